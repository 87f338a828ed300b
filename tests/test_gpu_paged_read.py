"""The paged read, a measurement aid timed beside the decode, reads each K/V
tile the decode reads exactly once and no other: with both pools zero but
for one marker word, the sink ends with the marker exactly when the plan's
pages cover the marked tile (the lane that reads it folds it in once)."""

from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
P = None

MARK = 0x9E3779B9  # the value a lane writes to the sink when its data folds to it
LENS = [300, 0, 1000, 17, 64]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    global P
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_04_amd  # fails loudly if the library is not built
    P = paged_kv_gqa_04_amd


def _setup(mode, S, chunk, Hkv, D):
    """A plan over LENS with its rows' pages scattered over pages 1.. of the
    pool; page 0 and a few more are used by no row, and the table entries
    past each row's last page point at unused pages."""
    pages = [(n + 15) // 16 for n in LENS]
    stride = max(pages) + 3
    num_pages = sum(pages) + 6
    rng = np.random.default_rng(7)
    perm = 1 + rng.permutation(num_pages - 1)
    bt = np.zeros((len(LENS), stride), np.int32)
    off = 0
    for b, pg in enumerate(pages):
        bt[b, :pg] = perm[off:off + pg]
        off += pg
    unused = [0] + [int(p) for p in perm[off:]]
    for b, pg in enumerate(pages):
        bt[b, pg:] = unused[1 + b % (len(unused) - 1)]
    shape = P.make_shape(len(LENS), 4 * Hkv, Hkv, D, stride, num_pages, "bf16")
    plan = P.Plan(shape, np.asarray(LENS, np.int32), P.make_opts(mode, S, chunk))
    plan.upload()
    return plan, bt, unused, num_pages


def _read(plan, bt, num_pages, Hkv, D, phys, g, which, word):
    words = 16 * D // 2  # int32 words of one (page, KV head) tile
    k = torch.zeros(num_pages * Hkv * words, dtype=torch.int32, device="cuda")
    v = torch.zeros_like(k)
    (k if which == "k" else v)[(phys * Hkv + g) * words + word] = MARK - (1 << 32)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    lens = torch.from_numpy(np.asarray(LENS, np.int32)).cuda()
    P.pkv_paged_read(plan.handle, k, v, torch.from_numpy(bt).cuda(), lens, sink,
                     torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return int(sink.item()) & 0xFFFFFFFF


CASES = [("split", 3, 0), ("workqueue", 0, 8), ("unsplit", 0, 0)]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mode,S,chunk", CASES)
def test_every_read_tile_is_read_once(mode, S, chunk, D):
    Hkv = 2
    plan, bt, unused, num_pages = _setup(mode, S, chunk, Hkv, D)
    words = 16 * D // 2
    rng = np.random.default_rng(11)
    for b, n in enumerate(LENS):
        pg = (n + 15) // 16
        for lp in sorted({0, pg // 2, pg - 1}) if pg else []:
            g = int(rng.integers(Hkv))
            which = "kv"[int(rng.integers(2))]
            word = int(rng.integers(words))
            got = _read(plan, bt, num_pages, Hkv, D, int(bt[b, lp]), g, which, word)
            assert got == MARK, (mode, D, b, lp, g, which, word)
    plan.close()


@pytest.mark.parametrize("mode,S,chunk", CASES)
def test_pages_no_row_uses_are_not_read(mode, S, chunk):
    Hkv, D = 2, 128
    plan, bt, unused, num_pages = _setup(mode, S, chunk, Hkv, D)
    for phys in unused:
        for which in "kv":
            assert _read(plan, bt, num_pages, Hkv, D, phys, 1, which, 5) == 0, (mode, phys)
    plan.close()


def test_an_entry_outside_the_pool_reads_page_zero_instead():
    Hkv, D = 2, 128
    plan, bt, unused, num_pages = _setup("split", 3, 0, Hkv, D)
    replaced = int(bt[2, 7])
    bt[2, 7] = num_pages + 3  # page 0 is used by no row, so it is read once
    assert _read(plan, bt, num_pages, Hkv, D, 0, 1, "v", 9) == MARK
    assert _read(plan, bt, num_pages, Hkv, D, replaced, 1, "v", 9) == 0
    plan.close()
