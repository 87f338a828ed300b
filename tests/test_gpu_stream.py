"""The plain streaming read that the bench times as the HBM floor reads every
16-byte piece of both buffers exactly as asked: with all words zero but one
marker word, only the thread that reads the marker ends with it as its
running XOR and writes it to the sink."""

from __future__ import annotations

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
P = None

MARK = 0x9E3779B9  # the value the kernel writes to the sink when it sees it


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    global P
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_04_amd  # fails loudly if the library is not built
    P = paged_kv_gqa_04_amd


def _read(a, b, n16, grid):
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    P.pkv_stream_read(a, b, n16 * 16, grid, sink, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return int(sink.item()) & 0xFFFFFFFF


# (pieces of 16 bytes per buffer, workgroups): remainders only, exact unrolled
# rounds, and unrolled rounds followed by a remainder
@pytest.mark.parametrize("n16,grid", [(1, 1), (1000, 3), (4096, 4), (10007, 2)])
@pytest.mark.parametrize("which", ["a", "b"])
def test_every_piece_is_read(n16, grid, which):
    for pos in sorted({0, n16 // 2, n16 - 1}):
        a = torch.zeros(n16 * 4, dtype=torch.int32, device="cuda")
        b = torch.zeros_like(a)
        word = 4 * pos + (pos % 4)  # each of the piece's four words in turn
        (a if which == "a" else b)[word] = MARK - (1 << 32)
        assert _read(a, b, n16, grid) == MARK, (n16, grid, which, pos)


def test_zero_data_and_zero_size_leave_the_sink_alone():
    a = torch.zeros(4096, dtype=torch.int32, device="cuda")
    assert _read(a, a, 1024, 2) == 0
    assert _read(a, a, 0, 2) == 0
