"""Re-planning between steps without a copy: when a row's length changes
inside its last page, the queue image (whole-page ranges) is unchanged, the
plan stays uploaded, and the next decode reads the new exact lengths from
the device. The ai-trend study note ("How it works", step four) has the
scheduler re-form the batch every step, so this is the per-step path."""

from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from oracle import paged_gqa as O

from .gpu_helpers import assert_parity, run_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
P = None


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    global P
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_04_amd  # fails loudly if the library is not built
    P = paged_kv_gqa_04_amd

LENS = [3000, 517, 1203, 45]  # none a multiple of 16: +1 stays in the last page


def _decode(plan, dev, lens, out):
    dev["seq_lens"].copy_(torch.from_numpy(np.asarray(lens, dtype=np.int32)))
    out.fill_(float("nan"))
    plan.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"], dev["seq_lens"], out)
    torch.cuda.synchronize()
    return out.to(torch.float64).cpu().numpy()


def _want(c, lens):
    return O.decode(c.q, c.k_pool, c.v_pool, c.block_table, np.asarray(lens, dtype=np.int32),
                    c.dtype, c.sm_scale)


@pytest.mark.parametrize("mode,S,chunk", [("workqueue", 0, 8), ("auto", 0, 0), ("split", 5, 0)])
def test_replan_inside_pages_keeps_the_upload(mode, S, chunk):
    c = W.make_case_from_lengths("replan", LENS, num_q_heads=8, num_kv_heads=2, head_dim=128,
                                 dtype=W.BF16, seed=31, poison=False)
    dev = W.case_to_device(c)
    got, plan, out = run_case(c, dev, mode=mode, num_splits=S, chunk_pages=chunk,
                              return_plan=True)
    assert_parity(got, _want(c, LENS), f"{mode} step 0")
    assert not P.pkv_plan_upload_needed(plan.handle)

    # Every row one token longer, no row gains a page: same image, no copy.
    lens1 = [n + 1 for n in LENS]
    plan.update(np.asarray(lens1, dtype=np.int32))
    assert not P.pkv_plan_upload_needed(plan.handle)
    assert_parity(_decode(plan, dev, lens1, out), _want(c, lens1), f"{mode} +1 without upload")

    # Row 1 gains a page (its table already names one there).
    lens2 = list(lens1)
    lens2[1] = 16 * ((lens1[1] + 15) // 16) + 3
    plan.update(np.asarray(lens2, dtype=np.int32))
    if mode == "split":
        # The split grid's image holds only the zeroed counters: the ranges
        # follow from the device lengths, so no copy is ever needed.
        assert not P.pkv_plan_upload_needed(plan.handle)
    else:
        # The work queue's last range of row 1 ends one page later.
        assert P.pkv_plan_upload_needed(plan.handle)
        with pytest.raises(P.PkvError):
            _decode(plan, dev, lens2, out)
        plan.upload()
        assert not P.pkv_plan_upload_needed(plan.handle)
    assert_parity(_decode(plan, dev, lens2, out), _want(c, lens2), f"{mode} new page")

    # A forced copy of the same image changes nothing.
    ref = out.clone()
    plan.upload(force=True)
    _decode(plan, dev, lens2, out)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    plan.close()


def test_replan_that_outgrows_the_workspace_needs_an_upload():
    lens = [40, 40]
    c = W.make_case_from_lengths("grow", [4000, 4000], num_q_heads=8, num_kv_heads=2,
                                 head_dim=64, dtype=W.F16, seed=32, poison=False)
    dev = W.case_to_device(c)
    plan = P.Plan(P.make_shape(2, 8, 2, 64, c.stride, c.num_pages, c.dtype, c.sm_scale), lens,
                  P.make_opts("workqueue", 0, 8))
    plan.upload()
    small = plan.workspace_bytes()
    out = torch.empty_like(dev["q"])
    assert_parity(_decode(plan, dev, lens, out), _want(c, lens), "short rows")
    lens = [4000, 3990]
    plan.update(np.asarray(lens, dtype=np.int32))
    assert plan.workspace_bytes() > small
    assert P.pkv_plan_upload_needed(plan.handle)
    plan.upload()  # grows the workspace
    assert_parity(_decode(plan, dev, lens, out), _want(c, lens), "long rows")
    plan.close()
