"""pkv_decode_static, the entry point that allocates nothing (the plan's
workspace lives in the library's own device scratch), against pkv_decode
with a caller-bound workspace, through the C ABI: identical bits and oracle
parity, on two calls in a row with the second input smaller (the scratch
keeps whatever the previous call left), in every mode."""

import numpy as np
import pytest

import workloads as W
from oracle import paged_gqa as O
from tests.gpu_helpers import assert_parity, out_bits, shape_of

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_04_amd  # noqa: F401  (fails loudly if not built)


MODES = [("split", "fused", 6, 0), ("workqueue", "fused", 0, 5), ("workqueue", "kernel", 0, 5),
         ("auto", "fused", 0, 0), ("unsplit", "fused", 0, 0), ("bucketed", "fused", 0, 0),
         ("bucketed", "kernel", 0, 0)]


def _pair(mode, merge, S, chunk, c):
    import paged_kv_gqa_04_amd as P
    dev = W.case_to_device(c)
    args = (dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"], dev["seq_lens"])
    stream = torch.cuda.current_stream().cuda_stream
    with P.Plan(shape_of(c), c.seq_lens, P.make_opts(mode, S, chunk, merge=merge)) as plan:
        got = torch.full_like(dev["q"], float("nan"))
        P.pkv_decode_static(plan.handle, *args, got, stream)  # no upload needed
        torch.cuda.synchronize()
        plan.upload()
        ref = torch.full_like(dev["q"], float("nan"))
        plan.decode(*args, ref)
        torch.cuda.synchronize()
        return got, ref


@pytest.mark.parametrize("mode,merge,S,chunk", MODES)
def test_static_scratch_matches_the_bound_workspace(mode, merge, S, chunk):
    big = W.make_case_from_lengths("big", [9000, 300, 0, 4100, 17], num_q_heads=32,
                                   num_kv_heads=8, head_dim=128, dtype=W.BF16, seed=41)
    small = W.make_case_from_lengths("small", [700, 33], num_q_heads=32, num_kv_heads=8,
                                     head_dim=128, dtype=W.BF16, seed=42)
    for c in (big, small):  # the second call is smaller
        got, ref = _pair(mode, merge, S, chunk, c)
        np.testing.assert_array_equal(out_bits(got), out_bits(ref), err_msg=f"{mode}/{c.name}")
        assert_parity(got.to(torch.float64).cpu().numpy(), O.decode_case(c), f"{mode}/{c.name}")


def test_static_scratch_across_plans_and_steps():
    """Plans of different shapes take turns on the one scratch, several
    steps each, fp16 and bf16: every call equals its own bound-workspace
    result."""
    import paged_kv_gqa_04_amd as P
    cases = [W.make_case_from_lengths("a", [20000, 5000, 12000, 1], num_q_heads=16,
                                      num_kv_heads=2, head_dim=128, dtype=W.BF16, seed=51),
             W.make_case_from_lengths("b", [300, 40], num_q_heads=8, num_kv_heads=1,
                                      head_dim=64, dtype=W.F16, seed=52)]
    stream = torch.cuda.current_stream().cuda_stream
    plans, refs, devs = [], [], []
    for c in cases:
        dev = W.case_to_device(c)
        plan = P.Plan(shape_of(c), c.seq_lens, P.make_opts("workqueue", chunk_pages=16))
        plan.upload()
        ref = torch.full_like(dev["q"], float("nan"))
        plan.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"], dev["seq_lens"],
                    ref)
        plans.append(plan)
        refs.append(out_bits(ref))
        devs.append(dev)
    torch.cuda.synchronize()
    for step in range(6):
        i = step % 2
        d = devs[i]
        got = torch.full_like(d["q"], float("nan"))
        P.pkv_decode_static(plans[i].handle, d["q"], d["k_pool"], d["v_pool"], d["block_table"],
                            d["seq_lens"], got, stream)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out_bits(got), refs[i], err_msg=f"step {step}")
    for plan in plans:
        plan.close()
