"""The decode step captured in a HIP graph (one launch, or partial + merge,
or one launch per bucket) and replayed: each replay matches the eager
result bit for bit, also after the inputs change in place between replays
and with eager steps in between (the fused merge's counters are reset by
the kernel itself, with no memset node)."""

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


@pytest.mark.parametrize("mode,merge", [("split", "fused"), ("workqueue", "fused"),
                                        ("workqueue", "kernel"), ("bucketed", "kernel"),
                                        ("unsplit", "fused")])
def test_decode_graph_replays_match_eager(mode, merge):
    import paged_kv_gqa_04_amd as P
    c = W.make_case_from_lengths("graph", [3000, 17, 0, 900, 4100, 900], num_q_heads=8,
                                 num_kv_heads=2, head_dim=128, dtype=W.BF16, seed=31)
    dev = W.case_to_device(c)
    plan = P.Plan(shape_of(c), c.seq_lens, P.make_opts(mode, num_splits=5 if mode == "split" else 0,
                                                       chunk_pages=16, merge=merge))
    plan.upload()
    args = (dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"], dev["seq_lens"])

    def eager():
        o = torch.full_like(dev["q"], float("nan"))
        plan.decode(*args, o)
        torch.cuda.synchronize()
        return o

    ref = eager()
    assert_parity(ref.to(torch.float64).cpu().numpy(), O.decode_case(c), f"{mode}/{merge}")
    out = torch.full_like(dev["q"], float("nan"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream's kind of stream
        plan.decode(*args, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.decode(*args, out)
    for i in range(4):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out_bits(out), out_bits(ref), err_msg=f"replay {i}")
        np.testing.assert_array_equal(out_bits(eager()), out_bits(ref))  # eager in between
    # new query values in place: the replay reads them
    rng = np.random.default_rng(32)
    c.q = W.to_bits(rng.standard_normal(c.q.shape, dtype=np.float32), c.dtype)
    dev["q"].copy_(torch.from_numpy(c.q.view(np.int16)).view(dev["q"].dtype))
    graph.replay()
    torch.cuda.synchronize()
    assert_parity(out.to(torch.float64).cpu().numpy(), O.decode_case(c), "replay, new q")
    np.testing.assert_array_equal(out_bits(out), out_bits(eager()))
    plan.close()
