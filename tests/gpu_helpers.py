"""Shared helpers for the GPU tests: run the HIP path through the C ABI on a
host case, and compare with the oracle under the parity bar."""

from __future__ import annotations

import numpy as np

import workloads as W

# Parity bar for fp16/bf16 K/V with fp32 accumulation: an element passes when
# |gpu - oracle| <= max(ATOL, RTOL * |oracle|).
ATOL = 2e-3
RTOL = 1e-2


def parity(got: np.ndarray, want: np.ndarray) -> dict:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    bound = np.maximum(ATOL, RTOL * np.abs(want))
    big = np.abs(want) >= 0.2
    rel = (err[big] / np.abs(want[big])).max() if big.any() else 0.0
    norm = np.linalg.norm(want)
    return {
        "ok": bool(np.isfinite(got).all() and (err <= bound).all()),
        "max_abs": float(err.max()) if err.size else 0.0,
        "max_rel": float(rel),
        "normwise": float(np.linalg.norm(got - want) / norm) if norm > 0 else float(np.linalg.norm(got)),
        "worst": float((err / bound).max()) if err.size else 0.0,
    }


def assert_parity(got, want, label=""):
    r = parity(got, want)
    assert r["ok"], f"{label} parity failed: {r}"
    return r


def shape_of(case, num_pages=None):
    import paged_kv_gqa_04_amd as P
    return P.make_shape(case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim,
                        case.stride, case.num_pages if num_pages is None else num_pages,
                        case.dtype, case.sm_scale)


def run_case(case, dev=None, mode="auto", num_splits=0, chunk_pages=0, queue_seed=0,
             return_plan=False, merge="fused"):
    """Decode ``case`` on the GPU; returns float64 out (and the Plan)."""
    import torch

    import paged_kv_gqa_04_amd as P
    if dev is None:
        dev = W.case_to_device(case)
    out = torch.full_like(dev["q"], float("nan"))
    plan = P.Plan(shape_of(case), case.seq_lens,
                  P.make_opts(mode, num_splits, chunk_pages, 0, queue_seed, merge))
    plan.upload()
    plan.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                dev["seq_lens"], out)
    torch.cuda.synchronize()
    res = out.to(torch.float64).cpu().numpy()
    if return_plan:
        return res, plan, out
    plan.close()
    return res


def out_bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy()
