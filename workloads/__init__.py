"""Seeded synthetic inputs for one paged GQA decode step.

This module only *makes inputs*: sequence lengths, a shuffled physical page
pool, a block table, and N(0, 1) query / key / value data rounded to the
storage dtype. It holds none of the attention arithmetic, so both the CPU
oracle (``oracle/``) and the HIP path can consume the same bytes without
sharing any method code.

Storage conventions (the readings the library documents in its C header):

* ``q``: ``[B, Hq, d]``; ``k_pool`` / ``v_pool``: ``[num_pages, Hkv, P, d]``;
  all three are returned as ``uint16`` arrays holding the raw fp16 or bf16
  bits, so no host float type has to represent bf16.
* ``block_table``: int32 ``[B, stride]``; entry ``j`` of row ``b`` is the
  physical page that holds logical tokens ``[j*P, (j+1)*P)`` of sequence
  ``b`` (PagedAttention block tables: LLM Primer ch. 8, section 8.1; the
  ZimaSpace paged-attention post, "PagedAttention splits KV state into
  fixed-size blocks").
* ``seq_lens``: int32 ``[B]``; rows may be 0 (an idle slot).

Sub-streams come from ``np.random.default_rng([seed, config_id])`` and are
drawn in the fixed order: lengths, page permutation, q, K, V.

The two seeds follow the PersistentKV explainer, Technical summary, Results:
thresholds are calibrated on 20260622 and reported on the hold-out 20260623.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

SEED_CALIBRATION = 20260622
SEED_HOLDOUT = 20260623
PAGE_TOKENS = 16

F16 = "f16"
BF16 = "bf16"


@dataclass(frozen=True)
class ConfigSpec:
    """Shape and length distribution of one named synthetic workload."""

    name: str
    config_id: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    lengths: tuple  # ("fixed", n) | ("uniform", lo, hi) | ("loguniform", lo, hi)
    #                 | ("bucketed", n1, n2, ...) | ("bimodal", lo1, hi1, lo2, hi2, p)
    #                 | ("zipf", unit, kmax, a)
    pool_pages: int | None = None  # None: exactly the pages the batch uses
    num_splits: int | None = None  # S named by the workload, if any
    mode: str = "auto"  # the dispatch mode the workload is quoted in
    description: str = ""

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


CONFIGS: dict[str, ConfigSpec] = {
    "tiny": ConfigSpec(
        "tiny", 1, 1, 8, 2, 64, F16, ("fixed", 512), pool_pages=64, num_splits=4,
        mode="split",
        description="B=1, Hq=8, Hkv=2 (G=4), d=64, 512 tokens, fp16, 64-page "
                    "shuffled pool, S=4",
    ),
    "long": ConfigSpec(
        "long", 2, 1, 32, 8, 128, BF16, ("fixed", 32768), pool_pages=4096,
        num_splits=32, mode="split",
        description="B=1, Hq=32, Hkv=8 (G=4), d=128, 32768 tokens, bf16, "
                    "4096-page shuffled pool, S=32",
    ),
    "mixed8": ConfigSpec(
        "mixed8", 3, 8, 32, 8, 128, BF16, ("loguniform", 256, 32768),
        mode="workqueue",
        description="B=8, Hq=32, Hkv=8, d=128, bf16, lengths log-uniform in "
                    "[256, 32768], pages interleaved across sequences, work queue",
    ),
    "b4": ConfigSpec(
        "b4", 4, 4, 32, 8, 128, BF16, ("uniform", 2048, 16384), mode="auto",
        description="B=4, Hq=32, Hkv=8, d=128, bf16, lengths uniform in "
                    "[2048, 16384]; unsplit vs split vs work queue vs auto",
    ),
    "b64": ConfigSpec(
        "b64", 5, 64, 64, 8, 128, BF16, ("loguniform", 4096, 131072),
        mode="workqueue",
        description="B=64, Hq=64, Hkv=8 (G=8), d=128, bf16, lengths "
                    "log-uniform in [4096, 131072], work queue",
    ),
    # Trace families of the PersistentKV explainer (Evaluation protocol,
    # traces isolating context length, active batch size and raggedness).
    # The pages give no parameters; these are plain readings of the names.
    "bucketed1": ConfigSpec(
        "bucketed1", 6, 1, 32, 8, 128, BF16, ("bucketed", 8192, 16384, 32768, 65536),
        mode="auto",
        description="B=1, Hq=32, Hkv=8, d=128, bf16, length drawn from the "
                    "power-of-two buckets {8192, 16384, 32768, 65536}",
    ),
    "bimodal8": ConfigSpec(
        "bimodal8", 7, 8, 32, 8, 128, BF16, ("bimodal", 256, 1024, 16384, 32768, 0.5),
        mode="auto",
        description="B=8, Hq=32, Hkv=8, d=128, bf16, lengths short U[256, 1024] or "
                    "long U[16384, 32768] with probability 1/2 each",
    ),
    "uniform8": ConfigSpec(
        "uniform8", 8, 8, 32, 8, 128, BF16, ("uniform", 256, 32768), mode="auto",
        description="B=8, Hq=32, Hkv=8, d=128, bf16, lengths uniform in [256, 32768]",
    ),
    "zipf8": ConfigSpec(
        "zipf8", 9, 8, 32, 8, 128, BF16, ("zipf", 256, 128, 1.1), mode="auto",
        description="B=8, Hq=32, Hkv=8, d=128, bf16, lengths 256 k with k in 1..128 "
                    "drawn with probability proportional to k^-1.1 (Zipf-like)",
    ),
}

# The B=8 trace families, in the order the pages list them.
TRACE_FAMILIES = ("bimodal8", "uniform8", "zipf8")


def pages_for(n: int, page: int = PAGE_TOKENS) -> int:
    return (int(n) + page - 1) // page


def draw_lengths(lengths: tuple, batch: int, rng: np.random.Generator) -> np.ndarray:
    """Draw ``batch`` sequence lengths.

    * fixed: every row has ``n`` tokens;
    * uniform: integers in ``[lo, hi]`` inclusive;
    * loguniform: ``clip(round(exp(U(ln lo, ln hi))), lo, hi)``;
    * bucketed: each row takes one of the listed values, uniformly;
    * bimodal: with probability ``p`` uniform in ``[lo1, hi1]``, else in
      ``[lo2, hi2]``;
    * zipf: ``unit * k`` with ``k`` in ``1..kmax``, ``P(k)`` proportional to
      ``k^-a`` (inverse-CDF draw from one uniform per row).
    """
    kind = lengths[0]
    if kind == "fixed":
        return np.full(batch, int(lengths[1]), dtype=np.int32)
    if kind == "uniform":
        lo, hi = int(lengths[1]), int(lengths[2])
        return rng.integers(lo, hi + 1, size=batch).astype(np.int32)
    if kind == "loguniform":
        lo, hi = int(lengths[1]), int(lengths[2])
        u = rng.uniform(math.log(lo), math.log(hi), size=batch)
        return np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int32)
    if kind == "bucketed":
        values = np.asarray(lengths[1:], dtype=np.int64)
        return values[rng.integers(0, len(values), size=batch)].astype(np.int32)
    if kind == "bimodal":
        lo1, hi1, lo2, hi2, p = lengths[1:]
        first = rng.uniform(size=batch) < float(p)
        a = rng.integers(int(lo1), int(hi1) + 1, size=batch)
        b = rng.integers(int(lo2), int(hi2) + 1, size=batch)
        return np.where(first, a, b).astype(np.int32)
    if kind == "zipf":
        unit, kmax, a = int(lengths[1]), int(lengths[2]), float(lengths[3])
        w = np.arange(1, kmax + 1, dtype=np.float64) ** -a
        cdf = np.cumsum(w) / w.sum()
        k = np.searchsorted(cdf, rng.uniform(size=batch), side="right") + 1
        return (unit * np.minimum(k, kmax)).astype(np.int32)
    raise ValueError(f"unknown length distribution {kind!r}")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); raw bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE fp16 (numpy rounds to nearest even); raw bits."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    if dtype == F16:
        return f32_to_f16_bits(x)
    raise ValueError(f"unsupported dtype {dtype!r}")


NAN_BITS = {BF16: np.uint16(0x7FC0), F16: np.uint16(0x7E00)}


@dataclass
class Case:
    """One decode step's inputs, as raw host arrays."""

    name: str
    seed: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    dtype: str
    seq_lens: np.ndarray  # int32 [B]
    block_table: np.ndarray  # int32 [B, stride]
    q: np.ndarray  # uint16 bits [B, Hq, d]
    k_pool: np.ndarray  # uint16 bits [num_pages, Hkv, P, d]
    v_pool: np.ndarray  # uint16 bits [num_pages, Hkv, P, d]
    sm_scale: float
    num_splits: int | None = None
    mode: str = "auto"
    poison_page: int | None = None  # a NaN page that unused table entries name
    meta: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def stride(self) -> int:
        return int(self.block_table.shape[1])


def _layout_pool(seq_lens, rng, pool_pages, extra_pages, page):
    """Deal a seeded permutation of physical pages to the sequences in order.

    Returns (block_table, num_pages, poison_page). ``poison_page`` is a page no
    sequence owns, or None when the pool has no spare page.
    """
    pages = [pages_for(n, page) for n in seq_lens]
    need = int(sum(pages))
    total = need if pool_pages is None else int(pool_pages)
    if total < need:
        raise ValueError(f"pool of {total} pages cannot hold {need}")
    total += int(extra_pages)
    perm = rng.permutation(total).astype(np.int32)
    stride = max(1, max(pages) if pages else 1)
    bt = np.zeros((len(seq_lens), stride), dtype=np.int32)
    used = np.zeros(total, dtype=bool)
    cur = 0
    for b, np_b in enumerate(pages):
        bt[b, :np_b] = perm[cur:cur + np_b]
        used[perm[cur:cur + np_b]] = True
        cur += np_b
    spare = np.flatnonzero(~used)
    poison_page = int(spare[0]) if spare.size else None
    fill = poison_page if poison_page is not None else 0
    for b, np_b in enumerate(pages):
        bt[b, np_b:] = fill
    return bt, total, poison_page


def _poison(case: Case) -> None:
    """NaN-fill every pool slot that no sequence's first seq_len tokens name."""
    nan = NAN_BITS[case.dtype]
    P = case.page_size
    live = np.zeros((case.num_pages, P), dtype=bool)
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        for j in range(pages_for(n, P)):
            valid = min(P, n - j * P)
            live[case.block_table[b, j], :valid] = True
    pages, slots = np.nonzero(~live)
    case.k_pool[pages, :, slots, :] = nan
    case.v_pool[pages, :, slots, :] = nan


def make_case_from_lengths(
    name: str,
    seq_lens,
    *,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    dtype: str,
    seed: int,
    config_id: int = 0,
    pool_pages: int | None = None,
    extra_pages: int = 1,
    poison: bool = True,
    identity: bool = False,
    num_splits: int | None = None,
    mode: str = "auto",
    sm_scale: float | None = None,
    page_size: int = PAGE_TOKENS,
    rng: np.random.Generator | None = None,
) -> Case:
    """Build a case for explicit lengths (used by tests and the named configs)."""
    if rng is None:
        rng = np.random.default_rng([seed, config_id])
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = int(seq_lens.shape[0])
    if identity:
        pages = [pages_for(n, page_size) for n in seq_lens]
        stride = max(1, max(pages) if pages else 1)
        total = int(sum(pages)) + int(extra_pages)
        bt = np.zeros((B, stride), dtype=np.int32)
        cur = 0
        for b, np_b in enumerate(pages):
            bt[b, :np_b] = np.arange(cur, cur + np_b, dtype=np.int32)
            cur += np_b
        poison_page = cur if extra_pages > 0 else None
        for b, np_b in enumerate(pages):
            bt[b, np_b:] = poison_page if poison_page is not None else 0
        num_pages = total
    else:
        bt, num_pages, poison_page = _layout_pool(
            seq_lens, rng, pool_pages, extra_pages, page_size)
    shape_q = (B, num_q_heads, head_dim)
    shape_kv = (num_pages, num_kv_heads, page_size, head_dim)
    q = to_bits(rng.standard_normal(shape_q, dtype=np.float32), dtype)
    k = to_bits(rng.standard_normal(shape_kv, dtype=np.float32), dtype)
    v = to_bits(rng.standard_normal(shape_kv, dtype=np.float32), dtype)
    case = Case(
        name=name, seed=seed, batch=B, num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, page_size=page_size,
        dtype=dtype, seq_lens=seq_lens, block_table=bt, q=q, k_pool=k,
        v_pool=v,
        sm_scale=float(sm_scale) if sm_scale else 1.0 / math.sqrt(head_dim),
        num_splits=num_splits, mode=mode, poison_page=poison_page,
    )
    if poison:
        _poison(case)
    return case


def make_case(name: str, seed: int = SEED_HOLDOUT, *, poison: bool = True,
              extra_pages: int | None = None) -> Case:
    """Host-generated inputs for a named workload (all but the largest)."""
    spec = CONFIGS[name]
    rng = np.random.default_rng([seed, spec.config_id])
    seq_lens = draw_lengths(spec.lengths, spec.batch, rng)
    if extra_pages is None:
        extra_pages = 0 if spec.pool_pages is not None else 1
    return make_case_from_lengths(
        name, seq_lens, num_q_heads=spec.num_q_heads,
        num_kv_heads=spec.num_kv_heads, head_dim=spec.head_dim,
        dtype=spec.dtype, seed=seed, config_id=spec.config_id,
        pool_pages=spec.pool_pages, extra_pages=extra_pages, poison=poison,
        num_splits=spec.num_splits, mode=spec.mode, rng=rng,
    )


def algorithmic_bytes(seq_lens, num_q_heads, num_kv_heads, head_dim,
                      elem_bytes=2, page=PAGE_TOKENS) -> int:
    """Bytes one decode step must move: K/V of the exact tokens, q, out, the
    used block-table entries and seq_lens."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    kv = int(seq_lens.sum()) * num_kv_heads * head_dim * 2 * elem_bytes
    qo = 2 * len(seq_lens) * num_q_heads * head_dim * elem_bytes
    bt = int(sum(pages_for(n, page) for n in seq_lens)) * 4
    return kv + qo + bt + 4 * len(seq_lens)


# --------------------------------------------------------------------------
# Device-side helpers (torch is plumbing only: device memory and generators).
# --------------------------------------------------------------------------

def torch_dtype(dtype: str):
    import torch
    return torch.bfloat16 if dtype == BF16 else torch.float16


def case_to_device(case: Case, device="cuda"):
    """Copy a host case to device tensors (bit-exact)."""
    import torch
    td = torch_dtype(case.dtype)

    def bits(a):
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
        return t.to(device).view(td)

    return {
        "q": bits(case.q),
        "k_pool": bits(case.k_pool),
        "v_pool": bits(case.v_pool),
        "block_table": torch.from_numpy(np.ascontiguousarray(case.block_table)).to(device),
        "seq_lens": torch.from_numpy(np.ascontiguousarray(case.seq_lens)).to(device),
    }


def make_device_case(name: str, seed: int = SEED_HOLDOUT, device="cuda",
                     chunk_pages: int = 4096):
    """Generate a named workload directly in device memory.

    Lengths and the page permutation come from numpy (so the host knows the
    layout); q/K/V are N(0,1) from a seeded torch device generator, rounded to
    the storage dtype. Used for the largest workload, whose pools do not fit
    comfortably in host memory; the host keeps only the metadata.
    """
    import torch
    spec = CONFIGS[name]
    rng = np.random.default_rng([seed, spec.config_id])
    seq_lens = draw_lengths(spec.lengths, spec.batch, rng)
    bt, num_pages, poison_page = _layout_pool(
        seq_lens, rng, spec.pool_pages, 0, PAGE_TOKENS)
    td = torch_dtype(spec.dtype)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1000 + spec.config_id)
    Hkv, d, P = spec.num_kv_heads, spec.head_dim, PAGE_TOKENS

    def pool():
        t = torch.empty((num_pages, Hkv, P, d), dtype=td, device=device)
        for s in range(0, num_pages, chunk_pages):
            e = min(num_pages, s + chunk_pages)
            t[s:e] = torch.randn((e - s, Hkv, P, d), generator=gen,
                                 device=device, dtype=torch.float32).to(td)
        return t

    q = torch.randn((spec.batch, spec.num_q_heads, d), generator=gen,
                    device=device, dtype=torch.float32).to(td)
    k_pool = pool()
    v_pool = pool()
    return {
        "spec": spec,
        "seq_lens_host": seq_lens,
        "block_table_host": bt,
        "num_pages": num_pages,
        "q": q,
        "k_pool": k_pool,
        "v_pool": v_pool,
        "block_table": torch.from_numpy(bt).to(device),
        "seq_lens": torch.from_numpy(seq_lens).to(device),
        "sm_scale": 1.0 / math.sqrt(d),
    }


def host_subcase_from_device(dev: dict, rows, name="sample") -> Case:
    """Copy the pages that ``rows`` of a device case use back to the host,
    renumbered into a compact pool, as a host Case (for sampled checks)."""
    import torch
    spec = dev["spec"]
    rows = [int(r) for r in rows]
    sl = dev["seq_lens_host"][rows].astype(np.int32)
    bt_full = dev["block_table_host"]
    pages = [pages_for(n) for n in sl]
    stride = max(1, max(pages))
    phys = np.concatenate([bt_full[r, :p] for r, p in zip(rows, pages)]).astype(np.int64)
    idx = torch.from_numpy(phys).to(dev["k_pool"].device)
    k = dev["k_pool"].index_select(0, idx).view(torch.int16).cpu().numpy().view(np.uint16)
    v = dev["v_pool"].index_select(0, idx).view(torch.int16).cpu().numpy().view(np.uint16)
    q = dev["q"][rows].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    bt = np.zeros((len(rows), stride), dtype=np.int32)
    cur = 0
    for i, p in enumerate(pages):
        bt[i, :p] = np.arange(cur, cur + p, dtype=np.int32)
        cur += p
    return Case(
        name=name, seed=-1, batch=len(rows), num_q_heads=spec.num_q_heads,
        num_kv_heads=spec.num_kv_heads, head_dim=spec.head_dim,
        page_size=PAGE_TOKENS, dtype=spec.dtype, seq_lens=sl, block_table=bt,
        q=q, k_pool=k, v_pool=v, sm_scale=dev["sm_scale"],
    )
