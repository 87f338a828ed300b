"""CPU float64 oracle for one paged grouped-query-attention decode step.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The library's
product path never calls it, and it shares no code with the HIP path: the two
meet only in the input bytes that ``workloads`` generates.

What it computes
----------------
For every sequence ``b`` and query head ``h`` (sources, by page and section):

* GQA grouping: ``G = Hq / Hkv`` query heads share one KV head
  (PersistentKV explainer, Technical summary, Methodology 1, native
  block-table decode engine). Grouping is contiguous: head ``h`` reads KV
  head ``h // G``, the usual repeat-KV convention (the page fixes only G).
* Paged storage: the cache is a flat pool of fixed 16-token blocks and a
  per-sequence block table maps logical block ``j`` to a physical page; keys
  and values are fetched through that table (LLM Primer ch. 8, section 8.1).
  The mapping moves storage only, never the logical token order (ZimaSpace
  post, section on fixed-size blocks). Logical token ``t`` of sequence ``b``
  is therefore slot ``t % P`` of page ``block_table[b, t // P]``.
* The decode step reads the cache directly through the table with no
  repacking (PersistentKV explainer, Methodology 1, layout).
* The attention itself is not printed on the pages; the plainest reading is
  standard scaled dot-product attention of one new query token over the
  ``N_b`` cached tokens: ``out = softmax(sm_scale * q K^T) V`` with
  ``sm_scale = 1/sqrt(d)`` unless another scale is given.
* An empty sequence (``N_b == 0``) yields zeros (the pages are silent; zero is
  the value the neutral merge state normalises to).

Computation is the plain definition: gather, exact two-pass softmax in float64
(max, exponentials, one normalisation), using numpy's matmul as the only
library primitive. Stored fp16 / bf16 bits are widened exactly, so no
rounding happens before accumulation.

``append_tokens`` is the step before decode: every sequence's new token is
stored at its next logical position ``N_b``, i.e. slot ``N_b % P`` of page
``block_table[b, N_b // P]`` (the same mapping; ZimaSpace post, fixed-size
blocks: a sequence takes further blocks from the shared pool as tokens
arrive). The oracle writes raw storage bits into copies of the pools.

``range_state`` and ``merge_states`` restate the split form from the same
page (Methodology 1, sequence splitting): the sequence axis is cut into
disjoint ranges, each summarised by a partial online-softmax state
``(m, l, acc)``, which a merge combines exactly. These exist to check the GPU
partial kernel on its own and to pin the split invariance; ``decode`` never
uses them.
"""

from __future__ import annotations

import math

import numpy as np

F16 = "f16"
BF16 = "bf16"


def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Widen raw fp16 / bf16 storage bits to float64 exactly.

    bf16 is the top half of an IEEE binary32, so its value is the binary32
    whose high 16 bits are the stored bits and whose low 16 bits are zero.
    """
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("expected raw uint16 storage bits")
    if dtype == BF16:
        wide = bits.astype(np.uint32) << np.uint32(16)
        return wide.view(np.float32).astype(np.float64)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float64)
    raise ValueError(f"unsupported dtype {dtype!r}")


def _scale(sm_scale, head_dim):
    return float(sm_scale) if sm_scale else 1.0 / math.sqrt(head_dim)


def gather_tokens(pool: np.ndarray, table_row: np.ndarray, t_begin: int,
                  t_end: int, kv_head: int, dtype: str) -> np.ndarray:
    """Rows ``[t_begin, t_end)`` of one sequence's keys (or values) for one
    KV head, fetched through the block table, as float64 ``[n, d]``."""
    P = pool.shape[2]
    t = np.arange(t_begin, t_end, dtype=np.int64)
    phys = np.asarray(table_row, dtype=np.int64)[t // P]
    return bits_to_f64(pool[phys, kv_head, t % P, :], dtype)


def decode(q, k_pool, v_pool, block_table, seq_lens, dtype, sm_scale=None,
           rows=None) -> np.ndarray:
    """One decode step; returns float64 ``[len(rows), Hq, d]``.

    ``q``: uint16 bits ``[B, Hq, d]``; pools: uint16 bits
    ``[num_pages, Hkv, P, d]``; ``block_table``: int ``[B, stride]``;
    ``seq_lens``: int ``[B]``. ``rows`` limits the work to some sequences.
    """
    B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    scale = _scale(sm_scale, d)
    rows = range(B) if rows is None else [int(r) for r in rows]
    out = np.zeros((len(rows), Hq, d), dtype=np.float64)
    for i, b in enumerate(rows):
        n = int(seq_lens[b])
        if n == 0:
            continue
        for g in range(Hkv):
            K = gather_tokens(k_pool, block_table[b], 0, n, g, dtype)
            V = gather_tokens(v_pool, block_table[b], 0, n, g, dtype)
            Q = bits_to_f64(q[b, g * G:(g + 1) * G, :], dtype)
            x = scale * (Q @ K.T)  # [G, n] logits
            m = x.max(axis=1, keepdims=True)
            w = np.exp(x - m)
            out[i, g * G:(g + 1) * G, :] = (w @ V) / w.sum(axis=1, keepdims=True)
    return out


def decode_case(case, rows=None) -> np.ndarray:
    return decode(case.q, case.k_pool, case.v_pool, case.block_table,
                  case.seq_lens, case.dtype, case.sm_scale, rows=rows)


def range_state(q, k_pool, v_pool, block_table, seq_lens, dtype, b, kv_head,
                t_begin, t_end, sm_scale=None):
    """Partial online-softmax state of tokens ``[t_begin, t_end)`` of sequence
    ``b`` (clipped to its length) for the G query heads of ``kv_head``.

    Returns ``(m, l, acc)`` with ``m[G]`` the largest scaled logit of the
    range, ``l[G] = sum exp(x - m)`` and ``acc[G, d] = sum exp(x - m) v``
    (unnormalised). An empty range is the neutral state ``(-inf, 0, 0)``.
    """
    B, Hq, d = q.shape
    G = Hq // k_pool.shape[1]
    t_end = min(int(t_end), int(seq_lens[b]))
    if t_end <= t_begin:
        return (np.full(G, -np.inf), np.zeros(G), np.zeros((G, d)))
    scale = _scale(sm_scale, d)
    K = gather_tokens(k_pool, block_table[b], t_begin, t_end, kv_head, dtype)
    V = gather_tokens(v_pool, block_table[b], t_begin, t_end, kv_head, dtype)
    Q = bits_to_f64(q[b, kv_head * G:(kv_head + 1) * G, :], dtype)
    x = scale * (Q @ K.T)
    m = x.max(axis=1)
    w = np.exp(x - m[:, None])
    return (m, w.sum(axis=1), w @ V)


def merge_states(states) -> np.ndarray:
    """Combine partial states of disjoint ranges into the normalised output.

    With ``M = max_s m_s``, each state is weighted by ``exp(m_s - M)``; a
    neutral state (``m = -inf``) weighs zero. If every state is neutral the
    result is zero. Returns float64 ``[G, d]``.
    """
    ms = np.stack([s[0] for s in states])  # [S, G]
    ls = np.stack([s[1] for s in states])  # [S, G]
    accs = np.stack([s[2] for s in states])  # [S, G, d]
    M = ms.max(axis=0)  # [G]
    out = np.zeros(accs.shape[1:], dtype=np.float64)
    for h in range(ms.shape[1]):
        if M[h] == -np.inf:
            continue
        w = np.where(ms[:, h] == -np.inf, 0.0, np.exp(ms[:, h] - M[h]))
        out[h] = (w[:, None] * accs[:, h, :]).sum(axis=0) / (w * ls[:, h]).sum()
    return out


def append_tokens(k_pool, v_pool, block_table, seq_lens, k_new, v_new, page=16):
    """Pools after one append step, as new arrays (inputs unchanged).

    Row ``b`` stores ``k_new[b]`` / ``v_new[b]`` (raw bits, [Hkv, d]) as its
    logical token ``N_b = seq_lens[b]``: page ``block_table[b, N_b // page]``,
    slot ``N_b % page``, every KV head. A row whose table entry is outside
    the pool stores nothing (the kernels' rule for untrusted entries).
    """
    k = np.array(k_pool, copy=True)
    v = np.array(v_pool, copy=True)
    for b, n in enumerate(np.asarray(seq_lens)):
        n = int(n)
        if n < 0 or n // page >= block_table.shape[1]:
            continue
        pg = int(block_table[b, n // page])
        if not 0 <= pg < k.shape[0]:
            continue
        k[pg, :, n % page, :] = k_new[b]
        v[pg, :, n % page, :] = v_new[b]
    return k, v
