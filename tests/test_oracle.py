"""Pins for the CPU oracle, each against something other than the oracle.

* IEEE binary16 / bfloat16 definitions for the bit widening;
* PyTorch's scaled_dot_product_attention (float64, GQA mode, default scale)
  on dense tensors that the test scatters into a shuffled pool itself;
* closed forms (one token, constant values, zero query, a dominant key);
* invariants: page permutation, split count and merge order, GQA = MHA on
  repeated KV heads, NaN in storage no sequence owns;
* planted mistakes in the oracle (on the CPU) that these pins must catch.
"""

import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import paged_gqa as O

# ----------------------------------------------------------------- helpers


def torch_widen(bits: np.ndarray, dtype: str) -> torch.Tensor:
    """float64 values of storage bits, decoded by torch (not by the oracle)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    td = torch.bfloat16 if dtype == W.BF16 else torch.float16
    return t.view(td).to(torch.float64)


def scatter_dense(kd: np.ndarray, vd: np.ndarray, lens, perm_seed, page=16,
                  extra=3, identity=False):
    """Lay dense per-sequence K/V bits ``[B][Hkv, N_b, d]`` into a paged pool.

    Written independently of the oracle: logical block j of sequence b goes
    to page ``perm[cursor + j]``; slot s of that page holds token j*page+s.
    Free pages and tail slots hold NaN bits.
    """
    B = len(lens)
    Hkv, d = kd[0].shape[0], kd[0].shape[2]
    npg = [(n + page - 1) // page for n in lens]
    total = sum(npg) + extra
    rng = np.random.default_rng(perm_seed)
    perm = np.arange(total) if identity else rng.permutation(total)
    nan = np.uint16(0x7FC0)
    kp = np.full((total, Hkv, page, d), nan, dtype=np.uint16)
    vp = np.full((total, Hkv, page, d), nan, dtype=np.uint16)
    stride = max(1, max(npg))
    bt = np.full((B, stride), perm[-1], dtype=np.int32)  # a free NaN page
    cur = 0
    for b in range(B):
        for j in range(npg[b]):
            p = perm[cur + j]
            bt[b, j] = p
            for s in range(page):
                t = j * page + s
                if t < lens[b]:
                    kp[p, :, s, :] = kd[b][:, t, :]
                    vp[p, :, s, :] = vd[b][:, t, :]
        cur += npg[b]
    return kp, vp, bt


def random_dense(rng, B, Hq, Hkv, d, lens, dtype):
    q = W.to_bits(rng.standard_normal((B, Hq, d), dtype=np.float32), dtype)
    kd = [W.to_bits(rng.standard_normal((Hkv, n, d), dtype=np.float32), dtype)
          for n in lens]
    vd = [W.to_bits(rng.standard_normal((Hkv, n, d), dtype=np.float32), dtype)
          for n in lens]
    return q, kd, vd


def sdpa_reference(q, kd, vd, lens, dtype):
    """torch SDPA (float64, enable_gqa, default 1/sqrt(d) scale) per sequence."""
    B, Hq, d = q.shape
    out = np.zeros((B, Hq, d))
    for b in range(B):
        if lens[b] == 0:
            continue
        qq = torch_widen(q[b], dtype)[None, :, None, :]  # [1, Hq, 1, d]
        kk = torch_widen(kd[b], dtype)[None]  # [1, Hkv, N, d]
        vv = torch_widen(vd[b], dtype)[None]
        o = torch.nn.functional.scaled_dot_product_attention(
            qq, kk, vv, enable_gqa=True)
        out[b] = o[0, :, 0, :].numpy()
    return out


# ----------------------------------------------------- bit widening (IEEE)


@pytest.mark.parametrize("bits,value", [
    (0x3F80, 1.0), (0xC000, -2.0), (0x4049, 3.140625), (0x0001, 2.0 ** -133),
    (0x0080, 2.0 ** -126), (0x7F7F, (2 - 2.0 ** -7) * 2.0 ** 127),
    (0x8000, -0.0), (0x7F80, math.inf), (0xFF80, -math.inf),
])
def test_bf16_widening_ieee(bits, value):
    got = O.bits_to_f64(np.array([bits], dtype=np.uint16), O.BF16)[0]
    assert got == value and math.copysign(1, got) == math.copysign(1, value)


@pytest.mark.parametrize("bits,value", [
    (0x3C00, 1.0), (0xC000, -2.0), (0x0001, 2.0 ** -24), (0x0400, 2.0 ** -14),
    (0x7BFF, 65504.0), (0x3555, 0.333251953125), (0xFC00, -math.inf),
])
def test_f16_widening_ieee(bits, value):
    got = O.bits_to_f64(np.array([bits], dtype=np.uint16), O.F16)[0]
    assert got == value


def test_bf16_nan_bits_widen_to_nan():
    assert np.isnan(O.bits_to_f64(np.array([0x7FC0], np.uint16), O.BF16)[0])
    assert np.isnan(O.bits_to_f64(np.array([0x7E00], np.uint16), O.F16)[0])


# ------------------------------------------- brute force via library SDPA

DENSE_LENS = [0, 1, 2, 15, 16, 17, 33, 100]


@pytest.mark.parametrize("dtype", [W.BF16, W.F16])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("Hkv,d", [(1, 8), (2, 64), (2, 8)])
def test_oracle_matches_torch_sdpa(dtype, G, Hkv, d):
    rng = np.random.default_rng([7, G, Hkv, d, dtype == W.BF16])
    Hq = G * Hkv
    for trial in range(3):
        B = int(rng.integers(1, 4))
        lens = [int(x) for x in rng.choice(DENSE_LENS, size=B)]
        q, kd, vd = random_dense(rng, B, Hq, Hkv, d, lens, dtype)
        kp, vp, bt = scatter_dense(kd, vd, lens, perm_seed=trial)
        got = O.decode(q, kp, vp, bt, np.array(lens), dtype)
        want = sdpa_reference(q, kd, vd, lens, dtype)
        assert np.isfinite(got).all()
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)
        for b, n in enumerate(lens):
            if n == 0:
                assert (got[b] == 0).all()


# ------------------------------------------------------------- closed forms


def _case(lens, G=4, Hkv=2, d=64, dtype=W.BF16, seed=3):
    return W.make_case_from_lengths(
        "pin", lens, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=d,
        dtype=dtype, seed=seed)


def test_single_token_returns_its_value_exactly():
    c = _case([1, 1, 1])
    out = O.decode_case(c)
    for b in range(3):
        for h in range(c.num_q_heads):
            v0 = O.bits_to_f64(c.v_pool[c.block_table[b, 0], h // c.group, 0], c.dtype)
            assert np.array_equal(out[b, h], v0)


def test_constant_values_return_the_constant():
    c = _case([37, 200])
    val = W.to_bits(np.linspace(-3, 3, c.head_dim, dtype=np.float32), c.dtype)
    c.v_pool[:, :, :, :] = val  # every token of every head has the same row
    out = O.decode_case(c)
    np.testing.assert_allclose(out, np.broadcast_to(O.bits_to_f64(val, c.dtype), out.shape),
                               rtol=1e-14, atol=0)


def test_zero_query_gives_uniform_average():
    c = _case([50, 129])
    c.q[:] = 0
    out = O.decode_case(c)
    for b, n in enumerate(c.seq_lens):
        for g in range(c.num_kv_heads):
            t = np.arange(n)
            V = O.bits_to_f64(
                c.v_pool[c.block_table[b, t // 16], g, t % 16], c.dtype)
            mean = np.sum(V, axis=0) / n
            for h in range(g * c.group, (g + 1) * c.group):
                np.testing.assert_allclose(out[b, h], mean, rtol=1e-12, atol=1e-13)


def test_dominant_key_selects_its_value():
    # q = e_0 * 16, key t* has k_0 = 64, all other keys have k_0 = 0 and the
    # rest of q is zero, so logit(t*) - logit(t) = 16*64/sqrt(d) = 128 > 50.
    c = _case([77], G=2, Hkv=1, d=64)
    c.q[:] = W.to_bits(np.zeros((1, 2, 64), np.float32), c.dtype)
    c.q[:, :, 0] = W.to_bits(np.array([16.0], np.float32), c.dtype)[0]
    t = np.arange(77)
    pages, slots = c.block_table[0, t // 16], t % 16
    c.k_pool[pages, 0, slots, 0] = W.to_bits(np.array([0.0], np.float32), c.dtype)[0]
    star = 41
    c.k_pool[pages[star], 0, slots[star], 0] = W.to_bits(np.array([64.0], np.float32), c.dtype)[0]
    out = O.decode_case(c)
    v_star = O.bits_to_f64(c.v_pool[pages[star], 0, slots[star]], c.dtype)
    vmax = np.abs(O.bits_to_f64(c.v_pool[pages, 0, slots], c.dtype)).max()
    for h in range(2):
        assert np.abs(out[0, h] - v_star).max() <= 77 * math.exp(-128) * 2 * vmax + 1e-300


def test_empty_rows_are_zero():
    c = _case([0, 33, 0])
    out = O.decode_case(c)
    assert (out[0] == 0).all() and (out[2] == 0).all()
    assert np.abs(out[1]).max() > 0


def test_two_token_closed_form():
    # Two tokens: out = (v0 + e^D v1) / (1 + e^D), D = scale*(q.k1 - q.k0).
    c = _case([2], G=1, Hkv=1, d=64, seed=11)
    out = O.decode_case(c)
    bt = c.block_table[0, 0]
    q = torch_widen(c.q[0, 0], c.dtype).numpy()
    k0, k1 = (torch_widen(c.k_pool[bt, 0, s], c.dtype).numpy() for s in (0, 1))
    v0, v1 = (torch_widen(c.v_pool[bt, 0, s], c.dtype).numpy() for s in (0, 1))
    D = (math.fsum(q * k1) - math.fsum(q * k0)) / 8.0
    want = (v0 + math.exp(D) * v1) / (1 + math.exp(D))
    np.testing.assert_allclose(out[0, 0], want, rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------- invariants


def test_page_permutation_is_exactly_invariant():
    rng = np.random.default_rng(5)
    lens = [16, 100, 1, 257]
    q, kd, vd = random_dense(rng, 4, 8, 2, 64, lens, W.BF16)
    outs = []
    for seed, ident in [(0, True), (1, False), (2, False)]:
        kp, vp, bt = scatter_dense(kd, vd, lens, perm_seed=seed, identity=ident)
        outs.append(O.decode(q, kp, vp, bt, np.array(lens), W.BF16))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_nan_in_unowned_storage_does_not_reach_output():
    clean = W.make_case("tiny", seed=99, poison=False)
    dirty = W.make_case("tiny", seed=99, poison=True)
    assert np.isnan(O.bits_to_f64(dirty.k_pool, dirty.dtype)).any()
    a, b = O.decode_case(clean), O.decode_case(dirty)
    assert np.isfinite(b).all() and np.array_equal(a, b)


@pytest.mark.parametrize("S", [1, 2, 3, 4, 7, 32, "pages"])
def test_split_merge_equals_plain(S):
    c = _case([513, 16, 300, 1], seed=21)
    plain = O.decode_case(c)
    rng = np.random.default_rng(hash(str(S)) % 1000)
    for b, n in enumerate(c.seq_lens):
        pages = (n + 15) // 16
        s_count = pages if S == "pages" else S
        chunk = max(1, -(-pages // s_count))
        bounds = [min(pages, i * chunk) * 16 for i in range(s_count + 1)]
        for g in range(c.num_kv_heads):
            states = [O.range_state(c.q, c.k_pool, c.v_pool, c.block_table,
                                    c.seq_lens, c.dtype, b, g, bounds[i],
                                    bounds[i + 1], c.sm_scale)
                      for i in range(s_count)]
            merged = O.merge_states(states)
            hs = slice(g * c.group, (g + 1) * c.group)
            np.testing.assert_allclose(merged, plain[b, hs], rtol=1e-12, atol=1e-14)
            # merge is order independent (commutative and associative)
            order = rng.permutation(len(states))
            again = O.merge_states([states[i] for i in order])
            np.testing.assert_allclose(again, merged, rtol=1e-13, atol=1e-15)
            # random (not page-aligned) cut points give the same result
            cuts = np.sort(rng.integers(0, n + 1, size=5))
            edges = [0, *cuts.tolist(), int(n)]
            st = [O.range_state(c.q, c.k_pool, c.v_pool, c.block_table,
                                c.seq_lens, c.dtype, b, g, edges[i], edges[i + 1],
                                c.sm_scale) for i in range(len(edges) - 1)]
            np.testing.assert_allclose(O.merge_states(st), plain[b, hs],
                                       rtol=1e-12, atol=1e-14)


def test_neutral_states_merge_to_zero_and_weigh_nothing():
    G, d = 4, 8
    neutral = (np.full(G, -np.inf), np.zeros(G), np.zeros((G, d)))
    assert (O.merge_states([neutral, neutral]) == 0).all()
    rng = np.random.default_rng(0)
    real = (rng.standard_normal(G), rng.random(G) + 0.5, rng.standard_normal((G, d)))
    np.testing.assert_array_equal(O.merge_states([neutral, real, neutral]),
                                  O.merge_states([real]))


def test_gqa_equals_mha_on_repeated_heads():
    c = _case([70, 5, 160], G=4, Hkv=2, d=64, seed=8)
    out = O.decode_case(c)
    rep = lambda p: np.repeat(p, c.group, axis=1)  # KV head h//G -> head h
    mha = O.decode(c.q, rep(c.k_pool), rep(c.v_pool), c.block_table, c.seq_lens,
                   c.dtype, c.sm_scale)
    np.testing.assert_allclose(out, mha, rtol=1e-13, atol=1e-15)


# ------------------------------------------------ planted mistakes are seen


def _dense_mismatch(monkeypatch=None, q_perm=None, scale=None):
    rng = np.random.default_rng(17)
    lens = [40, 77]
    q, kd, vd = random_dense(rng, 2, 8, 2, 8, lens, W.BF16)
    kp, vp, bt = scatter_dense(kd, vd, lens, perm_seed=4)
    qq = q if q_perm is None else q[:, q_perm, :]
    got = O.decode(qq, kp, vp, bt, np.array(lens), W.BF16, sm_scale=scale)
    want = sdpa_reference(q, kd, vd, lens, W.BF16)
    diff = np.abs(got - want)
    return math.inf if np.isnan(diff).any() else diff.max()


def test_planted_gather_swap_is_caught(monkeypatch):
    real = O.gather_tokens

    def swapped(pool, row, t0, t1, g, dtype):
        P = pool.shape[2]
        t = np.arange(t0, t1)
        phys = np.asarray(row)[t % P % len(row)]  # page/slot roles swapped
        return O.bits_to_f64(pool[phys, g, (t // P) % P, :], dtype)

    assert _dense_mismatch() < 1e-12
    monkeypatch.setattr(O, "gather_tokens", swapped)
    assert _dense_mismatch() > 1e-3
    monkeypatch.setattr(O, "gather_tokens", real)


def test_planted_wrong_grouping_and_scale_are_caught():
    # head h reading KV head h % Hkv instead of h // G is the same as
    # permuting the query heads; a dropped 1/sqrt(d) is scale 1.
    G, Hkv = 4, 2
    interleaved = [(h % G) * Hkv + h // G for h in range(G * Hkv)]
    assert _dense_mismatch(q_perm=interleaved) > 1e-3
    assert _dense_mismatch(scale=1.0) > 1e-3


# --------------------------------------------------------------- KV append


@pytest.mark.parametrize("lens", [[0, 1, 15, 16, 17, 31, 32, 100]])
@pytest.mark.parametrize("dtype", [W.BF16, W.F16])
def test_append_stores_the_next_token_where_decode_reads_it(lens, dtype):
    """Build the cache of N_b + 1 tokens independently, erase token N_b, let
    the oracle append it back: the pools must match bit for bit, and decode
    over N_b + 1 tokens must equal torch SDPA on the dense sequences."""
    rng = np.random.default_rng([11, dtype == W.BF16])
    B, Hq, Hkv, d = len(lens), 8, 2, 16
    full = [n + 1 for n in lens]
    q, kd, vd = random_dense(rng, B, Hq, Hkv, d, full, dtype)
    kp, vp, bt = scatter_dense(kd, vd, full, perm_seed=5)
    before_k, before_v = kp.copy(), vp.copy()
    k_new = np.stack([kd[b][:, n, :] for b, n in enumerate(lens)])  # [B, Hkv, d]
    v_new = np.stack([vd[b][:, n, :] for b, n in enumerate(lens)])
    nan = np.uint16(0x7FC0)
    for b, n in enumerate(lens):  # erase token N_b
        before_k[bt[b, n // 16], :, n % 16, :] = nan
        before_v[bt[b, n // 16], :, n % 16, :] = nan
    k2, v2 = O.append_tokens(before_k, before_v, bt, np.array(lens), k_new, v_new)
    np.testing.assert_array_equal(k2, kp)
    np.testing.assert_array_equal(v2, vp)
    assert (before_k[bt[0, 0], :, 0, :] == nan).all()  # inputs untouched
    got = O.decode(q, k2, v2, bt, np.array(full), dtype)
    np.testing.assert_allclose(got, sdpa_reference(q, kd, vd, full, dtype), rtol=1e-12,
                               atol=1e-14)


def test_append_skips_rows_whose_page_is_outside_the_pool():
    k = np.zeros((4, 1, 16, 8), np.uint16)
    v = np.zeros_like(k)
    bt = np.array([[2], [9], [-1]], np.int32)
    kn = np.full((3, 1, 8), 7, np.uint16)
    k2, v2 = O.append_tokens(k, v, bt, np.array([5, 5, 5]), kn, kn)
    assert (k2[2, 0, 5] == 7).all() and (v2[2, 0, 5] == 7).all()
    assert int((k2 != 0).sum()) == 8  # rows 1 and 2 wrote nothing
