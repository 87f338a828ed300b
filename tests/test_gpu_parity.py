"""GPU parity: the HIP path (called through the C ABI) against the float64
CPU oracle on the same seeded inputs, plus bitwise invariants and the
partial states on their own."""

import math

import numpy as np
import pytest

import workloads as W
from oracle import paged_gqa as O
from tests.gpu_helpers import assert_parity, out_bits, run_case, shape_of

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_04_amd  # noqa: F401  (fails loudly if not built)


def _mini(lens, G=4, Hkv=2, d=128, dtype=W.BF16, seed=1, **kw):
    return W.make_case_from_lengths(
        "mini", lens, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=d,
        dtype=dtype, seed=seed, **kw)


# ------------------------------------------------------ named workloads


@pytest.mark.parametrize("mode", ["split", "auto", "workqueue", "unsplit"])
def test_tiny(mode):
    c = W.make_case("tiny")  # fp16, S = 4, 32 unreferenced NaN pages
    want = O.decode_case(c)
    got = run_case(c, mode=mode, num_splits=c.num_splits if mode == "split" else 0)
    assert_parity(got, want, f"tiny/{mode}")


@pytest.fixture(scope="module")
def long_case():
    c = W.make_case("long", poison=False)
    return c, W.case_to_device(c), O.decode_case(c)


@pytest.mark.parametrize("mode,S", [("split", 32), ("auto", 0), ("workqueue", 0),
                                    ("unsplit", 0), ("split", 7)])
def test_long(long_case, mode, S):
    c, dev, want = long_case
    got = run_case(c, dev, mode=mode, num_splits=S)
    assert_parity(got, want, f"long/{mode}/S={S}")


@pytest.fixture(scope="module")
def mixed_case():
    c = W.make_case("mixed8")
    return c, W.case_to_device(c), O.decode_case(c)


@pytest.mark.parametrize("mode,chunk", [("workqueue", 0), ("auto", 0), ("split", 0),
                                        ("unsplit", 0), ("workqueue", 5), ("workqueue", 64),
                                        ("bucketed", 0)])
def test_mixed8(mixed_case, mode, chunk):
    c, dev, want = mixed_case
    got = run_case(c, dev, mode=mode, chunk_pages=chunk)
    assert_parity(got, want, f"mixed8/{mode}/chunk={chunk}")


@pytest.mark.parametrize("seed", [20260622, 7, 12345])
@pytest.mark.parametrize("name", ["mixed8", "b4"])
def test_ragged_batches_other_seeds(name, seed):
    """The ragged workloads at full size on other draws of lengths, page
    placement and values, in the mode the policy picks."""
    c = W.make_case(name, seed)
    got = run_case(c)
    assert_parity(got, O.decode_case(c), f"{name}/seed={seed}")


@pytest.mark.parametrize("dtype", [W.BF16, W.F16])
@pytest.mark.parametrize("mode,S,chunk", [("split", 7, 0), ("workqueue", 0, 8), ("unsplit", 0, 0)])
def test_wide_logit_range_and_rising_maxima(dtype, mode, S, chunk):
    """Logits with a wide dynamic range whose maximum keeps rising along the
    sequence: a softmax scale 6x the default, and each key scaled by
    1 + 3 t / N (token t of N), so the running maximum of every range is
    raised again and again (each raise rescales the accumulator) and most
    weights underflow against the last tokens'. Checked against the
    float64 oracle at the usual bar."""
    lens = [3000, 700, 1, 160]
    c = _mini(lens, dtype=dtype, seed=41, poison=False)
    k = O.bits_to_f64(c.k_pool, dtype)
    for b, n in enumerate(lens):
        for t in range(n):
            k[c.block_table[b, t // 16], :, t % 16, :] *= 1.0 + 3.0 * t / n
    c.k_pool = W.to_bits(k.astype(np.float32), dtype)
    c.sm_scale = 6.0 / math.sqrt(c.head_dim)
    got = run_case(c, mode=mode, num_splits=S, chunk_pages=chunk)
    assert_parity(got, O.decode_case(c), f"wide range/{dtype}/{mode}")


@pytest.mark.parametrize("mode", ["unsplit", "split", "workqueue", "auto"])
def test_b4(mode):
    c = W.make_case("b4")
    got = run_case(c, mode=mode)
    assert_parity(got, O.decode_case(c), f"b4/{mode}")


_TRACE_CACHE = {}


def _trace_case(name):
    if name not in _TRACE_CACHE:
        c = W.make_case(name)  # hold-out seed; unowned pool pages poisoned
        _TRACE_CACHE.clear()  # keep one case (and its oracle) in memory
        _TRACE_CACHE[name] = (c, W.case_to_device(c), O.decode_case(c))
    return _TRACE_CACHE[name]


@pytest.mark.parametrize("mode", ["auto", "bucketed", "split"])
@pytest.mark.parametrize("name", ["bucketed1"] + list(W.TRACE_FAMILIES))
def test_trace_families(name, mode):
    """The Bucketed / Bimodal / Uniform / Zipf-like traces in the policy's
    choice, exact-length bucketing and the rectangular split grid."""
    c, dev, want = _trace_case(name)
    assert_parity(run_case(c, dev, mode=mode, merge="kernel" if mode == "bucketed" else "fused"),
                  want, f"{name}/{mode}")


@pytest.mark.slow
def test_b64_full_size():
    """The largest workload at full size (64 sequences, G = 8, about 2.3M
    tokens), in the work-queue launch the bench times, checked element by
    element on every row and head: the rows go to the host four at a time
    (their pages only), so host memory stays bounded."""
    import paged_kv_gqa_04_amd as P
    dev = W.make_device_case("b64")
    spec = dev["spec"]
    shape = P.make_shape(spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                         dev["block_table_host"].shape[1], dev["num_pages"], spec.dtype)
    out = torch.full_like(dev["q"], float("nan"))
    with P.Plan(shape, dev["seq_lens_host"], P.make_opts("workqueue")) as plan:
        plan.upload()
        plan.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                    dev["seq_lens"], out)
        torch.cuda.synchronize()
    got = out.to(torch.float64).cpu().numpy()
    assert np.isfinite(got).all()
    for r0 in range(0, spec.batch, 4):
        rows = list(range(r0, min(spec.batch, r0 + 4)))
        sub = W.host_subcase_from_device(dev, rows)
        assert_parity(got[rows], O.decode_case(sub), f"b64 rows {rows[0]}..{rows[-1]}")
        del sub


# ----------------------------------------------------------- split counts


@pytest.mark.parametrize("dtype", [W.BF16, W.F16])
@pytest.mark.parametrize("mode,S,chunk", [("auto", 0, 0), ("split", 16, 0), ("workqueue", 0, 32),
                                          ("unsplit", 0, 0)])
def test_g8_d64_mid_size(dtype, mode, S, chunk):
    """The G=8, d=64 kernel on rows of thousands of tokens (many pages per
    wave, several table chunks per unsplit row, tens of ranges per row to
    merge), with NaN-poisoned unused pool pages and row tails."""
    c = _mini([12000, 8000, 3000, 517, 1], G=8, Hkv=4, d=64, dtype=dtype, seed=88)
    got = run_case(c, mode=mode, num_splits=S, chunk_pages=chunk)
    assert_parity(got, O.decode_case(c), f"G8/d64/{dtype}/{mode}")


@pytest.mark.parametrize("G,Hkv,d,dtype", [(1, 8, 128, W.F16), (2, 4, 64, W.BF16),
                                           (4, 8, 128, W.F16), (8, 8, 128, W.F16)])
@pytest.mark.parametrize("mode", ["auto", "split"])
def test_other_shapes_mid_size(G, Hkv, d, dtype, mode):
    """Every other built (G, d) and the fp16 caches on rows of thousands of
    tokens, in the policy's mode and on the split grid."""
    c = _mini([16384, 5000, 777, 33], G=G, Hkv=Hkv, d=d, dtype=dtype, seed=G * 10 + d)
    got = run_case(c, mode=mode, num_splits=8 if mode == "split" else 0)
    assert_parity(got, O.decode_case(c), f"G{G}/Hkv{Hkv}/d{d}/{dtype}/{mode}")


@pytest.fixture(scope="module")
def longest_row_case():
    c = W.make_case_from_lengths("longest_row", [262144, 100], num_q_heads=32, num_kv_heads=8,
                                 head_dim=128, dtype=W.BF16, seed=3, poison=False)
    return c, W.case_to_device(c), O.decode_case(c)


@pytest.mark.parametrize("mode,S", [("auto", 0), ("unsplit", 0), ("split", 32)])
def test_longest_row(longest_row_case, mode, S):
    """A row of 262,144 tokens (16,384 pages: twice the longest row of the
    batch-of-64 workload) beside a short one: unsplit, each of its
    workgroups walks 32 staged block-table chunks; in the work queue and
    the split grid, 32 ranges per (row, KV head) are merged."""
    c, dev, want = longest_row_case
    got = run_case(c, dev, mode=mode, num_splits=S)
    assert_parity(got, want, f"longest row/{mode}/S={S}")


@pytest.mark.parametrize("S", [1, 2, 4, 7, 32, 200])
def test_split_counts(S):
    c = _mini([2000, 300, 16, 1, 4097], seed=S)
    got = run_case(c, mode="split", num_splits=S)
    assert_parity(got, O.decode_case(c), f"S={S}")


def test_split_count_changes_only_rounding():
    c = _mini([3000, 1234], seed=5)
    outs = [run_case(c, mode="split", num_splits=S) for S in (1, 3, 16)]
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 2 * 2.0 ** -8 * np.abs(outs[0]).max()


# ------------------------------------------------------------ edge cases


@pytest.mark.parametrize("dtype", [W.BF16, W.F16])
@pytest.mark.parametrize("G,Hkv,d", [(1, 4, 128), (2, 2, 64), (4, 1, 64), (8, 2, 128), (8, 1, 64),
                                     (4, 3, 128), (1, 1, 64)])
@pytest.mark.parametrize("mode", ["unsplit", "split", "workqueue", "bucketed"])
def test_shapes_and_ragged_tails(dtype, G, Hkv, d, mode):
    lens = [0, 1, 15, 16, 17, 33, 255, 1000]
    c = _mini(lens, G=G, Hkv=Hkv, d=d, dtype=dtype, seed=G * 100 + Hkv * 10 + d)
    got = run_case(c, mode=mode, num_splits=3 if mode == "split" else 0,
                   chunk_pages=2 if mode in ("workqueue", "bucketed") else 0)
    want = O.decode_case(c)
    assert_parity(got, want, f"{dtype}/G{G}/Hkv{Hkv}/d{d}/{mode}")
    assert (got[0] == 0).all()  # empty row -> zeros


def _random_cases(n, seed=20260705):
    """Seeded random small cases across every built shape: batch 1..6,
    lengths drawn from edge values (0, 1, page boundaries) and uniform
    ones, G in {1, 2, 4, 8}, d in {64, 128}, both dtypes, every mode and
    both merge paths, with chunk / split counts that force several ranges
    per row."""
    rng = np.random.default_rng(seed)
    edge = [0, 1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129]
    out = []
    for i in range(n):
        B = int(rng.integers(1, 7))
        lens = [int(rng.choice(edge)) if rng.random() < 0.5 else int(rng.integers(1, 1500))
                for _ in range(B)]
        G = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.integers(1, 4))
        d = int(rng.choice([64, 128]))
        dtype = W.BF16 if rng.random() < 0.5 else W.F16
        mode = str(rng.choice(["unsplit", "split", "workqueue", "bucketed", "auto"]))
        merge = "kernel" if (mode == "bucketed" or rng.random() < 0.3) else "fused"
        splits = int(rng.integers(1, 9)) if mode == "split" else 0
        chunk = int(rng.integers(1, 13)) if mode in ("workqueue", "bucketed") else 0
        out.append(dict(lens=lens, G=G, Hkv=Hkv, d=d, dtype=dtype, mode=mode, merge=merge,
                        splits=splits, chunk=chunk, seed=int(rng.integers(1, 1 << 30))))
    return out


@pytest.mark.parametrize("k", range(40))
def test_random_small_cases(k):
    c = _random_cases(40)[k]
    case = _mini(c["lens"], G=c["G"], Hkv=c["Hkv"], d=c["d"], dtype=c["dtype"], seed=c["seed"])
    got = run_case(case, mode=c["mode"], num_splits=c["splits"], chunk_pages=c["chunk"],
                   merge=c["merge"])
    assert_parity(got, O.decode_case(case), str(c))
    empty = [b for b, n in enumerate(c["lens"]) if n == 0]
    assert all((got[b] == 0).all() for b in empty)


@pytest.mark.parametrize("mode", ["unsplit", "split", "workqueue", "auto"])
def test_all_rows_empty(mode):
    c = _mini([0, 0, 0])
    got = run_case(c, mode=mode, num_splits=4 if mode == "split" else 0)
    assert (got == 0).all()


def test_zero_batch_is_a_noop():
    import paged_kv_gqa_04_amd as P
    shape = P.make_shape(0, 8, 2, 128, 1, 1, "bf16")
    with P.Plan(shape, np.zeros(0, np.int32)) as plan:
        plan.upload()
        plan.decode(0, 0, 0, 0, 0, 0)
        torch.cuda.synchronize()


def test_single_token_rows_return_v0():
    c = _mini([1, 1], G=4, Hkv=2, d=64)
    got = run_case(c, mode="unsplit")
    for b in range(2):
        for h in range(8):
            v0 = O.bits_to_f64(c.v_pool[c.block_table[b, 0], h // 4, 0], c.dtype)
            np.testing.assert_array_equal(got[b, h], v0)  # exact: weight 1, bf16 in/out


def test_shared_pages_between_rows():
    c = _mini([64, 64, 40])
    c.block_table[1, :4] = c.block_table[0, :4]  # rows 0 and 1 share their pages
    c.q[1] = c.q[0]  # ... and their query, so their outputs must be identical
    c.block_table[2, :3] = c.block_table[0, [3, 0, 2]]
    got = run_case(c, mode="workqueue", chunk_pages=2)
    want = O.decode_case(c)
    assert_parity(got, want, "shared pages")
    np.testing.assert_array_equal(got[0], got[1])


def test_out_of_range_table_entries_contribute_nothing():
    c = _mini([48, 48], G=4, Hkv=2, d=64, poison=False)
    good = run_case(c, mode="unsplit")
    c.block_table[1, :] = c.num_pages + 5  # whole row points outside the pool
    got = run_case(c, mode="unsplit")
    np.testing.assert_array_equal(got[0], good[0])
    assert (got[1] == 0).all()


# ----------------------------------------------------- bitwise invariants


def _permute_pages(c, seed):
    """Same logical cache, pages moved to other physical slots."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(c.num_pages)  # old page p -> new slot perm[p]
    k = np.empty_like(c.k_pool)
    v = np.empty_like(c.v_pool)
    k[perm] = c.k_pool
    v[perm] = c.v_pool
    c2 = W.Case(**{**c.__dict__})
    c2.k_pool, c2.v_pool = k, v
    c2.block_table = perm[c.block_table].astype(np.int32)
    return c2


@pytest.mark.parametrize("mode", ["unsplit", "split", "workqueue"])
def test_page_permutation_bitwise(mode):
    c = _mini([700, 33, 4096, 5], seed=9)
    kw = dict(mode=mode, num_splits=5 if mode == "split" else 0)
    a, pa, oa = run_case(c, return_plan=True, **kw)
    b, pb, ob = run_case(_permute_pages(c, 1), return_plan=True, **kw)
    np.testing.assert_array_equal(out_bits(oa), out_bits(ob))
    pa.close()
    pb.close()


def test_queue_order_bitwise():
    c = _mini([700, 33, 4096, 5, 1500], seed=10)
    ref = None
    for seed in [0, 1, 2, 12345]:
        _, plan, o = run_case(c, mode="workqueue", chunk_pages=4, queue_seed=seed,
                              return_plan=True)
        bits = out_bits(o)
        plan.close()
        if ref is None:
            ref = bits
        np.testing.assert_array_equal(bits, ref)


def test_repeated_runs_bitwise():
    c = W.make_case("mixed8", seed=W.SEED_CALIBRATION)
    dev = W.case_to_device(c)
    ref = None
    for _ in range(5):
        _, plan, o = run_case(c, dev, mode="workqueue", return_plan=True)
        bits = out_bits(o)
        plan.close()
        if ref is None:
            ref = bits
        np.testing.assert_array_equal(bits, ref)


# ------------------------------------------------------ merge placement


@pytest.mark.parametrize("mode", ["split", "workqueue", "bucketed"])
def test_fused_and_kernel_merge_give_identical_bits(mode):
    c = _mini([3000, 17, 0, 900, 4100], seed=12)
    kw = dict(mode=mode, num_splits=6 if mode == "split" else 0,
              chunk_pages=5 if mode == "workqueue" else 0, return_plan=True)
    _, pf, of = run_case(c, merge="fused", **kw)
    _, pk, ok = run_case(c, merge="kernel", **kw)
    if mode != "bucketed":
        assert pf.stats()["launches"] == 1 and pk.stats()["launches"] == 2
    else:  # 4 distinct lengths and an empty row: 5 buckets
        assert pf.stats()["launches"] == 5 and pk.stats()["launches"] == 10
    np.testing.assert_array_equal(out_bits(of), out_bits(ok))
    assert_parity(of.to(torch.float64).cpu().numpy(), O.decode_case(c), f"fused/{mode}")
    pf.close()
    pk.close()


@pytest.mark.parametrize("mode", ["split", "workqueue"])
def test_fused_counters_reset_between_steps(mode):
    """One upload, several decodes: each step's last workgroup resets the
    per-row arrival counters, so later steps merge exactly as the first."""
    c = _mini([2000, 33, 700], seed=13)
    dev = W.case_to_device(c)
    _, plan, out = run_case(c, dev, mode=mode, num_splits=4 if mode == "split" else 0,
                            return_plan=True)
    first = out_bits(out)
    for _ in range(4):
        out.fill_(float("nan"))
        plan.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                    dev["seq_lens"], out)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out_bits(out), first)
    lay = plan.layout()
    rows = c.batch * c.num_kv_heads
    import paged_kv_gqa_04_amd as P
    cnt = plan.workspace[lay["counters_offset"]:lay["counters_offset"] + P.COUNTER_STRIDE * rows]
    assert (cnt.cpu().numpy().view(np.int32) == 0).all()
    plan.close()


@pytest.mark.parametrize("mode", ["split", "workqueue"])
def test_consecutive_steps_with_new_inputs(mode):
    """One plan and workspace, steps alternating between two different input
    sets of the same lengths: every step's merge must read the states of
    that step (written by workgroups on other XCDs), never an earlier one."""
    lens = [20000, 5000, 12000, 1]
    cases = [_mini(lens, seed=s) for s in (21, 22)]
    devs = [W.case_to_device(c) for c in cases]
    wants = [O.decode_case(c) for c in cases]
    kw = dict(mode=mode, num_splits=48 if mode == "split" else 0,
              chunk_pages=8 if mode == "workqueue" else 0)
    _, plan, out = run_case(cases[0], devs[0], return_plan=True, **kw)
    assert plan.stats()["grid"] >= 256
    assert_parity(out.to(torch.float64).cpu().numpy(), wants[0], f"{mode} step 0")
    first = [out_bits(out), None]
    for step in range(1, 7):
        i = step % 2
        d = devs[i]
        out.fill_(float("nan"))
        plan.decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"], out)
        torch.cuda.synchronize()
        got = out_bits(out)
        if first[i] is None:
            assert_parity(out.to(torch.float64).cpu().numpy(), wants[i], f"{mode} step {step}")
            first[i] = got
        np.testing.assert_array_equal(got, first[i])
    plan.close()


# --------------------------------------------- partial states on their own


@pytest.mark.parametrize("mode", ["workqueue", "split"])
def test_partial_states_match_oracle(mode):
    c = _mini([1000, 77, 300], G=4, Hkv=2, d=128, seed=4)
    _, plan, out = run_case(c, mode=mode, num_splits=4 if mode == "split" else 0,
                            chunk_pages=8 if mode == "workqueue" else 0, return_plan=True)
    lay = plan.layout()
    ws = plan.workspace.cpu().numpy()
    G, d = c.group, c.head_dim
    S = lay["num_splits"]
    f32 = lambda off, n: ws[off:off + 4 * n].view(np.float32)
    m2 = f32(lay["m_offset"], lay["num_slots"] * G).reshape(-1, G)
    ls = f32(lay["l_offset"], lay["num_slots"] * G).reshape(-1, G)
    acc = f32(lay["acc_offset"], lay["num_slots"] * G * d).reshape(-1, G, d)
    meta = ws[lay["meta_offset"]:lay["meta_offset"] + 8 * c.batch].view(np.int32).reshape(-1, 2)
    checked = 0
    for b, n in enumerate(c.seq_lens):
        pages = (n + 15) // 16
        if mode == "workqueue":
            base, Sb = meta[b]
            chunk = plan.stats()["chunk_pages"]
        else:
            Sb, chunk = S, max(1, math.ceil(pages / S))
        for g in range(c.num_kv_heads):
            for s in range(Sb):
                slot = (base + g * Sb + s) if mode == "workqueue" else ((b * c.num_kv_heads + g) * S + s)
                t0, t1 = s * chunk * 16, min(n, (s + 1) * chunk * 16)
                mo, lo, ao = O.range_state(c.q, c.k_pool, c.v_pool, c.block_table, c.seq_lens,
                                           c.dtype, b, g, t0, t1, c.sm_scale)
                if t1 <= t0:
                    assert (m2[slot] == -np.inf).all() and (ls[slot] == 0).all()
                    assert (acc[slot] == 0).all()
                    continue
                mg = m2[slot].astype(np.float64) * math.log(2)
                # the reference may sit below the range maximum by < 8 log2 units
                assert (mo - mg >= -1e-4).all() and (mo - mg <= 8 * math.log(2) + 1e-4).all()
                f = np.exp(mg - mo)
                np.testing.assert_allclose(ls[slot] * f, lo, rtol=1e-4)
                np.testing.assert_allclose(acc[slot] * f[:, None], ao, rtol=1e-3,
                                           atol=1e-4 * np.abs(ao).max())
                checked += 1
    assert checked > 0
    plan.close()


# ------------------------------------------------------- ABI error paths


def test_abi_errors_on_device():
    import paged_kv_gqa_04_amd as P
    c = _mini([100, 50])
    dev = W.case_to_device(c)
    out = torch.empty_like(dev["q"])
    plan = P.Plan(shape_of(c), c.seq_lens, P.make_opts("workqueue", chunk_pages=2))
    args = (dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"], dev["seq_lens"], out)
    with pytest.raises(P.PkvError) as e:
        plan.decode(*args)  # not uploaded yet
    assert e.value.status == P.PKV_ERR_STATE
    nb = plan.workspace_bytes()
    ws = torch.empty(nb + 512, dtype=torch.uint8, device="cuda")
    with pytest.raises(P.PkvError) as e:
        P.pkv_plan_upload(plan.handle, ws, nb - 1, torch.cuda.current_stream().cuda_stream)
    assert e.value.status == P.PKV_ERR_WORKSPACE
    with pytest.raises(P.PkvError) as e:
        P.pkv_plan_upload(plan.handle, ws.data_ptr() + 4, nb, 0)
    assert e.value.status == P.PKV_ERR_WORKSPACE
    plan.upload()
    with pytest.raises(P.PkvError) as e:
        P.pkv_decode(plan.handle, dev["q"].data_ptr() + 2, *[a for a in args[1:]])
    assert e.value.status == P.PKV_ERR_INVALID
    plan.decode(*args)
    torch.cuda.synchronize()
    assert_parity(out.to(torch.float64).cpu().numpy(), O.decode_case(c), "after errors")
    plan.close()
