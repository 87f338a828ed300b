"""GPU tests of the paged KV append step through the C ABI: the device
writes match the oracle bit for bit, and append + decode over many steps
(pages taken as rows grow, a finished row's pages reused) matches the
oracle's append + decode."""

import numpy as np
import pytest

import workloads as W
from oracle import paged_gqa as O
from tests.gpu_helpers import assert_parity, run_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_04_amd  # noqa: F401  (fails loudly if not built)


def _case(lens, G=4, Hkv=2, d=128, dtype=W.BF16, seed=1, extra=24):
    c = W.make_case_from_lengths("append", lens, num_q_heads=G * Hkv, num_kv_heads=Hkv,
                                 head_dim=d, dtype=dtype, seed=seed, extra_pages=extra)
    # room in every row for the steps below
    stride = c.block_table.shape[1] + 8
    bt = np.full((c.batch, stride), -1, np.int32)
    bt[:, :c.block_table.shape[1]] = c.block_table
    c.block_table = bt
    return c


def _pool_for(case):
    """An allocator whose free pages are the pool pages no row uses."""
    import paged_kv_gqa_04_amd as P
    pool = P.Pool(case.num_pages)
    pool.alloc(case.num_pages)
    used = set()
    for b, n in enumerate(case.seq_lens):
        used.update(int(x) for x in case.block_table[b, :W.pages_for(n)])
    pool.free(np.array(sorted(set(range(case.num_pages)) - used), np.int32))
    return pool


def _new_token_bits(rng, case):
    x = rng.standard_normal((case.batch, case.num_kv_heads, case.head_dim), dtype=np.float32)
    return W.to_bits(x, case.dtype)


def _shape(case):
    import paged_kv_gqa_04_amd as P
    return P.make_shape(case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim,
                        case.block_table.shape[1], case.num_pages, case.dtype, case.sm_scale)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("d,dtype", [(128, W.BF16), (64, W.F16)])
def test_append_writes_match_the_oracle_bitwise(d, dtype):
    import paged_kv_gqa_04_amd as P
    c = _case([0, 1, 15, 16, 17, 31, 32, 100], d=d, dtype=dtype)
    rng = np.random.default_rng(3)
    with _pool_for(c) as pool:
        assert pool.prepare(c.seq_lens, c.block_table) == 3  # positions 0, 16 and 32
    c.block_table[5, 1] = c.num_pages + 3  # a bad entry: row 5 writes nothing
    kn, vn = _new_token_bits(rng, c), _new_token_bits(rng, c)
    want_k, want_v = O.append_tokens(c.k_pool, c.v_pool, c.block_table, c.seq_lens, kn, vn)
    kp, vp = _dev(c.k_pool.view(np.int16)), _dev(c.v_pool.view(np.int16))
    lens_d = _dev(c.seq_lens)
    new_lens = torch.full_like(lens_d, -7)
    P.pkv_append(_shape(c), _dev(kn.view(np.int16)), _dev(vn.view(np.int16)), kp, vp,
                 _dev(c.block_table), lens_d, new_lens)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(kp.cpu().numpy().view(np.uint16), want_k)
    np.testing.assert_array_equal(vp.cpu().numpy().view(np.uint16), want_v)
    np.testing.assert_array_equal(new_lens.cpu().numpy(), c.seq_lens + 1)


def test_append_then_decode_over_many_steps():
    """24 steps of host prepare, device append, device decode; row 2 ends at
    step 10 and a new row takes its place (its pages go back to the pool and
    are reused). Every step's output matches the oracle's append + decode."""
    import paged_kv_gqa_04_amd as P
    c = _case([30, 15, 47, 1], extra=12, seed=4)
    rng = np.random.default_rng(5)
    host_k, host_v = c.k_pool.copy(), c.v_pool.copy()
    kp, vp = _dev(c.k_pool.view(np.int16)), _dev(c.v_pool.view(np.int16))
    lens = c.seq_lens.copy()
    with _pool_for(c) as pool:
        for step in range(24):
            if step == 10:  # row 2 finishes; a new sequence starts in its slot
                row = np.ascontiguousarray(c.block_table[2])
                pool.release_row(row, int(lens[2]))
                c.block_table[2] = row
                lens[2] = 0
            pool.prepare(lens, c.block_table)
            kn, vn = _new_token_bits(rng, c), _new_token_bits(rng, c)
            host_k, host_v = O.append_tokens(host_k, host_v, c.block_table, lens, kn, vn)
            bt_d, lens_d = _dev(c.block_table), _dev(lens)
            new_lens = torch.empty_like(lens_d)
            P.pkv_append(_shape(c), _dev(kn.view(np.int16)), _dev(vn.view(np.int16)), kp, vp,
                         bt_d, lens_d, new_lens)
            lens = lens + 1
            np.testing.assert_array_equal(new_lens.cpu().numpy(), lens)
            q = W.to_bits(rng.standard_normal((c.batch, c.num_q_heads, c.head_dim),
                                              dtype=np.float32), c.dtype)
            c2 = W.Case(**{**c.__dict__})
            c2.seq_lens, c2.q, c2.k_pool, c2.v_pool = lens.copy(), q, host_k, host_v
            td = W.torch_dtype(c.dtype)
            dev = dict(q=_dev(q.view(np.int16)).view(td), k_pool=kp.view(td), v_pool=vp.view(td),
                       block_table=bt_d, seq_lens=new_lens)
            got = run_case(c2, dev, mode="auto")
            assert_parity(got, O.decode_case(c2), f"step {step}")
        np.testing.assert_array_equal(kp.cpu().numpy().view(np.uint16), host_k)


def test_append_argument_errors():
    import paged_kv_gqa_04_amd as P
    c = _case([5, 6])
    x = _dev(np.zeros((2, 2, 128), np.int16))
    lens = _dev(c.seq_lens)
    kp = _dev(c.k_pool.view(np.int16))
    bt = _dev(c.block_table)
    with pytest.raises(P.PkvError) as e:
        P.pkv_append(_shape(c), x, x, kp, kp, bt, lens, lens)  # aliasing lengths
    assert e.value.status == P.PKV_ERR_INVALID
    with pytest.raises(P.PkvError) as e:
        P.pkv_append(_shape(c), 0, x, kp, kp, bt, lens)
    assert e.value.status == P.PKV_ERR_INVALID
    bad = P.make_shape(2, 8, 2, 96, c.block_table.shape[1], c.num_pages, c.dtype)
    with pytest.raises(P.PkvError) as e:
        P.pkv_append(bad, x, x, kp, kp, bt, lens)
    assert e.value.status == P.PKV_ERR_UNSUPPORTED
    P.pkv_append(P.make_shape(0, 8, 2, 128, 1, 1, c.dtype), 0, 0, 0, 0, 0, 0)  # B = 0: no-op


# ------------------------------------------ append folded into the decode


def _plan_for(case, lens, mode, S=0, chunk=0):
    import paged_kv_gqa_04_amd as P
    plan = P.Plan(_shape(case), lens, P.make_opts(mode, S, chunk))
    plan.upload()
    return plan


@pytest.mark.parametrize("mode,S,chunk", [("auto", 0, 0), ("split", 3, 0), ("workqueue", 0, 2),
                                          ("unsplit", 0, 0), ("bucketed", 0, 0)])
@pytest.mark.parametrize("d,dtype", [(128, W.BF16), (64, W.F16)])
def test_decode_append_equals_append_then_decode(mode, S, chunk, d, dtype):
    """One launch (pkv_decode_append) against two (pkv_append, then
    pkv_decode with the same plan): outputs, pools and new lengths equal bit
    for bit, and the output matches the oracle's append + decode. Rows cover
    a token opening a page, filling one, mid-page, an empty row and a bad
    table entry for the new token's page."""
    import paged_kv_gqa_04_amd as P
    c = _case([0, 1, 15, 16, 17, 31, 32, 100, 700], d=d, dtype=dtype, seed=7)
    rng = np.random.default_rng(8)
    with _pool_for(c) as pool:
        pool.prepare(c.seq_lens, c.block_table)
    c.block_table[6, 2] = c.num_pages + 5  # row 6 (32 tokens) opens page 2: a bad entry
    kn, vn = _new_token_bits(rng, c), _new_token_bits(rng, c)
    td = W.torch_dtype(c.dtype)
    q = _dev(c.q.view(np.int16)).view(td)
    bt, lens_d = _dev(c.block_table), _dev(c.seq_lens)
    kn_d, vn_d = _dev(kn.view(np.int16)).view(td), _dev(vn.view(np.int16)).view(td)
    new_lens = c.seq_lens + 1
    plan = _plan_for(c, new_lens, mode, S, chunk)
    # two launches
    kp2, vp2 = _dev(c.k_pool.view(np.int16)), _dev(c.v_pool.view(np.int16))
    nl2 = torch.full_like(lens_d, -1)
    P.pkv_append(_shape(c), kn_d, vn_d, kp2, vp2, bt, lens_d, nl2)
    out2 = torch.full_like(q, float("nan"))
    plan.decode(q, kp2.view(td), vp2.view(td), bt, nl2, out2)
    # one launch
    kp1, vp1 = _dev(c.k_pool.view(np.int16)), _dev(c.v_pool.view(np.int16))
    nl1 = torch.full_like(lens_d, -1)
    out1 = torch.full_like(q, float("nan"))
    plan.decode_append(q, kn_d, vn_d, kp1.view(td), vp1.view(td), bt, lens_d, out1, nl1)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(nl1.cpu().numpy(), new_lens)
    np.testing.assert_array_equal(nl2.cpu().numpy(), new_lens)
    np.testing.assert_array_equal(out1.view(torch.int16).cpu().numpy(),
                                  out2.view(torch.int16).cpu().numpy())
    np.testing.assert_array_equal(kp1.cpu().numpy(), kp2.cpu().numpy())
    np.testing.assert_array_equal(vp1.cpu().numpy(), vp2.cpu().numpy())
    want_k, want_v = O.append_tokens(c.k_pool, c.v_pool, c.block_table, c.seq_lens, kn, vn)
    np.testing.assert_array_equal(kp1.cpu().numpy().view(np.uint16), want_k)
    c2 = W.Case(**{**c.__dict__})
    c2.seq_lens, c2.k_pool, c2.v_pool = new_lens.copy(), want_k, want_v
    c2.seq_lens[6] -= 1  # its new token's page is outside the pool: it contributes nothing
    assert_parity(out1.to(torch.float64).cpu().numpy(), O.decode_case(c2), f"fused {mode}")
    plan.close()


def test_decode_append_over_many_steps():
    """The 24-step loop of the test above with the append folded into the
    decode launch, the device lengths carried from step to step by the
    kernel itself (new_seq_lens), row 2 replaced at step 10."""
    import paged_kv_gqa_04_amd as P
    c = _case([30, 15, 47, 1], extra=12, seed=4)
    rng = np.random.default_rng(5)
    host_k, host_v = c.k_pool.copy(), c.v_pool.copy()
    td = W.torch_dtype(c.dtype)
    kp, vp = _dev(c.k_pool.view(np.int16)), _dev(c.v_pool.view(np.int16))
    lens = c.seq_lens.copy()
    lens_d = _dev(lens)
    with _pool_for(c) as pool:
        for step in range(24):
            if step == 10:
                row = np.ascontiguousarray(c.block_table[2])
                pool.release_row(row, int(lens[2]))
                c.block_table[2] = row
                lens[2] = 0
                lens_d = _dev(lens)
            pool.prepare(lens, c.block_table)
            kn, vn = _new_token_bits(rng, c), _new_token_bits(rng, c)
            host_k, host_v = O.append_tokens(host_k, host_v, c.block_table, lens, kn, vn)
            q = W.to_bits(rng.standard_normal((c.batch, c.num_q_heads, c.head_dim),
                                              dtype=np.float32), c.dtype)
            plan = _plan_for(c, lens + 1, "auto")
            out = torch.full((c.batch, c.num_q_heads, c.head_dim), float("nan"), dtype=td,
                             device="cuda")
            new_lens = torch.empty_like(lens_d)
            plan.decode_append(_dev(q.view(np.int16)).view(td), _dev(kn.view(np.int16)).view(td),
                               _dev(vn.view(np.int16)).view(td), kp.view(td), vp.view(td),
                               _dev(c.block_table), lens_d, out, new_lens)
            torch.cuda.synchronize()
            plan.close()
            lens = lens + 1
            np.testing.assert_array_equal(new_lens.cpu().numpy(), lens)
            lens_d = new_lens
            c2 = W.Case(**{**c.__dict__})
            c2.seq_lens, c2.q, c2.k_pool, c2.v_pool = lens.copy(), q, host_k, host_v
            assert_parity(out.to(torch.float64).cpu().numpy(), O.decode_case(c2), f"step {step}")
        np.testing.assert_array_equal(kp.cpu().numpy().view(np.uint16), host_k)
        np.testing.assert_array_equal(vp.cpu().numpy().view(np.uint16), host_v)


def test_decode_append_argument_errors():
    import paged_kv_gqa_04_amd as P
    c = _case([5, 6])
    plan = _plan_for(c, c.seq_lens + 1, "auto")
    td = W.torch_dtype(c.dtype)
    x = _dev(np.zeros((2, 2, 128), np.int16)).view(td)
    q = _dev(c.q.view(np.int16)).view(td)
    kp = _dev(c.k_pool.view(np.int16)).view(td)
    bt, lens = _dev(c.block_table), _dev(c.seq_lens)
    out = torch.empty_like(q)
    for args in [(q, 0, x, kp, kp, bt, lens, out, None),      # v_new without k_new
                 (q, x, x, kp, kp, bt, lens, out, lens),      # aliasing lengths
                 (q, x[:, :, 1:], x, kp, kp, bt, lens, out, None)]:  # misaligned k_new
        with pytest.raises(P.PkvError) as e:
            P.pkv_decode_append(plan.handle, *args)
        assert e.value.status == P.PKV_ERR_INVALID
    plan.close()
