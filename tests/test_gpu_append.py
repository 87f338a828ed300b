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
