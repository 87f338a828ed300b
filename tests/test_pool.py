"""Host page allocator and the host half of the append step (CPU, through
the C ABI): pages are taken when a row's next token opens a page, returned
when a row ends, reused, and never handed out twice."""

import numpy as np
import pytest

P = pytest.importorskip("paged_kv_gqa_04_amd")


def test_alloc_order_free_reuse():
    with P.Pool(6) as pool:
        assert pool.free_pages() == 6
        np.testing.assert_array_equal(pool.alloc(3), [0, 1, 2])
        pool.free([1])
        np.testing.assert_array_equal(pool.alloc(2), [1, 3])  # freed page first
        assert pool.free_pages() == 2


def test_exhaustion_takes_nothing():
    with P.Pool(3) as pool:
        pool.alloc(2)
        with pytest.raises(P.PkvError) as e:
            pool.alloc(2)
        assert e.value.status == P.PKV_ERR_POOL
        assert pool.free_pages() == 1


@pytest.mark.parametrize("bad", [[7], [-1], [0, 0], [2]])
def test_bad_frees_are_rejected_whole(bad):
    with P.Pool(4) as pool:
        pool.alloc(2)  # pages 0, 1 taken; 2, 3 free
        with pytest.raises(P.PkvError) as e:
            pool.free([1] + bad)
        assert e.value.status == P.PKV_ERR_INVALID
        assert pool.free_pages() == 2  # page 1 was not returned either
        pool.free([1, 0])
        assert pool.free_pages() == 4


def test_prepare_takes_pages_only_at_page_boundaries():
    lens = np.array([0, 1, 15, 16, 17, 32, 47], np.int32)
    bt = np.full((len(lens), 4), -1, np.int32)
    with P.Pool(10) as pool:
        taken = pool.prepare(lens, bt)
        opens = [b for b, n in enumerate(lens) if n % 16 == 0]
        assert taken == len(opens) == 3 and pool.free_pages() == 7
        for b, n in enumerate(lens):
            row = bt[b]
            if b in opens:
                assert row[n // 16] >= 0
                assert (np.delete(row, n // 16) == -1).all()
            else:
                assert (row == -1).all()
        new = bt[bt >= 0]
        assert len(set(new.tolist())) == len(new)


def test_prepare_failures_leave_everything_unchanged():
    bt = np.full((3, 2), -1, np.int32)
    with P.Pool(1) as pool:
        with pytest.raises(P.PkvError) as e:  # two rows open a page, one page free
            pool.prepare(np.array([0, 16, 3], np.int32), bt)
        assert e.value.status == P.PKV_ERR_POOL
        assert (bt == -1).all() and pool.free_pages() == 1
        for lens in ([32, 0, 0], [-1, 0, 0]):  # past the row; negative
            with pytest.raises(P.PkvError) as e:
                pool.prepare(np.array(lens, np.int32), bt)
            assert e.value.status == P.PKV_ERR_INVALID
            assert (bt == -1).all() and pool.free_pages() == 1


def test_release_row_returns_pages_for_reuse():
    with P.Pool(4) as pool:
        bt = np.full((2, 4), -1, np.int32)
        lens = np.zeros(2, np.int32)
        for step in range(40):  # row 0 grows to 40 tokens, row 1 to 10
            grow = np.array([1, 1 if step < 10 else 0], np.int32)
            sub = np.ascontiguousarray(bt[grow == 1])
            pool.prepare(lens[grow == 1], sub)
            bt[grow == 1] = sub
            lens += grow
        assert pool.free_pages() == 0  # 3 pages + 1 page
        row1 = bt[1].copy()
        r = np.ascontiguousarray(bt[1])
        pool.release_row(r, 10)
        bt[1] = r
        assert (bt[1] == -1).all() and pool.free_pages() == 1
        with pytest.raises(P.PkvError):  # released already: rejected, nothing changes
            pool.release_row(row1.copy(), 10)
        assert pool.free_pages() == 1
        for _ in range(9):  # row 0 stores tokens 40..48: 48 opens a page, row 1's
            sub = np.ascontiguousarray(bt[:1])
            pool.prepare(lens[:1], sub)
            bt[:1] = sub
            lens[0] += 1
        assert bt[0, 3] == row1[0] and pool.free_pages() == 0


def test_simulated_serving_never_shares_a_page():
    """Random arrivals, one token per step per active row, random finishes:
    the live rows' pages are always distinct, and every page is either live
    or free (none leaks)."""
    rng = np.random.default_rng(0)
    B, stride, npages = 8, 16, 64
    with P.Pool(npages) as pool:
        bt = np.full((B, stride), -1, np.int32)
        lens = np.full(B, -1, np.int32)  # -1: slot empty
        for step in range(600):
            for b in range(B):
                if lens[b] < 0 and rng.uniform() < 0.3:
                    lens[b] = 0
            active = np.where(lens >= 0)[0]
            if len(active):
                sub_bt = bt[active].copy()
                try:
                    pool.prepare(lens[active], sub_bt)
                except P.PkvError as e:
                    assert e.value.status == P.PKV_ERR_POOL
                    sub_bt = None
                if sub_bt is not None:
                    bt[active] = sub_bt
                    lens[active] += 1
            for b in active:
                full = lens[b] >= stride * 16
                if full or rng.uniform() < 0.02:
                    row = np.ascontiguousarray(bt[b])
                    pool.release_row(row, int(lens[b]))
                    bt[b] = row
                    lens[b] = -1
            live = np.concatenate([bt[b, :(lens[b] + 15) // 16] for b in range(B) if lens[b] > 0]
                                  or [np.zeros(0, np.int32)])
            assert len(set(live.tolist())) == len(live)
            assert len(live) + pool.free_pages() == npages
