"""The seeded input generators (CPU): length distributions of the named
workloads and trace families, pool layout, and determinism."""

import math

import numpy as np
import pytest

import workloads as W


def draw(lengths, n, seed=0):
    return W.draw_lengths(lengths, n, np.random.default_rng(seed))


def test_fixed_uniform_loguniform_bounds():
    assert (draw(("fixed", 77), 5) == 77).all()
    u = draw(("uniform", 10, 20), 20000)
    assert u.min() == 10 and u.max() == 20
    lu = draw(("loguniform", 256, 32768), 20000)
    assert lu.min() >= 256 and lu.max() <= 32768
    # log-uniform: the median sits at the geometric mean of the bounds
    assert abs(math.log(np.median(lu)) - 0.5 * (math.log(256) + math.log(32768))) < 0.05


def test_bucketed_takes_only_bucket_values_evenly():
    vals = (8192, 16384, 32768, 65536)
    x = draw(("bucketed",) + vals, 40000)
    assert set(np.unique(x).tolist()) == set(vals)
    frac = np.array([(x == v).mean() for v in vals])
    assert np.abs(frac - 0.25).max() < 0.01


def test_bimodal_two_bands_in_proportion():
    x = draw(("bimodal", 256, 1024, 16384, 32768, 0.5), 40000)
    short = (x >= 256) & (x <= 1024)
    long_ = (x >= 16384) & (x <= 32768)
    assert (short | long_).all()
    assert abs(short.mean() - 0.5) < 0.01


def test_zipf_probabilities_follow_the_power_law():
    unit, kmax, a = 256, 128, 1.1
    x = draw(("zipf", unit, kmax, a), 200000)
    assert (x % unit == 0).all() and x.min() >= unit and x.max() <= unit * kmax
    k = x // unit
    w = np.arange(1, kmax + 1, dtype=np.float64) ** -a
    pmf = w / w.sum()
    for kk in (1, 2, 3, 10):
        assert abs((k == kk).mean() - pmf[kk - 1]) < 4 * math.sqrt(pmf[kk - 1] / len(k)) + 1e-3


@pytest.mark.parametrize("name", ["bucketed1"] + list(W.TRACE_FAMILIES))
def test_trace_family_layouts_are_seeded_and_consistent(name):
    spec = W.CONFIGS[name]

    def layout(seed):
        rng = np.random.default_rng([seed, spec.config_id])
        lens = W.draw_lengths(spec.lengths, spec.batch, rng)
        bt, num_pages, _ = W._layout_pool(lens, rng, spec.pool_pages, 1, W.PAGE_TOKENS)
        return lens, bt, num_pages

    la, ba, na = layout(W.SEED_CALIBRATION)
    lb, bb, nb = layout(W.SEED_CALIBRATION)
    lc, _, _ = layout(W.SEED_HOLDOUT)
    np.testing.assert_array_equal(la, lb)
    np.testing.assert_array_equal(ba, bb)
    assert not np.array_equal(la, lc)
    # every used page appears exactly once in the block table
    used = np.concatenate([ba[i, :W.pages_for(n)] for i, n in enumerate(la)])
    assert len(np.unique(used)) == len(used) and used.max() < na


def test_make_case_is_deterministic():
    a = W.make_case("zipf8", W.SEED_HOLDOUT, poison=False)
    b = W.make_case("zipf8", W.SEED_HOLDOUT, poison=False)
    for f in ("seq_lens", "block_table", "q", "k_pool", "v_pool"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
