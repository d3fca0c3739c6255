"""Pins of the oracle's sampler (oracle/sampling.py) to things other than itself: numpy's
own Philox generator, closed-form filtered distributions worked out by hand, the greedy
limits, and a chi-square test of the draws against the exact distribution."""
import numpy as np
import pytest

from oracle import sampling as S

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _np_philox_block(counter, key):
    # numpy's Philox (4x64, 10 rounds) adds one to its 256-bit counter before generating a
    # block, so start it one below
    m = 1 << 64
    whole = sum(int(c) << (64 * i) for i, c in enumerate(counter))
    prev = (whole - 1) % (1 << 256)
    ctr = np.array([(prev >> (64 * i)) % m for i in range(4)], dtype=np.uint64)
    bg = np.random.Philox(counter=ctr, key=np.array(key, dtype=np.uint64))
    return [int(v) for v in bg.random_raw(4)]


@pytest.mark.parametrize("counter,key", [((0, 0, 0, 0), (0, 0)), ((1, 0, 0, 0), (0, 0)),
                                         ((7, 0, 0, 0), (12345, 0)),
                                         ((2**64 - 1, 3, 5, 7), (2**64 - 1, 2**63 + 11)),
                                         ((0, 0, 0, 0), (1, 0)), ((123456789, 0, 0, 0), (2**40 + 1, 0))])
def test_philox_matches_numpy(counter, key):
    assert S.philox4x64(counter, key) == _np_philox_block(counter, key)


def test_uniform_matches_numpy_random_and_is_in_range():
    for seed in (0, 1, 99, 2**63 + 5):
        for c in (1, 2, 50, 10**9):
            ctr = np.array([c - 1, 0, 0, 0], dtype=np.uint64)
            g = np.random.Generator(np.random.Philox(counter=ctr, key=np.array([seed, 0], dtype=np.uint64)))
            assert S.uniform(seed, c) == g.random()
    us = [S.uniform(3, c) for c in range(2000)]
    assert min(us) >= 0 and max(us) < 1
    assert S.uniform(3, 5) != S.uniform(4, 5)


Q = np.array([0.05, 0.4, 0.1, 0.3, 0.15])
LQ = np.log(Q)


def _probs(s):
    p, _ = S.filtered_probs(LQ, s)
    return p


def test_temperature_one_is_the_softmax_and_two_is_its_square_root():
    assert np.allclose(_probs(S.Sampler(temperature=1.0)), Q, rtol=1e-13)
    r = np.sqrt(Q)
    assert np.allclose(_probs(S.Sampler(temperature=2.0)), r / r.sum(), rtol=1e-13)
    r = Q ** 2
    assert np.allclose(_probs(S.Sampler(temperature=0.5)), r / r.sum(), rtol=1e-13)


def test_top_k_keeps_the_k_largest_renormalised():
    p = _probs(S.Sampler(temperature=1.0, top_k=2))
    assert np.allclose(p, [0, 0.4 / 0.7, 0, 0.3 / 0.7, 0], rtol=1e-13, atol=0)


def test_top_p_keeps_the_shortest_run_reaching_p():
    # 0.4 + 0.3 = 0.7 < 0.75 <= 0.85
    p = _probs(S.Sampler(temperature=1.0, top_p=0.75))
    assert np.allclose(p, [0, 0.4 / 0.85, 0, 0.3 / 0.85, 0.15 / 0.85], rtol=1e-13, atol=0)
    p = _probs(S.Sampler(temperature=1.0, top_p=0.65))
    assert np.allclose(p, [0, 0.4 / 0.7, 0, 0.3 / 0.7, 0], rtol=1e-13, atol=0)


def test_filters_apply_in_order_each_on_the_renormalised_distribution():
    # top-k 3 leaves 0.4, 0.3, 0.15 (/0.85): 0.47, 0.35, 0.18; top-p 0.8 then stops after two
    p = _probs(S.Sampler(temperature=1.0, top_k=3, top_p=0.8))
    assert np.allclose(p, [0, 4 / 7, 0, 3 / 7, 0], rtol=1e-13, atol=0)
    # top-p 0.75 leaves 0.47, 0.35, 0.176; min-p 0.16 compares against those, keeping all three
    p = _probs(S.Sampler(temperature=1.0, top_p=0.75, min_p=0.16))
    assert np.allclose(p, [0, 0.4 / 0.85, 0, 0.3 / 0.85, 0.15 / 0.85], rtol=1e-13, atol=0)
    p = _probs(S.Sampler(temperature=1.0, top_p=0.75, min_p=0.2))
    assert np.allclose(p, [0, 4 / 7, 0, 3 / 7, 0], rtol=1e-13, atol=0)
    p = _probs(S.Sampler(temperature=1.0, min_p=0.12))
    assert np.allclose(p, [0, 0.4 / 0.85, 0, 0.3 / 0.85, 0.15 / 0.85], rtol=1e-13, atol=0)


def test_equal_logits_order_by_index():
    l = np.array([1.0, 3.0, 2.0, 3.0, 2.0, 3.0])
    p, _ = S.filtered_probs(l, S.Sampler(temperature=1.0, top_k=2))
    assert list(np.flatnonzero(p)) == [1, 3]
    p, _ = S.filtered_probs(l, S.Sampler(temperature=1.0, top_k=4))
    assert list(np.flatnonzero(p)) == [1, 2, 3, 5]
    assert S.greedy(l) == 1
    assert S.sample(l, S.Sampler(), 0).token == 1


def test_greedy_limits():
    rng = np.random.default_rng(0)
    l = rng.standard_normal(300) * 3
    top = int(np.argmax(l))
    for c in range(200):
        assert S.sample(l, S.Sampler(temperature=0.0, seed=1), c).token == top
        assert S.sample(l, S.Sampler(temperature=1.5, top_k=1, seed=c), c).token == top
        assert S.sample(l, S.Sampler(temperature=1.5, top_p=1e-9, seed=c), c).token == top
        assert S.sample(l, S.Sampler(temperature=1.5, min_p=1.0, seed=c), c).token == top
    # temperature towards 0: the distribution collapses onto the largest logit
    gap = np.sort(l)[-1] - np.sort(l)[-2]
    t = gap / 40.0
    assert all(S.sample(l, S.Sampler(temperature=t, seed=9), c).token == top for c in range(300))


def test_draw_is_the_inverse_cdf_at_u():
    rng = np.random.default_rng(1)
    l = rng.standard_normal(50)
    for c in range(300):
        d = S.sample(l, S.Sampler(temperature=0.8, top_k=20, top_p=0.9, seed=4), c)
        cdf = np.cumsum(d.probs)
        lo = cdf[d.token - 1] if d.token else 0.0
        assert lo <= d.u < cdf[d.token] and d.probs[d.token] > 0
        assert d.u == S.uniform(4, c)


@pytest.mark.parametrize("s", [S.Sampler(temperature=1.0, seed=5), S.Sampler(temperature=0.7, seed=6),
                               S.Sampler(temperature=1.3, top_k=3, seed=7),
                               S.Sampler(temperature=1.0, top_p=0.75, seed=8),
                               S.Sampler(temperature=1.0, top_p=0.75, min_p=0.2, seed=9)])
def test_chi_square_of_draws_against_the_exact_distribution(s):
    scipy_stats = pytest.importorskip("scipy.stats")
    n = 20000
    p = _probs(s)
    counts = np.bincount([S.sample(LQ, s, c).token for c in range(n)], minlength=Q.size)
    assert np.all(counts[p == 0] == 0)
    live = p > 0
    res = scipy_stats.chisquare(counts[live], p[live] * n)
    assert res.pvalue > 1e-4, (counts, p * n)


def test_same_seed_same_tokens():
    rng = np.random.default_rng(2)
    l = rng.standard_normal(1000) * 2
    s = S.Sampler(temperature=1.0, top_p=0.95, seed=77)
    a = [S.sample(l, s, c).token for c in range(50)]
    b = [S.sample(l, s, c).token for c in range(50)]
    assert a == b and len(set(a)) > 5
