"""Pins of the oracle's sampled tokens (the sampled-token alternative to argmax).

The draw (openai-hub page "从零拆开DiffusionGemma", step 4: real samplers draw from the
tempered distribution) is the inverse CDF over the whole vocabulary with one Philox
uniform per position. The tests check the frequencies against p with chi-square tests,
the closed forms of the inverse CDF on two-token and uniform distributions with the
uniform taken from numpy's own Philox4x64-10 (an implementation independent of the
oracle's), its monotonicity under stochastic dominance, the degenerate cases by hand, and
that the Philox counters make positions, steps and canvases independent draws.
"""
import math

import numpy as np
import scipy.stats as st

import oracle as O


def numpy_uniform(seed, canvas, step, pos):
    """u = (word 0 >> 11) / 2^53 of Philox4x64-10 with key (seed, canvas) and counter
    (pos, step, 2, 0), computed by numpy's generator. numpy emits the block of counter
    c + 1 first (the counter read as one 256-bit number, word 0 lowest), so it is
    started at that number minus one."""
    value = pos + (step << 64) + (2 << 128) - 1
    ctr = [(value >> (64 * i)) & (2 ** 64 - 1) for i in range(4)]
    g = np.random.Philox(key=np.array([seed, canvas], np.uint64), counter=np.array(ctr, np.uint64))
    w = int(g.random_raw(1)[0])
    return (w >> 11) * 2.0 ** -53


def draws(p_row, n, seed=3, canvas=0, pos=0):
    p = np.asarray(p_row, dtype=np.float64)[None]
    return np.array([O.sample_tokens(p, seed, canvas, step)[0] for step in range(n)])


def test_uniform_matches_numpy_philox():
    for seed, canvas, step, pos in ((3, 0, 0, 0), (1, 7, 5, 9), (2 ** 40 + 5, 3, 47, 255), (9, 1, 0, 4)):
        assert O.sample_uniform(seed, canvas, step, pos) == numpy_uniform(seed, canvas, step, pos)


def test_two_token_closed_form():
    # p = (a, 1 - a): the inverse CDF takes id 0 exactly when u < a
    for a in (0.1, 0.5, 0.73):
        p = np.array([[a, 1.0 - a]])
        for step in range(60):
            u = numpy_uniform(5, 2, step, 3)
            x = O.sample_tokens(p, 5, 2, step, positions=[3])[0]
            assert x == (0 if u < a else 1), (a, step, u, x)


def test_uniform_distribution_closed_form():
    # uniform p over V ids: token = floor(u V) (away from the exact multiples of 1/V)
    V = 1000
    p = np.full((1, V), 1.0 / V)
    for step in range(40):
        u = numpy_uniform(8, 0, step, 0)
        x = O.sample_tokens(p, 8, 0, step)[0]
        if abs(u * V - round(u * V)) > 1e-9:
            assert x == math.floor(u * V), (step, u, x)


def test_frequencies_match_p():
    # 20 ids with mass spread over a 300-id vocabulary, unequal weights
    V = 300
    p = np.zeros(V)
    ids = list(range(0, 10)) + list(range(256, 266))
    w = np.array([1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 2, 2, 2, 2, 2, 4, 4, 4, 4, 4], float)
    p[ids] = w / w.sum()
    n = 4000
    x = draws(p, n)
    assert set(np.unique(x)) <= set(ids)
    counts = np.array([(x == i).sum() for i in ids])
    chi = st.chisquare(counts, f_exp=p[ids] * n)
    assert chi.pvalue > 1e-3, chi


def test_frequencies_over_a_wide_vocabulary():
    # mass over 1536 ids, grouped into six bins of 256 for the chi-square test
    V = 256 * 6
    rng = np.random.default_rng(11)
    p = rng.random(V) ** 4
    p[256:512] *= 5.0
    p /= p.sum()
    n = 3000
    x = draws(p, n, seed=9)
    bins = x // 256
    masses = np.array([p[t * 256:(t + 1) * 256].sum() for t in range(6)])
    counts = np.bincount(bins, minlength=6)
    chi = st.chisquare(counts, f_exp=masses * n)
    assert chi.pvalue > 1e-3, chi


def test_stochastic_dominance_is_monotone():
    # moving mass towards lower ids can only lower the drawn id for the same uniform
    rng = np.random.default_rng(14)
    for trial in range(30):
        p = rng.dirichlet(np.ones(64) * 0.5)
        q = p.copy()
        i, j = sorted(rng.choice(64, 2, replace=False))
        move = q[j] * rng.random()
        q[j] -= move
        q[i] += move
        for step in range(5):
            a = O.sample_tokens(p[None], 4, trial, step)[0]
            b = O.sample_tokens(q[None], 4, trial, step)[0]
            assert b <= a


def test_one_hot_and_tail_mass():
    p = np.zeros(700)
    p[517] = 1.0
    assert set(draws(p, 50)) == {517}
    p = np.zeros(700)
    p[600:700] = 1.0 / 100                          # mass only at the end of the vocabulary
    x = draws(p, 200)
    assert np.all((x >= 600) & (x < 700))
    p = np.zeros(700)
    p[0] = 1.0                                      # all mass on the first id
    assert set(draws(p, 20)) == {0}


def test_counters_separate_positions_steps_canvases():
    rng = np.random.default_rng(12)
    p = rng.dirichlet(np.ones(512), size=4)
    a = O.sample_tokens(p, 1, 0, 0, B=2)
    assert np.array_equal(a, O.sample_tokens(p, 1, 0, 0, B=2))          # deterministic
    # canvas ids: rows of canvas b equal a one-canvas call with canvas_base + b
    for b in range(2):
        np.testing.assert_array_equal(a[2 * b:2 * b + 2], O.sample_tokens(p[2 * b:2 * b + 2], 1, b, 0))
    # different steps and seeds give different draws over many rows
    q = rng.dirichlet(np.ones(512) * 0.2, size=64)
    s0, s1, s2 = (O.sample_tokens(q, 1, 0, 0), O.sample_tokens(q, 1, 0, 1), O.sample_tokens(q, 2, 0, 0))
    assert (s0 != s1).mean() > 0.5 and (s0 != s2).mean() > 0.5


def test_margin_is_the_distance_to_the_nearest_boundary():
    p = np.random.default_rng(13).dirichlet(np.ones(600), size=3)
    x, margin = O.sample_tokens(p, 1, 0, 0, with_margins=True)
    for r in range(3):
        u = O.sample_uniform(1, 0, 0, r)
        cum = np.cumsum(p[r])
        t = u * cum[-1]
        lo = cum[x[r] - 1] if x[r] else 0.0
        assert lo <= t < cum[x[r]]
        assert margin[r] == min(t - lo, cum[x[r]] - t) and margin[r] >= 0
