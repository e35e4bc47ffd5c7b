"""Pins of the oracle's sampled tokens (the sampled-token alternative to argmax).

The draw (openai-hub page "从零拆开DiffusionGemma", step 4: real samplers draw with
temperature and Gumbel noise) must be a sample from p^0: the tests check the frequencies
against p with chi-square tests, the degenerate and boundary cases by hand, and that the
Philox counters make positions, steps and canvases independent draws.
"""
import math

import numpy as np
import pytest
import scipy.stats as st

import oracle as O


def draws(p_row, n, seed=3, canvas=0, pos=0):
    p = np.asarray(p_row, dtype=np.float64)[None]
    return np.array([O.sample_tokens(p, seed, canvas, step)[0] for step in range(n)])


def test_frequencies_match_p_across_two_chunks():
    # 20 ids with mass, 10 in chunk 0 and 10 in chunk 1 (V = 300: chunks of 256 and 44),
    # unequal weights and unequal chunk masses
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


def test_chunk_stage_follows_chunk_masses():
    # many chunks, mass concentrated unevenly: the chunk of the draw ~ the chunk masses
    V = 256 * 6
    rng = np.random.default_rng(11)
    p = rng.random(V) ** 4
    p[256:512] *= 5.0
    p /= p.sum()
    n = 3000
    x = draws(p, n, seed=9)
    chunks = x // 256
    masses = np.array([p[t * 256:(t + 1) * 256].sum() for t in range(6)])
    counts = np.bincount(chunks, minlength=6)
    chi = st.chisquare(counts, f_exp=masses * n)
    assert chi.pvalue > 1e-3, chi


def test_one_hot_and_single_chunk_mass():
    p = np.zeros(700)
    p[517] = 1.0
    assert set(draws(p, 50)) == {517}
    p = np.zeros(700)
    p[600:700] = 1.0 / 100                          # mass only in the partial last chunk
    x = draws(p, 200)
    assert np.all((x >= 600) & (x < 700))


def test_gumbel_noise_definition():
    # G = -ln(-ln((h + 1/2) / 2^32)) from the stated word and half
    for v in (0, 1, 7, 8, 255, 1000):
        w = O.philox4x64_10((5, 2, 3, v // 8), (1, 4))[(v % 8) // 2]
        h = (w >> 32) if v % 2 else (w & 0xFFFFFFFF)
        g = -math.log(-math.log((h + 0.5) / 2 ** 32))
        assert O.gumbel_noise(1, 4, 2, 5, v) == g
    # standard Gumbel over many ids: mean = Euler-Mascheroni, var = pi^2 / 6
    g = np.array([O.gumbel_noise(7, 0, 0, 0, v) for v in range(20000)])
    assert abs(g.mean() - 0.5772156649) < 0.03
    assert abs(g.var() - math.pi ** 2 / 6) < 0.08


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


def test_margins_reported():
    p = np.random.default_rng(13).dirichlet(np.ones(600), size=3)
    x, mc, mg = O.sample_tokens(p, 1, 0, 0, with_margins=True)
    assert np.all(mc >= 0) and np.all(mc <= 1) and np.all(mg >= 0)
