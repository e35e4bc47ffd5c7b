"""Pins of the oracle's confidence rule against what the pages and the mathematics fix.

The rule (openai-hub page "从零拆开DiffusionGemma", step 4, confidence decoding; "Text
diffusion models" survey, section 5): a position's confidence is its largest tempered
probability, and each step keeps the most confident positions, as many as the page's
simplified decoder has revealed by then (ceil(unresolved / remaining steps) per step),
pinned by the closed form that rule reduces to.
"""
import math

import numpy as np
import pytest
import scipy.special as sps

import dg_inputs as di
import oracle as O
from dg_inputs import f32_to_bf16_bits


def bf16(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


# ------------------------------------------------------------------ confidence
@pytest.mark.parametrize("V", [2, 512, 32768])
def test_uniform_logits_confidence_is_one_over_v(V):
    E = bf16(np.random.default_rng(3).standard_normal((V, 8)))
    conf = O.confidence(bf16(np.zeros((3, 8))), E, 0.8)
    np.testing.assert_allclose(conf, 1.0 / V, rtol=1e-6)


@pytest.mark.parametrize("gap", [0.0, 0.25, 1.0, 3.0, -2.0])
@pytest.mark.parametrize("tau", [0.8, 0.4])
def test_two_token_confidence_closed_form(gap, tau):
    # logits (gap, 0): p = 1 / (1 + exp(-gap / tau)); confidence = max(p, 1 - p)
    conf = O.confidence(bf16([[gap]]), bf16([[1.0], [0.0]]), tau)
    t = float(np.float32(tau))
    g = float(np.float32(gap))
    pr = 1.0 / (1.0 + math.exp(-g / t))
    assert abs(float(conf[0]) - max(pr, 1.0 - pr)) < 1e-7


def test_confidence_one_hot_limit_and_scipy():
    rng = np.random.default_rng(4)
    E = bf16(rng.standard_normal((300, 6)))
    H = bf16(rng.standard_normal((5, 6)))
    for tau in (0.8, 0.4, 0.05):
        conf = O.confidence(H, E, tau)
        u = (di.bf16_bits_to_f32(H).astype(np.float64) @ di.bf16_bits_to_f32(E).astype(np.float64).T) / float(np.float32(tau))
        ref = sps.softmax(u, axis=1).max(axis=1)
        np.testing.assert_allclose(conf, ref, rtol=1e-6)
    # a dominant logit: confidence -> 1
    Eb = bf16(np.vstack([np.full((1, 4), 4.0), np.zeros((99, 4))]))
    conf = O.confidence(bf16(np.full((1, 4), 4.0)), Eb, 0.4)
    assert conf[0] > 1 - 1e-30 or conf[0] == np.float32(1.0)


# ------------------------------------------------------------------ reveal schedule
# The rule as the page states it: each step reveals ceil(unresolved / remaining steps),
# i.e. n_t = n_{t-1} + ceil((C - n_{t-1}) / (N - t)) with n_{-1} = 0. Writing C = qN + r
# (0 <= r < N): while t < r the unresolved count is (N - t) q + (r - t) with
# 0 < r - t < N - t, so the step reveals q + 1; from t = r on it is (N - t) q, so the step
# reveals q. Hence the closed form n_t = (t + 1) q + min(t + 1, r).
def closed_form(C, N):
    q, r = divmod(C, N)
    return [(t + 1) * q + min(t + 1, r) for t in range(N)]


def test_reveal_schedule_hand_worked():
    # C = 5 over N = 9: one position per step until all five are out, then none
    assert O.reveal_schedule(5, 9) == [1, 2, 3, 4, 5, 5, 5, 5, 5]
    # C = 256 over N = 48: 256 = 5 * 48 + 16, six per step for 16 steps, then five
    sched = O.reveal_schedule(256, 48)
    assert sched[:4] == [6, 12, 18, 24]
    assert sched[15:18] == [96, 101, 106]
    assert sched[-2:] == [251, 256]
    assert [b - a for a, b in zip([0] + sched, sched)] == [6] * 16 + [5] * 32
    # C = 1 over N = 1 and C = 0
    assert O.reveal_schedule(1, 1) == [1]
    assert O.reveal_schedule(0, 4) == [0, 0, 0, 0]


@pytest.mark.parametrize("C,N", [(256, 48), (16, 8), (100, 7), (5, 9), (1, 1), (1000, 48), (47, 48), (49, 48)])
def test_reveal_schedule_closed_form(C, N):
    sched = O.reveal_schedule(C, N)
    assert sched == closed_form(C, N)
    assert sched[-1] == C
    assert all(a <= b for a, b in zip(sched, sched[1:]))


def test_reveal_schedule_linear_when_divisible():
    # C a multiple of N: the page's "linear reveal progress", C/N positions per step
    for C, N in ((256, 8), (96, 48), (48, 48)):
        assert O.reveal_schedule(C, N) == [(t + 1) * C // N for t in range(N)]


# ------------------------------------------------------------------ top-k acceptance
def test_topk_brute_force_random_with_ties():
    rng = np.random.default_rng(5)
    for trial in range(200):
        C = int(rng.integers(1, 40))
        vals = rng.choice(np.array([0.1, 0.2, 0.2, 0.5, 0.9, np.nan], np.float32), size=C)
        k = int(rng.integers(0, C + 3))
        acc, n = O.topk_accept(vals[None], k)
        valid = [i for i in range(C) if not np.isnan(vals[i])]
        # brute force: accepted = the first k of all valid positions ranked by counting,
        # for each position, how many valid positions beat it
        def beats(j, i):
            return vals[j] > vals[i] or (vals[j] == vals[i] and j < i)
        rank = {i: sum(beats(j, i) for j in valid if j != i) for i in valid}
        ref = np.zeros(C, np.uint8)
        for i in valid:
            if rank[i] < k:
                ref[i] = 1
        np.testing.assert_array_equal(acc[0], ref)
        assert n[0] == min(k, len(valid))
        # invariant: every accepted score >= every rejected valid score
        a = vals[acc[0] == 1]
        r = np.array([vals[i] for i in valid if acc[0, i] == 0])
        if len(a) and len(r):
            assert a.min() >= r.max()


def test_topk_special_cases():
    s = np.array([[0.3, np.nan, 0.3, 0.7]], np.float32)
    np.testing.assert_array_equal(O.topk_accept(s, 0)[0], [[0, 0, 0, 0]])
    np.testing.assert_array_equal(O.topk_accept(s, 1)[0], [[0, 0, 0, 1]])
    np.testing.assert_array_equal(O.topk_accept(s, 2)[0], [[1, 0, 0, 1]])   # tie -> lower position
    np.testing.assert_array_equal(O.topk_accept(s, 10)[0], [[1, 0, 1, 1]])  # NaN never
    z = np.array([[-0.0, 0.0]], np.float32)
    np.testing.assert_array_equal(O.topk_accept(z, 1)[0], [[0, 1]])         # +0 above -0


def test_topk_segments_independent():
    rng = np.random.default_rng(6)
    s = rng.random((4, 30)).astype(np.float32)
    acc, n = O.topk_accept(s, 7)
    for b in range(4):
        a1, n1 = O.topk_accept(s[b], 7)
        np.testing.assert_array_equal(acc[b], a1[0])
        assert n[b] == n1[0] == 7


# ------------------------------------------------------------------ loop with the rule
def test_confidence_rule_loop_accepts_schedule_and_keeps_argmax():
    cfg = di.config(0)
    W = di.weights(cfg)
    Kp, Vp = di.prefix_kv(cfg, cfg.P0 + cfg.C)
    tgt = di.targets(cfg, 0)
    sched = O.reveal_schedule(cfg.C, cfg.N)
    P, recs = O.run_canvas(W, Kp, Vp, cfg.P0, lambda k: di.hidden(cfg, W["E"], 0, k, tgt),
                           V=cfg.V, C=cfg.C, Hq=cfg.Hq, Hkv=cfg.Hkv, hd=cfg.hd, N=cfg.N,
                           seed=cfg.seed, canvas=0, rule="confidence", with_attn=False)
    assert len(recs) == cfg.N and P == cfg.P0 + cfg.C
    for r in recs:
        assert r["n_accept"] == sched[r["k"]]
        acc = r["accept"].astype(bool)
        np.testing.assert_array_equal(r["tokens"][acc], r["argmax"][acc])
    assert recs[-1]["accept"].all()                 # the last step accepts every position
