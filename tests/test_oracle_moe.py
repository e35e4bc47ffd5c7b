"""Pins of the oracle's canvas MoE FFN (DiffusionGemma Technical Report page,
"Prerequisites", mixture of experts: 8 of 128 experts plus one shared expert per token;
"Text diffusion models" survey, sections 11 and 13: router top-k, expert GEMM, token
permutation).
"""
import numpy as np
import pytest
import torch

import oracle as O
from dg_inputs import f32_to_bf16_bits


def bf16(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def make(C=10, d=16, E=8, Fe=12, Fs=10, seed=0):
    r = np.random.default_rng(seed)
    return (bf16(r.standard_normal((C, d))), bf16(r.standard_normal((E, d))),
            bf16(r.standard_normal((E, Fe, d)) * 0.3), bf16(r.standard_normal((E, d, Fe)) * 0.3),
            bf16(r.standard_normal((Fs, d)) * 0.3), bf16(r.standard_normal((d, Fs)) * 0.3))


def ffn_torch(x, W1, W2):
    """Independent FFW route: torch F.linear and the exact-erf GELU, float64."""
    h = torch.nn.functional.gelu(torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(W1)),
                                 approximate="none")
    return torch.nn.functional.linear(h, torch.from_numpy(W2)).numpy()


def test_routing_is_brute_force_top_k_with_ties_and_softmax_gates():
    rng = np.random.default_rng(1)
    for trial in range(30):
        X, Wr, *_ = make(C=6, E=9, seed=trial)
        if trial % 3 == 0:                       # duplicated router rows force tied logits
            Wr[4] = Wr[1]
            Wr[7] = Wr[1]
        K = int(rng.integers(1, 9))
        sel, gates, r = O.moe_route(X, Wr, K)
        for t in range(X.shape[0]):
            # brute force: rank every expert by how many beat it
            beats = [sum((r[t, j] > r[t, e]) or (r[t, j] == r[t, e] and j < e) for j in range(9))
                     for e in range(9)]
            ref = sorted(range(9), key=lambda e: beats[e])[:K]
            assert list(sel[t]) == ref
            v = r[t, ref].astype(np.float64)
            np.testing.assert_allclose(gates[t], np.exp(v - v.max()) / np.exp(v - v.max()).sum(), rtol=1e-15)
            assert abs(gates[t].sum() - 1.0) < 1e-12


def test_single_expert_is_the_ffw_plus_shared():
    X, Wr, W1, W2, W1s, W2s = make(E=1)
    Y, sel, gates, n = O.moe_ffn(X, Wr, W1, W2, W1s, W2s, K=1)
    assert n == 1 and np.all(gates == 1.0)
    x = O.from_bf16(X)
    y = O.from_bf16(O.to_bf16(O.from_bf16(O.to_bf16(
        ffn_torch(x, O.from_bf16(W1[0]), np.eye(W1.shape[1])))) @ O.from_bf16(W2[0]).T))
    ys = O.from_bf16(O.to_bf16(O.from_bf16(O.to_bf16(
        ffn_torch(x, O.from_bf16(W1s), np.eye(W1s.shape[0])))) @ O.from_bf16(W2s).T))
    np.testing.assert_array_equal(Y, O.to_bf16(y + ys))


def test_identical_experts_cancel_the_gates():
    # every expert the same: the K gates sum to 1, so y = E(x) + S(x) whatever the routing
    X, Wr, W1, W2, W1s, W2s = make(E=8)
    W1[:] = W1[3]
    W2[:] = W2[3]
    Y, sel, _, _ = O.moe_ffn(X, Wr, W1, W2, W1s, W2s, K=3)
    x = O.from_bf16(X)
    y = O.from_bf16(O.to_bf16(O.from_bf16(O.to_bf16(O.gelu_erf(x @ O.from_bf16(W1[3]).T))) @ O.from_bf16(W2[3]).T))
    ys = O.from_bf16(O.to_bf16(O.from_bf16(O.to_bf16(O.gelu_erf(x @ O.from_bf16(W1s).T))) @ O.from_bf16(W2s).T))
    got, ref = O.from_bf16(Y), y + ys
    assert np.abs(got - ref).max() <= 2.0 ** -7 * np.abs(ref).max()    # bf16 rounding of y
    assert len(np.unique(sel)) > 3                                       # routing did vary


def test_token_permutation_equivariant_and_row_independent():
    X, Wr, W1, W2, W1s, W2s = make(C=12, E=8, seed=5)
    Y, sel, gates, _ = O.moe_ffn(X, Wr, W1, W2, W1s, W2s, K=2)
    perm = np.random.default_rng(6).permutation(12)
    Yp, selp, _, _ = O.moe_ffn(X[perm], Wr, W1, W2, W1s, W2s, K=2)
    np.testing.assert_array_equal(Yp, Y[perm])
    np.testing.assert_array_equal(selp, sel[perm])
    Y1, _, _, _ = O.moe_ffn(X[[4]], Wr, W1, W2, W1s, W2s, K=2)
    np.testing.assert_array_equal(Y1[0], Y[4])


def test_gate_weighting_matters():
    # a mistake in the gates (e.g. uniform 1/K) would change the output
    X, Wr, W1, W2, W1s, W2s = make(E=8, seed=7)
    Y, sel, gates, _ = O.moe_ffn(X, Wr, W1, W2, W1s, W2s, K=3)
    x = O.from_bf16(X)
    acc = np.zeros((X.shape[0], X.shape[1]))
    for t in range(X.shape[0]):
        for k in range(3):
            e = sel[t, k]
            h = O.from_bf16(O.to_bf16(O.gelu_erf(x[t:t + 1] @ O.from_bf16(W1[e]).T)))
            acc[t] += (1.0 / 3) * O.from_bf16(O.to_bf16(h @ O.from_bf16(W2[e]).T))[0]
    ys = O.from_bf16(O.to_bf16(O.from_bf16(O.to_bf16(O.gelu_erf(x @ O.from_bf16(W1s).T))) @ O.from_bf16(W2s).T))
    assert np.any(O.to_bf16(acc + ys) != Y)
    assert not np.allclose(gates, 1.0 / 3)


def test_canvas_share_gives_the_pages_expert_count():
    # the MoE workload's input recipe: canvas rows sharing part of their direction route a
    # 256-token canvas to about 84 of 128 experts at top-8 (DiffusionGemma Technical Report
    # page, "Prerequisites"); independent rows reach nearly all of them
    import dg_inputs as di
    for seed in (51, 61):
        inp = di.moe_inputs(256, 2048, 128, 8, 32, 32, seed=seed, share=di.MOE_CANVAS_SHARE)
        sel, _, _ = O.moe_route(inp["X"], inp["Wr"], 8)
        assert 72 <= len(np.unique(sel)) <= 96
        x = O.from_bf16(inp["X"])
        assert abs(x.std() - 1.0) < 0.05                 # rows stay N(0, 1) per element
    inp = di.moe_inputs(256, 2048, 128, 8, 32, 32, seed=51)
    assert len(np.unique(O.moe_route(inp["X"], inp["Wr"], 8)[0])) >= 120
