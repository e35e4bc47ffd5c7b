"""Pins of the oracle's rotary positions and causal block prefill (the re-encode commit).

The commit of a finalized block re-encodes it causally into the KV cache (tutorial
chapter "DiffusionGemma": the data-flow pseudocode's incremental prefill and the KV-cache
write timing); rotary position encoding is part of the full model (openai-hub page
"从零拆开DiffusionGemma", closing remarks of step 3). These tests pin the oracle against
independent formulations: complex rotation, torch's causal attention, causality itself.
"""
import math

import numpy as np
import pytest
import torch

import dg_inputs as di
import oracle as O
from dg_inputs import f32_to_bf16_bits


def bf16(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


# ------------------------------------------------------------------ rotary positions
def rope_complex(x, positions, base):
    """Independent formulation: pair d as the complex number x_d + i x_{d+h}, times
    exp(i * pos * theta_d)."""
    n, H, hd = x.shape
    h = hd // 2
    z = x[..., :h] + 1j * x[..., h:]
    theta = np.array([base ** (-2.0 * d / hd) for d in range(h)])
    rot = np.exp(1j * np.outer(np.asarray(positions, float), theta))[:, None, :]
    w = z * rot
    return np.concatenate([w.real, w.imag], axis=-1)


@pytest.mark.parametrize("hd", [16, 64, 128])
def test_rope_equals_complex_rotation(hd):
    rng = np.random.default_rng(hd)
    x = rng.standard_normal((7, 3, hd))
    pos = [0, 1, 5, 255, 8192, 34559, 262399]
    np.testing.assert_allclose(O.rope(x, pos, 10000.0), rope_complex(x, pos, 10000.0), rtol=0, atol=1e-9)


def test_rope_identity_norm_and_first_pair():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 2, 32))
    np.testing.assert_array_equal(O.rope(x, [0] * 4, 10000.0), x)           # position 0
    assert O.rope(x, [3, 4, 5, 6], 0.0) is x                                # base 0: off
    y = O.rope(x, [3, 4, 5, 6], 10000.0)
    np.testing.assert_allclose(np.hypot(y[..., :16], y[..., 16:]), np.hypot(x[..., :16], x[..., 16:]), atol=1e-12)
    # theta_0 = 1: the first pair turns by exactly pos radians
    p = 5
    c, s = math.cos(p), math.sin(p)
    np.testing.assert_allclose(y[2, :, 0], x[2, :, 0] * c - x[2, :, 16] * s, atol=1e-12)


def test_rope_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))
    for m, n in ((10, 3), (300, 299), (0, 40)):
        a = float((O.rope(q, [m], 10000.0) * O.rope(k, [n], 10000.0)).sum())
        b = float((O.rope(q, [m + 1234], 10000.0) * O.rope(k, [n + 1234], 10000.0)).sum())
        assert abs(a - b) < 1e-9


# ------------------------------------------------------------------ causal prefill
def small_cfg():
    return di.Config("pf", V=300, d=64, C=24, Hq=4, Hkv=2, hd=16, F=32, P0=0, N=2,
                     alpha_max=8.0, seed=41)


def test_prefill_empty_prefix_is_torch_causal_attention():
    cfg = small_cfg()
    W = di.weights(cfg)
    tok = np.random.default_rng(3).integers(0, cfg.V, cfg.C)
    Kp = np.zeros((cfg.Hkv, cfg.C, cfg.hd), np.uint16)
    Vp = np.zeros_like(Kp)
    A, P = O.prefill_block(tok, W["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], Kp, Vp, 0,
                           cfg.Hq, cfg.Hkv, cfg.hd)
    assert P == cfg.C
    X = O.from_bf16(W["E"][tok])
    q = O.from_bf16(O.to_bf16(X @ O.from_bf16(W["Wq"]).T)).reshape(cfg.C, cfg.Hq, cfg.hd)
    k = O.from_bf16(Kp).transpose(1, 0, 2)          # [C, Hkv, hd], as stored
    v = O.from_bf16(Vp).transpose(1, 0, 2)
    G = cfg.Hq // cfg.Hkv
    qt = torch.from_numpy(q.transpose(1, 0, 2))[None]
    kt = torch.from_numpy(np.repeat(k.transpose(1, 0, 2), G, axis=0))[None]
    vt = torch.from_numpy(np.repeat(v.transpose(1, 0, 2), G, axis=0))[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)[0]
    ref = O.to_bf16(o.numpy().transpose(1, 0, 2).reshape(cfg.C, -1) @ O.from_bf16(W["Wo"]).T)
    d = np.abs(O.from_bf16(A) - O.from_bf16(ref))
    assert d.max() <= 1e-2 * np.abs(O.from_bf16(ref)).max()
    # the written rows are the projections of the block
    np.testing.assert_array_equal(Kp.transpose(1, 0, 2).reshape(cfg.C, -1),
                                  O.to_bf16(X @ O.from_bf16(W["Wk"]).T))


@pytest.mark.parametrize("rope_base", [0.0, 10000.0])
def test_prefill_is_causal(rope_base):
    cfg = small_cfg()
    W = di.weights(cfg)
    rng = np.random.default_rng(4)
    P0 = 10
    Kp0 = bf16(rng.standard_normal((cfg.Hkv, P0 + cfg.C, cfg.hd)))
    Vp0 = bf16(rng.standard_normal((cfg.Hkv, P0 + cfg.C, cfg.hd)))
    tok = rng.integers(0, cfg.V, cfg.C)
    tok2 = tok.copy()
    tok2[9:] = (tok2[9:] + 7) % cfg.V               # change every token from position 9 on
    out = []
    for t in (tok, tok2):
        Kp, Vp = Kp0.copy(), Vp0.copy()
        A, P = O.prefill_block(t, W["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], Kp, Vp, P0,
                               cfg.Hq, cfg.Hkv, cfg.hd, rope_base)
        out.append((A, Kp, Vp))
        np.testing.assert_array_equal(Kp[:, :P0], Kp0[:, :P0])              # prefix untouched
        np.testing.assert_array_equal(Vp[:, :P0], Vp0[:, :P0])
    (A1, K1, V1), (A2, K2, V2) = out
    np.testing.assert_array_equal(A1[:9], A2[:9])                           # rows before 9 unchanged
    np.testing.assert_array_equal(K1[:, :P0 + 9], K2[:, :P0 + 9])
    assert np.any(A1[9:] != A2[9:])


def test_prefill_single_token_without_prefix_returns_its_value():
    cfg = small_cfg()
    W = di.weights(cfg)
    Kp = np.zeros((cfg.Hkv, 8, cfg.hd), np.uint16)
    Vp = np.zeros_like(Kp)
    A, P = O.prefill_block(np.array([17]), W["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], Kp, Vp, 0,
                           cfg.Hq, cfg.Hkv, cfg.hd, 10000.0)
    v = O.from_bf16(O.to_bf16(O.from_bf16(W["E"][[17]]) @ O.from_bf16(W["Wv"]).T)).reshape(cfg.Hkv, cfg.hd)
    o = np.concatenate([v[(h * cfg.Hkv) // cfg.Hq] for h in range(cfg.Hq)])[None]
    np.testing.assert_array_equal(A, O.to_bf16(o @ O.from_bf16(W["Wo"]).T))
    assert P == 1


def test_prefill_rotated_keys_and_capacity():
    cfg = small_cfg()
    W = di.weights(cfg)
    tok = np.arange(cfg.C)
    Kp = np.zeros((cfg.Hkv, 40, cfg.hd), np.uint16)
    Vp = np.zeros_like(Kp)
    O.prefill_block(tok, W["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], Kp, Vp, 5, cfg.Hq, cfg.Hkv, cfg.hd, 500.0)
    X = O.from_bf16(W["E"][tok])
    k = O.from_bf16(O.to_bf16(X @ O.from_bf16(W["Wk"]).T)).reshape(cfg.C, cfg.Hkv, cfg.hd)
    kr = O.to_bf16(rope_complex(k, 5 + np.arange(cfg.C), 500.0))
    np.testing.assert_array_equal(Kp[:, 5:5 + cfg.C], kr.transpose(1, 0, 2))
    with pytest.raises(ValueError):
        O.prefill_block(tok, W["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], Kp, Vp, 20, cfg.Hq, cfg.Hkv, cfg.hd)


def test_canvas_attention_rope_rows_match_full():
    cfg = small_cfg()
    W = di.weights(cfg)
    rng = np.random.default_rng(5)
    Kp = bf16(rng.standard_normal((cfg.Hkv, 30, cfg.hd)))
    Vp = bf16(rng.standard_normal((cfg.Hkv, 30, cfg.hd)))
    tok = rng.integers(0, cfg.V, cfg.C)
    A, _ = O.canvas_attn(tok, None, W["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], Kp, Vp, 30,
                         cfg.Hq, cfg.Hkv, cfg.hd, rope_base=10000.0)
    Ar, _ = O.canvas_attn(tok, None, W["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], Kp, Vp, 30,
                          cfg.Hq, cfg.Hkv, cfg.hd, rows=[0, 7, 23], rope_base=10000.0)
    np.testing.assert_array_equal(A[[0, 7, 23]], Ar)
    A0, _ = O.canvas_attn(tok, None, W["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], Kp, Vp, 30,
                          cfg.Hq, cfg.Hkv, cfg.hd)
    assert np.any(A0 != A)                                                  # positions matter
