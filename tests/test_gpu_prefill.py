"""Parity of the block prefill (the causal re-encode commit) and of rotary positions in
canvas attention, HIP path against the oracle (needs an MI355X).

Bars: A and the appended K/V rows within 2e-2 max relative error (bf16 inputs, fp32
accumulation, float64 oracle), the prefix rows byte-unchanged, P advanced by C; causality
checked bit-exactly (changing later block tokens leaves earlier rows' outputs and keys
byte-identical).
"""
import numpy as np
import pytest
import torch

import block_ar_canvas_amd as dg
import dg_inputs as di
import oracle as O
from gpu_util import DEV, bits_np, cache_logical, i32_dev, maxrel, maxrel_rows, upload_cache
from test_gpu_calls import SHAPES, setup, ws_for

pytestmark = pytest.mark.gpu


def run_prefill(ctx, cfg, Wd, Kp, Vp, Pcap, P, tokens, rope_base):
    Kd, Vtd = upload_cache(Kp[:, :P], Vp[:, :P], Pcap)
    ws = ws_for(cfg, Pcap)
    A = torch.empty(cfg.C, cfg.d, dtype=torch.bfloat16, device=DEV)
    ctx.set_rope(rope_base)
    try:
        P2 = ctx.prefill_block(cfg, i32_dev(tokens), Wd["E"], Wd["Wq"], Wd["Wk"], Wd["Wv"], Wd["Wo"],
                               Kd, Vtd, P, ws, A)
        ctx.sync()
    finally:
        ctx.set_rope(0.0)
    return P2, bits_np(A), cache_logical(Kd, Vtd)


# "wide" (C = 300, two query heads per KV head) puts the canvas into more than one key
# split, and its 32-row waves straddle the two heads: under the causal mask a split that
# starts inside the canvas has lanes that see keys next to lanes that see none yet.
@pytest.mark.parametrize("name", ["tiny", "small", "ragged", "hd64", "wide"])
@pytest.mark.parametrize("rope_base", [0.0, 10000.0])
@pytest.mark.parametrize("prefix", ["full", "empty"])
def test_prefill_block(dg_ctx, name, rope_base, prefix):
    cfg, W, Kp, Vp, Pcap, Wd = setup(name)
    P = cfg.P0 if prefix == "full" else 0
    tok = np.random.default_rng(cfg.seed + 5).integers(0, cfg.V, cfg.C).astype(np.int32)
    P2, A, (Kg, Vg) = run_prefill(dg_ctx, cfg, Wd, Kp, Vp, Pcap, P, tok, rope_base)
    Ko, Vo = Kp.copy(), Vp.copy()
    Ao, Po = O.prefill_block(tok, W["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], Ko, Vo, P,
                             cfg.Hq, cfg.Hkv, cfg.hd, rope_base)
    assert P2 == Po == P + cfg.C
    assert maxrel_rows(O.from_bf16(A), O.from_bf16(Ao)) <= 2e-2
    np.testing.assert_array_equal(Kg[:, :P], Kp[:, :P])
    np.testing.assert_array_equal(Vg[:, :P], Vp[:, :P])
    assert maxrel(O.from_bf16(Kg[:, P:P2]), O.from_bf16(Ko[:, P:P2])) <= 2e-2
    assert maxrel(O.from_bf16(Vg[:, P:P2]), O.from_bf16(Vo[:, P:P2])) <= 2e-2


@pytest.mark.parametrize("rope_base", [0.0, 10000.0])
def test_prefill_block_is_causal_bit_exact(dg_ctx, rope_base):
    cfg, W, Kp, Vp, Pcap, Wd = setup("small")
    rng = np.random.default_rng(9)
    tok = rng.integers(0, cfg.V, cfg.C).astype(np.int32)
    tok2 = tok.copy()
    cut = 150
    tok2[cut:] = (tok2[cut:] + 11) % cfg.V
    _, A1, (K1, V1) = run_prefill(dg_ctx, cfg, Wd, Kp, Vp, Pcap, cfg.P0, tok, rope_base)
    _, A2, (K2, V2) = run_prefill(dg_ctx, cfg, Wd, Kp, Vp, Pcap, cfg.P0, tok2, rope_base)
    np.testing.assert_array_equal(A1[:cut], A2[:cut])
    np.testing.assert_array_equal(K1[:, :cfg.P0 + cut], K2[:, :cfg.P0 + cut])
    np.testing.assert_array_equal(V1[:, :cfg.P0 + cut], V2[:, :cfg.P0 + cut])
    assert np.any(A1[cut:] != A2[cut:])


@pytest.mark.parametrize("name", ["tiny", "small", "ragged", "hd64"])
def test_canvas_attention_rotary(dg_ctx, name):
    cfg, W, Kp, Vp, Pcap, Wd = setup(name)
    P = cfg.P0
    Kd, Vtd = upload_cache(Kp[:, :P], Vp[:, :P], Pcap)
    ws = ws_for(cfg, Pcap)
    tok = np.random.default_rng(cfg.seed + 6).integers(0, cfg.V, cfg.C).astype(np.int32)
    A = torch.empty(cfg.C, cfg.d, dtype=torch.bfloat16, device=DEV)
    dg_ctx.set_rope(10000.0)
    try:
        dg_ctx.canvas_attn(cfg, i32_dev(tok), None, Wd["E"], Wd["Wq"], Wd["Wk"], Wd["Wv"], Wd["Wo"],
                           Kd, Vtd, P, ws, A)
        dg_ctx.sync()
    finally:
        dg_ctx.set_rope(0.0)
    Ao, _ = O.canvas_attn(tok, None, W["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], Kp, Vp, P,
                          cfg.Hq, cfg.Hkv, cfg.hd, rope_base=10000.0)
    assert maxrel_rows(O.from_bf16(bits_np(A)), O.from_bf16(Ao)) <= 2e-2


def test_prefill_block_errors(dg_ctx):
    cfg, W, Kp, Vp, Pcap, Wd = setup("tiny")
    Kd, Vtd = upload_cache(Kp[:, :cfg.P0], Vp[:, :cfg.P0], Pcap)
    ws = ws_for(cfg, Pcap)
    A = torch.empty(cfg.C, cfg.d, dtype=torch.bfloat16, device=DEV)
    tok = i32_dev(np.zeros(cfg.C, np.int32))
    with pytest.raises(dg.DGError):                  # P + C > Pcap: nothing enqueued
        dg_ctx.prefill_block(cfg, tok, Wd["E"], Wd["Wq"], Wd["Wk"], Wd["Wv"], Wd["Wo"], Kd, Vtd,
                             Pcap - cfg.C + 8, ws, A)
    with pytest.raises(dg.DGError):
        dg_ctx.set_rope(-1.0)
    Kg, Vg = cache_logical(Kd, Vtd)
    np.testing.assert_array_equal(Kg[:, :cfg.P0], Kp[:, :cfg.P0])
