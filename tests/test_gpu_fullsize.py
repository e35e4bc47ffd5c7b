"""Parity of single calls at the full workload sizes (needs an MI355X).

These tests make the same library calls, with the same workspace layout and launch
configuration, that the benchmark times: the 262144-token vocabulary (d 2048, C 256),
an 8192-token prefix cache, and the commits at the end of an 8-canvas chain. The float64
oracle evaluates every canvas position (E converted to float64 once). Tolerances are those
of the per-call parity tests (entropy 1e-3 nats; argmax exact unless the oracle's top-2
gap is a near-tie; A and z within 2e-2 largest per-row relative error; committed K/V
within one bf16 ulp). The whole loops at these sizes are in test_gpu_headline.py.
"""
import math

import numpy as np
import pytest
import torch

import block_ar_canvas_amd as dg
import dg_inputs as di
import oracle as O
from gpu_util import (DEV, argmax_mismatch_unexcused, bf16_dev, bits_np, cache_logical, i32_dev,
                      maxrel, maxrel_rows, sample_excused, upload_cache, upload_weights, workload)

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

def full(name):
    return workload(name)


def ws_for(cfg, Pcap):
    return torch.empty(dg.workspace_bytes(cfg, Pcap), dtype=torch.uint8, device=DEV)


@pytest.mark.parametrize("k", [24, 47])
def test_sampler_head_and_selfcond_full_vocab(dg_ctx, k):
    cfg, W, W64, Wd = full("gemma_head")
    ws = ws_for(cfg, cfg.Pcap)
    H = di.hidden(cfg, W["E"], 0, k)
    tau = O.temperature(k, cfg.N)
    Hd = bf16_dev(H)
    runs = []
    for rep in range(2):                                # run twice: byte-identical outputs
        ent = torch.empty(cfg.C, dtype=torch.float32, device=DEV)
        am = torch.empty(cfg.C, dtype=torch.int32, device=DEV)
        dg_ctx.logits_entropy(cfg, Hd, Wd["E"], tau, ws, ent, am)
        conf = torch.empty(cfg.C, dtype=torch.float32, device=DEV)
        dg_ctx.confidence(cfg, ws, conf)
        tok = torch.empty(cfg.C, dtype=torch.int32, device=DEV)
        dg_ctx.sample(cfg, ws, 1, 99, 3, k, tok)
        z = torch.empty(cfg.C, cfg.d, dtype=torch.bfloat16, device=DEV)
        dg_ctx.selfcond(cfg, ws, Wd["E"], Wd["W1"], Wd["W2"], z)
        dg_ctx.sync()
        runs.append((ent.cpu().numpy(), am.cpu().numpy(), conf.cpu().numpy(), tok.cpu().numpy(),
                     bits_np(z)))
    for x, y in zip(*runs):
        assert x.tobytes() == y.tobytes()
    e, a, c, g, zg = runs[0]
    assert np.all(np.isfinite(e))
    assert e.min() >= 0.0 and e.max() <= math.log(cfg.V) + 1e-3
    # every position against the oracle
    ent_r, am_r, p_r, u_r = O.logits_entropy(H, W64["E"], tau)
    assert np.max(np.abs(e - ent_r)) <= 1e-3, np.max(np.abs(e - ent_r))
    assert argmax_mismatch_unexcused(a, am_r, u_r) == 0
    del u_r
    np.testing.assert_allclose(c, p_r.max(axis=1), rtol=2e-5, atol=0)
    assert g.min() >= 0 and g.max() < cfg.V
    ref, margin = O.sample_tokens(p_r, 99, 3, k, with_margins=True)
    for i in np.nonzero(g != ref)[0]:
        assert sample_excused(p_r[i], int(ref[i]), float(margin[i])), (i, g[i], ref[i])
    assert np.mean(g == ref) >= 0.95
    z_r, _ = O.selfcond(p_r, W64["E"], W["W1"], W["W2"])
    assert np.all(np.isfinite(O.from_bf16(zg)))
    assert maxrel_rows(O.from_bf16(zg), O.from_bf16(z_r)) <= 2e-2


def test_canvas_attention_full_prefix(dg_ctx):
    # gemma_head's 8192-token prefix, every row; the 262144-token prefix is compared on
    # every row by the loop steps in test_gpu_headline.py
    cfg, W, W64, Wd = full("gemma_head")
    P = cfg.P0
    Pcap = -(-(P + cfg.C) // 8) * 8
    Kp, Vp = di.prefix_kv(cfg, Pcap)
    rng = np.random.default_rng(cfg.seed + 300)
    tok = di.targets(cfg, 0)
    z = di.f32_to_bf16_bits(rng.standard_normal((cfg.C, cfg.d)).astype(np.float32) * 0.3)
    Kd, Vtd = upload_cache(Kp, Vp, Pcap)
    ws = ws_for(cfg, Pcap)
    outs = []
    for rep in range(2):                                # run twice: byte-identical outputs
        A = torch.empty(cfg.C, cfg.d, dtype=torch.bfloat16, device=DEV)
        dg_ctx.canvas_attn(cfg, i32_dev(tok), bf16_dev(z), Wd["E"], Wd["Wq"], Wd["Wk"], Wd["Wv"],
                           Wd["Wo"], Kd, Vtd, P, ws, A)
        dg_ctx.sync()
        outs.append(bits_np(A))
    assert outs[0].tobytes() == outs[1].tobytes()
    Ag = O.from_bf16(outs[0])
    assert np.all(np.isfinite(Ag))
    A_r, _ = O.canvas_attn(tok, z, W64["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], Kp, Vp, P,
                           cfg.Hq, cfg.Hkv, cfg.hd)
    assert maxrel_rows(Ag, O.from_bf16(A_r)) <= 2e-2


def test_batched_sampler_head_full_vocab(dg_ctx):
    # the B = 2 batched line's launch configuration: both canvases' 512 columns in one
    # dg_logits_entropy / dg_selfcond pass over the 262144-token vocabulary
    cfg, W, W64, Wd = full("gemma_head")
    B, k = 2, 40
    dims = dg.Dims(cfg.V, cfg.d, B * cfg.C, cfg.Hq, cfg.Hkv, cfg.hd, cfg.F)
    ws = torch.empty(dg.workspace_bytes(dims, cfg.Pcap), dtype=torch.uint8, device=DEV)
    H = np.concatenate([di.hidden(cfg, W["E"], b, k) for b in range(B)], axis=0)
    tau = O.temperature(k, cfg.N)
    ent = torch.empty(B * cfg.C, dtype=torch.float32, device=DEV)
    am = torch.empty(B * cfg.C, dtype=torch.int32, device=DEV)
    dg_ctx.logits_entropy(dims, bf16_dev(H), Wd["E"], tau, ws, ent, am)
    z = torch.empty(B * cfg.C, cfg.d, dtype=torch.bfloat16, device=DEV)
    dg_ctx.selfcond(dims, ws, Wd["E"], Wd["W1"], Wd["W2"], z)
    dg_ctx.sync()
    e, a = ent.cpu().numpy(), am.cpu().numpy()
    assert np.all(np.isfinite(e)) and e.min() >= 0.0 and e.max() <= math.log(cfg.V) + 1e-3
    ent_r, am_r, p_r, u_r = O.logits_entropy(H, W64["E"], tau)   # all 512 columns
    assert np.max(np.abs(e - ent_r)) <= 1e-3
    assert argmax_mismatch_unexcused(a, am_r, u_r) == 0
    del u_r
    z_r, _ = O.selfcond(p_r, W64["E"], W["W1"], W["W2"])
    assert maxrel_rows(O.from_bf16(bits_np(z)), O.from_bf16(z_r)) <= 2e-2


def test_commit_at_end_of_chain(dg_ctx):
    cfg, W, W64, Wd = full("chain8")
    Pcap = cfg.Pcap
    P = cfg.P0 + (cfg.n_canvas - 1) * cfg.C          # the last canvas of the chain
    Kp, Vp = di.prefix_kv(cfg, Pcap)
    rng = np.random.default_rng(cfg.seed + 400)
    Kp[:, cfg.P0:P] = di.f32_to_bf16_bits(rng.standard_normal((cfg.Hkv, P - cfg.P0, cfg.hd)).astype(np.float32))
    Vp[:, cfg.P0:P] = di.f32_to_bf16_bits(rng.standard_normal((cfg.Hkv, P - cfg.P0, cfg.hd)).astype(np.float32))
    tok = rng.integers(0, cfg.V, cfg.C).astype(np.int32)
    Kd, Vtd = upload_cache(Kp, Vp, Pcap)
    P_new = dg_ctx.commit_kv(cfg, i32_dev(tok), Wd["E"], Wd["Wk"], Wd["Wv"], Kd, Vtd, P)
    dg_ctx.sync()
    assert P_new == P + cfg.C == Pcap
    Kg, Vg = cache_logical(Kd, Vtd)
    K_r, V_r = Kp.copy(), Vp.copy()
    assert O.commit_kv(tok, W64["E"], W["Wk"], W["Wv"], K_r, V_r, P, cfg.Hkv, cfg.hd) == Pcap
    np.testing.assert_array_equal(Kg[:, :P], Kp[:, :P])
    np.testing.assert_array_equal(Vg[:, :P], Vp[:, :P])
    for got, ref in ((Kg[:, P:], K_r[:, P:]), (Vg[:, P:], V_r[:, P:])):
        g = O.from_bf16(got)
        r = O.from_bf16(ref)
        assert maxrel(g, r) <= 2e-2
        # one bf16 ulp, plus the fp32 accumulation error of a 2048-term dot product for
        # results that cancel to far below the tensor's scale
        err = np.abs(g - r)
        bound = np.abs(r) * 2.0 ** -7 + 2.0 ** -16 * np.max(np.abs(r))
        worst = np.unravel_index(np.argmax(err - bound), err.shape)
        assert np.all(err <= bound), (int(np.sum(err > bound)), worst, g[worst], r[worst])


def test_prefill_commit_at_end_of_chain(dg_ctx):
    # the chain8_prefill configuration: the last canvas's block re-encoded causally over a
    # 34560-token cache with rotary positions (base 10000), filling the cache to Pcap
    cfg, W, W64, Wd = full("chain8")
    Pcap = cfg.Pcap
    P = cfg.P0 + (cfg.n_canvas - 1) * cfg.C
    Kp, Vp = di.prefix_kv(cfg, Pcap)
    rng = np.random.default_rng(cfg.seed + 500)
    Kp[:, cfg.P0:P] = di.f32_to_bf16_bits(rng.standard_normal((cfg.Hkv, P - cfg.P0, cfg.hd)).astype(np.float32))
    Vp[:, cfg.P0:P] = di.f32_to_bf16_bits(rng.standard_normal((cfg.Hkv, P - cfg.P0, cfg.hd)).astype(np.float32))
    tok = rng.integers(0, cfg.V, cfg.C).astype(np.int32)
    Kd, Vtd = upload_cache(Kp, Vp, Pcap)
    ws = ws_for(cfg, Pcap)
    A = torch.empty(cfg.C, cfg.d, dtype=torch.bfloat16, device=DEV)
    dg_ctx.set_rope(10000.0)
    try:
        P_new = dg_ctx.prefill_block(cfg, i32_dev(tok), Wd["E"], Wd["Wq"], Wd["Wk"], Wd["Wv"], Wd["Wo"],
                                     Kd, Vtd, P, ws, A)
        dg_ctx.sync()
    finally:
        dg_ctx.set_rope(0.0)
    assert P_new == P + cfg.C == Pcap
    Kg, Vg = cache_logical(Kd, Vtd)
    K_r, V_r = Kp.copy(), Vp.copy()
    A_r, P_r = O.prefill_block(tok, W64["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], K_r, V_r, P,
                               cfg.Hq, cfg.Hkv, cfg.hd, 10000.0)
    assert P_r == Pcap
    np.testing.assert_array_equal(Kg[:, :P], Kp[:, :P])
    np.testing.assert_array_equal(Vg[:, :P], Vp[:, :P])
    assert maxrel_rows(O.from_bf16(Kg[:, P:]), O.from_bf16(K_r[:, P:])) <= 2e-2
    assert maxrel_rows(O.from_bf16(Vg[:, P:]), O.from_bf16(V_r[:, P:])) <= 2e-2
    Ag = O.from_bf16(bits_np(A))
    assert np.all(np.isfinite(Ag))
    assert maxrel_rows(Ag, O.from_bf16(A_r)) <= 2e-2
