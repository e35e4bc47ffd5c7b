"""Edge shapes of the per-call API against the oracle (needs an MI355X).

- "c1000g2": a 1000-token canvas with two query heads per KV head. The canvas spans
  sixteen 64-key tiles and several key splits, and the 32-row waves straddle the two
  heads (1000 is not a multiple of 32), both without and with the causal mask.
- "c1": a one-token canvas (the smallest C).
- "v3": a three-token vocabulary (one vocabulary tile holding 253 padding rows).

Bars as in test_gpu_calls: A, z and appended K/V within 2e-2 (per-row max relative),
entropy within 1e-3 nats, argmax exact outside near-ties.
"""
import numpy as np
import pytest
import torch

import block_ar_canvas_amd as dg
import dg_inputs as di
import oracle as O
from gpu_util import (DEV, argmax_mismatch_unexcused, bf16_dev, bits_np, cache_logical, i32_dev,
                      maxrel, maxrel_rows, upload_cache, upload_weights)

pytestmark = pytest.mark.gpu

EDGES = {
    "c1000g2": di.Config("c1000g2", V=2000, d=128, C=1000, Hq=4, Hkv=2, hd=32, F=64, P0=70, N=4,
                         alpha_max=8.0, seed=61),
    "c1": di.Config("c1", V=700, d=128, C=1, Hq=2, Hkv=1, hd=64, F=64, P0=100, N=4,
                    alpha_max=8.0, seed=62),
    "v3": di.Config("v3", V=3, d=64, C=16, Hq=4, Hkv=2, hd=16, F=32, P0=40, N=6,
                    alpha_max=4.0, seed=63),
}
_cache = {}


def setup(name):
    if name not in _cache:
        cfg = EDGES[name]
        W = di.weights(cfg)
        Pcap = -(-(cfg.P0 + cfg.C) // 8) * 8
        Kp, Vp = di.prefix_kv(cfg, Pcap)
        _cache[name] = (cfg, W, Kp, Vp, Pcap, upload_weights(W))
    return _cache[name]


def ws_for(cfg, Pcap):
    return torch.empty(dg.workspace_bytes(cfg, Pcap), dtype=torch.uint8, device=DEV)


@pytest.mark.parametrize("name", list(EDGES))
@pytest.mark.parametrize("prefix", ["full", "empty"])
def test_edge_canvas_attention(dg_ctx, name, prefix):
    cfg, W, Kp, Vp, Pcap, Wd = setup(name)
    P = cfg.P0 if prefix == "full" else 0
    rng = np.random.default_rng(cfg.seed + 100)
    tok = rng.integers(0, cfg.V, cfg.C).astype(np.int32)
    z = di.f32_to_bf16_bits(rng.standard_normal((cfg.C, cfg.d)).astype(np.float32) * 0.3)
    Kd, Vtd = upload_cache(Kp[:, :P], Vp[:, :P], Pcap)
    A = torch.empty(cfg.C, cfg.d, dtype=torch.bfloat16, device=DEV)
    dg_ctx.canvas_attn(cfg, i32_dev(tok), bf16_dev(z), Wd["E"], Wd["Wq"], Wd["Wk"], Wd["Wv"],
                       Wd["Wo"], Kd, Vtd, P, ws_for(cfg, Pcap), A)
    dg_ctx.sync()
    A_r, _ = O.canvas_attn(tok, z, W["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], Kp, Vp, P,
                           cfg.Hq, cfg.Hkv, cfg.hd)
    assert maxrel_rows(O.from_bf16(bits_np(A)), O.from_bf16(A_r)) <= 2e-2


@pytest.mark.parametrize("name", list(EDGES))
@pytest.mark.parametrize("prefix", ["full", "empty"])
def test_edge_prefill(dg_ctx, name, prefix):
    cfg, W, Kp, Vp, Pcap, Wd = setup(name)
    P = cfg.P0 if prefix == "full" else 0
    tok = np.random.default_rng(cfg.seed + 5).integers(0, cfg.V, cfg.C).astype(np.int32)
    Kd, Vtd = upload_cache(Kp[:, :P], Vp[:, :P], Pcap)
    A = torch.empty(cfg.C, cfg.d, dtype=torch.bfloat16, device=DEV)
    P2 = dg_ctx.prefill_block(cfg, i32_dev(tok), Wd["E"], Wd["Wq"], Wd["Wk"], Wd["Wv"], Wd["Wo"],
                              Kd, Vtd, P, ws_for(cfg, Pcap), A)
    dg_ctx.sync()
    Kg, Vg = cache_logical(Kd, Vtd)
    Ko, Vo = Kp.copy(), Vp.copy()
    Ao, Po = O.prefill_block(tok, W["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], Ko, Vo, P,
                             cfg.Hq, cfg.Hkv, cfg.hd, 0.0)
    assert P2 == Po == P + cfg.C
    assert maxrel_rows(O.from_bf16(bits_np(A)), O.from_bf16(Ao)) <= 2e-2
    np.testing.assert_array_equal(Kg[:, :P], Kp[:, :P])
    np.testing.assert_array_equal(Vg[:, :P], Vp[:, :P])
    assert maxrel(O.from_bf16(Kg[:, P:P2]), O.from_bf16(Ko[:, P:P2])) <= 2e-2
    assert maxrel(O.from_bf16(Vg[:, P:P2]), O.from_bf16(Vo[:, P:P2])) <= 2e-2


@pytest.mark.parametrize("name", list(EDGES))
def test_edge_head_and_selfcond(dg_ctx, name):
    cfg, W, Kp, Vp, Pcap, Wd = setup(name)
    ws = ws_for(cfg, Pcap)
    tgt = di.targets(cfg, 0)
    for k in (0, cfg.N - 1):
        H = di.hidden(cfg, W["E"], 0, k, tgt)
        tau = O.temperature(k, cfg.N)
        ent = torch.empty(cfg.C, dtype=torch.float32, device=DEV)
        am = torch.empty(cfg.C, dtype=torch.int32, device=DEV)
        dg_ctx.logits_entropy(cfg, bf16_dev(H), Wd["E"], tau, ws, ent, am)
        z = torch.empty(cfg.C, cfg.d, dtype=torch.bfloat16, device=DEV)
        dg_ctx.selfcond(cfg, ws, Wd["E"], Wd["W1"], Wd["W2"], z)
        dg_ctx.sync()
        ent_r, am_r, p_r, u_r = O.logits_entropy(H, W["E"], tau)
        e = ent.cpu().numpy()
        assert np.all(np.isfinite(e))
        assert np.max(np.abs(e - ent_r)) <= 1e-3, (k, np.max(np.abs(e - ent_r)))
        assert argmax_mismatch_unexcused(am.cpu().numpy(), am_r, u_r) == 0
        z_r, _ = O.selfcond(p_r, W["E"], W["W1"], W["W2"])
        assert maxrel_rows(O.from_bf16(bits_np(z)), O.from_bf16(z_r)) <= 2e-2


@pytest.mark.parametrize("name", list(EDGES))
def test_edge_commit_kv(dg_ctx, name):
    cfg, W, Kp, Vp, Pcap, Wd = setup(name)
    tok = np.random.default_rng(cfg.seed + 51).integers(0, cfg.V, cfg.C).astype(np.int32)
    Kd, Vtd = upload_cache(Kp, Vp, Pcap)
    K0, V0 = bits_np(Kd), bits_np(Vtd)
    P2 = dg_ctx.commit_kv(cfg, i32_dev(tok), Wd["E"], Wd["Wk"], Wd["Wv"], Kd, Vtd, cfg.P0)
    dg_ctx.sync()
    assert P2 == cfg.P0 + cfg.C
    Ko, Vo = Kp.copy(), Vp.copy()
    O.commit_kv(tok, W["E"], W["Wk"], W["Wv"], Ko, Vo, cfg.P0, cfg.Hkv, cfg.hd)
    Kg, Vtg = bits_np(Kd), bits_np(Vtd)
    P0 = cfg.P0
    np.testing.assert_array_equal(Kg[:, :P0], K0[:, :P0])
    np.testing.assert_array_equal(Vtg[:, :, :P0], V0[:, :, :P0])
    np.testing.assert_array_equal(Kg[:, P2:], K0[:, P2:])
    np.testing.assert_array_equal(Vtg[:, :, P2:], V0[:, :, P2:])
    assert maxrel(O.from_bf16(Kg[:, P0:P2]), O.from_bf16(Ko[:, P0:P2])) <= 2e-2
    assert maxrel(O.from_bf16(Vtg[:, :, P0:P2].transpose(0, 2, 1)), O.from_bf16(Vo[:, P0:P2])) <= 2e-2


@pytest.mark.parametrize("name", list(EDGES))
def test_edge_loop_parity(dg_ctx, name):
    """Two whole canvases (all steps, commits between them) against the oracle's loop.
    With one canvas position, or three vocabulary ids, a fraction-of-positions cap on
    excused mismatches means nothing, so every mismatch must be excused (cutoff or tie)."""
    from test_gpu_loop import run_both
    s = run_both(dg_ctx, EDGES[name], n_canvas=2)
    assert s["unexcused"] == 0, s


@pytest.mark.parametrize("name", list(EDGES))
def test_edge_sample_tokens_and_confidence(dg_ctx, name):
    """dg_sample (inverse-CDF draw over the whole vocabulary) and dg_confidence at the edge
    shapes; a drawn token may differ only where the oracle's target lies within the
    device's rounding of a cumulative boundary."""
    from gpu_util import sample_excused
    cfg, W, Kp, Vp, Pcap, Wd = setup(name)
    ws = ws_for(cfg, Pcap)
    tgt = di.targets(cfg, 0)
    for k in (0, cfg.N - 1):
        H = di.hidden(cfg, W["E"], 0, k, tgt)
        tau = O.temperature(k, cfg.N)
        ent = torch.empty(cfg.C, dtype=torch.float32, device=DEV)
        am = torch.empty(cfg.C, dtype=torch.int32, device=DEV)
        dg_ctx.logits_entropy(cfg, bf16_dev(H), Wd["E"], tau, ws, ent, am)
        tok = torch.full((cfg.C,), -1, dtype=torch.int32, device=DEV)
        dg_ctx.sample(cfg, ws, 1, 4321 + k, 3, k, tok)
        conf = torch.empty(cfg.C, dtype=torch.float32, device=DEV)
        dg_ctx.confidence(cfg, ws, conf)
        dg_ctx.sync()
        _, _, p_r, _ = O.logits_entropy(H, W["E"], tau)
        np.testing.assert_allclose(conf.cpu().numpy(), p_r.max(axis=1), rtol=2e-5, atol=0)
        ref, margin = O.sample_tokens(p_r, 4321 + k, 3, k, B=1, with_margins=True)
        g = tok.cpu().numpy()
        assert np.all((g >= 0) & (g < cfg.V))
        for i in np.nonzero(g != ref)[0]:
            assert sample_excused(p_r[i], int(ref[i]), float(margin[i])), (k, i, g[i], ref[i])
