"""Two contexts on one device, each on its own stream, with their calls interleaved
(needs an MI355X). Each context keeps its own state (the sampler head -> self-conditioning
hand-off in its workspace, the MoE FFN's second stream and events, the sticky status), so
every output must be byte-identical to the same calls made on one context alone."""
import numpy as np
import pytest
import torch

import block_ar_canvas_amd as dg
import dg_inputs as di
import oracle as O
from gpu_util import DEV, bf16_dev, bits_np, upload_weights

pytestmark = pytest.mark.gpu

CFG = di.Config("ctx2", V=5000, d=96, C=100, Hq=6, Hkv=3, hd=32, F=64, P0=77, N=6,
                alpha_max=8.0, seed=41)


def head_and_selfcond(ctx, cfg, Wd, H, tau, ws):
    ent = torch.empty(cfg.C, dtype=torch.float32, device=DEV)
    am = torch.empty(cfg.C, dtype=torch.int32, device=DEV)
    z = torch.empty(cfg.C, cfg.d, dtype=torch.bfloat16, device=DEV)
    ctx.logits_entropy(cfg, bf16_dev(H), Wd["E"], tau, ws, ent, am)
    return ent, am, z


def test_interleaved_contexts_match_one_context(dg_ctx):
    cfg = CFG
    W = di.weights(cfg)
    Wd = upload_weights(W)
    tgt = di.targets(cfg, 0)
    Hs = [di.hidden(cfg, W["E"], 0, k, tgt) for k in (0, cfg.N - 1)]
    taus = [O.temperature(k, cfg.N) for k in (0, cfg.N - 1)]
    nbytes = dg.workspace_bytes(cfg, 0)

    # reference: both inputs on the session context alone, one after the other
    ref = []
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    for H, tau in zip(Hs, taus):
        ent, am, z = head_and_selfcond(dg_ctx, cfg, Wd, H, tau, ws)
        dg_ctx.selfcond(cfg, ws, Wd["E"], Wd["W1"], Wd["W2"], z)
        dg_ctx.sync()
        ref.append((ent.cpu().numpy().copy(), am.cpu().numpy().copy(), bits_np(z).copy()))

    # two contexts on two streams: both sampler heads enqueued before either
    # self-conditioning call, each reading its own context's workspace
    side = torch.cuda.Stream(device=DEV)
    ctx2 = dg.Context(0, stream=side)
    try:
        wss = [torch.empty(nbytes, dtype=torch.uint8, device=DEV) for _ in range(2)]
        ctxs = [dg_ctx, ctx2]
        outs = [head_and_selfcond(c, cfg, Wd, H, tau, w) for c, H, tau, w in zip(ctxs, Hs, taus, wss)]
        for c, w, (_, _, z) in zip(ctxs, wss, outs):
            c.selfcond(cfg, w, Wd["E"], Wd["W1"], Wd["W2"], z)
        dg_ctx.sync()
        ctx2.sync()
        for (ent, am, z), (ent_r, am_r, z_r) in zip(outs, ref):
            np.testing.assert_array_equal(ent.cpu().numpy(), ent_r)
            np.testing.assert_array_equal(am.cpu().numpy(), am_r)
            np.testing.assert_array_equal(bits_np(z), z_r)
    finally:
        ctx2.close()


def test_moe_ffn_on_two_contexts_matches_one(dg_ctx):
    C, d, E, K, Fe, Fs = 64, 128, 16, 4, 64, 64
    inp = di.moe_inputs(C, d, E, K, Fe, Fs, seed=42)
    X2 = di.moe_inputs(C, d, E, K, Fe, Fs, seed=43)["X"]
    md = dg.MoeDims(d, E, K, Fe, Fs)
    dv = {k: bf16_dev(v) for k, v in inp.items()}
    Xs = [dv["X"], bf16_dev(X2)]
    nbytes = dg.moe_workspace_bytes(md, C)

    ref = []
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    for X in Xs:
        Y = torch.empty(C, d, dtype=torch.bfloat16, device=DEV)
        dg_ctx.moe_ffn(md, X, dv["Wr"], dv["W1"], dv["W2"], dv["W1s"], dv["W2s"], ws, Y, None)
        dg_ctx.sync()
        ref.append(bits_np(Y).copy())

    ctx2 = dg.Context(0, stream=torch.cuda.Stream(device=DEV))
    try:
        ctxs = [dg_ctx, ctx2]
        wss = [torch.empty(nbytes, dtype=torch.uint8, device=DEV) for _ in range(2)]
        Ys = [torch.empty(C, d, dtype=torch.bfloat16, device=DEV) for _ in range(2)]
        for c, X, w, Y in zip(ctxs, Xs, wss, Ys):
            c.moe_ffn(md, X, dv["Wr"], dv["W1"], dv["W2"], dv["W1s"], dv["W2s"], w, Y, None)
        dg_ctx.sync()
        ctx2.sync()
        for Y, Yr in zip(Ys, ref):
            np.testing.assert_array_equal(bits_np(Y), Yr)
    finally:
        ctx2.close()
