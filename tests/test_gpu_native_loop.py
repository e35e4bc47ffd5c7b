"""dg_run_canvas, the canvas loop sequenced inside the library, against CanvasLoop, the same
calls sequenced from Python (needs an MI355X): the entropy rule with argmax draws and the
projection commit, the causal re-encode commit with rotary positions, and the confidence
rule and sampled-token draws. CanvasLoop is held to the oracle's loop by test_gpu_loop, so
byte equality here carries that parity over: the same steps per canvas, the same
committed blocks, and byte-identical caches after chained canvases."""
import numpy as np
import pytest
import torch

import block_ar_canvas_amd as dg
from block_ar_canvas_amd.loop import CanvasLoop
import dg_inputs as di
from gpu_util import DEV, bf16_dev, bits_np, upload_cache, upload_weights

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": di.config("tiny"),
    "ragged": di.Config("ragged", V=5000, d=96, C=100, Hq=6, Hkv=3, hd=32, F=64, P0=77, N=6,
                        alpha_max=8.0, seed=21),
    # two steps and a weak driver: the stop never fires, every canvas ends at the cap
    "cap": di.Config("cap", V=700, d=64, C=40, Hq=2, Hkv=1, hd=32, F=64, P0=30, N=2,
                     alpha_max=1.0, seed=26),
}


@pytest.mark.parametrize("name", list(CASES))
def test_native_loop_matches_python_loop(dg_ctx, name):
    cfg = CASES[name]
    n_canvas = 2
    W = di.weights(cfg)
    Wd = upload_weights(W)
    Pcap = -(-(cfg.P0 + cfg.C * n_canvas) // 8) * 8
    Kp, Vp = di.prefix_kv(cfg, Pcap)
    K1, V1 = upload_cache(Kp, Vp, Pcap)
    K2, V2 = upload_cache(Kp, Vp, Pcap)
    loop = CanvasLoop(dg_ctx, cfg, Wd, K1, V1, cfg.P0, N=cfg.N, seed=cfg.seed)
    ws = torch.empty(dg.workspace_bytes(cfg, Pcap), dtype=torch.uint8, device=DEV)
    lws = torch.empty(dg.loop_workspace_bytes(cfg), dtype=torch.uint8, device=DEV)
    x0 = torch.full((cfg.C,), -1, dtype=torch.int32, device=DEV)
    P2 = cfg.P0
    for c in range(n_canvas):
        tgt = di.targets(cfg, c)
        Hd = [bf16_dev(di.hidden(cfg, W["E"], c, k, tgt)) for k in range(cfg.N)]
        steps1 = loop.run_canvas(c, lambda k: Hd[k])
        dg_ctx.sync()
        x1 = loop.final_tokens(steps1 - 1).cpu().numpy().copy()
        steps2, P2 = dg_ctx.run_canvas(cfg, Wd, K2, V2, P2, lambda k: Hd[k], ws, lws, x0, N=cfg.N,
                                       seed=cfg.seed, canvas=c)
        dg_ctx.sync()
        assert steps2 == steps1, (c, steps1, steps2)
        assert P2 == loop.P
        np.testing.assert_array_equal(x0.cpu().numpy(), x1)
        if name == "cap":
            assert steps2 == cfg.N
    np.testing.assert_array_equal(bits_np(K2), bits_np(K1))
    np.testing.assert_array_equal(bits_np(V2), bits_np(V1))


def test_native_loop_prefill_commit_with_rotary_positions(dg_ctx):
    """The causal re-encode commit with rotary positions: byte-equal to CanvasLoop with the
    same commit over two chained canvases (the second attends the first's prefilled rows)."""
    cfg = CASES["ragged"]
    n_canvas = 2
    W = di.weights(cfg)
    Wd = upload_weights(W)
    Pcap = -(-(cfg.P0 + cfg.C * n_canvas) // 8) * 8
    Kp, Vp = di.prefix_kv(cfg, Pcap)
    K1, V1 = upload_cache(Kp, Vp, Pcap)
    K2, V2 = upload_cache(Kp, Vp, Pcap)
    try:
        loop = CanvasLoop(dg_ctx, cfg, Wd, K1, V1, cfg.P0, N=cfg.N, seed=cfg.seed, commit="prefill",
                          rope_base=10000.0)
        ws = torch.empty(dg.workspace_bytes(cfg, Pcap), dtype=torch.uint8, device=DEV)
        lws = torch.empty(dg.loop_workspace_bytes(cfg), dtype=torch.uint8, device=DEV)
        x0 = torch.full((cfg.C,), -1, dtype=torch.int32, device=DEV)
        P2 = cfg.P0
        for c in range(n_canvas):
            tgt = di.targets(cfg, c)
            Hd = [bf16_dev(di.hidden(cfg, W["E"], c, k, tgt)) for k in range(cfg.N)]
            steps1 = loop.run_canvas(c, lambda k: Hd[k])
            dg_ctx.sync()
            x1 = loop.final_tokens(steps1 - 1).cpu().numpy().copy()
            steps2, P2 = dg_ctx.run_canvas(cfg, Wd, K2, V2, P2, lambda k: Hd[k], ws, lws, x0, N=cfg.N,
                                           seed=cfg.seed, canvas=c, commit="prefill")
            dg_ctx.sync()
            assert steps2 == steps1, (c, steps1, steps2)
            assert P2 == loop.P
            np.testing.assert_array_equal(x0.cpu().numpy(), x1)
        np.testing.assert_array_equal(bits_np(K2), bits_np(K1))
        np.testing.assert_array_equal(bits_np(V2), bits_np(V1))
    finally:
        dg_ctx.set_rope(0.0)


VARIANTS = [("confidence", "argmax"), ("entropy", "sample"), ("confidence", "sample")]


@pytest.mark.parametrize("rule,draw", VARIANTS, ids=[f"{r}-{d}" for r, d in VARIANTS])
def test_native_loop_rules_and_draws(dg_ctx, rule, draw):
    """The confidence rule and sampled-token draws: byte-equal to CanvasLoop with the same
    rule and draw over two chained canvases at the ragged shape (steps, committed blocks,
    whole caches)."""
    cfg = CASES["ragged"]
    n_canvas = 2
    W = di.weights(cfg)
    Wd = upload_weights(W)
    Pcap = -(-(cfg.P0 + cfg.C * n_canvas) // 8) * 8
    Kp, Vp = di.prefix_kv(cfg, Pcap)
    K1, V1 = upload_cache(Kp, Vp, Pcap)
    K2, V2 = upload_cache(Kp, Vp, Pcap)
    loop = CanvasLoop(dg_ctx, cfg, Wd, K1, V1, cfg.P0, N=cfg.N, seed=cfg.seed, rule=rule, draw=draw)
    ws = torch.empty(dg.workspace_bytes(cfg, Pcap), dtype=torch.uint8, device=DEV)
    lws = torch.empty(dg.loop_workspace_bytes(cfg), dtype=torch.uint8, device=DEV)
    x0 = torch.full((cfg.C,), -1, dtype=torch.int32, device=DEV)
    P2 = cfg.P0
    for c in range(n_canvas):
        tgt = di.targets(cfg, c)
        Hd = [bf16_dev(di.hidden(cfg, W["E"], c, k, tgt)) for k in range(cfg.N)]
        steps1 = loop.run_canvas(c, lambda k: Hd[k])
        dg_ctx.sync()
        x1 = loop.final_tokens(steps1 - 1).cpu().numpy().copy()
        steps2, P2 = dg_ctx.run_canvas(cfg, Wd, K2, V2, P2, lambda k: Hd[k], ws, lws, x0, N=cfg.N,
                                       seed=cfg.seed, canvas=c, rule=rule, draw=draw)
        dg_ctx.sync()
        assert steps2 == steps1, (c, steps1, steps2)
        assert P2 == loop.P
        np.testing.assert_array_equal(x0.cpu().numpy(), x1)
    np.testing.assert_array_equal(bits_np(K2), bits_np(K1))
    np.testing.assert_array_equal(bits_np(V2), bits_np(V1))


def test_native_loop_refusals(dg_ctx):
    cfg = CASES["tiny"]
    W = di.weights(cfg)
    Wd = upload_weights(W)
    Pcap = -(-(cfg.P0 + cfg.C) // 8) * 8
    Kp, Vp = di.prefix_kv(cfg, Pcap)
    K, V = upload_cache(Kp, Vp, Pcap)
    K0, V0 = bits_np(K).copy(), bits_np(V).copy()
    ws = torch.empty(dg.workspace_bytes(cfg, Pcap), dtype=torch.uint8, device=DEV)
    lws = torch.zeros(dg.loop_workspace_bytes(cfg), dtype=torch.uint8, device=DEV)
    x0 = torch.full((cfg.C,), -1, dtype=torch.int32, device=DEV)
    Hd = [bf16_dev(di.hidden(cfg, W["E"], 0, k, di.targets(cfg, 0))) for k in range(cfg.N)]
    # no room for the commit: refused before anything is enqueued
    with pytest.raises(dg.DGError) as ei:
        dg_ctx.run_canvas(cfg, Wd, K, V, Pcap - cfg.C + 1, lambda k: Hd[k], ws, lws, x0, N=cfg.N,
                          seed=cfg.seed, canvas=0)
    assert ei.value.name == "DG_ERR_CAPACITY"
    # a schedule with a non-positive temperature, a step cap below 1, an unknown commit
    for kw in ({"commit": "append"}, {"rule": "random"}, {"draw": "topp"}):
        with pytest.raises(ValueError):
            dg_ctx.run_canvas(cfg, Wd, K, V, cfg.P0, lambda k: Hd[k], ws, lws, x0, N=cfg.N, seed=cfg.seed,
                              canvas=0, **kw)
    for kw in ({"tau1": 0.0}, {"N": 0}):
        args = {"N": cfg.N, "seed": cfg.seed, "canvas": 0, **kw}
        with pytest.raises(dg.DGError) as ei:
            dg_ctx.run_canvas(cfg, Wd, K, V, cfg.P0, lambda k: Hd[k], ws, lws, x0, **args)
        assert ei.value.name == "DG_ERR_RANGE"
    dg_ctx.sync()
    assert int(lws.sum().item()) == 0 and int(x0.min().item()) == -1
    np.testing.assert_array_equal(bits_np(K), K0)
    np.testing.assert_array_equal(bits_np(V), V0)
    # a hidden source that fails at step 1 ends the loop with its own error; the steps
    # already enqueued stay ordered on the stream
    def bad(k):
        if k >= 1:
            raise ValueError("no hidden state")
        return Hd[k]
    with pytest.raises(ValueError):
        dg_ctx.run_canvas(cfg, Wd, K, V, cfg.P0, bad, ws, lws, x0, N=cfg.N, seed=cfg.seed, canvas=0)
    dg_ctx.sync()
    np.testing.assert_array_equal(bits_np(K), K0)
