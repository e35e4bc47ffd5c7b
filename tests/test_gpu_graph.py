"""A whole canvas captured in a HIP graph and replayed (needs an MI355X).

CanvasLoop.enqueue_canvas_fixed enqueues init, every step and the commit with no host
wait, so the sequence can be captured. Each replay must reproduce the eagerly enqueued
canvas bit for bit (tokens, z, A, entropies, argmax, acceptance and the committed K/V
rows), with the program's own eager library work and synchronizations between replays.
None of the captured calls records a memset node: every buffer is written by kernels.
"""
import numpy as np
import pytest
import torch

import block_ar_canvas_amd as dg
import dg_inputs as di
from block_ar_canvas_amd.loop import CanvasLoop
from gpu_util import DEV, bf16_dev, bits_np, upload_cache, upload_weights

pytestmark = pytest.mark.gpu

RAGGED = di.Config("ragged_graph", V=5000, d=96, C=100, Hq=6, Hkv=3, hd=32, F=64, P0=77, N=6,
                   alpha_max=9.0, seed=27)


def snapshot(loop):
    k = loop.N - 1
    Kg = bits_np(loop.Kp)[:, loop.P - loop.dims.C:loop.P]
    Vg = bits_np(loop.Vt)[:, :, loop.P - loop.dims.C:loop.P]
    return [t.cpu().numpy().tobytes() for t in
            (loop.tokens, loop.z.view(torch.int16), loop.A.view(torch.int16), loop.entropy,
             loop.argmax[k & 1], loop.accept)] + [Kg.tobytes(), Vg.tobytes()]


@pytest.mark.parametrize("cfg", [di.config(0), RAGGED], ids=["tiny", "ragged"])
def test_canvas_graph_replays_match_eager(cfg):
    W = di.weights(cfg)
    Pcap = -(-(cfg.P0 + cfg.C) // 8) * 8
    Kp, Vp = di.prefix_kv(cfg, Pcap)
    Wd = upload_weights(W)
    Kd, Vtd = upload_cache(Kp, Vp, Pcap)
    tgt = di.targets(cfg, 0)
    Hd = [bf16_dev(di.hidden(cfg, W["E"], 0, k, tgt)) for k in range(cfg.N)]
    s = torch.cuda.Stream()
    ctx = dg.Context(0, stream=s)
    loop = CanvasLoop(ctx, cfg, Wd, Kd, Vtd, cfg.P0, N=cfg.N, seed=cfg.seed)
    with torch.cuda.stream(s):
        loop.enqueue_canvas_fixed(5, lambda k: Hd[k])      # eager reference
    ctx.sync()
    ref = snapshot(loop)
    loop.P = cfg.P0
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        loop.enqueue_canvas_fixed(5, lambda k: Hd[k])
    loop.P = cfg.P0 + cfg.C                              # where the captured commit writes
    # eager work of the program between replays: another sampler-head call on its own buffers
    ws2 = torch.empty(dg.workspace_bytes(cfg, Pcap), dtype=torch.uint8, device=DEV)
    ent2 = torch.empty(cfg.C, dtype=torch.float32, device=DEV)
    am2 = torch.empty(cfg.C, dtype=torch.int32, device=DEV)
    for rep in range(3):
        with torch.cuda.stream(s):                       # clobber the outputs first
            for t in (loop.tokens, loop.entropy, loop.argmax[0], loop.argmax[1]):
                t.fill_(-7)
            loop.z.fill_(3.0)
            loop.A.fill_(3.0)
            Kd[:, cfg.P0:cfg.P0 + cfg.C].fill_(0.0)         # the rows the commit writes
            Vtd[:, :, cfg.P0:cfg.P0 + cfg.C].fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert snapshot(loop) == ref, rep
        with torch.cuda.stream(s):
            ctx.logits_entropy(cfg, Hd[rep], Wd["E"], 0.5, ws2, ent2, am2)
        ctx.sync()
    ctx.close()
