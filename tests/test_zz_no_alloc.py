"""dg_canvas_attn_static, the allocation-free variant of dg_canvas_attn (needs an MI355X).

It runs the same kernels on the library's static per-device scratch instead of a
caller's workspace, so its output must equal dg_canvas_attn's bit for bit, and both
stay within the oracle's bar (A within 2e-2 largest per-row relative error). Two calls
in a row, the second with a smaller input, check that nothing left in the shared
scratch by the first call leaks into the second.
"""
import numpy as np
import pytest
import torch

import block_ar_canvas_amd as dg
import dg_inputs as di
import oracle as O
from gpu_util import DEV, bf16_dev, bits_np, i32_dev, maxrel_rows, upload_cache, upload_weights

pytestmark = pytest.mark.gpu

SMALL = di.config(1)                                 # V 32768, d 1024, C 256, prefix 2048
RAGGED = di.Config("ragged_static", V=5000, d=96, C=100, Hq=6, Hkv=3, hd=32, F=64, P0=77, N=6,
                   alpha_max=8.0, seed=25)


def inputs(cfg, seed):
    W = di.weights(cfg)
    Pcap = -(-(cfg.P0 + cfg.C) // 8) * 8
    Kp, Vp = di.prefix_kv(cfg, Pcap)
    rng = np.random.default_rng(seed)
    tok = rng.integers(0, cfg.V, cfg.C).astype(np.int32)
    z = di.f32_to_bf16_bits(rng.standard_normal((cfg.C, cfg.d)).astype(np.float32) * 0.3)
    return W, Kp, Vp, Pcap, tok, z


def test_static_scratch_matches_workspace_call(dg_ctx):
    for cfg, seed in ((SMALL, 71), (RAGGED, 72)):     # the second call is smaller
        W, Kp, Vp, Pcap, tok, z = inputs(cfg, seed)
        Wd = upload_weights(W)
        Kd, Vtd = upload_cache(Kp, Vp, Pcap)
        td, zd = i32_dev(tok), bf16_dev(z)
        A_static = torch.full((cfg.C, cfg.d), float("nan"), dtype=torch.bfloat16, device=DEV)
        dg_ctx.canvas_attn_static(cfg, td, zd, Wd["E"], Wd["Wq"], Wd["Wk"], Wd["Wv"], Wd["Wo"],
                                  Kd, Vtd, cfg.P0, A_static)
        ws = torch.empty(dg.workspace_bytes(cfg, Pcap), dtype=torch.uint8, device=DEV)
        A_ws = torch.empty(cfg.C, cfg.d, dtype=torch.bfloat16, device=DEV)
        dg_ctx.canvas_attn(cfg, td, zd, Wd["E"], Wd["Wq"], Wd["Wk"], Wd["Wv"], Wd["Wo"], Kd, Vtd,
                           cfg.P0, ws, A_ws)
        dg_ctx.sync()
        assert torch.equal(A_static.view(torch.int16), A_ws.view(torch.int16)), cfg.name
        A_r, _ = O.canvas_attn(tok, z, W["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], Kp, Vp, cfg.P0,
                               cfg.Hq, cfg.Hkv, cfg.hd)
        assert maxrel_rows(O.from_bf16(bits_np(A_static)), O.from_bf16(A_r)) <= 2e-2, cfg.name


def test_static_scratch_without_selfcond_term_and_empty_prefix(dg_ctx):
    cfg = RAGGED
    W, Kp, Vp, Pcap, tok, _ = inputs(cfg, 73)
    Wd = upload_weights(W)
    Kd, Vtd = upload_cache(Kp, Vp, Pcap)
    A = torch.empty(cfg.C, cfg.d, dtype=torch.bfloat16, device=DEV)
    dg_ctx.canvas_attn_static(cfg, i32_dev(tok), None, Wd["E"], Wd["Wq"], Wd["Wk"], Wd["Wv"],
                              Wd["Wo"], Kd, Vtd, 0, A)
    dg_ctx.sync()
    A_r, _ = O.canvas_attn(tok, None, W["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], Kp, Vp, 0,
                           cfg.Hq, cfg.Hkv, cfg.hd)
    assert maxrel_rows(O.from_bf16(bits_np(A)), O.from_bf16(A_r)) <= 2e-2


def test_static_scratch_rejects_dims_beyond_its_size(dg_ctx):
    # 1024 positions over 64 query heads of 128 at d 4096: about 60 MiB of scratch;
    # the call is refused on the host before anything is enqueued
    dims = dg.Dims(512, 4096, 1024, 64, 8, 128, 64)
    dev = lambda n, dt: torch.zeros(n, dtype=dt, device=DEV)
    tok = dev(1024, torch.int32)
    E = dev(512 * 4096, torch.bfloat16)
    Wq = dev(8192 * 4096, torch.bfloat16)   # [Hq*hd, d]; also passed as Wo [d, Hq*hd]
    Wkv = dev(1024 * 4096, torch.bfloat16)
    A = dev(1024 * 4096, torch.bfloat16)
    Kd = torch.zeros(8, 8, 128, dtype=torch.bfloat16, device=DEV)
    Vtd = torch.zeros(8, 128, 8, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(dg.DGError) as ei:
        dg_ctx.canvas_attn_static(dims, tok, None, E, Wq, Wkv, Wkv, Wq, Kd, Vtd, 0, A)
    assert ei.value.name == "DG_ERR_CAPACITY" and "static scratch" in str(ei.value)
    dg_ctx.sync()
