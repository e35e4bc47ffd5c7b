"""Failure paths and resumption of the HIP path (needs an MI355X).

Every condition is forced from the host with data or arguments; every kernel still runs
to completion. A block may not settle within the step budget and the method gives no
guarantee (tutorial chapter "DiffusionGemma", KV-cache write timing), so the library's
error reporting and its behaviour on bad data are part of the contract:
  * a position with non-finite hidden states gets a NaN entropy, is never accepted,
    blocks the stop, contributes z = 0, leaves every other position in parity, and
    dg_sync reports DG_ERR_NONFINITE until the status is cleared;
  * a token id outside [0, V) is read as id 0 and dg_sync reports DG_ERR_RANGE;
  * a commit over capacity is refused before anything is enqueued (cache unchanged);
  * NULL and misaligned pointers are refused before anything is enqueued;
  * a loop restarted from a saved state (canvas tokens, z, previous argmax, step)
    reproduces the remaining steps bit for bit.
"""
import ctypes

import numpy as np
import pytest
import torch

import block_ar_canvas_amd as dg
import dg_inputs as di
import oracle as O
from block_ar_canvas_amd.loop import CanvasLoop
from gpu_util import (DEV, bf16_dev, bits_np, cache_logical, i32_dev, maxrel_rows, upload_cache,
                      upload_weights)

pytestmark = pytest.mark.gpu

RAGGED = di.Config("ragged_fail", V=5000, d=96, C=100, Hq=6, Hkv=3, hd=32, F=64, P0=77, N=6,
                   alpha_max=9.0, seed=26)
NAN_ROW = 37


def setup(cfg):
    W = di.weights(cfg)
    Pcap = -(-(cfg.P0 + 2 * cfg.C) // 8) * 8
    Kp, Vp = di.prefix_kv(cfg, Pcap)
    return W, upload_weights(W), Kp, Vp, Pcap


def sharp_hidden(cfg, W, nan_row=None):
    # 200 E[target]: entropies ~0 and a stable argmax, so the stop fires at step 1
    tgt = di.targets(cfg, 0)
    H = di.f32_to_bf16_bits(200.0 * di.bf16_bits_to_f32(W["E"][tgt]))
    if nan_row is not None:
        H = H.copy()
        H[nan_row] = 0x7FC0                             # bf16 quiet NaN
    return H


def two_steps(ctx, cfg, Wd, Kd, Vtd, H):
    """Steps 0 and 1 of canvas 0 on constant hidden states; returns per-step host copies."""
    loop = CanvasLoop(ctx, cfg, Wd, Kd, Vtd, cfg.P0, N=cfg.N, seed=cfg.seed)
    loop.init_canvas(0)
    Hd = bf16_dev(H)
    out = []
    for k in range(2):
        loop.step(k, Hd)
        out.append({"entropy": loop.entropy.cpu().numpy().copy(),
                    "argmax": loop.argmax[k & 1].cpu().numpy().copy(),
                    "accept": loop.accept.cpu().numpy().copy(),
                    "tokens": loop.tokens.cpu().numpy().copy(),
                    "z": bits_np(loop.z), "flag": loop.wait_flag(k)})
    return out


def test_nonfinite_row_is_isolated_and_reported(dg_ctx):
    cfg = RAGGED
    W, Wd, Kp, Vp, Pcap = setup(cfg)
    Kd, Vtd = upload_cache(Kp, Vp, Pcap)
    # control: without the bad row the sharp driver stops at step 1
    good = two_steps(dg_ctx, cfg, Wd, Kd, Vtd, sharp_hidden(cfg, W))
    dg_ctx.sync()
    assert [g["flag"] for g in good] == [O.STOP_GO, O.STOP_STOP]
    H = sharp_hidden(cfg, W, NAN_ROW)
    bad = two_steps(dg_ctx, cfg, Wd, Kd, Vtd, H)
    with pytest.raises(dg.DGError) as ei:
        dg_ctx.sync()
    assert ei.value.name == "DG_ERR_NONFINITE"
    dg_ctx.clear_status()
    dg_ctx.sync()                                       # cleared: no error any more
    others = np.arange(cfg.C) != NAN_ROW
    for k, g in enumerate(bad):
        ent_r, am_r, p_r, _ = O.logits_entropy(H, W["E"], O.temperature(k, cfg.N))
        z_r, _ = O.selfcond(p_r[others], W["E"], W["W1"], W["W2"])
        assert np.isnan(g["entropy"][NAN_ROW]) and g["argmax"][NAN_ROW] == 0
        assert g["accept"][NAN_ROW] == 0                 # never accepted
        assert np.max(np.abs(g["entropy"][others] - ent_r[others])) <= 1e-3
        np.testing.assert_array_equal(g["argmax"][others], am_r[others])
        # acceptance of the rest: the fixed-point rule on the device's own entropies
        acc_o, _ = O.entropy_accept(g["entropy"][None], 0.1)
        np.testing.assert_array_equal(g["accept"], acc_o[0])
        assert np.all(g["z"][NAN_ROW] == 0)              # flushed position: s = 0, z = 0
        assert maxrel_rows(O.from_bf16(g["z"][others]), O.from_bf16(z_r)) <= 2e-2
    assert [g["flag"] for g in bad] == [O.STOP_GO, O.STOP_GO]   # the NaN entropy blocks the stop
    assert int(O.stop_test(bad[1]["entropy"][None], bad[1]["argmax"][None], bad[0]["argmax"][None],
                           0.005, 1, cfg.N)[0]) == O.STOP_GO


def test_token_out_of_range_reads_as_zero_and_is_reported(dg_ctx):
    cfg = RAGGED
    W, Wd, Kp, Vp, Pcap = setup(cfg)
    Kd, Vtd = upload_cache(Kp, Vp, Pcap)
    rng = np.random.default_rng(7)
    tok = rng.integers(0, cfg.V, cfg.C).astype(np.int32)
    tok[5], tok[60] = cfg.V, -3
    z = di.f32_to_bf16_bits(rng.standard_normal((cfg.C, cfg.d)).astype(np.float32) * 0.3)
    tok0 = tok.copy()
    tok0[[5, 60]] = 0
    ws = torch.empty(dg.workspace_bytes(cfg, Pcap), dtype=torch.uint8, device=DEV)
    for zz in (z, None):                                 # the xgather path and the gather GEMM
        A = torch.empty(cfg.C, cfg.d, dtype=torch.bfloat16, device=DEV)
        dg_ctx.canvas_attn(cfg, i32_dev(tok), None if zz is None else bf16_dev(zz), Wd["E"], Wd["Wq"],
                           Wd["Wk"], Wd["Wv"], Wd["Wo"], Kd, Vtd, cfg.P0, ws, A)
        with pytest.raises(dg.DGError) as ei:
            dg_ctx.sync()
        assert ei.value.name == "DG_ERR_RANGE"
        dg_ctx.clear_status()
        A_r, _ = O.canvas_attn(tok0, zz, W["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], Kp, Vp, cfg.P0,
                               cfg.Hq, cfg.Hkv, cfg.hd)
        assert maxrel_rows(O.from_bf16(bits_np(A)), O.from_bf16(A_r)) <= 2e-2
    # the commit reads the ids the same way
    P2 = dg_ctx.commit_kv(cfg, i32_dev(tok), Wd["E"], Wd["Wk"], Wd["Wv"], Kd, Vtd, cfg.P0)
    with pytest.raises(dg.DGError) as ei:
        dg_ctx.sync()
    assert ei.value.name == "DG_ERR_RANGE"
    dg_ctx.clear_status()
    Kg, Vg = cache_logical(Kd, Vtd)
    K_r, V_r = Kp.copy(), Vp.copy()
    O.commit_kv(tok0, W["E"], W["Wk"], W["Wv"], K_r, V_r, cfg.P0, cfg.Hkv, cfg.hd)
    assert maxrel_rows(O.from_bf16(Kg[:, cfg.P0:P2]), O.from_bf16(K_r[:, cfg.P0:P2])) <= 2e-2


def test_commit_over_capacity_writes_nothing(dg_ctx):
    cfg = RAGGED
    W, Wd, Kp, Vp, _ = setup(cfg)
    Pcap = -(-(cfg.P0 + cfg.C) // 8) * 8                # room for one block only
    Kd, Vtd = upload_cache(Kp[:, :cfg.P0], Vp[:, :cfg.P0], Pcap)
    tok = i32_dev(np.arange(cfg.C) % cfg.V)
    ws = torch.empty(dg.workspace_bytes(cfg, Pcap), dtype=torch.uint8, device=DEV)
    A = torch.empty(cfg.C, cfg.d, dtype=torch.bfloat16, device=DEV)
    K0, V0 = bits_np(Kd), bits_np(Vtd)
    P_full = Pcap - cfg.C + 1                           # P + C > Pcap by one row
    with pytest.raises(dg.DGError) as ei:
        dg_ctx.commit_kv(cfg, tok, Wd["E"], Wd["Wk"], Wd["Wv"], Kd, Vtd, P_full)
    assert ei.value.name == "DG_ERR_CAPACITY"
    with pytest.raises(dg.DGError) as ei:
        dg_ctx.prefill_block(cfg, tok, Wd["E"], Wd["Wq"], Wd["Wk"], Wd["Wv"], Wd["Wo"], Kd, Vtd, P_full,
                             ws, A)
    assert ei.value.name == "DG_ERR_CAPACITY"
    dg_ctx.sync()
    assert bits_np(Kd).tobytes() == K0.tobytes() and bits_np(Vtd).tobytes() == V0.tobytes()


def test_null_and_misaligned_pointers_enqueue_nothing(dg_ctx):
    cfg = RAGGED
    W, Wd, Kp, Vp, Pcap = setup(cfg)
    Kd, Vtd = upload_cache(Kp, Vp, Pcap)
    lib, h = dg_ctx._lib, dg_ctx._h
    dims = dg.Dims.of(cfg)
    ws = torch.empty(dg.workspace_bytes(cfg, Pcap) + 64, dtype=torch.uint8, device=DEV)
    tok = i32_dev(np.arange(cfg.C) % cfg.V)
    A = torch.full((cfg.C, cfg.d), 7.0, dtype=torch.bfloat16, device=DEV)
    ent = torch.full((cfg.C,), -5.0, dtype=torch.float32, device=DEV)
    am = torch.full((cfg.C,), -5, dtype=torch.int32, device=DEV)
    H = bf16_dev(di.hidden(cfg, W["E"], 0, 3))
    p = lambda t: t.data_ptr()
    args = dict(tokens=p(tok), z=None, E=p(Wd["E"]), Wq=p(Wd["Wq"]), Wk=p(Wd["Wk"]), Wv=p(Wd["Wv"]),
                Wo=p(Wd["Wo"]), Kp=p(Kd), Vt=p(Vtd), ws=p(ws), A=p(A))

    def attn(**kw):
        a = dict(args, **kw)
        return lib.dg_canvas_attn(h, ctypes.byref(dims), a["tokens"], a["z"], a["E"], a["Wq"], a["Wk"],
                                  a["Wv"], a["Wo"], a["Kp"], a["Vt"], cfg.P0, Pcap, a["ws"], a["A"])

    for name in ("tokens", "E", "Wq", "Wk", "Wv", "Wo", "Kp", "Vt", "ws", "A"):
        assert attn(**{name: None}) == 1, name           # DG_ERR_NULL
        assert attn(**{name: args[name] + 2}) == 3, name  # DG_ERR_ALIGN
    assert attn(z=p(A) + 2) == 3
    assert lib.dg_canvas_attn_static(h, ctypes.byref(dims), p(tok), None, p(Wd["E"]), None, p(Wd["Wk"]),
                                     p(Wd["Wv"]), p(Wd["Wo"]), p(Kd), p(Vtd), cfg.P0, Pcap, p(A)) == 1
    assert lib.dg_logits_entropy(h, ctypes.byref(dims), None, p(Wd["E"]), ctypes.c_float(0.8), p(ws),
                                 p(ent), p(am)) == 1
    assert lib.dg_logits_entropy(h, ctypes.byref(dims), p(H) + 2, p(Wd["E"]), ctypes.c_float(0.8), p(ws),
                                 p(ent), p(am)) == 3
    assert lib.dg_logits_entropy(h, ctypes.byref(dims), p(H), p(Wd["E"]), ctypes.c_float(0.0), p(ws),
                                 p(ent), p(am)) == 4  # tau <= 0: DG_ERR_RANGE
    assert lib.dg_selfcond(h, ctypes.byref(dims), p(ws), p(Wd["E"]), p(Wd["W1"]), None, p(A)) == 1
    assert lib.dg_entropy_accept(h, 1, cfg.C, None, ctypes.c_float(0.1), p(am), p(am)) == 1
    assert lib.dg_stop_test(h, 1, cfg.C, p(ent), None, None, ctypes.c_float(0.005), 1, cfg.N, p(am)) == 1
    assert lib.dg_renoise(h, 1, cfg.C, cfg.V, None, p(am), ctypes.c_uint64(1), 0, 0, p(tok)) == 1
    assert lib.dg_canvas_attn(None, ctypes.byref(dims), *[None] * 9, 0, 0, None, None) == 1
    dg_ctx.sync()
    # nothing ran: every output still holds its fill value
    assert torch.all(A == 7.0) and torch.all(ent == -5.0) and torch.all(am == -5)


def test_resume_from_saved_state_is_bit_exact(dg_ctx):
    cfg = RAGGED
    W, Wd, Kp, Vp, Pcap = setup(cfg)
    tgt = di.targets(cfg, 0)
    Hd = [bf16_dev(di.hidden(cfg, W["E"], 0, k, tgt)) for k in range(cfg.N)]
    k_save = 3

    def run(loop, k_from, state=None):
        if state is None:
            loop.init_canvas(0)
        else:                                           # restore (tokens, z, previous argmax)
            loop.canvas = 0
            loop.tokens.copy_(state[0])
            loop.z.copy_(state[1])
            loop.argmax[(k_from - 1) & 1].copy_(state[2])
        out, saved = [], None
        for k in range(k_from, cfg.N):
            if k == k_save and state is None:
                saved = (loop.tokens.clone(), loop.z.clone(), loop.argmax[(k - 1) & 1].clone())
            loop.step(k, Hd[k])
            out.append([t.cpu().numpy().tobytes() for t in
                        (loop.entropy, loop.argmax[k & 1], loop.accept, loop.tokens,
                         loop.z.view(torch.int16), loop.A.view(torch.int16))] + [loop.wait_flag(k)])
        return out, saved

    Kd, Vtd = upload_cache(Kp, Vp, Pcap)
    full, saved = run(CanvasLoop(dg_ctx, cfg, Wd, Kd, Vtd, cfg.P0, N=cfg.N, seed=cfg.seed), 0)
    Kd2, Vtd2 = upload_cache(Kp, Vp, Pcap)
    resumed, _ = run(CanvasLoop(dg_ctx, cfg, Wd, Kd2, Vtd2, cfg.P0, N=cfg.N, seed=cfg.seed), k_save, saved)
    dg_ctx.sync()
    assert resumed == full[k_save:]
