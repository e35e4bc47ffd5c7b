"""Parity of the batched lockstep loop against the oracle (needs an MI355X).

BatchLoop denoises B canvases together, one per request, each request with its own
prefix KV cache; the sampler head and self-conditioning see all B*C positions as one
set of columns, and acceptance, renoise and the stop test run with B segments. The
oracle runs every canvas on its own (same canvas id, same request prefix, same driver
states), so these tests also check that batching couples nothing across canvases.
Bars are those of the single-canvas loop test: tokens agree at >= 99.9% of positions
with every mismatch excused by a near-cutoff entropy or a near-tie argmax, entropies
within 1e-3 nats, A and z within 2e-2 max relative error, identical stop flags, and the
committed cache rows within 2e-2 with the prefix rows untouched.
"""
import numpy as np
import pytest
import torch

import dg_inputs as di
import oracle as O
from block_ar_canvas_amd.loop import BatchLoop
from gpu_util import bf16_dev, bits_np, cache_logical, maxrel, maxrel_rows, near_tie, upload_cache, upload_weights
from test_gpu_loop import cutoff_confidence, cutoff_entropy

pytestmark = pytest.mark.gpu

# B * C > 256 in both cases, so the vocabulary-wide kernels run several canvas blocks:
# "wide" with a tile count divisible by 8 and 8 self-conditioning splits (the mappings
# that keep a tile's or a split's canvas blocks on one XCD), "ragged" with neither.
WIDE = di.config(1).with_(name="batch_wide", N=6, seed=31)
RAGGED = di.Config("batch_ragged", V=5000, d=96, C=100, Hq=6, Hkv=3, hd=32, F=64, P0=77, N=8,
                   alpha_max=9.0, seed=32)


def run_batch_both(dg_ctx, cfg, B, batch=1, rule="entropy"):
    W = di.weights(cfg)
    Pcap = -(-(cfg.P0 + cfg.C) // 8) * 8
    Wd = upload_weights(W)
    host, caches = [], []
    for r in range(B):
        Kp, Vp = di.prefix_kv(cfg, Pcap, request=r)
        Kd, Vtd = upload_cache(Kp, Vp, Pcap)
        host.append([Kp, Vp])
        caches.append((Kd, Vtd, cfg.P0))
    loop = BatchLoop(dg_ctx, cfg, Wd, caches, N=cfg.N, seed=cfg.seed, rule=rule)
    ids = [batch * B + i for i in range(B)]
    Hs = [[di.hidden(cfg, W["E"], c, k, di.targets(cfg, c)) for k in range(cfg.N)] for c in ids]
    Hd = [bf16_dev(np.concatenate([Hs[i][k] for i in range(B)], axis=0)) for k in range(cfg.N)]
    rec = []

    def on_step(k, lp):
        rec.append({"entropy": lp.entropy.cpu().numpy().copy(),
                    "argmax": lp.argmax[k & 1].cpu().numpy().copy(),
                    "accept": lp.accept.cpu().numpy().copy(),
                    "tokens": lp.tokens.cpu().numpy().copy(),
                    "z": bits_np(lp.z), "A": bits_np(lp.A),
                    "flags": lp.wait_flags(k)})

    steps = loop.run_batch(batch, lambda k: Hd[k], on_step=on_step)
    torch.cuda.synchronize()
    stats = {"positions": 0, "mismatch": 0, "unexcused": 0}
    for i, c in enumerate(ids):
        Kp, Vp = host[i]
        P_o, recs = O.run_canvas(W, Kp, Vp, cfg.P0, lambda k: Hs[i][k], V=cfg.V, C=cfg.C,
                                 Hq=cfg.Hq, Hkv=cfg.Hkv, hd=cfg.hd, N=cfg.N, seed=cfg.seed,
                                 canvas=c, rule=rule)
        assert steps[i] == len(recs)
        for k, r in enumerate(recs):
            g = rec[k]
            assert g["flags"][i] == r["flag"]
            assert np.max(np.abs(g["entropy"][i] - r["entropy"])) <= 1e-3
            assert maxrel_rows(O.from_bf16(g["A"][i]), O.from_bf16(r["A"])) <= 2e-2
            assert maxrel_rows(O.from_bf16(g["z"][i]), O.from_bf16(r["z"])) <= 2e-2
            _, _, _, u = O.logits_entropy(Hs[i][r["k"]], W["E"], r["tau"])
            if rule == "confidence":
                assert int(g["accept"][i].sum()) == int(r["accept"].sum())
                cut = cutoff_confidence(r["conf"], r["accept"])
            else:
                cut = cutoff_entropy(r["entropy"], r["accept"])
            gt, ga, gm = g["tokens"][i], g["accept"][i], g["argmax"][i]
            mism = np.nonzero(gt != r["tokens"])[0]
            stats["positions"] += cfg.C
            stats["mismatch"] += len(mism)
            for j in mism:
                if rule == "confidence":
                    near_cut = ga[j] != r["accept"][j] and any(abs(float(r["conf"][j]) - x) <= 2e-5 * x for x in cut)
                else:
                    near_cut = ga[j] != r["accept"][j] and any(abs(float(r["entropy"][j]) - x) <= 1e-4 for x in cut)
                tie = gm[j] != r["argmax"][j] and near_tie(u[j])
                if not (near_cut or tie):
                    stats["unexcused"] += 1
        assert loop.P[i] == P_o
        Kg, Vg = cache_logical(caches[i][0], caches[i][1])
        K0, V0 = di.prefix_kv(cfg, Pcap, request=i)
        np.testing.assert_array_equal(Kg[:, :cfg.P0], K0[:, :cfg.P0])
        np.testing.assert_array_equal(Vg[:, :cfg.P0], V0[:, :cfg.P0])
        assert maxrel(O.from_bf16(Kg[:, cfg.P0:P_o]), O.from_bf16(Kp[:, cfg.P0:P_o])) <= 2e-2
        assert maxrel(O.from_bf16(Vg[:, cfg.P0:P_o]), O.from_bf16(Vp[:, cfg.P0:P_o])) <= 2e-2
    return stats


@pytest.mark.parametrize("cfg,B", [(WIDE, 2), (RAGGED, 3)], ids=["wide_b2", "ragged_b3"])
def test_batch_loop_parity(dg_ctx, cfg, B):
    s = run_batch_both(dg_ctx, cfg, B)
    assert s["unexcused"] == 0, s
    assert s["mismatch"] <= 0.001 * s["positions"], s


def test_batch_loop_parity_confidence_rule(dg_ctx):
    s = run_batch_both(dg_ctx, RAGGED, 2, rule="confidence")
    assert s["unexcused"] == 0, s
    assert s["mismatch"] <= 0.001 * s["positions"], s


def test_batch_of_one_matches_single_canvas_loop(dg_ctx):
    """B = 1 runs exactly the calls of the single-canvas loop: bit-identical records."""
    from block_ar_canvas_amd.loop import CanvasLoop
    cfg = di.config(0)
    W = di.weights(cfg)
    Pcap = -(-(cfg.P0 + cfg.C) // 8) * 8
    Wd = upload_weights(W)
    Hd = [bf16_dev(di.hidden(cfg, W["E"], 0, k, di.targets(cfg, 0))) for k in range(cfg.N)]
    out = []
    for batched in (False, True):
        Kp, Vp = di.prefix_kv(cfg, Pcap)
        Kd, Vtd = upload_cache(Kp, Vp, Pcap)
        rec = []

        def on_step(k, lp):
            rec.append((bits_np(lp.z).reshape(-1).copy(), lp.tokens.cpu().numpy().reshape(-1).copy(),
                        lp.entropy.cpu().numpy().reshape(-1).copy()))

        if batched:
            lp = BatchLoop(dg_ctx, cfg, Wd, [(Kd, Vtd, cfg.P0)], N=cfg.N, seed=cfg.seed)
            lp.run_batch(0, lambda k: Hd[k], on_step=on_step)
        else:
            lp = CanvasLoop(dg_ctx, cfg, Wd, Kd, Vtd, cfg.P0, N=cfg.N, seed=cfg.seed)
            lp.run_canvas(0, lambda k: Hd[k], on_step=on_step)
        torch.cuda.synchronize()
        out.append((rec, cache_logical(Kd, Vtd)))
    (ra, ca), (rb, cb) = out
    assert len(ra) == len(rb)
    for x, y in zip(ra, rb):
        for u, v in zip(x, y):
            np.testing.assert_array_equal(u, v)
    np.testing.assert_array_equal(ca[0], cb[0])
    np.testing.assert_array_equal(ca[1], cb[1])
