"""End-to-end parity at the headline workload sizes (needs an MI355X).

The same library calls, in the same launch configuration, that the benchmark times, on
the full shapes: a 262144-token vocabulary, d 2048, a 256-token canvas, 16 query and 8
KV heads of 128, against the float64 oracle on every canvas position.
  * gemma_head (8192-token prefix): the whole 48-step loop of one canvas;
  * long_prefix (262144-token prefix): the first two steps of a canvas, attention
    compared on every row;
  * chain8 (from a 32768-token prefix): two consecutive canvases with their commits,
    once with the projection commit and once with the causal prefill commit and rotary
    positions; attention is compared on every row at steps 0, 24 and 47 of each canvas.
Bars (the loop bars of the smaller loop tests): entropies within 1e-3 nats; argmax equal
except at oracle near-ties; canvas tokens equal at >= 99.9% of positions, a mismatch
excused only where acceptance differs at an oracle entropy within 1e-4 of the cutoff or
at an argmax near-tie; A and z within 2e-2 largest per-row relative error; stop flags
identical; committed K/V within 2e-2 and the prefix byte-unchanged.
The oracle takes E converted to float64 once per workload (the same values).
"""
import numpy as np
import pytest
import torch

import dg_inputs as di
import oracle as O
from block_ar_canvas_amd.loop import CanvasLoop
from gpu_util import (DEV, bf16_dev, bits_np, cache_logical, maxrel, maxrel_rows, near_tie,
                      upload_cache, upload_weights, workload)

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

_head = {}


def cutoff_entropy(ent, acc):
    order = sorted(range(len(ent)), key=lambda i: (float(ent[i]), i))
    n = int(acc.sum())
    cands = []
    if n > 0:
        cands.append(float(ent[order[n - 1]]))
    if n < len(ent):
        cands.append(float(ent[order[n]]))
    return cands


def run_device_canvas(loop, canvas, Hd):
    rec = []

    def on_step(k, lp):
        rec.append({"entropy": lp.entropy.cpu().numpy().copy(),
                    "argmax": lp.argmax[k & 1].cpu().numpy().copy(),
                    "accept": lp.accept.cpu().numpy().copy(),
                    "tokens": lp.tokens.cpu().numpy().copy(),
                    "z": bits_np(lp.z), "A": bits_np(lp.A), "flag": lp.wait_flag(k)})

    loop.run_canvas(canvas, lambda k: Hd[k], on_step=on_step)
    return rec


def compare_steps(rec, recs, Hs, E64, stats):
    """Per-step sampler-head, acceptance, token and z bars (A is compared by the caller)."""
    assert [g["flag"] for g in rec] == [r["flag"] for r in recs]
    for g, r in zip(rec, recs):
        assert np.max(np.abs(g["entropy"] - r["entropy"])) <= 1e-3, r["k"]
        assert maxrel_rows(O.from_bf16(g["z"]), O.from_bf16(r["z"])) <= 2e-2, r["k"]
        amis = np.nonzero(g["argmax"] != r["argmax"])[0]
        tmis = np.nonzero(g["tokens"] != r["tokens"])[0]
        ties = set()
        rows = sorted(set(amis) | set(tmis))
        if rows:                                        # the oracle's logits of those rows only
            _, _, _, u = O.logits_entropy(Hs[r["k"]], E64, r["tau"], rows=rows)
            ties = {i for i, ur in zip(rows, u) if near_tie(ur)}
        assert all(i in ties for i in amis), (r["k"], amis)
        cut = cutoff_entropy(r["entropy"], r["accept"])
        stats["positions"] += len(r["tokens"])
        stats["mismatch"] += len(tmis)
        for i in tmis:
            near_cut = g["accept"][i] != r["accept"][i] and any(
                abs(float(r["entropy"][i]) - x) <= 1e-4 for x in cut)
            if not (near_cut or (g["argmax"][i] != r["argmax"][i] and i in ties)):
                stats["unexcused"] += 1


def compare_attention(g_A, dev_input, r, W, W64, Kp, Vp, P, cfg, rope_base=0.0):
    """A of one step on every row; on the device's own input canvas where an excused
    token mismatch left it different from the oracle's."""
    tokens, z = r["tokens_in"], r["z_in"]
    if dev_input is not None and not np.array_equal(dev_input[0], tokens):
        tokens, z = dev_input
    A_r, _ = O.canvas_attn(tokens, z, W64["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], Kp, Vp, P,
                           cfg.Hq, cfg.Hkv, cfg.hd, rope_base=rope_base)
    err = maxrel_rows(O.from_bf16(g_A), O.from_bf16(A_r))
    assert err <= 2e-2, (r["k"], err)


ATTN_STEPS = (0, 24, 47)


def head_records(cfg, W, W64, canvas):
    """The oracle's sampler-head records of one chain canvas (they do not depend on the
    cache or on the commit): cached across the two commit variants."""
    if (cfg.name, canvas) not in _head:
        for key in [k for k in _head if k[0] != cfg.name]:
            del _head[key]
        Kp, Vp = di.prefix_kv(cfg.with_(P0=0), cfg.Pcap)     # scratch cache for the commit
        tgt = di.targets(cfg, canvas)
        Hs = [di.hidden(cfg, W["E"], canvas, k, tgt) for k in range(cfg.N)]
        _, recs = O.run_canvas(W64, Kp, Vp, 0, lambda k: Hs[k], V=cfg.V, C=cfg.C, Hq=cfg.Hq,
                               Hkv=cfg.Hkv, hd=cfg.hd, N=cfg.N, seed=cfg.seed, canvas=canvas,
                               with_attn=False)
        _head[(cfg.name, canvas)] = (Hs, recs)
    return _head[(cfg.name, canvas)]


@pytest.mark.parametrize("commit", ["projection", "prefill"])
def test_chain_two_canvases(dg_ctx, commit):
    cfg, W, W64, Wd = workload("chain8")
    rope = 10000.0 if commit == "prefill" else 0.0
    Pcap = cfg.Pcap
    Kp, Vp = di.prefix_kv(cfg, Pcap)
    Kd, Vtd = upload_cache(Kp, Vp, Pcap)
    try:
        loop = CanvasLoop(dg_ctx, cfg, Wd, Kd, Vtd, cfg.P0, N=cfg.N, seed=cfg.seed, commit=commit,
                          rope_base=rope)
        Kp_o, Vp_o, P_o = Kp.copy(), Vp.copy(), cfg.P0
        stats = {"positions": 0, "mismatch": 0, "unexcused": 0}
        keep = []
        for c in range(2):
            Hs, recs = head_records(cfg, W, W64, c)
            rec = run_device_canvas(loop, c, [bf16_dev(h) for h in Hs])
            A_commit = bits_np(loop.A) if commit == "prefill" else None
            dg_ctx.sync()
            assert len(rec) == len(recs) == cfg.N
            compare_steps(rec, recs, Hs, W64["E"], stats)
            for j in ATTN_STEPS:                       # attention over this canvas's cache
                dev_in = None if j == 0 else (rec[j - 1]["tokens"], rec[j - 1]["z"])
                compare_attention(rec[j]["A"], dev_in, recs[j], W, W64, Kp_o, Vp_o, P_o, cfg, rope)
            # the committed block: a position's K/V row depends on its own token only, and
            # prefill row i of A on tokens 0..i; a final argmax excused at a near-tie
            # leaves that row (and later prefill rows of A) out of the comparison
            x0 = recs[-1]["argmax"]
            same = rec[-1]["argmax"] == x0
            keep.append(same)
            if commit == "prefill":
                A_r, P_o = O.prefill_block(x0, W64["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], Kp_o,
                                           Vp_o, P_o, cfg.Hq, cfg.Hkv, cfg.hd, rope)
                n_ok = int(np.argmin(same)) if not same.all() else cfg.C
                assert maxrel_rows(O.from_bf16(A_commit[:n_ok]), O.from_bf16(A_r[:n_ok])) <= 2e-2
            else:
                P_o = O.commit_kv(x0, W64["E"], W["Wk"], W["Wv"], Kp_o, Vp_o, P_o, cfg.Hkv, cfg.hd)
            assert loop.P == P_o
        assert stats["unexcused"] == 0 and stats["mismatch"] <= 0.001 * stats["positions"], stats
    finally:
        dg_ctx.set_rope(0.0)
    Kg, Vg = cache_logical(Kd, Vtd)
    np.testing.assert_array_equal(Kg[:, :cfg.P0], Kp[:, :cfg.P0])
    np.testing.assert_array_equal(Vg[:, :cfg.P0], Vp[:, :cfg.P0])
    new = cfg.P0 + np.nonzero(np.concatenate(keep))[0]
    assert len(new) >= 0.99 * (P_o - cfg.P0)
    assert maxrel_rows(O.from_bf16(Kg[:, new]), O.from_bf16(Kp_o[:, new])) <= 2e-2
    assert maxrel_rows(O.from_bf16(Vg[:, new]), O.from_bf16(Vp_o[:, new])) <= 2e-2


def test_gemma_head_loop_48_steps(dg_ctx):
    cfg, W, W64, Wd = workload("gemma_head")
    Pcap = cfg.Pcap
    Kp, Vp = di.prefix_kv(cfg, Pcap)
    Kd, Vtd = upload_cache(Kp, Vp, Pcap)
    loop = CanvasLoop(dg_ctx, cfg, Wd, Kd, Vtd, cfg.P0, N=cfg.N, seed=cfg.seed)
    tgt = di.targets(cfg, 0)
    Hs = [di.hidden(cfg, W["E"], 0, k, tgt) for k in range(cfg.N)]
    rec = run_device_canvas(loop, 0, [bf16_dev(h) for h in Hs])
    dg_ctx.sync()
    Kg, Vg = cache_logical(Kd, Vtd)
    P_o, recs = O.run_canvas(W64, Kp, Vp, cfg.P0, lambda k: Hs[k], V=cfg.V, C=cfg.C, Hq=cfg.Hq,
                             Hkv=cfg.Hkv, hd=cfg.hd, N=cfg.N, seed=cfg.seed, canvas=0)
    assert len(rec) == len(recs) == cfg.N and loop.P == P_o == cfg.P0 + cfg.C
    stats = {"positions": 0, "mismatch": 0, "unexcused": 0}
    compare_steps(rec, recs, Hs, W64["E"], stats)
    assert stats["unexcused"] == 0 and stats["mismatch"] <= 0.001 * stats["positions"], stats
    for j, r in enumerate(recs):
        dev_in = None if j == 0 else (rec[j - 1]["tokens"], rec[j - 1]["z"])
        err = maxrel_rows(O.from_bf16(rec[j]["A"]), O.from_bf16(r["A"]))
        if err > 2e-2:                                  # only an earlier excused mismatch may explain it
            compare_attention(rec[j]["A"], dev_in, r, W, W64, Kp, Vp, cfg.P0, cfg)
    np.testing.assert_array_equal(Kg[:, :cfg.P0], Kp[:, :cfg.P0])
    np.testing.assert_array_equal(Vg[:, :cfg.P0], Vp[:, :cfg.P0])
    rows = np.arange(cfg.P0, P_o)
    final_same = rec[-1]["argmax"] == recs[-1]["argmax"]
    rows = rows[final_same]
    assert maxrel_rows(O.from_bf16(Kg[:, rows]), O.from_bf16(Kp[:, rows])) <= 2e-2
    assert maxrel_rows(O.from_bf16(Vg[:, rows]), O.from_bf16(Vp[:, rows])) <= 2e-2


def test_long_prefix_two_steps(dg_ctx):
    # the first two denoise steps of a canvas over the 262144-token cache: step 0 on the
    # initial uniform canvas (X = E[x]), step 1 on the renoised canvas and step 0's z
    cfg, W, W64, Wd = workload("long_prefix")
    Pcap = cfg.Pcap
    Kp, Vp = di.prefix_kv(cfg, Pcap)
    Kd, Vtd = upload_cache(Kp, Vp, Pcap)
    loop = CanvasLoop(dg_ctx, cfg, Wd, Kd, Vtd, cfg.P0, N=cfg.N, seed=cfg.seed)
    tgt = di.targets(cfg, 0)
    Hs = [di.hidden(cfg, W["E"], 0, k, tgt) for k in range(2)]
    loop.init_canvas(0)
    x0 = loop.tokens.cpu().numpy().copy()
    rec = []
    for k in range(2):
        loop.step(k, bf16_dev(Hs[k]))
        rec.append({"entropy": loop.entropy.cpu().numpy().copy(),
                    "argmax": loop.argmax[k & 1].cpu().numpy().copy(),
                    "accept": loop.accept.cpu().numpy().copy(),
                    "tokens": loop.tokens.cpu().numpy().copy(),
                    "z": bits_np(loop.z), "A": bits_np(loop.A), "flag": loop.wait_flag(k)})
    dg_ctx.sync()
    # the oracle's two steps, call by call
    x = O.renoise(np.zeros(cfg.C, np.int32), None, cfg.seed, 0, 0, cfg.V)[0]
    np.testing.assert_array_equal(x0, x)
    z = np.zeros((cfg.C, cfg.d), np.uint16)
    prev = None
    recs = []
    for k in range(2):
        tau = O.temperature(k, cfg.N)
        r = {"k": k, "tau": tau, "tokens_in": x.copy(), "z_in": z.copy()}
        r["A"], _ = O.canvas_attn(x, z, W64["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], Kp, Vp,
                                  cfg.P0, cfg.Hq, cfg.Hkv, cfg.hd)
        ent, am, p, _ = O.logits_entropy(Hs[k], W64["E"], tau)
        acc, _ = O.entropy_accept(ent[None], 0.1)
        x = O.renoise(am[None], acc, cfg.seed, 0, k, cfg.V)[0]
        z, _ = O.selfcond(p, W64["E"], W["W1"], W["W2"])
        del p
        flag = int(O.stop_test(ent[None], am[None], None if prev is None else prev[None],
                               0.005, k, cfg.N)[0])
        prev = am
        r.update(entropy=ent, argmax=am, accept=acc[0], tokens=x.copy(), z=z.copy(), flag=flag)
        recs.append(r)
    stats = {"positions": 0, "mismatch": 0, "unexcused": 0}
    compare_steps(rec, recs, Hs, W64["E"], stats)
    assert stats["unexcused"] == 0 and stats["mismatch"] <= 0.001 * stats["positions"], stats
    for j, r in enumerate(recs):
        dev_in = None if j == 0 else (rec[j - 1]["tokens"], rec[j - 1]["z"])
        err = maxrel_rows(O.from_bf16(rec[j]["A"]), O.from_bf16(r["A"]))
        if err > 2e-2:
            compare_attention(rec[j]["A"], dev_in, r, W, W64, Kp, Vp, cfg.P0, cfg)
    Kg, Vg = cache_logical(Kd, Vtd)                      # denoising only reads the cache
    np.testing.assert_array_equal(Kg[:, :cfg.P0], Kp[:, :cfg.P0])
    np.testing.assert_array_equal(Vg[:, :cfg.P0], Vp[:, :cfg.P0])
