"""Per-call parity of the HIP path against the CPU oracle (needs an MI355X).

Sizes span several tiles of every kernel and ragged tails (V, C, P and d not multiples
of the tile sizes). Tolerances:
  * entropy within 1e-3 nats; argmax exact except where the oracle's top-2 gap of the
    tempered logits is within 1e-3 max(1, |u_top|);
  * attention output A, self-conditioning z and committed K/V: max|g - r| / max|r| <= 2e-2
    (bf16 inputs, fp32 accumulation vs the float64 oracle);
  * acceptance, renoise and the stop flag bit-exact when fed the oracle's vectors.
"""
import math

import numpy as np
import pytest
import torch

import block_ar_canvas_amd as dg
import dg_inputs as di
import oracle as O
from gpu_util import (DEV, argmax_mismatch_unexcused, bf16_dev, bits_np, cache_logical, f32_dev, i32_dev,
                      maxrel, maxrel_rows, sample_excused, u8_dev, upload_cache, upload_weights)

pytestmark = pytest.mark.gpu

SHAPES = {
    "tiny": di.config(0),
    "small": di.config(1),
    "ragged": di.Config("ragged", V=5000, d=96, C=100, Hq=6, Hkv=3, hd=32, F=64, P0=77, N=6,
                        alpha_max=8.0, seed=21),
    "hd64": di.Config("hd64", V=3000, d=128, C=40, Hq=4, Hkv=1, hd=64, F=96, P0=300, N=6,
                      alpha_max=9.0, seed=22),
    "c1000": di.Config("c1000", V=1000, d=64, C=1000, Hq=2, Hkv=2, hd=16, F=32, P0=5, N=4,
                       alpha_max=6.0, seed=23),
    # two canvas blocks over a tile count divisible by 8 and 8 self-conditioning splits:
    # the workgroup mappings that keep a tile's (a split's) canvas blocks on one XCD
    "wide": di.Config("wide", V=32768, d=256, C=300, Hq=4, Hkv=2, hd=64, F=128, P0=100, N=4,
                      alpha_max=8.0, seed=24),
    # 257 vocabulary tiles (so 256-column canvas blocks), the last one holding 77 ids, a
    # tile count the self-conditioning splits do not divide (plain dispatch order), a
    # model width whose last 64-wide chunk is half full, and a ragged canvas; the shapes
    # above with few tiles or at most 128 padded columns take 128-column blocks
    "wide_tail": di.Config("wide_tail", V=65613, d=96, C=130, Hq=2, Hkv=1, hd=32, F=64, P0=50, N=4,
                           alpha_max=8.0, seed=25),
}

_cache = {}


def setup(name):
    if name not in _cache:
        cfg = SHAPES[name]
        W = di.weights(cfg)
        Pcap = -(-(cfg.P0 + cfg.C) // 8) * 8
        Kp, Vp = di.prefix_kv(cfg, Pcap)
        _cache[name] = (cfg, W, Kp, Vp, Pcap, upload_weights(W))
    return _cache[name]


def ws_for(cfg, Pcap):
    return torch.empty(dg.workspace_bytes(cfg, Pcap), dtype=torch.uint8, device=DEV)


def run_head(ctx, cfg, Wd, H, tau, ws):
    ent = torch.empty(cfg.C, dtype=torch.float32, device=DEV)
    am = torch.empty(cfg.C, dtype=torch.int32, device=DEV)
    ctx.logits_entropy(cfg, bf16_dev(H), Wd["E"], tau, ws, ent, am)
    return ent, am


@pytest.mark.parametrize("name", list(SHAPES))
def test_logits_entropy_and_selfcond(dg_ctx, name):
    cfg, W, Kp, Vp, Pcap, Wd = setup(name)
    ws = ws_for(cfg, Pcap)
    tgt = di.targets(cfg, 0)
    for k in sorted({0, cfg.N // 2, cfg.N - 1}):
        H = di.hidden(cfg, W["E"], 0, k, tgt)
        tau = O.temperature(k, cfg.N)
        assert np.float32(dg.temperature(k, cfg.N)) == tau
        ent, am = run_head(dg_ctx, cfg, Wd, H, tau, ws)
        conf = torch.empty(cfg.C, dtype=torch.float32, device=DEV)
        dg_ctx.confidence(cfg, ws, conf)
        z = torch.empty(cfg.C, cfg.d, dtype=torch.bfloat16, device=DEV)
        dg_ctx.selfcond(cfg, ws, Wd["E"], Wd["W1"], Wd["W2"], z)
        dg_ctx.sync()
        ent_r, am_r, p_r, u_r = O.logits_entropy(H, W["E"], tau)
        # confidence = largest probability; fp32 statistics vs float64: 2e-5 relative
        conf_r = p_r.max(axis=1)
        np.testing.assert_allclose(conf.cpu().numpy(), conf_r, rtol=2e-5, atol=0)
        e = ent.cpu().numpy()
        assert np.all(np.isfinite(e))
        assert np.max(np.abs(e - ent_r)) <= 1e-3, (k, np.max(np.abs(e - ent_r)))
        assert argmax_mismatch_unexcused(am.cpu().numpy(), am_r, u_r) == 0
        z_r, _ = O.selfcond(p_r, W["E"], W["W1"], W["W2"])
        assert maxrel_rows(O.from_bf16(bits_np(z)), O.from_bf16(z_r)) <= 2e-2


@pytest.mark.parametrize("name", ["tiny", "small", "ragged", "wide"])
def test_sample_tokens(dg_ctx, name):
    """dg_sample against the oracle's inverse-CDF draw over the whole vocabulary. A token
    may differ only where the oracle's target u times the total lies within the device's
    rounding of a cumulative boundary (gpu_util.sample_excused)."""
    cfg, W, Kp, Vp, Pcap, Wd = setup(name)
    ws = ws_for(cfg, Pcap)
    tgt = di.targets(cfg, 0)
    B = 2 if cfg.C % 2 == 0 else 1
    total = bad = same = 0
    for k in sorted({0, cfg.N // 2, cfg.N - 1}):
        H = di.hidden(cfg, W["E"], 0, k, tgt)
        tau = O.temperature(k, cfg.N)
        run_head(dg_ctx, cfg, Wd, H, tau, ws)
        tok = torch.full((cfg.C,), -1, dtype=torch.int32, device=DEV)
        dg_ctx.sample(cfg, ws, B, 1234 + k, 7, k, tok)
        dg_ctx.sync()
        _, _, p_r, _ = O.logits_entropy(H, W["E"], tau)
        ref, margin = O.sample_tokens(p_r, 1234 + k, 7, k, B=B, with_margins=True)
        g = tok.cpu().numpy()
        assert np.all((g >= 0) & (g < cfg.V))
        for i in np.nonzero(g != ref)[0]:
            if not sample_excused(p_r[i], int(ref[i]), float(margin[i])):
                bad += 1
        total += cfg.C
        same += int((g == ref).sum())
    assert bad == 0, (bad, total)
    assert same >= 0.95 * total, (same, total)     # excuses stay rare


def test_sample_rejects_bad_segments_and_stale_ws(dg_ctx):
    cfg, W, Kp, Vp, Pcap, Wd = setup("ragged")
    ws = ws_for(cfg, Pcap)
    tok = torch.empty(cfg.C, dtype=torch.int32, device=DEV)
    with pytest.raises(dg.DGError):                 # no dg_logits_entropy on this ws yet
        dg_ctx.sample(cfg, ws, 1, 0, 0, 0, tok)
    run_head(dg_ctx, cfg, Wd, di.hidden(cfg, W["E"], 0, 0, di.targets(cfg, 0)), 0.8, ws)
    with pytest.raises(dg.DGError):                 # 3 does not divide C = 100
        dg_ctx.sample(cfg, ws, 3, 0, 0, 0, tok)


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("prefix", ["full", "empty"])
def test_canvas_attention(dg_ctx, name, prefix):
    cfg, W, Kp, Vp, Pcap, Wd = setup(name)
    P = cfg.P0 if prefix == "full" else 0
    rng = np.random.default_rng(cfg.seed + 100)
    tok = rng.integers(0, cfg.V, cfg.C).astype(np.int32)
    z = di.f32_to_bf16_bits(rng.standard_normal((cfg.C, cfg.d)).astype(np.float32) * 0.3)
    Kd, Vtd = upload_cache(Kp, Vp)
    ws = ws_for(cfg, Pcap)
    A = torch.empty(cfg.C, cfg.d, dtype=torch.bfloat16, device=DEV)
    dg_ctx.canvas_attn(cfg, i32_dev(tok), bf16_dev(z), Wd["E"], Wd["Wq"], Wd["Wk"], Wd["Wv"],
                       Wd["Wo"], Kd, Vtd, P, ws, A)
    dg_ctx.sync()
    A_r, _ = O.canvas_attn(tok, z, W["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], Kp, Vp, P,
                           cfg.Hq, cfg.Hkv, cfg.hd)
    assert maxrel_rows(O.from_bf16(bits_np(A)), O.from_bf16(A_r)) <= 2e-2
    # the cache is only read
    Kb, Vb = upload_cache(Kp, Vp)
    assert torch.equal(Kd.view(torch.int16), Kb.view(torch.int16))
    assert torch.equal(Vtd.view(torch.int16), Vb.view(torch.int16))


def test_canvas_attention_without_selfcond_term(dg_ctx):
    cfg, W, Kp, Vp, Pcap, Wd = setup("ragged")
    tok = np.random.default_rng(5).integers(0, cfg.V, cfg.C).astype(np.int32)
    Kd, Vtd = upload_cache(Kp, Vp)
    A = torch.empty(cfg.C, cfg.d, dtype=torch.bfloat16, device=DEV)
    dg_ctx.canvas_attn(cfg, i32_dev(tok), None, Wd["E"], Wd["Wq"], Wd["Wk"], Wd["Wv"], Wd["Wo"],
                       Kd, Vtd, cfg.P0, ws_for(cfg, Pcap), A)
    dg_ctx.sync()
    A_r, _ = O.canvas_attn(tok, None, W["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], Kp, Vp,
                           cfg.P0, cfg.Hq, cfg.Hkv, cfg.hd)
    assert maxrel_rows(O.from_bf16(bits_np(A)), O.from_bf16(A_r)) <= 2e-2


def _accept_cases_synthetic():
    rng = np.random.default_rng(31)
    cases = []
    for C in (1, 7, 16, 100, 256, 1000, 1024):
        h = rng.exponential(10 ** rng.uniform(-3, -1), (3, C)).astype(np.float32)
        h[1, ::3] = h[1, 0]                               # ties
        h[2, : C // 2] = np.float32(0.0)
        cases.append(h)
    edge = np.array([[np.nan, 0.0, np.inf, 70000.0, 0.01, -0.0, -1.0, -np.inf,
                      0.05, 0.05, 0.05, 65535.0]], np.float32)
    cases.append(edge)
    cases.append(np.full((2, 3), 0.05, np.float32))
    return cases


def _accept_cases():
    cases = _accept_cases_synthetic()
    # the oracle's own entropies along a small-config trajectory
    cfg, W, *_ = setup("small")
    tgt = di.targets(cfg, 0)
    rows = [O.logits_entropy(di.hidden(cfg, W["E"], 0, k, tgt), W["E"], O.temperature(k, cfg.N))[0]
            for k in (30, 38, 42, 47)]
    cases.append(np.stack(rows))
    return cases


@pytest.mark.parametrize("b", [0.1, 0.0, 0.37, 65000.0])
def test_entropy_accept_bit_exact(dg_ctx, b):
    for h in _accept_cases():
        B, C = h.shape
        acc = torch.full((B, C), 7, dtype=torch.uint8, device=DEV)
        n = torch.empty(B, dtype=torch.int32, device=DEV)
        dg_ctx.entropy_accept(f32_dev(h), b, acc, n)
        acc_r, n_r = O.entropy_accept(h, b)
        np.testing.assert_array_equal(acc.cpu().numpy(), acc_r)
        np.testing.assert_array_equal(n.cpu().numpy(), n_r)


def _topk_cases():
    rng = np.random.default_rng(77)
    cases = []
    for B, C in ((1, 16), (3, 100), (2, 256), (1, 257), (2, 1000), (1, 1024)):
        # few distinct values (many ties), NaNs and signed zeros
        s = rng.choice(np.array([0.05, 0.2, 0.2, 0.5, 0.9], np.float32), size=(B, C))
        s[rng.random((B, C)) < 0.05] = np.nan
        s[rng.random((B, C)) < 0.03] = -0.0
        s[rng.random((B, C)) < 0.03] = 0.0
        cases.append(s.astype(np.float32))
        cases.append(rng.random((B, C)).astype(np.float32))
    return cases


def test_topk_accept_bit_exact(dg_ctx):
    for s in _topk_cases():
        B, C = s.shape
        for k in sorted({0, 1, C // 3, C - 1, C, C + 5}):
            acc = torch.full((B, C), 7, dtype=torch.uint8, device=DEV)
            n = torch.empty(B, dtype=torch.int32, device=DEV)
            dg_ctx.topk_accept(f32_dev(s), k, acc, n)
            acc_r, n_r = O.topk_accept(s, k)
            np.testing.assert_array_equal(acc.cpu().numpy(), acc_r)
            np.testing.assert_array_equal(n.cpu().numpy(), n_r)


def test_topk_accept_rejects_negative_k(dg_ctx):
    s = f32_dev(np.zeros((1, 8), np.float32))
    acc = torch.empty(1, 8, dtype=torch.uint8, device=DEV)
    n = torch.empty(1, dtype=torch.int32, device=DEV)
    with pytest.raises(dg.DGError):
        dg_ctx.topk_accept(s, -1, acc, n)


@pytest.mark.parametrize("V", [2, 3, 512, 5000, 262144, 2 ** 31 - 1])
def test_renoise_bit_exact(dg_ctx, V):
    rng = np.random.default_rng(V % 1000)
    B, C = 3, 257
    am = rng.integers(0, V, (B, C)).astype(np.int32)
    acc = (rng.random((B, C)) < 0.4).astype(np.uint8)
    for seed, base, step in ((0, 0, 0), (2 ** 63 + 5, 7, 47), (12345, 2 ** 31, 3)):
        tok = torch.empty(B, C, dtype=torch.int32, device=DEV)
        dg_ctx.renoise(V, i32_dev(am), u8_dev(acc), seed, base, step, tok)
        np.testing.assert_array_equal(tok.cpu().numpy(), O.renoise(am, acc, seed, base, step, V))
        dg_ctx.renoise(V, None, None, seed, base, 0, tok)
        np.testing.assert_array_equal(tok.cpu().numpy(), O.renoise(am, None, seed, base, 0, V))


def test_stop_test_bit_exact(dg_ctx):
    C, N = 256, 48
    am = np.arange(C, dtype=np.int32)
    h = np.full(C, 0.005, np.float32)
    h_up = h.copy()
    h_up[7] = np.nextafter(np.float32(0.005), np.float32(1))
    am2 = am.copy()
    am2[100] += 1
    h_nan = np.zeros(C, np.float32)
    h_nan[0] = np.nan
    cases = [(h, am, am, 3), (h_up, am, am, 3), (h, am2, am, 3), (h, am, None, 0), (h, am, am, 0),
             (h_up, am, am, N - 1), (h, am, am, N - 1), (h_nan, am, am, 3), (h_up, am, None, N - 1)]
    rng = np.random.default_rng(41)
    for _ in range(10):
        hh = rng.exponential(0.004, C).astype(np.float32)
        cases.append((hh, am, am, int(rng.integers(1, N))))
    for hh, a, p, step in cases:
        flag = torch.full((1,), -1, dtype=torch.int32, device=DEV)
        dg_ctx.stop_test(f32_dev(hh), i32_dev(a), None if p is None else i32_dev(p), 0.005, step, N, flag)
        assert int(flag.item()) == int(O.stop_test(hh, a, p, 0.005, step, N)[0])
    # segments
    hb = np.zeros((3, 16), np.float32)
    hb[1, 3] = 1.0
    ab = np.zeros((3, 16), np.int32)
    pb = ab.copy()
    pb[2, 5] = 1
    flag = torch.empty(3, dtype=torch.int32, device=DEV)
    dg_ctx.stop_test(f32_dev(hb), i32_dev(ab), i32_dev(pb), 0.005, 2, 8, flag)
    np.testing.assert_array_equal(flag.cpu().numpy(), O.stop_test(hb, ab, pb, 0.005, 2, 8))


def _ars_cases():
    """(entropy [B, C], b, prev relation, step, N) for the one-launch acceptance, renoise
    and stop test: the acceptance cases (NaN, infinities, ties, zeros, C up to 1024),
    plus canvases whose mean entropy is under the threshold so the stop can fire."""
    cases = []
    for i, h in enumerate(_accept_cases_synthetic()):
        B, C = h.shape
        cases.append((h, (0.1, 0.0, 0.37, 65000.0)[i % 4], ("same", "one_changed", None)[i % 3],
                      (0, 3, 47)[i % 3], 48))
    rng = np.random.default_rng(53)
    for B, C, step in ((1, 256, 5), (3, 100, 1), (2, 1024, 47), (4, 1, 2)):
        h = rng.exponential(0.002, (B, C)).astype(np.float32)
        cases.append((h, 0.1, "same", step, 48))
        cases.append((h, 0.1, "one_changed", step, 48))
    return cases


@pytest.mark.parametrize("case", range(len(_ars_cases())))
def test_accept_renoise_stop_matches_the_three_calls(dg_ctx, case):
    """dg_accept_renoise_stop against the oracle's acceptance, renoise and stop test and
    against the three separate calls, bit for bit (x0 differs from the argmax so the
    kept tokens are checked to come from x0)."""
    h, b, rel, step, N = _ars_cases()[case]
    B, C = h.shape
    V, thr, seed, base = 5000, 0.005, 2 ** 63 + 9 + case, 11 * case
    rng = np.random.default_rng(100 + case)
    am = rng.integers(0, V, (B, C)).astype(np.int32)
    x0 = rng.integers(0, V, (B, C)).astype(np.int32)
    prev = None
    if rel is not None:
        prev = am.copy()
        if rel == "one_changed":
            prev[-1, C // 2] = (prev[-1, C // 2] + 1) % V
    acc_r, n_r = O.entropy_accept(h, b)
    tok_r = O.renoise(x0, acc_r, seed, base, step, V)
    flag_r = O.stop_test(h, am, prev, thr, step, N)

    def fresh():
        return (torch.full((B, C), 7, dtype=torch.uint8, device=DEV), torch.full((B,), -5, dtype=torch.int32, device=DEV),
                torch.full((B, C), -1, dtype=torch.int32, device=DEV), torch.full((B,), -1, dtype=torch.int32, device=DEV))

    hd, amd, x0d = f32_dev(h), i32_dev(am), i32_dev(x0)
    prevd = None if prev is None else i32_dev(prev)
    acc, n, tok, flag = fresh()
    dg_ctx.accept_renoise_stop(V, hd, b, x0d, amd, prevd, seed, base, step, thr, N, acc, n, tok, flag)
    acc2, n2, tok2, flag2 = fresh()
    dg_ctx.entropy_accept(hd, b, acc2, n2)
    dg_ctx.renoise(V, x0d, acc2, seed, base, step, tok2)
    dg_ctx.stop_test(hd, amd, prevd, thr, step, N, flag2)
    dg_ctx.sync()
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_r)
    np.testing.assert_array_equal(n.cpu().numpy(), n_r)
    np.testing.assert_array_equal(tok.cpu().numpy(), tok_r)
    np.testing.assert_array_equal(flag.cpu().numpy(), flag_r)
    for got, ref in ((acc, acc2), (n, n2), (tok, tok2), (flag, flag2)):
        np.testing.assert_array_equal(got.cpu().numpy(), ref.cpu().numpy())


def test_accept_renoise_stop_refusals(dg_ctx):
    h = f32_dev(np.zeros((1, 8), np.float32))
    a = i32_dev(np.zeros((1, 8), np.int32))
    acc = torch.empty(1, 8, dtype=torch.uint8, device=DEV)
    n = torch.empty(1, dtype=torch.int32, device=DEV)
    tok = torch.full((1, 8), -1, dtype=torch.int32, device=DEV)
    flag = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    for kw, err in (({"b": -0.5}, "DG_ERR_RANGE"), ({"thr": 70000.0}, "DG_ERR_RANGE"),
                    ({"step": -1}, "DG_ERR_RANGE"), ({"N": 0}, "DG_ERR_RANGE"), ({"V": 0}, "DG_ERR_SHAPE")):
        args = {"V": 10, "b": 0.1, "thr": 0.005, "step": 1, "N": 4, **kw}
        with pytest.raises(dg.DGError) as ei:
            dg_ctx.accept_renoise_stop(args["V"], h, args["b"], a, a, a, 1, 0, args["step"], args["thr"],
                                       args["N"], acc, n, tok, flag)
        assert ei.value.name == err
    dg_ctx.sync()
    assert int(tok.min().item()) == -1 and int(flag.item()) == -1


# (shape, canvases B): up to 256 positions per canvas the acceptance work runs beside the
# reduce (tiny, ragged, hd64, small, wide_tail; ragged as 4 canvases of 25 and wide as 3
# of 100); c1000 and wide (300 positions) take a launch of their own
SELFCOND_ACCEPT = [("tiny", 1), ("ragged", 1), ("ragged", 4), ("hd64", 1), ("small", 1), ("wide_tail", 1),
                   ("wide", 3), ("wide", 1), ("c1000", 1)]


@pytest.mark.parametrize("name,B", SELFCOND_ACCEPT, ids=[f"{n}-B{b}" for n, b in SELFCOND_ACCEPT])
def test_selfcond_accept_matches_the_separate_calls(dg_ctx, name, B):
    """dg_selfcond_accept against dg_accept_renoise_stop followed by dg_selfcond on the same
    sampler-head outputs, bit for bit: z, acceptance, tokens, counts and flags (a stop that
    fires at the last step, where the argmax is unchanged, and one that cannot)."""
    cfg, W, Kp, Vp, Pcap, Wd = setup(name)
    tgt = di.targets(cfg, 0)
    k = cfg.N - 1
    H = bf16_dev(di.hidden(cfg, W["E"], 0, k, tgt))
    tau = O.temperature(k, cfg.N)
    Cs = cfg.C // B
    rng = np.random.default_rng(7 + B)
    x0 = i32_dev(rng.integers(0, cfg.V, (B, Cs)).astype(np.int32))
    outs = []
    for fused in (False, True):
        ws = ws_for(cfg, Pcap)
        ent = torch.empty(B, Cs, dtype=torch.float32, device=DEV)
        am = torch.empty(B, Cs, dtype=torch.int32, device=DEV)
        dg_ctx.logits_entropy(cfg, H, Wd["E"], tau, ws, ent.view(-1), am.view(-1))
        z = torch.full((cfg.C, cfg.d), -1.0, dtype=torch.bfloat16, device=DEV)
        acc = torch.full((B, Cs), 7, dtype=torch.uint8, device=DEV)
        n = torch.full((B,), -5, dtype=torch.int32, device=DEV)
        tok = torch.full((B, Cs), -1, dtype=torch.int32, device=DEV)
        flag = torch.full((B,), -1, dtype=torch.int32, device=DEV)
        # prev = argmax: the stop fires wherever the mean entropy is under the threshold
        args = (0.1, x0, am, am.clone(), 2 ** 62 + 3, 5, k, 10.0, cfg.N, acc, n, tok, flag)
        if fused:
            dg_ctx.selfcond_accept(cfg, ws, Wd["E"], Wd["W1"], Wd["W2"], z, ent, *args)
        else:
            dg_ctx.accept_renoise_stop(cfg.V, ent, *args)
            dg_ctx.selfcond(cfg, ws, Wd["E"], Wd["W1"], Wd["W2"], z)
        dg_ctx.sync()
        outs.append((bits_np(z).copy(), acc.cpu().numpy(), n.cpu().numpy(), tok.cpu().numpy(), flag.cpu().numpy()))
        e = ent.cpu().numpy()
    assert int((outs[1][3] < 0).sum()) == 0
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)
    # the flags themselves against the oracle's stop test on the same entropies
    am_np = am.cpu().numpy()
    np.testing.assert_array_equal(outs[1][4], O.stop_test(e, am_np, am_np, 10.0, k, cfg.N))


@pytest.mark.parametrize("name,B", [("ragged", 1), ("small", 1), ("ragged", 4), ("c1000", 1)],
                         ids=["ragged", "small", "ragged-B4", "c1000"])
def test_next_input_and_canvas_attn_x(dg_ctx, name, B):
    """selfcond_accept's x_next is bf16(E[tokens] + z) of its own new tokens and z, bit for
    bit (float32 add of the two bf16 values, rounded to nearest even, computed here on the
    host from the device's tokens and z); canvas_attn_x on it gives canvas_attn's bytes."""
    cfg, W, Kp, Vp, Pcap, Wd = setup(name)
    ws = ws_for(cfg, Pcap)
    k = 1
    H = bf16_dev(di.hidden(cfg, W["E"], 0, k, di.targets(cfg, 0)))
    Cs = cfg.C // B
    ent = torch.empty(B, Cs, dtype=torch.float32, device=DEV)
    am = torch.empty(B, Cs, dtype=torch.int32, device=DEV)
    dg_ctx.logits_entropy(cfg, H, Wd["E"], O.temperature(k, cfg.N), ws, ent.view(-1), am.view(-1))
    z = torch.empty(cfg.C, cfg.d, dtype=torch.bfloat16, device=DEV)
    X = torch.full((cfg.C, cfg.d), -1.0, dtype=torch.bfloat16, device=DEV)
    acc = torch.empty(B, Cs, dtype=torch.uint8, device=DEV)
    n = torch.empty(B, dtype=torch.int32, device=DEV)
    tok = torch.empty(B, Cs, dtype=torch.int32, device=DEV)
    flag = torch.empty(B, dtype=torch.int32, device=DEV)
    dg_ctx.selfcond_accept(cfg, ws, Wd["E"], Wd["W1"], Wd["W2"], z, ent, 0.1, am, am, None, 5, 0, k, 0.005, cfg.N,
                           acc, n, tok, flag, x_next=X)
    dg_ctx.sync()
    t = tok.cpu().numpy().reshape(-1)
    e = O.from_bf16(W["E"][t]).astype(np.float32)
    ref = O.to_bf16(e + O.from_bf16(bits_np(z)).astype(np.float32))
    np.testing.assert_array_equal(bits_np(X), ref)
    # attention of one canvas on X against attention on (tokens, z)
    Kd, Vtd = upload_cache(Kp, Vp)
    cfg1 = cfg.with_(C=Cs)
    ws1 = ws_for(cfg1, Pcap)
    A1 = torch.empty(Cs, cfg.d, dtype=torch.bfloat16, device=DEV)
    A2 = torch.empty(Cs, cfg.d, dtype=torch.bfloat16, device=DEV)
    # the last canvas's rows, copied to 16-byte-aligned buffers
    t1, z1, X1 = tok[B - 1].clone(), z[(B - 1) * Cs:].clone(), X[(B - 1) * Cs:].clone()
    dg_ctx.canvas_attn(cfg1, t1, z1, Wd["E"], Wd["Wq"], Wd["Wk"], Wd["Wv"], Wd["Wo"], Kd, Vtd, cfg.P0, ws1, A1)
    dg_ctx.canvas_attn_x(cfg1, X1, Wd["Wq"], Wd["Wk"], Wd["Wv"], Wd["Wo"], Kd, Vtd, cfg.P0, ws1, A2)
    dg_ctx.sync()
    np.testing.assert_array_equal(bits_np(A2), bits_np(A1))


def test_selfcond_accept_refusals(dg_ctx):
    cfg, W, Kp, Vp, Pcap, Wd = setup("ragged")
    ws = ws_for(cfg, Pcap)
    H = bf16_dev(di.hidden(cfg, W["E"], 0, 0, di.targets(cfg, 0)))
    ent = torch.empty(cfg.C, dtype=torch.float32, device=DEV)
    am = torch.empty(cfg.C, dtype=torch.int32, device=DEV)
    dg_ctx.logits_entropy(cfg, H, Wd["E"], 0.8, ws, ent, am)
    z = torch.full((cfg.C, cfg.d), 1.0, dtype=torch.bfloat16, device=DEV)
    acc = torch.empty(cfg.C, dtype=torch.uint8, device=DEV)
    n = torch.empty(1, dtype=torch.int32, device=DEV)
    tok = torch.full((cfg.C,), -1, dtype=torch.int32, device=DEV)
    flag = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    # 3 canvases do not divide C = 100
    with pytest.raises(dg.DGError) as ei:
        dg_ctx.selfcond_accept(cfg, ws, Wd["E"], Wd["W1"], Wd["W2"], z, ent.view(1, -1).expand(3, -1).contiguous(),
                               0.1, am, am, None, 1, 0, 0, 0.005, 4, acc, n, tok, flag)
    assert ei.value.name == "DG_ERR_SHAPE"
    for kw, err in (({"b": -1.0}, "DG_ERR_RANGE"), ({"N": 0}, "DG_ERR_RANGE"), ({"step": -2}, "DG_ERR_RANGE")):
        a = {"b": 0.1, "N": 4, "step": 0, **kw}
        with pytest.raises(dg.DGError) as ei:
            dg_ctx.selfcond_accept(cfg, ws, Wd["E"], Wd["W1"], Wd["W2"], z, ent, a["b"], am, am, None, 1, 0,
                                   a["step"], 0.005, a["N"], acc, n, tok, flag)
        assert ei.value.name == err
    # a workspace without the sampler head's p0
    with pytest.raises(dg.DGError) as ei:
        dg_ctx.selfcond_accept(cfg, ws_for(cfg, Pcap), Wd["E"], Wd["W1"], Wd["W2"], z, ent, 0.1, am, am, None, 1,
                               0, 0, 0.005, 4, acc, n, tok, flag)
    assert ei.value.name == "DG_ERR_STATE"
    dg_ctx.sync()
    assert int(tok.min().item()) == -1 and int(flag.item()) == -1
    assert bool((z == 1.0).all().item())


def test_stop_flag_in_pinned_host_memory(dg_ctx):
    """The stop kernel's system-scope store reaches a pinned host flag without any copy:
    pre-filled with -1, the flag is polled until it changes, and it must equal both the
    oracle's flag and the device-memory result."""
    import time
    C, N = 256, 48
    rng = np.random.default_rng(43)
    for step in (0, 3, N - 1):
        hh = rng.exponential(0.002, C).astype(np.float32)
        am = rng.integers(0, 1000, C).astype(np.int32)
        prev = am.copy()
        if step == 3:
            prev[5] += 1
        host = torch.full((1,), -1, dtype=torch.int32, pin_memory=True)
        dev = torch.full((1,), -1, dtype=torch.int32, device=DEV)
        dg_ctx.stop_test(f32_dev(hh), i32_dev(am), i32_dev(prev), 0.005, step, N, host)
        dg_ctx.stop_test(f32_dev(hh), i32_dev(am), i32_dev(prev), 0.005, step, N, dev)
        deadline = time.monotonic() + 30.0
        while int(host[0]) < 0 and time.monotonic() < deadline:
            pass
        dg_ctx.sync()
        want = int(O.stop_test(hh, am, prev, 0.005, step, N)[0])
        assert int(host[0]) == int(dev.item()) == want


@pytest.mark.parametrize("name", ["tiny", "ragged", "hd64"])
def test_commit_kv(dg_ctx, name):
    cfg, W, Kp, Vp, Pcap, Wd = setup(name)
    rng = np.random.default_rng(51)
    tok = rng.integers(0, cfg.V, cfg.C).astype(np.int32)
    Kd, Vtd = upload_cache(Kp, Vp, Pcap)
    K0, V0 = bits_np(Kd), bits_np(Vtd)
    P2 = dg_ctx.commit_kv(cfg, i32_dev(tok), Wd["E"], Wd["Wk"], Wd["Wv"], Kd, Vtd, cfg.P0)
    dg_ctx.sync()
    assert P2 == cfg.P0 + cfg.C
    Ko, Vo = Kp.copy(), Vp.copy()
    O.commit_kv(tok, W["E"], W["Wk"], W["Wv"], Ko, Vo, cfg.P0, cfg.Hkv, cfg.hd)
    Kg, Vtg = bits_np(Kd), bits_np(Vtd)
    P0 = cfg.P0
    np.testing.assert_array_equal(Kg[:, :P0], K0[:, :P0])           # prefix untouched
    np.testing.assert_array_equal(Vtg[:, :, :P0], V0[:, :, :P0])
    np.testing.assert_array_equal(Kg[:, P2:], K0[:, P2:])           # beyond the block
    np.testing.assert_array_equal(Vtg[:, :, P2:], V0[:, :, P2:])
    for got, ref in ((O.from_bf16(Kg[:, P0:P2]), O.from_bf16(Ko[:, P0:P2])),
                     (O.from_bf16(Vtg[:, :, P0:P2].transpose(0, 2, 1)), O.from_bf16(Vo[:, P0:P2]))):
        assert maxrel(got, ref) <= 2e-2
        assert np.all(np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-30)   # <= 1 bf16 ulp


def test_determinism(dg_ctx):
    cfg, W, Kp, Vp, Pcap, Wd = setup("ragged")
    H = di.hidden(cfg, W["E"], 0, cfg.N - 1)
    outs = []
    for _ in range(2):
        ws = ws_for(cfg, Pcap)
        ent, am = run_head(dg_ctx, cfg, Wd, H, 0.4, ws)
        z = torch.empty(cfg.C, cfg.d, dtype=torch.bfloat16, device=DEV)
        dg_ctx.selfcond(cfg, ws, Wd["E"], Wd["W1"], Wd["W2"], z)
        Kd, Vtd = upload_cache(Kp, Vp, Pcap)
        A = torch.empty(cfg.C, cfg.d, dtype=torch.bfloat16, device=DEV)
        dg_ctx.canvas_attn(cfg, am, z, Wd["E"], Wd["Wq"], Wd["Wk"], Wd["Wv"], Wd["Wo"], Kd, Vtd,
                           cfg.P0, ws, A)
        dg_ctx.sync()
        outs.append([x.cpu().numpy().tobytes() for x in (ent, am, z.view(torch.int16), A.view(torch.int16))])
    assert outs[0] == outs[1]


@pytest.mark.parametrize("C", [256, 200])
def test_sampler_head_does_not_depend_on_the_canvas_block_width(dg_ctx, C):
    """At a 32768-token vocabulary one canvas runs the sampler head in 128-column blocks
    (256-column blocks would leave CUs idle), and the same canvas stacked with a second
    one runs it in 256-column blocks. Tile statistics are per (tile, column), so the
    entropy, argmax and confidence of the shared columns must agree bit for bit."""
    cfg = di.Config("blocks", V=32768, d=256, C=C, Hq=2, Hkv=1, hd=64, F=64, P0=0, N=4,
                    alpha_max=8.0, seed=27)
    W = di.weights(cfg)
    Wd = upload_weights(W)
    tgt = di.targets(cfg, 0)
    H1 = di.hidden(cfg, W["E"], 0, 1, tgt)
    H2 = di.hidden(cfg, W["E"], 1, 2, di.targets(cfg, 1))
    tau = O.temperature(1, cfg.N)
    outs = []
    for cf, H in ((cfg, H1), (cfg.with_(C=2 * C), np.concatenate([H1, H2], axis=0))):
        ws = torch.empty(dg.workspace_bytes(cf, 0), dtype=torch.uint8, device=DEV)
        ent, am = run_head(dg_ctx, cf, Wd, H, tau, ws)
        conf = torch.empty(cf.C, dtype=torch.float32, device=DEV)
        dg_ctx.confidence(cf, ws, conf)
        dg_ctx.sync()
        outs.append((ent.cpu().numpy()[:C], am.cpu().numpy()[:C], conf.cpu().numpy()[:C]))
    for a, b in zip(outs[0], outs[1]):
        np.testing.assert_array_equal(a, b)


def test_selfcond_does_not_depend_on_the_canvas_block_width(dg_ctx):
    """At a 32768-token vocabulary and d = 2048, a 128-position canvas runs the
    self-conditioning split in 128-column blocks (at most 128 columns padded in) and a
    256-position canvas, whose first 128 positions are the same, in 256-column blocks
    (8 model-width slices x 32 splits fill 256 CUs). The split count is 32 in both (it
    depends on the 256-column block count, 1 in both). Every element of s sums its
    split's vocabulary rows in the same order, and the FFW GEMMs do not depend on their
    tile shape, so the shared rows of z must agree bit for bit."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if 8 * 32 < cus:
        pytest.skip(f"{cus} CUs: the 256-position canvas would also take 128-column blocks")
    cfg = di.Config("blocks_sc", V=32768, d=2048, C=128, Hq=2, Hkv=1, hd=64, F=256, P0=0, N=4,
                    alpha_max=8.0, seed=28)
    W = di.weights(cfg)
    Wd = upload_weights(W)
    H1 = di.hidden(cfg, W["E"], 0, 1, di.targets(cfg, 0))
    H2 = di.hidden(cfg, W["E"], 1, 2, di.targets(cfg, 1))
    tau = O.temperature(1, cfg.N)
    outs = []
    for cf, H in ((cfg, H1), (cfg.with_(C=256), np.concatenate([H1, H2], axis=0))):
        ws = torch.empty(dg.workspace_bytes(cf, 0), dtype=torch.uint8, device=DEV)
        ent, am = run_head(dg_ctx, cf, Wd, H, tau, ws)
        z = torch.empty(cf.C, cf.d, dtype=torch.bfloat16, device=DEV)
        dg_ctx.selfcond(cf, ws, Wd["E"], Wd["W1"], Wd["W2"], z)
        dg_ctx.sync()
        outs.append(bits_np(z)[:128].copy())
    np.testing.assert_array_equal(outs[0], outs[1])


def test_gemm_results_do_not_depend_on_the_tile_shape(dg_ctx):
    """The projection GEMM picks its tile shape from the output size: committing 256
    tokens (1024 key and 1024 value features) runs 32 x 64 tiles, committing 512 runs
    64 x 64. Each output element takes the same k order and the same fixed sum over the
    workgroup's waves in both, so the first 256 rows must be bit-identical."""
    cfg = di.Config("shapes", V=4000, d=256, C=256, Hq=16, Hkv=8, hd=128, F=64, P0=8, N=4,
                    alpha_max=8.0, seed=28)
    W = di.weights(cfg)
    Wd = upload_weights(W)
    Pcap = cfg.P0 + 512
    Kp, Vp = di.prefix_kv(cfg, Pcap)
    tok = np.random.default_rng(5).integers(0, cfg.V, 512).astype(np.int32)
    rows = []
    for C in (256, 512):
        Kd, Vtd = upload_cache(Kp, Vp, Pcap)
        dg_ctx.commit_kv(cfg.with_(C=C), i32_dev(tok[:C]), Wd["E"], Wd["Wk"], Wd["Wv"], Kd, Vtd, cfg.P0)
        dg_ctx.sync()
        Kg, Vg = cache_logical(Kd, Vtd)
        rows.append((Kg[:, cfg.P0:cfg.P0 + 256].copy(), Vg[:, cfg.P0:cfg.P0 + 256].copy()))
    np.testing.assert_array_equal(rows[0][0], rows[1][0])
    np.testing.assert_array_equal(rows[0][1], rows[1][1])
