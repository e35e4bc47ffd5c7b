"""Pins of the CPU oracle against facts fixed outside it (no GPU).

Each test checks the oracle against something it cannot agree with by construction:
values the pages print (the sampler hyper-parameter table), closed forms, textbook /
library routines (numpy's Philox4x64-10, scipy's softmax and entropy, torch's bf16
conversion and scaled-dot-product attention), invariants, and brute force on tiny
inputs. A plausible slip in the oracle (a dropped term, a wrong sign or index, a
transposed operand, an off-by-one in the budget) fails at least one of them.
"""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special as sps
import torch

import oracle as O
from dg_inputs import f32_to_bf16_bits, bf16_bits_to_f32
import dg_inputs as di

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden_hparams():
    vals = {}
    with open(os.path.join(GOLDEN, "sampler_hparams.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                vals[k] = float(v)
    return vals


def bf16(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


# ------------------------------------------------------------------ bf16 rounding
def test_to_bf16_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 20000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, 1e-40], np.float32)])
    x = x.astype(np.float32)
    ours = O.to_bf16(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_to_bf16_ties_to_even_and_roundtrip():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1.0
    assert O.from_bf16(O.to_bf16(np.array([1.0 + 2 ** -8]))) == 1.0
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6: even mantissa is 1 + 2^-6
    assert O.from_bf16(O.to_bf16(np.array([1.0 + 3 * 2 ** -8]))) == 1.0 + 2 ** -6
    bits = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    np.testing.assert_array_equal(O.to_bf16(O.from_bf16(bits)), bits)


# ------------------------------------------------------------------ temperature
def test_temperature_endpoints_from_table():
    g = golden_hparams()
    N = int(g["max_steps"])
    assert O.temperature(0, N) == np.float32(g["temperature_start"])
    assert O.temperature(N - 1, N) == np.float32(g["temperature_end"])
    for n in range(2, 65):
        assert O.temperature(0, n) == np.float32(0.8)
        assert O.temperature(n - 1, n) == np.float32(0.4)
    assert O.temperature(0, 1) == np.float32(0.8)


def test_temperature_linear_equal_steps():
    N = 48
    taus = np.array([O.temperature(k, N) for k in range(N)], dtype=np.float64)
    steps = np.diff(taus)
    step = (0.4 - 0.8) / (N - 1)
    ulp = np.spacing(np.float32(0.8))
    assert np.all(steps < 0)
    assert np.max(np.abs(steps - step)) <= 2 * ulp


def test_default_hparams_are_the_tables():
    g = golden_hparams()
    import inspect
    sig = inspect.signature(O.run_canvas)
    assert sig.parameters["b"].default == g["entropy_bound"]
    assert sig.parameters["thr"].default == g["stop_mean_entropy"]
    assert sig.parameters["tau0"].default == g["temperature_start"]
    assert sig.parameters["tau1"].default == g["temperature_end"]
    from dg_inputs import config
    for i in (2, 3, 4):
        assert config(i).C == g["canvas_length"] and config(i).N == g["max_steps"]


# ------------------------------------------------------------------ entropy / argmax
def _head(H, E, tau):
    return O.logits_entropy(bf16(H), bf16(E), tau)


@pytest.mark.parametrize("V", [512, 32768])
def test_uniform_logits_give_log_v(V):
    d = 8
    E = np.random.default_rng(1).standard_normal((V, d))
    H = np.zeros((3, d))
    ent, am, p, _ = _head(H, E, 0.8)
    np.testing.assert_allclose(ent, math.log(V), rtol=1e-6)
    assert np.all(am == 0)                       # all tied -> lowest id
    np.testing.assert_allclose(p, 1.0 / V)


def test_uniform_logits_gemma_vocab_closed_form():
    # ln 262144 = 18 ln 2
    V = 262144
    E = np.ones((V, 4))
    ent, am, _, _ = _head(np.zeros((1, 4)), E, 0.4)
    assert abs(float(ent[0]) - 12.476649250079015) < 2e-6
    assert am[0] == 0


@pytest.mark.parametrize("gap", [0.0, 0.25, 1.0, 3.0])
@pytest.mark.parametrize("tau", [0.8, 0.4])
def test_two_token_closed_form(gap, tau):
    # logits (gap, 0): p = 1/(1+exp(-gap/tau)); H = -p ln p - (1-p) ln(1-p)
    E = np.array([[1.0], [0.0]])
    H = np.array([[gap]])
    ent, am, p, _ = _head(H, E, tau)
    t = float(np.float32(tau))
    pr = 1.0 / (1.0 + math.exp(-gap / t))
    ref = -pr * math.log(pr) - (1 - pr) * math.log(1 - pr)
    assert abs(float(ent[0]) - ref) < 1e-6
    assert am[0] == 0
    assert abs(p[0, 0] - pr) < 1e-12
    if gap == 0.0:
        assert abs(float(ent[0]) - math.log(2)) < 1e-7


def test_entropy_shift_invariance_and_tau_limits():
    rng = np.random.default_rng(2)
    V, d = 300, 6
    E = rng.standard_normal((V, d))
    H = rng.standard_normal((4, d))
    # append a constant column: every logit of a row shifts by the same amount
    E1 = np.concatenate([E, np.ones((V, 1))], axis=1)
    H1 = np.concatenate([H, np.full((4, 1), 5.0)], axis=1)
    H0 = np.concatenate([H, np.zeros((4, 1))], axis=1)
    a, am_a, _, _ = _head(H0, E1, 0.6)
    b, am_b, _, _ = _head(H1, E1, 0.6)
    np.testing.assert_allclose(a, b, atol=2e-6)
    np.testing.assert_array_equal(am_a, am_b)
    hot, _, _, _ = O.logits_entropy(bf16(H * 1e4), bf16(E), 1e-3)   # one-hot limit
    assert np.all(hot < 1e-6)
    flat, _, _, _ = O.logits_entropy(bf16(H), bf16(E), 1e30)         # tau -> inf
    np.testing.assert_allclose(flat, math.log(V), rtol=1e-6)


def test_entropy_matches_scipy_softmax_entr():
    rng = np.random.default_rng(3)
    V, d = 1000, 16
    Eb, Hb = bf16(rng.standard_normal((V, d))), bf16(3 * rng.standard_normal((8, d)))
    tau = np.float32(0.55)
    ent, am, p, u = O.logits_entropy(Hb, Eb, tau)
    logits = bf16_bits_to_f32(Hb).astype(np.float64) @ bf16_bits_to_f32(Eb).astype(np.float64).T
    sp = sps.softmax(logits / float(tau), axis=1)
    np.testing.assert_allclose(p, sp, rtol=1e-10, atol=1e-300)
    ref = sps.entr(sp).sum(axis=1)
    np.testing.assert_allclose(ent, ref, rtol=1e-6, atol=1e-7)
    np.testing.assert_array_equal(am, np.argmax(logits, axis=1))


def test_argmax_ties_lowest_id():
    E = np.array([[0.0], [1.0], [1.0], [0.5], [1.0]])
    ent, am, _, _ = _head(np.array([[2.0], [-2.0]]), E, 0.8)
    assert am[0] == 1          # ids 1, 2, 4 tie for the max
    assert am[1] == 0          # -2 * 0 = 0 is the max at id 0


# ------------------------------------------------------------------ acceptance
def _fixed(h):
    return O.entropy_fixed(np.float32(h))


def _brute_accept(h, b):
    """Max-cardinality subset with fixed-point sum <= floor(b 2^32); ties: min sum,
    then the lexicographically smallest (entropy, position) list."""
    C = len(h)
    budget = math.floor(float(np.float32(b)) * 2 ** 32)
    best = None
    for r in range(C, -1, -1):
        cands = []
        for S in itertools.combinations(range(C), r):
            s = sum(_fixed(h[i]) for i in S)
            if s <= budget:
                key = sorted((float(h[i]), i) for i in S)
                cands.append((s, key, S))
        if cands:
            best = min(cands)
            break
    acc = np.zeros(C, np.uint8)
    acc[list(best[2])] = 1
    return acc


def test_accept_brute_force_random():
    rng = np.random.default_rng(4)
    for trial in range(300):
        C = int(rng.integers(1, 11))
        scale = 10.0 ** rng.uniform(-3, 0)
        h = (rng.exponential(scale, C)).astype(np.float32)
        if trial % 5 == 0:           # force ties
            h[rng.integers(0, C, C // 2)] = h[0]
        b = np.float32(rng.choice([0.1, 0.05, 0.3, 0.0]))
        acc, n = O.entropy_accept(h[None], b)
        np.testing.assert_array_equal(acc[0], _brute_accept(h, b))
        assert n[0] == acc.sum()


def test_accept_budget_never_exceeded_real_and_fixed():
    rng = np.random.default_rng(5)
    h = rng.exponential(0.01, (50, 256)).astype(np.float32)
    acc, n = O.entropy_accept(h, 0.1)
    for s in range(50):
        sel = h[s][acc[s] == 1].astype(np.float64)
        assert sel.sum() <= float(np.float32(0.1)) + 0.0
        assert sum(_fixed(x) for x in h[s][acc[s] == 1]) <= 429496736
        # maximality: adding the cheapest rejected position would exceed the budget
        rej = h[s][acc[s] == 0]
        if len(rej):
            assert sum(_fixed(x) for x in sel.astype(np.float32)) + _fixed(rej.min()) > 429496736


def test_accept_special_cases():
    acc, n = O.entropy_accept(np.zeros((1, 16), np.float32), 0.1)
    assert acc.all() and n[0] == 16
    acc, n = O.entropy_accept(np.full((1, 16), 0.2, np.float32), 0.1)
    assert not acc.any() and n[0] == 0
    # exact boundary: 3 x 0.05f -> q = 214748368 each, two sum to 429496736 == floor(0.1f 2^32)
    assert _fixed(0.05) == 214748368
    assert math.floor(float(np.float32(0.1)) * 2 ** 32) == 429496736
    acc, n = O.entropy_accept(np.full((1, 3), 0.05, np.float32), 0.1)
    assert n[0] == 2 and list(acc[0]) == [1, 1, 0]   # position order breaks the tie
    # NaN and out-of-domain entropies are never accepted, even with a huge budget
    h = np.array([[np.nan, 0.0, np.inf, 70000.0, 0.01]], np.float32)
    acc, n = O.entropy_accept(h, 60000.0)
    assert list(acc[0]) == [0, 1, 0, 0, 1]
    # negative entropy counts as zero
    acc, n = O.entropy_accept(np.array([[-1.0, 0.1]], np.float32), 0.1)
    assert list(acc[0]) == [1, 1]


def test_accept_monotone():
    rng = np.random.default_rng(6)
    for _ in range(100):
        h = rng.exponential(0.03, 12).astype(np.float32)
        acc, _ = O.entropy_accept(h[None], 0.1)
        i = int(rng.integers(0, 12))
        if acc[0, i]:
            h2 = h.copy()
            h2[i] = np.float32(h[i] * rng.uniform(0, 1))
            acc2, _ = O.entropy_accept(h2[None], 0.1)
            assert acc2[0, i] == 1


def test_accept_tiny_vocab_enumeration():
    # V in {2, 3}, C <= 6: enumerate logit rows on a grid, entropies from the oracle's
    # head, acceptance against brute force.
    for V in (2, 3):
        grid = [-2.0, 0.0, 1.5, 6.0]
        rows = np.array(list(itertools.product(grid, repeat=V)))
        E = np.eye(V)
        ent, _, _, _ = O.logits_entropy(bf16(rows), bf16(E), 0.4)
        rng = np.random.default_rng(V)
        for _ in range(60):
            C = int(rng.integers(1, 7))
            h = ent[rng.integers(0, len(rows), C)]
            for b in (0.1, 0.02):
                acc, _ = O.entropy_accept(h[None], b)
                np.testing.assert_array_equal(acc[0], _brute_accept(h, b))


def test_accept_segments_independent():
    rng = np.random.default_rng(7)
    h = rng.exponential(0.02, (3, 20)).astype(np.float32)
    acc, n = O.entropy_accept(h, 0.1)
    for s in range(3):
        a1, n1 = O.entropy_accept(h[s:s + 1], 0.1)
        np.testing.assert_array_equal(acc[s], a1[0])


# ------------------------------------------------------------------ Philox / renoise
def test_philox_matches_numpy():
    # numpy's Philox(counter=c) emits the block of counter c + 1 first.
    rng = np.random.default_rng(8)
    for _ in range(20):
        key = [int(x) for x in rng.integers(0, 2 ** 63, 2)]
        ctr = [int(x) for x in rng.integers(0, 2 ** 63, 4)]
        g = np.random.Philox(key=np.array(key, np.uint64), counter=np.array(ctr, np.uint64))
        want = [int(x) for x in g.random_raw(4)]
        nxt = list(ctr)
        nxt[0] += 1
        assert list(O.philox4x64_10(nxt, key)) == want


def test_philox_published_known_answer():
    # Random123 known-answer vector for philox4x64_10 with zero counter and key.
    assert O.philox4x64_10((0, 0, 0, 0), (0, 0)) == (
        0x16554D9ECA36314C, 0xDB20FE9D672D0FDC, 0xD7E772CEE186176B, 0x7E68B68AEC7BA23B)


def test_renoise_keeps_accepted_and_draws_rest():
    am = np.arange(10, dtype=np.int32)[None] * 3
    acc = np.array([[1, 0, 1, 0, 0, 1, 1, 0, 0, 1]], np.uint8)
    x = O.renoise(am, acc, seed=11, canvas_base=2, step=5, V=512)
    for i in range(10):
        if acc[0, i]:
            assert x[0, i] == am[0, i]
        else:
            r = O.philox4x64_10((i, 5, O.STREAM_RENOISE, 0), (11, 2))[0]
            assert x[0, i] == r >> (64 - 9)              # power-of-two V: top 9 bits
    assert np.array_equal(x, O.renoise(am, acc, 11, 2, 5, 512))   # deterministic
    init = O.renoise(am, None, 11, 2, 0, 512)
    for i in range(10):
        r = O.philox4x64_10((i, 0, O.STREAM_INIT, 0), (11, 2))[0]
        assert init[0, i] == r >> 55


def test_renoise_uniform_chi2():
    for V in (2, 3, 512):
        n = 20000 if V < 512 else 51200
        toks = np.array([O.uniform_token(123, 0, 3, 0, i, V) for i in range(n)])
        assert toks.min() >= 0 and toks.max() < V
        counts = np.bincount(toks, minlength=V)
        chi2 = ((counts - n / V) ** 2 / (n / V)).sum()
        p = 1 - __import__("scipy.stats").stats.chi2.cdf(chi2, V - 1)
        assert p > 1e-4, (V, chi2)


def test_renoise_segments_use_canvas_id():
    am = np.zeros((2, 4), np.int32)
    acc = np.zeros((2, 4), np.uint8)
    x = O.renoise(am, acc, 5, 7, 1, 1000)
    np.testing.assert_array_equal(x[1], O.renoise(am[1:], acc[1:], 5, 8, 1, 1000)[0])


# ------------------------------------------------------------------ self-conditioning
def test_gelu_points():
    xs = np.array([-3.0, -1.0, -0.1, 0.0, 0.5, 2.0])
    ref = [x * 0.5 * (1 + math.erf(x / math.sqrt(2))) for x in xs]
    np.testing.assert_allclose(O.gelu_erf(xs), ref, rtol=1e-15, atol=1e-300)
    assert O.gelu_erf(np.array([0.0]))[0] == 0.0
    # Phi(1) = 0.8413447460685429 (normal CDF table value)
    assert abs(O.gelu_erf(np.array([1.0]))[0] - 0.8413447460685429) < 1e-15


def test_selfcond_projection_pins():
    rng = np.random.default_rng(9)
    V, d, F = 40, 8, 12
    E = bf16(rng.standard_normal((V, d)))
    W1, W2 = bf16(rng.standard_normal((F, d))), bf16(rng.standard_normal((d, F)))
    onehot = np.zeros((3, V))
    onehot[[0, 1, 2], [5, 0, 39]] = 1.0
    _, aux = O.selfcond(onehot, E, W1, W2)
    np.testing.assert_array_equal(aux["s"], bf16_bits_to_f32(E)[[5, 0, 39]].astype(np.float64))
    uni = np.full((1, V), 1.0 / V)
    _, aux = O.selfcond(uni, E, W1, W2)
    np.testing.assert_allclose(aux["s"][0], bf16_bits_to_f32(E).astype(np.float64).mean(axis=0), rtol=1e-12)
    p1, p2 = rng.dirichlet(np.ones(V), 2)
    _, a1 = O.selfcond(p1[None], E, W1, W2)
    _, a2 = O.selfcond(p2[None], E, W1, W2)
    _, a12 = O.selfcond((0.3 * p1 + 0.7 * p2)[None], E, W1, W2)
    np.testing.assert_allclose(a12["s"], 0.3 * a1["s"] + 0.7 * a2["s"], rtol=1e-12, atol=1e-14)
    z, _ = O.selfcond(uni, E, W1, np.zeros_like(W2))
    assert not z.any()
    # FFW orientation: torch Linear layers with the same weights
    lin1 = torch.nn.functional.linear(torch.from_numpy(a1["s"]), torch.from_numpy(bf16_bits_to_f32(W1).astype(np.float64)))
    g = torch.nn.functional.gelu(lin1)
    out = torch.nn.functional.linear(g, torch.from_numpy(bf16_bits_to_f32(W2).astype(np.float64)))
    z1, _ = O.selfcond(p1[None], E, W1, W2)
    np.testing.assert_array_equal(z1, torch.from_numpy(out.numpy().astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


# ------------------------------------------------------------------ stop test
def test_stop_hand_cases():
    C, N = 256, 48
    am = np.arange(C, dtype=np.int32)
    h = np.full(C, 0.005, np.float32)
    assert _fixed(0.005) == 21474836
    assert math.floor(float(np.float32(0.005)) * C * 2 ** 32) == 5497558016
    assert O.stop_test(h, am, am, 0.005, 3, N)[0] == O.STOP_STOP           # inclusive
    h2 = h.copy()
    h2[7] = np.nextafter(np.float32(0.005), np.float32(1))
    assert O.stop_test(h2, am, am, 0.005, 3, N)[0] == O.STOP_GO            # +1 ulp
    am2 = am.copy()
    am2[100] += 1
    assert O.stop_test(h, am2, am, 0.005, 3, N)[0] == O.STOP_GO            # argmax moved
    assert O.stop_test(h, am, None, 0.005, 0, N)[0] == O.STOP_GO           # k = 0
    assert O.stop_test(h, am, am, 0.005, 0, N)[0] == O.STOP_GO
    assert O.stop_test(h2, am, am, 0.005, N - 1, N)[0] == O.STOP_CAP       # cap
    assert O.stop_test(h, am, am, 0.005, N - 1, N)[0] == O.STOP_STOP
    h3 = np.zeros(C, np.float32)
    h3[0] = np.nan
    assert O.stop_test(h3, am, am, 0.005, 3, N)[0] == O.STOP_GO            # NaN blocks
    # the mean, not the max: one high entropy balanced by zeros still stops
    h4 = np.zeros(C, np.float32)
    h4[0] = np.float32(0.005 * C * 0.999)
    assert O.stop_test(h4, am, am, 0.005, 5, N)[0] == O.STOP_STOP


def test_stop_segments():
    h = np.zeros((2, 16), np.float32)
    h[1, 3] = 1.0
    am = np.zeros((2, 16), np.int32)
    f = O.stop_test(h, am, am, 0.005, 2, 8)
    assert list(f) == [1, 0]


# ------------------------------------------------------------------ attention
def _attn_setup(C=12, P=10, Hq=4, Hkv=2, hd=8, d=16, V=50, seed=10):
    rng = np.random.default_rng(seed)
    E = bf16(rng.standard_normal((V, d)) / 4)
    W = {n: bf16(rng.standard_normal(s) / 4) for n, s in
         (("Wq", (Hq * hd, d)), ("Wk", (Hkv * hd, d)), ("Wv", (Hkv * hd, d)), ("Wo", (d, Hq * hd)))}
    Kp = bf16(rng.standard_normal((Hkv, P + C, hd)))
    Vp = bf16(rng.standard_normal((Hkv, P + C, hd)))
    tok = rng.integers(0, V, C).astype(np.int32)
    z = bf16(rng.standard_normal((C, d)) / 8)
    return E, W, Kp, Vp, tok, z


def _attn(tok, z, E, W, Kp, Vp, P, Hq=4, Hkv=2, hd=8):
    return O.canvas_attn(tok, z, E, W["Wq"], W["Wk"], W["Wv"], W["Wo"], Kp, Vp, P, Hq, Hkv, hd)


def test_attention_permutation_equivariant():
    E, W, Kp, Vp, tok, z = _attn_setup()
    A, aux = _attn(tok, z, E, W, Kp, Vp, 10)
    perm = np.random.default_rng(1).permutation(len(tok))
    A2, aux2 = _attn(tok[perm], z[perm], E, W, Kp, Vp, 10)
    np.testing.assert_allclose(aux2["O"], aux["O"][perm], rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(A2, A[perm])


def test_attention_empty_prefix_is_full_attention_torch():
    E, W, Kp, Vp, tok, z = _attn_setup()
    A, aux = _attn(tok, z, E, W, Kp, Vp, 0)
    q = torch.from_numpy(aux["Q"]).permute(1, 0, 2)[None]             # [1, Hq, C, hd]
    k = torch.from_numpy(aux["Kc"]).permute(1, 0, 2).repeat_interleave(2, dim=0)[None]
    v = torch.from_numpy(aux["Vc"]).permute(1, 0, 2).repeat_interleave(2, dim=0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v)     # no mask
    np.testing.assert_allclose(aux["O"], ref[0].permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def test_attention_prefix_matches_torch_with_concat():
    E, W, Kp, Vp, tok, z = _attn_setup(seed=12)
    P = 10
    A, aux = _attn(tok, z, E, W, Kp, Vp, P)
    kp = torch.from_numpy(O.from_bf16(Kp[:, :P]))
    vp = torch.from_numpy(O.from_bf16(Vp[:, :P]))
    k = torch.cat([kp, torch.from_numpy(aux["Kc"]).permute(1, 0, 2)], dim=1).repeat_interleave(2, 0)
    v = torch.cat([vp, torch.from_numpy(aux["Vc"]).permute(1, 0, 2)], dim=1).repeat_interleave(2, 0)
    q = torch.from_numpy(aux["Q"]).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None])[0]
    np.testing.assert_allclose(aux["O"], ref.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)
    # the denoiser input is E[x] + z rounded to bf16
    np.testing.assert_array_equal(aux["X"], O.from_bf16(O.to_bf16(O.from_bf16(E[tok]) + O.from_bf16(z))))
    # Q is X Wq^T (nn.Linear orientation), rounded to bf16
    ql = torch.nn.functional.linear(torch.from_numpy(aux["X"]), torch.from_numpy(O.from_bf16(W["Wq"])))
    np.testing.assert_array_equal(O.to_bf16(ql.numpy()).reshape(aux["Q"].shape), O.to_bf16(aux["Q"]))


def test_attention_single_key_and_identical_keys():
    E, W, Kp, Vp, tok, z = _attn_setup(C=1, P=0)
    _, aux = _attn(tok, z, E, W, Kp, Vp, 0)
    # one key: the output is that key's value row for every head of its group
    for h in range(4):
        np.testing.assert_allclose(aux["O"][0, h], aux["Vc"][0, h // 2], rtol=1e-14)
    # identical keys: uniform weights -> mean of the values
    E, W, Kp, Vp, tok, z = _attn_setup(C=6, P=8)
    Kp[:] = Kp[:, :1]
    W2 = dict(W)
    W2["Wk"] = np.zeros_like(W["Wk"])          # canvas keys = 0, prefix keys equal
    Kp[:] = 0
    _, aux = _attn(tok, z, E, W2, Kp, Vp, 8)
    for h in range(4):
        g = h // 2
        allv = np.concatenate([O.from_bf16(Vp[g, :8]), aux["Vc"][:, g]])
        np.testing.assert_allclose(aux["O"][:, h], np.broadcast_to(allv.mean(0), (6, 8)), rtol=1e-12)


def test_attention_mha_when_hq_equals_hkv():
    E, W, Kp, Vp, tok, z = _attn_setup(Hq=2, Hkv=2)
    _, aux = O.canvas_attn(tok, z, E, W["Wq"][:16], W["Wk"], W["Wv"], W["Wo"][:, :16], Kp, Vp, 10, 2, 2, 8)
    for h in range(2):
        K = np.concatenate([O.from_bf16(Kp[h, :10]), aux["Kc"][:, h]])
        V = np.concatenate([O.from_bf16(Vp[h, :10]), aux["Vc"][:, h]])
        np.testing.assert_allclose(aux["O"][:, h], O.attention_rows(aux["Q"][:, h], K, V, 8), rtol=1e-12)


# ------------------------------------------------------------------ commit
def test_commit_rows_and_capacity():
    rng = np.random.default_rng(13)
    V, d, Hkv, hd, C, P = 30, 16, 2, 8, 5, 7
    E = bf16(rng.standard_normal((V, d)))
    Wk, Wv = bf16(rng.standard_normal((Hkv * hd, d))), bf16(rng.standard_normal((Hkv * hd, d)))
    Kp = bf16(rng.standard_normal((Hkv, P + C, hd)))
    Vp = bf16(rng.standard_normal((Hkv, P + C, hd)))
    K0, V0 = Kp.copy(), Vp.copy()
    tok = rng.integers(0, V, C).astype(np.int32)
    P2 = O.commit_kv(tok, E, Wk, Wv, Kp, Vp, P, Hkv, hd)
    assert P2 == P + C
    np.testing.assert_array_equal(Kp[:, :P], K0[:, :P])
    np.testing.assert_array_equal(Vp[:, :P], V0[:, :P])
    Ef = torch.from_numpy(bf16_bits_to_f32(E[tok]).astype(np.float64))
    kref = torch.nn.functional.linear(Ef, torch.from_numpy(bf16_bits_to_f32(Wk).astype(np.float64)))
    kref = kref.float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).reshape(C, Hkv, hd)
    np.testing.assert_array_equal(Kp[:, P:P + C], kref.transpose(1, 0, 2))
    with pytest.raises(ValueError):
        O.commit_kv(tok, E, Wk, Wv, Kp, Vp, P + 1, Hkv, hd)


def test_attention_row_restriction_matches_full():
    """canvas_attn(rows=r) returns exactly the rows r of the full computation."""
    cfg = di.config(0)
    W = di.weights(cfg)
    Kp, Vp = di.prefix_kv(cfg)
    rng = np.random.default_rng(7)
    tok = rng.integers(0, cfg.V, cfg.C).astype(np.int32)
    z = di.f32_to_bf16_bits(rng.standard_normal((cfg.C, cfg.d)).astype(np.float32) * 0.3)
    A, _ = O.canvas_attn(tok, z, W["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], Kp, Vp, cfg.P0,
                         cfg.Hq, cfg.Hkv, cfg.hd)
    rows = [0, 5, 15]
    Ar, _ = O.canvas_attn(tok, z, W["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], Kp, Vp, cfg.P0,
                          cfg.Hq, cfg.Hkv, cfg.hd, rows=rows)
    np.testing.assert_array_equal(Ar, A[rows])
