"""Plain CPU oracle for one DiffusionGemma canvas-denoise step and its block-AR chain.

TEST INFRASTRUCTURE ONLY. Nothing in the product library calls, imports or links this
module; only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it. It shares no code with the HIP path: it has its own bf16
rounding, its own Philox and its own fixed-point acceptance, written from the pages.

Everything is numpy float64 over the same bf16-rounded inputs the GPU receives (bf16 is
carried as uint16 bits). It rounds to bf16 only where the method's data crosses a bf16
storage boundary: the denoiser input X = E[x] + z, the projected Q/K/V, the attention
output A, the self-conditioning vector z and the committed K/V rows.

Sources (web pages on DiffusionGemma):
  [TR]  "DiffusionGemma Technical Report" summary (paper.rainbus.top/paper/2608.00146),
        section "Method steps" (inference steps (1)-(5)), section "Prerequisites /
        Self-conditioning", section "Reproducibility" (the sampler hyper-parameter table).
  [TUT] Tutorial chapter "DiffusionGemma" (papers-3lj.pages.dev, diffusion docs ch. 12),
        the data-flow pseudocode, the sampler configuration (temperature 0.8 -> 0.4,
        linear), the KV-cache write timing and the per-phase attention masks.
  [GGL] Google "DiffusionGemma explained" (ai.google.dev), sections "Uniform State
        Diffusion", "Architecture: incremental prefill and denoising", "Self-conditioning",
        "Multi-canvas sampling".
  [SRV] "Text diffusion models" survey (papers.franksyz.com), section 11 (DiffusionGemma
        defaults: 48 steps, entropy bound 0.1, temperature 0.8 -> 0.4), section 5 (reverse
        generation: predict, select, accept, remask).
  [MOE] the DiffusionGemma Technical Report page, section "Prerequisites" (mixture of
        experts: 8 of 128 experts plus one shared expert per token; about 84 distinct
        experts active per canvas against 8 per token), and the survey's section 11
        (128 experts per layer, 8 routed, 1 shared) and section 13 (router top-k, expert
        GEMM, token permutation).
  [HUB] openai-hub page "从零拆开DiffusionGemma" (news 2086), step 4 (confidence decoding:
        predict every position, keep the most confident ones, the simplified decoder's
        reveal count ceil(unresolved / remaining steps)); the closing remarks of step 3
        (the full model adds MoE layers, rotary position encoding, prompt prefill and a KV
        cache to the teaching model).

Readings taken where the pages leave a step open (each restated where it is used):
  * temperature: tau_k = tau0 + (tau1 - tau0) * k / (N - 1) over the step budget N,
    computed in float64 and passed on as float32 (N = 1 gives tau0);
  * p^0 is the softmax of logits / tau_k; entropy is Shannon entropy in nats;
  * the accepted token is argmax p^0 (x^0), ties to the lowest vocabulary id;
  * acceptance sorts positions by (entropy, position) ascending and accepts the longest
    prefix whose entropy sum stays within b, summed in 2^-32 fixed point
    (q = ceil(h * 2^32), budget floor(b * 2^32)); zero accepted positions is legal;
  * every non-accepted position is redrawn uniformly over the whole vocabulary from
    Philox4x64-10 keyed by (seed, canvas) with counter (position, step, stream, 0);
  * self-conditioning: z = W2 . GELU_erf(W1 . (p^0 E)), no bias, next input X = E[x] + z;
  * stop: step >= 1, sum of q <= floor(thr * C * 2^32) and argmax unchanged from the
    previous step; otherwise the step cap N - 1 commits anyway;
  * commit: the finalized block is x^0 = argmax at the stopping step; its K/V rows are
    E[x^0] Wk^T and E[x^0] Wv^T (stand-in for the causal re-encode), appended at [P, P+C).
  * sampled tokens (an alternative to x^0 = argmax): x~ ~ p^0 drawn by inverse CDF over
    the whole vocabulary with one Philox uniform per position; accepted positions and
    the commit take x~, the stop test still compares argmaxes;
  * the commit as a causal re-encode (an alternative to the projection stand-in): one
    attention layer over the prefix and the block's earlier tokens, with rotary positions
    when a base is given, appends the block's rotated K and its V;
  * the confidence rule (an alternative to the entropy budget): a position's confidence
    is its largest tempered probability; step k accepts the n_k most confident positions
    (ties to the lower position, NaN never), n_k the number the [HUB] decoder has revealed
    after step k; accepted positions keep x^0, the rest are renoised as above, and every
    position is ranked afresh each step.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf

TWO32 = 1 << 32
# Entropies at or above this bound (and NaN/Inf) are outside the sampler's domain
# (a valid entropy never exceeds ln V); they are never accepted and block the stop.
H_LIMIT = 65536.0
Q_SENTINEL = 1 << 48


# ------------------------------------------------------------------ bf16 storage
def from_bf16(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 values (exact). A float64 array is taken as values
    already converted (callers may convert a large table such as E once)."""
    if isinstance(bits, np.ndarray) and bits.dtype == np.float64:
        return bits
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def to_bf16(x) -> np.ndarray:
    """float64 -> bf16 bits, rounding once to nearest with ties to even.

    bf16 keeps 8 significant bits: the quantum of a value with binary exponent e
    (x = f * 2^e, 0.5 <= |f| < 1) is 2^(e-8), never finer than the subnormal quantum
    2^-133. Values past the largest bf16 become infinities.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    y = np.rint(x / q) * q                      # numpy rint rounds half to even
    with np.errstate(over="ignore"):
        y32 = y.astype(np.float32)              # y is exactly representable (or inf)
    return (np.ascontiguousarray(y32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ------------------------------------------------------------------ (a1) temperature
def temperature(k: int, N: int, tau0: float = 0.8, tau1: float = 0.4) -> np.float32:
    """Linearly annealed sampling temperature for denoise step k of a budget of N.

    [TUT] sampler configuration: logits are divided by a temperature that decreases
    linearly from 0.8 to 0.4; [TR] "Method steps" (3). Endpoints are the float32 values
    0.8f at k = 0 and 0.4f at k = N - 1.
    """
    t0 = float(np.float32(tau0))
    t1 = float(np.float32(tau1))
    if N <= 1:
        return np.float32(t0)
    return np.float32(t0 + (t1 - t0) * k / (N - 1))


# ------------------------------------------------------------------ (a2-a4) attention
def rope(x, positions, base):
    """Rotary position embedding, half-split pairing: for d < hd/2 the pair
    (x_d, x_{d+hd/2}) is rotated by the angle pos * base^(-2d/hd). base 0 is the identity.
    [HUB] names rotary position encoding as part of the full model; the pairing and the
    base are readings (the Gemma family's convention). x float64 [n, H, hd]."""
    if not base:
        return x
    n, H, hd = x.shape
    h = hd // 2
    theta = float(base) ** (-2.0 * np.arange(h) / hd)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def canvas_attn(tokens, z_bits, E_bits, Wq, Wk, Wv, Wo, Kp, Vp, P, Hq, Hkv, hd, rows=None,
                rope_base=0.0):
    """Bidirectional canvas attention over the static prefix KV cache, then Wo.

    [GGL] "Architecture": in denoise mode a query at any canvas position attends to all
    other canvas tokens and to the KV cache (no mask). [TUT] pseudocode: the denoiser
    input is embed(canvas) + self_conditioning. Head h reads KV head floor(h*Hkv/Hq).
    No positional encoding, soft-cap or bias (none is named for the canvas pass).

    tokens [C] int; z_bits [C, d] bf16 or None (z = 0); E_bits [V, d]; Wq [Hq*hd, d];
    Wk, Wv [Hkv*hd, d]; Wo [d, Hq*hd]; Kp, Vp [Hkv, >=P, hd] bf16 (logical layout).
    ``rows`` restricts the queries (and the returned A) to those canvas positions; the
    keys and values still come from every canvas token. rope_base > 0 rotates the canvas
    queries and keys at their token positions P + i (the prefix keys are stored rotated).
    Returns (A bits [C or len(rows), d], dict of intermediates as float64).
    """
    tokens = np.asarray(tokens)
    C = tokens.shape[0]
    Ex = from_bf16(E_bits[tokens])
    z = 0.0 if z_bits is None else from_bf16(z_bits)
    X = from_bf16(to_bf16(Ex + z))
    Xq = X if rows is None else X[np.asarray(rows)]
    nq = Xq.shape[0]
    Q = from_bf16(to_bf16(Xq @ from_bf16(Wq).T)).reshape(nq, Hq, hd)
    Kc = from_bf16(to_bf16(X @ from_bf16(Wk).T)).reshape(C, Hkv, hd)
    Vc = from_bf16(to_bf16(X @ from_bf16(Wv).T)).reshape(C, Hkv, hd)
    if rope_base:
        qpos = P + (np.arange(C) if rows is None else np.asarray(rows))
        Q = from_bf16(to_bf16(rope(Q, qpos, rope_base)))
        Kc = from_bf16(to_bf16(rope(Kc, P + np.arange(C), rope_base)))
    O = np.zeros((nq, Hq, hd))
    scale = 1.0 / math.sqrt(hd)
    for h in range(Hq):
        g = (h * Hkv) // Hq
        K = np.concatenate([from_bf16(Kp[g, :P]), Kc[:, g]], axis=0)
        V = np.concatenate([from_bf16(Vp[g, :P]), Vc[:, g]], axis=0)
        S = (Q[:, h] @ K.T) * scale
        S = S - S.max(axis=1, keepdims=True)
        W = np.exp(S)
        W /= W.sum(axis=1, keepdims=True)
        O[:, h] = W @ V
    A = to_bf16(O.reshape(nq, Hq * hd) @ from_bf16(Wo).T)
    return A, {"X": X, "Q": Q, "Kc": Kc, "Vc": Vc, "O": O}


def attention_rows(Q_rows, K, V, hd):
    """softmax(Q K^T / sqrt(hd)) V for a few query rows (used for sampled checks)."""
    S = (Q_rows @ K.T) / math.sqrt(hd)
    S = S - S.max(axis=1, keepdims=True)
    W = np.exp(S)
    return (W / W.sum(axis=1, keepdims=True)) @ V


# ------------------------------------------------------------------ (a5) sampler head
def logits_entropy(H_bits, E_bits, tau, rows=None):
    """Logits, tempered softmax p^0, per-position entropy (nats) and argmax.

    [TR] "Method steps" (3): the decoder's logits L_t go through a softmax at the
    annealed temperature tau_t giving p^0; positions are then ranked by entropy.
    u = (H E^T) / tau; p = exp(u - max u) / Z; H(p) = ln Z - sum p (u - max u), clamped
    at 0 and stored as float32. argmax ties go to the lowest vocabulary id.

    Returns (entropy f32 [C], argmax int32 [C], p float64 [C, V], u float64 [C, V]).
    ``rows`` restricts the computation to those canvas positions.
    """
    H = from_bf16(H_bits if rows is None else np.asarray(H_bits)[rows])
    E = from_bf16(E_bits)
    u = (H @ E.T) / float(np.float32(tau))
    m = u.max(axis=1, keepdims=True)
    e = np.exp(u - m)
    Z = e.sum(axis=1)
    S = (e * (u - m)).sum(axis=1)
    ent = np.maximum(np.log(Z) - S / Z, 0.0).astype(np.float32)
    am = np.argmax(u, axis=1).astype(np.int32)   # first maximal index = lowest id
    p = e / Z[:, None]
    return ent, am, p, u


# ------------------------------------------------------------------ (a6) acceptance
def entropy_fixed(h) -> int:
    """2^-32 fixed-point entropy used for budget sums: ceil(h * 2^32).

    h*2^32 is exact in float64 for a float32 h. Out-of-domain entropies (NaN, Inf,
    >= 2^16) map to a sentinel larger than any admissible budget; negatives count as 0.
    """
    h = float(h)
    if not (h < H_LIMIT):          # NaN, +Inf, too large
        return Q_SENTINEL
    if h <= 0.0:
        return 0
    return math.ceil(h * TWO32)


def _sort_key(h, i):
    h = float(h)
    valid = h < H_LIMIT
    return (0 if valid else 1, max(h, 0.0) if valid else 0.0, i)


def entropy_accept(entropy, b):
    """Entropy-bounded acceptance for B segments of C positions.

    [TR] "Method steps" (3): sort positions by entropy from small to large and accept
    them while the cumulative entropy stays within the budget b = 0.1; the rest are
    renoised. [TR] "Technical novelty": entropy-bounded acceptance, similar to MaskGIT.
    Reading: the accepted set is the longest prefix of the (entropy, position) order
    whose fixed-point sum is <= floor(b * 2^32) (inclusive); an empty set is legal.

    entropy float32 [B, C] -> (accept uint8 [B, C], n_accept int32 [B]).
    """
    ent = np.asarray(entropy, dtype=np.float32)
    if ent.ndim == 1:
        ent = ent[None]
    B, C = ent.shape
    budget = math.floor(float(np.float32(b)) * TWO32)
    accept = np.zeros((B, C), dtype=np.uint8)
    n_acc = np.zeros(B, dtype=np.int32)
    for s in range(B):
        order = sorted(range(C), key=lambda i: _sort_key(ent[s, i], i))
        total = 0
        for i in order:
            q = entropy_fixed(ent[s, i])
            if total + q > budget:
                break
            total += q
            accept[s, i] = 1
            n_acc[s] += 1
    return accept, n_acc


# ------------------------------------------------------------------ confidence rule
def confidence(H_bits, E_bits, tau, rows=None):
    """Confidence of every position: its largest tempered probability max_v p^0[c][v].

    [HUB] step 4: the decoder computes probs = softmax(logits / temperature) and takes
    (confidence, candidates) = probs.max(-1). Stored as float32.
    """
    _, _, p, _ = logits_entropy(H_bits, E_bits, tau, rows)
    return p.max(axis=1).astype(np.float32)


def reveal_schedule(C: int, N: int):
    """Number of positions revealed after each step of confidence decoding.

    [HUB] step 4: each step reveals ceil(unresolved / remaining steps) positions, so the
    count after step t is n_t = n_{t-1} + ceil((C - n_{t-1}) / (N - t)) with n_{-1} = 0.
    Returns [n_0, ..., n_{N-1}]; n_{N-1} = C.
    """
    out = []
    n = 0
    for t in range(N):
        n += -(-(C - n) // (N - t))
        out.append(n)
    return out


def topk_accept(score, k):
    """Accept the k highest-scoring positions of each of B segments.

    Order: score descending, then position ascending (equal scores go to the lower
    position; -0.0 counts as below +0.0, the order of their bit patterns); NaN scores
    are never accepted. score float32 [B, C] -> (accept uint8 [B, C], n_accept int32 [B]).
    """
    sc = np.asarray(score, dtype=np.float32)
    if sc.ndim == 1:
        sc = sc[None]
    B, C = sc.shape
    accept = np.zeros((B, C), dtype=np.uint8)
    n_acc = np.zeros(B, dtype=np.int32)
    for s in range(B):
        valid = [i for i in range(C) if not math.isnan(float(sc[s, i]))]
        # value descending; for equal values +0.0 before -0.0; then position ascending
        order = sorted(valid, key=lambda i: (-float(sc[s, i]), math.copysign(1.0, float(sc[s, i])) < 0, i))
        for i in order[:max(0, int(k))]:
            accept[s, i] = 1
            n_acc[s] += 1
    return accept, n_acc


# ------------------------------------------------------------------ (a7, a11) renoise
_M0, _M1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157      # Philox4x64 multipliers
_W0, _W1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B      # Weyl key increments
_MASK64 = (1 << 64) - 1


def philox4x64_10(counter, key):
    """Philox4x64 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel random numbers:
    as easy as 1, 2, 3", SC'11): each round multiplies words 0 and 2 by the two
    multipliers, swaps the high halves crosswise into the odd words XORed with the key,
    and the key is bumped by the Weyl constants between rounds."""
    c0, c1, c2, c3 = (int(x) & _MASK64 for x in counter)
    k0, k1 = (int(x) & _MASK64 for x in key)
    for _ in range(10):
        p0 = _M0 * c0
        p1 = _M1 * c2
        c0, c1, c2, c3 = ((p1 >> 64) ^ c1 ^ k0, p1 & _MASK64,
                          (p0 >> 64) ^ c3 ^ k1, p0 & _MASK64)
        k0 = (k0 + _W0) & _MASK64
        k1 = (k1 + _W1) & _MASK64
    return c0, c1, c2, c3


STREAM_RENOISE, STREAM_INIT = 0, 1
STREAM_SAMPLE = 2           # the uniform of a sampled token


def uniform_token(seed, canvas, step, stream, pos, V) -> int:
    """A vocabulary id drawn uniformly: floor(r * V / 2^64), r = Philox word 0 with
    key (seed, canvas) and counter (pos, step, stream, 0)."""
    r = philox4x64_10((pos, step, stream, 0), (seed, canvas))[0]
    return (r * V) >> 64


def renoise(argmax, accept, seed, canvas_base, step, V):
    """Uniform-state renoise: accepted positions keep x^0 = argmax, every other
    position is replaced by a token drawn uniformly from the whole vocabulary.

    [TR] "Method steps" (2) and (3): the canvas starts as 256 uniform draws from the
    vocabulary and, after acceptance, "the rest are uniformly renoised". [GGL] "Uniform
    State Diffusion": noise replaces words with fully random vocabulary tokens and a
    position whose probability falls is renoised with a new random token.
    accept=None is canvas initialization: every position drawn on the init stream.
    Segment s uses canvas id canvas_base + s.
    """
    am = np.asarray(argmax, dtype=np.int64)
    if am.ndim == 1:
        am = am[None]
    B, C = am.shape
    acc = None if accept is None else np.asarray(accept).reshape(B, C)
    stream = STREAM_INIT if accept is None else STREAM_RENOISE
    out = np.zeros((B, C), dtype=np.int32)
    for s in range(B):
        for i in range(C):
            if acc is not None and acc[s, i]:
                out[s, i] = am[s, i]
            else:
                out[s, i] = uniform_token(seed, canvas_base + s, step, stream, i, V)
    return out


# ------------------------------------------------------------------ sampled tokens
def sample_uniform(seed, canvas, step, pos) -> float:
    """The uniform of a sampled token: u = (word 0 >> 11) / 2^53 in [0, 1), from
    Philox4x64-10 with key (seed, canvas) and counter (pos, step, 2, 0)."""
    w = philox4x64_10((pos, step, STREAM_SAMPLE, 0), (seed, canvas))[0]
    return (w >> 11) * 2.0 ** -53


def sample_tokens(p, seed, canvas_base, step, B=1, with_margins=False, positions=None):
    """Sampled tokens x~ ~ p^0, the sampled-token alternative to x^0 = argmax.

    [HUB] step 4 notes that real samplers draw from the tempered distribution instead of
    always taking the most likely token. The draw is the textbook inverse CDF over the
    whole vocabulary in id order: with one uniform u per position (sample_uniform), the
    token is the first id v whose cumulative probability sum_{v' <= v} p_v' exceeds
    u times the total.
    p float64 [B * Cs, V] (rows = canvas b position i at b * Cs + i); canvas id =
    canvas_base + b. Returns int32 tokens; with_margins also returns, per row, the
    distance (in probability) from u times the total to the nearest cumulative boundary,
    i.e. how far the draw is from picking a neighbouring id. ``positions`` (B = 1 only)
    gives the canvas position of each row when p holds a subset of rows.
    """
    p = np.asarray(p, dtype=np.float64)
    rows, V = p.shape
    Cs = rows // B
    out = np.zeros(rows, dtype=np.int32)
    margin = np.zeros(rows)
    for r in range(rows):
        b, i = divmod(r, Cs)
        if positions is not None:
            b, i = 0, int(positions[r])
        u = sample_uniform(seed, canvas_base + b, step, i)
        cum = np.cumsum(p[r])
        target = u * cum[-1]
        v = int(np.searchsorted(cum, target, side="right"))
        if v >= V:                                  # u * total rounded onto the total
            v = int(np.nonzero(p[r] > 0)[0][-1])
        out[r] = v
        lo = cum[v - 1] if v > 0 else 0.0
        margin[r] = min(target - lo, cum[v] - target)
    if with_margins:
        return out, margin
    return out


# ------------------------------------------------------------------ (a8) self-cond
def gelu_erf(x):
    """GELU in its exact form x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2))."""
    return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))


def selfcond(p, E_bits, W1, W2):
    """Self-conditioning vector z = FFW(p^0 E).

    [TR] "Method steps" (3): z = FFW(p^0 E); [TR] prerequisites: the previous softmax
    is projected through the embedding matrix and fed back through a small FFW block;
    [GGL] "Self-conditioning": the probability matrix times the token embedding table
    gives the vector passed to the next step. FFW = W2 . GELU(W1 . s), no bias.
    p float64 [C, V]; W1 [F, d]; W2 [d, F] -> z bf16 bits [C, d].
    """
    s = p @ from_bf16(E_bits)
    g = gelu_erf(s @ from_bf16(W1).T)
    return to_bf16(g @ from_bf16(W2).T), {"s": s, "g": g}


# ------------------------------------------------------------------ (a9) stop test
STOP_GO, STOP_STOP, STOP_CAP = 0, 1, 2


def stop_test(entropy, argmax, prev_argmax, thr, step, N):
    """Adaptive stop: 1 when mean canvas entropy <= thr and the argmax prediction is
    the same as at the previous step (checked from step 1 on); else 2 at the step cap
    N - 1; else 0.

    [TR] "Method steps" (4): stop early when the canvas mean entropy is <= 0.005 and
    the argmax prediction is unchanged over two consecutive steps. The mean is tested
    in 2^-32 fixed point: sum ceil(h * 2^32) <= floor(thr * C * 2^32). Any out-of-domain
    entropy blocks the stop. Works on B segments: entropy/argmax [B, C] -> flag [B].
    """
    ent = np.asarray(entropy, dtype=np.float32)
    am = np.asarray(argmax)
    if ent.ndim == 1:
        ent, am = ent[None], am[None]
        prev = None if prev_argmax is None else np.asarray(prev_argmax)[None]
    else:
        prev = None if prev_argmax is None else np.asarray(prev_argmax)
    B, C = ent.shape
    limit = math.floor(float(np.float32(thr)) * C * TWO32)
    flags = np.zeros(B, dtype=np.int32)
    for s in range(B):
        stop = False
        if step >= 1 and prev is not None:
            valid = all(float(h) < H_LIMIT for h in ent[s])
            total = sum(entropy_fixed(h) for h in ent[s])
            stop = valid and total <= limit and bool(np.all(am[s] == prev[s]))
        if stop:
            flags[s] = STOP_STOP
        elif step >= N - 1:
            flags[s] = STOP_CAP
    return flags


# ------------------------------------------------------------------ (a10) commit
def commit_kv(tokens, E_bits, Wk, Wv, Kp, Vp, P, Hkv, hd):
    """Append the finalized block's K/V rows at [P, P + C) of every KV head.

    [TR] "Method steps" (5): x^0 goes through the encoder and is appended to the KV
    cache, then the next canvas starts. [TUT] KV-cache timing: the canvas writes nothing
    to the cache until it is committed. Stand-in for the causal re-encode: K = E[x^0] Wk^T,
    V = E[x^0] Wv^T, rounded to bf16. Kp/Vp [Hkv, Pcap, hd] bf16 are modified in place;
    returns the new length P + C. Rows [0, P) are untouched.
    """
    tokens = np.asarray(tokens)
    C = tokens.shape[0]
    if P + C > Kp.shape[1]:
        raise ValueError("KV capacity exceeded")
    X = from_bf16(E_bits[tokens])
    Kn = to_bf16(X @ from_bf16(Wk).T).reshape(C, Hkv, hd)
    Vn = to_bf16(X @ from_bf16(Wv).T).reshape(C, Hkv, hd)
    Kp[:, P:P + C] = Kn.transpose(1, 0, 2)
    Vp[:, P:P + C] = Vn.transpose(1, 0, 2)
    return P + C


def prefill_block(tokens, E_bits, Wq, Wk, Wv, Wo, Kp, Vp, P, Hq, Hkv, hd, rope_base=0.0):
    """Causal re-encode of a finalized block, appending its K/V to the cache.

    [TUT] data-flow pseudocode (incremental_prefill of the finalized block into the KV
    cache) and KV-cache write timing: the output KV comes from the backbone re-encoding
    the finalized block in causal (prefill) mode, not from the denoiser's states. One
    attention layer stands in for the backbone: X = E[x], Q/K/V = bf16(X W^T), Q and K
    rotated at positions P + i (rope_base > 0) and rounded to bf16; block token i attends
    to the prefix [0, P) and to block tokens j <= i; A = bf16(O Wo^T). The rotated K and V
    rows are written at [P, P + C) of Kp/Vp (in place).
    Returns (A bits [C, d], new P = P + C).
    """
    tokens = np.asarray(tokens)
    C = tokens.shape[0]
    if P + C > Kp.shape[1]:
        raise ValueError("KV capacity exceeded")
    X = from_bf16(E_bits[tokens])
    pos = P + np.arange(C)
    Q = from_bf16(to_bf16(X @ from_bf16(Wq).T)).reshape(C, Hq, hd)
    Kb = from_bf16(to_bf16(X @ from_bf16(Wk).T)).reshape(C, Hkv, hd)
    Vb = from_bf16(to_bf16(X @ from_bf16(Wv).T)).reshape(C, Hkv, hd)
    if rope_base:
        Q = from_bf16(to_bf16(rope(Q, pos, rope_base)))
        Kb = from_bf16(to_bf16(rope(Kb, pos, rope_base)))
    Kp[:, P:P + C] = to_bf16(Kb).transpose(1, 0, 2)
    Vp[:, P:P + C] = to_bf16(Vb).transpose(1, 0, 2)
    O = np.zeros((C, Hq, hd))
    scale = 1.0 / math.sqrt(hd)
    causal = np.tril(np.ones((C, C), dtype=bool))
    for h in range(Hq):
        g = (h * Hkv) // Hq
        K = np.concatenate([from_bf16(Kp[g, :P]), Kb[:, g]], axis=0)
        V = np.concatenate([from_bf16(Vp[g, :P]), Vb[:, g]], axis=0)
        S = (Q[:, h] @ K.T) * scale
        S[:, P:][~causal] = -np.inf
        S = S - S.max(axis=1, keepdims=True)
        W = np.exp(S)
        W /= W.sum(axis=1, keepdims=True)
        O[:, h] = W @ V
    A = to_bf16(O.reshape(C, Hq * hd) @ from_bf16(Wo).T)
    return A, P + C


# ------------------------------------------------------------------ canvas MoE FFN
def moe_route(X_bits, Wr, K):
    """Router of the canvas MoE FFN ([MOE]): logits r = X Wr^T; each token takes the K
    experts with the largest logits (ties to the lower expert id) and gates them with a
    softmax over those K logits. Selection and gates are taken on the float64 logits.
    Returns (experts int32 [C, K] in rank order, gates float64 [C, K], logits float64 [C, E])."""
    X = from_bf16(X_bits)
    r = X @ from_bf16(Wr).T
    C, E = r.shape
    sel = np.zeros((C, K), dtype=np.int32)
    gates = np.zeros((C, K))
    for t in range(C):
        order = sorted(range(E), key=lambda e: (-float(r[t, e]), e))[:K]
        sel[t] = order
        v = r[t, order]
        w = np.exp(v - v.max())
        gates[t] = w / w.sum()
    return sel, gates, r


def moe_ffn(X_bits, Wr, W1, W2, W1s, W2s, K):
    """Canvas MoE FFN ([MOE]): y = sum over the token's K routed experts of gate * E_e(x)
    + S(x), every expert and the shared one of the FFW form W2 GELU_erf(W1 x) (the form of
    the self-conditioning FFW; the pages name no gating). Expert and shared outputs are
    stored as bf16, combined in float64, and y is rounded to bf16.
    X [C, d]; Wr [E, d]; W1 [E, Fe, d]; W2 [E, d, Fe]; W1s [Fs, d]; W2s [d, Fs] (bf16 bits).
    Returns (Y bits [C, d], experts [C, K], gates [C, K], number of distinct experts used)."""
    X = from_bf16(X_bits)
    sel, gates, _ = moe_route(X_bits, Wr, K)
    C, d = X.shape
    acc = np.zeros((C, d))
    for e in np.unique(sel):
        rows, ranks = np.nonzero(sel == e)
        h = from_bf16(to_bf16(gelu_erf(X[rows] @ from_bf16(W1[e]).T)))
        y = from_bf16(to_bf16(h @ from_bf16(W2[e]).T))
        acc[rows] += gates[rows, ranks][:, None] * y
    hs = from_bf16(to_bf16(gelu_erf(X @ from_bf16(W1s).T)))
    ys = from_bf16(to_bf16(hs @ from_bf16(W2s).T))
    return to_bf16(acc + ys), sel, gates, int(len(np.unique(sel)))


# ------------------------------------------------------------------ the step loop
def run_canvas(W, Kp, Vp, P, hidden_of_step, *, V, C, Hq, Hkv, hd, N, seed, canvas,
               b=0.1, thr=0.005, tau0=0.8, tau1=0.4, record=True, with_attn=True,
               rule="entropy", draw="argmax", commit="projection", rope_base=0.0):
    """One canvas of the block-AR loop: init, up to N denoise steps, commit.

    [TR] "Method steps" (2)-(5) in order; [TUT] data-flow pseudocode. The sampler head's
    hidden states come from ``hidden_of_step(k)`` (the synthetic driver standing in for
    the denoiser stack); the attention output A_k is computed on the true denoiser input
    X_k = E[x_k] + z_k every step and recorded, but does not feed H_k.
    rule "confidence" replaces the entropy budget by the confidence rule; draw "sample"
    gives accepted positions, and the commit, x~ ~ p^0 instead of x^0; commit "prefill"
    re-encodes the block causally (prefill_block) instead of projecting it; rope_base > 0
    rotates canvas (and block) queries and keys to their positions (module header).
    Returns (new P, list of per-step records).
    """
    d = W["E"].shape[1]
    schedule = reveal_schedule(C, N)
    x = renoise(np.zeros(C, np.int32), None, seed, canvas, 0, V)[0]
    z = np.zeros((C, d), dtype=np.uint16)            # z_1 = 0 (bf16 zero bits)
    prev = None
    recs = []
    k = 0
    am = None
    for k in range(N):
        tau = temperature(k, N, tau0, tau1)
        rec = {"k": k, "tau": tau, "tokens_in": x.copy(), "z_in": z.copy()}
        if with_attn:
            A, _ = canvas_attn(x, z, W["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"],
                               Kp, Vp, P, Hq, Hkv, hd, rope_base=rope_base)
            rec["A"] = A
        ent, am, p, _ = logits_entropy(hidden_of_step(k), W["E"], tau)
        x0 = am
        if draw == "sample":
            x0, margin = sample_tokens(p, seed, canvas, k, with_margins=True)
            rec.update(sampled=x0, sample_margin=margin)
        if rule == "confidence":
            conf = p.max(axis=1).astype(np.float32)
            acc, nacc = topk_accept(conf[None], schedule[k])
            rec["conf"] = conf
        else:
            acc, nacc = entropy_accept(ent[None], b)
        x = renoise(x0[None], acc, seed, canvas, k, V)[0]
        z, _ = selfcond(p, W["E"], W["W1"], W["W2"])
        flag = int(stop_test(ent[None], am[None], None if prev is None else prev[None],
                             thr, k, N)[0])
        rec.update(entropy=ent, argmax=am, accept=acc[0], n_accept=int(nacc[0]),
                   tokens=x.copy(), z=z.copy(), flag=flag)
        if record:
            recs.append(rec)
        prev = am
        if flag != STOP_GO:
            break
    if commit == "prefill":
        A_block, P = prefill_block(x0, W["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], Kp, Vp, P,
                                   Hq, Hkv, hd, rope_base)
        if record and recs:
            recs[-1]["A_commit"] = A_block
    else:
        P = commit_kv(x0, W["E"], W["Wk"], W["Wv"], Kp, Vp, P, Hkv, hd)
    return P, recs
