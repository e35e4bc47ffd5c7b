"""Seeded synthetic inputs for the canvas-denoise step (shared by tests, bench and oracle).

This module only *generates* inputs: Gaussian weights, a random prefix KV cache,
per-canvas target tokens and the synthetic hidden-state driver that stands in for
the trained 30-layer denoiser stack. It holds none of the method's arithmetic
(no softmax, entropy, acceptance, renoise, attention or self-conditioning).

Every tensor is drawn from ``numpy.random.default_rng([seed, tag, ...])`` in float32
and rounded to bfloat16 with round-to-nearest-even; bf16 tensors are carried as
``uint16`` bit patterns (numpy has no bf16 dtype).

Workload shapes follow the pages' sampler head: a 256-token canvas, a ~262K vocabulary,
at most 48 denoise steps (DiffusionGemma Technical Report summary, "method steps";
tutorial chapter "DiffusionGemma", sampler configuration). Everything else about the
workloads (model width, heads, FFW width, prefix length, weight scales, the driver) is
a synthetic stand-in defined here, because the pages name no such sizes and the trained
weights are not available.

Driver (stand-in for the denoiser forward): at step k of canvas c,
    alpha_k = alpha_max * k / (N - 1)
    H_k     = bf16(alpha_k * E[target_c] + eps_{c,k}),   eps ~ N(0, 1) drawn per step
so the sampler head sees logits that sharpen towards a per-canvas target sequence.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

__all__ = [
    "Config", "CONFIGS", "config", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "weights", "prefix_kv", "targets", "hidden", "hidden_all", "alpha",
    "gaussian_bf16",
]

# Fixed stream tags, one per generated tensor.
TAG_E, TAG_WQ, TAG_WK, TAG_WV, TAG_WO, TAG_W1, TAG_W2 = 1, 2, 3, 4, 5, 6, 7
TAG_KP, TAG_VP = 8, 9
TAG_TARGET, TAG_NOISE = 10, 11
TAG_MOE_X, TAG_MOE_WR, TAG_MOE_W1, TAG_MOE_W2, TAG_MOE_W1S, TAG_MOE_W2S = 12, 13, 14, 15, 16, 17
TAG_MOE_XG = 18

# Large tensors are drawn in independent row blocks of this many elements so that
# generation can be chunked; the block index is part of the stream key.
_BLOCK_ELEMS = 1 << 24


@dataclass(frozen=True)
class Config:
    """One synthetic workload: shapes, step budget, driver strength and seed."""
    name: str
    V: int          # vocabulary size (rows of the tied embedding / lm_head E)
    d: int          # model width
    C: int          # canvas length (tokens denoised together)
    Hq: int         # query heads
    Hkv: int        # key/value heads (GQA: Hq % Hkv == 0)
    hd: int         # head dim
    F: int          # self-conditioning FFW hidden width
    P0: int         # prefix length in the KV cache at the first canvas
    N: int          # denoise step budget
    alpha_max: float
    seed: int
    n_canvas: int = 1

    @property
    def Pcap(self) -> int:
        """Cache capacity: the prefix plus every canvas the workload commits."""
        return self.P0 + self.C * self.n_canvas

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS = (
    # tiny CPU-checkable step loop
    Config("tiny", V=512, d=64, C=16, Hq=4, Hkv=2, hd=16, F=128, P0=32, N=8,
           alpha_max=8.0, seed=0),
    # small full canvas
    Config("small", V=32768, d=1024, C=256, Hq=8, Hkv=2, hd=128, F=1024, P0=2048, N=48,
           alpha_max=8.0, seed=1),
    # Gemma-scale sampler head (256-canvas, 262144 vocab)
    Config("gemma_head", V=262144, d=2048, C=256, Hq=16, Hkv=8, hd=128, F=1024, P0=8192,
           N=48, alpha_max=10.0, seed=2),
    # long prefix (262144 cached tokens)
    Config("long_prefix", V=262144, d=2048, C=256, Hq=16, Hkv=8, hd=128, F=1024,
           P0=262144, N=48, alpha_max=10.0, seed=3),
    # block-AR chain of 8 canvases from a 32768-token prefix
    Config("chain8", V=262144, d=2048, C=256, Hq=16, Hkv=8, hd=128, F=1024, P0=32768,
           N=48, alpha_max=10.0, seed=4, n_canvas=8),
)


def config(i_or_name) -> Config:
    if isinstance(i_or_name, int):
        return CONFIGS[i_or_name]
    for c in CONFIGS:
        if c.name == i_or_name:
            return c
    raise KeyError(i_or_name)


# ---------------------------------------------------------------- bf16 bit helpers
def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32)
    out = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16))
    return out.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- generators
def gaussian_bf16(seed: int, tag: int, shape, std: float) -> np.ndarray:
    """N(0, std^2) in float32, rounded to bf16 bits. Drawn in fixed element blocks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    std32 = np.float32(std)
    for blk, start in enumerate(range(0, n, _BLOCK_ELEMS)):
        stop = min(n, start + _BLOCK_ELEMS)
        g = np.random.default_rng([seed, tag, blk])
        x = g.standard_normal(stop - start, dtype=np.float32)
        x *= std32
        out[start:stop] = f32_to_bf16_bits(x)
    return out.reshape(shape)


def weights(cfg: Config) -> dict:
    """All weights as bf16 bits, in [out_features, in_features] row-major layout.

    E [V, d] is the tied embedding / lm_head table. Every weight is N(0, 1/fan_in).
    """
    s, d = cfg.seed, cfg.d
    qd, kd = cfg.Hq * cfg.hd, cfg.Hkv * cfg.hd
    return {
        "E": gaussian_bf16(s, TAG_E, (cfg.V, d), d ** -0.5),
        "Wq": gaussian_bf16(s, TAG_WQ, (qd, d), d ** -0.5),
        "Wk": gaussian_bf16(s, TAG_WK, (kd, d), d ** -0.5),
        "Wv": gaussian_bf16(s, TAG_WV, (kd, d), d ** -0.5),
        "Wo": gaussian_bf16(s, TAG_WO, (d, qd), qd ** -0.5),
        "W1": gaussian_bf16(s, TAG_W1, (cfg.F, d), d ** -0.5),
        "W2": gaussian_bf16(s, TAG_W2, (d, cfg.F), cfg.F ** -0.5),
    }


def prefix_kv(cfg: Config, Pcap: int | None = None, request: int = 0):
    """Prefix K and V caches, logical layout [Hkv, Pcap, hd], rows [0, P0) ~ N(0, 1).

    Rows [P0, Pcap) are zero (free capacity for committed canvases). ``request`` r > 0
    draws an independent prefix (tags offset by 32 r) for the r-th request of a batch.
    """
    Pcap = cfg.Pcap if Pcap is None else Pcap
    K = np.zeros((cfg.Hkv, Pcap, cfg.hd), dtype=np.uint16)
    V = np.zeros((cfg.Hkv, Pcap, cfg.hd), dtype=np.uint16)
    if cfg.P0:
        off = 32 * int(request)
        K[:, :cfg.P0] = gaussian_bf16(cfg.seed, TAG_KP + off, (cfg.Hkv, cfg.P0, cfg.hd), 1.0)
        V[:, :cfg.P0] = gaussian_bf16(cfg.seed, TAG_VP + off, (cfg.Hkv, cfg.P0, cfg.hd), 1.0)
    return K, V


# Share of a canvas row's variance that its canvas has in common: with the random router
# below, a 256-token canvas of such rows routes to about 84 distinct experts of 128 at
# top-8, the count the DiffusionGemma Technical Report page gives ("Prerequisites").
MOE_CANVAS_SHARE = 0.56


def moe_inputs(C: int, d: int, E: int, K: int, Fe: int, Fs: int, seed: int, share: float = 0.0) -> dict:
    """Canvas MoE FFN stand-in weights and activations (bf16 bits): every weight
    N(0, 1/fan_in); X rows N(0, 1) per element, x_t = sqrt(share) g + sqrt(1 - share) e_t
    with one direction g per canvas (share = 0: independent rows, which route to nearly
    every expert). Layouts: Wr [E, d], W1 [E, Fe, d], W2 [E, d, Fe], W1s [Fs, d],
    W2s [d, Fs]. K (experts per token) is not used for drawing."""
    if share > 0.0:
        g = np.random.default_rng([seed, TAG_MOE_XG]).standard_normal(d).astype(np.float32)
        e = np.random.default_rng([seed, TAG_MOE_X]).standard_normal((C, d)).astype(np.float32)
        X = f32_to_bf16_bits(np.float32(np.sqrt(share)) * g[None, :] + np.float32(np.sqrt(1.0 - share)) * e)
    else:
        X = gaussian_bf16(seed, TAG_MOE_X, (C, d), 1.0)
    return {
        "X": X,
        "Wr": gaussian_bf16(seed, TAG_MOE_WR, (E, d), d ** -0.5),
        "W1": gaussian_bf16(seed, TAG_MOE_W1, (E, Fe, d), d ** -0.5),
        "W2": gaussian_bf16(seed, TAG_MOE_W2, (E, d, Fe), Fe ** -0.5),
        "W1s": gaussian_bf16(seed, TAG_MOE_W1S, (Fs, d), d ** -0.5),
        "W2s": gaussian_bf16(seed, TAG_MOE_W2S, (d, Fs), Fs ** -0.5),
    }


def targets(cfg: Config, canvas: int) -> np.ndarray:
    """Per-canvas target token ids the driver sharpens towards, uniform over [0, V)."""
    g = np.random.default_rng([cfg.seed, TAG_TARGET, canvas])
    return g.integers(0, cfg.V, size=cfg.C, dtype=np.int64).astype(np.int32)


def alpha(cfg: Config, k: int) -> np.float32:
    if cfg.N <= 1:
        return np.float32(cfg.alpha_max)
    return np.float32(cfg.alpha_max * k / (cfg.N - 1))


def hidden(cfg: Config, E_bits: np.ndarray, canvas: int, k: int,
           tgt: np.ndarray | None = None) -> np.ndarray:
    """Driver hidden states H_k [C, d] as bf16 bits (see module docstring)."""
    if tgt is None:
        tgt = targets(cfg, canvas)
    g = np.random.default_rng([cfg.seed, TAG_NOISE, canvas, k])
    eps = g.standard_normal((cfg.C, cfg.d), dtype=np.float32)
    Et = bf16_bits_to_f32(E_bits[tgt])
    return f32_to_bf16_bits(alpha(cfg, k) * Et + eps)


def hidden_all(cfg: Config, E_bits: np.ndarray, canvas: int) -> np.ndarray:
    """All N driver states of one canvas, [N, C, d] bf16 bits."""
    tgt = targets(cfg, canvas)
    return np.stack([hidden(cfg, E_bits, canvas, k, tgt) for k in range(cfg.N)])
