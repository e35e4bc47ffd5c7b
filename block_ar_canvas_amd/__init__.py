"""Python binding of libdg, the MI355X canvas-denoise library (C ABI in include/dg.h).

Argument marshalling only: every call checks the torch tensors it is handed (device,
dtype, contiguity), passes their device pointers and the context's HIP stream to the
C entry point of the same name, and raises DGError on a non-OK status. All of the
step's arithmetic runs in the library's HIP kernels; there is no fallback path, and
importing this package fails loudly when libdg.so has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["DGError", "Dims", "MoeDims", "Context", "moe_workspace_bytes", "workspace_bytes", "loop_workspace_bytes",
           "temperature", "reveal_count", "lib_path",
           "STOP_GO", "STOP_STOP", "STOP_CAP", "PEAK_STREAM_BLOCKS", "PEAK_MFMA_BLOCKS", "STATIC_SCRATCH_BYTES"]

_HERE = os.path.dirname(os.path.abspath(__file__))
STOP_GO, STOP_STOP, STOP_CAP = 0, 1, 2
PEAK_STREAM_BLOCKS, PEAK_MFMA_BLOCKS = 2048, 1024     # DG_PEAK_STREAM_BLOCKS, DG_PEAK_MFMA_BLOCKS
STATIC_SCRATCH_BYTES = 48 << 20                         # DG_STATIC_SCRATCH_BYTES

_STATUS = {0: "DG_OK", 1: "DG_ERR_NULL", 2: "DG_ERR_SHAPE", 3: "DG_ERR_ALIGN", 4: "DG_ERR_RANGE",
           5: "DG_ERR_CAPACITY", 6: "DG_ERR_STATE", 7: "DG_ERR_NONFINITE", 8: "DG_ERR_HIP",
           9: "DG_ERR_UNSUPPORTED"}


class DGError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status
        self.name = _STATUS.get(status, str(status))


def lib_path() -> str:
    return os.path.join(_HERE, "libdg.so")


class MoeDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("d", "E", "K", "Fe", "Fs")]


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("V", "d", "C", "Hq", "Hkv", "hd", "F")]

    @classmethod
    def of(cls, obj) -> "Dims":
        if isinstance(obj, Dims):
            return obj
        g = (lambda k: obj[k]) if isinstance(obj, dict) else (lambda k: getattr(obj, k))
        return cls(*(int(g(k)) for k in ("V", "d", "C", "Hq", "Hkv", "hd", "F")))


class Weights(ctypes.Structure):
    """dg_weights: device pointers of the step's weights."""
    _fields_ = [(n, ctypes.c_void_p) for n in ("E", "Wq", "Wk", "Wv", "Wo", "W1", "W2")]


class LoopParams(ctypes.Structure):
    """dg_loop_params of dg_run_canvas."""
    _fields_ = [("N", ctypes.c_int32), ("b", ctypes.c_float), ("thr", ctypes.c_float),
                ("tau0", ctypes.c_float), ("tau1", ctypes.c_float), ("seed", ctypes.c_uint64),
                ("canvas", ctypes.c_uint32), ("commit", ctypes.c_int32), ("rule", ctypes.c_int32),
                ("draw", ctypes.c_int32)]


COMMIT_PROJECTION, COMMIT_PREFILL = 0, 1          # dg_loop_params.commit
RULE_ENTROPY, RULE_CONFIDENCE = 0, 1              # dg_loop_params.rule
DRAW_ARGMAX, DRAW_SAMPLE = 0, 1                   # dg_loop_params.draw


class AcceptArgs(ctypes.Structure):
    """dg_accept_args of dg_selfcond_accept."""
    _fields_ = [("B", ctypes.c_int32), ("entropy", ctypes.c_void_p), ("b", ctypes.c_float),
                ("x0", ctypes.c_void_p), ("argmax", ctypes.c_void_p), ("prev_argmax", ctypes.c_void_p),
                ("seed", ctypes.c_uint64), ("canvas_base", ctypes.c_uint32), ("step", ctypes.c_int32),
                ("thr", ctypes.c_float), ("N", ctypes.c_int32), ("accept", ctypes.c_void_p),
                ("n_accept", ctypes.c_void_p), ("tokens", ctypes.c_void_p), ("flag", ctypes.c_void_p),
                ("x_next", ctypes.c_void_p)]


# dg_hidden_fn: (user, step) -> device pointer of H_step
HIDDEN_FN = ctypes.CFUNCTYPE(ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32)

_P = ctypes.c_void_p
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(f"libdg.so is not built ({path}); run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    i32, i64, f32, u32, u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_uint32, ctypes.c_uint64
    D = ctypes.POINTER(Dims)
    sig = {
        "dg_create": (i32, [ctypes.POINTER(_P), ctypes.c_int, _P]),
        "dg_destroy": (None, [_P]),
        "dg_set_stream": (i32, [_P, _P]),
        "dg_last_error": (ctypes.c_char_p, [_P]),
        "dg_sync": (i32, [_P]),
        "dg_clear_status": (i32, [_P]),
        "dg_workspace_bytes": (ctypes.c_size_t, [D, i64]),
        "dg_temperature": (f32, [i32, i32, f32, f32]),
        "dg_canvas_attn": (i32, [_P, D, _P, _P, _P, _P, _P, _P, _P, _P, _P, i64, i64, _P, _P]),
        "dg_canvas_attn_static": (i32, [_P, D, _P, _P, _P, _P, _P, _P, _P, _P, _P, i64, i64, _P]),
        "dg_canvas_attn_x": (i32, [_P, D, _P, _P, _P, _P, _P, _P, _P, i64, i64, _P, _P]),
        "dg_logits_entropy": (i32, [_P, D, _P, _P, f32, _P, _P, _P]),
        "dg_entropy_accept": (i32, [_P, i32, i32, _P, f32, _P, _P]),
        "dg_confidence": (i32, [_P, D, _P, _P]),
        "dg_topk_accept": (i32, [_P, i32, i32, _P, i32, _P, _P]),
        "dg_reveal_count": (i32, [i32, i32, i32]),
        "dg_sample": (i32, [_P, D, _P, i32, u64, u32, u32, _P]),
        "dg_set_rope": (i32, [_P, f32]),
        "dg_moe_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(MoeDims), i32]),
        "dg_moe_ffn": (i32, [_P, ctypes.POINTER(MoeDims), i32, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
        "dg_prefill_block": (i32, [_P, D, _P, _P, _P, _P, _P, _P, _P, _P, i64, i64, _P, _P,
                                   ctypes.POINTER(i64)]),
        "dg_renoise": (i32, [_P, i32, i32, i32, _P, _P, u64, u32, u32, _P]),
        "dg_selfcond": (i32, [_P, D, _P, _P, _P, _P, _P]),
        "dg_stop_test": (i32, [_P, i32, i32, _P, _P, _P, f32, i32, i32, _P]),
        "dg_accept_renoise_stop": (i32, [_P, i32, i32, i32, _P, f32, _P, _P, _P, u64, u32, i32, f32, i32,
                                         _P, _P, _P, _P]),
        "dg_selfcond_accept": (i32, [_P, D, _P, _P, _P, _P, _P, ctypes.POINTER(AcceptArgs)]),
        "dg_commit_kv": (i32, [_P, D, _P, _P, _P, _P, _P, _P, i64, i64, ctypes.POINTER(i64)]),
        "dg_peak_stream_read": (i32, [_P, _P, ctypes.c_size_t, _P]),
        "dg_peak_mfma_bf16": (i32, [_P, i32, _P]),
        "dg_loop_workspace_bytes": (ctypes.c_size_t, [D]),
        "dg_run_canvas": (i32, [_P, D, ctypes.POINTER(Weights), _P, _P, i64, i64, ctypes.POINTER(LoopParams),
                                HIDDEN_FN, _P, _P, _P, _P, ctypes.POINTER(i32), ctypes.POINTER(i64)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def workspace_bytes(dims, Pcap: int) -> int:
    d = Dims.of(dims)
    n = _load().dg_workspace_bytes(ctypes.byref(d), int(Pcap))
    if n == 0:
        raise DGError(2, "dg_workspace_bytes: unsupported dims")
    return int(n)


def loop_workspace_bytes(dims) -> int:
    """Bytes of the device state dg_run_canvas keeps for one canvas."""
    d = Dims.of(dims)
    n = _load().dg_loop_workspace_bytes(ctypes.byref(d))
    if n == 0:
        raise DGError(2, "dg_loop_workspace_bytes: unsupported dims")
    return int(n)


def temperature(k: int, N: int, tau0: float = 0.8, tau1: float = 0.4) -> float:
    return float(_load().dg_temperature(int(k), int(N), float(tau0), float(tau1)))


def moe_workspace_bytes(md, C: int) -> int:
    n = _load().dg_moe_workspace_bytes(ctypes.byref(md), int(C))
    if n == 0:
        raise DGError(2, "dg_moe_workspace_bytes: bad dims")
    return int(n)


def reveal_count(C: int, N: int, step: int) -> int:
    """Positions accepted at `step` under the confidence rule's reveal schedule."""
    n = int(_load().dg_reveal_count(int(C), int(N), int(step)))
    if n < 0:
        raise ValueError(f"reveal_count: bad arguments C={C} N={N} step={step}")
    return n


def _ptr(t, dtype, name, optional=False, pinned_ok=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda and not (pinned_ok and t.is_pinned()):
        raise ValueError(f"{name} must live on the GPU" + (" or in pinned host memory" if pinned_ok else ""))
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


_BF16, _F32, _I32, _U8 = torch.bfloat16, torch.float32, torch.int32, torch.uint8


class Context:
    """One dg_ctx: a device, a HIP stream and the sticky device status word."""

    def __init__(self, device: int = 0, stream=None):
        self._lib = _load()
        self.device = int(device)
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        self._stream = stream
        h = _P()
        st = self._lib.dg_create(ctypes.byref(h), self.device, self._raw_stream(stream))
        if st != 0:
            raise DGError(st, "dg_create failed")
        self._h = h

    @staticmethod
    def _raw_stream(stream):
        if stream is None:
            return None
        if isinstance(stream, int):
            return stream
        return stream.cuda_stream

    def close(self):
        if getattr(self, "_h", None):
            self._lib.dg_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, st: int):
        if st != 0:
            raise DGError(st, self._lib.dg_last_error(self._h).decode())

    def set_stream(self, stream):
        self._stream = stream
        self._check(self._lib.dg_set_stream(self._h, self._raw_stream(stream)))

    @property
    def stream(self):
        return self._stream

    def torch_stream(self):
        """The context's stream as a torch stream object, for torch work (fills, copies)
        that must stay ordered with the library's calls."""
        s = self._stream
        if isinstance(s, torch.cuda.Stream):
            return s
        return torch.cuda.ExternalStream(self._raw_stream(s) or 0, device=torch.device("cuda", self.device))

    def sync(self):
        self._check(self._lib.dg_sync(self._h))

    def clear_status(self):
        self._check(self._lib.dg_clear_status(self._h))

    # ------------------------------------------------------------ the seven calls
    def canvas_attn_x(self, dims, X, Wq, Wk, Wv, Wo, Kp, Vt, P, ws, A):
        """canvas_attn on a pre-formed input X [C, d] bf16 (e.g. selfcond_accept's x_next)."""
        d = Dims.of(dims)
        Pcap = Kp.shape[1] if Kp is not None else 0
        self._check(self._lib.dg_canvas_attn_x(
            self._h, ctypes.byref(d), _ptr(X, _BF16, "X"), _ptr(Wq, _BF16, "Wq"), _ptr(Wk, _BF16, "Wk"),
            _ptr(Wv, _BF16, "Wv"), _ptr(Wo, _BF16, "Wo"), _ptr(Kp, _BF16, "Kp", True),
            _ptr(Vt, _BF16, "Vt", True), int(P), int(Pcap), _ptr(ws, _U8, "ws"), _ptr(A, _BF16, "A")))

    def canvas_attn(self, dims, tokens, z, E, Wq, Wk, Wv, Wo, Kp, Vt, P, ws, A):
        d = Dims.of(dims)
        Pcap = Kp.shape[1] if Kp is not None else 0
        self._check(self._lib.dg_canvas_attn(
            self._h, ctypes.byref(d), _ptr(tokens, _I32, "tokens"), _ptr(z, _BF16, "z", True),
            _ptr(E, _BF16, "E"), _ptr(Wq, _BF16, "Wq"), _ptr(Wk, _BF16, "Wk"), _ptr(Wv, _BF16, "Wv"),
            _ptr(Wo, _BF16, "Wo"), _ptr(Kp, _BF16, "Kp", True), _ptr(Vt, _BF16, "Vt", True),
            int(P), int(Pcap), _ptr(ws, _U8, "ws"), _ptr(A, _BF16, "A")))

    def canvas_attn_static(self, dims, tokens, z, E, Wq, Wk, Wv, Wo, Kp, Vt, P, A):
        """dg_canvas_attn on the library's static per-device scratch (no workspace)."""
        d = Dims.of(dims)
        Pcap = Kp.shape[1] if Kp is not None else 0
        self._check(self._lib.dg_canvas_attn_static(
            self._h, ctypes.byref(d), _ptr(tokens, _I32, "tokens"), _ptr(z, _BF16, "z", True),
            _ptr(E, _BF16, "E"), _ptr(Wq, _BF16, "Wq"), _ptr(Wk, _BF16, "Wk"), _ptr(Wv, _BF16, "Wv"),
            _ptr(Wo, _BF16, "Wo"), _ptr(Kp, _BF16, "Kp", True), _ptr(Vt, _BF16, "Vt", True),
            int(P), int(Pcap), _ptr(A, _BF16, "A")))

    def logits_entropy(self, dims, H, E, tau, ws, entropy, argmax):
        d = Dims.of(dims)
        self._check(self._lib.dg_logits_entropy(
            self._h, ctypes.byref(d), _ptr(H, _BF16, "H"), _ptr(E, _BF16, "E"), float(tau),
            _ptr(ws, _U8, "ws"), _ptr(entropy, _F32, "entropy"), _ptr(argmax, _I32, "argmax")))

    def entropy_accept(self, entropy, b, accept, n_accept):
        B, C = (1, entropy.shape[0]) if entropy.dim() == 1 else tuple(entropy.shape)
        self._check(self._lib.dg_entropy_accept(
            self._h, B, C, _ptr(entropy, _F32, "entropy"), float(b), _ptr(accept, _U8, "accept"),
            _ptr(n_accept, _I32, "n_accept")))

    def confidence(self, dims, ws, conf):
        d = Dims.of(dims)
        self._check(self._lib.dg_confidence(self._h, ctypes.byref(d), _ptr(ws, _U8, "ws"),
                                            _ptr(conf, _F32, "confidence")))

    def topk_accept(self, score, k, accept, n_accept):
        B, C = (1, score.shape[0]) if score.dim() == 1 else tuple(score.shape)
        self._check(self._lib.dg_topk_accept(
            self._h, B, C, _ptr(score, _F32, "score"), int(k), _ptr(accept, _U8, "accept"),
            _ptr(n_accept, _I32, "n_accept")))

    def sample(self, dims, ws, B, seed, canvas_base, step, tokens):
        d = Dims.of(dims)
        self._check(self._lib.dg_sample(self._h, ctypes.byref(d), _ptr(ws, _U8, "ws"), int(B),
                                        int(seed), int(canvas_base), int(step),
                                        _ptr(tokens, _I32, "tokens")))

    def renoise(self, V, argmax, accept, seed, canvas_base, step, tokens):
        B, C = (1, tokens.shape[0]) if tokens.dim() == 1 else tuple(tokens.shape)
        self._check(self._lib.dg_renoise(
            self._h, B, C, int(V), _ptr(argmax, _I32, "argmax", True), _ptr(accept, _U8, "accept", True),
            int(seed), int(canvas_base), int(step), _ptr(tokens, _I32, "tokens")))

    def selfcond(self, dims, ws, E, W1, W2, z):
        d = Dims.of(dims)
        self._check(self._lib.dg_selfcond(
            self._h, ctypes.byref(d), _ptr(ws, _U8, "ws"), _ptr(E, _BF16, "E"), _ptr(W1, _BF16, "W1"),
            _ptr(W2, _BF16, "W2"), _ptr(z, _BF16, "z")))

    def stop_test(self, entropy, argmax, prev_argmax, thr, step, N, flag):
        B, C = (1, entropy.shape[0]) if entropy.dim() == 1 else tuple(entropy.shape)
        self._check(self._lib.dg_stop_test(
            self._h, B, C, _ptr(entropy, _F32, "entropy"), _ptr(argmax, _I32, "argmax"),
            _ptr(prev_argmax, _I32, "prev_argmax", True), float(thr), int(step), int(N),
            _ptr(flag, _I32, "flag", pinned_ok=True)))

    def accept_renoise_stop(self, V, entropy, b, x0, argmax, prev_argmax, seed, canvas_base, step,
                            thr, N, accept, n_accept, tokens, flag):
        """entropy_accept, renoise (with accept) and stop_test in one launch, same results."""
        B, C = (1, entropy.shape[0]) if entropy.dim() == 1 else tuple(entropy.shape)
        self._check(self._lib.dg_accept_renoise_stop(
            self._h, B, C, int(V), _ptr(entropy, _F32, "entropy"), float(b), _ptr(x0, _I32, "x0"),
            _ptr(argmax, _I32, "argmax"), _ptr(prev_argmax, _I32, "prev_argmax", True), int(seed),
            int(canvas_base), int(step), float(thr), int(N), _ptr(accept, _U8, "accept"),
            _ptr(n_accept, _I32, "n_accept"), _ptr(tokens, _I32, "tokens"),
            _ptr(flag, _I32, "flag", pinned_ok=True)))

    def selfcond_accept(self, dims, ws, E, W1, W2, z, entropy, b, x0, argmax, prev_argmax, seed,
                        canvas_base, step, thr, N, accept, n_accept, tokens, flag, x_next=None):
        """accept_renoise_stop then selfcond, same results; the acceptance work runs beside
        self-conditioning's reduce. B canvases = the rows of entropy. x_next [C, d] bf16,
        optional: receives bf16(E[tokens] + z), the next step's canvas_attn_x input."""
        d = Dims.of(dims)
        B = 1 if entropy.dim() == 1 else entropy.shape[0]
        a = AcceptArgs(int(B), _ptr(entropy, _F32, "entropy"), float(b), _ptr(x0, _I32, "x0"),
                       _ptr(argmax, _I32, "argmax"), _ptr(prev_argmax, _I32, "prev_argmax", True), int(seed),
                       int(canvas_base), int(step), float(thr), int(N), _ptr(accept, _U8, "accept"),
                       _ptr(n_accept, _I32, "n_accept"), _ptr(tokens, _I32, "tokens"),
                       _ptr(flag, _I32, "flag", pinned_ok=True), _ptr(x_next, _BF16, "x_next", True))
        self._check(self._lib.dg_selfcond_accept(
            self._h, ctypes.byref(d), _ptr(ws, _U8, "ws"), _ptr(E, _BF16, "E"), _ptr(W1, _BF16, "W1"),
            _ptr(W2, _BF16, "W2"), _ptr(z, _BF16, "z"), ctypes.byref(a)))

    def moe_ffn(self, md, X, Wr, W1, W2, W1s, W2s, ws, Y, n_active=None):
        C = X.shape[0]
        self._check(self._lib.dg_moe_ffn(
            self._h, ctypes.byref(md), int(C), _ptr(X, _BF16, "X"), _ptr(Wr, _BF16, "Wr"),
            _ptr(W1, _BF16, "W1"), _ptr(W2, _BF16, "W2"), _ptr(W1s, _BF16, "W1s"),
            _ptr(W2s, _BF16, "W2s"), _ptr(ws, _U8, "ws"), _ptr(Y, _BF16, "Y"),
            _ptr(n_active, _I32, "n_active", True)))

    def peak_stream_read(self, buf, sink):
        """Streaming read of the whole of buf (measured HBM ceiling); sink: int32
        [PEAK_STREAM_BLOCKS] receives per-workgroup XORs of the 16-byte words read."""
        self._check(self._lib.dg_peak_stream_read(self._h, _ptr(buf, buf.dtype, "buf"),
                                                  buf.numel() * buf.element_size(),
                                                  _ptr(sink, _I32, "sink")))

    def peak_mfma(self, iters: int, sink):
        """Back-to-back bf16 MFMAs (measured MFMA ceiling); sink: float32
        [PEAK_MFMA_BLOCKS * 4], each entry 1024 * iters. Returns the FLOP enqueued."""
        self._check(self._lib.dg_peak_mfma_bf16(self._h, int(iters), _ptr(sink, _F32, "sink")))
        return PEAK_MFMA_BLOCKS * 4 * int(iters) * 4 * 32768

    def set_rope(self, base: float):
        self._check(self._lib.dg_set_rope(self._h, float(base)))

    def prefill_block(self, dims, tokens, E, Wq, Wk, Wv, Wo, Kp, Vt, P, ws, A) -> int:
        d = Dims.of(dims)
        out = ctypes.c_int64(0)
        self._check(self._lib.dg_prefill_block(
            self._h, ctypes.byref(d), _ptr(tokens, _I32, "tokens"), _ptr(E, _BF16, "E"),
            _ptr(Wq, _BF16, "Wq"), _ptr(Wk, _BF16, "Wk"), _ptr(Wv, _BF16, "Wv"), _ptr(Wo, _BF16, "Wo"),
            _ptr(Kp, _BF16, "Kp"), _ptr(Vt, _BF16, "Vt"), int(P), int(Kp.shape[1]),
            _ptr(ws, _U8, "ws"), _ptr(A, _BF16, "A"), ctypes.byref(out)))
        return int(out.value)

    def commit_kv(self, dims, tokens, E, Wk, Wv, Kp, Vt, P) -> int:
        d = Dims.of(dims)
        out = ctypes.c_int64(0)
        self._check(self._lib.dg_commit_kv(
            self._h, ctypes.byref(d), _ptr(tokens, _I32, "tokens"), _ptr(E, _BF16, "E"),
            _ptr(Wk, _BF16, "Wk"), _ptr(Wv, _BF16, "Wv"), _ptr(Kp, _BF16, "Kp"), _ptr(Vt, _BF16, "Vt"),
            int(P), int(Kp.shape[1]), ctypes.byref(out)))
        return int(out.value)

    def run_canvas(self, dims, weights, Kp, Vt, P, hidden, ws, loop_ws, x0, *, N, seed, canvas,
                   b=0.1, thr=0.005, tau0=0.8, tau1=0.4, commit="projection", rule="entropy",
                   draw="argmax"):
        """dg_run_canvas: one whole canvas (init, steps until the stop test or the cap N,
        the commit) sequenced in the library. hidden(k) -> H_k bf16 device tensor [C, d].
        commit: "projection" (dg_commit_kv) or "prefill" (dg_prefill_block, the causal
        re-encode; rotary positions as set by set_rope); rule: "entropy" or "confidence";
        draw: "argmax" or "sample" (as in CanvasLoop). Returns (steps run, new cache
        length P); x0 [C] int32 receives the committed block."""
        d = Dims.of(dims)
        w = Weights(*(_ptr(weights[k], _BF16, k) for k in ("E", "Wq", "Wk", "Wv", "Wo", "W1", "W2")))
        commits = {"projection": COMMIT_PROJECTION, "prefill": COMMIT_PREFILL}
        rules = {"entropy": RULE_ENTROPY, "confidence": RULE_CONFIDENCE}
        draws = {"argmax": DRAW_ARGMAX, "sample": DRAW_SAMPLE}
        if commit not in commits or rule not in rules or draw not in draws:
            raise ValueError(f"commit must be one of {tuple(commits)}, rule one of {tuple(rules)}, "
                             f"draw one of {tuple(draws)}")
        prm = LoopParams(int(N), float(b), float(thr), float(tau0), float(tau1), int(seed), int(canvas),
                         commits[commit], rules[rule], draws[draw])
        held, err = [], []

        def cb(_user, k):
            try:
                t = hidden(int(k))
                held.append(t)                  # alive until the kernels reading it have run
                return _ptr(t, _BF16, "H")
            except Exception as e:              # reported after the call; NULL ends the loop
                err.append(e)
                return None

        fn = HIDDEN_FN(cb)
        steps, p_out = ctypes.c_int32(0), ctypes.c_int64(0)
        st = self._lib.dg_run_canvas(
            self._h, ctypes.byref(d), ctypes.byref(w), _ptr(Kp, _BF16, "Kp"), _ptr(Vt, _BF16, "Vt"),
            int(P), int(Kp.shape[1]), ctypes.byref(prm), fn, None, _ptr(ws, _U8, "ws"),
            _ptr(loop_ws, _U8, "loop_ws"), _ptr(x0, _I32, "x0"), ctypes.byref(steps), ctypes.byref(p_out))
        # the last steps may still run on the device: keep their inputs until the next call
        self._held = held
        if err:
            raise err[0]
        self._check(st)
        return int(steps.value), int(p_out.value)
