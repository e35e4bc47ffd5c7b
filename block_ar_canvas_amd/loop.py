"""Block-autoregressive canvas loop over the libdg calls.

The loop follows the DiffusionGemma inference steps (Technical Report page, "Method
steps" (2)-(5); tutorial chapter "DiffusionGemma", data-flow pseudocode): initialize
a canvas with uniform tokens and z = 0, run at most N denoise steps (attention,
sampler head, acceptance, renoise, stop test, self-conditioning; under the entropy rule
acceptance, renoise and the stop test run beside self-conditioning's reduce, since they
read only the sampler head's entropies and argmaxes), then commit the finalized block
x0 = argmax to the KV cache and start the next canvas.

This module only sequences calls and owns the device buffers of one canvas; every
step of the arithmetic is a libdg kernel. The sampler head reads hidden states from
a caller-supplied source (the synthetic driver standing in for the denoiser stack).
"""
from __future__ import annotations

import time

import torch

from . import STOP_GO, Context, Dims, reveal_count, temperature, workspace_bytes

RULES = ("entropy", "confidence")
DRAWS = ("argmax", "sample")
COMMITS = ("projection", "prefill")


class CanvasLoop:
    """Device state and buffers for denoising canvases of one model/cache shape.

    weights: dict of bf16 device tensors E, Wq, Wk, Wv, Wo, W1, W2 ([out, in] layout).
    Kp [Hkv, Pcap, hd] and Vt [Hkv, hd, Pcap] bf16 device tensors: the KV cache.
    rule: "entropy" (entropy-bounded acceptance with budget b) or "confidence" (the
    reveal_count(C, N, k) most confident positions of step k are accepted).
    draw: "argmax" (accepted positions and the commit take x0 = argmax) or "sample"
    (they take x~ ~ p0 drawn by dg_sample); the stop test compares argmaxes either way.
    commit: "projection" (dg_commit_kv: K/V = E[x0] W^T) or "prefill" (dg_prefill_block:
    the causal re-encode); rope_base > 0 sets the context's rotary positions (used by
    canvas attention and the prefill).
    """

    def __init__(self, ctx: Context, dims, weights, Kp, Vt, P: int, *, N: int, seed: int,
                 b: float = 0.1, thr: float = 0.005, tau0: float = 0.8, tau1: float = 0.4,
                 rule: str = "entropy", draw: str = "argmax", commit: str = "projection",
                 rope_base: float = 0.0):
        if rule not in RULES or draw not in DRAWS or commit not in COMMITS:
            raise ValueError(f"rule must be one of {RULES}, draw one of {DRAWS}, commit one of {COMMITS}")
        self.rule, self.draw, self.commit_mode = rule, draw, commit
        self.ctx, self.dims = ctx, Dims.of(dims)
        ctx.set_rope(rope_base)
        self.W, self.Kp, self.Vt, self.P = weights, Kp, Vt, int(P)
        self.N, self.seed, self.b, self.thr, self.tau0, self.tau1 = N, seed, b, thr, tau0, tau1
        dev = Kp.device
        C, d = self.dims.C, self.dims.d
        self.ws = torch.empty(workspace_bytes(self.dims, Kp.shape[1]), dtype=torch.uint8, device=dev)
        self.tokens = torch.empty(C, dtype=torch.int32, device=dev)
        self.z = torch.zeros(C, d, dtype=torch.bfloat16, device=dev)
        self.A = torch.empty(C, d, dtype=torch.bfloat16, device=dev)
        self.entropy = torch.empty(C, dtype=torch.float32, device=dev)
        self.conf = torch.empty(C, dtype=torch.float32, device=dev)
        self.argmax = [torch.empty(C, dtype=torch.int32, device=dev) for _ in range(2)]
        self.sampled = [torch.empty(C, dtype=torch.int32, device=dev) for _ in range(2)]
        self.accept = torch.empty(C, dtype=torch.uint8, device=dev)
        self.n_accept = torch.empty(1, dtype=torch.int32, device=dev)
        # The next step's attention input bf16(E[tokens] + z), formed by the entropy rule's
        # self-conditioning call; _x_for records the (canvas, step) that formed it and the
        # torch version counters of tokens and z then, so a step uses it only if nothing
        # has rewritten them since (a restored state, a caller's edit).
        self.X = torch.empty(C, d, dtype=torch.bfloat16, device=dev)
        self._x_for = None
        # Stop flags live in pinned host memory; the stop test writes them with
        # system-scope stores, the host pre-fills -1 when it enqueues the step and polls,
        # so no copy or event sits between two steps' kernels on the stream. Steps take
        # the four buffers in enqueue order: when a step is enqueued, at most the two
        # steps before it may still be pending (the driving loop enqueues step k + 1 before
        # waiting for step k, and a canvas switch adds one speculative step), so a buffer
        # is never refilled while an older step's stop test may still write it.
        self.flags = [torch.full((1,), -1, dtype=torch.int32, pin_memory=True) for _ in range(4)]
        self._seq = 0
        self._slot = {}
        # When lists, every step appends a (start, end) pair of timing events recorded
        # on the context's stream around its dg_logits_entropy / dg_selfcond call.
        self.logits_events = None
        self.selfcond_events = None

    def init_canvas(self, canvas: int):
        """Uniform random canvas (init stream) and z = 0."""
        self.ctx.renoise(self.dims.V, None, None, self.seed, canvas, 0, self.tokens)
        self.canvas = canvas
        self._slot = {}
        self._x_for = None

    def step(self, k: int, H):
        """Enqueues denoise step k on hidden states H [C, d]; wait_flag(k) returns its flag."""
        W, dm = self.W, self.dims
        am, prev = self.argmax[k & 1], (self.argmax[(k - 1) & 1] if k > 0 else None)
        if k > 0 and self._x_for == (self.canvas, k - 1, self.tokens._version, self.z._version):
            self.ctx.canvas_attn_x(dm, self.X, W["Wq"], W["Wk"], W["Wv"], W["Wo"], self.Kp, self.Vt, self.P,
                                   self.ws, self.A)
        else:
            self.ctx.canvas_attn(dm, self.tokens, self.z if k > 0 else None, W["E"], W["Wq"], W["Wk"],
                                 W["Wv"], W["Wo"], self.Kp, self.Vt, self.P, self.ws, self.A)
        tau = temperature(k, self.N, self.tau0, self.tau1)
        ev = self.logits_events
        if ev is not None:
            e0 = torch.cuda.Event(enable_timing=True)
            e0.record(self.ctx.torch_stream())
        self.ctx.logits_entropy(dm, H, W["E"], tau, self.ws, self.entropy, am)
        if ev is not None:
            e1 = torch.cuda.Event(enable_timing=True)
            e1.record(self.ctx.torch_stream())
            ev.append((e0, e1))
        x0 = am
        if self.draw == "sample":
            x0 = self.sampled[k & 1]
            self.ctx.sample(dm, self.ws, 1, self.seed, self.canvas, k, x0)
        slot = self._seq % len(self.flags)
        self._seq += 1
        self._slot[k] = slot
        self.flags[slot].fill_(-1)
        if self.rule == "confidence":
            self.ctx.confidence(dm, self.ws, self.conf)
            self.ctx.topk_accept(self.conf, reveal_count(dm.C, self.N, k), self.accept, self.n_accept)
            self.ctx.renoise(dm.V, x0, self.accept, self.seed, self.canvas, k, self.tokens)
            self.ctx.stop_test(self.entropy, am, prev, self.thr, k, self.N, self.flags[slot])
        sev = self.selfcond_events
        if sev is not None:
            s0 = torch.cuda.Event(enable_timing=True)
            s0.record(self.ctx.torch_stream())
        if self.rule == "confidence":
            self.ctx.selfcond(dm, self.ws, W["E"], W["W1"], W["W2"], self.z)
            self._x_for = None
        else:
            # acceptance, renoise and the stop test run beside self-conditioning's reduce,
            # and its FFW forms the next step's attention input
            self.ctx.selfcond_accept(dm, self.ws, W["E"], W["W1"], W["W2"], self.z, self.entropy, self.b, x0,
                                     am, prev, self.seed, self.canvas, k, self.thr, self.N, self.accept,
                                     self.n_accept, self.tokens, self.flags[slot], x_next=self.X)
            self._x_for = (self.canvas, k, self.tokens._version, self.z._version)
        if sev is not None:
            s1 = torch.cuda.Event(enable_timing=True)
            s1.record(self.ctx.torch_stream())
            sev.append((s0, s1))
        return am

    def wait_flag(self, k: int, timeout_s: float = 60.0) -> int:
        """Returns step k's stop flag once the device has written it (polls the pinned
        flag; after timeout_s a full device synchronization settles it or raises)."""
        f = self.flags[self._slot[k]]
        deadline = time.monotonic() + timeout_s
        while True:
            v = int(f[0])
            if v >= 0:
                return v
            if time.monotonic() > deadline:
                torch.cuda.synchronize(self.Kp.device)
                v = int(f[0])
                if v >= 0:
                    return v
                raise RuntimeError(f"stop flag of step {k} was never written")

    def commit(self, x0):
        W = self.W
        if self.commit_mode == "prefill":
            self.P = self.ctx.prefill_block(self.dims, x0, W["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"],
                                            self.Kp, self.Vt, self.P, self.ws, self.A)
        else:
            self.P = self.ctx.commit_kv(self.dims, x0, W["E"], W["Wk"], W["Wv"], self.Kp, self.Vt, self.P)
        return self.P

    def run_canvas(self, canvas: int, hidden, on_step=None):
        """Init, denoise until the stop test or the cap, commit. Returns steps run.

        hidden(k) -> H_k device tensor; on_step(k, loop) is called with the state right
        after step k (before step k + 1 is enqueued). Step k + 1 is enqueued before the
        host waits for step k's flag, so the device never idles on the flag read; when
        step k stops the canvas, the speculative step k + 1 is discarded (the commit
        uses step k's own argmax buffer, which step k + 1 does not write).
        """
        self.init_canvas(canvas)
        with torch.cuda.stream(self.ctx.torch_stream()):
            self.z.zero_()
        k = 0
        self.step(0, hidden(0))
        if on_step is not None:
            on_step(0, self)
        while True:
            if k + 1 < self.N:
                self.step(k + 1, hidden(k + 1))
            if self.wait_flag(k) != STOP_GO:
                break
            k += 1
            if on_step is not None:
                on_step(k, self)
        self.commit(self.final_tokens(k))
        return k + 1

    def enqueue_canvas_fixed(self, canvas: int, hidden):
        """Enqueues a whole canvas without any host wait: init, all N steps, and the commit
        of the last step's block. There is no adaptive stop (the host reads no flag; the
        stop test still writes its flags), so the sequence is fixed and can be captured in
        a HIP graph and replayed. hidden(k) -> H_k device tensor, read at enqueue time.
        Returns the commit's new cache length."""
        self.init_canvas(canvas)
        for k in range(self.N):
            self.step(k, hidden(k))
        return self.commit(self.final_tokens(self.N - 1))

    def final_tokens(self, k: int):
        """The block step k commits: its argmax, or its sampled tokens under draw="sample"."""
        return (self.sampled if self.draw == "sample" else self.argmax)[k & 1]


class BatchLoop:
    """B canvases denoised in lockstep, one per request, each request with its own
    prefix KV cache (the pages' multi-request serving: several users' canvases share one
    pass of the vocabulary-wide kernels).

    Per step, canvas attention runs once per canvas against that canvas's cache; the
    sampler head and self-conditioning run once over all B*C positions (every position
    is its own column of the logits and of p0 E), and acceptance, renoise and the stop
    test run once with B segments of C positions. Canvas b of batch j has canvas id
    j*B + b (the renoise key). A batch ends when every canvas has stopped or reached
    the cap; a canvas that stops earlier keeps the argmax of its stop step, which is what
    its commit writes, while the others go on (its later steps are computed and ignored).

    caches: list of B (Kp [Hkv, Pcap, hd], Vt [Hkv, hd, Pcap], P) per request.
    rule, draw, commit and rope_base as in CanvasLoop.
    """

    def __init__(self, ctx: Context, dims, weights, caches, *, N: int, seed: int,
                 b: float = 0.1, thr: float = 0.005, tau0: float = 0.8, tau1: float = 0.4,
                 rule: str = "entropy", draw: str = "argmax", commit: str = "projection",
                 rope_base: float = 0.0):
        if rule not in RULES or draw not in DRAWS or commit not in COMMITS:
            raise ValueError(f"rule must be one of {RULES}, draw one of {DRAWS}, commit one of {COMMITS}")
        self.rule, self.draw, self.commit_mode = rule, draw, commit
        self.ctx, self.W = ctx, weights
        ctx.set_rope(rope_base)
        self.B = len(caches)
        self.dims = Dims.of(dims)                       # one canvas
        C, d = self.dims.C, self.dims.d
        self.dims_all = Dims(self.dims.V, d, self.B * C, self.dims.Hq, self.dims.Hkv,
                             self.dims.hd, self.dims.F)  # all B canvases as columns
        self.Kp = [c[0] for c in caches]
        self.Vt = [c[1] for c in caches]
        self.P = [int(c[2]) for c in caches]
        self.N, self.seed, self.b, self.thr, self.tau0, self.tau1 = N, seed, b, thr, tau0, tau1
        dev = self.Kp[0].device
        B = self.B
        self.ws_attn = torch.empty(workspace_bytes(self.dims, max(k.shape[1] for k in self.Kp)),
                                   dtype=torch.uint8, device=dev)
        self.ws = torch.empty(workspace_bytes(self.dims_all, 0), dtype=torch.uint8, device=dev)
        self.tokens = torch.empty(B, C, dtype=torch.int32, device=dev)
        self.z = torch.zeros(B, C, d, dtype=torch.bfloat16, device=dev)
        self.A = torch.empty(B, C, d, dtype=torch.bfloat16, device=dev)
        self.entropy = torch.empty(B, C, dtype=torch.float32, device=dev)
        self.conf = torch.empty(B, C, dtype=torch.float32, device=dev)
        self.argmax = [torch.empty(B, C, dtype=torch.int32, device=dev) for _ in range(2)]
        self.sampled = [torch.empty(B, C, dtype=torch.int32, device=dev) for _ in range(2)]
        self.accept = torch.empty(B, C, dtype=torch.uint8, device=dev)
        self.n_accept = torch.empty(B, dtype=torch.int32, device=dev)
        self.X = torch.empty(B, C, d, dtype=torch.bfloat16, device=dev)   # as in CanvasLoop
        self._x_for = None
        # Same protocol as CanvasLoop: pinned flags written by the stop kernel, four
        # buffers taken in enqueue order.
        self.flags = [torch.full((B,), -1, dtype=torch.int32, pin_memory=True) for _ in range(4)]
        self._seq = 0
        self._slot = {}
        self.logits_events = None          # as in CanvasLoop

    def init_batch(self, batch: int):
        """Uniform random canvases (init stream) for canvas ids batch*B .. batch*B+B-1, z = 0."""
        self.batch = batch
        self.ctx.renoise(self.dims.V, None, None, self.seed, batch * self.B, 0, self.tokens)
        with torch.cuda.stream(self.ctx.torch_stream()):
            self.z.zero_()
        self._slot = {}
        self._x_for = None

    def step(self, k: int, H):
        """Enqueues denoise step k of every canvas; H [B*C, d] holds the canvases' hidden
        states in canvas order."""
        W, dm = self.W, self.dims
        am, prev = self.argmax[k & 1], (self.argmax[(k - 1) & 1] if k > 0 else None)
        use_x = k > 0 and self._x_for == (self.batch, k - 1, self.tokens._version, self.z._version)
        for i in range(self.B):
            if use_x:
                self.ctx.canvas_attn_x(dm, self.X[i], W["Wq"], W["Wk"], W["Wv"], W["Wo"], self.Kp[i], self.Vt[i],
                                       self.P[i], self.ws_attn, self.A[i])
            else:
                self.ctx.canvas_attn(dm, self.tokens[i], self.z[i] if k > 0 else None, W["E"], W["Wq"],
                                     W["Wk"], W["Wv"], W["Wo"], self.Kp[i], self.Vt[i], self.P[i],
                                     self.ws_attn, self.A[i])
        tau = temperature(k, self.N, self.tau0, self.tau1)
        ev = self.logits_events
        if ev is not None:
            e0 = torch.cuda.Event(enable_timing=True)
            e0.record(self.ctx.torch_stream())
        self.ctx.logits_entropy(self.dims_all, H, W["E"], tau, self.ws, self.entropy.view(-1),
                                am.view(-1))
        if ev is not None:
            e1 = torch.cuda.Event(enable_timing=True)
            e1.record(self.ctx.torch_stream())
            ev.append((e0, e1))
        x0 = am
        if self.draw == "sample":
            x0 = self.sampled[k & 1]
            self.ctx.sample(self.dims_all, self.ws, self.B, self.seed, self.batch * self.B, k, x0.view(-1))
        slot = self._seq % len(self.flags)
        self._seq += 1
        self._slot[k] = slot
        self.flags[slot].fill_(-1)
        base = self.batch * self.B
        if self.rule == "confidence":
            self.ctx.confidence(self.dims_all, self.ws, self.conf.view(-1))
            self.ctx.topk_accept(self.conf, reveal_count(dm.C, self.N, k), self.accept, self.n_accept)
            self.ctx.renoise(dm.V, x0, self.accept, self.seed, base, k, self.tokens)
            self.ctx.stop_test(self.entropy, am, prev, self.thr, k, self.N, self.flags[slot])
            self.ctx.selfcond(self.dims_all, self.ws, W["E"], W["W1"], W["W2"], self.z.view(-1, dm.d))
            self._x_for = None
        else:
            self.ctx.selfcond_accept(self.dims_all, self.ws, W["E"], W["W1"], W["W2"], self.z.view(-1, dm.d),
                                     self.entropy, self.b, x0, am, prev, self.seed, base, k, self.thr, self.N,
                                     self.accept, self.n_accept, self.tokens, self.flags[slot],
                                     x_next=self.X.view(-1, dm.d))
            self._x_for = (self.batch, k, self.tokens._version, self.z._version)
        return am

    def wait_flags(self, k: int, timeout_s: float = 60.0):
        """Step k's stop flags (one per canvas) once the device has written them all."""
        f = self.flags[self._slot[k]]
        deadline = time.monotonic() + timeout_s
        while True:
            v = f.tolist()
            if min(v) >= 0:
                return v
            if time.monotonic() > deadline:
                torch.cuda.synchronize(self.Kp[0].device)
                v = f.tolist()
                if min(v) >= 0:
                    return v
                raise RuntimeError(f"stop flags of step {k} were never written")

    def run_batch(self, batch: int, hidden, on_step=None):
        """Init, denoise until every canvas has stopped or capped, commit every canvas.
        Returns each canvas's step count. hidden(k) -> [B*C, d] device tensor; on_step as
        in CanvasLoop.run_canvas. Step k + 1 is enqueued before the host reads step k's
        flags; x0 of a canvas that stops at step k is copied from step k's argmax buffer
        before step k + 2, the next writer of that buffer, is enqueued."""
        self.init_batch(batch)
        B, C = self.B, self.dims.C
        x0 = [None] * B
        steps = [0] * B
        k = 0
        self.step(0, hidden(0))
        if on_step is not None:
            on_step(0, self)
        while True:
            if k + 1 < self.N:
                self.step(k + 1, hidden(k + 1))
            flags = self.wait_flags(k)
            for i in range(B):
                if x0[i] is None and flags[i] != STOP_GO:
                    # the copy is ordered on the context's stream before step k + 2, the
                    # next writer of this buffer
                    with torch.cuda.stream(self.ctx.torch_stream()):
                        x0[i] = (self.sampled if self.draw == "sample" else self.argmax)[k & 1][i].clone()
                    steps[i] = k + 1
            if all(x is not None for x in x0):
                break
            k += 1
            if on_step is not None:
                on_step(k, self)
        W = self.W
        for i in range(B):
            if self.commit_mode == "prefill":
                self.P[i] = self.ctx.prefill_block(self.dims, x0[i], W["E"], W["Wq"], W["Wk"], W["Wv"],
                                                   W["Wo"], self.Kp[i], self.Vt[i], self.P[i],
                                                   self.ws_attn, self.A[i])
            else:
                self.P[i] = self.ctx.commit_kv(self.dims, x0[i], W["E"], W["Wk"], W["Wv"], self.Kp[i],
                                               self.Vt[i], self.P[i])
        return steps
