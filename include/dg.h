/*
 * dg.h - C ABI of the MI355X (gfx950) canvas-denoise step of a block-autoregressive
 * uniform-state text diffusion model (DiffusionGemma's sampler loop).
 *
 * One denoise step of the 256-token canvas is, in call order:
 *   dg_canvas_attn     bidirectional canvas attention over the static prefix KV cache
 *   dg_logits_entropy  lm_head logits fused with tempered softmax, entropy and argmax
 *   dg_entropy_accept  entropy-bounded acceptance (segmented sort + fixed-point scan)
 *   dg_renoise         accepted positions keep the argmax, the rest are redrawn
 *   dg_selfcond        self-conditioning z = FFW(p0 . E)
 *   dg_stop_test       adaptive stop (mean entropy and stable argmax) / step cap
 * and, once per canvas, dg_commit_kv appends the finalized block to the KV cache.
 * dg_accept_renoise_stop runs acceptance, renoise and the stop test in one launch, and
 * dg_selfcond_accept runs them beside self-conditioning's reduce (and can form the next
 * step's attention input, which dg_canvas_attn_x takes).
 * Beyond that step: dg_prefill_block (the causal re-encode commit) with dg_set_rope,
 * dg_confidence / dg_topk_accept / dg_reveal_count (confidence-ranked acceptance),
 * dg_sample (sampled tokens), dg_moe_ffn (the canvas mixture-of-experts FFN),
 * dg_run_canvas (a whole canvas of the loop, sequenced in the library), and the
 * measured ceilings dg_peak_stream_read / dg_peak_mfma_bf16.
 * The method is the DiffusionGemma inference loop as summarized by the
 * "DiffusionGemma Technical Report" page (paper.rainbus.top/paper/2608.00146),
 * section "Method steps" (1)-(5), with the sampler hyper-parameters of its
 * "Reproducibility" section (canvas 256, N = 48, b = 0.1, stop 0.005, tau 0.8 -> 0.4).
 *
 * Conventions for every call
 *  - Tensor arguments are DEVICE pointers owned by the caller (contiguous, row-major,
 *    16-byte aligned). bf16 values are raw IEEE bfloat16 bit patterns (dg_bf16).
 *  - Weights use the [out_features, in_features] row-major layout.
 *  - The KV cache of one layer is two arrays:
 *        Kp [Hkv][Pcap][hd]   keys, one row per cached token
 *        Vt [Hkv][hd][Pcap]   values stored transposed (token index fastest)
 *    Rows / columns [0, P) hold the prefix; [P, Pcap) is free capacity.
 *  - Calls validate their arguments on the host, enqueue work on the context's HIP
 *    stream and return without waiting. No call allocates or frees device memory;
 *    scratch space comes from the caller's workspace (dg_workspace_bytes,
 *    dg_moe_workspace_bytes). The context itself holds a status word, a second
 *    stream and two events (for dg_moe_ffn), all made by dg_create.
 *  - On a non-OK return nothing was enqueued; dg_last_error() describes the problem.
 *  - Conditions only the device can see (a token id outside [0, V), non-finite
 *    logits) set a sticky status word in the context, reported by dg_sync().
 *  - A context is used by one host thread at a time. Every call that enqueues work or
 *    waits on the device first makes the context's device current on the calling thread.
 *    No C++ exception crosses the ABI.
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t dg_bf16;
typedef struct dg_ctx_s *dg_ctx;

typedef enum {
  DG_OK = 0,
  DG_ERR_NULL = 1,        /* a required pointer is NULL                                  */
  DG_ERR_SHAPE = 2,       /* a dimension is out of the supported set                     */
  DG_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned / Pcap not a multiple of 8 */
  DG_ERR_RANGE = 4,       /* a scalar is out of range (tau <= 0, b < 0, token id, ...)   */
  DG_ERR_CAPACITY = 5,    /* P + C > Pcap (the KV cache has no room), or static scratch  */
  DG_ERR_STATE = 6,       /* dg_selfcond without a matching dg_logits_entropy            */
  DG_ERR_NONFINITE = 7,   /* device saw non-finite logits (sticky, via dg_sync)          */
  DG_ERR_HIP = 8,         /* a HIP runtime call failed                                   */
  DG_ERR_UNSUPPORTED = 9
} dg_status;

/* Model / canvas shape.
 *  V   vocabulary size (rows of the tied embedding / lm_head table E)      1 <= V < 2^31
 *  d   model width                                               multiple of 32, <= 16384
 *  C   canvas length (positions denoised together)                              1..1024
 *  Hq  query heads, Hkv key/value heads (Hq % Hkv == 0)
 *  hd  head dimension                                                 16, 32, 64 or 128
 *  F   self-conditioning FFW hidden width                        multiple of 32, <= 16384 */
typedef struct {
  int32_t V, d, C, Hq, Hkv, hd, F;
} dg_dims;

/* ---------------------------------------------------------------- context */
/* Creates a context on HIP device `device` that enqueues on `hip_stream`
 * (a hipStream_t; NULL = the device's null stream). Allocates the context's status
 * word on the device and makes its second stream (default priority) and the two events
 * dg_moe_ffn forks and joins with. */
dg_status dg_create(dg_ctx *out, int device, void *hip_stream);
void dg_destroy(dg_ctx ctx);
/* Switches the stream later calls enqueue on. */
dg_status dg_set_stream(dg_ctx ctx, void *hip_stream);
/* Human-readable description of the last non-OK status of this context. */
const char *dg_last_error(dg_ctx ctx);
/* Waits for the stream; returns the sticky device status (DG_ERR_RANGE for an
 * out-of-range token id, DG_ERR_NONFINITE for non-finite logits) or DG_OK. */
dg_status dg_sync(dg_ctx ctx);
/* Clears the sticky device status (enqueued, stream-ordered). */
dg_status dg_clear_status(dg_ctx ctx);

/* Bytes of device workspace one step needs for these dims and cache capacity.
 * The same workspace is passed to dg_canvas_attn, dg_logits_entropy and dg_selfcond;
 * dg_selfcond consumes what the preceding dg_logits_entropy left in it. */
size_t dg_workspace_bytes(const dg_dims *dims, int64_t Pcap);

/* Annealed temperature of step k of a budget of N steps (host only, pure):
 * tau_k = float(tau0 + (tau1 - tau0) * k / (N - 1)) evaluated in double; N <= 1 gives
 * tau0. Linear decrease 0.8 -> 0.4: tutorial chapter "DiffusionGemma" (sampler
 * configuration) and the Technical Report page, "Method steps" (3). */
float dg_temperature(int32_t k, int32_t N, float tau0, float tau1);

/* ---------------------------------------------------------------- the step */
/* Bidirectional canvas attention (Google "DiffusionGemma explained", section
 * "Architecture: incremental prefill and denoising": in denoise mode a query at any
 * canvas position attends to every canvas token and to the KV cache, with no mask).
 *   X  = bf16(E[tokens] + z)                   denoiser input [C, d] (z NULL: 0)
 *   Q  = bf16(X Wq^T), Kc = bf16(X Wk^T), Vc = bf16(X Wv^T)
 *   O_h = softmax(Q_h [Kp_g ; Kc_g]^T / sqrt(hd)) [Vp_g ; Vc_g],  g = floor(h*Hkv/Hq)
 *   A  = bf16(O Wo^T)                           [C, d]
 * tokens [C] int32 (an id outside [0, V) sets DG_ERR_RANGE on the device and is read as id 0);
 * z [C, d] or NULL; E [V, d]; Wq [Hq*hd, d]; Wk, Wv [Hkv*hd, d]; Wo [d, Hq*hd];
 * Kp, Vt: the KV cache (layout above) holding P tokens (0 <= P <= Pcap, Pcap % 8 == 0);
 * the cache is only read. ws: workspace; A [C, d] output. */
dg_status dg_canvas_attn(dg_ctx ctx, const dg_dims *dims, const int32_t *tokens,
                         const dg_bf16 *z, const dg_bf16 *E, const dg_bf16 *Wq,
                         const dg_bf16 *Wk, const dg_bf16 *Wv, const dg_bf16 *Wo,
                         const dg_bf16 *Kp, const dg_bf16 *Vt, int64_t P, int64_t Pcap,
                         void *ws, dg_bf16 *A);

/* dg_canvas_attn on a denoiser input the caller formed: X [C, d] bf16 in place of
 * bf16(E[tokens] + z) (for instance the x_next of the previous step's dg_selfcond_accept,
 * which saves the gather launch). Same results as dg_canvas_attn given the tokens and z
 * that X was formed from; same layouts, workspace and errors (X must be 16-byte aligned). */
dg_status dg_canvas_attn_x(dg_ctx ctx, const dg_dims *dims, const dg_bf16 *X, const dg_bf16 *Wq,
                           const dg_bf16 *Wk, const dg_bf16 *Wv, const dg_bf16 *Wo,
                           const dg_bf16 *Kp, const dg_bf16 *Vt, int64_t P, int64_t Pcap,
                           void *ws, dg_bf16 *A);

/* dg_canvas_attn without a workspace argument and without any allocation, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation. Same arguments (minus ws), validation,
 * kernels and results as dg_canvas_attn; its scratch (the denoiser input, Q and canvas
 * K/V, the attention output before Wo and the split partials) lives in one
 * DG_STATIC_SCRATCH_BYTES array per device inside the library, held until the process
 * ends. Every call on a device shares that device's array, so calls that overlap on one
 * device (several streams or host threads, or contexts on different streams) race and
 * must be serialized by the caller; nothing in it needs to start zeroed.
 * DG_ERR_CAPACITY (nothing enqueued) when the dims need more than the array holds
 * (about 20.5 MiB at C 256, d 2048, 16 query / 8 KV heads of 128, any prefix length);
 * DG_ERR_HIP when the array's address could not be found on this device. */
#define DG_STATIC_SCRATCH_BYTES ((size_t)48 << 20)
dg_status dg_canvas_attn_static(dg_ctx ctx, const dg_dims *dims, const int32_t *tokens,
                                const dg_bf16 *z, const dg_bf16 *E, const dg_bf16 *Wq,
                                const dg_bf16 *Wk, const dg_bf16 *Wv, const dg_bf16 *Wo,
                                const dg_bf16 *Kp, const dg_bf16 *Vt, int64_t P, int64_t Pcap,
                                dg_bf16 *A);

/* Sampler head (Technical Report page, "Method steps" (3)): logits H E^T, softmax at
 * temperature tau giving p0, per-position Shannon entropy in nats (clamped at 0) and
 * argmax (ties to the lowest id). H [C, d]; E [V, d]; tau > 0. Writes entropy [C]
 * float32 and argmax [C] int32, and leaves p0 (as bf16 per-tile scaled probabilities
 * plus fp32 tile statistics) in ws for dg_selfcond; the C x V probabilities are never
 * materialized in fp32. Non-finite logits give a NaN entropy and argmax 0 for that
 * position and set DG_ERR_NONFINITE. */
dg_status dg_logits_entropy(dg_ctx ctx, const dg_dims *dims, const dg_bf16 *H,
                            const dg_bf16 *E, float tau, void *ws, float *entropy,
                            int32_t *argmax);

/* Entropy-bounded acceptance for B independent canvases of C positions (Technical
 * Report page, "Method steps" (3) and "Technical novelty": sort by entropy ascending,
 * accept within the cumulative entropy budget b). Sums use 2^-32 fixed point:
 * q = ceil(h * 2^32), order = (h, position) ascending, accept the longest prefix with
 * sum q <= floor(b * 2^32). Zero accepted positions is legal. Entropies that are NaN,
 * infinite or >= 65536 are never accepted; negative ones count as 0.
 * entropy [B, C] float32; 0 <= b < 65536; accept [B, C] uint8 (0/1); n_accept [B]. */
dg_status dg_entropy_accept(dg_ctx ctx, int32_t B, int32_t C, const float *entropy,
                            float b, uint8_t *accept, int32_t *n_accept);

/* Confidence of every canvas position: the largest probability of its tempered p0,
 * max_v p0[c][v] = 2^(m - R) / Z in the log2-unit statistics the logits pass keeps (m the
 * column's largest tempered logit, R its reference, Z the sum relative to 2^R); NaN for
 * a column whose logits were not finite. It is the score confidence decoding ranks
 * positions by (openai-hub page "从零拆开DiffusionGemma", step 4; "Text diffusion
 * models" survey, section 5). ws must hold the p0 of the immediately preceding
 * dg_logits_entropy with these dims (DG_ERR_STATE otherwise).
 * confidence [C] float32 output. */
dg_status dg_confidence(dg_ctx ctx, const dg_dims *dims, const void *ws, float *confidence);

/* Confidence-ranked acceptance (same pages): in each of B segments of C positions,
 * accept the k positions with the highest score; equal scores are taken in position
 * order (compared by value bits, so -0 ranks below +0), and NaN scores are never
 * accepted. k > C accepts every non-NaN position; k < 0 is DG_ERR_RANGE.
 * score [B, C] float32; accept [B, C] uint8 (0/1); n_accept [B] int32. */
dg_status dg_topk_accept(dg_ctx ctx, int32_t B, int32_t C, const float *score, int32_t k,
                         uint8_t *accept, int32_t *n_accept);

/* Sampled tokens x~ ~ p0, the sampled-token alternative to x0 = argmax (openai-hub page
 * "从零拆开DiffusionGemma", step 4: real samplers draw from the tempered distribution
 * rather than always taking the most likely token). ws must hold the p0 of the
 * immediately preceding dg_logits_entropy with these dims (DG_ERR_STATE otherwise).
 * The draw is the inverse CDF over the whole vocabulary in id order: for column
 * c = b * Cs + i (canvas canvas_base + b, position i, Cs = C / B), with
 * u = (word 0 of Philox4x64-10 under key (seed, canvas_base + b) and counter
 * (i, step, 2, 0)) >> 11, divided by 2^53, the token is the first id v whose cumulative
 * probability sum_{v' <= v} p0[c][v'] exceeds u times the total. On the device the
 * cumulative comes from the float32 per-tile sums and, inside the tile that holds the
 * crossing, from the stored bf16 probabilities, so a draw within about 2^-9 of that
 * tile's mass of a boundary may take the neighbouring id.
 * tokens [C] int32 output (0 for a column with non-finite logits).
 * DG_ERR_SHAPE unless B >= 1 divides C. */
dg_status dg_sample(dg_ctx ctx, const dg_dims *dims, const void *ws, int32_t B, uint64_t seed,
                    uint32_t canvas_base, uint32_t step, int32_t *tokens);

/* Host-side reveal schedule of confidence decoding (openai-hub page, step 4: each step
 * reveals ceil(unresolved / remaining steps) positions): the number of positions
 * revealed after steps 0..step of an N-step run over C positions,
 *   n_{-1} = 0,  n_t = n_{t-1} + ceil((C - n_{t-1}) / (N - t)),
 * so n_{N-1} = C; steps past N - 1 give C. Pure; -1 for C < 0, N < 1 or step < 0. */
int32_t dg_reveal_count(int32_t C, int32_t N, int32_t step);

/* Uniform-state renoise (Technical Report page, "Method steps" (2)-(3); Google page,
 * "Uniform State Diffusion"): accepted positions take argmax, every other position a
 * token drawn uniformly over [0, V):
 *   token = floor(r * V / 2^64),  r = word 0 of Philox4x64-10 with
 *   key (seed, canvas_base + s) and counter (position, step, stream, 0)
 * (Salmon et al., SC'11). stream = 0 for renoise; accept == NULL initializes a canvas:
 * every position is drawn on stream 1 and argmax may be NULL.
 * argmax, tokens [B, C] int32; accept [B, C] uint8 or NULL. */
dg_status dg_renoise(dg_ctx ctx, int32_t B, int32_t C, int32_t V, const int32_t *argmax,
                     const uint8_t *accept, uint64_t seed, uint32_t canvas_base,
                     uint32_t step, int32_t *tokens);

/* Self-conditioning (Technical Report page, "Method steps" (3): z = FFW(p0 E); Google
 * page, "Self-conditioning"): s = p0 E with p0 from the immediately preceding
 * dg_logits_entropy on the same workspace and dims, then z = bf16(GELU_erf(s W1^T) W2^T).
 * E [V, d]; W1 [F, d]; W2 [d, F]; z [C, d] output. A position whose logits were not
 * finite contributes s = 0, so its z row is 0. DG_ERR_STATE if ws does not hold the p0
 * of a matching dg_logits_entropy. */
dg_status dg_selfcond(dg_ctx ctx, const dg_dims *dims, void *ws, const dg_bf16 *E,
                      const dg_bf16 *W1, const dg_bf16 *W2, dg_bf16 *z);

/* Adaptive stop (Technical Report page, "Method steps" (4)): flag 1 when step >= 1,
 * the mean entropy is <= thr (sum ceil(h 2^32) <= floor(thr * C * 2^32), every entropy
 * in the valid domain) and argmax equals prev_argmax at every position; else 2 when
 * step >= N - 1 (step cap: commit anyway); else 0. prev_argmax may be NULL (no stop).
 * entropy [B, C]; argmax, prev_argmax [B, C]; 0 <= thr < 65536; flag [B] int32.
 * flag may be device memory or pinned host memory (hipHostMalloc): it is written with
 * system-scope stores, so a host that pre-fills it with a value outside {0, 1, 2} can
 * poll it for the result without a stream synchronization. */
dg_status dg_stop_test(dg_ctx ctx, int32_t B, int32_t C, const float *entropy,
                       const int32_t *argmax, const int32_t *prev_argmax, float thr,
                       int32_t step, int32_t N, int32_t *flag);

/* The acceptance, renoise and stop test of one step in one launch (the same passages as
 * the three calls): the results are those of
 *   dg_entropy_accept(B, C, entropy, b, accept, n_accept);
 *   dg_renoise(B, C, V, x0, accept, seed, canvas_base, step, tokens);
 *   dg_stop_test(B, C, entropy, argmax, prev_argmax, thr, step, N, flag);
 * in that order, bit for bit. x0 is what accepted positions keep (the argmax, or the
 * dg_sample draws); argmax and prev_argmax are what the stop test compares (prev_argmax
 * may be NULL). tokens must not overlap entropy, x0, argmax or prev_argmax.
 * Shapes and errors as in the three calls: 1 <= C <= 1024, V >= 1, 0 <= b, thr < 65536,
 * step >= 0, N >= 1. */
dg_status dg_accept_renoise_stop(dg_ctx ctx, int32_t B, int32_t C, int32_t V,
                                 const float *entropy, float b, const int32_t *x0,
                                 const int32_t *argmax, const int32_t *prev_argmax,
                                 uint64_t seed, uint32_t canvas_base, int32_t step, float thr,
                                 int32_t N, uint8_t *accept, int32_t *n_accept,
                                 int32_t *tokens, int32_t *flag);

/* dg_accept_renoise_stop and dg_selfcond of one step in one call, with the results of
 *   dg_accept_renoise_stop(B, C / B, V, entropy, b, x0, argmax, prev_argmax, seed,
 *                          canvas_base, step, thr, N, accept, n_accept, tokens, flag);
 *   dg_selfcond(dims, ws, E, W1, W2, z);
 * bit for bit (C and V from dims; the other arguments from *acc). For canvases of up to
 * 256 positions the acceptance work runs as extra workgroups of the self-conditioning
 * reduce launch, beside the reduce, instead of in a launch of its own; the stop flag is
 * then written while s is reduced. Larger canvases take a launch of its own first.
 * accept, n_accept, tokens and flag must not overlap ws or z. With x_next non-NULL it also
 * writes x_next = bf16(E[tokens] + z) for the new tokens and z, the input the next step's
 * dg_canvas_attn would form (bit for bit), so that step can take dg_canvas_attn_x.
 * Errors: those of both calls, checked before anything is enqueued; DG_ERR_SHAPE unless
 * B >= 1 divides C; DG_ERR_ALIGN for an x_next that is not 16-byte aligned. */
typedef struct {
  int32_t B;                 /* canvases; dims->C / B positions each */
  const float *entropy;      /* [B, C/B] */
  float b;                   /* acceptance budget */
  const int32_t *x0;         /* what accepted positions keep */
  const int32_t *argmax, *prev_argmax;  /* compared by the stop test; prev may be NULL */
  uint64_t seed;
  uint32_t canvas_base;
  int32_t step;
  float thr;                 /* stop threshold */
  int32_t N;                 /* step cap */
  uint8_t *accept;           /* [B, C/B] output */
  int32_t *n_accept;         /* [B] output */
  int32_t *tokens;           /* [B, C/B] output */
  int32_t *flag;             /* [B] output, device or pinned host memory */
  dg_bf16 *x_next;           /* [C, d] output or NULL: bf16(E[tokens] + z), the next step's
                                dg_canvas_attn_x input (formed in the FFW's epilogue) */
} dg_accept_args;
dg_status dg_selfcond_accept(dg_ctx ctx, const dg_dims *dims, void *ws, const dg_bf16 *E,
                             const dg_bf16 *W1, const dg_bf16 *W2, dg_bf16 *z,
                             const dg_accept_args *acc);

/* Rotary positions (openai-hub page "从零拆开DiffusionGemma", closing remarks of step 3:
 * the full model has rotary position encoding) for dg_canvas_attn and dg_prefill_block
 * of this context: base 0 (the default) turns them off; base > 0 rotates, in every head,
 * the pair (q_d, q_{d+hd/2}) of a token at position p by p * base^(-2d/hd) (half-split
 * pairing), in queries and keys, after the bf16 projection, re-rounded to bf16. Canvas
 * and block token i sits at position P + i; cached prefix keys are taken as rotated.
 * DG_ERR_RANGE for a negative or non-finite base. */
dg_status dg_set_rope(dg_ctx ctx, float base);

/* Causal re-encode of a finalized block (tutorial chapter "DiffusionGemma": the data-flow
 * pseudocode's incremental prefill of the finalized block, and the KV-cache write
 * timing: the next context comes from the backbone re-encoding the block causally, not
 * from the denoiser's states). One attention layer stands in for the backbone:
 * X = E[tokens]; Q, K, V = bf16(X W^T), Q and K rotated to positions P + i when the
 * context has a rotary base; block token i attends to the prefix [0, P) and to block
 * tokens j <= i; A = bf16(O Wo^T). The block's (rotated) K and V rows are appended at
 * [P, P + C), and *P_out (host) = P + C. Same layouts as dg_canvas_attn; A [C, d] output.
 * DG_ERR_CAPACITY (nothing enqueued) when P + C > Pcap. */
dg_status dg_prefill_block(dg_ctx ctx, const dg_dims *dims, const int32_t *tokens,
                           const dg_bf16 *E, const dg_bf16 *Wq, const dg_bf16 *Wk,
                           const dg_bf16 *Wv, const dg_bf16 *Wo, dg_bf16 *Kp, dg_bf16 *Vt,
                           int64_t P, int64_t Pcap, void *ws, dg_bf16 *A, int64_t *P_out);

/* Canvas MoE FFN (Technical Report page, "Prerequisites", mixture of experts: 8 of 128
 * experts plus one shared expert per token, about 84 distinct experts per 256-token
 * canvas; "Text diffusion models" survey, sections 11 and 13: router top-k, expert GEMM,
 * token permutation). For every row x of X:
 *   router logits r = x Wr^T (float32); the K experts with the largest logits (ties to the
 *   lower expert id) with gates g = softmax of those K logits;
 *   y = bf16( sum_k g_k * bf16(W2_e GELU_erf(W1_e x)) + bf16(W2s GELU_erf(W1s x)) ),
 *   each expert's hidden layer rounded to bf16 as well (the self-conditioning FFW's form).
 * X [C, d]; Wr [E, d]; W1 [E][Fe][d]; W2 [E][d][Fe]; W1s [Fs, d]; W2s [d, Fs]; Y [C, d]
 * output; n_active (device, optional) = the number of distinct experts used. The
 * workspace holds dg_moe_workspace_bytes(m, C) bytes. DG_ERR_SHAPE unless d, Fe, Fs are
 * positive multiples of 32, 1 <= K <= min(E, 32), E <= 256, C <= 1024 and C * K <= 8192.
 * The shared expert runs on a second stream of the context (made by dg_create,
 * default priority), forked from and joined back into the context's stream with events:
 * the call stays ordered on the context's stream like every other call. */
typedef struct { int32_t d, E, K, Fe, Fs; } dg_moe_dims;
size_t dg_moe_workspace_bytes(const dg_moe_dims *m, int32_t C);
dg_status dg_moe_ffn(dg_ctx ctx, const dg_moe_dims *m, int32_t C, const dg_bf16 *X,
                     const dg_bf16 *Wr, const dg_bf16 *W1, const dg_bf16 *W2, const dg_bf16 *W1s,
                     const dg_bf16 *W2s, void *ws, dg_bf16 *Y, int32_t *n_active);

/* Commit (Technical Report page, "Method steps" (5); tutorial chapter "DiffusionGemma",
 * KV-cache write timing): appends the finalized block's keys and values at token
 * positions [P, P + C) of every KV head: K = bf16(E[tokens] Wk^T), V = bf16(E[tokens]
 * Wv^T) (a stand-in for the causal re-encode of the block). Rows [0, P) are not touched.
 * tokens [C] int32 (x0 = argmax); Kp, Vt in/out; *P_out (host) = P + C.
 * An id outside [0, V) sets DG_ERR_RANGE on the device and is read as id 0.
 * DG_ERR_CAPACITY (nothing written) when P + C > Pcap. */
dg_status dg_commit_kv(dg_ctx ctx, const dg_dims *dims, const int32_t *tokens,
                       const dg_bf16 *E, const dg_bf16 *Wk, const dg_bf16 *Wv,
                       dg_bf16 *Kp, dg_bf16 *Vt, int64_t P, int64_t Pcap, int64_t *P_out);

/* ---------------------------------------------------------------- the canvas loop */
/* One whole canvas of the block-autoregressive loop (Technical Report page, "Method
 * steps" (2)-(5); tutorial chapter "DiffusionGemma", data-flow pseudocode), sequenced in
 * the library: a uniform random canvas (dg_renoise with accept = NULL), then denoise
 * steps k = 0, 1, ... of
 *   dg_canvas_attn (z = 0 at k = 0), dg_logits_entropy on H_k at dg_temperature(k, N,
 *   tau0, tau1), dg_selfcond_accept (acceptance with budget b, renoise of the rejected
 *   positions, the stop test against the previous step's argmax, self-conditioning),
 * until the stop test fires or the cap N is reached, then the commit of that step's
 * block. With rule = DG_RULE_CONFIDENCE the step runs dg_confidence, dg_topk_accept with
 * dg_reveal_count(C, N, k), dg_renoise, dg_stop_test and dg_selfcond instead of
 * dg_selfcond_accept; with draw = DG_DRAW_SAMPLE, dg_sample draws x~ after the sampler
 * head, accepted positions keep x~ and the commit takes the last step's x~ instead of its
 * argmax (the stop test compares argmaxes either way). The commit: dg_commit_kv (commit = DG_COMMIT_PROJECTION) or the causal re-encode
 * dg_prefill_block (commit = DG_COMMIT_PREFILL; its attention output goes to loop_ws);
 * both attention calls use the context's rotary setting (dg_set_rope). Step k + 1 is enqueued before the host waits for step k's flag (pinned host
 * memory of the context, polled: no stream synchronization between steps); when step k
 * stops the canvas, step k + 1's results are discarded (it writes the other argmax
 * buffer, and the commit reads step k's).
 * hidden(user, k) is called on the host before step k is enqueued and returns the device
 * pointer of H_k [C, d] bf16; it may enqueue work producing H_k on the context's stream.
 * loop_ws holds dg_loop_workspace_bytes(dims) bytes (the canvas tokens, z, the attention
 * output, entropies, both argmax and sampled-token buffers, acceptance, confidences, and
 * the next step's attention input, which the entropy rule's steps form for
 * dg_canvas_attn_x). Outputs: x0 [C] device int32, the
 * committed block; *steps (host) the steps run; *P_out (host) = P + C. Returns after the
 * commit is enqueued (dg_sync waits for it). A flag not written within 60 s of waiting
 * ends the call with DG_ERR_HIP after a stream synchronization. */
typedef struct {
  const dg_bf16 *E, *Wq, *Wk, *Wv, *Wo, *W1, *W2;
} dg_weights;
typedef struct {
  int32_t N;                 /* step cap, >= 1 */
  float b, thr;              /* acceptance budget and stop threshold (nats) */
  float tau0, tau1;          /* temperature schedule endpoints */
  uint64_t seed;             /* Philox key of the canvas draws */
  uint32_t canvas;           /* canvas index (the Philox key's second word) */
  int32_t commit;            /* DG_COMMIT_PROJECTION or DG_COMMIT_PREFILL */
  int32_t rule;              /* DG_RULE_ENTROPY or DG_RULE_CONFIDENCE */
  int32_t draw;              /* DG_DRAW_ARGMAX or DG_DRAW_SAMPLE */
} dg_loop_params;
enum { DG_COMMIT_PROJECTION = 0, DG_COMMIT_PREFILL = 1 };
enum { DG_RULE_ENTROPY = 0, DG_RULE_CONFIDENCE = 1 };
enum { DG_DRAW_ARGMAX = 0, DG_DRAW_SAMPLE = 1 };
typedef const dg_bf16 *(*dg_hidden_fn)(void *user, int32_t step);
size_t dg_loop_workspace_bytes(const dg_dims *dims);
dg_status dg_run_canvas(dg_ctx ctx, const dg_dims *dims, const dg_weights *w, dg_bf16 *Kp,
                        dg_bf16 *Vt, int64_t P, int64_t Pcap, const dg_loop_params *prm,
                        dg_hidden_fn hidden, void *user, void *ws, void *loop_ws, int32_t *x0,
                        int32_t *steps, int64_t *P_out);

/* Measured ceilings for the rooflines (measurement utilities, not steps of the method).
 * dg_peak_stream_read reads bytes (a positive multiple of 16) of the device buffer buf
 * (16-byte aligned) once with 16-byte streaming loads over DG_PEAK_STREAM_BLOCKS
 * workgroups, each writing the XOR of the words it read to sink[block] (device uint32,
 * DG_PEAK_STREAM_BLOCKS entries): the achievable HBM read rate when buf is larger than
 * the last-level cache.
 * dg_peak_mfma_bf16 runs DG_PEAK_MFMA_BLOCKS x 4 waves, each issuing iters rounds of four
 * independent v_mfma_f32_32x32x16_bf16 on register operands (bf16 1.0 everywhere), i.e.
 * DG_PEAK_MFMA_BLOCKS * 4 * iters * 4 * 32768 FLOP; lane 0 of wave w writes its
 * accumulator sum, exactly 1024 * iters, to sink[w] (device float, DG_PEAK_MFMA_BLOCKS * 4
 * entries). 1 <= iters <= 16384 (DG_ERR_RANGE otherwise). Both are enqueued on the
 * context's stream; the caller times them. */
#define DG_PEAK_STREAM_BLOCKS 2048
#define DG_PEAK_MFMA_BLOCKS 1024
dg_status dg_peak_stream_read(dg_ctx ctx, const void *buf, size_t bytes, uint32_t *sink);
dg_status dg_peak_mfma_bf16(dg_ctx ctx, int32_t iters, float *sink);

#ifdef __cplusplus
}
#endif
#endif /* DG_H */
