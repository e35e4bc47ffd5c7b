// C ABI of the canvas-denoise library (declarations and contracts in include/dg.h).
//
// Host-side responsibilities: validate every argument before anything is enqueued,
// carve the caller's workspace, and launch the kernels of each call in order on the
// context's stream. No call allocates device memory (the context's 4-byte status word
// and its pinned stop flags are allocated once in dg_create) and no call waits for the
// device except dg_sync and dg_run_canvas (which polls its steps' stop flags).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <chrono>
#include <climits>
#include <mutex>
#include <new>
#include <thread>

#include "../../include/dg.h"
#include "dg_common.h"

// Scratch of dg_canvas_attn_static: one copy per device, alive until the process ends.
// In host code `scratch` only names the symbol; its device address comes from
// hipGetSymbolAddress, looked up once per device by scratch_setup() and used everywhere
// the host hands this memory to a kernel.
static __device__ __align__(256) uint8_t scratch[DG_STATIC_SCRATCH_BYTES];

struct dg_ctx_s {
  int device = 0;
  hipStream_t stream = nullptr;
  int *d_status = nullptr;
  char err[512] = {0};
  // Rotary base for dg_canvas_attn and dg_prefill_block (0: no rotary positions).
  double rope_base = 0.0;
  // p0 hand-off between dg_logits_entropy and dg_selfcond.
  const void *p0_ws = nullptr;
  dg_dims p0_dims = {0, 0, 0, 0, 0, 0, 0};
  bool p0_valid = false;
  // Second stream (default priority) and fork/join events of dg_moe_ffn, made by
  // dg_create: the shared expert runs beside the routed experts.
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  // Stop flags of dg_run_canvas's steps, pinned host memory, four taken in enqueue order
  // across calls: when a step is enqueued at most two older ones are pending (including
  // the discarded step a stopped canvas leaves behind), so no slot is refilled while an
  // older stop kernel may still write it.
  int32_t *host_flags = nullptr;
  unsigned flag_seq = 0;
  // Device address of this device's static scratch (NULL if the lookup failed).
  void *scratch = nullptr;
  hipError_t scratch_err = hipSuccess;
};

namespace {

dg_status fail(dg_ctx ctx, dg_status st, const char *fmt, ...) {
  if (ctx) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(ctx->err, sizeof ctx->err, fmt, ap);
    va_end(ap);
  }
  return st;
}

dg_status hip_fail(dg_ctx ctx, hipError_t e, const char *where) {
  return fail(ctx, DG_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Null check, then the context's device is made current for what follows (the null
// stream, launch attributes and CU counts are per device).
#define DG_ENTER()                                                                \
  do {                                                                            \
    if (!ctx) return DG_ERR_NULL;                                                 \
    const hipError_t e_dev = hipSetDevice(ctx->device);                           \
    if (e_dev != hipSuccess) return hip_fail(ctx, e_dev, __func__);               \
  } while (0)

#define DG_REQUIRE_PTR(p)                                                         \
  do {                                                                            \
    if (!(p)) return fail(ctx, DG_ERR_NULL, "%s: %s is NULL", __func__, #p);      \
    if (!aligned16(p)) return fail(ctx, DG_ERR_ALIGN, "%s: %s is not 16-byte aligned", __func__, #p); \
  } while (0)

dg_status check_dims(dg_ctx ctx, const dg_dims *m, const char *fn) {
  if (!m) return fail(ctx, DG_ERR_NULL, "%s: dims is NULL", fn);
  if (m->V < 1) return fail(ctx, DG_ERR_SHAPE, "%s: V=%d must be >= 1", fn, m->V);
  if (m->d < 32 || m->d % 32 || m->d > 16384)
    return fail(ctx, DG_ERR_SHAPE, "%s: d=%d must be a multiple of 32 in [32, 16384]", fn, m->d);
  if (m->C < 1 || m->C > 1024) return fail(ctx, DG_ERR_SHAPE, "%s: C=%d must be in [1, 1024]", fn, m->C);
  if (m->Hq < 1 || m->Hkv < 1 || m->Hq % m->Hkv)
    return fail(ctx, DG_ERR_SHAPE, "%s: Hq=%d must be a positive multiple of Hkv=%d", fn, m->Hq, m->Hkv);
  if (m->hd != 16 && m->hd != 32 && m->hd != 64 && m->hd != 128)
    return fail(ctx, DG_ERR_SHAPE, "%s: hd=%d must be 16, 32, 64 or 128", fn, m->hd);
  if ((m->Hq * m->hd) % 32 || (m->Hkv * m->hd) % 8)
    return fail(ctx, DG_ERR_SHAPE, "%s: Hq*hd=%d must be a multiple of 32", fn, m->Hq * m->hd);
  if ((int64_t)m->V * m->d >= ((int64_t)1 << 31))
    return fail(ctx, DG_ERR_SHAPE, "%s: V*d=%lld must be < 2^31", fn, (long long)m->V * m->d);
  if (m->F < 32 || m->F % 32 || m->F > 16384)
    return fail(ctx, DG_ERR_SHAPE, "%s: F=%d must be a multiple of 32 in [32, 16384]", fn, m->F);
  return DG_OK;
}

dg_status check_cache(dg_ctx ctx, int64_t P, int64_t Pcap, const char *fn) {
  if (P < 0 || Pcap < 0 || P > Pcap)
    return fail(ctx, DG_ERR_RANGE, "%s: need 0 <= P=%lld <= Pcap=%lld", fn, (long long)P, (long long)Pcap);
  if (Pcap % 8) return fail(ctx, DG_ERR_ALIGN, "%s: Pcap=%lld must be a multiple of 8", fn, (long long)Pcap);
  if (Pcap > (int64_t)1 << 30) return fail(ctx, DG_ERR_SHAPE, "%s: Pcap=%lld too large", fn, (long long)Pcap);
  return DG_OK;
}

template <typename T>
T *ws_at(void *ws, size_t off) {
  return (T *)((char *)ws + off);
}

// Per-device address of the static scratch, looked up once per device (the device must
// be current) and kept for the life of the process, like the array itself.
std::mutex g_scratch_mu;
bool g_scratch_done[DG_MAX_DEVICES];
void *g_scratch_ptr[DG_MAX_DEVICES];
hipError_t g_scratch_err[DG_MAX_DEVICES];

hipError_t scratch_setup(int device, void **out) {
  *out = nullptr;
  if (device < 0 || device >= DG_MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_done[device]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_err[device] = e;
    g_scratch_ptr[device] = e == hipSuccess ? p : nullptr;
    g_scratch_done[device] = true;
  }
  *out = g_scratch_ptr[device];
  return g_scratch_err[device];
}

// Workspace regions canvas attention writes: the denoiser input, Q / canvas K, V, the
// attention output before Wo and the split partials.
struct AttnRegions {
  int Cpad;
  u16 *x, *q, *kc, *vct, *o;
  u16 *po;
  float *pml;
};

// Validation shared by dg_canvas_attn and dg_canvas_attn_static (fn names the caller).
dg_status check_canvas_attn(dg_ctx ctx, const char *fn, const dg_dims *dims, const int32_t *tokens,
                            const dg_bf16 *z, const dg_bf16 *E, const dg_bf16 *Wq, const dg_bf16 *Wk,
                            const dg_bf16 *Wv, const dg_bf16 *Wo, const dg_bf16 *Kp, const dg_bf16 *Vt,
                            int64_t P, int64_t Pcap, const dg_bf16 *A) {
  dg_status st = check_dims(ctx, dims, fn);
  if (st) return st;
  if ((st = check_cache(ctx, P, Pcap, fn))) return st;
  // the attention copies address one head's cache array with 32-bit byte offsets
  if ((int64_t)dims->Hkv * dims->hd * Pcap * 2 > (int64_t)UINT32_MAX)
    return fail(ctx, DG_ERR_SHAPE, "%s: Hkv*hd*Pcap*2 = %lld bytes exceeds 4 GiB", fn,
                (long long)dims->Hkv * dims->hd * Pcap * 2);
  const struct {
    const void *p;
    const char *name;
  } req[] = {{tokens, "tokens"}, {E, "E"}, {Wq, "Wq"}, {Wk, "Wk"}, {Wv, "Wv"}, {Wo, "Wo"}, {A, "A"},
             {P > 0 ? Kp : (const void *)A, "Kp"}, {P > 0 ? Vt : (const void *)A, "Vt"}};
  for (const auto &r : req) {
    if (!r.p) return fail(ctx, DG_ERR_NULL, "%s: %s is NULL", fn, r.name);
    if (!aligned16(r.p)) return fail(ctx, DG_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, r.name);
  }
  if (z && !aligned16(z)) return fail(ctx, DG_ERR_ALIGN, "%s: z is not 16-byte aligned", fn);
  return DG_OK;
}

// Enqueues canvas attention (gather, QKV, rotary positions, split attention and merge,
// Wo) over the given workspace regions. Arguments already validated.
dg_status enqueue_canvas_attn(dg_ctx ctx, const char *fn, const dg_dims &m, const int32_t *tokens,
                              const dg_bf16 *z, const dg_bf16 *E, const dg_bf16 *Wq, const dg_bf16 *Wk,
                              const dg_bf16 *Wv, const dg_bf16 *Wo, const dg_bf16 *Kp,
                              const dg_bf16 *Vt, int64_t P, int64_t Pcap, const AttnRegions &r,
                              dg_bf16 *A, const dg_bf16 *X = nullptr) {
  const int qd = m.Hq * m.hd, kd = m.Hkv * m.hd;

  // Q, K, V of the denoiser input X = bf16(E[tokens] + z) (or the caller's X).
  GemmArgs g{};
  g.M = m.C;
  g.K = m.d;
  g.V = m.V;
  g.status = ctx->d_status;
  if (X) {
    g.A = X;
  } else if (z) {
    hipError_t e = dg_launch_xgather(tokens, E, z, m.V, m.C, m.d, r.x, ctx->d_status, ctx->stream);
    if (e != hipSuccess) return hip_fail(ctx, e, fn);
    g.A = r.x;
  } else {
    g.tokens = tokens;
    g.E = E;
  }
  g.nseg = 3;
  g.seg[0] = GemmSeg{Wq, qd, r.q, qd, 0, 1, INT_MAX, m.C, 0};
  g.seg[1] = GemmSeg{Wk, kd, r.kc, kd, 0, 1, INT_MAX, r.Cpad, 0};
  g.seg[2] = GemmSeg{Wv, kd, r.vct, 1, 0, r.Cpad, INT_MAX, r.Cpad, 0};
  hipError_t e = dg_launch_gemm(g, ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, fn);
  if (ctx->rope_base > 0.0) {                        // canvas token i sits at position P + i
    e = dg_launch_rope_store(r.q, r.kc, nullptr, m.C, r.Cpad, m.Hq, m.Hkv, m.hd, P, ctx->rope_base, nullptr,
                             nullptr, 0, 0, ctx->stream);
    if (e != hipSuccess) return hip_fail(ctx, e, fn);
  }

  AttnArgs at{};
  at.Q = r.q;
  at.Kp = Kp;
  at.Vt = Vt;
  at.Kc = r.kc;
  at.Vct = r.vct;
  at.P = P;
  at.Pcap = Pcap;
  at.C = m.C;
  at.Cpad = r.Cpad;
  at.Hq = m.Hq;
  at.Hkv = m.Hkv;
  at.hd = m.hd;
  at.nsplit = dg_attn_nsplit(m.Hkv, m.Hq, m.C, P);
  at.scale_log2 = (float)(1.4426950408889634 / sqrt((double)m.hd));
  at.po = r.po;
  at.pml = r.pml;
  at.O = r.o;
  e = dg_launch_attention(at, ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, fn);

  GemmArgs go{};
  go.M = m.C;
  go.K = qd;
  go.A = r.o;
  go.nseg = 1;
  go.seg[0] = GemmSeg{Wo, m.d, A, m.d, 0, 1, INT_MAX, m.C, 0};
  e = dg_launch_gemm(go, ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, fn);
  return DG_OK;
}

}  // namespace

extern "C" {

dg_status dg_create(dg_ctx *out, int device, void *hip_stream) {
  if (!out) return DG_ERR_NULL;
  *out = nullptr;
  dg_ctx ctx = new (std::nothrow) dg_ctx_s;
  if (!ctx) return DG_ERR_UNSUPPORTED;
  ctx->device = device;
  ctx->stream = (hipStream_t)hip_stream;
  hipError_t e = hipSetDevice(device);
  if (e == hipSuccess) e = hipMalloc((void **)&ctx->d_status, sizeof(int));
  if (e == hipSuccess) e = hipMemset(ctx->d_status, 0, sizeof(int));
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&ctx->side, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&ctx->ev_fork, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&ctx->ev_join, hipEventDisableTiming);
  if (e == hipSuccess) e = hipHostMalloc((void **)&ctx->host_flags, 4 * sizeof(int32_t), hipHostMallocDefault);
  if (e != hipSuccess) {
    if (ctx->d_status) (void)hipFree(ctx->d_status);
    if (ctx->side) (void)hipStreamDestroy(ctx->side);
    if (ctx->ev_fork) (void)hipEventDestroy(ctx->ev_fork);
    if (ctx->ev_join) (void)hipEventDestroy(ctx->ev_join);
    delete ctx;
    return DG_ERR_HIP;
  }
  // the device is current: its static scratch address (dg_canvas_attn_static reports a
  // failed lookup; every other call works without it)
  ctx->scratch_err = scratch_setup(device, &ctx->scratch);
  *out = ctx;
  return DG_OK;
}

void dg_destroy(dg_ctx ctx) {
  if (!ctx) return;
  if (ctx->d_status) {
    (void)hipSetDevice(ctx->device);
    (void)hipStreamSynchronize(ctx->stream);
    (void)hipFree(ctx->d_status);
  }
  if (ctx->side) {
    (void)hipStreamSynchronize(ctx->side);
    (void)hipStreamDestroy(ctx->side);
  }
  if (ctx->ev_fork) (void)hipEventDestroy(ctx->ev_fork);
  if (ctx->ev_join) (void)hipEventDestroy(ctx->ev_join);
  if (ctx->host_flags) (void)hipHostFree(ctx->host_flags);
  delete ctx;
}

dg_status dg_set_stream(dg_ctx ctx, void *hip_stream) {
  if (!ctx) return DG_ERR_NULL;
  ctx->stream = (hipStream_t)hip_stream;
  return DG_OK;
}

const char *dg_last_error(dg_ctx ctx) { return ctx ? ctx->err : "NULL context"; }

dg_status dg_sync(dg_ctx ctx) {
  DG_ENTER();
  hipError_t e = hipStreamSynchronize(ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "dg_sync");
  int st = 0;
  e = hipMemcpy(&st, ctx->d_status, sizeof(int), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(ctx, e, "dg_sync");
  if (st == DGS_NONFINITE) return fail(ctx, DG_ERR_NONFINITE, "device saw non-finite logits");
  if (st == DGS_RANGE) return fail(ctx, DG_ERR_RANGE, "device saw a token id outside [0, V)");
  if (st) return fail(ctx, DG_ERR_UNSUPPORTED, "device status %d", st);
  return DG_OK;
}

dg_status dg_clear_status(dg_ctx ctx) {
  DG_ENTER();
  hipError_t e = hipMemsetAsync(ctx->d_status, 0, sizeof(int), ctx->stream);
  return e == hipSuccess ? DG_OK : hip_fail(ctx, e, "dg_clear_status");
}

size_t dg_workspace_bytes(const dg_dims *m, int64_t Pcap) {
  if (!m || check_dims(nullptr, m, "dg_workspace_bytes") != DG_OK || Pcap < 0) return 0;
  return dg_ws_layout(m->V, m->d, m->C, m->Hq, m->Hkv, m->hd, m->F, Pcap).total;
}

float dg_temperature(int32_t k, int32_t N, float tau0, float tau1) {
  if (N <= 1) return tau0;
  return (float)((double)tau0 + ((double)tau1 - (double)tau0) * (double)k / (double)(N - 1));
}

dg_status dg_canvas_attn(dg_ctx ctx, const dg_dims *dims, const int32_t *tokens,
                         const dg_bf16 *z, const dg_bf16 *E, const dg_bf16 *Wq,
                         const dg_bf16 *Wk, const dg_bf16 *Wv, const dg_bf16 *Wo,
                         const dg_bf16 *Kp, const dg_bf16 *Vt, int64_t P, int64_t Pcap,
                         void *ws, dg_bf16 *A) {
  DG_ENTER();
  dg_status st = check_canvas_attn(ctx, __func__, dims, tokens, z, E, Wq, Wk, Wv, Wo, Kp, Vt, P, Pcap, A);
  if (st) return st;
  DG_REQUIRE_PTR(ws);
  const dg_dims &m = *dims;
  const DgWs w = dg_ws_layout(m.V, m.d, m.C, m.Hq, m.Hkv, m.hd, m.F, Pcap);
  const AttnRegions r{w.Cpad, ws_at<u16>(ws, w.x), ws_at<u16>(ws, w.q), ws_at<u16>(ws, w.kc),
                      ws_at<u16>(ws, w.vct), ws_at<u16>(ws, w.o), ws_at<u16>(ws, w.po),
                      ws_at<float>(ws, w.pml)};
  return enqueue_canvas_attn(ctx, __func__, m, tokens, z, E, Wq, Wk, Wv, Wo, Kp, Vt, P, Pcap, r, A);
}

dg_status dg_canvas_attn_x(dg_ctx ctx, const dg_dims *dims, const dg_bf16 *X, const dg_bf16 *Wq,
                           const dg_bf16 *Wk, const dg_bf16 *Wv, const dg_bf16 *Wo, const dg_bf16 *Kp,
                           const dg_bf16 *Vt, int64_t P, int64_t Pcap, void *ws, dg_bf16 *A) {
  DG_ENTER();
  if (!X) return fail(ctx, DG_ERR_NULL, "%s: X is NULL", __func__);
  if (!aligned16(X)) return fail(ctx, DG_ERR_ALIGN, "%s: X is not 16-byte aligned", __func__);
  // the shared checks, X standing in for the token ids and E (neither is read here)
  dg_status st = check_canvas_attn(ctx, __func__, dims, (const int32_t *)X, nullptr, X, Wq, Wk, Wv, Wo, Kp, Vt, P,
                                   Pcap, A);
  if (st) return st;
  DG_REQUIRE_PTR(ws);
  const dg_dims &m = *dims;
  const DgWs w = dg_ws_layout(m.V, m.d, m.C, m.Hq, m.Hkv, m.hd, m.F, Pcap);
  const AttnRegions r{w.Cpad, ws_at<u16>(ws, w.x), ws_at<u16>(ws, w.q), ws_at<u16>(ws, w.kc),
                      ws_at<u16>(ws, w.vct), ws_at<u16>(ws, w.o), ws_at<u16>(ws, w.po),
                      ws_at<float>(ws, w.pml)};
  return enqueue_canvas_attn(ctx, __func__, m, nullptr, nullptr, nullptr, Wq, Wk, Wv, Wo, Kp, Vt, P, Pcap, r, A, X);
}

dg_status dg_canvas_attn_static(dg_ctx ctx, const dg_dims *dims, const int32_t *tokens,
                                const dg_bf16 *z, const dg_bf16 *E, const dg_bf16 *Wq,
                                const dg_bf16 *Wk, const dg_bf16 *Wv, const dg_bf16 *Wo,
                                const dg_bf16 *Kp, const dg_bf16 *Vt, int64_t P, int64_t Pcap,
                                dg_bf16 *A) {
  DG_ENTER();
  dg_status st = check_canvas_attn(ctx, __func__, dims, tokens, z, E, Wq, Wk, Wv, Wo, Kp, Vt, P, Pcap, A);
  if (st) return st;
  if (!ctx->scratch)
    return fail(ctx, DG_ERR_HIP, "%s: no static scratch on device %d (%s)", __func__, ctx->device,
                hipGetErrorString(ctx->scratch_err == hipSuccess ? hipErrorInvalidSymbol : ctx->scratch_err));
  const dg_dims &m = *dims;
  const DgAttnWs w = dg_attn_ws_layout(m.d, m.C, m.Hq, m.Hkv, m.hd, dg_attn_nsplit(m.Hkv, m.Hq, m.C, P));
  if (w.total > DG_STATIC_SCRATCH_BYTES)
    return fail(ctx, DG_ERR_CAPACITY, "%s: these dims need %zu bytes of scratch; the static scratch holds %zu",
                __func__, w.total, (size_t)DG_STATIC_SCRATCH_BYTES);
  void *ws = ctx->scratch;
  const AttnRegions r{w.Cpad, ws_at<u16>(ws, w.x), ws_at<u16>(ws, w.q), ws_at<u16>(ws, w.kc),
                      ws_at<u16>(ws, w.vct), ws_at<u16>(ws, w.o), ws_at<u16>(ws, w.po),
                      ws_at<float>(ws, w.pml)};
  return enqueue_canvas_attn(ctx, __func__, m, tokens, z, E, Wq, Wk, Wv, Wo, Kp, Vt, P, Pcap, r, A);
}

static dg_status check_moe(dg_ctx ctx, const dg_moe_dims *m, int32_t C, const char *fn) {
  if (!m) return fail(ctx, DG_ERR_NULL, "%s: moe dims is NULL", fn);
  if (C < 1 || C > 1024) return fail(ctx, DG_ERR_SHAPE, "%s: need 1 <= C <= 1024", fn);
  // the GEMMs take K in whole 16-deep MFMA steps, and every width is also an N or a K
  if (m->d < 32 || m->d % 32 || m->Fe < 32 || m->Fe % 32 || m->Fs < 32 || m->Fs % 32)
    return fail(ctx, DG_ERR_SHAPE, "%s: d, Fe, Fs must be positive multiples of 32", fn);
  if (m->E < 1 || m->E > 256 || m->K < 1 || m->K > m->E || m->K > 32 || (int64_t)C * m->K > 8192)
    return fail(ctx, DG_ERR_SHAPE, "%s: need 1 <= K <= min(E, 32), E <= 256, C * K <= 8192", fn);
  return DG_OK;
}

size_t dg_moe_workspace_bytes(const dg_moe_dims *m, int32_t C) {
  if (!m || check_moe(nullptr, m, C, "dg_moe_workspace_bytes") != DG_OK) return 0;
  return dg_moe_ws_layout(C, m->d, m->E, m->K, m->Fe, m->Fs).total;
}

dg_status dg_moe_ffn(dg_ctx ctx, const dg_moe_dims *m, int32_t C, const dg_bf16 *X,
                     const dg_bf16 *Wr, const dg_bf16 *W1, const dg_bf16 *W2, const dg_bf16 *W1s,
                     const dg_bf16 *W2s, void *ws, dg_bf16 *Y, int32_t *n_active) {
  DG_ENTER();
  dg_status st = check_moe(ctx, m, C, __func__);
  if (st) return st;
  DG_REQUIRE_PTR(X);
  DG_REQUIRE_PTR(Wr);
  DG_REQUIRE_PTR(W1);
  DG_REQUIRE_PTR(W2);
  DG_REQUIRE_PTR(W1s);
  DG_REQUIRE_PTR(W2s);
  DG_REQUIRE_PTR(ws);
  DG_REQUIRE_PTR(Y);
  const DgMoeWs w = dg_moe_ws_layout(C, m->d, m->E, m->K, m->Fe, m->Fs);
  float *logits = ws_at<float>(ws, w.logits), *gate = ws_at<float>(ws, w.gate);
  int *sel = ws_at<int>(ws, w.sel), *off = ws_at<int>(ws, w.off);
  int *perm = ws_at<int>(ws, w.perm), *pos = ws_at<int>(ws, w.pos), *tiles = ws_at<int>(ws, w.tiles);
  u16 *h = ws_at<u16>(ws, w.h), *yg = ws_at<u16>(ws, w.yg), *hs = ws_at<u16>(ws, w.hs);
  u16 *ys = ws_at<u16>(ws, w.ys);

  hipError_t e = hipSuccess;

  // shared expert on the side stream: it needs only X, and overlaps the routing and the
  // routed experts; the combine waits for it
  GemmArgs s1{};
  s1.M = C;
  s1.K = m->d;
  s1.A = X;
  s1.gelu = 1;
  s1.nseg = 1;
  s1.seg[0] = GemmSeg{W1s, m->Fs, hs, m->Fs, 0, 1, INT_MAX, C, 0};
  GemmArgs s2{};
  s2.M = C;
  s2.K = m->Fs;
  s2.A = hs;
  s2.nseg = 1;
  s2.seg[0] = GemmSeg{W2s, m->d, ys, m->d, 0, 1, INT_MAX, C, 0};
  e = hipEventRecord(ctx->ev_fork, ctx->stream);
  if (e == hipSuccess) e = hipStreamWaitEvent(ctx->side, ctx->ev_fork, 0);
  if (e == hipSuccess) e = dg_launch_gemm(s1, ctx->side);
  if (e == hipSuccess) e = dg_launch_gemm(s2, ctx->side);
  if (e == hipSuccess) e = hipEventRecord(ctx->ev_join, ctx->side);
  if (e != hipSuccess) return hip_fail(ctx, e, "dg_moe_ffn(shared)");

  // router logits in float32 (the routing decision is taken on them)
  GemmArgs gr{};
  gr.M = C;
  gr.K = m->d;
  gr.A = X;
  gr.nseg = 1;
  gr.seg[0] = GemmSeg{Wr, m->E, nullptr, m->E, 0, 1, INT_MAX, C, 0};
  gr.out32 = logits;
  gr.ld32 = m->E;
  const int rsplit = dg_moe_router_splits(m->d);
  gr.ksplit = rsplit;
  gr.split_stride = (int64_t)C * m->E;
  e = dg_launch_gemm(gr, ctx->stream);
  if (e == hipSuccess) e = dg_launch_moe_route(logits, rsplit, C, m->E, m->K, sel, gate, ctx->stream);
  if (e == hipSuccess) e = dg_launch_moe_group(sel, C, m->K, m->E, off, perm, pos, n_active, tiles, ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "dg_moe_ffn(route)");

  // routed experts over the tile list: hidden = GELU(X W1_e^T), out = hidden W2_e^T
  const int max_tiles = dg_moe_max_tiles(C, m->E, m->K);
  const MoeGemmArgs g1{X, W1, off, perm, tiles, h, m->Fe, m->d, m->Fe, 1, max_tiles};
  e = dg_launch_moe_expert(g1, ctx->stream);
  const MoeGemmArgs g2{h, W2, off, nullptr, tiles, yg, m->d, m->Fe, m->d, 0, max_tiles};
  if (e == hipSuccess) e = dg_launch_moe_expert(g2, ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "dg_moe_ffn(experts)");

  e = hipStreamWaitEvent(ctx->stream, ctx->ev_join, 0);
  if (e == hipSuccess) e = dg_launch_moe_combine(yg, ys, gate, pos, C, m->K, m->d, Y, ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "dg_moe_ffn(shared, combine)");
  return DG_OK;
}

dg_status dg_set_rope(dg_ctx ctx, float base) {
  if (!ctx) return DG_ERR_NULL;
  if (!(base >= 0.f) || !isfinite(base)) return fail(ctx, DG_ERR_RANGE, "%s: base=%g must be >= 0", __func__, base);
  ctx->rope_base = (double)base;
  return DG_OK;
}

dg_status dg_prefill_block(dg_ctx ctx, const dg_dims *dims, const int32_t *tokens,
                           const dg_bf16 *E, const dg_bf16 *Wq, const dg_bf16 *Wk,
                           const dg_bf16 *Wv, const dg_bf16 *Wo, dg_bf16 *Kp, dg_bf16 *Vt,
                           int64_t P, int64_t Pcap, void *ws, dg_bf16 *A, int64_t *P_out) {
  DG_ENTER();
  dg_status st = check_dims(ctx, dims, __func__);
  if (st) return st;
  if ((st = check_cache(ctx, P, Pcap, __func__))) return st;
  if ((int64_t)dims->Hkv * dims->hd * Pcap * 2 > (int64_t)UINT32_MAX)
    return fail(ctx, DG_ERR_SHAPE, "%s: Hkv*hd*Pcap*2 = %lld bytes exceeds 4 GiB", __func__,
                (long long)dims->Hkv * dims->hd * Pcap * 2);
  DG_REQUIRE_PTR(tokens);
  DG_REQUIRE_PTR(E);
  DG_REQUIRE_PTR(Wq);
  DG_REQUIRE_PTR(Wk);
  DG_REQUIRE_PTR(Wv);
  DG_REQUIRE_PTR(Wo);
  DG_REQUIRE_PTR(Kp);
  DG_REQUIRE_PTR(Vt);
  DG_REQUIRE_PTR(ws);
  DG_REQUIRE_PTR(A);
  DG_REQUIRE_PTR(P_out);
  const dg_dims &m = *dims;
  if (P + m.C > Pcap)
    return fail(ctx, DG_ERR_CAPACITY, "%s: P + C = %lld exceeds Pcap = %lld", __func__,
                (long long)(P + m.C), (long long)Pcap);
  const DgWs w = dg_ws_layout(m.V, m.d, m.C, m.Hq, m.Hkv, m.hd, m.F, Pcap);
  const int qd = m.Hq * m.hd, kd = m.Hkv * m.hd;
  u16 *q = ws_at<u16>(ws, w.q), *kc = ws_at<u16>(ws, w.kc), *vct = ws_at<u16>(ws, w.vct);
  u16 *o = ws_at<u16>(ws, w.o);

  // Q, K, V of the block X = E[tokens], rotated to positions P + i.
  GemmArgs g{};
  g.M = m.C;
  g.K = m.d;
  g.V = m.V;
  g.status = ctx->d_status;
  g.tokens = tokens;
  g.E = E;
  g.nseg = 3;
  g.seg[0] = GemmSeg{Wq, qd, q, qd, 0, 1, INT_MAX, m.C, 0};
  g.seg[1] = GemmSeg{Wk, kd, kc, kd, 0, 1, INT_MAX, w.Cpad, 0};
  g.seg[2] = GemmSeg{Wv, kd, vct, 1, 0, w.Cpad, INT_MAX, w.Cpad, 0};
  hipError_t e = dg_launch_gemm(g, ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "dg_prefill_block(qkv)");
  // Rotation of the block's queries and keys, and the block's rotated keys and its values
  // into the cache rows [P, P + C) (the attention below reads the cache only below P).
  e = dg_launch_rope_store(q, kc, vct, m.C, w.Cpad, m.Hq, m.Hkv, m.hd, P, ctx->rope_base, Kp, Vt, P, Pcap,
                           ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "dg_prefill_block(rope, store)");

  // Causal attention: the prefix [0, P) and block keys j <= i.
  AttnArgs at{};
  at.Q = q;
  at.Kp = Kp;
  at.Vt = Vt;
  at.Kc = kc;
  at.Vct = vct;
  at.P = P;
  at.Pcap = Pcap;
  at.C = m.C;
  at.Cpad = w.Cpad;
  at.Hq = m.Hq;
  at.Hkv = m.Hkv;
  at.hd = m.hd;
  at.nsplit = dg_attn_nsplit(m.Hkv, m.Hq, m.C, P);
  at.causal = 1;
  at.scale_log2 = (float)(1.4426950408889634 / sqrt((double)m.hd));
  at.po = ws_at<u16>(ws, w.po);
  at.pml = ws_at<float>(ws, w.pml);
  at.O = o;
  e = dg_launch_attention(at, ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "dg_prefill_block(attention)");

  GemmArgs go{};
  go.M = m.C;
  go.K = qd;
  go.A = o;
  go.nseg = 1;
  go.seg[0] = GemmSeg{Wo, m.d, A, m.d, 0, 1, INT_MAX, m.C, 0};
  e = dg_launch_gemm(go, ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "dg_prefill_block(wo)");

  *P_out = P + m.C;
  return DG_OK;
}

dg_status dg_logits_entropy(dg_ctx ctx, const dg_dims *dims, const dg_bf16 *H,
                            const dg_bf16 *E, float tau, void *ws, float *entropy,
                            int32_t *argmax) {
  DG_ENTER();
  dg_status st = check_dims(ctx, dims, __func__);
  if (st) return st;
  DG_REQUIRE_PTR(H);
  DG_REQUIRE_PTR(E);
  DG_REQUIRE_PTR(ws);
  DG_REQUIRE_PTR(entropy);
  DG_REQUIRE_PTR(argmax);
  if (!(tau > 0.f) || !isfinite(tau)) return fail(ctx, DG_ERR_RANGE, "%s: tau=%g must be > 0", __func__, tau);
  const dg_dims &m = *dims;
  const DgWs w = dg_ws_layout(m.V, m.d, m.C, m.Hq, m.Hkv, m.hd, m.F, 0);
  LogitsArgs a{};
  a.H = H;
  a.E = E;
  a.V = m.V;
  a.d = m.d;
  a.C = m.C;
  a.Cpad = w.Cpad;
  a.T = w.T;
  a.nsc = w.nsc;
  a.inv_tau = 1.0f / tau;
  a.ptilde = ws_at<u16>(ws, w.ptilde);
  a.tmax = ws_at<float>(ws, w.tmax);
  a.trho = ws_at<float>(ws, w.trho);
  a.tsum = ws_at<float>(ws, w.tsum);
  a.tent = ws_at<float>(ws, w.tent);
  a.targ = ws_at<int>(ws, w.targ);
  a.colR = ws_at<float>(ws, w.colR);
  a.colZ = ws_at<float>(ws, w.colZ);
  a.colP = ws_at<float>(ws, w.colP);
  a.entropy = entropy;
  a.argmax = argmax;
  a.status = ctx->d_status;
  hipError_t e = dg_launch_logits(a, ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "dg_logits_entropy");
  ctx->p0_ws = ws;
  ctx->p0_dims = m;
  ctx->p0_valid = true;
  return DG_OK;
}

dg_status dg_entropy_accept(dg_ctx ctx, int32_t B, int32_t C, const float *entropy, float b,
                            uint8_t *accept, int32_t *n_accept) {
  DG_ENTER();
  if (B < 1 || C < 1 || C > 1024) return fail(ctx, DG_ERR_SHAPE, "%s: need B >= 1, 1 <= C <= 1024", __func__);
  if (!entropy || !accept || !n_accept) return fail(ctx, DG_ERR_NULL, "%s: NULL buffer", __func__);
  if (!(b >= 0.f && b < 65536.f)) return fail(ctx, DG_ERR_RANGE, "%s: b=%g must be in [0, 65536)", __func__, b);
  const uint64_t budget = (uint64_t)floor((double)b * 4294967296.0);
  hipError_t e = dg_launch_accept(B, C, entropy, budget, accept, n_accept, ctx->stream);
  return e == hipSuccess ? DG_OK : hip_fail(ctx, e, "dg_entropy_accept");
}

dg_status dg_confidence(dg_ctx ctx, const dg_dims *dims, const void *ws, float *confidence) {
  DG_ENTER();
  dg_status st = check_dims(ctx, dims, __func__);
  if (st) return st;
  DG_REQUIRE_PTR(ws);
  DG_REQUIRE_PTR(confidence);
  const dg_dims &m = *dims;
  if (!ctx->p0_valid || ctx->p0_ws != ws || memcmp(&ctx->p0_dims, &m, sizeof m) != 0)
    return fail(ctx, DG_ERR_STATE, "%s: ws does not hold p0 of a dg_logits_entropy with these dims", __func__);
  const DgWs w = dg_ws_layout(m.V, m.d, m.C, m.Hq, m.Hkv, m.hd, m.F, 0);
  hipError_t e = dg_launch_confidence(m.C, ws_at<float>(const_cast<void *>(ws), w.colP), confidence,
                                      ctx->stream);
  return e == hipSuccess ? DG_OK : hip_fail(ctx, e, "dg_confidence");
}

dg_status dg_topk_accept(dg_ctx ctx, int32_t B, int32_t C, const float *score, int32_t k,
                         uint8_t *accept, int32_t *n_accept) {
  DG_ENTER();
  if (B < 1 || C < 1 || C > 1024) return fail(ctx, DG_ERR_SHAPE, "%s: need B >= 1, 1 <= C <= 1024", __func__);
  if (!score || !accept || !n_accept) return fail(ctx, DG_ERR_NULL, "%s: NULL buffer", __func__);
  if (k < 0) return fail(ctx, DG_ERR_RANGE, "%s: k=%d must be >= 0", __func__, (int)k);
  hipError_t e = dg_launch_topk(B, C, score, k > C ? C : k, accept, n_accept, ctx->stream);
  return e == hipSuccess ? DG_OK : hip_fail(ctx, e, "dg_topk_accept");
}

dg_status dg_sample(dg_ctx ctx, const dg_dims *dims, const void *ws, int32_t B, uint64_t seed,
                    uint32_t canvas_base, uint32_t step, int32_t *tokens) {
  DG_ENTER();
  dg_status st = check_dims(ctx, dims, __func__);
  if (st) return st;
  DG_REQUIRE_PTR(ws);
  DG_REQUIRE_PTR(tokens);
  const dg_dims &m = *dims;
  if (B < 1 || m.C % B != 0)
    return fail(ctx, DG_ERR_SHAPE, "%s: B=%d must divide C=%d", __func__, (int)B, (int)m.C);
  if (!ctx->p0_valid || ctx->p0_ws != ws || memcmp(&ctx->p0_dims, &m, sizeof m) != 0)
    return fail(ctx, DG_ERR_STATE, "%s: ws does not hold p0 of a dg_logits_entropy with these dims", __func__);
  const DgWs w = dg_ws_layout(m.V, m.d, m.C, m.Hq, m.Hkv, m.hd, m.F, 0);
  void *wsm = const_cast<void *>(ws);
  SampleArgs a{};
  a.ptilde = ws_at<u16>(wsm, w.ptilde);
  a.tsum = ws_at<float>(wsm, w.tsum);
  a.trho = ws_at<float>(wsm, w.trho);
  a.colR = ws_at<float>(wsm, w.colR);
  a.T = w.T;
  a.VS = w.Vpad / 16;
  a.V = m.V;
  a.B = B;
  a.Cs = m.C / B;
  a.seed = seed;
  a.canvas_base = canvas_base;
  a.step = step;
  a.tokens = tokens;
  hipError_t e = dg_launch_sample(a, ctx->stream);
  return e == hipSuccess ? DG_OK : hip_fail(ctx, e, "dg_sample");
}

int32_t dg_reveal_count(int32_t C, int32_t N, int32_t step) {
  if (C < 0 || N < 1 || step < 0) return -1;
  if (step >= N) step = N - 1;
  int64_t n = 0;
  for (int32_t t = 0; t <= step; ++t) n += (C - n + (N - t) - 1) / (N - t);
  return (int32_t)n;
}

dg_status dg_renoise(dg_ctx ctx, int32_t B, int32_t C, int32_t V, const int32_t *argmax,
                     const uint8_t *accept, uint64_t seed, uint32_t canvas_base, uint32_t step,
                     int32_t *tokens) {
  DG_ENTER();
  if (B < 1 || C < 1 || V < 1) return fail(ctx, DG_ERR_SHAPE, "%s: need B, C, V >= 1", __func__);
  if (!tokens) return fail(ctx, DG_ERR_NULL, "%s: tokens is NULL", __func__);
  if (accept && !argmax) return fail(ctx, DG_ERR_NULL, "%s: argmax is NULL", __func__);
  hipError_t e = dg_launch_renoise(B, C, V, argmax, accept, seed, canvas_base, step, tokens, ctx->stream);
  return e == hipSuccess ? DG_OK : hip_fail(ctx, e, "dg_renoise");
}

namespace {

// Self-conditioning after its arguments passed dg_selfcond's checks; with ars non-null the
// reduce launch also runs acceptance, renoise and the stop test (ars->tpp * ars->C <= 256).
dg_status selfcond_enqueue(dg_ctx ctx, const dg_dims &m, void *ws, const dg_bf16 *E, const dg_bf16 *W1,
                           const dg_bf16 *W2, dg_bf16 *z, const ArsArgs *ars, dg_bf16 *x_next = nullptr,
                           const int32_t *x_tokens = nullptr) {
  const DgWs w = dg_ws_layout(m.V, m.d, m.C, m.Hq, m.Hkv, m.hd, m.F, 0);
  SelfcondArgs a{};
  a.ptilde = ws_at<u16>(ws, w.ptilde);
  a.trho = ws_at<float>(ws, w.trho);
  a.colR = ws_at<float>(ws, w.colR);
  a.colZ = ws_at<float>(ws, w.colZ);
  a.rhoS = ws_at<float>(ws, w.rhoS);
  a.E = E;
  a.V = m.V;
  a.d = m.d;
  a.C = m.C;
  a.Cpad = w.Cpad;
  a.T = w.T;
  a.nsc = w.nsc;
  a.ps = ws_at<float>(ws, w.ps);
  a.s = ws_at<u16>(ws, w.s);
  hipError_t e = dg_launch_selfcond(a, ars, ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "dg_selfcond(p0 E)");

  u16 *gbuf = ws_at<u16>(ws, w.g);
  GemmArgs g1{};
  g1.M = m.C;
  g1.K = m.d;
  g1.A = a.s;
  g1.gelu = 1;
  g1.nseg = 1;
  g1.seg[0] = GemmSeg{W1, m.F, gbuf, m.F, 0, 1, INT_MAX, m.C, 0};
  e = dg_launch_gemm(g1, ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "dg_selfcond(W1)");
  GemmArgs g2{};
  g2.M = m.C;
  g2.K = m.F;
  g2.A = gbuf;
  g2.nseg = 1;
  g2.seg[0] = GemmSeg{W2, m.d, z, m.d, 0, 1, INT_MAX, m.C, 0};
  g2.status = ctx->d_status;
  const bool fused = x_next && dg_gemm_can_xsum(g2);
  if (fused) {                                       // X = bf16(E[x] + z) in the W2 epilogue
    g2.xsum = x_next;
    g2.xtok = x_tokens;
    g2.xE = E;
    g2.xV = m.V;
  }
  e = dg_launch_gemm(g2, ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "dg_selfcond(W2)");
  if (x_next && !fused) {
    e = dg_launch_xgather(x_tokens, E, z, m.V, m.C, m.d, x_next, ctx->d_status, ctx->stream);
    if (e != hipSuccess) return hip_fail(ctx, e, "dg_selfcond(next input)");
  }
  return DG_OK;
}

}  // namespace

dg_status dg_selfcond(dg_ctx ctx, const dg_dims *dims, void *ws, const dg_bf16 *E,
                      const dg_bf16 *W1, const dg_bf16 *W2, dg_bf16 *z) {
  DG_ENTER();
  dg_status st = check_dims(ctx, dims, __func__);
  if (st) return st;
  DG_REQUIRE_PTR(ws);
  DG_REQUIRE_PTR(E);
  DG_REQUIRE_PTR(W1);
  DG_REQUIRE_PTR(W2);
  DG_REQUIRE_PTR(z);
  const dg_dims &m = *dims;
  if (!ctx->p0_valid || ctx->p0_ws != ws || memcmp(&ctx->p0_dims, &m, sizeof m) != 0)
    return fail(ctx, DG_ERR_STATE, "%s: ws does not hold p0 of a dg_logits_entropy with these dims", __func__);
  return selfcond_enqueue(ctx, m, ws, E, W1, W2, z, nullptr);
}

dg_status dg_stop_test(dg_ctx ctx, int32_t B, int32_t C, const float *entropy,
                       const int32_t *argmax, const int32_t *prev_argmax, float thr, int32_t step,
                       int32_t N, int32_t *flag) {
  DG_ENTER();
  if (B < 1 || C < 1 || C > 1024) return fail(ctx, DG_ERR_SHAPE, "%s: need B >= 1, 1 <= C <= 1024", __func__);
  if (!entropy || !argmax || !flag) return fail(ctx, DG_ERR_NULL, "%s: NULL buffer", __func__);
  if (!(thr >= 0.f && thr < 65536.f)) return fail(ctx, DG_ERR_RANGE, "%s: thr=%g must be in [0, 65536)", __func__, thr);
  if (step < 0 || N < 1) return fail(ctx, DG_ERR_RANGE, "%s: need step >= 0, N >= 1", __func__);
  const uint64_t limit = (uint64_t)floor((double)thr * (double)C * 4294967296.0);
  hipError_t e = dg_launch_stop(B, C, entropy, argmax, prev_argmax, limit, step, N, flag, ctx->stream);
  return e == hipSuccess ? DG_OK : hip_fail(ctx, e, "dg_stop_test");
}

namespace {

// The checks of dg_accept_renoise_stop; fills r (tpp left 0) when they pass.
dg_status check_ars(dg_ctx ctx, int32_t B, int32_t C, int32_t V, const float *entropy, float b,
                    const int32_t *x0, const int32_t *argmax, const int32_t *prev_argmax, uint64_t seed,
                    uint32_t canvas_base, int32_t step, float thr, int32_t N, uint8_t *accept,
                    int32_t *n_accept, int32_t *tokens, int32_t *flag, const char *fn, ArsArgs &r) {
  if (B < 1 || C < 1 || C > 1024 || V < 1)
    return fail(ctx, DG_ERR_SHAPE, "%s: need B, V >= 1 and 1 <= C <= 1024", fn);
  if (!entropy || !x0 || !argmax || !accept || !n_accept || !tokens || !flag)
    return fail(ctx, DG_ERR_NULL, "%s: NULL buffer", fn);
  if (!(b >= 0.f && b < 65536.f)) return fail(ctx, DG_ERR_RANGE, "%s: b=%g must be in [0, 65536)", fn, b);
  if (!(thr >= 0.f && thr < 65536.f)) return fail(ctx, DG_ERR_RANGE, "%s: thr=%g must be in [0, 65536)", fn, thr);
  if (step < 0 || N < 1) return fail(ctx, DG_ERR_RANGE, "%s: need step >= 0, N >= 1", fn);
  r = ArsArgs{};
  r.B = B;
  r.C = C;
  r.V = V;
  r.step = step;
  r.N = N;
  r.ent = entropy;
  r.x0 = x0;
  r.am = argmax;
  r.prev = prev_argmax;
  r.budget = (uint64_t)floor((double)b * 4294967296.0);
  r.limit = (uint64_t)floor((double)thr * (double)C * 4294967296.0);
  r.seed = seed;
  r.canvas_base = canvas_base;
  r.acc = accept;
  r.nacc = n_accept;
  r.tok = tokens;
  r.flag = flag;
  return DG_OK;
}

}  // namespace

dg_status dg_accept_renoise_stop(dg_ctx ctx, int32_t B, int32_t C, int32_t V, const float *entropy,
                                 float b, const int32_t *x0, const int32_t *argmax,
                                 const int32_t *prev_argmax, uint64_t seed, uint32_t canvas_base,
                                 int32_t step, float thr, int32_t N, uint8_t *accept,
                                 int32_t *n_accept, int32_t *tokens, int32_t *flag) {
  DG_ENTER();
  ArsArgs r;
  dg_status st = check_ars(ctx, B, C, V, entropy, b, x0, argmax, prev_argmax, seed, canvas_base, step, thr, N,
                           accept, n_accept, tokens, flag, __func__, r);
  if (st) return st;
  hipError_t e = dg_launch_accept_renoise_stop(r, ctx->stream);
  return e == hipSuccess ? DG_OK : hip_fail(ctx, e, __func__);
}

dg_status dg_selfcond_accept(dg_ctx ctx, const dg_dims *dims, void *ws, const dg_bf16 *E,
                             const dg_bf16 *W1, const dg_bf16 *W2, dg_bf16 *z,
                             const dg_accept_args *acc) {
  DG_ENTER();
  dg_status st = check_dims(ctx, dims, __func__);
  if (st) return st;
  DG_REQUIRE_PTR(ws);
  DG_REQUIRE_PTR(E);
  DG_REQUIRE_PTR(W1);
  DG_REQUIRE_PTR(W2);
  DG_REQUIRE_PTR(z);
  DG_REQUIRE_PTR(acc);
  const dg_dims &m = *dims;
  if (!ctx->p0_valid || ctx->p0_ws != ws || memcmp(&ctx->p0_dims, &m, sizeof m) != 0)
    return fail(ctx, DG_ERR_STATE, "%s: ws does not hold p0 of a dg_logits_entropy with these dims", __func__);
  if (acc->B < 1 || m.C % acc->B != 0)
    return fail(ctx, DG_ERR_SHAPE, "%s: B=%d must divide C=%d", __func__, (int)acc->B, (int)m.C);
  ArsArgs r;
  if ((st = check_ars(ctx, acc->B, m.C / acc->B, m.V, acc->entropy, acc->b, acc->x0, acc->argmax,
                      acc->prev_argmax, acc->seed, acc->canvas_base, acc->step, acc->thr, acc->N, acc->accept,
                      acc->n_accept, acc->tokens, acc->flag, __func__, r)))
    return st;
  if (acc->x_next && !aligned16(acc->x_next))
    return fail(ctx, DG_ERR_ALIGN, "%s: x_next is not 16-byte aligned", __func__);
  if (r.C <= 256) {                                  // one reduce workgroup (256 threads) per canvas
    r.tpp = r.C <= 64 ? 4 : r.C <= 128 ? 2 : 1;
    return selfcond_enqueue(ctx, m, ws, E, W1, W2, z, &r, acc->x_next, acc->tokens);
  }
  hipError_t e = dg_launch_accept_renoise_stop(r, ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, __func__);
  return selfcond_enqueue(ctx, m, ws, E, W1, W2, z, nullptr, acc->x_next, acc->tokens);
}

dg_status dg_commit_kv(dg_ctx ctx, const dg_dims *dims, const int32_t *tokens, const dg_bf16 *E,
                       const dg_bf16 *Wk, const dg_bf16 *Wv, dg_bf16 *Kp, dg_bf16 *Vt, int64_t P,
                       int64_t Pcap, int64_t *P_out) {
  DG_ENTER();
  dg_status st = check_dims(ctx, dims, __func__);
  if (st) return st;
  if ((st = check_cache(ctx, P, Pcap, __func__))) return st;
  DG_REQUIRE_PTR(tokens);
  DG_REQUIRE_PTR(E);
  DG_REQUIRE_PTR(Wk);
  DG_REQUIRE_PTR(Wv);
  DG_REQUIRE_PTR(Kp);
  DG_REQUIRE_PTR(Vt);
  if (!P_out) return fail(ctx, DG_ERR_NULL, "%s: P_out is NULL", __func__);
  const dg_dims &m = *dims;
  if (P + m.C > Pcap)
    return fail(ctx, DG_ERR_CAPACITY, "%s: P=%lld + C=%d exceeds Pcap=%lld", __func__, (long long)P, m.C,
                (long long)Pcap);
  const int hd = m.hd, kd = m.Hkv * m.hd;
  GemmArgs g{};
  g.M = m.C;
  g.K = m.d;
  g.tokens = tokens;
  g.E = E;
  g.V = m.V;
  g.status = ctx->d_status;
  g.nseg = 2;
  // K rows: Kp[g][P + m][e] = base + m*hd + g*Pcap*hd + e, n = g*hd + e
  g.seg[0] = GemmSeg{Wk, kd, Kp + P * hd, hd, Pcap * hd, 1, hd, m.C, 0};
  // V columns: Vt[g][e][P + m] = base + (g*hd + e)*Pcap + m = base + n*Pcap + m
  g.seg[1] = GemmSeg{Wv, kd, Vt + P, 1, 0, Pcap, INT_MAX, m.C, 0};
  hipError_t e = dg_launch_gemm(g, ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, "dg_commit_kv");
  *P_out = P + m.C;
  return DG_OK;
}

}  // extern "C"

namespace {

// Device state of one canvas in dg_run_canvas's loop workspace, 256-byte aligned regions.
struct LoopWs {
  size_t tokens, z, A, entropy, am0, am1, accept, n_accept, smp0, smp1, conf, X, total;
};
LoopWs loop_ws_layout(const dg_dims &m) {
  LoopWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (size_t)dg_round_up((int64_t)bytes, 256);
    return o;
  };
  const size_t C = (size_t)m.C, cd = C * (size_t)m.d;
  w.tokens = take(4 * C);
  w.z = take(2 * cd);
  w.A = take(2 * cd);
  w.entropy = take(4 * C);
  w.am0 = take(4 * C);
  w.am1 = take(4 * C);
  w.accept = take(C);
  w.n_accept = take(4);
  w.smp0 = take(4 * C);                              // sampled tokens of even / odd steps
  w.smp1 = take(4 * C);
  w.conf = take(4 * C);                              // confidence scores (confidence rule)
  w.X = take(2 * cd);                                // the next step's attention input
  w.total = off;
  return w;
}

// Polls a pinned stop flag until the stop kernel's system-scope store lands (a value in
// {0, 1, 2}); after 60 s a stream synchronization settles it or the step is reported lost.
dg_status wait_flag(dg_ctx ctx, int slot, int k, int32_t *value) {
  volatile int32_t *f = ctx->host_flags + slot;
  const auto t0 = std::chrono::steady_clock::now();
  for (int spins = 0; *f < 0; ++spins) {
    if ((spins & 1023) == 1023) {
      if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(60)) {
        const hipError_t e = hipStreamSynchronize(ctx->stream);
        if (e != hipSuccess) return hip_fail(ctx, e, "dg_run_canvas");
        if (*f < 0) return fail(ctx, DG_ERR_HIP, "dg_run_canvas: the stop flag of step %d was never written", k);
        break;
      }
      std::this_thread::yield();
    }
  }
  *value = *f;
  return DG_OK;
}

}  // namespace

extern "C" {

size_t dg_loop_workspace_bytes(const dg_dims *m) {
  if (!m || check_dims(nullptr, m, "dg_loop_workspace_bytes") != DG_OK) return 0;
  return loop_ws_layout(*m).total;
}

dg_status dg_run_canvas(dg_ctx ctx, const dg_dims *dims, const dg_weights *w, dg_bf16 *Kp,
                        dg_bf16 *Vt, int64_t P, int64_t Pcap, const dg_loop_params *prm,
                        dg_hidden_fn hidden, void *user, void *ws, void *loop_ws, int32_t *x0,
                        int32_t *steps, int64_t *P_out) {
  DG_ENTER();
  // Everything a later call of the loop could refuse is checked here, so a refused call
  // enqueues nothing; only a NULL or misaligned H_k from the callback is found mid-loop.
  dg_status st = check_dims(ctx, dims, __func__);
  if (st) return st;
  if ((st = check_cache(ctx, P, Pcap, __func__))) return st;
  if (!w || !prm || !hidden || !steps || !P_out)
    return fail(ctx, DG_ERR_NULL, "%s: weights, params, hidden, steps and P_out must not be NULL", __func__);
  DG_REQUIRE_PTR(Kp);
  DG_REQUIRE_PTR(Vt);
  DG_REQUIRE_PTR(ws);
  DG_REQUIRE_PTR(loop_ws);
  DG_REQUIRE_PTR(x0);
  const dg_bf16 *E = w->E, *Wq = w->Wq, *Wk = w->Wk, *Wv = w->Wv, *Wo = w->Wo, *W1 = w->W1, *W2 = w->W2;
  DG_REQUIRE_PTR(E);
  DG_REQUIRE_PTR(Wq);
  DG_REQUIRE_PTR(Wk);
  DG_REQUIRE_PTR(Wv);
  DG_REQUIRE_PTR(Wo);
  DG_REQUIRE_PTR(W1);
  DG_REQUIRE_PTR(W2);
  const dg_dims &m = *dims;
  const int N = prm->N;
  if (N < 1) return fail(ctx, DG_ERR_RANGE, "%s: N=%d must be >= 1", __func__, N);
  if (!(prm->b >= 0.f && prm->b < 65536.f) || !(prm->thr >= 0.f && prm->thr < 65536.f))
    return fail(ctx, DG_ERR_RANGE, "%s: b=%g and thr=%g must be in [0, 65536)", __func__, prm->b, prm->thr);
  if ((prm->rule != DG_RULE_ENTROPY && prm->rule != DG_RULE_CONFIDENCE) ||
      (prm->draw != DG_DRAW_ARGMAX && prm->draw != DG_DRAW_SAMPLE))
    return fail(ctx, DG_ERR_RANGE, "%s: rule=%d or draw=%d unknown", __func__, (int)prm->rule, (int)prm->draw);
  if (prm->commit != DG_COMMIT_PROJECTION && prm->commit != DG_COMMIT_PREFILL)
    return fail(ctx, DG_ERR_RANGE, "%s: commit=%d is not DG_COMMIT_PROJECTION or DG_COMMIT_PREFILL", __func__,
                (int)prm->commit);
  if (!(prm->tau0 > 0.f) || !(prm->tau1 > 0.f) || !isfinite(prm->tau0) || !isfinite(prm->tau1))
    return fail(ctx, DG_ERR_RANGE, "%s: tau0=%g and tau1=%g must be finite and > 0", __func__, prm->tau0, prm->tau1);
  if (P + m.C > Pcap)
    return fail(ctx, DG_ERR_CAPACITY, "%s: P=%lld + C=%d exceeds Pcap=%lld", __func__, (long long)P, m.C,
                (long long)Pcap);

  const LoopWs L = loop_ws_layout(m);
  int32_t *tok = ws_at<int32_t>(loop_ws, L.tokens);
  dg_bf16 *z = ws_at<dg_bf16>(loop_ws, L.z), *A = ws_at<dg_bf16>(loop_ws, L.A);
  float *ent = ws_at<float>(loop_ws, L.entropy);
  int32_t *am[2] = {ws_at<int32_t>(loop_ws, L.am0), ws_at<int32_t>(loop_ws, L.am1)};
  uint8_t *acc = ws_at<uint8_t>(loop_ws, L.accept);
  int32_t *nacc = ws_at<int32_t>(loop_ws, L.n_accept);
  int32_t *smp[2] = {ws_at<int32_t>(loop_ws, L.smp0), ws_at<int32_t>(loop_ws, L.smp1)};
  float *conf = ws_at<float>(loop_ws, L.conf);
  dg_bf16 *X = ws_at<dg_bf16>(loop_ws, L.X);
  const bool sample = prm->draw == DG_DRAW_SAMPLE;
  const bool x_ready = prm->rule == DG_RULE_ENTROPY;   // each step forms the next one's input

  // a uniform random canvas (stream 1 of the canvas's draws)
  if ((st = dg_renoise(ctx, 1, m.C, m.V, nullptr, nullptr, prm->seed, prm->canvas, 0, tok))) return st;
  int slot[2] = {0, 0};
  auto step = [&](int k) -> dg_status {
    const dg_bf16 *H = hidden(user, k);
    if (!H) return fail(ctx, DG_ERR_NULL, "dg_run_canvas: hidden state of step %d is NULL", k);
    if (!aligned16(H)) return fail(ctx, DG_ERR_ALIGN, "dg_run_canvas: hidden state of step %d is not 16-byte aligned", k);
    int32_t *a = am[k & 1], *prev = k > 0 ? am[(k - 1) & 1] : nullptr;
    dg_status r = k > 0 && x_ready
                      ? dg_canvas_attn_x(ctx, dims, X, Wq, Wk, Wv, Wo, Kp, Vt, P, Pcap, ws, A)
                      : dg_canvas_attn(ctx, dims, tok, k > 0 ? z : nullptr, E, Wq, Wk, Wv, Wo, Kp, Vt, P, Pcap, ws, A);
    if (!r) r = dg_logits_entropy(ctx, dims, H, E, dg_temperature(k, N, prm->tau0, prm->tau1), ws, ent, a);
    int32_t *x0k = a;                                // what accepted positions keep
    if (!r && sample) {
      x0k = smp[k & 1];
      r = dg_sample(ctx, dims, ws, 1, prm->seed, prm->canvas, (uint32_t)k, x0k);
    }
    if (r) return r;
    const int sl = (int)(ctx->flag_seq++ % 4);
    slot[k & 1] = sl;
    ctx->host_flags[sl] = -1;
    if (prm->rule == DG_RULE_CONFIDENCE) {
      r = dg_confidence(ctx, dims, ws, conf);
      if (!r) r = dg_topk_accept(ctx, 1, m.C, conf, dg_reveal_count(m.C, N, k), acc, nacc);
      if (!r) r = dg_renoise(ctx, 1, m.C, m.V, x0k, acc, prm->seed, prm->canvas, (uint32_t)k, tok);
      if (!r) r = dg_stop_test(ctx, 1, m.C, ent, a, prev, prm->thr, k, N, ctx->host_flags + sl);
      if (!r) r = dg_selfcond(ctx, dims, ws, E, W1, W2, z);
      return r;
    }
    dg_accept_args aa{};
    aa.B = 1;
    aa.entropy = ent;
    aa.b = prm->b;
    aa.x0 = x0k;
    aa.argmax = a;
    aa.prev_argmax = prev;
    aa.seed = prm->seed;
    aa.canvas_base = prm->canvas;
    aa.step = k;
    aa.thr = prm->thr;
    aa.N = N;
    aa.accept = acc;
    aa.n_accept = nacc;
    aa.tokens = tok;
    aa.flag = ctx->host_flags + sl;
    aa.x_next = X;
    return dg_selfcond_accept(ctx, dims, ws, E, W1, W2, z, &aa);
  };

  if ((st = step(0))) return st;
  int k = 0;
  for (;;) {
    if (k + 1 < N && (st = step(k + 1))) return st;
    int32_t flag = 0;
    if ((st = wait_flag(ctx, slot[k & 1], k, &flag))) return st;
    if (flag != 0) break;                            // stop (1) or the cap (2): commit step k
    ++k;
  }
  const int32_t *fin = sample ? smp[k & 1] : am[k & 1];   // the block step k commits
  if (prm->commit == DG_COMMIT_PREFILL)
    st = dg_prefill_block(ctx, dims, fin, E, Wq, Wk, Wv, Wo, Kp, Vt, P, Pcap, ws, A, P_out);
  else
    st = dg_commit_kv(ctx, dims, fin, E, Wk, Wv, Kp, Vt, P, Pcap, P_out);
  if (st) return st;
  const hipError_t e = hipMemcpyAsync(x0, fin, (size_t)m.C * 4, hipMemcpyDeviceToDevice, ctx->stream);
  if (e != hipSuccess) return hip_fail(ctx, e, __func__);
  *steps = k + 1;
  return DG_OK;
}

dg_status dg_peak_stream_read(dg_ctx ctx, const void *buf, size_t bytes, uint32_t *sink) {
  DG_ENTER();
  DG_REQUIRE_PTR(buf);
  DG_REQUIRE_PTR(sink);
  if (bytes == 0 || bytes % 16 || ((uintptr_t)buf & 15))
    return fail(ctx, DG_ERR_SHAPE, "%s: bytes must be a positive multiple of 16, buf 16-byte aligned", __func__);
  const hipError_t e = dg_launch_stream_read(buf, (int64_t)bytes, sink, DG_PEAK_STREAM_BLOCKS, ctx->stream);
  return e == hipSuccess ? DG_OK : hip_fail(ctx, e, __func__);
}

dg_status dg_peak_mfma_bf16(dg_ctx ctx, int32_t iters, float *sink) {
  DG_ENTER();
  DG_REQUIRE_PTR(sink);
  if (iters < 1 || iters > 16384) return fail(ctx, DG_ERR_RANGE, "%s: iters=%d outside [1, 16384]", __func__, iters);
  const hipError_t e = dg_launch_mfma_peak(iters, sink, DG_PEAK_MFMA_BLOCKS, ctx->stream);
  return e == hipSuccess ? DG_OK : hip_fail(ctx, e, __func__);
}

}  // extern "C"
