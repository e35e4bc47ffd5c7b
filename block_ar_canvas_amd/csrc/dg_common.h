// Shared device helpers and the workspace layout of the canvas-denoise library.
//
// Matrix-core convention used by every kernel (CDNA4 / gfx950, wave64):
//   v_mfma_f32_32x32x16_bf16 computes D[32x32] += A[32x16] * B[16x32] where lane l
//   holds A[l%32][8*(l/32) .. +8], B[8*(l/32) .. +8][l%32], and accumulator register r
//   holds D[8*(r/4) + 4*(l/32) + r%4][l%32].
// Kernels put the "long" operand (vocabulary rows, keys, weight rows) in A and the
// canvas-side operand in B, so each lane's accumulator column is one canvas position
// (or query row): row reductions over vocabulary / keys stay inside a lane pair.
//
// Row permutation trick: when an accumulator tile is fed back into a second MFMA as
// its B operand (attention probabilities into P.V, softmax probabilities into p0.E),
// A-row i of the first MFMA is loaded from physical row pi(i) = i with bits 2 and 3
// swapped. Then accumulator registers [8s, 8s+8) of lane (c, h) hold physical rows
// 16s + 8h + [0, 8): exactly the B fragment of k-step s of the second MFMA, in
// natural order, with no data movement.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>
#include <initializer_list>

typedef uint16_t u16;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

#define DG_DEV __device__ __forceinline__

DG_DEV f32x16_t mfma_32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Physical row of MFMA A-row i (swap bits 2 and 3), see the header comment.
DG_DEV int perm_row(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

// Row of accumulator register r for the lane half h (natural A-row order).
DG_DEV int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }
// Physical row of accumulator register r when A rows were loaded through perm_row.
DG_DEV int acc_row_perm(int r, int h) { return 16 * (r >> 3) + 8 * h + (r & 7); }

DG_DEV float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
DG_DEV float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bf16, round to nearest even; NaN stays NaN.
DG_DEV u16 f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u16)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (u16)(u >> 16);
}
// Two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32 on gfx950).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
DG_DEV uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Max / sum over the lane pair (l, l ^ 32) without an LDS round trip: one
// v_permlane32_swap leaves {v[l], v[l ^ 32]} in the two registers of every lane (in an
// order that depends on the half, which neither symmetric operation sees).
DG_DEV float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
DG_DEV float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// 2^x by the hardware instruction (no denormal-range fix-up: results below 2^-126 may
// flush to zero, which no softmax weight here can notice).
DG_DEV float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Direct global -> LDS copy of 16 bytes per lane (gfx950 global_load_lds_dwordx4):
// lane l's 16 bytes land at LDS byte address lds_base + 16*l, lds_base wave-uniform.
// Issued through inline asm so that only the explicit dma_wait<N>() (s_waitcnt
// vmcnt(N): at most N of this wave's vector-memory loads still outstanding) orders
// the copies against LDS reads; callers follow it with a workgroup barrier.
DG_DEV void dma16(const void *gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}
template <int N>
DG_DEV void dma_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
DG_DEV uint32_t lds_addr(const void *p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

// Sticky device status codes (mirror dg_status).
#define DGS_RANGE 4
#define DGS_NONFINITE 7
DG_DEV void set_status(int *status, int code) {
  if (status) atomicMax(status, code);
}

// ------------------------------------------------------------------ tiling constants
#define DG_CT 32        // canvas columns per MFMA tile
#define DG_BV 256       // vocabulary rows per logits tile (one set of tile statistics)
#define DG_KT 64        // keys per attention tile

static inline int64_t dg_round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
static inline int64_t dg_cdiv(int64_t x, int64_t m) { return (x + m - 1) / m; }

// ------------------------------------------------------------------ host: per-device state
// Launchers run with the calling context's device current (every API call that enqueues
// work makes it current first). Launch attributes and the CU count are properties of a
// device, so their caches are kept per device.
#define DG_MAX_DEVICES 64
static inline int dg_current_device() {
  int d = 0;
  return hipGetDevice(&d) == hipSuccess && d >= 0 && d < DG_MAX_DEVICES ? d : 0;
}
// Compute units of the current device (256 on an MI355X if the query fails).
static inline int dg_device_cus() {
  static std::atomic<int> cus[DG_MAX_DEVICES];
  const int dev = dg_current_device();
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}
// Raises the dynamic LDS limit of the given kernels to `bytes` on the current device, the
// first time a launcher asks on that device (`done` is the launcher's own per-device flag
// array). Setting it twice is harmless, so concurrent first calls need no lock.
static inline hipError_t dg_smem_attr_once(std::atomic<bool> (&done)[DG_MAX_DEVICES], int bytes,
                                           std::initializer_list<const void *> kernels) {
  const int dev = dg_current_device();
  if (done[dev].load(std::memory_order_acquire)) return hipSuccess;
  for (const void *k : kernels) {
    const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
  }
  done[dev].store(true, std::memory_order_release);
  return hipSuccess;
}

// ------------------------------------------------------------------ workspace layout
// All regions are 256-byte aligned. Sizes depend on the dims and the cache capacity
// only, so one workspace serves every step of a run.
struct DgWs {
  int Cpad;        // C rounded up to 32
  int Vpad;        // V rounded up to DG_BV
  int T;           // vocabulary tiles = Vpad / DG_BV
  int nsc;         // self-conditioning split-K parts over the vocabulary
  int nsplit_max;  // attention split-K parts at Pcap
  size_t ptilde;   // bf16 p~ in MFMA fragment order: [Cpad/32][Vpad/16][64 lanes][8]
  size_t tmax, trho, tsum, tent, targ;  // per-(column, tile) statistics [Cpad][T]
  size_t colR;     // per-column reference R = max_t rho_t                  [Cpad]
  size_t colZ;     // per-column softmax sum relative to 2^R                 [Cpad]
  size_t colP;     // per-column confidence: the largest probability of p0   [Cpad]
  size_t rhoS;     // per-(split, column) reference rho_S = max over the split [nsc][Cpad]
  size_t q;        // Q   bf16 [Cpad][Hq*hd]
  size_t kc;       // canvas keys   bf16 [Cpad][Hkv*hd]
  size_t vct;      // canvas values bf16 [Hkv*hd][Cpad] (transposed)
  size_t o;        // attention output before Wo, bf16 [Cpad][Hq*hd]
  size_t po;       // attention partial O bf16 [nsplit][Hq][Cpad][hd]
  size_t pml;      // attention partial (max, sum) fp32 [nsplit][Hq][Cpad][2]
  size_t ps;       // self-cond partial s^T fp32 [nsc][d][Cpad]
  size_t s;        // s = p0 E rounded to bf16 [Cpad][d]
  size_t g;        // GELU(s W1^T) bf16 [Cpad][F]
  size_t x;        // denoiser input E[x] + z, bf16 [Cpad][d]
  size_t total;
};

// Attention split count for a given number of cached tokens (non-decreasing in P):
// about one workgroup (one KV head, 256 query rows, one key range) per CU, with at
// least 4 key tiles of 64 per range.
static inline int dg_attn_nsplit(int Hkv, int Hq, int C, int64_t P) {
  const int64_t nq = dg_cdiv((int64_t)(Hq / Hkv) * C, 256);
  const int64_t tiles = dg_cdiv(C, DG_KT) + dg_cdiv(P, DG_KT);
  int64_t ns = dg_cdiv(256, (int64_t)Hkv * nq);
  const int64_t by_len = dg_cdiv(tiles, 4);
  if (ns > by_len) ns = by_len;
  if (ns < 1) ns = 1;
  if (ns > 256) ns = 256;
  return (int)ns;
}

// Self-conditioning split count over the T vocabulary tiles: aim at >= 256 workgroups
// (256-wide j slices x 256-canvas blocks x splits), >= 4 tiles per split, and at most
// 128 tiles per split (the split's shift table is staged in 32 KiB of LDS). With a short
// vocabulary the splits are short and many, so the grid fills most of the chip; the
// reduce then reads more partials. Measured at 32768 ids (128 tiles, d = 1024): 32
// splits of 4 tiles ran the step about 1% faster than 64 splits of 2 (fewer partials to
// write and reduce, half the CUs idle in the split pass), 16 and 8 splits 12% and 32%
// slower.
static inline int dg_selfcond_nsplit(int d, int Cpad, int T) {
  const int64_t jt = dg_cdiv(d, 256) * dg_cdiv(Cpad, 256);
  int64_t ns = dg_cdiv(256, jt);
  const int64_t by_len = T / 4;
  if (ns > by_len) ns = by_len;
  const int64_t min_ns = dg_cdiv(T, 128);
  if (ns < min_ns) ns = min_ns;
  if (ns < 1) ns = 1;
  return (int)ns;
}

static inline DgWs dg_ws_layout(int V, int d, int C, int Hq, int Hkv, int hd, int F,
                                int64_t Pcap) {
  DgWs w;
  w.Cpad = (int)dg_round_up(C, DG_CT);
  w.Vpad = (int)dg_round_up(V, DG_BV);
  w.T = w.Vpad / DG_BV;
  w.nsc = dg_selfcond_nsplit(d, w.Cpad, w.T);
  w.nsplit_max = dg_attn_nsplit(Hkv, Hq, C, Pcap);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = (size_t)dg_round_up((int64_t)(off + bytes), 256);
    return at;
  };
  const size_t CT = (size_t)w.T * w.Cpad;
  w.ptilde = take((size_t)w.Cpad * w.Vpad * 2);
  w.tmax = take(CT * 4);
  w.trho = take(CT * 4);
  w.tsum = take(CT * 4);
  w.tent = take(CT * 4);
  w.targ = take(CT * 4);
  w.colR = take((size_t)w.Cpad * 4);
  w.colZ = take((size_t)w.Cpad * 4);
  w.colP = take((size_t)w.Cpad * 4);
  w.rhoS = take((size_t)w.nsc * w.Cpad * 4);
  w.q = take((size_t)w.Cpad * Hq * hd * 2);
  w.kc = take((size_t)w.Cpad * Hkv * hd * 2);
  w.vct = take((size_t)w.Cpad * Hkv * hd * 2);
  w.o = take((size_t)w.Cpad * Hq * hd * 2);
  w.ps = take((size_t)w.nsc * w.Cpad * d * 4);
  w.s = take((size_t)w.Cpad * d * 2);
  w.g = take((size_t)w.Cpad * F * 2);
  w.x = take((size_t)w.Cpad * d * 2);
  // Regions sized by the cache capacity come last, so every other offset is the same
  // whatever Pcap the layout is computed for.
  w.po = take((size_t)w.nsplit_max * Hq * w.Cpad * hd * 2);
  w.pml = take((size_t)w.nsplit_max * Hq * w.Cpad * 2 * 4);
  w.total = off;
  return w;
}

// Regions of canvas attention only (X, Q, canvas K/V, O, split partials), packed for
// the allocation-free variant, whose scratch holds nothing else. 256-byte aligned.
struct DgAttnWs {
  int Cpad;
  size_t x, q, kc, vct, o, po, pml, total;
};
static inline DgAttnWs dg_attn_ws_layout(int d, int C, int Hq, int Hkv, int hd, int nsplit) {
  DgAttnWs w;
  w.Cpad = (int)dg_round_up(C, DG_CT);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = (size_t)dg_round_up((int64_t)(off + bytes), 256);
    return at;
  };
  w.x = take((size_t)w.Cpad * d * 2);
  w.q = take((size_t)w.Cpad * Hq * hd * 2);
  w.kc = take((size_t)w.Cpad * Hkv * hd * 2);
  w.vct = take((size_t)w.Cpad * Hkv * hd * 2);
  w.o = take((size_t)w.Cpad * Hq * hd * 2);
  w.po = take((size_t)nsplit * Hq * w.Cpad * hd * 2);
  w.pml = take((size_t)nsplit * Hq * w.Cpad * 2 * 4);
  w.total = off;
  return w;
}

// ------------------------------------------------------------------ launcher API
// Host-side launchers implemented by the kernel translation units.
struct GemmSeg {
  const u16 *W;        // [N][K] weight rows (output features x input features)
  int N;               // output features of this segment
  u16 *out;            // output: out + m*sm + (n/seg)*sg + (n%seg)*se
  int64_t sm, sg, se;
  int seg;
  int m_store;         // rows m >= m_store are computed but not stored
  int nblk0;           // first n-block of this segment in the grid
};
struct GemmArgs {
  int M, K;
  const u16 *A;        // plain activation [M][K], or NULL for the embedding gather
  const int *tokens;   // gather: row m = E[tokens[m]]
  const u16 *E;
  int V;
  int *status;
  int gelu;            // apply exact GELU before storing
  int nseg;
  GemmSeg seg[3];
  int store_mode[3];   // set by the launcher
  // fp32 output (segment 0 only): out32[m * ld32 + n] = D[m][n] instead of bf16 stores
  float *out32;
  int ld32;
  // fp32 output only: K split into ksplit equal parts (each a multiple of 32); part s of
  // the sum goes to out32 + s * split_stride, and the consumer adds the parts in order.
  int ksplit;
  int64_t split_stride;
  // bf16 output of segment 0 with 16-byte stores along n (ST_NVEC) only: also writes
  // xsum[m * N + n] = bf16(E[xtok[m]][n] + D[m][n]), the next denoise step's input, with
  // xE rows of N elements (an id outside [0, xV) sets the range status and reads row 0)
  u16 *xsum;
  const int *xtok;
  const u16 *xE;
  int xV;
};
// 1 when the launch can form xsum in its epilogue (segment 0 stored with ST_NVEC).
int dg_gemm_can_xsum(const GemmArgs &a);
hipError_t dg_launch_gemm(const GemmArgs &a, hipStream_t st);

// Canvas MoE FFN workspace (256-byte aligned regions).
struct DgMoeWs {
  size_t logits;   // router logit parts fp32 [splits][C][E]
  size_t sel;      // selected experts int32 [C][K] (rank order)
  size_t gate;     // gates fp32 [C][K]
  size_t off;      // group offsets int32 [E + 1]
  size_t perm;     // tokens in grouped order int32 [C * K]
  size_t pos;      // grouped row of (token, rank) int32 [C * K]
  size_t tiles;    // expert GEMM work list int32: count, then (expert | row block << 16)
  size_t h;        // expert hidden bf16 [C * K][Fe] (grouped order)
  size_t yg;       // expert outputs bf16 [C * K][d] (grouped order)
  size_t hs;       // shared hidden bf16 [C][Fs]
  size_t ys;       // shared output bf16 [C][d]
  size_t total;
};
// Rows per expert GEMM tile, and the most tiles a routing can produce: every non-empty
// group has ceil(rows / MOE_TM) <= rows / MOE_TM + 1 tiles, and at most min(E, C * K)
// groups are non-empty.
constexpr int MOE_TM = 32;
static inline int dg_moe_max_tiles(int C, int E, int K) {
  const int ck = C * K;
  return (E < ck ? E : ck) + ck / MOE_TM;
}
// Router logits are computed in this many k parts (more workgroups on a short GEMM):
// halve the depth while it stays a multiple of 32 and at least 256, up to 8 parts.
static inline int dg_moe_router_splits(int d) {
  int s = 1;
  while (s < 8 && d % (2 * s * 32) == 0 && d / (2 * s) >= 256) s *= 2;
  return s;
}
static inline DgMoeWs dg_moe_ws_layout(int C, int d, int E, int K, int Fe, int Fs) {
  DgMoeWs w;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = (size_t)dg_round_up((int64_t)(off + bytes), 256);
    return at;
  };
  const size_t CK = (size_t)C * K;
  w.logits = take((size_t)dg_moe_router_splits(d) * C * E * 4);
  w.sel = take(CK * 4);
  w.gate = take(CK * 4);
  w.off = take((size_t)(E + 1) * 4);
  w.perm = take(CK * 4);
  w.pos = take(CK * 4);
  w.tiles = take((size_t)(1 + dg_moe_max_tiles(C, E, K)) * 4);
  w.h = take(CK * Fe * 2);
  w.yg = take(CK * d * 2);
  w.hs = take((size_t)C * Fs * 2);
  w.ys = take((size_t)C * d * 2);
  w.total = off;
  return w;
}
hipError_t dg_launch_moe_route(const float *logits, int splits, int C, int E, int K, int *sel, float *gate,
                               hipStream_t st);
hipError_t dg_launch_moe_group(const int *sel, int C, int K, int E, int *off, int *perm, int *pos,
                               int *nact, int *tiles, hipStream_t st);
// Grouped expert GEMM: for each listed tile (expert e, rows [m0, m0 + MOE_TM) of its group),
// Y[off[e] + m][n] = act(sum_k X[row][k] W[e][n][k]), row = perm[off[e] + m] (perm
// non-NULL) or off[e] + m. N, K multiples of 32; Y row stride ldY.
struct MoeGemmArgs {
  const u16 *X, *W;
  const int *off, *perm, *tiles;
  u16 *Y;
  int N, K, ldY, gelu, max_tiles;
};
hipError_t dg_launch_moe_expert(const MoeGemmArgs &a, hipStream_t st);

// Measured ceilings (streaming read, back-to-back bf16 MFMAs).
hipError_t dg_launch_stream_read(const void *buf, int64_t bytes, uint32_t *sink, int blocks, hipStream_t st);
hipError_t dg_launch_mfma_peak(int iters, float *sink, int blocks, hipStream_t st);
hipError_t dg_launch_moe_combine(const u16 *Yg, const u16 *Ys, const float *gate, const int *pos,
                                 int C, int K, int d, u16 *Y, hipStream_t st);
hipError_t dg_launch_xgather(const int *tokens, const u16 *E, const u16 *z, int V, int M, int K,
                             u16 *X, int *status, hipStream_t st);

struct AttnArgs {
  const u16 *Q;        // [Cpad][Hq*hd]
  const u16 *Kp;       // [Hkv][Pcap][hd]
  const u16 *Vt;       // [Hkv][hd][Pcap]
  const u16 *Kc;       // [Cpad][Hkv*hd]
  const u16 *Vct;      // [Hkv*hd][Cpad]
  int64_t P, Pcap;
  int C, Cpad, Hq, Hkv, hd;
  int nsplit;
  int causal;          // 1: canvas-segment key j visible to query i only for j <= i
  float scale_log2;    // log2(e) / sqrt(hd)
  u16 *po;             // [nsplit][Hq][Cpad][hd] bf16, relative to the split's max
  float *pml;          // [nsplit][Hq][Cpad][2]
  u16 *O;              // merged output [Cpad][Hq*hd]
};
hipError_t dg_launch_attention(const AttnArgs &a, hipStream_t st);
// Rotates the block's queries q [C][Hq*hd] and keys kc [C][Hkv*hd] to positions pos0 + r in
// place (base > 0), and, when Kp is given, writes the keys to Kp rows [P, P + C) and the
// values vct [Hkv*hd][Cpad] to Vt columns [P, P + C). One launch.
hipError_t dg_launch_rope_store(u16 *q, u16 *kc, const u16 *vct, int C, int Cpad, int Hq, int Hkv, int hd,
                                int64_t pos0, double base, u16 *Kp, u16 *Vt, int64_t P, int64_t Pcap,
                                hipStream_t st);

struct LogitsArgs {
  const u16 *H;        // [C][d]
  const u16 *E;        // [V][d]
  int V, d, C, Cpad, T;
  int nsc;             // self-conditioning splits (sets the tile dispatch order)
  float inv_tau;
  u16 *ptilde;
  float *tmax, *trho, *tsum, *tent;
  int *targ;
  float *colR, *colZ;  // per-column reference and softmax sum
  float *colP;         // per-column largest probability
  float *entropy;      // [C]
  int *argmax;         // [C]
  int *status;
};
hipError_t dg_launch_logits(const LogitsArgs &a, hipStream_t st);

// Acceptance, renoise and stop test of B canvases of C positions (see dg_sampler_dev.h).
struct ArsArgs {
  int B, C, tpp, V, step, N;
  const float *ent;
  const int *x0, *am, *prev;
  uint64_t budget, limit, seed;
  uint32_t canvas_base;
  uint8_t *acc;
  int *nacc, *tok, *flag;
};

struct SelfcondArgs {
  const u16 *ptilde;
  const float *trho;   // [Cpad][T] tile references
  const float *colR, *colZ;
  float *rhoS;         // [nsc][Cpad] split references (written here)
  const u16 *E;        // [V][d]
  int V, d, C, Cpad, T, nsc;
  float *ps;           // [nsc][d][Cpad]
  u16 *s;              // [Cpad][d]
};
// With ars non-null (ars->tpp * ars->C <= 256), acceptance, renoise and the stop test of
// ars->B canvases run as extra workgroups of the reduce launch.
hipError_t dg_launch_selfcond(const SelfcondArgs &a, const ArsArgs *ars, hipStream_t st);

hipError_t dg_launch_accept(int B, int C, const float *ent, uint64_t budget, uint8_t *acc,
                            int *nacc, hipStream_t st);
hipError_t dg_launch_topk(int B, int C, const float *score, int k, uint8_t *acc, int *nacc,
                          hipStream_t st);
struct SampleArgs {
  const u16 *ptilde;   // p~ in MFMA fragment order (see DgWs)
  const float *tsum, *trho, *colR;
  int T, VS, V;        // tiles, Vpad / 16, vocabulary
  int B, Cs;           // canvases and positions per canvas (columns = B * Cs)
  uint64_t seed;
  uint32_t canvas_base, step;
  int *tokens;         // [B * Cs]
};
hipError_t dg_launch_sample(const SampleArgs &a, hipStream_t st);
hipError_t dg_launch_confidence(int C, const float *colP, float *conf, hipStream_t st);
hipError_t dg_launch_renoise(int B, int C, int V, const int *am, const uint8_t *acc,
                             uint64_t seed, uint32_t canvas_base, uint32_t step, int *tok,
                             hipStream_t st);
hipError_t dg_launch_stop(int B, int C, const float *ent, const int *am, const int *prev,
                          uint64_t limit, int step, int N, int *flag, hipStream_t st);
// dg_launch_accept, dg_launch_renoise (with acc) and dg_launch_stop in one launch (r.tpp
// is chosen here).
hipError_t dg_launch_accept_renoise_stop(const ArsArgs &r, hipStream_t st);
