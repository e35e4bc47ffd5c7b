// Small-M bf16 GEMM with fp32 accumulation: D[m][n] = sum_k X[m][k] W[n][k].
//
// Used for every dense projection of the step whose M is the canvas (C <= 1024):
// the Q/K/V projections of the denoiser input X = E[x] + z, the attention output
// projection Wo, the two self-conditioning FFW layers (exact-erf GELU fused into the
// epilogue of the first) and the K/V projection of a committed block. Up to three
// weight segments share one launch; each segment has its own output address map
// out + m*sm + (n/seg)*sg + (n%seg)*se, which covers row-major outputs, the transposed
// canvas V, and the [Hkv][Pcap][hd] / [Hkv][hd][Pcap] cache layouts.
//
// With M this small every workgroup streams a long K range for a small output tile, so
// the kernel is bound by how fast operand bytes reach the CUs, not by the MFMAs:
//   * Workgroup tile TN n x TM m (64 x 64, 32 x 64 or 32 x 32, chosen per launch so
//     that the operand bytes each CU streams are fewest while the grid fills the
//     chip), K in stages of 128 (256-byte row pieces), fed by direct global -> LDS
//     copies (global_load_lds_dwordx4) into an NS-stage ring with one barrier per
//     stage; 256-byte LDS rows are XOR-swizzled by (row & 15) so the fragment reads
//     are conflict-free on 64 banks.
//   * 8 waves; wave w computes the whole tile (up to four independent 32 x 32
//     accumulators) for k16-step w of every stage, so a wave's MFMAs per stage do not
//     form a dependent chain. The eight partial tiles are summed through LDS in a fixed
//     wave order (deterministic), so every output element takes the same additions in
//     the same order whatever the tile shape: results do not depend on the shape.
//   * The epilogue (GELU, bf16 rounding) writes the tile to LDS and stores it with
//     16-byte stores along whichever output direction is contiguous.
//   * Workgroups that share a weight tile (same n tile, other m tiles) are placed on
//     the same XCD, so each weight tile is fetched from HBM once per L2.
// The embedding gather X = E[tokens] (rows read through per-lane addresses) is done by
// the copies themselves. The self-conditioned input bf16(E[tokens] + z) needs ALU work
// that a direct copy cannot do: xgather_kernel forms it, or the FFW W2 launch does in
// its epilogue (xsum), reading the E rows of the new tokens at the positions where it
// stores z and adding with the gather kernel's routine, so both give the same bits.
#include "dg_common.h"

namespace {

constexpr int BK = 128, NW = 8;
constexpr int RB = BK * 2;                  // bytes of one row piece per stage

DG_DEV int swz(int row, int chunk) { return row * RB + ((chunk ^ (row & 15)) << 4); }

// Shape of a launch: TN weight rows (n) x TM activation rows (m) per workgroup, each a
// multiple of 32, and NS ring stages.
template <int TN, int TM, int NS>
struct Tile {
  static constexpr int QN = TN / 32, QM = TM / 32, NQ = QN * QM;   // 32 x 32 MFMA tiles
  static constexpr int WT = TN * RB;                // weight bytes of one stage
  static constexpr int STAGE = WT + TM * RB;
  static constexpr int CPW = QN + QM;               // copies per wave and stage (4 rows each)
  static constexpr int RED = NW * NQ * 16 * 64 * 4; // fp32 partial tiles of all waves
  static constexpr int SMEM = NS * STAGE > RED ? NS * STAGE : RED;
  static constexpr int OPITCH = TN + 8;             // bf16 output tile pitch (elements)
  static constexpr int RPW = NQ * 2;                // summed accumulator registers per wave
};

// s_waitcnt for "at most CPW*rem of this wave's copies still in flight" (rem <= 6).
template <int CPW>
DG_DEV void wait_stages(int rem) {
  switch (rem) {
    case 0: dma_wait<0>(); break;
    case 1: dma_wait<CPW>(); break;
    case 2: dma_wait<2 * CPW>(); break;
    case 3: dma_wait<3 * CPW>(); break;
    case 4: dma_wait<4 * CPW>(); break;
    case 5: dma_wait<5 * CPW>(); break;
    default: dma_wait<6 * CPW>(); break;
  }
}

// Output store modes of a segment (chosen on the host).
enum { ST_SCALAR = 0, ST_NVEC = 1, ST_MVEC = 2 };

// Eight bf16 sums e + z, each added in float32 and rounded to bf16 (the denoiser input
// X = bf16(E[x] + z), wherever it is formed).
DG_DEV uint4 add_bf16x8(uint4 ee, uint4 zz) {
  const uint32_t *e = (const uint32_t *)&ee, *zw = (const uint32_t *)&zz;
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(bf16lo(e[j]) + bf16lo(zw[j]), bf16hi(e[j]) + bf16hi(zw[j]));
  return make_uint4(o[0], o[1], o[2], o[3]);
}

template <int TN, int TM, int NS, bool GATHER>
__global__ __launch_bounds__(512) void gemm_kernel(GemmArgs a, int MB) {
  using T = Tile<TN, TM, NS>;
  static_assert(TN % 32 == 0 && TM % 32 == 0 && TN <= 64 && TM <= 64 && NS >= 2 && NS <= 8, "shape");
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;

  // Tile of this workgroup; consecutive m tiles of one n tile share an XCD.
  // With a k split (fp32 output only) the grid holds ksplit copies of the tile grid.
  const int S = (a.out32 && a.ksplit > 1) ? a.ksplit : 1;
  const int total = gridDim.x / S;
  const int ks = blockIdx.x / total;
  int idx = blockIdx.x % total;
  if ((total & 7) == 0 && ((total >> 3) % MB) == 0) idx = (idx & 7) * (total >> 3) + (idx >> 3);
  const int mb = idx % MB, nbg = idx / MB;
  int si = 0;
  for (int s = 1; s < a.nseg; ++s)
    if (nbg >= a.seg[s].nblk0) si = s;
  const GemmSeg &sg = a.seg[si];
  const int nb0 = (nbg - sg.nblk0) * TN, m0 = mb * TM;
  const int K = a.K / S;                             // depth of this part
  const int kbase = ks * K;
  const int nst = (K + BK - 1) / BK;

  // Copy assignment: wave w fills rows [w*TN/8, +TN/8) of the weight tile and
  // [w*TM/8, +TM/8) of the activation tile, 4 rows (1 KiB) per instruction; lane l
  // covers row base + l/16, physical 16-byte chunk l % 16.
  const u16 *wrow[T::QN], *xrow[T::QM];
  int wchunk[T::QN], xchunk[T::QM];
#pragma unroll
  for (int j = 0; j < T::QN; ++j) {
    const int R = (TN / 8) * wave + 4 * j + (lane >> 4);
    wchunk[j] = (lane & 15) ^ (R & 15);
    const int n = min(nb0 + R, sg.N - 1);
    wrow[j] = sg.W + (int64_t)n * a.K + kbase;
  }
#pragma unroll
  for (int j = 0; j < T::QM; ++j) {
    const int R = (TM / 8) * wave + 4 * j + (lane >> 4);
    xchunk[j] = (lane & 15) ^ (R & 15);
    const int m = min(m0 + R, a.M - 1);
    if (GATHER) {
      int tok = a.tokens[m];
      if (tok < 0 || tok >= a.V) {
        set_status(a.status, DGS_RANGE);
        tok = 0;
      }
      xrow[j] = a.E + (int64_t)tok * a.K + kbase;
    } else {
      xrow[j] = a.A + (int64_t)m * a.K + kbase;
    }
  }
  const uint32_t lbase = lds_addr(smem);
  auto issue = [&](int i) {
    const int k0 = i * BK;
    const uint32_t wb = lbase + (uint32_t)((i % NS) * T::STAGE);
#pragma unroll
    for (int j = 0; j < T::QN; ++j) {
      const int k = min(k0 + 8 * wchunk[j], K - 8);   // chunks past K: any valid data
      dma16(wrow[j] + k, wb + (uint32_t)(((TN / 8) * wave + 4 * j) * RB));
    }
#pragma unroll
    for (int j = 0; j < T::QM; ++j) {
      const int k = min(k0 + 8 * xchunk[j], K - 8);
      dma16(xrow[j] + k, wb + (uint32_t)(T::WT + ((TM / 8) * wave + 4 * j) * RB));
    }
  };

  // Wave w computes the whole tile for k16-step w of every stage; tile q = i + QN*j
  // covers n [32i, +32) x m [32j, +32).
  f32x16_t acc[T::NQ] = {};
  for (int i = 0; i < NS - 1 && i < nst; ++i) issue(i);
  for (int i = 0; i < nst; ++i) {
    wait_stages<T::CPW>(min(nst - 1 - i, NS - 2));
    __syncthreads();
    if (i + NS - 1 < nst) issue(i + NS - 1);
    if (i * BK + 16 * wave < K) {
      const uint8_t *Ws = smem + (i % NS) * T::STAGE, *Xs = Ws + T::WT;
      const int c = 2 * wave + h;
      u32x4_t af[T::QN], bf[T::QM];
#pragma unroll
      for (int j = 0; j < T::QN; ++j) af[j] = *(const u32x4_t *)(Ws + swz(32 * j + l32, c));
#pragma unroll
      for (int j = 0; j < T::QM; ++j) bf[j] = *(const u32x4_t *)(Xs + swz(32 * j + l32, c));
#pragma unroll
      for (int jm = 0; jm < T::QM; ++jm)
#pragma unroll
        for (int jn = 0; jn < T::QN; ++jn)
          acc[jn + T::QN * jm] = mfma_32x32x16(af[jn], bf[jm], acc[jn + T::QN * jm]);
    }
  }

  // The next step's input (segment 0, 16-byte stores along n): this thread's 16 bytes of
  // E[x] are loaded now, so their latency overlaps the reduction below.
  uint4 xe = make_uint4(0u, 0u, 0u, 0u);
  const bool xdo = a.xsum && si == 0 && a.store_mode[0] == ST_NVEC && tid < TM * (TN / 8);
  if (xdo) {
    const int m = m0 + tid / (TN / 8), n = nb0 + (tid % (TN / 8)) * 8;
    if (m < sg.m_store && n < sg.N) {
      int tok = a.xtok[m];
      if (tok < 0 || tok >= a.xV) {                  // read as id 0, like the gather GEMM
        set_status(a.status, DGS_RANGE);
        tok = 0;
      }
      xe = *(const uint4 *)(a.xE + (int64_t)tok * sg.N + n);
    }
  }

  // Sum of the eight waves' tiles in a fixed wave order; wave w then owns registers
  // [w*RPW, +RPW) of the tile sequence (tile q = index / 16, register = index % 16).
  __syncthreads();
  float *red = (float *)smem;
#pragma unroll
  for (int q = 0; q < T::NQ; ++q)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[((wave * T::NQ + q) * 16 + r) * 64 + lane] = acc[q][r];
  __syncthreads();
  const int q = (wave * T::RPW) >> 4, rb = (wave * T::RPW) & 15;
  const int qn = q % T::QN, qm = q / T::QN;
  float v[T::RPW];
#pragma unroll
  for (int r = 0; r < T::RPW; ++r) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += red[((w * T::NQ + q) * 16 + rb + r) * 64 + lane];
    if (a.gelu) s = 0.5f * s * (1.0f + erff(s * 0.70710678118654752f));
    v[r] = s;
  }
  if (a.out32) {                                     // fp32 output, row-major
    const int m = m0 + qm * 32 + l32;
    if (m < sg.m_store) {
#pragma unroll
      for (int r = 0; r < T::RPW; ++r) {
        const int n = nb0 + qn * 32 + acc_row(rb + r, h);
        if (n < sg.N) a.out32[ks * a.split_stride + (int64_t)m * a.ld32 + n] = v[r];
      }
    }
    return;
  }
  __syncthreads();
  u16 *ot = (u16 *)smem;   // [TM m][OPITCH] bf16
  const int ml = qm * 32 + l32;
#pragma unroll
  for (int r = 0; r < T::RPW; ++r) ot[ml * T::OPITCH + qn * 32 + acc_row(rb + r, h)] = f32_to_bf16(v[r]);
  __syncthreads();

  const int mode = a.store_mode[si];
  if (mode == ST_MVEC) {
    if (tid >= TN * (TM / 8)) return;
    const int col = tid / (TM / 8), r8 = (tid % (TM / 8)) * 8;
    const int m = m0 + r8, n = nb0 + col;
    if (n < sg.N && m + 8 > sg.m_store) {
      for (int i = 0; i < 8 && m + i < sg.m_store; ++i)
        sg.out[(int64_t)(m + i) + (int64_t)(n / sg.seg) * sg.sg + (int64_t)(n % sg.seg) * sg.se] =
            ot[(r8 + i) * T::OPITCH + col];
    } else if (n < sg.N) {
      uint32_t w4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w4[i] = (uint32_t)ot[(r8 + 2 * i) * T::OPITCH + col] |
                ((uint32_t)ot[(r8 + 2 * i + 1) * T::OPITCH + col] << 16);
      *(uint4 *)(sg.out + (int64_t)m + (int64_t)(n / sg.seg) * sg.sg + (int64_t)(n % sg.seg) * sg.se) =
          make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
    return;
  }
  if (tid >= TM * (TN / 8)) return;
  const int row = tid / (TN / 8), c8 = (tid % (TN / 8)) * 8;
  const int m = m0 + row;
  if (mode == ST_NVEC) {
    const int n = nb0 + c8;
    if (m < sg.m_store && n < sg.N) {
      const uint4 zz = *(const uint4 *)(ot + row * T::OPITCH + c8);
      *(uint4 *)(sg.out + (int64_t)m * sg.sm + (int64_t)(n / sg.seg) * sg.sg + (int64_t)(n % sg.seg) * sg.se) = zz;
      if (xdo) *(uint4 *)(a.xsum + (int64_t)m * sg.N + n) = add_bf16x8(xe, zz);   // E[x] + this output
    }
  } else if (m < sg.m_store) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n = nb0 + c8 + i;
      if (n < sg.N)
        sg.out[(int64_t)m * sg.sm + (int64_t)(n / sg.seg) * sg.sg + (int64_t)(n % sg.seg) * sg.se] =
            ot[row * T::OPITCH + c8 + i];
    }
  }
}

// X[m][k] = bf16(E[tokens[m]][k] + z[m][k]) for m < M; an out-of-range token sets the
// range status and contributes a zero embedding row.
__global__ __launch_bounds__(256) void xgather_kernel(const int *tokens, const u16 *E,
                                                      const u16 *z, int V, int K, u16 *X,
                                                      int *status) {
  const int m = blockIdx.x;
  int tok = tokens[m];
  if (tok < 0 || tok >= V) {                         // read as id 0, like the gather GEMM
    if (threadIdx.x == 0) set_status(status, DGS_RANGE);
    tok = 0;
  }
  for (int k = threadIdx.x * 8; k < K; k += 256 * 8) {
    const uint4 zz = *(const uint4 *)(z + (int64_t)m * K + k);
    const uint4 ee = *(const uint4 *)(E + (int64_t)tok * K + k);
    *(uint4 *)(X + (int64_t)m * K + k) = add_bf16x8(ee, zz);
  }
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

// 16-byte stores are used when eight consecutive n (or m) map to one aligned run.
int store_mode(const GemmSeg &s) {
  if (!aligned16(s.out)) return ST_SCALAR;
  const bool seg8 = s.seg % 8 == 0 || s.seg >= (1 << 30);   // INT_MAX: one segment
  if (s.se == 1 && seg8 && s.sm % 8 == 0 && s.sg % 8 == 0) return ST_NVEC;
  if (s.sm == 1 && seg8 && s.se % 8 == 0 && s.sg % 8 == 0) return ST_MVEC;
  return ST_SCALAR;
}

}  // namespace

namespace {

// Sets the segments' first n blocks and store modes for tile width TN and launches one
// tile shape.
template <int TN, int TM, int NS>
hipError_t launch_tile(GemmArgs a, int S, hipStream_t st) {
  constexpr int smem = Tile<TN, TM, NS>::SMEM;
  static std::atomic<bool> attr[DG_MAX_DEVICES];
  const hipError_t e = dg_smem_attr_once(attr, smem, {(const void *)gemm_kernel<TN, TM, NS, false>,
                                                      (const void *)gemm_kernel<TN, TM, NS, true>});
  if (e != hipSuccess) return e;
  int nblk = 0, mmax = a.M;
  for (int s = 0; s < a.nseg; ++s) {
    a.seg[s].nblk0 = nblk;
    nblk += (a.seg[s].N + TN - 1) / TN;
    if (a.seg[s].m_store > mmax) mmax = a.seg[s].m_store;
    a.store_mode[s] = store_mode(a.seg[s]);
  }
  const int MB = (mmax + TM - 1) / TM;
  const dim3 grid(nblk * MB * S);
  if (a.A)
    hipLaunchKernelGGL((gemm_kernel<TN, TM, NS, false>), grid, dim3(512), smem, st, a, MB);
  else
    hipLaunchKernelGGL((gemm_kernel<TN, TM, NS, true>), grid, dim3(512), smem, st, a, MB);
  return hipGetLastError();
}

}  // namespace

// Tile shape: every workgroup streams (TN + TM) rows of K through its CU, so the shape
// with the fewest operand bytes per CU, rounds of workgroups x (TN + TM), is taken; on
// a tie the one with fewer workgroups (less total copying).
int dg_gemm_can_xsum(const GemmArgs &a) {
  const GemmSeg &s = a.seg[0];
  return a.nseg >= 1 && !a.out32 && store_mode(s) == ST_NVEC && s.sm == s.N && s.seg >= (1 << 30) ? 1 : 0;
}

hipError_t dg_launch_gemm(const GemmArgs &a, hipStream_t st) {
  const int S = (a.out32 && a.ksplit > 1) ? a.ksplit : 1;
  if (S > 1 && a.K % (32 * S) != 0) return hipErrorInvalidValue;
  int mmax = a.M;
  for (int s = 0; s < a.nseg; ++s)
    if (a.seg[s].m_store > mmax) mmax = a.seg[s].m_store;
  const int ncu = dg_device_cus();
  static const int shapes[3][2] = {{64, 64}, {32, 64}, {32, 32}};
  int best = 0;
  int64_t best_cost = INT64_MAX, best_wg = INT64_MAX;
  for (int c = 0; c < 3; ++c) {
    const int tn = shapes[c][0], tm = shapes[c][1];
    int64_t nblk = 0;
    for (int s = 0; s < a.nseg; ++s) nblk += (a.seg[s].N + tn - 1) / tn;
    const int64_t wg = nblk * ((mmax + tm - 1) / tm) * S;
    const int64_t cost = (wg + ncu - 1) / ncu * (tn + tm);
    if (cost < best_cost || (cost == best_cost && wg < best_wg)) {
      best = c;
      best_cost = cost;
      best_wg = wg;
    }
  }
  switch (best) {
    case 0: return launch_tile<64, 64, 4>(a, S, st);
    case 1: return launch_tile<32, 64, 5>(a, S, st);
    default: return launch_tile<32, 32, 4>(a, S, st);
  }
}

namespace {

// Rotary positions and the block's entry into the cache, in one launch. Three kinds of
// work items, in this order over the grid:
//   Q pairs (only when rotating): the pair (x_d, x_{d+hd/2}) of query head h of block row
//     r turns by (pos0 + r) * base^(-2d/hd), in place (half-split pairing; the openai-hub
//     page "从零拆开DiffusionGemma", closing remarks of step 3, names rotary positions as
//     part of the full model);
//   K pairs: the same turn for the block keys kc (when rotating), written back to kc for
//     the attention call and, when storing, to the cache rows Kp[g][P + r];
//   V elements (only when storing): vct [Hkv*hd][Cpad] to the cache columns Vt[g][e][P + r].
// Angle, sine, cosine and rotation in float64: token positions reach 2^18 and more, where
// a float32 angle is already off by about 1e-2 rad. The attention calls read the cache
// only below P, so storing the block before they run changes nothing they read.
struct RopeStoreArgs {
  u16 *q, *kc;
  const u16 *vct;
  int C, Cpad, Hq, Hkv, hd;
  int64_t pos0;
  double base;         // 0: no rotation
  u16 *Kp, *Vt;        // NULL: no store
  int64_t P, Pcap;
};

__global__ __launch_bounds__(256) void rope_store_kernel(RopeStoreArgs a, int64_t nq, int64_t nk) {
  const int half = a.hd / 2;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < nq + nk) {
    const bool isq = i < nq;
    if (!isq) i -= nq;
    const int heads = isq ? a.Hq : a.Hkv, ld = heads * a.hd;
    const int d = (int)(i % half);
    const int64_t rh = i / half;
    const int h = (int)(rh % heads), r = (int)(rh / heads);
    u16 *p = (isq ? a.q : a.kc) + (int64_t)r * ld + h * a.hd;
    u16 y1 = p[d], y2 = p[d + half];
    if (a.base > 0.0) {
      const double ang = (double)(a.pos0 + r) * pow(a.base, -2.0 * d / a.hd);
      double sn, cs;
      sincos(ang, &sn, &cs);
      const double x1 = __uint_as_float((uint32_t)y1 << 16);
      const double x2 = __uint_as_float((uint32_t)y2 << 16);
      y1 = f32_to_bf16((float)(x1 * cs - x2 * sn));
      y2 = f32_to_bf16((float)(x1 * sn + x2 * cs));
      p[d] = y1;
      p[d + half] = y2;
    }
    if (!isq && a.Kp) {
      u16 *kr = a.Kp + ((int64_t)h * a.Pcap + a.P + r) * a.hd;
      kr[d] = y1;
      kr[d + half] = y2;
    }
    return;
  }
  i -= nq + nk;
  if (a.Kp && i < (int64_t)a.C * a.Hkv * a.hd) {
    const int r = (int)(i % a.C);
    const int64_t ge = i / a.C;                      // g * hd + e
    a.Vt[ge * a.Pcap + a.P + r] = a.vct[ge * a.Cpad + r];
  }
}

}  // namespace

hipError_t dg_launch_rope_store(u16 *q, u16 *kc, const u16 *vct, int C, int Cpad, int Hq, int Hkv, int hd,
                                int64_t pos0, double base, u16 *Kp, u16 *Vt, int64_t P, int64_t Pcap,
                                hipStream_t st) {
  const RopeStoreArgs a{q, kc, vct, C, Cpad, Hq, Hkv, hd, pos0, base, Kp, Vt, P, Pcap};
  const int64_t nq = base > 0.0 ? (int64_t)C * Hq * (hd / 2) : 0;
  const int64_t nk = (base > 0.0 || Kp) ? (int64_t)C * Hkv * (hd / 2) : 0;
  const int64_t nv = Kp ? (int64_t)C * Hkv * hd : 0;
  const int64_t n = nq + nk + nv;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_store_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a, nq, nk);
  return hipGetLastError();
}

hipError_t dg_launch_xgather(const int *tokens, const u16 *E, const u16 *z, int V, int M, int K,
                             u16 *X, int *status, hipStream_t st) {
  hipLaunchKernelGGL(xgather_kernel, dim3(M), dim3(256), 0, st, tokens, E, z, V, K, X, status);
  return hipGetLastError();
}
