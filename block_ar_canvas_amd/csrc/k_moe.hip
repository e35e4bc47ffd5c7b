// Canvas MoE FFN: router top-K, token grouping by expert, combine.
//
// Method (DiffusionGemma Technical Report page, "Prerequisites", mixture of experts: each
// token uses 8 of 128 experts plus one shared expert, and a 256-token canvas touches
// about 84 distinct experts where one token touches 8; "Text diffusion models" survey,
// section 13: router top-k, expert GEMM, token permutation). The router logits and the
// shared expert use the plain GEMM; the kernels here route, group, run the routed
// experts and combine.
//
// moe_route_kernel: one workgroup per token; each thread holds one expert's logit (float32,
//   from the router GEMM) and counts the experts that beat it (larger logit, or equal
//   with a lower id); rank < K selects it. Gates: softmax over the K selected logits.
// moe_group_kernel: one workgroup; per expert, the number of tokens routed to it, the
//   exclusive offsets, the token list in token order (from per-expert token bitmasks:
//   deterministic), and for every (token, rank) the row of its expert output in grouped
//   order.
//   It also lists the work tiles of the expert GEMMs: one entry (expert, 64-row block) per
//   non-empty row block of every group.
// moe_expert_kernel: Y[off[e] + m] = act(X_e[m] . W[e]^T) for the grouped rows of
//   expert e. The weights are read once per tile, straight from memory into the MFMA A
//   operands (each wave owns 32 weight rows); the tile's activation rows (at most 64) are
//   staged per 128-deep k chunk in LDS and shared by the four waves.
// moe_combine_kernel: y[t] = bf16(sum over ranks k of gate[t][k] * Yg[pos[t][k]] + Ys[t]),
//   float32, ranks in order.
#include <float.h>

#include "dg_common.h"

namespace {

__global__ __launch_bounds__(256) void moe_route_kernel(const float *logits, int E, int K, int *sel,
                                                        float *gate) {
  __shared__ float lv[256];
  __shared__ float sv[32];
  const int t = blockIdx.x, tid = threadIdx.x;
  float v = -INFINITY;
  if (tid < E) {
    v = logits[(int64_t)t * E + tid];
    if (!(v == v)) v = -INFINITY;                    // a NaN logit ranks last
  }
  lv[tid] = v;
  __syncthreads();
  if (tid < E) {
    int rank = 0;
    for (int j = 0; j < E; ++j) {
      const float w = lv[j];
      rank += (w > v || (w == v && j < tid)) ? 1 : 0;
    }
    if (rank < K) {
      sel[(int64_t)t * K + rank] = tid;
      sv[rank] = v;
    }
  }
  __syncthreads();
  if (tid < K) {
    const float mx = sv[0];                          // rank 0 holds the largest logit
    float den = 0.f;
    for (int k = 0; k < K; ++k) den += expf(sv[k] - mx);
    gate[(int64_t)t * K + tid] = expf(sv[tid] - mx) / den;
  }
}

// Token sets as bitmasks: mask[e] holds bit t when token t routes to expert e (LDS
// atomic OR, so the result does not depend on the order of the updates). A token's row in
// its expert's group is the expert's offset plus the number of set bits below t: the
// grouped order is token order within each expert, the same on every run.
__global__ __launch_bounds__(256) void moe_group_kernel(const int *sel, int C, int K, int E, int *off,
                                                        int *perm, int *pos, int *nact, int *tiles) {
  extern __shared__ uint32_t mask[];                 // [E][W], W = C / 32 rounded up
  __shared__ int loff[257];
  const int tid = threadIdx.x, n = C * K, W = (C + 31) / 32;
  for (int i = tid; i < E * W; i += 256) mask[i] = 0u;
  __syncthreads();
  for (int i = tid; i < n; i += 256) {
    const int t = i / K, e = sel[i];
    atomicOr(&mask[e * W + (t >> 5)], 1u << (t & 31));
  }
  __syncthreads();
  // per expert: rows, 64-row tiles and a non-empty flag, packed as 14 + 9 + 9 bits (the
  // totals stay below 8192 rows, 384 tiles and 256 experts); one inclusive scan
  // (Hillis-Steele over the 256 threads) gives every offset at once
  __shared__ uint32_t scan[256];
  uint32_t v = 0;
  if (tid < E) {
    int c = 0;
    for (int w = 0; w < W; ++w) c += __popc(mask[tid * W + w]);
    v = (uint32_t)c | ((uint32_t)((c + MOE_TM - 1) / MOE_TM) << 14) | ((c > 0 ? 1u : 0u) << 23);
  }
  scan[tid] = v;
  __syncthreads();
  for (int dd = 1; dd < 256; dd <<= 1) {
    const uint32_t add = tid >= dd ? scan[tid - dd] : 0u;
    __syncthreads();
    scan[tid] += add;
    __syncthreads();
  }
  const uint32_t incl = scan[tid], excl = incl - v;
  if (tid < E) {
    const int o = (int)(excl & 0x3FFF), t0 = (int)((excl >> 14) & 0x1FF), nt = (int)((v >> 14) & 0x1FF);
    loff[tid] = o;
    off[tid] = o;
    for (int mt = 0; mt < nt; ++mt) tiles[1 + t0 + mt] = tid | (mt << 16);
  }
  if (tid == 255) {
    off[E] = (int)(incl & 0x3FFF);
    tiles[0] = (int)((incl >> 14) & 0x1FF);
    if (nact) nact[0] = (int)(incl >> 23);
  }
  __syncthreads();
  for (int i = tid; i < n; i += 256) {
    const int t = i / K, e = sel[i];
    const uint32_t *m = mask + e * W;
    int p = loff[e];
    for (int w = 0; w < (t >> 5); ++w) p += __popc(m[w]);
    p += __popc(m[t >> 5] & ((1u << (t & 31)) - 1u));
    perm[p] = t;
    pos[i] = p;
  }
}

// LDS slot of the 16-byte chunk q (of 16) of activation row m: XOR swizzle so that the
// 32 rows read by one MFMA operand load fall in distinct banks.
DG_DEV int xslot(int m, int q) { return m * 256 + ((q ^ (m & 15)) << 4); }

DG_DEV f32x4_t mfma_16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// One workgroup = 4 waves = 128 weight rows of one tile (expert e, rows [m0, m0 + 64) of
// its group); each wave owns 32 weight rows as two 16-row A operands.
// v_mfma_f32_16x16x32_bf16: lane l supplies row l % 16 of A (and column l % 16 of B) with
// 8 k values; the four lane groups g = l / 16 cover the 32 k of a step. Lane group g takes
// k [32j + 8g, +8) of the chunk in step j for both operands, so one weight load
// instruction reads 16 rows x 64 contiguous bytes (16 cache lines per KiB; the memory
// pipeline, not HBM, is what a weight stream with 32 lines per KiB saturates).
// Accumulator register i of lane l holds D[4(l / 16) + i][l % 16]: four consecutive
// weight rows of one activation row.
// Every memory load is unconditional, with row and k addresses clamped into the operands
// (rows past the group repeat its last row, k past K repeats the last 32 k), and loads of
// the chunk after the last read one fixed line: the compiler then counts the loads in
// flight exactly and keeps the next chunk's loads outstanding during the MFMAs. Clamped
// rows are never stored, and k steps past K are skipped (a wave-uniform test).
__global__ __launch_bounds__(256) void moe_expert_kernel(MoeGemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][MOE_TM * 256];
  const int NB = (a.N + 127) / 128;
  const int ti = blockIdx.x / NB, nb = blockIdx.x % NB;
  if (ti >= a.tiles[0]) return;
  const int tile = a.tiles[1 + ti], e = tile & 0xFFFF, m0 = (tile >> 16) * MOE_TM;
  const int o0 = a.off[e], mrows = min(MOE_TM, a.off[e + 1] - o0 - m0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int K = a.K, nch = (K + 127) / 128;
  const int n0 = nb * 128 + 32 * wave;
  const int nbop = (mrows + 15) >> 4;                // B operands (16 rows each) in use
  const u16 *wp[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
    wp[s] = a.W + ((int64_t)e * a.N + min(n0 + 16 * s + r16, a.N - 1)) * K + 8 * g;

  // activation staging: thread t moves 16-byte chunk (t & 15) of rows t/16 + 16q
  const u16 *xr[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int mm = m0 + min((tid >> 4) + 16 * q, mrows - 1);
    const int row = a.perm ? a.perm[o0 + mm] : o0 + mm;
    xr[q] = a.X + (int64_t)row * K;
  }
  auto xload = [&](int ch, u32x4_t *v) {
    const int k = min(ch * 128 + 8 * (tid & 15), K - 8);
    const bool real = ch < nch;
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = *(const u32x4_t *)(real ? xr[q] + k : a.X);
  };
  auto xstore = [&](int ch, const u32x4_t *v) {
#pragma unroll
    for (int q = 0; q < 4; ++q) *(u32x4_t *)(xs[ch & 1] + xslot((tid >> 4) + 16 * q, tid & 15)) = v[q];
  };
  // w[2j + s]: k step j, row half s
  auto wload = [&](int ch, u32x4_t *w) {
    const bool real = ch < nch;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int s = 0; s < 2; ++s)
        w[2 * j + s] = *(const u32x4_t *)(real ? wp[s] + min(ch * 128 + 32 * j, K - 32) : a.W);
  };

  f32x4_t acc[2][4] = {};
  auto compute = [&](int ch, const u32x4_t *w) {
    if (ch >= nch) return;
    const int nj = min(4, (K - ch * 128) >> 5);
    const uint8_t *xb = xs[ch & 1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < nj) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          if (b < nbop) {
            const u32x4_t bv = *(const u32x4_t *)(xb + xslot(16 * b + r16, 4 * j + g));
            acc[0][b] = mfma_16x16x32(w[2 * j], bv, acc[0][b]);
            acc[1][b] = mfma_16x16x32(w[2 * j + 1], bv, acc[1][b]);
          }
        }
      }
    }
  };

  // Chunk ch is computed from weight registers W[ch & 1] and LDS buffer ch & 1; step ch
  // first loads chunk ch + 1 (activations before weights, so waiting for the activations
  // leaves the weight loads in flight), then computes chunk ch, then stores the
  // activations of chunk ch + 1 into the other LDS buffer.
  u32x4_t W[2][8], X[4];
  xload(0, X);
  wload(0, W[0]);
  xstore(0, X);
  __syncthreads();
  for (int ch = 0; ch < nch; ch += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      xload(ch + u + 1, X);
      __builtin_amdgcn_sched_barrier(0);             // keep the issue order: activations first
      wload(ch + u + 1, W[u ^ 1]);
      __builtin_amdgcn_sched_barrier(0);
      compute(ch + u, W[u]);
      xstore(ch + u + 1, X);
      __syncthreads();
    }
  }
  if (n0 >= a.N) return;                             // wave past the output width

  // lane l, register i of acc[s][b]: D[n0 + 16s + 4g + i][m0 + 16b + r16]
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int mc = 16 * b + r16;
    if (b >= nbop || mc >= mrows) continue;
    u16 *yp = a.Y + (int64_t)(o0 + m0 + mc) * a.ldY + n0 + 4 * g;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float t = acc[s][b][i];
        if (a.gelu) t = 0.5f * t * (1.0f + erff(t * 0.70710678118654752f));
        v[i] = t;
      }
      uint2 o;
      o.x = pack_bf16x2(v[0], v[1]);
      o.y = pack_bf16x2(v[2], v[3]);
      *(uint2 *)(yp + 16 * s) = o;
    }
  }
}

__global__ __launch_bounds__(256) void moe_combine_kernel(const u16 *Yg, const u16 *Ys, const float *gate,
                                                          const int *pos, int K, int d, u16 *Y) {
  const int t = blockIdx.x;
  for (int j0 = threadIdx.x * 8; j0 < d; j0 += 256 * 8) {
    float acc[8] = {};
    for (int k = 0; k < K; ++k) {
      const float g = gate[(int64_t)t * K + k];
      const uint4 w = *(const uint4 *)(Yg + (int64_t)pos[(int64_t)t * K + k] * d + j0);
      const uint32_t *ww = (const uint32_t *)&w;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(g, bf16lo(ww[i]), acc[2 * i]);
        acc[2 * i + 1] = fmaf(g, bf16hi(ww[i]), acc[2 * i + 1]);
      }
    }
    const uint4 s = *(const uint4 *)(Ys + (int64_t)t * d + j0);
    const uint32_t *ss = (const uint32_t *)&s;
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i] + bf16lo(ss[i]), acc[2 * i + 1] + bf16hi(ss[i]));
    *(uint4 *)(Y + (int64_t)t * d + j0) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

}  // namespace

hipError_t dg_launch_moe_route(const float *logits, int C, int E, int K, int *sel, float *gate,
                               hipStream_t st) {
  hipLaunchKernelGGL(moe_route_kernel, dim3(C), dim3(256), 0, st, logits, E, K, sel, gate);
  return hipGetLastError();
}

hipError_t dg_launch_moe_group(const int *sel, int C, int K, int E, int *off, int *perm, int *pos,
                               int *nact, int *tiles, hipStream_t st) {
  hipLaunchKernelGGL(moe_group_kernel, dim3(1), dim3(256), (size_t)E * ((C + 31) / 32) * 4, st, sel, C,
                     K, E, off, perm, pos, nact, tiles);
  return hipGetLastError();
}

hipError_t dg_launch_moe_expert(const MoeGemmArgs &a, hipStream_t st) {
  if (a.N < 32 || a.N % 32 || a.K < 32 || a.K % 32 || a.max_tiles < 1) return hipErrorInvalidValue;
  const int NB = (a.N + 127) / 128;
  hipLaunchKernelGGL(moe_expert_kernel, dim3(a.max_tiles * NB), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t dg_launch_moe_combine(const u16 *Yg, const u16 *Ys, const float *gate, const int *pos,
                                 int C, int K, int d, u16 *Y, hipStream_t st) {
  hipLaunchKernelGGL(moe_combine_kernel, dim3(C), dim3(256), 0, st, Yg, Ys, gate, pos, K, d, Y);
  return hipGetLastError();
}
