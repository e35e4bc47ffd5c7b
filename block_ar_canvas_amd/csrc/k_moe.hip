// Canvas MoE FFN: router top-K, token grouping by expert, combine.
//
// Method (DiffusionGemma Technical Report page, "Prerequisites", mixture of experts: each
// token uses 8 of 128 experts plus one shared expert, and a 256-token canvas touches
// about 84 distinct experts where one token touches 8; "Text diffusion models" survey,
// section 13: router top-k, expert GEMM, token permutation). The expert GEMMs are the
// grouped mode of gemm_kernel (one workgroup per expert x row block x column block,
// weights streamed once per expert); the kernels here route, group and combine.
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
// moe_expert_kernel: Y[g_off[e] + m] = act(X_e[m] . W[e]^T) for the grouped rows of
//   expert e. The weights are read once per tile, straight from memory into the MFMA A
//   operand (each wave owns 32 weight rows); the tile's activation rows (at most 64) are
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

// One workgroup = 4 waves = 128 weight rows of one tile (expert e, rows [m0, m0 + 64) of
// its group). Lane (c, h) of a wave: A rows n0 + c, B rows m0 + c (and m0 + 32 + c).
// MFMA j of a 128-deep chunk covers k [16j, 16j + 16) of it; lane half h holds 8 of them.
// Every memory load is unconditional, with row and k addresses clamped into the operands
// (rows past the group repeat its last row, k past K repeats the last 16 k): the
// compiler then counts the loads in flight exactly and keeps the next chunk's loads
// outstanding during the MFMAs. Clamped rows are never stored, and the MFMAs of k steps
// past K are skipped (a wave-uniform test), so the repeats never reach a result.
__global__ __launch_bounds__(256) void moe_expert_kernel(MoeGemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][MOE_TM * 256];
  const int NB = (a.N + 127) / 128;
  const int ti = blockIdx.x / NB, nb = blockIdx.x % NB;
  if (ti >= a.tiles[0]) return;
  const int tile = a.tiles[1 + ti], e = tile & 0xFFFF, m0 = (tile >> 16) * MOE_TM;
  const int o0 = a.off[e], mrows = min(MOE_TM, a.off[e + 1] - o0 - m0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, h = lane >> 5;
  const int K = a.K, nch = (K + 127) / 128;
  const int n0 = nb * 128 + 32 * wave;
  const bool upper = mrows > 32;
  const u16 *wp = a.W + ((int64_t)e * a.N + min(n0 + c, a.N - 1)) * K + 8 * h;

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
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = *(const u32x4_t *)(xr[q] + k);
  };
  auto xstore = [&](int ch, const u32x4_t *v) {
#pragma unroll
    for (int q = 0; q < 4; ++q) *(u32x4_t *)(xs[ch & 1] + xslot((tid >> 4) + 16 * q, tid & 15)) = v[q];
  };
  auto wload = [&](int ch, u32x4_t *w) {
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = *(const u32x4_t *)(wp + min(ch * 128 + 16 * j, K - 16));
  };

  f32x16_t acc0 = {}, acc1 = {};
  auto compute = [&](int ch, const u32x4_t *w) {
    const int nj = min(8, (K - ch * 128) >> 4);
    const uint8_t *xb = xs[ch & 1];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < nj) {
        const u32x4_t b0 = *(const u32x4_t *)(xb + xslot(c, 2 * j + h));
        acc0 = mfma_32x32x16(w[j], b0, acc0);
        if (upper) {
          const u32x4_t b1 = *(const u32x4_t *)(xb + xslot(32 + c, 2 * j + h));
          acc1 = mfma_32x32x16(w[j], b1, acc1);
        }
      }
    }
  };

  u32x4_t wa[8], wb[8], xv[4];
  xload(0, xv);
  wload(0, wa);
  xstore(0, xv);
  __syncthreads();
  // chunk ch (not the last): its weights are in registers and its activations in LDS
  // buffer ch & 1. The next chunk's activations are loaded before its weights, so
  // waiting for them leaves the weight loads in flight.
  auto step = [&](int ch, const u32x4_t *cur, u32x4_t *nxt) {
    xload(ch + 1, xv);
    wload(ch + 1, nxt);
    compute(ch, cur);
    xstore(ch + 1, xv);
    __syncthreads();
  };
  int ch = 0;
  for (; ch + 2 < nch; ch += 2) {
    step(ch, wa, wb);
    step(ch + 1, wb, wa);
  }
  if (ch + 2 == nch) {
    step(ch, wa, wb);
    compute(ch + 1, wb);
  } else {
    compute(ch, wa);
  }
  if (n0 >= a.N) return;                             // wave past the output width

  // lane (c, h), register r: D[n0 + acc_row(r, h)][m0 + c]; four consecutive n per store
  auto store = [&](const f32x16_t &acc, int mc) {
    if (mc >= mrows) return;
    u16 *yp = a.Y + (int64_t)(o0 + m0 + mc) * a.ldY + n0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float s = acc[4 * g + i];
        if (a.gelu) s = 0.5f * s * (1.0f + erff(s * 0.70710678118654752f));
        v[i] = s;
      }
      uint2 o;
      o.x = pack_bf16x2(v[0], v[1]);
      o.y = pack_bf16x2(v[2], v[3]);
      *(uint2 *)(yp + 8 * g + 4 * h) = o;
    }
  };
  store(acc0, c);
  if (upper) store(acc1, 32 + c);
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
