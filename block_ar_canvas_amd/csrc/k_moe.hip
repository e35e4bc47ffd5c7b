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
                                                        int *perm, int *pos, int *nact) {
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
  int c = 0;
  if (tid < E)
    for (int w = 0; w < W; ++w) c += __popc(mask[tid * W + w]);
  loff[tid] = c;
  __syncthreads();
  if (tid == 0) {                                    // at most 256 experts: a short walk
    int run = 0, na = 0;
    for (int e = 0; e < E; ++e) {
      const int ce = loff[e];
      loff[e] = run;
      off[e] = run;
      run += ce;
      na += ce > 0 ? 1 : 0;
    }
    off[E] = run;
    if (nact) nact[0] = na;
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
                               int *nact, hipStream_t st) {
  hipLaunchKernelGGL(moe_group_kernel, dim3(1), dim3(256), (size_t)E * ((C + 31) / 32) * 4, st, sel, C,
                     K, E, off, perm, pos, nact);
  return hipGetLastError();
}

hipError_t dg_launch_moe_combine(const u16 *Yg, const u16 *Ys, const float *gate, const int *pos,
                                 int C, int K, int d, u16 *Y, hipStream_t st) {
  hipLaunchKernelGGL(moe_combine_kernel, dim3(C), dim3(256), 0, st, Yg, Ys, gate, pos, K, d, Y);
  return hipGetLastError();
}
