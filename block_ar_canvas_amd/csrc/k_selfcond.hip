// Self-conditioning product s = p0 E over the whole vocabulary.
//
// Method (DiffusionGemma Technical Report page, "Method steps" (3): z = FFW(p0 E);
// Google "DiffusionGemma explained", section "Self-conditioning": the step's
// probability matrix is multiplied by the token embedding table and the result is
// passed to the next step). The report's limitations single out this 262K-wide
// product as slow in plain framework code; here it is one split-K MFMA pass over E.
//
// selfcond_split_kernel computes s^T[j][c] = sum_v E[v][j] p0[c][v] for a 128-wide
// slice of the model width j, up to 256 canvas columns c and one contiguous range of
// vocabulary tiles. Operands:
//   B = p0^T: the bf16 p~ fragments written by the logits epilogue, already in MFMA
//       B-fragment order. Each 16-byte fragment holds 8 probabilities of one column c
//       and one 128-row tile t; it is scaled by exp(m_t - m_c) / Z_c (the finalize
//       factor) and rounded back to bf16 while it is copied into LDS.
//   A = E^T: E rows (vocabulary-major, j contiguous) are staged in LDS as loaded; each
//       lane gathers its 8 vocabulary values of one j column (the transpose happens in
//       the LDS read, E is never copied).
// Partial sums (one per vocabulary range) are reduced in range order by
// selfcond_reduce_kernel, which also rounds s to bf16 for the FFW.
#include "dg_common.h"

namespace {

constexpr int BJ = 128, BC = 256, BKV = 64, EPITCH = BJ + 8;

__global__ __launch_bounds__(256) void selfcond_split_kernel(SelfcondArgs a, int nj) {
  __shared__ __attribute__((aligned(16))) u16 Es[BKV * EPITCH];
  __shared__ __attribute__((aligned(16))) u16 Ps[8 * (BKV / 16) * 64 * 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wj = wave & 1, wc = wave >> 1;
  const int hh = lane >> 5, l32 = lane & 31;

  // blockIdx.x -> (split, j-slice); the j-slices of one split share the p~ range and
  // are kept on one XCD when the split count allows it.
  const int b = blockIdx.x;
  const int units = a.nsc;
  int split, jb;
  if ((units & 7) == 0) {
    const int xcd = b & 7, r = b >> 3;
    split = xcd + 8 * (r / nj);
    jb = r % nj;
  } else {
    split = b / nj;
    jb = b % nj;
  }
  const int j0 = jb * BJ;
  const int cb = blockIdx.y * BC;
  const int ct0 = cb / 32;                        // first canvas tile of this block
  const int nct = a.Cpad / 32;
  const int VS = a.T * (DG_BV / 16);
  const int tile0 = (int)((int64_t)split * a.T / a.nsc);
  const int tile1 = (int)((int64_t)(split + 1) * a.T / a.nsc);
  const int vbeg = tile0 * DG_BV, vend = tile1 * DG_BV;

  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};

  uint4 pe[4], pp[8];
  float pf[8];
  auto load = [&](int v0) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int q = tid + 256 * it;
      const int row = q >> 4, col = (q & 15) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (v0 + row < a.V && j0 + col < a.d) v = *(const uint4 *)(a.E + (int64_t)(v0 + row) * a.d + j0 + col);
      pe[it] = v;
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int q = tid + 256 * it;             // chunk = (canvas tile, vocab step, lane)
      const int ctl = q >> 8, vs = (q >> 6) & 3, ln = q & 63;
      const int ctile = ct0 + ctl;
      uint4 v = make_uint4(0, 0, 0, 0);
      float f = 0.f;
      if (ctile < nct) {
        const int vstep = v0 / 16 + vs;
        v = *(const uint4 *)(a.ptilde + (((int64_t)ctile * VS + vstep) * 64 + ln) * 8);
        const int c = ctile * 32 + (ln & 31);
        if (c < a.C) f = a.fac[(int64_t)(vstep / (DG_BV / 16)) * a.Cpad + c];
      }
      pp[it] = v;
      pf[it] = f;
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int q = tid + 256 * it;
      *(uint4 *)(Es + (q >> 4) * EPITCH + (q & 15) * 8) = pe[it];
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int q = tid + 256 * it;
      const uint32_t *w = (const uint32_t *)&pp[it];
      const float f = pf[it];
      const uint4 o = make_uint4(pack_bf16x2(bf16lo(w[0]) * f, bf16hi(w[0]) * f),
                                 pack_bf16x2(bf16lo(w[1]) * f, bf16hi(w[1]) * f),
                                 pack_bf16x2(bf16lo(w[2]) * f, bf16hi(w[2]) * f),
                                 pack_bf16x2(bf16lo(w[3]) * f, bf16hi(w[3]) * f));
      *(uint4 *)(Ps + q * 8) = o;
    }
  };

  if (vbeg < vend) load(vbeg);
  for (int v0 = vbeg; v0 < vend; v0 += BKV) {
    __syncthreads();
    store();
    __syncthreads();
    if (v0 + BKV < vend) load(v0 + BKV);
#pragma unroll
    for (int ks = 0; ks < BKV / 16; ++ks) {
      u32x4_t af[2];
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        const u16 *src = Es + (ks * 16 + 8 * hh) * EPITCH + wj * 64 + jt * 32 + l32;
        uint32_t w[4];
#pragma unroll
        for (int p = 0; p < 4; ++p)
          w[p] = (uint32_t)src[(2 * p) * EPITCH] | ((uint32_t)src[(2 * p + 1) * EPITCH] << 16);
        af[jt] = u32x4_t{w[0], w[1], w[2], w[3]};
      }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        if (ct0 + wc * 4 + ct >= nct) continue;   // wave-uniform
        const u32x4_t bf = *(const u32x4_t *)(Ps + (((wc * 4 + ct) * 4 + ks) * 64 + lane) * 8);
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) acc[jt][ct] = mfma_32x32x16(af[jt], bf, acc[jt][ct]);
      }
    }
  }

  // Partial s for this vocabulary range: ps[split][c][j], 4 consecutive j per store.
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const int c = cb + wc * 128 + ct * 32 + l32;
    if (c >= a.Cpad) continue;
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = j0 + wj * 64 + jt * 32 + 8 * q + 4 * hh;
        if (j >= a.d) continue;
        const float4 v = make_float4(acc[jt][ct][4 * q], acc[jt][ct][4 * q + 1],
                                     acc[jt][ct][4 * q + 2], acc[jt][ct][4 * q + 3]);
        *(float4 *)(a.ps + ((int64_t)split * a.Cpad + c) * a.d + j) = v;
      }
    }
  }
}

__global__ __launch_bounds__(256) void selfcond_reduce_kernel(SelfcondArgs a) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;   // element of [Cpad][d]
  const int64_t n = (int64_t)a.Cpad * a.d;
  if (i >= n) return;
  const int c = (int)(i / a.d);
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int p = 0; p < a.nsc; ++p) {
    const float4 v = *(const float4 *)(a.ps + (int64_t)p * n + i);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  if (c >= a.C) s = make_float4(0.f, 0.f, 0.f, 0.f);
  const uint2 o = make_uint2(pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w));
  *(uint2 *)(a.s + i) = o;
}

}  // namespace

hipError_t dg_launch_selfcond(const SelfcondArgs &a, hipStream_t st) {
  const int nj = (a.d + BJ - 1) / BJ;
  hipLaunchKernelGGL(selfcond_split_kernel, dim3(nj * a.nsc, (a.Cpad + BC - 1) / BC), dim3(256), 0,
                     st, a, nj);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n4 = (int64_t)a.Cpad * a.d / 4;
  hipLaunchKernelGGL(selfcond_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}
