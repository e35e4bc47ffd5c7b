// Small-M bf16 GEMM with fp32 accumulation: D[m][n] = sum_k X[m][k] W[n][k].
//
// Used for every dense projection of the step whose M is the canvas (C <= 1024):
// the Q/K/V projections of the denoiser input X = E[x] + z (the gather and the bf16
// rounding of the sum happen in the operand loader, so X never exists in memory),
// the attention output projection Wo, the two self-conditioning FFW layers (exact-erf
// GELU fused into the epilogue of the first) and the K/V projection of a committed
// block. Up to three weight segments share one launch; each segment has its own output
// address map out + m*sm + (n/seg)*sg + (n%seg)*se, which covers row-major outputs,
// the transposed canvas V, and the [Hkv][Pcap][hd] / [Hkv][hd][Pcap] cache layouts.
//
// Tiling: 256 threads = 4 waves in a 2 (n) x 2 (m) grid, block tile 64 n x 64 m,
// K in steps of 64 staged through LDS with a register prefetch of the next step.
// Weight rows are MFMA A operands, activation rows B operands (see dg_common.h).
#include "dg_common.h"

namespace {

constexpr int BN = 64, BM = 64, BK = 64, PITCH = BK + 8;

struct Prefetch {
  uint4 w[2];
  uint4 x[2];
  uint4 zx[2];
};

__device__ __forceinline__ void load_tile(const GemmArgs &a, const GemmSeg &sg, int nb0, int m0,
                                          int k0, int tid, Prefetch &pf) {
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int q = tid + 256 * it;
    const int row = q >> 3, col = (q & 7) * 8;
    const int n = nb0 + row, k = k0 + col;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (n < sg.N && k < a.K) v = *(const uint4 *)(sg.W + (int64_t)n * a.K + k);
    pf.w[it] = v;
    const int m = m0 + row;
    uint4 x = make_uint4(0, 0, 0, 0), zx = make_uint4(0, 0, 0, 0);
    if (m < a.M && k < a.K) {
      if (a.A) {
        x = *(const uint4 *)(a.A + (int64_t)m * a.K + k);
      } else {
        int t = a.tokens[m];
        if (t < 0 || t >= a.V) {
          if (k0 == 0 && col == 0) set_status(a.status, DGS_RANGE);
          t = -1;
        }
        if (t >= 0) x = *(const uint4 *)(a.E + (int64_t)t * a.K + k);
        if (a.z) zx = *(const uint4 *)(a.z + (int64_t)m * a.K + k);
      }
    }
    pf.x[it] = x;
    pf.zx[it] = zx;
  }
}

__device__ __forceinline__ void store_tile(const GemmArgs &a, u16 *Ws, u16 *Xs, int tid,
                                           const Prefetch &pf) {
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int q = tid + 256 * it;
    const int row = q >> 3, col = (q & 7) * 8;
    *(uint4 *)(Ws + row * PITCH + col) = pf.w[it];
    uint4 x = pf.x[it];
    if (!a.A && a.z) {
      // X = bf16(E[x] + z): the sum of two bf16 values in fp32, rounded once to bf16.
      const uint32_t *e = (const uint32_t *)&pf.x[it];
      const uint32_t *z = (const uint32_t *)&pf.zx[it];
      uint32_t o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        o[j] = pack_bf16x2(bf16lo(e[j]) + bf16lo(z[j]), bf16hi(e[j]) + bf16hi(z[j]));
      x = make_uint4(o[0], o[1], o[2], o[3]);
    }
    *(uint4 *)(Xs + row * PITCH + col) = x;
  }
}

__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) u16 Ws[BN * PITCH];
  __shared__ __attribute__((aligned(16))) u16 Xs[BM * PITCH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int h = lane >> 5, l32 = lane & 31;

  int si = 0;
  for (int s = 1; s < a.nseg; ++s)
    if ((int)blockIdx.x >= a.seg[s].nblk0) si = s;
  const GemmSeg &sg = a.seg[si];
  const int nb0 = ((int)blockIdx.x - sg.nblk0) * BN;
  const int m0 = blockIdx.y * BM;

  f32x16_t acc = {};
  Prefetch pf;
  load_tile(a, sg, nb0, m0, 0, tid, pf);
  for (int k0 = 0; k0 < a.K; k0 += BK) {
    __syncthreads();
    store_tile(a, Ws, Xs, tid, pf);
    __syncthreads();
    if (k0 + BK < a.K) load_tile(a, sg, nb0, m0, k0 + BK, tid, pf);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const u32x4_t af = *(const u32x4_t *)(Ws + (wn * 32 + l32) * PITCH + ks * 16 + 8 * h);
      const u32x4_t bf = *(const u32x4_t *)(Xs + (wm * 32 + l32) * PITCH + ks * 16 + 8 * h);
      acc = mfma_32x32x16(af, bf, acc);
    }
  }

  const int m = m0 + wm * 32 + l32;
  if (m >= sg.m_store) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int n = nb0 + wn * 32 + acc_row(r, h);
    if (n >= sg.N) continue;
    float v = acc[r];
    if (a.gelu) v = 0.5f * v * (1.0f + erff(v * 0.70710678118654752f));
    sg.out[(int64_t)m * sg.sm + (int64_t)(n / sg.seg) * sg.sg + (int64_t)(n % sg.seg) * sg.se] =
        f32_to_bf16(v);
  }
}

}  // namespace

hipError_t dg_launch_gemm(const GemmArgs &a0, hipStream_t st) {
  GemmArgs a = a0;
  int nblk = 0;
  int mmax = a.M;
  for (int s = 0; s < a.nseg; ++s) {
    a.seg[s].nblk0 = nblk;
    nblk += (a.seg[s].N + BN - 1) / BN;
    if (a.seg[s].m_store > mmax) mmax = a.seg[s].m_store;
  }
  dim3 grid(nblk, (mmax + BM - 1) / BM);
  hipLaunchKernelGGL(gemm_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}
