// Sampler head: lm_head logits fused with the tempered softmax statistics.
//
// Method (DiffusionGemma Technical Report page, "Method steps" (3)): the decoder's
// logits are divided by the annealed temperature and soft-maxed into p0; positions
// are then ranked by the entropy of p0, and x0 = argmax p0 is what acceptance keeps.
// The text-diffusion survey (section 13) and the report's limitations note that the
// vocabulary projection over every canvas position is a bandwidth and temporary-tensor
// hog; here the C x V logits never reach memory in fp32.
//
// logits_tile_kernel: one workgroup = 128 vocabulary rows x up to 256 canvas columns,
// K (model width) in steps of 64 through LDS with a register prefetch. E rows are the
// MFMA A operand (loaded through perm_row), H rows the B operand, so each lane owns a
// canvas column and its share of the tile's 128 logits. The epilogue, per column:
//   u = logit / tau, m_t = max u, a_t = argmax (lowest id), Z_t = sum exp(u - m_t),
//   S_t = sum exp(u - m_t) (u - m_t),
// and stores p~ = bf16(exp(u - m_t)) in the exact MFMA-fragment order dg_selfcond
// consumes (no re-layout), plus (m_t, Z_t, S_t, a_t) per (tile, column).
//
// row_finalize_kernel: per canvas column, merges the tile statistics in tile order:
//   m = max m_t, Z = sum Z_t e^(m_t - m), S = sum (S_t + Z_t (m_t - m)) e^(m_t - m),
//   entropy = ln Z - S / Z  (= -sum p ln p, both terms >= 0: no cancellation),
// argmax from the first tile reaching m, and the per-tile scale e^(m_t - m) / Z that
// turns p~ into p0 for the self-conditioning product.
#include <float.h>

#include "dg_common.h"

namespace {

constexpr int BV = DG_BV, BC = 256, BK = 64, PITCH = BK + 8;
constexpr float LOG2E = 1.4426950408889634f;

DG_DEV bool better(float u, int v, float best, int bi) {
  return u > best || (u == best && v < bi);
}

__global__ __launch_bounds__(256) void logits_tile_kernel(LogitsArgs a) {
  __shared__ __attribute__((aligned(16))) u16 Es[BV * PITCH];
  __shared__ __attribute__((aligned(16))) u16 Hs[BC * PITCH];
  __shared__ float red_m[2][BC];
  __shared__ int red_i[2][BC];
  __shared__ float red_z[2][BC];
  __shared__ float red_s[2][BC];
  __shared__ int red_bad[2][BC];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = wave & 1, wc = wave >> 1;
  const int hh = lane >> 5, l32 = lane & 31;
  const int vt = blockIdx.x;
  const int v0 = vt * BV;
  const int cb = blockIdx.y * BC;

  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};

  uint4 pe[4], ph[8];
  auto load = [&](int k0) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int q = tid + 256 * it;
      const int row = q >> 3, col = (q & 7) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (v0 + row < a.V && k0 + col < a.d) v = *(const uint4 *)(a.E + (int64_t)(v0 + row) * a.d + k0 + col);
      pe[it] = v;
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int q = tid + 256 * it;
      const int row = q >> 3, col = (q & 7) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (cb + row < a.C && k0 + col < a.d) v = *(const uint4 *)(a.H + (int64_t)(cb + row) * a.d + k0 + col);
      ph[it] = v;
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int q = tid + 256 * it;
      *(uint4 *)(Es + (q >> 3) * PITCH + (q & 7) * 8) = pe[it];
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int q = tid + 256 * it;
      *(uint4 *)(Hs + (q >> 3) * PITCH + (q & 7) * 8) = ph[it];
    }
  };

  const int wcol0 = cb + wc * 128;   // first canvas column of this wave
  load(0);
  for (int k0 = 0; k0 < a.d; k0 += BK) {
    __syncthreads();
    store();
    __syncthreads();
    if (k0 + BK < a.d) load(k0 + BK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      u32x4_t af[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        af[mt] = *(const u32x4_t *)(Es + (wv * 64 + mt * 32 + perm_row(l32)) * PITCH + ks * 16 + 8 * hh);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        if (wcol0 + nt * 32 >= a.C) continue;   // wave-uniform: columns past the canvas
        const u32x4_t bf = *(const u32x4_t *)(Hs + (wc * 128 + nt * 32 + l32) * PITCH + ks * 16 + 8 * hh);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) acc[mt][nt] = mfma_32x32x16(af[mt], bf, acc[mt][nt]);
      }
    }
  }

  // ---------------- epilogue, phase 1: tile max / argmax per column
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int lc = wc * 128 + nt * 32 + l32;
    float best = -INFINITY;
    int bi = 0x7FFFFFFF, bad = 0;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int v = v0 + wv * 64 + mt * 32 + acc_row_perm(r, hh);
        float u = acc[mt][nt][r] * a.inv_tau;
        if (v < a.V) {
          bad |= !(fabsf(u) <= FLT_MAX);
          if (better(u, v, best, bi)) { best = u; bi = v; }
        } else {
          u = -INFINITY;
        }
        acc[mt][nt][r] = u;
      }
    }
    const float ob = wave_xor32(best);
    const int oi = wave_xor32(bi);
    if (better(ob, oi, best, bi)) { best = ob; bi = oi; }
    bad |= wave_xor32(bad);
    if (hh == 0) {
      red_m[wv][lc] = best;
      red_i[wv][lc] = bi;
      red_bad[wv][lc] = bad;
    }
  }
  __syncthreads();

  // ---------------- phase 2: exp, Z_t, S_t, and p~ fragments
  const int VS = a.T * (BV / 16);            // 16-row vocabulary steps in p~
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int lc = wc * 128 + nt * 32 + l32;
    float m = red_m[0][lc];
    if (red_m[1][lc] > m) m = red_m[1][lc];
    float Z = 0.f, S = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float du = acc[mt][nt][r] - m;
        const float e = exp2f(du * LOG2E);
        Z += e;
        S += (e > 0.f) ? e * du : 0.f;
        acc[mt][nt][r] = e;
      }
    }
    Z += wave_xor32(Z);
    S += wave_xor32(S);
    if (hh == 0) {
      red_z[wv][lc] = Z;
      red_s[wv][lc] = S;
    }
    const int ctile = (cb + wc * 128 + nt * 32) / 32;
    if (ctile * 32 < a.Cpad) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int vstep = (v0 + wv * 64 + mt * 32) / 16 + s;
          const f32x16_t &e = acc[mt][nt];
          const uint4 w = make_uint4(pack_bf16x2(e[8 * s + 0], e[8 * s + 1]), pack_bf16x2(e[8 * s + 2], e[8 * s + 3]),
                                     pack_bf16x2(e[8 * s + 4], e[8 * s + 5]), pack_bf16x2(e[8 * s + 6], e[8 * s + 7]));
          *(uint4 *)(a.ptilde + (((int64_t)ctile * VS + vstep) * 64 + lane) * 8) = w;
        }
      }
    }
  }
  __syncthreads();

  // ---------------- phase 3: tile statistics (one writer per column)
  if (wv == 0 && hh == 0) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int lc = wc * 128 + nt * 32 + l32;
      const int c = cb + lc;
      if (c >= a.Cpad) continue;
      float m = red_m[0][lc];
      int ai = red_i[0][lc];
      if (better(red_m[1][lc], red_i[1][lc], m, ai)) { m = red_m[1][lc]; ai = red_i[1][lc]; }
      const bool bad = red_bad[0][lc] | red_bad[1][lc];
      const int64_t o = (int64_t)vt * a.Cpad + c;
      a.tmax[o] = bad ? __builtin_nanf("") : m;
      a.tsum[o] = red_z[0][lc] + red_z[1][lc];
      a.tent[o] = red_s[0][lc] + red_s[1][lc];
      a.targ[o] = ai;
    }
  }
}

// One workgroup per canvas column; tile order is fixed, so the result is deterministic.
__global__ __launch_bounds__(256) void row_finalize_kernel(LogitsArgs a) {
  __shared__ float sm[256];
  __shared__ int si[256];
  __shared__ float sz[256], ss[256];
  __shared__ int sbad[256];
  const int c = blockIdx.x, tid = threadIdx.x;

  float m = -INFINITY;
  int tb = 0x7FFFFFFF, bad = 0;
  for (int t = tid; t < a.T; t += 256) {
    const float mt = a.tmax[(int64_t)t * a.Cpad + c];
    if (mt != mt) bad = 1;
    else if (mt > m) { m = mt; tb = t; }
  }
  sm[tid] = m; si[tid] = tb; sbad[tid] = bad;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) {
      const float m2 = sm[tid + w];
      const int t2 = si[tid + w];
      if (m2 > sm[tid] || (m2 == sm[tid] && t2 < si[tid])) { sm[tid] = m2; si[tid] = t2; }
      sbad[tid] |= sbad[tid + w];
    }
    __syncthreads();
  }
  m = sm[0];
  tb = si[0];
  bad = sbad[0];
  __syncthreads();

  float Z = 0.f, S = 0.f;
  for (int t = tid; t < a.T; t += 256) {
    const int64_t o = (int64_t)t * a.Cpad + c;
    const float dm = a.tmax[o] - m;
    const float w = expf(dm);
    Z += a.tsum[o] * w;
    S += (a.tent[o] + a.tsum[o] * dm) * w;
  }
  sz[tid] = Z; ss[tid] = S;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) { sz[tid] += sz[tid + w]; ss[tid] += ss[tid + w]; }
    __syncthreads();
  }
  Z = sz[0];
  S = ss[0];
  const float invZ = 1.0f / Z;
  for (int t = tid; t < a.T; t += 256) {
    const int64_t o = (int64_t)t * a.Cpad + c;
    a.fac[o] = bad ? 0.f : expf(a.tmax[o] - m) * invZ;
  }
  if (tid == 0) {
    float ent = logf(Z) - S / Z;
    ent = ent > 0.f ? ent : 0.f;
    if (bad || !(ent == ent)) {
      ent = __builtin_nanf("");
      set_status(a.status, DGS_NONFINITE);
    }
    a.entropy[c] = ent;
    a.argmax[c] = bad ? 0 : a.targ[(int64_t)tb * a.Cpad + c];
  }
}

}  // namespace

hipError_t dg_launch_logits(const LogitsArgs &a, hipStream_t st) {
  hipLaunchKernelGGL(logits_tile_kernel, dim3(a.T, (a.Cpad + BC - 1) / BC), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(row_finalize_kernel, dim3(a.C), dim3(256), 0, st, a);
  return hipGetLastError();
}
