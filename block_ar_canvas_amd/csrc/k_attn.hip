// Bidirectional canvas attention over the static prefix KV cache.
//
// Method: in denoise mode every canvas query attends, with no mask, to all canvas
// tokens and to the prompt / finished-block KV cache (Google "DiffusionGemma
// explained", section "Architecture: incremental prefill and denoising"; tutorial
// chapter "DiffusionGemma", the per-phase attention masks: the current canvas uses
// full bidirectional attention and reads the cache). Attention is a softmax over a
// set of keys, so the key order is free: the kernel walks the canvas keys first, then
// the prefix, in tiles of 32 that never straddle the two segments.
//
// Work split (split-K / "flash decoding" over keys): a workgroup owns one KV head g,
// 256 query rows of that head's group (row = (head in group, canvas position)) and
// a contiguous range of key tiles. It streams K and V^T tiles HBM -> registers -> LDS
// (the next tile is prefetched into registers while the current one is consumed) and
// keeps an online softmax per query row in the log2 domain. Partial (O, max, sum) go
// to the workspace; attn_merge_kernel combines the parts in a fixed order.
//
// Orientation: S^T = K Q^T (keys are MFMA rows, loaded through perm_row so that the
// probabilities come out as ready B fragments), O^T = V^T P^T (V is stored transposed
// in the cache, so its A fragments are contiguous 16-byte LDS reads). Each lane owns
// one query row: its softmax statistics need only one cross-lane exchange (lane ^ 32).
#include "dg_common.h"

namespace {

constexpr int KT = DG_KT;

template <int HD>
struct AttnCfg {
  static constexpr int EROWS = HD < 32 ? 32 : HD;   // V^T rows padded to an MFMA tile
  static constexpr int ET = EROWS / 32;             // e-tiles of O^T
  static constexpr int KS = HD / 16;                // k-steps of S = K Q^T
  static constexpr int KPITCH = HD + 8;
  static constexpr int VPITCH = KT + 8;
  static constexpr int KCHUNKS = KT * HD / 8;       // 16-byte chunks per K tile
  static constexpr int VCHUNKS = HD * KT / 8;
};

template <int HD>
__global__ __launch_bounds__(256) void attn_split_kernel(AttnArgs a, int nq, int ntc,
                                                         int ntiles, int units) {
  using Cfg = AttnCfg<HD>;
  __shared__ __attribute__((aligned(16))) u16 Ks[KT * Cfg::KPITCH];
  __shared__ __attribute__((aligned(16))) u16 Vs[Cfg::EROWS * Cfg::VPITCH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;

  // Workgroups that read the same key range (same unit) land on the same XCD.
  const int b = blockIdx.x;
  int unit, qb;
  if ((units & 7) == 0) {
    const int xcd = b & 7, r = b >> 3;
    unit = xcd + 8 * (r / nq);
    qb = r % nq;
  } else {
    unit = b / nq;
    qb = b % nq;
  }
  const int g = unit / a.nsplit, split = unit % a.nsplit;
  const int G = a.Hq / a.Hkv;
  const int t0 = (int)((int64_t)split * ntiles / a.nsplit);
  const int t1 = (int)((int64_t)(split + 1) * ntiles / a.nsplit);

  // Zero the padded V^T rows once (head dims below one MFMA tile).
  if (Cfg::EROWS > HD) {
    for (int i = tid; i < (Cfg::EROWS - HD) * Cfg::VPITCH; i += 256) Vs[HD * Cfg::VPITCH + i] = 0;
  }

  // Query rows of this wave: two 32-row column tiles.
  int qrow_c[2], qrow_h[2];
  bool qrow_ok[2];
  u32x4_t qf[2][Cfg::KS];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int r = qb * 256 + wave * 64 + ct * 32 + l32;
    qrow_ok[ct] = r < G * a.C;
    const int hi = qrow_ok[ct] ? r / a.C : 0;
    qrow_c[ct] = qrow_ok[ct] ? r % a.C : 0;
    qrow_h[ct] = g * G + hi;
#pragma unroll
    for (int ks = 0; ks < Cfg::KS; ++ks) {
      u32x4_t v = {0, 0, 0, 0};
      if (qrow_ok[ct])
        v = *(const u32x4_t *)(a.Q + (int64_t)qrow_c[ct] * a.Hq * HD + qrow_h[ct] * HD +
                               ks * 16 + 8 * hh);
      qf[ct][ks] = v;
    }
  }

  f32x16_t O[2][Cfg::ET];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int et = 0; et < Cfg::ET; ++et) O[ct][et] = f32x16_t{};
  float mrun[2] = {-INFINITY, -INFINITY}, lrun[2] = {0.f, 0.f};

  // Register prefetch of one K tile and one V^T tile (at most 2 chunks each per thread).
  uint4 pk[2], pv[2];
  auto load = [&](int t) {
    const bool canvas = t < ntc;
    const int kbase = canvas ? t * KT : (t - ntc) * KT;
    const int64_t nvalid = canvas ? a.C : a.P;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int q = tid + 256 * it;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (q < Cfg::KCHUNKS) {
        const int kr = q / (HD / 8), col = (q % (HD / 8)) * 8;
        const int key = kbase + kr;
        if (key < nvalid) {
          const u16 *src = canvas ? a.Kc + (int64_t)key * a.Hkv * HD + g * HD + col
                                  : a.Kp + ((int64_t)g * a.Pcap + key) * HD + col;
          v = *(const uint4 *)src;
        }
      }
      pk[it] = v;
      uint4 w = make_uint4(0, 0, 0, 0);
      if (q < Cfg::VCHUNKS) {
        const int e = q / (KT / 8), col = (q % (KT / 8)) * 8;
        const int start = kbase + col;
        if (canvas) {
          w = *(const uint4 *)(a.Vct + ((int64_t)g * HD + e) * a.Cpad + start);
        } else if (start < a.P) {
          w = *(const uint4 *)(a.Vt + ((int64_t)g * HD + e) * a.Pcap + start);
          const int64_t nv = a.P - start;   // zero the tail beyond the cached length
          if (nv < 8) {
            uint32_t *ww = (uint32_t *)&w;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              if (2 * j >= nv) ww[j] = 0;
              else if (2 * j + 1 >= nv) ww[j] &= 0xFFFFu;
            }
          }
        }
      }
      pv[it] = w;
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int q = tid + 256 * it;
      if (q < Cfg::KCHUNKS) {
        const int kr = q / (HD / 8), col = (q % (HD / 8)) * 8;
        *(uint4 *)(Ks + kr * Cfg::KPITCH + col) = pk[it];
      }
      if (q < Cfg::VCHUNKS) {
        const int e = q / (KT / 8), col = (q % (KT / 8)) * 8;
        *(uint4 *)(Vs + e * Cfg::VPITCH + col) = pv[it];
      }
    }
  };

  if (t0 < t1) load(t0);
  for (int t = t0; t < t1; ++t) {
    __syncthreads();
    store();
    __syncthreads();
    if (t + 1 < t1) load(t + 1);

    const bool canvas = t < ntc;
    const int kbase = canvas ? t * KT : (t - ntc) * KT;
    const int64_t nvalid = canvas ? a.C : a.P;

    // S^T tile: 32 keys x 32 query rows per column tile.
    f32x16_t S[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
    for (int ks = 0; ks < Cfg::KS; ++ks) {
      const u32x4_t af = *(const u32x4_t *)(Ks + perm_row(l32) * Cfg::KPITCH + ks * 16 + 8 * hh);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) S[ct] = mfma_32x32x16(af, qf[ct][ks], S[ct]);
    }

    // Online softmax (log2 domain) per query row; probabilities become B fragments.
    u32x4_t pf[2][2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      float x[16];
      float mt = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kbase + acc_row_perm(r, hh);
        x[r] = key < nvalid ? S[ct][r] * a.scale_log2 : -INFINITY;
        mt = fmaxf(mt, x[r]);
      }
      mt = fmaxf(mt, wave_xor32(mt));
      const float mnew = fmaxf(mrun[ct], mt);
      const float alpha = exp2f(mrun[ct] - mnew);
      float ls = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x[r] = exp2f(x[r] - mnew);
        ls += x[r];
      }
      ls += wave_xor32(ls);
      lrun[ct] = lrun[ct] * alpha + ls;
      mrun[ct] = mnew;
#pragma unroll
      for (int et = 0; et < Cfg::ET; ++et) O[ct][et] *= alpha;
#pragma unroll
      for (int s = 0; s < 2; ++s)
        pf[ct][s] = u32x4_t{pack_bf16x2(x[8 * s + 0], x[8 * s + 1]), pack_bf16x2(x[8 * s + 2], x[8 * s + 3]),
                            pack_bf16x2(x[8 * s + 4], x[8 * s + 5]), pack_bf16x2(x[8 * s + 6], x[8 * s + 7])};
    }

    // O^T += V^T P^T
#pragma unroll
    for (int et = 0; et < Cfg::ET; ++et) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const u32x4_t af = *(const u32x4_t *)(Vs + (et * 32 + l32) * Cfg::VPITCH + 16 * s + 8 * hh);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) O[ct][et] = mfma_32x32x16(af, pf[ct][s], O[ct][et]);
      }
    }
  }

  // Partial results of this key range.
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    if (!qrow_ok[ct]) continue;
    const int64_t row = ((int64_t)split * a.Hq + qrow_h[ct]) * a.Cpad + qrow_c[ct];
    if (hh == 0) {
      a.pml[2 * row] = mrun[ct];
      a.pml[2 * row + 1] = lrun[ct];
    }
#pragma unroll
    for (int et = 0; et < Cfg::ET; ++et) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int e = et * 32 + acc_row(r, hh);
        if (e < HD) a.po[row * HD + e] = O[ct][et][r];
      }
    }
  }
}

// Log-sum-exp merge of the key-range partials, in split order.
template <int HD>
__global__ __launch_bounds__(128) void attn_merge_kernel(AttnArgs a) {
  const int h = blockIdx.x / a.C, c = blockIdx.x % a.C, e = threadIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s) {
    const int64_t row = ((int64_t)s * a.Hq + h) * a.Cpad + c;
    M = fmaxf(M, a.pml[2 * row]);
  }
  float L = 0.f, o = 0.f;
  for (int s = 0; s < a.nsplit; ++s) {
    const int64_t row = ((int64_t)s * a.Hq + h) * a.Cpad + c;
    const float w = exp2f(a.pml[2 * row] - M);
    L += a.pml[2 * row + 1] * w;
    if (e < HD) o += a.po[row * HD + e] * w;
  }
  if (e < HD) a.O[(int64_t)c * a.Hq * HD + h * HD + e] = f32_to_bf16(o / L);
}

template <int HD>
hipError_t launch(const AttnArgs &a, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  const int nq = (G * a.C + 255) / 256;
  const int ntc = a.Cpad / KT;
  const int ntiles = ntc + (int)((a.P + KT - 1) / KT);
  const int units = a.Hkv * a.nsplit;
  hipLaunchKernelGGL(attn_split_kernel<HD>, dim3(units * nq), dim3(256), 0, st, a, nq, ntc,
                     ntiles, units);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_merge_kernel<HD>, dim3(a.Hq * a.C), dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t dg_launch_attention(const AttnArgs &a, hipStream_t st) {
  switch (a.hd) {
    case 16: return launch<16>(a, st);
    case 32: return launch<32>(a, st);
    case 64: return launch<64>(a, st);
    case 128: return launch<128>(a, st);
    default: return hipErrorInvalidValue;
  }
}
