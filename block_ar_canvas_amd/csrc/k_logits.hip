// Sampler head: lm_head logits fused with the tempered softmax statistics.
//
// Method (DiffusionGemma Technical Report page, "Method steps" (3)): the decoder's
// logits are divided by the annealed temperature and soft-maxed into p0; positions
// are then ranked by the entropy of p0, and x0 = argmax p0 is what acceptance keeps.
// The text-diffusion survey (section 13) and the report's limitations note that the
// vocabulary projection over every canvas position is a bandwidth and temporary-tensor
// hog; here the C x V logits never reach memory in fp32.
//
// logits_tile_kernel: one workgroup = 256 vocabulary rows x up to 256 canvas columns,
// the model width streamed through LDS rings of direct global -> LDS copies. E rows
// are the MFMA A operand (loaded through perm_row), H rows the B operand, so each lane
// owns a canvas column and its share of the tile's 256 logits. The epilogue works in
// log2 units x = logit * log2(e) / tau; per column it finds the tile max m_t and argmax
// a_t (lowest id), the reference rho_t = ceil(m_t) (an integer), and
//   Z_t = sum 2^(x - rho_t),   S_t = ln2 * sum 2^(x - rho_t) (x - rho_t)   (nats),
// and stores p~ = bf16(2^(x - rho_t)) in the exact MFMA-fragment order dg_selfcond
// consumes. Because every reference is an integer in log2 units, moving p~ from one
// tile's reference to another's is an exact power-of-two scale.
//
// row_finalize_kernel: per canvas column, merges the tile statistics in tile order with
// the column reference R = max rho_t:
//   Z = sum Z_t 2^(rho_t - R),  S = sum 2^(rho_t - R) (S_t + Z_t (rho_t - R) ln2),
//   entropy = ln Z - S / Z  (= -sum p ln p, both terms >= 0: no cancellation),
// and the argmax from the first tile reaching the largest m_t. It keeps R and Z per
// column: p0 = p~ * 2^(rho_t - R) / Z, which the self-conditioning product applies
// as exact power-of-two shifts plus one scale per column.
#include <float.h>

#include "dg_common.h"

namespace {

// Workgroup tile 256 vocabulary rows x BCT canvas columns (BCT = 256, or 128 when the
// vocabulary tiles alone would leave CUs idle), 8 waves (4 along the vocabulary x 2
// along the canvas), each wave 64 x BCT/2 = 2 x BCT/64 MFMA tiles (up to 128
// accumulators, two waves per SIMD so one wave's LDS-read latency hides behind the
// other's MFMAs). The model width is consumed in steps of BK = 64 through LDS rings
// filled by direct global -> LDS copies: E (streamed from HBM) has 3 stages, so two are
// in flight while one is consumed; H (L2-resident, re-read by every workgroup) has 2.
// Each copy instruction moves 8 rows x 128 contiguous bytes (one full cache line per 8
// lanes). LDS rows are 128 bytes with XOR-swizzled 16-byte chunks (see swz), so
// fragment reads are free of bank conflicts. E rows are stored in perm_row order within
// each 32-row tile, so fragment reads are plain row reads.
constexpr int BV = DG_BV, BK = 64, NSE = 3, NSH = 2;
constexpr int TILE = 256 * 128;                  // bytes of one 256-row x 64-k E stage
template <int BCT>
constexpr int smem_bytes() { return NSE * TILE + NSH * BCT * 128; }   // 160 or 128 KiB
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

DG_DEV bool better(float u, int v, float best, int bi) {
  return u > best || (u == best && v < bi);
}

// Byte offset of logical 16-byte chunk c (0..7) of LDS row R. A 128-byte row covers
// half of the 64 LDS banks, so rows alternate bank halves; XOR-ing the chunk with
// (R >> 1) & 7 gives the 16 rows read by a 16-lane group 16 distinct 16-byte slots.
DG_DEV int swz(int R, int c) { return R * 128 + ((c ^ ((R >> 1) & 7)) << 4); }

// HALF_TAIL: d is an odd multiple of 32, so the last K chunk holds 32 valid columns.
template <bool HALF_TAIL, int BCT>
__global__ __launch_bounds__(512) void logits_tile_kernel(LogitsArgs a) {
  static_assert(BCT == 128 || BCT == 256, "canvas block");
  constexpr int BC = BCT, NTW = BCT / 64;          // MFMA tiles per wave along the canvas
  constexpr int HC = BCT / 64;                     // H copy instructions per wave and stage
  constexpr int HT = BCT * 128;                    // bytes of one H stage
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  // epilogue scratch aliases the stage rings once the main loop is done
  float(*red_m)[BC] = (float(*)[BC])(smem);
  int(*red_i)[BC] = (int(*)[BC])(smem + 4 * BC * 4);
  float(*red_z)[BC] = (float(*)[BC])(smem + 8 * BC * 4);
  float(*red_s)[BC] = (float(*)[BC])(smem + 12 * BC * 4);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wv = wave & 3, wc = wave >> 2;
  const int hh = lane >> 5, l32 = lane & 31;
  // Workgroup -> (vocabulary tile, canvas block). With more than one canvas block (a
  // batch of canvases), the blocks of one tile run back to back on one XCD (workgroups
  // b, b + 8, ... share an XCD), so all but the first read the tile's E rows from that
  // XCD's L2 while the first streams them from HBM.
  const int ncb = (a.Cpad + BC - 1) / BC;
  int vt, cbk;
  if (ncb > 1 && (a.T & 7) == 0) {
    const int q = blockIdx.x >> 3;
    cbk = q % ncb;
    vt = (q / ncb) * 8 + (blockIdx.x & 7);
  } else {
    vt = blockIdx.x / ncb;
    cbk = blockIdx.x % ncb;
  }
  // Dispatch order: when the vocabulary tiles split evenly into the self-conditioning
  // splits, the t-th tile in dispatch order is tile L-1-t/nsc of split t%nsc (L tiles
  // per split). The self-conditioning pass walks every split from its first tile to its
  // last, so the first workgroups here read the E rows it read last, which may still be
  // in the memory-side cache (measured: about 3% off this kernel at V = 262144).
  if (a.nsc > 0 && a.T % a.nsc == 0) {
    const int L = a.T / a.nsc;
    vt = (vt % a.nsc) * L + (L - 1 - vt / a.nsc);
  }
  const int v0 = vt * BV;
  const int cb = cbk * BC;

  // Copy duties per stage: rows [32*wave, +32) of E and [BCT/8*wave, +BCT/8) of H, in
  // copy instructions of 8 rows each. Lane l of instruction j fills LDS row
  // R = base + 8*j + l/8 at chunk slot l%8, i.e. logical chunk (l%8) ^ ((R>>1)&7).
  const u16 *ge[4], *gh[HC];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int R = 32 * wave + 8 * j + (lane >> 3);
    const int c = (lane & 7) ^ ((R >> 1) & 7);
    int er = v0 + (R & ~31) + perm_row(R & 31);
    er = er < a.V ? er : a.V - 1;                    // clamp: masked in the epilogue
    ge[j] = a.E + (int64_t)er * a.d + c * 8;
  }
#pragma unroll
  for (int j = 0; j < HC; ++j) {
    const int R = (BCT / 8) * wave + 8 * j + (lane >> 3);
    const int c = (lane & 7) ^ ((R >> 1) & 7);
    int hr = cb + R;
    hr = hr < a.C ? hr : a.C - 1;                    // clamp: columns never stored
    gh[j] = a.H + (int64_t)hr * a.d + c * 8;
  }
  const uint32_t sbase = lds_addr(smem);

  // K order: workgroups start at different chunks (rotation by the tile index) so the
  // GPU's concurrent copies spread over the address space. With HALF_TAIL the partial
  // chunk comes last; its upper four 16-byte chunks are copied from the lower four of
  // the same row (never past the row end) and the k-steps reading them are skipped.
  const int KI = (a.d + BK - 1) / BK;
  const int KF = a.d / BK;
  const int rot = KF > 0 ? vt % KF : 0;
  auto kcol = [&](int it) { return (it < KF ? (it + rot) % KF : it) * BK; };
  // Copies of one stage: NJ instructions of 8 rows from rows `row0` of the stage.
  auto issue = [&](int it, const u16 *const *g, int nj, int row0, uint32_t st) {
    const int k = kcol(it);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j >= nj) break;
      int kk = k;
      if (HALF_TAIL && it == KI - 1) {
        const int R = row0 + 8 * j + (lane >> 3);
        const int c = (lane & 7) ^ ((R >> 1) & 7);   // logical chunk of this copy lane
        kk = k - (c >= 4 ? 32 : 0);
      }
      dma16(g[j] + kk, st + (uint32_t)(row0 * 128 + j * 1024));
    }
  };
  auto issue_e = [&](int it) { issue(it, ge, 4, 32 * wave, sbase + (uint32_t)(it % NSE) * TILE); };
  auto issue_h = [&](int it) {
    issue(it, gh, HC, (BCT / 8) * wave, sbase + (uint32_t)(NSE * TILE + (it % NSH) * HT));
  };

  f32x16_t acc[2][NTW];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[i][j] = f32x16_t{};

  auto compute = [&](int it, int nks) {
    const char *se = smem + (it % NSE) * TILE;
    const char *sh = smem + NSE * TILE + (it % NSH) * HT;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      if (ks >= nks) break;
      u32x4_t af[2], bf[NTW];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        af[mt] = *(const u32x4_t *)(se + swz(wv * 64 + mt * 32 + l32, 2 * ks + hh));
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
        bf[nt] = *(const u32x4_t *)(sh + swz(wc * (BCT / 2) + nt * 32 + l32, 2 * ks + hh));
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) acc[mt][nt] = mfma_32x32x16(af[mt], bf[nt], acc[mt][nt]);
    }
  };

  // Issue order keeps the in-order vmcnt simple: stage it's H copies go out one
  // iteration ahead, its E copies two iterations ahead; at the top of iteration it
  // only E(it+1) (the last 4 copies of this wave) may still be in flight.
  issue_e(0);
  issue_h(0);
  if (KI > 1) issue_e(1);
  for (int it = 0; it < KI - 1; ++it) {
    dma_wait<4>();
    __syncthreads();
    issue_h(it + 1);
    if (it + 2 < KI) issue_e(it + 2);
    compute(it, BK / 16);
  }
  dma_wait<0>();
  __syncthreads();
  compute(KI - 1, HALF_TAIL ? 2 : BK / 16);
  __syncthreads();   // the rings become epilogue scratch

  // ---------------- epilogue, phase 1: tile max / argmax per column on the raw
  // logits (the scale k2 = log2(e) / tau is positive, so the order is the same as in
  // the log2 domain x = logit * k2). Within a lane the registers are visited in
  // ascending vocabulary order, so a strict '>' keeps the lowest id among ties. Rows
  // past V (last tile only) become -inf.
  const float k2 = a.inv_tau * LOG2E;
  const bool full = v0 + BV <= a.V;
  if (!full) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (v0 + wv * 64 + mt * 32 + acc_row_perm(r, hh) >= a.V)
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt) acc[mt][nt][r] = -INFINITY;
  }
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int lc = wc * (BCT / 2) + nt * 32 + l32;
    float best = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int vb = v0 + wv * 64 + mt * 32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = acc[mt][nt][r];
        if (x > best) { best = x; bi = vb + acc_row_perm(r, hh); }
      }
    }
    // lane pair (l, l ^ 32): the swap leaves both candidates in every lane, and the
    // choice between them is symmetric.
    const auto pb = __builtin_amdgcn_permlane32_swap(__float_as_uint(best), __float_as_uint(best), false, false);
    const auto pi = __builtin_amdgcn_permlane32_swap((uint32_t)bi, (uint32_t)bi, false, false);
    const float b0 = __uint_as_float(pb[0]), b1 = __uint_as_float(pb[1]);
    const int i0 = (int)pi[0], i1 = (int)pi[1];
    const bool take1 = better(b1, i1, b0, i0);
    best = take1 ? b1 : b0;
    bi = take1 ? i1 : i0;
    if (hh == 0) {
      red_m[wv][lc] = best * k2;
      red_i[wv][lc] = bi;
    }
  }
  __syncthreads();

  // ---------------- phase 2: exp2, Z_t, S_t (log2 units), and p~ fragments
  const int VS = a.T * (BV / 16);            // 16-row vocabulary steps in p~
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int lc = wc * (BCT / 2) + nt * 32 + l32;
    const float m = ceilf(fmaxf(fmaxf(red_m[0][lc], red_m[1][lc]), fmaxf(red_m[2][lc], red_m[3][lc])));
    const float nm = -m;
    float Z = 0.f, S = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float dx = fmaf(acc[mt][nt][r], k2, nm);
        if (!full) dx = fmaxf(dx, -1e30f);                 // masked rows: e = 0, e*dx = 0
        const float e = exp2_fast(dx);
        Z += e;
        S = fmaf(e, dx, S);
        acc[mt][nt][r] = e;
      }
    }
    Z = pair_sum(Z);
    S = pair_sum(S);
    if (hh == 0) {
      red_z[wv][lc] = Z;
      red_s[wv][lc] = S;
    }
    const int ctile = (cb + wc * (BCT / 2) + nt * 32) / 32;
    if (ctile * 32 < a.Cpad) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int vs0 = (v0 + wv * 64 + mt * 32) / 16;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const f32x16_t &e = acc[mt][nt];
          const uint4 w = make_uint4(pack_bf16x2(e[8 * s + 0], e[8 * s + 1]), pack_bf16x2(e[8 * s + 2], e[8 * s + 3]),
                                     pack_bf16x2(e[8 * s + 4], e[8 * s + 5]), pack_bf16x2(e[8 * s + 6], e[8 * s + 7]));
          *(uint4 *)(a.ptilde + (((int64_t)ctile * VS + vs0 + s) * 64 + lane) * 8) = w;
        }
      }
    }
  }
  __syncthreads();

  // ---------------- phase 3: tile statistics in natural units (one writer per column).
  // A non-finite logit makes m, Z or S non-finite; the tile max is then stored as NaN.
  if (tid < BC) {
    const int lc = tid;
    const int c = cb + lc;
    if (c < a.Cpad) {
      float m = red_m[0][lc];
      int ai = red_i[0][lc];
      float Z = red_z[0][lc], S = red_s[0][lc];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        if (better(red_m[w][lc], red_i[w][lc], m, ai)) { m = red_m[w][lc]; ai = red_i[w][lc]; }
        Z += red_z[w][lc];
        S += red_s[w][lc];
      }
      const float rho = ceilf(m);
      const bool bad = !(fabsf(m) <= FLT_MAX) || !(Z <= FLT_MAX) || !(fabsf(S) <= FLT_MAX);
      const int64_t o = (int64_t)c * a.T + vt;       // statistics are [column][tile]
      a.tmax[o] = bad ? __builtin_nanf("") : m;
      a.trho[o] = rho;
      a.tsum[o] = Z;
      a.tent[o] = S * LN2;
      a.targ[o] = ai;
    }
  }
}

// One workgroup per canvas column merges that column's tile statistics ([column][tile]
// layout: contiguous reads) in a fixed order, so the result is deterministic. Besides
// entropy and argmax it leaves the column reference R and the sum Z (relative to R)
// for the self-conditioning product, and the column's largest probability (the
// confidence that confidence-ranked acceptance orders positions by).
__global__ __launch_bounds__(256) void row_finalize_kernel(LogitsArgs a) {
  __shared__ float sm[4], sr[4], sz[4], ss[4];
  __shared__ int si[4], sbad[4];
  const int c = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float *tmax = a.tmax + (int64_t)c * a.T;
  const float *trho = a.trho + (int64_t)c * a.T;
  const float *tsum = a.tsum + (int64_t)c * a.T;
  const float *tent = a.tent + (int64_t)c * a.T;

  // (tile max, first tile reaching it), NaN flag and R, in ascending tile order.
  // Chunks of 1024 tiles, four per thread, loads issued before use (clamped indices,
  // so every load is valid): one memory round trip per chunk and pass.
  constexpr int U = 4;
  float m = -INFINITY, R = -INFINITY;
  int tb = 0x7FFFFFFF, bad = 0;
  for (int t0 = 0; t0 < a.T; t0 += 256 * U) {
    float vm[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = min(t0 + tid + 256 * u, a.T - 1);
      vm[u] = tmax[t];
      vr[u] = trho[t];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + tid + 256 * u;
      if (t < a.T) {
        const float mt = vm[u];
        if (mt != mt) bad = 1;
        else if (mt > m) { m = mt; tb = t; }
        R = fmaxf(R, vr[u]);
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64);
    const int t2 = __shfl_xor(tb, o, 64);
    if (m2 > m || (m2 == m && t2 < tb)) { m = m2; tb = t2; }
    bad |= __shfl_xor(bad, o, 64);
    R = fmaxf(R, __shfl_xor(R, o, 64));
  }
  if (lane == 0) { sm[wave] = m; si[wave] = tb; sbad[wave] = bad; sr[wave] = R; }
  __syncthreads();
  m = sm[0]; tb = si[0]; bad = sbad[0]; R = sr[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    if (sm[w] > m || (sm[w] == m && si[w] < tb)) { m = sm[w]; tb = si[w]; }
    bad |= sbad[w];
    R = fmaxf(R, sr[w]);
  }

  float Z = 0.f, S = 0.f;
  for (int t0 = 0; t0 < a.T; t0 += 256 * U) {
    float vr[U], vz[U], ve[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = min(t0 + tid + 256 * u, a.T - 1);
      vr[u] = trho[t];
      vz[u] = tsum[t];
      ve[u] = tent[t];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (t0 + tid + 256 * u < a.T) {
        const float dr = vr[u] - R;                  // integer <= 0
        const float w = exp2_fast(dr);
        Z += vz[u] * w;
        S += (ve[u] + vz[u] * dr * LN2) * w;
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    Z += __shfl_xor(Z, o, 64);
    S += __shfl_xor(S, o, 64);
  }
  if (lane == 0) { sz[wave] = Z; ss[wave] = S; }
  __syncthreads();
  if (tid == 0) {
    Z = (sz[0] + sz[1]) + (sz[2] + sz[3]);
    S = (ss[0] + ss[1]) + (ss[2] + ss[3]);
    float ent = logf(Z) - S / Z;
    ent = ent > 0.f ? ent : 0.f;
    if (bad || !(ent == ent)) {
      ent = __builtin_nanf("");
      set_status(a.status, DGS_NONFINITE);
    }
    a.entropy[c] = ent;
    a.argmax[c] = bad ? 0 : a.targ[(int64_t)c * a.T + tb];
    a.colR[c] = bad ? __builtin_nanf("") : R;
    a.colZ[c] = bad ? __builtin_nanf("") : Z;
    // confidence = the largest probability = 2^(m - R) / Z (m: the column's largest x)
    a.colP[c] = bad ? __builtin_nanf("") : exp2_fast(m - R) / Z;
  }
}

// Copies the finalize kernel's per-column confidence out of the workspace.
__global__ __launch_bounds__(256) void confidence_kernel(int C, const float *colP, float *conf) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < C) conf[i] = colP[i];
}

}  // namespace

hipError_t dg_launch_confidence(int C, const float *colP, float *conf, hipStream_t st) {
  hipLaunchKernelGGL(confidence_kernel, dim3((C + 255) / 256), dim3(256), 0, st, C, colP, conf);
  return hipGetLastError();
}

namespace {

template <int BCT>
hipError_t launch_tiles(const LogitsArgs &a, hipStream_t st) {
  constexpr int smem = smem_bytes<BCT>();
  static std::atomic<bool> attr[DG_MAX_DEVICES];
  const hipError_t e = dg_smem_attr_once(attr, smem, {(const void *)logits_tile_kernel<false, BCT>,
                                                      (const void *)logits_tile_kernel<true, BCT>});
  if (e != hipSuccess) return e;
  const dim3 grid(a.T * ((a.Cpad + BCT - 1) / BCT));
  if (a.d % BK)
    hipLaunchKernelGGL((logits_tile_kernel<true, BCT>), grid, dim3(512), smem, st, a);
  else
    hipLaunchKernelGGL((logits_tile_kernel<false, BCT>), grid, dim3(512), smem, st, a);
  return hipGetLastError();
}

}  // namespace

// Canvas blocks of 128 columns when at most 128 columns are padded in, or when blocks of
// 256 would give fewer workgroups than CUs (a short vocabulary): each workgroup then
// streams its E tile and half as many H rows, the two blocks of a tile share the E rows
// through L2, and twice as many CUs work. Otherwise blocks of 256 (more FLOP per copied
// byte).
hipError_t dg_launch_logits(const LogitsArgs &a, hipStream_t st) {
  const bool narrow = a.Cpad <= 128 || (int64_t)a.T * ((a.Cpad + 255) / 256) < dg_device_cus();
  hipError_t e = narrow ? launch_tiles<128>(a, st) : launch_tiles<256>(a, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(row_finalize_kernel, dim3(a.C), dim3(256), 0, st, a);
  return hipGetLastError();
}
