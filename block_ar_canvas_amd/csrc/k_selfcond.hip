// Self-conditioning product s = p0 E over the whole vocabulary.
//
// Method (DiffusionGemma Technical Report page, "Method steps" (3): z = FFW(p0 E);
// Google "DiffusionGemma explained", section "Self-conditioning": the step's
// probability matrix is multiplied by the token embedding table and the result is
// passed to the next step). The report's limitations single out this 262K-wide
// product as slow in plain framework code; here it is one split-K MFMA pass over E.
//
// selfcond_split_kernel computes s^T[j][c] = sum_v E[v][j] p~[c][v] 2^-n(t,c) for a
// 256-wide slice of the model width j, a block of BC = 256 (or 128) canvas columns c
// and one split S (a
// contiguous range of 256-row vocabulary tiles t). p~ holds bf16 2^(x - rho_t) from the
// logits epilogue; n(t, c) = rho_S - rho_t is an integer, so the rescale to the split's
// common reference is an exact exponent shift, applied to the bf16 fragments with packed
// 16-bit integer arithmetic. The remaining per-(split, column) factor 2^(rho_S - R) / Z
// (R = the column reference, Z = the softmax sum relative to 2^R, both from the logits
// finalize) is applied by selfcond_reduce_kernel, which sums the split partials in
// split order (deterministic) and rounds s to bf16 for the FFW.
//
// Data movement: a ring of 4 LDS stages, 32 vocabulary rows each, filled by direct
// global -> LDS copies (three stages in flight while one is consumed):
//   E tile [32 v][256 j] bf16, copied as 512-byte row segments (32 lanes per row) with
//     16-byte chunks XOR-swizzled by 4*(v & 3);
//   p~ fragments, copied as the 1 KiB blocks the logits epilogue wrote.
// MFMA operands: A = E^T (j rows, vocabulary k) via two ds_read_b64_tr_b16 transposing
// reads per fragment; B = p~ (canvas columns) via linear 16-byte reads. Each wave owns
// 128 j x BC/4 canvas (4 x BC/128 MFMA tiles, up to 128 accumulators, two waves per
// SIMD). Every output element sums its split's vocabulary rows in stage order whatever
// BC is, so both block widths give the same bits; 128-column blocks double the
// workgroups where 256-column ones would leave CUs idle (a short vocabulary).
#include "dg_sampler_dev.h"

namespace {

constexpr int BJ = 256, BKV = 32, NS = 4;
constexpr int ESTAGE = BKV * BJ * 2;           // 16 KiB
constexpr int NTAB_MAX = 32 * 1024;            // LDS bytes for the split's shift table
// p~ stage: BC/32 canvas tiles x 2 k-steps of 1 KiB; SMEM 160 KiB (BC 256) or 128 KiB
template <int BC> constexpr int pstage() { return BC / 32 * 2 * 1024; }
template <int BC> constexpr int stage() { return ESTAGE + pstage<BC>(); }
template <int BC> constexpr int smem_bytes() { return NS * stage<BC>() + NTAB_MAX; }

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v2i16_t __attribute__((ext_vector_type(2)));
#define LDS3 __attribute__((address_space(3)))

// Byte offset of element (row v, column j) in the E stage.
DG_DEV int eoff(int v, int j) { return v * 512 + ((((j >> 3) ^ (4 * (v & 3))) & 31) << 4) + ((j & 7) << 1); }

// bf16 pair scaled by 2^-n (n >= 0) through the exponent field, flushing to zero below
// the smallest normal (values are non-negative probabilities).
DG_DEV uint32_t shift2(uint32_t w, v2i16_t dn) {
  v2i16_t x = __builtin_bit_cast(v2i16_t, w) - dn;
  const v2i16_t z = {0, 0};
  x = x > z ? x : z;
  return __builtin_bit_cast(uint32_t, x);
}

template <int BC>
__global__ __launch_bounds__(512) void selfcond_split_kernel(SelfcondArgs a, int nj) {
  static_assert(BC == 128 || BC == 256, "canvas block");
  constexpr int STAGE = stage<BC>();
  constexpr int CTW = BC / 128;                   // canvas tiles per wave
  constexpr int PQ = BC / 128;                    // p~ copy instructions per wave and stage
  constexpr int CPS = 2 + PQ;                     // copies per wave and stage
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  unsigned char *ntab = (unsigned char *)(smem + NS * STAGE);   // [tile in split][BC columns]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wj = wave & 1, wc = wave >> 1;
  const int hh = lane >> 5, l32 = lane & 31;

  // blockIdx.x -> (split, j-slice, canvas block). The j-slices of one split share its
  // p~ range and its canvas blocks share its E rows; all of a split's workgroups are
  // dispatched together and kept on one XCD when the split count allows it.
  const int b = blockIdx.x;
  const int ncb = (a.Cpad + BC - 1) / BC;
  const int per = nj * ncb;                       // workgroups of one split
  int split, rem;
  if ((a.nsc & 7) == 0) {
    const int xcd = b & 7, r = b >> 3;
    split = xcd + 8 * (r / per);
    rem = r % per;
  } else {
    split = b / per;
    rem = b % per;
  }
  const int jb = rem % nj;
  const int j0 = jb * BJ;
  const int cb = (rem / nj) * BC;
  const int ct0 = cb / 32;                        // first canvas tile of this block
  const int nct = a.Cpad / 32;
  const int VS = a.T * (DG_BV / 16);
  const int tile0 = (int)((int64_t)split * a.T / a.nsc);
  const int tile1 = (int)((int64_t)(split + 1) * a.T / a.nsc);
  const int vbeg = tile0 * DG_BV;
  const int NIT = (tile1 - tile0) * (DG_BV / BKV);

  // Copy duties per stage (2 E and PQ p~ instructions per wave). E instruction `ins`
  // fills stage rows 2*ins and 2*ins + 1 (32 lanes per 512-byte row segment); p~
  // instruction `pin` copies k-step pin & 1 of canvas tile pin >> 1.
  int erow[2], ecol[2];
  const u16 *gp[PQ];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int ins = wave * 2 + q;                   // 0..15
    const int v = 2 * ins + (lane >> 5);             // E row in the stage
    const int lchunk = (lane & 31) ^ (4 * (v & 3));
    int jc = j0 + 8 * lchunk;
    jc = jc < a.d ? jc : a.d - 8;                    // clamp: columns past d never stored
    erow[q] = v;
    ecol[q] = jc;
  }
#pragma unroll
  for (int q = 0; q < PQ; ++q) {
    const int pin = wave * PQ + q;                  // 0 .. BC/16 - 1
    int ctile = ct0 + (pin >> 1);
    ctile = ctile < nct ? ctile : nct - 1;           // clamp: columns never stored
    gp[q] = a.ptilde + (((int64_t)ctile * VS + vbeg / 16 + (pin & 1)) * 64 + lane) * 8;
  }
  const uint32_t sbase = lds_addr(smem);
  auto issue = [&](int it) {
    const uint32_t st = sbase + (uint32_t)(it % NS) * STAGE;
    const int vo = it * BKV;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int ins = wave * 2 + q;
      int vr = vbeg + vo + erow[q];
      vr = vr < a.V ? vr : a.V - 1;                  // rows past V meet p~ = 0
      dma16(a.E + (int64_t)vr * a.d + ecol[q], st + ins * 1024);
    }
#pragma unroll
    for (int q = 0; q < PQ; ++q)
      dma16(gp[q] + (int64_t)(vo / 16) * 64 * 8, st + ESTAGE + (wave * PQ + q) * 1024);
  };

  f32x16_t acc[4][CTW];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < CTW; ++j) acc[i][j] = f32x16_t{};

  // Transposing-read source addresses: lane i of 16-lane group g reads 4 consecutive
  // j of row 4r + i/4 (+ 16ks + 8h); the group returns E^T rows j = 16(g&1) + i.
  const int g = lane >> 4, gi = lane & 15;
  const int trow = 8 * (g >> 1) + (gi >> 2);
  const int tcol = wj * 128 + 16 * (g & 1) + 4 * (gi & 3);

  // Operands of one 16-deep k-step: 4 E^T fragments, 2 raw p~ fragments and their
  // shift counts (the shift is applied just before the MFMAs).
  struct Frag {
    u32x4_t af[4], bf[CTW];
    short n[CTW];
  };
  auto load = [&](int it, int ks, Frag &f) {
    const char *se = smem + (it % NS) * STAGE;
    const char *sp = se + ESTAGE;
    const int tl = (it * BKV) / DG_BV;               // tile of this stage within the split
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      uint32_t w[4];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int off = eoff(16 * ks + 4 * r + trow, tcol + 32 * jt);
        const v4i16_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS3 v4i16_t *)(se + off));
        const uint2 u = __builtin_bit_cast(uint2, t);
        w[2 * r] = u.x;
        w[2 * r + 1] = u.y;
      }
      f.af[jt] = u32x4_t{w[0], w[1], w[2], w[3]};
    }
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) {
      f.n[ct] = (short)ntab[tl * BC + (wc * CTW + ct) * 32 + l32];
      f.bf[ct] = *(const u32x4_t *)(sp + ((wc * CTW + ct) * 2 + ks) * 1024 + lane * 16);
    }
  };
  auto mma = [&](const Frag &f) {
    u32x4_t bf[CTW];
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) {
      const v2i16_t dn = v2i16_t{(short)(f.n[ct] << 7), (short)(f.n[ct] << 7)};
      const u32x4_t v = f.bf[ct];
      bf[ct] = u32x4_t{shift2(v[0], dn), shift2(v[1], dn), shift2(v[2], dn), shift2(v[3], dn)};
    }
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) acc[jt][ct] = mfma_32x32x16(f.af[jt], bf[ct], acc[jt][ct]);
  };

  // Three stages' copies fly while one is consumed; each iteration waits for its own
  // stage, passes one barrier (which also frees the slot read in the previous
  // iteration) and refills that slot before computing.
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < NIT) issue(s);
  // Split reference rho_S = max of the split's tile references per column, and the
  // shift table n(t, c) = rho_S - rho_t (uint8; 255 flushes a tile, a column past C or
  // a column whose statistics are not finite). Staged while the first stages' copies
  // are in flight: 8 lanes share a column (consecutive tiles, so a wave's load touches
  // 8 columns' contiguous references), 64 columns per pass, and the lane group's
  // maximum comes from three xor shuffles.
  {
    constexpr int TPL = 16;                        // tiles per lane: ntl <= 128 = 8 * TPL
    const int ntl = tile1 - tile0;
    const int sub = tid & 7, cg = tid >> 3;
#pragma unroll
    for (int pass = 0; pass < BC / 64; ++pass) {
      const int cl = pass * 64 + cg, c = cb + cl;
      const bool live = c < a.C;
      const float *tr = a.trho + (int64_t)(live ? c : 0) * a.T + tile0;
      float v[TPL];
      float rs = -INFINITY;
#pragma unroll
      for (int k = 0; k < TPL; ++k) {
        const int t = sub + 8 * k;
        v[k] = (live && t < ntl) ? tr[t] : -INFINITY;
        rs = fmaxf(rs, v[k]);
      }
      rs = fmaxf(rs, __shfl_xor(rs, 1));
      rs = fmaxf(rs, __shfl_xor(rs, 2));
      rs = fmaxf(rs, __shfl_xor(rs, 4));
      const bool ok = live && rs - rs == 0.f;
#pragma unroll
      for (int k = 0; k < TPL; ++k) {
        const int t = sub + 8 * k;
        if (t < ntl) {
          const float n = ok ? fminf(rs - v[k], 255.f) : 255.f;
          ntab[t * BC + cl] = (unsigned char)(n == n ? n : 255.f);
        }
      }
      if (jb == 0 && sub == 0 && c < a.Cpad) a.rhoS[(int64_t)split * a.Cpad + c] = rs;
    }
  }

  Frag f0, f1;
  for (int it = 0; it < NIT; ++it) {
    const int ahead = NIT - 1 - it;                  // stages issued beyond this one
    if (ahead >= 2) dma_wait<2 * CPS>();
    else if (ahead == 1) dma_wait<CPS>();
    else dma_wait<0>();
    __syncthreads();
    if (it + NS - 1 < NIT) issue(it + NS - 1);
    load(it, 0, f0);
    load(it, 1, f1);
    mma(f0);
    mma(f1);
  }

  // Partial s^T for this split, stored as ps[split][j][c]: for each accumulator
  // register the 32 lanes of a half-wave write 32 consecutive columns (128 bytes).
#pragma unroll
  for (int ct = 0; ct < CTW; ++ct) {
    const int c = cb + (wc * CTW + ct) * 32 + l32;
    if (c >= a.Cpad) continue;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = j0 + wj * 128 + jt * 32 + acc_row(r, hh);
        if (j < a.d) a.ps[((int64_t)split * a.d + j) * a.Cpad + c] = acc[jt][ct][r];
      }
    }
  }
}

// s[c][j] = bf16( sum over splits S, in split order, of
//                 2^(rho_S - R_c) / Z_c * ps[S][j][c] ).
// A workgroup owns 16 j x 64 c (one float4 of columns per thread): reads run along c,
// the bf16 result is transposed through LDS and written along j. Splits are taken 16
// at a time; a chunk's 16 partial loads are issued together, ahead of the scale
// computation, so each chunk costs one memory round trip. (32 at a time took 190 VGPRs
// and two workgroups per CU, so at 512 workgroups an acceptance workgroup waited for a
// slot; 16 take 104 VGPRs, four per CU, and measured slightly faster at every size.)
// The summation order is the split order whatever the chunk size.
// The grid is one-dimensional: ars.B workgroups first, then nx x ny reduce workgroups
// in row order (j fastest). The first ars.B run acceptance, renoise and the stop test of
// canvas blockIdx.x instead: that work needs only the sampler head's outputs, so it
// overlaps the reduce instead of taking a launch of its own, and it comes first in
// dispatch order so that it starts at once even when the reduce fills every CU slot.
__global__ __launch_bounds__(256) void selfcond_reduce_kernel(SelfcondArgs a, ArsArgs ars, int nx) {
  if ((int)blockIdx.x < ars.B) {
    dgs::ars_canvas(ars, blockIdx.x);
    return;
  }
  const int wg = (int)blockIdx.x - ars.B, bx = wg % nx, by = wg / nx;
  constexpr int PC = 16;                             // splits per chunk
  __shared__ float scale[64 * (PC + 1)];             // [c][split in chunk]
  __shared__ u16 out[64][24];
  const int tid = threadIdx.x;
  const int j0 = bx * 16, c0 = by * 64;
  const int jj = tid >> 4, c4 = (tid & 15) * 4;
  const int j = j0 + jj;
  const bool live = j < a.d && c0 + c4 < a.Cpad;
  const float *src = a.ps + (int64_t)(live ? j : 0) * a.Cpad + (live ? c0 + c4 : 0);
  const int64_t pstride = (int64_t)a.d * a.Cpad;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < a.nsc; p0 += PC) {
    const int np = min(PC, a.nsc - p0);
    float4 x[PC];
#pragma unroll
    for (int p = 0; p < PC; ++p)                     // clamped split: always a valid address
      x[p] = *(const float4 *)(src + (int64_t)(p0 + min(p, np - 1)) * pstride);
    __syncthreads();                                 // previous chunk's scales consumed
    // clamped (always valid) addresses, loads first: they all go out together
    constexpr int SK = 64 * PC / 256;
    float R[SK], Z[SK], rs[SK];
#pragma unroll
    for (int k = 0; k < SK; ++k) {
      const int i = min(tid + 256 * k, 64 * np - 1);
      const int cc = min(c0 + i / np, a.C - 1);
      R[k] = a.colR[cc];
      Z[k] = a.colZ[cc];
      rs[k] = a.rhoS[(int64_t)(p0 + i % np) * a.Cpad + cc];
    }
#pragma unroll
    for (int k = 0; k < SK; ++k) {                  // branch-free, so no load is sunk
      const int i = tid + 256 * k;
      const int cl = i / np, p = i % np;
      const float e = exp2_fast(rs[k] - R[k]) / Z[k];
      const bool ok = c0 + cl < a.C && Z[k] > 0.f && Z[k] <= 3.0e38f && rs[k] - rs[k] == 0.f;
      if (i < 64 * np) scale[cl * (PC + 1) + p] = ok ? e : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < PC; ++p) {
      if (p < np) {
        v[0] += scale[(c4 + 0) * (PC + 1) + p] * x[p].x;
        v[1] += scale[(c4 + 1) * (PC + 1) + p] * x[p].y;
        v[2] += scale[(c4 + 2) * (PC + 1) + p] * x[p].z;
        v[3] += scale[(c4 + 3) * (PC + 1) + p] * x[p].w;
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) out[c4 + q][jj] = f32_to_bf16(v[q]);
  __syncthreads();
  if (tid < 128) {
    const int cl = tid >> 1, j8 = (tid & 1) * 8;
    const int c = c0 + cl, jo = j0 + j8;
    if (c < a.Cpad && jo < a.d) *(uint4 *)(a.s + (int64_t)c * a.d + jo) = *(const uint4 *)(&out[cl][j8]);
  }
}

template <int BC>
hipError_t launch_split(const SelfcondArgs &a, int nj, hipStream_t st) {
  constexpr int smem = smem_bytes<BC>();
  static std::atomic<bool> attr[DG_MAX_DEVICES];
  hipError_t e = dg_smem_attr_once(attr, smem, {(const void *)selfcond_split_kernel<BC>});
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(selfcond_split_kernel<BC>, dim3(nj * a.nsc * ((a.Cpad + BC - 1) / BC)), dim3(512), smem,
                     st, a, nj);
  return hipGetLastError();
}

}  // namespace

// Canvas blocks of 128 columns when at most 128 columns are padded in, or when blocks
// of 256 would give fewer workgroups than CUs (a short vocabulary); else 256 (each
// copied E byte feeds twice the columns).
hipError_t dg_launch_selfcond(const SelfcondArgs &a, const ArsArgs *ars, hipStream_t st) {
  const int nj = (a.d + BJ - 1) / BJ;
  const bool narrow = a.Cpad <= 128 || (int64_t)nj * a.nsc * ((a.Cpad + 255) / 256) < dg_device_cus();
  hipError_t e = narrow ? launch_split<128>(a, nj, st) : launch_split<256>(a, nj, st);
  if (e != hipSuccess) return e;
  const int nx = (a.d + 15) / 16, ny = (a.Cpad + 63) / 64;
  ArsArgs r{};                                       // r.B = 0: no acceptance workgroups
  if (ars) r = *ars;                                 // ars->tpp * ars->C <= 256 (caller)
  hipLaunchKernelGGL(selfcond_reduce_kernel, dim3(r.B + nx * ny), dim3(256), 0, st, a, r, nx);
  return hipGetLastError();
}
