// Bidirectional canvas attention over the static prefix KV cache.
//
// Method: in denoise mode every canvas query attends, with no mask, to all canvas
// tokens and to the prompt / finished-block KV cache (Google "DiffusionGemma
// explained", section "Architecture: incremental prefill and denoising"; tutorial
// chapter "DiffusionGemma", the per-phase attention masks: the current canvas uses
// full bidirectional attention and reads the cache). Attention is a softmax over a
// set of keys, so the key order is free: the kernel walks the canvas keys first, then
// the prefix, in tiles of 64 that never straddle the two segments.
//
// Work split (split-K / "flash decoding" over keys): a workgroup owns one KV head g,
// 256 query rows of that head's group (row = (head in group, canvas position)) and a
// contiguous range of 64-key tiles. Eight waves of 32 query rows each, two per SIMD,
// every wave on whole tiles with its own online softmax. K and V^T tiles stream
// HBM -> registers -> LDS into a 4-slot ring (two tiles ahead), one barrier per tile.
// The split's partial O goes to the workspace row-major in bf16 (coalesced 16-byte
// stores; it is relative to the split's own max, so rounding it costs one bf16 ulp
// before the merge, and A is bf16 anyway), its (max, sum) in fp32, and
// attn_merge_kernel combines the splits in a fixed order.
//
// Orientation: S^T = K Q^T (keys are MFMA rows, loaded through perm_row so that the
// probabilities come out as ready B fragments), O^T = V^T P^T (V is stored transposed
// in the cache, so its A fragments are contiguous 16-byte LDS reads). Each lane owns
// one query row: its softmax statistics need only one cross-lane exchange (lane ^ 32).
//
// Softmax reference: a lane keeps the reference m_ref its probabilities are scaled
// against and moves it (rescaling O and the sum) only when the running maximum
// exceeds it by more than 8 in log2 units, so probabilities stay below 2^8 and the
// O rescale (64 accumulator registers per lane) is rare after the first tiles.
#include <type_traits>

#include "dg_common.h"

namespace {

constexpr int KT = 64;      // keys per tile
constexpr int NS = 4;       // LDS ring slots
constexpr int NW = 8;       // waves per workgroup (two per SIMD)
constexpr int QB = NW * 32; // query rows per workgroup
constexpr float RESCALE_LOG2 = 8.f;

template <int HD>
struct Cfg {
  static constexpr int ER = HD < 32 ? 32 : HD;       // V^T rows padded to an MFMA tile
  static constexpr int ET = ER / 32;                 // e-tiles of O^T
  static constexpr int KS = HD / 16;                 // k-steps of S = K Q^T
  static constexpr int KRB = HD * 2;                 // bytes per K row
  static constexpr int KTILE = KT * KRB;             // K tile bytes
  static constexpr int VTILE = ER * KT * 2;          // V^T tile bytes (128-byte rows)
  static constexpr int STAGE = KTILE + VTILE;
  static constexpr int KI = KTILE / 1024;            // copy instructions for K
  static constexpr int VI = HD * KT * 2 / 1024;      // copy instructions for V^T
  static constexpr int TI = KI + VI;
  static constexpr int PER_WAVE = TI >= NW ? TI / NW : 1;   // copies per issuing wave
  static constexpr int KSH = HD == 128 ? 0 : HD == 64 ? 1 : HD == 32 ? 2 : 3;
  static constexpr int OPITCH = HD + 4;              // floats per row of the O transpose
  static constexpr int OSLOT = 32 * OPITCH * 4;      // one wave's 32 x HD fp32 tile
  static constexpr int SMEM_RING = NS * STAGE;
  static constexpr int SMEM_END = NW * OSLOT;
  static constexpr int SMEM = SMEM_RING > SMEM_END ? SMEM_RING : SMEM_END;
  static_assert(TI < NW || TI % NW == 0, "copy split");
};

// K rows: physical 16-byte chunk = logical ^ fk(row) (conflict-free A-fragment reads).
template <int HD>
DG_DEV int kswz(int row, int chunk) {
  return row * Cfg<HD>::KRB + ((chunk ^ ((row >> Cfg<HD>::KSH) & (HD / 8 - 1))) << 4);
}
DG_DEV int vswz(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

// CAUSAL (the block prefill): key j of the canvas segment (the block) is visible to
// query i only for j <= i; prefix keys are always visible.
template <int HD, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void attn_split_kernel(AttnArgs a, int nq, int ntc,
                                                             int ntiles, int units) {
  using F = Cfg<HD>;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  // Padded V^T rows (head dims below one MFMA tile) are zero in every ring slot.
  if constexpr (F::ER > HD) {
    constexpr int PW = (F::ER - HD) * 32;            // 32-bit words of padding per slot
    for (int i = tid; i < NS * PW; i += NW * 64)
      *(uint32_t *)(smem + (i / PW) * F::STAGE + F::KTILE + HD * 128 + 4 * (i % PW)) = 0;
  }

  // Query rows of this wave: r = qb*256 + wave*32 + l32 -> (head, canvas position).
  const int r = qb * QB + wave * 32 + l32;
  const bool qok = r < G * a.C;
  const int qh = g * G + (qok ? r / a.C : 0), qc = qok ? r % a.C : 0;
  u32x4_t qf[F::KS];
#pragma unroll
  for (int ks = 0; ks < F::KS; ++ks) {
    u32x4_t v = {0, 0, 0, 0};
    if (qok) v = *(const u32x4_t *)(a.Q + (int64_t)qc * a.Hq * HD + qh * HD + ks * 16 + 8 * hh);
    qf[ks] = v;
  }
  // Settle the Q loads once, here. Passing the fragments through an empty asm makes
  // them plain register values for the compiler; otherwise its wait-count tracking
  // carries "maybe pending" across the tile loop's back edge and puts a full
  // vector-memory wait (which also waits for the tile prefetch) before every score
  // MFMA.
#pragma unroll
  for (int ks = 0; ks < F::KS; ++ks) asm volatile("" : "+v"(qf[ks]));

  // Tile t is fetched into registers (one 16-byte load per lane per KiB of the stage:
  // K tile bytes for copy index i < KI, V^T tile bytes after that) and written to its
  // ring slot one iteration later. Ordinary loads plus LDS writes keep the matrix core
  // fed: with direct global -> LDS copies (global_load_lds) of the same bytes the MFMA
  // work of this loop took about 45% more cycles on gfx950.
  // Source of lane `lane` in copy index i: K row / V^T row and logical 16-byte chunk
  // follow from the lane (the LDS layout is swizzled by chunk). The element offset at
  // key 0 of each segment is precomputed per lane; a tile adds its first key times the
  // key stride, plus (only ever nonzero in a segment's last tile) the clamp of the key
  // to the segment, so every load stays inside the valid rows. Loads use a wave-uniform
  // base and a 32-bit byte offset (the API caps each cache array below 4 GiB).
  uint32_t ofc[F::PER_WAVE], ofp[F::PER_WAVE];
#pragma unroll
  for (int j = 0; j < F::PER_WAVE; ++j) {
    const int i = wave + NW * j;
    const int off = (i < F::KI ? i : i - F::KI) * 1024 + 16 * lane;
    if (i < F::KI) {
      const int row = off / F::KRB, pc = (off % F::KRB) >> 4;
      const int lc = pc ^ ((row >> F::KSH) & (HD / 8 - 1));
      ofc[j] = (uint32_t)(row * a.Hkv * HD + g * HD + 8 * lc);
      ofp[j] = (uint32_t)((g * (uint32_t)a.Pcap + row) * HD + 8 * lc);
    } else {
      const int e = off >> 7, pc = (off & 127) >> 4;
      const int lc = pc ^ ((e >> 1) & 7);
      ofc[j] = (uint32_t)((g * HD + e) * a.Cpad + 8 * lc);
      ofp[j] = (uint32_t)((g * HD + e) * (uint32_t)a.Pcap + 8 * lc);
    }
  }
  u32x4_t rbuf[F::PER_WAVE];
  auto fetch = [&](int t, u32x4_t (&rb)[F::PER_WAVE]) {
    const bool canvas = t < ntc;
    const int k0 = (canvas ? t : t - ntc) * KT;
    const int seglen = canvas ? a.C : (int)a.P;
#pragma unroll
    for (int j = 0; j < F::PER_WAVE; ++j) {
      const int i = wave + NW * j;
      if (F::TI < NW && i >= F::TI) break;   // only when fewer copies than waves
      const int off = (i < F::KI ? i : i - F::KI) * 1024 + 16 * lane;
      const u16 *base;
      uint32_t eo;
      if (i < F::KI) {
        const int key = k0 + off / F::KRB;                    // unclamped key of this row
        const int kst = canvas ? a.Hkv * HD : HD;
        base = canvas ? a.Kc : a.Kp;
        eo = (canvas ? ofc[j] : ofp[j]) + (uint32_t)((k0 + min(0, seglen - 1 - key)) * kst);
      } else {
        const int e = off >> 7, pc = (off & 127) >> 4;
        const int ks = k0 + 8 * (pc ^ ((e >> 1) & 7));        // unclamped first key
        base = canvas ? a.Vct : a.Vt;
        eo = (canvas ? ofc[j] : ofp[j]) + (uint32_t)(k0 + min(0, ((seglen - 1) & ~7) - ks));
      }
      rb[j] = *(const u32x4_t *)((const char *)base + 2u * eo);
    }
  };
  auto put = [&](int slot, const u32x4_t (&rb)[F::PER_WAVE]) {
#pragma unroll
    for (int j = 0; j < F::PER_WAVE; ++j) {
      const int i = wave + NW * j;
      if (F::TI < NW && i >= F::TI) break;   // only when fewer copies than waves
      *(u32x4_t *)(smem + slot * F::STAGE + (i < F::KI ? i * 1024 : F::KTILE + (i - F::KI) * 1024) + 16 * lane) = rb[j];
    }
  };

  f32x16_t O[F::ET];
#pragma unroll
  for (int et = 0; et < F::ET; ++et) O[et] = f32x16_t{};
  float mref = -INFINITY, lsum = 0.f;

  // The two waves of a SIMD (w and w + 4) run the same loop with opposite issue
  // priorities: the first is favoured in the MFMA phases (scores, P.V), the second in
  // the softmax phases. Both meet at every tile barrier; without the asymmetry they
  // stay in lockstep and contend for the matrix core and the vector ALU in turn.
  auto run = [&](auto PM, auto PL) {
    // Tiles 0 and 1 go to their slots up front (both loads in flight together) and tile
    // 2 into registers; iteration i writes tile i + 2 (slot of tile i - 2, free after
    // the barrier) and fetches i + 3.
    const int nt = t1 - t0;
    {
      u32x4_t rb1[F::PER_WAVE];
      if (nt > 0) fetch(t0, rbuf);
      if (nt > 1) fetch(t0 + 1, rb1);
      if (nt > 0) put(0, rbuf);
      if (nt > 1) put(1, rb1);
    }
    if (nt > 2) fetch(t0 + 2, rbuf);
    for (int i = 0; i < nt; ++i) {
      const int t = t0 + i;
      __syncthreads();
      if (i + 2 < nt) {
        put((i + 2) % NS, rbuf);
        if (i + 3 < nt) fetch(t + 3, rbuf);
      }
      const bool canvas = t < ntc;
      const int k0 = (canvas ? t : t - ntc) * KT;
      const int nvalid = min(KT, (canvas ? a.C : (int)a.P) - k0);
      const uint8_t *Ks = smem + (i % NS) * F::STAGE;
      uint8_t *Vs = smem + (i % NS) * F::STAGE + F::KTILE;
      if (nvalid < KT) {
        // Tail tile: zero V^T at keys >= nvalid (cache slots past the valid length may
        // hold any bit pattern, and 0 * NaN would poison O). The K rows there are copies
        // of the last valid key (finite) and their scores are masked.
        for (int x = tid; x < HD * (KT - nvalid); x += NW * 64) {
          const int e = x / (KT - nvalid), key = nvalid + x % (KT - nvalid);
          *(u16 *)(Vs + vswz(e, key >> 3) + 2 * (key & 7)) = 0;
        }
        __syncthreads();
      }

      // S^T for both 32-key halves of the tile (two independent MFMA chains), then one
      // online-softmax update and O^T += V^T P^T per half. Both halves always run, with
      // no branch between the MFMAs: in a tail tile the keys past nvalid have finite
      // (clamped) K rows, masked scores and zeroed V^T, so they add exactly nothing, and
      // the first half always holds a valid key, so the reference is finite before an
      // all-masked second half is seen.
      // The K fragments of k-step ks + 1 are read while k-step ks's two MFMAs run
      // (scheduling groups: 2 LDS reads, then 2 MFMAs).
      __builtin_amdgcn_s_setprio(decltype(PM)::value);
      f32x16_t S[2] = {f32x16_t{}, f32x16_t{}};
      u32x4_t ka[2][2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        ka[0][kt] = *(const u32x4_t *)(Ks + kswz<HD>(32 * kt + perm_row(l32), hh));
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int ks = 0; ks < F::KS; ++ks) {
        if (ks + 1 < F::KS) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
            ka[(ks + 1) & 1][kt] = *(const u32x4_t *)(Ks + kswz<HD>(32 * kt + perm_row(l32), 2 * (ks + 1) + hh));
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) S[kt] = mfma_32x32x16(ka[ks & 1][kt], qf[ks], S[kt]);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
      // One reference update per tile, from the maximum over both halves (so the
      // softmax and P.V code below is branch-free and the compiler can overlap half
      // 1's softmax with half 0's MFMAs).
      __builtin_amdgcn_s_setprio(decltype(PL)::value);
      if (nvalid < KT) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr)
            if (32 * kt + acc_row_perm(rr, hh) >= nvalid) S[kt][rr] = -INFINITY;
      }
      if (CAUSAL && canvas && k0 + KT - 1 > qc) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr)
            if (k0 + 32 * kt + acc_row_perm(rr, hh) > qc) S[kt][rr] = -INFINITY;
      }
      float mt = fmaxf(S[0][0], S[1][0]);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) mt = fmaxf(mt, S[kt][rr]);
      mt = pair_max(mt) * a.scale_log2;     // the scale is positive: max commutes with it
      if (__builtin_amdgcn_ballot_w64(mt > mref + RESCALE_LOG2)) {
        const float mnew = fmaxf(mref, mt);
        // The ballot is per wave, and under the causal mask a wave can mix lanes that see
        // keys with lanes that have seen none yet (a split starting inside the canvas, a
        // wave straddling two heads): those keep m_ref = -inf and O = 0, and must not take
        // exp2(-inf - -inf) = NaN.
        const float alpha = mnew == -INFINITY ? 1.f : exp2_fast(mref - mnew);
        lsum *= alpha;
#pragma unroll
        for (int et = 0; et < F::ET; ++et) O[et] *= alpha;
        mref = mnew;
      }
      // Under the causal mask a split may start with tiles that hide every key from a
      // query: its reference stays -inf, and those tiles must contribute 0, not NaN.
      const float nm = CAUSAL && mref == -INFINITY ? 0.f : -mref;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        float y[16], ls = 0.f;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          y[rr] = exp2_fast(fmaf(S[kt][rr], a.scale_log2, nm));
          ls += y[rr];
        }
        lsum += pair_sum(ls);
        u32x4_t pf[2];
#pragma unroll
        for (int s = 0; s < 2; ++s)
          pf[s] = u32x4_t{pack_bf16x2(y[8 * s + 0], y[8 * s + 1]), pack_bf16x2(y[8 * s + 2], y[8 * s + 3]),
                          pack_bf16x2(y[8 * s + 4], y[8 * s + 5]), pack_bf16x2(y[8 * s + 6], y[8 * s + 7])};
        if (kt == 0) __builtin_amdgcn_s_setprio(decltype(PM)::value);
#pragma unroll
        for (int et = 0; et < F::ET; ++et) {
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const u32x4_t af = *(const u32x4_t *)(Vs + vswz(et * 32 + l32, 4 * kt + 2 * s + hh));
            O[et] = mfma_32x32x16(af, pf[s], O[et]);
          }
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  if (wave < NW / 2) run(std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{});
  else run(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{});

  // The split's partial O, row-major through a per-wave LDS transpose, and (max, sum).
  __syncthreads();
  float *ot = (float *)(smem + wave * F::OSLOT);   // [32 query rows][OPITCH]
#pragma unroll
  for (int et = 0; et < F::ET; ++et)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int e = et * 32 + acc_row(rr, hh);
      if (e < HD) ot[l32 * F::OPITCH + e] = O[et][rr];
    }
  if (hh == 0 && qok) {
    const int64_t row = ((int64_t)split * a.Hq + qh) * a.Cpad + qc;
    a.pml[2 * row] = mref;
    a.pml[2 * row + 1] = lsum;
  }
  // The partial O is stored rounded to bf16 (its own reference and fp32 sum keep the
  // scale): one 16-byte store per eight head dims.
  constexpr int F8 = HD / 8;
  for (int f = lane; f < 32 * F8; f += 64) {
    const int rl = f / F8, c8 = f % F8;
    const int rq = qb * QB + wave * 32 + rl;
    if (rq >= G * a.C) continue;
    const int h = g * G + rq / a.C, c = rq % a.C;
    const float *src = ot + rl * F::OPITCH + 8 * c8;
    *(uint4 *)(a.po + (((int64_t)split * a.Hq + h) * a.Cpad + c) * HD + 8 * c8) =
        uint4{pack_bf16x2(src[0], src[1]), pack_bf16x2(src[2], src[3]), pack_bf16x2(src[4], src[5]),
              pack_bf16x2(src[6], src[7])};
  }
}

// Log-sum-exp merge of the key-range partials, in split order. HD/8 threads per
// output row, eight head dims each. Splits are taken eight at a time with clamped
// (always valid) indices, so a chunk's loads go out together: one memory round trip
// per eight splits instead of one per split.
template <int HD>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  constexpr int TPR = HD / 8, RPB = 256 / TPR, U = 8;
  const int row = blockIdx.x * RPB + threadIdx.x / TPR;
  if (row >= a.Hq * a.C) return;
  const int h = row / a.C, c = row % a.C, e0 = (threadIdx.x % TPR) * 8;
  const int ns = a.nsplit;
  auto prow = [&](int s) { return ((int64_t)s * a.Hq + h) * a.Cpad + c; };
  float M = -INFINITY;
  for (int s0 = 0; s0 < ns; s0 += U) {
    float m[U];
#pragma unroll
    for (int u = 0; u < U; ++u) m[u] = a.pml[2 * prow(min(s0 + u, ns - 1))];
#pragma unroll
    for (int u = 0; u < U; ++u) M = fmaxf(M, m[u]);   // clamped repeats do not change a max
  }
  float L = 0.f, o[8] = {};
  for (int s0 = 0; s0 < ns; s0 += U) {
    float ms[U], ls[U];
    uint4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t pr = prow(min(s0 + u, ns - 1));
      ms[u] = a.pml[2 * pr];
      ls[u] = a.pml[2 * pr + 1];
      x[u] = *(const uint4 *)(a.po + pr * HD + e0);   // eight bf16
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {                  // branch-free: clamped repeats weigh 0
      const float e = exp2_fast(ms[u] - M);
      const float w = (s0 + u < ns && ms[u] != -INFINITY) ? e : 0.f;
      L += ls[u] * w;
      const uint32_t wd[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        o[2 * k] += __uint_as_float(wd[k] << 16) * w;
        o[2 * k + 1] += __uint_as_float(wd[k] & 0xffff0000u) * w;
      }
    }
  }
  const float inv = 1.f / L;
  uint4 out;
  out.x = pack_bf16x2(o[0] * inv, o[1] * inv);
  out.y = pack_bf16x2(o[2] * inv, o[3] * inv);
  out.z = pack_bf16x2(o[4] * inv, o[5] * inv);
  out.w = pack_bf16x2(o[6] * inv, o[7] * inv);
  *(uint4 *)(a.O + (int64_t)c * a.Hq * HD + h * HD + e0) = out;
}

template <int HD, bool CAUSAL>
hipError_t launch(const AttnArgs &a, hipStream_t st) {
  static std::atomic<bool> attr[DG_MAX_DEVICES];
  hipError_t e = dg_smem_attr_once(attr, Cfg<HD>::SMEM, {(const void *)attn_split_kernel<HD, CAUSAL>});
  if (e != hipSuccess) return e;
  const int G = a.Hq / a.Hkv;
  const int nq = (G * a.C + QB - 1) / QB;
  const int ntc = (a.C + KT - 1) / KT;
  const int ntiles = ntc + (int)((a.P + KT - 1) / KT);
  const int units = a.Hkv * a.nsplit;
  hipLaunchKernelGGL((attn_split_kernel<HD, CAUSAL>), dim3(units * nq), dim3(NW * 64), Cfg<HD>::SMEM,
                     st, a, nq, ntc, ntiles, units);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int RPB = 256 / (HD / 8);
  hipLaunchKernelGGL(attn_merge_kernel<HD>, dim3((a.Hq * a.C + RPB - 1) / RPB), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t dg_launch_attention(const AttnArgs &a, hipStream_t st) {
  if (a.causal) {
    switch (a.hd) {
      case 16: return launch<16, true>(a, st);
      case 32: return launch<32, true>(a, st);
      case 64: return launch<64, true>(a, st);
      case 128: return launch<128, true>(a, st);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.hd) {
    case 16: return launch<16, false>(a, st);
    case 32: return launch<32, false>(a, st);
    case 64: return launch<64, false>(a, st);
    case 128: return launch<128, false>(a, st);
    default: return hipErrorInvalidValue;
  }
}
