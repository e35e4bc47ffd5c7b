// Device routines of acceptance, renoise and the stop test, shared by their own kernels,
// by the one-launch kernel of the three, and by the self-conditioning reduce, which can
// run the three as extra workgroups. Every result is an integer computed by the same
// code wherever it runs, so the placements agree bit for bit.
#pragma once

#include "dg_common.h"

namespace dgs {

constexpr float H_LIMIT = 65536.0f;
constexpr uint64_t Q_SENTINEL = 1ull << 48;

// Fixed-point entropy; out-of-domain entropies (NaN, +Inf, >= 2^16) get the sentinel.
DG_DEV uint64_t entropy_q(float h) {
  if (!(h < H_LIMIT)) return Q_SENTINEL;
  if (!(h > 0.f)) return 0;
  return (uint64_t)ceil((double)h * 4294967296.0);
}

// Acceptance of one canvas, workgroup-wide (one barrier inside): tpp threads per
// position (1, 2 or 4; tpp * C <= 1024) share that position's sum; h is position pos's
// entropy (read by the caller, unused for pos >= C). Returns whether position pos is
// accepted (the same answer in all tpp threads); q receives the position's fixed-point
// entropy, the sentinel for an entropy outside the domain.
DG_DEV bool accept_rank(int C, int tpp, int pos, int sub, float h, uint64_t budget,
                        ulonglong2 *kq, uint64_t &q_out) {
  uint64_t key = ~0ull, q = 0;
  if (pos < C) {
    uint32_t bits;
    if (!(h < H_LIMIT)) bits = 0xFFFFFFFFu;
    else bits = h > 0.f ? __float_as_uint(h) : 0u;
    key = ((uint64_t)bits << 32) | (uint32_t)pos;
    q = bits == 0xFFFFFFFFu ? Q_SENTINEL : entropy_q(__uint_as_float(bits));
    if (sub == 0) kq[pos] = make_ulonglong2(key, q);
  }
  __syncthreads();
  // The inclusive scan of q in ascending key order, evaluated at this position's own
  // place in that order: the sum of q over all keys <= this key (keys are distinct).
  // The tpp threads of a position take every tpp-th key; integer sums, so the split
  // and its order do not change the result.
  uint64_t sum = 0, sum2 = 0;
  int j = sub;
#pragma unroll 4
  for (; j + tpp < C; j += 2 * tpp) {
    const ulonglong2 v = kq[j], w = kq[j + tpp];
    sum += v.x <= key ? v.y : 0ull;
    sum2 += w.x <= key ? w.y : 0ull;
  }
  if (j < C) sum += kq[j].x <= key ? kq[j].y : 0ull;
  sum += sum2;
  for (int o = 1; o < tpp; o <<= 1) sum += __shfl_xor(sum, o);
  q_out = q;
  return pos < C && sum <= budget;
}

// Philox4x64-10.
DG_DEV void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t hi0 = __umul64hi(M0, c[0]), lo0 = M0 * c[0];
    const uint64_t hi1 = __umul64hi(M1, c[2]), lo1 = M1 * c[2];
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
    k0 += W0;
    k1 += W1;
  }
}

// A token drawn uniformly over [0, V): floor(r V / 2^64), r = word 0 of Philox4x64-10
// under key (seed, canvas) and counter (position, step, stream, 0).
DG_DEV int uniform_token(int pos, uint32_t step, uint64_t stream, uint64_t seed, uint32_t canvas, int V) {
  uint64_t c[4] = {(uint64_t)pos, (uint64_t)step, stream, 0ull};
  philox4x64_10(c, seed, (uint64_t)canvas);
  return (int)__umul64hi(c[0], (uint64_t)V);
}

// Stop flag: 1 = stop, else 2 at the step cap, else 0. A system-scope store: the flag
// may live in pinned host memory that the host polls.
DG_DEV void store_flag(int *flag, bool stop, int step, int N) {
  __hip_atomic_store(flag, stop ? 1 : (step >= N - 1 ? 2 : 0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Acceptance, renoise and stop test of canvas b by the calling workgroup (blockDim.x
// threads, a.tpp * a.C <= blockDim.x <= 1024): the same arithmetic as accept_kernel,
// renoise_kernel (stream 0) and stop_kernel run in that order. Every position is
// handled by one thread (sub == 0), which reads only its own x0, argmax and previous
// argmax. The draw and those reads do not depend on the acceptance, so they are issued
// first, their latency and the draw's arithmetic overlapping the read of the entropies.
DG_DEV void ars_canvas(const ArsArgs &a, int b) {
  __shared__ ulonglong2 kq[1024];
  __shared__ int sdraw[1024];
  __shared__ uint64_t ssum[16];
  __shared__ int sok[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pos = tid / a.tpp, sub = tid % a.tpp;
  const int64_t o = (int64_t)b * a.C + pos;
  const bool own = pos < a.C && sub == 0;
  const float h = pos < a.C ? a.ent[o] : 0.f;
  int keep = 0, ok = 1;
  if (own) {
    keep = a.x0[o];
    if (a.prev && a.am[o] != a.prev[o]) ok = 0;
  }
  // thread t draws for position t (whole waves busy), published through LDS; the
  // acceptance's barrier orders it before the reads below
  if (tid < a.C)
    sdraw[tid] = uniform_token(tid, (uint32_t)a.step, 0ull, a.seed, a.canvas_base + (uint32_t)b, a.V);
  uint64_t q;
  const bool take = accept_rank(a.C, a.tpp, pos, sub, h, a.budget, kq, q);
  uint64_t s = 0;
  if (own) {
    a.acc[o] = take ? 1 : 0;
    a.tok[o] = take ? keep : sdraw[pos];
    // stop-test terms: q is ceil(h 2^32) for an entropy in the domain (as the stop
    // test sums it) and the sentinel for one outside it (which blocks the stop)
    if (q == Q_SENTINEL) ok = 0;
    else s = q;
  }
  for (int off = 32; off > 0; off >>= 1) {           // integer sums: order-free
    s += __shfl_xor(s, off);
    ok &= __shfl_xor(ok, off);
  }
  if (lane == 0) {
    ssum[wave] = s;
    sok[wave] = ok;
  }
  const int n = __syncthreads_count(take && sub == 0);
  if (tid == 0) {
    uint64_t tot = 0;
    int all = 1;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
      tot += ssum[w];
      all &= sok[w];
    }
    a.nacc[b] = n;
    store_flag(a.flag + b, a.step >= 1 && a.prev != nullptr && all && tot <= a.limit, a.step, a.N);
  }
}

}  // namespace dgs
