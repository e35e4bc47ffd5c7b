// Integer part of the sampler: acceptance, renoise, stop test.
//
// Entropy-bounded acceptance (DiffusionGemma Technical Report page, "Method steps"
// (3): sort by entropy ascending and accept within the cumulative entropy budget
// b = 0.1; "Technical novelty": MaskGIT-like entropy-bounded acceptance). The budget
// sum runs in 2^-32 fixed point, q = ceil(h * 2^32) and budget floor(b * 2^32), so a
// parallel scan gives the same bits as a sequential loop and the accepted real-valued
// entropy sum never exceeds b. One workgroup per canvas. The 64-bit sort keys
// (entropy bits << 32 | position) are distinct, so the inclusive scan of q in
// ascending key order, taken at a position's own place, is the sum of q over all keys
// not above its key: each thread evaluates that sum directly over the canvas (no sort
// is materialised). Since q >= 0 the scan is monotone, and the accepted set is the
// sorted prefix whose scan stays within the budget.
//
// Uniform renoise (Technical Report page, "Method steps" (2)-(3); Google
// "DiffusionGemma explained", "Uniform State Diffusion"): rejected positions get a
// token drawn uniformly from the whole vocabulary. The generator is Philox4x64-10
// (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11),
// counter-based, so every (seed, canvas, step, position) draw is independent of
// launch shape and a resumed run needs no generator state.
//
// Stop test (Technical Report page, "Method steps" (4)): the canvas stops when its
// mean entropy is <= the threshold and the argmax did not change since the previous
// step; the step cap commits anyway.
//
// accept_renoise_stop_kernel runs acceptance, renoise and the stop test of a step in one
// launch. The routines are in dg_sampler_dev.h, shared with the three kernels here and
// with the self-conditioning reduce, which can run them beside itself; every placement
// gives the three kernels' results bit for bit.
//
// Confidence-ranked acceptance (the openai-hub page "从零拆开DiffusionGemma", step 4,
// confidence decoding; the "Text diffusion models" survey, section 5): each step keeps
// the k positions the model is most confident about. Same rank construction as the
// entropy rule: distinct 64-bit keys (score order, position), rank = keys below one's
// own, accepted iff rank < k.
//
// Sampled tokens (same openai-hub step: real samplers draw from the tempered
// distribution instead of taking the argmax): x~ ~ p0 by inverse CDF over the whole
// vocabulary in id order, with one uniform u = (word 0 of counter (position, step, 2, 0)
// >> 11) / 2^53 per position: the token is the first id whose cumulative probability
// exceeds u times the total. Here in two levels that reach the same id: (1) the logits
// tile t (256 ids) holding the crossing, from the running sum of the tile masses
// M_t = Z_t 2^(rho_t - R) (float32 tile sums, prefix in float64); (2) inside the tile,
// the first id whose running sum of the stored bf16 p~_v = 2^(x_v - rho_t) exceeds the
// rest of the target, rescaled to the tile's units by the exact power 2^(R - rho_t).
#include <float.h>

#include <climits>

#include "dg_sampler_dev.h"

namespace {

using namespace dgs;

__global__ __launch_bounds__(1024) void accept_kernel(int C, int tpp, const float *ent,
                                                      uint64_t budget, uint8_t *acc, int *nacc) {
  __shared__ ulonglong2 kq[1024];                    // (sort key, fixed-point entropy)
  const int b = blockIdx.x, tid = threadIdx.x;
  const int pos = tid / tpp, sub = tid % tpp;
  const float h = pos < C ? ent[(int64_t)b * C + pos] : 0.f;
  uint64_t q;
  const bool take = accept_rank(C, tpp, pos, sub, h, budget, kq, q);
  if (pos < C && sub == 0) acc[(int64_t)b * C + pos] = take ? 1 : 0;
  const int n = __syncthreads_count(take && sub == 0);
  if (tid == 0 && nacc) nacc[b] = n;
}

// Order-preserving code of a float score (ascending score = ascending code).
DG_DEV uint32_t score_code(float s) {
  const uint32_t b = __float_as_uint(s);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// tpp threads per position as in accept_kernel. Keys: (~code(score) << 32 | position),
// so ascending keys = descending score, ties to the lower position; NaN scores get the
// largest keys and are never accepted.
__global__ __launch_bounds__(1024) void topk_kernel(int C, int tpp, const float *score, int k,
                                                    uint8_t *acc, int *nacc) {
  __shared__ uint64_t keys[1024];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int pos = tid / tpp, sub = tid % tpp;
  uint64_t key = ~0ull;
  bool valid = false;
  if (pos < C) {
    const float s = score[(int64_t)b * C + pos];
    valid = s == s;
    const uint32_t hi = valid ? ~score_code(s) : 0xFFFFFFFFu;
    key = ((uint64_t)hi << 32) | (uint32_t)pos;
    if (sub == 0) keys[pos] = key;
  }
  __syncthreads();
  int rank = 0, rank2 = 0;
  int j = sub;
#pragma unroll 4
  for (; j + tpp < C; j += 2 * tpp) {
    rank += keys[j] < key ? 1 : 0;
    rank2 += keys[j + tpp] < key ? 1 : 0;
  }
  if (j < C) rank += keys[j] < key ? 1 : 0;
  rank += rank2;
  for (int o = 1; o < tpp; o <<= 1) rank += __shfl_xor(rank, o);
  const bool take = pos < C && valid && rank < k;
  if (pos < C && sub == 0) acc[(int64_t)b * C + pos] = take ? 1 : 0;
  const int n = __syncthreads_count(take && sub == 0);
  if (tid == 0 && nacc) nacc[b] = n;
}

__global__ __launch_bounds__(256) void renoise_kernel(int B, int C, int V, const int *am,
                                                      const uint8_t *acc, uint64_t seed,
                                                      uint32_t canvas_base, uint32_t step,
                                                      int *tok) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)B * C) return;
  const int b = (int)(i / C), pos = (int)(i % C);
  if (acc && acc[i]) {
    tok[i] = am[i];
    return;
  }
  tok[i] = uniform_token(pos, step, acc ? 0ull : 1ull, seed, canvas_base + (uint32_t)b, V);
}

// One workgroup per canvas column (canvas b = column / Cs, position = column % Cs).
__global__ __launch_bounds__(256) void sample_kernel(SampleArgs a) {
  __shared__ double swave[4];
  __shared__ double sbefore;
  __shared__ int st_star;
  __shared__ int sfirst[4], slast[4];
  const int c = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = c / a.Cs, pos = c % a.Cs;
  const uint64_t key1 = (uint64_t)(a.canvas_base + (uint32_t)b);
  const float R = a.colR[c];
  if (!(fabsf(R) <= FLT_MAX)) {                       // non-finite logits (status already set)
    if (tid == 0) a.tokens[c] = 0;
    return;
  }
  const float *tz = a.tsum + (int64_t)c * a.T;
  const float *tr = a.trho + (int64_t)c * a.T;
  auto mass = [&](int t) { return (double)tz[t] * ldexp(1.0, (int)(tr[t] - R)); };

  // (1) the tile: thread tid owns tiles [t0, t1); masses summed in tile order
  const int per = (a.T + 255) / 256;
  const int t0 = min(tid * per, a.T), t1 = min(t0 + per, a.T);
  double loc = 0.0;
  for (int t = t0; t < t1; ++t) loc += mass(t);
  // exclusive prefix of the per-thread sums: a wave scan, then the wave totals in order
  // (a fixed association, so every run gives the same bits)
  double incl = loc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  double ex = __shfl_up(incl, 1);
  if (lane == 0) ex = 0.0;
  if (lane == 63) swave[wave] = incl;
  if (tid == 0) st_star = -1;
  __syncthreads();
  double woff = 0.0;
  for (int i = 0; i < wave; ++i) woff += swave[i];
  const double total = ((swave[0] + swave[1]) + swave[2]) + swave[3];
  uint64_t w[4] = {(uint64_t)pos, (uint64_t)a.step, 2ull, 0ull};
  philox4x64_10(w, a.seed, key1);
  const double u = (double)(w[0] >> 11) * 0x1.0p-53;
  const double target = u * total;
  const double excl = woff + ex;
  if (t0 < t1 && excl <= target && excl + loc > target) {
    double run = excl;
    int t = t0;
    for (; t < t1 - 1; ++t) {
      const double next = run + mass(t);
      if (next > target) break;
      run = next;
    }
    st_star = t;                                     // exactly one thread crosses
    sbefore = run;                                   // mass of the tiles before t
  }
  __syncthreads();
  int ts = st_star;
  const bool past_end = ts < 0;                      // rounding left target >= total:
  if (past_end) {                                    // the last id with mass
    ts = a.T - 1;
    while (ts > 0 && !(mass(ts) > 0.0)) --ts;
  }
  // the rest of the target in the tile's own units (p~ sums to about Z_t there)
  const double rest = past_end ? INFINITY : (target - sbefore) * ldexp(1.0, (int)(R - tr[ts]));

  // (2) inverse CDF inside the tile: inclusive running sum of p~ over the tile's ids
  const int v = ts * 256 + tid;
  double pv = 0.0;
  if (v < a.V) {
    const int64_t off = (((int64_t)(c >> 5) * a.VS + (v >> 4)) * 64 + ((v & 15) >> 3) * 32 + (c & 31)) * 8 + (v & 7);
    pv = (double)__uint_as_float((uint32_t)a.ptilde[off] << 16);
  }
  double cum = pv;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(cum, o);
    if (lane >= o) cum += y;
  }
  __syncthreads();                                   // swave reuse
  if (lane == 63) swave[wave] = cum;
  __syncthreads();
  for (int i = 0; i < wave; ++i) cum += swave[i];
  // the first id whose running sum exceeds the rest (it has p~ > 0); if rounding left
  // none, the last id with p~ > 0
  const uint64_t over = __ballot(cum > rest);
  const uint64_t pos_mask = __ballot(pv > 0.0);
  if (lane == 0) {
    sfirst[wave] = over ? wave * 64 + __builtin_ctzll(over) : INT_MAX;
    slast[wave] = pos_mask ? wave * 64 + 63 - __builtin_clzll(pos_mask) : -1;
  }
  __syncthreads();
  if (tid == 0) {
    int first = INT_MAX, last = -1;
    for (int i = 0; i < 4; ++i) {
      first = min(first, sfirst[i]);
      last = max(last, slast[i]);
    }
    const int j = first != INT_MAX ? first : (last >= 0 ? last : 0);
    a.tokens[c] = ts * 256 + j;
  }
}

__global__ __launch_bounds__(256) void stop_kernel(int C, const float *ent, const int *am,
                                                   const int *prev, uint64_t limit, int step,
                                                   int N, int *flag) {
  __shared__ uint64_t ssum[4];
  __shared__ int sok[4];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t s = 0;
  int ok = 1;
  for (int i = tid; i < C; i += 256) {
    const int64_t o = (int64_t)b * C + i;
    const float h = ent[o];
    if (!(h < H_LIMIT)) ok = 0;
    else s += entropy_q(h);
    if (prev && am[o] != prev[o]) ok = 0;
  }
  // integer sums: any reduction order gives the same bits
  for (int o = 32; o > 0; o >>= 1) {
    s += __shfl_xor(s, o);
    ok &= __shfl_xor(ok, o);
  }
  if (lane == 0) {
    ssum[wave] = s;
    sok[wave] = ok;
  }
  __syncthreads();
  if (tid == 0) {
    const uint64_t tot = ssum[0] + ssum[1] + ssum[2] + ssum[3];
    const int all = sok[0] & sok[1] & sok[2] & sok[3];
    store_flag(flag + b, step >= 1 && prev != nullptr && all && tot <= limit, step, N);
  }
}

__global__ __launch_bounds__(1024) void accept_renoise_stop_kernel(ArsArgs a) { ars_canvas(a, blockIdx.x); }

}  // namespace

hipError_t dg_launch_accept(int B, int C, const float *ent, uint64_t budget, uint8_t *acc,
                            int *nacc, hipStream_t st) {
  // C <= 1024 (checked by the caller); up to 4 threads per position
  const int tpp = C <= 256 ? 4 : C <= 512 ? 2 : 1;
  const int n = (C * tpp + 63) / 64 * 64;
  hipLaunchKernelGGL(accept_kernel, dim3(B), dim3(n), 0, st, C, tpp, ent, budget, acc, nacc);
  return hipGetLastError();
}

hipError_t dg_launch_topk(int B, int C, const float *score, int k, uint8_t *acc, int *nacc,
                          hipStream_t st) {
  // C <= 1024 (checked by the caller); up to 4 threads per position
  const int tpp = C <= 256 ? 4 : C <= 512 ? 2 : 1;
  const int n = (C * tpp + 63) / 64 * 64;
  hipLaunchKernelGGL(topk_kernel, dim3(B), dim3(n), 0, st, C, tpp, score, k, acc, nacc);
  return hipGetLastError();
}

hipError_t dg_launch_sample(const SampleArgs &a, hipStream_t st) {
  hipLaunchKernelGGL(sample_kernel, dim3(a.B * a.Cs), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t dg_launch_renoise(int B, int C, int V, const int *am, const uint8_t *acc,
                             uint64_t seed, uint32_t canvas_base, uint32_t step, int *tok,
                             hipStream_t st) {
  const int64_t n = (int64_t)B * C;
  hipLaunchKernelGGL(renoise_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, B, C, V,
                     am, acc, seed, canvas_base, step, tok);
  return hipGetLastError();
}

hipError_t dg_launch_stop(int B, int C, const float *ent, const int *am, const int *prev,
                          uint64_t limit, int step, int N, int *flag, hipStream_t st) {
  hipLaunchKernelGGL(stop_kernel, dim3(B), dim3(256), 0, st, C, ent, am, prev, limit, step, N, flag);
  return hipGetLastError();
}

hipError_t dg_launch_accept_renoise_stop(const ArsArgs &r, hipStream_t st) {
  // C <= 1024 (checked by the caller); up to 4 threads per position as in acceptance
  ArsArgs a = r;
  a.tpp = a.C <= 256 ? 4 : a.C <= 512 ? 2 : 1;
  const int n = (a.C * a.tpp + 63) / 64 * 64;
  hipLaunchKernelGGL(accept_renoise_stop_kernel, dim3(a.B), dim3(n), 0, st, a);
  return hipGetLastError();
}
