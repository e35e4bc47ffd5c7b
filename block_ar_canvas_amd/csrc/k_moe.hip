// Canvas MoE FFN: router top-K, token grouping by expert, combine.
//
// Method (DiffusionGemma Technical Report page, "Prerequisites", mixture of experts: each
// token uses 8 of 128 experts plus one shared expert, and a 256-token canvas touches
// about 84 distinct experts where one token touches 8; "Text diffusion models" survey,
// section 13: router top-k, expert GEMM, token permutation). The router logits and the
// shared expert use the plain GEMM; the kernels here route, group, run the routed
// experts and combine.
//
// moe_route_kernel: one workgroup per token; each thread holds one expert's logit (float32,
//   the router GEMM's k parts added in order) and counts the experts that beat it (larger logit, or equal
//   with a lower id); rank < K selects it. Gates: softmax over the K selected logits.
// moe_group_kernel: one workgroup; per expert, the number of tokens routed to it, the
//   exclusive offsets, the token list in token order (from per-expert token bitmasks:
//   deterministic), and for every (token, rank) the row of its expert output in grouped
//   order.
//   It also lists the work tiles of the expert GEMMs: one entry (expert, 32-row block) per
//   non-empty row block of every group.
// moe_expert_kernel: Y[off[e] + m] = act(X_e[m] . W[e]^T) for the grouped rows of
//   expert e. The weights are read once per tile, straight from memory into the MFMA A
//   tile: 128 weight rows and at most 32 grouped rows, both copied straight into LDS.
// moe_combine_kernel: y[t] = bf16(sum over ranks k of gate[t][k] * Yg[pos[t][k]] + Ys[t]),
//   float32, ranks in order.
#include <float.h>

#include "dg_common.h"

namespace {

__global__ __launch_bounds__(256) void moe_route_kernel(const float *logits, int splits, int64_t pstride,
                                                        int E, int K, int *sel, float *gate) {
  __shared__ float lv[256];
  __shared__ float sv[32];
  const int t = blockIdx.x, tid = threadIdx.x;
  float v = -INFINITY;
  if (tid < E) {
    // up to 8 parts, loaded together (a clamped index keeps every load valid), added in order
    float p[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) p[s] = logits[min(s, splits - 1) * pstride + (int64_t)t * E + tid];
    v = p[0];
#pragma unroll
    for (int s = 1; s < 8; ++s)
      if (s < splits) v += p[s];
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
                                                        int *perm, int *pos, int *nact, int *tiles) {
  extern __shared__ uint32_t mask[];                 // [E][W], W = C / 32 rounded up
  __shared__ int loff[257];
  const int tid = threadIdx.x, n = C * K, W = (C + 31) / 32;
  // this thread's selections (n <= 8192: at most 32), loaded once and kept in registers
  int es[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) es[j] = sel[min(tid + 256 * j, n - 1)];
  for (int i = tid; i < E * W; i += 256) mask[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const int i = tid + 256 * j;
    if (i < n) atomicOr(&mask[es[j] * W + ((i / K) >> 5)], 1u << ((i / K) & 31));
  }
  __syncthreads();
  // per expert: rows, 32-row tiles and a non-empty flag, packed as 14 + 9 + 9 bits (the
  // totals stay at most 8192 rows, 504 tiles and 256 experts); one inclusive scan
  // (Hillis-Steele over the 256 threads) gives every offset at once
  __shared__ uint32_t scan[256];
  uint32_t v = 0;
  if (tid < E) {
    int c = 0;
    for (int w = 0; w < W; ++w) c += __popc(mask[tid * W + w]);
    v = (uint32_t)c | ((uint32_t)((c + MOE_TM - 1) / MOE_TM) << 14) | ((c > 0 ? 1u : 0u) << 23);
  }
  scan[tid] = v;
  __syncthreads();
  for (int dd = 1; dd < 256; dd <<= 1) {
    const uint32_t add = tid >= dd ? scan[tid - dd] : 0u;
    __syncthreads();
    scan[tid] += add;
    __syncthreads();
  }
  const uint32_t incl = scan[tid], excl = incl - v;
  if (tid < E) {
    const int o = (int)(excl & 0x3FFF), t0 = (int)((excl >> 14) & 0x1FF), nt = (int)((v >> 14) & 0x1FF);
    loff[tid] = o;
    off[tid] = o;
    for (int mt = 0; mt < nt; ++mt) tiles[1 + t0 + mt] = tid | (mt << 16);
  }
  if (tid == 255) {
    off[E] = (int)(incl & 0x3FFF);
    tiles[0] = (int)((incl >> 14) & 0x1FF);
    if (nact) nact[0] = (int)(incl >> 23);
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const int i = tid + 256 * j;
    if (i >= n) break;
    const int t = i / K, e = es[j];
    const uint32_t *m = mask + e * W;
    int p = loff[e];
    for (int w = 0; w < (t >> 5); ++w) p += __popc(m[w]);
    p += __popc(m[t >> 5] & ((1u << (t & 31)) - 1u));
    perm[p] = t;
    pos[i] = p;
  }
}

DG_DEV f32x4_t mfma_16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// One workgroup = 4 waves = 128 weight rows of one tile (expert e, rows [m0, m0 + 32) of
// its group); wave w computes weight rows [32w, 32w + 32) as two 16-row A operands.
// v_mfma_f32_16x16x32_bf16: lane l supplies row l % 16 of A (and column l % 16 of B) with
// 8 k values; lane group g = l / 16 takes k [32j + 8g, +8) of the chunk in step j for
// both operands. Accumulator register i of lane l holds D[4(l / 16) + i][l % 16].
//
// Both operands come through LDS by direct global -> LDS copies (the weights once, the
// activations once per workgroup): a stage holds a 128-deep chunk of the 128 weight rows
// (32 KiB) and of the 32 activation rows (8 KiB), 256 bytes per row with its 16-byte
// chunks XOR-swizzled by the row's low 4 bits. Two stages: the next chunk's copies are in
// flight while the MFMAs read the current one. Every wave issues the same copies every
// stage (8 of weight rows, and the 0-2 of activation rows that reach into the tile; rows
// past the group repeat its last row, k past K repeats the last 16 bytes), so one
// s_waitcnt vmcnt(8 + those) waits for the current stage. 80 KiB of LDS per workgroup:
// two workgroups per CU.
constexpr int XW = 128 * 256, XX = MOE_TM * 256, XSTAGE = XW + XX, XSMEM = 2 * XSTAGE;

// LDS byte offset of 16-byte chunk q (of 16) of a 256-byte row: XOR-swizzled by the row's
// low 4 bits, so the 16 rows one operand read touches fall in distinct bank groups.
DG_DEV int xswz(int row, int q) { return row * 256 + ((q ^ (row & 15)) << 4); }

__global__ __launch_bounds__(256) void moe_expert_kernel(MoeGemmArgs a) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int NB = (a.N + 127) / 128;
  const int ti = blockIdx.x / NB, nb = blockIdx.x % NB;
  if (ti >= a.tiles[0]) return;
  const int tile = a.tiles[1 + ti], e = tile & 0xFFFF, m0 = (tile >> 16) * MOE_TM;
  const int o0 = a.off[e], mrows = min(MOE_TM, a.off[e + 1] - o0 - m0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int K = a.K, nch = (K + 127) / 128;
  const int nw0 = nb * 128, n0 = nw0 + 32 * wave;
  const int nbop = (mrows + 15) >> 4;                // B operands (16 rows each) in use

  // copy sources: instruction i of this wave fills 4 rows x 256 bytes; lane l covers row
  // base + l / 16 and loads global chunk (l & 15) ^ (row & 15) into LDS slot l & 15
  const u16 *wsrc[8], *xsrc[2];
  int wch[8], xch[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int R = 32 * wave + 4 * i + (lane >> 4);
    wch[i] = 8 * ((lane & 15) ^ (R & 15));
    wsrc[i] = a.W + ((int64_t)e * a.N + min(nw0 + R, a.N - 1)) * K;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int R = 8 * wave + 4 * i + (lane >> 4);
    xch[i] = 8 * ((lane & 15) ^ (R & 15));
    const int mm = m0 + min(R, mrows - 1);
    const int row = a.perm ? a.perm[o0 + mm] : o0 + mm;
    xsrc[i] = a.X + (int64_t)row * K;
  }
  // activation copies of this wave: rows [8w + 4i, +4) are copied only when the first of
  // them is in the tile (wave-uniform); rows past the tile are never stored, so what LDS
  // holds there does not matter
  const int nx = __builtin_amdgcn_readfirstlane(min(2, max(0, (mrows - 8 * wave + 3) >> 2)));
  const uint32_t lbase = lds_addr(smem);
  auto issue = [&](int ch) {
    const uint32_t sb = lbase + (uint32_t)((ch & 1) * XSTAGE);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      dma16(wsrc[i] + min(ch * 128 + wch[i], K - 8), sb + (uint32_t)((32 * wave + 4 * i) * 256));
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (i < nx) dma16(xsrc[i] + min(ch * 128 + xch[i], K - 8), sb + (uint32_t)(XW + (8 * wave + 4 * i) * 256));
  };
  // this wave's copies per stage: 8 weight copies plus its activation copies in flight
  auto wait_current = [&](bool more) {
    if (!more) {
      dma_wait<0>();
    } else if (nx == 2) {
      dma_wait<10>();
    } else if (nx == 1) {
      dma_wait<9>();
    } else {
      dma_wait<8>();
    }
  };

  f32x4_t acc[2][2] = {};
  issue(0);
  for (int ch = 0; ch < nch; ++ch) {
    if (ch + 1 < nch) issue(ch + 1);
    wait_current(ch + 1 < nch);
    __syncthreads();
    const uint8_t *Ws = smem + (ch & 1) * XSTAGE, *Xs = Ws + XW;
    const int nj = min(4, (K - ch * 128) >> 5);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < nj) {
        const int q = 4 * j + g;
        u32x4_t av[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) av[s] = *(const u32x4_t *)(Ws + xswz(32 * wave + 16 * s + r16, q));
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          if (b < nbop) {
            const u32x4_t bv = *(const u32x4_t *)(Xs + xswz(16 * b + r16, q));
            acc[0][b] = mfma_16x16x32(av[0], bv, acc[0][b]);
            acc[1][b] = mfma_16x16x32(av[1], bv, acc[1][b]);
          }
        }
      }
    }
    __syncthreads();                                 // stage ch & 1 is refilled next round
  }
  if (n0 >= a.N) return;                             // wave past the output width

  // lane l, register i of acc[s][b]: D[n0 + 16s + 4g + i][m0 + 16b + r16]
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int mc = 16 * b + r16;
    if (b >= nbop || mc >= mrows) continue;
    u16 *yp = a.Y + (int64_t)(o0 + m0 + mc) * a.ldY + n0 + 4 * g;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float t = acc[s][b][i];
        if (a.gelu) t = 0.5f * t * (1.0f + erff(t * 0.70710678118654752f));
        v[i] = t;
      }
      uint2 o;
      o.x = pack_bf16x2(v[0], v[1]);
      o.y = pack_bf16x2(v[2], v[3]);
      *(uint2 *)(yp + 16 * s) = o;
    }
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

hipError_t dg_launch_moe_route(const float *logits, int splits, int C, int E, int K, int *sel, float *gate,
                               hipStream_t st) {
  hipLaunchKernelGGL(moe_route_kernel, dim3(C), dim3(256), 0, st, logits, splits, (int64_t)C * E, E, K, sel,
                     gate);
  return hipGetLastError();
}

hipError_t dg_launch_moe_group(const int *sel, int C, int K, int E, int *off, int *perm, int *pos,
                               int *nact, int *tiles, hipStream_t st) {
  hipLaunchKernelGGL(moe_group_kernel, dim3(1), dim3(256), (size_t)E * ((C + 31) / 32) * 4, st, sel, C,
                     K, E, off, perm, pos, nact, tiles);
  return hipGetLastError();
}

hipError_t dg_launch_moe_expert(const MoeGemmArgs &a, hipStream_t st) {
  if (a.N < 32 || a.N % 32 || a.K < 32 || a.K % 32 || a.max_tiles < 1) return hipErrorInvalidValue;
  static std::atomic<bool> attr[DG_MAX_DEVICES];
  const hipError_t e = dg_smem_attr_once(attr, XSMEM, {(const void *)moe_expert_kernel});
  if (e != hipSuccess) return e;
  const int NB = (a.N + 127) / 128;
  hipLaunchKernelGGL(moe_expert_kernel, dim3(a.max_tiles * NB), dim3(256), XSMEM, st, a);
  return hipGetLastError();
}

hipError_t dg_launch_moe_combine(const u16 *Yg, const u16 *Ys, const float *gate, const int *pos,
                                 int C, int K, int d, u16 *Y, hipStream_t st) {
  hipLaunchKernelGGL(moe_combine_kernel, dim3(C), dim3(256), 0, st, Yg, Ys, gate, pos, K, d, Y);
  return hipGetLastError();
}
