// Smoothing and quantisation kernels for gfx950.
//
//   Q and K: "SageAttention2 Technical Report" abstract (smooth Q; quantize Q, K
//   to INT4/INT8 with fine-grained scales; SageAttention's K smoothing among its
//   precision-enhancing methods) and the SageAttention2++ summary, section 2.1
//   (per-block scale factors for Q and K).
//   V: same abstract (smooth V; V to FP8) and section 2.1 (per-channel scaling).
//
// Every value that decides a code is computed in IEEE fp32 with round to
// nearest even and no contraction, and every mean uses one fixed summation
// tree (pairwise in token order, +0.0 padding up to 128 * 2^k tokens), so the
// codes, scales and means are exactly reproducible on any implementation that
// follows the same definition.
//
// These kernels stream their inputs once per pass (plus the K and V statistic
// passes) and are bound by HBM bandwidth: loads are 16 bytes per lane over
// whole 128-token blocks, reductions stay in registers, lane butterflies and
// LDS.
#pragma clang fp contract(off)

#include "sage_internal.h"

namespace sage {
namespace {

constexpr int kThreads = 256;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Thread layout over a 128-token x D block: TPR threads share one token row
// (8 channels each); every thread holds TOK consecutive tokens.
template <int D>
struct Tile {
  static constexpr int TPR = D / 8;
  static constexpr int TOK = 128 * TPR / kThreads;
  static_assert(TOK >= 1 && (TOK & (TOK - 1)) == 0, "tokens per thread must be a power of two");
};

template <bool BF16>
__device__ __forceinline__ float to_f32(uint16_t b) {
  if constexpr (BF16) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
  } else {
    return static_cast<float>(__builtin_bit_cast(_Float16, b));
  }
}

// Load rows [row0, row0 + 128) of one head; rows >= N read as 0.
template <int D, bool BF16>
__device__ __forceinline__ void load_block(const uint16_t* __restrict__ base, int64_t sN, int row0, int N,
                                           float (&x)[Tile<D>::TOK][8]) {
  const int t = threadIdx.x;
  const int g = t / Tile<D>::TPR, cg = t % Tile<D>::TPR;
#pragma unroll
  for (int u = 0; u < Tile<D>::TOK; ++u) {
    const int r = row0 + g * Tile<D>::TOK + u;
    uint4 raw = make_uint4(0u, 0u, 0u, 0u);
    if (r < N) raw = *reinterpret_cast<const uint4*>(base + static_cast<int64_t>(r) * sN + 8 * cg);
    const uint16_t* hv = reinterpret_cast<const uint16_t*>(&raw);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[u][e] = to_f32<BF16>(hv[e]);
  }
}

// Pairwise tree over the block's 128 token positions, per channel: in-register
// pairs over each thread's TOK consecutive tokens, lane butterflies over
// neighbouring token groups (fp32 addition is commutative, so both partners
// hold identical bits), then the four 32-token wave sums as (w0+w1)+(w2+w3).
// On return every thread holds the sums of its 8 channels.  lds: 4*D floats.
template <int D>
__device__ __forceinline__ void block_tree_sum(const float (&x)[Tile<D>::TOK][8], float (&s)[8], float* lds) {
  constexpr int TOK = Tile<D>::TOK, TPR = Tile<D>::TPR;
  float v[TOK][8];
#pragma unroll
  for (int u = 0; u < TOK; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) v[u][e] = x[u][e];
#pragma unroll
  for (int step = 1; step < TOK; step <<= 1)
#pragma unroll
    for (int u = 0; u < TOK; u += 2 * step)
#pragma unroll
      for (int e = 0; e < 8; ++e) v[u][e] = v[u][e] + v[u + step][e];
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = v[0][e];
#pragma unroll
  for (int m = TPR; m < 64; m <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = s[e] + __shfl_xor(s[e], m);
  const int w = threadIdx.x / 64, lane = threadIdx.x % 64, cg = threadIdx.x % TPR;
  if (lane < TPR)
#pragma unroll
    for (int e = 0; e < 8; ++e) lds[w * D + 8 * lane + e] = s[e];
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = 8 * cg + e;
    s[e] = (lds[c] + lds[D + c]) + (lds[2 * D + c] + lds[3 * D + c]);
  }
  __syncthreads();
}

// Group of row r (0..127 inside a block) and the number of groups per block.
__device__ __forceinline__ int q_group_in_block(int gran, int r) {
  return gran == SAGE_GRAN_THREAD ? r : (gran == SAGE_GRAN_WARP ? (r >> 5) : 0);
}
__host__ __device__ __forceinline__ int q_groups_per_block(int gran) {
  return gran == SAGE_GRAN_THREAD ? 128 : (gran == SAGE_GRAN_WARP ? 4 : 1);
}
__device__ __forceinline__ int k_group_in_block(int gran, int r) {
  return gran == SAGE_GRAN_THREAD ? (2 * (r >> 5) + ((r & 7) >> 2)) : (r >> 6);
}
__host__ __device__ __forceinline__ int k_groups_per_block(int gran) { return gran == SAGE_GRAN_THREAD ? 8 : 2; }

// Smoothed rows xs -> codes and per-group scales (symmetric, round half to even).
// gmax: 128 unsigned in LDS.  Writes the block's codes (N_pad rows, so padded
// rows get 0) and its group scales.
template <int D, bool IS_Q>
__device__ __forceinline__ void quantize_block(const float (&xs)[Tile<D>::TOK][8], int gran, int qmax,
                                               unsigned* gmax, int8_t* __restrict__ codes_blk,
                                               float* __restrict__ scale_blk) {
  constexpr int TOK = Tile<D>::TOK, TPR = Tile<D>::TPR;
  const int t = threadIdx.x, g = t / TPR, cg = t % TPR;
  if (t < 128) gmax[t] = 0u;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < TOK; ++u) {
    float ra = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ra = fmaxf(ra, fabsf(xs[u][e]));
#pragma unroll
    for (int m = 1; m < TPR; m <<= 1) ra = fmaxf(ra, __shfl_xor(ra, m));
    const int r = g * TOK + u;
    const int grp = IS_Q ? q_group_in_block(gran, r) : k_group_in_block(gran, r);
    if (cg == 0) atomicMax(&gmax[grp], __float_as_uint(ra));  // non-negative floats order as unsigned
  }
  __syncthreads();
  const float qm = static_cast<float>(qmax);
  const int ng = IS_Q ? q_groups_per_block(gran) : k_groups_per_block(gran);
  if (t < ng) scale_blk[t] = __uint_as_float(gmax[t]) / qm;
#pragma unroll
  for (int u = 0; u < TOK; ++u) {
    const int r = g * TOK + u;
    const int grp = IS_Q ? q_group_in_block(gran, r) : k_group_in_block(gran, r);
    const float am = __uint_as_float(gmax[grp]);
    const float inv = am > 0.f ? qm / am : 0.f;
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float c = rintf(xs[u][e] * inv);
      c = fminf(fmaxf(c, -qm), qm);
      packed[e >> 2] |= (static_cast<uint32_t>(static_cast<int>(c)) & 0xffu) << (8 * (e & 3));
    }
    *reinterpret_cast<uint2*>(codes_blk + static_cast<int64_t>(r) * D + 8 * cg) = make_uint2(packed[0], packed[1]);
  }
}

struct QKArgs {
  const uint16_t* q;
  const uint16_t* k;
  int64_t qsB, qsH, qsN, ksB, ksH, ksN;
  sage_qk_buffers out;
  int H, N, n_pad, nblk, gran, qmax, smooth_q, smooth_k;
  float scale_log2;  // sm_scale * log2(e): the bias is stored in the exp2 domain
};

// Pass 1, one work-group per (128-token block, head): Q block mean, Q codes and
// scales; per-block K channel sums (subtrees of the K mean's tree).
template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) void q_quant_k_sums_kernel(QKArgs a) {
  __shared__ float lds[4 * D];
  __shared__ unsigned gmax[128];
  const int blk = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;
  const int row0 = blk * 128;
  const int t = threadIdx.x, g = t / Tile<D>::TPR, cg = t % Tile<D>::TPR;
  float x[Tile<D>::TOK][8];
  float s[8];

  // K block sums.
  load_block<D, BF16>(a.k + b * a.ksB + h * a.ksH, a.ksN, row0, a.N, x);
  block_tree_sum<D>(x, s, lds);
  if (g == 0)
#pragma unroll
    for (int e = 0; e < 8; ++e) a.out.k_partial[(static_cast<int64_t>(bh) * a.nblk + blk) * D + 8 * cg + e] = s[e];

  // Q block mean and codes.
  load_block<D, BF16>(a.q + b * a.qsB + h * a.qsH, a.qsN, row0, a.N, x);
  const int valid = min(128, a.N - row0);
  float mu[8];
  if (a.smooth_q) {
    block_tree_sum<D>(x, s, lds);
    const float cnt = static_cast<float>(valid);
#pragma unroll
    for (int e = 0; e < 8; ++e) mu[e] = s[e] / cnt;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) mu[e] = 0.f;
  }
  if (g == 0)
#pragma unroll
    for (int e = 0; e < 8; ++e) a.out.q_mean[(static_cast<int64_t>(bh) * a.nblk + blk) * D + 8 * cg + e] = mu[e];
#pragma unroll
  for (int u = 0; u < Tile<D>::TOK; ++u) {
    const bool ok = g * Tile<D>::TOK + u < valid;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[u][e] = ok ? x[u][e] - mu[e] : 0.f;
  }
  const int ngq = q_groups_per_block(a.gran);
  quantize_block<D, true>(x, a.gran, a.qmax, gmax, a.out.q_codes + (static_cast<int64_t>(bh) * a.n_pad + row0) * D,
                          a.out.q_scale + (static_cast<int64_t>(bh) * a.nblk + blk) * ngq);
}

// Binary-counter evaluation of the pairwise tree over n leaves padded with
// +0.0 up to the next power of two; leaves are read through `leaf(i)`.
template <typename F>
__device__ __forceinline__ float tree_over_blocks(int n, F leaf) {
  float stk[24];
  int lvl[24];
  int sp = 0;
  int P = 1;
  while (P < n) P <<= 1;
  for (int i = 0; i < P; ++i) {
    float x = i < n ? leaf(i) : 0.f;
    int L = 0;
    while (sp > 0 && lvl[sp - 1] == L) {
      x = stk[sp - 1] + x;
      --sp;
      ++L;
    }
    stk[sp] = x;
    lvl[sp] = L;
    ++sp;
  }
  return stk[0];
}

// K mean from the per-block sums: one thread per channel of one head.
template <int D>
__global__ __launch_bounds__(D) void k_mean_kernel(QKArgs a) {
  const int bh = blockIdx.x, c = threadIdx.x;
  const float* part = a.out.k_partial + static_cast<int64_t>(bh) * a.nblk * D + c;
  float mu = 0.f;
  if (a.smooth_k) {
    const float sum = tree_over_blocks(a.nblk, [&](int i) { return part[static_cast<int64_t>(i) * D]; });
    mu = sum / static_cast<float>(a.N);
  }
  a.out.k_mean[static_cast<int64_t>(bh) * D + c] = mu;
}

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Pass 2, one work-group per (128-key block, head): K' = K - mean, K codes and
// scales, then the bias dS[qb, j] = mu_Q(qb) . K'_j for the block's keys and
// every Q block, on the bf16 matrix cores with a three-product hi/lo split of
// both operands (about 16 significant bits), stored times sm_scale * log2(e).
template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) void k_quant_bias_kernel(QKArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* khi = reinterpret_cast<uint16_t*>(smem);        // [128][D]
  uint16_t* klo = khi + 128 * D;                             // [128][D]
  unsigned* gmax = reinterpret_cast<unsigned*>(klo + 128 * D);
  const int blk = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;
  const int row0 = blk * 128;
  const int t = threadIdx.x, g = t / Tile<D>::TPR, cg = t % Tile<D>::TPR;
  float x[Tile<D>::TOK][8];
  load_block<D, BF16>(a.k + b * a.ksB + h * a.ksH, a.ksN, row0, a.N, x);
  const float* kmean = a.out.k_mean + static_cast<int64_t>(bh) * D + 8 * cg;
  float mu[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mu[e] = kmean[e];
  const int valid = min(128, a.N - row0);
#pragma unroll
  for (int u = 0; u < Tile<D>::TOK; ++u) {
    const int r = g * Tile<D>::TOK + u;
    const bool ok = r < valid;
    uint16_t hv[8], lv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[u][e] = ok ? x[u][e] - mu[e] : 0.f;
      hv[e] = bf16_rne(x[u][e]);
      lv[e] = bf16_rne(x[u][e] - __uint_as_float(static_cast<uint32_t>(hv[e]) << 16));
    }
    *reinterpret_cast<uint4*>(khi + r * D + 8 * cg) = *reinterpret_cast<const uint4*>(hv);
    *reinterpret_cast<uint4*>(klo + r * D + 8 * cg) = *reinterpret_cast<const uint4*>(lv);
  }
  const int ngk = k_groups_per_block(a.gran);
  quantize_block<D, false>(x, a.gran, a.qmax, gmax, a.out.k_codes + (static_cast<int64_t>(bh) * a.n_pad + row0) * D,
                           a.out.k_scale + (static_cast<int64_t>(bh) * a.nblk + blk) * ngk);
  // quantize_block passed a barrier after khi/klo were written, so they are complete here.

  const int w = t / 64, l = t % 64, col = l & 31, hh = l >> 5;
  const int key = 32 * w + col;
  const float* qmean = a.out.q_mean + static_cast<int64_t>(bh) * a.nblk * D;
  float* bias = a.out.bias + static_cast<int64_t>(bh) * a.nblk * a.n_pad + row0 + key;
  for (int qb0 = 0; qb0 < a.nblk; qb0 += 32) {
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    const int qrow = qb0 + col;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const int c0 = 16 * ks + 8 * hh;
      float mv[8];
      if (qrow < a.nblk) {
        const float4 m0 = *reinterpret_cast<const float4*>(qmean + static_cast<int64_t>(qrow) * D + c0);
        const float4 m1 = *reinterpret_cast<const float4*>(qmean + static_cast<int64_t>(qrow) * D + c0 + 4);
        mv[0] = m0.x; mv[1] = m0.y; mv[2] = m0.z; mv[3] = m0.w;
        mv[4] = m1.x; mv[5] = m1.y; mv[6] = m1.z; mv[7] = m1.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) mv[e] = 0.f;
      }
      uint16_t ah[8], al[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ah[e] = bf16_rne(mv[e]);
        al[e] = bf16_rne(mv[e] - __uint_as_float(static_cast<uint32_t>(ah[e]) << 16));
      }
      const bf16x8 A_hi = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ah));
      const bf16x8 A_lo = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(al));
      const bf16x8 B_hi = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(khi + key * D + c0));
      const bf16x8 B_lo = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(klo + key * D + c0));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A_hi, B_hi, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A_hi, B_lo, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A_lo, B_hi, acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int qb = qb0 + 8 * (i >> 2) + 4 * hh + (i & 3);
      if (qb < a.nblk) bias[static_cast<int64_t>(qb) * a.n_pad] = acc[i] * a.scale_log2;
    }
  }
}

struct VArgs {
  const uint16_t* v;
  int64_t sB, sH, sN;
  sage_v_buffers out;
  int H, N, n_pad, nblk, smooth_v;
  float v_range;
};

// V pass 1: per-block channel sums (tree), maxima and minima over valid tokens.
template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) void v_stats_kernel(VArgs a) {
  __shared__ float lds[4 * D];
  __shared__ float mm[2][4][D];
  const int blk = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;
  const int row0 = blk * 128;
  const int t = threadIdx.x, g = t / Tile<D>::TPR, cg = t % Tile<D>::TPR;
  float x[Tile<D>::TOK][8];
  float s[8];
  load_block<D, BF16>(a.v + b * a.sB + h * a.sH, a.sN, row0, a.N, x);
  const int valid = min(128, a.N - row0);
  float mx[8], mn[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    mx[e] = -INFINITY;
    mn[e] = INFINITY;
  }
#pragma unroll
  for (int u = 0; u < Tile<D>::TOK; ++u) {
    if (g * Tile<D>::TOK + u < valid) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        mx[e] = fmaxf(mx[e], x[u][e]);
        mn[e] = fminf(mn[e], x[u][e]);
      }
    }
  }
#pragma unroll
  for (int m = Tile<D>::TPR; m < 64; m <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mx[e] = fmaxf(mx[e], __shfl_xor(mx[e], m));
      mn[e] = fminf(mn[e], __shfl_xor(mn[e], m));
    }
  const int w = t / 64, lane = t % 64;
  if (lane < Tile<D>::TPR)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mm[0][w][8 * lane + e] = mx[e];
      mm[1][w][8 * lane + e] = mn[e];
    }
  block_tree_sum<D>(x, s, lds);  // contains the barriers that publish mm
  if (g == 0) {
    float* part = a.out.v_partial + (static_cast<int64_t>(bh) * a.nblk + blk) * 3 * D;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = 8 * cg + e;
      part[c] = s[e];
      part[D + c] = fmaxf(fmaxf(mm[0][0][c], mm[0][1][c]), fmaxf(mm[0][2][c], mm[0][3][c]));
      part[2 * D + c] = fminf(fminf(mm[1][0][c], mm[1][1][c]), fminf(mm[1][2][c], mm[1][3][c]));
    }
  }
}

// V pass 2: mean, amax, scale and reciprocal scale per channel of one head.
// The reciprocal is parked in block 0's sum slot (only this thread reads it).
template <int D>
__global__ __launch_bounds__(D) void v_finalize_kernel(VArgs a) {
  const int bh = blockIdx.x, c = threadIdx.x;
  float* part = a.out.v_partial + static_cast<int64_t>(bh) * a.nblk * 3 * D;
  float mu = 0.f;
  if (a.smooth_v) {
    const float sum = tree_over_blocks(a.nblk, [&](int i) { return part[static_cast<int64_t>(i) * 3 * D + c]; });
    mu = sum / static_cast<float>(a.N);
  }
  float vmax = -INFINITY, vmin = INFINITY;
  for (int i = 0; i < a.nblk; ++i) {
    vmax = fmaxf(vmax, part[static_cast<int64_t>(i) * 3 * D + D + c]);
    vmin = fminf(vmin, part[static_cast<int64_t>(i) * 3 * D + 2 * D + c]);
  }
  // max_n |fl(V_n - mu)| = max(fl(vmax - mu), fl(mu - vmin)): fl(x - mu) is monotone in x.
  const float amax = fmaxf(vmax - mu, mu - vmin);
  a.out.v_scale[static_cast<int64_t>(bh) * D + c] = amax / a.v_range;
  a.out.v_mean[static_cast<int64_t>(bh) * D + c] = mu;
  part[c] = amax > 0.f ? a.v_range / amax : 0.f;
}

// Position of key r (0..127 inside a 128-key block) in the permuted V layout.
__device__ __forceinline__ int v_perm(int r) {
  const int g = r >> 6, k = r & 63;
  const int st2 = k >> 5, a = (k & 31) >> 3, hh = (k & 7) >> 2, bb = k & 3;
  return 64 * g + 32 * hh + 16 * st2 + 4 * a + bb;
}

// V pass 3: encode V' * (V_r / amax) to E4M3 (hardware conversion: OCP E4M3,
// round to nearest even) into the channel-major permuted layout.
template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) void v_encode_kernel(VArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[D * 128];
  const int blk = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;
  const int row0 = blk * 128;
  const int t = threadIdx.x, g = t / Tile<D>::TPR, cg = t % Tile<D>::TPR;
  float x[Tile<D>::TOK][8];
  load_block<D, BF16>(a.v + b * a.sB + h * a.sH, a.sN, row0, a.N, x);
  const float* part = a.out.v_partial + static_cast<int64_t>(bh) * a.nblk * 3 * D;
  const float* vmean = a.out.v_mean + static_cast<int64_t>(bh) * D;
  float mu[8], inv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    mu[e] = vmean[8 * cg + e];
    inv[e] = part[8 * cg + e];
  }
  const int valid = min(128, a.N - row0);
#pragma unroll
  for (int u = 0; u < Tile<D>::TOK; ++u) {
    const int r = g * Tile<D>::TOK + u;
    const bool ok = r < valid;
    const int pos = v_perm(r);
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float p0 = (x[u][e] - mu[e]) * inv[e];
      const float p1 = (x[u][e + 1] - mu[e + 1]) * inv[e + 1];
      const int pk = ok ? __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false) : 0;
      tile[(8 * cg + e) * 128 + pos] = static_cast<uint8_t>(pk & 0xff);
      tile[(8 * cg + e + 1) * 128 + pos] = static_cast<uint8_t>((pk >> 8) & 0xff);
    }
  }
  __syncthreads();
  uint8_t* dst = a.out.v_codes + static_cast<int64_t>(bh) * D * a.n_pad + row0;
#pragma unroll
  for (int i = 0; i < D * 8 / kThreads; ++i) {
    const int q = t + kThreads * i;
    const int c = q >> 3, part16 = q & 7;
    *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(c) * a.n_pad + 16 * part16) =
        *reinterpret_cast<const uint4*>(tile + c * 128 + 16 * part16);
  }
}

template <int D, bool BF16>
hipError_t quant_qk_impl(const Problem& p, TensorView q, TensorView k, const sage_qk_buffers& out, hipStream_t st) {
  QKArgs a;
  a.q = static_cast<const uint16_t*>(q.ptr);
  a.k = static_cast<const uint16_t*>(k.ptr);
  a.qsB = q.sB; a.qsH = q.sH; a.qsN = q.sN;
  a.ksB = k.sB; a.ksH = k.sH; a.ksN = k.sN;
  a.out = out;
  a.H = p.H; a.N = p.N; a.n_pad = p.n_pad; a.nblk = p.nblk;
  a.gran = p.gran; a.qmax = p.qmax; a.smooth_q = p.smooth_q; a.smooth_k = p.smooth_k;
  a.scale_log2 = p.sm_scale * 1.4426950408889634f;
  const dim3 grid(p.nblk, p.B * p.H);
  hipLaunchKernelGGL((q_quant_k_sums_kernel<D, BF16>), grid, dim3(kThreads), 0, st, a);
  hipLaunchKernelGGL((k_mean_kernel<D>), dim3(p.B * p.H), dim3(D), 0, st, a);
  const size_t smem = 2 * 128 * D * sizeof(uint16_t) + 128 * sizeof(unsigned);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_quant_bias_kernel<D, BF16>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((k_quant_bias_kernel<D, BF16>), grid, dim3(kThreads), smem, st, a);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t quant_v_impl(const Problem& p, TensorView v, const sage_v_buffers& out, hipStream_t st) {
  VArgs a;
  a.v = static_cast<const uint16_t*>(v.ptr);
  a.sB = v.sB; a.sH = v.sH; a.sN = v.sN;
  a.out = out;
  a.H = p.H; a.N = p.N; a.n_pad = p.n_pad; a.nblk = p.nblk; a.smooth_v = p.smooth_v;
  a.v_range = p.v_range;
  const dim3 grid(p.nblk, p.B * p.H);
  hipLaunchKernelGGL((v_stats_kernel<D, BF16>), grid, dim3(kThreads), 0, st, a);
  hipLaunchKernelGGL((v_finalize_kernel<D>), dim3(p.B * p.H), dim3(D), 0, st, a);
  hipLaunchKernelGGL((v_encode_kernel<D, BF16>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_qk(const Problem& p, TensorView q, TensorView k, const sage_qk_buffers& out,
                           hipStream_t st) {
  if (p.D == 128) return p.bf16 ? quant_qk_impl<128, true>(p, q, k, out, st) : quant_qk_impl<128, false>(p, q, k, out, st);
  return p.bf16 ? quant_qk_impl<64, true>(p, q, k, out, st) : quant_qk_impl<64, false>(p, q, k, out, st);
}

hipError_t launch_quant_v(const Problem& p, TensorView v, const sage_v_buffers& out, hipStream_t st) {
  if (p.D == 128) return p.bf16 ? quant_v_impl<128, true>(p, v, out, st) : quant_v_impl<128, false>(p, v, out, st);
  return p.bf16 ? quant_v_impl<64, true>(p, v, out, st) : quant_v_impl<64, false>(p, v, out, st);
}

}  // namespace sage
