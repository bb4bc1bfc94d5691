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

// Lane exchanges on the vector ALU instead of the LDS crossbar
// (ds_bpermute).  xor_combine<M>(x, op) = op(x of lane l, x of lane l ^ M) on
// every lane, for M = 1, 2 (quad permutes), 8 (a rotation by 8 inside each
// row of 16 lanes), 16 and 32 (the permlane swaps, which deliver the two
// values of a pair to both of its lanes).  op must be commutative (+, max,
// min): both lanes of a pair then hold identical bits.
template <int M, typename Op>
__device__ __forceinline__ float xor_combine(float x, Op op) {
  const uint32_t u = __float_as_uint(x);
  if constexpr (M == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  } else {
    static_assert(M == 1 || M == 2 || M == 8, "lane distance without a one-instruction exchange");
    constexpr int kCtrl = M == 1 ? 0xB1 : (M == 2 ? 0x4E : 0x128);   // quad_perm [1,0,3,2], [2,3,0,1]; row_ror:8
    return op(x, __uint_as_float(static_cast<uint32_t>(
                     __builtin_amdgcn_update_dpp(0, static_cast<int>(u), kCtrl, 0xf, 0xf, false))));
  }
}
struct FAdd { __device__ float operator()(float a, float b) const { return a + b; } };
struct FMax { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };
struct FMin { __device__ float operator()(float a, float b) const { return fminf(a, b); } };

// Maximum over the L = 8 or 16 lanes of a row group (l / L equal): the two
// quad exchanges, then the mirror inside 8 lanes and inside 16 (after the
// quads agree, a mirrored partner holds the other quad's maximum).
template <int L>
__device__ __forceinline__ float row_max(float x) {
  static_assert(L == 8 || L == 16, "row groups of 8 or 16 lanes");
  x = xor_combine<1>(x, FMax{});
  x = xor_combine<2>(x, FMax{});
  x = fmaxf(x, __uint_as_float(static_cast<uint32_t>(
                   __builtin_amdgcn_update_dpp(0, static_cast<int>(__float_as_uint(x)), 0x141, 0xf, 0xf, false))));
  if constexpr (L == 16)
    x = fmaxf(x, __uint_as_float(static_cast<uint32_t>(
                     __builtin_amdgcn_update_dpp(0, static_cast<int>(__float_as_uint(x)), 0x140, 0xf, 0xf, false))));
  return x;
}

// op over the token groups of a wave that hold the same channels (lanes
// l ^ TPR, l ^ 2 TPR, ..., l ^ 32), in that order.
template <int TPR, typename Op>
__device__ __forceinline__ float across_rows(float x, Op op) {
  static_assert(TPR == 8 || TPR == 16, "8 or 16 lanes per token row");
  if constexpr (TPR == 8) x = xor_combine<8>(x, op);
  x = xor_combine<16>(x, op);
  return xor_combine<32>(x, op);
}

template <bool BF16>
__device__ __forceinline__ float to_f32(uint16_t b) {
  if constexpr (BF16) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
  } else {
    return static_cast<float>(__builtin_bit_cast(_Float16, b));
  }
}

// Raw buffer resource over `bytes` bytes from p, and its 16-byte loads: a
// load at a byte offset at or past `bytes` returns zeros.  Rows past N are
// read through it with no guard; a guarded load compiles to a branch whose
// result is waited for before the next load is issued, which serialises a
// block's loads.  bytes < 2^31 (the N stride limit keeps 128 rows below it).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), kBufferWord3);
}
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t rs, int byte_off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Load rows [row0, row0 + 128) of one head; rows >= N read as 0.
template <int D, bool BF16>
__device__ __forceinline__ void load_block(const uint16_t* __restrict__ base, int64_t sN, int row0, int N,
                                           float (&x)[Tile<D>::TOK][8]) {
  const int t = threadIdx.x;
  const int g = t / Tile<D>::TPR, cg = t % Tile<D>::TPR;
  const auto rs = rows_rsrc(base + static_cast<int64_t>(row0) * sN, static_cast<int64_t>(min(128, N - row0)) * sN * 2);
#pragma unroll
  for (int u = 0; u < Tile<D>::TOK; ++u) {
    const int r = g * Tile<D>::TOK + u;
    const uint4 raw = load16(rs, r * static_cast<int>(sN) * 2 + 16 * cg);
    const uint16_t* hv = reinterpret_cast<const uint16_t*>(&raw);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[u][e] = to_f32<BF16>(hv[e]);
  }
}

// Pairwise tree over the block's 128 token positions, per channel: in-register
// pairs over each thread's TOK consecutive tokens, lane butterflies over
// neighbouring token groups (fp32 addition is commutative, so both partners
// hold identical bits), then the four 32-token wave sums as (w0+w1)+(w2+w3).
// On return every thread holds the sums of its 8 channels.  lds: 4*D floats,
// read after the one barrier and never written again by any caller (each
// kernel forms one tree sum), so no barrier follows the reads.
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
  for (int e = 0; e < 8; ++e) s[e] = across_rows<TPR>(s[e], FAdd{});
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
__device__ __forceinline__ void quantize_block(const float (&xs)[Tile<D>::TOK][8], int gran, int qmax, int held,
                                               unsigned* gmax, int8_t* __restrict__ codes_blk,
                                               float* __restrict__ scale_blk) {
  constexpr int TOK = Tile<D>::TOK, TPR = Tile<D>::TPR;
  const int t = threadIdx.x, g = t / TPR, cg = t % TPR;
  const float qm = static_cast<float>(qmax);
  // Group maxima of this thread's rows.  THREAD granularity: every group lies
  // inside one wave (a Q group is one row; a K group is one half of the
  // wave's 32-key subtile), so lane exchanges finish it.  Otherwise the
  // groups span waves and meet in LDS.
  float am_row[TOK];
  if (gran == SAGE_GRAN_THREAD) {
    if constexpr (IS_Q) {
#pragma unroll
      for (int u = 0; u < TOK; ++u) {
        float ra = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ra = fmaxf(ra, fabsf(xs[u][e]));
        ra = row_max<TPR>(ra);
        am_row[u] = ra;
        if (cg == 0) scale_blk[g * TOK + u] = ra / qm;
      }
    } else {
      // rows r of key group half (r & 7) >> 2 of the wave's subtile r >> 5
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int u = 0; u < TOK; ++u) {
        float ra = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ra = fmaxf(ra, fabsf(xs[u][e]));
        if ((((g * TOK + u) & 7) >> 2) == 0) a0 = fmaxf(a0, ra);
        else a1 = fmaxf(a1, ra);
      }
      a0 = xor_combine<32>(xor_combine<16>(row_max<16>(a0), FMax{}), FMax{});
      a1 = xor_combine<32>(xor_combine<16>(row_max<16>(a1), FMax{}), FMax{});
#pragma unroll
      for (int u = 0; u < TOK; ++u) am_row[u] = (((g * TOK + u) & 7) >> 2) == 0 ? a0 : a1;
      if ((t & 63) == 0) {
        scale_blk[2 * (t >> 6)] = a0 / qm;
        scale_blk[2 * (t >> 6) + 1] = a1 / qm;
      }
    }
  } else {
    if (t < 128) gmax[t] = 0u;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < TOK; ++u) {
      float ra = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ra = fmaxf(ra, fabsf(xs[u][e]));
      ra = row_max<TPR>(ra);
      const int r = g * TOK + u;
      const int grp = IS_Q ? q_group_in_block(gran, r) : k_group_in_block(gran, r);
      if (cg == 0) atomicMax(&gmax[grp], __float_as_uint(ra));  // non-negative floats order as unsigned
    }
    __syncthreads();
    const int ng = IS_Q ? q_groups_per_block(gran) : k_groups_per_block(gran);
    if (t < ng) scale_blk[t] = __uint_as_float(gmax[t]) / qm;
#pragma unroll
    for (int u = 0; u < TOK; ++u) {
      const int r = g * TOK + u;
      am_row[u] = __uint_as_float(gmax[IS_Q ? q_group_in_block(gran, r) : k_group_in_block(gran, r)]);
    }
  }
#pragma unroll
  for (int u = 0; u < TOK; ++u) {
    const int r = g * TOK + u;
    const float am = am_row[u];
    const float inv = am > 0.f ? qm / am : 0.f;
    // code = clamp(rint(x' * inv)) as an exact small integer in fp32, then its
    // low byte; four bytes per word, assembled with byte permutes.
    uint32_t packed[2];
    if (held == 2) {
      // The same integer codes as 6-bit FP6 E2M3 codes (exact for |code| <= 7),
      // packed into the slot layout of the 64-deep FP6 matrix product: slot
      // (group j, half h) holds channels 64j + 16h + i (i < 16) and
      // 64j + 32 + 16h + i - 16 (i >= 16), value i at bits 6i..6i+5 of 24
      // bytes; the slot's bytes 0..15 sit at row byte 16(4j + h), bytes
      // 16..23 at 16(4j + 2 + h), followed by 8 zero bytes.
      uint32_t c24[2];
#pragma unroll
      for (int hq = 0; hq < 2; ++hq) {
        uint32_t mag = 0u, sgn = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float f = __builtin_amdgcn_fmed3f(rintf(xs[u][e + 4 * hq] * inv), -qm, qm);
          mag |= static_cast<uint32_t>(fabsf(f)) << (8 * e);
          sgn |= (f < 0.f ? 0x20u : 0u) << (8 * e);
        }
        // E2M3 codes of 0..7: 0, 8, 16, 20, 24, 26, 28, 30 (one byte each)
        const uint32_t c = __builtin_amdgcn_perm(0x1E1C1A18u, 0x14100800u, mag) | sgn;
        c24[hq] = (c & 0x3Fu) | (((c >> 8) & 0x3Fu) << 6) | (((c >> 16) & 0x3Fu) << 12) | (((c >> 24) & 0x3Fu) << 18);
      }
      // 48 bits of this thread's 8 channels: bytes b0..b5.  Slot (j, h) comes
      // from the threads 8j + 2h + {0, 1, 4, 5} of the row (slot bytes 0, 6,
      // 12, 18); the first and the third of them gather their neighbours'
      // bytes and write one 16-byte unit each.
      const uint32_t lo4 = c24[0] | (c24[1] << 24);
      const uint32_t hi2 = c24[1] >> 8;
      // the values of lanes l + 1 and l + 4 (inside the lane's 8-group, so a
      // row shift of the 16-lane DPP row; the lanes past its end are unused)
      const uint32_t lo_1 = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(lo4), 0x101, 0xf, 0xf, false));
      const uint32_t hi_1 = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(hi2), 0x101, 0xf, 0xf, false));
      const uint32_t lo_4 = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(lo4), 0x104, 0xf, 0xf, false));
      const int j = cg / 8, m = cg % 8;
      uint8_t* row = reinterpret_cast<uint8_t*>(codes_blk) + static_cast<int64_t>(r) * D;
      if (m == 0 || m == 2) {          // slot bytes 0..15 -> unit 4j + h
        *reinterpret_cast<uint4*>(row + 16 * (4 * j + m / 2)) =
            make_uint4(lo4, (hi2 & 0xffffu) | (lo_1 << 16), (lo_1 >> 16) | (hi_1 << 16), lo_4);
      } else if (m == 4 || m == 6) {   // slot bytes 16..23 and 8 zero bytes -> unit 4j + 2 + h
        *reinterpret_cast<uint4*>(row + 16 * (4 * j + 2 + (m - 4) / 2)) =
            make_uint4((hi2 & 0xffffu) | (lo_1 << 16), (lo_1 >> 16) | (hi_1 << 16), 0u, 0u);
      }
      continue;
    }
    if (held == 1) {
      // The same integer codes held as E4M3 bytes (exact for |code| <= 15);
      // adding +0 turns -0 into +0, so that code 0 is byte 0.
      float cf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) cf[e] = __builtin_amdgcn_fmed3f(rintf(xs[u][e] * inv), -qm, qm) + 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(cf[4 * h], cf[4 * h + 1], 0, false);
        packed[h] = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(cf[4 * h + 2], cf[4 * h + 3], lo, true));
      }
      *reinterpret_cast<uint2*>(codes_blk + static_cast<int64_t>(r) * D + 8 * cg) = make_uint2(packed[0], packed[1]);
      continue;
    }
    int ci[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      ci[e] = static_cast<int>(__builtin_amdgcn_fmed3f(rintf(xs[u][e] * inv), -qm, qm));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t lo = __builtin_amdgcn_perm(static_cast<uint32_t>(ci[4 * h + 1]), static_cast<uint32_t>(ci[4 * h]),
                                                0x0c0c0400u);
      const uint32_t hi = __builtin_amdgcn_perm(static_cast<uint32_t>(ci[4 * h + 3]),
                                                static_cast<uint32_t>(ci[4 * h + 2]), 0x04000c0cu);
      packed[h] = lo | hi;
    }
    *reinterpret_cast<uint2*>(codes_blk + static_cast<int64_t>(r) * D + 8 * cg) = make_uint2(packed[0], packed[1]);
  }
}

// MXFP4 quantisation of smoothed rows (SageAttention3 abstract: FP4 with
// microscaling, read as OCP MXFP4).  Each 32-channel block of a token gets
// the smallest exponent s with 6 * 2^s >= its max |x| (from the fp32 bit
// pattern: amax = (1 + M/2^23) 2^e is covered by 1.5 * 2^e iff M <= 2^22),
// stored as the E8M0 byte s + 127, and the codes E2M1(x * 2^-s) (exact
// power-of-two scaling, then the hardware conversion: nearest, ties to even,
// saturating, sign kept).  A thread holds 8 channels of TOK rows; the 4
// threads of a 32-channel block share the max through lane exchanges.  Row
// stride of the codes D/2 bytes (channel 2i in the low nibble of byte i), of
// the scales D/32 bytes.
template <int D>
__device__ __forceinline__ void quantize_block_mx(const float (&xs)[Tile<D>::TOK][8], uint8_t* __restrict__ codes_blk,
                                                  uint8_t* __restrict__ scale_blk) {
  constexpr int TOK = Tile<D>::TOK, TPR = Tile<D>::TPR;
  static_assert(TPR % 4 == 0, "a 32-channel block spans 4 threads");
  const int t = threadIdx.x, g = t / TPR, cg = t % TPR;
#pragma unroll
  for (int u = 0; u < TOK; ++u) {
    float am = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(xs[u][e]));
    am = xor_combine<2>(xor_combine<1>(am, FMax{}), FMax{});
    const uint32_t bits = __float_as_uint(am);
    const int ef = static_cast<int>((bits >> 23) & 0xffu);
    int s = ef - 127 - ((bits & 0x7fffffu) <= 0x400000u ? 2 : 1);
    s = ef == 0 ? -127 : max(s, -127);
    uint32_t word = 0u;
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, ldexpf(xs[u][0], -s), ldexpf(xs[u][1], -s), 1.f, 0);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, ldexpf(xs[u][2], -s), ldexpf(xs[u][3], -s), 1.f, 1);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, ldexpf(xs[u][4], -s), ldexpf(xs[u][5], -s), 1.f, 2);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, ldexpf(xs[u][6], -s), ldexpf(xs[u][7], -s), 1.f, 3);
    const int r = g * TOK + u;
    *reinterpret_cast<uint32_t*>(codes_blk + static_cast<int64_t>(r) * (D / 2) + 4 * cg) = word;
    if ((cg & 3) == 0) scale_blk[static_cast<int64_t>(r) * (D / 32) + cg / 4] = static_cast<uint8_t>(s + 127);
  }
}

struct QKArgs {
  const uint16_t* q;
  const uint16_t* k;
  int64_t qsB, qsH, qsN, ksB, ksH, ksN;
  sage_qk_buffers out;
  int H, N, n_pad, nblk, gran, qmax, smooth_q, smooth_k;
  int held;   // INT4-range integer codes written as 1: E4M3 bytes, 2: packed FP6 E2M3 (0: int8)
  int with_bias;     // 0: K codes and scales only; the bias buffer is left as it is
  int k_sums;        // 0: pass 1 skips the K block sums (k_partial and k_mean are left as they are)
  int q_blk0;        // pass 1's first Q block (its grid spans the Q blocks it quantizes)
  float scale_log2;  // sm_scale * log2(e): the bias is stored in the exp2 domain
};

// Pass 1, two work-groups per (128-token block, head): blockIdx.z = 0 writes
// the Q block mean, Q codes and scales, z = 1 the block's K channel sums
// (subtrees of the K mean's tree).  Work-groups start in z order, so K is the
// input read last, the one most likely still cached when pass 2 reads it
// again.  With k_sums = 0 every work-group is a Q one, for Q blocks q_blk0 +
// blockIdx.x.
template <int D, bool BF16, bool MX>
__global__ __launch_bounds__(kThreads) void q_quant_k_sums_kernel(QKArgs a) {
  __shared__ float lds[4 * D];
  __shared__ unsigned gmax[128];
  const bool k_part = a.k_sums && blockIdx.z == 1;
  const int blk = k_part ? static_cast<int>(blockIdx.x) : a.q_blk0 + static_cast<int>(blockIdx.x);
  const int bh = blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;
  const int row0 = blk * 128;
  const int t = threadIdx.x, g = t / Tile<D>::TPR, cg = t % Tile<D>::TPR;
  float x[Tile<D>::TOK][8];
  float s[8];

  if (k_part) {
    // K block sums.
    load_block<D, BF16>(a.k + b * a.ksB + h * a.ksH, a.ksN, row0, a.N, x);
    block_tree_sum<D>(x, s, lds);
    if (g == 0)
#pragma unroll
      for (int e = 0; e < 8; ++e) a.out.k_partial[(static_cast<int64_t>(bh) * a.nblk + blk) * D + 8 * cg + e] = s[e];
    return;
  }

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
  if constexpr (MX) {
    quantize_block_mx<D>(x, reinterpret_cast<uint8_t*>(a.out.q_codes) + (static_cast<int64_t>(bh) * a.n_pad + row0) * (D / 2),
                         reinterpret_cast<uint8_t*>(a.out.q_scale) + (static_cast<int64_t>(bh) * a.n_pad + row0) * (D / 32));
  } else {
    const int ngq = q_groups_per_block(a.gran);
    quantize_block<D, true>(x, a.gran, a.qmax, a.held, gmax, a.out.q_codes + (static_cast<int64_t>(bh) * a.n_pad + row0) * D,
                            a.out.q_scale + (static_cast<int64_t>(bh) * a.nblk + blk) * ngq);
  }
}

// Pairwise tree over the n per-block partial sums of one channel (leaves
// padded with +0.0 up to P = 2^ceil(log2 n)), for 32 channels of one head per
// work-group: S = min(8, P) threads per channel each reduce one aligned segment
// of P/S leaves (8-leaf subtrees formed in registers from batched loads, then
// merged by a binary counter kept in LDS), and the S segment sums are merged as
// a tree in LDS.  Exactly the canonical tree, with no padding beyond P.
template <typename F>
__device__ __forceinline__ float segment_tree_sum(int n, int c32, int seg, F leaf, float (*stk)[32][14],
                                                  float (*segsum)[32]) {
  int P = 1;
  while (P < n) P <<= 1;
  const int S = P < 8 ? P : 8;
  const int L = P / S;
  float result = 0.f;
  if (seg < S) {
    const int first = seg * L;
    int sp = 0, cnt = 0;
    auto push = [&](float x) {
      int k = cnt;
      while (k & 1) {
        x = stk[seg][c32][--sp] + x;
        k >>= 1;
      }
      stk[seg][c32][sp++] = x;
      ++cnt;
    };
    if (L >= 8) {
      for (int i0 = 0; i0 < L; i0 += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          // the index is clamped so that every load is issued unconditionally
          // (a guarded load would wait for the one before it)
          const int i = first + i0 + u;
          const float lv = leaf(min(i, n - 1));
          v[u] = i < n ? lv : 0.f;
        }
        push(((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7])));
      }
    } else {
      for (int i = first; i < first + L; ++i) {
        const float lv = leaf(min(i, n - 1));
        push(i < n ? lv : 0.f);
      }
    }
    result = stk[seg][c32][0];
    segsum[seg][c32] = result;
  }
  __syncthreads();
  for (int st = 1; st < S; st <<= 1) {
    if (seg % (2 * st) == 0 && seg + st < S) segsum[seg][c32] = segsum[seg][c32] + segsum[seg + st][c32];
    __syncthreads();
  }
  return segsum[0][c32];
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two-term bf16 split of a pair of floats (hardware conversion, round to
// nearest even): hi = bf16(x), lo = bf16(x - hi), each returned packed.
__device__ __forceinline__ void split_bf16x2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x0, x1}, bf16x2));
  const float h0 = __uint_as_float(hi << 16), h1 = __uint_as_float(hi & 0xffff0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x0 - h0, x1 - h1}, bf16x2));
}

// K mean: one work-group per (32-channel group, head); 256 threads = 32
// channels x 8 segments.  When the bias follows, the work-group then stores
// the bf16 split of the Q block means of its channels in the k_partial words
// it has just reduced (word (qb, c) = bf16 hi | bf16 lo << 16): the bias
// kernel reads the split from there instead of forming it once per key block.
template <int D>
__global__ __launch_bounds__(256) void k_mean_kernel(QKArgs a) {
  __shared__ float stk[8][32][14];
  __shared__ float segsum[8][32];
  const int bh = blockIdx.y, c = 32 * blockIdx.x + (threadIdx.x & 31), seg = threadIdx.x >> 5;
  float* part = a.out.k_partial + static_cast<int64_t>(bh) * a.nblk * D + c;
  const float sum = segment_tree_sum(a.nblk, threadIdx.x & 31, seg, [&](int i) { return part[static_cast<int64_t>(i) * D]; },
                                     stk, segsum);   // every leaf is read before its first barrier
  if (seg == 0) a.out.k_mean[static_cast<int64_t>(bh) * D + c] = a.smooth_k ? sum / static_cast<float>(a.N) : 0.f;
  if (a.with_bias) {
    const float* qm = a.out.q_mean + static_cast<int64_t>(bh) * a.nblk * D + c;
    for (int qb0 = seg; qb0 < a.nblk; qb0 += 64) {
      float mu[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) mu[u] = qm[static_cast<int64_t>(min(qb0 + 8 * u, a.nblk - 1)) * D];   // unused past nblk
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        uint32_t hi, lo;
        split_bf16x2(mu[u], 0.f, hi, lo);
        if (qb0 + 8 * u < a.nblk)
          reinterpret_cast<uint32_t*>(part)[static_cast<int64_t>(qb0 + 8 * u) * D] = (hi & 0xffffu) | (lo << 16);
      }
    }
  }
}

// Pass 2, one work-group per (128-key block, head): K' = K - mean, K codes and
// scales, then the bias dS[qb, j] = mu_Q(qb) . K'_j for the block's keys and
// every Q block, on the bf16 matrix cores with a three-product hi/lo split of
// both operands (about 16 significant bits), stored times sm_scale * log2(e).
// Each wave keeps the split of its 32 keys in registers; the split mu_Q rows
// (formed once per head by k_mean_kernel, word (qb, c) = bf16 hi | bf16 lo <<
// 16) go through LDS in chunks of kBiasChunk Q blocks, shared by the four
// waves.  A store instruction writes 32 consecutive keys (128 bytes) of two Q
// blocks.  LDS row of D bf16 values (2D bytes): 16-byte chunk c of row r lives
// at chunk c ^ (r & (2D/16 - 1)), so the 32 rows read together by an MFMA
// operand load spread over the banks.
constexpr int kBiasChunk = 64;

template <int D>
__device__ __forceinline__ int bf_off(int r, int c16) {
  constexpr int CH = 2 * D / 16;
  return r * 2 * D + 16 * (c16 ^ (r & (CH - 1)));
}

template <int D, bool BF16, bool MX>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void k_quant_bias_kernel(QKArgs a) {
  constexpr int QC = kBiasChunk;
  constexpr int PPT = QC * D / 8 / kThreads;    // 8-channel pieces of a mu_Q chunk per thread
  __shared__ __attribute__((aligned(16))) uint8_t ahi[QC * 2 * D];   // [QC Q blocks][D] bf16, swizzled rows
  __shared__ __attribute__((aligned(16))) uint8_t alo[QC * 2 * D];
  __shared__ unsigned gmax[128];
  const int blk = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;
  const int row0 = blk * 128;
  const int t = threadIdx.x, g = t / Tile<D>::TPR, cg = t % Tile<D>::TPR;
  const uint16_t* kin = a.k + b * a.ksB + h * a.ksH;
  const float* kmean = a.out.k_mean + static_cast<int64_t>(bh) * D;
  const uint32_t* musplit = reinterpret_cast<const uint32_t*>(a.out.k_partial) + static_cast<int64_t>(bh) * a.nblk * D;
  const int valid = min(128, a.N - row0);
  const int w = t / 64, l = t % 64, col = l & 31, hh = l >> 5;
  const int key = 32 * w + col;

  // The first chunk of split-mean words is fetched before the quantisation,
  // so that its latency overlaps it.
  uint4 mq[PPT][2];
  const auto mu_rs = rows_rsrc(musplit, static_cast<int64_t>(a.nblk) * D * 4);
  auto fetch_mu = [&](int qc0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int piece = t + kThreads * i;
      const int row = piece / (D / 8), c8 = piece % (D / 8);
      const int w0 = 4 * ((qc0 + row) * D + 8 * c8);   // rows past nblk read as zeros
      mq[i][0] = load16(mu_rs, w0);
      mq[i][1] = load16(mu_rs, w0 + 16);
    }
  };
  if (a.with_bias) fetch_mu(0);

  {
    float x[Tile<D>::TOK][8];
    load_block<D, BF16>(kin, a.ksN, row0, a.N, x);
    float mu[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) mu[e] = kmean[8 * cg + e];
#pragma unroll
    for (int u = 0; u < Tile<D>::TOK; ++u) {
      const bool ok = g * Tile<D>::TOK + u < valid;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[u][e] = ok ? x[u][e] - mu[e] : 0.f;
    }
    if constexpr (MX) {
      quantize_block_mx<D>(x, reinterpret_cast<uint8_t*>(a.out.k_codes) + (static_cast<int64_t>(bh) * a.n_pad + row0) * (D / 2),
                           reinterpret_cast<uint8_t*>(a.out.k_scale) + (static_cast<int64_t>(bh) * a.n_pad + row0) * (D / 32));
    } else {
      const int ngk = k_groups_per_block(a.gran);
      quantize_block<D, false>(x, a.gran, a.qmax, a.held, gmax, a.out.k_codes + (static_cast<int64_t>(bh) * a.n_pad + row0) * D,
                               a.out.k_scale + (static_cast<int64_t>(bh) * a.nblk + blk) * ngk);
    }
  }

  if (!a.with_bias) return;   // uniform over the launch

  // B operand: the split K' of this wave's 32 keys (the block's rows read
  // again, from L2), 16 channels per MFMA step, lane half hh holding 8.
  bf16x8 Bhi[D / 16], Blo[D / 16];
  {
    const bool ok = key < valid;
    uint4 kraw[D / 16];
    const auto krs = rows_rsrc(kin + static_cast<int64_t>(row0) * a.ksN, static_cast<int64_t>(valid) * a.ksN * 2);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)   // keys past N read as zeros (and are masked below)
      kraw[ks] = load16(krs, key * static_cast<int>(a.ksN) * 2 + 32 * ks + 16 * hh);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const int c0 = 16 * ks + 8 * hh;
      const uint16_t* hv = reinterpret_cast<const uint16_t*>(&kraw[ks]);
      const float4 m0 = *reinterpret_cast<const float4*>(kmean + c0);
      const float4 m1 = *reinterpret_cast<const float4*>(kmean + c0 + 4);
      const float mk[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
      float kp[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) kp[e] = ok ? to_f32<BF16>(hv[e]) - mk[e] : 0.f;
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) split_bf16x2(kp[2 * p], kp[2 * p + 1], hi[p], lo[p]);
      Bhi[ks] = __builtin_bit_cast(bf16x8, make_uint4(hi[0], hi[1], hi[2], hi[3]));
      Blo[ks] = __builtin_bit_cast(bf16x8, make_uint4(lo[0], lo[1], lo[2], lo[3]));
    }
  }
  float* bias = a.out.bias + static_cast<int64_t>(bh) * a.nblk * a.n_pad + row0 + key;
  for (int qc0 = 0; qc0 < a.nblk; qc0 += QC) {
    // Unpack this chunk's split words into the hi and lo rows in LDS (the
    // previous chunk's reads finished at the barrier ending the last
    // iteration), then fetch the next chunk.
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int piece = t + kThreads * i;
      const int row = piece / (D / 8), c8 = piece % (D / 8);
      const uint32_t wd[8] = {mq[i][0].x, mq[i][0].y, mq[i][0].z, mq[i][0].w,
                              mq[i][1].x, mq[i][1].y, mq[i][1].z, mq[i][1].w};
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        hi[p] = __builtin_amdgcn_perm(wd[2 * p + 1], wd[2 * p], 0x05040100u);   // low halves of the two words
        lo[p] = __builtin_amdgcn_perm(wd[2 * p + 1], wd[2 * p], 0x07060302u);   // high halves
      }
      *reinterpret_cast<uint4*>(ahi + bf_off<D>(row, c8)) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      *reinterpret_cast<uint4*>(alo + bf_off<D>(row, c8)) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
    __syncthreads();
    if (qc0 + QC < a.nblk) fetch_mu(qc0 + QC);
#pragma unroll 1
    for (int s0 = 0; s0 < QC && qc0 + s0 < a.nblk; s0 += 32) {
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
      // A operands (the split mu_Q rows s0 + col) are read one step ahead of
      // their three products, so that the LDS latency overlaps them.
      bf16x8 A_hi[2], A_lo[2];
      auto read_a = [&](int ks) __attribute__((always_inline)) {
        const int c16 = 2 * ks + hh;
        A_hi[ks & 1] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ahi + bf_off<D>(s0 + col, c16)));
        A_lo[ks & 1] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(alo + bf_off<D>(s0 + col, c16)));
      };
      read_a(0);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        if (ks + 1 < D / 16) read_a(ks + 1);
        __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of this step's products
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A_hi[ks & 1], Bhi[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A_hi[ks & 1], Blo[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A_lo[ks & 1], Bhi[ks], acc, 0, 0, 0);
      }
      // acc[i]: Q block qc0 + s0 + 8 (i / 4) + 4 hh + i % 4, this lane's key.
      float* dst = bias + static_cast<int64_t>(qc0 + s0 + 4 * hh) * a.n_pad;
      if (qc0 + s0 + 32 <= a.nblk) {   // uniform: all 32 Q blocks of the group exist
#pragma unroll
        for (int i = 0; i < 16; ++i) dst[static_cast<int64_t>(8 * (i >> 2) + (i & 3)) * a.n_pad] = acc[i] * a.scale_log2;
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (qc0 + s0 + 8 * (i >> 2) + 4 * hh + (i & 3) < a.nblk)
            dst[static_cast<int64_t>(8 * (i >> 2) + (i & 3)) * a.n_pad] = acc[i] * a.scale_log2;
      }
    }
    __syncthreads();   // every wave is done with this chunk's LDS rows
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
  if (valid == 128) {
    // Whole block: canonicalise each value once, then three-input max/min.
    float c[Tile<D>::TOK][8];
#pragma unroll
    for (int u = 0; u < Tile<D>::TOK; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) c[u][e] = __builtin_canonicalizef(x[u][e]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mx[e] = c[0][e];
      mn[e] = c[0][e];
    }
#pragma unroll
    for (int u = 1; u + 1 < Tile<D>::TOK; u += 2)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        mx[e] = fmaxf(fmaxf(mx[e], c[u][e]), c[u + 1][e]);
        mn[e] = fminf(fminf(mn[e], c[u][e]), c[u + 1][e]);
      }
    if constexpr (Tile<D>::TOK % 2 == 0)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        mx[e] = fmaxf(mx[e], c[Tile<D>::TOK - 1][e]);
        mn[e] = fminf(mn[e], c[Tile<D>::TOK - 1][e]);
      }
  } else {
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
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    mx[e] = across_rows<Tile<D>::TPR>(mx[e], FMax{});
    mn[e] = across_rows<Tile<D>::TPR>(mn[e], FMin{});
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

// V pass 2: mean, amax, scale and reciprocal scale per channel, one
// work-group per (32-channel group, head).  The reciprocal scale is parked in
// block 0's sum slot, which only this work-group reads (before the write).
template <int D>
__global__ __launch_bounds__(256) void v_finalize_kernel(VArgs a) {
  __shared__ float stk[8][32][14];
  __shared__ float segsum[8][32];
  __shared__ float mx[8][32], mn[8][32];
  const int bh = blockIdx.y, c32 = threadIdx.x & 31, c = 32 * blockIdx.x + c32, seg = threadIdx.x >> 5;
  float* part = a.out.v_partial + static_cast<int64_t>(bh) * a.nblk * 3 * D;
  float vmax = -INFINITY, vmin = INFINITY;
  // blocks seg, seg + 8, ..., eight at a time with every load issued before
  // the first is used; indices past the last block re-read it (max and min
  // are idempotent)
  for (int i0 = seg; i0 < a.nblk; i0 += 64) {
    float hx[8], lx[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t i = min(i0 + 8 * j, a.nblk - 1);
      hx[j] = part[i * 3 * D + D + c];
      lx[j] = part[i * 3 * D + 2 * D + c];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      vmax = fmaxf(vmax, hx[j]);
      vmin = fminf(vmin, lx[j]);
    }
  }
  mx[seg][c32] = vmax;
  mn[seg][c32] = vmin;
  const float sum = segment_tree_sum(a.nblk, c32, seg, [&](int i) { return part[static_cast<int64_t>(i) * 3 * D + c]; },
                                     stk, segsum);   // its barriers publish mx, mn
  if (seg == 0) {
    for (int s2 = 1; s2 < 8; ++s2) {
      vmax = fmaxf(vmax, mx[s2][c32]);
      vmin = fminf(vmin, mn[s2][c32]);
    }
    const float mu = a.smooth_v ? sum / static_cast<float>(a.N) : 0.f;
    // max_n |fl(V_n - mu)| = max(fl(vmax - mu), fl(mu - vmin)): fl(x - mu) is monotone in x.
    const float amax = fmaxf(vmax - mu, mu - vmin);
    a.out.v_scale[static_cast<int64_t>(bh) * D + c] = amax / a.v_range;
    a.out.v_mean[static_cast<int64_t>(bh) * D + c] = mu;
    part[c] = amax > 0.f ? a.v_range / amax : 0.f;
  }
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
  // Four consecutive tokens 4k..4k+3 of one channel sit at four consecutive
  // permuted positions, so they are converted as two token pairs and written
  // as one 32-bit word.
#pragma unroll
  for (int u4 = 0; u4 < Tile<D>::TOK; u4 += 4) {
    const int r = g * Tile<D>::TOK + u4;
    const int pos = v_perm(r);
    float pv[4][8];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[j][e] = r + j < valid ? (x[u4 + j][e] - mu[e]) * inv[e] : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int wd = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0][e], pv[1][e], 0, false);
      wd = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2][e], pv[3][e], wd, true);
      *reinterpret_cast<int*>(tile + (8 * cg + e) * 128 + pos) = wd;
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

// 16-bit P~V (SAGE_PV_F16): V as given, channel-major, keys of every 32-key
// group in the order of the 16-bit MFMA operand (swap bits 2 and 3 of the key
// offset: position 16m + 8h + 4a + r holds key 16m + 8a + 4h + r), zeros past
// N.  The work-groups of block 0 also write v_scale = 1 and v_mean = 0.
template <int D>
__global__ __launch_bounds__(kThreads) void v_pack16_kernel(VArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[D * 128];
  const int blk = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;
  const int row0 = blk * 128;
  const int t = threadIdx.x, g = t / Tile<D>::TPR, cg = t % Tile<D>::TPR;
  const uint16_t* base = a.v + b * a.sB + h * a.sH;
  const auto rs = rows_rsrc(base + static_cast<int64_t>(row0) * a.sN, static_cast<int64_t>(min(128, a.N - row0)) * a.sN * 2);
  // Four consecutive tokens 4k..4k+3 keep consecutive positions (only bits 2
  // and 3 swap), so each thread writes them per channel as one 8-byte word.
#pragma unroll
  for (int u4 = 0; u4 < Tile<D>::TOK; u4 += 4) {
    uint4 raw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = g * Tile<D>::TOK + u4 + j;   // rows past N read as zeros
      raw[j] = load16(rs, r * static_cast<int>(a.sN) * 2 + 16 * cg);
    }
    const int k = g * Tile<D>::TOK + u4;
    const int pos = (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint16_t v4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v4[j] = reinterpret_cast<const uint16_t*>(&raw[j])[e];
      *reinterpret_cast<uint2*>(tile + (8 * cg + e) * 128 + pos) = *reinterpret_cast<const uint2*>(v4);
    }
  }
  __syncthreads();
  uint16_t* dst = reinterpret_cast<uint16_t*>(a.out.v_codes) + static_cast<int64_t>(bh) * D * a.n_pad + row0;
#pragma unroll
  for (int i = 0; i < D * 16 / kThreads; ++i) {
    const int q = t + kThreads * i;
    const int c = q >> 4, part = q & 15;
    *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(c) * a.n_pad + 8 * part) =
        *reinterpret_cast<const uint4*>(tile + c * 128 + 8 * part);
  }
  if (blk == 0 && t < D) {
    a.out.v_scale[static_cast<int64_t>(bh) * D + t] = 1.f;
    a.out.v_mean[static_cast<int64_t>(bh) * D + t] = 0.f;
  }
}

template <int D, bool BF16>
hipError_t quant_qk_impl(const Problem& p, TensorView q, TensorView k, const sage_qk_buffers& out, hipStream_t st,
                         const QKPart& part) {
  QKArgs a;
  a.q = static_cast<const uint16_t*>(q.ptr);
  a.k = static_cast<const uint16_t*>(k.ptr);
  a.qsB = q.sB; a.qsH = q.sH; a.qsN = q.sN;
  a.ksB = k.sB; a.ksH = k.sH; a.ksN = k.sN;
  a.out = out;
  a.H = p.H; a.N = p.N; a.n_pad = p.n_pad; a.nblk = p.nblk;
  a.gran = p.gran; a.qmax = p.qmax; a.smooth_q = p.smooth_q; a.smooth_k = p.smooth_k;
  a.held = p.qk_held;
  a.with_bias = part.bias ? 1 : 0;
  a.k_sums = part.k_sums ? 1 : 0;
  a.q_blk0 = part.k_sums ? 0 : part.q_blk0;
  a.scale_log2 = p.sm_scale * 1.4426950408889634f;
  const dim3 grid(p.nblk, p.B * p.H);
  // with the K sums, pass 1 covers every Q block; without them, q_nblk blocks from q_blk0
  const int qn = part.k_sums ? p.nblk : min(part.q_nblk, p.nblk - part.q_blk0);
  const dim3 grid1(part.k_sums ? p.nblk : qn, p.B * p.H, part.k_sums ? 2 : 1);
  if (p.qk_mx) {
    if (qn > 0) hipLaunchKernelGGL((q_quant_k_sums_kernel<D, BF16, true>), grid1, dim3(kThreads), 0, st, a);
    if (part.k_sums) hipLaunchKernelGGL((k_mean_kernel<D>), dim3(D / 32, p.B * p.H), dim3(256), 0, st, a);
    if (part.k_codes) hipLaunchKernelGGL((k_quant_bias_kernel<D, BF16, true>), grid, dim3(kThreads), 0, st, a);
  } else {
    if (qn > 0) hipLaunchKernelGGL((q_quant_k_sums_kernel<D, BF16, false>), grid1, dim3(kThreads), 0, st, a);
    if (part.k_sums) hipLaunchKernelGGL((k_mean_kernel<D>), dim3(D / 32, p.B * p.H), dim3(256), 0, st, a);
    if (part.k_codes) hipLaunchKernelGGL((k_quant_bias_kernel<D, BF16, false>), grid, dim3(kThreads), 0, st, a);
  }
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
  if (p.pv_f16) {
    hipLaunchKernelGGL((v_pack16_kernel<D>), grid, dim3(kThreads), 0, st, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((v_stats_kernel<D, BF16>), grid, dim3(kThreads), 0, st, a);
  hipLaunchKernelGGL((v_finalize_kernel<D>), dim3(D / 32, p.B * p.H), dim3(256), 0, st, a);
  hipLaunchKernelGGL((v_encode_kernel<D, BF16>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_qk(const Problem& p, TensorView q, TensorView k, const sage_qk_buffers& out,
                           hipStream_t st, const QKPart& part) {
  // the bias is written by the K-code kernel from the Q-mean split that the K-mean kernel forms
  if (part.bias && (!part.k_codes || !part.k_sums)) return hipErrorInvalidValue;
  if (p.D == 128)
    return p.bf16 ? quant_qk_impl<128, true>(p, q, k, out, st, part)
                  : quant_qk_impl<128, false>(p, q, k, out, st, part);
  return p.bf16 ? quant_qk_impl<64, true>(p, q, k, out, st, part)
                : quant_qk_impl<64, false>(p, q, k, out, st, part);
}

hipError_t launch_quant_v(const Problem& p, TensorView v, const sage_v_buffers& out, hipStream_t st) {
  if (p.D == 128) return p.bf16 ? quant_v_impl<128, true>(p, v, out, st) : quant_v_impl<128, false>(p, v, out, st);
  return p.bf16 ? quant_v_impl<64, true>(p, v, out, st) : quant_v_impl<64, false>(p, v, out, st);
}

}  // namespace sage
