// Quantized attention forward kernel for gfx950 (CDNA4).
//
// Method: the FlashAttention-based quantized attention of the SageAttention2++
// summary ("2. Preliminary", "2.1 SageAttention2"): INT8 (or INT4-range)
// Q, K codes with per-group scales, dequantised S plus the Q-smoothing bias,
// online softmax, P~ to FP8 with the fixed scale 1/P_r, FP8 V with per-channel
// scales, rescale and normalise at the end.
//
// Mapping to the hardware:
//  * one work-group of 4 waves per 128-query block; wave w owns 32 queries.
//  * S^T = K^ Q^T on v_mfma_i32_32x32x32_i8: the A operand is 32 keys x 32
//    channels of K^ (from LDS), the B operand 32 channels x 32 queries of Q^
//    (registers for the whole kernel).  In the 32x32 accumulator lane l holds
//    query l%32 and the 16 keys 8a + 4(l/32) + b, so row max and row sum are
//    in-lane work plus one exchange with lane l^32.
//  * the 16 fp8-packed P~ values of two consecutive 32-key S tiles are
//    exactly one lane's 32-byte B operand of v_mfma_f32_32x32x64_f8f6f4
//    (O^T += V^T P~^T, keys as the reduction index).  The V codes are stored
//    channel-major with the matching in-group key order, so P~ never leaves
//    registers.
//  * one online-softmax update per 128-key tile; exp2 on v_exp_f32 with the
//    log2(e) softmax scale and log2(P_r) folded into the exponent.
#include "sage_internal.h"

namespace sage {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct AttnArgs {
  const int8_t* q_codes;
  const float* q_scale;
  const int8_t* k_codes;
  const float* k_scale;
  const float* bias;
  const uint8_t* v_codes;
  const float* v_scale;
  const float* v_mean;
  void* o;
  int64_t oB, oH, oN;
  int H, N, n_pad, nblk, gran, causal;
  float scale_log2;  // sm_scale * log2(e)
  float log2_pr;     // log2(P_r)
};

// 16-byte chunk swizzle inside a tile row so that the 16 lanes served together
// by one ds_read_b128 pass touch distinct banks.
template <int ROW_BYTES>
__device__ __forceinline__ int swz(int row, int chunk) {
  constexpr int CPR = ROW_BYTES / 16;
  constexpr int RPW = 256 / ROW_BYTES;  // rows per 256-byte bank window
  return chunk ^ ((row / RPW) & (CPR - 1));
}

__device__ __forceinline__ uint16_t to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Work-group -> (head, query block).  Work-groups are dispatched round-robin
// over the 8 XCDs (each with its own L2), so consecutive ids are regrouped to
// give every XCD a contiguous run of (head, block) items: the K/V codes of one
// head then stay in that XCD's L2 while its blocks run.  Causal runs visit the
// blocks of a head from the last (longest) to the first.
__device__ __forceinline__ void map_block(int id, int total, int nblk, int causal, int& bh, int& qb) {
  constexpr int kXcd = 8;
  int w = id;
  if (total % kXcd == 0) w = (id % kXcd) * (total / kXcd) + id / kXcd;
  bh = w / nblk;
  qb = w % nblk;
  if (causal) qb = nblk - 1 - qb;
}

typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ lds_void* lds_ptr(void* p) { return (lds_void*)(p); }

template <int D>
struct TileBuf {
  static constexpr int K_BYTES = 128 * D;          // K codes, 128 keys x D, rows swizzled
  static constexpr int V_BYTES = D * 128;          // V codes, D channels x 128 keys, rows swizzled
  static constexpr int B_BYTES = 128 * 4;          // bias of the 128 keys
  static constexpr int S_BYTES = 64 * 4;           // K scales of the tile (8 or 2 used)
  static constexpr int BYTES = K_BYTES + V_BYTES + B_BYTES + S_BYTES;
};

// Direct global->LDS copies of one key tile through buffer resources (raw
// buffers: reads past num_records return zero instead of faulting).  Lane L of
// a wave-wide copy always lands at (LDS base + 16 L), so each lane fetches the
// chunk that belongs at its destination in the swizzled layout.  With chunk
// p = 256 j + threadIdx.x, the swizzled column does not depend on j, so one
// per-lane offset serves every copy of a stream and j moves only the scalar
// offset (4096 j bytes of K rows, 32 j channel rows of V).
struct TileSrc {
  __amdgpu_buffer_rsrc_t k, v, b, s;
  uint32_t k_off, v_off, b_off;   // per-lane byte offsets for j = 0 and k0 = 0
  uint32_t v_row;                 // bytes per V channel row (n_pad)
  uint32_t s_per_tile;            // K scale groups per 128-key tile (8 or 2)
};

template <int D>
__device__ __forceinline__ TileSrc make_tile_src(const int8_t* kbase, const uint8_t* vbase, const float* brow,
                                                 const float* kscale, int n_scale, int n_pad, int t) {
  constexpr int CPR = D / 16;
  TileSrc s;
  const uint32_t flags = 0x00020000u;   // raw 32-bit data format, no swizzle
  s.k = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(kbase), 0, n_pad * D, flags);
  s.v = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(vbase), 0, n_pad * D, flags);
  s.b = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(brow), 0, n_pad * 4, flags);
  s.s = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(kscale), 0, n_scale * 4, flags);
  s.s_per_tile = static_cast<uint32_t>(n_scale / (n_pad / 128));
  const int r = t / CPR, pc = t % CPR;
  s.k_off = static_cast<uint32_t>(r * D + 16 * swz<D>(r, pc));
  const int ch = t >> 3, vc = t & 7;
  s.v_off = static_cast<uint32_t>(ch * n_pad + 16 * swz<128>(ch, vc));
  s.b_off = static_cast<uint32_t>(4 * t);
  s.v_row = static_cast<uint32_t>(n_pad);
  return s;
}

template <int D>
__device__ __forceinline__ void issue_tile(uint8_t* buf, const TileSrc& s, int k0, int w) {
#pragma unroll
  for (int j = 0; j < D / 32; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(s.k, lds_ptr(buf + (4 * j + w) * 1024), 16, s.k_off,
                                             static_cast<uint32_t>(k0 * D + 4096 * j), 0, 0);
  uint8_t* vb = buf + TileBuf<D>::K_BYTES;
#pragma unroll
  for (int j = 0; j < D / 32; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(s.v, lds_ptr(vb + (4 * j + w) * 1024), 16, s.v_off,
                                             static_cast<uint32_t>(k0) + 32u * j * s.v_row, 0, 0);
  if (w < 2) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(s.b, lds_ptr(buf + TileBuf<D>::K_BYTES + TileBuf<D>::V_BYTES + 256 * w),
                                             4, s.b_off, static_cast<uint32_t>(4 * k0), 0, 0);
  } else if (w == 2 && s.b_off - 512u < 4u * s.s_per_tile) {
    // lanes 0 .. s_per_tile-1 of wave 2 copy the tile's K scales (lane l reads scale l)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        s.s, lds_ptr(buf + TileBuf<D>::K_BYTES + TileBuf<D>::V_BYTES + TileBuf<D>::B_BYTES), 4, s.b_off - 512u,
        static_cast<uint32_t>(4 * (k0 / 128) * s.s_per_tile), 0, 0);
  }
}

template <int D, bool BF16>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(AttnArgs a) {
  constexpr int KS = D / 32;  // 32-channel k-steps of the QK product
  constexpr int CT = D / 32;  // 32-channel tiles of the output
  // Two distinct LDS objects (not halves of one array) so the compiler can see
  // that reads of the current tile do not alias the copies into the other.
  __shared__ __attribute__((aligned(1024))) uint8_t buf0[TileBuf<D>::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t buf1[TileBuf<D>::BYTES];

  const int t = threadIdx.x, l = t & 63, col = l & 31, hh = l >> 5;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);   // wave index, held in a scalar register
  int bh, qb;
  map_block(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x), a.nblk, a.causal, bh, qb);
  const int q0 = qb * 128;
  const int qi = q0 + 32 * w + col;

  const int key_end = a.causal ? min(a.N, q0 + 128) : a.N;
  const int ntiles = (key_end + 127) / 128;
  const int8_t* kbase = a.k_codes + static_cast<int64_t>(bh) * a.n_pad * D;
  const uint8_t* vbase = a.v_codes + static_cast<int64_t>(bh) * D * a.n_pad;
  const float* brow = a.bias + (static_cast<int64_t>(bh) * a.nblk + qb) * a.n_pad;
  const int n_kscale = a.gran == SAGE_GRAN_THREAD ? a.n_pad / 16 : a.n_pad / 64;
  const float* kscale = a.k_scale + static_cast<int64_t>(bh) * n_kscale;
  const TileSrc src = make_tile_src<D>(kbase, vbase, brow, kscale, n_kscale, a.n_pad, t);
  issue_tile<D>(buf0, src, 0, w);

  i32x4 qf[KS];
  {
    const int8_t* qrow = a.q_codes + (static_cast<int64_t>(bh) * a.n_pad + qi) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = *reinterpret_cast<const i32x4*>(qrow + 32 * s + 16 * hh);
  }
  float dq;
  if (a.gran == SAGE_GRAN_THREAD) {
    dq = a.q_scale[static_cast<int64_t>(bh) * a.n_pad + qi];
  } else if (a.gran == SAGE_GRAN_WARP) {
    dq = a.q_scale[static_cast<int64_t>(bh) * (a.n_pad / 32) + (qi >> 5)];
  } else {
    dq = a.q_scale[static_cast<int64_t>(bh) * a.nblk + qb];
  }
  const float dq2 = dq * a.scale_log2;

  f32x16 oacc[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[c][i] = 0.f;
  float m = -INFINITY, lsum = 0.f;

  auto step = [&](const int tt, uint8_t* cur, uint8_t* nxt) __attribute__((always_inline)) {
    const int k0 = tt * 128;
    // This thread's copies of tile tt are complete; after the barrier everyone's
    // are, and every wave has finished reading `nxt` (it held tile tt-1).
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tt + 1 < ntiles) issue_tile<D>(nxt, src, k0 + 128, w);

    const int8_t* ks = reinterpret_cast<const int8_t*>(cur);
    const uint8_t* vs = cur + TileBuf<D>::K_BYTES;
    const float* bs = reinterpret_cast<const float*>(cur + TileBuf<D>::K_BYTES + TileBuf<D>::V_BYTES);
    const float* ksc = reinterpret_cast<const float*>(cur + TileBuf<D>::K_BYTES + TileBuf<D>::V_BYTES +
                                                      TileBuf<D>::B_BYTES);
    float cs[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) cs[st] = dq2 * (a.gran == SAGE_GRAN_THREAD ? ksc[2 * st + hh] : ksc[st >> 1]);

    // S^T tile: 4 subtiles of 32 keys.
    i32x16 sacc[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[st][i] = 0;
      const int r = 32 * st + col;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const i32x4 kf = *reinterpret_cast<const i32x4*>(ks + r * D + 16 * swz<D>(r, 2 * s + hh));
        sacc[st] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qf[s], sacc[st], 0, 0, 0);
      }
    }

    float x[4][16];
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const float4 bv = *reinterpret_cast<const float4*>(bs + 32 * st + 8 * a4 + 4 * hh);
        x[st][4 * a4 + 0] = static_cast<float>(sacc[st][4 * a4 + 0]) * cs[st] + bv.x;
        x[st][4 * a4 + 1] = static_cast<float>(sacc[st][4 * a4 + 1]) * cs[st] + bv.y;
        x[st][4 * a4 + 2] = static_cast<float>(sacc[st][4 * a4 + 2]) * cs[st] + bv.z;
        x[st][4 * a4 + 3] = static_cast<float>(sacc[st][4 * a4 + 3]) * cs[st] + bv.w;
        __builtin_amdgcn_sched_barrier(0);   // consume each bias quad before fetching the next
      }
    const bool need_mask = (k0 + 128 > a.N) || (a.causal && k0 + 127 > q0 + 32 * w);
    if (need_mask) {
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = k0 + 32 * st + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (j >= a.N || (a.causal && j > qi)) x[st][r] = -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, x[st][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mnew = fmaxf(m, mt);
    const float alpha = (m == mnew) ? 1.f : ((m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mnew));
    const float base = (mnew == -INFINITY) ? 0.f : mnew - a.log2_pr;
    float ps = 0.f;
    i32x8 pb[2];
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float p0 = __builtin_amdgcn_exp2f(x[st][4 * q4 + 0] - base);
        const float p1 = __builtin_amdgcn_exp2f(x[st][4 * q4 + 1] - base);
        const float p2 = __builtin_amdgcn_exp2f(x[st][4 * q4 + 2] - base);
        const float p3 = __builtin_amdgcn_exp2f(x[st][4 * q4 + 3] - base);
        ps += (p0 + p1) + (p2 + p3);
        int v = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, __float_as_int(p0), false);
        v = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, v, true);
        pb[st >> 1][4 * (st & 1) + q4] = v;
      }
    lsum = alpha * lsum + ps;
    m = mnew;
    // Exact skip: when no row maximum of this wave moved, alpha == 1 everywhere.
    if (!__all(alpha == 1.f)) {
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[c][i] *= alpha;
    }

#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const int ch = 32 * c + col;
        const uint4 v0 = *reinterpret_cast<const uint4*>(vs + ch * 128 + 16 * swz<128>(ch, 4 * kc + 2 * hh));
        const uint4 v1 = *reinterpret_cast<const uint4*>(vs + ch * 128 + 16 * swz<128>(ch, 4 * kc + 2 * hh + 1));
        i32x8 va;
        va[0] = static_cast<int>(v0.x); va[1] = static_cast<int>(v0.y);
        va[2] = static_cast<int>(v0.z); va[3] = static_cast<int>(v0.w);
        va[4] = static_cast<int>(v1.x); va[5] = static_cast<int>(v1.y);
        va[6] = static_cast<int>(v1.z); va[7] = static_cast<int>(v1.w);
        oacc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb[kc], oacc[c], 0, 0, 0, 0, 0, 0);
      }
    }
  };
  for (int tt = 0; tt < ntiles; tt += 2) {
    step(tt, buf0, buf1);
    if (tt + 1 < ntiles) step(tt + 1, buf1, buf0);
  }

  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float inv = 1.f / ltot;
  if (qi < a.N) {
    const int b = bh / a.H, h = bh % a.H;
    uint16_t* orow = static_cast<uint16_t*>(a.o) + b * a.oB + h * a.oH + static_cast<int64_t>(qi) * a.oN;
    const float* vsc = a.v_scale + static_cast<int64_t>(bh) * D;
    const float* vmn = a.v_mean + static_cast<int64_t>(bh) * D;
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int c0 = 32 * c + 8 * a4 + 4 * hh;
        const float4 dv = *reinterpret_cast<const float4*>(vsc + c0);
        const float4 mv = *reinterpret_cast<const float4*>(vmn + c0);
        const float o0 = oacc[c][4 * a4 + 0] * (dv.x * inv) + mv.x;
        const float o1 = oacc[c][4 * a4 + 1] * (dv.y * inv) + mv.y;
        const float o2 = oacc[c][4 * a4 + 2] * (dv.z * inv) + mv.z;
        const float o3 = oacc[c][4 * a4 + 3] * (dv.w * inv) + mv.w;
        uint16_t hv[4];
        if constexpr (BF16) {
          hv[0] = to_bf16_rne(o0); hv[1] = to_bf16_rne(o1); hv[2] = to_bf16_rne(o2); hv[3] = to_bf16_rne(o3);
        } else {
          hv[0] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(o0));
          hv[1] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(o1));
          hv[2] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(o2));
          hv[3] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(o3));
        }
        *reinterpret_cast<uint2*>(orow + c0) = *reinterpret_cast<const uint2*>(hv);
      }
  }
}

template <int D, bool BF16>
hipError_t attn_impl(const Problem& p, const sage_qk_buffers& qk, const sage_v_buffers& vb, int causal, void* o,
                     const int64_t o_stride[3], hipStream_t st) {
  AttnArgs a;
  a.q_codes = qk.q_codes; a.q_scale = qk.q_scale; a.k_codes = qk.k_codes; a.k_scale = qk.k_scale;
  a.bias = qk.bias; a.v_codes = vb.v_codes; a.v_scale = vb.v_scale; a.v_mean = vb.v_mean;
  a.o = o; a.oB = o_stride[0]; a.oH = o_stride[1]; a.oN = o_stride[2];
  a.H = p.H; a.N = p.N; a.n_pad = p.n_pad; a.nblk = p.nblk; a.gran = p.gran; a.causal = causal ? 1 : 0;
  a.scale_log2 = p.sm_scale * 1.4426950408889634f;
  a.log2_pr = log2f(p.p_range);
  hipLaunchKernelGGL((attn_fwd_kernel<D, BF16>), dim3(p.nblk * p.B * p.H), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const Problem& p, const sage_qk_buffers& qk, const sage_v_buffers& vb, int causal,
                           void* o, const int64_t o_stride[3], hipStream_t st) {
  if (p.D == 128) return p.bf16 ? attn_impl<128, true>(p, qk, vb, causal, o, o_stride, st)
                                : attn_impl<128, false>(p, qk, vb, causal, o, o_stride, st);
  return p.bf16 ? attn_impl<64, true>(p, qk, vb, causal, o, o_stride, st)
                : attn_impl<64, false>(p, qk, vb, causal, o, o_stride, st);
}

}  // namespace sage
