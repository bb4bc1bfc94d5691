// Adaptive INT4/INT8 choice: exact reference attention on one sampled query
// block of every head, and the accuracy sums of two quantized outputs of the
// same rows against it.
//
// Method: the SageAttention2 abstract measures the accuracy of the quantized
// attention across layers and timesteps and picks the QK precision from it
// ("adaptive quantization"); accuracy is measured as in the SageAttention2++
// summary ("A.2 Datasets and Metrics"): cosine similarity and relative L1
// distance against full-precision attention.
//
//  * exact_part_kernel: work-group (split s, head bh) runs a plain fp32 online
//    softmax over the keys of split s for the 128 rows of the block, on the
//    fp32 matrix cores (v_mfma_f32_32x32x2_f32, fp32 products and sums).  As
//    in the quantized kernel, S^T = K Q^T puts one query and 16 keys in each
//    lane, so the row maximum takes one exchange with lane l ^ 32 and the
//    lane's P values are directly the B operand of O^T += V^T P^T.  K and V
//    sub-tiles of 64 keys are staged in LDS as fp32 (V transposed), the next
//    one's loads in flight during the current one's products.
//  * exact_merge_kernel: one work-group per (head, row), one lane per channel,
//    combines the splits (max of the running maxima, then the weighted sums)
//    into the reference rows.
//  * probe_sums_kernel / probe_total_kernel: fp64 sums over the valid rows of
//    every head, then over the heads in order.
#include "sage_internal.h"

namespace sage {
namespace {

constexpr int kRows = kProbeRows;   // one query block
constexpr int kSub = kProbeSub;     // split lengths past 64 Ki keys are multiples of this

template <bool BF16>
__device__ __forceinline__ float ld16(const void* base, int64_t i) {
  const uint16_t u = static_cast<const uint16_t*>(base)[i];
  if constexpr (BF16) return __uint_as_float(static_cast<uint32_t>(u) << 16);
  else return static_cast<float>(__builtin_bit_cast(_Float16, u));
}

struct ExactArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t qs0, qs1, qs2, ks0, ks1, ks2, vs0, vs1, vs2;   // element strides
  int H, N, q0, key_end, chunk, causal;
  float scale_log2;    // sm_scale * log2(e)
  float* part;         // [S, BH, 128, D + 2]: unnormalised row, running max, row sum
};

// 8 bf16/fp16 values (16 bytes) to fp32
template <bool BF16>
__device__ __forceinline__ void cvt8(uint4 u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (BF16) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    } else {
      f[2 * i] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i] & 0xffffu)));
      f[2 * i + 1] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i] >> 16)));
    }
  }
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int D, bool BF16>
__global__ __launch_bounds__(256, 2) void exact_part_kernel(ExactArgs a) {
  constexpr int KT = 64;                 // keys per LDS sub-tile
  constexpr int KR = D + 4;              // K row stride (floats): a wave's 32 rows fall in different banks
  constexpr int VR = KT + 4;             // V^T row stride (floats)
  constexpr int HC = D / 2;              // channels per lane half
  constexpr int CT = D / 32;             // 32-channel output tiles
  constexpr int PF = KT * D / 8 / 256;   // 16-byte loads per thread, tensor and sub-tile
  __shared__ __attribute__((aligned(16))) float kl[KT * KR];   // K [key][channel]
  __shared__ __attribute__((aligned(16))) float vt[D * VR];    // V^T [channel][key]
  const int t = threadIdx.x, l = t & 63, w = t >> 6, col = l & 31, hh = l >> 5;
  const int split = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;
  const int qi = a.q0 + 32 * w + col;    // this lane's query (column of the 32x32 products)

  // B operand of product i (i < HC): Q[qi][HC hh + i], so that one product
  // pairs channel i (lanes 0-31) with channel HC + i (lanes 32-63).
  float qr[HC];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + b * a.qs0 + h * a.qs1 +
                           static_cast<int64_t>(min(qi, a.N - 1)) * a.qs2 + HC * hh;
#pragma unroll
    for (int c8 = 0; c8 < HC / 8; ++c8) {
      float f[8];
      cvt8<BF16>(*reinterpret_cast<const uint4*>(qrow + 8 * c8), f);
#pragma unroll
      for (int e = 0; e < 8; ++e) qr[8 * c8 + e] = qi < a.N ? f[e] : 0.f;
    }
  }
  f32x16 oacc[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[c][i] = 0.f;
  float m = -INFINITY, lsum = 0.f;

  const int kb = split * a.chunk, ke = min(a.key_end, kb + a.chunk);
  const uint16_t* kg = static_cast<const uint16_t*>(a.k) + b * a.ks0 + h * a.ks1;
  const uint16_t* vg = static_cast<const uint16_t*>(a.v) + b * a.vs0 + h * a.vs1;
  // Load p of a sub-tile: key (t + 256 p) / (D/8), channels 8 ((t + 256 p) % (D/8)) ..; keys past ke read as 0.
  // The loads go through raw buffer resources over the sub-tile's keys below
  // ke (a load past the end returns zeros), so that none is guarded by a
  // branch and all of them issue back to back.
  uint4 kp[PF], vp[PF];
  auto fetch = [&](int j0) __attribute__((always_inline)) {
    const int64_t nk = max(0, min(KT, ke - j0));
    const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kg + static_cast<int64_t>(j0) * a.ks2), 0,
                                                      static_cast<int>(nk * a.ks2 * 2), kBufferWord3);
    const auto rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vg + static_cast<int64_t>(j0) * a.vs2), 0,
                                                      static_cast<int>(nk * a.vs2 * 2), kBufferWord3);
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int idx = t + 256 * p, kk = idx / (D / 8), c = 8 * (idx % (D / 8));
      const auto xk = __builtin_amdgcn_raw_buffer_load_b128(rk, kk * static_cast<int>(a.ks2) * 2 + 2 * c, 0, 0);
      const auto xv = __builtin_amdgcn_raw_buffer_load_b128(rv, kk * static_cast<int>(a.vs2) * 2 + 2 * c, 0, 0);
      kp[p] = make_uint4(xk[0], xk[1], xk[2], xk[3]);
      vp[p] = make_uint4(xv[0], xv[1], xv[2], xv[3]);
    }
  };
  if (kb < ke) fetch(kb);
  for (int j0 = kb; j0 < ke; j0 += KT) {
    __syncthreads();   // every wave is done with the previous sub-tile
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int idx = t + 256 * p, kk = idx / (D / 8), c = 8 * (idx % (D / 8));
      float fk[8], fv[8];
      cvt8<BF16>(kp[p], fk);
      cvt8<BF16>(vp[p], fv);
      *reinterpret_cast<float4*>(&kl[kk * KR + c]) = make_float4(fk[0], fk[1], fk[2], fk[3]);
      *reinterpret_cast<float4*>(&kl[kk * KR + c + 4]) = make_float4(fk[4], fk[5], fk[6], fk[7]);
#pragma unroll
      for (int e = 0; e < 8; ++e) vt[(c + e) * VR + kk] = fv[e];
    }
    __syncthreads();
    if (j0 + KT < ke) fetch(j0 + KT);   // the next sub-tile's loads fly during this one's products
#pragma unroll
    for (int s = 0; s < KT / 32; ++s) {
      // S^T of keys j0 + 32 s ..: A operand of product i is K[key 32 s + col][HC hh + i].
      f32x16 sacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
      const float* krow = &kl[(32 * s + col) * KR + HC * hh];
#pragma unroll
      for (int i4 = 0; i4 < HC / 4; ++i4) {
        const float4 kv = *reinterpret_cast<const float4*>(krow + 4 * i4);
        sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.x, qr[4 * i4 + 0], sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.y, qr[4 * i4 + 1], sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.z, qr[4 * i4 + 2], sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.w, qr[4 * i4 + 3], sacc, 0, 0, 0);
      }
      // sacc[i]: key j0 + 32 s + 8 (i / 4) + 4 hh + i % 4 of query qi; lane l ^ 32 holds the other 16 keys.
      float sc[16];
      float mt = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = j0 + 32 * s + 8 * (i >> 2) + 4 * hh + (i & 3);
        const bool vis = j < ke && (!a.causal || j <= qi);
        sc[i] = vis ? sacc[i] * a.scale_log2 : -INFINITY;
        mt = fmaxf(mt, sc[i]);
      }
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float mn = fmaxf(m, mt);
      // alpha = 0 while m is -inf; a row with no visible key yet keeps m = -inf, o = 0, l = 0
      const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - mn);
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sc[i] = mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[i] - mn);
        ps += sc[i];
      }
      lsum = lsum * alpha + ps;
      m = mn;
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[c][i] *= alpha;
      // O^T += V^T P^T: A operand V[key 32 s + 8 jq + 4 hh + e][32 c + col], B operand this lane's P.
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const float* vrow = &vt[(32 * c + col) * VR + 32 * s + 4 * hh];
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          const float4 vv = *reinterpret_cast<const float4*>(vrow + 8 * jq);
          oacc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.x, sc[4 * jq + 0], oacc[c], 0, 0, 0);
          oacc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.y, sc[4 * jq + 1], oacc[c], 0, 0, 0);
          oacc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.z, sc[4 * jq + 2], oacc[c], 0, 0, 0);
          oacc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.w, sc[4 * jq + 3], oacc[c], 0, 0, 0);
        }
      }
    }
  }
  // oacc[c][i]: channel 32 c + 8 (i / 4) + 4 hh + i % 4 of query qi
  const float ltot = lsum + __shfl_xor(lsum, 32);
  float* dst = a.part + ((static_cast<int64_t>(split) * gridDim.y + bh) * kRows + 32 * w + col) * (D + 2);
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      float* d = dst + 32 * c + 8 * jq + 4 * hh;    // rows are (D + 2) floats: 8-byte aligned
      *reinterpret_cast<float2*>(d) = make_float2(oacc[c][4 * jq + 0], oacc[c][4 * jq + 1]);
      *reinterpret_cast<float2*>(d + 2) = make_float2(oacc[c][4 * jq + 2], oacc[c][4 * jq + 3]);
    }
  if (hh == 0) {
    dst[D] = m;
    dst[D + 1] = ltot;
  }
}

struct MergeArgs {
  const float* part;
  float* ref;        // [BH, 128, D]
  int S, BH, q0, N;
};

template <int D>
__global__ __launch_bounds__(D) void exact_merge_kernel(MergeArgs a) {
  const int bh = blockIdx.x, r = blockIdx.y, c = threadIdx.x;
  const float* row0 = a.part + (static_cast<int64_t>(bh) * kRows + r) * (D + 2);
  const int64_t split_stride = static_cast<int64_t>(a.BH) * kRows * (D + 2);
  float mx = -INFINITY;
  for (int s = 0; s < a.S; ++s) mx = fmaxf(mx, row0[s * split_stride + D]);
  float lt = 0.f, ot = 0.f;
  for (int s = 0; s < a.S; ++s) {
    const float* p = row0 + s * split_stride;
    if (p[D] == -INFINITY) continue;
    const float wgt = __builtin_amdgcn_exp2f(p[D] - mx);
    lt = fmaf(wgt, p[D + 1], lt);
    ot = fmaf(wgt, p[c], ot);
  }
  a.ref[(static_cast<int64_t>(bh) * kRows + r) * D + c] = (a.q0 + r < a.N && lt > 0.f) ? ot / lt : 0.f;
}

struct SumArgs {
  const void* o4;    // [BH, 128, D] of the I/O type
  const void* o8;
  const float* ref;  // [BH, 128, D]
  double* part;      // [BH, 8]
  int rows;          // valid rows of the block
};

// Sums: <o4,r>, |o4|^2, <o8,r>, |o8|^2, |r|^2, |o4-r|_1, |o8-r|_1, |r|_1
template <int D, bool BF16>
__global__ __launch_bounds__(256) void probe_sums_kernel(SumArgs a) {
  __shared__ double red[8][256];
  const int t = threadIdx.x, bh = blockIdx.x;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const int64_t base = static_cast<int64_t>(bh) * kRows * D;
  for (int e = t; e < a.rows * D; e += 256) {
    const double r = a.ref[base + e];
    const double x4 = ld16<BF16>(a.o4, base + e), x8 = ld16<BF16>(a.o8, base + e);
    acc[0] += x4 * r;
    acc[1] += x4 * x4;
    acc[2] += x8 * r;
    acc[3] += x8 * x8;
    acc[4] += r * r;
    acc[5] += fabs(x4 - r);
    acc[6] += fabs(x8 - r);
    acc[7] += fabs(r);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[i][t] = acc[i];
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s)
#pragma unroll
      for (int i = 0; i < 8; ++i) red[i][t] += red[i][t + s];
    __syncthreads();
  }
  if (t < 8) a.part[bh * 8 + t] = red[t][0];
}

__global__ void probe_total_kernel(const double* part, double* out, int BH) {
  const int t = threadIdx.x;
  if (t < 8) {
    double s = 0.0;
    for (int bh = 0; bh < BH; ++bh) s += part[bh * 8 + t];
    out[t] = s;
  }
}

}  // namespace

hipError_t launch_probe_reference(const Problem& p, TensorView q, TensorView k, TensorView v, int causal, int q_block,
                                  char* scratch, hipStream_t st) {
  const ProbeLayout L = probe_layout(p.B, p.H, p.N, p.D, 2);
  ExactArgs a;
  a.q = q.ptr; a.k = k.ptr; a.v = v.ptr;
  a.qs0 = q.sB; a.qs1 = q.sH; a.qs2 = q.sN;
  a.ks0 = k.sB; a.ks1 = k.sH; a.ks2 = k.sN;
  a.vs0 = v.sB; a.vs1 = v.sH; a.vs2 = v.sN;
  a.H = p.H; a.N = p.N; a.q0 = kRows * q_block;
  a.key_end = causal ? min(p.N, a.q0 + kRows) : p.N;
  a.chunk = L.chunk; a.causal = causal;
  a.scale_log2 = p.sm_scale * 1.4426950408889634f;
  a.part = reinterpret_cast<float*>(scratch + L.part);
  const int BH = p.B * p.H;
  const dim3 grid(L.splits, BH);
  if (p.D == 128) {
    if (p.bf16) hipLaunchKernelGGL((exact_part_kernel<128, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((exact_part_kernel<128, false>), grid, dim3(256), 0, st, a);
  } else {
    if (p.bf16) hipLaunchKernelGGL((exact_part_kernel<64, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((exact_part_kernel<64, false>), grid, dim3(256), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  MergeArgs mg{a.part, reinterpret_cast<float*>(scratch + L.ref), L.splits, BH, a.q0, p.N};
  if (p.D == 128) hipLaunchKernelGGL((exact_merge_kernel<128>), dim3(BH, kRows), dim3(128), 0, st, mg);
  else hipLaunchKernelGGL((exact_merge_kernel<64>), dim3(BH, kRows), dim3(64), 0, st, mg);
  return hipGetLastError();
}

hipError_t launch_probe_sums(const Problem& p, int q_block, char* scratch, hipStream_t st) {
  const ProbeLayout L = probe_layout(p.B, p.H, p.N, p.D, 2);
  SumArgs a;
  a.o4 = scratch + L.o4;
  a.o8 = scratch + L.o8;
  a.ref = reinterpret_cast<const float*>(scratch + L.ref);
  a.part = reinterpret_cast<double*>(scratch + L.sums);
  a.rows = min(kRows, p.N - kRows * q_block);
  const int BH = p.B * p.H;
  if (p.D == 128) {
    if (p.bf16) hipLaunchKernelGGL((probe_sums_kernel<128, true>), dim3(BH), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((probe_sums_kernel<128, false>), dim3(BH), dim3(256), 0, st, a);
  } else {
    if (p.bf16) hipLaunchKernelGGL((probe_sums_kernel<64, true>), dim3(BH), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((probe_sums_kernel<64, false>), dim3(BH), dim3(256), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(probe_total_kernel, dim3(1), dim3(64), 0, st, a.part,
                     reinterpret_cast<double*>(scratch + L.total), BH);
  return hipGetLastError();
}

}  // namespace sage
