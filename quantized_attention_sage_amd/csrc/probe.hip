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
//    softmax over the keys of split s for the 128 rows of the block.  Eight
//    lanes share four rows, each holding an eighth of q and of the four output
//    rows, so that every K or V value read from LDS feeds four FMAs (LDS
//    bandwidth, not the FMA rate, bounds this loop otherwise); a score is the
//    sum of the eight partial dot products.  K and V sub-tiles of 8 keys are
//    staged in LDS as fp32.
//  * exact_merge_kernel: one work-group per (head, row), one lane per channel,
//    combines the splits (max of the running maxima, then the weighted sums)
//    into the reference rows.
//  * probe_sums_kernel / probe_total_kernel: fp64 sums over the valid rows of
//    every head, then over the heads in order.
#include "sage_internal.h"

namespace sage {
namespace {

constexpr int kRows = 128;   // one query block
constexpr int kSub = 8;      // keys per LDS sub-tile

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

// Sum over each aligned group of 8 lanes, with DPP lane moves (no LDS
// round trip): swap neighbours, swap pairs, then mirror within the 8.
__device__ __forceinline__ float dpp_f(float x, int ctrl_sel) {
  const int v = __float_as_int(x);
  int r;
  if (ctrl_sel == 0) r = __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);        // quad_perm [1,0,3,2]
  else if (ctrl_sel == 1) r = __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  else r = __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);                     // row_half_mirror
  return __int_as_float(r);
}
__device__ __forceinline__ float sum8(float x) {
  x += dpp_f(x, 0);
  x += dpp_f(x, 1);
  return x + dpp_f(x, 2);
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void exact_part_kernel(ExactArgs a) {
  constexpr int LPR = 8;          // lanes sharing a row
  constexpr int RPL = 4;          // rows per lane: each value read from LDS feeds RPL FMAs
  constexpr int DQ = D / LPR;     // channels per lane
  constexpr int RS = DQ + 4;      // segment stride in LDS: the eight segments fall in different banks
  __shared__ __attribute__((aligned(16))) float ks[kSub][LPR][RS];
  __shared__ __attribute__((aligned(16))) float vs[kSub][LPR][RS];
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
  const int g = l / LPR, qd = l % LPR;
  // rows of this lane: 32 w + g + 8 u, u < RPL; channels DQ qd ..
  const int split = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;

  float q[RPL][DQ], o[RPL][DQ], m[RPL], lsum[RPL];
  int qi[RPL];
#pragma unroll
  for (int u = 0; u < RPL; ++u) {
    qi[u] = a.q0 + 32 * w + g + 8 * u;
    const int64_t base = b * a.qs0 + h * a.qs1 + static_cast<int64_t>(min(qi[u], a.N - 1)) * a.qs2 + qd * DQ;
#pragma unroll
    for (int c = 0; c < DQ; ++c) {
      q[u][c] = qi[u] < a.N ? ld16<BF16>(a.q, base + c) : 0.f;
      o[u][c] = 0.f;
    }
    m[u] = -INFINITY;
    lsum[u] = 0.f;
  }

  const int kb = split * a.chunk, ke = min(a.key_end, kb + a.chunk);
  const int64_t kbase = b * a.ks0 + h * a.ks1, vbase = b * a.vs0 + h * a.vs1;
  constexpr int LOADS = kSub * D / 8;   // 16-byte loads per sub-tile and tensor
  for (int j0 = kb; j0 < ke; j0 += kSub) {
    __syncthreads();
    if (t < LOADS) {
      const int jj = t / (D / 8), c = 8 * (t % (D / 8)), j = j0 + jj;
      float fk[8], fv[8];
      if (j < ke) {
        cvt8<BF16>(*reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k) + kbase +
                                                   static_cast<int64_t>(j) * a.ks2 + c), fk);
        cvt8<BF16>(*reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.v) + vbase +
                                                   static_cast<int64_t>(j) * a.vs2 + c), fv);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) fk[i] = fv[i] = 0.f;
      }
      float* kd = &ks[jj][c / DQ][c % DQ];
      float* vd = &vs[jj][c / DQ][c % DQ];
#pragma unroll
      for (int i = 0; i < 8; i += 4) {
        *reinterpret_cast<float4*>(kd + i) = make_float4(fk[i], fk[i + 1], fk[i + 2], fk[i + 3]);
        *reinterpret_cast<float4*>(vd + i) = make_float4(fv[i], fv[i + 1], fv[i + 2], fv[i + 3]);
      }
    }
    __syncthreads();
    float sc[RPL][kSub];
    float mt[RPL];
#pragma unroll
    for (int u = 0; u < RPL; ++u) mt[u] = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < kSub; ++jj) {
      float kr[DQ];
#pragma unroll
      for (int c = 0; c < DQ; ++c) kr[c] = ks[jj][qd][c];
      const int j = j0 + jj;
      float dot[RPL];
#pragma unroll
      for (int u = 0; u < RPL; ++u) dot[u] = 0.f;
#pragma unroll
      for (int c = 0; c < DQ; ++c)     // rows innermost: RPL independent FMA chains
#pragma unroll
        for (int u = 0; u < RPL; ++u) dot[u] = fmaf(q[u][c], kr[c], dot[u]);
#pragma unroll
      for (int u = 0; u < RPL; ++u) {
        const float d8 = sum8(dot[u]);
        const bool vis = j < ke && (!a.causal || j <= qi[u]);
        sc[u][jj] = vis ? d8 * a.scale_log2 : -INFINITY;
        mt[u] = fmaxf(mt[u], sc[u][jj]);
      }
    }
    float mn[RPL];
#pragma unroll
    for (int u = 0; u < RPL; ++u) {
      mn[u] = fmaxf(m[u], mt[u]);
      // alpha = 0 while m is -inf; a row with no visible key yet keeps m = -inf, o = 0, l = 0
      const float alpha = mn[u] == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[u] - mn[u]);
      lsum[u] *= alpha;
#pragma unroll
      for (int c = 0; c < DQ; ++c) o[u][c] *= alpha;
#pragma unroll
      for (int jj = 0; jj < kSub; ++jj)
        sc[u][jj] = mn[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[u][jj] - mn[u]);
      m[u] = mn[u];
    }
#pragma unroll
    for (int jj = 0; jj < kSub; ++jj) {
      float vr[DQ];
#pragma unroll
      for (int c = 0; c < DQ; ++c) vr[c] = vs[jj][qd][c];
#pragma unroll
      for (int u = 0; u < RPL; ++u) {
        lsum[u] += sc[u][jj];
#pragma unroll
        for (int c = 0; c < DQ; ++c) o[u][c] = fmaf(sc[u][jj], vr[c], o[u][c]);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < RPL; ++u) {
    const int r = 32 * w + g + 8 * u;
    float* dst = a.part + ((static_cast<int64_t>(split) * gridDim.y + bh) * kRows + r) * (D + 2);
#pragma unroll
    for (int c = 0; c < DQ; ++c) dst[qd * DQ + c] = o[u][c];
    if (qd == 0) {
      dst[D] = m[u];
      dst[D + 1] = lsum[u];
    }
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

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

ProbeLayout probe_layout(int B, int H, int N, int D, int io_bytes) {
  ProbeLayout L;
  const int64_t BH = static_cast<int64_t>(B) * H;
  const int n_pad = (N + 127) / 128 * 128;
  // at most 64 key splits; splits are whole 32-key sub-tiles
  L.chunk = n_pad <= 64 * 1024 ? 1024 : ((n_pad + 63) / 64 + kSub - 1) / kSub * kSub;
  L.splits = (n_pad + L.chunk - 1) / L.chunk;
  size_t off = 0;
  L.ref = off;  off = align256(off + BH * kRows * D * 4);
  L.o4 = off;   off = align256(off + BH * kRows * D * io_bytes);
  L.o8 = off;   off = align256(off + BH * kRows * D * io_bytes);
  L.part = off; off = align256(off + static_cast<size_t>(L.splits) * BH * kRows * (D + 2) * 4);
  L.sums = off; off = align256(off + BH * 8 * 8);
  L.total = off; off = align256(off + 8 * 8);
  L.bytes = off;
  return L;
}

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
