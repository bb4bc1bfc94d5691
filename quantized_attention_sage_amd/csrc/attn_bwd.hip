// 8-bit attention backward for gfx950 (CDNA4).
//
// The SageAttention3 abstract's 8-bit attention for backward propagation,
// read as FlashAttention's backward (D = rowsum(dO o O); P = 2^(s - L);
// dV = P^T dO; dP = dO V^T; dS = P o (dP - D); dQ = c dS K'; dK = c dS^T Q)
// with every product on 8-bit operands whose scales are constant along the
// product's reduction axis (include/sage.h, sage_attn_bwd):
//   * S and dP on v_mfma_i32_32x32x32_i8: the forward's own Q/K codes, and
//     dO / V as INT8 with the THREAD granularity's groups;
//   * dV, dQ and dK on v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands:
//     P with the fixed scale 1/P_r; dS with one power-of-two (E8M0) scale per
//     64-element group along the reduced axis, which the instruction applies
//     per lane; dO, K' and Q with per-channel scales applied at the end.
//
// Three kernels, each the layout of the forward kernel, two with roles
// exchanged:
//  * bwd_dq_kernel: one work-group of 4 waves per 128-query block; wave w
//    owns 32 queries, lane l query l%32.  S^T = K^ Q^T and dP^T = V^ dO^T put
//    a query's 16 keys of each 32-key subtile in one lane, so the dS group of
//    a query row and 64 keys is that lane plus lane l^32, and the lane's FP8
//    dS codes are its B operand of dQ^T += K'^T dS^T.
//  * bwd_dkv_kernel<D, 1> (dV) and <D, 2> (dK): one work-group per 128-key
//    block; lane l holds key l%32.  S = Q^ K^T (and dP = dO^ V^T) put a key's
//    16 queries of each 32-query subtile in one lane, for dV^T += dO^T P and
//    dK^T += Q^T dS.  Split in two so that each holds one accumulator set and
//    two work-groups fit on a CU (dV: three; the dK kernel recomputes S and P).
// Each walks the other axis in 64-row half tiles through a three-slot LDS
// ring filled by direct global-to-LDS copies two half tiles ahead; work-group
// ids are regrouped so that each XCD runs a contiguous run of (head, block)
// items, whose streamed rows are then fetched into that XCD's L2.
#include <hip/hip_runtime.h>

#include <cmath>

#include "sage_internal.h"

namespace sage {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kT = 128;   // queries per block and keys per tile

struct BwdArgs {
  // forward quantisation (S recompute)
  const int8_t* q_codes;
  const float* q_scale;     // THREAD granularity: one per token
  const int8_t* k_codes;
  const float* k_scale;     // one per 16-key group
  const float* bias;        // [B, H, nblk, n_pad], in log2 units
  const float* lse;         // [B, H, n_pad]
  // INT8 dO (query side) and V (key side) for dP
  const int8_t* do_codes;
  const float* do_scale;
  const int8_t* v_codes;
  const float* v_scale;
  // E4M3 channel-major [B, H, d, n_pad] (64-token permuted groups) with per-channel scales
  const uint8_t* do8_codes;
  const float* do8_scale;
  const uint8_t* q8_codes;
  const float* q8_scale;
  const uint8_t* k8_codes;
  const float* k8_scale;
  const float* dsum;        // [B, H, n_pad]
  float* dq;
  float* dk;
  float* dv;                // [B, H, N, d] fp32, contiguous
  int H, N, n_pad, nblk, causal;
  float scale_log2;         // sm_scale * log2(e)
  float sm_scale;
  float p_range;
  float p_range_log2;       // log2(p_range): P P_r = 2^(s - L + log2 P_r)
  const float* lse_do;      // L - log2 s_dO per row (+inf where s_dO = 0)
  const float* dsum_do;     // D / s_dO per row (0 where s_dO = 0)
};

// 16-byte chunk swizzle inside an LDS row (bank-conflict-free fragment reads;
// self-inverse in `chunk`).
template <int ROW_BYTES>
__device__ __forceinline__ int swz(int row, int chunk) {
  constexpr int CPR = ROW_BYTES / 16;
  constexpr int RPW = 256 / ROW_BYTES;
  return chunk ^ ((row / RPW) & (CPR - 1));
}

// Global -> LDS copies without registers (buffer_load ... lds: lane L's 16
// bytes land at M0 + 16 L).  Written as inline assembly so that the compiler
// does not track these LDS writes; each kernel waits for them by hand
// (s_waitcnt vmcnt) before the barrier that publishes them.
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ i32x4 buffer_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(a & 0xffffffffu));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>((a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  r[3] = kBufferWord3;
  return r;
}

__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "s"(lds) : "memory", "m0");
}

// Per-lane source offsets of the 16-byte chunks a lane copies: chunk
// 256 j + t of a tile (t = thread) sits at LDS chunk 256 j + t and holds
// (row-major tile) row r, chunk swz(r, c) of the source, or (channel-major
// tile) channel ch, chunk swz(ch, c).  The swizzle term does not depend on j,
// which moves only the scalar offset: 4096 j bytes of rows, 32 j channels.
template <int D>
__device__ __forceinline__ uint32_t rows_off(int t) {
  constexpr int CPR = D / 16;
  const int r = t / CPR, pc = t % CPR;
  return static_cast<uint32_t>(r * D + 16 * swz<D>(r, pc));
}
__device__ __forceinline__ uint32_t cm_off(int t, int n_pad) {
  const int ch = t >> 3, vc = t & 7;
  return static_cast<uint32_t>(ch * n_pad + 16 * swz<128>(ch, vc));
}

// Copies of a 128-row tile starting at row r0 (D / 32 per wave) and of a
// channel-major tile starting at token c0 into the LDS tile at `lds`.
template <int D>
__device__ __forceinline__ void copy_rows(uint32_t lds, i32x4 rs, uint32_t voff, int r0, int w) {
#pragma unroll
  for (int j = 0; j < D / 32; ++j)
    dma16(rs, voff, static_cast<uint32_t>(r0 * D + 4096 * j), lds + (4 * j + w) * 1024);
}
template <int D>
__device__ __forceinline__ void copy_cm(uint32_t lds, i32x4 rs, uint32_t voff, int c0, int n_pad, int w) {
#pragma unroll
  for (int j = 0; j < D / 32; ++j)
    dma16(rs, voff, static_cast<uint32_t>(c0) + 32u * j * static_cast<uint32_t>(n_pad), lds + (4 * j + w) * 1024);
}

// A or B fragment of an INT8 product from a row-major tile: row 32 st + col,
// channels 32 kk + 16 hh .. + 16.
template <int D>
__device__ __forceinline__ i32x4 frag_rows(const uint8_t* tile, int st, int kk, int col, int hh) {
  const int r = 32 * st + col;
  return *reinterpret_cast<const i32x4*>(tile + r * D + 16 * swz<D>(r, 2 * kk + hh));
}

// A fragment of an E4M3 product from a channel-major tile: channel 32 c + col,
// tokens 64 kc + 32 hh .. + 32 (the permuted order of the stored group).
__device__ __forceinline__ i32x8 frag_cm(const uint8_t* tile, int kc, int c, int col, int hh) {
  const int r = 32 * c + col;
  const i32x4 a = *reinterpret_cast<const i32x4*>(tile + r * kT + 16 * swz<128>(r, 4 * kc + 2 * hh));
  const i32x4 b = *reinterpret_cast<const i32x4*>(tile + r * kT + 16 * swz<128>(r, 4 * kc + 2 * hh + 1));
  i32x8 v;
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  return v;
}

// Smallest e with 448 2^e >= amax (amax >= 0), in [-127, 127]: from the bits
// of amax = (1 + M/2^23) 2^E, e = E - 8 when M <= 0.75 2^23, else E - 7.
__device__ __forceinline__ int e8m0_exponent(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int ef = static_cast<int>((u >> 23) & 0xffu);
  if (ef == 0) return -127;
  const int e = (u & 0x7fffffu) <= 0x600000u ? ef - 135 : ef - 134;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// E4M3 codes of 32 values a lane holds for one 64-element step (two subtiles
// of 16), times 2^-e, packed as the 32-byte operand: word 4 sub + q4 holds
// values 4 q4 .. 4 q4 + 3 of subtile sub.  The scaled conversion divides by
// the power of two its scale operand's exponent field encodes (its mantissa is
// ignored), so the scale 2^e (exponent field e + 127, the E8M0 byte) applies
// 2^-e exactly before the rounding; |x| 2^-e <= 448 by the choice of e.
typedef short s16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ i32x8 pack_e4m3(const float (&x)[2][16], int e) {
  const float sc = __uint_as_float(static_cast<uint32_t>(e + 127) << 23);
  i32x8 r;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      s16x2 v = {0, 0};
      v = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v, x[sub][4 * q4 + 0], x[sub][4 * q4 + 1], sc, false);
      v = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v, x[sub][4 * q4 + 2], x[sub][4 * q4 + 3], sc, true);
      r[4 * sub + q4] = __builtin_bit_cast(int, v);
    }
  return r;
}

__device__ __forceinline__ float amax32(const float (&x)[2][16]) {
  float m = 0.f;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(x[sub][r]));
  return fmaxf(m, __shfl_xor(m, 32));
}

// Copies of a 64-key half tile: 64 rows (row-major codes, rows r0..) and D
// channel rows of 64 keys (channel-major codes, keys c0..; 16-byte chunk c of
// channel row r at chunk swz<64>(r, c)).  Lane t's source chunk sits at LDS
// chunk 256 j + t; j moves only the scalar offset (32 rows, or 64 channels).
template <int D>
__device__ __forceinline__ void copy_rows64(uint32_t lds, i32x4 rs, uint32_t voff, int r0, int w) {
#pragma unroll
  for (int j = 0; j < D / 64; ++j)
    dma16(rs, voff, static_cast<uint32_t>(r0 * D + 4096 * j), lds + (4 * j + w) * 1024);
}
__device__ __forceinline__ uint32_t cm64_off(int t, int n_pad) {
  const int ch = t >> 2, c = t & 3;
  return static_cast<uint32_t>(ch * n_pad + 16 * swz<64>(ch, c));
}
template <int D>
__device__ __forceinline__ void copy_cm64(uint32_t lds, i32x4 rs, uint32_t voff, int c0, int n_pad, int w) {
#pragma unroll
  for (int j = 0; j < D / 64; ++j)
    dma16(rs, voff, static_cast<uint32_t>(c0) + 64u * j * static_cast<uint32_t>(n_pad), lds + (4 * j + w) * 1024);
}
__device__ __forceinline__ void dma4(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dword %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "s"(lds) : "memory", "m0");
}
// A fragment of an E4M3 product from a channel-major half tile: channel
// 32 c + col, keys 32 hh .. + 32.
__device__ __forceinline__ i32x8 frag_cm64(const uint8_t* tile, int c, int col, int hh) {
  const int r = 32 * c + col;
  const i32x4 x = *reinterpret_cast<const i32x4*>(tile + r * 64 + 16 * swz<64>(r, 2 * hh));
  const i32x4 y = *reinterpret_cast<const i32x4*>(tile + r * 64 + 16 * swz<64>(r, 2 * hh + 1));
  i32x8 v;
  v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
  v[4] = y[0]; v[5] = y[1]; v[6] = y[2]; v[7] = y[3];
  return v;
}

// Work-group id -> item (head-major, then block).  Work-groups are dispatched
// round-robin over the 8 XCDs, each with its own L2; regrouping consecutive
// ids gives every XCD a contiguous run of items, so the rows that a head's
// blocks all stream through their rings are fetched into one L2.
__device__ __forceinline__ int xcd_item(int id, int total) {
  constexpr int kXcd = 8;
  return total % kXcd == 0 ? (id % kXcd) * (total / kXcd) + id / kXcd : id;
}

// dQ of one 128-query block.  Keys advance in 64-key half tiles through a
// three-slot LDS ring: half tile h + 2 is copied straight from global memory
// (buffer_load ... lds) while half tile h is used.  Each wave issues the same
// number of copies per half tile (NC), so at the top of step h the copies of
// h + 1 are the only ones of this wave that may still run: a wave's vector
// memory loads return in issue order, and the loop issues no others.
template <int D>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a) {
  constexpr int KS = D / 32, CT = D / 32;
  constexpr int KH = 64;                                   // keys per half tile
  constexpr int ROWS = KH * D;                             // bytes of one row-major half tile
  constexpr int AUX = 3 * ROWS;                            // bias (64 floats), K scales, V scales, spare
  constexpr int SLOT = AUX + 4 * 256;
  constexpr int NC = 3 * (D / 64) + 1;                     // copies per wave and half tile
  __shared__ __attribute__((aligned(1024))) uint8_t lds[3 * SLOT];
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)lds));

  const int t = threadIdx.x, l = t & 63, col = l & 31, hh = l >> 5;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int item = xcd_item(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
  const int bh = item / a.nblk;
  int qb = item % a.nblk;
  if (a.causal) qb = a.nblk - 1 - qb;   // longest blocks first
  const int q0 = qb * kT, qi = q0 + 32 * w + col;
  const int64_t row = static_cast<int64_t>(bh) * a.n_pad + qi;

  const int nh = 2 * (a.causal ? qb + 1 : a.nblk);     // half tiles of this block
  const uint32_t head_rows = static_cast<uint32_t>(a.n_pad * D);
  const i32x4 rk = buffer_rsrc(a.k_codes + static_cast<int64_t>(bh) * a.n_pad * D, head_rows);
  const i32x4 rv = buffer_rsrc(a.v_codes + static_cast<int64_t>(bh) * a.n_pad * D, head_rows);
  const i32x4 rk8 = buffer_rsrc(a.k8_codes + static_cast<int64_t>(bh) * D * a.n_pad, head_rows);
  const i32x4 rb = buffer_rsrc(a.bias + (static_cast<int64_t>(bh) * a.nblk + qb) * a.n_pad,
                               static_cast<uint32_t>(a.n_pad * 4));
  const uint32_t nsc = static_cast<uint32_t>(a.n_pad / 16 * 4);
  const i32x4 rks = buffer_rsrc(a.k_scale + static_cast<int64_t>(bh) * (a.n_pad / 16), nsc);
  const i32x4 rvs = buffer_rsrc(a.v_scale + static_cast<int64_t>(bh) * (a.n_pad / 16), nsc);
  const uint32_t off_rows = rows_off<D>(t), off_cm = cm64_off(t, a.n_pad);
  // Slot layout: K rows, V rows, K' E4M3 channel rows, then the half tile's
  // 64 bias values, K scales (4 used) and V scales (4 used); wave 3 copies the
  // bias again into the spare row so that every wave issues NC copies.
  auto copies = [&](int h, int slot) __attribute__((always_inline)) {
    const int k0 = min(h, nh - 1) * KH;        // past the end: the last half tile again (never read)
    const uint32_t base = lds0 + slot * SLOT;
    copy_rows64<D>(base, rk, off_rows, k0, w);
    copy_rows64<D>(base + ROWS, rv, off_rows, k0, w);
    copy_cm64<D>(base + 2 * ROWS, rk8, off_cm, k0, a.n_pad, w);
    const uint32_t lane4 = 4u * static_cast<uint32_t>(l);
    if (w == 1) dma4(rks, lane4, static_cast<uint32_t>(4 * (k0 / 16)), base + AUX + 256);
    else if (w == 2) dma4(rvs, lane4, static_cast<uint32_t>(4 * (k0 / 16)), base + AUX + 512);
    else dma4(rb, lane4, static_cast<uint32_t>(4 * k0), base + AUX + (w == 0 ? 0 : 768));
  };
  copies(0, 0);
  copies(1, 1);

  i32x4 qf[KS], df[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    qf[s] = *reinterpret_cast<const i32x4*>(a.q_codes + row * D + 32 * s + 16 * hh);
    df[s] = *reinterpret_cast<const i32x4*>(a.do_codes + row * D + 32 * s + 16 * hh);
  }
  const float dq2 = a.q_scale[row] * a.scale_log2;
  const float sdo = a.do_scale[row];
  const float Li = a.lse[row], Di = a.dsum[row];

  f32x16 acc[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;

  // entry (query qi, key j) is visible iff j <= lim_q (-1 for padded rows)
  const int lim_q = qi < a.N ? (a.causal ? min(a.N - 1, qi) : a.N - 1) : -1;
#pragma unroll 1
  for (int h = 0; h < nh; ++h) {
    // This wave's copies of half tile h are complete (only the NC of h + 1
    // may still run); after the barrier every wave's are, and every wave is
    // done with the slot of h - 1, which the copies of h + 2 refill.
    if constexpr (NC == 7) asm volatile("s_waitcnt vmcnt(7) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    copies(h + 2, (h + 2) % 3);
    const uint8_t* slot = lds + (h % 3) * SLOT;
    const uint8_t* tk = slot;
    const uint8_t* tv = slot + ROWS;
    const uint8_t* tk8 = slot + 2 * ROWS;
    const float* tb = reinterpret_cast<const float*>(slot + AUX);
    const float* tks = tb + 64;
    const float* tvs = tb + 128;
    const int k0 = h * KH;
    // every entry of the half tile visible (uniform): no per-entry mask
    const bool full = q0 + kT <= a.N && k0 + KH <= a.N && (!a.causal || k0 + KH - 1 <= q0);

    float ds[2][16];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      i32x16 S = {}, dP = {};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        S = __builtin_amdgcn_mfma_i32_32x32x32_i8(frag_rows<D>(tk, sub, kk, col, hh), qf[kk], S, 0, 0, 0);
        dP = __builtin_amdgcn_mfma_i32_32x32x32_i8(frag_rows<D>(tv, sub, kk, col, hh), df[kk], dP, 0, 0, 0);
      }
      const float cs = dq2 * tks[2 * sub + hh];
      const float cd = sdo * tvs[2 * sub + hh];
      // P = exp2(s - L), with s taken as -inf where the entry is masked (P = 0
      // there, and so is dS: D and the dP of padded rows and keys are finite).
      // Key k0 + jt is visible iff jt <= rel, jt = 32 sub + 8 (r / 4) + 4 hh + r % 4.
      const int rel = lim_q - k0 - 4 * hh - 32 * sub;
      float4 b4[4];
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) b4[a4] = *reinterpret_cast<const float4*>(tb + 32 * sub + 4 * hh + 8 * a4);
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        x[r] = static_cast<float>(S[r]) * cs + reinterpret_cast<const float*>(&b4[r >> 2])[r & 3] - Li;
      if (!full)   // uniform
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = 8 * (r >> 2) + (r & 3) <= rel ? x[r] : -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(x[r]);
        const float tdp = static_cast<float>(dP[r]) * cd - Di;
        ds[sub][r] = p * tdp;
      }
    }
    const int e = e8m0_exponent(amax32(ds));
    const i32x8 db = pack_e4m3(ds, e);
#pragma unroll
    for (int c = 0; c < CT; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(frag_cm64(tk8, c, col, hh), db, acc[c], 0, 0, 0,
                                                               127, 0, e + 127);
  }
  // the copies past the end write LDS: they complete before the work-group ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if (qi < a.N) {
    const float* s8 = a.k8_scale + static_cast<int64_t>(bh) * D;
    float* out = a.dq + (static_cast<int64_t>(bh) * a.N + qi) * D;
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int c0 = 32 * c + 8 * a4 + 4 * hh;
        float4 o;
        o.x = acc[c][4 * a4 + 0] * (a.sm_scale * s8[c0 + 0]);
        o.y = acc[c][4 * a4 + 1] * (a.sm_scale * s8[c0 + 1]);
        o.z = acc[c][4 * a4 + 2] * (a.sm_scale * s8[c0 + 2]);
        o.w = acc[c][4 * a4 + 3] * (a.sm_scale * s8[c0 + 3]);
        *reinterpret_cast<float4*>(out + c0) = o;
      }
  }
}

// dV (PART 1) or dK (PART 2) of one 128-key block: lane l holds key l%32 of
// its wave's 32 keys; S = Q^ K^T (and, for dK, dP = dO^ V^T) put a key's 16
// queries of a subtile in one lane.  Queries advance in 64-query half tiles
// through a three-slot LDS ring filled by direct copies two half tiles ahead,
// as in the dQ kernel (NC copies per wave and half tile, waited for by count).
// One accumulator set per kernel keeps two work-groups on a CU (dV, with the
// smaller ring and at most 168 registers: three).
//   dV^T += dO'^T P^ (P^ = E4M3(P P_r)): Q rows, dO' (E4M3) channel rows, Q
//     scale and L per query.
//   dK^T += Q'^T dS^ (dS^ = E4M3(dS 2^-e) per 64-query group): Q rows, dO
//     rows, Q' (E4M3) channel rows, Q scale, L - log2 s_dO and D / s_dO per
//     query (the dO scale s_dO rides on P: see bwd_dsum_kernel).
template <int D, int PART>
__global__ __launch_bounds__(256, PART == 1 ? 3 : 2) void bwd_dkv_kernel(BwdArgs a) {
  constexpr bool DK = PART == 2;
  constexpr int KS = D / 32, CT = D / 32;
  constexpr int QH = 64;                                   // queries per half tile
  constexpr int ROWS = QH * D;                             // bytes of one row-major half tile
  constexpr int NT = DK ? 3 : 2;                           // code tiles per slot
  constexpr int AUX = NT * ROWS;                           // 4 x 64 floats of per-query scalars
  constexpr int BIASB = AUX + 4 * 256;                     // the key block's bias row for the half tile's Q block
  constexpr int SLOT = BIASB + 2 * 256;
  constexpr int NC = NT * (D / 64) + 2;                    // copies per wave and half tile
  __shared__ __attribute__((aligned(1024))) uint8_t lds[3 * SLOT];
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)lds));

  const int t = threadIdx.x, l = t & 63, col = l & 31, hh = l >> 5;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int item = xcd_item(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
  const int bh = item / a.nblk;
  const int kb = item % a.nblk;   // causal: low blocks have the most queries, first
  const int k0 = kb * kT, kj = k0 + 32 * w + col;
  const int64_t krow = static_cast<int64_t>(bh) * a.n_pad + kj;
  const bool k_ok = kj < a.N;

  // The key's K (and V) codes, B operands of S (and dP), held for the kernel.
  i32x4 kcode[KS], vcode[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    kcode[kk] = *reinterpret_cast<const i32x4*>(a.k_codes + krow * D + 32 * kk + 16 * hh);
    if constexpr (DK) vcode[kk] = *reinterpret_cast<const i32x4*>(a.v_codes + krow * D + 32 * kk + 16 * hh);
  }
  // THREAD granularity: key j is in group 2 (j / 32) + ((j % 8) / 4); the
  // exp2-domain factor sm_scale log2 e rides on the key's scale
  const int kg = 2 * (kj >> 5) + ((kj & 7) >> 2);
  const float dk_j = a.k_scale[static_cast<int64_t>(bh) * (a.n_pad / 16) + kg] * a.scale_log2;
  const float sv_j = DK ? a.v_scale[static_cast<int64_t>(bh) * (a.n_pad / 16) + kg] : 0.f;

  f32x16 acc[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;

  const uint32_t head_rows = static_cast<uint32_t>(a.n_pad * D);
  const i32x4 rq = buffer_rsrc(a.q_codes + static_cast<int64_t>(bh) * a.n_pad * D, head_rows);
  const i32x4 rdo = buffer_rsrc(a.do_codes + static_cast<int64_t>(bh) * a.n_pad * D, head_rows);
  const i32x4 r8 = buffer_rsrc((DK ? a.q8_codes : a.do8_codes) + static_cast<int64_t>(bh) * D * a.n_pad, head_rows);
  const uint32_t head_f = static_cast<uint32_t>(a.n_pad * 4);
  const int64_t rbase = static_cast<int64_t>(bh) * a.n_pad;
  const i32x4 rqs = buffer_rsrc(a.q_scale + rbase, head_f);
  const i32x4 rl = buffer_rsrc((DK ? a.lse_do : a.lse) + rbase, head_f);
  const i32x4 rd = buffer_rsrc(a.dsum_do + rbase, head_f);
  const uint32_t off_rows = rows_off<D>(t), off_cm = cm64_off(t, a.n_pad);

  const int h0 = a.causal ? 2 * kb : 0, nh = 2 * a.nblk;
  // Slot layout: Q rows, [dO rows,] the E4M3 channel rows (dO' for dV, Q' for
  // dK), then 64 floats each of Q scale, L (dK: L - log2 s_dO), a spare copy
  // of the Q scale and D / s_dO (dV: the Q scale again), so that every wave
  // issues NC copies.
  auto copies = [&](int h, int slot) __attribute__((always_inline)) {
    const int q0 = min(h, nh - 1) * QH;        // past the end: the last half tile again (never read)
    const uint32_t base = lds0 + slot * SLOT;
    copy_rows64<D>(base, rq, off_rows, q0, w);
    if constexpr (DK) copy_rows64<D>(base + ROWS, rdo, off_rows, q0, w);
    copy_cm64<D>(base + (NT - 1) * ROWS, r8, off_cm, q0, a.n_pad, w);
    const uint32_t lane4 = 4u * static_cast<uint32_t>(l), so = static_cast<uint32_t>(4 * q0);
    const uint32_t dst = base + AUX + 256 * w;
    if (w == 0 || w == 2 || (!DK && w == 3)) dma4(rqs, lane4, so, dst);
    else if (w == 1) dma4(rl, lane4, so, dst);
    else dma4(rd, lane4, so, dst);
    // the bias of this block's 128 keys against the half tile's query block
    // (512 bytes): waves 0 and 1 copy a half each, waves 2 and 3 the same
    // halves again (identical bytes), so that every wave issues NC copies
    // (a resource over that one bias row: a head's rows can pass 2^32 bytes)
    const i32x4 rb = buffer_rsrc(a.bias + (static_cast<int64_t>(bh) * a.nblk + (q0 >> 7)) * a.n_pad,
                                 static_cast<uint32_t>(a.n_pad) * 4u);
    const uint32_t bh_off = 256u * static_cast<uint32_t>(w & 1);
    dma4(rb, lane4 + bh_off, static_cast<uint32_t>(4 * k0), base + BIASB + bh_off);
  };
  copies(h0, 0);
  copies(h0 + 1, 1);

#pragma unroll 1
  for (int h = h0; h < nh; ++h) {
    // This wave's copies of half tile h are complete (only the NC of h + 1
    // may still run); after the barrier every wave's are, and every wave is
    // done with the slot of h - 1, which the copies of h + 2 refill.
    static_assert(NC == 8 || NC == 6 || NC == 5 || NC == 4, "one wait per copy count");
    if constexpr (NC == 8) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if constexpr (NC == 6) asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if constexpr (NC == 5) asm volatile("s_waitcnt vmcnt(5) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    copies(h + 2, (h + 2 - h0) % 3);
    const uint8_t* slot = lds + ((h - h0) % 3) * SLOT;
    const uint8_t* tq = slot;
    const uint8_t* tdo = slot + ROWS;
    const uint8_t* t8 = slot + (NT - 1) * ROWS;
    const float* tqs = reinterpret_cast<const float*>(slot + AUX);
    const float* tl = tqs + 64;
    const float* td = tqs + 192;
    const int q0 = h * QH;
    // from the slot: a global load here would be waited for together with
    // the copies issued just before it (the compiler cannot count those)
    // (dV: P^ = E4M3(P P_r) with P P_r = 2^(s - L + log2 P_r), so log2 P_r
    // rides on the key's bias and no product per entry is needed)
    const float bj = reinterpret_cast<const float*>(slot + BIASB)[32 * w + col] + (DK ? 0.f : a.p_range_log2);
    // every entry of the half tile visible (uniform): no per-entry mask
    const bool full = q0 + QH <= a.N && k0 + kT <= a.N && (!a.causal || k0 + kT - 1 <= q0);

    float ds[2][16];
    i32x8 pb;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      i32x16 S = {};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        S = __builtin_amdgcn_mfma_i32_32x32x32_i8(frag_rows<D>(tq, sub, kk, col, hh), kcode[kk], S, 0, 0, 0);
      // query q0 + it is visible iff lo <= it <= hi, it = 32 sub + 8 (r / 4) + 4 hh + r % 4;
      // masked entries take s = -inf, so P = 0 (and dS = 0)
      const int base_it = 32 * sub + 4 * hh;
      const int lo = (a.causal ? kj - q0 : 0) - base_it, hi = (k_ok ? a.N - 1 - q0 : -1) - base_it;
      float x[16], p[16];
      if constexpr (DK) {
        float4 qs4[4], l4[4];
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          qs4[a4] = *reinterpret_cast<const float4*>(tqs + base_it + 8 * a4);
          l4[a4] = *reinterpret_cast<const float4*>(tl + base_it + 8 * a4);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float qs = reinterpret_cast<const float*>(&qs4[r >> 2])[r & 3];
          const float lr = reinterpret_cast<const float*>(&l4[r >> 2])[r & 3];
          x[r] = static_cast<float>(S[r]) * (qs * dk_j) + bj - lr;
        }
      } else {
        // each quad of per-query scalars loaded where it is used: fewer live
        // registers, so that three dV work-groups fit on a CU
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const float4 qs4 = *reinterpret_cast<const float4*>(tqs + base_it + 8 * a4);
          const float4 l4 = *reinterpret_cast<const float4*>(tl + base_it + 8 * a4);
#pragma unroll
          for (int u = 0; u < 4; ++u)
            x[4 * a4 + u] = static_cast<float>(S[4 * a4 + u]) * (reinterpret_cast<const float*>(&qs4)[u] * dk_j) + bj -
                            reinterpret_cast<const float*>(&l4)[u];
        }
      }
      if (!full)   // uniform
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int o = 8 * (r >> 2) + (r & 3);
          x[r] = ((o >= lo) & (o <= hi)) ? x[r] : -INFINITY;
        }
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(x[r]);
      if constexpr (!DK) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          int v = __builtin_amdgcn_cvt_pk_fp8_f32(p[4 * q4 + 0], p[4 * q4 + 1], 0, false);
          v = __builtin_amdgcn_cvt_pk_fp8_f32(p[4 * q4 + 2], p[4 * q4 + 3], v, true);
          pb[4 * sub + q4] = v;
        }
      } else {
        i32x16 dP = {};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
          dP = __builtin_amdgcn_mfma_i32_32x32x32_i8(frag_rows<D>(tdo, sub, kk, col, hh), vcode[kk], dP, 0, 0, 0);
        // p = P s_dO (the row's L - log2 s_dO in tl), so p (dP s_V - D / s_dO)
        // = P (dP s_dO s_V - D) with no product of two scales per entry
        float4 d4[4];
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) d4[a4] = *reinterpret_cast<const float4*>(td + base_it + 8 * a4);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float dr = reinterpret_cast<const float*>(&d4[r >> 2])[r & 3];
          ds[sub][r] = p[r] * (static_cast<float>(dP[r]) * sv_j - dr);   // 0 wherever p is
        }
      }
    }
    if constexpr (!DK) {
#pragma unroll
      for (int c = 0; c < CT; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(frag_cm64(t8, c, col, hh), pb, acc[c], 0, 0, 0, 0, 0, 0);
    } else {
      const int e = e8m0_exponent(amax32(ds));
      const i32x8 db = pack_e4m3(ds, e);
#pragma unroll
      for (int c = 0; c < CT; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(frag_cm64(t8, c, col, hh), db, acc[c], 0, 0, 0, 127, 0,
                                                                 e + 127);
    }
  }
  // the copies past the end write LDS: they complete before the work-group ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if (kj < a.N) {
    const float* s8 = (DK ? a.q8_scale : a.do8_scale) + static_cast<int64_t>(bh) * D;
    const float f = DK ? a.sm_scale : 1.f / a.p_range;
    float* out = (DK ? a.dk : a.dv) + (static_cast<int64_t>(bh) * a.N + kj) * D;
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int c0 = 32 * c + 8 * a4 + 4 * hh;
        float4 o;
        o.x = acc[c][4 * a4 + 0] * (f * s8[c0 + 0]);
        o.y = acc[c][4 * a4 + 1] * (f * s8[c0 + 1]);
        o.z = acc[c][4 * a4 + 2] * (f * s8[c0 + 2]);
        o.w = acc[c][4 * a4 + 3] * (f * s8[c0 + 3]);
        *reinterpret_cast<float4*>(out + c0) = o;
      }
  }
}

// D_i = sum_c dO_ic O_ic (fp32) of every padded row; 0 for rows >= N; and
// from it, L_i and the row's INT8 dO scale, the dK kernel's per-row terms.  A
// row is TPR = D/8 lanes of 8 channels (one 16-byte load of O and of dO
// each), a work-group 256/TPR rows.  Both tensors are read through raw buffer
// resources over the work-group's rows below N, so rows past N read as zeros
// and every load issues unconditionally.  The row sum: the lane's 8 products,
// then DPP exchanges inside the row's lanes.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void bwd_dsum_kernel(const uint16_t* o, const uint16_t* dout, int64_t sB, int64_t sH,
                                                       int64_t sN, int H, int N, int n_pad, const float* do_scale,
                                                       const float* lse, float* dsum, float* lse_do, float* dsum_do) {
  constexpr int TPR = D / 8, RPW = 256 / TPR;
  const int t = threadIdx.x, cg = t % TPR, rl = t / TPR;
  const int row0 = static_cast<int>(blockIdx.x) * RPW;
  const int bh = static_cast<int>(blockIdx.y);
  const int b = bh / H, h = bh % H;
  const int64_t base = b * sB + h * sH + static_cast<int64_t>(row0) * sN;
  const int64_t bytes = static_cast<int64_t>(max(0, min(RPW, N - row0))) * sN * 2;
  const auto ro = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(o + base), 0, static_cast<int>(bytes), kBufferWord3);
  const auto rd = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(dout + base), 0, static_cast<int>(bytes), kBufferWord3);
  const int off = rl * static_cast<int>(sN) * 2 + 16 * cg;
  const auto xo = __builtin_amdgcn_raw_buffer_load_b128(ro, off, 0, 0);
  const auto xd = __builtin_amdgcn_raw_buffer_load_b128(rd, off, 0, 0);
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint16_t ho = static_cast<uint16_t>(xo[e / 2] >> (16 * (e & 1)));
    const uint16_t hd = static_cast<uint16_t>(xd[e / 2] >> (16 * (e & 1)));
    float x, y;
    if constexpr (BF16) {
      x = __uint_as_float(static_cast<uint32_t>(ho) << 16);
      y = __uint_as_float(static_cast<uint32_t>(hd) << 16);
    } else {
      x = static_cast<float>(__builtin_bit_cast(_Float16, ho));
      y = static_cast<float>(__builtin_bit_cast(_Float16, hd));
    }
    acc = __builtin_fmaf(x, y, acc);
  }
  // sum over the row's TPR lanes: quad exchanges, then the mirrors inside 8 and 16 lanes
  auto dpp_add = [](float v, int ctrl_sel) __attribute__((always_inline)) {
    int u = __float_as_int(v), w;
    if (ctrl_sel == 0) w = __builtin_amdgcn_update_dpp(0, u, 0xB1, 0xf, 0xf, false);        // quad_perm [1,0,3,2]
    else if (ctrl_sel == 1) w = __builtin_amdgcn_update_dpp(0, u, 0x4E, 0xf, 0xf, false);   // quad_perm [2,3,0,1]
    else if (ctrl_sel == 2) w = __builtin_amdgcn_update_dpp(0, u, 0x141, 0xf, 0xf, false);  // row_half_mirror
    else w = __builtin_amdgcn_update_dpp(0, u, 0x140, 0xf, 0xf, false);                     // row_mirror
    return v + __int_as_float(w);
  };
  acc = dpp_add(acc, 0);
  acc = dpp_add(acc, 1);
  acc = dpp_add(acc, 2);
  if constexpr (TPR == 16) acc = dpp_add(acc, 3);
  if (cg == 0) {
    const int64_t i = static_cast<int64_t>(bh) * n_pad + row0 + rl;
    dsum[i] = acc;
    // the dK kernel's per-row terms, with the row's INT8 dO scale s:
    // 2^(s_ij - (L - log2 s)) (dP s_V - D / s) = P (dP s s_V - D)
    const float sc = do_scale[i];
    lse_do[i] = sc > 0.f ? lse[i] - log2f(sc) : INFINITY;
    dsum_do[i] = sc > 0.f ? acc / sc : 0.f;
  }
}

template <int D>
hipError_t bwd_impl(const Problem& p, const BwdBuffers& bb, int causal, hipStream_t st) {
  BwdArgs a;
  a.q_codes = bb.qk.q_codes; a.q_scale = bb.qk.q_scale; a.k_codes = bb.qk.k_codes; a.k_scale = bb.qk.k_scale;
  a.bias = bb.qk.bias; a.lse = bb.lse;
  a.do_codes = bb.dov.q_codes; a.do_scale = bb.dov.q_scale; a.v_codes = bb.dov.k_codes; a.v_scale = bb.dov.k_scale;
  a.do8_codes = bb.do8.v_codes; a.do8_scale = bb.do8.v_scale;
  a.q8_codes = bb.q8.v_codes; a.q8_scale = bb.q8.v_scale;
  a.k8_codes = bb.k8.v_codes; a.k8_scale = bb.k8.v_scale;
  a.dsum = bb.dsum;
  a.lse_do = bb.lse_do; a.dsum_do = bb.dsum_do;
  a.dq = bb.dq; a.dk = bb.dk; a.dv = bb.dv;
  a.H = p.H; a.N = p.N; a.n_pad = p.n_pad; a.nblk = p.nblk; a.causal = causal ? 1 : 0;
  a.scale_log2 = p.sm_scale * 1.4426950408889634f;
  a.sm_scale = p.sm_scale;
  a.p_range = p.p_range;
  a.p_range_log2 = static_cast<float>(std::log2(static_cast<double>(p.p_range)));
  const dim3 grid(p.nblk * p.B * p.H);
  hipLaunchKernelGGL((bwd_dq_kernel<D>), grid, dim3(256), 0, st, a);
  hipLaunchKernelGGL((bwd_dkv_kernel<D, 1>), grid, dim3(256), 0, st, a);
  hipLaunchKernelGGL((bwd_dkv_kernel<D, 2>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dsum(const Problem& p, TensorView o, TensorView dout, const BwdBuffers& bb, hipStream_t st) {
  const dim3 grid(p.n_pad / (256 / (p.D / 8)), p.B * p.H);
  const uint16_t* op = static_cast<const uint16_t*>(o.ptr);
  const uint16_t* dp = static_cast<const uint16_t*>(dout.ptr);
  auto kernel = p.D == 128 ? (p.bf16 ? bwd_dsum_kernel<128, true> : bwd_dsum_kernel<128, false>)
                           : (p.bf16 ? bwd_dsum_kernel<64, true> : bwd_dsum_kernel<64, false>);
  hipLaunchKernelGGL(kernel, grid, dim3(256), 0, st, op, dp, o.sB, o.sH, o.sN, p.H, p.N, p.n_pad, bb.dov.q_scale,
                     bb.lse, bb.dsum, bb.lse_do, bb.dsum_do);
  return hipGetLastError();
}

hipError_t launch_attn_bwd(const Problem& p, const BwdBuffers& bb, int causal, hipStream_t st) {
  return p.D == 128 ? bwd_impl<128>(p, bb, causal, st) : bwd_impl<64>(p, bb, causal, st);
}

}  // namespace sage
