// Quantized attention forward kernel for gfx950 (CDNA4).
//
// Method: the FlashAttention-based quantized attention of the SageAttention2++
// summary ("2. Preliminary", "2.1 SageAttention2"): INT8 (or INT4-range)
// Q, K codes with per-group scales, dequantised S plus the Q-smoothing bias,
// online softmax, P~ to FP8 with a fixed scale, FP8 V with per-channel
// scales, rescale and normalise at the end.
//
// Mapping to the hardware:
//  * one work-group of 4 waves per 128-query block; wave w owns 32 queries;
//    keys advance in tiles of 128.
//  * S^T = K^ Q^T on v_mfma_i32_32x32x32_i8: the A operand is 32 keys x 32
//    channels of K^ (from LDS), the B operand 32 channels x 32 queries of Q^
//    (registers for the whole kernel).  In the 32x32 accumulator lane l holds
//    query l%32 and the 16 keys 8a + 4(l/32) + b, so row max and row sum are
//    in-lane work plus one exchange with lane l^32.
//  * the 16 fp8-packed P~ values of two consecutive 32-key S subtiles are
//    exactly one lane's 32-byte B operand of v_mfma_f32_32x32x64_f8f6f4
//    (O^T += V^T P~^T, keys as the reduction index).  The V codes are stored
//    channel-major with the matching in-group key order, so P~ never leaves
//    registers.
//  * a single wave issues vector instructions only every few cycles, so its
//    matrix-core work is interleaved with its own vector work: tile t's
//    dequantisation and row maximum run beside the PV product of tile t-1,
//    and tile t's exp2 / FP8 packing beside the QK product of tile t+1.
//  * online softmax against the running row maximum m (log2 units): P~ =
//    2^(s - m) <= 1 is encoded as E4M3(P~ * P_r); O and l are rescaled when
//    some row of the wave has a new maximum (the rescale is skipped, exactly,
//    when none has).
//  * K codes, V codes and each tile's bias row and K scales are copied straight
//    from global memory into two-slot LDS rings, one tile ahead of their use.
#include "sage_internal.h"

namespace sage {
namespace {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 128;        // keys per tile (one online-softmax update)

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
  int lpt_g;         // causal: heads per longest-first group (map_block)
  float* lse;        // optional: log2 sum_j 2^(s_ij) of every query row [B, H, n_pad] (nullptr: not written)
  int probe_qb;      // PROBE kernels: the one query block of every head (work-group id = head);
                     // their output row of query i is i - 128 probe_qb ([B, H, 128, d] spans)
};

// 16-byte chunk swizzle inside a tile row so that the 16 lanes served together
// by one ds_read_b128 pass touch distinct banks (self-inverse in `chunk`).
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
__device__ __forceinline__ void map_block(int id, int total, int nblk, int causal, int lpt_g, int& bh, int& qb) {
  constexpr int kXcd = 8;
  int w = id;
  if (total % kXcd == 0) w = (id % kXcd) * (total / kXcd) + id / kXcd;
  bh = w / nblk;
  qb = w % nblk;
  if (causal) {
    qb = nblk - 1 - qb;
    // Groups of lpt_g heads that stay within one XCD run block-major, so the
    // longest blocks of the group go first (the K/V codes of lpt_g heads fit
    // that XCD's L2; the host picks lpt_g).
    const int span = lpt_g * nblk, g0 = (w / span) * span;
    if (lpt_g > 1 && total % kXcd == 0 && (total / kXcd) % span == 0) {
      const int loc = w - g0;
      bh = g0 / nblk + loc % lpt_g;
      qb = nblk - 1 - loc / lpt_g;
    }
  }
}

typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ lds_void* lds_ptr(void* p) { return (lds_void*)(p); }

// LDS rings of two slots; tile u lives in slot u % 2.  K slot: 128 keys x D
// codes (rows swizzled).  V slot: D channels x 128 keys (rows swizzled).  Aux
// slot: the tile's 128 bias values, then its K scales (8 or 2 used).
template <int D>
struct Rings {
  static constexpr int K = kTile * D;
  static constexpr int V = D * kTile;
  static constexpr int AUX = 1024;   // bias (512 B), K scales, spare row at 768
  static constexpr int K0 = 0, V0 = 2 * K, A0 = 2 * K + 2 * V;
  static constexpr int BYTES = 2 * (K + V + AUX);
  static constexpr int J = D / 32;   // 1 KiB copies per wave for one K or V slot
};

// Buffer resource (raw, 32-bit data format) over `bytes` bytes at p, in SGPRs.
// Reads past the end return zero.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(a & 0xffffffffu));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>((a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  r[3] = kBufferWord3;
  return r;
}

// Direct global->LDS copies (buffer_load ... lds): lane L's 16 (or 4) bytes
// land at M0 + 16 L (4 L).  Written as inline assembly so that the compiler
// does not track these LDS writes: the slots a tile reads are never the ones
// being filled (the ring schedule and the barriers guarantee it), and the
// copies are waited for by hand (s_waitcnt vmcnt) before the barrier that
// publishes them.  The "memory" clobber keeps LDS reads on their side.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma4(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dword %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "s"(lds) : "memory", "m0");
}

// Sources of the tile copies.  With chunk p = 256 j + threadIdx.x the swizzled
// column does not depend on j, so one per-lane offset per stream serves every
// copy and j moves only the scalar offset (4096 j bytes of K rows, 32 j
// channel rows of V).
struct TileSrc {
  i32x4 k, v, b, s;
  uint32_t k_off, v_off;          // per-lane byte offsets for j = 0 and k0 = 0
  uint32_t v_row;                 // bytes per V channel row (n_pad)
  uint32_t s_per_tile;            // K scale groups per 128-key tile (8 or 2)
};

template <int D>
__device__ __forceinline__ TileSrc make_tile_src(const int8_t* kbase, const uint8_t* vbase, const float* brow,
                                                 const float* kscale, int n_scale, int n_pad, int t) {
  constexpr int CPR = D / 16;
  TileSrc s;
  s.k = buffer_rsrc(kbase, static_cast<uint32_t>(n_pad * D));
  s.v = buffer_rsrc(vbase, static_cast<uint32_t>(n_pad * D));
  s.b = buffer_rsrc(brow, static_cast<uint32_t>(n_pad * 4));
  s.s = buffer_rsrc(kscale, static_cast<uint32_t>(n_scale * 4));
  s.s_per_tile = static_cast<uint32_t>(n_scale / (n_pad / kTile));
  const int r = t / CPR, pc = t % CPR;
  s.k_off = static_cast<uint32_t>(r * D + 16 * swz<D>(r, pc));
  const int ch = t >> 3, vc = t & 7;
  s.v_off = static_cast<uint32_t>(ch * n_pad + 16 * swz<128>(ch, vc));
  s.v_row = static_cast<uint32_t>(n_pad);
  return s;
}

// K codes of the 128 keys from k0 into the K slot at LDS address `slot`.
template <int D>
__device__ __forceinline__ void copy_k(uint32_t slot, const TileSrc& s, int k0, int w) {
#pragma unroll
  for (int j = 0; j < Rings<D>::J; ++j)
    dma16(s.k, s.k_off, static_cast<uint32_t>(k0 * D + 4096 * j), slot + (4 * j + w) * 1024);
}

// V codes of the 128 keys from k0 (all D channels) into a V slot.
template <int D>
__device__ __forceinline__ void copy_v(uint32_t slot, const TileSrc& s, int k0, int w) {
#pragma unroll
  for (int j = 0; j < Rings<D>::J; ++j)
    dma16(s.v, s.v_off, static_cast<uint32_t>(k0) + 32u * j * s.v_row, slot + (4 * j + w) * 1024);
}

// Bias row (waves 0, 1) and K scales (wave 2) of the 128 keys from k0 into an
// aux slot; wave 3 copies the bias again into a spare row so that every wave
// issues exactly one copy.  The K scales are spread so that subtile st, lane
// half h reads entry 2 st + h for every granularity (64-key groups: entry j holds
// group j / 4).  The lane's offsets are recomputed at every call (two
// instructions the compiler may not hoist): held across the loop they are
// spilled, and a reload's wait would also wait for the tile copies in flight.
__device__ __forceinline__ void copy_aux(uint32_t slot, const TileSrc& s, bool thread_gran, int k0, int w) {
  uint32_t lane;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  if (w != 2) {
    const uint32_t b_off = 4u * (64u * static_cast<uint32_t>(w) + lane);
    dma4(s.b, w == 3 ? (b_off & 255u) : b_off, static_cast<uint32_t>(4 * k0), slot + (w == 3 ? 768 : 256 * w));
  } else {
    const uint32_t lane4 = 4u * lane;
    const uint32_t src = lane4 >= 32u ? 0u : (thread_gran ? lane4 : (lane4 >> 4) << 2);
    dma4(s.s, src, static_cast<uint32_t>(4 * (k0 / kTile)) * s.s_per_tile, slot + 512);
  }
}

// 24 bytes of FP6 codes as an 8-register MFMA operand (the top two registers unused).
__device__ __forceinline__ i32x8 cat6(i32x4 a, i32x2 b) {
  const i32x4 bw = __builtin_shufflevector(b, b, 0, 1, -1, -1);
  return __builtin_shufflevector(a, bw, 0, 1, 2, 3, 4, 5, -1, -1);
}

// QKF: how the Q and K codes are held.  0: int8 on v_mfma_i32_32x32x32_i8.
// 1 (E4M3) and 2 (packed FP6 E2M3): small integers in a float format on
// v_mfma_f32_32x32x64_f8f6f4, 64 channels per instruction (FP6 at twice the FP8
// rate).  Every product and partial sum is an integer below 2^24, so the fp32
// result equals the integer product exactly and the int->float conversion
// disappears.
// PROBE: one work-group per head, on query block a.probe_qb only.
// LSE: also write log2 sum_j 2^(s_ij) of every query row to a.lse (a separate
// instantiation, so that the inference kernel's code is untouched).
template <int D, bool BF16, int QKF, bool PROBE, bool LSE = false>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(AttnArgs a) {
  constexpr int KS = D / 32;          // 32-channel fragments of Q^ and K^ per row
  constexpr bool F8QK = QKF != 0;          // a float-format QK product (E4M3 or E2M3)
  constexpr int CBSZ = QKF == 2 ? 2 : 0;    // operand format of that product: FP8 E4M3, or FP6 E2M3
  constexpr int KSF = F8QK ? KS / 2 : KS;  // QK MFMAs per 32-key subtile
  constexpr int CT = D / 32;          // 32-channel tiles of the output
  constexpr int NQK = 4 * KSF;        // QK MFMAs per tile
  constexpr int NPV = 2 * CT;         // PV MFMAs per tile
  constexpr int QK_EVERY = 16 / NQK;  // softmax quads per QK MFMA
  constexpr int PV_EVERY = 16 / NPV;  // dequant quads per PV MFMA
  constexpr int J = Rings<D>::J;
  using R = Rings<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[R::BYTES];
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_ptr(lds)));

  const int t = threadIdx.x, l = t & 63, col = l & 31, hh = l >> 5;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);   // wave index, held in a scalar register
  int bh, qb;
  if constexpr (PROBE) {
    bh = static_cast<int>(blockIdx.x);
    qb = a.probe_qb;
  } else {
    map_block(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x), a.nblk, a.causal, a.lpt_g, bh, qb);
  }
  const int q0 = qb * 128;
  const int qi = q0 + 32 * w + col;

  const int key_end = a.causal ? min(a.N, q0 + 128) : a.N;
  const int ntiles = (key_end + kTile - 1) / kTile;
  const int8_t* kbase = a.k_codes + static_cast<int64_t>(bh) * a.n_pad * D;
  const uint8_t* vbase = a.v_codes + static_cast<int64_t>(bh) * D * a.n_pad;
  const float* brow = a.bias + (static_cast<int64_t>(bh) * a.nblk + qb) * a.n_pad;
  const int n_kscale = a.gran == SAGE_GRAN_THREAD ? a.n_pad / 16 : a.n_pad / 64;
  const float* kscale = a.k_scale + static_cast<int64_t>(bh) * n_kscale;

  i32x4 qf[KS];
  i32x8 qf8[KSF];   // F8QK: fragments 2j, 2j+1 as one operand (E2M3: 16 + 8 bytes of a 24-byte slot)
  {
    const int8_t* qrow = a.q_codes + (static_cast<int64_t>(bh) * a.n_pad + qi) * D;
    if constexpr (F8QK) {
#pragma unroll
      for (int j = 0; j < KSF; ++j) {
        const i32x4 a0 = *reinterpret_cast<const i32x4*>(qrow + 64 * j + 16 * hh);
        if constexpr (QKF == 2) {
          const i32x2 a1 = *reinterpret_cast<const i32x2*>(qrow + 64 * j + 32 + 16 * hh);
          qf8[j] = cat6(a0, a1);
        } else {
          const i32x4 a1 = *reinterpret_cast<const i32x4*>(qrow + 64 * j + 32 + 16 * hh);
          qf8[j][0] = a0[0]; qf8[j][1] = a0[1]; qf8[j][2] = a0[2]; qf8[j][3] = a0[3];
          qf8[j][4] = a1[0]; qf8[j][5] = a1[1]; qf8[j][6] = a1[2]; qf8[j][7] = a1[3];
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) qf[s] = *reinterpret_cast<const i32x4*>(qrow + 32 * s + 16 * hh);
    }
  }
  auto qf2 = [&](int j) __attribute__((always_inline)) { return qf8[j]; };
  float dq;
  if (a.gran == SAGE_GRAN_THREAD) {
    dq = a.q_scale[static_cast<int64_t>(bh) * a.n_pad + qi];
  } else if (a.gran == SAGE_GRAN_WARP) {
    dq = a.q_scale[static_cast<int64_t>(bh) * (a.n_pad / 32) + (qi >> 5)];
  } else {
    dq = a.q_scale[static_cast<int64_t>(bh) * a.nblk + qb];
  }
  const float dq2 = dq * a.scale_log2;
  // exp2(x - (m + base_shift)) = P~ * P_r with P~ = exp2(x - m)
  const float base_shift = -a.log2_pr;
  const bool thread_gran = a.gran == SAGE_GRAN_THREAD;

  // First key of tile u; tiles past the end copy the last tile again (their
  // data is never used, and every wave keeps one copy count per issue point).
  auto kofs = [&](int u) __attribute__((always_inline)) { return min(u, ntiles - 1) * kTile; };

  const TileSrc src = make_tile_src<D>(kbase, vbase, brow, kscale, n_kscale, a.n_pad, t);
  // Tile t reads K of tile t+1 (and t's own K only in the prologue), V of tile
  // t-1 and the aux row of tile t.  It copies K of tile t+2 and the aux row of
  // tile t+1 when it starts, and V of tile t+1 once every wave has read V of
  // tile t-1 (mid-tile).  Tile 0's PV product reads the V slot of tile -1,
  // zero-filled here (its P~ is 0 too).
  copy_k<D>(lds0 + R::K0, src, kofs(0), w);
  copy_aux(lds0 + R::A0, src, thread_gran, kofs(0), w);
  {
    uint4* vz = reinterpret_cast<uint4*>(lds + R::V0 + R::V);
#pragma unroll
    for (int i = t; i < R::V / 16; i += 256) vz[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  // K(0) and aux(0) are needed now.  They are waited for by count 0, which
  // assumes nothing about the completion order of copies of different sizes;
  // the copies of K(1) and V(0) are issued after the barrier and run beside the first
  // QK product (they are what the first tile-start wait allows for).
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  copy_k<D>(lds0 + R::K0 + R::K, src, kofs(1), w);
  copy_v<D>(lds0 + R::V0, src, kofs(0), w);

  // Per-lane byte offsets of the LDS fragments, relative to a slot.  The
  // swizzle term does not depend on the subtile (K) or the channel tile (V),
  // so those move only the immediate offset of the read.
  //   K fragment, subtile st, channels 32kk..: kofl[kk] + 32 st D
  //   V fragment, keys 64kc.. (lane's 32), channels 32c..: vofl[kc][h2] + 32 c kTile, h2 = 0, 1
  //   bias quad (subtile st, a): 16 hh + 4 (32 st + 8 a)
  uint32_t kofl[KS], vofl[2][2];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) kofl[kk] = static_cast<uint32_t>(col * D + 16 * swz<D>(col, 2 * kk + hh));
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
      vofl[kc][h2] = static_cast<uint32_t>(col * kTile + 16 * swz<128>(col, 4 * kc + 2 * hh + h2));

  auto lds_i4 = [&](uint32_t off) __attribute__((always_inline)) {
    return *reinterpret_cast<const i32x4*>(lds + off);
  };
  auto k_frag = [&](const uint32_t* ko, int slot_off, int st, int kk) __attribute__((always_inline)) {
    return lds_i4(ko[kk] + slot_off + 32 * st * D);
  };
  // F8QK: channels 64j.. of a key as one 32-byte operand (fragments 2j, 2j+1)
  // (E2M3: the 24-byte slot, 16 bytes of fragment 2j and the first 8 of 2j+1)
  auto k_frag2 = [&](const uint32_t* ko, int slot_off, int st, int j) __attribute__((always_inline)) {
    const i32x4 a0 = lds_i4(ko[2 * j] + slot_off + 32 * st * D);
    if constexpr (QKF == 2) {
      return cat6(a0, *reinterpret_cast<const i32x2*>(lds + ko[2 * j + 1] + slot_off + 32 * st * D));
    } else {
      const i32x4 a1 = lds_i4(ko[2 * j + 1] + slot_off + 32 * st * D);
      i32x8 r;
      r[0] = a0[0]; r[1] = a0[1]; r[2] = a0[2]; r[3] = a0[3];
      r[4] = a1[0]; r[5] = a1[1]; r[6] = a1[2]; r[7] = a1[3];
      return r;
    }
  };
  auto v_frag = [&](const uint32_t (*vo)[2], int slot_off, int kc, int c) __attribute__((always_inline)) {
    const i32x4 v0 = lds_i4(vo[kc][0] + slot_off + 32 * c * kTile);
    const i32x4 v1 = lds_i4(vo[kc][1] + slot_off + 32 * c * kTile);
    i32x8 va;
    va[0] = v0[0]; va[1] = v0[1]; va[2] = v0[2]; va[3] = v0[3];
    va[4] = v1[0]; va[5] = v1[1]; va[6] = v1[2]; va[7] = v1[3];
    return va;
  };

  f32x16 oacc[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[c][i] = 0.f;
  float m = -INFINITY, lsum = 0.f;
  using SAcc = typename std::conditional<F8QK, f32x16, i32x16>::type;
  SAcc sA[4], sB[4];       // S^T of the tile whose softmax runs next (alternating sets)
  i32x8 pA[2], pB[2];      // FP8 P~ of the previous tile (alternating sets)
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int i = 0; i < 8; ++i) pA[kc][i] = 0;

  // QK product of tile 0 (not overlapped).
#pragma unroll
  for (int st = 0; st < 4; ++st) {
#pragma unroll
    for (int i = 0; i < 16; ++i) sA[st][i] = 0;
    if constexpr (F8QK) {
#pragma unroll
      for (int j = 0; j < KSF; ++j)
        sA[st] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k_frag2(kofl, R::K0, st, j), qf2(j), sA[st], CBSZ,
                                                                 CBSZ, 0, 0, 0, 0);
    } else {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        sA[st] = __builtin_amdgcn_mfma_i32_32x32x32_i8(k_frag(kofl, R::K0, st, kk), qf[kk], sA[st], 0, 0, 0);
    }
  }

  // One tile.  CUR: its ring slot (t % 2); S_cur / S_nxt: S^T of tiles t and
  // t+1; pb_prv / pb_cur: FP8 P~ of tiles t-1 and t.
  auto tile = [&](const int tt, auto cur_slot, SAcc* S_cur, SAcc* S_nxt, i32x8* pb_prv, i32x8* pb_cur)
                  __attribute__((always_inline)) {
    constexpr int CUR = decltype(cur_slot)::value, NXT = 1 - CUR;
    const int k0 = tt * kTile;
    // This wave's copy of aux(t) (issued when tile t-1 started) is complete:
    // only the 2J copies of K(t+1) and V(t), issued after it in phase B of tile
    // t-1, may still run (vector memory loads return in issue order, so the
    // count bounds the oldest).  K(t+1) is waited for at the mid-tile wait,
    // V(t) at the next tile's.  After the barrier every wave is done with
    // aux(t-1), whose slot is refilled below.
    if constexpr (J == 4) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    copy_aux(lds0 + R::A0 + NXT * R::AUX, src, thread_gran, kofs(tt + 1), w);

    // Fresh copies of the lane offsets: without this the compiler hoists one
    // address register per (slot, fragment) out of the loop and spills them.
    // (The F8QK form, free of the int->float conversions, fits without them;
    // with them its own offsets spill instead.)
    uint32_t ko[KS], vo[2][2], bo = 16u * hh;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) { ko[kk] = kofl[kk]; if constexpr (!F8QK) asm volatile("" : "+v"(ko[kk])); }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      vo[kc][0] = vofl[kc][0]; vo[kc][1] = vofl[kc][1];
      if constexpr (!F8QK) asm volatile("" : "+v"(vo[kc][0]), "+v"(vo[kc][1]));
    }
    if constexpr (!F8QK) asm volatile("" : "+v"(bo));
    const int aux = R::A0 + CUR * R::AUX;
    float cs[4];
    {
      const float* ksc = reinterpret_cast<const float*>(lds + aux + 512);
#pragma unroll
      for (int st = 0; st < 4; ++st)
        cs[st] = dq2 * ksc[2 * st + hh];
    }

    // Phase A: dequantise S(t) and take the row maximum, beside the PV product
    // of tile t-1 (V(t-1) is in slot NXT).  LDS operands are fetched ahead of
    // use (bias one quad, V fragments one PV interval) so that a quad's vector
    // work covers their latency.
    const int vslot_off = R::V0 + NXT * R::V;
    float x[4][16];
    float mx = -INFINITY, mx2 = -INFINITY;
    i32x8 vf[2];
    vf[0] = v_frag(vo, vslot_off, 0, 0);
    float4 bnext = *reinterpret_cast<const float4*>(lds + aux + bo);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int st = i >> 2, a4 = i & 3;
      const float4 bv = bnext;
      if (i + 1 < 16) {
        const int st1 = (i + 1) >> 2, a1 = (i + 1) & 3;
        bnext = *reinterpret_cast<const float4*>(lds + aux + bo + 4 * (32 * st1 + 8 * a1));
      }
      const int e = i / PV_EVERY;
      if (i % PV_EVERY == 0 && e + 1 < NPV) vf[(e + 1) & 1] = v_frag(vo, vslot_off, (e + 1) / CT, (e + 1) % CT);
      float* xs = &x[st][4 * a4];
      xs[0] = static_cast<float>(S_cur[st][4 * a4 + 0]) * cs[st] + bv.x;
      xs[1] = static_cast<float>(S_cur[st][4 * a4 + 1]) * cs[st] + bv.y;
      xs[2] = static_cast<float>(S_cur[st][4 * a4 + 2]) * cs[st] + bv.z;
      xs[3] = static_cast<float>(S_cur[st][4 * a4 + 3]) * cs[st] + bv.w;
      mx = fmaxf(fmaxf(mx, xs[0]), xs[1]);
      mx2 = fmaxf(fmaxf(mx2, xs[2]), xs[3]);
      // The empty asm statements pin each quad's vector work in place: compiler
      // passes must not move it across quads or across the rescale branch, or
      // the interleave with the matrix work is lost.  (Two running maxima keep
      // the max chains short: two v_max3 per quad.)
      asm volatile("" : "+v"(mx), "+v"(mx2));
      if (i % PV_EVERY == PV_EVERY - 1) {
        const int kc = e / CT, c = e % CT;
        oacc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[e & 1], pb_prv[kc], oacc[c], 0, 0, 0, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // Every wave has read V(t-1) (its slot is refilled in phase B) and this
    // wave's copies of K(t+1) are complete (only the aux copy issued at the
    // start of this tile may still run); after the barrier every wave's are.
    asm volatile("s_waitcnt vmcnt(1) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // K fragments of the first two QK MFMAs of phase B, read only now: K(t+1)
    // is copied by all four waves, and only the barrier above makes every
    // wave's part of it visible.
    const int kslot_off = R::K0 + NXT * R::K;
    i32x4 kf[3];
    i32x8 kf2[2];
    if constexpr (F8QK) {
      kf2[0] = k_frag2(ko, kslot_off, 0, 0);
    } else {
      kf[0] = k_frag(ko, kslot_off, 0, 0);
      if (NQK > 1) kf[1] = k_frag(ko, kslot_off, (1 / KS), 1 % KS);
    }

    mx = fmaxf(mx, mx2);
    const bool need_mask = (k0 + kTile > a.N) || (a.causal && k0 + kTile - 1 > q0 + 32 * w);
    if (need_mask) {
      // key j is visible to this query iff j <= lim
      const int lim = a.causal ? min(a.N - 1, qi) : a.N - 1;
      mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = k0 + 32 * st + 8 * (r >> 2) + 4 * hh + (r & 3);
          x[st][r] = j <= lim ? x[st][r] : -INFINITY;
          mx = fmaxf(mx, x[st][r]);
        }
    }
    const float mt = fmaxf(mx, __shfl_xor(mx, 32));
    // Running maximum: P~ of this tile is formed against max(m, tile maximum).
    const float mnew = mt > m ? mt : m;
    const float alpha = (m == mnew) ? 1.f : ((m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mnew));
    const float base = (mnew == -INFINITY) ? 0.f : mnew + base_shift;
    // Exact skip: alpha == 1 for every row of this wave unless a running maximum moved.
    if (!__all(alpha == 1.f)) {
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[c][i] *= alpha;
    }
    m = mnew;

    // Phase B: exp2 and FP8 packing of tile t, beside the QK product of tile
    // t+1 (K(t+1) is in slot NXT), subtile by subtile; K fragments are fetched
    // two MFMAs ahead.
    float ps = 0.f;
    const SAcc zero16 = {};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int st = i >> 2, q4 = i & 3;
      const int e = i / QK_EVERY;
      if constexpr (F8QK) {
        // one MFMA (QK_EVERY quads) ahead
        if (i % QK_EVERY == 0 && e + 1 < NQK) kf2[(e + 1) & 1] = k_frag2(ko, kslot_off, (e + 1) / KSF, (e + 1) % KSF);
      } else {
        if (i % QK_EVERY == 0 && e + 2 < NQK) kf[(e + 2) % 3] = k_frag(ko, kslot_off, (e + 2) / KS, (e + 2) % KS);
      }
      // Copies for later tiles, one every 16/(2J) quads: K(t+2) into slot CUR
      // (K(t) was last read in tile t-1) and V(t+1) into slot NXT (freed at
      // the mid-tile barrier).
      if (i % (8 / J) == 0) {
        const int cj = i / (8 / J);
        if (cj < J) dma16(src.k, src.k_off, static_cast<uint32_t>(kofs(tt + 2) * D + 4096 * cj),
                          lds0 + R::K0 + CUR * R::K + (4 * cj + w) * 1024);
        else dma16(src.v, src.v_off, static_cast<uint32_t>(kofs(tt + 1)) + 32u * (cj - J) * src.v_row,
                   lds0 + R::V0 + NXT * R::V + (4 * (cj - J) + w) * 1024);
      }
      const float p0 = __builtin_amdgcn_exp2f(x[st][4 * q4 + 0] - base);
      const float p1 = __builtin_amdgcn_exp2f(x[st][4 * q4 + 1] - base);
      const float p2 = __builtin_amdgcn_exp2f(x[st][4 * q4 + 2] - base);
      const float p3 = __builtin_amdgcn_exp2f(x[st][4 * q4 + 3] - base);
      ps += (p0 + p1) + (p2 + p3);
      int v = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, __float_as_int(p0), false);
      v = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, v, true);
      asm volatile("" : "+v"(v), "+v"(ps));
      pb_cur[st >> 1][4 * (st & 1) + q4] = v;
      if (i % QK_EVERY == 0) {
        if constexpr (F8QK) {
          const int sn = e / KSF, j = e % KSF;
          S_nxt[sn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf2[e & 1], qf2(j), j == 0 ? zero16 : S_nxt[sn],
                                                                      CBSZ, CBSZ, 0, 0, 0, 0);
        } else {
          const int sn = e / KS, kk = e % KS;
          S_nxt[sn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[e % 3], qf[kk], kk == 0 ? zero16 : S_nxt[sn], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    lsum = alpha * lsum + ps;
  };

  int tt = 0;
  for (; tt + 1 < ntiles; tt += 2) {
    tile(tt, std::integral_constant<int, 0>{}, sA, sB, pA, pB);
    tile(tt + 1, std::integral_constant<int, 1>{}, sB, sA, pB, pA);
  }
  if (tt < ntiles) {
    tile(tt, std::integral_constant<int, 0>{}, sA, sB, pA, pB);
    pA[0] = pB[0];
    pA[1] = pB[1];
  }

  // PV product of the last tile (V(ntiles-1) was copied mid tile ntiles-2).
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  {
    const int lv = R::V0 + ((ntiles - 1) & 1) * R::V;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int c = 0; c < CT; ++c)
        oacc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v_frag(vofl, lv, kc, c), pA[kc], oacc[c], 0, 0, 0,
                                                                  0, 0, 0);
  }

  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float inv = 1.f / ltot;
  // l sums P~ * P_r against the running maximum m: log2 sum_j 2^(s_j) = m + log2(l) - log2(P_r).
  if (LSE && hh == 0)
    a.lse[static_cast<int64_t>(bh) * a.n_pad + qi] = (m + __builtin_amdgcn_logf(ltot)) - a.log2_pr;
  if (qi < a.N) {
    const int b = bh / a.H, h = bh % a.H;
    const int orow_i = PROBE ? qi - q0 : qi;
    uint16_t* orow = static_cast<uint16_t*>(a.o) + b * a.oB + h * a.oH + static_cast<int64_t>(orow_i) * a.oN;
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

template <int D, bool BF16, int QKF>
hipError_t attn_impl(const Problem& p, const sage_qk_buffers& qk, const sage_v_buffers& vb, int causal, void* o,
                     const int64_t o_stride[3], hipStream_t st, int probe_qb, float* lse) {
  AttnArgs a;
  a.lse = lse;
  a.q_codes = qk.q_codes; a.q_scale = qk.q_scale; a.k_codes = qk.k_codes; a.k_scale = qk.k_scale;
  a.bias = qk.bias; a.v_codes = vb.v_codes; a.v_scale = vb.v_scale; a.v_mean = vb.v_mean;
  a.o = o; a.oB = o_stride[0]; a.oH = o_stride[1]; a.oN = o_stride[2];
  a.H = p.H; a.N = p.N; a.n_pad = p.n_pad; a.nblk = p.nblk; a.gran = p.gran; a.causal = causal ? 1 : 0;
  a.scale_log2 = p.sm_scale * 1.4426950408889634f;
  a.log2_pr = log2f(p.p_range);
  a.lpt_g = lpt_group(p.B * p.H, static_cast<int64_t>(2) * p.n_pad * p.D);
  a.probe_qb = probe_qb;
  const int grid = probe_qb >= 0 ? p.B * p.H : p.nblk * p.B * p.H;
  if (probe_qb >= 0) hipLaunchKernelGGL((attn_fwd_kernel<D, BF16, QKF, true>), dim3(grid), dim3(256), 0, st, a);
  else if (lse) hipLaunchKernelGGL((attn_fwd_kernel<D, BF16, QKF, false, true>), dim3(grid), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((attn_fwd_kernel<D, BF16, QKF, false>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const Problem& p, const sage_qk_buffers& qk, const sage_v_buffers& vb, int causal,
                           void* o, const int64_t o_stride[3], hipStream_t st, int probe_qb, float* lse) {
  if (p.qk_held == 2) {
    if (p.D == 128) return p.bf16 ? attn_impl<128, true, 2>(p, qk, vb, causal, o, o_stride, st, probe_qb, lse)
                                  : attn_impl<128, false, 2>(p, qk, vb, causal, o, o_stride, st, probe_qb, lse);
    return p.bf16 ? attn_impl<64, true, 2>(p, qk, vb, causal, o, o_stride, st, probe_qb, lse)
                  : attn_impl<64, false, 2>(p, qk, vb, causal, o, o_stride, st, probe_qb, lse);
  }
  if (p.qk_held == 1) {
    if (p.D == 128) return p.bf16 ? attn_impl<128, true, 1>(p, qk, vb, causal, o, o_stride, st, probe_qb, lse)
                                  : attn_impl<128, false, 1>(p, qk, vb, causal, o, o_stride, st, probe_qb, lse);
    return p.bf16 ? attn_impl<64, true, 1>(p, qk, vb, causal, o, o_stride, st, probe_qb, lse)
                  : attn_impl<64, false, 1>(p, qk, vb, causal, o, o_stride, st, probe_qb, lse);
  }
  if (p.D == 128) return p.bf16 ? attn_impl<128, true, 0>(p, qk, vb, causal, o, o_stride, st, probe_qb, lse)
                                : attn_impl<128, false, 0>(p, qk, vb, causal, o, o_stride, st, probe_qb, lse);
  return p.bf16 ? attn_impl<64, true, 0>(p, qk, vb, causal, o, o_stride, st, probe_qb, lse)
                : attn_impl<64, false, 0>(p, qk, vb, causal, o, o_stride, st, probe_qb, lse);
}

}  // namespace sage
