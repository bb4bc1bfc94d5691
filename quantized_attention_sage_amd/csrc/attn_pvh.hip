// Quantized attention forward kernel for gfx950 (CDNA4), 16-bit P~V.
//
// The setting of the first SageAttention, which the SageAttention2 abstract
// describes (8-bit QK^T, 16-bit P~V) and improves on with FP8 P~ and V: Q, K
// codes, scales, smoothing bias and the online softmax are those of the FP8
// kernel in attn.hip, but P~ = 2^(s - m) is rounded to the input's 16-bit type
// (bf16 or fp16, nearest even) and multiplied with V itself on the bf16/fp16
// matrix cores (v_mfma_f32_32x32x16_{bf16,f16}, fp32 accumulation).
//
// The schedule mirrors attn.hip (one work-group of 4 waves per 128-query block,
// 128-key tiles, S^T = K^ Q^T on the INT8 matrix cores, tile t's
// dequantisation beside the PV product of tile t-1 and its exp2 beside the QK
// product of tile t+1, two-slot LDS rings fed by buffer-to-LDS copies).  What
// differs:
//  * the 16 P~ values a lane holds for a 32-key subtile s (keys 32s + 8a + 4h
//    + b) form two 8-value B operands (a in {0,1}, then a in {2,3}); V is
//    stored channel-major with keys ordered to match (sage.h, SAGE_PV_F16),
//    so P~ still never leaves registers.
//  * a tile has 8 such 16-key steps per 32-channel output tile: 32 PV MFMAs
//    per tile at d = 128 instead of 8.
//  * a V slot is 256 bytes per channel (32 KiB at d = 128), so the rings take
//    98 KiB of LDS and one work-group runs per CU.
#include <type_traits>

#include "sage_internal.h"

namespace sage {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

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

// LDS: K and aux rings of two slots (tile u in slot u % 2) and one V slot.
// K slot: 128 keys x D codes (rows swizzled).  V slot: D channels x 128 keys
// of 2 bytes (256-byte rows, swizzled); V(t) is copied in during phase B of
// tile t, after every wave has read V(t-1), and read in phase A of tile t+1.
// Aux slot: the tile's 128 bias values, then its K scales (8 or 2 used).
// 66 KiB at d = 128: two work-groups per CU.
template <int D>
struct Rings {
  static constexpr int K = kTile * D;
  static constexpr int V = D * kTile * 2;
  static constexpr int AUX = 1024;   // bias (512 B), K scales, spare row at 768
  static constexpr int K0 = 0, V0 = 2 * K, A0 = 2 * K + V;
  static constexpr int BYTES = 2 * (K + AUX) + V;
  static constexpr int J = D / 32;   // 1 KiB copies per wave for one K slot
  static constexpr int JV = D / 16;  // ... and for one V slot
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
// copy and j moves only the scalar offset (4096 j bytes of K rows, 16 j
// channel rows of V).
struct TileSrc {
  i32x4 k, v, b, s;
  uint32_t k_off, v_off, b_off;   // per-lane byte offsets for j = 0 and k0 = 0
  uint32_t v_row;                 // bytes per V channel row (2 n_pad)
  uint32_t s_per_tile;            // K scale groups per 128-key tile (8 or 2)
};

template <int D>
__device__ __forceinline__ TileSrc make_tile_src(const int8_t* kbase, const uint8_t* vbase, const float* brow,
                                                 const float* kscale, int n_scale, int n_pad, int t) {
  constexpr int CPR = D / 16;
  TileSrc s;
  s.k = buffer_rsrc(kbase, static_cast<uint32_t>(n_pad * D));
  s.v = buffer_rsrc(vbase, static_cast<uint32_t>(n_pad * D * 2));
  s.b = buffer_rsrc(brow, static_cast<uint32_t>(n_pad * 4));
  s.s = buffer_rsrc(kscale, static_cast<uint32_t>(n_scale * 4));
  s.s_per_tile = static_cast<uint32_t>(n_scale / (n_pad / kTile));
  const int r = t / CPR, pc = t % CPR;
  s.k_off = static_cast<uint32_t>(r * D + 16 * swz<D>(r, pc));
  const int ch = t >> 4, vc = t & 15;   // 16 channel rows of 256 bytes per 4 KiB copy
  s.v_off = static_cast<uint32_t>(ch * 2 * n_pad + 16 * swz<256>(ch, vc));
  s.b_off = static_cast<uint32_t>(4 * t);
  s.v_row = static_cast<uint32_t>(2 * n_pad);
  return s;
}

// K codes of the 128 keys from k0 into the K slot at LDS address `slot`.
template <int D>
__device__ __forceinline__ void copy_k(uint32_t slot, const TileSrc& s, int k0, int w) {
#pragma unroll
  for (int j = 0; j < Rings<D>::J; ++j)
    dma16(s.k, s.k_off, static_cast<uint32_t>(k0 * D + 4096 * j), slot + (4 * j + w) * 1024);
}

// V of the 128 keys from k0 (all D channels) into a V slot; copy j moves 16
// channel rows.
__device__ __forceinline__ void copy_v_part(uint32_t slot, const TileSrc& s, int k0, int w, int j) {
  dma16(s.v, s.v_off, static_cast<uint32_t>(2 * k0) + 16u * j * s.v_row, slot + (4 * j + w) * 1024);
}
template <int D>
__device__ __forceinline__ void copy_v(uint32_t slot, const TileSrc& s, int k0, int w) {
#pragma unroll
  for (int j = 0; j < Rings<D>::JV; ++j) copy_v_part(slot, s, k0, w, j);
}

// Bias row (waves 0, 1), K scales (wave 2, lanes below s_per_tile) of the 128
// keys from k0 into an aux slot; wave 3 copies the bias again into a spare row
// so that every wave issues exactly one copy.
// The lane's byte offset 4 (64 w + lane) is recomputed at every call (two
// instructions the compiler may not hoist): held across the loop it is
// spilled, and the reload's wait would also wait for the tile copies in flight.
__device__ __forceinline__ void copy_aux(uint32_t slot, const TileSrc& s, int k0, int w) {
  uint32_t lane;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  const uint32_t b_off = 4u * (64u * static_cast<uint32_t>(w) + lane);
  if (w != 2) {
    dma4(s.b, w == 3 ? (b_off & 255u) : b_off, static_cast<uint32_t>(4 * k0), slot + (w == 3 ? 768 : 256 * w));
  } else {
    const uint32_t lane4 = b_off - 512u;
    dma4(s.s, lane4 < 4u * s.s_per_tile ? lane4 : 0u, static_cast<uint32_t>(4 * (k0 / kTile) * s.s_per_tile),
         slot + 512);
  }
}

// 16-bit P~ pair for the bf16/fp16 P~V product (round to nearest even).
template <bool BF16>
__device__ __forceinline__ int pack16(float p0, float p1) {
  if constexpr (BF16) return __builtin_bit_cast(int, __builtin_convertvector((f32x2){p0, p1}, bf16x2));
  else return __builtin_bit_cast(int, __builtin_convertvector((f32x2){p0, p1}, f16x2));
}

// O += V^T P~^T for one 16-key step on the bf16/fp16 matrix cores.
template <bool BF16>
__device__ __forceinline__ f32x16 mfma_pv16(i32x4 v, i32x4 p, f32x16 acc) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v), __builtin_bit_cast(bf16x8, p), acc,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, v), __builtin_bit_cast(f16x8, p), acc,
                                                  0, 0, 0);
}

// 16-bit P~V: the V slots are twice the FP8 ones (98 KiB of LDS at d = 128),
// so one work-group runs per CU and the whole register file is available.
template <int D, bool BF16>
__global__ __launch_bounds__(256, 2) void attn_pvh_kernel(AttnArgs a) {
  constexpr int KS = D / 32;          // 32-channel k-steps of the QK product
  constexpr int CT = D / 32;          // 32-channel tiles of the output
  constexpr int NQK = 4 * KS;         // QK MFMAs per tile
  constexpr int NPV = 8 * CT;         // PV MFMAs (16-key steps x channel tiles) per tile
  constexpr int QK_EVERY = 16 / NQK;  // softmax quads per QK MFMA
  constexpr int PPQ = NPV / 16;       // PV MFMAs per dequant quad
  constexpr int J = Rings<D>::J;
  constexpr int JV = Rings<D>::JV;
  using R = Rings<D>;
  using PB = i32x4;                   // 16-bit P~ operand of one 16-key step
  constexpr int NPB = 8;              // ... per tile
  __shared__ __attribute__((aligned(1024))) uint8_t lds[R::BYTES];
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_ptr(lds)));

  const int t = threadIdx.x, l = t & 63, col = l & 31, hh = l >> 5;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);   // wave index, held in a scalar register
  int bh, qb;
  map_block(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x), a.nblk, a.causal, a.lpt_g, bh, qb);
  const int q0 = qb * 128;
  const int qi = q0 + 32 * w + col;

  const int key_end = a.causal ? min(a.N, q0 + 128) : a.N;
  const int ntiles = (key_end + kTile - 1) / kTile;
  const int8_t* kbase = a.k_codes + static_cast<int64_t>(bh) * a.n_pad * D;
  const uint8_t* vbase = a.v_codes + static_cast<int64_t>(bh) * D * a.n_pad * 2;
  const float* brow = a.bias + (static_cast<int64_t>(bh) * a.nblk + qb) * a.n_pad;
  const int n_kscale = a.gran == SAGE_GRAN_THREAD ? a.n_pad / 16 : a.n_pad / 64;
  const float* kscale = a.k_scale + static_cast<int64_t>(bh) * n_kscale;

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
  // exp2(x - (m + base_shift)) = P~ = exp2(x - m): the host passes log2_pr = 0
  const float base_shift = -a.log2_pr;
  const bool thread_gran = a.gran == SAGE_GRAN_THREAD;

  // First key of tile u; tiles past the end copy the last tile again (their
  // data is never used, and every wave keeps one copy count per issue point).
  auto kofs = [&](int u) __attribute__((always_inline)) { return min(u, ntiles - 1) * kTile; };

  const TileSrc src = make_tile_src<D>(kbase, vbase, brow, kscale, n_kscale, a.n_pad, t);
  // Tile t reads K of tile t+1 (and t's own K only in the prologue), V of tile
  // t-1 and the aux row of tile t.  It copies the aux row of tile t+1 when it
  // starts, and V of tile t, then K of tile t+2, once every wave has read V of
  // tile t-1 (mid-tile).  Tile 0's PV product reads the V slot as tile -1,
  // zero-filled here (its P~ is 0 too).
  copy_k<D>(lds0 + R::K0, src, kofs(0), w);
  copy_aux(lds0 + R::A0, src, kofs(0), w);
  {
    uint4* vz = reinterpret_cast<uint4*>(lds + R::V0);
#pragma unroll
    for (int i = t; i < R::V / 16; i += 256) vz[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  // K(0) and aux(0) are needed now.  They are waited for by count 0, which
  // assumes nothing about the completion order of copies of different sizes;
  // the copies of K(1) are issued after the barrier and run beside the first
  // QK product (they are what the first tile-start wait allows for).
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  copy_k<D>(lds0 + R::K0 + R::K, src, kofs(1), w);

  // Per-lane byte offsets of the LDS fragments, relative to a slot.  The
  // swizzle term does not depend on the subtile (K) or the channel tile (V),
  // so those move only the immediate offset of the read.
  //   K fragment, subtile st, channels 32kk..: kofl[kk] + 32 st D
  //   V fragment of 16-key step sm = 2 st + m (keys 32 st + 16 m..; the lane
  //   half hh holds the 8 at positions 8 hh..), channels 32c..: vofh[sm] + 32 c 256
  //   bias quad (subtile st, a): 16 hh + 4 (32 st + 8 a)
  uint32_t kofl[KS], vofh[8];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) kofl[kk] = static_cast<uint32_t>(col * D + 16 * swz<D>(col, 2 * kk + hh));
#pragma unroll
  for (int sm = 0; sm < 8; ++sm) vofh[sm] = static_cast<uint32_t>(col * 256 + 16 * swz<256>(col, 2 * sm + hh));

  auto lds_i4 = [&](uint32_t off) __attribute__((always_inline)) {
    return *reinterpret_cast<const i32x4*>(lds + off);
  };
  auto k_frag = [&](const uint32_t* ko, int slot_off, int st, int kk) __attribute__((always_inline)) {
    return lds_i4(ko[kk] + slot_off + 32 * st * D);
  };
  auto v_frag16 = [&](const uint32_t* vo, int slot_off, int sm, int c) __attribute__((always_inline)) {
    return lds_i4(vo[sm] + slot_off + 32 * 256 * c);
  };

  f32x16 oacc[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[c][i] = 0.f;
  float m = -INFINITY, lsum = 0.f;
  i32x16 sA[4], sB[4];     // S^T of the tile whose softmax runs next (alternating sets)
  PB pA[NPB], pB[NPB];     // 16-bit P~ of the previous tile (alternating sets)
#pragma unroll
  for (int kc = 0; kc < NPB; ++kc) pA[kc] = PB{};

  // QK product of tile 0 (not overlapped).
#pragma unroll
  for (int st = 0; st < 4; ++st) {
#pragma unroll
    for (int i = 0; i < 16; ++i) sA[st][i] = 0;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      sA[st] = __builtin_amdgcn_mfma_i32_32x32x32_i8(k_frag(kofl, R::K0, st, kk), qf[kk], sA[st], 0, 0, 0);
  }

  // One tile.  CUR: its ring slot (t % 2); S_cur / S_nxt: S^T of tiles t and
  // t+1; pb_prv / pb_cur: 16-bit P~ of tiles t-1 and t.
  auto tile = [&](const int tt, auto cur_slot, i32x16* S_cur, i32x16* S_nxt, PB* pb_prv, PB* pb_cur)
                  __attribute__((always_inline)) {
    constexpr int CUR = decltype(cur_slot)::value, NXT = 1 - CUR;
    const int k0 = tt * kTile;
    // This wave's copies of aux(t) (issued when tile t-1 started) and of V(t-1)
    // (issued first in phase B of tile t-1) are complete; only the J copies of
    // K(t+1) issued after them may still run (see the mid-tile wait).  After
    // the barrier every wave's V(t-1) is in the slot and every wave is done
    // with aux(t-1), whose slot is refilled below.
    static_assert(J == 4 || J == 2, "K copies per tile");
    if constexpr (J == 4) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    copy_aux(lds0 + R::A0 + NXT * R::AUX, src, kofs(tt + 1), w);

    // Fresh copies of the lane offsets: without this the compiler hoists one
    // address register per (slot, fragment) out of the loop and spills them.
    uint32_t ko[KS], voh[8], bo = 16u * hh;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) { ko[kk] = kofl[kk]; asm volatile("" : "+v"(ko[kk])); }
#pragma unroll
    for (int sm = 0; sm < 8; ++sm) { voh[sm] = vofh[sm]; asm volatile("" : "+v"(voh[sm])); }
    asm volatile("" : "+v"(bo));
    const int aux = R::A0 + CUR * R::AUX;
    float cs[4];
    {
      const float* ksc = reinterpret_cast<const float*>(lds + aux + 512);
#pragma unroll
      for (int st = 0; st < 4; ++st) cs[st] = dq2 * (thread_gran ? ksc[2 * st + hh] : ksc[st >> 1]);
    }

    // Phase A: dequantise S(t) and take the row maximum, beside the PV product
    // of tile t-1 (V(t-1) is in slot NXT).  LDS operands are fetched ahead of
    // use (bias one quad, V fragments one PV interval) so that a quad's vector
    // work covers their latency.
    const int vslot_off = R::V0;
    float x[4][16];
    float mx = -INFINITY, mx2 = -INFINITY;
    i32x4 vh[2 * PPQ];
#pragma unroll
    for (int u = 0; u < PPQ; ++u) vh[u] = v_frag16(voh, vslot_off, u / CT, u % CT);
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
      // V fragments of the next quad's PV steps (PPQ per quad; step e: 16-key step e / CT, channel tile e % CT).
      if (i + 1 < 16) {
#pragma unroll
        for (int u = 0; u < PPQ; ++u) {
          const int e1 = PPQ * (i + 1) + u;
          vh[((i + 1) & 1) * PPQ + u] = v_frag16(voh, vslot_off, e1 / CT, e1 % CT);
        }
      }
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
#pragma unroll
      for (int u = 0; u < PPQ; ++u) {
        const int ep = PPQ * i + u, c = ep % CT;
        oacc[c] = mfma_pv16<BF16>(vh[(i & 1) * PPQ + u], pb_prv[ep / CT], oacc[c]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // Every wave has read V(t-1) (the slot is refilled in phase B) and this
    // wave's copies of K(t+1) are complete (only the aux copy issued at the
    // start of this tile may still run); after the barrier every wave's are.
    asm volatile("s_waitcnt vmcnt(1) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // K fragments of the first two QK MFMAs of phase B, read only now: K(t+1)
    // is copied by all four waves, and only the barrier above makes every
    // wave's part of it visible.
    const int kslot_off = R::K0 + NXT * R::K;
    i32x4 kf[3];
    kf[0] = k_frag(ko, kslot_off, 0, 0);
    if (NQK > 1) kf[1] = k_frag(ko, kslot_off, (1 / KS), 1 % KS);

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
    const i32x16 zero16 = {};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int st = i >> 2, q4 = i & 3;
      const int e = i / QK_EVERY;
      if (i % QK_EVERY == 0 && e + 2 < NQK) kf[(e + 2) % 3] = k_frag(ko, kslot_off, (e + 2) / KS, (e + 2) % KS);
      // Copies, spread evenly over the 16 quads: first V(t) into the V slot
      // (freed at the mid-tile barrier; read in phase A of tile t+1), then
      // K(t+2) into K slot CUR (K(t) was last read in tile t-1).
      {
        constexpr int C = J + JV;   // copies per tile
#pragma unroll
        for (int cj = (i * C + 15) / 16; cj < ((i + 1) * C + 15) / 16; ++cj) {
          if (cj < JV) copy_v_part(lds0 + R::V0, src, kofs(tt), w, cj);
          else dma16(src.k, src.k_off, static_cast<uint32_t>(kofs(tt + 2) * D + 4096 * (cj - JV)),
                     lds0 + R::K0 + CUR * R::K + (4 * (cj - JV) + w) * 1024);
        }
      }
      const float p0 = __builtin_amdgcn_exp2f(x[st][4 * q4 + 0] - base);
      const float p1 = __builtin_amdgcn_exp2f(x[st][4 * q4 + 1] - base);
      const float p2 = __builtin_amdgcn_exp2f(x[st][4 * q4 + 2] - base);
      const float p3 = __builtin_amdgcn_exp2f(x[st][4 * q4 + 3] - base);
      ps += (p0 + p1) + (p2 + p3);
      {
        // quad q4 of subtile st holds keys 32 st + 8 q4 + 4 hh + 0..3: 16-key step 2 st + q4 / 2, dwords 2 (q4 % 2)..
        int v0 = pack16<BF16>(p0, p1), v1 = pack16<BF16>(p2, p3);
        asm volatile("" : "+v"(v0), "+v"(v1), "+v"(ps));
        pb_cur[2 * st + (q4 >> 1)][2 * (q4 & 1)] = v0;
        pb_cur[2 * st + (q4 >> 1)][2 * (q4 & 1) + 1] = v1;
      }
      if (i % QK_EVERY == 0) {
        const int sn = e / KS, kk = e % KS;
        S_nxt[sn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[e % 3], qf[kk], kk == 0 ? zero16 : S_nxt[sn], 0, 0, 0);
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
#pragma unroll
    for (int kc = 0; kc < NPB; ++kc) pA[kc] = pB[kc];
  }

  // PV product of the last tile (V(ntiles-1) was copied in its phase B).
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  {
    const int lv = R::V0;
#pragma unroll
    for (int sm = 0; sm < 8; ++sm)
#pragma unroll
      for (int c = 0; c < CT; ++c) oacc[c] = mfma_pv16<BF16>(v_frag16(vofh, lv, sm, c), pA[sm], oacc[c]);
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
  // P~ = 2^(s - m) itself (no E4M3 range to fill): base shift 0.
  a.log2_pr = 0.f;
  a.lpt_g = lpt_group(p.B * p.H, static_cast<int64_t>(3) * p.n_pad * p.D);
  hipLaunchKernelGGL((attn_pvh_kernel<D, BF16>), dim3(p.nblk * p.B * p.H), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_pvh(const Problem& p, const sage_qk_buffers& qk, const sage_v_buffers& vb, int causal,
                           void* o, const int64_t o_stride[3], hipStream_t st) {
  if (p.D == 128) return p.bf16 ? attn_impl<128, true>(p, qk, vb, causal, o, o_stride, st)
                                : attn_impl<128, false>(p, qk, vb, causal, o, o_stride, st);
  return p.bf16 ? attn_impl<64, true>(p, qk, vb, causal, o, o_stride, st)
                : attn_impl<64, false>(p, qk, vb, causal, o, o_stride, st);
}

}  // namespace sage
