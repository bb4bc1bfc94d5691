// Quantized attention forward kernel for gfx950 (CDNA4), MXFP4 Q and K.
//
// The FP4 microscaling of the SageAttention3 abstract, read as OCP MXFP4: Q
// and K codes are E2M1 with one E8M0 scale per 32 channels of a token
// (include/sage.h, SAGE_QK_MXFP4), and S^T = K^ Q^T runs on
// v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands: each lane's 32 codes of
// a 64-channel step come with the E8M0 scale of its 32-channel block, and the
// product arrives in fp32 with the scales applied.  The rest (smoothing bias,
// online softmax, FP8 P~ and V, epilogue) is the FP8 kernel of
// attn.hip, whose schedule this file keeps.  What differs:
//  * dequantisation is one FMA per score (s = S sm_scale log2 e + bias): no
//    integer-to-float conversion and no per-group scales;
//  * a QK step covers 64 channels (8 products per 128-key tile at d = 128,
//    half the INT8 count, each on the FP4 rate);
//  * a K slot holds 128 keys x d/2 bytes of codes followed by their scale
//    bytes, copied together one tile ahead; the aux slot carries the bias only.
#include "sage_internal.h"

namespace sage {
namespace {

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

// LDS rings of two slots; tile u lives in slot u % 2.  K slot: 128 keys x D/2
// bytes of E2M1 codes (rows swizzled), then 1 KiB for their scale bytes (key
// j's D/32 bytes at j D/32; the rest is spare).  V slot: D channels x 128 keys
// (rows swizzled).  Aux slot: the tile's 128 bias values (and spare rows).
template <int D>
struct Rings {
  static constexpr int KC = kTile * D / 2;   // code bytes of a K slot
  static constexpr int K = KC + 1024;
  static constexpr int V = D * kTile;
  static constexpr int AUX = 1024;
  static constexpr int K0 = 0, V0 = 2 * K, A0 = 2 * K + 2 * V;
  static constexpr int BYTES = 2 * (K + V + AUX);
  static constexpr int J = D / 64;    // 1 KiB code copies per wave for one K slot (plus one scale copy)
  static constexpr int JV = D / 32;   // 1 KiB copies per wave for one V slot
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
  uint32_t k_off, v_off, b_off;   // per-lane byte offsets for j = 0 and k0 = 0
  uint32_t s_off;                 // per-lane byte offset of the K scale copy
  uint32_t v_row;                 // bytes per V channel row (n_pad)
};

template <int D>
__device__ __forceinline__ TileSrc make_tile_src(const int8_t* kbase, const uint8_t* vbase, const float* brow,
                                                 const uint8_t* kscale, int n_scale, int n_pad, int t) {
  constexpr int CPR = D / 32;   // 16-byte chunks per K code row (D/2 bytes)
  TileSrc s;
  s.k = buffer_rsrc(kbase, static_cast<uint32_t>(n_pad * D / 2));
  s.v = buffer_rsrc(vbase, static_cast<uint32_t>(n_pad * D));
  s.b = buffer_rsrc(brow, static_cast<uint32_t>(n_pad * 4));
  s.s = buffer_rsrc(kscale, static_cast<uint32_t>(n_scale));
  const int r = t / CPR, pc = t % CPR;
  s.k_off = static_cast<uint32_t>(r * (D / 2) + 16 * swz<D / 2>(r, pc));
  s.s_off = static_cast<uint32_t>((4 * t) & (4 * D - 1));
  const int ch = t >> 3, vc = t & 7;
  s.v_off = static_cast<uint32_t>(ch * n_pad + 16 * swz<128>(ch, vc));
  s.b_off = static_cast<uint32_t>(4 * t);
  s.v_row = static_cast<uint32_t>(n_pad);
  return s;
}

// Copy j of the K codes of the 128 keys from k0 (j < J), or their scale bytes
// (j = J; waves past the 4 D bytes copy them again into the spare area), into
// the K slot at LDS address `slot`.
template <int D>
__device__ __forceinline__ void copy_k_part(uint32_t slot, const TileSrc& s, int k0, int w, int j) {
  if (j < Rings<D>::J)
    dma16(s.k, s.k_off, static_cast<uint32_t>(k0 * (D / 2) + 4096 * j), slot + (4 * j + w) * 1024);
  else
    dma4(s.s, s.s_off, static_cast<uint32_t>(k0 * (D / 32)), slot + Rings<D>::KC + 256 * w);
}
template <int D>
__device__ __forceinline__ void copy_k(uint32_t slot, const TileSrc& s, int k0, int w) {
#pragma unroll
  for (int j = 0; j <= Rings<D>::J; ++j) copy_k_part<D>(slot, s, k0, w, j);
}

// V codes of the 128 keys from k0 (all D channels) into a V slot.
template <int D>
__device__ __forceinline__ void copy_v_part(uint32_t slot, const TileSrc& s, int k0, int w, int j) {
  dma16(s.v, s.v_off, static_cast<uint32_t>(k0) + 32u * j * s.v_row, slot + (4 * j + w) * 1024);
}
template <int D>
__device__ __forceinline__ void copy_v(uint32_t slot, const TileSrc& s, int k0, int w) {
#pragma unroll
  for (int j = 0; j < Rings<D>::JV; ++j) copy_v_part<D>(slot, s, k0, w, j);
}

// Bias row of the 128 keys from k0 into an aux slot (waves 0, 1); waves 2 and
// 3 copy its first half again into the spare rows, so that every wave issues
// exactly one copy.
__device__ __forceinline__ void copy_aux(uint32_t slot, const TileSrc& s, int k0, int w) {
  dma4(s.b, w >= 2 ? (s.b_off & 255u) : s.b_off, static_cast<uint32_t>(4 * k0), slot + 256 * w);
}

// The QK step: S^T(32 keys x 32 queries) += K^ Q^T over 64 channels, FP4
// operands (4 registers each; the upper half of the 8-register operand is not
// read for FP4) with the E8M0 scale of each lane's 32-channel block.
__device__ __forceinline__ f32x16 mfma_qk_fp4(i32x4 k, i32x4 q, f32x16 acc, int ks, int qs) {
  const i32x8 k8 = __builtin_shufflevector(k, k, 0, 1, 2, 3, -1, -1, -1, -1);
  const i32x8 q8 = __builtin_shufflevector(q, q, 0, 1, 2, 3, -1, -1, -1, -1);
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k8, q8, acc, 4, 4, 0, ks, 0, qs);
}

template <int D, bool BF16>
__global__ __launch_bounds__(256, 2) void attn_fp4_kernel(AttnArgs a) {
  constexpr int KS = D / 64;          // 64-channel k-steps of the QK product
  constexpr int CT = D / 32;          // 32-channel tiles of the output
  constexpr int NQK = 4 * KS;         // QK MFMAs per tile
  constexpr int NPV = 2 * CT;         // PV MFMAs per tile
  constexpr int QK_EVERY = 16 / NQK;  // softmax quads per QK MFMA
  constexpr int PV_EVERY = 16 / NPV;  // dequant quads per PV MFMA
  constexpr int J = Rings<D>::J;
  constexpr int JV = Rings<D>::JV;
  using R = Rings<D>;
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
  const int8_t* kbase = a.k_codes + static_cast<int64_t>(bh) * a.n_pad * (D / 2);
  const uint8_t* vbase = a.v_codes + static_cast<int64_t>(bh) * D * a.n_pad;
  const float* brow = a.bias + (static_cast<int64_t>(bh) * a.nblk + qb) * a.n_pad;
  const int n_kscale = a.n_pad * (D / 32);   // scale bytes per head
  const uint8_t* kscale = reinterpret_cast<const uint8_t*>(a.k_scale) + static_cast<int64_t>(bh) * n_kscale;

  // Q codes of this lane's query for each 64-channel step (lane half hh: its
  // 32-channel block), and the E8M0 scale byte of that block.
  i32x4 qf[KS];
  int qsc[KS];
  {
    const int8_t* qrow = a.q_codes + (static_cast<int64_t>(bh) * a.n_pad + qi) * (D / 2);
    const uint8_t* qs = reinterpret_cast<const uint8_t*>(a.q_scale) + (static_cast<int64_t>(bh) * a.n_pad + qi) * (D / 32);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qf[s] = *reinterpret_cast<const i32x4*>(qrow + 32 * s + 16 * hh);
      qsc[s] = qs[2 * s + hh];
    }
  }
  const float c_log2 = a.scale_log2;
  // exp2(x - (m + base_shift)) = P~ * P_r with P~ = exp2(x - m)
  const float base_shift = -a.log2_pr;

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
  copy_aux(lds0 + R::A0, src, kofs(0), w);
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
  //   K fragment, subtile st, channels 64kk + 32 hh..: kofl[kk] + 32 st D/2;
  //   its scale byte: kscl[kk] + 32 st D/32
  //   V fragment, keys 64kc.. (lane's 32), channels 32c..: vofl[kc][h2] + 32 c kTile, h2 = 0, 1
  //   bias quad (subtile st, a): 16 hh + 4 (32 st + 8 a)
  uint32_t kofl[KS], kscl[KS], vofl[2][2];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    kofl[kk] = static_cast<uint32_t>(col * (D / 2) + 16 * swz<D / 2>(col, 2 * kk + hh));
    kscl[kk] = static_cast<uint32_t>(R::KC + col * (D / 32) + 2 * kk + hh);
  }
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
      vofl[kc][h2] = static_cast<uint32_t>(col * kTile + 16 * swz<128>(col, 4 * kc + 2 * hh + h2));

  auto lds_i4 = [&](uint32_t off) __attribute__((always_inline)) {
    return *reinterpret_cast<const i32x4*>(lds + off);
  };
  auto k_frag = [&](const uint32_t* ko, int slot_off, int st, int kk) __attribute__((always_inline)) {
    return lds_i4(ko[kk] + slot_off + 32 * st * (D / 2));
  };
  auto k_scale = [&](const uint32_t* ks, int slot_off, int st, int kk) __attribute__((always_inline)) {
    return static_cast<int>(lds[ks[kk] + slot_off + 32 * st * (D / 32)]);
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
  f32x16 sA[4], sB[4];     // S^T of the tile whose softmax runs next (alternating sets)
  i32x8 pA[2], pB[2];      // FP8 P~ of the previous tile (alternating sets)
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int i = 0; i < 8; ++i) pA[kc][i] = 0;

  // QK product of tile 0 (not overlapped).
#pragma unroll
  for (int st = 0; st < 4; ++st) {
#pragma unroll
    for (int i = 0; i < 16; ++i) sA[st][i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      sA[st] = mfma_qk_fp4(k_frag(kofl, R::K0, st, kk), qf[kk], sA[st], k_scale(kscl, R::K0, st, kk), qsc[kk]);
  }

  // One tile.  CUR: its ring slot (t % 2); S_cur / S_nxt: S^T of tiles t and
  // t+1; pb_prv / pb_cur: FP8 P~ of tiles t-1 and t.
  auto tile = [&](const int tt, auto cur_slot, f32x16* S_cur, f32x16* S_nxt, i32x8* pb_prv, i32x8* pb_cur)
                  __attribute__((always_inline)) {
    constexpr int CUR = decltype(cur_slot)::value, NXT = 1 - CUR;
    const int k0 = tt * kTile;
    // This wave's copy of aux(t) (issued when tile t-1 started) is complete;
    // only the J + 1 + JV copies of K(t+1) and V(t) issued in phase B of tile
    // t-1 may still run (see the mid-tile wait).  After the barrier every wave
    // is done with aux(t-1), whose slot is refilled below.
    static_assert(J + 1 + JV == 7 || J + 1 + JV == 4, "copies per tile");
    if constexpr (J + 1 + JV == 7) asm volatile("s_waitcnt vmcnt(7) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    copy_aux(lds0 + R::A0 + NXT * R::AUX, src, kofs(tt + 1), w);

    // Fresh copies of the lane offsets: without this the compiler hoists one
    // address register per (slot, fragment) out of the loop and spills them.
    uint32_t ko[KS], ksl[KS], vo[2][2], bo = 16u * hh;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      ko[kk] = kofl[kk];
      ksl[kk] = kscl[kk];
      asm volatile("" : "+v"(ko[kk]), "+v"(ksl[kk]));
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      vo[kc][0] = vofl[kc][0]; vo[kc][1] = vofl[kc][1];
      asm volatile("" : "+v"(vo[kc][0]), "+v"(vo[kc][1]));
    }
    asm volatile("" : "+v"(bo));
    const int aux = R::A0 + CUR * R::AUX;

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
      xs[0] = S_cur[st][4 * a4 + 0] * c_log2 + bv.x;
      xs[1] = S_cur[st][4 * a4 + 1] * c_log2 + bv.y;
      xs[2] = S_cur[st][4 * a4 + 2] * c_log2 + bv.z;
      xs[3] = S_cur[st][4 * a4 + 3] * c_log2 + bv.w;
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
    int kfs[3];
    kf[0] = k_frag(ko, kslot_off, 0, 0);
    kfs[0] = k_scale(ksl, kslot_off, 0, 0);
    if (NQK > 1) {
      kf[1] = k_frag(ko, kslot_off, (1 / KS), 1 % KS);
      kfs[1] = k_scale(ksl, kslot_off, (1 / KS), 1 % KS);
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
    const f32x16 zero16 = {};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int st = i >> 2, q4 = i & 3;
      const int e = i / QK_EVERY;
      if (i % QK_EVERY == 0 && e + 2 < NQK) {
        kf[(e + 2) % 3] = k_frag(ko, kslot_off, (e + 2) / KS, (e + 2) % KS);
        kfs[(e + 2) % 3] = k_scale(ksl, kslot_off, (e + 2) / KS, (e + 2) % KS);
      }
      // Copies for later tiles, spread evenly over the 16 quads: K(t+2) codes
      // and scales into slot CUR (K(t) was last read in tile t-1) and V(t+1)
      // into slot NXT (freed at the mid-tile barrier).
      {
        constexpr int C = J + 1 + JV;
#pragma unroll
        for (int cj = (i * C + 15) / 16; cj < ((i + 1) * C + 15) / 16; ++cj) {
          if (cj <= J) copy_k_part<D>(lds0 + R::K0 + CUR * R::K, src, kofs(tt + 2), w, cj);
          else copy_v_part<D>(lds0 + R::V0 + NXT * R::V, src, kofs(tt + 1), w, cj - J - 1);
        }
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
        const int sn = e / KS, kk = e % KS;
        S_nxt[sn] = mfma_qk_fp4(kf[e % 3], qf[kk], kk == 0 ? zero16 : S_nxt[sn], kfs[e % 3], qsc[kk]);
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
  a.lpt_g = lpt_group(p.B * p.H, static_cast<int64_t>(p.n_pad) * (p.D + p.D / 2 + p.D / 32));
  hipLaunchKernelGGL((attn_fp4_kernel<D, BF16>), dim3(p.nblk * p.B * p.H), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fp4(const Problem& p, const sage_qk_buffers& qk, const sage_v_buffers& vb, int causal,
                           void* o, const int64_t o_stride[3], hipStream_t st) {
  if (p.D == 128) return p.bf16 ? attn_impl<128, true>(p, qk, vb, causal, o, o_stride, st)
                                : attn_impl<128, false>(p, qk, vb, causal, o, o_stride, st);
  return p.bf16 ? attn_impl<64, true>(p, qk, vb, causal, o, o_stride, st)
                : attn_impl<64, false>(p, qk, vb, causal, o, o_stride, st);
}

}  // namespace sage
