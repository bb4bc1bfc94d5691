/*
 * sage.h -- C ABI of a SageAttention2-style quantized attention forward pass
 * for AMD Instinct MI355X (gfx950).
 *
 * What is computed (the method of "SageAttention2 Technical Report: Accurate 4
 * Bit Attention for Plug-and-play Inference Acceleration", abstract, and of the
 * SageAttention2++ summary, sections "2. Preliminary" and "2.1 SageAttention2"):
 *
 *   K' = K - mean_tokens(K)                       (per channel, per head)
 *   Q' = Q - mean_block(Q)                        (per channel, per 128-token block qb)
 *   dS[qb, j] = mean_block(Q)(qb) . K'_j          (restores the Q mean)
 *   Q', K'  -> integer codes with per-group scales (INT8, or INT4-range [-7,7]
 *              held in int8 on the INT8 matrix cores or, with SAGE_QK_INT_E4M3
 *              / _E2M3, held as E4M3 / FP6 E2M3 on the FP8 / FP6 matrix cores,
 *              with the same S)
 *   V'  = V - mean_tokens(V); V' -> FP8 E4M3 with per-channel scales
 *   S   = dQ dK (q^ . k^) + dS;  online softmax over 128-key tiles against the
 *         running row maximum m, so P~ = 2^(s - m) <= 1 with s the score in
 *         log2 units (S sm_scale log2 e);
 *   P~  -> FP8 E4M3 with the fixed scale 1 / P_r;  O = sum P~ V' / l + mean(V),
 *         l = sum of the fp32 P~.
 *
 * All entry points are plain C with device pointers, sizes and a HIP stream
 * (passed as void*, a hipStream_t; NULL is the default stream).  The library
 * never allocates or frees memory: the caller owns every buffer (the one
 * exception is the static workspace of sage_attn_static, a device array the
 * library holds per GPU for callers that cannot allocate).  Apart from
 * sage_probe_qk_bits, which waits for its sums, nothing synchronises: every
 * call only enqueues work on the given stream.
 *
 * Error behaviour: every argument is validated on the host before anything is
 * enqueued.  A call that returns an error has launched nothing and written
 * nothing.  SAGE_EHIP reports a launch failure (hipGetLastError); device-side
 * faults surface at the caller's next synchronisation.  sage_last_error()
 * returns a thread-local message describing the last failure.  No C++
 * exception crosses this interface.
 */
#ifndef SAGE_H_
#define SAGE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SAGE_API __attribute__((visibility("default")))

/* Bumped whenever a buffer layout, a group map or a struct below changes. */
#define SAGE_ABI_VERSION 7

typedef enum {
  SAGE_OK = 0,
  SAGE_EINVAL = 1,       /* bad pointer, shape, stride, alignment or size */
  SAGE_EUNSUPPORTED = 2, /* valid request outside what this library supports */
  SAGE_EHIP = 3          /* the HIP runtime reported an error */
} sage_status;

typedef enum { SAGE_F16 = 0, SAGE_BF16 = 1 } sage_dtype;

/* Quantisation groups of Q and K (the pages' "per-block", "warp-level" and
 * "per-thread" granularities; the SageAttention2 abstract and the
 * SageAttention2++ summary, 2.1).  Token indices are per head.
 *   SAGE_GRAN_THREAD: Q group = one token; K group = the 16 keys
 *                     {32s + 8a + 4h + b : a, b in 0..3} for each 32-key block
 *                     s and h in {0,1}; K scale index = 2s + h.
 *   SAGE_GRAN_WARP:   Q group = 32 consecutive tokens; K group = 64 keys.
 *   SAGE_GRAN_BLOCK:  Q group = 128 consecutive tokens; K group = 64 keys. */
typedef enum { SAGE_GRAN_THREAD = 0, SAGE_GRAN_WARP = 1, SAGE_GRAN_BLOCK = 2 } sage_gran;

/* Precision of the P~V product.
 *   SAGE_PV_FP8: SageAttention2 (abstract; SageAttention2++ summary 2.1): V
 *                smoothed and encoded to FP8 E4M3 per channel, P~ to FP8
 *                with the fixed scale 1 / P_r, FP8 matrix cores.
 *   SAGE_PV_F16: the SageAttention (first version) setting the SageAttention2
 *                abstract builds on: P~ and V in the 16-bit type of the shape
 *                (round to nearest even for P~; V exactly as given, without
 *                smoothing, so smooth_v and v_range do not apply) on the
 *                bf16/fp16 matrix cores with fp32 accumulation. */
typedef enum { SAGE_PV_FP8 = 0, SAGE_PV_F16 = 1 } sage_pv_mode;

/* Format of the Q and K codes.
 *   SAGE_QK_INT:   integer codes with per-group scales (qk_bits, gran).
 *   SAGE_QK_MXFP4: the FP4 microscaling of the SageAttention3 abstract, read
 *                  as OCP MXFP4: E2M1 codes (nearest, ties to even,
 *                  saturating at 6) and one E8M0 scale 2^(e - 127) per 32
 *                  channels of a token, with the smallest power of two s such
 *                  that 6 s >= the block's max |x'|; the QK^T product runs on
 *                  the scaled FP4 matrix cores.  qk_bits and gran do not apply.
 *   SAGE_QK_INT_E4M3: the INT4-range integer codes of SAGE_QK_INT (qk_bits
 *                  must be 4; gran applies), each stored as the E4M3 byte of
 *                  the same integer (every integer in [-7, 7] is exact in
 *                  E4M3; code 0 is byte 0x00).  The QK^T product then runs on
 *                  the FP8 matrix cores with fp32 accumulation; every partial
 *                  sum is an integer below 2^24, so S is bit-identical to the
 *                  integer product of SAGE_QK_INT and so is the output.  With
 *                  SAGE_PV_FP8 only.
 *   SAGE_QK_INT_E2M3: the same INT4-range codes as 6-bit FP6 E2M3 codes (every
 *                  integer in [-7, 7] is exact; sign bit 5, exponent bits 4:3
 *                  with bias 1, mantissa bits 2:0), packed in the operand
 *                  layout of the 64-deep FP6 matrix product, which runs at
 *                  twice the FP8 rate.  Per token and per 64-channel group j,
 *                  half h (h in {0, 1}) is a slot of 32 values: value i is
 *                  channel 64j + 16h + i for i < 16 and 64j + 32 + 16h + i - 16
 *                  for i >= 16, at bits 6i .. 6i + 5 of 24 bytes.  The slot's
 *                  bytes 0..15 sit at byte 16(4j + h) of the token's d bytes,
 *                  bytes 16..23 at byte 16(4j + 2 + h), followed by 8 zero
 *                  bytes.  S and the output are bit-identical to SAGE_QK_INT.
 *                  qk_bits must be 4; SAGE_PV_FP8 only. */
typedef enum { SAGE_QK_INT = 0, SAGE_QK_MXFP4 = 1, SAGE_QK_INT_E4M3 = 2, SAGE_QK_INT_E2M3 = 3 } sage_qk_format;

/* Shape of Q, K, V ([B, H, N, d], element type dtype).  Strides are in
 * elements for the B, H and N dimensions; the d dimension is contiguous.
 * Every stride must be a multiple of 8 and every tensor pointer 16-byte
 * aligned; the N stride must be below 2^22 elements (SAGE_EUNSUPPORTED
 * otherwise).  Supported: d in {64, 128}; 1 <= N <= 2^20; B, H >= 1. */
typedef struct {
  int64_t B, H, N, d;
  int32_t dtype;         /* sage_dtype, shared by Q, K, V and O */
  int32_t reserved;
  int64_t q_stride[3];
  int64_t k_stride[3];
  int64_t v_stride[3];
} sage_shape;

/* Method settings.  sage_params_default() fills the defaults shown. */
typedef struct {
  int32_t qk_bits;   /* 8 (default) or 4 (INT4-range codes, qmax 7)           */
  int32_t gran;      /* sage_gran, default SAGE_GRAN_THREAD                   */
  int32_t smooth_q;  /* 1 (default): subtract the 128-token block mean of Q   */
  int32_t smooth_k;  /* 1 (default): subtract the token mean of K             */
  int32_t smooth_v;  /* 1 (default): subtract the token mean of V             */
  float p_range;     /* P_r in (0, 448], default 448: P~ code = E4M3(P~ * P_r)    */
  float v_range;     /* V_r in (0, 448], default 448: V code = E4M3(V' V_r/amax) */
  float sm_scale;    /* softmax scale; 0 (default) means 1/sqrt(d)            */
  int32_t pv_mode;   /* sage_pv_mode, default SAGE_PV_FP8                     */
  int32_t qk_format; /* sage_qk_format, default SAGE_QK_INT                   */
} sage_params;

/* Device buffers written by sage_quant_qk (N_pad = 128 * ceil(N / 128)).
 *   q_codes  int8  [B, H, N_pad, d]   row-major, rows >= N hold 0
 *   q_scale  fp32  [B, H, Gq]         Gq = N_pad (THREAD), N_pad/32 (WARP), N_pad/128 (BLOCK)
 *   q_mean   fp32  [B, H, N_pad/128, d]
 *   k_codes  int8  [B, H, N_pad, d]
 *   k_scale  fp32  [B, H, Gk]         Gk = N_pad/16 (THREAD), N_pad/64 (WARP, BLOCK)
 *   k_mean   fp32  [B, H, d]
 *   bias     fp32  [B, H, N_pad/128, N_pad]   dS[qb, j] * sm_scale * log2(e)
 *            (the bias in the exp2 domain of the softmax); 0 for j >= N
 *   k_partial fp32 [B, H, N_pad/128, d]       scratch (per-block K sums; then, when
 *            the bias is formed, the bf16 hi/lo split of each Q block mean)
 * With SAGE_QK_INT_E4M3 q_codes and k_codes hold E4M3 bytes (same layout);
 * with SAGE_QK_INT_E2M3 each d-byte row holds the packed E2M3 slots.
 * With SAGE_QK_MXFP4 the codes and scales of Q and K are instead
 *   q_codes, k_codes  uint8 [B, H, N_pad, d/2]   E2M1 codes, channel 2i in the
 *                     low nibble of byte i; rows >= N hold 0
 *   q_scale, k_scale  uint8 [B, H, N_pad, d/32]  E8M0 scale bytes, one per 32
 *                     channels of a token; rows >= N hold 0
 * (the pointers keep their types; the layout reports the byte sizes). */
typedef struct {
  int8_t* q_codes;
  float* q_scale;
  float* q_mean;
  int8_t* k_codes;
  float* k_scale;
  float* k_mean;
  float* bias;
  float* k_partial;
} sage_qk_buffers;

/* Device buffers written by sage_quant_v.
 *   SAGE_PV_FP8:
 *   v_codes  uint8 [B, H, d, N_pad]  E4M3 codes, channel-major.  Within every
 *            64-key group starting at key 64g, byte 32h + t (h in {0,1},
 *            t in 0..31) holds key 64g + 32(t/16) + 8((t%16)/4) + 4h + t%4.
 *            Keys >= N hold 0.
 *   v_scale  fp32  [B, H, d]   amax_c / V_r
 *   v_mean   fp32  [B, H, d]
 *   v_partial fp32 [B, H, N_pad/128, 3, d]   scratch (per-block sum, max, min)
 *   SAGE_PV_F16:
 *   v_codes  16-bit [B, H, d, N_pad]  V itself (the shape's dtype), channel-
 *            major.  Within every 32-key group starting at key 32g, element
 *            16m + 8h + 4a + r (m, h, a in {0,1}, r in 0..3) holds key
 *            32g + 16m + 8a + 4h + r.  Keys >= N hold 0.
 *   v_scale  fp32  [B, H, d]   1
 *   v_mean   fp32  [B, H, d]   0
 *   v_partial                  unused */
typedef struct {
  uint8_t* v_codes;
  float* v_scale;
  float* v_mean;
  float* v_partial;
} sage_v_buffers;

typedef struct {
  size_t offset; /* bytes from the start of the workspace (256-byte aligned) */
  size_t bytes;
} sage_span;

/* Byte layout of every intermediate buffer inside one workspace. */
typedef struct {
  int64_t n_pad, n_qblocks, q_groups, k_groups;
  sage_span q_codes, q_scale, q_mean, k_codes, k_scale, k_mean, bias, k_partial;
  sage_span v_codes, v_scale, v_mean, v_partial;
  size_t total_bytes;
} sage_layout;

/* Version of the buffer layouts and group maps (SAGE_ABI_VERSION). */
SAGE_API int sage_abi_version(void);

/* Fill *p with the defaults listed in sage_params. */
SAGE_API void sage_params_default(sage_params* p);

/* Host only.  Sizes and offsets of all intermediate buffers for this problem. */
SAGE_API sage_status sage_workspace_layout(const sage_shape* s, const sage_params* p, sage_layout* out);

/* Host only.  Point the buffer structs into a workspace laid out by
 * sage_workspace_layout (ws must be 256-byte aligned, ws_bytes >= total). */
SAGE_API sage_status sage_bind_workspace(const sage_layout* lay, void* ws, size_t ws_bytes,
                                         sage_qk_buffers* qk, sage_v_buffers* vb);

/* Smooth and quantize Q and K (SageAttention2 abstract: smoothing, INT4/INT8
 * Q and K; SageAttention2++ summary 2.1: per-block scales for Q and K).
 * Writes every field of *out (all must be non-NULL device pointers).
 * Codes, scales and means follow fp32 arithmetic with round-to-nearest-even
 * and a fixed pairwise summation tree in token order, so they are exactly
 * reproducible. */
SAGE_API sage_status sage_quant_qk(const void* q, const void* k, const sage_shape* s, const sage_params* p,
                                   const sage_qk_buffers* out, void* stream);

/* Smooth V by its token mean and encode V' to FP8 E4M3 with per-channel
 * scales (SageAttention2 abstract: FP8 V and V smoothing; SageAttention2++
 * summary 2.1: per-channel scaling of V). */
SAGE_API sage_status sage_quant_v(const void* v, const sage_shape* s, const sage_params* p,
                                  const sage_v_buffers* out, void* stream);

/* Attention on the quantized buffers (SageAttention2++ summary, "2.
 * Preliminary": FlashAttention-based tiled online softmax; INT8 matrix cores
 * for QK^T, FP8 matrix cores for P~V).  causal != 0 masks key j > query i.
 * o: [B, H, N, d] of the shape's dtype with element strides o_stride[0..2]
 * (multiples of 8, the N stride below 2^22; 16-byte aligned pointer). */
SAGE_API sage_status sage_attn_fwd(const sage_qk_buffers* qk, const sage_v_buffers* vb, const sage_shape* s,
                                   const sage_params* p, int causal, void* o, const int64_t o_stride[3],
                                   void* stream);

/* The plug-and-play call: sage_quant_qk, sage_quant_v and sage_attn_fwd in
 * order, with every intermediate buffer inside `workspace` (layout from
 * sage_workspace_layout; 256-byte aligned; ws_bytes >= total_bytes). */
SAGE_API sage_status sage_attn(const void* q, const void* k, const void* v, const sage_shape* s,
                               const sage_params* p, int causal, void* o, const int64_t o_stride[3],
                               void* workspace, size_t ws_bytes, void* stream);

/* Bytes of the library-held workspace of sage_attn_static (per GPU). */
#define SAGE_STATIC_WORKSPACE_BYTES (64u << 20)

/* sage_attn for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops and harnesses that forbid hipMalloc.
 * Arguments as sage_attn, without the workspace: every intermediate buffer
 * lives in a device array of SAGE_STATIC_WORKSPACE_BYTES that the library
 * holds on each GPU it runs on until the process ends (laid out as
 * sage_workspace_layout gives).  The caller still owns q, k, v and o.
 * Allocates nothing (no hipMalloc, hipFree or allocating library call).
 * Returns SAGE_EUNSUPPORTED, with nothing enqueued, when the layout's
 * total_bytes exceeds SAGE_STATIC_WORKSPACE_BYTES, and SAGE_EINVAL when a
 * non-NULL stream belongs to another device than the current one.  Every
 * call on a GPU shares that GPU's array and leaves its intermediates there:
 * calls that overlap on one GPU (other streams, other threads) race. */
SAGE_API sage_status sage_attn_static(const void* q, const void* k, const void* v, const sage_shape* s,
                                      const sage_params* p, int causal, void* o, const int64_t o_stride[3],
                                      void* stream);

/* ---- 8-bit training: the forward with its row log-sum-exp, and the backward ----
 * The SageAttention3 abstract (an 8-bit attention for forward and backward
 * propagation; no formats on the pages).  The readings, element by element:
 *   forward:  the method above; it also returns L_i = log2 sum_j 2^(s_ij) of
 *             its own log2-domain scores s (K smoothed, Q-smoothing bias
 *             added), so that P = 2^(s - L) is its softmax;
 *   backward: FlashAttention's formulas, D_i = sum_c dO_ic O_ic,
 *             dV = P^T dO, dP = dO V^T, dS = P o (dP - D), dQ = c dS K',
 *             dK = c dS^T Q (c = sm_scale, K' = K - mean(K); dS K = dS K'
 *             because each row of the exact dS sums to zero), every product
 *             on 8-bit operands with scales constant along its reduction axis:
 *             S from the forward's INT8 codes, scales and bias; dP in INT8
 *             (dO one scale per token, V one per 16-key group as the THREAD
 *             granularity's K groups; no smoothing); dV with P as E4M3 at the
 *             fixed scale 1/P_r and dO as E4M3 per channel; dQ and dK with dS
 *             as E4M3 under one power-of-two scale per 64-element group along
 *             the reduced axis (per query row and 64 keys for dQ, per key and
 *             64 queries for dK; the smallest 2^e with 448 2^e >= the group's
 *             max |dS|), K' and Q as E4M3 per channel.  Accumulation is fp32. */

/* sage_attn_fwd that also writes lse (float [B, H, N_pad], every padded row
 * included).  qk_format SAGE_QK_INT (qk_bits 8 or 4), _INT_E4M3 or _INT_E2M3
 * with SAGE_PV_FP8; other settings return SAGE_EUNSUPPORTED. */
SAGE_API sage_status sage_attn_fwd_lse(const sage_qk_buffers* qk, const sage_v_buffers* vb, const sage_shape* s,
                                       const sage_params* p, int causal, void* o, const int64_t o_stride[3],
                                       float* lse, void* stream);

/* Byte layout of the backward's intermediate buffers inside one workspace
 * (every span 256-byte aligned):
 *   do_codes int8 [B,H,N_pad,d], do_scale fp32 [B,H,N_pad], do_mean fp32
 *   [B,H,N_pad/128,d] (0): INT8 dO;  v_codes int8 [B,H,N_pad,d], v_scale fp32
 *   [B,H,N_pad/16], v_mean fp32 [B,H,d] (0), v_partial: INT8 V (the THREAD
 *   K-side groups) and its scratch;  do8_*, q8_*, k8_* as the FP8 V buffers of
 *   sage_v_buffers (codes uint8 [B,H,d,N_pad] in the permuted channel-major
 *   order, scale and mean fp32 [B,H,d]; k8 holds K' = K - mean(K) and its
 *   mean, do8 and q8 unsmoothed, means 0);  fp8_partial: their shared
 *   scratch;  dsum fp32 [B,H,N_pad]: D (0 past N);  lse_do and dsum_do
 *   fp32 [B,H,N_pad]: L - log2 s and D / s of each row with the row's INT8 dO
 *   scale s (+inf and 0 where s = 0), the dK kernel's per-row terms. */
typedef struct {
  int64_t n_pad;
  sage_span do_codes, do_scale, do_mean, v_codes, v_scale, v_mean, v_partial;
  sage_span do8_codes, do8_scale, do8_mean, q8_codes, q8_scale, q8_mean, k8_codes, k8_scale, k8_mean;
  sage_span fp8_partial, dsum, lse_do, dsum_do;
  size_t total_bytes;
} sage_bwd_layout;

/* Host only.  Layout of the backward workspace for this problem. */
SAGE_API sage_status sage_bwd_workspace_layout(const sage_shape* s, const sage_params* p, sage_bwd_layout* out);

/* The 8-bit backward.  q, k, v: the forward's inputs (shape s); o and dout:
 * the forward's output and its gradient, [B,H,N,d] of the shape's dtype with
 * element strides o_stride (shared by both); lse: from sage_attn_fwd_lse; qk:
 * the forward's sage_quant_qk buffers (same params).  Writes dq, dk, dv: fp32
 * [B,H,N,d], contiguous, 16-byte aligned.  Supported: qk_bits 8,
 * SAGE_GRAN_THREAD, SAGE_QK_INT, SAGE_PV_FP8 (else SAGE_EUNSUPPORTED).
 * workspace: 256-byte aligned, ws_bytes >= sage_bwd_workspace_layout's
 * total_bytes.  Enqueues kernels only. */
SAGE_API sage_status sage_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                   const int64_t o_stride[3], const float* lse, const sage_qk_buffers* qk,
                                   const sage_shape* s, const sage_params* p, int causal, float* dq, float* dk,
                                   float* dv, void* workspace, size_t ws_bytes, void* stream);

/* Result of sage_probe_qk_bits (host memory). */
typedef struct {
  double cos_int4, cos_int8;       /* cosine similarity with exact attention, over the probed rows */
  double rel_l1_int4, rel_l1_int8; /* relative L1 distance sum|O - O'| / sum|O| over the same rows */
  int32_t qk_bits;                 /* the choice: 4 if cos_int4 >= cos_min, else 8 */
  int32_t reserved;
} sage_probe_result;

/* Host only.  Bytes of device scratch sage_probe_qk_bits needs for this shape. */
SAGE_API sage_status sage_probe_scratch_bytes(const sage_shape* s, size_t* bytes);

/* Adaptive INT4/INT8 choice (SageAttention2 abstract: the QK precision is
 * picked per layer and timestep from measured accuracy; the metrics are those
 * of the SageAttention2++ summary, A.2).  On query block q_block (rows
 * 128 q_block .. 128 q_block + 127 that are < N) of every head it
 *   1. runs sage_quant_v, then the method with INT8 codes (qk_format
 *      SAGE_QK_INT) and with INT4-range codes (qk_bits 4, in p->qk_format:
 *      SAGE_QK_INT, _INT_E4M3 or _INT_E2M3), keeping both outputs in the I/O
 *      type;
 *   2. computes exact attention of the same rows in fp32 (fp32 dot products
 *      and online softmax, no quantisation, no smoothing);
 *   3. forms cosine similarity and relative L1 of each output against it over
 *      all probed rows of all heads (fp64 sums) and chooses INT4-range when
 *      cos_int4 >= cos_min.
 * On return *qk and *vb hold the quantisation for the chosen precision: call
 * sage_attn_fwd with p->qk_bits = result->qk_bits (and qk_format SAGE_QK_INT
 * when it is 8).  p->qk_bits is ignored; p->pv_mode must be SAGE_PV_FP8.
 * Blocks the calling thread until the sums are on the host (the stream is
 * synchronised).  Scratch layout (256-byte aligned spans, in order): the
 * exact rows fp32 [B, H, 128, d]; the INT4-range and the INT8 outputs,
 * [B, H, 128, d] of the I/O type; per-split partial rows; per-head and total
 * fp64 sums.  Rows past N are left unspecified in all of them. */
SAGE_API sage_status sage_probe_qk_bits(const void* q, const void* k, const void* v, const sage_shape* s,
                                        const sage_params* p, int causal, int64_t q_block, float cos_min,
                                        const sage_qk_buffers* qk, const sage_v_buffers* vb, void* scratch,
                                        size_t scratch_bytes, sage_probe_result* result, void* stream);

/* Static description of a status code. */
SAGE_API const char* sage_status_str(int status);

/* Thread-local message for the last failed call on this thread ("" if none). */
SAGE_API const char* sage_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SAGE_H_ */
