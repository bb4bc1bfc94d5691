// Internal launch interface between the C ABI (sage_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sage.h"

namespace sage {

constexpr int kQBlock = 128;   // queries per attention work-group and per Q-mean block
constexpr int kKTile = 128;    // keys per attention tile (one online-softmax update)

struct TensorView {
  const void* ptr;
  int64_t sB, sH, sN;  // element strides
};

// Largest N stride (elements) of an input or output: the quantisation kernels
// address a 128-row block through a buffer resource with 32-bit byte offsets,
// and 128 rows of 2-byte elements then stay below 2^31 bytes.
constexpr int64_t kMaxRowStride = int64_t(1) << 22;

// Word 3 of every raw buffer resource here: 32-bit data format, no swizzle,
// no index stride (byte offsets; an access at or past the record count
// returns zeros).
constexpr int kBufferWord3 = 0x00020000;

struct Problem {
  int B, H, N, D, n_pad, nblk;   // nblk = n_pad / 128
  int bf16;                      // 1: bfloat16 inputs/outputs, 0: float16
  int qmax;
  int gran;                      // sage_gran
  int smooth_q, smooth_k, smooth_v;
  float p_range, v_range, sm_scale;
  int pv_f16;                    // 1: P~ and V in the 16-bit input type (SAGE_PV_F16)
  int qk_mx;                     // 1: MXFP4 Q and K codes (SAGE_QK_MXFP4)
  int qk_held;                   // INT4-range codes held as 1: E4M3 bytes (SAGE_QK_INT_E4M3), 2: packed
                                 // FP6 E2M3 (SAGE_QK_INT_E2M3); 0: int8
};

// Parts of sage_quant_qk to run; the default is all of it.  The parts left out
// keep what the buffers hold, which is only valid when an earlier call on the
// same inputs wrote them: the K means and the bias do not depend on the code
// precision (they come from the smoothed K and the Q block means).
struct QKPart {
  bool bias = true;      // the bias (needs k_codes)
  bool k_sums = true;    // the K block sums and K means (and then every Q block)
  bool k_codes = true;   // the K codes and scales
  int q_blk0 = 0;        // without k_sums: the Q blocks [q_blk0, q_blk0 + q_nblk)
  int q_nblk = 1 << 30;
};
hipError_t launch_quant_qk(const Problem& p, TensorView q, TensorView k, const sage_qk_buffers& out,
                           hipStream_t st, const QKPart& part = QKPart());
hipError_t launch_quant_v(const Problem& p, TensorView v, const sage_v_buffers& out, hipStream_t st);
// probe_qb >= 0 runs only query block probe_qb of every head (B*H work-groups)
// and writes query 128 probe_qb + r of a head to output row r ([B, H, 128, d]).
// lse, when not null, receives log2 sum_j 2^(s_ij) of every query row, float [B, H, n_pad].
hipError_t launch_attn_fwd(const Problem& p, const sage_qk_buffers& qk, const sage_v_buffers& vb, int causal,
                           void* o, const int64_t o_stride[3], hipStream_t st, int probe_qb = -1,
                           float* lse = nullptr);
// The same attention with MXFP4 Q and K codes on the scaled FP4 matrix cores (Problem::qk_mx).
hipError_t launch_attn_fp4(const Problem& p, const sage_qk_buffers& qk, const sage_v_buffers& vb, int causal,
                           void* o, const int64_t o_stride[3], hipStream_t st);
// The same attention with the 16-bit P~V product (Problem::pv_f16).
hipError_t launch_attn_pvh(const Problem& p, const sage_qk_buffers& qk, const sage_v_buffers& vb, int causal,
                           void* o, const int64_t o_stride[3], hipStream_t st);

// Buffers of the 8-bit backward (sage_attn_bwd).
struct BwdBuffers {
  sage_qk_buffers qk;     // the forward's quantisation: Q/K codes and scales, bias (S recompute)
  const float* lse;       // the forward's log2 sum_j 2^(s_ij), [B, H, n_pad]
  sage_qk_buffers dov;    // INT8 dO (query side) and V (key side), THREAD groups, no smoothing
  sage_v_buffers do8;     // E4M3 dO per channel (no smoothing)
  sage_v_buffers q8;      // E4M3 Q per channel (no smoothing)
  sage_v_buffers k8;      // E4M3 K' = K - mean(K) per channel
  float* dsum;            // D = rowsum(dO o O), [B, H, n_pad]
  float* lse_do;          // L - log2 s_dO per row (+inf where s_dO = 0), [B, H, n_pad]
  float* dsum_do;         // D / s_dO per row (0 where s_dO = 0), [B, H, n_pad]
  float* dq;
  float* dk;
  float* dv;              // fp32 [B, H, N, d], contiguous
};
// D of every padded row (0 past N), and the dK kernel's per-row terms from D,
// the forward's L and the INT8 dO scales (bb.dov.q_scale, written before);
// o and dout share the strides of `o`.
hipError_t launch_bwd_dsum(const Problem& p, TensorView o, TensorView dout, const BwdBuffers& bb, hipStream_t st);
// dQ (one work-group per query block) and dK, dV (one per key block).
hipError_t launch_attn_bwd(const Problem& p, const BwdBuffers& bb, int causal, hipStream_t st);

// Device address of the library-held workspace of sage_attn_static
// (SAGE_STATIC_WORKSPACE_BYTES, 256-byte aligned) on the current device, looked
// up once per device; *device receives the current device.
hipError_t static_workspace(void** ptr, int* device);

// Heads per longest-first group of a causal grid: as many heads (a power of
// two dividing the heads of one XCD, at most 8) as keep their streamed K/V
// bytes within 4 MiB, one XCD's L2.
inline int lpt_group(int heads, int64_t head_bytes) {
  if (heads % 8 != 0) return 1;
  const int per_xcd = heads / 8;
  int g = 1;
  while (g < 8 && per_xcd % (2 * g) == 0 && 2 * g * head_bytes <= (int64_t(4) << 20)) g *= 2;
  return g;
}

constexpr int kProbeRows = 128;   // rows of the probed query block
constexpr int kProbeSub = 8;      // split lengths of the probe's exact reference past 64 Ki keys are multiples of this

// Scratch of the adaptive INT4/INT8 probe (byte offsets, 256-byte aligned).
struct ProbeLayout {
  size_t ref, o4, o8, part, sums, total, bytes;
  int chunk, splits;   // keys per split of the exact reference, number of splits
};
ProbeLayout probe_layout(int B, int H, int N, int D, int io_bytes);
// Exact fp32 attention of query block q_block of every head into scratch + ref.
hipError_t launch_probe_reference(const Problem& p, TensorView q, TensorView k, TensorView v, int causal, int q_block,
                                  char* scratch, hipStream_t st);
// fp64 accuracy sums of the o4 and o8 outputs against ref into scratch + total.
hipError_t launch_probe_sums(const Problem& p, int q_block, char* scratch, hipStream_t st);

}  // namespace sage
