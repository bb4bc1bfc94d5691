// Host side of the C ABI declared in include/sage.h: argument validation,
// buffer layout and dispatch to the gfx950 kernels.  Every check runs before
// the first launch, so a call that fails has enqueued nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <initializer_list>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "sage.h"
#include "sage_internal.h"

namespace {

thread_local char g_err[512] = "";

sage_status fail(sage_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

sage_status ok() {
  g_err[0] = '\0';
  return SAGE_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

sage_status check_params(const sage_params* p) {
  if (!p) return fail(SAGE_EINVAL, "params is NULL");
  if (p->qk_bits != 8 && p->qk_bits != 4) return fail(SAGE_EUNSUPPORTED, "qk_bits must be 8 or 4 (got %d)", p->qk_bits);
  if (p->gran < SAGE_GRAN_THREAD || p->gran > SAGE_GRAN_BLOCK) return fail(SAGE_EINVAL, "unknown granularity %d", p->gran);
  for (int f : {p->smooth_q, p->smooth_k, p->smooth_v})
    if (f != 0 && f != 1) return fail(SAGE_EINVAL, "smoothing flags must be 0 or 1");
  if (!(p->p_range > 0.f && p->p_range <= 448.f)) return fail(SAGE_EINVAL, "p_range must be in (0, 448]");
  if (!(p->v_range > 0.f && p->v_range <= 448.f)) return fail(SAGE_EINVAL, "v_range must be in (0, 448]");
  if (!(p->sm_scale >= 0.f) || !std::isfinite(p->sm_scale)) return fail(SAGE_EINVAL, "sm_scale must be finite and >= 0");
  if (p->pv_mode != SAGE_PV_FP8 && p->pv_mode != SAGE_PV_F16) return fail(SAGE_EINVAL, "unknown pv_mode %d", p->pv_mode);
  if (p->qk_format != SAGE_QK_INT && p->qk_format != SAGE_QK_MXFP4 && p->qk_format != SAGE_QK_INT_E4M3 &&
      p->qk_format != SAGE_QK_INT_E2M3)
    return fail(SAGE_EINVAL, "unknown qk_format %d", p->qk_format);
  if (p->qk_format == SAGE_QK_MXFP4 && p->pv_mode != SAGE_PV_FP8)
    return fail(SAGE_EUNSUPPORTED, "SAGE_QK_MXFP4 is built with SAGE_PV_FP8 only");
  const bool held = p->qk_format == SAGE_QK_INT_E4M3 || p->qk_format == SAGE_QK_INT_E2M3;
  if (held && p->qk_bits != 4)
    return fail(SAGE_EINVAL, "SAGE_QK_INT_E4M3 / _E2M3 hold INT4-range codes: qk_bits must be 4 (got %d)", p->qk_bits);
  if (held && p->pv_mode != SAGE_PV_FP8)
    return fail(SAGE_EUNSUPPORTED, "SAGE_QK_INT_E4M3 / _E2M3 are built with SAGE_PV_FP8 only");
  return SAGE_OK;
}

sage_status check_shape(const sage_shape* s) {
  if (!s) return fail(SAGE_EINVAL, "shape is NULL");
  if (s->B < 1 || s->H < 1) return fail(SAGE_EINVAL, "B and H must be >= 1");
  if (s->B * s->H > 65535) return fail(SAGE_EUNSUPPORTED, "B*H must be <= 65535");
  if (s->N < 1 || s->N > (1 << 20)) return fail(SAGE_EUNSUPPORTED, "N must be in [1, 2^20] (got %lld)", (long long)s->N);
  if (s->d != 64 && s->d != 128) return fail(SAGE_EUNSUPPORTED, "head dim d must be 64 or 128 (got %lld)", (long long)s->d);
  if (s->dtype != SAGE_F16 && s->dtype != SAGE_BF16) return fail(SAGE_EINVAL, "dtype must be SAGE_F16 or SAGE_BF16");
  const int64_t* st[3] = {s->q_stride, s->k_stride, s->v_stride};
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j)
      if (st[i][j] <= 0 || st[i][j] % 8 != 0) return fail(SAGE_EINVAL, "strides must be positive multiples of 8 elements");
  for (int i = 0; i < 3; ++i)
    if (st[i][2] >= sage::kMaxRowStride)
      return fail(SAGE_EUNSUPPORTED, "N strides must be below 2^22 elements (got %lld)", (long long)st[i][2]);
  return SAGE_OK;
}

sage::Problem make_problem(const sage_shape* s, const sage_params* p) {
  sage::Problem pr;
  pr.B = static_cast<int>(s->B);
  pr.H = static_cast<int>(s->H);
  pr.N = static_cast<int>(s->N);
  pr.D = static_cast<int>(s->d);
  pr.n_pad = static_cast<int>((s->N + 127) / 128 * 128);
  pr.nblk = pr.n_pad / 128;
  pr.bf16 = s->dtype == SAGE_BF16;
  pr.qmax = p->qk_bits == 8 ? 127 : 7;
  pr.gran = p->gran;
  pr.smooth_q = p->smooth_q;
  pr.smooth_k = p->smooth_k;
  pr.smooth_v = p->smooth_v;
  pr.p_range = p->p_range;
  pr.v_range = p->v_range;
  pr.sm_scale = p->sm_scale > 0.f ? p->sm_scale : 1.0f / std::sqrt(static_cast<float>(s->d));
  pr.pv_f16 = p->pv_mode == SAGE_PV_F16;
  pr.qk_mx = p->qk_format == SAGE_QK_MXFP4;
  pr.qk_held = p->qk_format == SAGE_QK_INT_E4M3 ? 1 : (p->qk_format == SAGE_QK_INT_E2M3 ? 2 : 0);
  return pr;
}

sage_status check_qk_buffers(const sage_qk_buffers* b) {
  if (!b) return fail(SAGE_EINVAL, "qk buffers is NULL");
  const void* ptrs[] = {b->q_codes, b->q_scale, b->q_mean, b->k_codes, b->k_scale, b->k_mean, b->bias, b->k_partial};
  for (const void* q : ptrs) {
    if (!q) return fail(SAGE_EINVAL, "a qk buffer pointer is NULL");
    if (!aligned(q, 16)) return fail(SAGE_EINVAL, "qk buffers must be 16-byte aligned");
  }
  return SAGE_OK;
}

sage_status check_v_buffers(const sage_v_buffers* b) {
  if (!b) return fail(SAGE_EINVAL, "v buffers is NULL");
  const void* ptrs[] = {b->v_codes, b->v_scale, b->v_mean, b->v_partial};
  for (const void* q : ptrs) {
    if (!q) return fail(SAGE_EINVAL, "a v buffer pointer is NULL");
    if (!aligned(q, 16)) return fail(SAGE_EINVAL, "v buffers must be 16-byte aligned");
  }
  return SAGE_OK;
}

sage_status check_tensor(const void* p, const char* name) {
  if (!p) return fail(SAGE_EINVAL, "%s is NULL", name);
  if (!aligned(p, 16)) return fail(SAGE_EINVAL, "%s must be 16-byte aligned", name);
  return SAGE_OK;
}

sage_status check_out(const void* o, const int64_t* os) {
  sage_status st = check_tensor(o, "o");
  if (st) return st;
  if (!os) return fail(SAGE_EINVAL, "o_stride is NULL");
  for (int j = 0; j < 3; ++j)
    if (os[j] <= 0 || os[j] % 8 != 0) return fail(SAGE_EINVAL, "o strides must be positive multiples of 8 elements");
  if (os[2] >= sage::kMaxRowStride) return fail(SAGE_EUNSUPPORTED, "the o N stride must be below 2^22 elements");
  return SAGE_OK;
}

sage_status launch_result(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SAGE_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

SAGE_API int sage_abi_version(void) { return SAGE_ABI_VERSION; }

SAGE_API void sage_params_default(sage_params* p) {
  if (!p) return;
  p->qk_bits = 8;
  p->gran = SAGE_GRAN_THREAD;
  p->smooth_q = 1;
  p->smooth_k = 1;
  p->smooth_v = 1;
  p->p_range = 448.f;
  p->v_range = 448.f;
  p->sm_scale = 0.f;
  p->pv_mode = SAGE_PV_FP8;
  p->qk_format = SAGE_QK_INT;
}

SAGE_API sage_status sage_workspace_layout(const sage_shape* s, const sage_params* p, sage_layout* out) {
  sage_status st;
  if ((st = check_shape(s)) || (st = check_params(p))) return st;
  if (!out) return fail(SAGE_EINVAL, "layout output is NULL");
  const int64_t BH = s->B * s->H, D = s->d;
  const int64_t n_pad = (s->N + 127) / 128 * 128, nblk = n_pad / 128;
  const bool mx = p->qk_format == SAGE_QK_MXFP4;
  // integer codes: groups of fp32 scales; MXFP4: one scale byte per 32 channels of a token
  const int64_t gq = mx ? n_pad * D / 32 : (p->gran == SAGE_GRAN_THREAD ? n_pad : (p->gran == SAGE_GRAN_WARP ? n_pad / 32 : nblk));
  const int64_t gk = mx ? n_pad * D / 32 : (p->gran == SAGE_GRAN_THREAD ? n_pad / 16 : n_pad / 64);
  const int64_t code_bytes = mx ? n_pad * D / 2 : n_pad * D;
  const int64_t scale_bytes = mx ? 1 : 4;
  sage_layout L;
  memset(&L, 0, sizeof(L));
  L.n_pad = n_pad;
  L.n_qblocks = nblk;
  L.q_groups = gq;
  L.k_groups = gk;
  size_t off = 0;
  auto put = [&](sage_span& sp, int64_t bytes) {
    sp.offset = off;
    sp.bytes = static_cast<size_t>(bytes);
    off = round_up(off + sp.bytes, 256);
  };
  put(L.q_codes, BH * code_bytes);
  put(L.q_scale, BH * gq * scale_bytes);
  put(L.q_mean, BH * nblk * D * 4);
  put(L.k_codes, BH * code_bytes);
  put(L.k_scale, BH * gk * scale_bytes);
  put(L.k_mean, BH * D * 4);
  put(L.bias, BH * nblk * n_pad * 4);
  put(L.k_partial, BH * nblk * D * 4);
  put(L.v_codes, BH * D * n_pad * (p->pv_mode == SAGE_PV_F16 ? 2 : 1));
  put(L.v_scale, BH * D * 4);
  put(L.v_mean, BH * D * 4);
  put(L.v_partial, BH * nblk * 3 * D * 4);
  L.total_bytes = off;
  *out = L;
  return ok();
}

SAGE_API sage_status sage_bind_workspace(const sage_layout* L, void* ws, size_t ws_bytes, sage_qk_buffers* qk,
                                         sage_v_buffers* vb) {
  if (!L || !qk || !vb) return fail(SAGE_EINVAL, "NULL argument");
  if (!ws) return fail(SAGE_EINVAL, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(SAGE_EINVAL, "workspace must be 256-byte aligned");
  if (ws_bytes < L->total_bytes)
    return fail(SAGE_EINVAL, "workspace too small: %zu < %zu bytes", ws_bytes, L->total_bytes);
  char* base = static_cast<char*>(ws);
  qk->q_codes = reinterpret_cast<int8_t*>(base + L->q_codes.offset);
  qk->q_scale = reinterpret_cast<float*>(base + L->q_scale.offset);
  qk->q_mean = reinterpret_cast<float*>(base + L->q_mean.offset);
  qk->k_codes = reinterpret_cast<int8_t*>(base + L->k_codes.offset);
  qk->k_scale = reinterpret_cast<float*>(base + L->k_scale.offset);
  qk->k_mean = reinterpret_cast<float*>(base + L->k_mean.offset);
  qk->bias = reinterpret_cast<float*>(base + L->bias.offset);
  qk->k_partial = reinterpret_cast<float*>(base + L->k_partial.offset);
  vb->v_codes = reinterpret_cast<uint8_t*>(base + L->v_codes.offset);
  vb->v_scale = reinterpret_cast<float*>(base + L->v_scale.offset);
  vb->v_mean = reinterpret_cast<float*>(base + L->v_mean.offset);
  vb->v_partial = reinterpret_cast<float*>(base + L->v_partial.offset);
  return ok();
}

SAGE_API sage_status sage_quant_qk(const void* q, const void* k, const sage_shape* s, const sage_params* p,
                                   const sage_qk_buffers* out, void* stream) {
  sage_status st;
  if ((st = check_shape(s)) || (st = check_params(p)) || (st = check_tensor(q, "q")) || (st = check_tensor(k, "k")) ||
      (st = check_qk_buffers(out)))
    return st;
  const sage::Problem pr = make_problem(s, p);
  const sage::TensorView qv{q, s->q_stride[0], s->q_stride[1], s->q_stride[2]};
  const sage::TensorView kv{k, s->k_stride[0], s->k_stride[1], s->k_stride[2]};
  return launch_result(sage::launch_quant_qk(pr, qv, kv, *out, static_cast<hipStream_t>(stream)), "sage_quant_qk");
}

SAGE_API sage_status sage_quant_v(const void* v, const sage_shape* s, const sage_params* p, const sage_v_buffers* out,
                                  void* stream) {
  sage_status st;
  if ((st = check_shape(s)) || (st = check_params(p)) || (st = check_tensor(v, "v")) || (st = check_v_buffers(out)))
    return st;
  const sage::Problem pr = make_problem(s, p);
  const sage::TensorView vv{v, s->v_stride[0], s->v_stride[1], s->v_stride[2]};
  return launch_result(sage::launch_quant_v(pr, vv, *out, static_cast<hipStream_t>(stream)), "sage_quant_v");
}

SAGE_API sage_status sage_attn_fwd(const sage_qk_buffers* qk, const sage_v_buffers* vb, const sage_shape* s,
                                   const sage_params* p, int causal, void* o, const int64_t o_stride[3],
                                   void* stream) {
  sage_status st;
  if ((st = check_shape(s)) || (st = check_params(p)) || (st = check_qk_buffers(qk)) || (st = check_v_buffers(vb)) ||
      (st = check_out(o, o_stride)))
    return st;
  if (causal != 0 && causal != 1) return fail(SAGE_EINVAL, "causal must be 0 or 1");
  const sage::Problem pr = make_problem(s, p);
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  return launch_result(pr.qk_mx    ? sage::launch_attn_fp4(pr, *qk, *vb, causal, o, o_stride, hs)
                       : pr.pv_f16 ? sage::launch_attn_pvh(pr, *qk, *vb, causal, o, o_stride, hs)
                                   : sage::launch_attn_fwd(pr, *qk, *vb, causal, o, o_stride, hs),
                       "sage_attn_fwd");
}

SAGE_API sage_status sage_attn(const void* q, const void* k, const void* v, const sage_shape* s, const sage_params* p,
                               int causal, void* o, const int64_t o_stride[3], void* workspace, size_t ws_bytes,
                               void* stream) {
  sage_status st;
  sage_layout L;
  if ((st = sage_workspace_layout(s, p, &L))) return st;
  if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k")) || (st = check_tensor(v, "v")) ||
      (st = check_out(o, o_stride)))
    return st;
  if (causal != 0 && causal != 1) return fail(SAGE_EINVAL, "causal must be 0 or 1");
  sage_qk_buffers qk;
  sage_v_buffers vb;
  if ((st = sage_bind_workspace(&L, workspace, ws_bytes, &qk, &vb))) return st;
  if ((st = sage_quant_qk(q, k, s, p, &qk, stream))) return st;
  if ((st = sage_quant_v(v, s, p, &vb, stream))) return st;
  return sage_attn_fwd(&qk, &vb, s, p, causal, o, o_stride, stream);
}

SAGE_API sage_status sage_attn_fwd_lse(const sage_qk_buffers* qk, const sage_v_buffers* vb, const sage_shape* s,
                                       const sage_params* p, int causal, void* o, const int64_t o_stride[3],
                                       float* lse, void* stream) {
  sage_status st;
  if ((st = check_shape(s)) || (st = check_params(p)) || (st = check_qk_buffers(qk)) || (st = check_v_buffers(vb)) ||
      (st = check_out(o, o_stride)) || (st = check_tensor(lse, "lse")))
    return st;
  if (causal != 0 && causal != 1) return fail(SAGE_EINVAL, "causal must be 0 or 1");
  if (p->qk_format == SAGE_QK_MXFP4 || p->pv_mode != SAGE_PV_FP8)
    return fail(SAGE_EUNSUPPORTED, "sage_attn_fwd_lse needs integer Q/K codes and SAGE_PV_FP8");
  const sage::Problem pr = make_problem(s, p);
  return launch_result(sage::launch_attn_fwd(pr, *qk, *vb, causal, o, o_stride, static_cast<hipStream_t>(stream),
                                             -1, lse),
                       "sage_attn_fwd_lse");
}

SAGE_API sage_status sage_bwd_workspace_layout(const sage_shape* s, const sage_params* p, sage_bwd_layout* out) {
  sage_status st;
  if ((st = check_shape(s)) || (st = check_params(p))) return st;
  if (!out) return fail(SAGE_EINVAL, "layout output is NULL");
  const int64_t BH = s->B * s->H, D = s->d;
  const int64_t n_pad = (s->N + 127) / 128 * 128, nblk = n_pad / 128;
  sage_bwd_layout L;
  memset(&L, 0, sizeof(L));
  L.n_pad = n_pad;
  size_t off = 0;
  auto put = [&](sage_span& sp, int64_t bytes) {
    sp.offset = off;
    sp.bytes = static_cast<size_t>(bytes);
    off = round_up(off + sp.bytes, 256);
  };
  put(L.do_codes, BH * n_pad * D);
  put(L.do_scale, BH * n_pad * 4);
  put(L.do_mean, BH * nblk * D * 4);
  put(L.v_codes, BH * n_pad * D);
  put(L.v_scale, BH * (n_pad / 16) * 4);
  put(L.v_mean, BH * D * 4);
  put(L.v_partial, BH * nblk * D * 4);
  put(L.do8_codes, BH * D * n_pad);
  put(L.do8_scale, BH * D * 4);
  put(L.do8_mean, BH * D * 4);
  put(L.q8_codes, BH * D * n_pad);
  put(L.q8_scale, BH * D * 4);
  put(L.q8_mean, BH * D * 4);
  put(L.k8_codes, BH * D * n_pad);
  put(L.k8_scale, BH * D * 4);
  put(L.k8_mean, BH * D * 4);
  put(L.fp8_partial, BH * nblk * 3 * D * 4);
  put(L.dsum, BH * n_pad * 4);
  put(L.lse_do, BH * n_pad * 4);
  put(L.dsum_do, BH * n_pad * 4);
  L.total_bytes = off;
  *out = L;
  return ok();
}

SAGE_API sage_status sage_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                   const int64_t o_stride[3], const float* lse, const sage_qk_buffers* qk,
                                   const sage_shape* s, const sage_params* p, int causal, float* dq, float* dk,
                                   float* dv, void* workspace, size_t ws_bytes, void* stream) {
  sage_status st;
  sage_bwd_layout L;
  if ((st = sage_bwd_workspace_layout(s, p, &L))) return st;
  if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k")) || (st = check_tensor(v, "v")) ||
      (st = check_out(o, o_stride)) || (st = check_tensor(dout, "dout")) || (st = check_tensor(lse, "lse")) ||
      (st = check_qk_buffers(qk)) || (st = check_tensor(dq, "dq")) || (st = check_tensor(dk, "dk")) ||
      (st = check_tensor(dv, "dv")))
    return st;
  if (causal != 0 && causal != 1) return fail(SAGE_EINVAL, "causal must be 0 or 1");
  if (p->qk_bits != 8 || p->gran != SAGE_GRAN_THREAD || p->qk_format != SAGE_QK_INT || p->pv_mode != SAGE_PV_FP8)
    return fail(SAGE_EUNSUPPORTED,
                "sage_attn_bwd needs qk_bits 8, SAGE_GRAN_THREAD, SAGE_QK_INT and SAGE_PV_FP8");
  if (!workspace || !aligned(workspace, 256)) return fail(SAGE_EINVAL, "workspace must be a 256-byte aligned pointer");
  if (ws_bytes < L.total_bytes)
    return fail(SAGE_EINVAL, "workspace too small: %zu < %zu bytes", ws_bytes, L.total_bytes);

  const sage::Problem pr = make_problem(s, p);
  char* base = static_cast<char*>(workspace);
  auto at = [&](const sage_span& sp) { return base + sp.offset; };
  sage::BwdBuffers bb;
  bb.qk = *qk;
  bb.lse = lse;
  bb.dov.q_codes = reinterpret_cast<int8_t*>(at(L.do_codes));
  bb.dov.q_scale = reinterpret_cast<float*>(at(L.do_scale));
  bb.dov.q_mean = reinterpret_cast<float*>(at(L.do_mean));
  bb.dov.k_codes = reinterpret_cast<int8_t*>(at(L.v_codes));
  bb.dov.k_scale = reinterpret_cast<float*>(at(L.v_scale));
  bb.dov.k_mean = reinterpret_cast<float*>(at(L.v_mean));
  bb.dov.bias = nullptr;                  // not written: the INT8 dO / V pass has no bias
  bb.dov.k_partial = reinterpret_cast<float*>(at(L.v_partial));
  float* fp8_partial = reinterpret_cast<float*>(at(L.fp8_partial));
  bb.do8 = {reinterpret_cast<uint8_t*>(at(L.do8_codes)), reinterpret_cast<float*>(at(L.do8_scale)),
            reinterpret_cast<float*>(at(L.do8_mean)), fp8_partial};
  bb.q8 = {reinterpret_cast<uint8_t*>(at(L.q8_codes)), reinterpret_cast<float*>(at(L.q8_scale)),
           reinterpret_cast<float*>(at(L.q8_mean)), fp8_partial};
  bb.k8 = {reinterpret_cast<uint8_t*>(at(L.k8_codes)), reinterpret_cast<float*>(at(L.k8_scale)),
           reinterpret_cast<float*>(at(L.k8_mean)), fp8_partial};
  bb.dsum = reinterpret_cast<float*>(at(L.dsum));
  bb.lse_do = reinterpret_cast<float*>(at(L.lse_do));
  bb.dsum_do = reinterpret_cast<float*>(at(L.dsum_do));
  bb.dq = dq;
  bb.dk = dk;
  bb.dv = dv;

  // INT8 dO (query side) and V (key side): the Q/K quantiser with the THREAD
  // groups and no smoothing, without the bias.
  sage::Problem pi = pr;
  pi.smooth_q = 0;
  pi.smooth_k = 0;
  pi.qmax = 127;
  pi.gran = SAGE_GRAN_THREAD;
  pi.qk_held = 0;
  pi.qk_mx = 0;
  sage::QKPart no_bias;
  no_bias.bias = false;
  // E4M3 per channel: the V quantiser at V_r = 448, smoothing only for K.
  sage::Problem pc = pr;
  pc.v_range = 448.f;
  pc.pv_f16 = 0;
  pc.smooth_v = 0;
  sage::Problem pk = pc;
  pk.smooth_v = 1;
  const sage::TensorView qv{q, s->q_stride[0], s->q_stride[1], s->q_stride[2]};
  const sage::TensorView kv{k, s->k_stride[0], s->k_stride[1], s->k_stride[2]};
  const sage::TensorView vv{v, s->v_stride[0], s->v_stride[1], s->v_stride[2]};
  const sage::TensorView ov{o, o_stride[0], o_stride[1], o_stride[2]};
  const sage::TensorView dov{dout, o_stride[0], o_stride[1], o_stride[2]};
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e;
  if ((e = sage::launch_quant_qk(pi, dov, vv, bb.dov, hs, no_bias)) != hipSuccess ||
      (e = sage::launch_quant_v(pc, dov, bb.do8, hs)) != hipSuccess ||
      (e = sage::launch_quant_v(pc, qv, bb.q8, hs)) != hipSuccess ||
      (e = sage::launch_quant_v(pk, kv, bb.k8, hs)) != hipSuccess ||
      (e = sage::launch_bwd_dsum(pr, ov, dov, bb, hs)) != hipSuccess)
    return launch_result(e, "sage_attn_bwd (operands)");
  return launch_result(sage::launch_attn_bwd(pr, bb, causal, hs), "sage_attn_bwd");
}

SAGE_API sage_status sage_attn_static(const void* q, const void* k, const void* v, const sage_shape* s,
                                      const sage_params* p, int causal, void* o, const int64_t o_stride[3],
                                      void* stream) {
  sage_status st;
  sage_layout L;
  if ((st = sage_workspace_layout(s, p, &L))) return st;
  if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k")) || (st = check_tensor(v, "v")) ||
      (st = check_out(o, o_stride)))
    return st;
  if (causal != 0 && causal != 1) return fail(SAGE_EINVAL, "causal must be 0 or 1");
  if (L.total_bytes > SAGE_STATIC_WORKSPACE_BYTES)
    return fail(SAGE_EUNSUPPORTED, "the problem needs a %zu-byte workspace; the static one holds %zu bytes",
                L.total_bytes, static_cast<size_t>(SAGE_STATIC_WORKSPACE_BYTES));
  void* ws = nullptr;
  int dev = -1;
  hipError_t e = sage::static_workspace(&ws, &dev);
  if (e != hipSuccess) return launch_result(e, "sage_attn_static (workspace address)");
  if (stream) {
    int sdev = -1;
    if ((e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev)) != hipSuccess)
      return launch_result(e, "sage_attn_static (stream device)");
    if (sdev != dev) return fail(SAGE_EINVAL, "the stream belongs to device %d, the current device is %d", sdev, dev);
  }
  return sage_attn(q, k, v, s, p, causal, o, o_stride, ws, SAGE_STATIC_WORKSPACE_BYTES, stream);
}

SAGE_API sage_status sage_probe_scratch_bytes(const sage_shape* s, size_t* bytes) {
  sage_status st;
  if ((st = check_shape(s))) return st;
  if (!bytes) return fail(SAGE_EINVAL, "bytes is NULL");
  *bytes = sage::probe_layout(static_cast<int>(s->B), static_cast<int>(s->H), static_cast<int>(s->N),
                              static_cast<int>(s->d), 2).bytes;
  return ok();
}

SAGE_API sage_status sage_probe_qk_bits(const void* q, const void* k, const void* v, const sage_shape* s,
                                        const sage_params* p, int causal, int64_t q_block, float cos_min,
                                        const sage_qk_buffers* qk, const sage_v_buffers* vb, void* scratch,
                                        size_t scratch_bytes, sage_probe_result* result, void* stream) {
  sage_status st;
  if (!p) return fail(SAGE_EINVAL, "params is NULL");
  if (p->qk_format == SAGE_QK_MXFP4)
    return fail(SAGE_EUNSUPPORTED, "the probe compares integer codes: qk_format must not be SAGE_QK_MXFP4");
  if (p->pv_mode != SAGE_PV_FP8) return fail(SAGE_EUNSUPPORTED, "the probe runs with SAGE_PV_FP8");
  // p->qk_bits is ignored: the two passes use 8 (SAGE_QK_INT) and 4 (p->qk_format)
  sage_params p8 = *p, p4 = *p;
  p8.qk_bits = 8;
  p8.qk_format = SAGE_QK_INT;
  p4.qk_bits = 4;
  if ((st = check_shape(s)) || (st = check_params(&p8)) || (st = check_params(&p4)) || (st = check_tensor(q, "q")) ||
      (st = check_tensor(k, "k")) || (st = check_tensor(v, "v")) || (st = check_qk_buffers(qk)) ||
      (st = check_v_buffers(vb)))
    return st;
  if (causal != 0 && causal != 1) return fail(SAGE_EINVAL, "causal must be 0 or 1");
  const int64_t nblk = (s->N + 127) / 128;
  if (q_block < 0 || q_block >= nblk)
    return fail(SAGE_EINVAL, "q_block must be in [0, %lld) (got %lld)", (long long)nblk, (long long)q_block);
  if (!std::isfinite(cos_min)) return fail(SAGE_EINVAL, "cos_min must be finite");
  if (!result) return fail(SAGE_EINVAL, "result is NULL");
  if (!scratch || !aligned(scratch, 256)) return fail(SAGE_EINVAL, "scratch must be a 256-byte aligned pointer");
  const sage::ProbeLayout PL = sage::probe_layout(static_cast<int>(s->B), static_cast<int>(s->H),
                                                  static_cast<int>(s->N), static_cast<int>(s->d), 2);
  if (scratch_bytes < PL.bytes) return fail(SAGE_EINVAL, "scratch too small: %zu < %zu bytes", scratch_bytes, PL.bytes);

  const sage::Problem pr8 = make_problem(s, &p8), pr4 = make_problem(s, &p4);
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const sage::TensorView qv{q, s->q_stride[0], s->q_stride[1], s->q_stride[2]};
  const sage::TensorView kv{k, s->k_stride[0], s->k_stride[1], s->k_stride[2]};
  const sage::TensorView vv{v, s->v_stride[0], s->v_stride[1], s->v_stride[2]};
  char* base = static_cast<char*>(scratch);
  // outputs [B, H, 128, d]: the probe instantiation writes query q0 + r of the
  // block to row r of its head
  const int64_t D = s->d;
  const int64_t os[3] = {s->H * 128 * D, 128 * D, D};
  void* o4 = base + PL.o4;
  void* o8 = base + PL.o8;
  const int qb = static_cast<int>(q_block);
  hipError_t e;
  if ((e = sage::launch_quant_v(pr8, vv, *vb, hs)) != hipSuccess) return launch_result(e, "sage_probe_qk_bits (quant_v)");
  if ((e = sage::launch_quant_qk(pr8, qv, kv, *qk, hs)) != hipSuccess ||
      (e = sage::launch_attn_fwd(pr8, *qk, *vb, causal, o8, os, hs, qb)) != hipSuccess)
    return launch_result(e, "sage_probe_qk_bits (INT8 pass)");
  // The INT4-range pass needs new K codes and the probed Q block's codes only:
  // the K means and the bias do not depend on the precision, and the INT8
  // pass's stay valid.
  sage::QKPart block_only;
  block_only.bias = false;
  block_only.k_sums = false;
  block_only.q_blk0 = qb;
  block_only.q_nblk = 1;
  if ((e = sage::launch_quant_qk(pr4, qv, kv, *qk, hs, block_only)) != hipSuccess ||
      (e = sage::launch_attn_fwd(pr4, *qk, *vb, causal, o4, os, hs, qb)) != hipSuccess)
    return launch_result(e, "sage_probe_qk_bits (INT4-range pass)");
  if ((e = sage::launch_probe_reference(pr8, qv, kv, vv, causal, qb, base, hs)) != hipSuccess ||
      (e = sage::launch_probe_sums(pr8, qb, base, hs)) != hipSuccess)
    return launch_result(e, "sage_probe_qk_bits (reference)");
  double sums[8];
  if ((e = hipMemcpyAsync(sums, base + PL.total, sizeof(sums), hipMemcpyDeviceToHost, hs)) != hipSuccess ||
      (e = hipStreamSynchronize(hs)) != hipSuccess)
    return launch_result(e, "sage_probe_qk_bits (sums)");
  // sums: <o4,r>, |o4|^2, <o8,r>, |o8|^2, |r|^2, |o4-r|_1, |o8-r|_1, |r|_1
  sage_probe_result r;
  memset(&r, 0, sizeof(r));
  r.cos_int4 = sums[0] / std::sqrt(sums[1] * sums[4]);
  r.cos_int8 = sums[2] / std::sqrt(sums[3] * sums[4]);
  r.rel_l1_int4 = sums[5] / sums[7];
  r.rel_l1_int8 = sums[6] / sums[7];
  r.qk_bits = r.cos_int4 >= static_cast<double>(cos_min) ? 4 : 8;
  // Leave the chosen precision's codes: INT8 needs its K codes and the probed
  // Q block back; INT4-range needs the Q codes of every block.
  sage::QKPart rest = block_only;
  if (r.qk_bits == 4) {
    rest.k_codes = false;
    rest.q_blk0 = 0;
    rest.q_nblk = 1 << 30;
  }
  if ((e = sage::launch_quant_qk(r.qk_bits == 8 ? pr8 : pr4, qv, kv, *qk, hs, rest)) != hipSuccess)
    return launch_result(e, "sage_probe_qk_bits (chosen codes)");
  *result = r;
  return ok();
}

SAGE_API const char* sage_status_str(int status) {
  switch (status) {
    case SAGE_OK: return "ok";
    case SAGE_EINVAL: return "invalid argument";
    case SAGE_EUNSUPPORTED: return "unsupported";
    case SAGE_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

SAGE_API const char* sage_last_error(void) { return g_err; }

}  // extern "C"
