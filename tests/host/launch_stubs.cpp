// Host-only stand-ins for the kernel launchers, so that the C ABI's host
// logic (validation, layouts, binding) can be built with the address and
// undefined-behaviour sanitizers and exercised without a GPU.  Every stand-in
// reports an error: the tests that use this build never reach a launch.
#include "sage_internal.h"

namespace sage {

hipError_t launch_quant_qk(const Problem&, TensorView, TensorView, const sage_qk_buffers&, hipStream_t,
                           const QKPart&) { return hipErrorNotSupported; }
hipError_t launch_quant_v(const Problem&, TensorView, const sage_v_buffers&, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_attn_fwd(const Problem&, const sage_qk_buffers&, const sage_v_buffers&, int, void*,
                           const int64_t[3], hipStream_t, int, float*) { return hipErrorNotSupported; }
hipError_t launch_attn_fp4(const Problem&, const sage_qk_buffers&, const sage_v_buffers&, int, void*,
                           const int64_t[3], hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attn_pvh(const Problem&, const sage_qk_buffers&, const sage_v_buffers&, int, void*,
                           const int64_t[3], hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_probe_reference(const Problem&, TensorView, TensorView, TensorView, int, int, char*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_probe_sums(const Problem&, int, char*, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_dsum(const Problem&, TensorView, TensorView, const BwdBuffers&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attn_bwd(const Problem&, const BwdBuffers&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t static_workspace(void**, int*) { return hipErrorNotSupported; }

}  // namespace sage
