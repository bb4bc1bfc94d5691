// Host-only layout arithmetic shared by the C ABI and the kernels' launchers.
#include "sage_internal.h"

namespace sage {
namespace {

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

ProbeLayout probe_layout(int B, int H, int N, int D, int io_bytes) {
  ProbeLayout L;
  const int64_t BH = static_cast<int64_t>(B) * H;
  const int n_pad = (N + 127) / 128 * 128;
  // at most 64 key splits (a split's last sub-tile may be partly past its end, masked)
  L.chunk = n_pad <= 64 * 1024 ? 1024 : ((n_pad + 63) / 64 + kProbeSub - 1) / kProbeSub * kProbeSub;
  L.splits = (n_pad + L.chunk - 1) / L.chunk;
  size_t off = 0;
  L.ref = off;  off = align256(off + BH * kProbeRows * D * 4);
  L.o4 = off;   off = align256(off + BH * kProbeRows * D * io_bytes);
  L.o8 = off;   off = align256(off + BH * kProbeRows * D * io_bytes);
  L.part = off; off = align256(off + static_cast<size_t>(L.splits) * BH * kProbeRows * (D + 2) * 4);
  L.sums = off; off = align256(off + BH * 8 * 8);
  L.total = off; off = align256(off + 8 * 8);
  L.bytes = off;
  return L;
}

}  // namespace sage
