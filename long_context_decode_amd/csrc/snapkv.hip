// SnapKV prefill compression kernels (placeholder until the MFMA scorer lands).
#include <hip/hip_runtime.h>

#include "lcd_internal.h"

namespace lcd {

size_t snapkv_ws_bytes(int B, int H, int N, int Lobs) {
  (void)B; (void)H; (void)N; (void)Lobs;
  return 256;
}

hipError_t launch_snapkv(const SnapkvParams& p, hipStream_t s) {
  (void)p; (void)s;
  return hipErrorNotSupported;
}

}  // namespace lcd
