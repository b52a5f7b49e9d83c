// Paged prefill attention (MFMA path): not built yet in this revision.
#include "common.h"
#include "kernels.h"

namespace pkv {

bool prefill_supported(int, int, int, int) { return false; }

int launch_prefill(void*, const void*, const int32_t*, int, int, const void*, const void*, const int32_t*, int,
                   const int32_t*, int, int, int, int, int, int, float, hipStream_t) {
  return -2;
}

}  // namespace pkv
