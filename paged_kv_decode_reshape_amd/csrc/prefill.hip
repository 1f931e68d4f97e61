// Prefill-chunk causal attention on MFMA (gfx950).
#include "device_common.h"
#include "kernels.h"

namespace pkv {

hipError_t launch_prefill(const PrefillParams& prm, hipStream_t stream, const KernelTimer& timer) {
  (void)prm;
  (void)stream;
  (void)timer;
  return hipErrorNotSupported;
}

}  // namespace pkv
