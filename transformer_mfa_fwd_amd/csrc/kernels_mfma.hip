// kernels_mfma.hip -- bf16/fp16 MFMA prefill kernel (in progress).
#include "mfa_internal.h"

namespace mfa {
bool mfma_prefill_supported(int, int) { return false; }
hipError_t launch_mfma_prefill(const FwdArgs&, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace mfa
