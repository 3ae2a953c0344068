// kernels_decode.hip -- Lq = 1 split-over-keys decode and combine (in progress).
#include "mfa_internal.h"

namespace mfa {
bool split_decode_supported(int, int, int, int) { return false; }
int split_decode_default_splits(int, int, int, int) { return 1; }
size_t split_decode_workspace_bytes(int B, int Hq, int D, int splits) {
    return (size_t)B * Hq * splits * (D + 2) * sizeof(float);
}
hipError_t launch_split_decode(const FwdArgs&, int, int, float*, hipStream_t) { return hipErrorNotSupported; }
}  // namespace mfa
