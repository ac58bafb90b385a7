// Launchers whose kernels are not written yet.
#include "tsa_internal.h"

namespace tsa {
hipError_t launch_nsa_fwd(const NsaParams&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_nsa_bwd(const NsaParams&, int, hipStream_t, void* const*, int) { return hipErrorNotSupported; }
int sfa_splits(const SfaParams&) { return 1; }
hipError_t launch_sfa_fwd(const SfaParams&, int, hipStream_t, void* const*, int) { return hipErrorNotSupported; }
hipError_t launch_sfa_check(const SfaParams&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace tsa
