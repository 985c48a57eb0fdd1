// Host-only stand-ins for the device launchers of libgdn, so that the C ABI shim
// (gdn_abi.cpp) can be built with AddressSanitizer and UndefinedBehaviorSanitizer
// and driven on a machine without a GPU.  Every launcher counts its calls and
// returns an error, which the shim reports as GDN_ERR_HIP.
#include "gdn_internal.h"

int g_launches = 0;

namespace gdn {
hipError_t launch_chunk_fwd(const FwdParams&, int, bool, bool, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_state_chain(const FwdParams&, int, bool, bool, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_chunk_fwd_states(const FwdParams&, int, bool, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_chunk_fwd_save(const FwdParams&, int, bool, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_chunk_bwd(const BwdParams&, int, bool, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_recurrent(const RecParams&, int, bool, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_prologue(const PrologueParams&, int, bool, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_epilogue(const EpilogueParams&, int, bool, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_kda_fwd(const KdaParams&, int, bool, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_kda_bwd(const KdaBwdParams&, int, bool, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
size_t recurrent_bwd_ws_floats(int N, int H, int Dk, int Dv, int64_t max_len) {
  return static_cast<size_t>(N) * H * (static_cast<size_t>(max_len) + 1) * (Dk + Dv);
}
}  // namespace gdn
