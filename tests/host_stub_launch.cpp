// Launch stubs for a host-only sanitizer build of the C ABI (tests/test_host_sanitizers.py).  The
// ABI tests never reach a launch; if one did, the stub aborts and the test fails.
#include "conv1d_launch.h"
#include <cstdlib>
namespace cconv {
static hipError_t fail() { std::abort(); }
hipError_t launch_fwd(const FwdArgs&, int, bool, bool, hipStream_t) { return fail(); }
hipError_t launch_decode(const DecodeArgs&, bool, bool, hipStream_t) { return fail(); }
hipError_t launch_bwd(const BwdArgs&, int, bool, bool, hipStream_t) { return fail(); }
hipError_t launch_reduce(const BwdArgs&, hipStream_t) { return fail(); }
hipError_t launch_fwd_cf(const CfArgs&, bool, bool, hipStream_t) { return fail(); }
hipError_t launch_bwd_cf(const CfArgs&, bool, bool, hipStream_t) { return fail(); }
hipError_t launch_combine(const CombineArgs&, hipStream_t) { return fail(); }
hipError_t bwd_scratch(hipStream_t, void**) { return fail(); }
}
