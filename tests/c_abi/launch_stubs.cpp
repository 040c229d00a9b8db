// Launch functions of the C ABI layer replaced by stubs that abort: the
// sanitizer build of kda_api.hip links against these, so any call in the host
// checks that got as far as launching a kernel ends the test program.
#include <cstdlib>

#include "kda_internal.h"

namespace kda {
hipError_t launch_window_table(const int32_t*, int, int64_t, int, int, int, int, int32_t*, int32_t*, int32_t*,
                               hipStream_t) { std::abort(); }
hipError_t launch_window_segments(const int32_t*, const int32_t*, int, int, int, int32_t*, int32_t*, int32_t*,
                                  hipStream_t) { std::abort(); }
hipError_t launch_prep(const PrepArgs&, hipStream_t) { std::abort(); }
hipError_t launch_carry(const CarryArgs&, hipStream_t) { std::abort(); }
hipError_t launch_decode(const DecodeArgs&, hipStream_t) { std::abort(); }
hipError_t launch_replay(const ReplayArgs&, hipStream_t) { std::abort(); }
hipError_t run_checks(const CheckArgs&, hipStream_t, uint32_t*) { std::abort(); }
hipError_t launch_worklist(const int32_t*, int, int32_t*, hipStream_t) { std::abort(); }
hipError_t launch_scan(const ScanArgs&, hipStream_t) { std::abort(); }
hipError_t launch_bwd_prep(const BwdArgs&, hipStream_t) { std::abort(); }
hipError_t launch_bwd_carry(const BwdArgs&, hipStream_t) { std::abort(); }
hipError_t launch_bwd_grad(const BwdArgs&, hipStream_t) { std::abort(); }
}  // namespace kda
