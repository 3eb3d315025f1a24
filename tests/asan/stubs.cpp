// Host-only stand-ins for the kernel launchers, so that the C-ABI entry points
// (fa_api.cpp) can be built with g++ and a sanitizer and driven on a host
// without a GPU.  A call that passed every check would reach one of these:
// each records the call and reports a launch failure.
#include <hip/hip_runtime.h>

#include "fa_fp8.h"
#include "fa_internal.h"

int g_launches = 0;

namespace fa {
hipError_t launch_fwd(const FwdParams&, int, int, hipStream_t) { ++g_launches; return hipErrorNoDevice; }
hipError_t launch_bwd(const BwdParams&, int, int, hipStream_t) { ++g_launches; return hipErrorNoDevice; }
hipError_t launch_decode(const DecodeParams&, int, int, hipStream_t) { ++g_launches; return hipErrorNoDevice; }
hipError_t launch_fp8_quantize(const Fp8QuantParams&, hipStream_t) { ++g_launches; return hipErrorNoDevice; }
hipError_t launch_fwd_fp8(const Fp8FwdParams&, int, hipStream_t) { ++g_launches; return hipErrorNoDevice; }
hipError_t decode_scratch(void** ptr) { ++g_launches; *ptr = nullptr; return hipErrorNoDevice; }
}  // namespace fa
