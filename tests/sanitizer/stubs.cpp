// Host-only stand-ins for the kernel launchers of libfa, so that the C ABI
// (fa_api.cpp) can be built with AddressSanitizer and UndefinedBehaviorSanitizer
// and driven on a machine without a GPU. Test infrastructure: every stub
// records what it was given and launches nothing.
#include <hip/hip_runtime_api.h>

#include "fa_launch.h"

namespace fa {

FwdParams g_fwd;
BwdParams g_bwd;
DecodeParams g_dec;
Fp8QuantParams g_q8;
Fp8FwdParams g_f8;
int g_calls = 0;
alignas(256) float g_scratch[64];

hipError_t launch_fwd(const FwdParams& p, hipStream_t) { g_fwd = p; ++g_calls; return hipSuccess; }
hipError_t launch_bwd(const BwdParams& p, hipStream_t) { g_bwd = p; ++g_calls; return hipSuccess; }
hipError_t launch_decode(const DecodeParams& p, hipStream_t) { g_dec = p; ++g_calls; return hipSuccess; }
hipError_t launch_fp8_quant(const Fp8QuantParams& p, hipStream_t) { g_q8 = p; ++g_calls; return hipSuccess; }
hipError_t launch_fwd_fp8(const Fp8FwdParams& p, hipStream_t) { g_f8 = p; ++g_calls; return hipSuccess; }
int decode_waves() { return 768; }
hipError_t decode_scratch(void** ptr) { *ptr = g_scratch; return hipSuccess; }

}  // namespace fa

extern "C" const char* hipGetErrorString(hipError_t) { return "stub"; }
