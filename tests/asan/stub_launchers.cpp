// Host-only stand-ins for the library's kernel launchers and device scratch,
// for the AddressSanitizer build of the C-ABI layer (tests/test_abi_asan.py):
// that build compiles sa_api.cpp with the host compiler alone, so every call
// that passes its checks ends here with a launch error (SA_ERR_HIP), having
// exercised the argument checks, the split table and the workspace layout
// with real host memory only.
#include "sa_internal.h"

namespace sa {

int g_launches = 0;   // calls that got past their checks

hipError_t scratch_pointer(void**) { ++g_launches; return hipErrorNoDevice; }
hipError_t launch_kv_append(const AppendArgs&, hipStream_t) { ++g_launches; return hipErrorNoDevice; }
hipError_t launch_decode_mfma(const DecodeArgs&, bool, int, hipStream_t) {
    ++g_launches;
    return hipErrorNoDevice;
}
hipError_t launch_decode_stream(const DecodeArgs&, bool, bool, hipStream_t) {
    ++g_launches;
    return hipErrorNoDevice;
}
hipError_t launch_decode_valu(const DecodeArgs&, hipStream_t) { ++g_launches; return hipErrorNoDevice; }
hipError_t launch_combine(const CombineArgs&, hipStream_t) { ++g_launches; return hipErrorNoDevice; }
hipError_t launch_read_probe(const void*, size_t, unsigned*, hipStream_t) {
    ++g_launches;
    return hipErrorNoDevice;
}
hipError_t launch_tile_probe(const void*, size_t, const int*, long long, int, unsigned*,
                             hipStream_t) {
    ++g_launches;
    return hipErrorNoDevice;
}

}  // namespace sa

extern "C" int sa_test_launch_count(void) { return sa::g_launches; }
