// Host-only stand-ins for the gfx950 kernel launchers and the scratch-area lookup of libffd, so
// that the C-ABI layer (csrc/ffd_api.cpp: argument validation, split heuristic, workspace layout)
// can be built with g++ and the address and undefined-behaviour sanitizers and driven by the ABI
// tests.  Test infrastructure: nothing here launches, reads or writes device memory; each
// launcher only counts its calls (ffd_stub_launches), and the next n launches (or scratch-area
// lookups) can be made to report a HIP error (ffd_stub_fail_next), to drive the error paths.
#include "../../long_context_decoding_amd/csrc/ffd_internal.h"

namespace {
int g_launches = 0;
int g_fail = 0;
hipError_t count()
{
    ++g_launches;
    if (g_fail > 0) {
        --g_fail;
        return hipErrorLaunchFailure;
    }
    return hipSuccess;
}
}  // namespace

namespace ffd {
hipError_t launch_bounds(const BoundsParams&, bool, hipStream_t) { return count(); }
hipError_t launch_scores(const ScoreParams&, int, bool, hipStream_t) { return count(); }
hipError_t launch_select(const SelectParams&, int, hipStream_t) { return count(); }
hipError_t launch_append(const AppendParams&, bool, hipStream_t) { return count(); }
hipError_t launch_decode(const DecodeParams&, bool, bool, hipStream_t) { return count(); }
hipError_t launch_quantize(const QuantParams&, bool, hipStream_t) { return count(); }
hipError_t launch_decode_res(const DecodeParams&, int, hipStream_t) { return count(); }
hipError_t launch_quantize_res(const QuantParams&, int, hipStream_t) { return count(); }
hipError_t launch_zero_counters(uint32_t*, int, hipStream_t) { return count(); }
hipError_t scratch_area(size_t, hipStream_t, void** ptr)
{
    if (g_fail > 0) {
        --g_fail;
        return hipErrorInvalidSymbol;
    }
    *ptr = reinterpret_cast<void*>(static_cast<uintptr_t>(1) << 20);  // aligned, never dereferenced
    return hipSuccess;
}
}  // namespace ffd

extern "C" int ffd_stub_launches(void) { return g_launches; }
extern "C" void ffd_stub_fail_next(int n) { g_fail = n; }
