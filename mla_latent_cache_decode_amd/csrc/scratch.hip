// Device scratch of the decode entry point that allocates nothing
// (mla_decode_run_noalloc).
//
// The array is a file-scope device variable: every GPU the library runs on
// holds its own copy, at its own address, from the code object's load until
// the process ends.  In host code its name is only a stand-in, never a
// device address; the address of a device's copy comes from
// hipGetSymbolAddress with that device current, taken once per device at
// init and kept here.  Host code passes that address, never the name.
#include "mla_internal.h"

#include <mutex>

namespace mla {

static __device__ __attribute__((aligned(256))) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 128;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_address(int device, void** out) {
    *out = nullptr;
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[device] = p;
    }
    *out = g_scratch_ptr[device];
    return hipSuccess;
}

}  // namespace mla
