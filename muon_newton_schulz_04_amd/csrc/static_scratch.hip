// The library's own device workspace, for callers that cannot allocate
// device memory (muon_init_static in include/libmuon.h).
//
// `scratch` is a file-scope device array of MUON_STATIC_WORKSPACE_BYTES; every
// GPU the library runs on holds its own copy until the process ends. In host
// code its name is only a host-side stand-in, so the device address is looked
// up once per device with hipGetSymbolAddress (with that device current) and
// kept here; kernels, copies and fills get that address, never the name.

#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/libmuon.h"

static __device__ __align__(256) char scratch[MUON_STATIC_WORKSPACE_BYTES];

namespace muon {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};
}  // namespace

// Device address of `scratch` on `device`, which must be the current device.
hipError_t static_scratch_address(int device, void** addr) {
    if (device < 0 || device >= kMaxDevices || !addr) return hipErrorInvalidValue;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_addr[device]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_addr[device] = p;
    }
    *addr = g_addr[device];
    return hipSuccess;
}

}  // namespace muon
