// The library's one fixed device buffer: the workspace of pa_decode_noalloc,
// for callers that cannot allocate device memory.  gfx950 / CDNA4.
//
// `scratch` is a file-scope device array of kStaticWorkspaceBytes.  Each GPU
// the library runs on gets its own copy, at its own address, when the code
// object is loaded there, and keeps it until the process ends.  In host code
// the name `scratch` is only a host-side stand-in for the symbol, never a
// device address: every host use goes through the pointer that
// hipGetSymbolAddress returns for the current device, looked up once per
// device and cached here.  Nothing in the buffer has to start at zero: every
// byte a decode call reads was written earlier in the same call.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace pa {
namespace {

static __device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];

constexpr int kMaxDevices = 64;
void* g_ptr[kMaxDevices];              // the device address of `scratch` on each device
hipError_t g_err[kMaxDevices];
std::once_flag g_once[kMaxDevices];

}  // namespace

int static_workspace(void** ptr, size_t* bytes) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
    // with `dev` current: the address of this device's copy of the array
    std::call_once(g_once[dev], [dev] {
        void* p = nullptr;
        g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
    });
    if (g_err[dev] != hipSuccess) return (int)g_err[dev];
    if (g_ptr[dev] == nullptr) return (int)hipErrorInvalidSymbol;
    *ptr = g_ptr[dev];
    *bytes = kStaticWorkspaceBytes;
    return 0;
}

}  // namespace pa
