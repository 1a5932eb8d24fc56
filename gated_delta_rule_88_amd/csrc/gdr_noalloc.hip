// gdr_noalloc.hip -- the chunked forward for callers that cannot allocate
// device memory: its workspace is a fixed array in the library's own device
// memory instead of a caller-provided buffer.
//
// The array is a file-scope __device__ variable, so each GPU the library
// runs on holds its own copy (allocated when the runtime loads the code
// object on that device) until the process ends.  Host code must not use the
// variable's name as an address: on the host it names a stand-in, not device
// memory.  The device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept; kernels are then
// handed that address exactly as they are handed a caller's workspace.
//
// Every call on a device shares that device's array and finds in it what
// the last call left.  No kernel of the forward reads a workspace byte it
// has not written earlier in the same call, so nothing needs clearing; but
// two calls that overlap on one device (different streams or host threads)
// race on the array and must be serialised by the caller.
#include "../../include/gdr.h"

#include <mutex>

#include "gdr_internal.h"

#define GDR_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kScratchBytes = (size_t)GDR_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];   // device address of `scratch`, per device (null until looked up)

// The scratch array's address on the current device, looked up on the first
// call made with that device current.
hipError_t scratch_address(void** out)
{
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

GDR_EXPORT int gdr_fwd_chunked_noalloc(int B, int H, int L, int d_k, int d_v, int C, int dtype,
                                       const void* q, const void* k, const void* v,
                                       const float* beta, int alpha_mode, const float* log_alpha,
                                       const float* S0, void* o, float* S_final, hipStream_t stream)
{
    const size_t need = gdr::fwd_chunked_workspace_checked(B, H, L, d_k, d_v, C, dtype, alpha_mode);
    if (need == (size_t)-1) {
        // sizes outside the domain: the full checks give the precise status
        return gdr::fwd_chunked_checked(B, H, L, d_k, d_v, C, dtype, q, k, v, beta, alpha_mode,
                                        log_alpha, S0, o, S_final, nullptr, 0, stream, 0u);
    }
    if (need > kScratchBytes) return GDR_ERR_SCRATCH_TOO_SMALL;
    void* ws = nullptr;
    if (need > 0 && scratch_address(&ws) != hipSuccess) return GDR_ERR_HIP;
    return gdr::fwd_chunked_checked(B, H, L, d_k, d_v, C, dtype, q, k, v, beta, alpha_mode, log_alpha,
                                    S0, o, S_final, ws, need > 0 ? kScratchBytes : 0, stream, 0u);
}
