// swa_decode_split_noalloc: the split-window ring decode with its partial
// results in a static device array instead of a caller workspace, for
// callers that cannot allocate (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).  Contract in include/swa.h.

#include "../../include/swa.h"
#include "swa_internal.h"

#include <mutex>

namespace {

// The partial (max, sum, unnormalised output) triples of the split decode.
// Every GPU the library runs on holds its own copy until the process ends.
// In host code `scratch` names a host-side stand-in: only the device
// address from hipGetSymbolAddress may reach a kernel or a copy.
constexpr int64_t kScratchBytes = SWA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device (guarded by g_mu)

// Device address of this device's `scratch`, looked up once per device with
// that device current.
hipError_t scratch_on(int dev, void** ptr) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" int swa_decode_split_noalloc(const void* q, const void* kring, const void* vring,
                                        const int64_t* pos, void* out, int64_t S, int64_t H,
                                        int64_t D, int64_t W, int dtype, void* stream) {
    if (!q || !kring || !vring || !pos || !out) return SWA_ERR_INVALID_ARG;
    const int64_t need = swa_decode_workspace_bytes(S, H, D, W, dtype);
    if (need < 0) return (int)-need;
    if (need > kScratchBytes) return SWA_ERR_SCRATCH_LIMIT;
    if (need == 0)   // no split for these sizes: swa_decode's kernels, no scratch
        return swa_decode_split(q, kring, vring, pos, out, S, H, D, W, dtype, nullptr, 0, stream);
    hipStream_t st = (hipStream_t)stream;
    int dev = -1;
    if (hipStreamGetDevice(st, &dev) != hipSuccess) return SWA_ERR_LAUNCH;
    void* ws = nullptr;
    if (scratch_on(dev, &ws) != hipSuccess) return SWA_ERR_LAUNCH;
    return swa_decode_split(q, kring, vring, pos, out, S, H, D, W, dtype, ws, kScratchBytes,
                            stream);
}
