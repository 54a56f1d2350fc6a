// noalloc.hip -- based_prefill_noalloc: based_prefill for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).
//
// The segment split of the bf16 matrix-core prefill needs a scratch area for
// the carried per-segment states (and for an initial state shared by several
// column groups).  based_prefill takes it from the caller; this variant
// takes it from `scratch`, a fixed device array of this library, which every
// GPU holds from the first call on it until the process ends.
//
// `scratch` names a host-side stand-in in host code: its device address is
// taken once per device with hipGetSymbolAddress (that device current) and
// only that address is ever passed to kernels.
//
// Nothing in `scratch` has to start at zero: the state pass writes every slot
// a call reads (the initial state, or zeros, into slot 0 and each segment's
// increment into the next) before the prefix sum and the output pass read
// them.  All calls on one GPU share its array, so calls that overlap in time
// on one GPU (different streams, different host threads) race: the caller
// must order them.
#include <hip/hip_runtime.h>

#include <mutex>

#include "based.h"
#include "kernels.hpp"

#define BASED_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kScratchBytes = BASED_PREFILL_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device (null until taken)

// Device address of `scratch` on device dev, taken on the first call for
// that device (with dev current; the caller's current device is restored).
hipError_t scratch_on(int dev, void** out) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        int cur = 0;
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
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

BASED_API based_status_t based_prefill_noalloc(const void* q, const void* k, const void* v, based_dtype_t dtype,
                                               int B, int H, int L, int d_feat, int d_v, int chunk, float eps,
                                               float* y, float* S, float* z, int use_initial_state, void* stream) {
    // Scratch this call's launch plan uses (0 when it uses none; malformed
    // arguments need none here and are refused by based_prefill below).
    size_t need = 0;
    if (dtype == BASED_BF16 && d_feat == 16 && (d_v == 64 || d_v == 128) && B >= 1 && H >= 1 && L >= 1 &&
        L <= INT32_MAX - 1023 && (long long)B * H <= (1ll << 27))
        need = based::prefill_mfma_plan_bytes(B * H, L, d_v, use_initial_state ? 1 : 0);
    if (need > kScratchBytes) return BASED_E_TOO_LARGE;
    void* ws = nullptr;
    size_t ws_bytes = 0;
    if (need > 0) {
        int dev = 0;
        hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
        if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) return BASED_E_LAUNCH;
        if (scratch_on(dev, &ws) != hipSuccess) return BASED_E_LAUNCH;
        ws_bytes = kScratchBytes;
    }
    return based_prefill(q, k, v, dtype, B, H, L, d_feat, d_v, chunk, eps, y, S, z, use_initial_state, ws, ws_bytes,
                         stream);
}
