// spec_verify_noalloc: spec_verify for callers that cannot allocate (code under HIP
// graph capture, serving loops that forbid allocation): the workspace is a static
// device array of this file, one copy per GPU, instead of a caller buffer.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "spec_verify.h"
#include "sv_common.h"

namespace {

constexpr size_t kScratchBytes = SV_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// The workspace of every spec_verify_noalloc call on a GPU.  In host code this name is
// only a handle for hipGetSymbolAddress: the kernels get the device address it returns.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up on the first call
// there (with that device current) and kept.
sv_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SV_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SV_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return SV_OK;
}

}  // namespace

extern "C" sv_status spec_verify_noalloc(const void* target_logits, const void* draft_logits,
                                         int dtype, const int32_t* draft_tokens,
                                         const float* uniforms, const float* temperature, int B,
                                         int K, int V, int32_t* out_tokens,
                                         int32_t* out_accept_len, float* out_p, float* out_q,
                                         int32_t* out_status, void* stream) {
    // every argument check first, on the host (a stand-in address for the scratch array,
    // which validation does not dereference), then the size limit
    void* const stand_in = reinterpret_cast<void*>(static_cast<uintptr_t>(256));
    sv_status st = (sv_status)sv::verify_dense_call(
        target_logits, draft_logits, dtype, draft_tokens, uniforms, temperature, B, K, V,
        out_tokens, out_accept_len, out_p, out_q, out_status, stand_in, ~(size_t)0, stream,
        false, false);
    if (st != SV_OK || B == 0) return st;
    if (sv::workspace_need(B, K, V) > kScratchBytes) return SV_ERR_SCRATCH;
    // the stream must belong to the current device, whose copy of scratch is used
    if (stream) {
        int sdev = -1, cur = -1;
        if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess ||
            hipGetDevice(&cur) != hipSuccess)
            return SV_ERR_HIP;
        if (sdev != cur) return SV_ERR_ARG;
    }
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != SV_OK) return st;
    // the same validation and kernels as spec_verify; no benchmark events (creating one
    // would allocate)
    return (sv_status)sv::verify_dense_call(target_logits, draft_logits, dtype, draft_tokens,
                                            uniforms, temperature, B, K, V, out_tokens,
                                            out_accept_len, out_p, out_q, out_status, ws,
                                            kScratchBytes, stream, false, true);
}
