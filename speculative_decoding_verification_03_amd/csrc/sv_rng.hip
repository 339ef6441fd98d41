// Counter-based uniforms for the verify step: u[b][t] for the ratio tests of the exact
// rule ("A Regra de Exatidão" on the lesson page "Decodificação Especulativa e EAGLE":
// one r ~ Uniform(0, 1) per drafted token) and, in slot K, the final categorical draw.
//
// Generator: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC'11): 10 rounds of two 64x64->128-bit multiplies and a
// permutation, with a Weyl-sequence key schedule.  Contract:
//   key = (seed, domain), counter = (t, b, step, 0), u = (word0 >> 40) * 2^-24.
#include <hip/hip_runtime.h>

#include "sv_common.h"
#include "sv_device.h"

namespace sv {

namespace {


// dense [B][K1]: thread i is (b, t) = (i / K1, i % K1)
__global__ __launch_bounds__(kThreads) void uniforms_kernel(uint64_t seed, uint64_t domain,
                                                            uint64_t step, int64_t total, int K1,
                                                            float* __restrict__ u) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= total) return;
    u[i] = philox_uniform(seed, domain, (uint64_t)(i % K1), (uint64_t)(i / K1), step);
}

// packed: thread i is (b, t) = (i / (K+1), i % (K+1)), K the bound on the drafts; writes
// u[cu[b] + b + t] for t <= K_b of sequences whose offsets are valid
__global__ __launch_bounds__(kThreads) void uniforms_packed_kernel(VerifyArgs a, uint64_t seed,
                                                                   uint64_t domain, uint64_t step,
                                                                   float* __restrict__ u) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int K1 = a.K + 1;
    if (i >= (int64_t)a.B * K1) return;
    const int b = (int)(i / K1), t = (int)(i % K1);
    const SeqRows s = seq_rows(a, b);
    if (t > s.K) return;  // also when the offsets are invalid (s.K = -1)
    u[s.t0 + t] = philox_uniform(seed, domain, (uint64_t)t, (uint64_t)b, step);
}

}  // namespace

int launch_uniforms(uint64_t seed, uint64_t domain, uint64_t step, int B, int K, float* u,
                    void* stream) {
    const int64_t total = (int64_t)B * (K + 1);
    if (total == 0) return 0;
    const int64_t blocks = (total + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(uniforms_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), seed, domain, step, total, K + 1, u);
    return (int)hipGetLastError();
}

int launch_uniforms_packed(uint64_t seed, uint64_t domain, uint64_t step, int B, int K,
                           const int32_t* cu, int total, float* u, void* stream) {
    const int64_t n = (int64_t)B * (K + 1);
    if (n == 0) return 0;
    VerifyArgs a{};
    a.cu = cu;
    a.total = total;
    a.B = B;
    a.K = K;
    const int64_t blocks = (n + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(uniforms_packed_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), a, seed, domain, step, u);
    return (int)hipGetLastError();
}

}  // namespace sv
