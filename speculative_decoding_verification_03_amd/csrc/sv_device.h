// Device helpers of the verify kernels (gfx950, wave64): logit loads, NaN-propagating
// maxima, wavefront/workgroup reductions and scans.  All reductions combine in a fixed
// order, so every result is bit-reproducible from run to run.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sv_common.h"

namespace sv {

// IEEE 754-2019 maximum: NaN if either operand is NaN (v_maximum3_f32 on gfx950).
__device__ __forceinline__ float nmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// A pointer to device global memory, marked so: the compiler then emits global loads
// rather than flat ones, whose completion every wait for an LDS read would include too.
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* gbl(const T* p) {
    return (const __attribute__((address_space(1))) T*)p;
}

// A pointer to LDS, marked so.
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(3))) T* lds(const T* p) {
    return (const __attribute__((address_space(3))) T*)p;
}

// One 16-byte streaming load from global memory (non-temporal: logits are read once).
__device__ __forceinline__ u32x4 load16(const void* p) {
    return __builtin_nontemporal_load(gbl(reinterpret_cast<const u32x4*>(p)));
}

// Logit element access: fp32 rows or bf16 rows (stored as uint16_t bit patterns).
template <typename E>
struct Logit;

template <>
struct Logit<float> {
    static constexpr int kVec = 4;  // elements per 16-byte load
    __device__ static __forceinline__ float at(const float* p, int64_t i) { return gbl(p)[i]; }
    __device__ static __forceinline__ u32x4 neg_inf16() {
        const uint32_t n = 0xff800000u;
        return u32x4{n, n, n, n};
    }
    __device__ static __forceinline__ void unpack(u32x4 v, float (&z)[4]) {
        z[0] = __uint_as_float(v.x); z[1] = __uint_as_float(v.y);
        z[2] = __uint_as_float(v.z); z[3] = __uint_as_float(v.w);
    }
};

template <>
struct Logit<uint16_t> {
    static constexpr int kVec = 8;
    __device__ static __forceinline__ float at(const uint16_t* p, int64_t i) {
        return __uint_as_float((uint32_t)gbl(p)[i] << 16);
    }
    __device__ static __forceinline__ u32x4 neg_inf16() {
        const uint32_t n = 0xff80ff80u;  // two bf16 -inf
        return u32x4{n, n, n, n};
    }
    __device__ static __forceinline__ void unpack(u32x4 v, float (&z)[8]) {
        z[0] = bf16_lo(v.x); z[1] = bf16_hi(v.x);
        z[2] = bf16_lo(v.y); z[3] = bf16_hi(v.y);
        z[4] = bf16_lo(v.z); z[5] = bf16_hi(v.z);
        z[6] = bf16_lo(v.w); z[7] = bf16_hi(v.w);
    }
};

// ---------------------------------------------------------------------------------
// fp64 2^y for the categorical draws (about 12 VALU operations and one LDS read):
// y = k/256 + f with k = rint(256 y) and |f| <= 1/512;  2^y = 2^(k>>8) * 2^((k&255)/256) * 2^f,
// the middle factor from a 256-entry table, 2^f from its Taylor series in f*ln2 to degree 4
// (truncation below 4e-17).  rint comes from adding 1.5 * 2^52, which leaves k in the low
// word of the sum.  y is clamped to [-1080, 1100], which maps -inf and every argument that
// underflows to 0, and +inf and every argument that overflows to inf.  Relative error a
// few 1e-16.
// ---------------------------------------------------------------------------------

constexpr int kExpTable = 256;

// Fill the table (kExpTable doubles of LDS) once per workgroup, without a barrier:
// 2^x for x = j/256 in [0, 1) from the Taylor series of exp(x ln2) to degree 17 (truncation
// below 2e-19), evaluated by Horner: a few registers, unlike a library exp2.
__device__ __forceinline__ void exp2_table_fill(double* t) {
    constexpr double c[18] = {1.0,
                              0.6931471805599453,
                              0.2402265069591007,
                              0.055504108664821576,
                              0.009618129107628477,
                              0.0013333558146428441,
                              0.00015403530393381606,
                              1.5252733804059838e-05,
                              1.3215486790144305e-06,
                              1.0178086009239696e-07,
                              7.054911620801121e-09,
                              4.44553827187081e-10,
                              2.5678435993488196e-11,
                              1.3691488853904124e-12,
                              6.778726354822543e-14,
                              3.132436707088427e-15,
                              1.357024794875514e-16,
                              5.533046532458238e-18};
    for (int j = threadIdx.x; j < kExpTable; j += blockDim.x) {
        const double x = (double)j / kExpTable;
        double p = c[17];
#pragma unroll
        for (int n = 16; n >= 0; --n) p = __builtin_fma(p, x, c[n]);
        t[j] = p;
    }
}

// The same, then __syncthreads().
__device__ __forceinline__ void exp2_table_init(double* t) {
    exp2_table_fill(t);
    __syncthreads();
}

// 2^(Y / 256) for Y in units of 1/256 of a binary order of magnitude (the caller folds the
// 256 into its scale factor).  Y = 256 k' + j + F with the table giving 2^(j/256) and
// |F| <= 1/2; 2^(F/256) by its Taylor polynomial of degree 4, whose truncation error is
// below (ln 2 / 512)^5 / 120 = 4e-17 relative: the weights stay fp64-accurate even where
// p - q cancels to a small fraction of p.  Y below -1080*256 (including -inf) gives 0.
__device__ __forceinline__ double exp2_256(double Y, const double* t) {
#pragma clang fp contract(off)
    constexpr double kRound = 6755399441055744.0;  // 1.5 * 2^52: rounds to an integer
    constexpr double kL = 0.6931471805599453 / 256.0;
    Y = fmin(fmax(Y, -1080.0 * 256.0), 1100.0 * 256.0);
    const double tk = Y + kRound;
    const int k = __double2loint(tk);
    const double F = Y - (tk - kRound);
    double p = kL * kL * kL * kL / 24.0;
    p = __builtin_fma(p, F, kL * kL * kL / 6.0);
    p = __builtin_fma(p, F, kL * kL / 2.0);
    p = __builtin_fma(p, F, kL);
    p = __builtin_fma(p, F, 1.0);
    return ldexp(t[k & (kExpTable - 1)] * p, k >> 8);
}

// (z - ref) * c, never fused into a following add: every caller that evaluates a weight as
// exp2_256(exp2_arg(...)), tabulated or direct, gets the same bits for the same operands.
__device__ __forceinline__ double exp2_arg(double z, double ref, double c) {
#pragma clang fp contract(off)
    return (z - ref) * c;
}

// ---------------------------------------------------------------------------------
// counter-based uniforms: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC'11): 10 rounds of two 64x64->128-bit multiplies and a
// permutation, with a Weyl-sequence key schedule.  Contract:
//   key = (seed, domain), counter = (t, b, step, 0), u = (word0 >> 40) * 2^-24.
// ---------------------------------------------------------------------------------

__device__ __forceinline__ float philox_uniform(uint64_t seed, uint64_t domain, uint64_t t,
                                                uint64_t b, uint64_t step) {
    constexpr uint64_t kM0 = 0xD2E7470EE14C6C93ull;
    constexpr uint64_t kM1 = 0xCA5A826395121157ull;
    constexpr uint64_t kW0 = 0x9E3779B97F4A7C15ull;
    constexpr uint64_t kW1 = 0xBB67AE8584CAA73Bull;
    uint64_t c0 = t, c1 = b, c2 = step, c3 = 0;
    uint64_t k0 = seed, k1 = domain;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t lo0 = kM0 * c0, hi0 = __umul64hi(kM0, c0);
        const uint64_t lo1 = kM1 * c2, hi1 = __umul64hi(kM1, c2);
        const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
        k0 += kW0;
        k1 += kW1;
    }
    return (float)(uint32_t)(c0 >> 40) * 0x1p-24f;
}

// ---------------------------------------------------------------------------------
// where a sequence's rows live (dense or packed layout, see VerifyArgs)
// ---------------------------------------------------------------------------------

struct SeqRows {
    int K;       // drafts of the sequence; -1 when its packed offsets are invalid
    int64_t t0;  // index of its target row 0 (also of its first uniform and output token)
    int64_t d0;  // index of its draft row 0 (also of its first draft token, p and q)
};

// Packed offsets are valid when 0 <= cu[b] <= cu[b+1] <= total and K_b <= K: then every
// row, token, uniform and output slot the sequence touches lies inside the packed arrays.
__device__ __forceinline__ SeqRows seq_rows(const VerifyArgs& a, int b) {
    SeqRows s;
    if (!a.cu) {
        s.K = a.K;
        s.d0 = (int64_t)b * a.K;
        s.t0 = s.d0 + b;
        return s;
    }
    const int c0 = a.cu[b], c1 = a.cu[b + 1];
    if (c0 < 0 || c1 < c0 || c1 > a.total || c1 - c0 > a.K) {
        s.K = -1;
        s.t0 = s.d0 = 0;
        return s;
    }
    s.K = c1 - c0;
    s.d0 = c0;
    s.t0 = (int64_t)c0 + b;
    return s;
}

// ---------------------------------------------------------------------------------
// wavefront reductions (butterfly: every lane ends with the same value)
// ---------------------------------------------------------------------------------

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float wave_nmax(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = nmax(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ int wave_or(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o, 64);
    return v;
}

// (value, index) maximum with the lowest index on ties; NaN handled by the caller.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) {
        v = v2;
        i = i2;
    }
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float v2 = __shfl_xor(v, o, 64);
        const int i2 = __shfl_xor(i, o, 64);
        argmax_merge(v, i, v2, i2);
    }
}

// ---------------------------------------------------------------------------------
// workgroup reductions over NW waves (NW * 64 threads); every thread gets the result.
// `sh` must hold NW entries of the value type.  Contains __syncthreads().
// ---------------------------------------------------------------------------------

template <int NW = kWaves>
__device__ __forceinline__ double block_sum(double v, double* sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    v = wave_sum(v);
    if (lane == 0) sh[w] = v;
    __syncthreads();
    double t = sh[0];
#pragma unroll
    for (int k = 1; k < NW; ++k) t += sh[k];
    __syncthreads();
    return t;
}

template <int NW = kWaves>
__device__ __forceinline__ float block_nmax(float v, float* sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    v = wave_nmax(v);
    if (lane == 0) sh[w] = v;
    __syncthreads();
    float t = sh[0];
#pragma unroll
    for (int k = 1; k < NW; ++k) t = nmax(t, sh[k]);
    __syncthreads();
    return t;
}

// Maximum of floats (fmaxf: a NaN operand is ignored).
template <int NW = kWaves>
__device__ __forceinline__ float block_max_f(float v, float* sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    if (lane == 0) sh[w] = v;
    __syncthreads();
    float t = sh[0];
#pragma unroll
    for (int k = 1; k < NW; ++k) t = fmaxf(t, sh[k]);
    __syncthreads();
    return t;
}

template <int NW = kWaves>
__device__ __forceinline__ int block_min(int v, int* sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    v = wave_min(v);
    if (lane == 0) sh[w] = v;
    __syncthreads();
    int t = sh[0];
#pragma unroll
    for (int k = 1; k < NW; ++k) t = min(t, sh[k]);
    __syncthreads();
    return t;
}

template <int NW = kWaves>
__device__ __forceinline__ int block_max(int v, int* sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    v = wave_max(v);
    if (lane == 0) sh[w] = v;
    __syncthreads();
    int t = sh[0];
#pragma unroll
    for (int k = 1; k < NW; ++k) t = max(t, sh[k]);
    __syncthreads();
    return t;
}

template <int NW = kWaves>
__device__ __forceinline__ int block_or(int v, int* sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    v = wave_or(v);
    if (lane == 0) sh[w] = v;
    __syncthreads();
    int t = sh[0];
#pragma unroll
    for (int k = 1; k < NW; ++k) t |= sh[k];
    __syncthreads();
    return t;
}

template <int NW = kWaves>
__device__ __forceinline__ void block_argmax(float& v, int& i, float* shv, int* shi) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    wave_argmax(v, i);
    if (lane == 0) {
        shv[w] = v;
        shi[w] = i;
    }
    __syncthreads();
    v = shv[0];
    i = shi[0];
#pragma unroll
    for (int k = 1; k < NW; ++k) argmax_merge(v, i, shv[k], shi[k]);
    __syncthreads();
}

// Inclusive prefix sum over the wave's lanes in lane order (Hillis-Steele: a fixed
// combination order, so the result is reproducible).
__device__ __forceinline__ double wave_inclusive_scan(double v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double y = __shfl_up(v, o, 64);
        if (lane >= o) v += y;
    }
    return v;
}

// Exclusive prefix sum of one fp64 value per thread, in thread order; also returns
// the workgroup total.  Fixed combination order (Hillis-Steele inside each wave, then
// wave totals left to right), so results are reproducible.
template <int NW = kWaves>
__device__ __forceinline__ double block_exclusive_scan(double v, double& total, double* sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    double incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
    }
    if (lane == 63) sh[w] = incl;
    __syncthreads();
    double before = 0.0, tot = 0.0;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
        if (k < w) before += sh[k];
        tot += sh[k];
    }
    __syncthreads();
    total = tot;
    // exclusive = inclusive minus own value would round differently; shift instead
    double excl = __shfl_up(incl, 1, 64);
    if (lane == 0) excl = 0.0;
    return before + excl;
}

}  // namespace sv
