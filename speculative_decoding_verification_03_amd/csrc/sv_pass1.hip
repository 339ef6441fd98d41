// Pass 1 of the verify step and the per-sequence resolve.
//
// Pass 1 streams every logit row a sequence needs exactly once from HBM: target rows
// t = 0..K always, draft rows t = 0..K-1 for sampled sequences.  Greedy rows keep the
// maximum and its lowest index (the temperature-0 rule, "Caso ganancioso" on the lesson
// page "Decodificação Especulativa e EAGLE").  Sampled rows keep the maximum m and
// S = sum_i exp((z_i - m) / T): the normaliser of the temperature softmax of that
// page's "Desenvolva" listing, accumulated online with a lazily moved reference.
//
// Each workgroup handles one (row, chunk) tile.  The workgroup that completes the
// last tile of a sequence (a per-sequence counter, self-resetting) merges the tiles and
// runs the resolve: the left-to-right test r_t < p_t(x_t)/q_t(x_t) of "A Regra de
// Exatidão", evaluated in fp64 log space, or the greedy comparison; it writes the
// accepted prefix and hands the final draw to pass 2 through a SeqDesc.
#include <float.h>
#include <hip/hip_runtime.h>
#include <math.h>

#include "sv_common.h"
#include "sv_device.h"

namespace sv {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
// Lazy rescale threshold of the running sum, in log2 units: elements may exceed the
// running reference by up to 2^32 before the reference moves.
constexpr float kRescaleLog2 = 32.0f;

// ------------------------------------------------------------------------------------
// per-thread accumulators
// ------------------------------------------------------------------------------------

struct SumExpAcc {
    float mx;   // NaN-propagating maximum of everything seen
    float ref;  // reference of s (s = sum exp2((z - ref) * c2))
    double s;
};

template <int N>
__device__ __forceinline__ void sumexp_step(const float (&z)[N], float c2, SumExpAcc& a) {
    float tm = z[0];
#pragma unroll
    for (int k = 1; k < N; ++k) tm = nmax(tm, z[k]);
    a.mx = nmax(a.mx, tm);
    if ((tm - a.ref) * c2 > kRescaleLog2) {
        // rare: the reference moves up; rescale the sum exactly enough in fp64
        if (a.s != 0.0) a.s *= exp2(((double)a.ref - (double)tm) * (double)c2);
        a.ref = tm;
    }
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < N; ++k) acc += __builtin_amdgcn_exp2f((z[k] - a.ref) * c2);
    a.s += (double)acc;
}

struct ArgmaxAcc {
    float mx;   // strict running maximum (NaN never enters)
    int idx;    // lowest index reaching mx
    int bad;    // a NaN was seen
};

template <int N>
__device__ __forceinline__ void argmax_step(const float (&z)[N], int64_t base, ArgmaxAcc& a) {
    float tm = z[0];
#pragma unroll
    for (int k = 1; k < N; ++k) tm = nmax(tm, z[k]);
    a.bad |= (tm != tm);
    if (tm > a.mx) {
        int k0 = N - 1;
#pragma unroll
        for (int k = N - 1; k >= 0; --k)
            if (z[k] == tm) k0 = k;
        a.mx = tm;
        a.idx = (int)base + k0;
    }
}

// ------------------------------------------------------------------------------------
// one (row, chunk) tile, whole workgroup
// ------------------------------------------------------------------------------------

// Calls f(z[N], first_index) over [lo, hi) of `row`: scalar head up to 16-byte
// alignment, 16-byte vectors, scalar tail.  Thread order inside the body is strided,
// so each thread sees its elements in increasing index order.
template <typename E, class FV, class FS>
__device__ __forceinline__ void for_tile(const E* row, int lo, int hi, FV&& fvec, FS&& fscalar) {
    constexpr int VEC = Logit<E>::kVec;
    const uintptr_t addr = reinterpret_cast<uintptr_t>(row + lo);
    int head = (int)(((16 - (addr & 15)) & 15) / sizeof(E));
    if (head > hi - lo) head = hi - lo;
    if ((int)threadIdx.x < head) fscalar(Logit<E>::at(row, lo + threadIdx.x), lo + threadIdx.x);
    const int body0 = lo + head;
    const int nvec = (hi - body0) / VEC;
    const E* p = row + body0;
    int v = threadIdx.x;
    // two independent 16-byte loads in flight per iteration
    for (; v + kThreads < nvec; v += 2 * kThreads) {
        float z0[VEC], z1[VEC];
        Logit<E>::vec(p + (int64_t)v * VEC, z0);
        Logit<E>::vec(p + (int64_t)(v + kThreads) * VEC, z1);
        fvec(z0, body0 + v * VEC);
        fvec(z1, body0 + (v + kThreads) * VEC);
    }
    if (v < nvec) {
        float z0[VEC];
        Logit<E>::vec(p + (int64_t)v * VEC, z0);
        fvec(z0, body0 + v * VEC);
    }
    const int tail0 = body0 + nvec * VEC;
    const int i = tail0 + threadIdx.x;
    if (i < hi) fscalar(Logit<E>::at(row, i), i);
}

template <typename E>
__device__ void tile_sumexp(const E* row, int lo, int hi, float T, RowPartial* out) {
    __shared__ float shf[kWaves];
    __shared__ double shd[kWaves];
    const float c2 = (float)(1.4426950408889634 / (double)T);
    SumExpAcc a{-INFINITY, -FLT_MAX, 0.0};
    for_tile<E>(
        row, lo, hi,
        [&](const float(&z)[Logit<E>::kVec], int) { sumexp_step(z, c2, a); },
        [&](float z, int) {
            const float zz[1] = {z};
            sumexp_step(zz, c2, a);
        });
    const float m = block_nmax(a.mx, shf);
    // rebase every thread's sum on the tile maximum in fp64
    double s = 0.0;
    if (a.s != 0.0) s = a.s * exp(((double)a.ref - (double)m) / (double)T);
    s = block_sum(s, shd);
    if (threadIdx.x == 0) {
        out->m = m;
        out->idx = 0;
        out->s = s;
    }
}

template <typename E>
__device__ void tile_argmax(const E* row, int lo, int hi, RowPartial* out) {
    __shared__ float shv[kWaves];
    __shared__ int shi[kWaves];
    ArgmaxAcc a{-INFINITY, 0x7fffffff, 0};
    for_tile<E>(
        row, lo, hi,
        [&](const float(&z)[Logit<E>::kVec], int base) { argmax_step(z, base, a); },
        [&](float z, int i) {
            const float zz[1] = {z};
            argmax_step(zz, i, a);
        });
    const int bad = block_or(a.bad, shi);
    float v = a.mx;
    int i = a.idx;
    block_argmax(v, i, shv, shi);
    if (threadIdx.x == 0) {
        out->m = bad ? __builtin_nanf("") : v;
        out->idx = i;
        out->s = 0.0;
    }
}

// ------------------------------------------------------------------------------------
// the resolve
// ------------------------------------------------------------------------------------

template <typename E>
__device__ __forceinline__ const E* target_row(const VerifyArgs& a, int b, int t) {
    return static_cast<const E*>(a.target) + ((int64_t)b * (a.K + 1) + t) * a.V;
}
template <typename E>
__device__ __forceinline__ const E* draft_row(const VerifyArgs& a, int b, int t) {
    return static_cast<const E*>(a.draft) + ((int64_t)b * a.K + t) * a.V;
}

// Merge the chunk partials of row j (0..K target, K+1..2K draft) of sequence b.
__device__ __forceinline__ void merge_greedy(const VerifyArgs& a, int b, int j, float& m, int& idx) {
    const RowPartial* p = a.part1 + ((int64_t)b * a.R + j) * a.nchunk1;
    m = -INFINITY;
    idx = 0x7fffffff;
    bool bad = false;
    for (int c = 0; c < a.nchunk1; ++c) {
        const float pm = p[c].m;
        if (pm != pm) bad = true;
        else if (pm > m) {  // strict: an earlier chunk keeps ties
            m = pm;
            idx = p[c].idx;
        }
    }
    if (bad) m = __builtin_nanf("");
}

__device__ __forceinline__ void merge_sampled(const VerifyArgs& a, int b, int j, double invT, float& m,
                                              double& S) {
    const RowPartial* p = a.part1 + ((int64_t)b * a.R + j) * a.nchunk1;
    m = -INFINITY;
    for (int c = 0; c < a.nchunk1; ++c) m = nmax(m, p[c].m);
    S = 0.0;
    for (int c = 0; c < a.nchunk1; ++c) {
        const double s = p[c].s;
        if (s != 0.0) S += s * exp(((double)p[c].m - (double)m) * invT);
    }
}

__device__ __forceinline__ bool row_bad(float m, bool sampled) {
    return (m != m) || m == -INFINITY || (sampled && m == INFINITY);
}

__device__ __forceinline__ bool temperature_bad(float T) {
    return (T != T) || T < 0.0f || T == INFINITY || (T > 0.0f && T < FLT_MIN);
}

template <typename E>
__device__ void resolve(const VerifyArgs& a, int b) {
    __shared__ int shi[kWaves];
    const int K = a.K, V = a.V;
    const int tid = threadIdx.x;
    const float T = a.temperature ? a.temperature[b] : 0.0f;
    const bool sampled = !(T == 0.0f);
    const int32_t* x = a.tokens + (int64_t)b * K;

    // ---- validation: every row read, every token, every uniform ----
    int err = 0;
    if (tid == 0 && temperature_bad(T)) err |= kSeqErrTemperature;
    for (int t = tid; t < K; t += kThreads) {
        const int xt = x[t];
        if (xt < 0 || xt >= V) err |= kSeqErrToken;
    }
    const double invT = sampled ? 1.0 / (double)T : 0.0;
    for (int j = tid; j < a.R; j += kThreads) {
        if (j > K && !sampled) continue;
        float m;
        if (sampled) {
            double S;
            merge_sampled(a, b, j, invT, m, S);
        } else {
            int i;
            merge_greedy(a, b, j, m, i);
        }
        if (row_bad(m, sampled)) err |= kSeqErrLogit;
    }
    if (sampled) {
        const float* u = a.uniforms + (int64_t)b * (K + 1);
        for (int t = tid; t <= K; t += kThreads) {
            const float ut = u[t];
            if (!(ut >= 0.0f && ut < 1.0f)) err |= kSeqErrUniform;
        }
    }
    err = block_or(err, shi);

    int32_t* tok = a.out_tokens + (int64_t)b * (K + 1);
    float* op = a.out_p ? a.out_p + (int64_t)b * K : nullptr;
    float* oq = a.out_q ? a.out_q + (int64_t)b * K : nullptr;
    if (err) {
        for (int t = tid; t <= K; t += kThreads) tok[t] = -1;
        for (int t = tid; t < K; t += kThreads) {
            if (op) op[t] = __builtin_nanf("");
            if (oq) oq[t] = __builtin_nanf("");
        }
        if (tid == 0) {
            a.out_n[b] = -1;
            a.out_status[b] = err;
            a.desc[b].mode = kModeNone;
        }
        return;
    }

    // ---- first position that fails ----
    int first = K;
    if (!sampled) {
        for (int t = tid; t < K; t += kThreads) {
            float m;
            int i;
            merge_greedy(a, b, t, m, i);
            if (i != x[t]) first = min(first, t);
            if (op) op[t] = __builtin_nanf("");
            if (oq) oq[t] = __builtin_nanf("");
        }
    } else {
        const float* u = a.uniforms + (int64_t)b * (K + 1);
        for (int t = tid; t < K; t += kThreads) {
            const int xt = x[t];
            float mt, md;
            double St, Sd;
            merge_sampled(a, b, t, invT, mt, St);
            merge_sampled(a, b, K + 1 + t, invT, md, Sd);
            const double zt = (double)Logit<E>::at(target_row<E>(a, b, t), xt);
            const double zd = (double)Logit<E>::at(draft_row<E>(a, b, t), xt);
            const double lp = (zt - (double)mt) / (double)T - log(St);
            const double lq = (zd - (double)md) / (double)T - log(Sd);
            if (op) op[t] = (float)exp(lp);
            if (oq) oq[t] = (float)exp(lq);
            // r < p/q, in log space; q = 0 with p > 0 accepts, p = 0 rejects
            const double ut = (double)u[t];
            bool accept;
            if (lp == -INFINITY) accept = false;
            else if (lq == -INFINITY) accept = true;
            else if (ut == 0.0) accept = true;
            else accept = log(ut) < lp - lq;
            if (!accept) first = min(first, t);
        }
    }
    const int n = block_min(first, shi);

    for (int t = tid; t <= K; t += kThreads) tok[t] = t < n ? x[t] : -1;
    __syncthreads();  // the -1 at tok[n] lands before the greedy token below
    if (tid == 0) {
        a.out_n[b] = n;
        a.out_status[b] = 0;
        SeqDesc d;
        d.n = n;
        d.T = T;
        d.status = 0;
        d.pad = 0;
        d.md = 0.0f;
        d.u = 0.0f;
        if (!sampled) {
            float m;
            int i;
            merge_greedy(a, b, n, m, i);
            tok[n] = i;
            d.mode = kModeNone;
            d.mt = m;
        } else {
            double S;
            merge_sampled(a, b, n, invT, d.mt, S);
            if (n < K) {
                merge_sampled(a, b, K + 1 + n, invT, d.md, S);
                d.mode = kModeResidual;
            } else {
                d.mode = kModeBonus;
            }
            d.u = a.uniforms[(int64_t)b * (K + 1) + K];
        }
        a.desc[b] = d;
    }
}

// ------------------------------------------------------------------------------------
// kernel
// ------------------------------------------------------------------------------------

template <typename E>
__global__ __launch_bounds__(kThreads) void pass1_kernel(VerifyArgs a) {
    __shared__ int sh_last;
    const int64_t blk = blockIdx.x;
    const int r = (int)(blk / a.nchunk1);
    const int c = (int)(blk - (int64_t)r * a.nchunk1);
    const int b = r / a.R;
    const int j = r - b * a.R;
    const float T = a.temperature ? a.temperature[b] : 0.0f;
    const bool sampled = !(T == 0.0f);
    RowPartial* out = a.part1 + blk;

    if (j <= a.K || sampled) {
        const E* row = j <= a.K ? target_row<E>(a, b, j) : draft_row<E>(a, b, j - a.K - 1);
        const int lo = c * a.ch1;
        const int hi = min(a.V, lo + a.ch1);
        if (sampled) tile_sumexp<E>(row, lo, hi, T, out);
        else tile_argmax<E>(row, lo, hi, out);
    }

    // last-tile-done: release this tile's partial, count it, acquire all partials
    if (threadIdx.x == 0) {
        const uint32_t tiles = (uint32_t)a.R * (uint32_t)a.nchunk1;
        __threadfence();
        const uint32_t old = atomicInc(&a.cnt1[b], tiles - 1);  // wraps to 0 on the last
        sh_last = (old == tiles - 1);
    }
    __syncthreads();
    if (sh_last) {
        __threadfence();
        resolve<E>(a, b);
    }
}

// Zero the per-sequence completion counters of pass 1 and pass 2 (a fill kernel rather
// than a memset node, so that the call stays safe to capture in a graph).
__global__ __launch_bounds__(kThreads) void zero_counters_kernel(uint32_t* c1, uint32_t* c2, int B) {
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i < B) {
        c1[i] = 0u;
        c2[i] = 0u;
    }
}

}  // namespace

int launch_zero_counters(const VerifyArgs& a, void* stream) {
    if (a.B == 0) return 0;
    const int blocks = (a.B + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(zero_counters_kernel, dim3(blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), a.cnt1, a.cnt2, a.B);
    return (int)hipGetLastError();
}

int launch_pass1(const VerifyArgs& a, int bf16, void* stream) {
    const int64_t blocks = (int64_t)a.B * a.R * a.nchunk1;
    if (blocks == 0) return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (bf16)
        hipLaunchKernelGGL(pass1_kernel<uint16_t>, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(pass1_kernel<float>, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    return (int)hipGetLastError();
}

}  // namespace sv
