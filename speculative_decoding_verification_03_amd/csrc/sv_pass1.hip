// Pass 1 of the verify step: stream every logit row a sequence needs exactly once.
//
// Rows read: target rows t = 0..K of every sequence, draft rows t = 0..K-1 of sampled
// sequences.  Greedy rows keep the maximum and its lowest index (the temperature-0 rule,
// "Caso ganancioso" on the lesson page "Decodificação Especulativa e EAGLE").  Sampled
// rows keep the maximum m and S = sum_i exp((z_i - m) / T): the normaliser of the
// temperature softmax of that page's "Desenvolva" listing.
//
// One workgroup per (row, chunk) tile of about 76 KB.  Each lane keeps kU or kUDeep 16-byte
// non-temporal loads in flight; the tail of a tile is handled by masking lanes to -inf,
// which adds nothing to a sum and never wins a maximum.  Sampled tiles evaluate
// 2^(z * c2 - R) with one FMA (the product is exact inside the FMA, so the only rounding
// is that of the small result) and v_exp_f32, against a per-lane reference R that moves
// up only when an element exceeds it by 2^32; 8-element sums are taken pairwise in fp32
// and accumulated in fp64.  The kernel carries no resolve code, so it keeps few registers
// and full occupancy.
#include <float.h>
#include <hip/hip_runtime.h>
#include <math.h>

#include "sv_common.h"
#include "sv_device.h"

namespace sv {

namespace {

constexpr double kLog2eD = 1.4426950408889634;
constexpr float kRescaleLog2 = 32.0f;
constexpr float kSkipLog2 = 50.0f;
// 16-byte loads in flight per lane: kU for small grids (8 waves per SIMD), kUDeep for
// large ones (4 waves per SIMD; a whole tile of at most kUDeep * kThreads vectors in one
// round of loads).  The deep variant's lower occupancy costs more in a short grid's last
// round than its longer queue saves, so it is taken from kDeepBlocks workgroups on, about
// 8 rounds of its resident workgroups (4 per CU on 256 CUs), and only for dense calls
// with sampled rows that read every row: all-greedy calls measured no faster with it, and
// in ragged and early-exit calls many workgroups of the grid find no row to read, so the
// grid's real work is short and it measured slower.
constexpr int kU = 4;
constexpr int kUDeep = 20;
constexpr int64_t kDeepBlocks = 8192;

struct SumExpAcc {
    float mx;   // NaN-propagating maximum of everything seen
    float R;    // reference, in log2 units: s = sum 2^(z * c2 - R)
    double s;
};

template <int N>
__device__ __forceinline__ float tree_sum(const float (&e)[N]) {
    if constexpr (N == 1) {
        return e[0];
    } else {
        float h[N / 2];
#pragma unroll
        for (int k = 0; k < N / 2; ++k) h[k] = e[2 * k] + e[2 * k + 1];
        return tree_sum(h);
    }
}

template <int N>
__device__ __forceinline__ void sumexp_vec(const float (&z)[N], float c2, SumExpAcc& a) {
    float tm = z[0];
#pragma unroll
    for (int k = 1; k < N; ++k) tm = nmax(tm, z[k]);
    a.mx = nmax(a.mx, tm);
    const float top = __builtin_fmaf(tm, c2, -a.R);
    if (top > kRescaleLog2) {
        // rare: move the reference up to this vector's maximum (exact in fp64)
        const float Rn = tm * c2;
        if (a.s != 0.0) a.s *= exp2((double)a.R - (double)Rn);
        a.R = Rn;
    }
    // the whole wave's terms are below 2^-kSkipLog2 of its references (each reference is at
    // most the row maximum times c2): over any row they add less than V 2^-kSkipLog2
    // relative to the sum, far below the fp32 rounding of the terms themselves
    if (__all(top < -kSkipLog2)) return;
    float e[N];
#pragma unroll
    for (int k = 0; k < N; ++k) e[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(z[k], c2, -a.R));
    a.s += (double)tree_sum(e);
}

struct ArgmaxAcc {
    float mx;   // strict running maximum (NaN never enters)
    int idx;    // lowest index reaching mx
    int bad;    // a NaN was seen
};

template <int N>
__device__ __forceinline__ void argmax_vec(const float (&z)[N], int base, ArgmaxAcc& a) {
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
        a.idx = base + k0;
    }
}

// Streams [lo, hi) of `row`: a scalar head up to 16-byte alignment, then 16-byte vectors
// in tiles of U per lane (lanes past the end see -inf), then a scalar tail.  fvec is
// called with VEC elements and the index of the first; fscal with one element.  Each
// lane sees its elements in increasing index order.
template <typename E, int U, class FV, class FS>
__device__ __forceinline__ void stream_tile(const E* row, int lo, int hi, FV&& fvec, FS&& fscal) {
    constexpr int VEC = Logit<E>::kVec;
    const int tid = threadIdx.x;
    const uintptr_t addr = reinterpret_cast<uintptr_t>(row + lo);
    int head = (int)(((16 - (addr & 15)) & 15) / sizeof(E));
    if (head > hi - lo) head = hi - lo;
    if (tid < head) fscal(Logit<E>::at(row, lo + tid), lo + tid);
    const int body0 = lo + head;
    const int nvec = (hi - body0) / VEC;
    const E* p = row + body0;
    for (int v0 = 0; v0 < nvec; v0 += U * kThreads) {
        u32x4 raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * kThreads + tid;
            raw[u] = v < nvec ? load16(p + (int64_t)v * VEC) : Logit<E>::neg_inf16();
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float z[VEC];
            Logit<E>::unpack(raw[u], z);
            fvec(z, body0 + (v0 + u * kThreads + tid) * VEC);
        }
    }
    const int i = body0 + nvec * VEC + tid;
    if (i < hi) fscal(Logit<E>::at(row, i), i);
}

// xi: the position of the row's draft token if it lies in this tile, else -1; its logit
// goes into the partial for the resolve.
template <typename E, int U>
__device__ void tile_sumexp(const E* row, int lo, int hi, float c2, int xi, RowPartial* out) {
    __shared__ float shf[kWaves];
    __shared__ double shd[kWaves];
    SumExpAcc a{-INFINITY, -FLT_MAX, 0.0};
    stream_tile<E, U>(
        row, lo, hi, [&](const float(&z)[Logit<E>::kVec], int) { sumexp_vec(z, c2, a); },
        [&](float z, int) {
            const float zz[1] = {z};
            sumexp_vec(zz, c2, a);
        });
    const float m = block_nmax(a.mx, shf);
    // rebase every lane's sum from its reference R to the tile maximum, in fp64
    double s = 0.0;
    if (a.s != 0.0) s = a.s * exp2((double)a.R - (double)m * (double)c2);
    s = block_sum(s, shd);
    if (threadIdx.x == 0) {
        RowPartial r;
        r.m = m;
        r.idx = xi >= 0 ? __float_as_int(Logit<E>::at(row, xi)) : 0;
        r.s = s;
        *out = r;
    }
}

template <typename E, int U>
__device__ void tile_argmax(const E* row, int lo, int hi, RowPartial* out) {
    __shared__ float shv[kWaves];
    __shared__ int shi[kWaves];
    ArgmaxAcc a{-INFINITY, 0x7fffffff, 0};
    stream_tile<E, U>(
        row, lo, hi,
        [&](const float(&z)[Logit<E>::kVec], int base) { argmax_vec(z, base, a); },
        [&](float z, int i) {
            const float zz[1] = {z};
            argmax_vec(zz, i, a);
        });
    const int bad = block_or(a.bad, shi);
    float v = a.mx;
    int i = a.idx;
    block_argmax(v, i, shv, shi);
    if (threadIdx.x == 0) {
        RowPartial r;
        r.m = bad ? __builtin_nanf("") : v;
        r.idx = i;
        r.s = 0.0;
        *out = r;
    }
}

template <typename E, int U>
__global__ __launch_bounds__(kThreads) void pass1_kernel(VerifyArgs a, int b0) {
    const int64_t blk = blockIdx.x;
    if (a.deal) {
        // the draw deal starts empty: no entries (a descriptor's mode is its first field)
        // and zero counts; the grid has at least B workgroups
        const int64_t i = blk * kThreads + threadIdx.x;
        if (i < a.B) reinterpret_cast<int32_t*>(static_cast<char*>(a.deal_desc) + i * kSeqDescBytes)[0] = kModeNone;
        else if (i < (int64_t)a.B + 2) a.deal[i - a.B] = 0;
    }
    if (a.u_gen) {
        // the uniforms of the call, one per thread of the first workgroups
        const int64_t i = blk * kThreads + threadIdx.x;
        if (i < (int64_t)a.B * (a.K + 1))
            a.u_gen[i] = philox_uniform(a.seed, a.domain, (uint64_t)(i % (a.K + 1)),
                                        (uint64_t)(i / (a.K + 1)), a.step);
    }
    const int r = (int)(blk / a.nchunk1);
    const int c = (int)(blk - (int64_t)r * a.nchunk1);
    const int b = b0 + r / a.R;
    const int j = r % a.R;  // 0..K target rows, K+1..2K draft rows (K the bound)
    const float T = a.temperature ? a.temperature[b] : 0.0f;
    const bool sampled = !(T == 0.0f);
    if (j > a.K && !sampled) return;  // greedy sequences never read draft rows
    const SeqRows s = seq_rows(a, b);
    const bool is_target = j <= a.K;
    const int t = is_target ? j : j - a.K - 1;
    if (t > s.K || (!is_target && t == s.K)) return;  // past this sequence's drafts, or bad offsets
    if (a.limit) {
        // early exit: this round's positions of the sequences still going
        if (t < a.t0 || t >= a.t1) return;
        if (a.t0 > 0 && a.limit[b] != a.t0) return;
    }
    const E* row = is_target ? static_cast<const E*>(a.target) + (s.t0 + t) * a.V
                             : static_cast<const E*>(a.draft) + (s.d0 + t) * a.V;
    const int lo = c * a.ch1;
    const int hi = min(a.V, lo + a.ch1);
    RowPartial* out = a.part1 + ((int64_t)b * a.R + j) * a.nchunk1 + c;
    if (sampled) {
        // target row t < K_b or draft row t: the draft token x_t, when it falls in this tile
        int xi = -1;
        if (t < s.K) {
            const int x = a.tokens[s.d0 + t];
            if (x >= lo && x < hi) xi = x;
        }
        tile_sumexp<E, U>(row, lo, hi, (float)(kLog2eD / (double)T), xi, out);
    }
    else tile_argmax<E, U>(row, lo, hi, out);
}

}  // namespace

int launch_pass1(const VerifyArgs& a, int bf16, int b0, int b1, void* stream) {
    const int64_t blocks = (int64_t)(b1 - b0) * a.R * a.nchunk1;
    if (blocks <= 0) return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 g((unsigned)blocks), t(kThreads);
    if (blocks >= kDeepBlocks && a.temperature && !a.cu && !a.limit) {
        if (bf16) hipLaunchKernelGGL((pass1_kernel<uint16_t, kUDeep>), g, t, 0, s, a, b0);
        else hipLaunchKernelGGL((pass1_kernel<float, kUDeep>), g, t, 0, s, a, b0);
    } else {
        if (bf16) hipLaunchKernelGGL((pass1_kernel<uint16_t, kU>), g, t, 0, s, a, b0);
        else hipLaunchKernelGGL((pass1_kernel<float, kU>), g, t, 0, s, a, b0);
    }
    return (int)hipGetLastError();
}

}  // namespace sv
