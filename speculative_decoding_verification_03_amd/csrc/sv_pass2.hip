// Pass 2 of the verify step: the one categorical draw of each sampled sequence.
//
// After a rejection at position n the draw uses (p_n - q_n)+, the positive part of
// the pointwise difference over the whole vocabulary ("A Regra de Exatidão" on the
// lesson page "Decodificação Especulativa e EAGLE"; the livestream "IA local 202"
// describes the same clamp-and-normalise at [12:30]).  After K acceptances it uses p_K
// (the bonus token, "O Conceito" step 4).  Only the row pair (or the one row) of that
// draw is read again.
//
// Everything here is fp64: normalisers, weights and prefix sums.  An fp32 weight
// carries a relative error near 1e-7, which at V ~ 1.5e5 moves CDF edges by far more
// than the width of most cells, so fp32 would change the drawn token on a visible
// fraction of draws; fp64 keeps those changes below 1e-9 per draw.
//
//   p2_norm_kernel   (residual only) per chunk: sum exp((zt - mt)/T), sum exp((zd - md)/T)
//   p2_sample_kernel per chunk and wave: sums of the draw weights over contiguous
//                    sub-chunks; the workgroup that finishes the last chunk of a
//                    sequence scans the sub-chunk sums, finds the sub-chunk holding
//                    u * S and scans inside it: token = min{ i : C_i > u * S }.
#include <float.h>
#include <hip/hip_runtime.h>
#include <math.h>

#include "sv_common.h"
#include "sv_device.h"

namespace sv {

namespace {

template <typename E>
struct DrawRows {
    const E* t;     // target row of the draw
    const E* d;     // draft row (residual only)
    double mt, md;  // row maxima
    double invT;
    double inv_sp, inv_sq;  // 1 / fp64 normalisers (residual only)
    int residual;           // 1: (p - q)+, 0: exp((zt - mt)/T) (bonus, or fallback to p)

    __device__ __forceinline__ double weight(int i) const {
        const double et = exp(((double)Logit<E>::at(t, i) - mt) * invT);
        if (!residual) return et;
        const double ed = exp(((double)Logit<E>::at(d, i) - md) * invT);
        const double w = et * inv_sp - ed * inv_sq;
        return w > 0.0 ? w : 0.0;
    }
};

template <typename E>
__device__ __forceinline__ DrawRows<E> draw_rows(const VerifyArgs& a, int b, const SeqDesc& d) {
    DrawRows<E> r;
    r.t = static_cast<const E*>(a.target) + ((int64_t)b * (a.K + 1) + d.n) * a.V;
    r.residual = d.mode == kModeResidual;
    r.d = r.residual ? static_cast<const E*>(a.draft) + ((int64_t)b * a.K + d.n) * a.V : nullptr;
    r.mt = d.mt;
    r.md = d.md;
    r.invT = 1.0 / (double)d.T;
    r.inv_sp = 1.0;
    r.inv_sq = 1.0;
    return r;
}

// Smallest i in [lo, hi) with base + (w_lo + ... + w_i) > target, each thread scanning a
// contiguous run.  standalone: base = 0 and target = u * (sum over the range).  If no
// index qualifies (rounding), the last index with positive weight; -1 if there is none.
template <typename E>
__device__ int block_search(const DrawRows<E>& r, int lo, int hi, double base, double target,
                            bool standalone, double u) {
    __shared__ double shd[kWaves];
    __shared__ int shi[kWaves];
    const int n = hi - lo;
    const int run = (n + kThreads - 1) / kThreads;
    const int a0 = min(hi, lo + (int)threadIdx.x * run);
    const int a1 = min(hi, a0 + run);
    double s = 0.0;
    for (int i = a0; i < a1; ++i) s += r.weight(i);
    double tot;
    const double ex = block_exclusive_scan(s, tot, shd);
    if (standalone) {
        base = 0.0;
        target = u * tot;
    }
    double acc = base + ex;
    int found = 0x7fffffff, lastpos = -1;
    for (int i = a0; i < a1; ++i) {
        const double w = r.weight(i);
        if (w > 0.0) lastpos = i;
        acc += w;
        if (found == 0x7fffffff && acc > target) found = i;
    }
    int f = block_min(found, shi);
    if (f == 0x7fffffff) f = block_max(lastpos, shi);
    return f;
}

template <typename E>
__device__ void final_draw(const VerifyArgs& a, int b, const SeqDesc& d, DrawRows<E> r) {
    __shared__ double shd[kWaves];
    __shared__ int shi[kWaves];
    __shared__ double sh_base;
    const int tid = threadIdx.x;
    const int nsub = a.nchunk2 * kWaves;
    const int sub = a.ch2 / kWaves;
    const double* e = a.part2b + (int64_t)b * nsub;
    int status = d.status;
    const double u = (double)d.u;

    // total draw mass, by the same tiled scan the search below repeats
    double carry = 0.0;
    for (int t0 = 0; t0 < nsub; t0 += kThreads) {
        const double v = (t0 + tid < nsub) ? e[t0 + tid] : 0.0;
        double tot;
        block_exclusive_scan(v, tot, shd);
        carry += tot;
    }
    const double total = carry;

    int y;
    if (!(total > 0.0)) {
        // Residual with zero fp64 mass (exact arithmetic rules it out): draw from p_n.
        status |= kSeqNoteFallback;
        r.residual = 0;
        y = block_search(r, 0, a.V, 0.0, 0.0, true, u);
    } else {
        const double target = u * total;
        carry = 0.0;
        int hit = 0x7fffffff;
        for (int t0 = 0; t0 < nsub; t0 += kThreads) {
            const int k = t0 + tid;
            const double v = (k < nsub) ? e[k] : 0.0;
            double tot;
            const double ex = block_exclusive_scan(v, tot, shd);
            const double incl = carry + ex + v;
            // a sub-chunk without mass never holds the first crossing (guards rounding)
            const int f = block_min((k < nsub && v > 0.0 && incl > target) ? k : 0x7fffffff, shi);
            if (f != 0x7fffffff) {
                if (k == f) sh_base = carry + ex;
                __syncthreads();
                hit = f;
                break;
            }
            carry += tot;
        }
        double base = 0.0, tgt = target;
        if (hit == 0x7fffffff) {
            // rounding put u*S past every prefix: the last sub-chunk with mass, last index
            int last = -1;
            for (int t0 = 0; t0 < nsub; t0 += kThreads) {
                const int k = t0 + tid;
                last = max(last, (k < nsub && e[k] > 0.0) ? k : -1);
            }
            hit = block_max(last, shi);
            tgt = INFINITY;
            status |= kSeqNoteFallback;
        } else {
            base = sh_base;
        }
        const int c = hit / kWaves, w = hit % kWaves;
        const int lo = min(a.V, c * a.ch2 + w * sub);
        const int hi = min(a.V, lo + sub);
        y = block_search(r, lo, hi, base, tgt, false, u);
    }
    if (tid == 0) {
        a.out_tokens[(int64_t)b * (a.K + 1) + d.n] = y;
        a.out_status[b] = status;
    }
}

template <typename E>
__global__ __launch_bounds__(kThreads) void p2_norm_kernel(VerifyArgs a) {
    __shared__ double shd[kWaves];
    const int b = blockIdx.x / a.nchunk2;
    const int c = blockIdx.x - b * a.nchunk2;
    const SeqDesc d = a.desc[b];
    if (d.mode != kModeResidual) return;  // whole workgroup
    const DrawRows<E> r = draw_rows<E>(a, b, d);
    const int lo = c * a.ch2;
    const int hi = min(a.V, lo + a.ch2);
    double sp = 0.0, sq = 0.0;
    for (int i = lo + threadIdx.x; i < hi; i += kThreads) {
        sp += exp(((double)Logit<E>::at(r.t, i) - r.mt) * r.invT);
        sq += exp(((double)Logit<E>::at(r.d, i) - r.md) * r.invT);
    }
    sp = block_sum(sp, shd);
    sq = block_sum(sq, shd);
    if (threadIdx.x == 0) {
        NormPartial np;
        np.sp = sp;
        np.sq = sq;
        a.part2a[(int64_t)b * a.nchunk2 + c] = np;
    }
}

template <typename E>
__global__ __launch_bounds__(kThreads) void p2_sample_kernel(VerifyArgs a) {
    __shared__ int sh_last;
    __shared__ double sh_inv[2];
    const int b = blockIdx.x / a.nchunk2;
    const int c = blockIdx.x - b * a.nchunk2;
    const SeqDesc d = a.desc[b];
    if (d.mode == kModeNone) return;  // whole workgroup, and every workgroup of b
    DrawRows<E> r = draw_rows<E>(a, b, d);
    if (r.residual) {
        if (threadIdx.x == 0) {
            const NormPartial* np = a.part2a + (int64_t)b * a.nchunk2;
            double sp = 0.0, sq = 0.0;
            for (int k = 0; k < a.nchunk2; ++k) {
                sp += np[k].sp;
                sq += np[k].sq;
            }
            sh_inv[0] = 1.0 / sp;
            sh_inv[1] = 1.0 / sq;
        }
        __syncthreads();
        r.inv_sp = sh_inv[0];
        r.inv_sq = sh_inv[1];
    }
    // each wave: one contiguous sub-chunk of this chunk
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int sub = a.ch2 / kWaves;
    const int lo = min(a.V, c * a.ch2 + w * sub);
    const int hi = min(a.V, lo + sub);
    double acc = 0.0;
    for (int i = lo + lane; i < hi; i += 64) acc += r.weight(i);
    acc = wave_sum(acc);
    if (lane == 0) a.part2b[((int64_t)b * a.nchunk2 + c) * kWaves + w] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        const uint32_t old = atomicInc(&a.cnt2[b], (uint32_t)a.nchunk2 - 1);
        sh_last = (old == (uint32_t)a.nchunk2 - 1);
    }
    __syncthreads();
    if (sh_last) {
        __threadfence();
        final_draw<E>(a, b, d, r);
    }
}

}  // namespace

int launch_pass2(const VerifyArgs& a, int bf16, void* stream) {
    const int64_t blocks = (int64_t)a.B * a.nchunk2;
    if (blocks == 0) return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (bf16) {
        hipLaunchKernelGGL(p2_norm_kernel<uint16_t>, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
        hipLaunchKernelGGL(p2_sample_kernel<uint16_t>, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    } else {
        hipLaunchKernelGGL(p2_norm_kernel<float>, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
        hipLaunchKernelGGL(p2_sample_kernel<float>, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    }
    return (int)hipGetLastError();
}

}  // namespace sv
