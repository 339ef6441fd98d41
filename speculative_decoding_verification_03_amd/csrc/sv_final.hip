// Pass 2 of the verify step: the final kernel, the draw of each sampled sequence from
// the partials of its segments.
#include "sv_draw.h"

namespace sv {

namespace {

// Smallest i in [lo, hi) (hi - lo <= PER * NT, lo a multiple of 16 bytes' worth of
// logits) with base + (w_lo + ... + w_i) > target, in one tile: each of the NT threads
// takes PER consecutive positions (a thread-local prefix, then a workgroup exclusive scan
// of the thread totals).  If no index qualifies (rounding), the last index with positive
// weight; -1 if none.
template <typename E, int NT, int PER>
__device__ __forceinline__ int segment_search(const DrawRows<E>& r, int lo, int hi, double base, double target) {
    constexpr int VEC = Logit<E>::kVec;
    constexpr int NW = NT / 64;
    static_assert(PER % VEC == 0, "whole vectors per thread");
    __shared__ double shd[NW];
    __shared__ int shi[NW];
    const int i0 = lo + PER * (int)threadIdx.x;
    double w[PER];
    double run = 0.0;
    int lastpos = -1;
#pragma unroll
    for (int v = 0; v < PER; v += VEC) {
        float zt[VEC], zd[VEC];
        load_vec(r.t, i0 + v, hi, r.vec_ok, zt);
        if (r.residual) load_vec(r.d, i0 + v, hi, r.vec_ok, zd);
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            w[v + k] = r.weight(zt[k], r.residual ? zd[k] : 0.0f);
            run += w[v + k];
            if (w[v + k] > 0.0) lastpos = i0 + v + k;
        }
    }
    double tot;
    double acc = base + block_exclusive_scan<NW>(run, tot, shd);
    int found = 0x7fffffff;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        acc += w[k];
        if (found == 0x7fffffff && w[k] > 0.0 && acc > target) found = i0 + k;
    }
    const int f = block_min<NW>(found, shi);
    if (f != 0x7fffffff) return f;
    return block_max<NW>(lastpos, shi);
}

// Sums of two doubles and an OR over the workgroup (NW waves), with one round of barriers.
// sh holds 2 NW doubles, shi NW ints.
template <int NW>
__device__ __forceinline__ void block_sum2_or(double& x, double& y, int& o, double* sh, int* shi) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    x = wave_sum(x);
    y = wave_sum(y);
    o = wave_or(o);
    if (lane == 0) {
        sh[w] = x;
        sh[NW + w] = y;
        shi[w] = o;
    }
    __syncthreads();
    x = sh[0];
    y = sh[NW];
    o = shi[0];
#pragma unroll
    for (int k = 1; k < NW; ++k) {
        x += sh[k];
        y += sh[NW + k];
        o |= shi[k];
    }
    __syncthreads();
}

// The draw of sequence b by a workgroup of NT threads when the sequence has at most NT
// segments of L positions (L <= PER * NT): thread k holds segment k's partial (part[k],
// bkt[k * kBuckets ...]), loaded once; one reduction, one scan, one segment search.
template <typename E, int NT, int PER>
__device__ __forceinline__ void final_seq_small(const VerifyArgs& a, DrawRows<E> r, const SeqDesc& d, int b,
                                                DrawPartial dp, Bucket bk0, const Bucket* bkt, int nsub, int L) {
    constexpr int NW = NT / 64;
    __shared__ double shd[2 * NW];
    __shared__ int shi[NW];
    __shared__ double sh_base;
    const int tid = threadIdx.x;
    const double u = (double)d.u;
    int status = 0;

    // dp, bk0: the partial and first bucket of segment k of this thread.  Up to 64
    // segments every wave holds all of them (k = lane) and reduces and scans them itself,
    // with no barrier; otherwise thread k holds segment k and the workgroup combines.
    const int lane = tid & 63;
    const bool per_wave = nsub <= 64;
    const int k = per_wave ? lane : tid;
    if (k >= nsub) dp = DrawPartial{};
    double sp = dp.sp, sq = dp.sq;
    int over = dp.nbkt > kBuckets;
    if (per_wave) {
        sp = wave_sum(sp);
        sq = wave_sum(sq);
        over = wave_or(over);
    } else {
        block_sum2_or<NW>(sp, sq, over, shd, shi);
    }
    // the classification by the pass-1 estimate stands if the exact threshold
    // T ln(S_p/S_q) + refA - refB lies well inside the bracket
    bool exact_ok = sp > 0.0;
    if (r.residual) {
        exact_ok = exact_ok && sq > 0.0 && !over;
        if (exact_ok) {
            const double T = (double)d.T;
            const double tau = T * (log(sp) - log(sq)) + (r.refA - r.refB);
            const double mid = 0.5 * (r.tau_lo + r.tau_hi);
            const double half = 0.5 * (r.tau_hi - r.tau_lo);
            exact_ok = fabs(tau - mid) <= 0.5 * half && half > 1e-12 * (fabs(mid) + 1.0);
        }
    }
    r.inv_sp = 1.0 / sp;
    r.inv_sq = r.residual ? 1.0 / sq : 1.0;

    int y = -1;
    if (!exact_ok) {
        // too many undecided positions, or the estimate was off: one exact sweep
        y = block_search<E, NT>(r, 0, a.V, 0.0, 0.0, true, u);
    } else {
        // this segment's mass in the units of the draw: its certain part and, per bucket
        // of undecided positions (one residual sign each), the bucket's residual if positive
        double v = 0.0;
        if (k < nsub) {
            if (!r.residual) {
                v = dp.sp;
            } else {
                v = dp.A * r.inv_sp - dp.B * r.inv_sq;
                const Bucket* bk = bkt + k * kBuckets;
                for (int q = 0; q < dp.nbkt; ++q) {
                    const Bucket bq = q == 0 ? bk0 : bk[q];
                    const double t = bq.a * r.inv_sp - bq.b * r.inv_sq;
                    if (t > 0.0) v += t;
                }
                v = v > 0.0 ? v : 0.0;
            }
        }
        double total, ex;
        if (per_wave) {
            const double incl = wave_inclusive_scan(v);
            total = __shfl(incl, 63, 64);
            ex = __shfl_up(incl, 1, 64);
            if (lane == 0) ex = 0.0;
        } else {
            ex = block_exclusive_scan<NW>(v, total, shd);
        }
        if (total > 0.0) {
            const double target = u * total;
            // a segment without mass never holds the first crossing (guards rounding)
            const bool crosses = k < nsub && v > 0.0 && ex + v > target;
            const bool mass = k < nsub && v > 0.0;
            int hit;
            double tgt = target, base;
            if (per_wave) {
                const uint64_t mc = __ballot(crosses), mm = __ballot(mass);
                if (mc) {
                    hit = __ffsll((unsigned long long)mc) - 1;
                } else {
                    // rounding put u*W past every prefix: the last segment with mass, last index
                    hit = 63 - __clzll((long long)mm);
                    tgt = INFINITY;
                    status |= kSeqNoteFallback;
                }
                base = __shfl(ex, hit, 64);
            } else {
                hit = block_min<NW>(crosses ? k : 0x7fffffff, shi);
                if (hit == 0x7fffffff) {
                    hit = block_max<NW>(mass ? k : -1, shi);
                    tgt = INFINITY;
                    status |= kSeqNoteFallback;
                }
                if (tid == hit) sh_base = ex;
                __syncthreads();
                base = sh_base;
            }
            int lo, hi;
            seg_range(a.V, L, hit, lo, hi);
            y = segment_search<E, NT, PER>(r, lo, hi, base, tgt);
        }
    }
    if (y < 0) {
        // residual without fp64 mass (exact arithmetic rules it out): draw from p_n
        status |= kSeqNoteFallback;
        r.residual = 0;
        y = block_search<E, NT>(r, 0, a.V, 0.0, 0.0, true, u);
    }
    if (tid == 0) {
        a.out_tokens[d.trow] = y;
        a.out_status[b] = status;
    }
}

// The draw of sequence b from the partials of all its segments, by one workgroup.
template <typename E, int NT>
__device__ __forceinline__ void final_seq(const VerifyArgs& a, DrawRows<E> r, const SeqDesc& d, int b) {
    constexpr int NW = NT / 64;
    __shared__ double shd[NW];
    __shared__ int shi[NW];
    __shared__ double sh_base;
    const int tid = threadIdx.x;
    const int nsub = a.nseg;
    const int64_t e0 = (int64_t)b * a.nseg;
    const double u = (double)d.u;
    int status = 0;

    // fp64 normalisers; the classification by the pass-1 estimate stands if the exact
    // threshold T ln(S_p/S_q) + refA - refB lies well inside the bracket
    double sp = 0.0, sq = 0.0;
    int over = 0;
    for (int k = tid; k < nsub; k += NT) {
        const DrawPartial dp = a.part2[e0 + k];
        sp += dp.sp;
        sq += dp.sq;
        over |= dp.nbkt > kBuckets;
    }
    sp = block_sum<NW>(sp, shd);
    sq = block_sum<NW>(sq, shd);
    over = block_or<NW>(over, shi);
    bool exact_ok = sp > 0.0;
    if (r.residual) {
        exact_ok = exact_ok && sq > 0.0 && !over;
        if (exact_ok) {
            const double T = (double)d.T;
            const double tau = T * (log(sp) - log(sq)) + (r.refA - r.refB);
            const double mid = 0.5 * (r.tau_lo + r.tau_hi);
            const double half = 0.5 * (r.tau_hi - r.tau_lo);
            // keep half of the bracket as the margin, and stay far above fp64 rounding
            exact_ok = fabs(tau - mid) <= 0.5 * half && half > 1e-12 * (fabs(mid) + 1.0);
        }
    }
    r.inv_sp = 1.0 / sp;
    r.inv_sq = r.residual ? 1.0 / sq : 1.0;

    int y;
    if (!exact_ok) {
        // too many undecided positions, or the estimate was off: one exact sweep
        y = block_search<E, NT>(r, 0, a.V, 0.0, 0.0, true, u);
    } else {
        // mass of sub-chunk k in the units of the draw: its certain part and, per bucket of
        // undecided positions (one residual sign each), the bucket's residual if positive
        auto mass = [&](int k) -> double {
            const DrawPartial dp = a.part2[e0 + k];
            if (!r.residual) return dp.sp;
            double w = dp.A * r.inv_sp - dp.B * r.inv_sq;
            const Bucket* bk = a.bkt + (e0 + k) * kBuckets;
            for (int q = 0; q < dp.nbkt; ++q) {
                const double t = bk[q].a * r.inv_sp - bk[q].b * r.inv_sq;
                if (t > 0.0) w += t;
            }
            return w > 0.0 ? w : 0.0;
        };
        double carry = 0.0;
        for (int t0 = 0; t0 < nsub; t0 += NT) {
            const int k = t0 + tid;
            const double v = k < nsub ? mass(k) : 0.0;
            double tot;
            block_exclusive_scan<NW>(v, tot, shd);
            carry += tot;
        }
        const double total = carry;
        if (!(total > 0.0)) {
            y = -1;
        } else {
            const double target = u * total;
            carry = 0.0;
            int hit = 0x7fffffff;
            for (int t0 = 0; t0 < nsub; t0 += NT) {
                const int k = t0 + tid;
                const double v = k < nsub ? mass(k) : 0.0;
                double tot;
                const double ex = block_exclusive_scan<NW>(v, tot, shd);
                const double incl = carry + ex + v;
                // a sub-chunk without mass never holds the first crossing (guards rounding)
                const int f = block_min<NW>((k < nsub && v > 0.0 && incl > target) ? k : 0x7fffffff, shi);
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
                // rounding put u*W past every prefix: the last sub-chunk with mass, last index
                int last = -1;
                for (int t0 = 0; t0 < nsub; t0 += NT) {
                    const int k = t0 + tid;
                    if (k < nsub && mass(k) > 0.0) last = max(last, k);
                }
                hit = block_max<NW>(last, shi);
                tgt = INFINITY;
                status |= kSeqNoteFallback;
            } else {
                base = sh_base;
            }
            int lo, hi;
            seg_range(a.V, a.seg, hit, lo, hi);
            y = block_search<E, NT>(r, lo, hi, base, tgt, false, u);
        }
    }
    if (y < 0) {
        // residual without fp64 mass (exact arithmetic rules it out): draw from p_n
        status |= kSeqNoteFallback;
        r.residual = 0;
        y = block_search<E, NT>(r, 0, a.V, 0.0, 0.0, true, u);
    }
    if (tid == 0) {
        a.out_tokens[d.trow] = y;
        a.out_status[b] = status;
    }
}

// grid = sequences: the draw of each sampled sequence from the partials of all its segments.
// Weights as in the sweep: the sequence's table in LDS for bf16 values it covers, the fp64
// exponential otherwise.
template <typename E>
__global__ __launch_bounds__(kFinalThreads) void final_kernel(VerifyArgs a, int b0) {
    __shared__ double tab[kExpTable];
    __shared__ double wt[DrawLds<E>::kWt];
    const int b = b0 + (int)blockIdx.x;
    // bf16: the sequence's weight table comes in with the descriptor (whether it holds a
    // table is known once the descriptor is: unused otherwise)
    TableCopy<kFinalThreads> tc;
    if constexpr (sizeof(E) == 2) tc.load(a.wtab + (int64_t)b * kWtabLen);
    const SeqDesc d = reinterpret_cast<const SeqDesc*>(a.desc)[b];
    // the segment partials and first buckets load together with the descriptor
    const bool small = a.nseg <= kFinalThreads;
    const DrawPartial* part = a.part2 + (int64_t)b * a.nseg;
    const Bucket* bkt = a.bkt + (int64_t)b * a.nseg * kBuckets;
    // the segment of this thread in final_seq_small: its lane up to 64 segments
    const int k = min(a.nseg <= 64 ? (int)(threadIdx.x & 63) : (int)threadIdx.x, a.nseg - 1);
    const DrawPartial dp = part[k];
    const Bucket bk0 = bkt[k * kBuckets];
    if (d.mode == kModeNone) return;  // whole workgroup
    if constexpr (sizeof(E) == 2) tc.store(wt);
    exp2_table_init(tab);  // its barrier also publishes wt
    const DrawRows<E> r = draw_rows<E>(a, d, tab, sizeof(E) == 2 ? wt : nullptr);
    if (small)
        final_seq_small<E, kFinalThreads, kSeg / kFinalThreads>(a, r, d, b, dp, bk0, bkt, a.nseg, a.seg);
    else
        final_seq<E, kFinalThreads>(a, r, d, b);
}

}  // namespace

int launch_final(const VerifyArgs& a, int bf16, int b0, int b1, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (bf16)
        hipLaunchKernelGGL(final_kernel<uint16_t>, dim3((unsigned)(b1 - b0)), dim3(kFinalThreads), 0, s, a, b0);
    else
        hipLaunchKernelGGL(final_kernel<float>, dim3((unsigned)(b1 - b0)), dim3(kFinalThreads), 0, s, a, b0);
    return (int)hipGetLastError();
}

}  // namespace sv
