// The draft-side sampler: one draw per row from softmax(z / T), argmax at T = 0 (the
// draft's temperature softmax and categorical draw of the "Desenvolva" listing on the
// lesson page "Decodificação Especulativa e EAGLE").
//
// One 1024-thread workgroup per row.  A sampled row is read once: its weights are taken
// against a provisional reference, kSampleLift binary orders of weight above R0 (the maximum
// of the row's first vectors).  Against the row maximum M that scales every weight by one
// common factor and so leaves the inverse CDF where it is.  The fp64 weights are summed per
// kSampleSeg-position segment (one wave per segment), then the segment sums are scanned for
// u * W and the segment that holds it is searched: token = min{ i : C_i > u * W }, C the
// prefix sums in index order.  The lift keeps M's weight at 2^-kSampleLift or more, so every
// weight within 2^-75 of it stays a normal fp64 number.
//
// The common path takes no per-element maximum: only the values read one by one pass
// through a maximum mr (every value outside the bf16 weight table's magnitude range, NaN and
// the infinities among them, and all values of rows without the table).  NaN or +inf there
// is a data error.  Otherwise R0 <= M <= max(mr, kTabTop), which bounds |M| for the
// scaled-range rule, and a total W of at most kSampleSumMax = 2^900 bounds every weight, so
// no sum overflowed.  A row that fails either bound (a far outlier at a very low
// temperature, many values near a far maximum, a row that opens with kSampleThreads vectors
// of -inf, a temperature near the range limit) takes the slow path: a maximum pass for M,
// the checks on it, and the sums again against M.  Greedy rows, and rows with a bad
// temperature or uniform, take one argmax pass.
#include "sv_draw.h"

namespace sv {

namespace {

// Largest row total the common path keeps: no weight and no partial sum above it can have
// overflowed.
constexpr double kSampleSumMax = 0x1p900;
// Binary orders of weight between R0 and the provisional reference above it (at most
// 1022 - 75, so that weights within 2^-75 of the row maximum's are normal numbers).
constexpr double kSampleLift = 900.0;
// 2^5: every magnitude the bf16 weight table holds lies below it.
constexpr float kTabTop = 32.0f;
static_assert(kTabHi == 132u * 128u, "the table ends at biased exponent 132, magnitude 2^5");
// 16-byte vectors per lane of one whole bf16 segment
constexpr int kSegVecs = kSampleSeg / (64 * 8);
static_assert(kSampleSeg % (64 * 8) == 0, "sampler segments are whole waves of bf16 vectors");
static_assert(kSampleMaxSeg <= 2 * kSampleThreads, "the scan takes two segments per thread");

// A thread's NaN-propagating maximum of the row's values (the threads stride the row).
template <typename E, int NT>
__device__ __forceinline__ float row_nmax(const E* row, int V, bool vec_ok) {
    constexpr int VEC = Logit<E>::kVec;
    const int nvec = vec_ok ? V / VEC : 0;
    float m = -INFINITY;
    for (int v = threadIdx.x; v < nvec; v += NT) {
        float z[VEC];
        Logit<E>::unpack(load16(row + (int64_t)v * VEC), z);
#pragma unroll
        for (int k = 0; k < VEC; ++k) m = nmax(m, z[k]);
    }
    for (int i = nvec * VEC + threadIdx.x; i < V; i += NT) m = nmax(m, Logit<E>::at(row, i));
    return m;
}

// Loads of one whole bf16 segment of a lane (positions lo + (k*64 + lane)*8 .. +7).
__device__ __forceinline__ void seg_load(const uint16_t* row, int lo, int lane, u32x4 (&v)[kSegVecs]) {
#pragma unroll
    for (int k = 0; k < kSegVecs; ++k) v[k] = load16(row + lo + (k * 64 + lane) * 8);
}

// A lane's fp64 weight sum over its vectors of a whole bf16 segment (already loaded), with
// table weights; a vector holding a value outside the table (its sum turns NaN on a
// sentinel) is read again and summed with the exact weights.  mx: the lane's
// NaN-propagating maximum of the values of the vectors read again, updated.
__device__ __forceinline__ double seg_sum_tab(const DrawRows<uint16_t>& r, const u32x4 (&v)[kSegVecs], int lo,
                                              int lane, float& mx) {
    double s = 0.0;
    uint32_t again = 0;
#pragma unroll
    for (int k = 0; k < kSegVecs; ++k) {
        const uint32_t x4[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
        double sk = 0.0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t o0, o1;
            tab_offsets(x4[q], o0, o1);
            sk += tab_at(r.wt, o0);
            sk += tab_at(r.wt, o1);
        }
        if (sk != sk) again |= 1u << k;
        else s += sk;
    }
    while (again) {  // rare
        const int k = __ffs(again) - 1;
        again &= again - 1;
        const u32x4 w = load16(r.t + lo + (k * 64 + lane) * 8);
        const uint32_t x4[4] = {w.x, w.y, w.z, w.w};
        double sk = 0.0;
#pragma unroll 1
        for (int q = 0; q < 8; ++q) {
            const uint32_t h = (x4[q >> 1] >> (16 * (q & 1))) & 0xffffu;
            const float z = __uint_as_float(h << 16);
            mx = nmax(mx, z);
            sk += r.a_of(z);
        }
        s += sk;
    }
    return s;
}

// A lane's weight sum over positions [lo, hi) element by element (exact weights), and the
// NaN-propagating maximum of what it reads; positions past hi read -inf (weight 0).
template <typename E>
__device__ __forceinline__ double seg_sum_exact(const DrawRows<E>& r, int lo, int hi, int lane, float& mx) {
    constexpr int VEC = Logit<E>::kVec;
    double s = 0.0;
    for (int i0 = lo; i0 < hi; i0 += 64 * VEC) {
        float z[VEC];
        load_vec(r.t, i0 + lane * VEC, hi, r.vec_ok, z);
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            mx = nmax(mx, z[k]);
            s += r.a_of(z[k]);
        }
    }
    return s;
}

// Sums of the weights of every segment of the row into segsum, one wave per segment
// (segments w, w + NW, ...), and each lane's NaN-propagating maximum of the values read one
// by one: with the table (bf16, aligned rows) those of the vectors that hold a value outside
// it and of the row's tail, else every value.  With the table every whole segment's loads
// go out before the previous one is summed.  first: the wave's first whole segment, already
// loaded (when have_first).  Contains no barrier.
template <typename E, int NT>
__device__ __forceinline__ float row_segment_sums(const DrawRows<E>& r, int V, double* segsum, bool have_first,
                                                  const u32x4 (&first)[kSegVecs]) {
    constexpr int NW = NT / 64;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nseg = (V + kSampleSeg - 1) / kSampleSeg;
    float mx = -INFINITY;
    if constexpr (sizeof(E) == 2) {
        if (r.use_tab && r.vec_ok) {
            const uint16_t* t = reinterpret_cast<const uint16_t*>(r.t);
            const int nwhole = V / kSampleSeg;
            u32x4 cur[kSegVecs];
            if (w < nwhole) {
                if (have_first) {
#pragma unroll
                    for (int k = 0; k < kSegVecs; ++k) cur[k] = first[k];
                } else {
                    seg_load(t, w * kSampleSeg, lane, cur);
                }
            }
            for (int k = w; k < nseg; k += NW) {
                const int lo = k * kSampleSeg;
                double s;
                if (k < nwhole) {
                    u32x4 nxt[kSegVecs];
                    const bool more = k + NW < nwhole;
                    if (more) seg_load(t, (k + NW) * kSampleSeg, lane, nxt);
                    s = seg_sum_tab(r, cur, lo, lane, mx);
                    if (more) {
#pragma unroll
                        for (int q = 0; q < kSegVecs; ++q) cur[q] = nxt[q];
                    }
                } else {
                    s = seg_sum_exact(r, lo, V, lane, mx);
                }
                s = wave_sum(s);
                if (lane == 0) segsum[k] = s;
            }
            return mx;
        }
    }
    for (int k = w; k < nseg; k += NW) {
        const int lo = k * kSampleSeg;
        double s = seg_sum_exact(r, lo, min(V, lo + kSampleSeg), lane, mx);
        s = wave_sum(s);
        if (lane == 0) segsum[k] = s;
    }
    return mx;
}

// The segment that holds u * W, found by one wave from the segment sums in LDS (every wave
// that calls it gets the same bits): each lane sums a run of consecutive segments in index
// order, a wave scan gives the runs' prefix sums, and the first segment with mass whose
// prefix passes u * W is the hit.  If rounding puts u * W past every prefix, the hit is the
// last segment with mass and the target becomes +inf (fallback).  hit = -1 when W = 0.
struct SegHit {
    double total;   // W
    double base;    // sum of the segments before the hit
    double target;  // u * W, or +inf on the fallback
    int hit;
    bool fallback;
};

__device__ __forceinline__ SegHit seg_hit(const double* segsum, int nseg, double u) {
    const int lane = threadIdx.x & 63;
    const int per = (nseg + 63) / 64;
    const int k0 = min(nseg, lane * per), k1 = min(nseg, k0 + per);
    double run = 0.0;
    for (int k = k0; k < k1; ++k) run += segsum[k];
    const double incl = wave_inclusive_scan(run);
    double ex = __shfl_up(incl, 1, 64);
    if (lane == 0) ex = 0.0;
    SegHit h;
    h.total = __shfl(incl, 63, 64);
    h.base = 0.0;
    h.target = (double)u * h.total;
    h.hit = -1;
    h.fallback = false;
    if (!(h.total > 0.0)) return h;
    int first = 0x7fffffff, last = -1;
    double fbase = 0.0, lbase = 0.0, acc = ex;
    for (int k = k0; k < k1; ++k) {
        const double v = segsum[k];
        if (v > 0.0) {
            // a segment without mass never holds the first crossing (guards rounding)
            if (first == 0x7fffffff && acc + v > h.target) {
                first = k;
                fbase = acc;
            }
            last = k;
            lbase = acc;
        }
        acc += v;
    }
    h.hit = wave_min(first);
    if (h.hit != 0x7fffffff) {
        h.base = __shfl(fbase, h.hit / per, 64);
    } else {
        h.hit = wave_max(last);  // W > 0: some segment has mass
        h.base = __shfl(lbase, h.hit / per, 64);
        h.target = INFINITY;
        h.fallback = true;
    }
    return h;
}

// grid = rows, one workgroup per row (see the top of this file).
template <typename E>
__global__ __launch_bounds__(kSampleThreads) void sample_kernel(VerifyArgs a) {
    constexpr int NT = kSampleThreads, NW = NT / 64;
    constexpr int VEC = Logit<E>::kVec;
    __shared__ double tab[kExpTable];
    __shared__ double wt[DrawLds<E>::kWt];
    __shared__ double segsum[kSampleMaxSeg];
    __shared__ float shv[NW];
    __shared__ int shi[NW];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int V = a.V;
    const float T = a.temperature[b];
    const bool sampled = !(T == 0.0f);
    const E* row = static_cast<const E*>(a.target) + (int64_t)b * V;
    const float u = sampled ? a.uniforms[b] : 0.0f;
    const bool vec_ok = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
    int err = 0;
    if (temperature_bad(T)) err |= kSeqErrTemperature;
    if (sampled && !(u >= 0.0f && u < 1.0f)) err |= kSeqErrUniform;

    if (!sampled || err) {
        // one pass: maximum, NaN and +inf (sampled rows), the lowest index of the maximum;
        // kU loads in flight per thread
        const int nvec = vec_ok ? V / VEC : 0;
        float mx = -INFINITY;
        int idx = 0x7fffffff;
        int bad = 0;
        constexpr int kU = 4;
        for (int v0 = 0; v0 < nvec; v0 += kU * NT) {
            u32x4 raw[kU];
#pragma unroll
            for (int k = 0; k < kU; ++k) {
                const int v = v0 + k * NT + tid;
                raw[k] = v < nvec ? load16(row + (int64_t)v * VEC) : Logit<E>::neg_inf16();
            }
#pragma unroll
            for (int k = 0; k < kU; ++k) {
                const int v = v0 + k * NT + tid;
                float z[VEC];
                Logit<E>::unpack(raw[k], z);
                // the vector's NaN-propagating maximum: NaN if it holds a NaN, else +inf if
                // it holds +inf; only a vector that beats the running maximum is searched
                // for the lowest index reaching it
                float tm = z[0];
#pragma unroll
                for (int e = 1; e < VEC; ++e) tm = nmax(tm, z[e]);
                bad |= (tm != tm) | (sampled && tm == INFINITY);
                if (tm > mx) {
                    int e0 = VEC - 1;
#pragma unroll
                    for (int e = VEC - 1; e >= 0; --e)
                        if (z[e] == tm) e0 = e;
                    mx = tm;
                    idx = v * VEC + e0;
                }
            }
        }
        for (int i = nvec * VEC + tid; i < V; i += NT) {
            const float z = Logit<E>::at(row, i);
            bad |= (z != z) | (sampled && z == INFINITY);
            if (z > mx) {
                mx = z;
                idx = i;
            }
        }
        err |= block_or<NW>(bad ? kSeqErrLogit : 0, shi);
        block_argmax<NW>(mx, idx, shv, shi);
        if (mx == -INFINITY) err |= kSeqErrLogit;
        if (sampled && scaled_range_bad(mx, (float)(kLog2eD / (double)T))) err |= kSeqErrLogit;
        if (tid == 0) {
            a.out_tokens[b] = err ? -1 : idx;
            a.out_status[b] = err;
        }
        return;
    }

    // a sampled row with a valid temperature and uniform: the provisional reference R0,
    // the maximum of the first NT vectors of the row, while the wave's first segment and
    // the 2^(j/256) table come in
    const int nwhole = V / kSampleSeg;
    u32x4 first[kSegVecs];
    const bool have_first = sizeof(E) == 2 && vec_ok && w < nwhole;
    if constexpr (sizeof(E) == 2) {
        if (have_first) seg_load(reinterpret_cast<const uint16_t*>(row), w * kSampleSeg, lane, first);
    }
    float z0[VEC];
    load_vec(row, tid * VEC, V, vec_ok, z0);
    exp2_table_fill(tab);
    float m0 = z0[0];
#pragma unroll
    for (int k = 1; k < VEC; ++k) m0 = nmax(m0, z0[k]);
    const float R0 = block_nmax<NW>(m0, shv);  // its barriers also publish tab

    SeqDesc d{};
    d.mode = kModeBonus;
    d.T = T;
    d.u = u;
    d.mt = d.md = R0;
    d.trow = d.drow = b;
    DrawRows<E> r = draw_rows<E>(a, d, tab, sizeof(E) == 2 ? wt : nullptr);
    r.t = row;
    r.d = row;
    r.vec_ok = vec_ok;
    // the lifted reference (a float step above R0; the flush threshold stays kFlushLog2
    // binary orders below R0)
    const double c2 = kLog2eD / (double)T;
    const double ref = (double)R0 + (double)(float)(kSampleLift / c2);
    r.refA = r.refB = ref;
    if constexpr (sizeof(E) == 2) {
        weight_table_write<E, NT>(r, wt);
        __syncthreads();
    }
    const float mx = row_segment_sums<E, NT>(r, V, segsum, have_first, first);
    const float mr = block_nmax<NW>(mx, shv);  // its barriers also publish segsum
    if (mr != mr || mr == INFINITY) {
        if (tid == 0) {
            a.out_tokens[b] = -1;
            a.out_status[b] = kSeqErrLogit;
        }
        return;
    }
    const int nseg = (V + kSampleSeg - 1) / kSampleSeg;
    SegHit h = seg_hit(segsum, nseg, (double)u);
    const float c2f = (float)(kLog2eD / (double)T);
    // R0 <= M <= max(mr, kTabTop): a bound on |M| for the scaled-range rule
    const float ub = fmaxf(fabsf(R0), fmaxf(mr, kTabTop));
    if (!(h.total <= kSampleSumMax) || scaled_range_bad(ub, c2f)) {
        // the slow path: the row maximum, its checks, the sums again against it
        const float M = block_nmax<NW>(row_nmax<E, NT>(row, V, vec_ok), shv);
        if ((M != M) || M == INFINITY || M == -INFINITY || scaled_range_bad(M, c2f)) {
            if (tid == 0) {
                a.out_tokens[b] = -1;
                a.out_status[b] = kSeqErrLogit;
            }
            return;
        }
        d.mt = d.md = M;
        r = draw_rows<E>(a, d, tab, sizeof(E) == 2 ? wt : nullptr);
        r.t = row;
        r.d = row;
        r.vec_ok = vec_ok;
        if constexpr (sizeof(E) == 2) {
            weight_table_write<E, NT>(r, wt);
            __syncthreads();
        }
        row_segment_sums<E, NT>(r, V, segsum, false, first);
        __syncthreads();
        h = seg_hit(segsum, nseg, (double)u);
    }
    // the index inside the hit segment
    int y = -1;
    if (h.hit >= 0) {
        int lo, hi;
        seg_range(V, kSampleSeg, h.hit, lo, hi);
        y = block_search<E, NT>(r, lo, hi, h.base, h.target, false, (double)u);
    }
    if (tid == 0) {
        // the finite row maximum has a positive weight: W > 0 and some index qualifies
        a.out_tokens[b] = y;
        a.out_status[b] = y < 0 ? kSeqErrLogit : (h.fallback ? kSeqNoteFallback : 0);
    }
}

}  // namespace

int launch_sample(const VerifyArgs& a, int bf16, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (bf16)
        hipLaunchKernelGGL(sample_kernel<uint16_t>, dim3((unsigned)a.B), dim3(kSampleThreads), 0, s, a);
    else
        hipLaunchKernelGGL(sample_kernel<float>, dim3((unsigned)a.B), dim3(kSampleThreads), 0, s, a);
    return (int)hipGetLastError();
}

}  // namespace sv
