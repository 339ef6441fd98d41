// The draft-side sampler: one draw per row from softmax(z / T), argmax at T = 0.
#include "sv_draw.h"

namespace sv {

namespace {

// ------------------------------------------------------------------------------------
// the draft-side sampler: one draw per row from softmax(z / T), the whole row in one
// workgroup
// ------------------------------------------------------------------------------------

// One wave's fp64 sum of the bonus weights over positions [lo, hi) of r.t: the table fast
// path over a whole segment of 16-byte vectors when it applies, the exact path otherwise.
// On the fast path a value outside the table reads NaN: its lane's vector is read again
// (from cache) and its values outside the table take the fp64 exponential (the callers
// have ruled out NaN and +inf logits).  bad: the exact path met a NaN or +inf logit
// (wave-uniform).
template <typename E>
__device__ __forceinline__ double wave_row_sum(const DrawRows<E>& r, int lo, int hi, bool& bad) {
    constexpr int VEC = Logit<E>::kVec;
    const int lane = threadIdx.x & 63;
    double s = 0.0;
    bool exact = true;
    if constexpr (sizeof(E) == 2) {
        constexpr int kU = kSeg / (64 * VEC);  // vectors per lane of a whole segment
        if (r.use_tab && r.vec_ok && hi - lo == kSeg) {
            u32x4 v[kU];  // every load of the segment in flight at once
#pragma unroll
            for (int k = 0; k < kU; ++k) v[k] = load16(r.t + lo + (k * 64 + lane) * VEC);
            uint32_t again = 0;  // this lane's vectors with a value outside the table
#pragma unroll
            for (int k = 0; k < kU; ++k) {
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
                const u32x4 w = load16(r.t + lo + (k * 64 + lane) * VEC);
                const uint32_t x4[4] = {w.x, w.y, w.z, w.w};
                double sk = 0.0;
#pragma unroll 1
                for (int q = 0; q < 8; ++q) {
                    const uint32_t h = (x4[q >> 1] >> (16 * (q & 1))) & 0xffffu;
                    sk += r.a_of(__uint_as_float(h << 16));
                }
                s += sk;
            }
            exact = false;
        }
    }
    bool b = false;
    if (exact) {
        s = 0.0;
        for (int i0 = lo; i0 < hi; i0 += 64 * VEC) {
            float z[VEC];
            load_vec(r.t, i0 + lane * VEC, hi, r.vec_ok, z);
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                b |= (z[k] != z[k]) | (z[k] == INFINITY);
                s += r.a_of(z[k]);
            }
        }
    }
    bad = __any(b);
    return wave_sum(s);
}

// Sums of the bonus weights of every segment of the row into segsum (one wave per
// segment); returns whether a NaN or +inf logit was met.  Contains __syncthreads().
template <typename E, int NT>
__device__ __forceinline__ bool row_segment_sums(const DrawRows<E>& r, int V, double* segsum, int* shi) {
    const int w = threadIdx.x >> 6, nseg = (V + kSeg - 1) / kSeg;
    int bad = 0;
    for (int k = w; k < nseg; k += NT / 64) {
        int lo, hi;
        seg_range(V, kSeg, k, lo, hi);
        bool bk;
        const double sk = wave_row_sum(r, lo, hi, bk);
        bad |= bk;
        if ((threadIdx.x & 63) == 0) segsum[k] = sk;
    }
    return block_or<NT / 64>(bad, shi) != 0;  // its barrier also publishes segsum
}

// grid = rows, one workgroup per row.  Phase 1 streams the row for its maximum (greedy
// rows: the lowest index reaching it), with normal loads so that the row stays in cache.
// Sampled rows then tabulate their weights against that maximum (bf16), sum the weights
// per kSeg segment (one wave per segment; the row is read again, mostly from cache), scan
// the segment sums for u * W and search the segment that holds it:
// token = min{ i : C_i > u * W }, C the prefix sums in index order.
template <typename E>
__global__ __launch_bounds__(kSampleThreads) void sample_kernel(VerifyArgs a) {
    constexpr int NT = kSampleThreads, NW = NT / 64;
    constexpr int VEC = Logit<E>::kVec;
    __shared__ double tab[kExpTable];
    __shared__ double wt[DrawLds<E>::kWt];
    __shared__ double segsum[kSampleMaxSeg];
    __shared__ float shv[NW];
    __shared__ int shi[NW];
    __shared__ double shd[2 * NW];
    __shared__ double sh_base;
    const int b = blockIdx.x, tid = threadIdx.x;
    const int V = a.V;
    const float T = a.temperature[b];
    const bool sampled = !(T == 0.0f);
    const E* row = static_cast<const E*>(a.target) + (int64_t)b * V;
    const float u = sampled ? a.uniforms[b] : 0.0f;
    const bool vec_ok = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
    const int nvec = vec_ok ? V / VEC : 0;
    int err = 0;
    if (temperature_bad(T)) err |= kSeqErrTemperature;
    if (sampled && !(u >= 0.0f && u < 1.0f)) err |= kSeqErrUniform;

    // phase 1: maximum, NaN and +inf (sampled rows), the lowest index of the maximum;
    // kU loads in flight per thread
    float mx = -INFINITY;
    int idx = 0x7fffffff;
    int bad = 0;
    constexpr int kU = 4;
    for (int v0 = 0; v0 < nvec; v0 += kU * NT) {
        u32x4 raw[kU];
#pragma unroll
        for (int k = 0; k < kU; ++k) {
            const int v = v0 + k * NT + tid;
            raw[k] = v < nvec ? *reinterpret_cast<const u32x4*>(row + (int64_t)v * VEC) : Logit<E>::neg_inf16();
        }
#pragma unroll
        for (int k = 0; k < kU; ++k) {
            const int v = v0 + k * NT + tid;
            float z[VEC];
            Logit<E>::unpack(raw[k], z);
            // the vector's NaN-propagating maximum: NaN if it holds a NaN, else +inf if it
            // holds +inf; only a vector that beats the running maximum is searched for the
            // lowest index reaching it
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
    if (err || !sampled) {
        if (tid == 0) {
            a.out_tokens[b] = err ? -1 : idx;
            a.out_status[b] = err;
        }
        return;
    }

    // phase 2: the weight table for reference mx (bf16)
    exp2_table_init(tab);
    SeqDesc d{};
    d.mode = kModeBonus;
    d.T = T;
    d.u = u;
    d.mt = d.md = mx;
    d.trow = d.drow = b;
    DrawRows<E> r = draw_rows<E>(a, d, tab, sizeof(E) == 2 ? wt : nullptr);
    r.t = row;
    r.d = row;
    r.vec_ok = vec_ok;
    if constexpr (sizeof(E) == 2) {
        weight_table_write<E, NT>(r, wt);
        __syncthreads();
    }

    // phase 3: weight sums per segment (no NaN or +inf is left to find)
    row_segment_sums<E, NT>(r, V, segsum, shi);

    // phase 4: the segment holding u * W, then the index inside it
    const int nseg = (V + kSeg - 1) / kSeg;
    int status = 0;
    const double v = tid < nseg ? segsum[tid] : 0.0;
    double total;
    const double ex = block_exclusive_scan<NW>(v, total, shd);
    int y = -1;
    if (total > 0.0) {
        const double target = (double)u * total;
        int hit = block_min<NW>((tid < nseg && v > 0.0 && ex + v > target) ? tid : 0x7fffffff, shi);
        double tgt = target;
        if (hit == 0x7fffffff) {
            // rounding put u*W past every prefix: the last segment with mass, last index
            hit = block_max<NW>((tid < nseg && v > 0.0) ? tid : -1, shi);
            tgt = INFINITY;
            status |= kSeqNoteFallback;
        }
        if (tid == hit) sh_base = ex;
        __syncthreads();
        int lo, hi;
        seg_range(V, kSeg, hit, lo, hi);
        y = block_search<E, NT>(r, lo, hi, sh_base, tgt, false, (double)u);
    }
    if (tid == 0) {
        // the finite row maximum has weight 1: total > 0 and some index qualifies
        a.out_tokens[b] = y;
        a.out_status[b] = y < 0 ? kSeqErrLogit : status;
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
