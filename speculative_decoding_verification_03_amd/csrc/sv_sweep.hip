// Pass 2 of the verify step: the sweep kernel, per-segment fp64 partials of the draw
// row(s) of each sampled sequence.
#include "sv_draw.h"

namespace sv {

namespace {

// ------------------------------------------------------------------------------------
// sweep
// ------------------------------------------------------------------------------------

struct SweepAcc {
    double sp, sq;  // this lane's sums of a_i, b_i
    double A, B;    // over the positions with a certainly positive residual
    // The wave's buckets of undecided positions, one per lane: lane j holds bucket j
    // (its difference value D and sums of a and b).  nbkt is wave-uniform.
    double bD, bA, bB;
    int nbkt;
    int lane;
    // fast path: the undecided positions whose difference equals `key` (wave-uniform; NaN
    // until the first one), and their sums of a and b
    float key;
    double kA, kB;

    __device__ __forceinline__ void reset() {
        sp = sq = A = B = 0.0;
        bD = bA = bB = 0.0;
        nbkt = 0;
        key = __builtin_nanf("");
        kA = kB = 0.0;
    }
};

// Adds the undecided positions of this call (flag u, difference D, weights a, b per lane)
// to the wave's buckets, one distinct D at a time.
__device__ __forceinline__ void bucket_add(SweepAcc& s, bool u, double D, double av, double bv) {
    uint64_t m = __ballot(u);
    while (m) {  // wave-uniform
        const int leader = __ffsll((unsigned long long)m) - 1;
        const double Dv = __shfl(D, leader, 64);
        const bool match = u && D == Dv;
        const double sa = wave_sum(match ? av : 0.0);
        const double sb = wave_sum(match ? bv : 0.0);
        const uint64_t hit = __ballot(s.lane < s.nbkt && s.bD == Dv);
        int slot;
        if (hit) {
            slot = __ffsll((unsigned long long)hit) - 1;
        } else {
            slot = s.nbkt;
            if (s.nbkt < kBuckets && s.lane == slot) s.bD = Dv;
            ++s.nbkt;  // past kBuckets: overflowed
        }
        if (slot < kBuckets && s.lane == slot) {
            s.bA += sa;
            s.bB += sb;
        }
        u = u && !match;
        m = __ballot(u);
    }
}

// The exact path for P positions of this lane: weights av, bv (0 where the position is
// not live), the fp32 difference Df (exact where dx_ok) or else the fp64 one.  Wave-wide
// votes: every lane of the wave calls this the same number of times.
template <typename E, int P>
__device__ __forceinline__ void accumulate(const DrawRows<E>& r, const double (&av)[P], const double (&bv)[P],
                                           const float (&zt)[P], const float (&zd)[P],
                                           const bool (&dx_ok)[P], const bool (&live)[P], SweepAcc& s) {
    bool pos[P], unc[P];
    bool any_unc = false, any_inexact = false;
#pragma unroll
    for (int k = 0; k < P; ++k) {
        const float Df = zt[k] - zd[k];
        pos[k] = Df > r.tau_hi_f;
        unc[k] = !pos[k] && Df >= r.tau_lo_f;
        any_inexact |= !dx_ok[k];
    }
    if (__any(any_inexact)) {  // a logit outside the table range: classify in fp64
#pragma unroll
        for (int k = 0; k < P; ++k) {
            if (!dx_ok[k]) {
                const double D = (double)zt[k] - (double)zd[k];
                pos[k] = D > r.tau_hi;
                unc[k] = !pos[k] && D >= r.tau_lo;
            }
        }
    }
#pragma unroll
    for (int k = 0; k < P; ++k) {
        unc[k] = unc[k] && live[k];
        any_unc |= unc[k];
        s.sp += av[k];
        s.sq += bv[k];
        const double sel = pos[k] ? 1.0 : 0.0;
        s.A = __builtin_fma(av[k], sel, s.A);
        s.B = __builtin_fma(bv[k], sel, s.B);
    }
    if (__any(any_unc)) {  // bucket by the exact logit difference
#pragma unroll
        for (int k = 0; k < P; ++k) bucket_add(s, unc[k], (double)zt[k] - (double)zd[k], av[k], bv[k]);
    }
}

// Exact path for two bf16 positions of each row (one 32-bit word each).
template <bool Residual>
__device__ __forceinline__ void exact_word_tab(const DrawRows<uint16_t>& r, uint32_t wt, uint32_t wd,
                                               SweepAcc& s) {
    const float zt[2] = {__uint_as_float(wt << 16), __uint_as_float(wt & 0xffff0000u)};
    const float zd[2] = {__uint_as_float(wd << 16), __uint_as_float(wd & 0xffff0000u)};
    double av[2], bv[2];
    bool dx_ok[2], live[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        uint32_t q;
        const bool it = tab_has(__float_as_uint(zt[k]) >> 16, q);
        av[k] = r.a_of(zt[k]);
        bool id = true;
        bv[k] = 0.0;
        if (Residual) {
            id = tab_has(__float_as_uint(zd[k]) >> 16, q);
            bv[k] = r.b_of(zd[k]);
        }
        live[k] = av[k] != 0.0 || bv[k] != 0.0;
        // a difference of two bf16 values with |z| in [2^-12, 32) is exact in fp32;
        // positions whose weights are both 0 need no sign
        dx_ok[k] = (it && id) || !live[k];
    }
    if (!Residual) {
        s.sp += av[0];
        s.sp += av[1];
        return;
    }
    accumulate<uint16_t, 2>(r, av, bv, zt, zd, dx_ok, live, s);
}

// One word of each row of a span that is taken again: words whose four values all lie in
// the table take the fast path's arithmetic with every undecided position bucketed by its
// exact difference (the differences of such values are exact in fp32); other words take
// the exact path.
template <bool Residual>
__device__ __forceinline__ void redo_word_tab(const DrawRows<uint16_t>& r, uint32_t xt, uint32_t xd,
                                              SweepAcc& s) {
    uint32_t ot0, ot1, od0 = 0, od1 = 0;
    tab_offsets(xt, ot0, ot1);
    if (Residual) tab_offsets(xd, od0, od1);
    const double a0 = tab_at(r.wt, ot0), a1 = tab_at(r.wt, ot1);
    const double b0 = Residual ? tab_at(r.wt, od0) : 0.0, b1 = Residual ? tab_at(r.wt, od1) : 0.0;
    // a sentinel (value outside the table) reads NaN
    const bool out = (a0 != a0) | (a1 != a1) | (b0 != b0) | (b1 != b1);
    if (__any(out)) {
        exact_word_tab<Residual>(r, xt, xd, s);
        return;
    }
    if (!Residual) {
        s.sp += a0;
        s.sp += a1;
        return;
    }
    const float D0 = __uint_as_float(xt << 16) - __uint_as_float(xd << 16);
    const float D1 = __uint_as_float(xt & 0xffff0000u) - __uint_as_float(xd & 0xffff0000u);
    const bool p0 = D0 > r.tau_hi_f, p1 = D1 > r.tau_hi_f;
    // positions with no weight on either side need no sign (as on the exact path)
    const bool u0 = !p0 && D0 >= r.tau_lo_f && (a0 != 0.0 || b0 != 0.0);
    const bool u1 = !p1 && D1 >= r.tau_lo_f && (a1 != 0.0 || b1 != 0.0);
    s.sp += a0;
    s.sq += b0;
    s.sp += a1;
    s.sq += b1;
    const double s0 = p0 ? 1.0 : 0.0, s1 = p1 ? 1.0 : 0.0;
    s.A = __builtin_fma(a0, s0, s.A);
    s.B = __builtin_fma(b0, s0, s.B);
    s.A = __builtin_fma(a1, s1, s.A);
    s.B = __builtin_fma(b1, s1, s.B);
    if (__any(u0 || u1)) {
        bucket_add(s, u0, (double)D0, a0, b0);
        bucket_add(s, u1, (double)D1, a1, b1);
    }
}

// Fast path for one word of each row: table weights without range checks (a value outside
// the table reads NaN), signs from the fp32 difference.  Undecided positions (difference
// inside the bracket) are summed into s.kA, s.kB when their difference equals the wave's
// key (set by the first one; typically every undecided position has the same difference,
// mt - md at low temperature); any other undecided position sets `odd`.
__device__ __forceinline__ void fast_word_res(const double* wt, uint32_t xt, uint32_t xd, float th, float tl,
                                              SweepAcc& s, bool& odd) {
    const float zt0 = __uint_as_float(xt << 16), zt1 = __uint_as_float(xt & 0xffff0000u);
    const float zd0 = __uint_as_float(xd << 16), zd1 = __uint_as_float(xd & 0xffff0000u);
    const float D0 = zt0 - zd0, D1 = zt1 - zd1;
    const bool p0 = D0 > th, p1 = D1 > th;
    const bool u0 = !p0 && D0 >= tl, u1 = !p1 && D1 >= tl;
    uint32_t ot0, ot1, od0, od1;
    tab_offsets(xt, ot0, ot1);
    tab_offsets(xd, od0, od1);
    const double a0 = tab_at(wt, ot0), a1 = tab_at(wt, ot1);
    const double b0 = tab_at(wt, od0), b1 = tab_at(wt, od1);
    if (__any(u0 || u1)) {
        if (s.key != s.key) {  // the first undecided difference becomes the key
            const uint64_t m = __ballot(u0 || u1);
            const int l = __ffsll((unsigned long long)m) - 1;
            s.key = __shfl(u0 ? D0 : D1, l, 64);
        }
        const bool k0 = u0 && D0 == s.key, k1 = u1 && D1 == s.key;
        odd = odd || (u0 && !k0) || (u1 && !k1);
        s.kA = __builtin_fma(a0, k0 ? 1.0 : 0.0, s.kA);
        s.kB = __builtin_fma(b0, k0 ? 1.0 : 0.0, s.kB);
        s.kA = __builtin_fma(a1, k1 ? 1.0 : 0.0, s.kA);
        s.kB = __builtin_fma(b1, k1 ? 1.0 : 0.0, s.kB);
    }
    s.sp += a0;
    s.sq += b0;
    s.sp += a1;
    s.sq += b1;
    const double s0 = p0 ? 1.0 : 0.0, s1 = p1 ? 1.0 : 0.0;
    s.A = __builtin_fma(a0, s0, s.A);
    s.B = __builtin_fma(b0, s0, s.B);
    s.A = __builtin_fma(a1, s1, s.A);
    s.B = __builtin_fma(b1, s1, s.B);
    // the sums exist here: no pass may sink this word's arithmetic towards the span end,
    // which would keep its table values in registers
    asm volatile("" ::"v"(s.sp), "v"(s.sq), "v"(s.A), "v"(s.B), "v"(s.kA), "v"(s.kB));
}

__device__ __forceinline__ void fast_word_bonus(const double* wt, uint32_t xt, SweepAcc& s) {
    uint32_t o0, o1;
    tab_offsets(xt, o0, o1);
    s.sp += tab_at(wt, o0);
    s.sp += tab_at(wt, o1);
    asm volatile("" ::"v"(s.sp));
}

// Writes a segment's partial (lane 0) and buckets (lanes below nbkt), then clears acc.  The
// fast path's keyed positions become (or join) the bucket of their difference.
__device__ __forceinline__ void store_partial(DrawPartial* part, Bucket* bkt, int e, SweepAcc& acc) {
    if (!(acc.key != acc.key)) bucket_add(acc, true, (double)acc.key, acc.kA, acc.kB);
    const double sp = wave_sum(acc.sp);
    const double sq = wave_sum(acc.sq);
    const double A = wave_sum(acc.A);
    const double Bm = wave_sum(acc.B);
    if (acc.lane < acc.nbkt && acc.lane < kBuckets) {
        Bucket bk;
        bk.a = acc.bA;
        bk.b = acc.bB;
        bkt[e * kBuckets + acc.lane] = bk;
    }
    if (acc.lane == 0) {
        DrawPartial dp;
        dp.sp = sp;
        dp.sq = sq;
        dp.A = A;
        dp.B = Bm;
        dp.nbkt = acc.nbkt;
        dp.pad[0] = dp.pad[1] = dp.pad[2] = 0;
        part[e] = dp;
    }
    acc.reset();
}

// The loads of the first whole span, issued before the weight table is built.
struct FirstSpan {
    u32x4 t[kG], d[kG];
};

template <bool Residual>
__device__ __forceinline__ void first_span(const DrawRows<uint16_t>& r, int lo, int lane, FirstSpan& f) {
#pragma unroll
    for (int g = 0; g < kG; ++g) {
        const int i = lo + (g * 64 + lane) * 8;
        f.t[g] = load16(r.t + i);
        f.d[g] = Residual ? load16(r.d + i) : f.t[g];
    }
}

// One wave over positions [lo, hi) of the draw row(s), bf16 with the LDS table, in
// segments of L positions (L a multiple of a span; lo a multiple of L): the partial of
// segment k goes to part[k], bkt[k * kBuckets ...].  Whole spans of 64 lanes x kG vectors
// per row go through the fast path, the next span's loads issued before the current one
// is processed; a span whose sums turned NaN or that held an undecided sign is redone by
// the exact path from a copy of the sums taken before it.  Positions outside whole spans
// (a partial last segment, or rows not 16-byte aligned) take the exact path one word per
// lane.  f holds the first whole span's loads when have_first.
template <bool Residual>
__device__ __forceinline__ void sweep_wave_tab(const DrawRows<uint16_t>& r, int lo, int hi, int L,
                                               DrawPartial* part, Bucket* bkt, SweepAcc& acc,
                                               const FirstSpan& f, bool have_first) {
    const int lane = acc.lane;
    const int hi_whole = r.vec_ok ? lo + ((hi - lo) / kSpan16) * kSpan16 : lo;
    const float th = r.tau_hi_f, tl = r.tau_lo_f;
    // segment by segment: a rolling pipeline over the segment's whole spans (group g of the
    // next span is loaded into rt[g], rd[g] as soon as group g of the current one has been
    // taken out of them), then the exact redo of the spans that needed it, with no loads
    // in flight
    for (int g0 = lo; g0 < hi_whole;) {
        const int g1 = min(hi_whole, (g0 / L + 1) * L);
        u32x4 rt[kG], rd[kG];
        if (have_first && g0 == lo) {
#pragma unroll
            for (int g = 0; g < kG; ++g) {
                rt[g] = f.t[g];
                rd[g] = f.d[g];
            }
        } else {
#pragma unroll
            for (int g = 0; g < kG; ++g) {
                const int i = g0 + (g * 64 + lane) * 8;
                rt[g] = load16(r.t + i);
                rd[g] = Residual ? load16(r.d + i) : rt[g];
            }
        }
        uint32_t redo = 0;  // wave-uniform: spans of this segment to redo exactly
        for (int i0 = g0, j = 0; i0 < g1; i0 += kSpan16, ++j) {  // wave-uniform trip count
            const bool more = i0 + kSpan16 < g1;
            const double keep_sp = acc.sp, keep_sq = acc.sq, keep_A = acc.A, keep_B = acc.B;
            const double keep_kA = acc.kA, keep_kB = acc.kB;
            bool odd = false;
#pragma unroll
            for (int g = 0; g < kG; ++g) {
                const u32x4 ct = rt[g], cd = rd[g];
                if (more) {
                    const int i = i0 + kSpan16 + (g * 64 + lane) * 8;
                    rt[g] = load16(r.t + i);
                    rd[g] = Residual ? load16(r.d + i) : rt[g];
                }
                // one word at a time: the scheduler must not hoist every table read of the
                // span (the registers they would take are better spent on loads in flight)
                const uint32_t xt4[4] = {ct.x, ct.y, ct.z, ct.w};
                const uint32_t xd4[4] = {cd.x, cd.y, cd.z, cd.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (Residual) fast_word_res(r.wt, xt4[q], xd4[q], th, tl, acc, odd);
                    else fast_word_bonus(r.wt, xt4[q], acc);
                    if ((q + 1) % kWordsPerFence == 0) __builtin_amdgcn_sched_barrier(0);
                }
            }
            if (__any(odd || acc.sp != acc.sp || acc.sq != acc.sq)) {  // rare
                acc.sp = keep_sp;
                acc.sq = keep_sq;
                acc.A = keep_A;
                acc.B = keep_B;
                acc.kA = keep_kA;
                acc.kB = keep_kB;
                redo |= 1u << j;
            }
        }
        while (redo) {  // wave-uniform
            const int j = __ffs(redo) - 1;
            redo &= redo - 1;
#pragma unroll 1
            for (int g = 0; g < kG; ++g) {
                const int i = g0 + j * kSpan16 + (g * 64 + lane) * 8;
                const u32x4 vt = *reinterpret_cast<const u32x4*>(r.t + i);
                const u32x4 vd = Residual ? *reinterpret_cast<const u32x4*>(r.d + i) : u32x4{0u, 0u, 0u, 0u};
                redo_word_tab<Residual>(r, vt.x, vd.x, acc);
                redo_word_tab<Residual>(r, vt.y, vd.y, acc);
                redo_word_tab<Residual>(r, vt.z, vd.z, acc);
                redo_word_tab<Residual>(r, vt.w, vd.w, acc);
            }
        }
        // a segment ends here (or the row does, exactly at a span)
        if (g1 % L == 0 || g1 == hi) store_partial(part, bkt, g0 / L, acc);
        g0 = g1;
    }
    // the rest, segment by segment, one word (two positions) per lane; positions at or
    // past the end read -inf (0xff80), whose weight is 0
    for (int t0 = hi_whole; t0 < hi;) {
        const int k = t0 / L;
        const int te = min(hi, (k + 1) * L);
#pragma unroll 1
        for (int j0 = t0; j0 < te; j0 += 128) {
            const int i = j0 + 2 * lane;
            const uint32_t x0 = i < te ? (uint32_t)r.t[i] : 0xff80u;
            const uint32_t x1 = i + 1 < te ? (uint32_t)r.t[i + 1] : 0xff80u;
            uint32_t y0 = 0xff80u, y1 = 0xff80u;
            if (Residual) {
                y0 = i < te ? (uint32_t)r.d[i] : 0xff80u;
                y1 = i + 1 < te ? (uint32_t)r.d[i + 1] : 0xff80u;
            }
            exact_word_tab<Residual>(r, x0 | (x1 << 16), y0 | (y1 << 16), acc);
        }
        store_partial(part, bkt, k, acc);
        t0 = te;
    }
}

// P positions of each row, weights by the fp64 exponential (fp32 logits, or rows that do
// not share a reference).
template <typename E, int P>
__device__ __forceinline__ void sweep_vec_exp(const DrawRows<E>& r, const float (&zt)[P], const float (&zd)[P],
                                              SweepAcc& s) {
    bool nt[P], nd[P], live[P];
    bool any = false;
#pragma unroll
    for (int k = 0; k < P; ++k) {
        nt[k] = zt[k] >= r.thr_t;
        nd[k] = r.residual && zd[k] >= r.thr_d;
        live[k] = nt[k] || nd[k];
        any |= live[k];
    }
    if (!__any(any)) return;
    double av[P], bv[P];
#pragma unroll
    for (int k = 0; k < P; ++k) {
        av[k] = nt[k] ? exp2_256(exp2_arg((double)zt[k], r.refA, r.c256), r.tab) : 0.0;
        bv[k] = nd[k] ? exp2_256(exp2_arg((double)zd[k], r.refB, r.c256), r.tab) : 0.0;
    }
    if (!r.residual) {
#pragma unroll
        for (int k = 0; k < P; ++k) s.sp += av[k];
        return;
    }
    bool dx_ok[P];
#pragma unroll
    for (int k = 0; k < P; ++k) dx_ok[k] = !live[k];  // fp32 differences may round: fp64
    accumulate<E, P>(r, av, bv, zt, zd, dx_ok, live, s);
}

// One wave over positions [lo, hi) in segments of L, weights by the fp64 exponential.
template <typename E>
__device__ __forceinline__ void sweep_wave_exp(const DrawRows<E>& r, int lo, int hi, int L, DrawPartial* part,
                                               Bucket* bkt, SweepAcc& acc) {
    constexpr int VEC = Logit<E>::kVec;
    constexpr int P = 4;
    constexpr int span = 64 * VEC;
    static_assert(kSpan16 % span == 0, "draw segments are whole spans");
    const int lane = acc.lane;
    const int hi_whole = r.vec_ok ? lo + ((hi - lo) / span) * span : lo;
    for (int i0 = lo; i0 < hi_whole; i0 += span) {
        const int i = i0 + lane * VEC;
        float zt[VEC], zd[VEC];
        Logit<E>::unpack(load16(r.t + i), zt);
        if (r.residual) {
            Logit<E>::unpack(load16(r.d + i), zd);
        } else {
#pragma unroll
            for (int k = 0; k < VEC; ++k) zd[k] = -INFINITY;
        }
#pragma unroll
        for (int h = 0; h < VEC; h += P) {
            float tp[P], dp[P];
#pragma unroll
            for (int k = 0; k < P; ++k) {
                tp[k] = zt[h + k];
                dp[k] = zd[h + k];
            }
            sweep_vec_exp<E, P>(r, tp, dp, acc);
        }
        // a segment ends here (or the row does, exactly at a span)
        if ((i0 + span) % L == 0 || i0 + span == hi) store_partial(part, bkt, i0 / L, acc);
    }
    for (int t0 = hi_whole; t0 < hi;) {
        const int k = t0 / L;
        const int te = min(hi, (k + 1) * L);
#pragma unroll 1
        for (int j0 = t0; j0 < te; j0 += 64) {
            const int i = j0 + lane;
            const bool in = i < te;
            const float t1[1] = {in ? Logit<E>::at(r.t, i) : -INFINITY};
            const float d1[1] = {(in && r.residual) ? Logit<E>::at(r.d, i) : -INFINITY};
            sweep_vec_exp<E, 1>(r, t1, d1, acc);
        }
        store_partial(part, bkt, k, acc);
        t0 = te;
    }
}

// grid = (sequences rounded up to a multiple of kXcds) x nchunk2.  Sampled sequences:
// workgroup c of a sequence sweeps segments
// [c spc, (c + 1) spc) of the draw row(s), each wave a contiguous run of them, into
// per-segment partials.
template <typename E>
__global__ __launch_bounds__(kSweepThreads) __attribute__((amdgpu_waves_per_eu(kDrawWaves)))
void sweep_kernel(VerifyArgs a, int b0) {
    constexpr int NW = kSweepThreads / 64;
    __shared__ double tab[kExpTable];
    __shared__ double wt[DrawLds<E>::kWt];
    // workgroups are handed to the XCDs in turn (workgroup id mod kXcds): every chunk of
    // entry k runs on XCD k mod kXcds, so a sequence's weight table is fetched into one
    // L2.  Entry k is the deal's (the draws dealt over the XCDs in turn, two-row residual
    // draws first, which balances the XCDs' work when the sweep takes several rounds of
    // workgroups; the entries between the two kinds of draws are empty), or else
    // sequence b0 + k, on the XCD of its resolve and final workgroups.  The grid is padded
    // to whole rounds of kXcds entries.
    const unsigned x = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
    const int k = (int)(x + kXcds * (j / (unsigned)a.nchunk2));
    if (k >= a.nseq2) return;
    const SeqDesc d = a.deal ? reinterpret_cast<const SeqDesc*>(a.deal_desc)[k]
                             : reinterpret_cast<const SeqDesc*>(a.desc)[b0 + k];
    if (d.mode == kModeNone || d.b < b0 || d.b >= b0 + a.nseq2) return;  // whole workgroup
    const int b = d.b;
    const int c = (int)(j % (unsigned)a.nchunk2);
    DrawRows<E> r = draw_rows<E>(a, d, tab, wt);
    const int w = threadIdx.x >> 6;
    SweepAcc acc;
    acc.lane = threadIdx.x & 63;
    acc.reset();
    const int c0 = c * a.spc, c1 = min(a.nseg, c0 + a.spc);
    const int per = (c1 - c0 + NW - 1) / NW;
    const int s0 = min(c1, c0 + w * per), s1 = min(c1, s0 + per);
    DrawPartial* part = a.part2 + (int64_t)b * a.nseg;
    Bucket* bkt = a.bkt + (int64_t)b * a.nseg * kBuckets;
    bool done = false;
    if constexpr (sizeof(E) == 2) {
        if (r.use_tab) {
            // the wave's first loads go out before the tables reach LDS
            const int lo = min(a.V, s0 * a.seg), hi = min(a.V, s1 * a.seg);
            const bool have_first = r.vec_ok && hi - lo >= kSpan16;
            FirstSpan f;
            if (have_first) {
                if (r.residual) first_span<true>(r, lo, acc.lane, f);
                else first_span<false>(r, lo, acc.lane, f);
            }
            TableCopy<kSweepThreads> tc;
            tc.load(a.wtab + (int64_t)b * kWtabLen);
            tc.store(wt);
            exp2_table_init(tab);  // its barrier also publishes wt
            if (s0 < s1) {
                if (r.residual) sweep_wave_tab<true>(r, lo, hi, a.seg, part, bkt, acc, f, have_first);
                else sweep_wave_tab<false>(r, lo, hi, a.seg, part, bkt, acc, f, have_first);
            }
            done = true;
        }
    }
    if (!done) {
        exp2_table_init(tab);
        if (s0 < s1) sweep_wave_exp<E>(r, min(a.V, s0 * a.seg), min(a.V, s1 * a.seg), a.seg, part, bkt, acc);
    }
}

}  // namespace

int launch_sweep(const VerifyArgs& a, int bf16, int b0, unsigned blocks, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (bf16)
        hipLaunchKernelGGL(sweep_kernel<uint16_t>, dim3(blocks), dim3(kSweepThreads), 0, s, a, b0);
    else
        hipLaunchKernelGGL(sweep_kernel<float>, dim3(blocks), dim3(kSweepThreads), 0, s, a, b0);
    return (int)hipGetLastError();
}

}  // namespace sv
