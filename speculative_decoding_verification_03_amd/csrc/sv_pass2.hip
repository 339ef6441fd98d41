// Pass 2 of the verify step: the resolve and the one categorical draw of each sequence,
// in three kernels: resolve_kernel (one workgroup per sequence), sweep_kernel ((sequence,
// chunk) workgroups) and final_kernel (one workgroup per sequence).
//
// Resolve: validation, then the left-to-right test r_t < p_t(x_t)/q_t(x_t) of "A Regra
// de Exatidão" (lesson page "Decodificação Especulativa e EAGLE"), evaluated in fp64 log
// space from the pass-1 row statistics, or for T = 0 the greedy comparison
// argmax(p_t) == x_t ("Caso ganancioso").  n = the first failing position (K if none).
//
// The draw.  After a rejection at n the token comes from (p_n - q_n)+, the positive part
// of the pointwise difference over the whole vocabulary ("A Regra de Exatidão"; the
// livestream "IA local 202" describes the same clamp-and-normalise at [12:30]); after K
// acceptances from p_K (the bonus token, "O Conceito" step 4).  Only that row pair (or
// row) is read again.  It is all fp64: an fp32 weight carries a relative error near 1e-7,
// which at V ~ 1.5e5 moves CDF edges past many narrow cells and would change the drawn
// token on a visible fraction of draws.
//
// Sweep (each workgroup, one contiguous sub-chunk per wave): a_i = exp((zt_i - mt)/T) and
// b_i = exp((zd_i - md)/T) in fp64 (a 256-entry LDS table of 2^(j/256) and a Taylor
// polynomial), their sums S_p, S_q, and the sums A, B of a_i, b_i over the positions whose
// residual is positive for every rho = S_p/S_q within 1 +- kDelta of the pass-1 estimate
// rho'.  The sign test uses the logit difference D_i = (zt_i - mt) - (zd_i - md):
// p_i > q_i exactly when D_i > T ln rho.  Positions whose D_i falls inside the bracket go to
// buckets of equal D_i (equal D, equal a/b ratio, one residual sign), each with its sums of
// a_i and b_i.
//
// Final (final_kernel, one workgroup per sequence, after the sweep): checks rho against rho' (else one exact sweep by this
// workgroup), forms each sub-chunk's residual mass A/S_p - B/S_q + sum over buckets of
// (a/S_p - b/S_q)+, scans the masses for u * W, and scans inside the sub-chunk that holds
// it: token = min{ i : C_i > u * W }, C the prefix sums in index order.
#include <float.h>
#include <hip/hip_runtime.h>
#include <math.h>

#include "sv_common.h"
#include "sv_device.h"

namespace sv {

namespace {

constexpr double kLog2eD = 1.4426950408889634;
// Classification margin around rho' and the acceptance test of rho: pass-1 normalisers
// are within ~1e-6 of the fp64 ones, so kDelta / 2 leaves a wide guard.
constexpr double kDelta = 8e-6;
// Positions whose a_i and b_i are both below 2^-80 of their row maxima are skipped: over
// any vocabulary they move the sums and CDF edges by less than V * 2^-80.
constexpr double kSkipLog2 = -80.0;
// Row statistics of the resolve kept in LDS; rows past this are merged again on demand.
constexpr int kRowsLds = 2 * kThreads;

// Sweep shape: 16-byte vectors per row whose loads are in flight together per lane, and
// positions whose exponentials are computed together (register pressure against overlap).
#ifndef SV_SWEEP_VECTORS
#define SV_SWEEP_VECTORS 2
#endif
#ifndef SV_SWEEP_POSITIONS
#define SV_SWEEP_POSITIONS 4
#endif
// Waves per SIMD the bf16 sweep's register allocation must allow.
#ifndef SV_TAB_WAVES
#define SV_TAB_WAVES 4
#endif

// The resolve's result for one sequence.
struct SeqDesc {
    int mode;      // kMode*
    int n;         // accepted drafts = row of the draw
    float T;       // temperature
    float u;       // uniform of the final draw
    float mt, md;  // maxima of target row n and draft row n
    double St, Sd; // pass-1 normalisers of those rows: sum exp((z - m) / T)
};
static_assert(sizeof(SeqDesc) <= kSeqDescBytes && kSeqDescBytes % alignof(SeqDesc) == 0,
              "workspace slot of the descriptor");

// ------------------------------------------------------------------------------------
// the resolve
// ------------------------------------------------------------------------------------

__device__ __forceinline__ bool row_bad(float m, bool sampled) {
    return (m != m) || m == -INFINITY || (sampled && m == INFINITY);
}

__device__ __forceinline__ bool temperature_bad(float T) {
    return (T != T) || T < 0.0f || T == INFINITY || (T > 0.0f && T < FLT_MIN);
}

struct RowStat {
    float m;   // row maximum (NaN if any chunk saw a NaN)
    int idx;   // greedy rows: lowest index reaching m
    double S;  // sampled rows: sum exp((z - m) / T)
};

// Row j (0..K target, K+1..2K draft) of sequence b from its pass-1 chunk partials.
// Greedy: max and lowest index (chunks in order, strict comparison keeps the earlier
// chunk on ties).  Sampled: max m and S from partials in the 2^((z - m_c) * c2) form.
__device__ __forceinline__ RowStat merge_row(const VerifyArgs& a, int b, int j, bool sampled, float c2) {
    const RowPartial* p = a.part1 + ((int64_t)b * a.R + j) * a.nchunk1;
    RowStat r{-INFINITY, 0x7fffffff, 0.0};
    if (!sampled) {
        bool bad = false;
#pragma unroll 4
        for (int c = 0; c < a.nchunk1; ++c) {
            const RowPartial q = p[c];
            if (q.m != q.m) bad = true;
            else if (q.m > r.m) {
                r.m = q.m;
                r.idx = q.idx;
            }
        }
        if (bad) r.m = __builtin_nanf("");
        return r;
    }
#pragma unroll 4
    for (int c = 0; c < a.nchunk1; ++c) r.m = nmax(r.m, p[c].m);
#pragma unroll 4
    for (int c = 0; c < a.nchunk1; ++c) {
        const RowPartial q = p[c];
        if (q.s != 0.0) r.S += q.s * exp2(((double)q.m - (double)r.m) * (double)c2);
    }
    return r;
}

// The resolve of sequence b by the whole workgroup.  write: also write the outputs (all
// but the drawn token of a sampled sequence, and its status).  Returns the same SeqDesc
// in every thread.  Contains __syncthreads().
template <typename E>
__device__ SeqDesc resolve_seq(const VerifyArgs& a, int b, bool write) {
    __shared__ RowStat rows[kRowsLds];
    __shared__ int shi[kWaves];
    __shared__ SeqDesc sd;
    const int tid = threadIdx.x;
    const int K = a.K, V = a.V, R = a.R;
    const float T = a.temperature ? a.temperature[b] : 0.0f;
    const bool sampled = !(T == 0.0f);
    const int32_t* x = a.tokens + (int64_t)b * K;
    const float* u = sampled ? a.uniforms + (int64_t)b * (K + 1) : nullptr;
    const float c2 = sampled ? (float)(kLog2eD / (double)T) : 0.0f;

    // loads that do not depend on the row statistics first: tokens, logits at x_t, uniforms
    int xt = 0;
    double zx = 0.0, dx = 0.0;
    float ut = 0.5f;
    int err = 0;
    if (tid < K) {
        xt = x[tid];
        if (sampled && xt >= 0 && xt < V) {
            zx = (double)Logit<E>::at(static_cast<const E*>(a.target) + ((int64_t)b * (K + 1) + tid) * V, xt);
            dx = (double)Logit<E>::at(static_cast<const E*>(a.draft) + ((int64_t)b * K + tid) * V, xt);
        }
    }
    if (sampled && tid <= K) ut = u[tid];
    for (int t = tid; t < K; t += kThreads) {
        const int v = x[t];
        if (v < 0 || v >= V) err |= kSeqErrToken;
    }
    if (sampled)
        for (int t = tid; t <= K; t += kThreads) {
            const float v = u[t];
            if (!(v >= 0.0f && v < 1.0f)) err |= kSeqErrUniform;
        }
    if (tid == 0 && temperature_bad(T)) err |= kSeqErrTemperature;
    // row statistics (draft rows only for sampled sequences)
    const int nrows = sampled ? R : K + 1;
    for (int j = tid; j < nrows; j += kThreads) {
        const RowStat r = merge_row(a, b, j, sampled, c2);
        if (row_bad(r.m, sampled)) err |= kSeqErrLogit;
        if (j < kRowsLds) rows[j] = r;
    }
    err = block_or(err, shi);  // also orders the rows[] writes before the reads below
    auto row = [&](int j) -> RowStat { return j < kRowsLds ? rows[j] : merge_row(a, b, j, sampled, c2); };

    int32_t* tok = a.out_tokens + (int64_t)b * (K + 1);
    float* op = a.out_p ? a.out_p + (int64_t)b * K : nullptr;
    float* oq = a.out_q ? a.out_q + (int64_t)b * K : nullptr;
    if (err) {
        if (write) {
            for (int t = tid; t <= K; t += kThreads) tok[t] = -1;
            for (int t = tid; t < K; t += kThreads) {
                if (op) op[t] = __builtin_nanf("");
                if (oq) oq[t] = __builtin_nanf("");
            }
            if (tid == 0) {
                a.out_n[b] = -1;
                a.out_status[b] = err;
            }
        }
        SeqDesc d{};
        d.mode = kModeNone;
        return d;
    }

    // the first position that fails
    int first = K;
    for (int t = tid; t < K; t += kThreads) {
        if (t >= kThreads) {  // K > kThreads: the early loads above covered t < kThreads only
            xt = x[t];
            if (sampled) {
                zx = (double)Logit<E>::at(static_cast<const E*>(a.target) + ((int64_t)b * (K + 1) + t) * V, xt);
                dx = (double)Logit<E>::at(static_cast<const E*>(a.draft) + ((int64_t)b * K + t) * V, xt);
                ut = u[t];
            }
        }
        if (!sampled) {
            if (row(t).idx != xt) first = min(first, t);
            if (write && op) op[t] = __builtin_nanf("");
            if (write && oq) oq[t] = __builtin_nanf("");
        } else {
            const RowStat rt = row(t), rd = row(K + 1 + t);
            const double lp = (zx - (double)rt.m) / (double)T - log(rt.S);
            const double lq = (dx - (double)rd.m) / (double)T - log(rd.S);
            if (write && op) op[t] = (float)exp(lp);
            if (write && oq) oq[t] = (float)exp(lq);
            // r < p/q in log space; q = 0 with p > 0 accepts, p = 0 rejects
            bool accept;
            if (lp == -INFINITY) accept = false;
            else if (lq == -INFINITY) accept = true;
            else if (ut == 0.0f) accept = true;
            else accept = log((double)ut) < lp - lq;
            if (!accept) first = min(first, t);
        }
    }
    const int n = block_min(first, shi);
    if (write)
        for (int t = tid; t <= K; t += kThreads)
            if (t != n) tok[t] = t < n ? x[t] : -1;
    if (tid == 0) {
        SeqDesc d{};
        d.n = n;
        d.T = T;
        if (write) a.out_n[b] = n;
        if (!sampled) {
            if (write) {
                tok[n] = row(n).idx;
                a.out_status[b] = 0;
            }
            d.mode = kModeNone;
        } else {
            const RowStat rt = row(n);
            d.mt = rt.m;
            d.St = rt.S;
            if (n < K) {
                const RowStat rd = row(K + 1 + n);
                d.md = rd.m;
                d.Sd = rd.S;
                d.mode = kModeResidual;
            } else {
                d.mode = kModeBonus;
            }
            d.u = a.uniforms[(int64_t)b * (K + 1) + K];
        }
        sd = d;
    }
    __syncthreads();
    const SeqDesc d = sd;
    __syncthreads();
    return d;
}

// ------------------------------------------------------------------------------------
// draw weights
// ------------------------------------------------------------------------------------

template <typename E>
struct DrawRows {
    const E* t;          // target row of the draw
    const E* d;          // draft row (residual; the target row again otherwise)
    double mt, md, c256; // row maxima, 256 log2(e)/T
    double inv_sp, inv_sq;
    int residual;        // 1: (a/S_p - b/S_q)+ ; 0: a (bonus, or the draw from p_n)
    int vec_ok;          // both rows 16-byte aligned
    const double* tab;

    // exp((z - m)/T) = 2^((z - m) * 256 log2(e)/T / 256); z - m is exact in fp64
    __device__ __forceinline__ double a_of(float z) const { return exp2_256(((double)z - mt) * c256, tab); }
    __device__ __forceinline__ double b_of(float z) const { return exp2_256(((double)z - md) * c256, tab); }
    __device__ __forceinline__ double weight(float zt, float zd) const {
        const double a = a_of(zt);
        if (!residual) return a;
        const double w = a * inv_sp - b_of(zd) * inv_sq;
        return w > 0.0 ? w : 0.0;
    }
};

template <typename E>
__device__ __forceinline__ DrawRows<E> draw_rows(const VerifyArgs& a, int b, const SeqDesc& d,
                                                 const double* tab) {
    DrawRows<E> r;
    r.residual = d.mode == kModeResidual;
    r.t = static_cast<const E*>(a.target) + ((int64_t)b * (a.K + 1) + d.n) * a.V;
    r.d = r.residual ? static_cast<const E*>(a.draft) + ((int64_t)b * a.K + d.n) * a.V : r.t;
    r.mt = d.mt;
    r.md = d.md;
    r.c256 = 256.0 * kLog2eD / (double)d.T;
    r.inv_sp = 1.0;
    r.inv_sq = 1.0;
    r.vec_ok = ((reinterpret_cast<uintptr_t>(r.t) | reinterpret_cast<uintptr_t>(r.d)) & 15) == 0;
    r.tab = tab;
    return r;
}

// Logits at positions i .. i+VEC-1: one 16-byte vector when aligned and inside [.., hi),
// else element by element with positions at or past hi reading -inf (weight 0).
template <typename E>
__device__ __forceinline__ void load_vec(const E* row, int i, int hi, bool vec_ok,
                                         float (&z)[Logit<E>::kVec]) {
    constexpr int VEC = Logit<E>::kVec;
    if (vec_ok && i + VEC <= hi) {
        Logit<E>::unpack(load16(row + i), z);
    } else {
#pragma unroll
        for (int k = 0; k < VEC; ++k) z[k] = (i + k < hi) ? Logit<E>::at(row, i + k) : -INFINITY;
    }
}

// ------------------------------------------------------------------------------------
// sweep: grid = sequences x nchunk2, each wave one contiguous sub-chunk
// ------------------------------------------------------------------------------------

struct SweepAcc {
    double sp = 0.0, sq = 0.0;  // this lane's sums of a_i, b_i
    double A = 0.0, B = 0.0;    // over the positions with a certainly positive residual
    // p_i > q_i  <=>  D_i = (zt_i - mt) - (zd_i - md) > T ln(S_p / S_q).  With the ratio
    // known to within 1 +- kDelta of rho', D_i above tau_hi is positive for certain and
    // D_i in [tau_lo, tau_hi] undecided.
    double tau_hi, tau_lo;
    // The same bracket on the computed ratio a_i / b_i (tabulated bf16 weights):
    // a_i > rho_hi b_i is positive for certain, rho_lo b_i <= a_i <= rho_hi b_i undecided.
    double rho_hi, rho_lo;
    // The wave's buckets of undecided positions, one per lane: lane j holds bucket j
    // (its D value and sums of a and b).  nbkt is wave-uniform.
    double bD = 0.0, bA = 0.0, bB = 0.0;
    int nbkt = 0;
    int lane;
};

// Adds the undecided positions of this call (flag u, values D, a, b per lane) to the
// wave's buckets, one distinct D value at a time.
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

// P positions of this lane.  Every lane of the wave calls this the same number of times
// (the votes below are wave-wide).
template <typename E, int P>
__device__ __forceinline__ void sweep_vec(const DrawRows<E>& r, const float (&zt)[P], const float (&zd)[P],
                                          SweepAcc& s) {
    double xt[P], xd[P], yt[P], yd[P];
    bool need = false;
#pragma unroll
    for (int k = 0; k < P; ++k) {
        xt[k] = (double)zt[k] - r.mt;
        xd[k] = r.residual ? (double)zd[k] - r.md : -INFINITY;
        yt[k] = xt[k] * r.c256;
        yd[k] = xd[k] * r.c256;
        need |= fmax(yt[k], yd[k]) >= kSkipLog2 * 256.0;
    }
    if (!__any(need)) return;  // the whole wave: weights below 2^-80 of the row maxima
    if (!r.residual) {
#pragma unroll
        for (int k = 0; k < P; ++k) s.sp += exp2_256(yt[k], r.tab);
        return;
    }
    double av[P], bv[P], D[P];
    bool unc[P];
    bool any_unc = false;
#pragma unroll
    for (int k = 0; k < P; ++k) {
        av[k] = exp2_256(yt[k], r.tab);
        bv[k] = exp2_256(yd[k], r.tab);
        s.sp += av[k];
        s.sq += bv[k];
        D[k] = xt[k] - xd[k];
        const bool pos = D[k] > s.tau_hi;
        unc[k] = !pos && D[k] >= s.tau_lo;
        any_unc |= unc[k];
        const double sel = pos ? 1.0 : 0.0;
        s.A = __builtin_fma(av[k], sel, s.A);
        s.B = __builtin_fma(bv[k], sel, s.B);
    }
    if (__any(any_unc)) {  // rare
#pragma unroll
        for (int k = 0; k < P; ++k) bucket_add(s, unc[k], D[k], av[k], bv[k]);
    }
}

// ---- the bf16 path: weights looked up in the per-sequence tables (kTabE0 .. kTabNE) ----

// Table index of the bf16 bit pattern h (in the low 16 bits), clamped into the table, and
// whether h lies inside it.
__device__ __forceinline__ uint32_t tab_index(uint32_t h, bool& in) {
    const uint32_t off = (h & 0x7fffu) - (uint32_t)(kTabE0 * 128);
    in = off < (uint32_t)kTabHalf;
    return min(off, (uint32_t)(kTabHalf - 1)) + (h >> 15) * (uint32_t)kTabHalf;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) { return __uint_as_float(h << 16); }

// P positions of this lane given as bf16 bit patterns; ta, tb the LDS tables of the target
// and draft rows.  Logits outside the tables take the polynomial (rare: tiny, very large
// or infinite values); both give the same fp64 value for the same logit.
template <bool Residual, int P>
__device__ __forceinline__ void sweep_tab(const DrawRows<uint16_t>& r, const double* ta, const double* tb,
                                          const uint32_t (&ht)[P], const uint32_t (&hd)[P], SweepAcc& s) {
    double av[P], bv[P];
    bool in_all = true;
#pragma unroll
    for (int k = 0; k < P; ++k) {
        bool it, id = true;
        av[k] = ta[tab_index(ht[k], it)];
        if (Residual) bv[k] = tb[tab_index(hd[k], id)];
        in_all = in_all && it && id;
    }
    if (!__all(in_all)) {
#pragma unroll
        for (int k = 0; k < P; ++k) {
            bool it, id = true;
            tab_index(ht[k], it);
            if (!it) av[k] = r.a_of(bf16_bits_to_float(ht[k]));
            if (Residual) {
                tab_index(hd[k], id);
                if (!id) bv[k] = r.b_of(bf16_bits_to_float(hd[k]));
            }
        }
    }
    if (!Residual) {
#pragma unroll
        for (int k = 0; k < P; ++k) s.sp += av[k];
        return;
    }
    bool unc[P];
    bool any_unc = false;
#pragma unroll
    for (int k = 0; k < P; ++k) {
        s.sp += av[k];
        s.sq += bv[k];
        const bool pos = av[k] > s.rho_hi * bv[k];
        unc[k] = !pos && av[k] > 0.0 && av[k] >= s.rho_lo * bv[k];
        any_unc |= unc[k];
        const double sel = pos ? 1.0 : 0.0;
        s.A = __builtin_fma(av[k], sel, s.A);
        s.B = __builtin_fma(bv[k], sel, s.B);
    }
    if (__any(any_unc)) {  // rare: bucket by the exact logit difference
#pragma unroll
        for (int k = 0; k < P; ++k) {
            const double D = ((double)bf16_bits_to_float(ht[k]) - r.mt) - ((double)bf16_bits_to_float(hd[k]) - r.md);
            bucket_add(s, unc[k], D, av[k], bv[k]);
        }
    }
}

// One wave per sub-chunk of chunk c of the draw row(s) of sequence b, bf16 logits, tables
// in LDS.
template <bool Residual>
__device__ __forceinline__ void sweep_chunk_tab(const VerifyArgs& a, const DrawRows<uint16_t>& r,
                                                const SeqDesc& d, const double* ta, const double* tb,
                                                int b, int c) {
    constexpr int VEC = 8;
    constexpr int kG = SV_SWEEP_VECTORS;
    const int V = a.V;
    const int lane = threadIdx.x & 63, w = (threadIdx.x >> 6) & (kWaves - 1);
    const int sub = a.ch2 / kWaves;
    const int lo = min(V, c * a.ch2 + w * sub);
    const int hi = min(V, lo + sub);
    const int64_t e = ((int64_t)b * a.ns2 + c) * kWaves + w;
    SweepAcc acc;
    acc.tau_hi = acc.tau_lo = 0.0;
    acc.rho_hi = acc.rho_lo = 1.0;
    if (Residual) {
        const double rho1 = d.St / d.Sd;
        acc.rho_hi = rho1 * (1.0 + kDelta);
        acc.rho_lo = rho1 * (1.0 - kDelta);
    }
    acc.lane = lane;

    const int span = 64 * kG * VEC;
    const int hi_whole = r.vec_ok ? lo + ((hi - lo) / span) * span : lo;
    u32x4 rt[kG], rd[kG];
    auto fetch = [&](int s0) {
#pragma unroll
        for (int g = 0; g < kG; ++g) {
            const int i = s0 + (g * 64 + lane) * VEC;
            rt[g] = load16(r.t + i);
            rd[g] = Residual ? load16(r.d + i) : rt[g];
        }
    };
    if (lo < hi_whole) fetch(lo);
    for (int s0 = lo; s0 < hi_whole; s0 += span) {  // wave-uniform trip count
        uint32_t wt[kG][4], wd[kG][4];
#pragma unroll
        for (int g = 0; g < kG; ++g) {
            wt[g][0] = rt[g].x; wt[g][1] = rt[g].y; wt[g][2] = rt[g].z; wt[g][3] = rt[g].w;
            wd[g][0] = rd[g].x; wd[g][1] = rd[g].y; wd[g][2] = rd[g].z; wd[g][3] = rd[g].w;
        }
        if (s0 + span < hi_whole) fetch(s0 + span);
#pragma unroll
        for (int g = 0; g < kG; ++g) {
#pragma unroll
            for (int q = 0; q < 4; q += 2) {  // 4 positions: two words of two bf16 each
                const uint32_t ht[4] = {wt[g][q] & 0xffffu, wt[g][q] >> 16, wt[g][q + 1] & 0xffffu, wt[g][q + 1] >> 16};
                const uint32_t hd[4] = {wd[g][q] & 0xffffu, wd[g][q] >> 16, wd[g][q + 1] & 0xffffu, wd[g][q + 1] >> 16};
                sweep_tab<Residual>(r, ta, tb, ht, hd, acc);
            }
        }
    }
    // the rest (a partial span, or rows not 16-byte aligned): one position per lane; lanes
    // past the end see -inf (0xff80), which lies outside the tables and weighs 0
#pragma unroll 1
    for (int i0 = hi_whole; i0 < hi; i0 += 64) {
        const int i = i0 + lane;
        const bool in = i < hi;
        const uint32_t t1[1] = {in ? (uint32_t)r.t[i] : 0xff80u};
        const uint32_t d1[1] = {(in && Residual) ? (uint32_t)r.d[i] : 0xff80u};
        sweep_tab<Residual>(r, ta, tb, t1, d1, acc);
    }
    const double sp = wave_sum(acc.sp);
    const double sq = wave_sum(acc.sq);
    const double A = wave_sum(acc.A);
    const double Bm = wave_sum(acc.B);
    if (lane < acc.nbkt && lane < kBuckets) {
        Bucket bk;
        bk.a = acc.bA;
        bk.b = acc.bB;
        a.bkt[e * kBuckets + lane] = bk;
    }
    if (lane == 0) {
        DrawPartial dp;
        dp.sp = sp;
        dp.sq = sq;
        dp.A = A;
        dp.B = Bm;
        dp.nbkt = acc.nbkt;
        dp.pad[0] = dp.pad[1] = dp.pad[2] = 0;
        a.part2[e] = dp;
    }
}

// One wave per sub-chunk of chunk c of the draw row(s) of sequence b.
template <typename E>
__device__ __forceinline__ void sweep_chunk(const VerifyArgs& a, const DrawRows<E>& r, const SeqDesc& d,
                                            int b, int c) {
    constexpr int VEC = Logit<E>::kVec;
    constexpr int kG = SV_SWEEP_VECTORS;  // 16-byte vectors per row in flight per lane
    constexpr int P = SV_SWEEP_POSITIONS < VEC ? SV_SWEEP_POSITIONS : VEC;

    const int V = a.V;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int sub = a.ch2 / kWaves;
    const int lo = min(V, c * a.ch2 + w * sub);
    const int hi = min(V, lo + sub);
    const int64_t e = ((int64_t)b * a.ns2 + c) * kWaves + w;
    SweepAcc acc;
    acc.tau_hi = acc.tau_lo = 0.0;
    if (r.residual) {
        const double rho1 = d.St / d.Sd;
        acc.tau_hi = (double)d.T * log(rho1 * (1.0 + kDelta));
        acc.tau_lo = (double)d.T * log(rho1 * (1.0 - kDelta));
    }
    acc.lane = lane;

    // whole, aligned spans of 64 lanes x kG vectors per row; the next span's loads are
    // issued before the current span is processed
    const int span = 64 * kG * VEC;
    const int hi_whole = r.vec_ok ? lo + ((hi - lo) / span) * span : lo;
    u32x4 rt[kG], rd[kG];
    auto fetch = [&](int s0) {
#pragma unroll
        for (int g = 0; g < kG; ++g) {
            const int i = s0 + (g * 64 + lane) * VEC;
            rt[g] = load16(r.t + i);
            rd[g] = r.residual ? load16(r.d + i) : rt[g];
        }
    };
    if (lo < hi_whole) fetch(lo);
    for (int s0 = lo; s0 < hi_whole; s0 += span) {  // wave-uniform trip count
        float zt[kG][VEC], zd[kG][VEC];
#pragma unroll
        for (int g = 0; g < kG; ++g) {
            Logit<E>::unpack(rt[g], zt[g]);
            Logit<E>::unpack(rd[g], zd[g]);
        }
        if (s0 + span < hi_whole) fetch(s0 + span);
#pragma unroll
        for (int g = 0; g < kG; ++g) {
#pragma unroll
            for (int h = 0; h < VEC; h += P) {  // P positions at a time (constant indices)
                float tp[P], dp[P];
#pragma unroll
                for (int k = 0; k < P; ++k) {
                    tp[k] = zt[g][h + k];
                    dp[k] = zd[g][h + k];
                }
                sweep_vec(r, tp, dp, acc);
            }
        }
    }
    // the rest (a partial span at the end, or rows not 16-byte aligned): one position per lane
#pragma unroll 1
    for (int i0 = hi_whole; i0 < hi; i0 += 64) {
        const int i = i0 + lane;
        const bool in = i < hi;
        const float t1[1] = {in ? Logit<E>::at(r.t, i) : -INFINITY};
        const float d1[1] = {(in && r.residual) ? Logit<E>::at(r.d, i) : -INFINITY};
        sweep_vec(r, t1, d1, acc);
    }
    const double sp = wave_sum(acc.sp);
    const double sq = wave_sum(acc.sq);
    const double A = wave_sum(acc.A);
    const double Bm = wave_sum(acc.B);
    if (lane < acc.nbkt && lane < kBuckets) {
        Bucket bk;
        bk.a = acc.bA;
        bk.b = acc.bB;
        a.bkt[e * kBuckets + lane] = bk;
    }
    if (lane == 0) {
        DrawPartial dp;
        dp.sp = sp;
        dp.sq = sq;
        dp.A = A;
        dp.B = Bm;
        dp.nbkt = acc.nbkt;
        dp.pad[0] = dp.pad[1] = dp.pad[2] = 0;
        a.part2[e] = dp;
    }
}

// ------------------------------------------------------------------------------------
// final: grid = sequences, one workgroup each
// ------------------------------------------------------------------------------------

// Smallest i in [lo, hi) with base + (w_lo + ... + w_i) > target, in tiles of VEC positions
// per thread (thread-local prefix, then a workgroup exclusive scan of the thread totals).
// standalone: base = 0 and target = u * (sum over the range), taken by a first sweep.
// If no index qualifies (rounding), the last index with positive weight; -1 if none.
// lo must be a multiple of VEC.
template <typename E>
__device__ int block_search(const DrawRows<E>& r, int lo, int hi, double base, double target,
                            bool standalone, double u) {
    constexpr int VEC = Logit<E>::kVec;
    constexpr int kTile = VEC * kThreads;
    __shared__ double shd[kWaves];
    __shared__ int shi[kWaves];
    const int tid = threadIdx.x;
    if (standalone) {
        double tot = 0.0;
        for (int t0 = lo; t0 < hi; t0 += kTile) {
            const int i = t0 + VEC * tid;
            float zt[VEC], zd[VEC];
            load_vec(r.t, i, hi, r.vec_ok, zt);
            if (r.residual) load_vec(r.d, i, hi, r.vec_ok, zd);
            double s = 0.0;
#pragma unroll
            for (int k = 0; k < VEC; ++k) s += r.weight(zt[k], r.residual ? zd[k] : 0.0f);
            tot += block_sum(s, shd);
        }
        base = 0.0;
        target = u * tot;
    }
    double carry = 0.0;
    int lastpos = -1;
    for (int t0 = lo; t0 < hi; t0 += kTile) {
        const int i = t0 + VEC * tid;
        float zt[VEC], zd[VEC];
        load_vec(r.t, i, hi, r.vec_ok, zt);
        if (r.residual) load_vec(r.d, i, hi, r.vec_ok, zd);
        double w[VEC];
        double run = 0.0;
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            w[k] = r.weight(zt[k], r.residual ? zd[k] : 0.0f);
            run += w[k];
            if (w[k] > 0.0) lastpos = i + k;
        }
        double tile_tot;
        const double ex = block_exclusive_scan(run, tile_tot, shd);
        double acc = base + carry + ex;
        int found = 0x7fffffff;
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            acc += w[k];
            if (found == 0x7fffffff && w[k] > 0.0 && acc > target) found = i + k;
        }
        const int f = block_min(found, shi);
        if (f != 0x7fffffff) return f;
        carry += tile_tot;
    }
    return block_max(lastpos, shi);
}

// The draw of sequence b from the partials of all its chunks.
template <typename E>
__device__ void final_seq(const VerifyArgs& a, DrawRows<E> r, const SeqDesc& d, int b) {
    __shared__ double shd[kWaves];
    __shared__ int shi[kWaves];
    __shared__ double sh_base;
    const int tid = threadIdx.x;
    const int nsub = a.nchunk2 * kWaves;
    const int sub = a.ch2 / kWaves;
    const int64_t e0 = (int64_t)b * a.ns2 * kWaves;
    const double u = (double)d.u;
    int status = 0;

    // fp64 normalisers and the check that rho' classified every position
    bool exact_ok = true;
    if (r.residual) {
        double sp = 0.0, sq = 0.0;
        int over = 0;
        for (int k = tid; k < nsub; k += kThreads) {
            const DrawPartial dp = a.part2[e0 + k];
            sp += dp.sp;
            sq += dp.sq;
            over |= dp.nbkt > kBuckets;
        }
        sp = block_sum(sp, shd);
        sq = block_sum(sq, shd);
        over = block_or(over, shi);
        r.inv_sp = 1.0 / sp;
        r.inv_sq = 1.0 / sq;
        const double rho = sp / sq;
        const double rho1 = d.St / d.Sd;
        exact_ok = !over && rho >= rho1 * (1.0 - 0.5 * kDelta) && rho <= rho1 * (1.0 + 0.5 * kDelta);
#ifdef SV_DEBUG_FINAL
        if (tid == 0 && a.out_p) {
            a.out_p[(int64_t)b * a.K] = (float)(rho / rho1 - 1.0);
            status |= (over ? 128 : 0) | (exact_ok ? 0 : 64);
        }
#endif
    }

    int y;
    if (!exact_ok) {
        // the pass-1 estimate was off, or too many undecided positions: one exact sweep
        y = block_search(r, 0, a.V, 0.0, 0.0, true, u);
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
        for (int t0 = 0; t0 < nsub; t0 += kThreads) {
            const int k = t0 + tid;
            const double v = k < nsub ? mass(k) : 0.0;
            double tot;
            block_exclusive_scan(v, tot, shd);
            carry += tot;
        }
        const double total = carry;
        if (!(total > 0.0)) {
            // residual without fp64 mass (exact arithmetic rules it out): draw from p_n
            status |= kSeqNoteFallback;
            r.residual = 0;
            y = block_search(r, 0, a.V, 0.0, 0.0, true, u);
        } else {
            const double target = u * total;
            carry = 0.0;
            int hit = 0x7fffffff;
            for (int t0 = 0; t0 < nsub; t0 += kThreads) {
                const int k = t0 + tid;
                const double v = k < nsub ? mass(k) : 0.0;
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
                // rounding put u*W past every prefix: the last sub-chunk with mass, last index
                int last = -1;
                for (int t0 = 0; t0 < nsub; t0 += kThreads) {
                    const int k = t0 + tid;
                    if (k < nsub && mass(k) > 0.0) last = max(last, k);
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
    }
    if (tid == 0) {
        a.out_tokens[(int64_t)b * (a.K + 1) + d.n] = y;
        a.out_status[b] = status;
    }
}


// ------------------------------------------------------------------------------------
// the kernels
// ------------------------------------------------------------------------------------

// grid = sequences: the resolve; writes its outputs and the sequence's SeqDesc, and for
// bf16 logits the weight tables of the draw row(s), entry by entry the same fp64 function
// as DrawRows::a_of / b_of.
template <typename E>
__global__ __launch_bounds__(kThreads) void resolve_kernel(VerifyArgs a, int b0) {
    __shared__ double tab[kExpTable];
    const int b = b0 + blockIdx.x;
    const SeqDesc d = resolve_seq<E>(a, b, true);
    if (threadIdx.x == 0) reinterpret_cast<SeqDesc*>(a.desc)[b] = d;
    if constexpr (sizeof(E) == 2) {
        if (d.mode == kModeNone) return;  // whole workgroup
        exp2_table_init(tab);
        const DrawRows<E> r = draw_rows<E>(a, b, d, tab);
        double* dst = a.wtab + (int64_t)b * 2 * kTabLen;
        for (int k = threadIdx.x; k < kTabLen; k += kThreads) {
            const uint32_t h = (k < kTabHalf ? 0u : 0x8000u) | (uint32_t)(kTabE0 * 128 + k % kTabHalf);
            const float z = bf16_bits_to_float(h);
            dst[k] = r.a_of(z);
            if (r.residual) dst[kTabLen + k] = r.b_of(z);
        }
    }
}

// Workgroups of the bf16 sweep: kTabChunks chunks of kThreads each, sharing one copy of
// the weight tables in LDS.
constexpr int kTabChunks = 2;

// grid = sequences x ceil(nchunk2 / kTabChunks), bf16: the sweep of kTabChunks chunks.
__global__ __launch_bounds__(kThreads * kTabChunks) __attribute__((amdgpu_waves_per_eu(SV_TAB_WAVES)))
void sweep_tab_kernel(VerifyArgs a, int b0) {
    __shared__ double tab[kExpTable];
    __shared__ double wt[2 * kTabLen];
    const int ngrp = (a.nchunk2 + kTabChunks - 1) / kTabChunks;
    const int b = b0 + (int)(blockIdx.x / (unsigned)ngrp);
    const int c = (int)(blockIdx.x % (unsigned)ngrp) * kTabChunks + (int)(threadIdx.x / kThreads);
    const SeqDesc d = reinterpret_cast<const SeqDesc*>(a.desc)[b];
    if (d.mode == kModeNone) return;  // whole workgroup
    const bool residual = d.mode == kModeResidual;
    const int n16 = (residual ? 2 * kTabLen : kTabLen) / 2;  // 16-byte pieces
    const u32x4* src = reinterpret_cast<const u32x4*>(a.wtab + (int64_t)b * 2 * kTabLen);
    u32x4* dst = reinterpret_cast<u32x4*>(wt);
    for (int k = threadIdx.x; k < n16; k += blockDim.x) dst[k] = src[k];
    exp2_table_init(tab);  // its barrier also publishes wt
    if (c >= a.nchunk2) return;  // no barrier follows
    const DrawRows<uint16_t> r = draw_rows<uint16_t>(a, b, d, tab);
    if (residual) sweep_chunk_tab<true>(a, r, d, wt, wt + kTabLen, b, c);
    else sweep_chunk_tab<false>(a, r, d, wt, wt, b, c);
}

// grid = sequences x nchunk2, fp32: the sweep of chunk c of the sequence's draw row(s).
template <typename E>
__global__ __launch_bounds__(kThreads) void sweep_kernel(VerifyArgs a, int b0) {
    __shared__ double tab[kExpTable];
    const int b = b0 + (int)(blockIdx.x / (unsigned)a.nchunk2);
    const int c = (int)(blockIdx.x % (unsigned)a.nchunk2);
    const SeqDesc d = reinterpret_cast<const SeqDesc*>(a.desc)[b];
    if (d.mode == kModeNone) return;  // whole workgroup
    exp2_table_init(tab);
    sweep_chunk<E>(a, draw_rows<E>(a, b, d, tab), d, b, c);
}

// grid = sequences: the draw from the partials of all chunks.
template <typename E>
__global__ __launch_bounds__(kThreads) void final_kernel(VerifyArgs a, int b0) {
    __shared__ double tab[kExpTable];
    const int b = b0 + blockIdx.x;
    const SeqDesc d = reinterpret_cast<const SeqDesc*>(a.desc)[b];
    if (d.mode == kModeNone) return;
    exp2_table_init(tab);
    final_seq<E>(a, draw_rows<E>(a, b, d, tab), d, b);
}

}  // namespace

template <typename E>
void launch_all(const VerifyArgs& a, int b0, int b1, hipStream_t s) {
    hipLaunchKernelGGL(resolve_kernel<E>, dim3(b1 - b0), dim3(kThreads), 0, s, a, b0);
    if (!a.temperature) return;  // greedy only: the resolve is everything
    if constexpr (sizeof(E) == 2) {
        const int ngrp = (a.nchunk2 + kTabChunks - 1) / kTabChunks;
        const unsigned blocks = (unsigned)((int64_t)(b1 - b0) * ngrp);
        hipLaunchKernelGGL(sweep_tab_kernel, dim3(blocks), dim3(kThreads * kTabChunks), 0, s, a, b0);
    } else {
        const unsigned blocks = (unsigned)((int64_t)(b1 - b0) * a.nchunk2);
        hipLaunchKernelGGL(sweep_kernel<E>, dim3(blocks), dim3(kThreads), 0, s, a, b0);
    }
    hipLaunchKernelGGL(final_kernel<E>, dim3(b1 - b0), dim3(kThreads), 0, s, a, b0);
}

int launch_draw(const VerifyArgs& a, int bf16, int b0, int b1, void* stream) {
    if (b1 <= b0) return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (bf16) launch_all<uint16_t>(a, b0, b1, s);
    else launch_all<float>(a, b0, b1, s);
    return (int)hipGetLastError();
}

}  // namespace sv
