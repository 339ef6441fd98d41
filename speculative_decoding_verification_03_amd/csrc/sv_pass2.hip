// Pass 2 of the verify step: the resolve and the one categorical draw of each sequence.
//
// resolve_kernel (one wave per sequence): validation, then the left-to-right test
// r_t < p_t(x_t)/q_t(x_t) of "A Regra de Exatidão" (lesson page "Decodificação
// Especulativa e EAGLE"), evaluated in fp64 log space from the pass-1 row statistics, or
// for T = 0 the greedy comparison argmax(p_t) == x_t ("Caso ganancioso").  n = the first
// failing position (K if none).  Writes every output except the drawn token of a sampled
// sequence, and a SeqDesc for the draw.
//
// The draw.  After a rejection at n the token comes from (p_n - q_n)+, the positive part
// of the pointwise difference over the whole vocabulary ("A Regra de Exatidão"; the
// livestream "IA local 202" describes the same clamp-and-normalise at [12:30]); after K
// acceptances from p_K (the bonus token, "O Conceito" step 4).  Only that row pair (or
// row) is read again.  It is all fp64: an fp32 weight carries a relative error near 1e-7,
// which at V ~ 1.5e5 moves CDF edges past many narrow cells and would change the drawn
// token on a visible fraction of draws.
//
// sweep_kernel (sequence x chunk workgroups, one contiguous sub-chunk per wave):
// a_i = exp((zt_i - mt)/T) and b_i = exp((zd_i - md)/T) in fp64 (a 256-entry LDS table of
// 2^(j/256) and a cubic), their sums S_p, S_q, and the sums A, B of a_i, b_i over the
// positions whose residual is positive for every rho = S_p/S_q within 1 +- kDelta of the
// pass-1 estimate rho'.  The sign test uses the logit difference
// D_i = (zt_i - mt) - (zd_i - md): p_i > q_i exactly when D_i > T ln rho.  Positions whose
// D_i falls inside the bracket go to buckets of equal D_i (equal D, equal a/b ratio, one
// residual sign), each with its sums of a_i and b_i.
//
// final_kernel (one workgroup per sequence): checks rho against rho' (else one exact
// sweep by this workgroup), forms each sub-chunk's residual mass
// A/S_p - B/S_q + sum over buckets of (a/S_p - b/S_q)+, scans the masses for u * W, and
// scans inside the sub-chunk that holds it: token = min{ i : C_i > u * W }, C the prefix
// sums in index order.
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

// Sweep shape: 16-byte vectors per row whose loads are in flight together per lane, and
// positions whose exponentials are computed together (register pressure against overlap).
#ifndef SV_SWEEP_VECTORS
#define SV_SWEEP_VECTORS 2
#endif
#ifndef SV_SWEEP_POSITIONS
#define SV_SWEEP_POSITIONS 4
#endif

// ------------------------------------------------------------------------------------
// the resolve
// ------------------------------------------------------------------------------------

__device__ __forceinline__ bool row_bad(float m, bool sampled) {
    return (m != m) || m == -INFINITY || (sampled && m == INFINITY);
}

__device__ __forceinline__ bool temperature_bad(float T) {
    return (T != T) || T < 0.0f || T == INFINITY || (T > 0.0f && T < FLT_MIN);
}

// Row j (0..K target, K+1..2K draft) of sequence b: max over chunks (NaN if any chunk saw
// a NaN) and the lowest index reaching it.
__device__ __forceinline__ void merge_greedy(const VerifyArgs& a, int b, int j, float& m, int& idx) {
    const RowPartial* p = a.part1 + ((int64_t)b * a.R + j) * a.nchunk1;
    m = -INFINITY;
    idx = 0x7fffffff;
    bool bad = false;
    for (int c = 0; c < a.nchunk1; ++c) {
        const RowPartial q = p[c];
        if (q.m != q.m) bad = true;
        else if (q.m > m) {  // strict: an earlier chunk keeps ties
            m = q.m;
            idx = q.idx;
        }
    }
    if (bad) m = __builtin_nanf("");
}

// Sampled row j: max m and S = sum exp((z - m)/T), from chunk partials in the
// 2^((z - m) * c2) form.
__device__ __forceinline__ void merge_sampled(const VerifyArgs& a, int b, int j, float c2, float& m,
                                              double& S) {
    const RowPartial* p = a.part1 + ((int64_t)b * a.R + j) * a.nchunk1;
    m = -INFINITY;
    for (int c = 0; c < a.nchunk1; ++c) m = nmax(m, p[c].m);
    S = 0.0;
    for (int c = 0; c < a.nchunk1; ++c) {
        const RowPartial q = p[c];
        if (q.s != 0.0) S += q.s * exp2(((double)q.m - (double)m) * (double)c2);
    }
}

// One wave per sequence.
template <typename E>
__global__ __launch_bounds__(64) void resolve_kernel(VerifyArgs a, int b0) {
    const int b = b0 + blockIdx.x;
    const int lane = threadIdx.x;
    const int K = a.K, V = a.V;
    const float T = a.temperature ? a.temperature[b] : 0.0f;
    const bool sampled = !(T == 0.0f);
    const int32_t* x = a.tokens + (int64_t)b * K;
    const float c2 = sampled ? (float)(kLog2eD / (double)T) : 0.0f;
    int32_t* tok = a.out_tokens + (int64_t)b * (K + 1);
    float* op = a.out_p ? a.out_p + (int64_t)b * K : nullptr;
    float* oq = a.out_q ? a.out_q + (int64_t)b * K : nullptr;
    SeqDesc d{};
    d.T = T;

    // ---- validation: every row read, every token, every uniform ----
    int err = 0;
    if (lane == 0 && temperature_bad(T)) err |= kSeqErrTemperature;
    for (int t = lane; t < K; t += 64) {
        const int xt = x[t];
        if (xt < 0 || xt >= V) err |= kSeqErrToken;
    }
    for (int j = lane; j < a.R; j += 64) {
        if (j > K && !sampled) continue;
        const RowPartial* p = a.part1 + ((int64_t)b * a.R + j) * a.nchunk1;
        float m = -INFINITY;
        for (int c = 0; c < a.nchunk1; ++c) m = nmax(m, p[c].m);
        if (row_bad(m, sampled)) err |= kSeqErrLogit;
    }
    if (sampled) {
        const float* u = a.uniforms + (int64_t)b * (K + 1);
        for (int t = lane; t <= K; t += 64) {
            const float ut = u[t];
            if (!(ut >= 0.0f && ut < 1.0f)) err |= kSeqErrUniform;
        }
    }
    err = wave_or(err);
    if (err) {
        for (int t = lane; t <= K; t += 64) tok[t] = -1;
        for (int t = lane; t < K; t += 64) {
            if (op) op[t] = __builtin_nanf("");
            if (oq) oq[t] = __builtin_nanf("");
        }
        if (lane == 0) {
            a.out_n[b] = -1;
            a.out_status[b] = err;
            d.mode = kModeNone;
            a.desc[b] = d;
        }
        return;
    }

    // ---- the first position that fails ----
    int first = K;
    if (!sampled) {
        for (int t = lane; t < K; t += 64) {
            float m;
            int i;
            merge_greedy(a, b, t, m, i);
            if (i != x[t]) first = min(first, t);
            if (op) op[t] = __builtin_nanf("");
            if (oq) oq[t] = __builtin_nanf("");
        }
    } else {
        const float* u = a.uniforms + (int64_t)b * (K + 1);
        for (int t = lane; t < K; t += 64) {
            const int xt = x[t];
            float mt, md;
            double St, Sd;
            merge_sampled(a, b, t, c2, mt, St);
            merge_sampled(a, b, K + 1 + t, c2, md, Sd);
            const E* trow = static_cast<const E*>(a.target) + ((int64_t)b * (K + 1) + t) * V;
            const E* drow = static_cast<const E*>(a.draft) + ((int64_t)b * K + t) * V;
            const double zt = (double)Logit<E>::at(trow, xt);
            const double zd = (double)Logit<E>::at(drow, xt);
            const double lp = (zt - (double)mt) / (double)T - log(St);
            const double lq = (zd - (double)md) / (double)T - log(Sd);
            if (op) op[t] = (float)exp(lp);
            if (oq) oq[t] = (float)exp(lq);
            // r < p/q in log space; q = 0 with p > 0 accepts, p = 0 rejects
            const double ut = (double)u[t];
            bool accept;
            if (lp == -INFINITY) accept = false;
            else if (lq == -INFINITY) accept = true;
            else if (ut == 0.0) accept = true;
            else accept = log(ut) < lp - lq;
            if (!accept) first = min(first, t);
        }
    }
    const int n = wave_min(first);
    for (int t = lane; t <= K; t += 64)
        if (t != n) tok[t] = t < n ? x[t] : -1;
    if (lane == 0) {
        a.out_n[b] = n;
        d.n = n;
        if (!sampled) {
            float m;
            int i;
            merge_greedy(a, b, n, m, i);
            tok[n] = i;
            a.out_status[b] = 0;
            d.mode = kModeNone;
        } else {
            merge_sampled(a, b, n, c2, d.mt, d.St);
            if (n < K) {
                merge_sampled(a, b, K + 1 + n, c2, d.md, d.Sd);
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

template <typename E>
__global__ __launch_bounds__(kThreads) void sweep_kernel(VerifyArgs a, int b0) {
    constexpr int VEC = Logit<E>::kVec;
    constexpr int kG = SV_SWEEP_VECTORS;  // 16-byte vectors per row in flight per lane
    constexpr int P = SV_SWEEP_POSITIONS < VEC ? SV_SWEEP_POSITIONS : VEC;
    __shared__ double tab[kExpTable];
    const int b = b0 + blockIdx.x / a.nchunk2;
    const int c = blockIdx.x % a.nchunk2;
    const SeqDesc d = a.desc[b];
    if (d.mode == kModeNone) return;  // whole workgroup
    exp2_table_init(tab);
    const DrawRows<E> r = draw_rows<E>(a, b, d, tab);

    const int V = a.V;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int sub = a.ch2 / kWaves;
    const int lo = min(V, c * a.ch2 + w * sub);
    const int hi = min(V, lo + sub);
    const int64_t e = ((int64_t)b * a.nchunk2 + c) * kWaves + w;
    SweepAcc acc;
    acc.tau_hi = acc.tau_lo = 0.0;
    if (r.residual) {
        const double rho1 = d.St / d.Sd;
        acc.tau_hi = (double)d.T * log(rho1 * (1.0 + kDelta));
        acc.tau_lo = (double)d.T * log(rho1 * (1.0 - kDelta));
    }
    acc.lane = lane;

    // whole, aligned spans of 64 lanes x kG vectors: all loads in flight together
    const int span = 64 * kG * VEC;
    const int hi_whole = r.vec_ok ? lo + ((hi - lo) / span) * span : lo;
    for (int s0 = lo; s0 < hi_whole; s0 += span) {  // wave-uniform trip count
        u32x4 rt[kG], rd[kG];
#pragma unroll
        for (int g = 0; g < kG; ++g) {
            const int i = s0 + (g * 64 + lane) * VEC;
            rt[g] = load16(r.t + i);
            rd[g] = r.residual ? load16(r.d + i) : rt[g];
        }
#pragma unroll
        for (int g = 0; g < kG; ++g) {
            const int i = s0 + (g * 64 + lane) * VEC;
            float zt[VEC], zd[VEC];
            Logit<E>::unpack(rt[g], zt);
            Logit<E>::unpack(rd[g], zd);
#pragma unroll
            for (int h = 0; h < VEC; h += P) {  // P positions at a time (constant indices)
                float tp[P], dp[P];
#pragma unroll
                for (int k = 0; k < P; ++k) {
                    tp[k] = zt[h + k];
                    dp[k] = zd[h + k];
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

template <typename E>
__global__ __launch_bounds__(kThreads) void final_kernel(VerifyArgs a, int b0) {
    __shared__ double tab[kExpTable];
    __shared__ double shd[kWaves];
    __shared__ int shi[kWaves];
    __shared__ double sh_base;
    const int b = b0 + blockIdx.x;
    const SeqDesc d = a.desc[b];
    if (d.mode == kModeNone) return;
    exp2_table_init(tab);
    DrawRows<E> r = draw_rows<E>(a, b, d, tab);
    const int tid = threadIdx.x;
    const int nsub = a.nchunk2 * kWaves;
    const int sub = a.ch2 / kWaves;
    const int64_t e0 = (int64_t)b * nsub;
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

}  // namespace

int launch_resolve(const VerifyArgs& a, int bf16, int b0, int b1, void* stream) {
    if (b1 <= b0) return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (bf16)
        hipLaunchKernelGGL(resolve_kernel<uint16_t>, dim3(b1 - b0), dim3(64), 0, s, a, b0);
    else
        hipLaunchKernelGGL(resolve_kernel<float>, dim3(b1 - b0), dim3(64), 0, s, a, b0);
    return (int)hipGetLastError();
}

int launch_draw(const VerifyArgs& a, int bf16, int b0, int b1, void* stream) {
    if (b1 <= b0) return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const unsigned sweep_blocks = (unsigned)((int64_t)(b1 - b0) * a.nchunk2);
    if (bf16) {
        hipLaunchKernelGGL(sweep_kernel<uint16_t>, dim3(sweep_blocks), dim3(kThreads), 0, s, a, b0);
        hipLaunchKernelGGL(final_kernel<uint16_t>, dim3(b1 - b0), dim3(kThreads), 0, s, a, b0);
    } else {
        hipLaunchKernelGGL(sweep_kernel<float>, dim3(sweep_blocks), dim3(kThreads), 0, s, a, b0);
        hipLaunchKernelGGL(final_kernel<float>, dim3(b1 - b0), dim3(kThreads), 0, s, a, b0);
    }
    return (int)hipGetLastError();
}

}  // namespace sv
