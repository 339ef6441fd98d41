// Pass 2 of the verify step, device code shared by its kernels: the resolve and the one
// categorical draw of each sequence, in three kernels: resolve_kernel (sv_resolve.hip, one
// workgroup per sequence), sweep_kernel (sv_sweep.hip) over (sequence, chunk) workgroups,
// then final_kernel (sv_final.hip, one workgroup per sequence); and the draft-side
// sampler, sample_kernel (sv_sample.hip, one workgroup per row).
//
// Resolve: validation, then the left-to-right test r_t < p_t(x_t)/q_t(x_t) of "A Regra
// de Exatidão" (lesson page "Decodificação Especulativa e EAGLE"), evaluated in fp64 from
// the pass-1 row statistics, or for T = 0 the greedy comparison argmax(p_t) == x_t ("Caso
// ganancioso").  n = the first failing position (K if none).  It also writes the draw's
// descriptor and, for bf16 logits, the sequence's weight table to the workspace.
//
// The draw.  After a rejection at n the token comes from (p_n - q_n)+, the positive part
// of the pointwise difference over the whole vocabulary ("A Regra de Exatidão"; the
// livestream "IA local 202" describes the same clamp-and-normalise at [12:30]); after K
// acceptances from p_K (the bonus token, "O Conceito" step 4).  Only that row pair (or
// row) is read again.  The weights are fp64: an fp32 weight carries a relative error near
// 1e-7, which at V ~ 1.5e5 moves CDF edges past many narrow cells and would change the
// drawn token on a visible fraction of draws.
//
// Weights.  a_i = 2^((zt_i - refA) c2), b_i = 2^((zd_i - refB) c2), c2 = log2(e)/T, so that
// p_i = a_i / S_p and q_i = b_i / S_q.  Both rows share one reference (the larger row
// maximum) unless that would push the smaller row toward fp64 underflow.  For bf16 logits
// the resolve tabulates the weight of every bf16 value with |z| in [2^-12, 32) (4352
// doubles); the sweep and final kernels copy the table into LDS and look weights up.
// Other values, and fp32 logits, take the fp64 exponential of sv_device.h.  A weight so
// computed below 2^-70 of its row maximum counts as 0: over any vocabulary that moves the
// normalisers by less than V 2^-70 relative.
//
// Sweep (each workgroup one chunk of the row, each wave a run of kSeg-position segments):
// per segment S_p, S_q, and the sums A, B of a_i, b_i over the positions whose residual is
// positive for every normaliser ratio within 1 +- kDelta of the pass-1 estimate.  The sign
// test is on the logit difference: p_i > q_i exactly when zt_i - zd_i > tau =
// T ln(S_p/S_q) + refA - refB.  Positions whose difference falls inside the bracket go to
// buckets of equal difference (equal difference, equal a/b ratio, one residual sign), each
// with its sums of a and b.
//
// Final (one workgroup per sequence, after every sweep): exact fp64 normalisers, the check
// that the estimate bracketed them (else one exact sweep by this workgroup), each
// segment's residual mass A/S_p - B/S_q plus the positive bucket masses, a scan of the
// masses for u * W, and a scan inside the segment that holds it:
// token = min{ i : C_i > u * W }, C the prefix sums in index order.
#pragma once

#include <float.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>

#include "sv_common.h"
#include "sv_device.h"

namespace sv {

namespace {

constexpr double kLog2eD = 1.4426950408889634;
// Bracket around the pass-1 normaliser ratio (pass-1 normalisers are within ~1e-6 of the
// fp64 ones), and the part of it the exact ratio must fall in for the classification to
// stand: ln(1 + kDelta) and ln(1 - kDelta).
constexpr double kDelta = 8e-6;
constexpr double kLnDeltaHi = 7.999968000170666e-06;
constexpr double kLnDeltaLo = -8.000032000170667e-06;
// ln(1 + x) < x < -ln(1 - x) for 0 < x < 1, to the digits given
static_assert(kLnDeltaHi < kDelta && kDelta < -kLnDeltaLo && kDelta - kLnDeltaHi < 3.3e-11 &&
                  -kLnDeltaLo - kDelta < 3.3e-11,
              "the bracket's logarithms");
// Weights below 2^-kFlushLog2 of their row maximum count as 0.
constexpr double kFlushLog2 = 70.0;
// One shared weight reference for both rows while the row maxima differ by at most this
// many binary orders of magnitude (then every weight that is not flushed stays normal).
constexpr double kMaxRefGapLog2 = 900.0;
// Row statistics of the resolve kept in LDS; rows past this are merged again on demand.
constexpr int kRowsLds = 64;
static_assert(kRowsLds <= 64, "with every row in LDS (2K + 1 <= kRowsLds) one wave holds the K tests");
// Pass-1 partials of one sequence the resolve stages in LDS (16 KB); more stay in memory.
constexpr int kPartsLds = 1024;
// Threads of a resolve workgroup (one workgroup per sequence).
#ifndef SV_RESOLVE_THREADS
#define SV_RESOLVE_THREADS 1024
#endif
constexpr int kResolveThreads = SV_RESOLVE_THREADS;
// Threads of a final workgroup (one workgroup per sequence; a multiple of kSeg / 8).
#ifndef SV_FINAL_THREADS
#define SV_FINAL_THREADS 512
#endif
constexpr int kFinalThreads = SV_FINAL_THREADS;

// bf16 weight table in LDS, the signs interleaved: slot 2q + s holds the weight of the bf16
// value with sign s whose 15-bit magnitude field is kTabLo + q, for q in [1, kTabN]: biased
// exponents 115..131, |z| in [2^-12, 32), the widest range in which the difference of two
// of its values is exact in fp32 (16 binary orders apart at most, 8 significant bits
// each).  Slots of q = 0 and q = kTabN + 1 hold NaN: a magnitude outside the range is
// clamped onto them, so a sum that met one turns NaN and its span is redone exactly.
constexpr uint32_t kTabLo = 115 * 128 - 1;
constexpr int kTabN = 17 * 128;
constexpr uint32_t kTabHi = kTabLo + kTabN + 1;
constexpr int kTabLen = 2 * (kTabN + 2);

// Waves per SIMD the sweep kernel's register allocation must allow (4 workgroups per CU).
#ifndef SV_DRAW_WAVES
#define SV_DRAW_WAVES 4
#endif

// 16-byte vectors per row whose loads are in flight together per lane; a span is what one
// wave covers with them.
#ifndef SV_SWEEP_G
#define SV_SWEEP_G 1
#endif
constexpr int kG = SV_SWEEP_G;
// Words of the fast path between scheduling fences (their table reads may overlap).
constexpr unsigned kXcds = 8;  // XCDs of an MI355X

#ifndef SV_SWEEP_WPF
#define SV_SWEEP_WPF 4
#endif
constexpr int kWordsPerFence = SV_SWEEP_WPF;
constexpr int kSpan16 = 64 * kG * 8;
static_assert(kSeg % kSpan16 == 0 && kSeg / kSpan16 <= 32, "draw segments are whole spans of bf16 vectors");


// The resolve's result for one sequence.
struct SeqDesc {
    int mode;      // kMode*
    int n;         // accepted drafts = row of the draw
    float T;       // temperature
    float u;       // uniform of the final draw
    float mt, md;  // maxima of target row n and draft row n
    int b;         // the sequence
    // residual draws: the bracket [tau_lo, tau_hi] on zt_i - zd_i around the sign threshold
    // T ln(St/Sd) + mt - md, St and Sd the pass-1 normalisers sum exp((z - m) / T) of the
    // two rows
    double tau_lo, tau_hi;
    int64_t trow;  // target row of the draw (also the output slot of the drawn token)
    int64_t drow;  // draft row of the draw (residual draws)
};

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
    float zx;  // sampled rows with a draft token: the logit at it
};

// ln x for finite x > 0 in fp64 (the resolve's few logarithms).
__device__ __forceinline__ double ln(double x) { return log(x); }

// Where the resolve finds a sequence's draft tokens and uniforms: the first kRowsLds
// tokens and kRowsLds + 1 uniforms in LDS, later ones in memory.
struct ResolveIn {
    const int32_t* xs;        // LDS tokens
    const float* us;          // LDS uniforms
    const int32_t* x;         // tokens in memory
    const float* u;           // uniforms in memory (null for greedy-only calls)
    __device__ __forceinline__ int token(int t) const { return t < kRowsLds ? xs[t] : x[t]; }
    __device__ __forceinline__ float uniform(int t) const { return t <= kRowsLds ? us[t] : u[t]; }
};

// Row i (0..K_b target rows, K_b+1..2K_b draft rows) of sequence b from its pass-1 chunk
// partials, by one thread.  Greedy: max and lowest index (chunks in order, strict
// comparison keeps the earlier chunk on ties).  Sampled: max m and S = the chunks' sums
// rebased from their own maxima to m, 2^((m_c - m) c2) in fp64, added in chunk order;
// `terms` (or null) holds those rebased sums, computed beforehand one per thread.
// `parts`: the sequence's partials (in LDS or in memory; the caller passes the array
// itself, so that the compiler sees which).
__device__ __forceinline__ RowStat merge_row(const VerifyArgs& a, const SeqRows& s, const ResolveIn& in,
                                             const RowPartial* parts, int i, bool sampled, float c2,
                                             const double* tab, const double* terms) {
    const bool is_target = i <= s.K;
    const int t = is_target ? i : i - s.K - 1;
    const int j = is_target ? t : a.K + 1 + t;  // workspace slot (dense layout, K the bound)
    const RowPartial* p = parts + (int64_t)j * a.nchunk1;
    RowStat r{-INFINITY, 0x7fffffff, 0.0, -INFINITY};
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
    // the chunk holding this row's draft token recorded the logit there
    int cx = -1;
    if (t < s.K) {
        const int x = in.token(t);
        if (x >= 0 && x < a.V) cx = x / a.ch1;
    }
    r.zx = -INFINITY;
#pragma unroll 4
    for (int c = 0; c < a.nchunk1; ++c) r.m = nmax(r.m, p[c].m);
#pragma unroll 4
    for (int c = 0; c < a.nchunk1; ++c) {
        const RowPartial q = p[c];
        if (q.s != 0.0)
            r.S += terms ? terms[(int64_t)i * a.nchunk1 + c]
                         : q.s * exp2_256(((double)q.m - (double)r.m) * ((double)c2 * 256.0), tab);
        if (c == cx) r.zx = __int_as_float(q.idx);
    }
    return r;
}

// The rebased chunk sum of sampled row i, chunk c (see merge_row).
__device__ __forceinline__ double chunk_term(const VerifyArgs& a, const SeqRows& s, const RowPartial* parts,
                                             int i, int c, float c2, const double* tab) {
    const bool is_target = i <= s.K;
    const int t = is_target ? i : i - s.K - 1;
    const int j = is_target ? t : a.K + 1 + t;
    const RowPartial* p = parts + (int64_t)j * a.nchunk1;
    float m = -INFINITY;
    for (int cc = 0; cc < a.nchunk1; ++cc) m = nmax(m, p[cc].m);
    const RowPartial q = p[c];
    return q.s != 0.0 ? q.s * exp2_256(((double)q.m - (double)m) * ((double)c2 * 256.0), tab) : 0.0;
}

// Every row of the sequence from its partials in LDS, by lane groups: G lanes per row (G the
// power of two at or above nchunk1), chunk c of row i on thread i G + c, which the caller
// guarantees covers them (G <= 64, so that a group lies inside one wave; nrows <= kRowsLds;
// nrows G <= blockDim.x).  Group maxima by
// shuffles; the rebased sums added in chunk order with the very operations of merge_row,
// so the result has merge_row's bits.  Rows past the first L positions (early exit) get
// the placeholder of rows not read.  Returns this thread's error bits.
__device__ __forceinline__ int merge_rows_grouped(const VerifyArgs& a, const SeqRows& s, const ResolveIn& in,
                                                  const RowPartial* parts, int nrows, bool sampled, float c2,
                                                  const double* tab, int L, RowStat* rows) {
    const int nc = a.nchunk1;
    int lg = 0;
    while ((1 << lg) < nc) ++lg;
    const int tid = threadIdx.x, i = tid >> lg, c = tid & ((1 << lg) - 1);
    const int base = (tid & 63) - c;  // lane of the group's chunk 0
    if (i >= nrows) return 0;  // whole groups
    const bool is_target = i <= s.K;
    const int t = is_target ? i : i - s.K - 1;
    if (t >= L) {
        if (c == 0) rows[i] = RowStat{0.0f, -1, 1.0, -INFINITY};
        return 0;
    }
    const int j = is_target ? t : a.K + 1 + t;  // workspace slot (dense layout, K the bound)
    const bool live = c < nc;
    RowPartial q;
    q.m = -INFINITY;
    q.idx = 0;
    q.s = 0.0;
    if (live) q = parts[(int64_t)j * nc + c];
    RowStat r{-INFINITY, 0x7fffffff, 0.0, -INFINITY};
    if (!sampled) {
        // the strict maximum over chunks in order: the first chunk reaching the maximum of
        // the chunk maxima that are not NaN; any NaN marks the row
        const bool nan = live && q.m != q.m;
        float m = nan ? -INFINITY : q.m;
        for (int o = 1; o < (1 << lg); o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
        int first = (live && !nan && q.m == m && m > -INFINITY) ? c : 0x7fff;
        int bad = nan;
        for (int o = 1; o < (1 << lg); o <<= 1) {
            first = min(first, __shfl_xor(first, o, 64));
            bad |= __shfl_xor(bad, o, 64);
        }
        const int idx = __shfl(q.idx, base + (first == 0x7fff ? 0 : first), 64);
        r.m = bad ? __builtin_nanf("") : m;
        r.idx = first == 0x7fff ? 0x7fffffff : idx;
    } else {
        float m = q.m;
        for (int o = 1; o < (1 << lg); o <<= 1) m = nmax(m, __shfl_xor(m, o, 64));
        r.m = m;
        const double term = (live && q.s != 0.0)
                                ? q.s * exp2_256(((double)q.m - (double)m) * ((double)c2 * 256.0), tab)
                                : 0.0;
        for (int cc = 0; cc < nc; ++cc) r.S += __shfl(term, base + cc, 64);
        // the chunk holding this row's draft token recorded the logit there
        int cx = -1;
        if (t < s.K) {
            const int x = in.token(t);
            if (x >= 0 && x < a.V) cx = x / a.ch1;
        }
        const int zbits = __shfl(q.idx, base + (cx < 0 ? 0 : cx), 64);
        r.zx = cx < 0 ? -INFINITY : __int_as_float(zbits);
    }
    if (c != 0) return 0;
    if (i < kRowsLds) rows[i] = r;
    return row_bad(r.m, sampled) ? kSeqErrLogit : 0;
}

// The test of position t: r < p/q, i.e. r St < Sd 2^((ex - dxm) c2) with ex = zx - mt and
// dxm = dx - md; q = 0 with p > 0 accepts, p = 0 rejects (2^y saturates to inf above and
// to 0 below the fp64 range).
__device__ __forceinline__ bool accept_test(const RowStat& rt, const RowStat& rd, float ut, double c256,
                                            const double* tab) {
    const double ex = (double)rt.zx - (double)rt.m, dxm = (double)rd.zx - (double)rd.m;
    if (rt.zx == -INFINITY) return false;
    if (rd.zx == -INFINITY) return true;
    if (ut == 0.0f) return true;
    return (double)ut * rt.S < rd.S * exp2_256((ex - dxm) * c256, tab);
}

// The resolve of sequence b by the whole workgroup of NT threads.  write: also write the
// outputs (all but the drawn token of a sampled sequence, and its status).  Returns the
// same SeqDesc in every thread, without the sign bracket of a residual draw (tau_lo,
// tau_hi; see desc_bracket).  Contains __syncthreads().
template <typename E, int NT>
__device__ __forceinline__ SeqDesc resolve_seq(const VerifyArgs& a, int b, bool write, double* tab,
                                               double& St, double& Sd) {
    constexpr int NW = NT / 64;
    __shared__ RowStat rows[kRowsLds];
    __shared__ RowPartial parts[kPartsLds];
    __shared__ double terms[kPartsLds];
    __shared__ int32_t xs[kRowsLds];
    __shared__ float us[kRowsLds + 1];
    __shared__ int shi[NW];
    const int tid = threadIdx.x;
    St = Sd = 0.0;
    const SeqRows s = seq_rows(a, b);
    if (s.K < 0) {
        // packed offsets that do not describe a sequence: nothing of it can be located
        if (write && tid == 0) {
            if (a.out_n) a.out_n[b] = -1;
            a.out_status[b] = kSeqErrOffsets;
        }
        SeqDesc d{};
        d.mode = kModeNone;
        return d;
    }
    const int K = s.K, V = a.V;
    const float T = a.temperature ? a.temperature[b] : 0.0f;
    // every load of the resolve goes out at once: the partials of all the sequence's
    // workspace rows (used or not), its tokens and uniforms (greedy sequences of a
    // sampled call read their uniforms too, unused)
    ResolveIn in;
    in.x = a.tokens + s.d0;
    in.u = a.uniforms ? a.uniforms + s.t0 : nullptr;
    in.xs = xs;
    in.us = us;
    const int nparts = a.R * a.nchunk1;
    const RowPartial* src = a.part1 + (int64_t)b * nparts;
    const bool staged = nparts <= kPartsLds;
    const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
    u32x4* d4 = reinterpret_cast<u32x4*>(parts);
    constexpr bool one_load = NT >= kPartsLds;  // one 16-byte load per thread stages them all
    if (staged && !one_load) {
        // two 16-byte loads in flight per thread (indices clamped, stores guarded)
        for (int i0 = 0; i0 < nparts; i0 += 2 * NT) {
            const int i1 = i0 + tid, i2 = i0 + NT + tid;
            const u32x4 q1 = s4[min(i1, nparts - 1)];
            const u32x4 q2 = s4[min(i2, nparts - 1)];
            if (i1 < nparts) d4[i1] = q1;
            if (i2 < nparts) d4[i2] = q2;
        }
    }
    const bool mine = staged && one_load && tid < nparts;
    const bool has_x = tid < K && tid < kRowsLds, has_u = in.u && tid <= K && tid <= kRowsLds;
    u32x4 qp{0u, 0u, 0u, 0u};
    int xv = 0;
    float uv = 0.0f;
    if (mine) qp = s4[tid];
    if (has_x) xv = in.x[tid];
    if (has_u) uv = in.u[tid];
    exp2_table_fill(tab);  // while the loads are in flight
    if (mine) d4[tid] = qp;
    if (has_x) xs[tid] = xv;
    if (has_u) us[tid] = uv;
    __syncthreads();  // publishes the staging and the exponential table
    const bool sampled = !(T == 0.0f);
    const float c2 = sampled ? (float)(kLog2eD / (double)T) : 0.0f;

    int err = 0;
    for (int t = tid; t < K; t += NT) {
        const int v = in.token(t);
        if (v < 0 || v >= V) err |= kSeqErrToken;
    }
    if (sampled)
        for (int t = tid; t <= K; t += NT) {
            const float v = in.uniform(t);
            if (!(v >= 0.0f && v < 1.0f)) err |= kSeqErrUniform;
        }
    if (tid == 0 && temperature_bad(T)) err |= kSeqErrTemperature;
    // row statistics (draft rows only for sampled sequences): with the partials in LDS
    // the rebasing exponentials of all (row, chunk) pairs first, one per thread, then one
    // thread per row
    const int nrows = sampled ? 2 * K + 1 : K + 1;
    // early exit: only the rows of the first L positions were read
    const int L = a.limit ? (a.limit[b] & ~kStopBit) : K + 1;
    auto row_read = [&](int i) { return (i <= K ? i : i - K - 1) < L; };
    int lg = 0;
    while ((1 << lg) < a.nchunk1) ++lg;
    // lane groups stay inside one wave (16 lanes at most: the chunk-order sum takes one
    // shuffle per chunk)
    const bool grouped = staged && lg <= 4 && nrows <= kRowsLds && (nrows << lg) <= NT;
    const bool by_pair = !grouped && staged && sampled && nrows <= kRowsLds;
    if (grouped) err |= merge_rows_grouped(a, s, in, parts, nrows, sampled, c2, tab, L, rows);
    if (by_pair) {
        for (int q = tid; q < nrows * a.nchunk1; q += NT) {
            const int i = q / a.nchunk1;
            if (row_read(i)) terms[q] = chunk_term(a, s, parts, i, q - i * a.nchunk1, c2, tab);
        }
        __syncthreads();
    }
    for (int i = grouped ? nrows : tid; i < nrows; i += NT) {
        if (!row_read(i)) {
            if (i < kRowsLds) rows[i] = RowStat{0.0f, -1, 1.0, -INFINITY};
            continue;
        }
        const RowStat r = staged ? merge_row(a, s, in, parts, i, sampled, c2, tab, by_pair ? terms : nullptr)
                                 : merge_row(a, s, in, src, i, sampled, c2, tab, nullptr);
        if (row_bad(r.m, sampled)) err |= kSeqErrLogit;
        if (i < kRowsLds) rows[i] = r;
    }
    err = block_or<NW>(err, shi);  // also orders the rows[] writes before the reads below
    auto row = [&](int i) -> RowStat {
        if (i < kRowsLds) return rows[i];
        return staged ? merge_row(a, s, in, parts, i, sampled, c2, tab, nullptr)
                      : merge_row(a, s, in, src, i, sampled, c2, tab, nullptr);
    };

    int32_t* tok = a.out_tokens + s.t0;
    float* op = a.out_p ? a.out_p + s.d0 : nullptr;
    float* oq = a.out_q ? a.out_q + s.d0 : nullptr;
    if (err) {
        if (write) {
            for (int t = tid; t <= K; t += NT) tok[t] = -1;
            for (int t = tid; t < K; t += NT) {
                if (op) op[t] = __builtin_nanf("");
                if (oq) oq[t] = __builtin_nanf("");
            }
            if (tid == 0) {
                if (a.out_n) a.out_n[b] = -1;
                a.out_status[b] = err;
            }
        }
        SeqDesc d{};
        d.mode = kModeNone;
        return d;
    }

    // the first position that fails.  With every row in LDS the tests and the reported
    // p, q go to separate threads; otherwise one thread per position (rows past kRowsLds
    // are merged again by the thread that needs them)
    const double c256 = sampled ? 256.0 * kLog2eD / (double)T : 0.0;
    const bool all_lds = nrows <= kRowsLds;
    const int Kt = min(K, L);  // positions whose rows were read (early exit: up to the stop)
    int first = K;
    if (!sampled) {
        for (int t = tid; t < K; t += NT) {
            if (write && op) op[t] = __builtin_nanf("");
            if (write && oq) oq[t] = __builtin_nanf("");
        }
        for (int t = tid; t < Kt; t += NT)
            if (row(t).idx != in.token(t)) first = min(first, t);
    } else if (all_lds && NT >= 192) {
        // the tests on wave 0, p on wave 1, q on wave 2 (K < kRowsLds <= 64 here): no wave
        // runs more than one kind
        const int kind = tid >> 6, t = tid & 63;
        if (kind < 3 && t < K) {
            const RowStat rt = rows[t], rd = rows[K + 1 + t];
            const double ex = (double)rt.zx - (double)rt.m, dxm = (double)rd.zx - (double)rd.m;
            if (kind == 1) {
                if (write && op) op[t] = t < Kt ? (float)(exp2_256(ex * c256, tab) / rt.S) : __builtin_nanf("");
            } else if (kind == 2) {
                if (write && oq) oq[t] = t < Kt ? (float)(exp2_256(dxm * c256, tab) / rd.S) : __builtin_nanf("");
            } else if (t < Kt) {
                if (!accept_test(rt, rd, in.uniform(t), c256, tab)) first = t;
            }
        }
    } else if (all_lds) {
        for (int q = tid; q < 3 * K; q += NT) {
            const int kind = q / K, t = q - kind * K;
            const RowStat rt = rows[t], rd = rows[K + 1 + t];
            // p = 2^((zx - mt) c2) / St and q = 2^((dx - md) c2) / Sd
            const double ex = (double)rt.zx - (double)rt.m, dxm = (double)rd.zx - (double)rd.m;
            if (kind == 1) {
                if (write && op) op[t] = t < Kt ? (float)(exp2_256(ex * c256, tab) / rt.S) : __builtin_nanf("");
            } else if (kind == 2) {
                if (write && oq) oq[t] = t < Kt ? (float)(exp2_256(dxm * c256, tab) / rd.S) : __builtin_nanf("");
            } else if (t < Kt) {
                if (!accept_test(rt, rd, in.uniform(t), c256, tab)) first = min(first, t);
            }
        }
    } else {
        for (int t = tid; t < K; t += NT) {
            if (t >= Kt) {
                if (write && op) op[t] = __builtin_nanf("");
                if (write && oq) oq[t] = __builtin_nanf("");
                continue;
            }
            const RowStat rt = row(t), rd = row(K + 1 + t);
            const double ex = (double)rt.zx - (double)rt.m, dxm = (double)rd.zx - (double)rd.m;
            if (write && op) op[t] = (float)(exp2_256(ex * c256, tab) / rt.S);
            if (write && oq) oq[t] = (float)(exp2_256(dxm * c256, tab) / rd.S);
            if (!accept_test(rt, rd, in.uniform(t), c256, tab)) first = min(first, t);
        }
    }
    const int n = block_min<NW>(first, shi);
    if (write)
        for (int t = tid; t <= K; t += NT)
            if (t != n) tok[t] = t < n ? in.token(t) : -1;
    // every thread reads the same rows: the descriptor in every thread
    const RowStat rt = row(n);
    SeqDesc d{};
    d.n = n;
    d.T = T;
    d.trow = s.t0 + n;
    d.drow = s.d0 + n;
    if (write && tid == 0 && a.out_n) a.out_n[b] = n;
    if (!sampled) {
        if (write && tid == 0) {
            tok[n] = rt.idx;
            a.out_status[b] = 0;
        }
        d.mode = kModeNone;
        return d;
    }
    d.mt = rt.m;
    d.md = rt.m;
    St = rt.S;
    if (n < K) {
        const RowStat rd = row(K + 1 + n);
        d.md = rd.m;
        Sd = rd.S;
        d.mode = kModeResidual;
    } else {
        d.mode = kModeBonus;
    }
    d.u = in.uniform(K);
    return d;
}

// The sign bracket of a residual draw: [tau_lo, tau_hi] on zt_i - zd_i around the
// threshold T ln(St/Sd) + mt - md, St and Sd the pass-1 normalisers of the two rows.
__device__ __forceinline__ void desc_bracket(SeqDesc& d, double St, double Sd) {
    d.tau_lo = d.tau_hi = 0.0;
    if (d.mode != kModeResidual) return;
    const double T = (double)d.T;
    const double base = T * ln(St / Sd) + ((double)d.mt - (double)d.md);
    d.tau_hi = base + T * kLnDeltaHi;
    d.tau_lo = base + T * kLnDeltaLo;
}

// ------------------------------------------------------------------------------------
// draw weights
// ------------------------------------------------------------------------------------

// Table slot of the bf16 value in the low 16 bits of x (higher bits ignored); values
// outside the table land on a NaN slot.
__device__ __forceinline__ uint32_t tab_slot(uint32_t x) {
    const uint32_t t = min(max(x & 0x7fffu, kTabLo), kTabHi);
    return 2 * (t - kTabLo) + ((x >> 15) & 1u);
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Byte offsets into the table of the two bf16 values packed in x (o0: low half, o1: high
// half): 8 tab_slot(...) of each, both halves at once with packed 16-bit integer
// arithmetic (saturating subtract, minimum, shift; 16 (kTabN + 1) + 8 < 2^16).
static_assert(16 * (kTabN + 1) + 8 < 65536, "table byte offsets fit 16 bits");
__device__ __forceinline__ void tab_offsets(uint32_t x, uint32_t& o0, uint32_t& o1) {
    const u16x2 m = __builtin_bit_cast(u16x2, x & 0x7fff7fffu);
    const u16x2 lo = {(unsigned short)kTabLo, (unsigned short)kTabLo};
    const u16x2 top = {(unsigned short)(kTabN + 1), (unsigned short)(kTabN + 1)};
    u16x2 c = __builtin_elementwise_sub_sat(m, lo);  // magnitude - kTabLo, or 0 below
    c = __builtin_elementwise_min(c, top);           // kTabN + 1 above
    c = c << (unsigned short)4;
    const uint32_t off = __builtin_bit_cast(uint32_t, c) | ((x >> 12) & 0x00080008u);  // + 8 sign
    o0 = off & 0xffffu;
    o1 = off >> 16;
}

__device__ __forceinline__ double tab_at(const double* wt, uint32_t off) {
    return *reinterpret_cast<const double*>(reinterpret_cast<const char*>(wt) + off);
}

// Whether the bf16 value in the low 16 bits of h has a table slot, and that slot.
__device__ __forceinline__ bool tab_has(uint32_t h, uint32_t& slot) {
    const uint32_t t = h & 0x7fffu;
    slot = 2 * (t - kTabLo) + ((h >> 15) & 1u);
    return t - (kTabLo + 1) < (uint32_t)kTabN;
}

template <typename E>
struct DrawRows {
    const E* t;            // target row of the draw
    const E* d;            // draft row (residual; the target row again otherwise)
    double refA, refB;     // weight references of the two rows
    double c256;           // 256 log2(e) / T
    double inv_sp, inv_sq; // 1 / S_p, 1 / S_q once known
    double tau_lo, tau_hi; // undecided bracket on zt - zd
    float tau_lo_f, tau_hi_f;  // the same, rounded outward to fp32
    float thr_t, thr_d;    // below these, computed weights are flushed (2^-70 of the row max)
    int residual;          // 1: (a/S_p - b/S_q)+ ; 0: a (bonus, or the draw from p_n)
    int vec_ok;            // both rows 16-byte aligned
    int one_ref;           // both rows share the reference (bf16: the table applies)
    int use_tab;           // bf16 with one shared reference: weights from the LDS table
    const double* tab;     // 2^(j/256), LDS
    const double* wt;      // bf16 weight table, LDS

    // exp((z - ref)/T) = 2^((z - ref) * 256 log2(e)/T / 256); z - ref is exact in fp64.
    // Table values are that same function of the same operands.
    __device__ __forceinline__ double a_of(float z) const {
        if constexpr (sizeof(E) == 2) {
            uint32_t k;
            if (use_tab && tab_has(__float_as_uint(z) >> 16, k)) return wt[k];
        }
        if (!(z >= thr_t)) return 0.0;
        return exp2_256(exp2_arg((double)z, refA, c256), tab);
    }
    __device__ __forceinline__ double b_of(float z) const {
        if constexpr (sizeof(E) == 2) {
            uint32_t k;
            if (use_tab && tab_has(__float_as_uint(z) >> 16, k)) return wt[k];
        }
        if (!(z >= thr_d)) return 0.0;
        return exp2_256(exp2_arg((double)z, refB, c256), tab);
    }
    __device__ __forceinline__ double weight(float zt, float zd) const {
        const double a = a_of(zt);
        if (!residual) return a;
        const double w = a * inv_sp - b_of(zd) * inv_sq;
        return w > 0.0 ? w : 0.0;
    }
};

// The draw rows of sequence b and their weight parameters (no LDS access).
template <typename E>
__device__ __forceinline__ DrawRows<E> draw_rows(const VerifyArgs& a, const SeqDesc& d,
                                                 const double* tab, const double* wt) {
    DrawRows<E> r;
    r.residual = d.mode == kModeResidual;
    r.t = static_cast<const E*>(a.target) + d.trow * a.V;
    r.d = r.residual ? static_cast<const E*>(a.draft) + d.drow * a.V : r.t;
    const double T = (double)d.T;
    const double c2 = kLog2eD / T;
    r.c256 = 256.0 * c2;
    const double mt = (double)d.mt, md = r.residual ? (double)d.md : mt;
    const bool one_ref = fabs(mt - md) * c2 <= kMaxRefGapLog2;
    const double M = fmax(mt, md);
    r.refA = one_ref ? M : mt;
    r.refB = one_ref ? M : md;
    r.one_ref = one_ref;
    r.use_tab = sizeof(E) == 2 && one_ref && wt != nullptr;
    r.thr_t = (float)(mt - kFlushLog2 / c2);
    r.thr_d = r.residual ? (float)(md - kFlushLog2 / c2) : INFINITY;
    r.inv_sp = 1.0;
    r.inv_sq = 1.0;
    r.tau_lo = r.tau_hi = 0.0;
    r.tau_lo_f = r.tau_hi_f = 0.0f;
    if (r.residual) {
        // p_i > q_i  <=>  zt_i - zd_i > T ln(S_p/S_q) + refA - refB, which in the pass-1
        // terms is T ln(St/Sd) + mt - md: the resolve's bracket around it
        r.tau_hi = d.tau_hi;
        r.tau_lo = d.tau_lo;
        r.tau_hi_f = __double2float_ru(r.tau_hi);
        r.tau_lo_f = __double2float_rd(r.tau_lo);
    }
    r.vec_ok = ((reinterpret_cast<uintptr_t>(r.t) | reinterpret_cast<uintptr_t>(r.d)) & 15) == 0;
    r.tab = tab;
    r.wt = wt;
    return r;
}

static_assert(sizeof(RowPartial) == sizeof(u32x4), "partials move as 16-byte vectors");
static_assert(kTabLen == kWtabLen, "workspace slot of the weight table");

// The bf16 weight table of a sequence (kTabLen doubles) for reference r.refA (= r.refB),
// written to `dst`: each entry is the fp64 exponential of its bf16 value, exactly what
// DrawRows evaluates without the table.
template <typename E, int NT = kThreads>
__device__ __forceinline__ void weight_table_write(const DrawRows<E>& r, double* dst) {
#pragma unroll 4
    for (int k = threadIdx.x; k < kTabLen; k += NT) {
        const uint32_t q = (uint32_t)k >> 1;
        double v = __builtin_nan("");
        if (q != 0 && q != (uint32_t)kTabN + 1) {
            const uint32_t h = ((uint32_t)k & 1u) << 15 | (kTabLo + q);
            v = exp2_256(exp2_arg((double)__uint_as_float(h << 16), r.refA, r.c256), r.tab);
        }
        dst[k] = v;
    }
}

// A sequence's weight table on its way from the workspace into LDS, in 16-byte pieces:
// load() puts every load in flight at once, store() writes LDS later (the caller's next
// __syncthreads() publishes it), so other loads can go out in between.
template <int NT>
struct TableCopy {
    static constexpr int kPieces = kTabLen / 2;
    static constexpr int kN = (kPieces + NT - 1) / NT;
    u32x4 v[kN];
    __device__ __forceinline__ void load(const double* src) {
        const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
#pragma unroll
        for (int k = 0; k < kN; ++k) {
            const int i = (int)threadIdx.x + k * NT;
            v[k] = s4[kPieces % NT == 0 ? i : min(i, kPieces - 1)];
        }
    }
    __device__ __forceinline__ void store(double* wt) const {
        u32x4* d4 = reinterpret_cast<u32x4*>(wt);
#pragma unroll
        for (int k = 0; k < kN; ++k) {
            const int i = (int)threadIdx.x + k * NT;
            if (kPieces % NT == 0 || i < kPieces) d4[i] = v[k];
        }
    }
};

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

// Positions of segment k of length L: [k * L, min(V, (k + 1) * L)).
__device__ __forceinline__ void seg_range(int V, int L, int k, int& lo, int& hi) {
    lo = min(V, k * L);
    hi = min(V, lo + L);
}

// ------------------------------------------------------------------------------------
// search inside a range of the draw row(s) (final kernel, sampler)
// ------------------------------------------------------------------------------------

// Smallest i in [lo, hi) with base + (w_lo + ... + w_i) > target, in tiles of VEC positions
// per thread (thread-local prefix, then a workgroup exclusive scan of the thread totals).
// standalone: base = 0 and target = u * (sum over the range), taken by a first sweep.
// If no index qualifies (rounding), the last index with positive weight; -1 if none.
// lo must be a multiple of VEC.
template <typename E, int NT = kThreads>
__device__ __forceinline__ int block_search(const DrawRows<E>& r, int lo, int hi, double base, double target,
                            bool standalone, double u) {
    constexpr int VEC = Logit<E>::kVec;
    constexpr int NW = NT / 64;
    constexpr int kTile = VEC * NT;
    __shared__ double shd[NW];
    __shared__ int shi[NW];
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
            tot += block_sum<NW>(s, shd);
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
        const double ex = block_exclusive_scan<NW>(run, tile_tot, shd);
        double acc = base + carry + ex;
        int found = 0x7fffffff;
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            acc += w[k];
            if (found == 0x7fffffff && w[k] > 0.0 && acc > target) found = i + k;
        }
        const int f = block_min<NW>(found, shi);
        if (f != 0x7fffffff) return f;
        carry += tile_tot;
    }
    return block_max<NW>(lastpos, shi);
}

// ------------------------------------------------------------------------------------
// LDS of the draw kernels
// ------------------------------------------------------------------------------------

template <typename E>
struct DrawLds {
    static constexpr int kWt = sizeof(E) == 2 ? kTabLen : 1;
};

static_assert(sizeof(SeqDesc) <= kSeqDescBytes && kSeqDescBytes % alignof(SeqDesc) == 0,
              "workspace slot of the descriptor");
static_assert(offsetof(SeqDesc, mode) == 0, "pass 1 clears deal entries through their first field");

}  // namespace

}  // namespace sv
