// Pass 2 of the verify step: the resolve and the one categorical draw of each sequence,
// in three kernels: resolve_kernel (one workgroup per sequence), sweep_kernel over
// (sequence, chunk) workgroups, then final_kernel (one workgroup per sequence); and the
// draft-side sampler, sample_kernel (one workgroup per row).
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

// Positions of segment k of length L: [k * L, min(V, (k + 1) * L)).
__device__ __forceinline__ void seg_range(int V, int L, int k, int& lo, int& hi) {
    lo = min(V, k * L);
    hi = min(V, lo + L);
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

// ------------------------------------------------------------------------------------
// final
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
            seg_range(a.V, kSeg, hit, lo, hi);
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

// ------------------------------------------------------------------------------------
// the kernel
// ------------------------------------------------------------------------------------

template <typename E>
struct DrawLds {
    static constexpr int kWt = sizeof(E) == 2 ? kTabLen : 1;
};

static_assert(sizeof(SeqDesc) <= kSeqDescBytes && kSeqDescBytes % alignof(SeqDesc) == 0,
              "workspace slot of the descriptor");
static_assert(offsetof(SeqDesc, mode) == 0, "pass 1 clears deal entries through their first field");

// grid = sequences: the resolve.  Writes the outputs (all but a sampled sequence's drawn
// token and status), the sequence's SeqDesc and, for bf16 draws with one reference, the
// sequence's weight table.
template <typename E>
__global__ __launch_bounds__(kResolveThreads) void resolve_kernel(VerifyArgs a, int b0) {
    __shared__ double tab[kExpTable];
    const int b = b0 + (int)blockIdx.x;
    double St, Sd;
    SeqDesc d = resolve_seq<E, kResolveThreads>(a, b, true, tab, St, Sd);  // fills tab
    d.b = b;
    // thread 0 takes the draw's slot in the deal (residual draws, two rows, from the front;
    // bonus draws, one row, from the back; the atomic's round trip overlaps the weight
    // table) and finishes the descriptor while the others start on the table
    int slot = -1;
    if (threadIdx.x == 0) {
        if (a.deal && (d.mode == kModeResidual || d.mode == kModeBonus))
            slot = d.mode == kModeResidual ? atomicAdd(&a.deal[0], 1) : a.nseq2 - 1 - atomicAdd(&a.deal[1], 1);
        desc_bracket(d, St, Sd);
        reinterpret_cast<SeqDesc*>(a.desc)[b] = d;
    }
    if constexpr (sizeof(E) == 2) {
        if (d.mode != kModeNone) {
            const DrawRows<E> r = draw_rows<E>(a, d, tab, nullptr);  // the bracket is not used
            if (r.one_ref) weight_table_write<E, kResolveThreads>(r, a.wtab + (int64_t)b * kWtabLen);
        }
    }
    if (slot >= 0) reinterpret_cast<SeqDesc*>(a.deal_desc)[slot] = d;
}

// grid = (sequences rounded up to a multiple of kXcds) x nchunk2.  Sampled sequences:
// workgroup c of a sequence sweeps segments
// [c spc, (c + 1) spc) of the draw row(s), each wave a contiguous run of them, into
// per-segment partials.
template <typename E>
__global__ __launch_bounds__(kSweepThreads) __attribute__((amdgpu_waves_per_eu(SV_DRAW_WAVES)))
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
            const int lo = min(a.V, s0 * kSeg), hi = min(a.V, s1 * kSeg);
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
                if (r.residual) sweep_wave_tab<true>(r, lo, hi, kSeg, part, bkt, acc, f, have_first);
                else sweep_wave_tab<false>(r, lo, hi, kSeg, part, bkt, acc, f, have_first);
            }
            done = true;
        }
    }
    if (!done) {
        exp2_table_init(tab);
        if (s0 < s1) sweep_wave_exp<E>(r, min(a.V, s0 * kSeg), min(a.V, s1 * kSeg), kSeg, part, bkt, acc);
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
        final_seq_small<E, kFinalThreads, kSeg / kFinalThreads>(a, r, d, b, dp, bk0, bkt, a.nseg, kSeg);
    else
        final_seq<E, kFinalThreads>(a, r, d, b);
}

// ------------------------------------------------------------------------------------
// early exit: the tests of one round of positions
// ------------------------------------------------------------------------------------

// grid = sequences.  For a sequence still going (limit == t0; every sequence in the first
// round), the tests of positions [t0, min(t1, K)) from the rows pass 1 has just read, with
// the resolve's arithmetic (merge_row, accept_test: the resolve, which tests these
// positions again, reaches the same decisions).  limit becomes (n + 1) | kStopBit at the
// first failing position n, else min(t1, K + 1).  Invalid data only ends the sequence;
// the resolve reports it.
template <typename E>
__global__ __launch_bounds__(kThreads) void prefix_kernel(VerifyArgs a) {
    __shared__ double tab[kExpTable];
    __shared__ int shi[kWaves];
    const int b = blockIdx.x, tid = threadIdx.x;
    if (a.t0 > 0 && a.limit[b] != a.t0) return;  // whole workgroup: stopped earlier
    exp2_table_init(tab);
    const SeqRows s = seq_rows(a, b);
    const int K = s.K;
    const float T = a.temperature ? a.temperature[b] : 0.0f;
    const bool sampled = !(T == 0.0f);
    const float c2 = sampled ? (float)(kLog2eD / (double)T) : 0.0f;
    const double c256 = sampled ? 256.0 * kLog2eD / (double)T : 0.0;
    ResolveIn in;
    in.x = a.tokens + s.d0;
    in.u = a.uniforms ? a.uniforms + s.t0 : nullptr;
    in.xs = in.x;  // tokens and uniforms straight from memory
    in.us = in.u;
    const RowPartial* parts = a.part1 + (int64_t)b * a.R * a.nchunk1;
    const int te = min(a.t1, K);
    int first = 0x7fffffff;
    for (int t = a.t0 + tid; t < te; t += kThreads) {
        const RowStat rt = merge_row(a, s, in, parts, t, sampled, c2, tab, nullptr);
        bool ok;
        if (!sampled) {
            ok = rt.idx == in.x[t];
        } else {
            const RowStat rd = merge_row(a, s, in, parts, K + 1 + t, true, c2, tab, nullptr);
            const float ut = in.u[t];
            ok = (ut >= 0.0f && ut < 1.0f) && accept_test(rt, rd, ut, c256, tab);
        }
        if (!ok) first = min(first, t);
    }
    first = block_min(first, shi);
    if (tid == 0) a.limit[b] = first != 0x7fffffff ? (first + 1) | kStopBit : min(a.t1, K + 1);
}

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

#ifndef SV_SAMPLE_LOADS
#define SV_SAMPLE_LOADS 4
#endif

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
    constexpr int kU = SV_SAMPLE_LOADS;
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
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                bad |= (z[e] != z[e]) | (sampled && z[e] == INFINITY);
                if (z[e] > mx) {
                    mx = z[e];
                    idx = v * VEC + e;
                }
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

// Waves the sweep keeps resident on the current device (kDrawWaves per SIMD, 4 SIMDs per
// compute unit), cached per device.
int sweep_resident_waves() {
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1 << 30;
    if (cache[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            return 1 << 30;
        cache[dev] = cus * 4 * SV_DRAW_WAVES;
    }
    return cache[dev];
}

template <typename E>
void launch_all(const VerifyArgs& a, int b0, int b1, hipStream_t s) {
    VerifyArgs a2 = a;
    a2.nseq2 = b1 - b0;
    // deal the draws over the XCDs only when the sweep takes more than one round of
    // resident waves: in a single round every workgroup runs at once and nothing is gained
    const int64_t sweep_waves = (int64_t)(b1 - b0) * a.nchunk2 * (kSweepThreads / 64);
    if (!a.temperature || sweep_waves <= sweep_resident_waves()) a2.deal = nullptr;
    hipLaunchKernelGGL(resolve_kernel<E>, dim3((unsigned)(b1 - b0)), dim3(kResolveThreads), 0, s, a2, b0);
    if (!a.temperature) return;  // greedy only: the resolve is everything
    const int64_t padded = ((int64_t)(b1 - b0) + kXcds - 1) / kXcds * kXcds;
    const unsigned blocks = (unsigned)(padded * a.nchunk2);
    hipLaunchKernelGGL(sweep_kernel<E>, dim3(blocks), dim3(kSweepThreads), 0, s, a2, b0);
    hipLaunchKernelGGL(final_kernel<E>, dim3((unsigned)(b1 - b0)), dim3(kFinalThreads), 0, s, a2, b0);
}

int launch_prefix(const VerifyArgs& a, int bf16, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (bf16)
        hipLaunchKernelGGL(prefix_kernel<uint16_t>, dim3((unsigned)a.B), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(prefix_kernel<float>, dim3((unsigned)a.B), dim3(kThreads), 0, s, a);
    return (int)hipGetLastError();
}

int launch_sample(const VerifyArgs& a, int bf16, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (bf16)
        hipLaunchKernelGGL(sample_kernel<uint16_t>, dim3((unsigned)a.B), dim3(kSampleThreads), 0, s, a);
    else
        hipLaunchKernelGGL(sample_kernel<float>, dim3((unsigned)a.B), dim3(kSampleThreads), 0, s, a);
    return (int)hipGetLastError();
}

int launch_draw(const VerifyArgs& a, int bf16, int b0, int b1, void* stream) {
    if (b1 <= b0) return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (bf16) launch_all<uint16_t>(a, b0, b1, s);
    else launch_all<float>(a, b0, b1, s);
    return (int)hipGetLastError();
}

}  // namespace sv
