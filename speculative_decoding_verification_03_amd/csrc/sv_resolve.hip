// Pass 2 of the verify step: the resolve kernel (accept tests, outputs, the draw's
// descriptor and weight table), the early-exit prefix kernel, and the launch of the
// resolve, sweep and final kernels.
#include <atomic>

#include "sv_draw.h"

namespace sv {

namespace {

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
// Row statistics of the resolve kept in LDS; rows past this are merged again on demand.
constexpr int kRowsLds = 64;
static_assert(kRowsLds <= 64, "with every row in LDS (2K + 1 <= kRowsLds) one wave holds the K tests");
// Pass-1 partials of one sequence the resolve stages in LDS (16 KB); more stay in memory.
constexpr int kPartsLds = 1024;
// Threads of a resolve workgroup (one workgroup per sequence).
constexpr int kResolveThreads = 1024;

// A row the sequence reads is bad when its maximum is NaN (a NaN anywhere) or -inf, or,
// sampled, +inf or out of the scaled range (c2 = fp32(log2(e) / T)).
__device__ __forceinline__ bool row_bad(float m, bool sampled, float c2) {
    return (m != m) || m == -INFINITY || (sampled && (m == INFINITY || scaled_range_bad(m, c2)));
}

struct RowStat {
    float m;   // row maximum (NaN if any chunk saw a NaN)
    int idx;   // greedy rows: lowest index reaching m
    double S;  // sampled rows: sum exp((z - m) / T)
    float zx;  // sampled rows with a draft token: the logit at it
};

// ln x for finite x > 0 in fp64 (the resolve's few logarithms).
__device__ __forceinline__ double ln(double x) { return log(x); }

// Where the resolve finds a sequence's draft tokens and uniforms: the first nx tokens and
// nu uniforms in LDS, later ones in memory.
struct ResolveIn {
    const int32_t* xs;        // LDS tokens
    const float* us;          // LDS uniforms
    const int32_t* x;         // tokens in memory
    const float* u;           // uniforms in memory (null for greedy-only calls)
    int nx, nu;
    __device__ __forceinline__ int token(int t) const { return t < nx ? lds(xs)[t] : gbl(x)[t]; }
    __device__ __forceinline__ float uniform(int t) const { return t < nu ? lds(us)[t] : gbl(u)[t]; }
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
    return row_bad(r.m, sampled, c2) ? kSeqErrLogit : 0;
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
    in.nx = kRowsLds;
    in.nu = kRowsLds + 1;
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
        if (row_bad(r.m, sampled, c2)) err |= kSeqErrLogit;
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
    in.xs = nullptr;  // tokens and uniforms straight from memory
    in.us = nullptr;
    in.nx = in.nu = 0;
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

}  // namespace

// Waves the sweep keeps resident on the current device (kDrawWaves per SIMD, 4 SIMDs
// per compute unit), cached per device; calls from several host threads may fill an entry
// together (with the same value).
static int sweep_resident_waves() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1 << 30;
    int w = cache[dev].load(std::memory_order_relaxed);
    if (w == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            return 1 << 30;
        w = cus * 4 * kDrawWaves;
        cache[dev].store(w, std::memory_order_relaxed);
    }
    return w;
}

int launch_draw(const VerifyArgs& a, int bf16, int b0, int b1, void* stream) {
    if (b1 <= b0) return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    VerifyArgs a2 = a;
    a2.nseq2 = b1 - b0;
    // deal the draws over the XCDs only when the sweep takes more than one round of
    // resident waves: in a single round every workgroup runs at once and nothing is gained
    const int64_t sweep_waves = (int64_t)(b1 - b0) * a.nchunk2 * (kSweepThreads / 64);
    if (!a.temperature || sweep_waves <= sweep_resident_waves()) a2.deal = nullptr;
    if (bf16)
        hipLaunchKernelGGL(resolve_kernel<uint16_t>, dim3((unsigned)(b1 - b0)), dim3(kResolveThreads), 0, s, a2, b0);
    else
        hipLaunchKernelGGL(resolve_kernel<float>, dim3((unsigned)(b1 - b0)), dim3(kResolveThreads), 0, s, a2, b0);
    if (!a.temperature) return (int)hipGetLastError();  // greedy only: the resolve is everything
    const int64_t padded = ((int64_t)(b1 - b0) + kXcds - 1) / kXcds * kXcds;
    const int e = launch_sweep(a2, bf16, b0, (unsigned)(padded * a.nchunk2), stream);
    if (e) return e;
    return launch_final(a2, bf16, b0, b1, stream);
}

int launch_prefix(const VerifyArgs& a, int bf16, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (bf16)
        hipLaunchKernelGGL(prefix_kernel<uint16_t>, dim3((unsigned)a.B), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(prefix_kernel<float>, dim3((unsigned)a.B), dim3(kThreads), 0, s, a);
    return (int)hipGetLastError();
}

}  // namespace sv
