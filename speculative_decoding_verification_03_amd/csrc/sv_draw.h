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
// descriptor and, for bf16 logits, the sequence's weight table to the workspace.  Its
// device code is in sv_resolve.hip; this header holds what the draw kernels share.
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
// Weights below 2^-kFlushLog2 of their row maximum count as 0.
constexpr double kFlushLog2 = 70.0;
// One shared weight reference for both rows while the row maxima differ by at most this
// many binary orders of magnitude (then every weight that is not flushed stays normal).
constexpr double kMaxRefGapLog2 = 900.0;
// Threads of a final workgroup (one workgroup per sequence; a multiple of kSeg / 8).
constexpr int kFinalThreads = 512;

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
constexpr int kDrawWaves = 4;

// 16-byte vectors per row whose loads are in flight together per lane; a span is what one
// wave covers with them.
constexpr int kG = 1;
// Words of the fast path between scheduling fences (their table reads may overlap).
constexpr unsigned kXcds = 8;  // XCDs of an MI355X

constexpr int kWordsPerFence = 4;
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
// validation shared by the resolve and the sampler
// ------------------------------------------------------------------------------------

__device__ __forceinline__ bool temperature_bad(float T) {
    return (T != T) || T < 0.0f || T == INFINITY || (T > 0.0f && T < FLT_MIN);
}

// A sampled row whose maximum m has |m| c2 >= 2^30, c2 = fp32(log2(e) / T), is a data
// error: pass 1 holds each lane's exponent reference R ~ m c2 as an fp32 number, whose
// rounding (up to half an ulp of R, 32 at 2^30) shifts the row maximum's own term
// 2^(m c2 - R); beyond 2^30 that shift could leave the range of an fp32 exponential and
// lose the term.  Checked only for a valid temperature (c2 finite and positive); the
// product of the two fp32 values is exact in fp64.
__device__ __forceinline__ bool scaled_range_bad(float m, float c2) {
    return c2 > 0.0f && c2 < INFINITY && fabs((double)m) * (double)c2 >= 0x1p30;
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
