// Pass 2 of the verify step: the resolve kernel (accept tests, outputs, the draw's
// descriptor and weight table), the early-exit prefix kernel, and the launch of the
// resolve, sweep and final kernels.
#include "sv_draw.h"

namespace sv {

namespace {

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

}  // namespace

// Waves the sweep keeps resident on the current device (kDrawWaves per SIMD, 4 SIMDs per
// compute unit), cached per device.
static int sweep_resident_waves() {
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
