// Shared host/device definitions of the verify library: workspace layout, chunking,
// kernel argument blocks and the internal launchers.  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace sv {

constexpr int kThreads = 256;  // workgroup size of the streaming, sweep and final kernels
constexpr int kWaves = kThreads / 64;

// Per-sequence status flags (same values as the public SV_SEQ_* macros).
constexpr int kSeqErrToken = 1;
constexpr int kSeqErrLogit = 2;
constexpr int kSeqErrTemperature = 4;
constexpr int kSeqErrUniform = 8;
constexpr int kSeqNoteFallback = 16;
constexpr int kSeqErrOffsets = 32;
constexpr int kSeqErrTree = 64;

// Largest token tree (nodes per sequence, root included) of the tree entry points.
constexpr int kTreeMaxNodes = 1024;

// Draw modes handed from the resolve to the sweep and final kernels.
constexpr int kModeNone = 0;      // greedy or failed: outputs complete after the resolve
constexpr int kModeResidual = 1;  // draw from (p_n - q_n)+
constexpr int kModeBonus = 2;     // draw from p_K

// One (row, chunk) result of pass 1.  Greedy rows: m = chunk max, idx = lowest index
// reaching it.  Sampled rows: m = chunk max, s = sum_i 2^((z_i - m) * c2) over the chunk,
// c2 = fp32(log2(e) / T) (fp32 exponentials, fp64 sum); idx = the bits of the fp32 logit at
// the row's draft token when that token lies in the chunk.
struct alignas(16) RowPartial {
    float m;
    int32_t idx;
    double s;
};

// Sweep results per (sequence, segment of kSeg positions), fp64, with
//   a_i = exp((zt_i - mt)/T) and b_i = exp((zd_i - md)/T):
//   sp, sq = sum a_i, sum b_i;
//   A, B   = sums of a_i, b_i over the positions whose residual is certainly positive;
//   nbkt   = buckets of undecided positions: positions whose logit difference
//            D_i = (zt_i - mt) - (zd_i - md) lies too close to the sign threshold, grouped
//            by equal D_i (equal D means equal a_i / b_i, hence one residual sign); each
//            bucket keeps its sums of a_i and b_i.  nbkt > kBuckets: the buckets overflowed.
// Bonus draws use sp only.
constexpr int kBuckets = 16;
struct alignas(16) DrawPartial {
    double sp, sq, A, B;
    int32_t nbkt;
    int32_t pad[3];
};
struct alignas(16) Bucket {
    double a, b;
};

constexpr int kSeg = 4096;         // longest draw segment (positions; one partial each)
constexpr int kSegMin = 512;       // shortest draw segment
constexpr int64_t kSegCount = 4096;  // segments a call aims for: one per resident sweep wave
constexpr int kWtabLen = 4356;     // doubles per sequence of the bf16 weight table
constexpr int kSeqDescBytes = 64;  // workspace slot of the resolve's per-sequence result

struct Layout {
    int nchunk1, ch1;  // pass-1 chunks per row and elements per chunk (multiple of 64)
    int seg;           // positions per draw segment of this call (seg_len)
    int nseg;          // draw segments per sequence: ceil(V / seg)
    size_t off_desc, off_part1, off_part2, off_bkt, off_wtab, off_limit, off_deal, off_deal_desc, total;
};

// Early exit: positions are read in rounds [t0, t1); limit[b] holds how many positions
// of sequence b have been read (target and draft rows), with kStopBit set once one of
// its tests has failed (nothing more of it is read).
constexpr int32_t kStopBit = 0x40000000;

// Pass-1 chunks of about kChunkBytes1 (long streams per workgroup), more when the batch
// is too small to fill the chip, never shorter than kMinChunk1 elements.
constexpr int64_t kChunkBytes1 = 76 * 1024;
constexpr int kTargetBlocks1 = 4096;
constexpr int kMinChunk1 = 4096;
constexpr int kTargetBlocks2 = 2560;
// Threads of a sweep workgroup: each wave sweeps its own run of draw segments.
constexpr int kSweepThreads = 256;
// The one-workgroup-per-row sampler: threads, positions per segment sum, and the longest
// row it takes (segments; longer rows take the verify kernels at K = 0).
constexpr int kSampleThreads = 1024;
constexpr int kSampleSeg = 2048;
constexpr int kSampleMaxSeg = 2 * kSampleThreads;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline void chunking1(int64_t rows, int V, int esize, int& nchunk1, int& ch1) {
    int64_t by_bytes = ceil_div((int64_t)V * esize, kChunkBytes1);
    int64_t want = rows > 0 ? ceil_div(kTargetBlocks1, rows) : 1;
    int64_t maxc = V / kMinChunk1;
    if (maxc < 1) maxc = 1;
    if (want > maxc) want = maxc;
    int64_t n = by_bytes > want ? by_bytes : want;
    if (n < 1) n = 1;
    const int64_t ch = ceil_div(ceil_div(V, n), 64) * 64;
    nchunk1 = (int)ceil_div(V, ch);
    ch1 = (int)ch;
}

// Draw segment length of a call over B sequences of V positions: the shortest power of two
// in [kSegMin, kSeg] that keeps the call's segments (one sweep wave each) near kSegCount,
// so that a small batch still spreads its draws over the chip's waves; large batches take
// kSeg (the sweep then needs several rounds of resident waves anyway).
inline int seg_len(int64_t B, int V) {
    int L = kSegMin;
    while (L < kSeg && B * ceil_div(V, (int64_t)L) > kSegCount) L *= 2;
    return L;
}

inline int segments(int V, int seg) { return (int)ceil_div(V, (int64_t)seg); }

// Draw chunks (workgroups) per sequence for a launch over `seqs` sequences: about
// kTargetBlocks2 workgroups in all; each chunk holds spc whole segments, at least one per
// wave of a workgroup when the row has that many (each workgroup copies the weight table
// once, so a chunk should keep all its waves busy).
inline void chunking2(int64_t seqs, int V, int seg, int& nchunk2, int& spc) {
    const int64_t nseg = segments(V, seg);
    const int64_t want = seqs > 0 ? ceil_div(kTargetBlocks2, seqs) : 1;
    const int64_t n = want < 1 ? 1 : (want > nseg ? nseg : want);
    int64_t per = ceil_div(nseg, n);
    const int64_t waves = kSweepThreads / 64;
    if (per < waves) per = nseg < waves ? nseg : waves;
    spc = (int)per;
    nchunk2 = (int)ceil_div(nseg, spc);
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// rows_per_seq = 2K+1 for spec_verify, K+1 for spec_verify_greedy.
inline Layout make_layout(int B, int K, int V, int esize, int rows_per_seq) {
    (void)K;
    Layout L;
    chunking1((int64_t)B * rows_per_seq, V, esize, L.nchunk1, L.ch1);
    L.seg = seg_len(B, V);
    L.nseg = segments(V, L.seg);
    size_t off = 0;
    L.off_desc = off;
    off = align256(off + kSeqDescBytes * (size_t)B);
    L.off_part1 = off;
    off = align256(off + sizeof(RowPartial) * (size_t)B * rows_per_seq * L.nchunk1);
    L.off_part2 = off;
    off = align256(off + sizeof(DrawPartial) * (size_t)B * L.nseg);
    L.off_bkt = off;
    off = align256(off + sizeof(Bucket) * kBuckets * (size_t)B * L.nseg);
    L.off_wtab = off;
    if (esize == 2) off = align256(off + sizeof(double) * kWtabLen * (size_t)B);
    L.off_limit = off;
    off = align256(off + sizeof(int32_t) * (size_t)B);
    L.off_deal = off;
    off = align256(off + 2 * sizeof(int32_t));
    L.off_deal_desc = off;
    off = align256(off + kSeqDescBytes * (size_t)B);
    L.total = off;
    return L;
}

// Row layout.  Dense calls (cu == nullptr): every sequence has K drafts; target rows
// [B][K+1], draft rows, tokens, p and q [B][K], uniforms and output tokens [B][K+1].
// Packed calls: sequence b has K_b = cu[b+1] - cu[b] <= K drafts; its draft rows, tokens,
// p and q start at index cu[b], its target rows, uniforms and output tokens at cu[b] + b.
// Workspace slots keep the dense [B][R] shape either way (R = 2K+1 or K+1, K the bound).
struct VerifyArgs {
    const void* target;        // target rows
    const void* draft;         // draft rows (may be null when greedy-only or K == 0)
    const int32_t* tokens;     // draft tokens
    const float* uniforms;     // (null when greedy-only)
    const float* temperature;  // [B] (null when greedy-only)
    const int32_t* cu;         // [B+1] packed offsets, or null (dense)
    int total;                 // packed calls: draft rows in all (cu[B] when valid)
    int B, K, V, R;            // R = rows per sequence handled by pass 1
    int nchunk1, ch1;          // pass-1 chunking
    int nchunk2, spc;          // draw chunking of this launch: chunks per sequence, segments
                               // per chunk
    int seg;                   // positions per draw segment (seg_len)
    int nseg;                  // draw segments per sequence
    int nseq2;                 // sequences of this draw launch (set by the launcher)
    // The draw deal of this call (null when no draw follows): deal_desc[nseq2] descriptors
    // (kSeqDescBytes each) and deal[2] counts.  Pass 1 resets it (counts 0, every entry's
    // mode kModeNone); each resolve workgroup with a draw copies its descriptor into it,
    // residual draws from the front, bonus draws from the back, deal[0] and deal[1]
    // counting them.
    int32_t* deal;
    void* deal_desc;
    void* desc;                // [B] the resolve's result per sequence (kSeqDescBytes each)
    RowPartial* part1;         // [B][R][nchunk1]
    DrawPartial* part2;        // [B][nseg]
    Bucket* bkt;               // [B][nseg][kBuckets]
    double* wtab;              // bf16: [B][kWtabLen] weight table of each sequence's draw
    // when u_gen is set, pass 1 also writes uniforms[B][K+1] (dense layout) from the
    // counter generator with these parameters; the resolve reads them after it
    float* u_gen;
    uint64_t seed, domain, step;
    // early exit (null: every row is read): pass 1 and the prefix test take the positions
    // [t0, t1) of the sequences still going; the resolve uses the rows read
    int32_t* limit;
    int t0, t1;
    int32_t* out_tokens;
    int32_t* out_n;            // may be null (plain sampling)
    float* out_p;
    float* out_q;
    int32_t* out_status;
};

// Tree verification: parents [B][N] (root -1, else in [0, j)), node tokens [B][N] (node
// 0's unused); part1 holds pass 1's greedy partials of the N target rows per sequence.
struct TreeArgs {
    const int32_t* parents;
    const int32_t* tokens;
    const RowPartial* part1;  // [B][N][nchunk1]
    int B, N, V, nchunk1;
    int32_t* out_tokens;      // [B][N]
    int32_t* out_nodes;       // [B][N] or null
    int32_t* out_n;           // [B]
    int32_t* out_status;      // [B]
    uint8_t* out_mask;        // [B][N][N] (mask kernel)
    int32_t* out_depth;       // [B][N] or null (mask kernel)
};

// Host helpers of the C entry points (sv_api.cpp): the shape check, the workspace size
// of (B, K, V), and spec_verify's validation and launches on a given workspace (returns
// an sv_status; profile: record the benchmark events while they are on; launch_it false:
// validate the arguments only, touching neither the workspace nor the GPU).
bool shape_ok(int B, int K, int V);
size_t workspace_need(int B, int K, int V);
int verify_dense_call(const void* target_logits, const void* draft_logits, int dtype,
                      const int32_t* draft_tokens, const float* uniforms,
                      const float* temperature, int B, int K, int V,
                      int32_t* out_tokens, int32_t* out_accept_len,
                      float* out_p, float* out_q, int32_t* out_status,
                      void* workspace, size_t workspace_bytes, void* stream, bool profile,
                      bool launch_it);

// Internal launchers (return hipError_t as int; 0 = success).  Sequences [b0, b1).
// launch_draw runs the resolve and the draws of those sequences (greedy-only calls: the
// resolve only) after their pass 1, on the same stream.
int launch_pass1(const VerifyArgs& a, int bf16, int b0, int b1, void* stream);
int launch_draw(const VerifyArgs& a, int bf16, int b0, int b1, void* stream);
// The two draw kernels after the resolve (launch_draw's steps): the sweep over `blocks`
// workgroups and the final kernel over sequences [b0, b1).
int launch_sweep(const VerifyArgs& a, int bf16, int b0, unsigned blocks, void* stream);
int launch_final(const VerifyArgs& a, int bf16, int b0, int b1, void* stream);
int launch_uniforms(uint64_t seed, uint64_t domain, uint64_t step, int B, int K, float* u,
                    void* stream);
int launch_tree(const TreeArgs& a, void* stream);
// Early exit: the tests of positions [a.t0, a.t1) of the sequences still going.
int launch_prefix(const VerifyArgs& a, int bf16, void* stream);
// sv_sample with at most kSampleMaxSeg segments per row: one workgroup per row.
int launch_sample(const VerifyArgs& a, int bf16, void* stream);
int launch_tree_mask(const TreeArgs& a, void* stream);
// Packed layout: u[cu[b] + b + t] for t <= K_b of each sequence with valid offsets.
int launch_uniforms_packed(uint64_t seed, uint64_t domain, uint64_t step, int B, int K,
                           const int32_t* cu, int total, float* u, void* stream);

}  // namespace sv
