// Shared host/device definitions of the verify library: workspace layout, chunking,
// kernel argument blocks and the internal launchers.  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace sv {

constexpr int kThreads = 256;  // every kernel: 4 wave64 per workgroup
constexpr int kWaves = kThreads / 64;

// Pass-2 descriptor modes.
constexpr int kModeNone = 0;      // greedy, failed, or nothing to draw
constexpr int kModeResidual = 1;  // draw from (p_n - q_n)+
constexpr int kModeBonus = 2;     // draw from p_K

// Per-sequence status flags (same values as the public SV_SEQ_* macros).
constexpr int kSeqErrToken = 1;
constexpr int kSeqErrLogit = 2;
constexpr int kSeqErrTemperature = 4;
constexpr int kSeqErrUniform = 8;
constexpr int kSeqNoteFallback = 16;

// One (row, chunk) result of pass 1.  Greedy rows: m = chunk max, idx = lowest index
// reaching it.  Sampled rows: m = chunk max, s = sum_i exp((z_i - m) / T) over the chunk.
struct alignas(16) RowPartial {
    float m;
    int32_t idx;
    double s;
};

// Work item handed from the resolve to pass 2, one per sequence.
struct alignas(32) SeqDesc {
    int32_t mode;   // kMode*
    int32_t n;      // accepted drafts: the row pair (residual) or K (bonus)
    float T;        // temperature
    float mt;       // max of target row n
    float md;       // max of draft row n (residual only)
    float u;        // uniform of the final draw
    int32_t status; // flags so far
    int32_t pad;
};

// Pass-2 normaliser partials for one chunk of the rejected row pair.
struct alignas(16) NormPartial {
    double sp;
    double sq;
};

struct Layout {
    int nchunk1, ch1;  // pass-1 chunks per row and elements per chunk (multiple of 64)
    int nchunk2, ch2;  // pass-2 chunks per row and elements per chunk (multiple of 256)
    size_t off_part1, off_cnt1, off_desc, off_part2a, off_part2b, off_cnt2, total;
};

// Pass-1 chunking: aim for enough workgroups to fill the chip, never chunks shorter
// than kMinChunk1 elements.  The same function sizes the workspace and the launches.
constexpr int kTargetBlocks1 = 4096;
constexpr int kMinChunk1 = 4096;
constexpr int kTargetBlocks2 = 2048;
constexpr int kMinChunk2 = 2048;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline void chunking(int64_t rows, int64_t seqs, int V, int& nchunk1, int& ch1,
                     int& nchunk2, int& ch2) {
    int64_t want = rows > 0 ? ceil_div(kTargetBlocks1, rows) : 1;
    int64_t maxc = V / kMinChunk1;
    if (maxc < 1) maxc = 1;
    int64_t n = want < 1 ? 1 : (want > maxc ? maxc : want);
    int64_t ch = ceil_div(ceil_div(V, n), 64) * 64;
    nchunk1 = (int)ceil_div(V, ch);
    ch1 = (int)ch;

    want = seqs > 0 ? ceil_div(kTargetBlocks2, seqs) : 1;
    maxc = V / kMinChunk2;
    if (maxc < 1) maxc = 1;
    n = want < 1 ? 1 : (want > maxc ? maxc : want);
    ch = ceil_div(ceil_div(V, n), 256) * 256;
    nchunk2 = (int)ceil_div(V, ch);
    ch2 = (int)ch;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// rows_per_seq = 2K+1 for spec_verify, K+1 for spec_verify_greedy.
inline Layout make_layout(int B, int K, int V, int rows_per_seq) {
    Layout L;
    chunking((int64_t)B * rows_per_seq, B, V, L.nchunk1, L.ch1, L.nchunk2, L.ch2);
    // completion counters first; every call zeroes them before its first kernel
    size_t off = 0;
    L.off_cnt1 = off;
    off = align256(off + sizeof(uint32_t) * (size_t)B);
    L.off_cnt2 = off;
    off = align256(off + sizeof(uint32_t) * (size_t)B);
    L.off_desc = off;
    off = align256(off + sizeof(SeqDesc) * (size_t)B);
    L.off_part1 = off;
    off = align256(off + sizeof(RowPartial) * (size_t)B * rows_per_seq * L.nchunk1);
    L.off_part2a = off;
    off = align256(off + sizeof(NormPartial) * (size_t)B * L.nchunk2);
    L.off_part2b = off;
    off = align256(off + sizeof(double) * kWaves * (size_t)B * L.nchunk2);
    L.total = off;
    return L;
}

struct VerifyArgs {
    const void* target;        // [B][K+1][V]
    const void* draft;         // [B][K][V] (may be null when greedy-only or K == 0)
    const int32_t* tokens;     // [B][K]
    const float* uniforms;     // [B][K+1] (null when greedy-only)
    const float* temperature;  // [B] (null when greedy-only)
    int B, K, V, R;            // R = rows per sequence handled by pass 1
    int nchunk1, ch1, nchunk2, ch2;
    RowPartial* part1;
    uint32_t* cnt1;
    SeqDesc* desc;
    NormPartial* part2a;
    double* part2b;
    uint32_t* cnt2;
    int32_t* out_tokens;
    int32_t* out_n;
    float* out_p;
    float* out_q;
    int32_t* out_status;
};

// Internal launchers (return hipError_t as int; 0 = success).
int launch_zero_counters(const VerifyArgs& a, void* stream);
int launch_pass1(const VerifyArgs& a, int bf16, void* stream);
int launch_pass2(const VerifyArgs& a, int bf16, void* stream);
int launch_uniforms(uint64_t seed, uint64_t domain, uint64_t step, int B, int K, float* u,
                    void* stream);

}  // namespace sv
