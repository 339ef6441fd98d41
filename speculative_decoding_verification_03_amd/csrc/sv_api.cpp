// C ABI of the verify library (include/spec_verify.h): argument validation on the host,
// workspace layout, kernel launches.  Validation runs before any HIP call, so every
// SV_ERR_ARG / SV_ERR_DTYPE / SV_ERR_WORKSPACE path works without a GPU.
#include "spec_verify.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <vector>

#include "sv_common.h"

namespace sv {

// B*(K+1)*V and the block counts must fit comfortably.
bool shape_ok(int B, int K, int V) {
    if (B < 0 || K < 0 || V < 1) return false;
    const __int128 cells = (__int128)B * (K + 1) * V;
    if (cells > (__int128)INT64_MAX / 8) return false;
    return true;
}

// Workspace for both entry points: the larger of the two layouts.
size_t workspace_need(int B, int K, int V) {
    size_t need = 0;
    for (int esize : {2, 4})
        for (int R : {2 * K + 1, K + 1}) {
            const size_t t = make_layout(B, K, V, esize, R).total;
            if (t > need) need = t;
        }
    return need;
}

}  // namespace sv

namespace {

using sv::shape_ok;
using sv::workspace_need;

// Benchmark timing: per recorded call three events (before pass 1, between the passes,
// after pass 2).  Events are created on demand and kept for reuse.
struct Profile {
    bool on = false;
    bool failed = false;
    std::vector<hipEvent_t> pool;
    size_t used = 0;
    int calls = 0;

    hipEvent_t next() {
        if (used == pool.size()) {
            hipEvent_t e = nullptr;
            if (hipEventCreate(&e) != hipSuccess) {
                failed = true;
                return nullptr;
            }
            pool.push_back(e);
        }
        return pool[used++];
    }
    void record(hipEvent_t e, void* stream) {
        if (!e || hipEventRecord(e, static_cast<hipStream_t>(stream)) != hipSuccess) failed = true;
    }
};
Profile g_prof;

using sv::Layout;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool grid_ok(int B, int R, const Layout& L) {
    const __int128 blocks1 = (__int128)B * R * L.nchunk1;
    const __int128 blocks2 = ((__int128)B + 7) * L.nseg;  // the sweep pads B to whole rounds of 8 XCDs
    return blocks1 <= 0x7fffffff && blocks2 <= 0x7fffffff;
}

sv::VerifyArgs make_args(const void* target, const void* draft, const int32_t* tokens,
                         const float* uniforms, const float* temperature, int B, int K, int V,
                         int R, const Layout& L, void* workspace, int32_t* out_tokens,
                         int32_t* out_n, float* out_p, float* out_q, int32_t* out_status) {
    sv::VerifyArgs a;
    memset(&a, 0, sizeof(a));
    char* ws = static_cast<char*>(workspace);
    a.target = target;
    a.draft = draft;
    a.tokens = tokens;
    a.uniforms = uniforms;
    a.temperature = temperature;
    a.cu = nullptr;
    a.total = 0;
    a.B = B;
    a.K = K;
    a.V = V;
    a.R = R;
    a.nchunk1 = L.nchunk1;
    a.ch1 = L.ch1;
    a.seg = L.seg;
    a.nseg = L.nseg;
    sv::chunking2(B, V, L.seg, a.nchunk2, a.spc);
    a.desc = ws + L.off_desc;
    a.part1 = reinterpret_cast<sv::RowPartial*>(ws + L.off_part1);
    a.part2 = reinterpret_cast<sv::DrawPartial*>(ws + L.off_part2);
    a.bkt = reinterpret_cast<sv::Bucket*>(ws + L.off_bkt);
    a.wtab = reinterpret_cast<double*>(ws + L.off_wtab);
    a.deal = temperature ? reinterpret_cast<int32_t*>(ws + L.off_deal) : nullptr;
    a.deal_desc = temperature ? ws + L.off_deal_desc : nullptr;
    a.out_tokens = out_tokens;
    a.out_n = out_n;
    a.out_p = out_p;
    a.out_q = out_q;
    a.out_status = out_status;
    a.u_gen = nullptr;
    a.seed = a.domain = a.step = 0;
    return a;
}

// pass 1, then `second` (the resolve and draws, or the tree resolve), with the
// benchmark events around each
template <class F>
sv_status launch_two(const sv::VerifyArgs& a, int bf16, void* stream, F&& second, bool profile = true) {
    hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
    const bool prof = profile && g_prof.on;
    if (prof) {
        for (auto& e : ev) e = g_prof.next();
        g_prof.calls++;
        g_prof.record(ev[0], stream);
    }
    if (sv::launch_pass1(a, bf16, 0, a.B, stream) != 0) return SV_ERR_HIP;
    if (prof) g_prof.record(ev[1], stream);
    if (second() != 0) return SV_ERR_HIP;
    if (prof) g_prof.record(ev[2], stream);
    return SV_OK;
}

sv_status launch(const sv::VerifyArgs& a, int bf16, void* stream, bool profile = true) {
    return launch_two(a, bf16, stream, [&] { return sv::launch_draw(a, bf16, 0, a.B, stream); },
                      profile);
}

// Packed-layout sizes: (total + B) target rows of V elements must fit comfortably.
bool packed_shape_ok(int B, int K, int total, int V) {
    if (B < 0 || K < 0 || total < 0 || V < 1) return false;
    const __int128 cells = ((__int128)total + B) * V;
    if (cells > (__int128)INT64_MAX / 8) return false;
    if ((__int128)total + B > 0x7fffffff) return false;
    return shape_ok(B, K, V);
}

}  // namespace

extern "C" {

int sv_abi_version(void) { return SV_ABI_VERSION; }

const char* sv_status_string(int status) {
    switch (status) {
        case SV_OK: return "ok";
        case SV_ERR_ARG: return "invalid argument";
        case SV_ERR_DTYPE: return "unsupported dtype";
        case SV_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case SV_ERR_HIP: return "HIP launch failed";
        case SV_ERR_SCRATCH: return "the call needs more than the static scratch buffer";
        default: return "unknown status";
    }
}

sv_status sv_workspace_bytes(int B, int K, int V, size_t* bytes) {
    if (!bytes) return SV_ERR_ARG;
    *bytes = 0;
    if (!shape_ok(B, K, V)) return SV_ERR_ARG;
    *bytes = workspace_need(B, K, V);
    return SV_OK;
}

sv_status spec_verify(const void* target_logits, const void* draft_logits, int dtype,
                      const int32_t* draft_tokens, const float* uniforms,
                      const float* temperature, int B, int K, int V,
                      int32_t* out_tokens, int32_t* out_accept_len,
                      float* out_p, float* out_q, int32_t* out_status,
                      void* workspace, size_t workspace_bytes, void* stream) {
    return (sv_status)sv::verify_dense_call(target_logits, draft_logits, dtype, draft_tokens,
                                            uniforms, temperature, B, K, V, out_tokens,
                                            out_accept_len, out_p, out_q, out_status, workspace,
                                            workspace_bytes, stream, true, true);
}

}  // extern "C"

namespace sv {

int verify_dense_call(const void* target_logits, const void* draft_logits, int dtype,
                      const int32_t* draft_tokens, const float* uniforms,
                      const float* temperature, int B, int K, int V,
                      int32_t* out_tokens, int32_t* out_accept_len,
                      float* out_p, float* out_q, int32_t* out_status,
                      void* workspace, size_t workspace_bytes, void* stream, bool profile,
                      bool launch_it) {
    if (dtype != SV_DTYPE_F32 && dtype != SV_DTYPE_BF16) return SV_ERR_DTYPE;
    if (!shape_ok(B, K, V)) return SV_ERR_ARG;
    if (B == 0) return SV_OK;
    const size_t esz = dtype == SV_DTYPE_BF16 ? 2 : 4;
    if (!target_logits || !uniforms || !temperature || !out_tokens || !out_accept_len ||
        !out_status)
        return SV_ERR_ARG;
    if (K > 0 && (!draft_logits || !draft_tokens)) return SV_ERR_ARG;
    if (!aligned(target_logits, esz) || (draft_logits && !aligned(draft_logits, esz)))
        return SV_ERR_ARG;
    if (!aligned(uniforms, 4) || !aligned(temperature, 4) || !aligned(out_tokens, 4) ||
        !aligned(out_accept_len, 4) || !aligned(out_status, 4) ||
        (draft_tokens && !aligned(draft_tokens, 4)) || (out_p && !aligned(out_p, 4)) ||
        (out_q && !aligned(out_q, 4)))
        return SV_ERR_ARG;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < workspace_need(B, K, V))
        return SV_ERR_WORKSPACE;
    const int R = 2 * K + 1;
    const Layout L = sv::make_layout(B, K, V, (int)esz, R);
    if (!grid_ok(B, R, L)) return SV_ERR_ARG;
    if (!launch_it) return SV_OK;

    const sv::VerifyArgs a = make_args(target_logits, draft_logits, draft_tokens, uniforms,
                                       temperature, B, K, V, R, L, workspace, out_tokens,
                                       out_accept_len, out_p, out_q, out_status);
    return launch(a, dtype == SV_DTYPE_BF16, stream, profile);
}

}  // namespace sv

extern "C" {

// Logit bytes of a full read above which early exit reads in three rounds, not two.
constexpr double kEarlyExitBytes = 4.0 * (1 << 30);

sv_status spec_verify_early_exit(const void* target_logits, const void* draft_logits, int dtype,
                                 const int32_t* draft_tokens, const float* uniforms,
                                 const float* temperature, int B, int K, int V,
                                 int32_t* out_tokens, int32_t* out_accept_len,
                                 float* out_p, float* out_q, int32_t* out_status,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    if (dtype != SV_DTYPE_F32 && dtype != SV_DTYPE_BF16) return SV_ERR_DTYPE;
    if (!shape_ok(B, K, V)) return SV_ERR_ARG;
    if (B == 0) return SV_OK;
    const size_t esz = dtype == SV_DTYPE_BF16 ? 2 : 4;
    if (!target_logits || !uniforms || !temperature || !out_tokens || !out_accept_len ||
        !out_status)
        return SV_ERR_ARG;
    if (K > 0 && (!draft_logits || !draft_tokens)) return SV_ERR_ARG;
    if (!aligned(target_logits, esz) || (draft_logits && !aligned(draft_logits, esz)))
        return SV_ERR_ARG;
    if (!aligned(uniforms, 4) || !aligned(temperature, 4) || !aligned(out_tokens, 4) ||
        !aligned(out_accept_len, 4) || !aligned(out_status, 4) ||
        (draft_tokens && !aligned(draft_tokens, 4)) || (out_p && !aligned(out_p, 4)) ||
        (out_q && !aligned(out_q, 4)))
        return SV_ERR_ARG;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < workspace_need(B, K, V))
        return SV_ERR_WORKSPACE;
    const int R = 2 * K + 1;
    const Layout L = sv::make_layout(B, K, V, (int)esz, R);
    if (!grid_ok(B, R, L)) return SV_ERR_ARG;
    sv::VerifyArgs a = make_args(target_logits, draft_logits, draft_tokens, uniforms,
                                 temperature, B, K, V, R, L, workspace, out_tokens,
                                 out_accept_len, out_p, out_q, out_status);
    a.limit = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + L.off_limit);
    const int bf16 = dtype == SV_DTYPE_BF16;
    // rounds of positions: [0, 2), then the rest for the sequences that accepted both; a
    // call over more than kEarlyExitBytes of logit rows (where a round's fixed cost is
    // small against the rows it can spare) also stops at position 5
    int bounds[4];
    int rounds = 0;
    bounds[rounds++] = 0;
    if (K + 1 > 2) bounds[rounds++] = 2;
    if (K + 1 > 5 && (double)B * R * V * esz > kEarlyExitBytes) bounds[rounds++] = 5;
    bounds[rounds] = K + 1;
    hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
    if (g_prof.on) {
        for (auto& e : ev) e = g_prof.next();
        g_prof.calls++;
        g_prof.record(ev[0], stream);
    }
    for (int r = 0; r < rounds; ++r) {
        a.t0 = bounds[r];
        a.t1 = r + 1 == rounds ? K + 1 : bounds[r + 1];
        if (sv::launch_pass1(a, bf16, 0, B, stream) != 0) return SV_ERR_HIP;
        if (sv::launch_prefix(a, bf16, stream) != 0) return SV_ERR_HIP;
    }
    if (g_prof.on) g_prof.record(ev[1], stream);
    if (sv::launch_draw(a, bf16, 0, B, stream) != 0) return SV_ERR_HIP;
    if (g_prof.on) g_prof.record(ev[2], stream);
    return SV_OK;
}

sv_status spec_verify_philox(const void* target_logits, const void* draft_logits, int dtype,
                             const int32_t* draft_tokens, const float* temperature,
                             int B, int K, int V, uint64_t seed, uint64_t domain, uint64_t step,
                             float* uniforms_out, int32_t* out_tokens, int32_t* out_accept_len,
                             float* out_p, float* out_q, int32_t* out_status,
                             void* workspace, size_t workspace_bytes, void* stream) {
    if (dtype != SV_DTYPE_F32 && dtype != SV_DTYPE_BF16) return SV_ERR_DTYPE;
    if (!shape_ok(B, K, V)) return SV_ERR_ARG;
    if (B == 0) return SV_OK;
    if (!uniforms_out || !aligned(uniforms_out, 4)) return SV_ERR_ARG;
    // the uniforms are written by the first workgroups of pass 1
    sv_status st = SV_OK;
    const size_t esz = dtype == SV_DTYPE_BF16 ? 2 : 4;
    if (!target_logits || !temperature || !out_tokens || !out_accept_len || !out_status)
        return SV_ERR_ARG;
    if (K > 0 && (!draft_logits || !draft_tokens)) return SV_ERR_ARG;
    if (!aligned(target_logits, esz) || (draft_logits && !aligned(draft_logits, esz)))
        return SV_ERR_ARG;
    if (!aligned(temperature, 4) || !aligned(out_tokens, 4) || !aligned(out_accept_len, 4) ||
        !aligned(out_status, 4) || (draft_tokens && !aligned(draft_tokens, 4)) ||
        (out_p && !aligned(out_p, 4)) || (out_q && !aligned(out_q, 4)))
        return SV_ERR_ARG;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < workspace_need(B, K, V))
        return SV_ERR_WORKSPACE;
    const int R = 2 * K + 1;
    const Layout L = sv::make_layout(B, K, V, (int)esz, R);
    if (!grid_ok(B, R, L)) return SV_ERR_ARG;
    sv::VerifyArgs a = make_args(target_logits, draft_logits, draft_tokens, uniforms_out,
                                 temperature, B, K, V, R, L, workspace, out_tokens,
                                 out_accept_len, out_p, out_q, out_status);
    a.u_gen = uniforms_out;
    a.seed = seed;
    a.domain = domain;
    a.step = step;
    st = launch(a, dtype == SV_DTYPE_BF16, stream);
    return st;
}

sv_status spec_verify_ragged(const void* target_logits, const void* draft_logits, int dtype,
                             const int32_t* cu_drafts, int total_drafts, int K_max,
                             const int32_t* draft_tokens, const float* uniforms,
                             const float* temperature, int B, int V,
                             int32_t* out_tokens, int32_t* out_accept_len,
                             float* out_p, float* out_q, int32_t* out_status,
                             void* workspace, size_t workspace_bytes, void* stream) {
    if (dtype != SV_DTYPE_F32 && dtype != SV_DTYPE_BF16) return SV_ERR_DTYPE;
    if (!packed_shape_ok(B, K_max, total_drafts, V)) return SV_ERR_ARG;
    if (B == 0) return SV_OK;
    const size_t esz = dtype == SV_DTYPE_BF16 ? 2 : 4;
    if (!target_logits || !cu_drafts || !uniforms || !temperature || !out_tokens ||
        !out_accept_len || !out_status)
        return SV_ERR_ARG;
    if (total_drafts > 0 && (!draft_logits || !draft_tokens)) return SV_ERR_ARG;
    if (!aligned(target_logits, esz) || (draft_logits && !aligned(draft_logits, esz)))
        return SV_ERR_ARG;
    if (!aligned(cu_drafts, 4) || !aligned(uniforms, 4) || !aligned(temperature, 4) ||
        !aligned(out_tokens, 4) || !aligned(out_accept_len, 4) || !aligned(out_status, 4) ||
        (draft_tokens && !aligned(draft_tokens, 4)) || (out_p && !aligned(out_p, 4)) ||
        (out_q && !aligned(out_q, 4)))
        return SV_ERR_ARG;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < workspace_need(B, K_max, V))
        return SV_ERR_WORKSPACE;
    const int R = 2 * K_max + 1;
    const Layout L = sv::make_layout(B, K_max, V, (int)esz, R);
    if (!grid_ok(B, R, L)) return SV_ERR_ARG;
    sv::VerifyArgs a = make_args(target_logits, draft_logits, draft_tokens, uniforms,
                                 temperature, B, K_max, V, R, L, workspace, out_tokens,
                                 out_accept_len, out_p, out_q, out_status);
    a.cu = cu_drafts;
    a.total = total_drafts;
    return launch(a, dtype == SV_DTYPE_BF16, stream);
}

sv_status sv_sample(const void* logits, int dtype, const float* uniforms,
                    const float* temperature, int B, int V, int32_t* out_tokens,
                    int32_t* out_status, void* workspace, size_t workspace_bytes, void* stream) {
    if (dtype != SV_DTYPE_F32 && dtype != SV_DTYPE_BF16) return SV_ERR_DTYPE;
    if (!shape_ok(B, 0, V)) return SV_ERR_ARG;
    if (B == 0) return SV_OK;
    const size_t esz = dtype == SV_DTYPE_BF16 ? 2 : 4;
    if (!logits || !uniforms || !temperature || !out_tokens || !out_status) return SV_ERR_ARG;
    if (!aligned(logits, esz) || !aligned(uniforms, 4) || !aligned(temperature, 4) ||
        !aligned(out_tokens, 4) || !aligned(out_status, 4))
        return SV_ERR_ARG;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < workspace_need(B, 0, V))
        return SV_ERR_WORKSPACE;
    const Layout L = sv::make_layout(B, 0, V, (int)esz, 1);
    if (!grid_ok(B, 1, L)) return SV_ERR_ARG;
    // the verify step with no drafts: the bonus draw from p_0, or its argmax at T = 0
    const sv::VerifyArgs a = make_args(logits, nullptr, nullptr, uniforms, temperature, B, 0, V,
                                       1, L, workspace, out_tokens, nullptr, nullptr, nullptr,
                                       out_status);
    const int bf16 = dtype == SV_DTYPE_BF16;
    if ((int64_t)V > (int64_t)sv::kSampleMaxSeg * sv::kSampleSeg) return launch(a, bf16, stream);
    // rows of at most kSampleMaxSeg segments: one workgroup per row does everything
    // (timed as the first phase)
    hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
    if (g_prof.on) {
        for (auto& e : ev) e = g_prof.next();
        g_prof.calls++;
        g_prof.record(ev[0], stream);
    }
    if (sv::launch_sample(a, bf16, stream) != 0) return SV_ERR_HIP;
    if (g_prof.on) {
        g_prof.record(ev[1], stream);
        g_prof.record(ev[2], stream);
    }
    return SV_OK;
}

sv_status spec_verify_greedy(const void* target_logits, int dtype,
                             const int32_t* draft_tokens, int B, int K, int V,
                             int32_t* out_tokens, int32_t* out_accept_len,
                             int32_t* out_status,
                             void* workspace, size_t workspace_bytes, void* stream) {
    if (dtype != SV_DTYPE_F32 && dtype != SV_DTYPE_BF16) return SV_ERR_DTYPE;
    if (!shape_ok(B, K, V)) return SV_ERR_ARG;
    if (B == 0) return SV_OK;
    const size_t esz = dtype == SV_DTYPE_BF16 ? 2 : 4;
    if (!target_logits || !out_tokens || !out_accept_len || !out_status) return SV_ERR_ARG;
    if (K > 0 && !draft_tokens) return SV_ERR_ARG;
    if (!aligned(target_logits, esz) || !aligned(out_tokens, 4) ||
        !aligned(out_accept_len, 4) || !aligned(out_status, 4) ||
        (draft_tokens && !aligned(draft_tokens, 4)))
        return SV_ERR_ARG;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < workspace_need(B, K, V))
        return SV_ERR_WORKSPACE;
    const int R = K + 1;
    const Layout L = sv::make_layout(B, K, V, (int)esz, R);
    if (!grid_ok(B, R, L)) return SV_ERR_ARG;

    const sv::VerifyArgs a = make_args(target_logits, nullptr, draft_tokens, nullptr, nullptr, B,
                                       K, V, R, L, workspace, out_tokens, out_accept_len, nullptr,
                                       nullptr, out_status);
    return launch(a, dtype == SV_DTYPE_BF16, stream);
}

sv_status spec_verify_greedy_ragged(const void* target_logits, int dtype,
                                    const int32_t* cu_drafts, int total_drafts, int K_max,
                                    const int32_t* draft_tokens, int B, int V,
                                    int32_t* out_tokens, int32_t* out_accept_len,
                                    int32_t* out_status,
                                    void* workspace, size_t workspace_bytes, void* stream) {
    if (dtype != SV_DTYPE_F32 && dtype != SV_DTYPE_BF16) return SV_ERR_DTYPE;
    if (!packed_shape_ok(B, K_max, total_drafts, V)) return SV_ERR_ARG;
    if (B == 0) return SV_OK;
    const size_t esz = dtype == SV_DTYPE_BF16 ? 2 : 4;
    if (!target_logits || !cu_drafts || !out_tokens || !out_accept_len || !out_status)
        return SV_ERR_ARG;
    if (total_drafts > 0 && !draft_tokens) return SV_ERR_ARG;
    if (!aligned(target_logits, esz) || !aligned(cu_drafts, 4) || !aligned(out_tokens, 4) ||
        !aligned(out_accept_len, 4) || !aligned(out_status, 4) ||
        (draft_tokens && !aligned(draft_tokens, 4)))
        return SV_ERR_ARG;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < workspace_need(B, K_max, V))
        return SV_ERR_WORKSPACE;
    const int R = K_max + 1;
    const Layout L = sv::make_layout(B, K_max, V, (int)esz, R);
    if (!grid_ok(B, R, L)) return SV_ERR_ARG;
    sv::VerifyArgs a = make_args(target_logits, nullptr, draft_tokens, nullptr, nullptr, B, K_max,
                                 V, R, L, workspace, out_tokens, out_accept_len, nullptr, nullptr,
                                 out_status);
    a.cu = cu_drafts;
    a.total = total_drafts;
    return launch(a, dtype == SV_DTYPE_BF16, stream);
}

sv_status sv_fill_uniforms(uint64_t seed, uint64_t domain, uint64_t step, int B, int K,
                           float* uniforms, void* stream) {
    if (B < 0 || K < 0) return SV_ERR_ARG;
    if ((__int128)B * (K + 1) > (__int128)0x7fffffff * sv::kThreads) return SV_ERR_ARG;
    if (B == 0) return SV_OK;
    if (!uniforms || !aligned(uniforms, 4)) return SV_ERR_ARG;
    if (sv::launch_uniforms(seed, domain, step, B, K, uniforms, stream) != 0) return SV_ERR_HIP;
    return SV_OK;
}

sv_status spec_verify_tree_greedy(const void* target_logits, int dtype, const int32_t* parents,
                                  const int32_t* node_tokens, int B, int N, int V,
                                  int32_t* out_tokens, int32_t* out_nodes,
                                  int32_t* out_accept_len, int32_t* out_status,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    if (dtype != SV_DTYPE_F32 && dtype != SV_DTYPE_BF16) return SV_ERR_DTYPE;
    if (B < 0 || N < 1 || N > sv::kTreeMaxNodes || !shape_ok(B, N - 1, V)) return SV_ERR_ARG;
    if (B == 0) return SV_OK;
    const size_t esz = dtype == SV_DTYPE_BF16 ? 2 : 4;
    if (!target_logits || !parents || !node_tokens || !out_tokens || !out_accept_len ||
        !out_status)
        return SV_ERR_ARG;
    if (!aligned(target_logits, esz) || !aligned(parents, 4) || !aligned(node_tokens, 4) ||
        !aligned(out_tokens, 4) || !aligned(out_accept_len, 4) || !aligned(out_status, 4) ||
        (out_nodes && !aligned(out_nodes, 4)))
        return SV_ERR_ARG;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < workspace_need(B, N - 1, V))
        return SV_ERR_WORKSPACE;
    const int R = N;
    const Layout L = sv::make_layout(B, N - 1, V, (int)esz, R);
    if (!grid_ok(B, R, L)) return SV_ERR_ARG;
    // pass 1 over the N target rows of every sequence as greedy rows (no temperature)
    const sv::VerifyArgs a = make_args(target_logits, nullptr, nullptr, nullptr, nullptr, B, N - 1,
                                       V, R, L, workspace, nullptr, nullptr, nullptr, nullptr,
                                       nullptr);
    sv::TreeArgs t;
    memset(&t, 0, sizeof(t));
    t.parents = parents;
    t.tokens = node_tokens;
    t.part1 = a.part1;
    t.B = B;
    t.N = N;
    t.V = V;
    t.nchunk1 = L.nchunk1;
    t.out_tokens = out_tokens;
    t.out_nodes = out_nodes;
    t.out_n = out_accept_len;
    t.out_status = out_status;
    return launch_two(a, dtype == SV_DTYPE_BF16, stream, [&] { return sv::launch_tree(t, stream); });
}

sv_status sv_tree_attention_mask(const int32_t* parents, int B, int N, uint8_t* out_mask,
                                 int32_t* out_depth, int32_t* out_status, void* stream) {
    if (B < 0 || N < 1 || N > sv::kTreeMaxNodes) return SV_ERR_ARG;
    if (B == 0) return SV_OK;
    if (!parents || !out_mask || !out_status || !aligned(parents, 4) || !aligned(out_status, 4) ||
        (out_depth && !aligned(out_depth, 4)))
        return SV_ERR_ARG;
    sv::TreeArgs t;
    memset(&t, 0, sizeof(t));
    t.parents = parents;
    t.B = B;
    t.N = N;
    t.out_mask = out_mask;
    t.out_depth = out_depth;
    t.out_status = out_status;
    if (sv::launch_tree_mask(t, stream) != 0) return SV_ERR_HIP;
    return SV_OK;
}

sv_status sv_fill_uniforms_ragged(uint64_t seed, uint64_t domain, uint64_t step, int B,
                                  const int32_t* cu_drafts, int total_drafts, int K_max,
                                  float* uniforms, void* stream) {
    if (B < 0 || K_max < 0 || total_drafts < 0) return SV_ERR_ARG;
    if ((__int128)B * (K_max + 1) > (__int128)0x7fffffff * sv::kThreads) return SV_ERR_ARG;
    if ((__int128)total_drafts + B > 0x7fffffff) return SV_ERR_ARG;
    if (B == 0) return SV_OK;
    if (!cu_drafts || !uniforms || !aligned(cu_drafts, 4) || !aligned(uniforms, 4))
        return SV_ERR_ARG;
    if (sv::launch_uniforms_packed(seed, domain, step, B, K_max, cu_drafts, total_drafts,
                                   uniforms, stream) != 0)
        return SV_ERR_HIP;
    return SV_OK;
}

sv_status sv_profile_begin(void) {
    g_prof.on = true;
    g_prof.failed = false;
    g_prof.used = 0;
    g_prof.calls = 0;
    return SV_OK;
}

sv_status sv_profile_end(int* calls, double* ms_pass1, double* ms_pass2) {
    double t1 = 0.0, t2 = 0.0;
    bool ok = !g_prof.failed;
    for (size_t i = 0; ok && i + 3 <= g_prof.used; i += 3) {
        float a = 0.f, b = 0.f;
        if (hipEventSynchronize(g_prof.pool[i + 2]) != hipSuccess ||
            hipEventElapsedTime(&a, g_prof.pool[i], g_prof.pool[i + 1]) != hipSuccess ||
            hipEventElapsedTime(&b, g_prof.pool[i + 1], g_prof.pool[i + 2]) != hipSuccess) {
            ok = false;
            break;
        }
        t1 += a;
        t2 += b;
    }
    if (calls) *calls = g_prof.calls;
    if (ms_pass1) *ms_pass1 = t1;
    if (ms_pass2) *ms_pass2 = t2;
    g_prof.on = false;
    g_prof.used = 0;
    return ok ? SV_OK : SV_ERR_HIP;
}

}  // extern "C"
