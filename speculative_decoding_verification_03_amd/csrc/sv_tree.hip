// Greedy verification of a draft token TREE, and the tree attention mask the target's
// forward pass over the tree uses.
//
// The draft proposes a tree instead of one chain: node 0 is the root (the last token
// already emitted), every other node j carries a drafted token and has a parent
// p(j) < j.  The target verifies all nodes in one forward pass under a tree attention
// mask in which each node sees only its ancestors and itself; the result is the longest
// prefix along any accepted root path ("Verificação de Atenção em Árvore" on the lesson
// page "Decodificação Especulativa e EAGLE"; "Kiểm tra sự chú ý của cây" on the Vietnamese
// page; the EAGLE section of "Accelerating Sonar through speculation" describes keeping
// the longest accepted candidate plus one extra token from the target).
//
// Greedy rule on a tree (the chain rule of "Caso ganancioso" applied along every root
// path): node j is accepted when its parent is accepted and its token equals the
// lowest-index argmax of the target row of its parent; the root is accepted.  The
// result is the deepest accepted node a (lowest index among equally deep ones); the
// emitted tokens are those along the path root -> a, then the argmax of a's row.
//
// Row j of the target logits is the target's next-token distribution after node j's
// path.  Pass 1 (sv_pass1.hip, greedy rows) gives each row's argmax; tree_kernel (one
// workgroup per sequence) merges them, marks accepted nodes by pointer jumping over the
// parent links (log2 N rounds) and walks the winning path.
#include <hip/hip_runtime.h>
#include <math.h>

#include "sv_common.h"
#include "sv_device.h"

namespace sv {

namespace {

constexpr int kPer = kTreeMaxNodes / kThreads;  // nodes per thread
static_assert(kTreeMaxNodes % kThreads == 0, "tree nodes spread evenly over the threads");

// parent of node j as read, and whether the link is legal (root: -1; else in [0, j))
__device__ __forceinline__ bool parent_ok(int j, int p) { return j == 0 ? p == -1 : (p >= 0 && p < j); }

__global__ __launch_bounds__(kThreads) void tree_kernel(TreeArgs a) {
    __shared__ int am[kTreeMaxNodes];   // argmax of row j
    __shared__ int par[kTreeMaxNodes];  // parent (root: itself)
    __shared__ int tk[kTreeMaxNodes];   // token of node j
    __shared__ int anc[kTreeMaxNodes];  // pointer-jumping ancestor
    __shared__ int ok[kTreeMaxNodes];   // path j .. anc[j] (exclusive) all matches
    __shared__ int dep[kTreeMaxNodes];  // edges j .. anc[j]
    __shared__ int shi[kWaves];
    const int b = blockIdx.x, tid = threadIdx.x, N = a.N, V = a.V;
    const int32_t* parent = a.parents + (int64_t)b * N;
    const int32_t* token = a.tokens + (int64_t)b * N;
    int err = 0;
    for (int j = tid; j < N; j += kThreads) {
        // row j: maximum and lowest index over the chunks in order (strict comparison
        // keeps the earlier chunk on ties)
        const RowPartial* p = a.part1 + ((int64_t)b * N + j) * a.nchunk1;
        float m = -INFINITY;
        int idx = 0;
        bool nan = false;
        for (int c = 0; c < a.nchunk1; ++c) {
            const RowPartial q = p[c];
            if (q.m != q.m) nan = true;
            else if (q.m > m) {
                m = q.m;
                idx = q.idx;
            }
        }
        if (nan || m == -INFINITY) err |= kSeqErrLogit;
        const int pj = parent[j];
        if (!parent_ok(j, pj)) err |= kSeqErrTree;
        const int x = j == 0 ? 0 : token[j];
        if (x < 0 || x >= V) err |= kSeqErrToken;
        am[j] = idx;
        par[j] = parent_ok(j, pj) ? (j == 0 ? 0 : pj) : 0;
        tk[j] = x;
    }
    err = block_or(err, shi);  // also publishes am, par, tk
    int32_t* out_tok = a.out_tokens + (int64_t)b * N;
    int32_t* out_nodes = a.out_nodes ? a.out_nodes + (int64_t)b * N : nullptr;
    if (err) {
        for (int t = tid; t < N; t += kThreads) {
            out_tok[t] = -1;
            if (out_nodes) out_nodes[t] = -1;
        }
        if (tid == 0) {
            a.out_n[b] = -1;
            a.out_status[b] = err;
        }
        return;
    }
    // pointer jumping: after round r, anc[j] is the 2^r-th ancestor of j (or the root),
    // ok[j] the AND of the matches of the nodes from j up to anc[j] (exclusive), dep[j]
    // the number of edges in between.  The root is a fixed point with an empty path.
    for (int j = tid; j < N; j += kThreads) {
        anc[j] = par[j];
        ok[j] = j == 0 ? 1 : (tk[j] == am[par[j]]);
        dep[j] = j == 0 ? 0 : 1;
    }
    __syncthreads();
    for (int span = 1; span < N; span <<= 1) {
        int na[kPer], nok[kPer], nd[kPer];
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int j = tid + k * kThreads;
            if (j < N) {
                const int q = anc[j];
                na[k] = anc[q];
                nok[k] = ok[j] & ok[q];
                nd[k] = dep[j] + dep[q];
            }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int j = tid + k * kThreads;
            if (j < N) {
                anc[j] = na[k];
                ok[j] = nok[k];
                dep[j] = nd[k];
            }
        }
        __syncthreads();
    }
    // deepest accepted node, lowest index among equals: the largest key depth * 2^11 +
    // (2^11 - 1 - j) over accepted nodes (the root, depth 0, is always accepted)
    int best = -1;
    for (int j = tid; j < N; j += kThreads)
        if (ok[j]) best = max(best, dep[j] * 2048 + (2047 - j));
    best = block_max(best, shi);
    const int win = 2047 - (best & 2047), d = best >> 11;
    // outputs: tokens along root -> win, then the argmax of win's row; -1 after
    for (int t = d + 1 + tid; t < N; t += kThreads) out_tok[t] = -1;
    if (out_nodes)
        for (int t = d + tid; t < N; t += kThreads) out_nodes[t] = -1;
    if (tid == 0) {
        out_tok[d] = am[win];
        int cur = win;
        for (int k = d - 1; k >= 0; --k) {
            out_tok[k] = tk[cur];
            if (out_nodes) out_nodes[k] = cur;
            cur = par[cur];
        }
        a.out_n[b] = d;
        a.out_status[b] = 0;
    }
}

// One workgroup per sequence; each wave builds whole mask rows.  Row i of the mask marks
// the ancestors of node i and i itself: the nodes its token may attend to.
__global__ __launch_bounds__(kThreads) void tree_mask_kernel(TreeArgs a) {
    __shared__ int par[kTreeMaxNodes];
    __shared__ int shi[kWaves];
    const int b = blockIdx.x, tid = threadIdx.x, N = a.N;
    const int lane = tid & 63, w = tid >> 6;
    const int32_t* parent = a.parents + (int64_t)b * N;
    int err = 0;
    for (int j = tid; j < N; j += kThreads) {
        const int pj = parent[j];
        if (!parent_ok(j, pj)) err |= kSeqErrTree;
        par[j] = j == 0 ? 0 : pj;
    }
    err = block_or(err, shi);
    uint8_t* mask = a.out_mask + (int64_t)b * N * N;
    int32_t* depth = a.out_depth ? a.out_depth + (int64_t)b * N : nullptr;
    if (tid == 0) a.out_status[b] = err;
    if (err) {
        // nothing is attendable in a malformed tree
        for (int64_t e = tid; e < (int64_t)N * N; e += kThreads) mask[e] = 0;
        if (depth)
            for (int j = tid; j < N; j += kThreads) depth[j] = -1;
        return;
    }
    for (int i = w; i < N; i += kWaves) {
        uint8_t* row = mask + (int64_t)i * N;
        // ancestors of i have smaller indices: walk up once per wave, marking as the
        // walk passes each 64-column block from the right
        int cur = i, steps = 0;
        for (int j0 = ((i >> 6) << 6); j0 >= 0; j0 -= 64) {
            bool mine = false;
            // the walk visits indices in decreasing order; consume those in [j0, j0 + 64)
            while (cur >= j0) {
                if (cur == j0 + lane) mine = true;
                if (cur == 0) {
                    cur = -1;
                    break;
                }
                cur = par[cur];
                ++steps;
            }
            const int j = j0 + lane;
            if (j < N) row[j] = mine ? 1 : 0;
        }
        for (int j = (((i >> 6) + 1) << 6) + lane; j < N; j += 64) row[j] = 0;
        if (depth && lane == 0) depth[i] = steps;
    }
}

}  // namespace

int launch_tree(const TreeArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(tree_kernel, dim3((unsigned)a.B), dim3(kThreads), 0, s, a);
    return (int)hipGetLastError();
}

int launch_tree_mask(const TreeArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(tree_mask_kernel, dim3((unsigned)a.B), dim3(kThreads), 0, s, a);
    return (int)hipGetLastError();
}

}  // namespace sv
