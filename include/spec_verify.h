/*
 * spec_verify.h -- C ABI of the batched speculative-sampling verify step (MI355X / gfx950).
 *
 * The operation.  For each of B sequences a draft model has proposed K tokens
 * x_0..x_{K-1}; the target model has produced logits at K+1 positions and the draft
 * at K positions.  With p_t = softmax(zt_t / T) and q_t = softmax(zd_t / T):
 *   - left to right, draft token x_t is accepted while r_t < p_t(x_t) / q_t(x_t);
 *   - at the first rejection one token is drawn from (p_t - q_t)+ / ||(p_t - q_t)+||_1,
 *     the positive part of the pointwise difference over the vocabulary, and the
 *     step stops;
 *   - if all K are accepted, a bonus token is drawn from p_K;
 *   - at temperature 0 the rule is argmax(p_t) == x_t, emitting argmax(p_t) on the
 *     first mismatch (argmax(p_K) after K matches).
 * Source: the lesson "Decodificação Especulativa e EAGLE" (ai-engineering.academy,
 * Phase 10 Lesson 25), sections "O Conceito" (steps 1-4), "A Regra de Exatidão"
 * and its "Caso ganancioso" paragraph; the same text as "Quy tắc chính xác" in
 * "Việc giải mã giả định và Eagle" (aiengineeringfromscratch.com).  The temperature
 * softmax on both sides follows those pages' "Desenvolva" / "Hãy xây dựng nó" listing.
 *
 * Readings fixed by this contract where the pages are silent:
 *   - argmax ties go to the LOWEST index;
 *   - a categorical draw with weights w and uniform u returns the smallest i with
 *     w_0 + ... + w_i > u * sum(w); if rounding leaves no such i, the last index
 *     with w_i > 0.  The draw that follows a rejection or the bonus uses u[b][K];
 *     test t uses u[b][t];
 *   - the draw after a rejection uses fp64 weights; should they sum to zero in fp64
 *     (impossible in exact arithmetic) it draws from p_t and flags NOTE_FALLBACK.
 *
 * Memory.  Every pointer named "device" is device memory owned by the caller.  The
 * library never allocates, frees or retains memory (spec_verify_noalloc uses a static
 * scratch array of the library instead of a caller workspace).  All calls are asynchronous on
 * `stream` (a hipStream_t passed as void*; NULL = the null stream) and never
 * synchronise the host.  Outputs stay on the device.  No call records a memset or any
 * operation other than kernel launches on `stream`, so calls can be captured in a HIP
 * graph (the profiling pair sv_profile_begin/end excepted: it records events).
 *
 * Errors.  Argument errors are detected on the host BEFORE any HIP call and
 * returned synchronously (SV_ERR_ARG, SV_ERR_DTYPE, SV_ERR_WORKSPACE); a failed
 * launch returns SV_ERR_HIP.  Data errors are detected on the device and reported
 * per sequence in out_status[b] (flags below); such a sequence emits tokens -1,
 * accept length -1 and p = q = NaN.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_ABI_VERSION 5

/* Host-side return codes. */
typedef enum sv_status {
    SV_OK = 0,
    SV_ERR_ARG = 1,        /* bad size, NULL required pointer, misaligned pointer        */
    SV_ERR_DTYPE = 2,      /* dtype is not one of sv_dtype                                */
    SV_ERR_WORKSPACE = 3,  /* workspace NULL, misaligned or smaller than required        */
    SV_ERR_HIP = 4,        /* a kernel launch failed                                      */
    SV_ERR_SCRATCH = 5     /* spec_verify_noalloc: the call needs more workspace than its
                              static scratch buffer holds (SV_NOALLOC_SCRATCH_BYTES)        */
} sv_status;

/* Logit storage.  bf16 = the upper 16 bits of an IEEE fp32 (round-trip exact widening). */
typedef enum sv_dtype {
    SV_DTYPE_F32 = 0,
    SV_DTYPE_BF16 = 1
} sv_dtype;

/* Per-sequence device status flags (out_status[b], OR-ed). */
#define SV_SEQ_OK               0
#define SV_SEQ_ERR_TOKEN        1   /* a draft token outside [0, V)                                 */
#define SV_SEQ_ERR_LOGIT        2   /* NaN in a row the sequence reads, a row whose max is -inf, or
                                       (sampled sequences) a +inf logit or a row whose maximum m
                                       has |m| * fp32(log2(e) / T) >= 2^30 (outside the supported
                                       range of scaled logits)                                      */
#define SV_SEQ_ERR_TEMPERATURE  4   /* T NaN, negative, infinite, or in (0, FLT_MIN)                */
#define SV_SEQ_ERR_UNIFORM      8   /* (sampled sequences) u NaN or outside [0, 1)                  */
#define SV_SEQ_NOTE_FALLBACK   16   /* not an error: a categorical draw fell back (see above)       */
#define SV_SEQ_ERR_TREE        64   /* (tree calls) parents[b][0] != -1, or a parents[b][j] outside
                                       [0, j) for j >= 1                                             */
#define SV_SEQ_ERR_OFFSETS     32   /* (ragged calls) cu[b], cu[b+1] not 0 <= cu[b] <= cu[b+1] <=
                                       total_drafts with cu[b+1] - cu[b] <= K_max                   */

/* Returns SV_ABI_VERSION of the loaded library. */
int sv_abi_version(void);

/* Static text for an sv_status value; "unknown status" otherwise.  Never NULL. */
const char* sv_status_string(int status);

/*
 * Bytes of device workspace spec_verify / spec_verify_greedy need for (B, K, V).
 * Pure host function.  Returns SV_ERR_ARG (and *bytes = 0) when B < 0, K < 0, V < 1,
 * or the sizes overflow; SV_OK otherwise.  The same size serves both entry points.
 *
 * Workspace contract: 256-byte aligned device memory of at least *bytes.  Its content
 * on entry does not matter (each call initialises what it uses); it can be reused for
 * any later (B, K, V) that fits.  Calls that share one workspace must be ordered (same
 * stream, or synchronised): overlapping calls on one workspace race.
 */
sv_status sv_workspace_bytes(int B, int K, int V, size_t* bytes);

/*
 * Sampled verify (temperature > 0), with the greedy rule for sequences whose T == 0.
 *
 *   target_logits  device, [B][K+1][V] of `dtype`, row-major and contiguous.
 *   draft_logits   device, [B][K][V]   of `dtype`; rows of T == 0 sequences are not
 *                  read.  May be NULL only when K == 0.
 *   dtype          sv_dtype.  Pointers must be aligned to the element size.
 *   draft_tokens   device, [B][K] int32.  May be NULL only when K == 0.
 *   uniforms       device, [B][K+1] fp32, each in [0, 1): slot t < K drives the ratio
 *                  test of x_t, slot K the final categorical draw.  Not read for T == 0.
 *   temperature    device, [B] fp32.  T > 0: sampled; T == 0: greedy rule.
 *   B, K, V        B >= 0 (B == 0 is a no-op), K >= 0 (K == 0 = plain sampling from
 *                  p_0), V >= 1; B*(K+1)*V must fit in int64.
 *   out_tokens     device, [B][K+1] int32: x_0..x_{n-1}, the drawn token, then -1.
 *   out_accept_len device, [B] int32: n in [0, K], the number of accepted drafts.
 *   out_p, out_q   device, [B][K] fp32, or NULL: p_t(x_t) and q_t(x_t) for every t < K
 *                  (also past the rejection); NaN for T == 0 sequences.
 *   out_status     device, [B] int32: SV_SEQ_* flags.
 *   workspace      device, see sv_workspace_bytes.
 *   stream         hipStream_t as void*.
 * Outputs are complete when the stream reaches the end of the call.  Bit-reproducible:
 * the same inputs give the same outputs on every call.
 */
sv_status spec_verify(const void* target_logits, const void* draft_logits, int dtype,
                      const int32_t* draft_tokens, const float* uniforms,
                      const float* temperature, int B, int K, int V,
                      int32_t* out_tokens, int32_t* out_accept_len,
                      float* out_p, float* out_q, int32_t* out_status,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_verify for callers that cannot allocate device memory, not even a workspace:
 * code being captured into a HIP graph, serving loops and harnesses that forbid
 * allocation.  The same computation, kernels and outputs as spec_verify (bit for bit);
 * the workspace is a static device array of the library, SV_NOALLOC_SCRATCH_BYTES
 * (64 MiB) per GPU, which each GPU the library runs on holds until the process ends.
 * The call itself allocates nothing (no hipMalloc, no events).
 *
 * Arguments as for spec_verify, without workspace and workspace_bytes.  The stream
 * must belong to the current device (whose copy of the array is used).  Returns
 * SV_ERR_SCRATCH, before any HIP call, when sv_workspace_bytes(B, K, V) exceeds
 * SV_NOALLOC_SCRATCH_BYTES (B=1024, K=10, V=262144 needs 55.5 MiB and fits), and
 * SV_ERR_ARG when the stream belongs to another device.  Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (different streams, or host threads
 * without ordering) race.  Nothing in the array needs to start at zero: each call
 * initialises what it reads.
 */
#define SV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
sv_status spec_verify_noalloc(const void* target_logits, const void* draft_logits, int dtype,
                              const int32_t* draft_tokens, const float* uniforms,
                              const float* temperature, int B, int K, int V,
                              int32_t* out_tokens, int32_t* out_accept_len,
                              float* out_p, float* out_q, int32_t* out_status, void* stream);

/*
 * spec_verify reading each sequence's rows only up to its first rejection: the tests run
 * left to right and stop there ("A Regra de Exatidão": the first rejection ends the step),
 * so the rows of later positions are never needed for the emitted tokens.  Positions are
 * read in rounds: [0, 2), then the rest for the sequences that accepted both (a call over
 * more than 4 GiB of logit rows also stops at position 5); a sequence whose test fails in
 * a round reads nothing more.  The
 * emitted tokens, accept lengths and draws are bit-identical to spec_verify's.
 * Differences: out_p / out_q hold p_t(x_t), q_t(x_t) only for the positions up to and
 * including the first rejection n (all K when every draft is accepted) and are NaN after
 * it, and a NaN or +inf logit in a row of a position after n is not reported (whether or
 * not its round read it).  Arguments as for spec_verify.
 */
sv_status spec_verify_early_exit(const void* target_logits, const void* draft_logits, int dtype,
                                 const int32_t* draft_tokens, const float* uniforms,
                                 const float* temperature, int B, int K, int V,
                                 int32_t* out_tokens, int32_t* out_accept_len,
                                 float* out_p, float* out_q, int32_t* out_status,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_verify with uniforms from the counter generator: the same as
 *   sv_fill_uniforms(seed, domain, step, B, K, uniforms_out, stream);
 *   spec_verify(..., uniforms_out, ...);
 * with one launch fewer (the first workgroups of the logit-streaming kernel write the
 * uniforms).  uniforms_out: device, [B][K+1] fp32, written by the call, owned by the
 * caller.  Every other argument as for spec_verify.  Outputs are bit-identical to the
 * two calls above.
 */
sv_status spec_verify_philox(const void* target_logits, const void* draft_logits, int dtype,
                             const int32_t* draft_tokens, const float* temperature,
                             int B, int K, int V, uint64_t seed, uint64_t domain, uint64_t step,
                             float* uniforms_out, int32_t* out_tokens, int32_t* out_accept_len,
                             float* out_p, float* out_q, int32_t* out_status,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Greedy verify (temperature 0 for every sequence): accept x_t while the lowest-index
 * argmax of target row t equals x_t; emit that argmax at the first mismatch, or the
 * argmax of row K after K matches.  Reads target logits only.  Arguments as for
 * spec_verify.  Bit-exact by construction (comparisons only).
 */
sv_status spec_verify_greedy(const void* target_logits, int dtype,
                             const int32_t* draft_tokens, int B, int K, int V,
                             int32_t* out_tokens, int32_t* out_accept_len,
                             int32_t* out_status,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Ragged verify: a different number of drafts K_b per sequence, in the packed layout an
 * engine's flattened verify batch has.  This serves adaptive verification, where each
 * request is verified on as many drafted tokens as is worth it (the Speculators talk in
 * the livestream "IA local 202", [44:15]-[45:16]); the rule applied to each sequence is
 * the one of spec_verify with K = K_b.  Rows past a sequence's K_b are never read.
 *
 *   cu_drafts      device, [B+1] int32 offsets: sequence b has K_b = cu[b+1] - cu[b]
 *                  drafts; its draft rows, draft tokens, out_p and out_q entries start at
 *                  index cu[b], its K_b + 1 target rows, uniforms and out_tokens entries at
 *                  index cu[b] + b.  Expected: cu[0] = 0, non-decreasing, cu[B] = total.
 *   total_drafts   host int, the number of packed draft rows (sum of K_b).
 *   K_max          host int, a bound on every K_b (sizes the launch and the workspace).
 *   target_logits  device, [total_drafts + B][V]; draft_logits device, [total_drafts][V]
 *                  (rows of T == 0 sequences are not read; NULL allowed iff total == 0).
 *   draft_tokens   device, [total_drafts] int32 (NULL allowed iff total == 0).
 *   uniforms       device, [total_drafts + B] fp32: u of test t of sequence b at
 *                  cu[b] + b + t, the final draw's at cu[b] + b + K_b.
 *   out_tokens     device, [total_drafts + B] int32: per sequence x_0..x_{n-1}, the
 *                  drawn token, then -1, over its K_b + 1 slots.
 *   out_p, out_q   device, [total_drafts] fp32, or NULL.
 *   temperature, out_accept_len, out_status: [B], as for spec_verify.
 *   workspace      at least sv_workspace_bytes(B, K_max, V).
 * A sequence whose offsets break the rule above is flagged SV_SEQ_ERR_OFFSETS, reads
 * nothing and writes only out_accept_len[b] = -1 and out_status[b]; every other sequence
 * reads and writes only inside the packed arrays (if cu decreases somewhere, sequences
 * may overlap and their outputs are unspecified).  Host errors: as spec_verify, plus
 * SV_ERR_ARG for total_drafts < 0, K_max < 0, a NULL cu_drafts, or sizes that overflow.
 */
sv_status spec_verify_ragged(const void* target_logits, const void* draft_logits, int dtype,
                             const int32_t* cu_drafts, int total_drafts, int K_max,
                             const int32_t* draft_tokens, const float* uniforms,
                             const float* temperature, int B, int V,
                             int32_t* out_tokens, int32_t* out_accept_len,
                             float* out_p, float* out_q, int32_t* out_status,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Greedy verify in the ragged layout of spec_verify_ragged (target rows only; the rule
 * of spec_verify_greedy with K = K_b per sequence).
 */
sv_status spec_verify_greedy_ragged(const void* target_logits, int dtype,
                                    const int32_t* cu_drafts, int total_drafts, int K_max,
                                    const int32_t* draft_tokens, int B, int V,
                                    int32_t* out_tokens, int32_t* out_accept_len,
                                    int32_t* out_status,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Largest token tree of the tree entry points (nodes per sequence, root included). */
#define SV_TREE_MAX_NODES 1024

/*
 * Greedy verification of a draft token tree.  Node 0 of each sequence's tree is the
 * root (the last token already emitted); node j >= 1 carries a drafted token and has a
 * parent p(j) < j.  The target has scored all nodes in one forward pass under the tree
 * attention mask (sv_tree_attention_mask): its row j is the next-token logits after the
 * path root -> j.  Rule: node j is accepted when its parent is accepted and its token is
 * the lowest-index argmax of its parent's row (the greedy rule of spec_verify_greedy
 * along every root path); the root is accepted.  The winner is the deepest accepted node
 * a, the lowest index among equally deep ones: the longest prefix along any accepted
 * path.  The emitted tokens are the tokens along root -> a, then the argmax of a's row.
 * Source: "Verificação de Atenção em Árvore" on the lesson page "Decodificação
 * Especulativa e EAGLE" ("Kiểm tra sự chú ý của cây" on the Vietnamese page); the EAGLE
 * section of "Accelerating Sonar through speculation" (the longest accepted candidate
 * plus one token from the target).  The pages give no sampled rule for trees.
 *
 *   target_logits  device, [B][N][V] of `dtype`.
 *   parents        device, [B][N] int32: -1 for node 0, else in [0, j).
 *   node_tokens    device, [B][N] int32, in [0, V) for j >= 1 (node 0's is not read).
 *   B, N, V        B >= 0, 1 <= N <= SV_TREE_MAX_NODES, V >= 1.
 *   out_tokens     device, [B][N] int32: the d tokens along the winning path, the
 *                  target's token after it, then -1.
 *   out_nodes      device, [B][N] int32, or NULL: the d node indices along the path
 *                  (root excluded), then -1 (which drafted nodes' KV entries to keep).
 *   out_accept_len device, [B] int32: d, the depth of the winning node.
 *   out_status     device, [B] int32: SV_SEQ_* flags (TREE, TOKEN, LOGIT); a flagged
 *                  sequence emits -1 everywhere.
 *   workspace      at least sv_workspace_bytes(B, N - 1, V).
 * Bit-exact by construction (comparisons only).
 */
sv_status spec_verify_tree_greedy(const void* target_logits, int dtype, const int32_t* parents,
                                  const int32_t* node_tokens, int B, int N, int V,
                                  int32_t* out_tokens, int32_t* out_nodes,
                                  int32_t* out_accept_len, int32_t* out_status,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * The tree attention mask of the same trees: out_mask[b][i][j] = 1 when node j is node i
 * or one of its ancestors (each token attends only to its ancestors, "Verificação de
 * Atenção em Árvore"), else 0; out_depth[b][i] (optional) = the number of edges from the
 * root to node i (the position offset of node i's token).  A sequence whose parents
 * break the rule of spec_verify_tree_greedy gets SV_SEQ_ERR_TREE in out_status[b], an
 * all-zero mask and depths -1; otherwise out_status[b] = 0.
 *   parents   device, [B][N] int32;  out_mask device, [B][N][N] uint8;
 *   out_depth device, [B][N] int32 or NULL;  out_status device, [B] int32.
 * Host errors: SV_ERR_ARG for B < 0, N outside [1, SV_TREE_MAX_NODES], NULL required
 * pointers or misaligned int32 pointers.
 */
sv_status sv_tree_attention_mask(const int32_t* parents, int B, int N, uint8_t* out_mask,
                                 int32_t* out_depth, int32_t* out_status, void* stream);

/*
 * Draft-side sampler: one token per row from softmax(z / T), the temperature softmax the
 * draft applies before its draw in the "Desenvolva" listing ("Decodificação Especulativa
 * e EAGLE"; "Hãy xây dựng nó" on the Vietnamese page), by the categorical-draw rule above
 * (fp64 weights, smallest i whose prefix exceeds u * sum); at T == 0 the lowest-index
 * argmax.  The same computation as spec_verify with K = 0.
 *
 *   logits         device, [B][V] of `dtype`.
 *   uniforms       device, [B] fp32 in [0, 1) (not read for T == 0).
 *   temperature    device, [B] fp32.
 *   out_tokens     device, [B] int32 (-1 for a sequence with a data error).
 *   out_status     device, [B] int32, SV_SEQ_* flags.
 *   workspace      at least sv_workspace_bytes(B, 0, V).
 */
sv_status sv_sample(const void* logits, int dtype, const float* uniforms,
                    const float* temperature, int B, int V, int32_t* out_tokens,
                    int32_t* out_status, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Fill uniforms[B][K+1] (device, fp32) with the counter-based draws of the exact
 * rule's r ~ Uniform(0, 1) ("A Regra de Exatidão") and of the final categorical draw:
 *   u[b][t] = (w0 >> 40) * 2^-24,   (w0, w1, w2, w3) = Philox4x64-10(counter, key),
 *   key = (seed, domain), counter = (t, b, step, 0),
 * Philox4x64-10 as published by Salmon, Moraes, Dror and Shaw ("Parallel random
 * numbers: as easy as 1, 2, 3", SC'11).  Every u is a multiple of 2^-24 in [0, 1).
 * B >= 0, K >= 0; uniforms may be NULL only when B == 0.
 */
sv_status sv_fill_uniforms(uint64_t seed, uint64_t domain, uint64_t step, int B, int K,
                           float* uniforms, void* stream);

/*
 * The same draws in the ragged layout: uniforms[cu[b] + b + t] (device, [total_drafts + B])
 * = the u that sv_fill_uniforms gives for (b, t), for t <= K_b, for every sequence whose
 * offsets are valid (see spec_verify_ragged; other sequences' slots are not written).
 */
sv_status sv_fill_uniforms_ragged(uint64_t seed, uint64_t domain, uint64_t step, int B,
                                  const int32_t* cu_drafts, int total_drafts, int K_max,
                                  float* uniforms, void* stream);

/*
 * Kernel timing for benchmarks (host state, not thread-safe).
 * sv_profile_begin: until sv_profile_end, every verify or sampling call records HIP
 * events on its stream around its pass-1 kernel (streaming of the logit rows) and around
 * its pass-2 kernels (the resolve and the categorical draw).
 * sv_profile_end: waits for those events, writes the number of calls and the summed
 * milliseconds of each phase (any pointer may be NULL), and stops recording.  Returns
 * SV_ERR_HIP if an event could not be created, recorded or read.
 */
sv_status sv_profile_begin(void);
sv_status sv_profile_end(int* calls, double* ms_pass1, double* ms_pass2);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
