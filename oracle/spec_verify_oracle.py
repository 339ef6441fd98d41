"""fp64 CPU oracle of the batched speculative-sampling verify step.

TEST INFRASTRUCTURE ONLY.  This is the plain, slow reference that the HIP library
is checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code, header,
table or constant with the HIP path; status codes are restated here from the
library's documented contract.

What it computes (per sequence b; sources are the lesson pages "Việc giải mã giả
định và Eagle" (aiengineeringfromscratch.com, Vietnamese) and "Decodificação
Especulativa e EAGLE" (ai-engineering.academy, Phase 10 Lesson 25), which carry
the same text):

* The draft proposes x_0..x_{K-1}; the target gives K+1 rows of logits and the
  draft K rows ("O Conceito", steps 1-2).
* p_t = softmax(zt_t / T), q_t = softmax(zd_t / T): the temperature softmax of the
  pseudocode in "Desenvolva" / "Hãy xây dựng nó", with the same T on both sides.
* Left to right, accept x_t while r_t < p_t(x_t) / q_t(x_t) ("A Regra de
  Exatidão" / "Quy tắc chính xác").
* On the first rejection, emit one token drawn from (p_t - q_t)+ / ||(p_t - q_t)+||_1,
  the positive part of the POINTWISE difference over the whole vocabulary
  ("A Regra de Exatidão"; the livestream "IA local 202" describes the same
  clamp-at-zero-then-normalise at [12:30]).  The pseudocode on those pages
  subtracts the scalar q(x_t) instead; that contradicts the rule text and does not
  preserve p, so the rule text is followed (see the negative test).
* If all K are accepted, emit a bonus token drawn from p_K ("O Conceito", step 4).
* Temperature 0: accept while argmax(p_t) == x_t, else emit argmax(p_t) and stop
  ("Caso ganancioso" / "Greedy case"); after K matches the bonus is argmax(p_K),
  the T -> 0 limit of the bonus rule.

Readings where the pages are silent (each is part of the library contract too):

* argmax ties go to the lowest index (numpy's documented first-occurrence rule).
* A categorical draw with weights w and uniform u returns the smallest i with
  C_i > u * S, where C_i = w_0 + ... + w_i accumulated left to right in fp64 and
  S = C_{V-1}.  Slot u[b][K] drives that draw; u[b][t] drives test t.
* If no index satisfies it (only possible through rounding) the last index with
  positive weight is returned.  If the residual has zero fp64 mass after a
  rejection (impossible in exact arithmetic, since p(x) < q(x) there), the draw
  uses p_t instead and the sequence is flagged NOTE_FALLBACK.
* Data errors, per sequence (bit flags, OR-ed):
    ERR_TOKEN        a draft token outside [0, V)
    ERR_LOGIT        a NaN in any row the sequence reads, a row whose maximum is
                     -inf, or (sampled sequences) a +inf logit, or (sampled sequences
                     with a valid T) a row whose maximum m has |m| * c2 >= 2^30,
                     c2 = log2(e) / T rounded to fp32 (the range of scaled logits
                     the verify path supports; see scaled_range_error)
    ERR_TEMPERATURE  T is NaN, negative, infinite, or positive but below the
                     smallest normal fp32 (1/T would not be finite in fp32)
    ERR_UNIFORM      (sampled sequences) a uniform that is NaN or outside [0, 1)
  A sequence with any error emits tokens -1, accept length -1, p = q = NaN.
  A sequence is "greedy" iff T == 0; otherwise it reads the draft rows too.

Precision: logits are decoded exactly (bf16 and fp32 widen exactly to fp64); all
arithmetic below is fp64 with numpy's exp/log.
"""

import math

import numpy as np

SEQ_OK = 0
SEQ_ERR_TOKEN = 1
SEQ_ERR_LOGIT = 2
SEQ_ERR_TEMPERATURE = 4
SEQ_ERR_UNIFORM = 8
SEQ_NOTE_FALLBACK = 16
SEQ_ERR_OFFSETS = 32
SEQ_ERR_TREE = 64
SEQ_ERROR_MASK = (SEQ_ERR_TOKEN | SEQ_ERR_LOGIT | SEQ_ERR_TEMPERATURE | SEQ_ERR_UNIFORM
                  | SEQ_ERR_OFFSETS | SEQ_ERR_TREE)

FP32_MIN_NORMAL = 2.0 ** -126


# ----------------------------------------------------------------------------
# Decoding
# ----------------------------------------------------------------------------

def decode_bf16(bits):
    """bf16 bit patterns (uint16) -> float64, exactly (a bf16 is the top half of an fp32)."""
    bits = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):  # NaN payloads widen to NaN
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def decode_logits(raw):
    """Logit rows as stored (uint16 = bf16 bits, float32) -> float64, exactly."""
    raw = np.asarray(raw)
    if raw.dtype == np.uint16:
        return decode_bf16(raw)
    if raw.dtype == np.float32:
        return raw.astype(np.float64)
    if raw.dtype == np.float64:
        return raw
    raise TypeError(f"unsupported logit storage {raw.dtype}")


# ----------------------------------------------------------------------------
# The steps of the method
# ----------------------------------------------------------------------------

def softmax_t(z, T):
    """p = softmax(z / T) in fp64, shifted by the row maximum (exact for the quotient)."""
    m = np.max(z)
    e = np.exp((z - m) / T)
    return e / np.sum(e)


def prob_at(z, T, x):
    """p(x) for p = softmax(z / T), fp64: exp((z_x - m)/T) / sum_i exp((z_i - m)/T)."""
    m = np.max(z)
    return math.exp((z[x] - m) / T) / float(np.sum(np.exp((z - m) / T)))


def argmax_first(z):
    """Index of the maximum; ties go to the lowest index (numpy.argmax's rule)."""
    return int(np.argmax(z))


def log_prob_at(z, T, x):
    """ln p(x) for p = softmax(z / T), fp64: (z_x - m)/T - ln sum_i exp((z_i - m)/T).
    -inf exactly when z_x is -inf; it does not underflow where p(x) itself would."""
    m = np.max(z)
    return (z[x] - m) / T - math.log(float(np.sum(np.exp((z - m) / T))))


def accept_test(u, lp_x, lq_x):
    """The exact rule's test r < p(x)/q(x) on log-probabilities: ln u < ln p - ln q.

    p = 0 (ln p = -inf) rejects, q = 0 with p > 0 accepts, u = 0 accepts any p > 0.
    In log space the test holds the real-number predicate even where p(x) and q(x)
    underflow fp64 on their own.
    """
    if lp_x == -math.inf:
        return False
    if lq_x == -math.inf:
        return True
    return (math.log(u) if u > 0.0 else -math.inf) < lp_x - lq_x


def replacement_weights(p, q, x):
    """Weights of the replacement draw after drafted token x was rejected.

    The rule text: (p - q)+ taken pointwise over the whole vocabulary, left
    unnormalised (the categorical draw normalises).  x does not enter; it is an
    argument so that tests can plant the variants the pages' code listings imply
    (subtracting the scalar q(x), or drawing from p) and show they break the law.
    """
    return np.maximum(p - q, 0.0)


def categorical_draw(w, u):
    """Smallest i with C_i > u*S (C = left-to-right fp64 prefix sums of w, S = C[-1]).

    Returns (index, margin, fell_through) where margin is the distance from u to the
    nearer edge of the chosen cell [C_{i-1}/S, C_i/S) and fell_through says that no
    index satisfied the predicate (then the last index with w > 0 is returned).
    """
    c = np.cumsum(w)
    s = c[-1]
    target = u * s
    i = int(np.searchsorted(c, target, side="right"))
    fell = False
    if i >= len(w):
        fell = True
        i = int(np.nonzero(w > 0)[0][-1])
    lo = (c[i - 1] if i > 0 else 0.0) / s
    hi = c[i] / s
    margin = min(abs(u - lo), abs(hi - u))
    return i, margin, fell


def expected_tokens(alpha, K):
    """E[tokens per target forward] = (1 - alpha^{K+1}) / (1 - alpha)  ("Aceleração Esperada").

    alpha is the token-level acceptance rate; at alpha = 1 the limit K + 1 is returned.
    """
    if alpha == 1.0:
        return float(K + 1)
    return (1.0 - alpha ** (K + 1)) / (1.0 - alpha)


def expected_tokens_general(alphas):
    """E[n+1] = sum_{j=0..K} prod_{i<j} alpha_i for per-position acceptance rates.

    Reduces to expected_tokens(alpha, K) when every alpha_i equals alpha.
    """
    total, run = 1.0, 1.0
    for a in alphas:
        run *= a
        total += run
    return total


def acceptance_rate(p, q):
    """alpha = sum_v min(p(v), q(v)) = E_{x~q}[min(1, p(x)/q(x))]."""
    return float(np.sum(np.minimum(p, q)))


# ----------------------------------------------------------------------------
# Validation (data errors)
# ----------------------------------------------------------------------------

def temperature_error(T):
    T = float(T)
    if math.isnan(T) or T < 0.0 or math.isinf(T):
        return True
    return 0.0 < T < FP32_MIN_NORMAL


LOG2E = 1.4426950408889634  # log2(e), rounded to fp64


SCALED_RANGE = 2.0 ** 30


def scaled_range_error(m, T):
    """|m| * c2 >= 2^30 with c2 = log2(e)/T rounded to fp32 (the product of two fp32
    values is exact in fp64).  The pages put no bound on logits or temperatures; this is
    the library's contract (its first pass holds the scaled row maximum as an fp32
    number whose rounding must stay far below the range of an fp32 exponential), and the
    oracle applies the same rule so that both sides flag the same rows."""
    c2 = float(np.float32(LOG2E / T))
    return abs(float(m)) * c2 >= SCALED_RANGE


def row_error(z, sampled, T=None):
    """NaN anywhere, a maximum of -inf, or (sampled rows) a +inf logit; with a valid
    temperature T > 0 also a maximum outside the scaled range (scaled_range_error)."""
    if np.isnan(z).any():
        return True
    m = np.max(z)
    if m == -np.inf:
        return True
    if sampled and m == np.inf:
        return True
    return bool(sampled and T is not None and T > 0.0 and not temperature_error(T)
                and scaled_range_error(m, T))


# ----------------------------------------------------------------------------
# One sequence
# ----------------------------------------------------------------------------

def verify_sequence(zt, zd, x, u, T):
    """Verify one sequence.

    zt: [K+1][V] target logits (any storage decode_logits accepts)
    zd: [K][V] draft logits, or None (only allowed when T == 0)
    x:  [K] draft tokens;  u: [K+1] uniforms (None allowed when T == 0);  T: float
    Returns a dict: tokens [K+1] (-1 padded), n (accepted drafts), p, q [K]
    (p_t(x_t), q_t(x_t), NaN on greedy or failed sequences), status, draws
    (list of (kind, t, margin) in the order the uniforms are consumed).
    """
    zt = np.asarray(zt)
    K = zt.shape[0] - 1
    V = zt.shape[1]
    x = [int(v) for v in x]
    T = float(T)
    greedy = (T == 0.0)

    status = SEQ_OK
    if temperature_error(T):
        status |= SEQ_ERR_TEMPERATURE
    if any(v < 0 or v >= V for v in x):
        status |= SEQ_ERR_TOKEN
    rows_t = [decode_logits(zt[t]) for t in range(K + 1)]
    rows_d = [] if greedy else [decode_logits(zd[t]) for t in range(K)]
    if any(row_error(r, not greedy, T) for r in rows_t + rows_d):
        status |= SEQ_ERR_LOGIT
    if not greedy:
        uu = [float(v) for v in u]
        if any(math.isnan(v) or v < 0.0 or v >= 1.0 for v in uu):
            status |= SEQ_ERR_UNIFORM

    nan_k = [math.nan] * K
    if status & SEQ_ERROR_MASK:
        return dict(tokens=[-1] * (K + 1), n=-1, p=nan_k, q=list(nan_k), status=status, draws=[])

    tokens = [-1] * (K + 1)
    if greedy:
        for t in range(K):
            a = argmax_first(rows_t[t])
            if a != x[t]:
                tokens[:t] = x[:t]
                tokens[t] = a
                return dict(tokens=tokens, n=t, p=nan_k, q=list(nan_k), status=status, draws=[])
        tokens[:K] = x
        tokens[K] = argmax_first(rows_t[K])
        return dict(tokens=tokens, n=K, p=nan_k, q=list(nan_k), status=status, draws=[])

    # Sampled: ln p_t(x_t) and ln q_t(x_t) for every drafted position.
    lp_x = [log_prob_at(rows_t[t], T, x[t]) for t in range(K)]
    lq_x = [log_prob_at(rows_d[t], T, x[t]) for t in range(K)]
    p_x = [math.exp(v) for v in lp_x]
    q_x = [math.exp(v) for v in lq_x]
    draws = []
    for t in range(K):
        # margin: |u - p/q|; p = 0 or q = 0 decide the test whatever u is
        if lp_x[t] == -math.inf or lq_x[t] == -math.inf:
            margin = math.inf
        else:
            d = lp_x[t] - lq_x[t]
            margin = abs(uu[t] - (math.exp(d) if d < 700.0 else math.inf))
        draws.append(("test", t, margin))
        if accept_test(uu[t], lp_x[t], lq_x[t]):
            continue
        # First rejection: replacement from the pointwise residual.
        p = softmax_t(rows_t[t], T)
        q = softmax_t(rows_d[t], T)
        w = replacement_weights(p, q, x[t])
        if not np.sum(w) > 0.0:
            status |= SEQ_NOTE_FALLBACK
            w = p
        y, margin, fell = categorical_draw(w, uu[K])
        if fell:
            status |= SEQ_NOTE_FALLBACK
        draws.append(("residual", t, margin))
        tokens[:t] = x[:t]
        tokens[t] = y
        return dict(tokens=tokens, n=t, p=p_x, q=q_x, status=status, draws=draws)

    # All K accepted: bonus token from p_K.
    y, margin, fell = categorical_draw(softmax_t(rows_t[K], T), uu[K])
    if fell:
        status |= SEQ_NOTE_FALLBACK
    draws.append(("bonus", K, margin))
    tokens[:K] = x
    tokens[K] = y
    return dict(tokens=tokens, n=K, p=p_x, q=q_x, status=status, draws=draws)


# ----------------------------------------------------------------------------
# A batch (same argument meaning as the library's entry points)
# ----------------------------------------------------------------------------

def verify(target_logits, draft_logits, draft_tokens, uniforms, temperature, seqs=None):
    """Batched sampled/greedy verify.

    target_logits [B][K+1][V], draft_logits [B][K][V] (uint16 bf16 bits or float32),
    draft_tokens [B][K] int, uniforms [B][K+1] float32, temperature [B] float32.
    ``seqs`` restricts the work to a subset of sequence indices (others are left
    as -1 / NaN with status -1 in the result).
    Returns dict of numpy arrays: tokens [B][K+1] int32, accept_len [B] int32,
    p, q [B][K] float32, status [B] int32, and ``draws``: {b: list of draws}.
    """
    target_logits = np.asarray(target_logits)
    B, K1, V = target_logits.shape
    K = K1 - 1
    out_tokens = np.full((B, K + 1), -1, dtype=np.int32)
    out_n = np.full(B, -1, dtype=np.int32)
    out_p = np.full((B, K), np.nan, dtype=np.float32)
    out_q = np.full((B, K), np.nan, dtype=np.float32)
    out_status = np.full(B, -1, dtype=np.int32)
    draws = {}
    for b in (range(B) if seqs is None else seqs):
        T = float(np.float32(temperature[b]))
        zd = None if draft_logits is None else draft_logits[b]
        r = verify_sequence(target_logits[b], zd, draft_tokens[b],
                            None if uniforms is None else uniforms[b], T)
        out_tokens[b] = r["tokens"]
        out_n[b] = r["n"]
        out_p[b] = np.asarray(r["p"], dtype=np.float64).astype(np.float32) if K else out_p[b]
        out_q[b] = np.asarray(r["q"], dtype=np.float64).astype(np.float32) if K else out_q[b]
        out_status[b] = r["status"]
        draws[b] = r["draws"]
    return dict(tokens=out_tokens, accept_len=out_n, p=out_p, q=out_q,
                status=out_status, draws=draws)


def verify_greedy(target_logits, draft_tokens, seqs=None):
    """All sequences greedy (temperature 0); no draft logits and no uniforms are read."""
    target_logits = np.asarray(target_logits)
    B = target_logits.shape[0]
    r = verify(target_logits, None, draft_tokens, None, np.zeros(B, dtype=np.float32), seqs)
    return dict(tokens=r["tokens"], accept_len=r["accept_len"], status=r["status"])


# ----------------------------------------------------------------------------
# Ragged batches and plain sampling
# ----------------------------------------------------------------------------

def verify_ragged(target_logits, draft_logits, cu_drafts, draft_tokens, uniforms,
                  temperature, K_max, seqs=None):
    """Verify with a different number of drafts per sequence (packed layout).

    Adaptive verification (the Speculators talk in the livestream "IA local 202",
    [44:15]-[45:16]) verifies each request on its own number of drafted tokens K_b; the
    rule per sequence is the one above with K = K_b.  Layout: sequence b owns draft rows,
    draft tokens and p/q slots cu[b] .. cu[b+1]-1, and target rows, uniforms and output
    token slots cu[b]+b .. cu[b+1]+b.  Offsets with cu[b] < 0, cu[b+1] < cu[b],
    cu[b+1] > total or K_b > K_max flag ERR_OFFSETS (accept length -1, nothing else
    written for that sequence).

    Returns dict: tokens [total+B] int32 (-1 where unwritten), accept_len [B],
    p, q [total] float32, status [B], draws {b: list}, and K [B] (K_b, or -1).
    """
    cu = [int(v) for v in cu_drafts]
    B = len(cu) - 1
    total = len(draft_tokens)
    out_tokens = np.full(total + B, -1, dtype=np.int32)
    out_n = np.full(B, -1, dtype=np.int32)
    out_p = np.full(total, np.nan, dtype=np.float32)
    out_q = np.full(total, np.nan, dtype=np.float32)
    out_status = np.full(B, -1, dtype=np.int32)
    ks = np.full(B, -1, dtype=np.int64)
    draws = {}
    for b in (range(B) if seqs is None else seqs):
        c0, c1 = cu[b], cu[b + 1]
        if c0 < 0 or c1 < c0 or c1 > total or c1 - c0 > K_max:
            out_status[b] = SEQ_ERR_OFFSETS
            draws[b] = []
            continue
        K = c1 - c0
        ks[b] = K
        T = float(np.float32(temperature[b]))
        zd = None if T == 0.0 else draft_logits[c0:c1]
        u = None if T == 0.0 else uniforms[c0 + b:c1 + b + 1]
        r = verify_sequence(target_logits[c0 + b:c1 + b + 1], zd, draft_tokens[c0:c1], u, T)
        out_tokens[c0 + b:c1 + b + 1] = r["tokens"]
        out_n[b] = r["n"]
        if K:
            out_p[c0:c1] = np.asarray(r["p"], dtype=np.float64).astype(np.float32)
            out_q[c0:c1] = np.asarray(r["q"], dtype=np.float64).astype(np.float32)
        out_status[b] = r["status"]
        draws[b] = r["draws"]
    return dict(tokens=out_tokens, accept_len=out_n, p=out_p, q=out_q, status=out_status,
                draws=draws, K=ks)


def sample(logits, uniforms, temperature):
    """One token per row from softmax(z / T) by the categorical-draw rule, argmax at T = 0.

    This is the draft model's own draw in the "Desenvolva" / "Hãy xây dựng nó" listing
    (temperature softmax, then a categorical draw), and exactly the verify step with no
    drafts: the bonus draw from p_0.  Returns dict: tokens [B] int32, status [B] int32,
    draws {b: list}.
    """
    logits = np.asarray(logits)
    B = logits.shape[0]
    tokens = np.full(B, -1, dtype=np.int32)
    status = np.zeros(B, dtype=np.int32)
    draws = {}
    for b in range(B):
        T = float(np.float32(temperature[b]))
        r = verify_sequence(logits[b:b + 1], None, [], None if T == 0.0 else [uniforms[b]], T)
        tokens[b] = r["tokens"][0]
        status[b] = r["status"]
        draws[b] = r["draws"]
    return dict(tokens=tokens, status=status, draws=draws)


# ----------------------------------------------------------------------------
# Token trees (greedy)
# ----------------------------------------------------------------------------

def tree_parents_ok(parents):
    """Node 0 is the root (parent -1); every other node's parent comes before it."""
    return all((p == -1) if j == 0 else (0 <= p < j) for j, p in enumerate(parents))


def verify_tree_sequence(zt, parents, tokens):
    """Greedy verification of one draft token tree.

    The target scores every node of the tree in one pass under a tree attention mask,
    and the output is the longest prefix along any accepted root path ("Verificação de
    Atenção em Árvore" on the lesson page "Decodificação Especulativa e EAGLE"; the EAGLE
    section of "Accelerating Sonar through speculation").  With the greedy rule
    ("Caso ganancioso") on every root path: the root (node 0) is accepted; node j is
    accepted when its parent p(j) is accepted and its token equals argmax of row p(j),
    row i being the target's logits after the path root -> i.  Reading (the pages do not
    say which of several equally long paths wins): the deepest accepted node, the lowest
    index among equally deep ones.  Emitted: the tokens along root -> winner, then the
    argmax of the winner's row.

    zt: [N][V] logits; parents: [N] ints; tokens: [N] ints (tokens[0] unused).
    Returns dict: tokens [N] (-1 padded), nodes [N] (path nodes, root excluded, -1
    padded), n (depth of the winner), status.
    """
    zt = np.asarray(zt)
    N, V = zt.shape
    parents = [int(p) for p in parents]
    tokens = [int(t) for t in tokens]
    status = SEQ_OK
    if not tree_parents_ok(parents):
        status |= SEQ_ERR_TREE
    if any(t < 0 or t >= V for t in tokens[1:]):
        status |= SEQ_ERR_TOKEN
    rows = [decode_logits(zt[j]) for j in range(N)]
    if any(row_error(r, False) for r in rows):
        status |= SEQ_ERR_LOGIT
    if status & SEQ_ERROR_MASK:
        return dict(tokens=[-1] * N, nodes=[-1] * N, n=-1, status=status)
    amax = [argmax_first(r) for r in rows]
    accepted = [True] + [False] * (N - 1)
    depth = [0] * N
    for j in range(1, N):
        p = parents[j]
        depth[j] = depth[p] + 1
        accepted[j] = accepted[p] and tokens[j] == amax[p]
    win = 0
    for j in range(N):
        if accepted[j] and depth[j] > depth[win]:
            win = j
    path = []
    cur = win
    while cur != 0:
        path.append(cur)
        cur = parents[cur]
    path.reverse()
    d = len(path)
    out_tokens = [tokens[j] for j in path] + [amax[win]] + [-1] * (N - d - 1)
    out_nodes = path + [-1] * (N - d)
    return dict(tokens=out_tokens, nodes=out_nodes, n=d, status=status)


def verify_tree_greedy(target_logits, parents, node_tokens):
    """Batched tree verification: target_logits [B][N][V], parents and node_tokens [B][N].
    Returns dict of numpy arrays tokens, nodes [B][N], accept_len [B], status [B]."""
    target_logits = np.asarray(target_logits)
    B, N, _ = target_logits.shape
    out = dict(tokens=np.full((B, N), -1, dtype=np.int32), nodes=np.full((B, N), -1, dtype=np.int32),
               accept_len=np.full(B, -1, dtype=np.int32), status=np.zeros(B, dtype=np.int32))
    for b in range(B):
        r = verify_tree_sequence(target_logits[b], parents[b], node_tokens[b])
        out["tokens"][b] = r["tokens"]
        out["nodes"][b] = r["nodes"]
        out["accept_len"][b] = r["n"]
        out["status"][b] = r["status"]
    return out


def tree_attention_mask(parents):
    """mask[i][j] = 1 when node j is node i or an ancestor of it (each token attends only
    to its ancestors, "Verificação de Atenção em Árvore"); depth[i] = edges from the root.
    A malformed tree gives an all-zero mask, depths -1 and ERR_TREE.  parents: [B][N]."""
    parents = np.asarray(parents)
    B, N = parents.shape
    mask = np.zeros((B, N, N), dtype=np.uint8)
    depth = np.full((B, N), -1, dtype=np.int32)
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        par = [int(p) for p in parents[b]]
        if not tree_parents_ok(par):
            status[b] = SEQ_ERR_TREE
            continue
        for i in range(N):
            cur, d = i, 0
            while True:
                mask[b, i, cur] = 1
                if cur == 0:
                    break
                cur = par[cur]
                d += 1
            depth[b, i] = d
    return dict(mask=mask, depth=depth, status=status)
