"""Pins of the fp64 oracle against what the pages and mathematics fix.

Each test would fail for a plausible mistake somewhere in the oracle:
  * exact enumeration at V=4, K=2 (distribution preservation, the exact rule on the
    lesson pages "Việc giải mã giả định và Eagle" / "Decodificação Especulativa e
    EAGLE", section "A Regra de Exatidão"): any wrong sign, index, dropped term,
    wrong temperature handling or wrong residual breaks the exact equality;
  * the closed form E[tokens] = (1 - a^{K+1})/(1 - a) and its printed value 3.36
    ("Aceleração Esperada"), on inputs constructed so that sum(min(p, q)) = a;
  * closed forms of the temperature softmax, exact rational CDFs for the
    categorical draw, brute force for argmax ties, special cases (p == q, disjoint
    supports, K = 0, V = 1, T -> 0 equals greedy) and negative tests showing that
    the pages' code-listing residual and the Q&A page's reject branch break the law.
"""
import math
from fractions import Fraction as F
import itertools
import os

import numpy as np
import pytest

from oracle import spec_verify_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------

def dist(ws):
    s = sum(ws)
    return [F(w, s) for w in ws]


def logits_of(p, T, shift=0.0):
    """Logits z with softmax(z/T) = p: z = T*ln(p) + shift (-inf where p = 0)."""
    return np.array([T * math.log(float(v)) + shift if v > 0 else -math.inf for v in p])


def positive_part(a, b):
    return [max(x - y, F(0)) for x, y in zip(a, b)]


def normalise(w):
    s = sum(w)
    return [x / s for x in w] if s > 0 else None


def breakpoints_of(w):
    """Exact CDF edges in (0, 1) of the categorical law with weights w."""
    w = normalise(w)
    if w is None:
        return []
    out, run = [], F(0)
    for x in w[:-1]:
        run += x
        out.append(run)
    return out


def cells(points):
    """Partition [0, 1) at the given points; returns (midpoint as float, exact width)."""
    pts = sorted({F(0), F(1)} | {p for p in points if 0 < p < 1})
    return [(float((a + b) / 2), b - a) for a, b in zip(pts[:-1], pts[1:]) if b > a]


# ----------------------------------------------------------------------------
# V = 4, K = 2 fixture: target conditionals p1, p2(.|a), p3(.|a,b); draft q1, q2(.|a)
# Rational, with zeros on both sides so that support corner cases are exercised.
# ----------------------------------------------------------------------------

V4 = 4
P1 = dist([3, 1, 4, 2])
P2 = {a: dist([(a + 1) % 3, 2 + a, 1, 5 - a]) for a in range(4)}  # a=2 gives p2[0] = 0
P3 = {(a, b): dist([1 + (a * b) % 3, (a + 2 * b) % 4, 2, 1 + a]) for a in range(4) for b in range(4)}
Q1 = dist([2, 5, 0, 3])
Q2 = {a: dist([4 - a, 1, a % 2 + 1, 3]) if a != 1 else dist([1, 0, 6, 2]) for a in range(4)}


def target_law(a, b, c):
    return P1[a] * P2[a][b] * P3[(a, b)][c]


def completion(emitted):
    """Exact law of (a, b, c) after emitting `emitted`, continuing with target samples."""
    out = {}
    if len(emitted) == 1:
        a = emitted[0]
        for b in range(V4):
            for c in range(V4):
                out[(a, b, c)] = P2[a][b] * P3[(a, b)][c]
    elif len(emitted) == 2:
        a, b = emitted
        for c in range(V4):
            out[(a, b, c)] = P3[(a, b)][c]
    else:
        out[tuple(emitted)] = F(1)
    return out


def enumerate_law(T, shift_t=0.0, shift_d=0.0):
    """Exact law of the completed 3-token output of one verify step (oracle decisions)."""
    law = {k: F(0) for k in itertools.product(range(V4), repeat=3)}
    for x1 in range(V4):
        for x2 in range(V4):
            W = Q1[x1] * Q2[x1][x2]
            if W == 0:
                continue
            p_rows = [P1, P2[x1], P3[(x1, x2)]]
            q_rows = [Q1, Q2[x1]]
            zt = np.stack([logits_of(r, T, shift_t) for r in p_rows])
            zd = np.stack([logits_of(r, T, shift_d) for r in q_rows])
            r0 = P1[x1] / Q1[x1]
            r1 = P2[x1][x2] / Q2[x1][x2]
            # every distribution the final draw could use, for the rule and the planted
            # variants, so that one partition of u2 is fine enough for all of them
            finals = [P3[(x1, x2)]]
            for p, q, x in ((P1, Q1, x1), (P2[x1], Q2[x1], x2)):
                finals += [positive_part(p, q), positive_part(p, [q[x]] * V4), p]
            u2_points = [bp for w in finals for bp in breakpoints_of(w)]
            for m0, w0 in cells([r0]):
                for m1, w1 in cells([r1]):
                    for m2, w2 in cells(u2_points):
                        r = O.verify_sequence(zt, zd, [x1, x2], [m0, m1, m2], T)
                        assert r["status"] & O.SEQ_ERROR_MASK == 0
                        emitted = r["tokens"][: r["n"] + 1]
                        for k, v in completion(emitted).items():
                            law[k] += W * w0 * w1 * w2 * v
    return law


@pytest.mark.parametrize("T,shift_t,shift_d", [(1.0, 0.0, 0.0), (0.7, 37.5, -12.0), (2.5, -3.0, 80.0)])
def test_exact_enumeration_preserves_target_law(T, shift_t, shift_d, monkeypatch):
    flags = []
    real = O.verify_sequence

    def spy(*a, **k):
        r = real(*a, **k)
        flags.append(r["status"])
        return r

    monkeypatch.setattr(O, "verify_sequence", spy)
    law = enumerate_law(T, shift_t, shift_d)
    assert set(flags) == {0}
    assert sum(law.values()) == 1
    for k, v in law.items():
        assert v == target_law(*k), (k, v, target_law(*k))


def test_negative_code_listing_residual_breaks_law(monkeypatch):
    """The pages' code listing subtracts the scalar q(x_t): (p - q(x_t))+.  Not exact."""
    monkeypatch.setattr(O, "replacement_weights", lambda p, q, x: np.maximum(p - q[x], 0.0))
    law = enumerate_law(1.0)
    dev = max(abs(float(v - target_law(*k))) for k, v in law.items())
    assert dev > 1e-3


def test_negative_reject_branch_sampling_from_p_breaks_law(monkeypatch):
    """The Q&A page resamples from p after a rejection.  Not exact."""
    monkeypatch.setattr(O, "replacement_weights", lambda p, q, x: p)
    law = enumerate_law(1.0)
    dev = max(abs(float(v - target_law(*k))) for k, v in law.items())
    assert dev > 1e-3


# ----------------------------------------------------------------------------
# Closed form E[tokens] = (1 - a^{K+1}) / (1 - a)
# ----------------------------------------------------------------------------

def read_golden_worked_example():
    with open(os.path.join(GOLDEN, "expected_tokens_worked_example.txt")) as f:
        line = [l for l in f if l.strip() and not l.startswith("#")][0]
    kv = dict(item.split("=") for item in line.split())
    return float(kv["alpha"]), int(kv["K"]), float(kv["tokens"]), int(kv["decimals"])


def constructed_position(alpha, a_w, bp_w, bq_w, V):
    """p = alpha*a + (1-alpha)*b_p, q = alpha*a + (1-alpha)*b_q on disjoint supports.

    a_w, bp_w, bq_w: dicts index -> weight.  Then sum(min(p, q)) = alpha exactly,
    drafts in supp(a) are always accepted (p/q = 1) and drafts in supp(b_q) always
    rejected (p = 0).
    """
    a, bp, bq = (normalise_dict(d) for d in (a_w, bp_w, bq_w))
    p = [F(0)] * V
    q = [F(0)] * V
    for i, v in a.items():
        p[i] += alpha * v
        q[i] += alpha * v
    for i, v in bp.items():
        p[i] += (1 - alpha) * v
    for i, v in bq.items():
        q[i] += (1 - alpha) * v
    return p, q


def normalise_dict(d):
    s = sum(d.values())
    return {k: F(v, s) for k, v in d.items()}


def enumerate_mean_tokens(positions, T=1.0):
    """Exact E[n+1] of the oracle over all drafts x ~ q (acceptance is deterministic)."""
    K = len(positions) - 1
    V = len(positions[0][0])
    zt = np.stack([logits_of(p, T) for p, _ in positions])
    zd = np.stack([logits_of(q, T, 5.0) for _, q in positions[:K]])
    supports = [[i for i in range(V) if q[i] > 0] for _, q in positions[:K]]
    total = F(0)
    for xs in itertools.product(*supports):
        W = F(1)
        for t, x in enumerate(xs):
            W *= positions[t][1][x]
        r = O.verify_sequence(zt, zd, list(xs), [0.999999] * K + [0.5], T)
        assert r["status"] == 0
        total += W * (r["n"] + 1)
    return total


def test_closed_form_worked_value_336():
    alpha, K, printed, decimals = read_golden_worked_example()
    a = F(alpha).limit_denominator(1000)
    pos = constructed_position(a, {0: 1}, {1: 1}, {2: 1}, 4)
    mean = enumerate_mean_tokens([pos] * (K + 1))
    assert mean == F(33616, 10000)
    assert round(float(mean), decimals) == printed
    assert abs(O.expected_tokens(alpha, K) - float(mean)) < 1e-14
    p, q = (np.array([float(v) for v in r]) for r in pos)
    assert abs(O.acceptance_rate(p, q) - alpha) < 1e-15


def test_closed_form_general_per_position_rates():
    alphas = [F(1, 2), F(7, 10), F(9, 10), F(3, 5), F(1, 3)]
    positions = [constructed_position(al, {0: 2, 1: 3, 2: 1}, {3: 1, 4: 4}, {5: 2, 6: 1}, 8)
                 for al in alphas]
    mean = enumerate_mean_tokens(positions, T=0.8)
    expect = sum(math.prod(alphas[:j]) for j in range(len(alphas)))
    assert mean == expect
    assert abs(O.expected_tokens_general([float(a) for a in alphas[:-1]]) - float(mean)) < 1e-14
    for al, (p, q) in zip(alphas, positions):
        pf = np.array([float(v) for v in p])
        qf = np.array([float(v) for v in q])
        assert abs(O.acceptance_rate(pf, qf) - float(al)) < 1e-15


def test_closed_form_formula_values():
    assert O.expected_tokens(0.0, 7) == 1.0                        # nothing accepted
    assert O.expected_tokens(1.0, 7) == 8.0                        # everything accepted
    assert abs(O.expected_tokens(0.5, 200) - 2.0) < 1e-12          # K -> inf: 1/(1-a)
    assert abs(O.expected_tokens(0.8, 4) - 3.3616) < 1e-12
    assert abs(O.expected_tokens_general([0.8] * 4) - 3.3616) < 1e-12


# ----------------------------------------------------------------------------
# Temperature softmax, closed forms
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("T", [0.3, 1.0, 2.5])
@pytest.mark.parametrize("shift", [0.0, 700.0, -900.0])
def test_softmax_closed_form(T, shift):
    rng = np.random.default_rng(3)
    p = rng.dirichlet(np.ones(37))
    p[5] = 0.0
    p /= p.sum()
    z = np.array([T * math.log(v) + shift if v > 0 else -math.inf for v in p])
    got = O.softmax_t(z, T)
    # the logits themselves carry a rounding error of about ulp(shift) / T in z / T
    tol = 1e-14 + 4 * abs(shift) * 2.0 ** -53 / T * 40
    np.testing.assert_allclose(got, p, rtol=tol, atol=0)
    for x in (0, 5, 17, 36):
        assert abs(O.prob_at(z, T, x) - p[x]) <= tol * p[x]
        lp = O.log_prob_at(z, T, x)
        if p[x] == 0:
            assert lp == -math.inf
        else:
            assert abs(lp - math.log(p[x])) <= tol


def test_bf16_decoding_matches_torch():
    torch = pytest.importorskip("torch")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = O.decode_bf16(bits)
    ref = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert (ours[~nan] == ref[~nan]).all()
    assert (np.signbit(ours[~nan]) == np.signbit(ref[~nan])).all()


# ----------------------------------------------------------------------------
# Categorical draw: exact rational CDF
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_categorical_draw_exact_cells(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(1, 12))
    num = rng.integers(0, 9, V)
    if num.sum() == 0:
        num[-1] = 1
    w_exact = [F(int(v), 64) for v in num]                  # dyadic: exact in fp64
    w = np.array([float(v) for v in w_exact])
    S = sum(w_exact)
    C = list(itertools.accumulate(w_exact))
    for k in range(0, 1 << 12):
        u = k / 4096
        i, margin, fell = O.categorical_draw(w, u)
        assert not fell
        lo = C[i - 1] if i > 0 else F(0)
        assert lo <= F(u) * S < C[i]
        assert w_exact[i] > 0
        assert abs(margin - float(min(F(u) - lo / S, C[i] / S - F(u)))) < 1e-15


def test_categorical_draw_law_on_fine_grid():
    p = np.array([0.1, 0.0, 0.25, 0.05, 0.6])
    n = 1 << 16
    counts = np.zeros(5)
    for k in range(n):
        counts[O.categorical_draw(p, (k + 0.5) / n)[0]] += 1
    np.testing.assert_allclose(counts / n, p, atol=1.5 / n)


# ----------------------------------------------------------------------------
# Greedy rule
# ----------------------------------------------------------------------------

def test_argmax_first_brute_force_ties():
    vals = [-math.inf, -1.0, 0.0, -0.0, 2.0]
    for combo in itertools.product(vals, repeat=4):
        z = np.array(combo)
        best = max(combo)
        expect = min(i for i in range(4) if combo[i] == best)
        assert O.argmax_first(z) == expect


def test_greedy_rule_brute_force():
    """V=3, K=2, every logit pattern over {0, 1}, every draft: accept while argmax matches."""
    for bits in itertools.product([0.0, 1.0], repeat=9):
        zt = np.array(bits).reshape(3, 3)
        amax = [min(i for i in range(3) if zt[t][i] == zt[t].max()) for t in range(3)]
        for x in itertools.product(range(3), repeat=2):
            r = O.verify_sequence(zt, None, list(x), None, 0.0)
            n = 0
            while n < 2 and amax[n] == x[n]:
                n += 1
            assert r["n"] == n
            assert r["tokens"][:n] == list(x[:n])
            assert r["tokens"][n] == amax[n]
            assert all(v == -1 for v in r["tokens"][n + 1:])
            assert all(math.isnan(v) for v in r["p"])


def test_small_temperature_limit_equals_greedy():
    """T -> 0 with well separated maxima: the sampled rule reproduces the greedy rule."""
    rng = np.random.default_rng(11)
    V, K = 40, 5
    for trial in range(30):
        zt = rng.normal(0, 3, (K + 1, V))
        zd = zt[:K] + rng.normal(0, 0.3 if trial % 2 else 3.0, (K, V))
        for row in list(zt) + list(zd):
            # force a unique maximum at least 0.5 above the runner-up
            i = int(np.argmax(row))
            row[i] = np.sort(row)[-2] + 0.5
        # a T -> 0 drafter proposes the argmax of its own logits
        greedy_x = [int(np.argmax(zd[t])) for t in range(K)]
        g = O.verify_sequence(zt, None, greedy_x, None, 0.0)
        for u in (2.0 ** -24, 0.3, 0.999):  # u = 0 picks any weight > 0, however tiny
            s = O.verify_sequence(zt, zd, greedy_x, [u] * (K + 1), 1e-3)
            assert s["n"] == g["n"] and s["tokens"] == g["tokens"], (trial, u)


# ----------------------------------------------------------------------------
# Special cases
# ----------------------------------------------------------------------------

def test_identical_draft_accepts_everything():
    rng = np.random.default_rng(5)
    V, K = 50, 6
    zt = rng.normal(0, 2, (K + 1, V))
    zd = zt[:K].copy()
    for trial in range(20):
        x = rng.integers(0, V, K)
        u = rng.random(K + 1) * 0.999
        r = O.verify_sequence(zt, zd, x, u, 0.9)
        assert r["n"] == K
        np.testing.assert_allclose(r["p"], r["q"], rtol=1e-15)


def test_disjoint_supports_reject_first_and_sample_target():
    V, K = 20, 3
    p = np.array([F(i + 1, 55) for i in range(10)] + [F(0)] * 10, dtype=object)
    q = [F(0)] * 10 + dist([1] * 10)
    zt = np.stack([logits_of(p, 1.0)] * (K + 1))
    zd = np.stack([logits_of(q, 1.0)] * K)
    C = list(itertools.accumulate(p))
    n = 997
    for k in range(n):
        u_final = (k + 0.5) / n
        x = [10 + k % 10, 11, 12]
        r = O.verify_sequence(zt, zd, x, [0.0, 0.5, 0.5, u_final], 1.0)
        assert r["n"] == 0
        y = r["tokens"][0]
        assert (C[y - 1] if y else 0) <= F(u_final) < C[y]


def test_k_zero_is_plain_sampling():
    p = [F(1, 8), F(0), F(3, 8), F(1, 2)]
    zt = logits_of(p, 0.5, 3.0)[None, :]
    C = list(itertools.accumulate(p))
    for k in range(512):
        u = (k + 0.5) / 512
        r = O.verify_sequence(zt, np.zeros((0, 4)), [], [u], 0.5)
        assert r["n"] == 0 and len(r["tokens"]) == 1
        y = r["tokens"][0]
        assert (C[y - 1] if y else 0) <= F(u) < C[y]
        g = O.verify_sequence(zt, None, [], None, 0.0)
        assert g["tokens"] == [3]


def test_single_token_vocabulary():
    r = O.verify_sequence(np.zeros((4, 1)), np.ones((3, 1)), [0, 0, 0], [0.99, 0.5, 0.0, 0.7], 1.3)
    assert r["n"] == 3 and r["tokens"] == [0, 0, 0, 0]


# ----------------------------------------------------------------------------
# Data errors
# ----------------------------------------------------------------------------

def base_case():
    rng = np.random.default_rng(1)
    zt = rng.normal(0, 1, (4, 10)).astype(np.float32)
    zd = rng.normal(0, 1, (3, 10)).astype(np.float32)
    return zt, zd, [1, 2, 3], [0.5, 0.5, 0.5, 0.5]


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_errors(T):
    zt, zd, x, u = base_case()
    ok = O.verify_sequence(zt, zd, x, u, T)
    assert ok["status"] == 0

    def st(zt=zt, zd=zd, x=x, u=u, T=T):
        r = O.verify_sequence(zt, zd, x, u, T)
        if r["status"] & O.SEQ_ERROR_MASK:
            assert r["n"] == -1 and r["tokens"] == [-1] * 4
            assert all(math.isnan(v) for v in r["p"] + r["q"])
        return r["status"]

    assert st(x=[1, 10, 3]) == O.SEQ_ERR_TOKEN
    assert st(x=[-1, 2, 3]) == O.SEQ_ERR_TOKEN
    bad = zt.copy(); bad[2, 4] = np.nan
    assert st(zt=bad) == O.SEQ_ERR_LOGIT
    bad = zt.copy(); bad[3, :] = -np.inf
    assert st(zt=bad) == O.SEQ_ERR_LOGIT
    bad = zt.copy(); bad[1, 7] = np.inf
    assert st(zt=bad) == (O.SEQ_ERR_LOGIT if T else 0)
    bad = zt.copy(); bad[1, 0:9] = -np.inf
    assert st(zt=bad) == 0                                  # one finite logit is enough
    badd = zd.copy(); badd[0, 0] = np.nan
    assert st(zd=badd) == (O.SEQ_ERR_LOGIT if T else 0)     # greedy never reads draft rows
    assert st(u=[0.5, 1.0, 0.5, 0.5]) == (O.SEQ_ERR_UNIFORM if T else 0)
    assert st(u=[0.5, 0.5, 0.5, np.nan]) == (O.SEQ_ERR_UNIFORM if T else 0)
    assert st(u=[-0.25, 0.5, 0.5, 0.5]) == (O.SEQ_ERR_UNIFORM if T else 0)
    if T:
        assert st(T=-1.0) & O.SEQ_ERR_TEMPERATURE
        assert st(T=float("nan")) & O.SEQ_ERR_TEMPERATURE
        assert st(T=float("inf")) & O.SEQ_ERR_TEMPERATURE
        assert st(T=1e-39) & O.SEQ_ERR_TEMPERATURE
        # the smallest legal temperature: logits of order 1 scale past 2^30 ...
        assert st(T=2.0 ** -126) == O.SEQ_ERR_LOGIT
        # ... logits below 2^-97 in magnitude do not
        assert st(zt=zt * 2.0 ** -99, zd=zd * 2.0 ** -99, T=2.0 ** -126) == 0
    assert st(x=[1, 10, 3], zt=np.where(np.arange(10) == 3, np.nan, zt).astype(np.float32)) == \
        O.SEQ_ERR_TOKEN | O.SEQ_ERR_LOGIT


def test_zero_residual_mass_falls_back_to_target():
    """A rejection whose fp64 residual is all zero (only reachable by planting it)."""
    zt, zd, x, u = base_case()
    r = O.verify_sequence(zt, zd, x, [0.999999, 0.5, 0.5, 0.25], 1.0)
    t = r["n"]
    assert t < 3
    real = O.replacement_weights
    try:
        O.replacement_weights = lambda p, q, x: np.zeros_like(p)
        f = O.verify_sequence(zt, zd, x, [0.999999, 0.5, 0.5, 0.25], 1.0)
    finally:
        O.replacement_weights = real
    assert f["status"] == O.SEQ_NOTE_FALLBACK and f["n"] == t
    p = O.softmax_t(zt[t].astype(np.float64), 1.0)
    assert f["tokens"][t] == O.categorical_draw(p, 0.25)[0]


def test_scaled_range_rule():
    """A sampled row whose maximum m has |m| * fp32(log2(e)/T) >= 2^30 is a data error
    (outside the scaled range the library supports); greedy rows and rows just inside
    are not."""
    V = 6
    c2 = float(np.float32(1.4426950408889634))           # T = 1
    assert c2 * 2.0 ** 29 < 2.0 ** 30 <= c2 * 2.0 ** 30

    def rows(top):
        """Rows whose maximum is top (the draft's too); the other logits lie below it."""
        base = np.array([1.0, 0.5, -0.25, -1.0, 1.0, 0.75])
        zt = np.array([top * base] * 3, dtype=np.float32)
        zd = np.array([top * base[::-1]] * 2, dtype=np.float32)
        return zt, zd

    for top, T, err in ((2.0 ** 29, 1.0, 0), (2.0 ** 30, 1.0, O.SEQ_ERR_LOGIT),
                        (3.0e38, 1.0, O.SEQ_ERR_LOGIT),
                        (10.0, 1e-8, O.SEQ_ERR_LOGIT), (0.5, 1e-8, 0),
                        (10.0, 2e-38, O.SEQ_ERR_LOGIT), (1e-30, 2e-38, 0)):
        zt, zd = rows(top)
        r = O.verify_sequence(zt, zd, [1, 3], [0.5, 0.5, 0.5], T)
        assert r["status"] == err, (top, T, r["status"])
        g = O.verify_sequence(zt, None, [1, 3], None, 0.0)
        assert g["status"] == 0                                   # greedy rows: exempt
    # a logit of -2^127 that is not the maximum is no error (its weight is 0) ...
    zt = np.array([[0.0, -(2.0 ** 127), 1.0, -2.0, 0.5, 0.0]] * 3, dtype=np.float32)
    zd = np.array([[1.0, -(2.0 ** 127), 0.0, 2.0, -3.0, 0.5]] * 2, dtype=np.float32)
    assert O.verify_sequence(zt, zd, [1, 3], [0.5] * 3, 1.0)["status"] == 0
    # ... but a row entirely at -2^30 has its maximum out of range
    zt = np.full((3, V), -(2.0 ** 30), dtype=np.float32)
    zd = np.zeros((2, V), dtype=np.float32)
    assert O.verify_sequence(zt, zd, [1, 3], [0.5] * 3, 1.0)["status"] == O.SEQ_ERR_LOGIT


def test_accept_test_where_p_and_q_underflow():
    """r < p(x)/q(x) holds its real-number value where p(x) and q(x) each underflow
    fp64: p(x)/q(x) = e^0.5 > 1 accepts for every u; e^-0.5 accepts exactly for
    u < e^-0.5.  Where only p(x) underflows the ratio is ~e^-1000: only u = 0 accepts."""
    zt = np.array([[0.0, -1000.0, -1e4], [0.0, 0.0, 0.0]])
    zd = np.array([[0.0, -1000.5, -1e4]])
    for u in (0.0, 0.3, 0.999999):
        r = O.verify_sequence(zt, zd, [1], [u, 0.5], 1.0)
        assert r["n"] == 1 and r["tokens"][0] == 1
        assert r["p"][0] == 0.0 and r["q"][0] == 0.0
    zd2 = np.array([[0.0, -999.5, -1e4]])
    e = math.exp(-0.5)
    for u, acc in ((0.0, True), (e * (1 - 1e-9), True), (e * (1 + 1e-9), False), (0.9, False)):
        r = O.verify_sequence(zt, zd2, [1], [u, 0.5], 1.0)
        assert (r["n"] == 1) == acc, (u, r)
    zd3 = np.array([[0.0, 0.0, -1e4]])
    for u, acc in ((0.0, True), (2.0 ** -24, False), (0.5, False)):
        r = O.verify_sequence(zt, zd3, [1], [u, 0.5], 1.0)
        assert (r["n"] == 1) == acc, (u, r)
