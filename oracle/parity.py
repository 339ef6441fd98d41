"""Near-tie accounting of a comparison between the HIP path and the fp64 oracle.

TEST INFRASTRUCTURE ONLY (part of the oracle's side): used by tests/ and by the
cpu_baseline leg of bench.py, never by the product path.

A sampled sequence matches when accept length, tokens and status agree.  Otherwise the
first draw on which the two diverge (the earlier of the two accept lengths' tests, or
the final draw) is looked up in the oracle's draw list: its margin is |u - p/q| for a
ratio test, or the distance from u to the nearer edge of the chosen CDF cell for a
categorical draw.  Margin < 1e-5 counts as a near-tie (excused, counted); anything else
is a hard failure.  Near-ties must stay below 1e-4 of the draws the oracle consumed
(the tests it evaluated and its final draw, on sampled sequences).  Greedy sequences and
data errors must match bit for bit.  Reported probabilities p_t(x_t), q_t(x_t) must lie
within 1e-5 relative of the oracle's (1e-35 absolute below 1e-30).

Besides the mismatch count, a tally also counts every oracle draw whose margin is below
1e-5 (``within``), whether or not the two sides agreed on it: the share of draws that
lie that close to a ratio threshold or a CDF edge at all.
"""
import math

import numpy as np

NEAR_TIE = 1e-5
NEAR_TIE_BUDGET = 1e-4
PROB_RTOL = 1e-5
PROB_TINY = 1e-30
PROB_ATOL_TINY = 1e-35



class Tally:
    def __init__(self):
        self.seqs = 0
        self.sampled = 0
        self.draws = 0
        self.within = 0
        self.near_ties = 0
        self.hard = []
        self.prob_max_rel = 0.0
        self.prob_bad = []
        self.fallbacks = 0

    def merge(self, other):
        for k in ("seqs", "sampled", "draws", "within", "near_ties", "fallbacks"):
            setattr(self, k, getattr(self, k) + getattr(other, k))
        self.hard += other.hard
        self.prob_bad += other.prob_bad
        self.prob_max_rel = max(self.prob_max_rel, other.prob_max_rel)

    def assert_ok(self, what=""):
        assert not self.hard, f"{what}: hard mismatches {self.hard[:5]}"
        assert not self.prob_bad, f"{what}: probability mismatches {self.prob_bad[:5]}"
        if self.draws:
            assert self.near_ties <= NEAR_TIE_BUDGET * self.draws, \
                f"{what}: {self.near_ties} near-ties in {self.draws} draws"

    def as_dict(self):
        return dict(sequences=self.seqs, sampled=self.sampled, draws=self.draws,
                    near_ties=self.near_ties, within_1e_5=self.within, hard=len(self.hard),
                    prob_max_rel=self.prob_max_rel, fallbacks=self.fallbacks)

    def __str__(self):
        return (f"seqs={self.seqs} sampled={self.sampled} draws={self.draws} "
                f"near_ties={self.near_ties} within_1e-5={self.within} hard={len(self.hard)} "
                f"prob_max_rel={self.prob_max_rel:.2e} fallbacks={self.fallbacks}")


def compare(gpu, orc, seqs, temperature, greedy_only=False):
    """gpu, orc: dicts of numpy arrays (tokens, accept_len, status, and p, q unless greedy)."""
    t = Tally()
    for b in seqs:
        t.seqs += 1
        T = float(temperature[b]) if temperature is not None else 0.0
        g_tok, o_tok = list(gpu["tokens"][b]), list(orc["tokens"][b])
        g_n, o_n = int(gpu["accept_len"][b]), int(orc["accept_len"][b])
        g_st, o_st = int(gpu["status"][b]), int(orc["status"][b])
        sampled = (T != 0.0) and not greedy_only
        if o_st & 16:
            t.fallbacks += 1
        if not sampled or (o_st & ~16):
            if (g_tok, g_n, g_st) != (o_tok, o_n, o_st):
                t.hard.append(("exact", b, g_n, o_n, g_tok, o_tok, g_st, o_st))
            continue
        t.sampled += 1
        draws = orc["draws"][b]
        t.draws += len(draws)
        t.within += sum(1 for d in draws if d[2] < NEAR_TIE)
        if (g_tok, g_n) != (o_tok, o_n) or (g_st & ~16) != (o_st & ~16):
            if g_n != o_n:
                first = draws[min(g_n, o_n)]
            else:
                first = draws[-1]
            if first[2] < NEAR_TIE and (g_st & ~16) == (o_st & ~16):
                t.near_ties += 1
            else:
                t.hard.append(("sampled", b, g_n, o_n, g_tok, o_tok, first))
        # reported probabilities, every drafted position
        for key in ("p", "q"):
            gv = np.asarray(gpu[key][b], dtype=np.float64)
            ov = np.asarray(orc[key][b], dtype=np.float64)
            for k in range(len(ov)):
                o, g = ov[k], gv[k]
                if math.isnan(o) or math.isnan(g):
                    if not (math.isnan(o) and math.isnan(g)):
                        t.prob_bad.append((key, b, k, g, o))
                    continue
                if o >= PROB_TINY:
                    rel = abs(g - o) / o
                    t.prob_max_rel = max(t.prob_max_rel, rel)
                    if rel > PROB_RTOL:
                        t.prob_bad.append((key, b, k, g, o, rel))
                elif abs(g - o) > PROB_ATOL_TINY:
                    t.prob_bad.append((key, b, k, g, o))
    return t
