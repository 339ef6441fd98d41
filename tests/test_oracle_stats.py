"""Statistical pins of the oracle (Monte Carlo; fixed seeds, so deterministic).

* The exercise on the lesson page "Decodificação Especulativa e EAGLE"
  ("Exercícios", item 1) runs 10k samples through speculative decoding and
  through plain target sampling and asks for a total-variation distance below
  0.01.  10^5 samples are used here so that the multinomial noise (about 0.004)
  sits well inside that bound.
* Mean tokens per step on context-free synthetic rows against the per-position
  closed form E[n+1] = sum_j prod_{i<j} alpha_i, alpha_i = sum(min(p_i, q_i)).
Drafts are drawn with numpy's own categorical sampler, uniforms from the counter
generator contract.
"""
import numpy as np

from oracle import philox
from oracle import spec_verify_oracle as O


def make_rows(rng, V, K, noise, T):
    zt = rng.normal(0, 2, (K + 1, V))
    zd = zt[:K] + rng.normal(0, noise, (K, V))
    p = np.stack([O.softmax_t(r, T) for r in zt])
    q = np.stack([O.softmax_t(r, T) for r in zd])
    return zt, zd, p, q


def run(zt, zd, q, T, n, seed, rng):
    K = zd.shape[0]
    out = []
    for s in range(n):
        x = [int(rng.choice(len(q[t]), p=q[t])) for t in range(K)]
        u = [philox.uniform(seed, 0, s, 0, t) for t in range(K + 1)]
        out.append(O.verify_sequence(zt, zd, x, u, T))
    return out


def test_first_token_total_variation_against_plain_sampling():
    rng = np.random.default_rng(2024)
    V, K, T = 5, 3, 0.8
    zt, zd, p, q = make_rows(rng, V, K, 1.5, T)
    n = 100_000
    res = run(zt, zd, q, T, n, 77, rng)
    spec = np.bincount([r["tokens"][0] for r in res], minlength=V) / n
    plain = np.bincount(rng.choice(V, size=n, p=p[0]), minlength=V) / n
    assert 0.5 * np.abs(spec - plain).sum() < 0.01
    assert 0.5 * np.abs(spec - p[0]).sum() < 0.01
    # joint law of the first two positions, completing a 1-token step with a target draw
    joint = np.zeros((V, V))
    for r in res:
        a = r["tokens"][0]
        b = r["tokens"][1] if r["n"] >= 1 else int(rng.choice(V, p=p[1]))
        joint[a, b] += 1
    expect = np.outer(p[0], p[1]) * n
    chi2 = ((joint - expect) ** 2 / expect).sum()
    assert chi2 < 52.6  # chi-square with 24 dof, p = 0.001


def test_mean_tokens_per_step_matches_closed_form():
    rng = np.random.default_rng(99)
    V, K, T = 1000, 4, 1.0
    zt, zd, p, q = make_rows(rng, V, K, 0.5, T)
    alphas = [O.acceptance_rate(p[t], q[t]) for t in range(K)]
    expect = O.expected_tokens_general(alphas)
    n = 3000
    lens = np.array([r["n"] + 1 for r in run(zt, zd, q, T, n, 5, rng)], dtype=float)
    se = lens.std() / np.sqrt(n)
    assert abs(lens.mean() - expect) < 4 * se, (lens.mean(), expect, se)
