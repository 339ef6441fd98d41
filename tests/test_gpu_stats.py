"""Statistical checks of the HIP verify path itself, independent of the oracle.

The guarantee of speculative sampling ("A Regra de Exatidão" on the lesson page
"Decodificação Especulativa e EAGLE"): every emitted token is distributed as the target's
temperature softmax p, whatever the draft.  The page's exercise ("Exercícios", item 1)
asks for a total-variation distance below 0.01 between speculative and plain sampling.
Here 10^5 sequences with fixed context-free rows go through one spec_verify call each
test, with Pearson's chi-square test of the emitted tokens against p at level 1e-4 (and
the exercise's bound where V is small enough for 10^5 draws to meet it; the multinomial
noise is then about 0.004).  The mean accept length is
checked against the closed form E[n] = sum_{j=1..K} prod_{i<j} alpha_i, alpha_i =
sum_v min(p_i(v), q_i(v)) (for rows that do not depend on context, P(n >= j) is the
product of the first j acceptance rates), within 5 standard errors.  The draft-side sampler's draws are tested against softmax(z / T) the
same way.  Fixed seeds, so the outcome is deterministic.
"""
import os

import numpy as np
import pytest
import torch

import speculative_decoding_verification_03_amd as sv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(sv.lib_path), "libspecverify.so is not built"
    return torch.device("cuda:0")


def chi2_ok(counts, probs, alpha=1e-4):
    """Pearson's goodness of fit of counts to probs at level alpha (bins expecting fewer
    than 5 draws are pooled)."""
    from scipy.stats import chi2
    n = counts.sum()
    e = probs * n
    big = e >= 5
    o = np.append(counts[big], counts[~big].sum())
    e = np.append(e[big], e[~big].sum())
    if e[-1] < 5:
        o, e = o[:-1], e[:-1]
    stat = ((o - e) ** 2 / e).sum()
    return stat, chi2.ppf(1 - alpha, len(e) - 1)


def softmax(z, T):
    w = np.exp((z - z.max()) / T)
    return w / w.sum()


@pytest.mark.parametrize("V,K,T,noise,seed", [(5, 3, 0.8, 1.5, 2024), (40, 4, 1.0, 0.7, 7),
                                              (7, 2, 0.3, 2.0, 31)])
def test_emitted_tokens_follow_target(dev, V, K, T, noise, seed):
    print(f"stats V={V} K={K} T={T} noise={noise}", flush=True)
    rng = np.random.default_rng(seed)
    zt = rng.normal(0, 2, (K + 1, V)).astype(np.float32)
    zd = (zt[:K] + rng.normal(0, noise, (K, V))).astype(np.float32)
    p = np.stack([softmax(r.astype(np.float64), T) for r in zt])
    q = np.stack([softmax(r.astype(np.float64), T) for r in zd])
    B = 100_000
    # drafts x_t ~ q_t, independently per sequence
    x = np.stack([rng.choice(V, size=B, p=q[t]) for t in range(K)], axis=1).astype(np.int32)
    tgt = torch.from_numpy(zt).to(dev).unsqueeze(0).expand(B, K + 1, V).contiguous()
    drf = torch.from_numpy(zd).to(dev).unsqueeze(0).expand(B, K, V).contiguous()
    tok = torch.from_numpy(x).to(dev)
    temp = torch.full((B,), T, dtype=torch.float32, device=dev)
    u = sv.sv_fill_uniforms(seed, 0, 0, B, K)
    r = sv.spec_verify(tgt, drf, tok, u, temp)
    torch.cuda.synchronize()
    n = r["accept_len"].cpu().numpy()
    tokens = r["tokens"].cpu().numpy()
    status = r["status"].cpu().numpy()
    assert (status == 0).all()
    assert ((n >= 0) & (n <= K)).all()
    # the first emitted token ~ p_0
    f0 = np.bincount(tokens[:, 0], minlength=V) / B
    tv0 = 0.5 * np.abs(f0 - p[0]).sum()
    # the second emitted token, over sequences that emitted a draft at position 0, ~ p_1
    m = n >= 1
    f1 = np.bincount(tokens[m, 1], minlength=V) / m.sum()
    tv1 = 0.5 * np.abs(f1 - p[1]).sum()
    # accepted drafts: closed form of E[n]
    alpha = np.minimum(p[:K], q).sum(axis=1)
    en = sum(np.prod(alpha[:j]) for j in range(1, K + 1))
    se = n.std() / np.sqrt(B)
    print(f"   tv0 {tv0:.4f} tv1 {tv1:.4f} (over {m.sum()}) mean n {n.mean():.4f} "
          f"closed form {en:.4f} se {se:.4f}", flush=True)
    c0, lim0 = chi2_ok(np.bincount(tokens[:, 0], minlength=V), p[0])
    c1, lim1 = chi2_ok(np.bincount(tokens[m, 1], minlength=V), p[1])
    print(f"   chi2 {c0:.1f} (limit {lim0:.1f}), {c1:.1f} (limit {lim1:.1f})", flush=True)
    assert c0 < lim0 and c1 < lim1
    if V <= 10:  # the exercise's criterion, where 10^5 draws put the noise well below it
        assert tv0 < 0.01 and tv1 < 0.02
    assert abs(n.mean() - en) < 5 * se
    # positions past the emitted tokens are padding
    k = np.arange(K + 1)[None, :]
    assert (tokens[k > n[:, None]] == -1).all()


@pytest.mark.parametrize("V,T,dt,seed", [(40, 0.9, torch.float32, 5), (300, 1.3, torch.bfloat16, 6)])
def test_sampler_draws_follow_softmax(dev, V, T, dt, seed):
    """sv_sample over 10^5 copies of one row: the draws fit softmax(z / T) of the row's
    logits as stored (bf16 values for bf16 rows)."""
    print(f"sampler stats V={V} T={T} {dt}", flush=True)
    rng = np.random.default_rng(seed)
    z = torch.from_numpy(rng.normal(0, 2, V).astype(np.float32)).to(dt)
    p = softmax(z.float().numpy().astype(np.float64), T)
    B = 100_000
    zz = z.to(dev).unsqueeze(0).expand(B, V).contiguous()
    temp = torch.full((B,), T, dtype=torch.float32, device=dev)
    u = sv.sv_fill_uniforms(seed, 1, 0, B, 0).reshape(B).contiguous()
    r = sv.sv_sample(zz, u, temp)
    torch.cuda.synchronize()
    assert (r["status"].cpu().numpy() == 0).all()
    c, lim = chi2_ok(np.bincount(r["tokens"].cpu().numpy(), minlength=V), p)
    print(f"   chi2 {c:.1f} (limit {lim:.1f})", flush=True)
    assert c < lim
