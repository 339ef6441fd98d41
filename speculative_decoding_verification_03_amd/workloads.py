"""Seeded synthetic inputs of the verify step (shared by tests and the benchmark).

Holds none of the verify arithmetic: it draws logits, temperatures and draft tokens.
Draft tokens stand in for a draft model: for T > 0 they are drawn from
q = softmax(zd / T) with the Gumbel-max trick (argmax(zd / T + G), G standard Gumbel),
for T == 0 they are argmax(zd), as a greedy drafter would propose.  The verify rule
assumes x ~ q ("O Conceito", step 1, on the lesson page "Decodificação Especulativa e
EAGLE").  Uniforms are not drawn here: they come from the counter generator.

Workloads (V = vocabulary size, K = drafted tokens, B = sequences):
  1  B=1,    K=4,  V=1000,   fp32  zt ~ N(0, 2^2), zd = zt + N(0, 0.5^2), T = 1
  2  B=8,    K=4,  V=32000,  fp32  zt ~ N(0, 3^2), zd = zt + N(0, 1), T = 1 (and greedy)
  3  B=64,   K=5,  V=128256, bf16  zt ~ N(0, 3^2) plus +8 at 16 random indices per target
                                   row, zd = zt + N(0, sigma^2), sigma = 0.4219 (mean
                                   alpha ~ 0.8), T = 0.7
  4  B=256,  K=8,  V=152064, bf16  zt = N(0, 3^2) - 1.1 * ln(rank), rank a random
                                   permutation of 1..V per sequence (Zipf(1.1) offsets);
                                   zd = zt + N(0, sigma_b^2), sigma_b in {0.3, 1, 3};
                                   T_b ~ U[0, 1.2] with exactly B/4 sequences at T = 0
  5  B=1024, K=10, V=262144, bf16  zt ~ N(0, 3^2), T = 1; four equal groups: sigma for
                                   alpha ~ 0.5 / 0.8 / 0.95 (1.3396 / 0.4980 / 0.1232),
                                   and an adversarial group zd = zt + N(0, 1) + 30 on the
                                   64 smallest target logits of each row (q sits where
                                   p is tiny, so the first draft is rejected)
The sigma values come from the oracle-side calibration script (oracle/calibrate_sigma.py).

Ragged batches (adaptive verification, a number of drafts K_b per sequence) are packed
from a dense batch: sequence b keeps its first K_b draft rows and K_b + 1 target rows.
The ragged workload draws K_b uniformly from {1, ..., K} on workload 4's rows.

Token trees (greedy tree verification): B trees of N nodes laid out level by level
(TREE_LEVELS nodes per level, 64 nodes, depth 8), each node's parent drawn uniformly
from the level above; target rows follow workload 4's recipe (Zipf(1.1)-offset
N(0, 3^2)); a node's token is the argmax of its parent's row with probability 0.75 (a
drafter that agrees with the target), else uniform on the vocabulary.
"""
import math

import torch

WORKLOADS = {
    1: dict(B=1, K=4, V=1000, dtype=torch.float32),
    2: dict(B=8, K=4, V=32000, dtype=torch.float32),
    3: dict(B=64, K=5, V=128256, dtype=torch.bfloat16),
    4: dict(B=256, K=8, V=152064, dtype=torch.bfloat16),
    5: dict(B=1024, K=10, V=262144, dtype=torch.bfloat16),
}

SIGMA_CFG3 = 0.4219
SIGMA_CFG4 = (0.3, 1.0, 3.0)
SIGMA_CFG5 = (1.3396, 0.4980, 0.1232)  # alpha ~ 0.5, 0.8, 0.95


def describe(cfg):
    c = WORKLOADS[cfg]
    return f"B={c['B']} K={c['K']} V={c['V']} {'bf16' if c['dtype'] == torch.bfloat16 else 'fp32'}"


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _draft_tokens(zd, T, g):
    """Draft tokens: Gumbel-max draws from softmax(zd / T) rows, argmax where T == 0."""
    B, K, V = zd.shape
    out = torch.empty((B, K), dtype=torch.int32, device=zd.device)
    for b in range(B):
        z = zd[b].float()
        t = float(T[b])
        if t == 0.0:
            out[b] = torch.argmax(z, dim=-1).to(torch.int32)
        else:
            u = torch.rand(z.shape, generator=g, device=z.device, dtype=torch.float64)
            gumbel = -torch.log(-torch.log(u.clamp_min(1e-300)))
            out[b] = torch.argmax(z.double() / t + gumbel, dim=-1).to(torch.int32)
    return out


def make_inputs(cfg, step=0, device="cuda", B=None, seed=None):
    """Inputs of workload `cfg` for one step.

    Returns dict(target [B][K+1][V], draft [B][K][V] (cfg dtype), tokens [B][K] int32,
    temperature [B] fp32, cfg, B, K, V).  B may be lowered for smaller test cases; the
    first B sequences then follow the same recipe.
    """
    c = WORKLOADS[cfg]
    Bf, K, V, dt = c["B"], c["K"], c["V"], c["dtype"]
    B = Bf if B is None else int(B)
    seed = (1000 + cfg) * 1_000_003 + step if seed is None else seed
    g = _gen(device, seed)
    target = torch.empty((B, K + 1, V), dtype=dt, device=device)
    draft = torch.empty((B, K, V), dtype=dt, device=device)
    T = torch.empty((B,), dtype=torch.float32)
    sig = torch.empty((B,), dtype=torch.float64)
    gh = torch.Generator().manual_seed(int(seed) + 17)  # host-side choices
    if cfg == 1:
        T.fill_(1.0)
    elif cfg == 2:
        T.fill_(1.0)
    elif cfg == 3:
        T.fill_(0.7)
    elif cfg == 4:
        T.copy_(torch.rand((B,), generator=gh) * 1.2)
        T[torch.randperm(B, generator=gh)[: B // 4]] = 0.0
        sig.copy_(torch.tensor(SIGMA_CFG4, dtype=torch.float64)[torch.randint(0, 3, (B,), generator=gh)])
    elif cfg == 5:
        T.fill_(1.0)
    # per-sequence generation keeps fp32 temporaries small at the large workloads
    for b in range(B):
        if cfg == 1:
            zt = 2.0 * torch.randn((K + 1, V), generator=g, device=device)
            zd = zt[:K] + 0.5 * torch.randn((K, V), generator=g, device=device)
        elif cfg == 2:
            zt = 3.0 * torch.randn((K + 1, V), generator=g, device=device)
            zd = zt[:K] + torch.randn((K, V), generator=g, device=device)
        elif cfg == 3:
            zt = 3.0 * torch.randn((K + 1, V), generator=g, device=device)
            peaks = torch.rand((K + 1, V), generator=g, device=device).argsort(dim=-1)[:, :16]
            zt.scatter_add_(1, peaks, torch.full((K + 1, 16), 8.0, device=device))
            zd = zt[:K] + SIGMA_CFG3 * torch.randn((K, V), generator=g, device=device)
        elif cfg == 4:
            rank = torch.randperm(V, generator=g, device=device).to(torch.float32) + 1.0
            zt = 3.0 * torch.randn((K + 1, V), generator=g, device=device) - 1.1 * torch.log(rank)
            zd = zt[:K] + float(sig[b]) * torch.randn((K, V), generator=g, device=device)
        elif cfg == 5:
            zt = 3.0 * torch.randn((K + 1, V), generator=g, device=device)
            group = (4 * b) // B
            if group < 3:
                zd = zt[:K] + SIGMA_CFG5[group] * torch.randn((K, V), generator=g, device=device)
            else:
                zd = zt[:K] + torch.randn((K, V), generator=g, device=device)
                low = torch.topk(zt[:K], 64, dim=-1, largest=False).indices
                zd.scatter_add_(1, low, torch.full((K, 64), 30.0, device=device))
        else:
            raise ValueError(f"unknown workload {cfg}")
        target[b] = zt.to(dt)
        draft[b] = zd.to(dt)
    tokens = _draft_tokens(draft, T, g)
    return dict(target=target, draft=draft, tokens=tokens, temperature=T.to(device),
                cfg=cfg, B=B, K=K, V=V)


def draft_counts(B, K, seed, kmin=1):
    """K_b for each sequence, uniform on {kmin, ..., K} (host generator, seeded)."""
    gh = torch.Generator().manual_seed(int(seed) + 29)
    return torch.randint(kmin, K + 1, (B,), generator=gh).tolist()


def pack_ragged(inp, kb):
    """Packed inputs from dense ones: kb[b] <= K drafts kept for sequence b.

    Returns dict(target [total+B][V], draft [total][V], tokens [total] int32,
    cu [B+1] int32 (device), kb (list), temperature [B], K_max, total, B, V).
    """
    B, K1, V = inp["target"].shape
    dev = inp["target"].device
    cu = [0]
    for k in kb:
        cu.append(cu[-1] + int(k))
    total = cu[-1]
    trow = torch.tensor([b * K1 + t for b in range(B) for t in range(kb[b] + 1)], device=dev)
    drow = torch.tensor([b * (K1 - 1) + t for b in range(B) for t in range(kb[b])],
                        dtype=torch.int64, device=dev)
    target = inp["target"].reshape(B * K1, V).index_select(0, trow).contiguous()
    draft = inp["draft"].reshape(B * (K1 - 1), V).index_select(0, drow).contiguous()
    tokens = inp["tokens"].reshape(-1).index_select(0, drow).contiguous()
    return dict(target=target, draft=draft, tokens=tokens,
                cu=torch.tensor(cu, dtype=torch.int32, device=dev), kb=list(kb),
                temperature=inp["temperature"], K_max=K1 - 1, total=total, B=B, V=V)


TREE_LEVELS = (1, 4, 8, 12, 12, 12, 8, 4, 3)


def make_tree_inputs(B=64, V=152064, dtype=torch.bfloat16, levels=TREE_LEVELS, step=0,
                     device="cuda", seed=None, agree=0.75):
    """Tree inputs: dict(target [B][N][V], parents [B][N] int32, tokens [B][N] int32)."""
    N = sum(levels)
    seed = 7_000_003 + 131 * step if seed is None else seed
    g = _gen(device, seed)
    gh = torch.Generator().manual_seed(int(seed) + 5)
    parents = torch.empty((B, N), dtype=torch.int32)
    for b in range(B):
        parents[b, 0] = -1
        start, prev = 1, (0, 1)
        for n in levels[1:]:
            parents[b, start:start + n] = torch.randint(prev[0], prev[1], (n,), generator=gh,
                                                        dtype=torch.int32)
            prev = (start, start + n)
            start += n
    target = torch.empty((B, N, V), dtype=dtype, device=device)
    for b in range(B):
        rank = torch.randperm(V, generator=g, device=device).to(torch.float32) + 1.0
        zt = 3.0 * torch.randn((N, V), generator=g, device=device) - 1.1 * torch.log(rank)
        target[b] = zt.to(dtype)
    amax = torch.stack([torch.argmax(target[b].float(), dim=-1) for b in range(B)]).cpu()
    agree_mask = torch.rand((B, N), generator=gh) < agree
    rand_tok = torch.randint(0, V, (B, N), generator=gh)
    par = parents.clamp_min(0).long()
    tokens = torch.where(agree_mask, torch.gather(amax, 1, par), rand_tok).to(torch.int32)
    tokens[:, 0] = 0
    return dict(target=target, parents=parents.to(device), tokens=tokens.to(device), B=B, N=N,
                V=V)


def logit_bytes(B, K, V, dtype, temperature):
    """Algorithmic pass-1 bytes: target rows of every sequence, draft rows of sampled ones."""
    e = 2 if dtype == torch.bfloat16 else 4
    sampled = int((temperature != 0).sum())
    return e * V * (B * (K + 1) + sampled * K)


def ragged_logit_bytes(kb, V, dtype, temperature):
    """Algorithmic pass-1 bytes of a ragged batch."""
    e = 2 if dtype == torch.bfloat16 else 4
    T = temperature.cpu()
    return e * V * sum(k + 1 + (k if float(T[b]) != 0.0 else 0) for b, k in enumerate(kb))


def expected_draw_bytes(B, K, V, dtype):
    """Upper bound of pass-2 bytes: one row pair per sequence."""
    e = 2 if dtype == torch.bfloat16 else 4
    return e * V * 2 * B


if __name__ == "__main__":
    for k in WORKLOADS:
        print(k, describe(k), f"{math.prod((WORKLOADS[k]['B'], WORKLOADS[k]['K'] + 1, WORKLOADS[k]['V']))} target logits")
