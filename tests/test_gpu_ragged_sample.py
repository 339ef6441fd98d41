"""Parity of the ragged verify and the draft-side sampler (HIP path through the C ABI)
with the fp64 oracle, on MI355X.  Same bar as the dense verify: greedy and data errors
bit-exact, sampled draws identical except near-ties (under 1e-4 of draws), reported
probabilities within 1e-5 relative.
"""
import math
import os

import numpy as np
import pytest
import torch

import speculative_decoding_verification_03_amd as sv
from speculative_decoding_verification_03_amd import workloads as W
from oracle import spec_verify_oracle as O
from parity_util import (Tally, compare, host_uniforms, host_uniforms_packed, logits_to_host,
                         to_host)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(sv.lib_path), "libspecverify.so is not built"
    return torch.device("cuda:0")


def dense_case(dev, B, K, V, dtype, temps, seed, sigma=1.0, scale=2.0):
    g = torch.Generator(device=dev).manual_seed(seed)
    zt = scale * torch.randn((B, K + 1, V), generator=g, device=dev)
    zd = zt[:, :K] + sigma * torch.randn((B, K, V), generator=g, device=dev)
    T = torch.tensor(temps, dtype=torch.float32)
    inp = dict(target=zt.to(dtype).contiguous(), draft=zd.to(dtype).contiguous(),
               temperature=T.to(dev))
    inp["tokens"] = W._draft_tokens(inp["draft"], T, g)
    return inp


def per_sequence(out, cu, with_probs=True):
    """Packed outputs -> per-sequence lists (the layout compare() walks)."""
    B = len(cu) - 1
    res = dict(tokens=[], accept_len=out["accept_len"], status=out["status"], p=[], q=[])
    for b in range(B):
        c0, c1 = int(cu[b]), int(cu[b + 1])
        res["tokens"].append(out["tokens"][c0 + b:c1 + b + 1])
        res["p"].append(out["p"][c0:c1] if with_probs else [])
        res["q"].append(out["q"][c0:c1] if with_probs else [])
    if "draws" in out:
        res["draws"] = out["draws"]
    return res


def run_ragged(P, u):
    out = sv.spec_verify_ragged(P["target"], P["draft"], P["cu"], P["tokens"], u,
                                P["temperature"], P["K_max"])
    torch.cuda.synchronize()
    return to_host(out)


def oracle_ragged(P, u):
    return O.verify_ragged(logits_to_host(P["target"]), logits_to_host(P["draft"]),
                           P["cu"].cpu().numpy(), P["tokens"].cpu().numpy(), u.cpu().numpy(),
                           P["temperature"].cpu().numpy(), P["K_max"])


RAGGED = [
    # B, K_max, V, dtype, temperatures, K_b
    (9, 6, 1003, torch.float32, [1.0, 0.0, 0.5, 1.3, 0.0, 0.8, 1.0, 0.2, 2.0],
     [0, 1, 2, 3, 4, 5, 6, 0, 6]),
    (6, 8, 40000, torch.bfloat16, [1.0, 0.7, 0.0, 1.1, 0.4, 0.9], [8, 1, 3, 0, 5, 2]),
    (4, 5, 130001, torch.bfloat16, [0.6, 0.0, 1.0, 1.2], [5, 5, 1, 3]),
    (5, 3, 777, torch.bfloat16, [1.0, 0.0, 0.5, 1.0, 0.3], [0, 0, 0, 0, 0]),  # no drafts
]


@pytest.mark.parametrize("case", range(len(RAGGED)))
def test_ragged_parity(dev, case):
    B, KM, V, dt, temps, kb = RAGGED[case]
    say(f"ragged case {case}: B={B} K_max={KM} V={V} {dt} K_b={kb}")
    t = Tally()
    for rep in range(3):
        inp = dense_case(dev, B, KM, V, dt, temps, seed=500 + 10 * case + rep)
        P = W.pack_ragged(inp, kb)
        cu = P["cu"].cpu().numpy()
        uh = host_uniforms_packed(91 + case, 0, rep, cu, P["total"])
        np.testing.assert_array_equal(
            sv.sv_fill_uniforms_ragged(91 + case, 0, rep, P["cu"], P["total"], KM).cpu().numpy(), uh)
        u = torch.from_numpy(uh).to(dev)
        g = run_ragged(P, u)
        o = oracle_ragged(P, u)
        assert list(o["K"]) == kb
        t.merge(compare(per_sequence(g, cu), per_sequence(o, cu), range(B),
                        inp["temperature"].cpu()))
        # greedy entry point on the same packed target rows
        gg = sv.spec_verify_greedy_ragged(P["target"], P["cu"], P["tokens"], KM)
        torch.cuda.synchronize()
        gg = to_host(gg)
        og = O.verify_ragged(logits_to_host(P["target"]), None, cu, P["tokens"].cpu().numpy(),
                             None, np.zeros(B, dtype=np.float32), KM)
        c = compare(per_sequence(gg, cu, False), per_sequence(og, cu, False), range(B), None,
                    greedy_only=True)
        c.assert_ok(f"ragged {case} greedy")
    say("  ", t)
    t.assert_ok(f"ragged {case}")


def test_ragged_uniforms_match_dense_generator(dev):
    kb = [3, 0, 7, 1, 5]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(kb)]), dtype=torch.int32, device=dev)
    u = sv.sv_fill_uniforms_ragged(1234, 2, 9, cu, sum(kb), 7).cpu().numpy()
    d = sv.sv_fill_uniforms(1234, 2, 9, len(kb), 7).cpu().numpy()
    for b, k in enumerate(kb):
        c0 = int(cu[b])
        np.testing.assert_array_equal(u[c0 + b:c0 + b + k + 1], d[b, :k + 1])


def test_ragged_full_rows_equal_dense(dev):
    """K_b = K for every sequence: the packed call is the dense call, bit for bit."""
    B, K, V = 16, 8, 152064
    inp = W.make_inputs(4, step=3, device=dev, B=B)
    P = W.pack_ragged(inp, [K] * B)
    u = sv.sv_fill_uniforms(1004, 0, 3, B, K)
    a = to_host(sv.spec_verify(inp["target"], inp["draft"], inp["tokens"], u, inp["temperature"]))
    r = run_ragged(P, u.reshape(-1).contiguous())
    np.testing.assert_array_equal(r["tokens"], a["tokens"].reshape(-1))
    np.testing.assert_array_equal(r["accept_len"], a["accept_len"])
    np.testing.assert_array_equal(r["status"], a["status"])
    np.testing.assert_array_equal(r["p"], a["p"].reshape(-1))
    np.testing.assert_array_equal(r["q"], a["q"].reshape(-1))


def test_ragged_workload_sampled_sequences(dev):
    """The ragged benchmark workload (workload-4 rows, K_b uniform on 1..8), a sample of
    its sequences against the oracle, in the launch configuration of the full batch."""
    inp = W.make_inputs(4, step=0, device=dev)
    kb = W.draft_counts(inp["B"], inp["K"], 4000)
    P = W.pack_ragged(inp, kb)
    del inp
    cu = P["cu"].cpu().numpy()
    u = torch.from_numpy(host_uniforms_packed(1004, 0, 0, cu, P["total"])).to(dev)
    g = run_ragged(P, u)
    seqs = list(range(0, P["B"], 8))
    # the oracle on the sampled sequences only (reads only their slices)
    o = O.verify_ragged(logits_to_host(P["target"]), logits_to_host(P["draft"]), cu,
                        P["tokens"].cpu().numpy(), u.cpu().numpy(),
                        P["temperature"].cpu().numpy(), P["K_max"], seqs=seqs)
    t = compare(per_sequence(g, cu), per_sequence(o, cu), seqs, P["temperature"].cpu())
    say("  ragged workload:", t)
    t.assert_ok("ragged workload")
    assert (g["status"] & ~16 == 0).all()


@pytest.mark.parametrize("cu,bad", [
    ([0, 2, 5, 6], {1}),     # K_b above the bound 2
    ([0, 2, 4, 9], {2}),     # past the packed arrays
    ([-1, 2, 4, 6], {0}),    # negative start
])
def test_ragged_invalid_offsets_flagged(dev, cu, bad):
    B, KM, V, total = 3, 2, 300, 6
    g = torch.Generator(device=dev).manual_seed(77)
    target = torch.randn((total + B, V), generator=g, device=dev)
    draft = torch.randn((total, V), generator=g, device=dev)
    tokens = torch.randint(0, V, (total,), generator=g, device=dev, dtype=torch.int32)
    u = torch.rand((total + B,), generator=g, device=dev)
    T = torch.tensor([1.0, 0.0, 0.8], device=dev)
    cu_d = torch.tensor(cu, dtype=torch.int32, device=dev)
    out = to_host(sv.spec_verify_ragged(target, draft, cu_d, tokens, u, T, KM))
    orc = O.verify_ragged(target.cpu().numpy(), draft.cpu().numpy(), np.array(cu),
                          tokens.cpu().numpy(), u.cpu().numpy(), T.cpu().numpy(), KM)
    for b in range(B):
        if b in bad:
            assert out["status"][b] == sv.SV_SEQ_ERR_OFFSETS and out["accept_len"][b] == -1
    good = [b for b in range(B) if b not in bad]
    cuv = np.array(cu)
    t = compare(per_sequence(out, cuv), per_sequence(orc, cuv), good, T.cpu())
    t.assert_ok("valid sequences next to invalid offsets")


# ------------------------------------------------------------------------------------
# draft-side sampler
# ------------------------------------------------------------------------------------

def sample_as_verify(r):
    """sv_sample / O.sample results in the per-sequence layout of compare()."""
    B = len(r["tokens"])
    out = dict(tokens=[[int(v)] for v in r["tokens"]],
               accept_len=np.where(np.asarray(r["status"]) & ~16, -1, 0), status=r["status"],
               p=[[] for _ in range(B)], q=[[] for _ in range(B)])
    if "draws" in r:
        out["draws"] = r["draws"]
    return out


@pytest.mark.parametrize("B,V,dt", [(64, 152064, torch.bfloat16), (37, 1000, torch.float32),
                                    (20, 131073, torch.float32), (3, 1, torch.bfloat16),
                                    (7, 4096 * 1024, torch.bfloat16),    # longest one-workgroup row
                                    (2, 4096 * 1024 + 5, torch.bfloat16)])  # the multi-kernel path
def test_sample_parity(dev, B, V, dt):
    say(f"sampler B={B} V={V} {dt}")
    t = Tally()
    for rep in range(3):
        g = torch.Generator(device=dev).manual_seed(900 + rep + V)
        z = (3.0 * torch.randn((B, V), generator=g, device=dev)).to(dt)
        T = torch.rand((B,), generator=g, device=dev) * 1.5
        T[::5] = 0.0
        u = torch.from_numpy(host_uniforms(55, 1, rep, B, 0).reshape(B)).to(dev)
        r = to_host(sv.sv_sample(z, u, T))
        o = O.sample(logits_to_host(z), u.cpu().numpy(), T.cpu().numpy())
        t.merge(compare(sample_as_verify(r), sample_as_verify(o), range(B), T.cpu()))
        # the same computation as spec_verify with K = 0, bit for bit
        v = to_host(sv.spec_verify(z.reshape(B, 1, V), None, torch.empty((B, 0), dtype=torch.int32,
                                                                            device=dev),
                                   u.reshape(B, 1).contiguous(), T))
        np.testing.assert_array_equal(r["tokens"], v["tokens"][:, 0])
    say("  ", t)
    t.assert_ok("sampler")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_sample_ties_and_bad_values(dev, dt):
    """Greedy rows whose maximum is tied many times over (lowest index wins), rows with a
    NaN, +inf or -inf planted at the first, a middle or the last position (the scalar tail,
    V not a multiple of 8), and rows of -inf only: tokens and status equal the oracle's."""
    B, V = 48, 10007
    say(f"sampler ties and bad values {dt}")
    g = torch.Generator(device=dev).manual_seed(4242)
    z = torch.randint(-3, 2, (B, V), generator=g, device=dev).float()
    T = torch.rand((B,), generator=g, device=dev) + 0.25
    T[::2] = 0.0
    spots = [0, V // 2 + 3, V - 1]
    for j, pos in enumerate(spots):
        z[8 + j, pos] = float("nan")          # greedy
        z[9 + 2 * j, pos] = float("nan")      # sampled (odd rows)
        z[20 + 2 * j, pos] = float("inf")     # greedy: a valid maximum
        z[21 + 2 * j, pos] = float("inf")     # sampled: an error
        z[30 + 2 * j, pos] = 5.0              # greedy: a single maximum there
    z[40] = -float("inf")
    z[41] = -float("inf")
    z = z.to(dt).contiguous()
    u = torch.from_numpy(host_uniforms(77, 1, 0, B, 0).reshape(B)).to(dev)
    r = to_host(sv.sv_sample(z, u, T))
    o = O.sample(logits_to_host(z), u.cpu().numpy(), T.cpu().numpy())
    np.testing.assert_array_equal(r["status"], o["status"])
    np.testing.assert_array_equal(r["tokens"], o["tokens"])
    assert (np.asarray(r["status"])[[8, 9, 21, 40, 41]] != 0).all()
    assert r["tokens"][30] == 0 and r["tokens"][20] == 0 and r["tokens"][34] == V - 1


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_sample_far_maximum(dev, dt):
    """Rows whose maximum lies far above that of their first few thousand positions, at a low
    temperature: a cluster of near-equal peaks beyond them, at two heights, one that the
    sampler's lifted provisional reference covers and one that needs its second pass over
    the row; plus the greedy row of the same values.  Tokens and status equal the oracle's
    and every sampled token is one of the peaks."""
    V, n_u = 20007, 8
    say(f"sampler far maximum {dt}")
    if dt == torch.bfloat16:
        T0 = 0.1       # 900 / (log2(e) / T) = 62 logits: 84 and 204 lie past it
        peaks = [(84.0, 84.0, 83.5), (204.0, 204.0, 203.0)]
    else:
        T0 = 0.05      # 31 logits: 44 and 104 lie past it
        peaks = [(44.0, 43.95, 43.9), (104.0, 103.95, 103.98)]
    spots = [9000, 15001, V - 1]
    rng = np.random.default_rng(31337)
    rows, temps = [], []
    for hi in peaks:
        for t in [T0] * n_u + [0.0]:
            z = rng.standard_normal(V).astype(np.float32)
            z[spots] = hi
            rows.append(z)
            temps.append(t)
    B = len(rows)
    z = torch.from_numpy(np.stack(rows)).to(dev).to(dt).contiguous()
    T = torch.tensor(temps, dtype=torch.float32, device=dev)
    u = torch.from_numpy(host_uniforms(91, 1, 0, B, 0).reshape(B)).to(dev)
    r = to_host(sv.sv_sample(z, u, T))
    o = O.sample(logits_to_host(z), u.cpu().numpy(), T.cpu().numpy())
    t = compare(sample_as_verify(r), sample_as_verify(o), range(B), T.cpu())
    say("  ", t)
    t.assert_ok("sampler, far maximum")
    np.testing.assert_array_equal(r["status"], o["status"])
    assert (np.asarray(r["status"]) & ~16 == 0).all()
    assert set(np.asarray(r["tokens"]).tolist()) <= set(spots)
    greedy = np.asarray(temps) == 0.0
    assert (np.asarray(r["tokens"])[greedy] == spots[0]).all()


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_sample_row_shapes_near_the_limits(dev, dt):
    """Sampled rows at the edges of the sampler's one-read path, each equal to the oracle:
    a row that opens with 8192 -inf; a finite mask value (-1e30) among ordinary logits;
    values whose weights against the provisional reference each lie just under 2^900, enough
    of them that the row total passes it; a row maximum just inside and one just outside
    the scaled-range rule at T = 1e-6 (an error in the oracle and on the GPU)."""
    V, n_u = 20007, 6
    say(f"sampler rows near the limits {dt}")
    rng = np.random.default_rng(777)
    nfirst = 8192 if dt == torch.bfloat16 else 4096   # the values the provisional max reads
    rows, temps = [], []

    def add(z, t):
        for _ in range(n_u):
            rows.append(z.copy())
            temps.append(t)

    def rnd(v=V):
        return rng.standard_normal(v).astype(np.float32)

    def cast(z):   # the values the kernel will see
        return torch.from_numpy(z).to(dt).float().numpy()

    z = rnd()
    z[:8192] = -np.inf
    add(z, 0.8)
    z = rnd()
    z[rng.choice(V, 500, replace=False)] = -1e30
    add(z, 1.1)
    z = cast(rnd())
    r0 = float(z[:nfirst].max())

    def down(v):   # the next value below v > 0 in the row's type
        if dt == torch.float32:
            return float(np.nextafter(np.float32(v), np.float32(0)))
        b = torch.tensor([v], dtype=torch.bfloat16).view(torch.int16) - 1
        return float(b.view(torch.bfloat16).float())

    # a temperature at which some value of the row's type weighs 2^e, 895 <= e < 899.9,
    # against the provisional reference (the lifted maximum of the first values)
    for T in np.linspace(0.08, 0.12, 401).astype(np.float32):
        c2 = math.log2(math.e) / float(T)
        ref = r0 + float(np.float32(900.0 / c2))
        spike = float(cast(np.array([ref + 899.6 / c2], dtype=np.float32))[0])
        while (spike - ref) * c2 >= 899.9:
            spike = down(spike)
        e = (spike - ref) * c2
        if e >= 895.0:
            break
    assert e >= 895.0
    n = max(2, math.ceil(2.0 ** (900.3 - e)))
    z[np.linspace(9000, V - 1, n).astype(np.int64)] = spike
    add(z, float(T))
    z = rnd()
    z[13000] = 700.0     # 700 * log2(e) / 1e-6 < 2^30
    add(z, 1e-6)
    z = rnd()
    z[13000] = 800.0     # 800 * log2(e) / 1e-6 >= 2^30: an error
    add(z, 1e-6)
    B = len(rows)
    zt = torch.from_numpy(np.stack(rows)).to(dev).to(dt).contiguous()
    Tt = torch.tensor(temps, dtype=torch.float32, device=dev)
    u = torch.from_numpy(host_uniforms(92, 1, 0, B, 0).reshape(B)).to(dev)
    r = to_host(sv.sv_sample(zt, u, Tt))
    o = O.sample(logits_to_host(zt), u.cpu().numpy(), Tt.cpu().numpy())
    np.testing.assert_array_equal(r["status"], o["status"])
    t = compare(sample_as_verify(r), sample_as_verify(o), range(B), Tt.cpu())
    say("  ", t)
    t.assert_ok("sampler, rows near the limits")
    st = np.asarray(r["status"]) & ~16
    assert (st[:4 * n_u] == 0).all() and (st[4 * n_u:] != 0).all()
    assert (np.asarray(r["tokens"])[3 * n_u:4 * n_u] == 13000).all()


# ------------------------------------------------------------------------------------
# token trees (greedy) and the tree attention mask
# ------------------------------------------------------------------------------------

def run_tree(inp):
    out = sv.spec_verify_tree_greedy(inp["target"], inp["parents"], inp["tokens"])
    torch.cuda.synchronize()
    return to_host(out)


def oracle_tree(inp):
    return O.verify_tree_greedy(logits_to_host(inp["target"]), inp["parents"].cpu().numpy(),
                                inp["tokens"].cpu().numpy())


def assert_tree_equal(g, o, what):
    for k in ("tokens", "nodes", "accept_len", "status"):
        np.testing.assert_array_equal(g[k], o[k], err_msg=f"{what}: {k}")


def random_trees(dev, B, N, V, dt, seed, shape, agree=0.7, ties=False):
    rng = np.random.default_rng(seed)
    par = np.full((B, N), -1, dtype=np.int32)
    for b in range(B):
        for j in range(1, N):
            if shape == "chain":
                par[b, j] = j - 1
            elif shape == "star":
                par[b, j] = 0
            elif shape == "binary":
                par[b, j] = (j - 1) // 2
            else:
                par[b, j] = rng.integers(max(0, j - 6), j)
    g = torch.Generator(device=dev).manual_seed(seed)
    if ties:
        z = torch.randint(-2, 2, (B, N, V), generator=g, device=dev).float()
    else:
        z = 2.0 * torch.randn((B, N, V), generator=g, device=dev)
    z = z.to(dt).contiguous()
    amax = torch.argmax(z.float(), dim=-1).cpu().numpy()
    tok = np.where(rng.random((B, N)) < agree,
                   np.take_along_axis(amax, np.maximum(par, 0).astype(np.int64), axis=1),
                   rng.integers(0, V, (B, N)))
    tok[:, 0] = 0
    return dict(target=z, parents=torch.tensor(par, device=dev),
                tokens=torch.tensor(tok.astype(np.int32), device=dev))


TREES = [
    # B, N, V, dtype, shape, ties
    (8, 9, 1000, torch.float32, "chain", False),
    (8, 31, 1003, torch.bfloat16, "binary", True),
    (6, 64, 40000, torch.bfloat16, "random", False),
    (4, 200, 777, torch.float32, "random", True),
    (3, 1024, 300, torch.bfloat16, "random", True),   # the largest tree
    (5, 1, 5000, torch.float32, "star", False),       # root only
    (3, 17, 130001, torch.bfloat16, "star", False),
]


@pytest.mark.parametrize("case", range(len(TREES)))
def test_tree_parity(dev, case):
    B, N, V, dt, shape, ties = TREES[case]
    say(f"tree case {case}: B={B} N={N} V={V} {dt} {shape} ties={ties}")
    for rep in range(2):
        inp = random_trees(dev, B, N, V, dt, 300 + 10 * case + rep, shape, ties=ties)
        g = run_tree(inp)
        o = oracle_tree(inp)
        assert_tree_equal(g, o, f"tree {case}")
        say("   accept", g["accept_len"].tolist()[:8])
        m = sv.sv_tree_attention_mask(inp["parents"])
        torch.cuda.synchronize()
        m = to_host(m)
        om = O.tree_attention_mask(inp["parents"].cpu().numpy())
        for k in ("mask", "depth", "status"):
            np.testing.assert_array_equal(m[k], om[k], err_msg=f"tree mask {case}: {k}")


def test_tree_chain_equals_linear_greedy(dev):
    """A chain tree is the linear verify: spec_verify_greedy on the same rows."""
    B, K, V = 16, 8, 152064
    inp = W.make_inputs(4, step=5, device=dev, B=B)
    par = torch.tensor([[-1] + list(range(K))] * B, dtype=torch.int32, device=dev)
    tok = torch.cat([torch.zeros((B, 1), dtype=torch.int32, device=dev), inp["tokens"]], dim=1)
    g = run_tree(dict(target=inp["target"], parents=par, tokens=tok.contiguous()))
    lin = to_host(sv.spec_verify_greedy(inp["target"], inp["tokens"]))
    np.testing.assert_array_equal(g["tokens"], lin["tokens"])
    np.testing.assert_array_equal(g["accept_len"], lin["accept_len"])


def test_tree_errors_flagged(dev):
    B, N, V = 4, 6, 500
    inp = random_trees(dev, B, N, V, torch.float32, 9, "random")
    par = inp["parents"].clone()
    par[1, 3] = 3            # not an earlier node
    par[2, 0] = 0            # root with a parent
    tok = inp["tokens"].clone()
    tok[3, 2] = V            # token outside the vocabulary
    tgt = inp["target"].clone()
    tgt[0, 4, 7] = float("nan")
    bad = dict(target=tgt, parents=par, tokens=tok)
    assert_tree_equal(run_tree(bad), oracle_tree(bad), "tree errors")
    m = to_host(sv.sv_tree_attention_mask(par))
    om = O.tree_attention_mask(par.cpu().numpy())
    for k in ("mask", "depth", "status"):
        np.testing.assert_array_equal(m[k], om[k])


def test_tree_workload_full_size(dev):
    """The tree benchmark workload (64 trees of 64 nodes, V=152064 bf16) against the oracle."""
    inp = W.make_tree_inputs(device=dev)
    g = run_tree(inp)
    o = oracle_tree(inp)
    assert_tree_equal(g, o, "tree workload")
    say("   tree workload mean accept", float(g["accept_len"].mean()))
