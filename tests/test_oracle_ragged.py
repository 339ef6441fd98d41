"""Pins of the oracle's ragged verify and its plain sampler.

* verify_ragged: a packed batch with a different K_b per sequence must give, for every
  sequence, exactly what the dense verify (pinned by enumeration and closed forms in
  test_oracle_exact) gives for that sequence in a batch of its own K.  Sequences are
  packed from several dense batches of different K in shuffled order, so a wrong
  offset, a swapped target/draft base or a misplaced uniform or output slot changes a
  result.  Invalid offsets are flagged without disturbing the other sequences.
* sample: the categorical draw from softmax(z / T) equals numpy's
  searchsorted(cumsum(w), u * sum(w), side="right") (a library routine, on the exact
  fp64 weights of the definition), and numpy's first-occurrence argmax at T = 0.
"""
import numpy as np
import pytest

from oracle import spec_verify_oracle as O


def dense_batch(rng, B, K, V, sigma=0.7):
    zt = rng.normal(0.0, 2.0, (B, K + 1, V))
    zd = zt[:, :K] + rng.normal(0.0, sigma, (B, K, V))
    T = rng.choice([0.0, 0.5, 1.0, 1.7], size=B).astype(np.float32)
    # drafts from q (argmax on greedy rows), as the method assumes
    x = np.zeros((B, K), dtype=np.int64)
    for b in range(B):
        for t in range(K):
            if T[b] == 0.0:
                x[b, t] = int(np.argmax(zd[b, t]))
            else:
                q = np.exp((zd[b, t] - zd[b, t].max()) / T[b])
                x[b, t] = int(rng.choice(V, p=q / q.sum()))
    u = (rng.integers(0, 2 ** 24, (B, K + 1)) * 2.0 ** -24).astype(np.float32)
    return dict(zt=zt.astype(np.float32), zd=zd.astype(np.float32), x=x, u=u, T=T, K=K)


def pack(parts, order):
    """order: list of (part index, sequence index); returns the packed arrays."""
    V = parts[0]["zt"].shape[-1]
    cu = [0]
    tgt, drf, tok, uni, T = [], [], [], [], []
    for (i, b) in order:
        d = parts[i]
        K = d["K"]
        tgt.append(d["zt"][b])
        drf.append(d["zd"][b].reshape(K, V))
        tok.extend(int(v) for v in d["x"][b])
        uni.extend(float(v) for v in d["u"][b])
        T.append(d["T"][b])
        cu.append(cu[-1] + K)
    return dict(target=np.concatenate(tgt), draft=np.concatenate(drf),
                cu=np.array(cu, dtype=np.int32), tokens=np.array(tok, dtype=np.int64),
                uniforms=np.array(uni, dtype=np.float32), T=np.array(T, dtype=np.float32))


def test_ragged_equals_dense_per_sequence():
    rng = np.random.default_rng(11)
    V = 37
    parts = [dense_batch(rng, 4, K, V) for K in (0, 1, 3, 5)]
    dense = [O.verify(d["zt"], d["zd"], d["x"], d["u"], d["T"]) for d in parts]
    order = [(i, b) for i in range(4) for b in range(4)]
    rng.shuffle(order)
    P = pack(parts, order)
    r = O.verify_ragged(P["target"], P["draft"], P["cu"], P["tokens"], P["uniforms"], P["T"], 5)
    cu = P["cu"]
    for s, (i, b) in enumerate(order):
        want = dense[i]
        K = parts[i]["K"]
        c0 = cu[s]
        assert r["K"][s] == K
        assert r["accept_len"][s] == want["accept_len"][b]
        assert r["status"][s] == want["status"][b]
        assert list(r["tokens"][c0 + s:c0 + s + K + 1]) == list(want["tokens"][b])
        np.testing.assert_array_equal(r["p"][c0:c0 + K], want["p"][b])
        np.testing.assert_array_equal(r["q"][c0:c0 + K], want["q"][b])
        assert r["draws"][s] == want["draws"][b]
    # every output slot belongs to exactly one sequence and was written
    assert (r["tokens"] != -1).sum() == sum(int(r["accept_len"][s]) + 1 for s in range(len(order)))


def test_ragged_uniform_slots_drive_the_right_tests():
    # one sequence with K_b = 2 whose first test is decided by its own first uniform:
    # p(x_0)/q(x_0) = 0.5, so u = 0.25 accepts and u = 0.75 rejects
    V = 2
    zt = np.log(np.array([[0.25, 0.75], [0.5, 0.5], [0.5, 0.5]]))
    zd = np.log(np.array([[0.5, 0.5], [0.5, 0.5]]))
    for u0, n_first in ((0.25, None), (0.75, 0)):
        # a zero-draft sequence before it shifts every slot of the second one by one
        target = np.concatenate([np.zeros((1, V)), zt]).astype(np.float32)
        P = dict(cu=np.array([0, 0, 2], dtype=np.int32), tokens=np.array([0, 0]),
                 uniforms=np.array([0.3, u0, 0.1, 0.9], dtype=np.float32),
                 T=np.array([1.0, 1.0], dtype=np.float32))
        r = O.verify_ragged(target, zd.astype(np.float32), P["cu"], P["tokens"], P["uniforms"],
                            P["T"], 2)
        if n_first is None:
            assert r["accept_len"][1] >= 1
        else:
            assert r["accept_len"][1] == 0
            # the residual (p - q)+ puts all mass on token 1
            assert r["tokens"][1] == 1 and list(r["tokens"][2:4]) == [-1, -1]
        # K_b = 0 sequence: plain draw from softmax(0, 0) with u = 0.3 -> token 0
        assert r["tokens"][0] == 0 and r["accept_len"][0] == 0


@pytest.mark.parametrize("cu,bad", [
    ([0, 2, 1, 3], {1}),           # decreasing pair
    ([0, 2, 5, 6], {1}),           # K_b above the bound 2
    ([0, 2, 4, 9], {2}),           # past total
    ([-1, 2, 4, 6], {0}),          # negative start
])
def test_ragged_invalid_offsets_are_flagged(cu, bad):
    rng = np.random.default_rng(5)
    V, total, B = 11, 6, 3
    target = rng.normal(size=(total + B, V)).astype(np.float32)
    draft = rng.normal(size=(total, V)).astype(np.float32)
    tokens = rng.integers(0, V, total)
    u = (rng.integers(0, 2 ** 24, total + B) * 2.0 ** -24).astype(np.float32)
    T = np.array([1.0, 0.0, 0.8], dtype=np.float32)
    r = O.verify_ragged(target, draft, np.array(cu, dtype=np.int32), tokens, u, T, 2)
    for b in range(B):
        if b in bad:
            assert r["status"][b] == O.SEQ_ERR_OFFSETS and r["accept_len"][b] == -1
        else:
            assert r["status"][b] & O.SEQ_ERROR_MASK == 0 and r["accept_len"][b] >= 0


@pytest.mark.parametrize("T", [0.35, 1.0, 2.5])
def test_sample_is_inverse_cdf_of_the_temperature_softmax(T):
    rng = np.random.default_rng(int(T * 100))
    B, V = 64, 257
    z = rng.normal(0.0, 3.0, (B, V)).astype(np.float32)
    u = (rng.integers(0, 2 ** 24, B) * 2.0 ** -24).astype(np.float32)
    r = O.sample(z, u, np.full(B, T, dtype=np.float32))
    for b in range(B):
        w = np.exp((z[b].astype(np.float64) - z[b].max()) / np.float64(np.float32(T)))
        c = np.cumsum(w)
        want = int(np.searchsorted(c, float(u[b]) * c[-1], side="right"))
        assert r["tokens"][b] == want
        assert r["status"][b] == 0


def test_sample_greedy_is_first_argmax():
    rng = np.random.default_rng(3)
    z = rng.integers(-3, 3, (50, 9)).astype(np.float32)  # many ties
    r = O.sample(z, np.zeros(50, dtype=np.float32), np.zeros(50, dtype=np.float32))
    assert list(r["tokens"]) == [int(np.argmax(row)) for row in z]
