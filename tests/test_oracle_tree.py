"""Pins of the oracle's greedy tree verification and its tree attention mask.

* A chain tree (parent of j is j - 1) is the linear greedy verify with K = N - 1, which
  is pinned by brute force in test_oracle_exact.
* On random trees the result equals what the linear greedy rule gives along root paths:
  the accepted depth is the longest linear accept length over all root-to-leaf paths,
  the winner is the lowest-index node of that depth whose whole path is accepted, and
  the emitted tokens are the linear verify's along any leaf path through the winner.
* The worked tree of "Verificação de Atenção em Árvore" (root; a, b; c, d under a; e, f
  under b) with hand-set argmaxes.
* The mask is the reflexive transitive closure of the child -> parent relation, computed
  here by boolean matrix powers instead of walks; depth = ancestors in the mask - 1.
"""
import numpy as np
import pytest

from oracle import spec_verify_oracle as O


def onehot_rows(amax, V, rng=None):
    """Logits whose lowest-index argmax is amax[j] (with a tie behind it sometimes)."""
    rng = rng or np.random.default_rng(0)
    z = rng.normal(0.0, 1.0, (len(amax), V)).astype(np.float32)
    for j, a in enumerate(amax):
        z[j, a] = 10.0
        if a + 1 < V and j % 3 == 0:
            z[j, a + 1] = 10.0  # a tie after the argmax: lowest index wins
    return z


def random_tree(rng, N, max_children=None):
    parents = [-1]
    for j in range(1, N):
        parents.append(int(rng.integers(0, j)))
    return parents


def leaf_paths(parents):
    N = len(parents)
    children = {j: [] for j in range(N)}
    for j in range(1, N):
        children[parents[j]].append(j)
    out = []

    def walk(j, path):
        if not children[j]:
            out.append(path)
        for c in children[j]:
            walk(c, path + [c])
    walk(0, [])
    return out


def test_chain_tree_is_linear_greedy():
    rng = np.random.default_rng(1)
    for rep in range(30):
        N, V = int(rng.integers(1, 9)), int(rng.integers(2, 12))
        z = rng.integers(-2, 3, (N, V)).astype(np.float32)  # many ties
        toks = [0] + [int(np.argmax(z[j - 1])) if rng.random() < 0.7 else int(rng.integers(0, V))
                      for j in range(1, N)]
        r = O.verify_tree_sequence(z, [-1] + list(range(N - 1)), toks)
        lin = O.verify_greedy(z[None], np.array([toks[1:]]))
        assert r["n"] == lin["accept_len"][0]
        assert r["tokens"] == list(lin["tokens"][0])
        assert r["nodes"][:r["n"]] == list(range(1, r["n"] + 1))


def test_tree_equals_best_linear_path():
    rng = np.random.default_rng(2)
    for rep in range(60):
        N, V = int(rng.integers(1, 25)), int(rng.integers(2, 6))
        parents = random_tree(rng, N)
        z = rng.integers(-2, 2, (N, V)).astype(np.float32)
        amax = [int(np.argmax(r)) for r in z]
        toks = [0] + [amax[parents[j]] if rng.random() < 0.6 else int(rng.integers(0, V))
                      for j in range(1, N)]
        r = O.verify_tree_sequence(z, parents, toks)
        best, through = -1, {}
        for path in leaf_paths(parents):
            rows = z[[0] + path]
            lin = O.verify_greedy(rows[None], np.array([[toks[j] for j in path]]))
            n = int(lin["accept_len"][0])
            best = max(best, n)
            through.setdefault(tuple([0] + path[:n]), lin)
        assert r["n"] == best
        # the winner: lowest-index node at that depth whose path is accepted
        cands = sorted(p[-1] for p in through if len(p) - 1 == best)
        win = cands[0]
        key = next(p for p in through if p[-1] == win and len(p) - 1 == best)
        lin = through[key]
        assert r["tokens"] == list(lin["tokens"][0][:best + 1]) + [-1] * (N - best - 1)
        assert r["nodes"] == list(key[1:]) + [-1] * (N - best)


def test_worked_tree_of_the_pages():
    # root=0; a=1, b=2 (children of root); c=3, d=4 under a; e=5, f=6 under b
    parents = [-1, 0, 0, 1, 1, 2, 2]
    V = 16
    tok = [0, 7, 9, 3, 4, 5, 6]
    # the target prefers b after the root, then f after b, then token 11
    amax = [9, 2, 6, 1, 1, 1, 11]
    r = O.verify_tree_sequence(onehot_rows(amax, V), parents, tok)
    assert r["n"] == 2 and r["nodes"][:2] == [2, 6]
    assert r["tokens"] == [9, 6, 11, -1, -1, -1, -1]
    # duplicate siblings: a and b both carry 9; the deeper path wins (through b)
    tok2 = [0, 9, 9, 3, 4, 5, 6]
    r = O.verify_tree_sequence(onehot_rows([9, 2, 6, 1, 1, 1, 11], V), parents, tok2)
    assert r["n"] == 2 and r["nodes"][:2] == [2, 6]
    # equally deep accepted paths (d under a, e under b): the lower node index wins
    tok3 = [0, 9, 9, 3, 8, 8, 6]
    r = O.verify_tree_sequence(onehot_rows([9, 8, 8, 1, 12, 13, 11], V), parents, tok3)
    assert r["n"] == 2 and r["nodes"][:2] == [1, 4] and r["tokens"][:3] == [9, 8, 12]
    # nothing accepted: the root's argmax is emitted
    r = O.verify_tree_sequence(onehot_rows([5, 0, 0, 0, 0, 0, 0], V), parents, tok)
    assert r["n"] == 0 and r["tokens"][0] == 5 and r["nodes"] == [-1] * 7


def test_tree_errors():
    z = np.zeros((3, 4), dtype=np.float32)
    assert O.verify_tree_sequence(z, [0, 0, 1], [0, 1, 1])["status"] == O.SEQ_ERR_TREE
    assert O.verify_tree_sequence(z, [-1, 0, 2], [0, 1, 1])["status"] == O.SEQ_ERR_TREE
    assert O.verify_tree_sequence(z, [-1, 0, 0], [0, 4, 1])["status"] == O.SEQ_ERR_TOKEN
    # node 0's token is never read
    assert O.verify_tree_sequence(z, [-1, 0, 0], [-7, 1, 1])["status"] == 0
    zn = z.copy()
    zn[2, 1] = np.nan
    assert O.verify_tree_sequence(zn, [-1, 0, 0], [0, 1, 1])["status"] == O.SEQ_ERR_LOGIT


@pytest.mark.parametrize("N", [1, 2, 7, 40])
def test_mask_is_transitive_closure(N):
    rng = np.random.default_rng(N)
    parents = np.array([random_tree(rng, N) for _ in range(5)])
    r = O.tree_attention_mask(parents)
    for b in range(5):
        A = np.zeros((N, N), dtype=np.int64)
        for j in range(1, N):
            A[j, parents[b, j]] = 1
        C, P = np.eye(N, dtype=np.int64), np.eye(N, dtype=np.int64)
        for _ in range(N):
            P = (P @ A > 0).astype(np.int64)
            C |= P
        np.testing.assert_array_equal(r["mask"][b], C.astype(np.uint8))
        np.testing.assert_array_equal(r["depth"][b], C.sum(axis=1) - 1)
        assert r["status"][b] == 0


def test_mask_of_malformed_tree():
    r = O.tree_attention_mask(np.array([[-1, 0, 1], [-1, 2, 0]]))
    assert list(r["status"]) == [0, O.SEQ_ERR_TREE]
    assert r["mask"][1].sum() == 0 and (r["depth"][1] == -1).all()
