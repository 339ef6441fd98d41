"""Pins of the plain-C fp64 oracle (oracle/verify_oracle.c).

The C oracle is a second transcription of the verify rule, used where many sequences
must be checked.  It is pinned the same way as the numpy oracle, not by itself:
  * the numpy oracle's pins that go through verify_sequence are run again with the C
    oracle in its place: exact enumeration at V=4, K=2 (the emitted law equals the
    target law, "A Regra de Exatidão" on the lesson page "Decodificação Especulativa e
    EAGLE"), the closed form 3.36 at alpha=0.8, K=4 ("Aceleração Esperada"), the general
    per-position form, greedy brute force ("Caso ganancioso"), T -> 0 equals greedy,
    p == q, disjoint supports, K = 0 (plain sampling), V = 1 and the data errors;
  * on random bf16, fp32 and fp64 batches it agrees with the numpy oracle: the same
    tokens, accept lengths, statuses and draws, p and q within 1e-12 relative.
"""
import math

import numpy as np
import pytest

from oracle import c_oracle as C
from oracle import spec_verify_oracle as O

import test_oracle_exact as E


@pytest.fixture
def c_impl(monkeypatch):
    monkeypatch.setattr(O, "verify_sequence", C.verify_sequence)


@pytest.mark.parametrize("T,shift_t,shift_d", [(1.0, 0.0, 0.0), (0.7, 37.5, -12.0), (2.5, -3.0, 80.0)])
def test_c_exact_enumeration_preserves_target_law(c_impl, T, shift_t, shift_d, monkeypatch):
    E.test_exact_enumeration_preserves_target_law(T, shift_t, shift_d, monkeypatch)


def test_c_closed_form_worked_value_336(c_impl):
    E.test_closed_form_worked_value_336()


def test_c_closed_form_general_per_position_rates(c_impl):
    E.test_closed_form_general_per_position_rates()


def test_c_greedy_rule_brute_force(c_impl):
    E.test_greedy_rule_brute_force()


def test_c_small_temperature_limit_equals_greedy(c_impl):
    E.test_small_temperature_limit_equals_greedy()


def test_c_identical_draft_accepts_everything(c_impl):
    E.test_identical_draft_accepts_everything()


def test_c_disjoint_supports_reject_first_and_sample_target(c_impl):
    E.test_disjoint_supports_reject_first_and_sample_target()


def test_c_k_zero_is_plain_sampling(c_impl):
    E.test_k_zero_is_plain_sampling()


def test_c_single_token_vocabulary(c_impl):
    E.test_single_token_vocabulary()


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_c_errors(c_impl, T):
    E.test_errors(T)


def test_c_scaled_range_rule(c_impl):
    E.test_scaled_range_rule()


def test_c_accept_test_where_p_and_q_underflow(c_impl):
    E.test_accept_test_where_p_and_q_underflow()


def _random_batch(rng, B, K, V, kind):
    zt = rng.normal(0, 2.5, (B, K + 1, V))
    zd = zt[:, :K] + rng.normal(0, rng.choice([0.2, 1.0, 3.0]), (B, K, V))
    if V > 3:
        zt[:, :, ::7] = -np.inf                       # impossible tokens for p
        zd[:, :, 3::11] = -np.inf                     # and for q
        zt[:, :, 1] = zt[:, :, 2] = np.max(zt, axis=2)  # argmax ties
    if kind == "bf16":
        f = zt.astype(np.float32)
        g = zd.astype(np.float32)
        zt = (f.view(np.uint32) >> 16).astype(np.uint16)
        zd = (g.view(np.uint32) >> 16).astype(np.uint16)
    elif kind == "fp32":
        zt, zd = zt.astype(np.float32), zd.astype(np.float32)
    x = rng.integers(0, V, (B, K)).astype(np.int32)
    u = rng.random((B, K + 1)).astype(np.float32)
    T = np.array([0.0 if b % 4 == 1 else float(rng.uniform(0.05, 2.0)) for b in range(B)],
                 dtype=np.float32)
    return zt, zd, x, u, T


@pytest.mark.parametrize("kind", ["bf16", "fp32", "fp64"])
def test_c_agrees_with_numpy_oracle(kind):
    rng = np.random.default_rng({"bf16": 1, "fp32": 2, "fp64": 3}[kind])
    for (B, K, V) in ((12, 0, 50), (8, 3, 1), (8, 4, 7), (10, 5, 1000), (6, 8, 3001), (3, 2, 20000)):
        zt, zd, x, u, T = _random_batch(rng, B, K, V, kind)
        for b in range(B):
            d = None if T[b] == 0 else zd[b]
            ref = O.verify_sequence(zt[b], d, x[b], None if T[b] == 0 else u[b], float(T[b]))
            got = C.verify_sequence(zt[b], d, x[b], None if T[b] == 0 else u[b], float(T[b]))
            for k in ("tokens", "n", "status"):
                assert got[k] == ref[k], (kind, B, K, V, b, k, got[k], ref[k])
            np.testing.assert_allclose(got["p"], ref["p"], rtol=1e-12, atol=0)
            np.testing.assert_allclose(got["q"], ref["q"], rtol=1e-12, atol=0)
            assert [dr[:2] for dr in got["draws"]] == [dr[:2] for dr in ref["draws"]]
            for g, r in zip(got["draws"], ref["draws"]):
                assert math.isclose(g[2], r[2], rel_tol=1e-9, abs_tol=1e-14), (g, r)


def test_c_batched_threads_equal_single_calls():
    rng = np.random.default_rng(9)
    zt, zd, x, u, T = _random_batch(rng, 40, 4, 2000, "bf16")
    one = C.verify(zt, zd, x, u, T, threads=1)
    many = C.verify(zt, zd, x, u, T, threads=6)
    ref = O.verify(zt, zd, x, u, T)
    for k in ("tokens", "accept_len", "status"):
        np.testing.assert_array_equal(one[k], many[k])
        np.testing.assert_array_equal(one[k], ref[k])
    for k in ("p", "q"):
        np.testing.assert_array_equal(one[k].view(np.uint32), many[k].view(np.uint32))
        np.testing.assert_allclose(one[k], ref[k], rtol=1e-6, equal_nan=True)
    assert one["draws"] == many["draws"]
