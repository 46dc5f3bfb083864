"""Pins of the oracle's gated-delta-rule step (CPU).

The pages name the per-head BLAS calls of the GatedDeltaNet update (scale, matrix-vector product,
rank-one update; Flash-MoE wiki, technique 4, "Accelerate BLAS linear attention") but print no formula.  These
tests fix the oracle to what the gated delta rule implies independently of how the oracle
computes it: a hand-derived fixture, the delta rule's exact recall of v for a unit key, the
untouched orthogonal complement of k, the beta = 0 and identity special cases, and the rule's
product form alpha S (I - beta k k^T) + beta v k^T.
"""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gdn_step_2x2.json")


def _case(rng, nh=3, dv=16, dk=8, unit_k=True):
    S = rng.standard_normal((nh, dv, dk))
    q = rng.standard_normal((nh, dk))
    k = rng.standard_normal((nh, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((nh, dv))
    alpha = rng.uniform(0.2, 1.0, nh)
    beta = rng.uniform(0.1, 1.0, nh)
    return S, q, k, v, alpha, beta


def test_hand_derived_fixture():
    for c in json.load(open(GOLDEN))["cases"]:
        S, o = oracle.gdn_step(c["state"], c["q"], c["k"], c["v"], c["alpha"], c["beta"])
        assert np.array_equal(S, np.array(c["new_state"], dtype=np.float64))
        assert np.array_equal(o, np.array(c["o"], dtype=np.float64))


def test_unit_key_with_beta_one_recalls_v_exactly():
    rng = np.random.default_rng(1)
    S, q, k, v, alpha, _ = _case(rng, nh=4, dv=128, dk=128)
    S1, _ = oracle.gdn_step(S, q, k, v, alpha, np.ones(4))
    for h in range(4):
        np.testing.assert_allclose(S1[h] @ k[h], v[h], rtol=0, atol=1e-12)


def test_orthogonal_complement_of_key_only_decays():
    rng = np.random.default_rng(2)
    S, q, k, v, alpha, beta = _case(rng, nh=3, dv=12, dk=10)
    S1, _ = oracle.gdn_step(S, q, k, v, alpha, beta)
    for h in range(3):
        w = rng.standard_normal(10)
        w -= (w @ k[h]) * k[h]  # w orthogonal to the unit key
        np.testing.assert_allclose(S1[h] @ w, alpha[h] * (S[h] @ w), rtol=0, atol=1e-12)


def test_beta_zero_is_pure_decay_and_alpha_one_beta_zero_is_identity():
    rng = np.random.default_rng(3)
    S, q, k, v, alpha, _ = _case(rng)
    S1, o = oracle.gdn_step(S, q, k, v, alpha, np.zeros(3))
    assert np.array_equal(S1, S * alpha[:, None, None])
    S2, o2 = oracle.gdn_step(S, q, k, v, np.ones(3), np.zeros(3))
    assert np.array_equal(S2, S)
    np.testing.assert_allclose(o2, np.einsum("hij,hj->hi", S, q), rtol=1e-14, atol=1e-14)


def test_product_form_of_the_rule():
    rng = np.random.default_rng(4)
    S, q, k, v, alpha, beta = _case(rng, nh=2, dv=9, dk=7, unit_k=False)
    S1, o = oracle.gdn_step(S, q, k, v, alpha, beta)
    for h in range(2):
        P = np.eye(7) - beta[h] * np.outer(k[h], k[h])
        ref = alpha[h] * (S[h] @ P) + beta[h] * np.outer(v[h], k[h])
        np.testing.assert_allclose(S1[h], ref, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(o[h], ref @ q[h], rtol=1e-12, atol=1e-12)


def test_heads_are_independent_and_inputs_untouched():
    rng = np.random.default_rng(5)
    S, q, k, v, alpha, beta = _case(rng, nh=5)
    S0 = S.copy()
    S1, o1 = oracle.gdn_step(S, q, k, v, alpha, beta)
    assert np.array_equal(S, S0)
    p = np.array([3, 0, 4, 1, 2])
    S2, o2 = oracle.gdn_step(S[p], q[p], k[p], v[p], alpha[p], beta[p])
    assert np.array_equal(S2, S1[p]) and np.array_equal(o2, o1[p])
