"""Oracle pins: hand-computed cases and closed forms of the KDA recurrence."""
import json
import math
import os

import numpy as np
import pytest

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _load("scalar_cases.json")["cases"], ids=lambda c: c["name"])
def test_hand_computed_recurrence(oracle, case):
    K, V = case["K"], case["V"]
    L = len(case["beta"])
    q = np.array(case["q"]).reshape(1, L, 1, K)
    k = np.array(case["k"]).reshape(1, L, 1, K)
    v = np.array(case["v"]).reshape(1, L, 1, V)
    g = np.log(np.array(case["exp_g"])).reshape(1, L, 1, K)
    beta = np.array(case["beta"]).reshape(1, L, 1)
    h0 = np.array(case["h0"]).reshape(1, 1, K, V)
    o, ht = oracle.recurrence(q, k, v, g, beta, h0)
    np.testing.assert_allclose(o.reshape(L, V), np.array(case["o"]), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(ht.reshape(K, V), np.array(case["ht"]), rtol=1e-14, atol=1e-14)
    # the explicit-matrix definition agrees too
    o2, s2 = oracle.forms.recurrence_explicit(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0],
                                              beta[0, :, 0], h0[0, 0])
    np.testing.assert_allclose(o2, np.array(case["o"]), rtol=1e-14, atol=1e-14)


def _rand(seed, L=9, K=8, V=6):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, L, 1, K))
    k = rng.standard_normal((1, L, 1, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, L, 1, V))
    g = -np.abs(rng.standard_normal((1, L, 1, K)))
    beta = 1 / (1 + np.exp(-rng.standard_normal((1, L, 1))))
    h0 = 0.3 * rng.standard_normal((1, 1, K, V))
    return q, k, v, g, beta, h0


def test_one_token_from_zero_state(oracle):
    q, k, v, g, beta, _ = _rand(1, L=1)
    o, ht = oracle.recurrence(q, k, v, g, beta, None)
    K = q.shape[-1]
    kk, vv, qq, bb = k[0, 0, 0], v[0, 0, 0], q[0, 0, 0], beta[0, 0, 0]
    np.testing.assert_allclose(ht[0, 0], bb * np.outer(kk, vv), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(o[0, 0, 0], bb * vv * (kk @ qq) / math.sqrt(K), rtol=1e-13, atol=1e-15)


def test_zero_beta_is_pure_decay(oracle):
    q, k, v, g, beta, h0 = _rand(2)
    beta[:] = 0.0
    o, ht = oracle.recurrence(q, k, v, g, beta, h0)
    G = np.cumsum(g[0, :, 0], axis=0)
    np.testing.assert_allclose(ht[0, 0], np.exp(G[-1])[:, None] * h0[0, 0], rtol=1e-13)
    K = q.shape[-1]
    for t in range(q.shape[1]):
        ref = (np.exp(G[t])[:, None] * h0[0, 0]).T @ q[0, t, 0] / math.sqrt(K)
        np.testing.assert_allclose(o[0, t, 0], ref, rtol=1e-12, atol=1e-14)


def test_full_forgetting_keeps_only_last_write(oracle):
    q, k, v, g, beta, h0 = _rand(3)
    g[:] = -800.0  # exp underflows to exactly 0: the state forgets everything
    o, ht = oracle.recurrence(q, k, v, g, beta, h0)
    np.testing.assert_allclose(ht[0, 0], beta[0, -1, 0] * np.outer(k[0, -1, 0], v[0, -1, 0]), rtol=1e-14)


def test_delta_rule_write(oracle):
    """beta = 1 and a unit key: after the write the state maps k_t exactly to v_t."""
    q, k, v, g, beta, h0 = _rand(4, L=12)
    beta[:] = 1.0
    L = q.shape[1]
    for t in range(1, L + 1):
        _, ht = oracle.recurrence(q[:, :t], k[:, :t], v[:, :t], g[:, :t], beta[:, :t], h0)
        np.testing.assert_allclose(ht[0, 0].T @ k[0, t - 1, 0], v[0, t - 1, 0], rtol=1e-12, atol=1e-13)


def test_query_scale_is_one_over_sqrt_k(oracle):
    q, k, v, g, beta, h0 = _rand(5, K=16)
    o, _ = oracle.recurrence(q, k, v, g, beta, h0)
    o1, _ = oracle.recurrence(q, k, v, g, beta, h0, scale=1.0)
    np.testing.assert_allclose(o, o1 / 4.0, rtol=1e-14)


def test_tiny_random_matches_explicit_definition(oracle):
    for seed in range(3):
        q, k, v, g, beta, h0 = _rand(10 + seed, L=7, K=5, V=3)
        o, ht = oracle.recurrence(q, k, v, g, beta, h0)
        o2, s2 = oracle.forms.recurrence_explicit(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0],
                                                  beta[0, :, 0], h0[0, 0])
        np.testing.assert_allclose(o[0, :, 0], o2, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(ht[0, 0], s2, rtol=1e-12, atol=1e-13)
