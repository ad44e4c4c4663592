"""Oracle pins for the KDA gate: activation, unit-scale default, chunk-local log2 cumsum."""
import json
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cases():
    with open(os.path.join(GOLDEN, "gate_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_gate_hand_computed(oracle, case):
    x = np.array(case["x"]).reshape(1, -1, 1, 1)
    a = None if case["A_log"] is None else np.array([case["A_log"]])
    g = oracle.gate_activation(x, a)
    np.testing.assert_allclose(g.ravel() * oracle.LOG2E, case["per_token_log2"], rtol=1e-14, atol=1e-14)
    G2 = oracle.gate_cumsum_log2(g, None, case["chunk_size"])
    np.testing.assert_allclose(G2.ravel(), case["cumsum_log2"], rtol=1e-14, atol=1e-14)


def test_softplus_matches_logaddexp(oracle):
    x = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(oracle.softplus(x), np.logaddexp(0.0, x), rtol=2e-9, atol=0)


def test_omitted_A_log_is_zero_A_log_bitwise(oracle):
    rng = np.random.default_rng(0)
    x = rng.standard_normal((2, 5, 3, 4))
    g0 = oracle.gate_activation(x, None)
    gz = oracle.gate_activation(x, np.zeros(3))
    assert g0.tobytes() == gz.tobytes()


def test_ones_A_log_scales_by_e(oracle):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((1, 7, 2, 4))
    g0 = oracle.gate_activation(x, None)
    g1 = oracle.gate_activation(x, np.ones(2))
    np.testing.assert_allclose(g1, math.e * g0, rtol=1e-15)


def test_chunk_size_one_is_per_token_log2(oracle):
    rng = np.random.default_rng(2)
    g = -np.abs(rng.standard_normal((2, 9, 3, 4)))
    G2 = oracle.gate_cumsum_log2(g, None, 1)
    np.testing.assert_allclose(G2, g * oracle.LOG2E, rtol=1e-15)


def test_cumsum_restarts_per_chunk_and_sequence(oracle):
    rng = np.random.default_rng(3)
    g = -np.abs(rng.standard_normal((1, 20, 1, 2)))
    cu = [0, 3, 3, 20]
    G2 = oracle.gate_cumsum_log2(g, cu, 4)
    # brute force: running sum reset at each sequence start and every 4 tokens within it
    ref = np.full_like(g, np.nan)
    for bos, eos in [(0, 3), (3, 3), (3, 20)]:
        acc = np.zeros(2)
        for t in range(bos, eos):
            if (t - bos) % 4 == 0:
                acc = np.zeros(2)
            acc = acc + g[0, t, 0]
            ref[0, t, 0] = acc / math.log(2.0)
    np.testing.assert_allclose(G2, ref, rtol=1e-14)


def test_log2_cumsum_roundtrip(oracle):
    rng = np.random.default_rng(4)
    g = -np.abs(rng.standard_normal((1, 30, 2, 3)))
    cu = [0, 7, 30]
    G2 = oracle.gate_cumsum_log2(g, cu, 8)
    np.testing.assert_allclose(oracle.g_from_log2_cumsum(G2, cu, 8), g, rtol=1e-12, atol=1e-15)
