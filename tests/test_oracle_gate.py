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


# ---------------------------------------------------------------- gate backward (dx, dA_log, d_dt_bias)

def _gate_bwd_case(seed, B=1, T=9, HV=2, K=3, cu=(0, 3, 3, 8)):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, T, HV, K))
    x[0, 1, 0, 0] = 24.0   # above the softplus threshold (derivative exactly 1 there)
    x[0, 2, 1, 2] = -27.0  # deep in the exponential tail
    A_log = 0.7 * rng.standard_normal(HV)
    dt_bias = rng.standard_normal((HV, K))
    dg = rng.standard_normal((B, T, HV, K))
    return x, A_log, dt_bias, dg, (None if cu is None else list(cu))


def _inside(B, T, cu):
    m = np.zeros((B, T), dtype=bool)
    if cu is None:
        m[:] = True
    else:
        for a, b in zip(cu[:-1], cu[1:]):
            m[0, a:b] = True
    return m


@pytest.mark.parametrize("cu", [None, (0, 3, 3, 8)])
def test_gate_bwd_matches_finite_differences(oracle, cu):
    """dx, dA_log and d_dt_bias against central differences of the scalar
    L = sum over tokens inside a sequence of dg * g(x, A_log, dt_bias)."""
    x, A_log, dt_bias, dg, cu = _gate_bwd_case(5, cu=cu)
    B, T = x.shape[:2]
    inside = _inside(B, T, cu)[:, :, None, None]

    def loss(x_, a_, b_):
        return float(np.sum(np.where(inside, dg * oracle.gate_activation(x_, a_, b_), 0.0)))

    dx, dA, db = oracle.gate_activation_bwd(x, A_log, dt_bias, dg, cu)
    eps = 1e-6
    for idx in np.ndindex(x.shape):
        p, m = x.copy(), x.copy()
        p[idx] += eps
        m[idx] -= eps
        fd = (loss(p, A_log, dt_bias) - loss(m, A_log, dt_bias)) / (2 * eps)
        if inside[idx[0], idx[1], 0, 0]:
            assert abs(fd - dx[idx]) <= 1e-7 * max(1.0, abs(fd)), (idx, fd, dx[idx])
        else:
            assert fd == 0.0 and np.isnan(dx[idx])
    for h in range(A_log.size):
        p, m = A_log.copy(), A_log.copy()
        p[h] += eps
        m[h] -= eps
        fd = (loss(x, p, dt_bias) - loss(x, m, dt_bias)) / (2 * eps)
        assert abs(fd - dA[h]) <= 1e-7 * max(1.0, abs(fd)), (h, fd, dA[h])
    for idx in np.ndindex(dt_bias.shape):
        p, m = dt_bias.copy(), dt_bias.copy()
        p[idx] += eps
        m[idx] -= eps
        fd = (loss(x, A_log, p) - loss(x, A_log, m)) / (2 * eps)
        assert abs(fd - db[idx]) <= 1e-7 * max(1.0, abs(fd)), (idx, fd, db[idx])


def test_gate_bias_zero_is_no_bias_bitwise(oracle):
    x, A_log, _, dg, _ = _gate_bwd_case(6, cu=None)
    g0 = oracle.gate_activation(x, A_log)
    gz = oracle.gate_activation(x, A_log, np.zeros((x.shape[2], x.shape[3])))
    assert g0.tobytes() == gz.tobytes()
    dx0, dA0, db0 = oracle.gate_activation_bwd(x, A_log, None, dg)
    dxz, dAz, dbz = oracle.gate_activation_bwd(x, A_log, np.zeros((x.shape[2], x.shape[3])), dg)
    assert db0 is None and dbz is not None
    assert dx0.tobytes() == dxz.tobytes() and dA0.tobytes() == dAz.tobytes()
    _, dAn, _ = oracle.gate_activation_bwd(x, None, None, dg)
    assert dAn is None


def test_gate_bwd_closed_form_at_zero_argument(oracle):
    """x + dt_bias = 0: softplus' = sigmoid(0) = 1/2 and softplus(0) = ln 2, so
    dx = -exp(A_log) dg / 2 and dA_log = -exp(A_log) ln 2 * sum(dg)."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((1, 4, 2, 3))
    dt_bias = -x[0, 0]                      # zero argument on token 0
    x[0, 1:] = x[0, 0]
    dg = rng.standard_normal((1, 4, 2, 3))
    A_log = np.array([0.0, math.log(3.0)])
    dx, dA, db = oracle.gate_activation_bwd(x, A_log, dt_bias, dg)
    s = np.exp(A_log)[None, None, :, None]
    np.testing.assert_allclose(dx, -s * dg / 2, rtol=1e-15, atol=0)
    np.testing.assert_allclose(dA, -np.exp(A_log) * math.log(2.0) * dg.sum(axis=(0, 1, 3)), rtol=1e-14)
    np.testing.assert_allclose(db, (-s * dg / 2).sum(axis=(0, 1)), rtol=1e-14)


def test_gate_bwd_through_the_scan_matches_finite_differences(oracle):
    """End to end: x -> g -> recurrence -> L = <o, W_o> + <h_T, W_h>. The
    recurrence's dg fed to gate_activation_bwd gives dL/dx, dL/dA_log and
    dL/d_dt_bias (checked on sampled entries)."""
    import workloads
    wl = workloads.tiny_case(72, T=11, H=1, HV=2, K=4, V=3, cu_seqlens=[0, 4, 4, 10], grads=True)
    A_log = np.array([0.3, -0.4])
    dt_bias = np.random.default_rng(8).standard_normal((2, 4))
    x = wl.x.astype(np.float64)
    W_o = np.nan_to_num(wl.dO.astype(np.float64))
    W_o[:, 10:] = 0.0
    W_h = wl.dht.astype(np.float64)

    def loss(x_, a_, b_):
        o, ht = oracle.recurrence(wl.q, wl.k, wl.v, oracle.gate_activation(x_, a_, b_), wl.beta, wl.h0,
                                  wl.cu_seqlens)
        return float(np.sum(np.nan_to_num(o) * W_o) + np.sum(ht * W_h))

    g = oracle.gate_activation(x, A_log, dt_bias)
    grads = oracle.recurrence_bwd(wl.q, wl.k, wl.v, g, wl.beta, W_o, wl.h0, W_h, wl.cu_seqlens)
    dx, dA, db = oracle.gate_activation_bwd(x, A_log, dt_bias, grads["dg"], wl.cu_seqlens)
    eps = 1e-6
    rng = np.random.default_rng(9)
    for fi in rng.choice(10 * 2 * 4, size=10, replace=False):
        idx = (0,) + np.unravel_index(fi, (10, 2, 4))
        p, m = x.copy(), x.copy()
        p[idx] += eps
        m[idx] -= eps
        fd = (loss(p, A_log, dt_bias) - loss(m, A_log, dt_bias)) / (2 * eps)
        assert abs(fd - dx[idx]) <= 1e-6 * max(1.0, abs(fd)), (idx, fd, dx[idx])
    for h in range(2):
        p, m = A_log.copy(), A_log.copy()
        p[h] += eps
        m[h] -= eps
        fd = (loss(x, p, dt_bias) - loss(x, m, dt_bias)) / (2 * eps)
        assert abs(fd - dA[h]) <= 1e-6 * max(1.0, abs(fd)), (h, fd, dA[h])
    for idx in [(0, 0), (1, 3)]:
        p, m = dt_bias.copy(), dt_bias.copy()
        p[idx] += eps
        m[idx] -= eps
        fd = (loss(x, A_log, p) - loss(x, A_log, m)) / (2 * eps)
        assert abs(fd - db[idx]) <= 1e-6 * max(1.0, abs(fd)), (idx, fd, db[idx])


# ---------------------------------------------------------------- q/k L2 normalisation

def test_l2norm_hand_computed(oracle):
    """(3, 4) has squared norm 25: y = (3, 4) / sqrt(25 + 1e-6)."""
    y = oracle.l2norm(np.array([[3.0, 4.0]]))
    s = 1.0 / math.sqrt(25.000001)
    np.testing.assert_allclose(y, [[3.0 * s, 4.0 * s]], rtol=1e-15, atol=0)
    assert abs(s - 0.2 * (1.0 - 2e-8)) < 1e-15


def test_l2norm_properties(oracle):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((5, 7, 3, 16)) * rng.uniform(0.01, 100.0, (5, 7, 3, 1))
    y = oracle.l2norm(x)
    n2 = np.sum(x * x, axis=-1)
    # parallel to x, squared norm n2 / (n2 + eps), zero stays zero
    np.testing.assert_allclose(np.sum(y * y, axis=-1), n2 / (n2 + oracle.L2NORM_EPS), rtol=1e-13)
    cos = np.sum(y * x, axis=-1) / np.sqrt(np.sum(y * y, axis=-1) * n2)
    np.testing.assert_allclose(cos, 1.0, rtol=1e-13)
    assert (oracle.l2norm(np.zeros((2, 8))) == 0.0).all()


def test_l2norm_of_unit_rows_changes_the_scan_by_eps_only(oracle):
    """Inputs already of unit norm: normalising q and k moves the outputs by
    O(eps); normalising v instead (a plausible slip) moves them by O(1)."""
    import workloads
    wl = workloads.tiny_case(12, B=1, T=40, H=1, HV=2, K=16, V=8)
    g = oracle.gate_activation(wl.x, wl.A_log)
    o1, h1 = oracle.recurrence(wl.q, wl.k, wl.v, g, wl.beta, wl.h0)
    o2, h2 = oracle.recurrence(oracle.l2norm(wl.q), oracle.l2norm(wl.k), wl.v, g, wl.beta, wl.h0)
    assert np.abs(o2 - o1).max() <= 1e-5 * np.abs(o1).max()
    o3, _ = oracle.recurrence(wl.q, wl.k, oracle.l2norm(wl.v), g, wl.beta, wl.h0)
    assert np.abs(o3 - o1).max() > 1e-2 * np.abs(o1).max()
