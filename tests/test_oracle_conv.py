"""Oracle pins for the short causal convolution + SiLU and the pre-processing order.

The pages name the step (ShortConvolution / causal_conv1d_silu on q, k and v)
without printing it; the pins fix the reading the oracle implements: a
per-channel causal cross-correlation with W - 1 rows of history in front of
every sequence (zeros, or a carried state whose hand-off splits a sequence
exactly), weight[:, W - 1] on the current token, then SiLU.
"""
import math

import numpy as np
import pytest
from scipy.special import expit


def _rng(seed=0):
    return np.random.default_rng(seed)


def test_silu_closed_forms(oracle):
    # logistic(ln 3) = 3/4, so silu(ln 3) = 0.75 ln 3; silu(0) = 0
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(oracle.silu(np.array([math.log(3.0)])), [0.75 * math.log(3.0)],
                               rtol=1e-15)
    # odd part: silu(z) - silu(-z) = z
    z = np.linspace(-40, 40, 801)
    np.testing.assert_allclose(oracle.silu(z) - oracle.silu(-z), z, rtol=1e-13, atol=1e-13)
    # far tails: silu(z) -> z above, -> 0 below (no overflow warning)
    assert abs(oracle.silu(np.array([800.0]))[0] - 800.0) == 0.0
    assert oracle.silu(np.array([-800.0]))[0] == 0.0


@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_conv_matches_numpy_convolve(oracle, W):
    r = _rng(W)
    B, T, D = 2, 37, 5
    x = r.standard_normal((B, T, D))
    w = r.standard_normal((D, W))
    b = r.standard_normal(D)
    y = oracle.short_conv_silu(x, w, b)
    for bb in range(B):
        for c in range(D):
            # full convolution with the reversed taps = causal cross-correlation
            z = np.convolve(x[bb, :, c], w[c, ::-1])[:T] + b[c]
            np.testing.assert_allclose(y[bb, :, c], z * expit(z), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("W", [2, 3, 4])
def test_conv_impulse_response_is_the_reversed_taps(oracle, W):
    T, D, t0 = 12, 3, 5
    w = np.arange(1, D * W + 1, dtype=np.float64).reshape(D, W) / 7.0
    x = np.zeros((1, T, D))
    x[0, t0, 1] = 1.0
    y = oracle.short_conv_silu(x, w, None)
    expect = np.zeros((T, D))
    for i in range(W):
        expect[t0 + i, 1] = w[1, W - 1 - i] / (1.0 + math.exp(-w[1, W - 1 - i]))
    np.testing.assert_allclose(y[0], expect, rtol=1e-15, atol=0)


def test_width_one_is_elementwise_and_bias_enters_before_silu(oracle):
    r = _rng(3)
    x = r.standard_normal((2, 9, 4))
    w = r.standard_normal((4, 1))
    b = r.standard_normal(4)
    z = x * w[:, 0] + b
    np.testing.assert_allclose(oracle.short_conv_silu(x, w, b), z * expit(z), rtol=1e-13)
    # zero input: every output is silu(bias)
    y0 = oracle.short_conv_silu(np.zeros((1, 6, 4)), r.standard_normal((4, 4)), b)
    np.testing.assert_allclose(y0[0], np.broadcast_to(b * expit(b), (6, 4)), rtol=1e-15)


def test_conv_is_causal_and_short(oracle):
    r = _rng(4)
    W, T, D, t = 4, 20, 3, 9
    x = r.standard_normal((1, T, D))
    w = r.standard_normal((D, W))
    y = oracle.short_conv_silu(x, w, None)
    x2 = x.copy()
    x2[0, t] += 10.0
    y2 = oracle.short_conv_silu(x2, w, None)
    assert np.array_equal(y[0, :t], y2[0, :t])          # nothing before t moves
    assert np.array_equal(y[0, t + W:], y2[0, t + W:])  # nothing after the window moves
    assert np.all(y[0, t:t + W] != y2[0, t:t + W])


def test_varlen_sequences_are_independent(oracle):
    r = _rng(5)
    W, D = 4, 6
    cu = [0, 0, 3, 3, 11, 12, 30]  # empty slots, a 1-token and a 2-token-shorter-than-W case
    cap = 33
    x = r.standard_normal((1, cap, D))
    w = r.standard_normal((D, W))
    b = r.standard_normal(D)
    y = oracle.short_conv_silu(x, w, b, cu)
    for n in range(len(cu) - 1):
        bos, eos = cu[n], cu[n + 1]
        if eos == bos:
            continue
        alone = oracle.short_conv_silu(x[:, bos:eos], w, b)
        np.testing.assert_array_equal(y[:, bos:eos], alone)
    assert np.isnan(y[0, cu[-1]:]).all()


def test_preprocess_order_conv_then_l2norm(oracle):
    r = _rng(6)
    B, T, H, K, HV, V, W = 1, 10, 2, 8, 4, 6, 3
    q, k = r.standard_normal((B, T, H, K)), r.standard_normal((B, T, H, K))
    v = r.standard_normal((B, T, HV, V))
    conv = tuple((r.standard_normal((n, W)), r.standard_normal(n)) for n in (H * K, H * K, HV * V))
    q1, k1, v1 = oracle.preprocess(q, k, v, conv, qk_l2norm=True)
    cq = oracle.short_conv_silu(q.reshape(B, T, -1), *conv[0]).reshape(q.shape)
    ck = oracle.short_conv_silu(k.reshape(B, T, -1), *conv[1]).reshape(k.shape)
    cv = oracle.short_conv_silu(v.reshape(B, T, -1), *conv[2]).reshape(v.shape)
    # normalised rows: |x|^2 = s / (s + eps) with s the squared norm of the conv output
    sq = np.sum(cq * cq, axis=-1)
    np.testing.assert_allclose(np.sum(q1 * q1, axis=-1), sq / (sq + oracle.L2NORM_EPS), rtol=1e-13)
    np.testing.assert_allclose(q1 * np.sqrt(sq + oracle.L2NORM_EPS)[..., None], cq, rtol=1e-12)
    sk = np.sum(ck * ck, axis=-1)
    np.testing.assert_allclose(k1 * np.sqrt(sk + oracle.L2NORM_EPS)[..., None], ck, rtol=1e-12)
    np.testing.assert_array_equal(v1, cv)  # v is convolved, never normalised
    # identity taps (1 on the current token) and no bias reduce the conv to silu(x)
    eye = tuple((np.concatenate([np.zeros((n, W - 1)), np.ones((n, 1))], axis=1), None)
                for n in (H * K, H * K, HV * V))
    q2, _, v2 = oracle.preprocess(q, k, v, eye, qk_l2norm=False)
    np.testing.assert_allclose(q2, q * expit(q), rtol=1e-15)
    np.testing.assert_allclose(v2, v * expit(v), rtol=1e-15)


@pytest.mark.parametrize("W", [1, 2, 4])
@pytest.mark.parametrize("m", [0, 1, 2, 5, 17])
def test_carried_state_splits_a_sequence_exactly(oracle, W, m):
    """Convolving a sequence in two segments, the second starting from the
    history the first returns, equals convolving it whole (outputs and the
    final history), for splits before, inside and after the first W - 1 tokens."""
    r = _rng(10 + W)
    L, D = 17, 5
    x = r.standard_normal((1, L, D))
    w = r.standard_normal((D, W))
    b = r.standard_normal(D)
    y, st = oracle.short_conv_silu(x, w, b, return_state=True)
    y1, st1 = oracle.short_conv_silu(x[:, :m], w, b, return_state=True)
    y2, st2 = oracle.short_conv_silu(x[:, m:], w, b, state=st1, return_state=True)
    np.testing.assert_allclose(np.concatenate([y1, y2], axis=1), y, rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(st2, st)
    assert st.shape == (1, W - 1, D)


def test_state_is_the_last_inputs_reaching_into_the_history(oracle):
    r = _rng(20)
    W, D = 4, 3
    hist = r.standard_normal((3, W - 1, D))
    x = r.standard_normal((1, 9, D))
    cu = [0, 1, 1, 9]  # a 1-token sequence, an empty slot, an 8-token sequence
    w = r.standard_normal((D, W))
    _, st = oracle.short_conv_silu(x, w, None, cu, state=hist, return_state=True)
    np.testing.assert_array_equal(st[0], np.concatenate([hist[0, 1:], x[0, 0:1]]))  # 2 old + 1 new
    np.testing.assert_array_equal(st[1], hist[1])                                    # empty: unchanged
    np.testing.assert_array_equal(st[2], x[0, 6:9])                                  # last 3 inputs
    # an impulse in the history at position -1 reaches the first W - 1 outputs
    h1 = np.zeros((1, W - 1, D))
    h1[0, W - 2, 0] = 1.0
    y = oracle.short_conv_silu(np.zeros((1, 5, D)), w, None, state=h1)
    z = np.array([w[0, W - 2], w[0, W - 3], w[0, W - 4], 0.0, 0.0])
    np.testing.assert_allclose(y[0, :, 0], z * expit(z), rtol=1e-15)
