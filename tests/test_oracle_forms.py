"""Oracle pins: the token recurrence against independent formulations, and
the varlen / empty-slot / GVA contracts."""
import numpy as np
import pytest

import workloads


def _case(seed, **kw):
    wl = workloads.tiny_case(seed, **kw)
    return wl


@pytest.mark.parametrize("C", [1, 16, 64, 73])
def test_chunk_form_matches_recurrence(oracle, C):
    wl = _case(7, T=73, K=8, V=6, gate_scale=1.5)
    g = oracle.gate_activation(wl.x, wl.A_log)
    o, ht = oracle.recurrence(wl.q, wl.k, wl.v, g, wl.beta, wl.h0)
    o2, ht2 = oracle.forms.chunk_form(wl.q, wl.k, wl.v, g, wl.beta, wl.h0, chunk_size=C)
    np.testing.assert_allclose(o2, o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(ht2, ht, rtol=1e-11, atol=1e-12)


def test_dense_form_matches_recurrence(oracle):
    for seed in range(3):
        wl = _case(20 + seed, T=40, K=16, V=12)
        g = oracle.gate_activation(wl.x, wl.A_log)
        o, ht = oracle.recurrence(wl.q, wl.k, wl.v, g, wl.beta, wl.h0)
        o2, s2 = oracle.forms.dense_form(wl.q[0, :, 0], wl.k[0, :, 0], wl.v[0, :, 0], g[0, :, 0],
                                         wl.beta[0, :, 0], wl.h0[0, 0])
        np.testing.assert_allclose(o2, o[0, :, 0], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(s2, ht[0, 0], rtol=1e-11, atol=1e-12)


def test_chunk_form_varlen_gva(oracle):
    wl = _case(30, T=50, H=2, HV=4, K=8, V=4, cu_seqlens=[0, 5, 5, 37, 50])
    g = oracle.gate_activation(wl.x, wl.A_log)
    o, ht = oracle.recurrence(wl.q, wl.k, wl.v, g, wl.beta, wl.h0, wl.cu_seqlens)
    o2, ht2 = oracle.forms.chunk_form(wl.q, wl.k, wl.v, g, wl.beta, wl.h0, wl.cu_seqlens, chunk_size=16)
    np.testing.assert_allclose(o2, o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(ht2, ht, rtol=1e-11, atol=1e-12)


def test_packed_equals_separate_bitwise(oracle):
    cu = [0, 6, 6, 19, 30]
    wl = _case(40, T=33, H=1, HV=2, K=8, V=5, cu_seqlens=cu)  # tokens 30..32: capacity tail
    g = oracle.gate_activation(wl.x, wl.A_log)
    o, ht = oracle.recurrence(wl.q, wl.k, wl.v, g, wl.beta, wl.h0, wl.cu_seqlens)
    for n in range(len(cu) - 1):
        a, b = cu[n], cu[n + 1]
        if a == b:
            continue
        sl = slice(a, b)
        o1, h1 = oracle.recurrence(wl.q[:, sl], wl.k[:, sl], wl.v[:, sl], g[:, sl], wl.beta[:, sl],
                                   wl.h0[n:n + 1])
        assert o1.tobytes() == o[:, sl].tobytes()
        assert h1.tobytes() == ht[n:n + 1].tobytes()
    # the capacity tail is never written
    assert np.isnan(o[:, 30:]).all()


def test_empty_slot_passthrough_bitwise(oracle):
    cu = [0, 0, 4, 4, 4, 9]
    wl = _case(41, T=9, HV=2, K=4, V=3, cu_seqlens=cu)
    h0 = wl.h0.astype(np.float64)
    h0[0, 0, 0, 0] = -0.0
    h0[2, 1, 1, 1] = np.nan  # NaN payload must survive an empty slot untouched
    g = oracle.gate_activation(wl.x, wl.A_log)
    _, ht = oracle.recurrence(wl.q, wl.k, wl.v, g, wl.beta, h0, cu)
    for n in (0, 2, 3):
        assert ht[n].tobytes() == h0[n].tobytes()
    _, ht0 = oracle.recurrence(wl.q, wl.k, wl.v, g, wl.beta, None, cu)
    for n in (0, 2, 3):
        assert (ht0[n] == 0).all() and not np.signbit(ht0[n]).any()


def test_gva_equals_expanded_heads(oracle):
    wl = _case(50, T=21, H=2, HV=6, K=8, V=4)
    g = oracle.gate_activation(wl.x, wl.A_log)
    o, ht = oracle.recurrence(wl.q, wl.k, wl.v, g, wl.beta, wl.h0)
    rep = wl.HV // wl.H
    qe = np.repeat(wl.q, rep, axis=2)
    ke = np.repeat(wl.k, rep, axis=2)
    o2, ht2 = oracle.recurrence(qe, ke, wl.v, g, wl.beta, wl.h0)
    assert o.tobytes() == o2.tobytes() and ht.tobytes() == ht2.tobytes()


def test_dense_batch_equals_varlen_rows(oracle):
    wl = _case(60, B=3, T=11, K=4, V=4)
    g = oracle.gate_activation(wl.x, wl.A_log)
    o, ht = oracle.recurrence(wl.q, wl.k, wl.v, g, wl.beta, wl.h0)
    cu = [0, 11, 22, 33]
    r = lambda a: a.reshape(1, 33, *a.shape[2:])
    o2, ht2 = oracle.recurrence(r(wl.q), r(wl.k), r(wl.v), r(g), r(wl.beta), wl.h0, cu)
    assert o.tobytes() == o2.reshape(o.shape).tobytes() and ht.tobytes() == ht2.tobytes()
