"""Oracle pin for the reverse pass: central finite differences of the FP64
forward recurrence on tiny shapes (varlen, empty slot, GVA, nonzero h0/dht)."""
import numpy as np
import pytest

import workloads


def _loss(oracle, wl, g, W_o, W_h, **over):
    args = dict(q=wl.q, k=wl.k, v=wl.v, g=g, beta=wl.beta, h0=wl.h0)
    args.update(over)
    o, ht = oracle.recurrence(args["q"], args["k"], args["v"], args["g"], args["beta"], args["h0"],
                              wl.cu_seqlens)
    o = np.nan_to_num(o, nan=0.0)
    return float(np.sum(o * W_o) + np.sum(ht * W_h))


@pytest.mark.parametrize("layout", ["dense", "varlen_gva"])
def test_bwd_matches_finite_differences(oracle, layout):
    if layout == "dense":
        wl = workloads.tiny_case(70, B=2, T=7, H=1, HV=1, K=5, V=4, grads=True)
    else:
        wl = workloads.tiny_case(71, T=12, H=1, HV=2, K=5, V=4, cu_seqlens=[0, 4, 4, 11], grads=True)
    g = oracle.gate_activation(wl.x, wl.A_log)
    W_o = np.nan_to_num(wl.dO.astype(np.float64))
    if wl.cu_seqlens is not None:
        W_o[:, int(wl.cu_seqlens[-1]):] = 0.0
    W_h = wl.dht.astype(np.float64)
    grads = oracle.recurrence_bwd(wl.q, wl.k, wl.v, g, wl.beta, W_o, wl.h0, W_h, wl.cu_seqlens)
    base = dict(q=wl.q.astype(np.float64), k=wl.k.astype(np.float64), v=wl.v.astype(np.float64),
                g=g, beta=wl.beta.astype(np.float64), h0=wl.h0.astype(np.float64))
    names = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", h0="dh0")
    rng = np.random.default_rng(0)
    eps = 1e-6
    for name, gname in names.items():
        arr = base[name]
        flat_idx = rng.choice(arr.size, size=min(arr.size, 12), replace=False)
        for fi in flat_idx:
            idx = np.unravel_index(fi, arr.shape)
            if wl.cu_seqlens is not None and name not in ("h0",) and idx[1] >= int(wl.cu_seqlens[-1]):
                continue
            p = arr.copy(); p[idx] += eps
            m = arr.copy(); m[idx] -= eps
            over_p = dict(base); over_p[name] = p
            over_m = dict(base); over_m[name] = m
            lp = _loss(oracle, wl, over_p["g"], W_o, W_h, **{k: v for k, v in over_p.items() if k != "g"})
            lm = _loss(oracle, wl, over_m["g"], W_o, W_h, **{k: v for k, v in over_m.items() if k != "g"})
            fd = (lp - lm) / (2 * eps)
            an = grads[gname][idx]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, an)


@pytest.mark.parametrize("C", [1, 5, 16, 64])
def test_chunk_backward_matches_reverse_recurrence(oracle, C):
    """The chunked backward (an independent derivation, reversed product by
    product) agrees with the token-level reverse recurrence."""
    wl = workloads.tiny_case(72, T=40, H=1, HV=2, K=6, V=5, cu_seqlens=[0, 3, 3, 29, 40],
                             grads=True, gate_scale=1.5)
    g = oracle.gate_activation(wl.x, wl.A_log)
    ref = oracle.recurrence_bwd(wl.q, wl.k, wl.v, g, wl.beta, wl.dO, wl.h0, wl.dht, wl.cu_seqlens)
    got = oracle.forms.chunk_backward(wl.q, wl.k, wl.v, g, wl.beta, wl.dO, wl.h0, wl.dht,
                                      wl.cu_seqlens, chunk_size=C)
    for name in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        np.testing.assert_allclose(got[name], ref[name], rtol=1e-9, atol=1e-11, err_msg=name)
