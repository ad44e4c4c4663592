"""Independent reformulations of the KDA scan -- TEST INFRASTRUCTURE ONLY.

Each function computes the same result as the token recurrence by another
route, so that the tests can pin the recurrence against it. All FP64 NumPy;
tiny and moderate sizes only.

* `recurrence_explicit`: the recurrence exactly as the definition is written,
  S_t = (I - b_t k_t k_t^T) Diag(exp g_t) S_{t-1} + b_t k_t v_t^T with explicit
  K x K matrices, o_t = S_t^T q_t / sqrt(K).
* `chunk_form`: the chunked (UT / WY) form. The pages name its steps for the
  gated delta rule sibling op ("[Fix] Use unit KDA gate scale ..." page,
  squashed commit bodies: kkt, solve_tril, recompute_w_u, fwd_h, fwd_o);
  the per-channel version written out here is our derivation, with G the
  natural-log cumulative gate inside the chunk and Gamma = exp(G):
      A_ij  = b_i sum_c k_ic k_jc exp(G_ic - G_jc)     (i > j, else 0)
      T     = (I + A)^-1
      W     = T diag(b) (K * Gamma),  U = T diag(b) V
      Delta = U - W S0
      O     = (Q~ * Gamma) S0 + (P o M) Delta,  P_ij = sum_c q~_ic k_jc exp(G_ic - G_jc), j <= i
      S_end = Diag(Gamma_last) S0 + (K * exp(G_last - G))^T Delta
* `dense_form`: one chunk spanning the whole sequence, solved with a
  unit-lower-triangular triangular solve instead of forming T.
"""
from __future__ import annotations

import math

import numpy as np
import scipy.linalg


def _seq(a, bos, eos, B, T):
    return a.reshape(B * T, *a.shape[2:])[bos:eos]


def recurrence_explicit(q, k, v, g, beta, h0=None, scale=None):
    """Single sequence, single head: q, k [L, K]; v [L, V]; g [L, K]; beta [L];
    h0 [K, V]. Returns (o [L, V], S [K, V]). Pure definition, O(L K^2 V)."""
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    L, K = k.shape
    V = v.shape[1]
    S = np.zeros((K, V)) if h0 is None else np.array(h0, dtype=np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    o = np.zeros((L, V))
    eye = np.eye(K)
    for t in range(L):
        kt = k[t][:, None]
        S = (eye - beta[t] * (kt @ kt.T)) @ np.diag(np.exp(g[t])) @ S + beta[t] * kt @ v[t][None, :]
        o[t] = S.T @ (q[t] * scale)
    return o, S


def _pair_decay(G_rows, G_cols, inclusive):
    """exp(G_i - G_j) per channel for j < i (or j <= i), zero elsewhere: [Lr, Lc, K]."""
    Lr, Lc = G_rows.shape[0], G_cols.shape[0]
    i = np.arange(Lr)[:, None]
    j = np.arange(Lc)[None, :]
    mask = (j <= i) if inclusive else (j < i)
    d = G_rows[:, None, :] - G_cols[None, :, :]
    d = np.where(mask[:, :, None], d, -np.inf)
    return np.exp(d)


def chunk_step(S0, q, k, v, g, beta, scale):
    """One chunk of the UT form. q, k, g [L, K]; v [L, V]; beta [L]; S0 [K, V].
    Returns (O [L, V], S_end [K, V], parts dict)."""
    L, K = k.shape
    G = np.cumsum(g, axis=0)
    Gam = np.exp(G)
    qs = q * scale
    Dk = _pair_decay(G, G, inclusive=False)
    A = beta[:, None] * np.einsum("ic,jc,ijc->ij", k, k, Dk)
    Tm = np.linalg.inv(np.eye(L) + A)
    W = Tm @ (beta[:, None] * (k * Gam))
    U = Tm @ (beta[:, None] * v)
    Delta = U - W @ S0
    Dq = _pair_decay(G, G, inclusive=True)
    P = np.einsum("ic,jc,ijc->ij", qs, k, Dq)
    O = (qs * Gam) @ S0 + P @ Delta
    Khat = k * np.exp(G[-1][None, :] - G)
    S1 = np.exp(G[-1])[:, None] * S0 + Khat.T @ Delta
    return O, S1, dict(A=A, T=Tm, W=W, U=U, Delta=Delta, P=P, Khat=Khat, G=G)


def chunk_form(q, k, v, g, beta, h0=None, cu_seqlens=None, chunk_size=64, scale=None):
    """Whole problem in the chunked form. Same shapes and outputs as
    `oracle.recurrence` (g natural log, per token)."""
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    G_ = HV // H
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    from . import seq_bounds
    bounds = seq_bounds(B, T, cu_seqlens)
    o = np.full((B * T, HV, V), np.nan)
    ht = np.zeros((len(bounds), HV, K, V))
    qf, kf = q.reshape(B * T, H, K), k.reshape(B * T, H, K)
    vf, gf, bf = v.reshape(B * T, HV, V), g.reshape(B * T, HV, K), beta.reshape(B * T, HV)
    for n, (bos, eos) in enumerate(bounds):
        for hv in range(HV):
            h = hv // G_
            S = np.zeros((K, V)) if h0 is None else np.array(h0[n, hv], dtype=np.float64)
            for c0 in range(bos, eos, chunk_size):
                c1 = min(c0 + chunk_size, eos)
                O, S, _ = chunk_step(S, qf[c0:c1, h], kf[c0:c1, h], vf[c0:c1, hv], gf[c0:c1, hv],
                                     bf[c0:c1, hv], scale)
                o[c0:c1, hv] = O
            ht[n, hv] = S
    return o.reshape(B, T, HV, V), ht


def dense_form(q, k, v, g, beta, h0=None, scale=None):
    """Single sequence, single head, one chunk over all L tokens, with the
    unit-lower-triangular system (I + A) Delta = diag(b)(V - (K*Gamma) S0)
    solved by forward substitution (scipy.linalg.solve_triangular)."""
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    L, K = k.shape
    V = v.shape[1]
    S0 = np.zeros((K, V)) if h0 is None else np.asarray(h0, dtype=np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    G = np.cumsum(g, axis=0)
    Gam = np.exp(G)
    A = beta[:, None] * np.einsum("ic,jc,ijc->ij", k, k, _pair_decay(G, G, False))
    rhs = beta[:, None] * (v - (k * Gam) @ S0)
    Delta = scipy.linalg.solve_triangular(np.eye(L) + A, rhs, lower=True, unit_diagonal=True)
    P = np.einsum("ic,jc,ijc->ij", q * scale, k, _pair_decay(G, G, True))
    O = (q * scale * Gam) @ S0 + P @ Delta
    S1 = np.exp(G[-1])[:, None] * S0 + (k * np.exp(G[-1][None, :] - G)).T @ Delta
    return O, S1


def chunk_step_bwd(S0, q, k, v, g, beta, scale, dO, dS1):
    """Reverse of `chunk_step` (our derivation, by hand): given the chunk's
    start state S0, upstream dO [L, V] and dS1 (gradient of the chunk's end
    state), return (dq, dk, dv, dg, dbeta, dS0) with dg w.r.t. the per-token
    natural-log gate. Every product of the forward chunk form is reversed in
    turn: O and S_end -> Delta, S0; Delta -> U, W; U, W -> T, beta, V, K*Gamma;
    T = (I + A)^-1 -> A; A, P -> k, q, G; G -> g (reverse cumsum)."""
    L, K = k.shape
    G = np.cumsum(g, axis=0)
    Gam = np.exp(G)
    gam = Gam[-1]
    qs = q * scale
    Dk = _pair_decay(G, G, inclusive=False)
    Dq = _pair_decay(G, G, inclusive=True)
    Abar = np.einsum("ic,jc,ijc->ij", k, k, Dk)
    A = beta[:, None] * Abar
    Tm = np.linalg.inv(np.eye(L) + A)
    Kg = k * Gam
    W = Tm @ (beta[:, None] * Kg)
    U = Tm @ (beta[:, None] * v)
    Delta = U - W @ S0
    P = np.einsum("ic,jc,ijc->ij", qs, k, Dq)
    QG = qs * Gam
    eL = np.exp(G[-1][None, :] - G)
    KH = k * eL
    # outputs O = QG S0 + P Delta, S1 = diag(gam) S0 + KH^T Delta
    dDelta = P.T @ dO + KH @ dS1
    dS0 = QG.T @ dO + gam[:, None] * dS1 - W.T @ dDelta
    dP = np.tril(dO @ Delta.T)
    dQG = dO @ S0.T
    dKH = Delta @ dS1.T
    dgam = np.sum(dS1 * S0, axis=1)
    # Delta = U - W S0
    dU = dDelta
    dW = -dDelta @ S0.T
    # U = T (b V), W = T (b Kg)
    dT = dU @ (beta[:, None] * v).T + dW @ (beta[:, None] * Kg).T
    TtdU = Tm.T @ dU
    TtdW = Tm.T @ dW
    dv = beta[:, None] * TtdU
    dKg = beta[:, None] * TtdW
    dbeta = np.sum(v * TtdU, axis=1) + np.sum(Kg * TtdW, axis=1)
    # T = (I + A)^-1, A strictly lower
    dA = np.tril(-Tm.T @ dT @ Tm.T, -1)
    dbeta += np.sum(Abar * dA, axis=1)
    dAb = beta[:, None] * dA
    # Abar_ij = sum_c k_ic k_jc exp(G_ic - G_jc), i > j
    X1 = np.einsum("ij,jc,ijc->ic", dAb, k, Dk)
    X2 = np.einsum("ij,ic,ijc->jc", dAb, k, Dk)
    dk = X1 + X2
    dG = k * X1 - k * X2
    # P_ij = sum_c q~_ic k_jc exp(G_ic - G_jc), j <= i
    Y1 = np.einsum("ij,jc,ijc->ic", dP, k, Dq)
    Y2 = np.einsum("ij,ic,ijc->jc", dP, qs, Dq)
    dqs = Y1.copy()
    dk += Y2
    dG += qs * Y1 - k * Y2
    # QG = q~ Gamma
    dqs += dQG * Gam
    dG += dQG * QG
    # KH = k exp(G_last - G)
    dk += dKH * eL
    t = dKH * KH
    dG -= t
    dG[-1] += t.sum(axis=0)
    # gam = exp(G_last)
    dG[-1] += dgam * gam
    # Kg = k Gamma
    dk += dKg * Gam
    dG += dKg * Kg
    dq = dqs * scale
    dg = np.cumsum(dG[::-1], axis=0)[::-1]
    return dq, dk, dv, dg, dbeta, dS0


def chunk_backward(q, k, v, g, beta, dO, h0=None, dht=None, cu_seqlens=None, chunk_size=64,
                   scale=None):
    """Gradients of the chunked form over a whole problem (same shapes and
    outputs as `oracle.recurrence_bwd`): a forward pass keeps each chunk's
    start state, then chunks are reversed from the last one."""
    q, k, v, g, beta, dO = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta, dO))
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    G_ = HV // H
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    from . import seq_bounds
    bounds = seq_bounds(B, T, cu_seqlens)
    N = len(bounds)
    qf, kf = q.reshape(B * T, H, K), k.reshape(B * T, H, K)
    vf, gf, bf = v.reshape(B * T, HV, V), g.reshape(B * T, HV, K), beta.reshape(B * T, HV)
    dOf = dO.reshape(B * T, HV, V)
    dq = np.zeros((B * T, H, K)); dk = np.zeros((B * T, H, K))
    dv = np.zeros((B * T, HV, V)); dg = np.zeros((B * T, HV, K)); db = np.zeros((B * T, HV))
    dh0 = np.zeros((N, HV, K, V))
    for n, (bos, eos) in enumerate(bounds):
        for hv in range(HV):
            h = hv // G_
            S = np.zeros((K, V)) if h0 is None else np.array(h0[n, hv], dtype=np.float64)
            starts = []
            chunks = [(c0, min(c0 + chunk_size, eos)) for c0 in range(bos, eos, chunk_size)]
            for c0, c1 in chunks:
                starts.append(S)
                _, S, _ = chunk_step(S, qf[c0:c1, h], kf[c0:c1, h], vf[c0:c1, hv], gf[c0:c1, hv],
                                     bf[c0:c1, hv], scale)
            dS = np.zeros((K, V)) if dht is None else np.array(dht[n, hv], dtype=np.float64)
            for (c0, c1), S0 in reversed(list(zip(chunks, starts))):
                a, b_, c, d_, e, dS = chunk_step_bwd(S0, qf[c0:c1, h], kf[c0:c1, h], vf[c0:c1, hv],
                                                     gf[c0:c1, hv], bf[c0:c1, hv], scale,
                                                     dOf[c0:c1, hv], dS)
                dq[c0:c1, h] += a
                dk[c0:c1, h] += b_
                dv[c0:c1, hv] = c
                dg[c0:c1, hv] = d_
                db[c0:c1, hv] = e
            dh0[n, hv] = dS
    r = lambda a, *s: a.reshape(B, T, *s)
    return dict(dq=r(dq, H, K), dk=r(dk, H, K), dv=r(dv, HV, V), dg=r(dg, HV, K), dbeta=r(db, HV),
                dh0=dh0)
