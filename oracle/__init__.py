"""CPU oracle for the KDA scan -- TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of `bench.py`
may import this package. The GPU library never loads it and shares no code,
headers or constants with it.

Contents
  * `kda_oracle.c`  FP64 token recurrence and its hand-written reverse pass
                    (C, OpenMP over (sequence, value head)), loaded via ctypes.
  * `gate_activation`, `gate_cumsum_log2`  FP64 NumPy gate: g = -exp(A_log) *
                    softplus(x + dt_bias) (omitted A_log = unit scale, omitted
                    dt_bias = no bias), then the chunk-local inclusive cumsum
                    in log2 units; `gate_activation_bwd` its reverse (dx,
                    dA_log, d_dt_bias); `l2norm` the optional q/k
                    normalisation of the fused forward; `short_conv_silu`
                    the short causal convolution + SiLU of q, k and v, and
                    `preprocess` the two in the layer's order.
  * `forms.py`      independent reformulations (single-chunk dense solve,
                    chunked UT form) used only to pin the recurrence.

Sources on the pages (the KDA recurrence itself is not printed there; the
form of record is S_t = (I - b k k^T) Diag(exp g) S_{t-1} + b k v^T,
o_t = S_t^T q / sqrt(K)):
  * "[Fix] Use unit KDA gate scale when A_log is omitted" (fla-org
    flash-linear-attention PR #1294), Summary and Breaking changes: the decay
    scale is exp(A_log); omitting A_log means unit scale, identical to an
    explicit zero A_log; an all-ones A_log reproduces exp(1).
  * "kda in torchtitan (training)" (pytorch/torchtitan PR #4164), quoted
    attention-gym description of `recurrent_kda`: packed varlen via int32
    cu_seqlens, repeated offsets are empty slots whose state passes through
    bitwise, a tail beyond the terminal offset is outside the contract, FP32
    states one per logical sequence, the gate is a per-token log2 decay
    (chunk-local cumulative for the chunked op), queries scaled by 1/sqrt(K).

Parity status: every function here is pinned by `tests/test_oracle_*.py`
(closed forms, invariants, brute force on tiny inputs, finite differences,
a hand-computed golden case).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None

LOG2E = 1.0 / math.log(2.0)
LN2 = math.log(2.0)


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (FP64, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
                               "-std=c11", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        i64, dbl, p = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.kda_oracle_fwd.argtypes = [i64, p, p, i64, i64, i64, i64, dbl] + [p] * 8
        lib.kda_oracle_fwd.restype = ctypes.c_int
        lib.kda_oracle_bwd.argtypes = [i64, p, p, i64, i64, i64, i64, dbl] + [p] * 14
        lib.kda_oracle_bwd.restype = ctypes.c_int
        lib.kda_oracle_num_threads.restype = ctypes.c_int
        lib.kda_oracle_set_threads.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def num_threads() -> int:
    return _load().kda_oracle_num_threads()


def set_threads(n: int) -> None:
    _load().kda_oracle_set_threads(int(n))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


# --------------------------------------------------------------------------- gate

def softplus(x: np.ndarray) -> np.ndarray:
    """softplus(x) = log(1 + exp(x)), returning x itself above 20 (PyTorch's
    default threshold; the pages name softplus without printing a formula)."""
    x = _f64(x)
    with np.errstate(over="ignore"):
        return np.where(x > 20.0, x, np.log1p(np.exp(np.minimum(x, 20.0))))


def gate_activation(x: np.ndarray, A_log: Optional[np.ndarray],
                    dt_bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Per-token natural-log decay g = -exp(A_log[hv]) * softplus(x + dt_bias[hv, c]).

    x: [..., HV, K]; A_log: [HV] or None. None means unit scale, which is
    identical to an explicit zero A_log (PR #1294 Summary). dt_bias: [HV, K]
    (or flat HV*K) or None (no bias); the pages name a gate bias and its
    gradient (PR #1294 commit list, "Reduce GDN/KDA gate bias gradients
    before downcasting") without printing where it enters: here it is added
    to the raw input before the softplus."""
    x = _f64(x)
    HV, K = x.shape[-2], x.shape[-1]
    scale = np.ones(HV) if A_log is None else np.exp(_f64(A_log))
    u = x if dt_bias is None else x + _f64(dt_bias).reshape(HV, K)
    return -scale[:, None] * softplus(u)


def sigmoid(x: np.ndarray) -> np.ndarray:
    """Derivative of `softplus` above: 1 / (1 + exp(-x)), exactly 1 above 20
    where softplus returns its argument."""
    x = _f64(x)
    with np.errstate(over="ignore"):
        return np.where(x > 20.0, 1.0, 1.0 / (1.0 + np.exp(-x)))


def gate_activation_bwd(x: np.ndarray, A_log: Optional[np.ndarray],
                        dt_bias: Optional[np.ndarray], dg: np.ndarray,
                        cu_seqlens=None):
    """Reverse of `gate_activation` for the gradient dg of the per-token gate g.

    x, dg: [B, T, HV, K]. Returns (dx, dA_log, d_dt_bias):
      dx[t, h, c]    = dg * dg/dx = -exp(A_log[h]) * sigmoid(x + dt_bias[h, c]) * dg
      dA_log[h]      = sum over tokens and channels of dg * g   (dg/dA_log = g)
      d_dt_bias[h, c] = sum over tokens of dx                  (dg/ddt_bias = dg/dx)
    dA_log is None when A_log is None and d_dt_bias is None when dt_bias is
    None (no parameter). Only tokens inside a sequence (dense: every token;
    varlen: [cu[n], cu[n+1])) enter the sums; dx of other tokens is NaN."""
    x, dg = _f64(x), _f64(dg)
    B, T, HV, K = x.shape
    scale = np.ones(HV) if A_log is None else np.exp(_f64(A_log))
    u = x if dt_bias is None else x + _f64(dt_bias).reshape(HV, K)
    g = -scale[:, None] * softplus(u)
    dx_all = -scale[:, None] * sigmoid(u) * dg
    inside = np.zeros(B * T, dtype=bool)
    for bos, eos in seq_bounds(B, T, cu_seqlens):
        inside[bos:eos] = True
    inside = inside.reshape(B, T)
    dx = np.where(inside[:, :, None, None], dx_all, np.nan)
    dA = None if A_log is None else (dg * g)[inside].sum(axis=(0, 2))
    db = None if dt_bias is None else dx_all[inside].sum(axis=0)
    return dx, dA, db


# Stabiliser of the q/k normalisation. The pages name an l2norm step applied to
# q and k before the scan ("kda in torchtitan (training)": the attention-gym
# imports next to recurrent_kda) without printing it; the plainest reading is
# x / sqrt(sum x^2 + eps) over the K channels of each (token, head), with eps
# chosen here as 1e-6.
L2NORM_EPS = 1e-6


def l2norm(x: np.ndarray, eps: float = L2NORM_EPS) -> np.ndarray:
    """x / sqrt(sum over the last axis of x^2 + eps), in FP64."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU z * logistic(z) = z / (1 + exp(-z)), in FP64 (no threshold)."""
    z = _f64(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


# Widths of the short convolution the fused forward accepts. The pages name a
# short causal depthwise convolution followed by SiLU on q, k and v
# (ShortConvolution and causal_conv1d_silu imports on the Paddle compatibility
# page and the torchtitan training page) without printing it.
CONV_MAX_WIDTH = 4


def short_conv_silu(x: np.ndarray, weight: np.ndarray, bias: Optional[np.ndarray],
                    cu_seqlens=None, state: Optional[np.ndarray] = None,
                    return_state: bool = False):
    """Causal depthwise convolution along the tokens of each sequence, then SiLU.

    x: [B, T, D] (any trailing shape is flattened to D channels); weight
    [D, W]; bias [D] or None. Reading of the pages' ShortConvolution: a
    PyTorch Conv1d cross-correlation per channel, so weight[c, W - 1]
    multiplies the current token:
        z[t, c] = bias[c] + sum_{j<W} weight[c, j] * x[t - (W - 1) + j, c]
        y[t, c] = silu(z[t, c]).
    Before a sequence's first token x is the sequence's carried history:
    state[n, W - 1 + p, c] for the p-th position before it (p = -1 .. -(W-1);
    state is [N, W - 1, D], oldest row first), or zero when state is None.
    Sequences are the batch rows (dense) or [cu[n], cu[n+1]) of the packed rows
    (varlen); tokens outside every sequence are NaN.
    return_state: also return the history a following segment would carry,
    [N, W - 1, D]: the last W - 1 inputs of each sequence, reaching back into
    `state` (or zeros) when the sequence is shorter than W - 1."""
    x = _f64(x)
    B, T = x.shape[:2]
    D = int(np.prod(x.shape[2:]))
    w = _f64(weight).reshape(D, -1)
    W = w.shape[1]
    b = np.zeros(D) if bias is None else _f64(bias).reshape(D)
    flat = x.reshape(B * T, D)
    out = np.full_like(flat, np.nan)
    bounds = seq_bounds(B, T, cu_seqlens)
    st_out = np.zeros((len(bounds), W - 1, D))
    for n, (bos, eos) in enumerate(bounds):
        hist = np.zeros((W - 1, D)) if state is None else _f64(state)[n].reshape(W - 1, D)
        seq = np.concatenate([hist, flat[bos:eos]], axis=0)  # position p at row W - 1 + p
        for t in range(bos, eos):
            r = W - 1 + (t - bos)
            z = b.copy()
            for j in range(W):
                z = z + w[:, j] * seq[r - (W - 1) + j]
            out[t] = silu(z)
        st_out[n] = seq[len(seq) - (W - 1):] if W > 1 else st_out[n]
    y = out.reshape(x.shape)
    return (y, st_out) if return_state else y


def preprocess(q: np.ndarray, k: np.ndarray, v: np.ndarray, conv=None, qk_l2norm: bool = False,
               cu_seqlens=None):
    """The pre-processing the fused forward applies before the scan: the short
    convolution + SiLU of q, k and v (conv = ((wq, bq), (wk, bk), (wv, bv)) or
    None), then the optional q/k L2 normalisation (after the convolution, as
    the layer applies them). Returns (q, k, v) in FP64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    if conv is not None:
        (wq, bq), (wk, bk), (wv, bv) = conv
        q = short_conv_silu(q, wq, bq, cu_seqlens)
        k = short_conv_silu(k, wk, bk, cu_seqlens)
        v = short_conv_silu(v, wv, bv, cu_seqlens)
    if qk_l2norm:
        q, k = l2norm(q), l2norm(k)
    return q, k, v


def seq_bounds(B: int, T: int, cu_seqlens: Optional[Sequence[int]]):
    if cu_seqlens is None:
        return [(b * T, (b + 1) * T) for b in range(B)]
    cu = [int(c) for c in cu_seqlens]
    return [(cu[n], cu[n + 1]) for n in range(len(cu) - 1)]


def gate_cumsum_log2(g: np.ndarray, cu_seqlens, chunk_size: int) -> np.ndarray:
    """Chunk-local inclusive cumsum of the natural-log gate, in log2 units.

    g: [B, T, HV, K] (natural log). Chunks tile each sequence from its own
    start (dense: each batch row is one sequence); the last chunk of a
    sequence may be partial. chunk_size=1 gives the per-token log2 decay that
    the recurrent op consumes. Tokens outside every sequence stay NaN."""
    g = _f64(g)
    B, T = g.shape[:2]
    flat = g.reshape(B * T, *g.shape[2:])
    out = np.full_like(flat, np.nan)
    for bos, eos in seq_bounds(B, T, cu_seqlens):
        for c0 in range(bos, eos, chunk_size):
            c1 = min(c0 + chunk_size, eos)
            out[c0:c1] = np.cumsum(flat[c0:c1], axis=0) * LOG2E
    return out.reshape(g.shape)


# --------------------------------------------------------------------------- recurrence

def recurrence(q, k, v, g, beta, h0=None, cu_seqlens=None, scale=None):
    """FP64 token recurrence (C). Shapes: q, k [B,T,H,K]; v [B,T,HV,V];
    g [B,T,HV,K] natural log; beta [B,T,HV]; h0 [N,HV,K,V] or None.
    Returns (o [B,T,HV,V] with NaN outside every sequence, ht [N,HV,K,V])."""
    q, k, v, g, beta = (_f64(a) for a in (q, k, v, g, beta))
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    bounds = seq_bounds(B, T, cu_seqlens)
    N = len(bounds)
    bos = np.array([b for b, _ in bounds], dtype=np.int64)
    eos = np.array([e for _, e in bounds], dtype=np.int64)
    h0d = None if h0 is None else _f64(h0)
    if h0d is not None:
        assert h0d.shape == (N, HV, K, V)
    o = np.full((B, T, HV, V), np.nan)
    ht = np.zeros((N, HV, K, V))
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    rc = _load().kda_oracle_fwd(N, _ptr(bos), _ptr(eos), H, HV, K, V, float(scale),
                                _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0d),
                                _ptr(o), _ptr(ht))
    if rc != 0:
        raise ValueError("kda_oracle_fwd rejected its arguments")
    return o, ht


def recurrence_bwd(q, k, v, g, beta, do, h0=None, dht=None, cu_seqlens=None, scale=None):
    """Reverse pass of `recurrence`. Returns dict dq, dk, dv, dg, dbeta, dh0 (FP64)."""
    q, k, v, g, beta, do = (_f64(a) for a in (q, k, v, g, beta, do))
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    bounds = seq_bounds(B, T, cu_seqlens)
    N = len(bounds)
    bos = np.array([b for b, _ in bounds], dtype=np.int64)
    eos = np.array([e for _, e in bounds], dtype=np.int64)
    h0d = None if h0 is None else _f64(h0)
    dhtd = None if dht is None else _f64(dht)
    dq = np.zeros((B, T, H, K)); dk = np.zeros((B, T, H, K))
    dv = np.zeros((B, T, HV, V)); dg = np.zeros((B, T, HV, K))
    dbeta = np.zeros((B, T, HV)); dh0 = np.zeros((N, HV, K, V))
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    rc = _load().kda_oracle_bwd(N, _ptr(bos), _ptr(eos), H, HV, K, V, float(scale),
                                _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0d),
                                _ptr(do), _ptr(dhtd), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
                                _ptr(dbeta), _ptr(dh0))
    if rc != 0:
        raise ValueError("kda_oracle_bwd rejected its arguments")
    return dict(dq=dq, dk=dk, dv=dv, dg=dg, dbeta=dbeta, dh0=dh0)


# --------------------------------------------------------------------------- workload helpers

def forward(wl, A_log="workload", h0="workload", g_override=None):
    """Oracle forward of a `workloads.Workload`: gate activation from the raw
    x (FP64) and the token recurrence. Returns (o, ht)."""
    a = wl.A_log if (isinstance(A_log, str) and A_log == "workload") else A_log
    s = wl.h0 if (isinstance(h0, str) and h0 == "workload") else h0
    g = gate_activation(wl.x, a) if g_override is None else g_override
    return recurrence(wl.q, wl.k, wl.v, g, wl.beta, s, wl.cu_seqlens)


def backward(wl):
    g = gate_activation(wl.x, wl.A_log)
    return recurrence_bwd(wl.q, wl.k, wl.v, g, wl.beta, wl.dO, wl.h0, wl.dht, wl.cu_seqlens)


def g_from_log2_cumsum(G2: np.ndarray, cu_seqlens, chunk_size: int) -> np.ndarray:
    """Inverse of gate_cumsum_log2 on exactly given values: per-token natural-log
    gate g_t = ln2 * (G2_t - G2_{t-1}) within each chunk (G2_{-1} = 0), in FP64.
    Lets a stage test feed a given fp32 log2 gate to the recurrence."""
    G2 = _f64(G2)
    B, T = G2.shape[:2]
    flat = G2.reshape(B * T, *G2.shape[2:])
    out = np.full_like(flat, np.nan)
    for bos, eos in seq_bounds(B, T, cu_seqlens):
        for c0 in range(bos, eos, chunk_size):
            c1 = min(c0 + chunk_size, eos)
            blk = flat[c0:c1]
            prev = np.concatenate([np.zeros_like(blk[:1]), blk[:-1]], axis=0)
            out[c0:c1] = (blk - prev) * LN2
    return out.reshape(G2.shape)


from . import forms  # noqa: E402,F401
