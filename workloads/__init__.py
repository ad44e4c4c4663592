"""Seeded synthetic inputs for the KDA (Kimi Delta Attention) scan.

This module is shared by the CPU oracle tests, the GPU parity tests and the
benchmark. It only draws random numbers and shapes them; it holds none of the
method's arithmetic (no gate activation, no cumsum, no recurrence). The
L2 normalisation of q and k and the sigmoid of the beta logits belong to the
input recipe of the workloads (q, k ~ N(0,1) then L2-normalised per head;
beta = sigmoid(N(0,1))), not to the scan itself.

Every tensor is returned as a NumPy float32 array whose values are exactly
representable in the workload's dtype (bf16-rounded where the workload is
bf16), so the oracle can upcast the very values the GPU receives.

Draw order (fixed): q, k, v, beta logits, gate x, A_log, h0, dO, dht, lengths.
One PCG64 stream per workload, seeded 20261200 + workload number.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = ["Workload", "make", "round_bf16", "WORKLOADS", "tiny_case"]


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even), returned as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    nan = np.isnan(a)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def _l2norm_last(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / np.maximum(n, 1e-12)).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


@dataclass
class Workload:
    """One synthetic KDA problem.

    Layouts (row-major): q, k [B, T, H, K]; v [B, T, HV, V]; beta [B, T, HV];
    x (raw gate input) [B, T, HV, K]; A_log [HV] or None (unit scale);
    h0 [N, HV, K, V] or None; cu_seqlens int32 [N+1] or None (dense);
    dO [B, T, HV, V] and dht [N, HV, K, V] only for backward workloads.
    For varlen workloads B == 1 and T is the physical capacity; tokens in
    [cu_seqlens[-1], T) are outside the contract (poisoned with NaN here).
    """

    name: str
    dtype: str  # "fp32" or "bf16": dtype of q, k, v, beta and o
    B: int
    T: int
    H: int
    HV: int
    K: int
    V: int
    chunk_size: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    beta: np.ndarray
    x: np.ndarray
    A_log: Optional[np.ndarray]
    h0: Optional[np.ndarray]
    cu_seqlens: Optional[np.ndarray]
    dO: Optional[np.ndarray] = None
    dht: Optional[np.ndarray] = None
    notes: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        return self.B if self.cu_seqlens is None else len(self.cu_seqlens) - 1

    @property
    def tokens(self) -> int:
        """In-contract tokens."""
        if self.cu_seqlens is None:
            return self.B * self.T
        return int(self.cu_seqlens[-1])

    def seq_bounds(self):
        """List of (bos, eos) flat token offsets per sequence (flat index = b*T + t)."""
        if self.cu_seqlens is None:
            return [(b * self.T, (b + 1) * self.T) for b in range(self.B)]
        cu = self.cu_seqlens
        return [(int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]


def _rnd(dtype, a):
    return round_bf16(a) if dtype == "bf16" else np.ascontiguousarray(a, dtype=np.float32)


def _draw_common(rng, dtype, B, T, H, HV, K, V):
    q = _l2norm_last(rng.standard_normal((B, T, H, K), dtype=np.float32))
    k = _l2norm_last(rng.standard_normal((B, T, H, K), dtype=np.float32))
    v = rng.standard_normal((B, T, HV, V), dtype=np.float32)
    bl = rng.standard_normal((B, T, HV), dtype=np.float32)
    x = rng.standard_normal((B, T, HV, K), dtype=np.float32)
    return _rnd(dtype, q), _rnd(dtype, k), _rnd(dtype, v), _rnd(dtype, _sigmoid(bl)), x


def workload1(dense: bool = False) -> Workload:
    """Tiny FP32 scan: B=1, T=73, H=1, HV=2, K=V=64, cu_seqlens [0,3,73]."""
    rng = np.random.Generator(np.random.PCG64(20261201))
    B, T, H, HV, K, V = 1, 73, 1, 2, 64, 64
    q, k, v, beta, x = _draw_common(rng, "fp32", B, T, H, HV, K, V)
    A_log = np.zeros(HV, dtype=np.float32)
    n = 1 if dense else 2
    h0 = (0.1 * rng.standard_normal((2, HV, K, V), dtype=np.float32))[:n].copy()
    cu = None if dense else np.array([0, 3, 73], dtype=np.int32)
    return Workload("tiny_fp32_dense" if dense else "tiny_fp32_varlen", "fp32", B, T, H, HV, K, V, 64,
                    q, k, v, beta, x, A_log, h0, cu)


def workload2(B: int = 4, T: int = 4096) -> Workload:
    """Dense bf16 chunk forward: B=4, T=4096, H=HV=16, K=V=128, A_log ~ U(0, ln 16)."""
    rng = np.random.Generator(np.random.PCG64(20261202))
    H = HV = 16
    K = V = 128
    q, k, v, beta, x = _draw_common(rng, "bf16", B, T, H, HV, K, V)
    A_log = rng.uniform(0.0, math.log(16.0), size=HV).astype(np.float32)
    return Workload(f"dense_bf16_B{B}_T{T}_H16_K128", "bf16", B, T, H, HV, K, V, 64,
                    q, k, v, beta, x, A_log, None, None)


def varlen_lengths(rng, n_seq: int, total: int, max_len: int) -> np.ndarray:
    """Lengths ~ exp(U(0, ln max_len)), renormalised to `total` (floor, each >= 1,
    remainder to the longest)."""
    raw = np.exp(rng.uniform(0.0, math.log(max_len), size=n_seq))
    lens = np.maximum(np.floor(raw / raw.sum() * total).astype(np.int64), 1)
    lens[int(np.argmax(lens))] += total - int(lens.sum())
    assert lens.sum() == total and (lens >= 1).all()
    return lens


def workload3(total: int = 32768, n_seq: int = 16, max_len: int = 8192, tail: int = 512,
              empty_at=(0, 9, 18), H: int = 16, HV: int = 32, K: int = 128, V: int = 128) -> Workload:
    """Packed varlen + GVA, bf16: 16 sequences + 3 empty slots, capacity tail of 512."""
    rng = np.random.Generator(np.random.PCG64(20261203))
    T = total + tail
    q, k, v, beta, x = _draw_common(rng, "bf16", 1, T, H, HV, K, V)
    N = n_seq + len(empty_at)
    h0 = 0.1 * rng.standard_normal((N, HV, K, V), dtype=np.float32)
    lens = varlen_lengths(rng, n_seq, total, max_len)
    seq_lens = []
    it = iter(lens.tolist())
    for slot in range(N):
        seq_lens.append(0 if slot in empty_at else next(it))
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seq_lens)
    # capacity tail: outside the contract, poisoned so any read shows up
    for a in (q, k):
        a[:, total:] = np.nan
    for a in (v, beta, x):
        a[:, total:] = np.nan
    return Workload(f"varlen_gva_bf16_{total}tok_HV{HV}", "bf16", 1, T, H, HV, K, V, 64,
                    q, k, v, beta, x, np.zeros(HV, dtype=np.float32), h0, cu,
                    notes={"lengths": seq_lens, "capacity": T})


def workload4(slots: int = 256, n_empty: int = 26, H: int = 16, HV: int = 32, K: int = 128,
              V: int = 128) -> Workload:
    """Varlen decode: 256 slots, 1 token each, 26 empty (0 and 255 among them)."""
    rng = np.random.Generator(np.random.PCG64(20261204))
    T = slots - n_empty
    q, k, v, beta, x = _draw_common(rng, "bf16", 1, T, H, HV, K, V)
    h0 = 0.1 * rng.standard_normal((slots, HV, K, V), dtype=np.float32)
    others = rng.permutation(np.arange(1, slots - 1))[: n_empty - 2]
    empty = set([0, slots - 1] + others.tolist())
    seq_lens = [0 if s in empty else 1 for s in range(slots)]
    cu = np.zeros(slots + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seq_lens)
    assert cu[-1] == T
    return Workload(f"decode_bf16_{slots}slots_HV{HV}", "bf16", 1, T, H, HV, K, V, 1,
                    q, k, v, beta, x, None, h0, cu, notes={"empty": sorted(empty)})


def workload5(T: int = 65536, H: int = 32, HV: int = 32, K: int = 128, V: int = 128,
              with_grads: bool = True) -> Workload:
    """Long-context bf16 forward + backward: B=1, T=65536, H=HV=32, nonzero h0."""
    rng = np.random.Generator(np.random.PCG64(20261205))
    q, k, v, beta, x = _draw_common(rng, "bf16", 1, T, H, HV, K, V)
    h0 = 0.1 * rng.standard_normal((1, HV, K, V), dtype=np.float32)
    dO = dht = None
    if with_grads:
        dO = round_bf16(rng.standard_normal((1, T, HV, V), dtype=np.float32))
        dht = 0.1 * rng.standard_normal((1, HV, K, V), dtype=np.float32)
    return Workload(f"long_bf16_T{T}_H{HV}", "bf16", 1, T, H, HV, K, V, 64,
                    q, k, v, beta, x, np.zeros(HV, dtype=np.float32), h0, None, dO, dht)


def tiny_case(seed: int, B: int = 1, T: int = 20, H: int = 1, HV: int = 1, K: int = 8, V: int = 6,
              dtype: str = "fp32", cu_seqlens=None, h0: bool = True, grads: bool = False,
              A_log: Optional[float] = 0.0, gate_scale: float = 1.0) -> Workload:
    """Small random case for oracle pins and small GPU parity runs.

    cu_seqlens (a list) selects the varlen layout (then B must be 1 and N = len-1).
    A_log=None leaves it omitted (unit scale). gate_scale multiplies the raw gate
    input x to reach stronger or weaker decays.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    q, k, v, beta, x = _draw_common(rng, dtype, B, T, H, HV, K, V)
    x = (x * np.float32(gate_scale)).astype(np.float32)
    N = B if cu_seqlens is None else len(cu_seqlens) - 1
    a = None if A_log is None else np.full(HV, A_log, dtype=np.float32)
    hs = (0.1 * rng.standard_normal((N, HV, K, V), dtype=np.float32)) if h0 else None
    dO = dht = None
    if grads:
        dO = _rnd(dtype, rng.standard_normal((B, T, HV, V), dtype=np.float32))
        dht = 0.1 * rng.standard_normal((N, HV, K, V), dtype=np.float32)
    cu = None if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int32)
    return Workload(f"tiny_{seed}", dtype, B, T, H, HV, K, V, 64, q, k, v, beta, x, a, hs, cu, dO, dht)


WORKLOADS = {
    1: workload1,
    2: workload2,
    3: workload3,
    4: workload4,
    5: workload5,
}


def make(n: int, **kw) -> Workload:
    return WORKLOADS[n](**kw)


def with_raw_projections(wl: Workload, seed: int, width: int = 4, bias: bool = True,
                         tap_scale: float = 1.0):
    """Inputs of the fused short-convolution forward: replaces q, k, v of `wl`
    by raw projections ~ N(0, 1) (rounded to the workload dtype) and draws the
    FP32 taps [channels, width] and biases [channels] of the q, k and v
    convolutions from U(-b, b), b = tap_scale / sqrt(width) (PyTorch's default
    Conv1d initialisation for a depthwise filter: fan-in = width). Returns
    (wl, taps) with taps = ((wq, bq), (wk, bk), (wv, bv)), biases None when
    bias is False."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B, T, H, HV, K, V = wl.B, wl.T, wl.H, wl.HV, wl.K, wl.V
    wl.q = _rnd(wl.dtype, rng.standard_normal((B, T, H, K), dtype=np.float32))
    wl.k = _rnd(wl.dtype, rng.standard_normal((B, T, H, K), dtype=np.float32))
    wl.v = _rnd(wl.dtype, rng.standard_normal((B, T, HV, V), dtype=np.float32))
    lim = tap_scale / math.sqrt(width)
    taps = []
    for D in (H * K, H * K, HV * V):
        w = rng.uniform(-lim, lim, (D, width)).astype(np.float32)
        b = rng.uniform(-lim, lim, D).astype(np.float32) if bias else None
        taps.append((w, b))
    return wl, tuple(taps)
