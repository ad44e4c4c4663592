"""Short-T, many-chain cases: enough (sequence, value head) chains that the
scans take their wide value-column blocks. The forward scan picks the widest of
64 / 32 / 16 value columns per workgroup that still gives every compute unit a
workgroup (FP32 with K = 128 stops at 32: the 64-column tile set does not fit
its register file); the backward's two recurrences pick 32 columns when that
still fills the device, else 16. Every chain is compared with the oracle."""
import numpy as np
import pytest
import torch

import gated_delta_rule_69_amd as kda
import oracle
import workloads
from helpers import (check_parity, device_inputs, in_contract_rows, normwise_max_err, rel_rms,
                     tdtype, to_dev, to_np)

pytestmark = pytest.mark.gpu


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _fwd_block(chains, V, dtype, K):
    bv = 64
    while bv > 16 and chains * (V // bv) < _cus():
        bv //= 2
    bv = min(bv, V)
    if dtype == "fp32" and K == 128:
        bv = min(bv, 32)
    return bv


def _varlen_cu(seed, n_seq, T_max):
    """n_seq ragged lengths in [0, T_max] (a few empty), packed."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(0, T_max + 1, n_seq)
    lens[::7] = 0
    lens[1] = T_max
    return [0] + np.cumsum(lens).tolist()


FWD = [
    # dtype, K, V, B, H, HV, varlen sequences (None: dense)
    ("bf16", 128, 128, 8, 16, 16, None),   # 128 chains -> 64 columns
    ("bf16", 128, 128, 4, 16, 16, None),   # 64 chains -> 32 columns
    ("bf16", 64, 64, 16, 16, 16, None),    # 256 chains -> 64 columns (= V)
    ("bf16", 64, 128, 8, 8, 16, None),     # GVA, 128 chains -> 64
    ("bf16", 128, 64, 16, 16, 16, None),   # 256 chains -> 64 (= V)
    ("bf16", 128, 128, 1, 2, 4, 40),       # varlen + GVA, 160 chains -> 64
    ("fp32", 128, 128, 8, 16, 16, None),   # FP32 K = 128 -> 32 columns
    ("fp32", 64, 64, 16, 16, 16, None),    # 64
    ("fp32", 64, 128, 4, 16, 16, None),    # 32
    ("fp32", 128, 64, 16, 16, 16, None),   # FP32 K = 128 -> 32 (of V = 64)
]


@pytest.mark.parametrize("dtype,K,V,B,H,HV,nseq", FWD)
def test_forward_wide_blocks(dtype, K, V, B, H, HV, nseq):
    T = 130  # two full chunks and a 2-token tail
    cu = None
    if nseq is not None:
        cu = _varlen_cu(600 + K + V, nseq, T)
        T = cu[-1] + 9  # a capacity tail
    wl = workloads.tiny_case(500 + K + V + B + HV, B=B, T=T, H=H, HV=HV, K=K, V=V, dtype=dtype,
                             cu_seqlens=cu, A_log=1.0)
    chains = wl.N * HV
    bv = _fwd_block(chains, V, dtype, K)
    d = device_inputs(wl)
    o = torch.full_like(d["v"], 3.0)
    G = kda.gate_cumsum(d["x"], d["A_log"], d["cu"], 64)
    o, ht = kda.chunk_kda(d["q"], d["k"], d["v"], G, d["beta"], d["h0"], cu_seqlens=d["cu"],
                          output_final_state=True, o=o)
    torch.cuda.synchronize()
    if cu is not None:
        assert (to_np(o[:, cu[-1]:]) == 3.0).all(), "capacity tail written"
    o_ref, h_ref = oracle.forward(wl)
    check_parity(wl, o, ht, o_ref, h_ref, f"{dtype} K{K} V{V} {chains} chains, {bv} columns")


BWD = [
    # dtype, K, V, B, H, HV, varlen sequences
    ("bf16", 128, 128, 4, 16, 16, None),   # 64 chains -> 32 columns
    ("bf16", 64, 64, 8, 16, 16, None),     # 128 chains -> 32
    ("bf16", 128, 64, 8, 16, 16, None),    # 128 chains -> 32
    ("bf16", 64, 128, 4, 8, 16, None),     # GVA, 64 chains -> 32
    ("bf16", 128, 128, 1, 2, 4, 20),       # varlen + GVA, 80 chains -> 32
    ("fp32", 64, 64, 8, 16, 16, None),     # 128 chains -> 32
    ("fp32", 64, 128, 4, 16, 16, None),    # 64 chains -> 32
    ("bf16", 128, 128, 2, 16, 16, None),   # 32 chains -> 16 (the narrow case beside them)
]


@pytest.mark.parametrize("dtype,K,V,B,H,HV,nseq", BWD)
def test_backward_wide_blocks(dtype, K, V, B, H, HV, nseq):
    T = 130
    cu = None
    if nseq is not None:
        cu = _varlen_cu(700 + K + V, nseq, T)
        T = cu[-1] + 5
    wl = workloads.tiny_case(520 + K + V + B + HV, B=B, T=T, H=H, HV=HV, K=K, V=V, dtype=dtype,
                             cu_seqlens=cu, A_log=1.0, grads=True)
    chains = wl.N * HV
    cols = 32 if chains * (V // 32) >= _cus() else 16
    d = device_inputs(wl)
    dt = tdtype(wl)
    dO = to_dev(np.nan_to_num(wl.dO), dt)
    G = kda.gate_cumsum(d["x"], d["A_log"], d["cu"], 64)
    got = kda.chunk_kda_bwd(d["q"], d["k"], d["v"], G, d["beta"], d["h0"], dO, to_dev(wl.dht),
                            cu_seqlens=d["cu"])
    torch.cuda.synchronize()
    g = oracle.gate_activation(wl.x, wl.A_log)
    dO_ref = np.nan_to_num(wl.dO.astype(np.float64))
    if cu is not None:
        dO_ref[:, cu[-1]:] = 0.0
    ref = oracle.recurrence_bwd(wl.q, wl.k, wl.v, g, wl.beta, dO_ref, wl.h0, wl.dht, cu)
    mask = in_contract_rows(wl)
    err = normwise_max_err if dtype == "fp32" else rel_rms
    tol = 2e-5 if dtype == "fp32" else 1e-2
    worst = {}
    bounds = wl.seq_bounds()
    for name in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        a = to_np(got[name])
        b = ref[name]
        if name == "dh0":
            worst[name] = max(err(a[n, h], b[n, h]) for n in range(wl.N) for h in range(HV))
            continue
        heads = a.shape[2]
        a = a.reshape(wl.B * wl.T, heads, -1)
        b = b.reshape(wl.B * wl.T, heads, -1)
        e = [err(a[s:t, h], b[s:t, h]) for (s, t) in bounds if t > s for h in range(heads)]
        worst[name] = max(e)
        assert err(a[mask.reshape(-1)], b[mask.reshape(-1)]) <= tol, name
    print(f"bwd {dtype} K{K} V{V} {chains} chains, {cols} columns: worst chain",
          {k_: f"{e_:.2e}" for k_, e_ in worst.items()})
    assert all(e <= tol for e in worst.values()), worst
