"""GPU edge cases of the chunked and recurrent paths: workspace contents,
batches with no tokens, one-token sequences, and beta = 0.

* The workspace is scratch the kernels fully write before they read it: a call
  with a workspace full of NaN bytes must give bitwise the outputs of a call
  with a zeroed one (forward and backward).
* A slot whose offset repeats holds no tokens and hands its state on unchanged,
  bit for bit (the attention-gym recurrent_kda description quoted in "kda in
  torchtitan (training)"); a batch where every slot is empty, or a dense batch
  with T = 0, is the degenerate case of that contract.
* beta = 0 removes the delta-rule write, so the state only decays:
  S_t = Diag(exp(sum_{s<=t} g_s)) S_0 and o_t = S_t^T q_t / sqrt(K), a closed
  form independent of the chunked algebra.
"""
import math

import numpy as np
import pytest
import torch

import gated_delta_rule_69_amd as kda
import oracle
import workloads
from helpers import (DEV, TOL_FP32, check_parity, device_inputs, in_contract_rows, normwise_max_err,
                     run_gpu, tdtype, to_dev, to_np)

pytestmark = pytest.mark.gpu


def _bits(t):
    """Integer view of a float tensor, for bitwise comparison (NaN == NaN)."""
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _same_bits(a, b):
    return torch.equal(_bits(a), _bits(b))


def _chunk_fwd(d, fused, ws):
    o = torch.full_like(d["v"], 7.0)  # rows outside the contract keep the sentinel
    if fused:
        return kda.chunk_kda(d["q"], d["k"], d["v"], d["x"], d["beta"], d["h0"], cu_seqlens=d["cu"],
                             output_final_state=True, o=o, workspace=ws, use_gate_in_kernel=True,
                             A_log=d["A_log"])
    G = kda.gate_cumsum(d["x"], d["A_log"], d["cu"], 64)
    return kda.chunk_kda(d["q"], d["k"], d["v"], G, d["beta"], d["h0"], cu_seqlens=d["cu"],
                         output_final_state=True, o=o, workspace=ws)


@pytest.mark.parametrize("dtype,K,V", [("fp32", 64, 64), ("bf16", 128, 128), ("bf16", 64, 128)])
@pytest.mark.parametrize("fused", [False, True])
def test_forward_workspace_contents_do_not_matter(dtype, K, V, fused):
    # varlen + GVA: a long sequence (3 chunks + tail), an empty slot, a short one
    wl = workloads.tiny_case(7100 + K + V, B=1, T=260, H=2, HV=4, K=K, V=V, dtype=dtype,
                             cu_seqlens=[0, 150, 150, 203, 250], A_log=1.0)
    d = device_inputs(wl)
    need = kda.chunk_workspace_bytes(d["q"], d["v"], d["cu"])
    outs = []
    for fill in (0, 0xFF):  # 0xFF bytes are NaN in both FP32 and bf16
        ws = torch.full((need,), fill, dtype=torch.uint8, device=DEV)
        outs.append(_chunk_fwd(d, fused, ws))
    torch.cuda.synchronize()
    (o0, h0), (o1, h1) = outs
    assert _same_bits(o0, o1) and _same_bits(h0, h1)
    assert not torch.isnan(h1).any()
    o_ref, ht_ref = oracle.forward(wl)
    check_parity(wl, o1, h1, o_ref, ht_ref, f"poisoned workspace {dtype} K{K} V{V}")


@pytest.mark.parametrize("dtype,K,V", [("fp32", 64, 64), ("bf16", 128, 128)])
def test_backward_workspace_contents_do_not_matter(dtype, K, V):
    wl = workloads.tiny_case(7200 + K, B=1, T=200, H=1, HV=2, K=K, V=V, dtype=dtype,
                             cu_seqlens=[0, 131, 131, 190], grads=True)
    d = device_inputs(wl)
    dt = tdtype(wl)
    dO = to_dev(wl.dO, dt)
    dht = to_dev(wl.dht)
    G = kda.gate_cumsum(d["x"], d["A_log"], d["cu"], 64)
    ws_bytes = kda.chunk_bwd_workspace_bytes(d["q"], d["v"], d["cu"])
    res = []
    for fill in (0, 0xFF):
        ws = torch.full((ws_bytes,), fill, dtype=torch.uint8, device=DEV)
        res.append(kda.chunk_kda_bwd(d["q"], d["k"], d["v"], G, d["beta"], d["h0"], dO, dht,
                                     cu_seqlens=d["cu"], workspace=ws))
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        assert _same_bits(res[0][name], res[1][name]), name
        assert not torch.isnan(res[1][name]).any(), name


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("with_h0", [True, False])
def test_every_slot_empty(dtype, with_h0):
    """cu_seqlens = [0, 0, 0, 0]: no token is in the contract. Inputs are NaN,
    the output keeps its sentinel, and every final state is the initial state
    bitwise (+0.0 without one), on the chunked (fused and two-call) and the
    recurrent path."""
    wl = workloads.tiny_case(7300, B=1, T=70, H=1, HV=2, K=64, V=64, dtype=dtype,
                             cu_seqlens=[0, 0, 0, 0], h0=with_h0)
    for a in (wl.q, wl.k, wl.v, wl.beta, wl.x):
        a[:] = np.nan
    d = device_inputs(wl)
    sentinel = torch.full_like(d["v"], 3.0)
    runs = []
    for fused in (False, True):
        o = sentinel.clone()
        if fused:
            runs.append(kda.chunk_kda(d["q"], d["k"], d["v"], d["x"], d["beta"], d["h0"],
                                      cu_seqlens=d["cu"], output_final_state=True, o=o,
                                      use_gate_in_kernel=True, A_log=d["A_log"]))
        else:
            G = kda.gate_cumsum(d["x"], d["A_log"], d["cu"], 64)
            runs.append(kda.chunk_kda(d["q"], d["k"], d["v"], G, d["beta"], d["h0"],
                                      cu_seqlens=d["cu"], output_final_state=True, o=o))
    G1 = kda.gate_cumsum(d["x"], d["A_log"], d["cu"], 1)
    runs.append(kda.recurrent_kda(d["q"], d["k"], d["v"], G1, d["beta"], d["h0"],
                                  cu_seqlens=d["cu"], output_final_state=True, o=sentinel.clone()))
    torch.cuda.synchronize()
    want = d["h0"] if with_h0 else torch.zeros((3, 2, 64, 64), device=DEV)
    for o, ht in runs:
        assert _same_bits(o, sentinel)
        assert _same_bits(ht, want)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_dense_batch_without_tokens(dtype):
    """B = 2, T = 0 (dense): every row is an empty sequence. The final state is
    the initial state bitwise, and the backward returns dh0 = dht bitwise (and
    +0.0 without dht), with grouped value heads (HV = 2H)."""
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    B, H, HV, K, V = 2, 1, 2, 64, 64
    g = torch.Generator(device="cpu").manual_seed(7400)
    q = torch.empty((B, 0, H, K), device=DEV, dtype=dt)
    k = torch.empty_like(q)
    v = torch.empty((B, 0, HV, V), device=DEV, dtype=dt)
    beta = torch.empty((B, 0, HV), device=DEV, dtype=dt)
    x = torch.empty((B, 0, HV, K), device=DEV, dtype=torch.float32)
    h0 = (0.1 * torch.randn((B, HV, K, V), generator=g)).to(DEV)
    dht = (0.1 * torch.randn((B, HV, K, V), generator=g)).to(DEV)
    G = kda.gate_cumsum(x, None, None, 64)
    G1 = kda.gate_cumsum(x, None, None, 1)
    _, ht_c = kda.chunk_kda(q, k, v, G, beta, h0, output_final_state=True)
    _, ht_f = kda.chunk_kda(q, k, v, x, beta, h0, output_final_state=True, use_gate_in_kernel=True)
    _, ht_r = kda.recurrent_kda(q, k, v, G1, beta, h0, output_final_state=True)
    torch.cuda.synchronize()
    for ht in (ht_c, ht_f, ht_r):
        assert _same_bits(ht, h0)
    do = torch.empty_like(v)
    r = kda.chunk_kda_bwd(q, k, v, G, beta, h0, do, dht)
    r0 = kda.chunk_kda_bwd(q, k, v, G, beta, h0, do, None)
    torch.cuda.synchronize()
    assert _same_bits(r["dh0"], dht)
    assert _same_bits(r0["dh0"], torch.zeros_like(dht))


@pytest.mark.parametrize("dtype,K,V", [("fp32", 64, 64), ("bf16", 128, 128)])
def test_one_token_sequences(dtype, K, V):
    """Sequences of one token between longer ones: each is a chunk of length 1
    whose only pair is the diagonal."""
    cu = [0, 1, 2, 3, 67, 68, 140]
    wl = workloads.tiny_case(7500 + K, B=1, T=150, H=1, HV=2, K=K, V=V, dtype=dtype,
                             cu_seqlens=cu, A_log=1.5)
    d = device_inputs(wl)
    o_ref, ht_ref = oracle.forward(wl)
    for path in ("chunk", "recurrent"):
        o, ht = run_gpu(wl, d, path)
        check_parity(wl, o, ht, o_ref, ht_ref, f"one-token {path} {dtype}")


def test_beta_zero_is_pure_decay():
    """beta = 0 on the chunked path (FP32) against the closed form of a pure
    per-channel decay: S_t = Diag(exp(G_t)) S_0 with G_t the running sum of the
    natural-log gate, o_t = S_t^T q_t / sqrt(K)."""
    cu = [0, 5, 150, 150, 200]
    wl = workloads.tiny_case(7600, B=1, T=210, H=1, HV=2, K=64, V=64, dtype="fp32",
                             cu_seqlens=cu, A_log=-3.0)  # decay scale e^-3: moderate total decay
    wl.beta[:] = 0.0
    d = device_inputs(wl)
    o, ht = run_gpu(wl, d, "chunk")
    g = np.asarray(oracle.gate_activation(wl.x, wl.A_log), dtype=np.float64)  # [1, T, HV, K]
    q = wl.q.astype(np.float64)
    K, HV = wl.K, wl.HV
    o_cf = np.zeros((wl.T, HV, wl.V))
    ht_cf = np.zeros((len(cu) - 1, HV, K, wl.V))
    for n in range(len(cu) - 1):
        bos, eos = cu[n], cu[n + 1]
        for hv in range(HV):
            h = hv // (HV // wl.H)
            S0 = wl.h0[n, hv].astype(np.float64)
            Gc = np.cumsum(g[0, bos:eos, hv, :], axis=0)  # [L, K]
            # o_t[v] = sum_c q_tc / sqrt(K) exp(G_tc) S0[c, v]
            o_cf[bos:eos, hv] = (q[0, bos:eos, h, :] / math.sqrt(K) * np.exp(Gc)) @ S0
            decay = np.exp(Gc[-1]) if eos > bos else np.ones(K)
            ht_cf[n, hv] = decay[:, None] * S0
    n_tok = cu[-1]
    og = to_np(o)[0, :n_tok]
    assert normwise_max_err(og, o_cf[:n_tok]) <= TOL_FP32
    assert normwise_max_err(to_np(ht), ht_cf) <= TOL_FP32
    # the empty slot passes its state through bitwise
    assert _same_bits(ht[2], d["h0"][2])


@pytest.mark.parametrize("N", [1023, 1100])
def test_many_sequences_in_any_order(N):
    """A packed batch of N sequences (empty ones, one-token ones, several
    chunks) on either side of the 1024 sequences up to which the chunk table
    orders the scans longest first: forward (every chain) and backward against
    the oracle, and the same batch with its sequences in reverse order gives
    the same per-sequence results bit for bit."""
    rng = np.random.default_rng(900 + N)
    lens = rng.integers(0, 40, size=N)
    lens[rng.choice(N, 6, replace=False)] = rng.integers(65, 200, size=6)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1]) + 5
    wl = workloads.tiny_case(901 + N, B=1, T=T, H=1, HV=2, K=64, V=64, dtype="fp32",
                             cu_seqlens=cu.tolist(), grads=True, A_log=0.5)
    d = device_inputs(wl)
    o, ht = _chunk_fwd(d, True, None)
    o_ref, ht_ref = oracle.forward(wl)
    check_parity(wl, o, ht, o_ref, ht_ref, label=f"{N} sequences")
    # reverse the sequences (the token rows move with them)
    order = np.arange(N)[::-1]
    rows = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in order] + [np.arange(cu[-1], T)])
    cu_r = np.concatenate([[0], np.cumsum(lens[order])]).astype(np.int32)
    dr = {kk: (t[:, torch.from_numpy(rows).to(DEV)] if kk in ("q", "k", "v", "beta", "x") else t)
          for kk, t in d.items()}
    dr["h0"] = d["h0"][torch.from_numpy(order.copy()).to(DEV)]
    dr["cu"] = torch.from_numpy(cu_r).to(DEV)
    o_r, ht_r = _chunk_fwd(dr, True, None)
    torch.cuda.synchronize()
    rows_t = torch.from_numpy(rows[: int(cu[-1])]).to(DEV)
    assert _same_bits(o[:, rows_t], o_r[:, : int(cu[-1])])
    assert _same_bits(ht[torch.from_numpy(order.copy()).to(DEV)], ht_r)
    # backward against the oracle's reverse pass
    dO = to_dev(np.nan_to_num(wl.dO))
    r = kda.chunk_kda_bwd(d["q"], d["k"], d["v"], d["x"], d["beta"], d["h0"], dO, to_dev(wl.dht),
                          cu_seqlens=d["cu"], use_gate_in_kernel=True, A_log=d["A_log"])
    g = oracle.gate_activation(wl.x, wl.A_log)
    dO_ref = np.nan_to_num(wl.dO.astype(np.float64))
    dO_ref[:, int(cu[-1]):] = 0.0
    ref = oracle.recurrence_bwd(wl.q, wl.k, wl.v, g, wl.beta, dO_ref, wl.h0, wl.dht, wl.cu_seqlens)
    m = in_contract_rows(wl)
    for name in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        a, b = to_np(r[name]), ref[name]
        if name != "dh0":
            a, b = a[m], b[m]
        assert normwise_max_err(a, b) <= TOL_FP32, name
