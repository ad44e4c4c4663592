"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times: the GPU runs the whole problem and the FP64 oracle the whole
problem too (OpenMP over chains); every (sequence, value head) chain is held
to the bar on its own. The backward is checked on a suffix of the long
context (the oracle's reverse pass over all of it is not needed for that)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_69_amd as kda
import oracle
import workloads
from helpers import chain_errors, check_parity, device_inputs, rel_rms, to_dev, to_np

pytestmark = pytest.mark.gpu


def _per_head_report(label, co, ch):
    """Print the worst chain of each value head (sorted worst first)."""
    worst_o = np.nanmax(co, axis=0)
    worst_h = ch.max(axis=0)
    order = np.argsort(-worst_o)
    print(f"{label}: worst chains by value head (o / state):",
          ", ".join(f"hv{hv} {worst_o[hv]:.2e}/{worst_h[hv]:.2e}" for hv in order[:6]))


def test_dense_B4_T4096_H16_every_chain():
    """The benchmark's dense workload, on the two-call path (kda_gate_cumsum +
    kda_chunk_fwd) and on the fused-gate call the benchmark times (bitwise
    equal to it); every one of the 64 (batch row, value head) chains against
    the oracle."""
    wl = workloads.workload2()
    d = device_inputs(wl)
    G = kda.gate_cumsum(d["x"], d["A_log"], None, 64)
    o, ht = kda.chunk_kda(d["q"], d["k"], d["v"], G, d["beta"], None, output_final_state=True)
    o2, h2 = kda.chunk_kda(d["q"], d["k"], d["v"], d["x"], d["beta"], None,
                           output_final_state=True, use_gate_in_kernel=True, A_log=d["A_log"])
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(ht.view(torch.int32), h2.view(torch.int32))
    o_ref, h_ref = oracle.forward(wl)
    check_parity(wl, o2, h2, o_ref, h_ref, "dense B4 T4096 H16 (fused gate)")
    co, ch = chain_errors(wl, o2, h2, o_ref, h_ref)
    _per_head_report("dense", co, ch)


def test_varlen_gva_32768_tokens_every_chain():
    """Packed varlen + GVA (16 sequences, 3 empty slots, capacity tail): every
    live (sequence, value head) chain against the oracle; empty slots bitwise;
    the tail untouched."""
    wl = workloads.workload3()
    d = device_inputs(wl)
    G = kda.gate_cumsum(d["x"], d["A_log"], d["cu"], 64)
    h_before = d["h0"].clone()
    o = torch.full_like(d["v"], 7.0)
    o, ht = kda.chunk_kda(d["q"], d["k"], d["v"], G, d["beta"], d["h0"], cu_seqlens=d["cu"],
                          output_final_state=True, o=o)
    torch.cuda.synchronize()
    tot = int(wl.cu_seqlens[-1])
    assert (to_np(o[:, tot:]) == 7.0).all(), "capacity tail written"
    lens = np.diff(wl.cu_seqlens)
    for s in np.nonzero(lens == 0)[0]:
        assert torch.equal(ht[s].view(torch.int32), h_before[s].view(torch.int32))
    o_ref, h_ref = oracle.forward(wl)
    check_parity(wl, o, ht, o_ref, h_ref, "varlen + GVA 32768 tokens")
    co, ch = chain_errors(wl, o, ht, o_ref, h_ref)
    live = int(np.isfinite(co).sum())
    assert live == int((lens > 0).sum()) * wl.HV
    print(f"varlen: {live} live chains compared")
    _per_head_report("varlen", co, ch)


def test_long_context_T65536_forward_every_head():
    wl = workloads.workload5(with_grads=False)
    d = device_inputs(wl)
    G = kda.gate_cumsum(d["x"], d["A_log"], None, 64)
    o, ht = kda.chunk_kda(d["q"], d["k"], d["v"], G, d["beta"], d["h0"], output_final_state=True)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle.forward(wl)
    check_parity(wl, o, ht, o_ref, h_ref, "long context T65536 H32")
    co, ch = chain_errors(wl, o, ht, o_ref, h_ref)
    _per_head_report("long context", co, ch)


def test_long_context_T65536_backward_suffix():
    """Full T=65536 backward on the GPU; the oracle checks the gradients of the
    last 256 tokens of every head: it runs the forward recurrence to token
    T-256 for the state there, then the reverse pass over the suffix with the
    same dht (a suffix's gradients depend on the past only through that
    state). dq and dk are compared per head (H == HV here)."""
    wl = workloads.workload5()
    d = device_inputs(wl)
    G = kda.gate_cumsum(d["x"], d["A_log"], None, 64)
    dO = to_dev(wl.dO, torch.bfloat16)
    got = kda.chunk_kda_bwd(d["q"], d["k"], d["v"], G, d["beta"], d["h0"], dO, to_dev(wl.dht))
    torch.cuda.synchronize()
    T, S = wl.T, 256
    pre = slice(0, T - S)
    g_all = oracle.gate_activation(wl.x, wl.A_log)
    _, s_mid = oracle.recurrence(wl.q[:, pre], wl.k[:, pre], wl.v[:, pre], g_all[:, pre],
                                 wl.beta[:, pre], wl.h0)
    sl = slice(T - S, T)
    ref = oracle.recurrence_bwd(wl.q[:, sl], wl.k[:, sl], wl.v[:, sl], g_all[:, sl],
                                wl.beta[:, sl], wl.dO[:, sl], s_mid, wl.dht)
    worst = {}
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        a = to_np(got[name][:, sl])
        per_head = [rel_rms(a[:, :, h], ref[name][:, :, h]) for h in range(a.shape[2])]
        worst[name] = max(per_head)
    print("long-context suffix, worst head per gradient:",
          {k_: f"{e_:.2e}" for k_, e_ in worst.items()})
    assert all(e <= 1e-2 for e in worst.values()), worst
