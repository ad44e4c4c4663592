"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times: the GPU runs the whole problem; the FP64 oracle recomputes
sampled (sequence, value head) chains one by one."""
import numpy as np
import pytest
import torch

import gated_delta_rule_69_amd as kda
import oracle
import workloads
from helpers import (DEV, TOL_BF16_O, TOL_BF16_STATE, device_inputs, rel_rms, to_dev, to_np)

pytestmark = pytest.mark.gpu


def _chain_ref(wl, n, hv, h0=None, upto=None):
    """Oracle forward of one (sequence n, value head hv) chain."""
    bos, eos = wl.seq_bounds()[n]
    if upto is not None:
        eos = min(eos, bos + upto)
    flat = lambda a: a.reshape(wl.B * wl.T, *a.shape[2:])
    h = hv // (wl.HV // wl.H)
    sl = slice(bos, eos)
    q = flat(wl.q)[sl, h][None, :, None]
    k = flat(wl.k)[sl, h][None, :, None]
    v = flat(wl.v)[sl, hv][None, :, None]
    b = flat(wl.beta)[sl, hv][None, :, None]
    x = flat(wl.x)[sl, hv][None, :, None]
    a = None if wl.A_log is None else wl.A_log[hv:hv + 1]
    g = oracle.gate_activation(x, a)
    s0 = None
    if h0 is not None:
        s0 = h0[n, hv][None, None]
    o, ht = oracle.recurrence(q, k, v, g, b, s0)
    return o[0, :, 0], ht[0, 0], (bos, eos)


def test_dense_B4_T4096_H16_sampled_chains():
    wl = workloads.workload2()
    d = device_inputs(wl)
    G = kda.gate_cumsum(d["x"], d["A_log"], None, 64)
    o, ht = kda.chunk_kda(d["q"], d["k"], d["v"], G, d["beta"], None, output_final_state=True)
    torch.cuda.synchronize()
    o = o.reshape(wl.B * wl.T, wl.HV, wl.V)
    # weakest and strongest decay heads, in different batch rows
    order = np.argsort(wl.A_log)
    for n, hv in ((0, int(order[0])), (3, int(order[-1])), (2, 7)):
        o_ref, h_ref, (bos, eos) = _chain_ref(wl, n, hv)
        eo = rel_rms(to_np(o[bos:eos, hv]), o_ref)
        eh = rel_rms(to_np(ht[n, hv]), h_ref)
        print(f"dense chain n={n} hv={hv} A_log={wl.A_log[hv]:.2f}: o {eo:.2e} state {eh:.2e}")
        assert eo <= TOL_BF16_O and eh <= TOL_BF16_STATE


def test_varlen_gva_32768_tokens_sampled():
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
    longest = int(np.argmax(lens))
    shortest = int(np.argmin(np.where(lens > 0, lens, 1 << 30)))
    o2 = o[0]
    for n, hv in ((longest, 0), (longest, 31), (shortest, 5), (4, 17)):
        o_ref, h_ref, (bos, eos) = _chain_ref(wl, n, hv, h0=wl.h0)
        eo = rel_rms(to_np(o2[bos:eos, hv]), o_ref)
        eh = rel_rms(to_np(ht[n, hv]), h_ref)
        print(f"varlen seq {n} (len {eos - bos}) hv={hv}: o {eo:.2e} state {eh:.2e}")
        assert eo <= TOL_BF16_O and eh <= TOL_BF16_STATE


def test_long_context_T65536_forward_sampled_heads():
    wl = workloads.workload5(with_grads=False)
    d = device_inputs(wl)
    G = kda.gate_cumsum(d["x"], d["A_log"], None, 64)
    o, ht = kda.chunk_kda(d["q"], d["k"], d["v"], G, d["beta"], d["h0"], output_final_state=True)
    torch.cuda.synchronize()
    for hv in (0, 21):
        o_ref, h_ref, (bos, eos) = _chain_ref(wl, 0, hv, h0=wl.h0)
        eo = rel_rms(to_np(o[0, :, hv]), o_ref)
        eh = rel_rms(to_np(ht[0, hv]), h_ref)
        print(f"long context hv={hv}: o {eo:.2e} state {eh:.2e}")
        assert eo <= TOL_BF16_O and eh <= TOL_BF16_STATE


def test_long_context_T65536_backward_suffix():
    """Full T=65536 backward on the GPU; the oracle checks the gradients of the
    last 256 tokens of two heads: it runs the forward recurrence to token
    T-256 for the state there, then the reverse pass over the suffix with the
    same dht (a suffix's gradients depend on the past only through that state)."""
    wl = workloads.workload5()
    d = device_inputs(wl)
    G = kda.gate_cumsum(d["x"], d["A_log"], None, 64)
    dO = to_dev(wl.dO, torch.bfloat16)
    got = kda.chunk_kda_bwd(d["q"], d["k"], d["v"], G, d["beta"], d["h0"], dO, to_dev(wl.dht))
    torch.cuda.synchronize()
    T, S = wl.T, 256
    for hv in (3, 30):
        _, s_mid, _ = _chain_ref(wl, 0, hv, h0=wl.h0, upto=T - S)
        sl = slice(T - S, T)
        q = wl.q[:, sl, hv:hv + 1]
        k = wl.k[:, sl, hv:hv + 1]
        v = wl.v[:, sl, hv:hv + 1]
        b = wl.beta[:, sl, hv:hv + 1]
        g = oracle.gate_activation(wl.x[:, sl, hv:hv + 1], wl.A_log[hv:hv + 1])
        ref = oracle.recurrence_bwd(q, k, v, g, b, wl.dO[:, sl, hv:hv + 1], s_mid[None, None],
                                    wl.dht[:, hv:hv + 1])
        errs = {}
        for name in ("dq", "dk", "dv", "dg", "dbeta"):
            a = to_np(got[name][:, sl, hv:hv + 1])
            errs[name] = rel_rms(a, ref[name])
        print(f"long-context suffix hv={hv}:", {k_: f"{e_:.2e}" for k_, e_ in errs.items()})
        assert all(e <= 1e-2 for e in errs.values()), errs
