"""torch.library ops (torch.ops.kda.chunk_kda_train with autograd,
torch.ops.kda.recurrent_kda): gradients through PyTorch autograd against the
FP64 oracle's reverse pass and gate backward, and opcheck of the
registrations (schema, fake tensors, autograd registration)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_69_amd as kda
import gated_delta_rule_69_amd.torch_ops  # noqa: F401  (registers torch.ops.kda.*)
import oracle
import workloads
from helpers import DEV, device_inputs, in_contract_rows, normwise_max_err, rel_rms, tdtype, to_dev, to_np

pytestmark = pytest.mark.gpu


def _case(dtype):
    wl = workloads.tiny_case(950, T=140, H=1, HV=2, K=64, V=64, dtype=dtype, cu_seqlens=[0, 3, 3, 130],
                             grads=True, A_log=0.4)
    wl.A_log = np.array([0.4, -0.3], dtype=np.float32)
    b = np.random.default_rng(951).standard_normal((2, 64)).astype(np.float32)
    return wl, b


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_chunk_kda_train_autograd_matches_oracle(dtype):
    wl, b = _case(dtype)
    dt = tdtype(wl)
    d = device_inputs(wl)
    leaves = dict(q=d["q"], k=d["k"], v=d["v"], x=d["x"], beta=d["beta"], A_log=d["A_log"],
                  dt_bias=to_dev(b), h0=d["h0"])
    for t in leaves.values():
        t.requires_grad_(True)
    n = int(wl.cu_seqlens[-1])
    W_o = np.nan_to_num(wl.dO.astype(np.float64))
    W_o[:, n:] = 0.0
    o, ht = torch.ops.kda.chunk_kda_train(leaves["q"], leaves["k"], leaves["v"], leaves["x"],
                                          leaves["beta"], leaves["A_log"], leaves["dt_bias"],
                                          leaves["h0"], d["cu"])
    loss = (o[:, :n].float() * to_dev(W_o[:, :n])).sum() + (ht * to_dev(wl.dht)).sum()
    grads = dict(zip(leaves, torch.autograd.grad(loss, list(leaves.values()))))
    torch.cuda.synchronize()
    # oracle: token recurrence reverse pass, then the gate backward
    g = oracle.gate_activation(wl.x, wl.A_log, b)
    r = oracle.recurrence_bwd(wl.q, wl.k, wl.v, g, wl.beta, W_o, wl.h0, wl.dht, wl.cu_seqlens)
    dx, dA, db = oracle.gate_activation_bwd(wl.x, wl.A_log, b, r["dg"], wl.cu_seqlens)
    ref = dict(q=r["dq"], k=r["dk"], v=r["dv"], x=dx, beta=r["dbeta"], A_log=dA, dt_bias=db, h0=r["dh0"])
    mask = in_contract_rows(wl)
    tol = 2e-5 if dtype == "fp32" else 1e-2
    errs = {}
    for name in ("q", "k", "v", "x", "beta", "h0"):
        a, c = to_np(grads[name]), ref[name]
        if name != "h0":
            a, c = a[mask], c[mask]
        errs[name] = normwise_max_err(a, c) if dtype == "fp32" else rel_rms(a, c)
    # the parameter gradients are sums with cancellation: bounded by tol times the
    # sum of the magnitudes of their terms
    mag_A = np.abs(r["dg"] * g)[mask].sum(axis=(0, 2))
    mag_b = np.abs(dx[mask]).sum(axis=0)
    errs["A_log"] = float(np.max(np.abs(to_np(grads["A_log"]) - dA) / mag_A))
    errs["dt_bias"] = float(np.max(np.abs(to_np(grads["dt_bias"]) - db) / mag_b))
    assert all(e <= tol for e in errs.values()), errs


def test_chunk_kda_train_forward_equals_entry_points_bitwise():
    wl, b = _case("bf16")
    d = device_inputs(wl)
    o, ht = torch.ops.kda.chunk_kda_train(d["q"], d["k"], d["v"], d["x"], d["beta"], d["A_log"],
                                          to_dev(b), d["h0"], d["cu"])
    G = kda.gate_cumsum(d["x"], d["A_log"], d["cu"], 64, dt_bias=to_dev(b))
    o2, ht2 = kda.chunk_kda(d["q"], d["k"], d["v"], G, d["beta"], d["h0"], cu_seqlens=d["cu"],
                            output_final_state=True)
    torch.cuda.synchronize()
    n = int(wl.cu_seqlens[-1])
    assert torch.equal(o[:, :n].view(torch.int16), o2[:, :n].view(torch.int16))
    assert torch.equal(ht.view(torch.int32), ht2.view(torch.int32))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_chunk_kda_train_without_bias_runs_fused_gate_bitwise(dtype):
    """Without dt_bias the op runs the gate step inside the kernels (fused-gate
    forward, kda_chunk_bwd_ex backward); with a zero dt_bias it forms the log2
    gate with kda_gate_cumsum_biased first (x + 0 = x). Outputs and every
    gradient agree bit for bit."""
    wl, _ = _case(dtype)
    d = device_inputs(wl)
    zero_b = torch.zeros((wl.HV, wl.K), device=DEV, dtype=torch.float32)
    n = int(wl.cu_seqlens[-1])
    W_o = np.nan_to_num(wl.dO.astype(np.float64))
    W_o[:, n:] = 0.0
    res = []
    for bias in (None, zero_b):
        leaves = dict(q=d["q"].clone(), k=d["k"].clone(), v=d["v"].clone(), x=d["x"].clone(),
                      beta=d["beta"].clone(), A_log=d["A_log"].clone(), h0=d["h0"].clone())
        for t in leaves.values():
            t.requires_grad_(True)
        o, ht = torch.ops.kda.chunk_kda_train(leaves["q"], leaves["k"], leaves["v"], leaves["x"],
                                              leaves["beta"], leaves["A_log"], bias, leaves["h0"],
                                              d["cu"])
        loss = (o[:, :n].float() * to_dev(W_o[:, :n])).sum() + (ht * to_dev(wl.dht)).sum()
        grads = torch.autograd.grad(loss, list(leaves.values()))
        res.append((o.detach(), ht.detach(), grads))
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
    (o1, h1, g1), (o2, h2, g2) = res
    assert torch.equal(bits(o1[:, :n]), bits(o2[:, :n]))
    assert torch.equal(bits(h1), bits(h2))
    mask = torch.from_numpy(in_contract_rows(wl)).to(DEV)
    for name, a, c in zip(("q", "k", "v", "x", "beta", "A_log", "h0"), g1, g2):
        if name not in ("A_log", "h0"):
            a, c = a[mask], c[mask]
        assert torch.equal(bits(a), bits(c)), name


def test_opcheck_registrations():
    wl, b = _case("fp32")
    d = device_inputs(wl)
    tests = ("test_schema", "test_faketensor", "test_autograd_registration")
    args = (d["q"], d["k"], d["v"], d["x"], d["beta"], d["A_log"], to_dev(b), d["h0"], d["cu"])
    torch.library.opcheck(torch.ops.kda.chunk_kda_train.default, args, test_utils=tests)
    rargs = (d["q"], d["k"], d["v"], d["x"], d["beta"], d["A_log"], d["h0"], d["cu"])
    torch.library.opcheck(torch.ops.kda.recurrent_kda.default, rargs,
                          test_utils=("test_schema", "test_faketensor"))
    o, ht = torch.ops.kda.recurrent_kda(*rargs)
    o_ref, ht_ref = oracle.forward(wl)
    n = int(wl.cu_seqlens[-1])
    assert normwise_max_err(to_np(o)[:, :n], o_ref[:, :n]) <= 2e-5
    assert normwise_max_err(to_np(ht), ht_ref) <= 2e-5


def test_prefill_and_decode_step_ops():
    """kda::chunk_kda_prefill and kda::recurrent_kda_step equal the direct
    binding calls bit for bit (the step op mutating state and history), and
    pass opcheck."""
    import gated_delta_rule_69_amd as kda
    import workloads as wls

    wl = wls.tiny_case(1200, T=150, H=2, HV=4, K=64, V=64, dtype="bf16", cu_seqlens=[0, 70, 70, 148],
                       A_log=0.3)
    wl, taps = wls.with_raw_projections(wl, 1201, 4, True)
    d = device_inputs(wl)
    tt = [to_dev(a) for pair in taps for a in pair]  # wq, bq, wk, bk, wv, bv
    wq, bq, wk, bk, wv, bv = tt
    conv_args = (wq, wk, wv, bq, bk, bv)
    o, ht, hist = torch.ops.kda.chunk_kda_prefill(d["q"], d["k"], d["v"], d["x"], d["beta"], d["A_log"],
                                                  d["h0"], d["cu"], True, *conv_args)
    o2, ht2 = kda.chunk_kda(d["q"], d["k"], d["v"], d["x"], d["beta"], d["h0"], cu_seqlens=d["cu"],
                            output_final_state=True, use_gate_in_kernel=True, A_log=d["A_log"],
                            qk_l2norm=True, short_conv=((wq, bq), (wk, bk), (wv, bv)))
    hist2 = torch.zeros_like(hist)
    kda.short_conv(d["q"], d["k"], d["v"], ((wq, bq), (wk, bk), (wv, bv)), cu_seqlens=d["cu"],
                   conv_state_out=hist2, outputs=False)
    torch.cuda.synchronize()
    n = 148
    assert torch.equal(o[:, :n].view(torch.int16), o2[:, :n].view(torch.int16))
    assert torch.equal(ht.view(torch.int32), ht2.view(torch.int32))
    assert torch.equal(hist.view(torch.int16), hist2.view(torch.int16))
    # one decode token per slot continuing from the prefill
    step = wls.tiny_case(1202, T=3, H=2, HV=4, K=64, V=64, dtype="bf16", cu_seqlens=[0, 1, 2, 3],
                         A_log=0.3)
    step, _ = wls.with_raw_projections(step, 1203, 4, True)
    s = device_inputs(step)
    st_a, st_b = ht.clone(), ht.clone()
    hi_a, hi_b = hist.clone(), hist.clone()
    oa = torch.ops.kda.recurrent_kda_step(s["q"], s["k"], s["v"], s["x"], s["beta"], s["A_log"], st_a,
                                          hi_a, s["cu"], True, *conv_args)
    ob, _ = kda.recurrent_kda(s["q"], s["k"], s["v"], s["x"], s["beta"], st_b, cu_seqlens=s["cu"],
                              output_final_state=True, final_state=st_b, use_gate_in_kernel=True,
                              A_log=s["A_log"], qk_l2norm=True,
                              short_conv=((wq, bq), (wk, bk), (wv, bv)), conv_state=hi_b,
                              conv_state_out=hi_b)
    torch.cuda.synchronize()
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))
    assert torch.equal(st_a.view(torch.int32), st_b.view(torch.int32))
    assert torch.equal(hi_a.view(torch.int16), hi_b.view(torch.int16))
    assert not torch.equal(hi_a.view(torch.int16), hist.view(torch.int16))  # it advanced
    torch.library.opcheck(torch.ops.kda.chunk_kda_prefill.default,
                          (d["q"], d["k"], d["v"], d["x"], d["beta"], d["A_log"], d["h0"], d["cu"],
                           True, *conv_args), test_utils=("test_schema", "test_faketensor"))
    torch.library.opcheck(torch.ops.kda.recurrent_kda_step.default,
                          (s["q"], s["k"], s["v"], s["x"], s["beta"], s["A_log"], ht.clone(),
                           hist.clone(), s["cu"], True, *conv_args),
                          test_utils=("test_schema", "test_faketensor"))
