"""GPU parity of the fused short convolution + SiLU forward (kda_chunk_fwd_conv)
against the oracle: short_conv_silu on q, k and v, then (optionally) the q/k
L2 normalisation, then the FP64 token recurrence. With bf16 inputs the kernel
rounds the convolution output (and the normalised rows) to bf16 where a
separate pass would store them; the reference rounds at the same points."""
import numpy as np
import pytest
import torch

import gated_delta_rule_69_amd as kda
import oracle
import workloads
from helpers import (TOL_BF16_O, TOL_BF16_STATE, check_parity, device_inputs, rel_rms, to_dev,
                     to_np)

pytestmark = pytest.mark.gpu


def _dev_taps(taps):
    return tuple((to_dev(w), to_dev(b)) for w, b in taps)


def _preprocessed(wl, taps, qn):
    """q, k, v as the scan sees them (FP64 values, bf16-rounded for bf16)."""
    if wl.dtype == "bf16":
        rnd = lambda a: workloads.round_bf16(a.astype(np.float32)).astype(np.float64)
    else:
        rnd = lambda a: a
    cu = wl.cu_seqlens
    out = []
    for a, (w, b) in zip((wl.q, wl.k, wl.v), taps):
        B, T = a.shape[:2]
        y = oracle.short_conv_silu(a.reshape(B, T, -1), w, b, cu).reshape(a.shape)
        out.append(rnd(np.nan_to_num(y)))  # rows outside every sequence: 0, never read
    q, k, v = out
    if qn:
        q, k = rnd(oracle.l2norm(q)), rnd(oracle.l2norm(k))
    return q, k, v


def _ref(wl, taps, qn):
    q, k, v = _preprocessed(wl, taps, qn)
    g = oracle.gate_activation(wl.x, wl.A_log)
    return oracle.recurrence(q, k, v, g, wl.beta, wl.h0, wl.cu_seqlens)


CASES = [
    # dtype, K, V, B, T, cu, width, bias, qk_l2norm, tap_scale
    ("fp32", 64, 64, 1, 150, [0, 1, 3, 3, 140], 4, True, True, 1.0),     # 1- and 2-token sequences
    ("bf16", 128, 128, 1, 300, [0, 0, 100, 230, 230, 290], 4, True, True, 1.0),
    ("fp32", 128, 64, 2, 130, None, 3, False, True, 1.0),
    ("bf16", 64, 128, 2, 200, None, 2, True, True, 1.0),
    ("fp32", 64, 64, 1, 100, None, 1, True, True, 1.0),
    ("fp32", 64, 128, 1, 140, [0, 70, 139], 4, True, False, 0.1),         # no normalisation
    ("bf16", 128, 128, 1, 200, None, 4, False, False, 0.1),
    ("fp32", 128, 128, 1, 257, [0, 65, 129, 193, 257], 4, True, True, 1.0),  # chunk-edge lengths
]


@pytest.mark.parametrize("dtype,K,V,B,T,cu,W,bias,qn,ts", CASES)
@pytest.mark.parametrize("fused_gate", [True, False])
def test_chunk_conv_matches_oracle(dtype, K, V, B, T, cu, W, bias, qn, ts, fused_gate):
    seed = 800 + K + V + T + W
    wl = workloads.tiny_case(seed, B=B, T=T, H=1, HV=2, K=K, V=V, dtype=dtype, cu_seqlens=cu,
                             A_log=0.5)
    wl, taps = workloads.with_raw_projections(wl, seed + 1, W, bias, ts)
    d = device_inputs(wl)
    dt = _dev_taps(taps)
    sentinel = 3.0
    o = torch.full_like(d["v"], sentinel)
    if fused_gate:
        o, ht = kda.chunk_kda(d["q"], d["k"], d["v"], d["x"], d["beta"], d["h0"], cu_seqlens=d["cu"],
                              output_final_state=True, use_gate_in_kernel=True, A_log=d["A_log"],
                              qk_l2norm=qn, short_conv=dt, o=o)
    else:
        G = kda.gate_cumsum(d["x"], d["A_log"], d["cu"], 64)
        o, ht = kda.chunk_kda(d["q"], d["k"], d["v"], G, d["beta"], d["h0"], cu_seqlens=d["cu"],
                              output_final_state=True, qk_l2norm=qn, short_conv=dt, o=o)
    torch.cuda.synchronize()
    o_ref, h_ref = _ref(wl, taps, qn)
    eo, eh = check_parity(wl, o, ht, o_ref, h_ref, f"conv {dtype} K{K} V{V} W{W}")
    print(f"conv {dtype} K{K} V{V} W{W} bias={bias} qn={qn}: o {eo:.2e} state {eh:.2e}")
    if cu is not None:
        assert (to_np(o[:, cu[-1]:]) == sentinel).all(), "capacity tail written"


def test_conv_identity_taps_equal_silu_inputs_on_the_plain_path():
    """Taps (0, .., 0, 1) and no bias: the fused call equals kda_chunk_fwd_ex
    on silu(q), silu(k), silu(v) formed by the oracle and rounded to bf16."""
    wl = workloads.tiny_case(840, B=1, T=200, H=2, HV=4, K=128, V=128, dtype="bf16",
                             cu_seqlens=[0, 90, 90, 199], A_log=0.3)
    wl, _ = workloads.with_raw_projections(wl, 841)
    eye = []
    for D in (2 * 128, 2 * 128, 4 * 128):
        w = np.zeros((D, 4), np.float32)
        w[:, 3] = 1.0
        eye.append((w, None))
    d = device_inputs(wl)
    o1, h1 = kda.chunk_kda(d["q"], d["k"], d["v"], d["x"], d["beta"], d["h0"], cu_seqlens=d["cu"],
                           output_final_state=True, use_gate_in_kernel=True, A_log=d["A_log"],
                           qk_l2norm=True, short_conv=_dev_taps(eye))
    s = lambda a: to_dev(workloads.round_bf16(np.nan_to_num(oracle.silu(a)).astype(np.float32)),
                         torch.bfloat16)
    o2, h2 = kda.chunk_kda(s(wl.q), s(wl.k), s(wl.v), d["x"], d["beta"], d["h0"], cu_seqlens=d["cu"],
                           output_final_state=True, use_gate_in_kernel=True, A_log=d["A_log"],
                           qk_l2norm=True)
    torch.cuda.synchronize()
    n = 199
    # the kernel's FP32 SiLU and the oracle's FP64 one may round a few
    # elements to neighbouring bf16 values; the scans then agree closely
    assert rel_rms(to_np(o1[:, :n]), to_np(o2[:, :n])) < 2e-3
    assert rel_rms(to_np(h1), to_np(h2)) < 2e-3


def test_dense_B4_T4096_H16_conv_every_chain():
    """The headline dense shape through the fused convolution (width 4, biases,
    q/k normalisation, gate in the kernel): every chain against the oracle."""
    wl = workloads.workload2()
    wl, taps = workloads.with_raw_projections(wl, 850, 4, True)
    d = device_inputs(wl)
    o, ht = kda.chunk_kda(d["q"], d["k"], d["v"], d["x"], d["beta"], None, output_final_state=True,
                          use_gate_in_kernel=True, A_log=d["A_log"], qk_l2norm=True,
                          short_conv=_dev_taps(taps))
    torch.cuda.synchronize()
    o_ref, h_ref = _ref(wl, taps, True)
    check_parity(wl, o, ht, o_ref, h_ref, "dense conv B4 T4096 H16")
