"""GPU parity of the short convolution with a carried history: the standalone
kda_short_conv_fwd, decode from raw projections (kda_recurrent_fwd_conv) and
the prefill -> decode hand-off, against the oracle's short_conv_silu (with its
state) and FP64 recurrence over the whole sequences."""
import numpy as np
import pytest
import torch

import gated_delta_rule_69_amd as kda
import oracle
import workloads
from helpers import TOL_FP32, check_parity, device_inputs, normwise_max_err, to_dev, to_np

pytestmark = pytest.mark.gpu


def _tdt(wl):
    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def _rnd(wl, a):
    """Values as the device holds them in the workload dtype (bf16 or FP32)."""
    if wl.dtype == "bf16":
        return workloads.round_bf16(np.asarray(a, np.float32)).astype(np.float64)
    return np.asarray(a, np.float32).astype(np.float64)


def _split_state(st, H, K, HV, V):
    """[N, W-1, 2HK + HV V] -> the q, k, v histories."""
    return st[..., :H * K], st[..., H * K:2 * H * K], st[..., 2 * H * K:]


def _oracle_conv(wl, taps, state):
    """Oracle outputs (q, k, v) and the new history, concatenated like the ABI."""
    B, T, H, K, HV, V = wl.B, wl.T, wl.H, wl.K, wl.HV, wl.V
    parts = (None, None, None) if state is None else _split_state(state, H, K, HV, V)
    outs, sts = [], []
    for a, (w, b), st in zip((wl.q, wl.k, wl.v), taps, parts):
        y, s = oracle.short_conv_silu(a.reshape(B, T, -1), w, b, wl.cu_seqlens, state=st,
                                      return_state=True)
        outs.append(y.reshape(a.shape))
        sts.append(s)
    return outs, np.concatenate(sts, axis=-1)


CASES = [
    # dtype, K, V, B, T, cu, W, bias, with_state
    ("bf16", 128, 128, 1, 12, [0, 1, 1, 2, 5, 12], 4, True, True),   # decode-like and short
    ("fp32", 64, 64, 1, 40, [0, 0, 3, 40], 4, False, True),
    ("bf16", 64, 128, 2, 7, None, 3, True, False),
    ("fp32", 128, 64, 1, 9, [0, 2, 9], 2, True, True),
    ("bf16", 128, 128, 1, 6, [0, 1, 2, 3, 4, 5, 6], 1, True, True),   # width 1: no history
]


@pytest.mark.parametrize("dtype,K,V,B,T,cu,W,bias,with_state", CASES)
def test_short_conv_op_matches_oracle(dtype, K, V, B, T, cu, W, bias, with_state):
    seed = 900 + K + V + T + W
    wl = workloads.tiny_case(seed, B=B, T=T, H=2, HV=4, K=K, V=V, dtype=dtype, cu_seqlens=cu)
    wl, taps = workloads.with_raw_projections(wl, seed + 1, W, bias)
    d = device_inputs(wl)
    tt = tuple((to_dev(w), to_dev(b)) for w, b in taps)
    N = B if cu is None else len(cu) - 1
    shape = (N, W - 1, 2 * 2 * K + 4 * V)
    rng = np.random.default_rng(seed + 2)
    st_np = _rnd(wl, rng.standard_normal(shape)) if with_state else None
    st_in = to_dev(st_np, _tdt(wl)) if with_state else None
    st_out = torch.full(shape, 5.0, device=d["q"].device, dtype=_tdt(wl))
    sentinel = 7.0
    outs = tuple(torch.full_like(d[n], sentinel) for n in ("q", "k", "v"))
    res, _ = kda.short_conv(d["q"], d["k"], d["v"], tt, cu_seqlens=d["cu"], conv_state=st_in,
                            conv_state_out=st_out, out=outs)
    # history only, in place on a copy of the input history
    st_inplace = st_in.clone() if with_state else torch.zeros(shape, device=d["q"].device,
                                                               dtype=_tdt(wl))
    kda.short_conv(d["q"], d["k"], d["v"], tt, cu_seqlens=d["cu"], conv_state=st_inplace,
                   conv_state_out=st_inplace, outputs=False)
    torch.cuda.synchronize()
    (qo, ko, vo), st_ref = _oracle_conv(wl, taps, st_np)
    n_tok = B * T if cu is None else cu[-1]
    for got, ref, name in zip(res, (qo, ko, vo), "qkv"):
        g = to_np(got).reshape(B * T, -1)[:n_tok]
        r = _rnd(wl, np.nan_to_num(ref)).reshape(B * T, -1)[:n_tok]
        if dtype == "fp32":
            assert normwise_max_err(g, r) <= 1e-6, name
        else:  # both sides round to bf16: at most one bf16 step apart
            assert np.all(np.abs(g - r) <= 2.0 ** -7 * np.abs(r) + 1e-30), name
        if cu is not None:
            assert (to_np(got).reshape(B * T, -1)[n_tok:] == sentinel).all(), "tail written"
    # the history is data movement: bitwise
    assert np.array_equal(to_np(st_out), _rnd(wl, st_ref)), "history"
    assert np.array_equal(to_np(st_inplace), _rnd(wl, st_ref)), "history in place"


DECODE = [
    # dtype, K, V, cu (tokens per slot), W, qk_l2norm
    ("bf16", 128, 128, [0, 1, 2, 2, 3, 4], 4, True),
    ("fp32", 64, 64, [0, 1, 1, 2], 3, True),
    ("fp32", 128, 128, [0, 5, 6, 20], 4, True),    # several tokens per sequence
    ("fp32", 64, 128, [0, 1, 2], 4, False),
]


@pytest.mark.parametrize("dtype,K,V,cu,W,qn", DECODE)
def test_decode_with_conv_matches_oracle(dtype, K, V, cu, W, qn):
    seed = 950 + K + V + W
    T = cu[-1]
    wl = workloads.tiny_case(seed, T=T, H=2, HV=4, K=K, V=V, dtype=dtype, cu_seqlens=cu, A_log=0.4)
    wl, taps = workloads.with_raw_projections(wl, seed + 1, W, True, 1.0 if qn else 0.1)
    d = device_inputs(wl)
    tt = tuple((to_dev(w), to_dev(b)) for w, b in taps)
    N = len(cu) - 1
    shape = (N, W - 1, 2 * 2 * K + 4 * V)
    st_np = _rnd(wl, np.random.default_rng(seed + 2).standard_normal(shape))
    st = to_dev(st_np, _tdt(wl))
    h = d["h0"].clone()
    o, ht = kda.recurrent_kda(d["q"], d["k"], d["v"], d["x"], d["beta"], h, cu_seqlens=d["cu"],
                              output_final_state=True, final_state=h, use_gate_in_kernel=True,
                              A_log=d["A_log"], qk_l2norm=qn, short_conv=tt, conv_state=st,
                              conv_state_out=st)
    torch.cuda.synchronize()
    (qc, kc, vc), st_ref = _oracle_conv(wl, taps, st_np)
    qc, kc, vc = (_rnd(wl, np.nan_to_num(a)) for a in (qc, kc, vc))
    if qn:
        qc, kc = _rnd(wl, oracle.l2norm(qc)), _rnd(wl, oracle.l2norm(kc))
    g = oracle.gate_activation(wl.x, wl.A_log)
    o_ref, h_ref = oracle.recurrence(qc, kc, vc, g, wl.beta, wl.h0, wl.cu_seqlens)
    eo, eh = check_parity(wl, o, ht, o_ref, h_ref, f"conv decode {dtype} K{K} V{V} W{W}")
    print(f"conv decode {dtype} K{K} V{V} W{W} qn={qn}: o {eo:.2e} state {eh:.2e}")
    assert np.array_equal(to_np(st), _rnd(wl, st_ref)), "history updated in place"


def test_prefill_then_decode_handoff():
    """Prefill the first part of each sequence with the fused chunked forward,
    hand over the recurrent state and the convolution history, decode the
    remaining tokens one at a time: the outputs match the oracle run over the
    whole sequences."""
    H, HV, K, V, W = 2, 4, 128, 128, 4
    lens_pre = [70, 1, 130, 3]          # prompts, some shorter than W - 1
    n_dec = 3
    lens = [p + n_dec for p in lens_pre]
    cu_all = np.concatenate([[0], np.cumsum(lens)]).tolist()
    wl = workloads.tiny_case(990, T=cu_all[-1], H=H, HV=HV, K=K, V=V, dtype="fp32", cu_seqlens=cu_all,
                             A_log=0.3, h0=False)
    wl, taps = workloads.with_raw_projections(wl, 991, W, True)
    tt = tuple((to_dev(w), to_dev(b)) for w, b in taps)
    # oracle over the whole sequences
    (qc, kc, vc), _ = _oracle_conv(wl, taps, None)
    qc, kc, vc = np.nan_to_num(qc), np.nan_to_num(kc), np.nan_to_num(vc)
    qc, kc = oracle.l2norm(qc), oracle.l2norm(kc)
    g = oracle.gate_activation(wl.x, wl.A_log)
    o_ref, h_ref = oracle.recurrence(qc, kc, vc, g, wl.beta, None, wl.cu_seqlens)

    def take(a, rows):
        return np.ascontiguousarray(a[:, rows])

    pre_rows = np.concatenate([np.arange(cu_all[n], cu_all[n] + lens_pre[n]) for n in range(4)])
    cu_pre = np.concatenate([[0], np.cumsum(lens_pre)]).astype(np.int32)
    dev = lambda a, dt=torch.float32: to_dev(a, dt)
    cu_pre_d = torch.from_numpy(cu_pre).to("cuda:0")
    q, k, v = dev(take(wl.q, pre_rows)), dev(take(wl.k, pre_rows)), dev(take(wl.v, pre_rows))
    x, beta = dev(take(wl.x, pre_rows)), dev(take(wl.beta, pre_rows))
    A = dev(wl.A_log)
    o_pre, state = kda.chunk_kda(q, k, v, x, beta, None, cu_seqlens=cu_pre_d, output_final_state=True,
                                 use_gate_in_kernel=True, A_log=A, qk_l2norm=True, short_conv=tt)
    hist = torch.zeros(kda.conv_state_shape(q, v, cu_pre_d, W), device="cuda:0")
    kda.short_conv(q, k, v, tt, cu_seqlens=cu_pre_d, conv_state_out=hist, outputs=False)
    outs = []
    cu_dec = torch.arange(5, dtype=torch.int32, device="cuda:0")
    for i in range(n_dec):
        rows = np.array([cu_all[n] + lens_pre[n] + i for n in range(4)])
        o_i, _ = kda.recurrent_kda(dev(take(wl.q, rows)), dev(take(wl.k, rows)), dev(take(wl.v, rows)),
                                   dev(take(wl.x, rows)), dev(take(wl.beta, rows)), state,
                                   cu_seqlens=cu_dec, output_final_state=True, final_state=state,
                                   use_gate_in_kernel=True, A_log=A, qk_l2norm=True, short_conv=tt,
                                   conv_state=hist, conv_state_out=hist)
        outs.append(to_np(o_i)[0])
    torch.cuda.synchronize()
    o_pre_ref = o_ref[0, pre_rows]
    assert normwise_max_err(to_np(o_pre)[0], o_pre_ref) <= TOL_FP32
    for i in range(n_dec):
        rows = [cu_all[n] + lens_pre[n] + i for n in range(4)]
        e = normwise_max_err(outs[i], o_ref[0, rows])
        print(f"decode step {i}: {e:.2e}")
        assert e <= TOL_FP32
    assert normwise_max_err(to_np(state), h_ref) <= TOL_FP32
