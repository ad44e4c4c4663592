"""The binding is the only guard on buffer sizes and dtypes (the C ABI takes
bare pointers): every scan argument's dtype and full shape is checked before
anything reaches the library. These run on the CPU: the checks come before the
device check and before the library is loaded."""
import pytest
import torch

import gated_delta_rule_69_amd as kda

B, T, H, HV, K, V = 1, 10, 2, 4, 8, 6


def _args(dtype=torch.bfloat16, varlen=True):
    q = torch.zeros(B, T, H, K, dtype=dtype)
    k = torch.zeros(B, T, H, K, dtype=dtype)
    v = torch.zeros(B, T, HV, V, dtype=dtype)
    gate = torch.zeros(B, T, HV, K)
    beta = torch.zeros(B, T, HV, dtype=dtype)
    cu = torch.tensor([0, 3, 3, 9], dtype=torch.int32) if varlen else None
    N = 3 if varlen else B
    h0 = torch.zeros(N, HV, K, V)
    return dict(q=q, k=k, v=v, gate=gate, beta=beta, initial_state=h0, cu_seqlens=cu)


def _call(fn, a, **kw):
    args = (a["q"], a["k"], a["v"], a["gate"], a["beta"], a["initial_state"])
    if fn is kda.chunk_kda_bwd:
        do = kw.pop("do", torch.zeros_like(a["v"]))
        return fn(*args, do, kw.pop("dht", None), cu_seqlens=a["cu_seqlens"], **kw)
    return fn(*args, cu_seqlens=a["cu_seqlens"], **kw)


FNS = [kda.chunk_kda, kda.recurrent_kda, kda.chunk_kda_bwd]


@pytest.mark.parametrize("fn", FNS)
def test_int64_cu_seqlens_rejected(fn):
    a = _args()
    a["cu_seqlens"] = a["cu_seqlens"].to(torch.int64)
    with pytest.raises(TypeError, match="int32"):
        _call(fn, a)


@pytest.mark.parametrize("fn", FNS)
def test_bf16_gate_rejected(fn):
    a = _args()
    a["gate"] = a["gate"].to(torch.bfloat16)
    with pytest.raises(TypeError, match="gate"):
        _call(fn, a)


@pytest.mark.parametrize("fn", FNS)
def test_wrong_state_count_rejected(fn):
    a = _args()
    a["initial_state"] = torch.zeros(2, HV, K, V)  # cu_seqlens holds 3 sequences
    with pytest.raises(ValueError, match="initial_state"):
        _call(fn, a)


@pytest.mark.parametrize("fn", FNS)
@pytest.mark.parametrize("name,bad,exc", [
    ("k", lambda a: a["k"].float(), TypeError),                      # dtype differs from q
    ("v", lambda a: torch.zeros(B, T + 1, HV, V, dtype=torch.bfloat16), ValueError),
    ("beta", lambda a: torch.zeros(B, T, H, dtype=torch.bfloat16), ValueError),  # per qk head
    ("beta", lambda a: a["beta"].float(), TypeError),
    ("gate", lambda a: torch.zeros(B, T, H, K), ValueError),          # per qk head
    ("initial_state", lambda a: a["initial_state"].to(torch.bfloat16), TypeError),
    ("initial_state", lambda a: torch.zeros(3, HV, V, K), ValueError),  # transposed
])
def test_bad_operand_rejected(fn, name, bad, exc):
    a = _args()
    a[name] = bad(a)
    with pytest.raises(exc, match=name):
        _call(fn, a)


def test_varlen_needs_one_batch_row():
    a = _args(varlen=False)
    for n in ("q", "k"):
        a[n] = torch.zeros(2, T, H, K, dtype=torch.bfloat16)
    a["v"] = torch.zeros(2, T, HV, V, dtype=torch.bfloat16)
    a["beta"] = torch.zeros(2, T, HV, dtype=torch.bfloat16)
    a["gate"] = torch.zeros(2, T, HV, K)
    a["initial_state"] = torch.zeros(3, HV, K, V)
    a["cu_seqlens"] = torch.tensor([0, 3, 3, 9], dtype=torch.int32)
    with pytest.raises(ValueError, match="B == 1"):
        _call(kda.chunk_kda, a)


def test_heads_must_group():
    a = _args()
    a["v"] = torch.zeros(B, T, 3, V, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="multiple"):
        _call(kda.chunk_kda, a)


def test_outputs_and_gradients_checked():
    a = _args()
    with pytest.raises(TypeError, match="o must be"):
        _call(kda.chunk_kda, a, o=torch.zeros(B, T, HV, V))  # FP32 o for bf16 inputs
    with pytest.raises(ValueError, match="final_state"):
        _call(kda.recurrent_kda, a, output_final_state=True, final_state=torch.zeros(3, HV, K, K))
    with pytest.raises(ValueError, match="dht"):
        _call(kda.chunk_kda_bwd, a, dht=torch.zeros(3, HV, K, V + 1))
    with pytest.raises(TypeError, match="do"):
        _call(kda.chunk_kda_bwd, a, do=torch.zeros(B, T, HV, V))
    with pytest.raises(ValueError, match="A_log"):
        _call(kda.chunk_kda, a, use_gate_in_kernel=True, A_log=torch.zeros(H))


def test_gate_entry_points_checked():
    x = torch.zeros(B, T, HV, K)
    cu = torch.tensor([0, 3, 9], dtype=torch.int32)
    with pytest.raises(TypeError, match="gate_in"):
        kda.gate_cumsum(x.to(torch.bfloat16), None, cu, 64)
    with pytest.raises(TypeError, match="int32"):
        kda.gate_cumsum(x, None, cu.long(), 64)
    with pytest.raises(ValueError, match="A_log"):
        kda.gate_cumsum(x, torch.zeros(HV + 1), cu, 64)
    with pytest.raises(ValueError, match="dt_bias"):
        kda.gate_cumsum(x, None, cu, 64, dt_bias=torch.zeros(HV, K + 1))
    with pytest.raises(ValueError, match="dg"):
        kda.gate_bwd(x, torch.zeros(B, T, HV, K + 1), None, None, cu)


def test_short_conv_inputs_checked():
    q = torch.zeros(B, T, H, K, dtype=torch.bfloat16)
    taps = ((torch.zeros(H * K, 4), None), (torch.zeros(H * K, 4), None), (torch.zeros(HV * V, 4), None))
    with pytest.raises(TypeError, match="k"):
        kda.short_conv(q, q.float(), torch.zeros(B, T, HV, V, dtype=torch.bfloat16), taps)
    with pytest.raises(TypeError, match="int32"):
        kda.short_conv(q, q, torch.zeros(B, T, HV, V, dtype=torch.bfloat16), taps,
                       cu_seqlens=torch.tensor([0, 10]))
