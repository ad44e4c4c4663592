"""GPU parity of step A7 (kda_recurrent_fwd) against the FP64 oracle."""
import numpy as np
import pytest
import torch

import gated_delta_rule_69_amd as kda
import oracle
import workloads
from helpers import (DEV, check_parity, device_inputs, in_contract_rows, run_gpu, to_np)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dense", [False, True])
def test_tiny_fp32_recurrent(dense):
    wl = workloads.workload1(dense=dense)
    d = device_inputs(wl)
    o, ht = run_gpu(wl, d, "recurrent")
    o_ref, ht_ref = oracle.forward(wl)
    check_parity(wl, o, ht, o_ref, ht_ref, "tiny")


@pytest.mark.parametrize("K,V", [(37, 50), (64, 100), (128, 128), (200, 256), (256, 24), (1, 1)])
def test_non_power_of_two_shapes_fp32(K, V):
    wl = workloads.tiny_case(200 + K, B=2, T=19, H=1, HV=2, K=K, V=V)
    d = device_inputs(wl)
    o, ht = run_gpu(wl, d, "recurrent")
    o_ref, ht_ref = oracle.forward(wl)
    check_parity(wl, o, ht, o_ref, ht_ref, f"K{K}V{V}")


def test_bf16_gva_varlen():
    wl = workloads.tiny_case(210, T=140, H=2, HV=8, K=128, V=128, dtype="bf16",
                             cu_seqlens=[0, 1, 1, 60, 140])
    d = device_inputs(wl)
    o, ht = run_gpu(wl, d, "recurrent")
    o_ref, ht_ref = oracle.forward(wl)
    check_parity(wl, o, ht, o_ref, ht_ref, "gva")


@pytest.mark.parametrize("dtype,B,T,H,HV,K,V", [
    ("bf16", 8, 37, 4, 32, 128, 128),   # 1024 waves at 16 rows per lane: the many-chain form
    ("fp32", 16, 12, 16, 64, 64, 64),   # 1024 waves, one column block each
    ("bf16", 2, 150, 1, 4, 256, 64),    # few chains, K = 256: 64 row lanes (both lane swaps)
    ("fp32", 1, 90, 1, 3, 128, 64),     # few chains, K = 128: 64 row lanes of 2 rows
    ("bf16", 3, 70, 1, 2, 64, 128),     # few chains, K = 64: 32 row lanes (one lane swap)
])
def test_row_split_forms_multi_token(dtype, B, T, H, HV, K, V):
    """The per-wave kernel takes 16 state rows per lane when there are enough
    (sequence, value head) waves to fill the device and 2 (K = 256: 4) rows per
    lane otherwise (many times the waves, a shorter per-token chain, the row
    sums over 32 or 64 lanes); both forms over multi-token sequences against
    the oracle."""
    wl = workloads.tiny_case(270 + K + B, B=B, T=T, H=H, HV=HV, K=K, V=V, dtype=dtype)
    d = device_inputs(wl)
    o, ht = run_gpu(wl, d, "recurrent")
    o_ref, ht_ref = oracle.forward(wl)
    check_parity(wl, o, ht, o_ref, ht_ref, f"rows split {dtype} B{B} HV{HV} K{K}")


def test_decode_in_place_and_empty_slots_bitwise():
    """Decode workload: 256 slots (26 empty), state updated in place."""
    wl = workloads.workload4()
    d = device_inputs(wl)
    h0_before = d["h0"].clone()
    o, ht = run_gpu(wl, d, "recurrent", in_place=True, o_fill=777.0)
    assert ht.data_ptr() == d["h0"].data_ptr()
    o_ref, ht_ref = oracle.forward(wl)
    check_parity(wl, o, ht, o_ref, ht_ref, "decode")
    for s in wl.notes["empty"]:
        assert torch.equal(ht[s].view(torch.int32), h0_before[s].view(torch.int32)), s


@pytest.mark.parametrize("K,V", [(16, 16), (64, 72), (128, 128)])
def test_empty_slot_copy_not_in_place_bitwise(K, V):
    """K=16 runs the general kernel; K in {64, 128} with V % 4 == 0 the per-wave one."""
    wl = workloads.tiny_case(220, T=10, HV=2, K=K, V=V, cu_seqlens=[0, 0, 10, 10])
    d = device_inputs(wl)
    h0 = d["h0"]
    h0[0, 0, 0, 0] = -0.0
    h0.view(torch.int32)[2, 1, 3, 3] = 0x7FC01234  # NaN with a payload
    o, ht = run_gpu(wl, d, "recurrent")
    for s in (0, 2):
        assert torch.equal(ht[s].view(torch.int32), h0[s].view(torch.int32))
    # the planted -0.0 and NaN live in the empty slots only (checked bitwise
    # above); slot 1 is computed and held to the parity bar
    o_ref, ht_ref = oracle.forward(wl)
    ht_cmp = ht.clone()
    ht_cmp[[0, 2]] = torch.from_numpy(ht_ref[[0, 2]]).float().to(ht.device)
    check_parity(wl, o, ht_cmp, o_ref, ht_ref, f"empty K{K}")


@pytest.mark.parametrize("K,V", [(16, 16), (128, 128)])
def test_empty_slot_without_initial_state_is_zero(K, V):
    wl = workloads.tiny_case(221, T=10, HV=2, K=K, V=V, cu_seqlens=[0, 0, 10, 10], h0=False)
    d = device_inputs(wl)
    o, ht = run_gpu(wl, d, "recurrent")
    z = ht[[0, 2]]
    assert torch.equal(z.view(torch.int32), torch.zeros_like(z).view(torch.int32))


def test_packed_equals_separate_bitwise():
    cu = [0, 7, 7, 30, 41]
    wl = workloads.tiny_case(230, T=48, H=1, HV=2, K=64, V=64, dtype="bf16", cu_seqlens=cu)
    d = device_inputs(wl)
    o, ht = run_gpu(wl, d, "recurrent")
    G = kda.gate_cumsum(d["x"], d["A_log"], d["cu"], 1)
    for n in range(len(cu) - 1):
        a, b = cu[n], cu[n + 1]
        if a == b:
            continue
        sl = slice(a, b)
        o1, h1 = kda.recurrent_kda(d["q"][:, sl].contiguous(), d["k"][:, sl].contiguous(),
                                   d["v"][:, sl].contiguous(), G[:, sl].contiguous(),
                                   d["beta"][:, sl].contiguous(), d["h0"][n:n + 1].contiguous(),
                                   output_final_state=True)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o[:, sl].view(torch.int16))
        assert torch.equal(h1.view(torch.int32), ht[n:n + 1].view(torch.int32))


@pytest.mark.parametrize("K", [32, 64])
def test_capacity_tail_untouched(K):
    cu = [0, 12, 30]
    wl = workloads.tiny_case(240, T=40, HV=2, K=K, V=32, cu_seqlens=cu)
    wl.q[:, 30:] = np.nan
    wl.v[:, 30:] = np.nan
    wl.x[:, 30:] = np.nan
    d = device_inputs(wl)
    o, ht = run_gpu(wl, d, "recurrent", o_fill=-9.0)
    assert (to_np(o)[:, 30:] == -9.0).all()
    o_ref, ht_ref = oracle.forward(wl)
    check_parity(wl, o, ht, o_ref, ht_ref, "tail")


def test_misaligned_operands_take_the_general_kernel():
    """q, k offset by one element (not 16-byte aligned): same results as aligned."""
    wl = workloads.tiny_case(260, T=33, H=1, HV=2, K=64, V=64, dtype="bf16")
    d = device_inputs(wl)
    o, ht = run_gpu(wl, d, "recurrent")
    G = kda.gate_cumsum(d["x"], d["A_log"], d["cu"], 1)
    qb = torch.empty(d["q"].numel() + 1, dtype=d["q"].dtype, device=DEV)
    kb = torch.empty(d["k"].numel() + 1, dtype=d["k"].dtype, device=DEV)
    q2 = qb[1:].view(d["q"].shape)
    k2 = kb[1:].view(d["k"].shape)
    q2.copy_(d["q"])
    k2.copy_(d["k"])
    o2, h2 = kda.recurrent_kda(q2, k2, d["v"], G, d["beta"], d["h0"], output_final_state=True)
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.forward(wl)
    check_parity(wl, o2, h2, o_ref, ht_ref, "misaligned")
    check_parity(wl, o, ht, o_ref, ht_ref, "aligned")


def test_rejects_inputs_that_require_grad():
    wl = workloads.tiny_case(250, T=4, K=8, V=8)
    d = device_inputs(wl)
    G = kda.gate_cumsum(d["x"], None, None, 1)
    q = d["q"].clone().requires_grad_(True)
    with pytest.raises(RuntimeError, match="chunk_kda"):
        kda.recurrent_kda(q, d["k"], d["v"], G, d["beta"])
