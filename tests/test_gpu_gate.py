"""GPU parity of step A1 (kda_gate_cumsum) against the oracle gate."""
import math

import numpy as np
import pytest
import torch

import gated_delta_rule_69_amd as kda
import oracle
import workloads
from helpers import DEV, device_inputs, in_contract_rows, to_np

pytestmark = pytest.mark.gpu


def _ref(wl, chunk):
    g = oracle.gate_activation(wl.x, wl.A_log)
    return oracle.gate_cumsum_log2(g, wl.cu_seqlens, chunk)


def _close(gpu, ref, mask):
    gpu, ref = gpu[mask], ref[mask]
    err = np.abs(gpu - ref) / (1.0 + np.abs(ref))
    return float(err.max())


@pytest.mark.parametrize("chunk", [1, 64, 7])
def test_gate_dense_matches_oracle(chunk):
    wl = workloads.tiny_case(101, B=2, T=150, HV=3, K=64, V=8, A_log=0.7, gate_scale=2.0)
    d = device_inputs(wl)
    out = kda.gate_cumsum(d["x"], d["A_log"], None, chunk)
    torch.cuda.synchronize()
    assert _close(to_np(out), _ref(wl, chunk), in_contract_rows(wl)) < 2e-6


@pytest.mark.parametrize("chunk", [1, 64])
def test_gate_varlen_tail_untouched(chunk):
    cu = [0, 0, 5, 70, 70, 200]
    wl = workloads.tiny_case(102, T=230, HV=2, K=128, V=8, cu_seqlens=cu, A_log=None)
    d = device_inputs(wl)
    out = torch.full_like(d["x"], 12345.0)
    kda.gate_cumsum(d["x"], None, d["cu"], chunk, out=out)
    torch.cuda.synchronize()
    o = to_np(out)
    assert (o[:, 200:] == 12345.0).all()
    assert _close(o, _ref(wl, chunk), in_contract_rows(wl)) < 2e-6


def test_gate_omitted_A_log_is_bitwise_zero_A_log():
    wl = workloads.tiny_case(103, B=1, T=100, HV=4, K=32, V=8)
    d = device_inputs(wl)
    a = kda.gate_cumsum(d["x"], None, None, 64)
    b = kda.gate_cumsum(d["x"], torch.zeros(4, device=DEV), None, 64)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_gate_ones_A_log_scales_by_e():
    wl = workloads.tiny_case(104, B=1, T=64, HV=2, K=16, V=8)
    d = device_inputs(wl)
    a = to_np(kda.gate_cumsum(d["x"], None, None, 1))
    b = to_np(kda.gate_cumsum(d["x"], torch.ones(2, device=DEV), None, 1))
    np.testing.assert_allclose(b, math.e * a, rtol=1e-6)


def test_gate_natural_log_input_mode():
    wl = workloads.tiny_case(105, B=1, T=90, HV=2, K=16, V=8)
    g = oracle.gate_activation(wl.x, None)
    gd = torch.from_numpy(g.astype(np.float32)).to(DEV)
    out = kda.gate_cumsum(gd, None, None, 64, is_raw=False)
    ref = oracle.gate_cumsum_log2(g.astype(np.float32), None, 64)
    assert _close(to_np(out), ref, np.ones((1, 90), bool)) < 2e-6


def test_gate_in_place_per_token():
    wl = workloads.tiny_case(106, B=1, T=77, HV=2, K=16, V=8)
    d = device_inputs(wl)
    ref = to_np(kda.gate_cumsum(d["x"], None, None, 1))
    x = d["x"].clone()
    kda.gate_cumsum(x, None, None, 1, out=x)
    assert np.array_equal(to_np(x), ref)
