"""kda_recurrent_fwd_conv_noalloc (decode from raw projections without a
workspace argument: the library's own static device scratch) against
kda_recurrent_fwd_conv, the entry point it mirrors: bitwise equal outputs,
final states and convolution histories on two calls in a row, the second
with a smaller input (the scratch keeps the first call's contents)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_69_amd as kda
import workloads
from helpers import DEV, to_dev

pytestmark = pytest.mark.gpu


def _decode_inputs(slots, n_empty, seed):
    wl = workloads.workload4(slots=slots, n_empty=n_empty)
    wl, taps = workloads.with_raw_projections(wl, seed, 4, True)
    bf = torch.bfloat16
    d = dict(q=to_dev(wl.q, bf), k=to_dev(wl.k, bf), v=to_dev(wl.v, bf), beta=to_dev(wl.beta, bf),
             x=to_dev(wl.x), h0=to_dev(wl.h0),
             cu=torch.from_numpy(wl.cu_seqlens.astype(np.int32)).to(DEV))
    taps = tuple((to_dev(w), to_dev(b)) for w, b in taps)
    gen = torch.Generator(device=DEV).manual_seed(seed)
    hist = torch.randn(kda.conv_state_shape(d["q"], d["v"], d["cu"], 4), device=DEV,
                       generator=gen).to(bf)
    return wl, d, taps, hist


def _step(d, taps, h, hist, o, no_alloc, ws=None):
    return kda.recurrent_kda(d["q"], d["k"], d["v"], d["x"], d["beta"], h, cu_seqlens=d["cu"],
                             output_final_state=True, o=o, final_state=h, use_gate_in_kernel=True,
                             qk_l2norm=True, short_conv=taps, conv_state=hist, conv_state_out=hist,
                             workspace=ws, no_alloc=no_alloc)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_noalloc_matches_workspace_entry_two_calls():
    for slots, n_empty, seed in ((256, 26, 900), (96, 10, 901)):  # second call smaller
        wl, d, taps, hist0 = _decode_inputs(slots, n_empty, seed)
        need = kda.load().kda_recurrent_fwd_conv_workspace_bytes(
            kda.KdaDims(1, wl.T, wl.N, wl.H, wl.HV, wl.K, wl.V), kda.KDA_BF16)
        assert 0 < need <= kda.NOALLOC_SCRATCH_BYTES
        print(f"no-alloc decode: {slots} slots, {wl.T} tokens, {need} scratch bytes", flush=True)
        h_a, h_b = d["h0"].clone(), d["h0"].clone()
        hist_a, hist_b = hist0.clone(), hist0.clone()
        o_a = torch.full_like(d["v"], 5.0)
        o_b = torch.full_like(d["v"], 5.0)
        ws = torch.empty(need, device=DEV, dtype=torch.uint8)
        _step(d, taps, h_a, hist_a, o_a, False, ws)
        _step(d, taps, h_b, hist_b, o_b, True)
        torch.cuda.synchronize()
        assert torch.equal(_bits(o_a), _bits(o_b))
        assert torch.equal(_bits(h_a), _bits(h_b))
        assert torch.equal(_bits(hist_a), _bits(hist_b))
        assert not torch.equal(_bits(hist_a), _bits(hist0))  # the history did advance


def test_noalloc_rejects_inputs_beyond_its_scratch():
    # 4096 tokens (one sequence) at these head sizes need 64 MiB of convolved q, k, v
    T = 4096
    d = kda.KdaDims(1, T, 1, 16, 32, 128, 128)
    lib = kda.load()
    assert lib.kda_recurrent_fwd_conv_workspace_bytes(d, kda.KDA_BF16) > kda.NOALLOC_SCRATCH_BYTES
    with pytest.raises(kda.KdaError, match="WORKSPACE"):
        bf = torch.bfloat16
        q = torch.zeros(1, T, 16, 128, device=DEV, dtype=bf)
        v = torch.zeros(1, T, 32, 128, device=DEV, dtype=bf)
        x = torch.zeros(1, T, 32, 128, device=DEV)
        beta = torch.zeros(1, T, 32, device=DEV, dtype=bf)
        h = torch.zeros(1, 32, 128, 128, device=DEV)
        cu = torch.tensor([0, T], device=DEV, dtype=torch.int32)
        taps = tuple((torch.zeros(D, 4, device=DEV), None) for D in (2048, 2048, 4096))
        kda.recurrent_kda(q, q, v, x, beta, h, cu_seqlens=cu, output_final_state=True,
                          final_state=h, use_gate_in_kernel=True, short_conv=taps, no_alloc=True)
