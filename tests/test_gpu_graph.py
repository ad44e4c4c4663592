"""HIP-graph capture and replay of the forward entry points: the library
reads cu_seqlens only on the device and enqueues nothing but kernels, so a
captured call replays correctly with new inputs and new sequence boundaries
(same N and capacity). Every replay is compared bit for bit with an eager call
on the same inputs, with eager work and synchronisations in between."""
import numpy as np
import pytest
import torch

import gated_delta_rule_69_amd as kda
import oracle
import workloads
from helpers import DEV, check_parity, device_inputs, to_dev

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _boundaries(rng, n_seq, total, empty):
    """cu_seqlens with n_seq slots summing to `total`, slots in `empty` of length 0."""
    live = [i for i in range(n_seq) if i not in empty]
    cuts = np.sort(rng.choice(np.arange(1, total), size=len(live) - 1, replace=False))
    lens = np.diff(np.concatenate([[0], cuts, [total]]))
    full = np.zeros(n_seq, dtype=np.int64)
    full[live] = lens
    return np.concatenate([[0], np.cumsum(full)]).astype(np.int32)


def test_decode_graph_replay_with_new_slots_and_inputs():
    wl = workloads.workload4()  # 256 slots, one token each, state in place, fused gate
    d = device_inputs(wl)
    h = d["h0"].clone()
    o = torch.empty_like(d["v"])
    st = {n: d[n].clone() for n in ("q", "k", "v", "x", "beta")}
    cu = d["cu"].clone()

    def step():
        kda.recurrent_kda(st["q"], st["k"], st["v"], st["x"], st["beta"], h, cu_seqlens=cu,
                          output_final_state=True, final_state=h, o=o, use_gate_in_kernel=True)

    g = _capture(step)
    rng = np.random.default_rng(900)
    N = int(wl.cu_seqlens.size) - 1
    total = int(wl.cu_seqlens[-1])
    for rep in range(3):
        # new inputs, new empty slots, new state
        for n in st:
            st[n].copy_(torch.randn_like(st[n], dtype=torch.float32).to(st[n].dtype) *
                        (1.0 if n != "beta" else 0.2))
        # slots of one token and a few of two, within the token capacity
        n_empty = 26 + 4 * rep
        empty = set(rng.choice(N, size=n_empty, replace=False).tolist())
        new_cu = _boundaries(rng, N, min(N - n_empty + 3 * rep, total), empty)
        cu.copy_(torch.from_numpy(new_cu).to(DEV))
        h0 = torch.randn_like(h) * 0.1
        h.copy_(h0)
        g.replay()
        torch.cuda.synchronize()
        o_g, h_g = o.clone(), h.clone()
        # eager on the same inputs
        h_e = h0.clone()
        o_e, _ = kda.recurrent_kda(st["q"], st["k"], st["v"], st["x"], st["beta"], h_e,
                                   cu_seqlens=cu, output_final_state=True, final_state=h_e,
                                   use_gate_in_kernel=True)
        torch.cuda.synchronize()
        n_tok = int(new_cu[-1])
        assert torch.equal(_bits(o_g[:, :n_tok]), _bits(o_e[:, :n_tok])), rep
        assert torch.equal(_bits(h_g), _bits(h_e)), rep
        for s in empty:
            assert torch.equal(_bits(h_g[s]), _bits(h0[s])), (rep, s)


def test_chunk_forward_graph_replay_with_new_boundaries():
    cu0 = [0, 0, 100, 230, 230, 400]
    wl = workloads.tiny_case(910, T=450, H=2, HV=4, K=128, V=128, dtype="bf16", cu_seqlens=cu0)
    d = device_inputs(wl)
    ws = torch.empty(kda.chunk_workspace_bytes(d["q"], d["v"], d["cu"]), device=DEV, dtype=torch.uint8)
    o = torch.empty_like(d["v"])
    ht = torch.empty_like(d["h0"])
    cu = d["cu"].clone()

    def step():
        kda.chunk_kda(d["q"], d["k"], d["v"], d["x"], d["beta"], d["h0"], cu_seqlens=cu,
                      output_final_state=True, o=o, final_state=ht, workspace=ws,
                      use_gate_in_kernel=True, A_log=d["A_log"])

    g = _capture(step)
    rng = np.random.default_rng(911)
    for rep in range(3):
        new_cu = _boundaries(rng, 5, 400 + 10 * rep, {rep % 5})
        cu.copy_(torch.from_numpy(new_cu).to(DEV))
        d["x"].copy_(torch.randn_like(d["x"]))
        g.replay()
        torch.cuda.synchronize()
        o_g, h_g = o.clone(), ht.clone()
        o_e, h_e = kda.chunk_kda(d["q"], d["k"], d["v"], d["x"], d["beta"], d["h0"], cu_seqlens=cu,
                                 output_final_state=True, use_gate_in_kernel=True, A_log=d["A_log"])
        torch.cuda.synchronize()
        n_tok = int(new_cu[-1])
        assert torch.equal(_bits(o_g[:, :n_tok]), _bits(o_e[:, :n_tok])), rep
        assert torch.equal(_bits(h_g), _bits(h_e)), rep
    # the last replay against the oracle too
    wl.cu_seqlens = new_cu
    wl.x = d["x"].cpu().numpy()
    o_ref, h_ref = oracle.forward(wl)
    check_parity(wl, o_g, h_g, o_ref, h_ref, "graph replay")


def test_conv_decode_graph_replay_advances_the_history():
    """A captured decode step from raw projections (short convolution with the
    history updated in place, then the scan with the state in place) replayed
    three times with new tokens equals three eager steps bit for bit, history
    and state included."""
    wl = workloads.workload4()
    wl, taps = workloads.with_raw_projections(wl, 905, 4, True)
    d = device_inputs(wl)
    tt = tuple((to_dev(w), to_dev(b)) for w, b in taps)
    hist0 = torch.randn(kda.conv_state_shape(d["q"], d["v"], d["cu"], 4), device=DEV).to(d["q"].dtype)
    h0 = d["h0"].clone()
    ws = torch.empty(1 << 24, device=DEV, dtype=torch.uint8)
    inp = {n: d[n].clone() for n in ("q", "k", "v", "x", "beta")}
    hist, h, o = hist0.clone(), h0.clone(), torch.empty_like(d["v"])

    def step(hist_, h_, o_, src):
        kda.recurrent_kda(src["q"], src["k"], src["v"], src["x"], src["beta"], h_, cu_seqlens=d["cu"],
                          output_final_state=True, final_state=h_, o=o_, use_gate_in_kernel=True,
                          qk_l2norm=True, short_conv=tt, conv_state=hist_, conv_state_out=hist_,
                          workspace=ws)

    g = _capture(lambda: step(hist, h, o, inp))
    # the capture's warm-up calls advanced the history and state: restart both
    hist.copy_(hist0)
    h.copy_(h0)
    hist_e, h_e, o_e = hist0.clone(), h0.clone(), torch.empty_like(o)
    gen = torch.Generator(device=DEV).manual_seed(906)
    for rep in range(3):
        for n in inp:
            inp[n].copy_((torch.randn(inp[n].shape, device=DEV, generator=gen) *
                          (1.0 if n != "beta" else 0.2)).to(inp[n].dtype))
        if "beta" in inp:
            inp["beta"].copy_(inp["beta"].abs())
        g.replay()
        torch.cuda.synchronize()
        step(hist_e, h_e, o_e, inp)
        torch.cuda.synchronize()
        rows = int(wl.cu_seqlens[-1])
        assert torch.equal(_bits(o[:, :rows]), _bits(o_e[:, :rows])), rep
        assert torch.equal(_bits(hist), _bits(hist_e)), rep
        assert torch.equal(_bits(h), _bits(h_e)), rep


def test_chunk_backward_graph_replay_with_new_boundaries():
    """The backward of a training step (gate recompute + kda_chunk_bwd, GVA,
    empty slots) captured once and replayed with new upstream gradients, gate
    inputs and sequence boundaries: every replay equals the eager call bit for
    bit (fixed-order reductions, no atomics)."""
    cu0 = [0, 0, 120, 250, 250, 400]
    wl = workloads.tiny_case(920, T=450, H=2, HV=4, K=128, V=128, dtype="bf16", cu_seqlens=cu0,
                             grads=True)
    d = device_inputs(wl)
    dO = to_dev(wl.dO, torch.bfloat16)
    dht = to_dev(wl.dht)
    ws = torch.empty(kda.chunk_bwd_workspace_bytes(d["q"], d["v"], d["cu"]), device=DEV,
                     dtype=torch.uint8)
    cu = d["cu"].clone()
    res = {}

    def step():
        G = kda.gate_cumsum(d["x"], d["A_log"], cu, 64)
        res.update(kda.chunk_kda_bwd(d["q"], d["k"], d["v"], G, d["beta"], d["h0"], dO, dht,
                                     cu_seqlens=cu, workspace=ws))

    g = _capture(step)
    rng = np.random.default_rng(921)
    for rep in range(3):
        new_cu = _boundaries(rng, 5, 400 + 10 * rep, {(rep + 1) % 5})
        cu.copy_(torch.from_numpy(new_cu).to(DEV))
        d["x"].copy_(torch.randn_like(d["x"]))
        dO.copy_(torch.randn_like(dO))
        g.replay()
        torch.cuda.synchronize()
        got = {n: t.clone() for n, t in res.items()}
        G = kda.gate_cumsum(d["x"], d["A_log"], cu, 64)
        want = kda.chunk_kda_bwd(d["q"], d["k"], d["v"], G, d["beta"], d["h0"], dO, dht,
                                 cu_seqlens=cu)
        torch.cuda.synchronize()
        n_tok = int(new_cu[-1])
        for n in ("dq", "dk", "dv", "dg", "dbeta"):
            assert torch.equal(_bits(got[n][:, :n_tok]), _bits(want[n][:, :n_tok])), (rep, n)
        assert torch.equal(_bits(got["dh0"]), _bits(want["dh0"])), rep
