"""Randomized shapes. Chunked path: 150 seeded small cases over dtype (bf16, FP32), K and V
in {64, 128}, grouped value heads, dense batches and packed varlen batches
(empty, single-token, chunk-boundary and ragged sequences, a capacity tail),
gate strength, the log2-gate and fused-gate entry points, and the
recomputing and saved (training-pair) backward. Every case is checked against
the FP64 oracle: forward output and final state, and all six gradients.

Tolerances: bf16 5e-3 rel-RMS (outputs), 1e-2 (states, gradients); FP32 2e-5
normwise, widened to ln2 * ulp(max |G2|) where the chunk-local log2 gate is
large (the FP32 representation bound of the two-call contract), and 4x that
for gradients. Token-sequential path: 200 cases with any K, V up to 256.
The cases are drawn from fixed seeds."""
import numpy as np
import pytest
import torch

import gated_delta_rule_69_amd as kda
import oracle
import workloads
from helpers import DEV, device_inputs, in_contract_rows, normwise_max_err, rel_rms, tdtype, to_dev, to_np

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def _cases(seed=12, n=150):
    rng = np.random.default_rng(seed)
    out = []
    for case in range(n):
        dtype = "bf16" if rng.random() < 0.6 else "fp32"
        K = int(rng.choice([64, 128]))
        V = int(rng.choice([64, 128]))
        if dtype == "fp32" and K == 128 and rng.random() < 0.7:
            K = 64
        H = int(rng.choice([1, 2]))
        HV = H * int(rng.choice([1, 2]))
        if rng.random() < 0.5:
            N = int(rng.integers(1, 6))
            lens = [int(rng.choice([0, 1, 2, 63, 64, 65, 127, 128, 129, 200]) if rng.random() < 0.5
                        else rng.integers(0, 260)) for _ in range(N)]
            cu = [0] + [int(c) for c in np.cumsum(lens)]
            B, T = 1, cu[-1] + int(rng.integers(0, 9))
        else:
            cu = None
            B, T = int(rng.integers(1, 3)), int(rng.choice([1, 5, 63, 64, 65, 130, 191, 256]))
        T = max(T, 1)
        A = float(rng.choice([0.0, 1.0, 2.7]))
        gs = float(rng.choice([1.0, 3.0]))
        s = int(rng.integers(1, 1 << 30))
        fused = bool(rng.random() < 0.5)
        saved = bool(rng.random() < 0.5)
        out.append((case, dtype, K, V, H, HV, B, T, cu, A, gs, s, fused, saved))
    return out


def test_random_shapes_forward_and_backward():
    failures = []
    for (case, dtype, K, V, H, HV, B, T, cu, A, gs, s, fused, saved) in _cases():
        label = (f"case {case}: {dtype} K{K} V{V} H{H} HV{HV} B{B} T{T} cu={cu} A_log={A} "
                 f"gate_scale={gs} fused={fused} saved={saved}")
        print(label, flush=True)
        wl = workloads.tiny_case(s, B=B, T=T, H=H, HV=HV, K=K, V=V, dtype=dtype, cu_seqlens=cu,
                                 grads=True, A_log=A, gate_scale=gs)
        d = device_inputs(wl)
        dt = tdtype(wl)
        fkw = dict(use_gate_in_kernel=True, A_log=d["A_log"]) if fused else {}
        gin = d["x"] if fused else kda.gate_cumsum(d["x"], d["A_log"], d["cu"], 64)
        o, ht = kda.chunk_kda(d["q"], d["k"], d["v"], gin, d["beta"], d["h0"], cu_seqlens=d["cu"],
                              output_final_state=True, **fkw)
        torch.cuda.synchronize()
        o_ref, ht_ref = oracle.forward(wl)
        mask = in_contract_rows(wl)
        err = normwise_max_err if dtype == "fp32" else rel_rms
        G_ref = oracle.gate_cumsum_log2(oracle.gate_activation(wl.x, wl.A_log), wl.cu_seqlens, 64)
        rep = float(np.log(2) * np.spacing(np.float32(np.nanmax(np.abs(G_ref)))))
        tol_o = max(2e-5, rep) if dtype == "fp32" else 5e-3
        tol_h = tol_o if dtype == "fp32" else 1e-2
        errs = {"o": err(to_np(o)[mask], o_ref[mask]) if mask.any() else 0.0,
                "state": err(to_np(ht), ht_ref)}
        bars = {"o": tol_o, "state": tol_h}
        if not (dtype == "fp32" and K == 128):  # the FP32 backward takes K = 64
            dO, dht = to_dev(np.nan_to_num(wl.dO), dt), to_dev(wl.dht)
            ws = None
            if saved:
                ws = torch.full((kda.chunk_bwd_workspace_bytes(d["q"], d["v"], d["cu"]),), 0xFF,
                                device=DEV, dtype=torch.uint8)
                kda.chunk_kda(d["q"], d["k"], d["v"], gin, d["beta"], d["h0"], cu_seqlens=d["cu"],
                              output_final_state=True, save_for_backward=ws, **fkw)
            r = kda.chunk_kda_bwd(d["q"], d["k"], d["v"], gin, d["beta"], d["h0"], dO, dht,
                                  cu_seqlens=d["cu"], saved=saved, workspace=ws, **fkw)
            torch.cuda.synchronize()
            dOr = np.nan_to_num(wl.dO.astype(np.float64))
            if cu is not None:
                dOr[:, cu[-1]:] = 0.0
            ref = oracle.recurrence_bwd(wl.q, wl.k, wl.v, oracle.gate_activation(wl.x, wl.A_log),
                                        wl.beta, dOr, wl.h0, wl.dht, wl.cu_seqlens)
            tol_g = 4 * tol_o if dtype == "fp32" else 1e-2
            for nm in GRADS:
                a, c = to_np(r[nm]), ref[nm]
                if nm != "dh0":
                    a, c = a[mask], c[mask]
                if c.size and np.any(c):
                    errs[nm], bars[nm] = err(a, c), tol_g
        over = {k: (v, bars[k]) for k, v in errs.items() if not v <= bars[k]}
        print("   " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()), flush=True)
        if over:
            failures.append((label, over))
    assert not failures, failures


def test_random_shapes_recurrent():
    """200 seeded cases of the token-sequential path: any K, V up to 256 (not
    only powers of two), grouped value heads, dense and packed batches with
    empty and short sequences, both gate entry points."""
    rng = np.random.default_rng(21)
    failures = []
    for case in range(200):
        dtype = "bf16" if rng.random() < 0.5 else "fp32"
        K = int(rng.integers(1, 257)) if rng.random() < 0.5 else int(rng.choice([16, 32, 64, 128, 256]))
        V = int(rng.integers(1, 257)) if rng.random() < 0.5 else int(rng.choice([16, 32, 64, 128, 256]))
        H = int(rng.choice([1, 2]))
        HV = H * int(rng.choice([1, 2, 4]))
        if rng.random() < 0.6:
            N = int(rng.integers(1, 7))
            lens = [int(rng.choice([0, 1, 2, 5]) if rng.random() < 0.6 else rng.integers(0, 90))
                    for _ in range(N)]
            cu = [0] + [int(c) for c in np.cumsum(lens)]
            B, T = 1, max(cu[-1] + int(rng.integers(0, 5)), 1)
        else:
            cu = None
            B, T = int(rng.integers(1, 4)), int(rng.choice([1, 2, 7, 40]))
        A = float(rng.choice([0.0, 1.0, 2.7]))
        fused = bool(rng.random() < 0.5)
        s = int(rng.integers(1, 1 << 30))
        label = f"case {case}: {dtype} K{K} V{V} H{H} HV{HV} B{B} T{T} cu={cu} A_log={A} fused={fused}"
        print(label, flush=True)
        wl = workloads.tiny_case(s, B=B, T=T, H=H, HV=HV, K=K, V=V, dtype=dtype, cu_seqlens=cu, A_log=A)
        d = device_inputs(wl)
        if fused:
            o, ht = kda.recurrent_kda(d["q"], d["k"], d["v"], d["x"], d["beta"], d["h0"],
                                      cu_seqlens=d["cu"], output_final_state=True,
                                      use_gate_in_kernel=True, A_log=d["A_log"])
        else:
            G1 = kda.gate_cumsum(d["x"], d["A_log"], d["cu"], 1)
            o, ht = kda.recurrent_kda(d["q"], d["k"], d["v"], G1, d["beta"], d["h0"],
                                      cu_seqlens=d["cu"], output_final_state=True)
        torch.cuda.synchronize()
        o_ref, ht_ref = oracle.forward(wl)
        mask = in_contract_rows(wl)
        err = normwise_max_err if dtype == "fp32" else rel_rms
        eo = err(to_np(o)[mask], o_ref[mask]) if mask.any() else 0.0
        eh = err(to_np(ht), ht_ref)
        ok = eo <= (2e-5 if dtype == "fp32" else 5e-3) and eh <= (2e-5 if dtype == "fp32" else 1e-2)
        print(f"   o {eo:.1e} state {eh:.1e}", flush=True)
        if not ok:
            failures.append((label, eo, eh))
    assert not failures, failures
