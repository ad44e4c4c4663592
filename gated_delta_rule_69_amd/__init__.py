"""MI355X-native Kimi Delta Attention (KDA) scan: thin Python binding of libkda.

Every step of the computation runs in the HIP kernels of `libkda.so`
(`csrc/`, built for gfx950 by `build.py`). This module only marshals
arguments: it reads shapes and device pointers from torch tensors, allocates
outputs and workspace with torch, and passes torch's current HIP stream. If the
library is missing it raises; there is no fallback path.

Entry points mirror the C ABI in `include/kda.h` (same names and argument
order as the `recurrent_kda(q, k, v, gate, beta, initial_state=None, *,
cu_seqlens=None, output_final_state=False)` contract described in "kda in
torchtitan (training)", quoted attention-gym description):
  gate_cumsum     step A1  (kda_gate_cumsum)
  chunk_kda       steps A2..A6 (kda_chunk_fwd); with use_gate_in_kernel=True
                  steps A1..A6 (kda_chunk_fwd_fused_gate)
  chunk_kda_bwd   steps B1..B3 (kda_chunk_bwd)
  recurrent_kda   step A7  (kda_recurrent_fwd); with use_gate_in_kernel=True
                  steps A1 + A7 (kda_recurrent_fwd_fused_gate)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_FP32, KDA_BF16 = 0, 1
_STATUS = {0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_SHAPE", 3: "KDA_ERR_DTYPE",
           4: "KDA_ERR_UNSUPPORTED", 5: "KDA_ERR_ALIAS", 6: "KDA_ERR_WORKSPACE", 7: "KDA_ERR_LAUNCH"}

EXPORTED = ("kda_status_string", "kda_gate_cumsum", "kda_gate_cumsum_biased",
            "kda_gate_bwd_workspace_bytes", "kda_gate_bwd", "kda_chunk_fwd_workspace_bytes",
            "kda_chunk_fwd", "kda_chunk_fwd_fused_gate", "kda_chunk_bwd_workspace_bytes",
            "kda_chunk_bwd", "kda_recurrent_fwd", "kda_recurrent_fwd_fused_gate",
            "kda_chunk_fwd_ex", "kda_recurrent_fwd_ex", "kda_chunk_fwd_conv", "kda_short_conv_fwd",
            "kda_recurrent_fwd_conv_workspace_bytes", "kda_recurrent_fwd_conv",
            "kda_recurrent_fwd_conv_noalloc", "kda_chunk_fwd_train", "kda_chunk_bwd_saved",
            "kda_chunk_fwd_train_ex", "kda_chunk_bwd_ex")
# bytes of the library's static device scratch behind kda_recurrent_fwd_conv_noalloc
NOALLOC_SCRATCH_BYTES = 16 << 20
KDA_GATE_LOG2, KDA_GATE_NAT, KDA_GATE_RAW = 0, 1, 2


class KdaDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "T", "N", "H", "HV", "K", "V")]


class KdaShortConv(ctypes.Structure):
    """kda_short_conv: FP32 taps [channels, width] and optional biases of the
    short convolution applied to q, k and v."""
    _fields_ = [("q_weight", ctypes.c_void_p), ("k_weight", ctypes.c_void_p),
                ("v_weight", ctypes.c_void_p), ("q_bias", ctypes.c_void_p),
                ("k_bias", ctypes.c_void_p), ("v_bias", ctypes.c_void_p), ("width", ctypes.c_int32)]


class KdaError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {_STATUS.get(code, code)} ({_lib().kda_status_string(code).decode()})")
        self.code = code


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m gated_delta_rule_69_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        p, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        dims = ctypes.POINTER(KdaDims)
        lib.kda_status_string.argtypes = [ctypes.c_int]
        lib.kda_status_string.restype = ctypes.c_char_p
        lib.kda_gate_cumsum.argtypes = [dims, p, i32, p, p, i32, p, p]
        lib.kda_gate_cumsum.restype = ctypes.c_int
        lib.kda_gate_cumsum_biased.argtypes = [dims, p, p, p, p, i32, p, p]
        lib.kda_gate_cumsum_biased.restype = ctypes.c_int
        lib.kda_gate_bwd_workspace_bytes.argtypes = [dims]
        lib.kda_gate_bwd_workspace_bytes.restype = sz
        lib.kda_gate_bwd.argtypes = [dims, p, p, p, p, p, p, p, p, p, sz, p]
        lib.kda_gate_bwd.restype = ctypes.c_int
        lib.kda_chunk_fwd_workspace_bytes.argtypes = [dims, ctypes.c_int, i32]
        lib.kda_chunk_fwd_workspace_bytes.restype = sz
        lib.kda_chunk_fwd.argtypes = [dims, ctypes.c_int, p, p, p, p, p, p, p, i32, i32, p, p, p, sz, p]
        lib.kda_chunk_fwd.restype = ctypes.c_int
        lib.kda_chunk_fwd_fused_gate.argtypes = [dims, ctypes.c_int, p, p, p, p, i32, p, p, p, p,
                                                 i32, i32, p, p, p, sz, p]
        lib.kda_chunk_fwd_fused_gate.restype = ctypes.c_int
        lib.kda_chunk_bwd_workspace_bytes.argtypes = [dims, ctypes.c_int, i32]
        lib.kda_chunk_bwd_workspace_bytes.restype = sz
        lib.kda_chunk_bwd.argtypes = [dims, ctypes.c_int] + [p] * 7 + [i32] + [p] * 8 + [p, sz, p]
        lib.kda_chunk_bwd.restype = ctypes.c_int
        lib.kda_chunk_bwd_saved.argtypes = lib.kda_chunk_bwd.argtypes
        lib.kda_chunk_bwd_saved.restype = ctypes.c_int
        lib.kda_chunk_fwd_train.argtypes = lib.kda_chunk_fwd.argtypes
        lib.kda_chunk_fwd_train.restype = ctypes.c_int
        lib.kda_chunk_fwd_train_ex.argtypes = [dims, ctypes.c_int, p, p, p, p, i32, p, p, p, p, i32,
                                               i32, p, p, p, sz, p]
        lib.kda_chunk_fwd_train_ex.restype = ctypes.c_int
        lib.kda_chunk_bwd_ex.argtypes = ([dims, ctypes.c_int] + [p] * 4 + [i32, p] + [p] * 3 + [i32]
                                         + [p] * 8 + [i32, p, sz, p])
        lib.kda_chunk_bwd_ex.restype = ctypes.c_int
        lib.kda_recurrent_fwd.argtypes = [dims, ctypes.c_int, p, p, p, p, p, p, p, i32, p, p, p]
        lib.kda_recurrent_fwd.restype = ctypes.c_int
        lib.kda_recurrent_fwd_fused_gate.argtypes = [dims, ctypes.c_int, p, p, p, p, i32, p, p, p, p,
                                                     i32, p, p, p]
        lib.kda_recurrent_fwd_fused_gate.restype = ctypes.c_int
        lib.kda_chunk_fwd_ex.argtypes = [dims, ctypes.c_int, p, p, p, p, i32, p, i32, p, p, p, i32, i32,
                                         p, p, p, sz, p]
        lib.kda_chunk_fwd_ex.restype = ctypes.c_int
        lib.kda_recurrent_fwd_ex.argtypes = [dims, ctypes.c_int, p, p, p, p, i32, p, i32, p, p, p, i32,
                                             p, p, p]
        lib.kda_recurrent_fwd_ex.restype = ctypes.c_int
        lib.kda_chunk_fwd_conv.argtypes = [dims, ctypes.c_int, p, p, p, ctypes.POINTER(KdaShortConv), p,
                                           i32, p, i32, p, p, p, i32, i32, p, p, p, sz, p]
        lib.kda_chunk_fwd_conv.restype = ctypes.c_int
        conv = ctypes.POINTER(KdaShortConv)
        lib.kda_short_conv_fwd.argtypes = [dims, ctypes.c_int, p, p, p, conv, p, p, p, p, p, p, p]
        lib.kda_short_conv_fwd.restype = ctypes.c_int
        lib.kda_recurrent_fwd_conv_workspace_bytes.argtypes = [dims, ctypes.c_int]
        lib.kda_recurrent_fwd_conv_workspace_bytes.restype = sz
        lib.kda_recurrent_fwd_conv.argtypes = [dims, ctypes.c_int, p, p, p, conv, p, p, p, i32, p, i32,
                                               p, p, p, i32, p, p, p, sz, p]
        lib.kda_recurrent_fwd_conv.restype = ctypes.c_int
        lib.kda_recurrent_fwd_conv_noalloc.argtypes = [dims, ctypes.c_int, p, p, p, conv, p, p, p, i32,
                                                       p, i32, p, p, p, i32, p, p, p]
        lib.kda_recurrent_fwd_conv_noalloc.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def load() -> ctypes.CDLL:
    """Load libkda.so (raises if it is not built)."""
    return _lib()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_FP32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _check(t: Optional[torch.Tensor], name: str):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dims(q, v, cu_seqlens) -> KdaDims:
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    return KdaDims(B, T, N, H, HV, K, V)


_I32_MAX = 2**31 - 1


def _expect(t: Optional[torch.Tensor], name: str, shape, dtype):
    """Raise unless `t` (if given) has exactly this shape and dtype."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _cu_dims(cu_seqlens: Optional[torch.Tensor], B: int) -> int:
    """Number of state entries N; checks cu_seqlens is a 1-D int32 tensor of
    N + 1 >= 1 offsets with B == 1 (the C ABI reads it as int32 on the device,
    so any other dtype would be misread rather than rejected there)."""
    if cu_seqlens is None:
        return B
    if not isinstance(cu_seqlens, torch.Tensor):
        raise TypeError("cu_seqlens must be a torch.Tensor")
    if cu_seqlens.dtype != torch.int32:
        raise TypeError(f"cu_seqlens must be torch.int32, got {cu_seqlens.dtype}")
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D tensor of N + 1 >= 1 offsets")
    if B != 1:
        raise ValueError(f"varlen inputs are packed into one batch row (B == 1), got B = {B}")
    return cu_seqlens.numel() - 1


def _validate_scan(q, k, v, gate, beta, initial_state, cu_seqlens, *, o=None, final_state=None,
                   A_log=None, do=None, dht=None):
    """Full dtype and shape check of the scan arguments before any pointer is
    handed to the C ABI, which cannot see buffer sizes: q, k [B, T, H, K] and
    v [B, T, HV, V] and beta [B, T, HV] in one dtype (bfloat16 or float32),
    gate [B, T, HV, K] float32, states [N, HV, K, V] float32, A_log [HV]
    float32, o like v, do like v, dht like the states."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (beta, "beta"), (gate, "gate")):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{n} must be a torch.Tensor")
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q must be [B, T, H, K] and v [B, T, HV, V]")
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    if tuple(v.shape[:2]) != (B, T):
        raise ValueError(f"v must be [{B}, {T}, HV, V], got {tuple(v.shape)}")
    if H < 1 or HV % H != 0:
        raise ValueError(f"HV ({HV}) must be a positive multiple of H ({H})")
    if max(B, T, H, HV, K, V) > _I32_MAX:
        raise ValueError("every size must fit the C ABI's int32 fields")
    dt = q.dtype
    if dt not in (torch.bfloat16, torch.float32):
        raise TypeError(f"q must be bfloat16 or float32, got {dt}")
    _expect(k, "k", (B, T, H, K), dt)
    _expect(v, "v", (B, T, HV, V), dt)
    _expect(beta, "beta", (B, T, HV), dt)
    _expect(gate, "gate", (B, T, HV, K), torch.float32)
    N = _cu_dims(cu_seqlens, B)
    st = (N, HV, K, V)
    _expect(initial_state, "initial_state", st, torch.float32)
    _expect(final_state, "final_state", st, torch.float32)
    _expect(o, "o", (B, T, HV, V), dt)
    _expect(A_log, "A_log", (HV,), torch.float32)
    _expect(do, "do", (B, T, HV, V), dt)
    _expect(dht, "dht", st, torch.float32)
    dev = q.device
    for t, n in ((k, "k"), (v, "v"), (gate, "gate"), (beta, "beta"), (initial_state, "initial_state"),
                 (cu_seqlens, "cu_seqlens"), (o, "o"), (final_state, "final_state"), (A_log, "A_log"),
                 (do, "do"), (dht, "dht")):
        if t is not None and t.device != dev:
            raise ValueError(f"{n} is on {t.device}, q on {dev}")


def _validate_gate(x, A_log, cu_seqlens, out=None, dt_bias=None, name="gate_in"):
    """x [B, T, HV, K] float32, A_log [HV], dt_bias [HV, K], out like x (all float32)."""
    if not isinstance(x, torch.Tensor) or x.dim() != 4:
        raise ValueError(f"{name} must be a [B, T, HV, K] tensor")
    B, T, HV, K = x.shape
    _expect(x, name, (B, T, HV, K), torch.float32)
    _expect(A_log, "A_log", (HV,), torch.float32)
    _expect(out, "out", (B, T, HV, K), torch.float32)
    if dt_bias is not None and dt_bias.numel() == HV * K and dt_bias.dim() == 1:
        _expect(dt_bias, "dt_bias", (HV * K,), torch.float32)
    else:
        _expect(dt_bias, "dt_bias", (HV, K), torch.float32)
    _cu_dims(cu_seqlens, B)


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def gate_cumsum(gate_in: torch.Tensor, A_log: Optional[torch.Tensor] = None,
                cu_seqlens: Optional[torch.Tensor] = None, chunk_size: int = 64,
                is_raw: bool = True, out: Optional[torch.Tensor] = None,
                dt_bias: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Step A1 (kda_gate_cumsum): [B, T, HV, K] FP32 raw gate input x (or the
    natural-log g if is_raw=False) -> chunk-local inclusive cumsum in log2 units.
    With dt_bias ([HV, K] FP32, raw input only) it is kda_gate_cumsum_biased."""
    _validate_gate(gate_in, A_log, cu_seqlens, out, dt_bias)
    for t, n in ((gate_in, "gate_in"), (A_log, "A_log"), (cu_seqlens, "cu_seqlens"), (out, "out"),
                 (dt_bias, "dt_bias")):
        _check(t, n)
    B, T, HV, K = gate_in.shape
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    d = KdaDims(B, T, N, 1, HV, K, 1)
    if out is None:
        out = torch.empty_like(gate_in)
    if dt_bias is not None:
        if not is_raw:
            raise ValueError("dt_bias applies to a raw gate input")
        rc = _lib().kda_gate_cumsum_biased(ctypes.byref(d), _ptr(gate_in), _ptr(A_log), _ptr(dt_bias),
                                           _ptr(cu_seqlens), int(chunk_size), _ptr(out), _stream())
        if rc:
            raise KdaError("kda_gate_cumsum_biased", rc)
        return out
    rc = _lib().kda_gate_cumsum(ctypes.byref(d), _ptr(gate_in), int(is_raw), _ptr(A_log),
                                _ptr(cu_seqlens), int(chunk_size), _ptr(out), _stream())
    if rc:
        raise KdaError("kda_gate_cumsum", rc)
    return out


def gate_bwd_workspace_bytes(x: torch.Tensor, cu_seqlens: Optional[torch.Tensor] = None) -> int:
    """Workspace bytes kda_gate_bwd needs for x [B, T, HV, K] when it reduces dA_log or d_dt_bias."""
    B, T, HV, K = x.shape
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    d = KdaDims(B, T, N, 1, HV, K, 1)
    return int(_lib().kda_gate_bwd_workspace_bytes(ctypes.byref(d)))


def gate_bwd(x: torch.Tensor, dg: torch.Tensor, A_log: Optional[torch.Tensor] = None,
             dt_bias: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None,
             dx: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Reverse of the raw gate activation (kda_gate_bwd): x, dg [B, T, HV, K] FP32
    (dg = gradient of the per-token natural-log gate, e.g. chunk_kda_bwd's dg) ->
    (dx, dA_log or None, d_dt_bias or None); the parameter gradients are
    produced exactly for the parameters given."""
    _validate_gate(x, A_log, cu_seqlens, dx, dt_bias, name="x")
    _expect(dg, "dg", tuple(x.shape), torch.float32)
    for t, n in ((x, "x"), (dg, "dg"), (A_log, "A_log"), (dt_bias, "dt_bias"),
                 (cu_seqlens, "cu_seqlens"), (dx, "dx"), (workspace, "workspace")):
        _check(t, n)
    B, T, HV, K = x.shape
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    d = KdaDims(B, T, N, 1, HV, K, 1)
    if dx is None:
        dx = torch.empty_like(x)
    dA = None if A_log is None else torch.empty(HV, device=x.device, dtype=torch.float32)
    db = None if dt_bias is None else torch.empty(HV, K, device=x.device, dtype=torch.float32)
    need = int(_lib().kda_gate_bwd_workspace_bytes(ctypes.byref(d)))
    if (dA is not None or db is not None) and workspace is None:
        workspace = torch.empty(max(need, 1), device=x.device, dtype=torch.uint8)
    ws_bytes = _nbytes(workspace)
    rc = _lib().kda_gate_bwd(ctypes.byref(d), _ptr(x), _ptr(A_log), _ptr(dt_bias), _ptr(dg),
                             _ptr(cu_seqlens), _ptr(dx), _ptr(dA), _ptr(db), _ptr(workspace),
                             ws_bytes, _stream())
    if rc:
        raise KdaError("kda_gate_bwd", rc)
    return dx, dA, db


def chunk_workspace_bytes(q: torch.Tensor, v: torch.Tensor, cu_seqlens=None, chunk_size: int = 64) -> int:
    d = _dims(q, v, cu_seqlens)
    return int(_lib().kda_chunk_fwd_workspace_bytes(ctypes.byref(d), _dtype_code(q), int(chunk_size)))


def chunk_kda(q, k, v, gate, beta, initial_state=None, *, cu_seqlens=None,
              output_final_state: bool = False, chunk_size: int = 64,
              o: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, use_gate_in_kernel: bool = False,
              A_log: Optional[torch.Tensor] = None, gate_is_raw: bool = True,
              qk_l2norm: bool = False, short_conv=None,
              save_for_backward: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Steps A2..A6 (kda_chunk_fwd). `gate` is the chunk-local cumulative log2
    gate (gate_cumsum with the same chunk_size). With use_gate_in_kernel=True,
    `gate` is gate_cumsum's input instead (raw x with optional A_log, or the
    natural-log g if gate_is_raw=False) and the gate step runs inside the
    chunk kernel (kda_chunk_fwd_fused_gate). qk_l2norm=True normalises q and k
    in the kernel (kda_chunk_fwd_ex). short_conv=((wq, bq), (wk, bk), (wv, bv))
    treats q, k, v as raw projections and applies the short causal convolution
    + SiLU to them in the kernel (kda_chunk_fwd_conv): FP32 taps [H*K, W] /
    [HV*V, W] (a [D, 1, W] Conv1d weight is accepted too), biases or None.
    save_for_backward: a device buffer of at least chunk_bwd_workspace_bytes()
    bytes: the forward runs as kda_chunk_fwd_train (kda_chunk_fwd_train_ex
    with use_gate_in_kernel=True) and leaves the chunk start states and Deltas
    there for chunk_kda_bwd(..., saved=True, workspace=that buffer, and the
    same gate arguments), which then skips the recurrence.
    Returns (o, final_state)."""
    _validate_scan(q, k, v, gate, beta, initial_state, cu_seqlens, o=o, final_state=final_state,
                   A_log=A_log)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (gate, "gate"), (beta, "beta"),
                 (initial_state, "initial_state"), (cu_seqlens, "cu_seqlens"), (A_log, "A_log"),
                 (o, "o"), (final_state, "final_state"), (workspace, "workspace")):
        _check(t, n)
    if A_log is not None and not use_gate_in_kernel:
        raise ValueError("A_log needs use_gate_in_kernel=True (else pass it to gate_cumsum)")
    d = _dims(q, v, cu_seqlens)
    dt = _dtype_code(q)
    if o is None:
        o = torch.empty_like(v)
    if output_final_state and final_state is None:
        final_state = torch.empty((d.N, d.HV, d.K, d.V), device=q.device, dtype=torch.float32)
    if not output_final_state:
        final_state = None
    need = int(_lib().kda_chunk_fwd_workspace_bytes(ctypes.byref(d), dt, int(chunk_size)))
    if save_for_backward is None and (workspace is None or _nbytes(workspace) < need):
        workspace = torch.empty(max(need, 1), device=q.device, dtype=torch.uint8)
    kind = (KDA_GATE_RAW if gate_is_raw else KDA_GATE_NAT) if use_gate_in_kernel else KDA_GATE_LOG2
    if save_for_backward is not None:
        if qk_l2norm or short_conv is not None:
            raise ValueError("save_for_backward runs without in-kernel normalisation or convolution")
        _check(save_for_backward, "save_for_backward")
        if use_gate_in_kernel:
            rc = _lib().kda_chunk_fwd_train_ex(
                ctypes.byref(d), dt, _ptr(q), _ptr(k), _ptr(v), _ptr(gate), kind, _ptr(A_log),
                _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens), int(chunk_size),
                int(bool(output_final_state)), _ptr(o), _ptr(final_state), _ptr(save_for_backward),
                _nbytes(save_for_backward), _stream())
            if rc:
                raise KdaError("kda_chunk_fwd_train_ex", rc)
            return o, final_state
        rc = _lib().kda_chunk_fwd_train(
            ctypes.byref(d), dt, _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta),
            _ptr(initial_state), _ptr(cu_seqlens), int(chunk_size), int(bool(output_final_state)),
            _ptr(o), _ptr(final_state), _ptr(save_for_backward), _nbytes(save_for_backward),
            _stream())
        if rc:
            raise KdaError("kda_chunk_fwd_train", rc)
        return o, final_state
    if short_conv is not None:
        sc = _short_conv(short_conv, d)
        rc = _lib().kda_chunk_fwd_conv(
            ctypes.byref(d), dt, _ptr(q), _ptr(k), _ptr(v), ctypes.byref(sc), _ptr(gate), kind,
            _ptr(A_log), int(bool(qk_l2norm)), _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens),
            int(chunk_size), int(bool(output_final_state)), _ptr(o), _ptr(final_state),
            _ptr(workspace), _nbytes(workspace), _stream())
        if rc:
            raise KdaError("kda_chunk_fwd_conv", rc)
        return o, final_state
    if qk_l2norm:
        rc = _lib().kda_chunk_fwd_ex(
            ctypes.byref(d), dt, _ptr(q), _ptr(k), _ptr(v), _ptr(gate), kind, _ptr(A_log), 1,
            _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens), int(chunk_size),
            int(bool(output_final_state)), _ptr(o), _ptr(final_state), _ptr(workspace),
            _nbytes(workspace), _stream())
        if rc:
            raise KdaError("kda_chunk_fwd_ex", rc)
        return o, final_state
    if use_gate_in_kernel:
        rc = _lib().kda_chunk_fwd_fused_gate(
            ctypes.byref(d), dt, _ptr(q), _ptr(k), _ptr(v), _ptr(gate), int(bool(gate_is_raw)),
            _ptr(A_log), _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens), int(chunk_size),
            int(bool(output_final_state)), _ptr(o), _ptr(final_state), _ptr(workspace),
            _nbytes(workspace), _stream())
        if rc:
            raise KdaError("kda_chunk_fwd_fused_gate", rc)
        return o, final_state
    rc = _lib().kda_chunk_fwd(ctypes.byref(d), dt, _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta),
                              _ptr(initial_state), _ptr(cu_seqlens), int(chunk_size),
                              int(bool(output_final_state)), _ptr(o), _ptr(final_state),
                              _ptr(workspace), _nbytes(workspace), _stream())
    if rc:
        raise KdaError("kda_chunk_fwd", rc)
    return o, final_state


def _short_conv(short_conv, d: KdaDims) -> KdaShortConv:
    """Marshal ((wq, bq), (wk, bk), (wv, bv)) into a kda_short_conv (the
    tensors must stay alive until the call returns; the caller holds them)."""
    (wq, bq), (wk, bk), (wv, bv) = short_conv
    widths = set()
    for t, n in ((wq, "wq"), (wk, "wk"), (wv, "wv"), (bq, "bq"), (bk, "bk"), (bv, "bv")):
        _check(t, n)
        if t is not None and t.dtype != torch.float32:
            raise TypeError(f"short_conv {n} must be float32")
    for w in (wq, wk, wv):
        if w.dim() not in (2, 3) or (w.dim() == 3 and w.shape[1] != 1):
            raise ValueError("short_conv weights are [D, W] or [D, 1, W]")
        widths.add(int(w.shape[-1]))
    if len(widths) != 1:
        raise ValueError("q, k and v convolutions must have one width")
    W = next(iter(widths))
    for w, b, n, D in ((wq, bq, "q", d.H * d.K), (wk, bk, "k", d.H * d.K), (wv, bv, "v", d.HV * d.V)):
        if w.numel() != D * W or (b is not None and b.numel() != D):
            raise ValueError(f"short_conv {n}: weight must be [{D}, {W}] and bias [{D}]")
    return KdaShortConv(wq.data_ptr(), wk.data_ptr(), wv.data_ptr(),
                        None if bq is None else bq.data_ptr(), None if bk is None else bk.data_ptr(),
                        None if bv is None else bv.data_ptr(), W)


def chunk_bwd_workspace_bytes(q: torch.Tensor, v: torch.Tensor, cu_seqlens=None,
                              chunk_size: int = 64) -> int:
    d = _dims(q, v, cu_seqlens)
    return int(_lib().kda_chunk_bwd_workspace_bytes(ctypes.byref(d), _dtype_code(q), int(chunk_size)))


def chunk_kda_bwd(q, k, v, gate, beta, initial_state, do, dht=None, *, cu_seqlens=None,
                  chunk_size: int = 64, workspace: Optional[torch.Tensor] = None,
                  saved: bool = False, use_gate_in_kernel: bool = False,
                  A_log: Optional[torch.Tensor] = None, gate_is_raw: bool = True):
    """Steps B1..B3 (kda_chunk_bwd). Returns a dict with dq, dk (shape of q),
    dv (shape of v), dg (FP32, w.r.t. the per-token natural-log gate), dbeta
    and dh0 (FP32 [N, HV, K, V]). saved=True (kda_chunk_bwd_saved): `workspace`
    is the buffer a chunk_kda(..., save_for_backward=workspace) call on the
    same inputs filled, and the recurrence is not run again. With
    use_gate_in_kernel=True (kda_chunk_bwd_ex), `gate` is gate_cumsum's input
    (raw x with optional A_log, or the natural-log g if gate_is_raw=False), as
    in chunk_kda, and the gate step runs inside the backward's kernels."""
    _validate_scan(q, k, v, gate, beta, initial_state, cu_seqlens, do=do, dht=dht, A_log=A_log)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (gate, "gate"), (beta, "beta"), (do, "do"),
                 (initial_state, "initial_state"), (dht, "dht"), (cu_seqlens, "cu_seqlens"),
                 (workspace, "workspace"), (A_log, "A_log")):
        _check(t, n)
    if A_log is not None and not (use_gate_in_kernel and gate_is_raw):
        raise ValueError("A_log needs use_gate_in_kernel=True with a raw gate")
    d = _dims(q, v, cu_seqlens)
    dt = _dtype_code(q)
    # the kernels write every row inside a sequence: dense inputs need no fill;
    # packed inputs get zeros in the capacity tail, which no kernel touches
    new = torch.empty_like if cu_seqlens is None else torch.zeros_like
    dq, dk, dv = new(q), new(k), new(v)
    dg = new(gate)
    dbeta = new(beta)
    dh0 = torch.empty((d.N, d.HV, d.K, d.V), device=q.device, dtype=torch.float32)
    need = int(_lib().kda_chunk_bwd_workspace_bytes(ctypes.byref(d), dt, int(chunk_size)))
    if saved:
        if workspace is None:
            raise ValueError("saved=True needs the workspace the training forward filled")
    elif workspace is None or _nbytes(workspace) < need:
        workspace = torch.empty(max(need, 1), device=q.device, dtype=torch.uint8)
    if use_gate_in_kernel:
        kind = KDA_GATE_RAW if gate_is_raw else KDA_GATE_NAT
        rc = _lib().kda_chunk_bwd_ex(
            ctypes.byref(d), dt, _ptr(q), _ptr(k), _ptr(v), _ptr(gate), kind, _ptr(A_log),
            _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens), int(chunk_size), _ptr(do),
            _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dh0),
            int(bool(saved)), _ptr(workspace), _nbytes(workspace), _stream())
        if rc:
            raise KdaError("kda_chunk_bwd_ex", rc)
        return dict(dq=dq, dk=dk, dv=dv, dg=dg, dbeta=dbeta, dh0=dh0)
    fn = _lib().kda_chunk_bwd_saved if saved else _lib().kda_chunk_bwd
    rc = fn(ctypes.byref(d), dt, _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta),
            _ptr(initial_state), _ptr(cu_seqlens), int(chunk_size), _ptr(do),
            _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta),
            _ptr(dh0), _ptr(workspace), _nbytes(workspace), _stream())
    if rc:
        raise KdaError("kda_chunk_bwd_saved" if saved else "kda_chunk_bwd", rc)
    return dict(dq=dq, dk=dk, dv=dv, dg=dg, dbeta=dbeta, dh0=dh0)


def conv_state_shape(q, v, cu_seqlens, width: int):
    """Shape of a short-convolution history: [N, width - 1, 2*H*K + HV*V]."""
    d = _dims(q, v, cu_seqlens)
    return (d.N, width - 1, 2 * d.H * d.K + d.HV * d.V)


def short_conv(q, k, v, short_conv, *, cu_seqlens=None, conv_state=None, conv_state_out=None,
               outputs: bool = True, out=None):
    """kda_short_conv_fwd: SiLU(causal conv) of raw q, k, v continuing each
    sequence from its carried history `conv_state` ([N, W-1, 2HK + HV V] in the
    input dtype, oldest row first; None = zeros). The new history goes to
    `conv_state_out` (may be conv_state itself; None = not kept). outputs=False
    computes the history only (prefill hand-off). `out` = (q_out, k_out, v_out)
    to write into (may be the inputs). Returns ((q, k, v) or None, conv_state_out)."""
    if q.dim() != 4 or v.dim() != 4 or q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q must be [B, T, H, K] and v [B, T, HV, V], bfloat16 or float32")
    _expect(k, "k", tuple(q.shape), q.dtype)
    _expect(v, "v", tuple(q.shape[:2]) + tuple(v.shape[2:]), q.dtype)
    _cu_dims(cu_seqlens, q.shape[0])
    if out is not None:
        for t, ref, n in zip(out, (q, k, v), ("q_out", "k_out", "v_out")):
            _expect(t, n, tuple(ref.shape), ref.dtype)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (cu_seqlens, "cu_seqlens"), (conv_state, "conv_state"),
                 (conv_state_out, "conv_state_out")):
        _check(t, n)
    d = _dims(q, v, cu_seqlens)
    dt = _dtype_code(q)
    sc = _short_conv(short_conv, d)
    for st, n in ((conv_state, "conv_state"), (conv_state_out, "conv_state_out")):
        if st is not None and (tuple(st.shape) != conv_state_shape(q, v, cu_seqlens, sc.width)
                               or st.dtype != q.dtype):
            raise ValueError(f"{n} must be {conv_state_shape(q, v, cu_seqlens, sc.width)} {q.dtype}")
    res = None
    if outputs:
        res = out if out is not None else (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    rc = _lib().kda_short_conv_fwd(ctypes.byref(d), dt, _ptr(q), _ptr(k), _ptr(v), ctypes.byref(sc),
                                   _ptr(cu_seqlens), _ptr(conv_state), _ptr(conv_state_out),
                                   *(_ptr(t) for t in (res or (None, None, None))), _stream())
    if rc:
        raise KdaError("kda_short_conv_fwd", rc)
    return res, conv_state_out


def recurrent_kda(q, k, v, gate, beta, initial_state=None, *, cu_seqlens=None,
                  output_final_state: bool = False, o: Optional[torch.Tensor] = None,
                  final_state: Optional[torch.Tensor] = None, use_gate_in_kernel: bool = False,
                  A_log: Optional[torch.Tensor] = None, gate_is_raw: bool = True,
                  qk_l2norm: bool = False, short_conv=None, conv_state=None, conv_state_out=None,
                  workspace: Optional[torch.Tensor] = None,
                  no_alloc: bool = False) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Step A7 (kda_recurrent_fwd). `gate` is the per-token log2 decay
    (gate_cumsum with chunk_size=1). With use_gate_in_kernel=True, `gate` is
    gate_cumsum's input instead (raw x with optional A_log, or the natural-log
    g if gate_is_raw=False), activated inside the scan kernel
    (kda_recurrent_fwd_fused_gate). qk_l2norm=True normalises q and k in the
    kernel (kda_recurrent_fwd_ex). short_conv=((wq, bq), (wk, bk), (wv, bv))
    treats q, k, v as raw projections and runs the short convolution + SiLU
    first, continuing each sequence from `conv_state` and writing the new
    history to `conv_state_out` (kda_recurrent_fwd_conv; see short_conv);
    with no_alloc=True that step runs kda_recurrent_fwd_conv_noalloc instead,
    which takes no workspace (the library's own static scratch; pass `o` and
    `final_state` too so that nothing is allocated at all). Inference only: inputs that require grad are rejected (use chunk_kda for
    training). Pass final_state=initial_state to update the states in place."""
    if any(t is not None and t.requires_grad for t in (q, k, v, gate, beta, initial_state)):
        raise RuntimeError("recurrent_kda is inference-only; inputs require grad (use chunk_kda)")
    _validate_scan(q, k, v, gate, beta, initial_state, cu_seqlens, o=o, final_state=final_state,
                   A_log=A_log)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (gate, "gate"), (beta, "beta"),
                 (initial_state, "initial_state"), (cu_seqlens, "cu_seqlens"), (A_log, "A_log"),
                 (o, "o"), (final_state, "final_state"), (workspace, "workspace")):
        _check(t, n)
    if A_log is not None and not use_gate_in_kernel:
        raise ValueError("A_log needs use_gate_in_kernel=True (else pass it to gate_cumsum)")
    if no_alloc and short_conv is None:
        raise ValueError("no_alloc applies to decode from raw projections (short_conv)")
    d = _dims(q, v, cu_seqlens)
    dt = _dtype_code(q)
    if o is None:
        o = torch.empty_like(v)
    if output_final_state and final_state is None:
        final_state = torch.empty((d.N, d.HV, d.K, d.V), device=q.device, dtype=torch.float32)
    if not output_final_state:
        final_state = None
    kind = (KDA_GATE_RAW if gate_is_raw else KDA_GATE_NAT) if use_gate_in_kernel else KDA_GATE_LOG2
    if short_conv is not None:
        sc = _short_conv(short_conv, d)
        for st, n in ((conv_state, "conv_state"), (conv_state_out, "conv_state_out")):
            _check(st, n)
            if st is not None and (tuple(st.shape) != conv_state_shape(q, v, cu_seqlens, sc.width)
                                   or st.dtype != q.dtype):
                raise ValueError(f"{n} must be {conv_state_shape(q, v, cu_seqlens, sc.width)} {q.dtype}")
        if no_alloc:
            rc = _lib().kda_recurrent_fwd_conv_noalloc(
                ctypes.byref(d), dt, _ptr(q), _ptr(k), _ptr(v), ctypes.byref(sc), _ptr(conv_state),
                _ptr(conv_state_out), _ptr(gate), kind, _ptr(A_log), int(bool(qk_l2norm)), _ptr(beta),
                _ptr(initial_state), _ptr(cu_seqlens), int(bool(output_final_state)), _ptr(o),
                _ptr(final_state), _stream())
            if rc:
                raise KdaError("kda_recurrent_fwd_conv_noalloc", rc)
            return o, final_state
        need = int(_lib().kda_recurrent_fwd_conv_workspace_bytes(ctypes.byref(d), dt))
        if workspace is None or _nbytes(workspace) < need:
            workspace = torch.empty(max(need, 1), device=q.device, dtype=torch.uint8)
        rc = _lib().kda_recurrent_fwd_conv(
            ctypes.byref(d), dt, _ptr(q), _ptr(k), _ptr(v), ctypes.byref(sc), _ptr(conv_state),
            _ptr(conv_state_out), _ptr(gate), kind, _ptr(A_log), int(bool(qk_l2norm)), _ptr(beta),
            _ptr(initial_state), _ptr(cu_seqlens), int(bool(output_final_state)), _ptr(o),
            _ptr(final_state), _ptr(workspace), _nbytes(workspace), _stream())
        if rc:
            raise KdaError("kda_recurrent_fwd_conv", rc)
        return o, final_state
    if qk_l2norm:
        rc = _lib().kda_recurrent_fwd_ex(
            ctypes.byref(d), dt, _ptr(q), _ptr(k), _ptr(v), _ptr(gate), kind, _ptr(A_log), 1,
            _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens), int(bool(output_final_state)), _ptr(o),
            _ptr(final_state), _stream())
        if rc:
            raise KdaError("kda_recurrent_fwd_ex", rc)
        return o, final_state
    if use_gate_in_kernel:
        rc = _lib().kda_recurrent_fwd_fused_gate(
            ctypes.byref(d), dt, _ptr(q), _ptr(k), _ptr(v), _ptr(gate), int(bool(gate_is_raw)),
            _ptr(A_log), _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens),
            int(bool(output_final_state)), _ptr(o), _ptr(final_state), _stream())
        if rc:
            raise KdaError("kda_recurrent_fwd_fused_gate", rc)
        return o, final_state
    rc = _lib().kda_recurrent_fwd(ctypes.byref(d), dt, _ptr(q), _ptr(k), _ptr(v), _ptr(gate),
                                  _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens),
                                  int(bool(output_final_state)), _ptr(o), _ptr(final_state), _stream())
    if rc:
        raise KdaError("kda_recurrent_fwd", rc)
    return o, final_state


__all__ = ["gate_cumsum", "chunk_kda", "chunk_kda_bwd", "recurrent_kda", "short_conv", "conv_state_shape",
           "chunk_workspace_bytes", "load",
           "KdaDims", "KdaShortConv", "KdaError", "LIB_PATH", "EXPORTED", "KDA_FP32", "KDA_BF16"]
