"""C-ABI checks that need no GPU: the library loads, exports every entry point
that include/kda.h declares, and rejects bad arguments before any launch."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_69_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    assert set(_declared()) == set(kda.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = kda.load()
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings():
    lib = kda.load()
    for code in range(8):
        assert lib.kda_status_string(code)


FAKE = [ctypes.c_void_p(0x10000 * (i + 1)) for i in range(16)]  # never dereferenced


def _dims(**kw):
    d = dict(B=1, T=64, N=1, H=1, HV=1, K=64, V=64)
    d.update(kw)
    return kda.KdaDims(**d)


def _chunk(lib, d, dt=1, chunk=64, ws=None, ws_bytes=1 << 40, h0=None, ht=None, o=None, cu=None, fin=1):
    return lib.kda_chunk_fwd(ctypes.byref(d), dt, FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4],
                             h0, cu, chunk, fin, o if o is not None else FAKE[5],
                             ht if ht is not None else FAKE[6],
                             ws if ws is not None else FAKE[7], ws_bytes, None)


def test_chunk_rejects_bad_arguments():
    lib = kda.load()
    assert lib.kda_chunk_fwd(None, 1, *[None] * 7, 64, 0, None, None, None, 0, None) == 1  # NULL dims
    assert _chunk(lib, _dims(H=2, HV=3)) == 2  # HV % H != 0
    assert _chunk(lib, _dims(N=2)) == 2  # dense needs N == B
    assert _chunk(lib, _dims(B=2, N=2), cu=FAKE[8]) == 2  # varlen needs B == 1
    assert _chunk(lib, _dims(), dt=7) == 3  # dtype
    assert _chunk(lib, _dims(), chunk=32) == 4  # chunk size
    assert _chunk(lib, _dims(K=96)) == 4  # head dim
    assert _chunk(lib, _dims(), ws_bytes=16) == 6  # workspace too small
    assert _chunk(lib, _dims(), o=FAKE[0]) == 5  # o aliases q
    assert _chunk(lib, _dims(), h0=ctypes.c_void_p(0x10000 * 7 + 64)) == 5  # partial state overlap
    d = _dims()
    assert lib.kda_chunk_fwd(ctypes.byref(d), 1, FAKE[0], None, FAKE[2], FAKE[3], FAKE[4], None, None,
                             64, 0, FAKE[5], None, FAKE[7], 1 << 40, None) == 1  # k NULL
    assert lib.kda_chunk_fwd(ctypes.byref(d), 1, FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4], None, None,
                             64, 1, FAKE[5], None, FAKE[7], 1 << 40, None) == 1  # final_state NULL


def test_recurrent_rejects_bad_arguments():
    lib = kda.load()
    d = _dims(K=300)
    assert lib.kda_recurrent_fwd(ctypes.byref(d), 0, FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4],
                                 None, None, 0, FAKE[5], None, None) == 4
    d = _dims(H=3, HV=4)
    assert lib.kda_recurrent_fwd(ctypes.byref(d), 0, FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4],
                                 None, None, 0, FAKE[5], None, None) == 2


def test_gate_rejects_bad_arguments():
    lib = kda.load()
    d = _dims()
    assert lib.kda_gate_cumsum(ctypes.byref(d), FAKE[0], 1, None, None, 0, FAKE[1], None) == 4
    assert lib.kda_gate_cumsum(ctypes.byref(d), FAKE[0], 1, None, None, 65, FAKE[1], None) == 4
    assert lib.kda_gate_cumsum(ctypes.byref(d), FAKE[0], 0, FAKE[2], None, 64, FAKE[1], None) == 2
    assert lib.kda_gate_cumsum(ctypes.byref(d), FAKE[0], 1, None, None, 64, FAKE[0], None) == 5


def test_workspace_bytes():
    lib = kda.load()
    d = _dims(B=4, T=4096, N=4, H=16, HV=16, K=128, V=128)
    b = lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(d), 1, 64)
    assert b > 4 * 64 * 16 * 64 * 128 * 2
    assert lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(d), 1, 32) == 0


def test_workspace_bindings_match_the_c_calls():
    """The binding's workspace helpers only marshal shapes (meta tensors, no
    device): they equal the C calls, grow with T, cover a varlen batch's extra
    partial chunks, and the backward's workspace holds at least the forward's."""
    import torch
    lib = kda.load()
    for T in (0, 1, 64, 4096):
        q = torch.empty((4, T, 16, 128), dtype=torch.bfloat16, device="meta")
        v = torch.empty((4, T, 16, 128), dtype=torch.bfloat16, device="meta")
        d = _dims(B=4, T=T, N=4, H=16, HV=16, K=128, V=128)
        f = kda.chunk_workspace_bytes(q, v)
        b = kda.chunk_bwd_workspace_bytes(q, v)
        assert f == lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(d), 1, 64)
        assert b == lib.kda_chunk_bwd_workspace_bytes(ctypes.byref(d), 1, 64)
        assert b >= f
    small = kda.chunk_workspace_bytes(torch.empty((1, 64, 16, 128), device="meta", dtype=torch.bfloat16),
                                      torch.empty((1, 64, 16, 128), device="meta", dtype=torch.bfloat16))
    big = kda.chunk_workspace_bytes(torch.empty((1, 4096, 16, 128), device="meta", dtype=torch.bfloat16),
                                    torch.empty((1, 4096, 16, 128), device="meta", dtype=torch.bfloat16))
    assert big > small
    cu = torch.empty((6,), dtype=torch.int32, device="meta")  # 5 sequences packed in one row
    q1 = torch.empty((1, 4096, 16, 128), dtype=torch.bfloat16, device="meta")
    assert kda.chunk_workspace_bytes(q1, q1, cu) > kda.chunk_workspace_bytes(q1, q1)


def test_fused_gate_entries_reject_bad_arguments():
    lib = kda.load()
    d = _dims()

    def chunk(is_raw, A_log, o=FAKE[5], chunk=64):
        return lib.kda_chunk_fwd_fused_gate(ctypes.byref(d), 1, FAKE[0], FAKE[1], FAKE[2], FAKE[3],
                                            is_raw, A_log, FAKE[4], None, None, chunk, 1, o,
                                            FAKE[6], FAKE[7], 1 << 40, None)

    def rec(is_raw, A_log, o=FAKE[5], dd=d):
        return lib.kda_recurrent_fwd_fused_gate(ctypes.byref(dd), 1, FAKE[0], FAKE[1], FAKE[2],
                                                FAKE[3], is_raw, A_log, FAKE[4], None, None, 1, o,
                                                FAKE[6], None)

    assert chunk(0, FAKE[9]) == 2  # A_log only with a raw gate input
    assert rec(0, FAKE[9]) == 2
    assert chunk(1, FAKE[9], chunk=32) == 4
    assert chunk(1, FAKE[5]) == 5  # A_log overlaps o
    assert rec(1, FAKE[5]) == 5
    assert chunk(1, FAKE[9], o=FAKE[3]) == 5  # o overlaps the gate input
    assert rec(1, None, dd=_dims(V=300)) == 4


def test_gate_bias_and_gate_bwd_reject_bad_arguments():
    lib = kda.load()
    d = _dims()
    # kda_gate_cumsum_biased(dims, x, A_log, dt_bias, cu, chunk, out, stream)
    assert lib.kda_gate_cumsum_biased(ctypes.byref(d), FAKE[0], None, FAKE[2], None, 0, FAKE[1], None) == 4
    assert lib.kda_gate_cumsum_biased(ctypes.byref(d), FAKE[0], None, FAKE[2], None, 64, FAKE[0], None) == 5
    assert lib.kda_gate_cumsum_biased(ctypes.byref(d), FAKE[0], None, FAKE[1], None, 64, FAKE[1], None) == 5
    need = lib.kda_gate_bwd_workspace_bytes(ctypes.byref(d))
    assert need >= 2 * 64 * 4

    # kda_gate_bwd(dims, x, A_log, dt_bias, dg, cu, dx, dA_log, d_dt_bias, ws, ws_bytes, stream)
    def bwd(A_log=None, bias=None, dx=FAKE[4], dA=None, db=None, ws=FAKE[7], ws_bytes=1 << 30, dd=d):
        return lib.kda_gate_bwd(ctypes.byref(dd), FAKE[0], A_log, bias, FAKE[3], None, dx, dA, db,
                                ws, ws_bytes, None)

    assert bwd(A_log=FAKE[1]) == 2                   # A_log given, dA_log missing
    assert bwd(dA=FAKE[5]) == 2                      # dA_log without A_log
    assert bwd(bias=FAKE[2]) == 2                    # dt_bias given, d_dt_bias missing
    assert bwd(A_log=FAKE[1], dA=FAKE[5], ws=None) == 6
    assert bwd(A_log=FAKE[1], dA=FAKE[5], ws_bytes=need - 1) == 6
    assert bwd(dx=FAKE[0]) == 5                      # dx overlaps x
    assert bwd(bias=FAKE[2], db=FAKE[4]) == 5        # d_dt_bias overlaps dx
    assert bwd(A_log=FAKE[1], dA=FAKE[5], ws=FAKE[4]) == 5  # workspace overlaps dx
    assert bwd(dd=_dims(K=5000)) == 4
    assert lib.kda_gate_bwd(ctypes.byref(d), None, None, None, FAKE[3], None, FAKE[4], None, None,
                            None, 0, None) == 1


def test_torch_ops_fake_shapes_on_meta_tensors():
    """The torch.library registrations import without a GPU and their fake
    implementations give the output shapes (dense and varlen, GVA)."""
    import torch

    import gated_delta_rule_69_amd.torch_ops  # noqa: F401

    m = dict(device="meta")
    q = torch.empty(1, 50, 2, 64, dtype=torch.bfloat16, **m)
    v = torch.empty(1, 50, 4, 32, dtype=torch.bfloat16, **m)
    x = torch.empty(1, 50, 4, 64, **m)
    beta = torch.empty(1, 50, 4, dtype=torch.bfloat16, **m)
    cu = torch.empty(4, dtype=torch.int32, **m)
    o, ht = torch.ops.kda.chunk_kda_train(q, q, v, x, beta, None, None, None, cu)
    assert o.shape == v.shape and o.dtype == v.dtype
    assert ht.shape == (3, 4, 64, 32) and ht.dtype == torch.float32
    o, ht = torch.ops.kda.recurrent_kda(q, q, v, x, beta, None, None, None)
    assert o.shape == v.shape and ht.shape == (1, 4, 64, 32)


def test_ex_entries_reject_bad_arguments():
    lib = kda.load()
    d = _dims()

    def chunk(kind, A_log):
        return lib.kda_chunk_fwd_ex(ctypes.byref(d), 1, FAKE[0], FAKE[1], FAKE[2], FAKE[3], kind,
                                    A_log, 1, FAKE[4], None, None, 64, 1, FAKE[5], FAKE[6], FAKE[7],
                                    1 << 40, None)

    def rec(kind, A_log):
        return lib.kda_recurrent_fwd_ex(ctypes.byref(d), 1, FAKE[0], FAKE[1], FAKE[2], FAKE[3], kind,
                                        A_log, 1, FAKE[4], None, None, 1, FAKE[5], FAKE[6], None)

    assert chunk(3, None) == 2 and rec(-1, None) == 2          # unknown gate kind
    assert chunk(0, FAKE[9]) == 2 and rec(1, FAKE[9]) == 2     # A_log only with a raw gate
    assert chunk(2, FAKE[5]) == 5                              # A_log overlaps o


def test_conv_entry_rejects_bad_arguments():
    lib = kda.load()
    d = _dims()

    def call(conv):
        return lib.kda_chunk_fwd_conv(ctypes.byref(d), 1, FAKE[0], FAKE[1], FAKE[2],
                                      None if conv is None else ctypes.byref(conv), FAKE[3], 2,
                                      None, 1, FAKE[4], None, None, 64, 1, FAKE[5], FAKE[6],
                                      FAKE[7], 1 << 40, None)

    def taps(width=4, **kw):
        f = dict(q_weight=FAKE[10].value, k_weight=FAKE[11].value, v_weight=FAKE[12].value,
                 q_bias=None, k_bias=None, v_bias=None, width=width)
        f.update(kw)
        return kda.KdaShortConv(**f)

    assert call(None) == 1                          # no taps
    assert call(taps(k_weight=None)) == 1           # a missing weight
    assert call(taps(width=0)) == 4                 # widths 1..4
    assert call(taps(width=5)) == 4
    assert call(taps(v_weight=FAKE[5].value)) == 5  # taps overlap o
    assert call(taps(q_bias=FAKE[6].value)) == 5    # bias overlaps the final state
    conv = taps()
    assert lib.kda_chunk_fwd_conv(ctypes.byref(d), 1, FAKE[0], FAKE[1], FAKE[2], ctypes.byref(conv),
                                  FAKE[3], 0, FAKE[9], 0, FAKE[4], None, None, 64, 1, FAKE[5],
                                  FAKE[6], FAKE[7], 1 << 40, None) == 2  # A_log with a log2 gate


def test_short_conv_and_conv_decode_reject_bad_arguments():
    lib = kda.load()
    d = _dims()

    def taps(width=4, **kw):
        f = dict(q_weight=FAKE[10].value, k_weight=FAKE[11].value, v_weight=FAKE[12].value,
                 q_bias=None, k_bias=None, v_bias=None, width=width)
        f.update(kw)
        return kda.KdaShortConv(**f)

    def sc(conv, outs=(FAKE[5], FAKE[6], FAKE[7]), st_in=None, st_out=None, dims=d, dt=1):
        return lib.kda_short_conv_fwd(ctypes.byref(dims), dt, FAKE[0], FAKE[1], FAKE[2],
                                      None if conv is None else ctypes.byref(conv), None, st_in,
                                      st_out, *outs, None)

    assert sc(None) == 1                                   # no taps
    assert sc(taps(v_weight=None)) == 1
    assert sc(taps(width=5)) == 4
    assert sc(taps(), outs=(FAKE[5], None, FAKE[7])) == 1  # outputs: all three or none
    assert sc(taps(), dims=_dims(K=60)) == 4               # 16-byte channel units
    assert sc(taps(), dt=9) == 3
    assert sc(taps(), outs=(FAKE[1], FAKE[6], FAKE[7])) == 5   # q_out over k
    assert sc(taps(q_weight=FAKE[6].value)) == 5               # taps under an output
    assert sc(taps(), outs=(ctypes.c_void_p(FAKE[5].value + 8), FAKE[6], FAKE[7])) == 4  # alignment
    # history-only mode with an in-place history is accepted up to the launch;
    # with N = 0 nothing is launched
    assert sc(taps(), outs=(None, None, None), st_in=FAKE[8], st_out=FAKE[8],
              dims=_dims(B=0, N=0)) == 0
    assert lib.kda_recurrent_fwd_conv_workspace_bytes(None, 1) == 0
    need = lib.kda_recurrent_fwd_conv_workspace_bytes(ctypes.byref(d), 1)
    assert need == 3 * 64 * 64 * 2

    def rec(conv, kind=2, A_log=None, ws=FAKE[13], ws_bytes=1 << 40):
        return lib.kda_recurrent_fwd_conv(ctypes.byref(d), 1, FAKE[0], FAKE[1], FAKE[2],
                                          None if conv is None else ctypes.byref(conv), None, None,
                                          FAKE[3], kind, A_log, 1, FAKE[4], None, None, 1, FAKE[5],
                                          FAKE[6], ws, ws_bytes, None)

    assert rec(taps(), kind=4) == 2
    assert rec(taps(), kind=0, A_log=FAKE[9]) == 2
    assert rec(None) == 1
    assert rec(taps(), ws=None) == 6
    assert rec(taps(), ws_bytes=need - 1) == 6
    assert rec(taps(), ws=FAKE[5]) == 5                    # workspace over o
    assert rec(taps(), ws=ctypes.c_void_p(FAKE[13].value + 16)) == 4

    def rec_hist(st_out, h0=None, A_log=None):
        return lib.kda_recurrent_fwd_conv(ctypes.byref(d), 1, FAKE[0], FAKE[1], FAKE[2],
                                          ctypes.byref(taps()), None, st_out, FAKE[3], 2, A_log, 1,
                                          FAKE[4], h0, None, 1, FAKE[5], FAKE[6], FAKE[13], 1 << 40,
                                          None)

    # the new history is written before the scan reads its inputs: it may overlap
    # none of them (initial state, gate, beta, A_log, taps), nor o or the states
    assert rec_hist(FAKE[9], h0=FAKE[9]) == 5      # history over the initial state
    assert rec_hist(FAKE[3]) == 5                  # over the gate
    assert rec_hist(FAKE[4]) == 5                  # over beta
    assert rec_hist(FAKE[8], A_log=FAKE[8]) == 5   # over A_log
    assert rec_hist(FAKE[10]) == 5                 # over the q taps
    assert rec_hist(FAKE[12]) == 5                 # over the v taps
    assert rec_hist(FAKE[5]) == 5                  # over o


def test_noalloc_conv_decode_checks_its_scratch_limit():
    """The allocation-free decode rejects a problem whose convolved q, k, v
    exceed the library's static scratch before touching any device."""
    lib = kda.load()
    assert lib.kda_recurrent_fwd_conv_noalloc(None, 1, *[None] * 4, None, None, None, 2, None, 1,
                                              None, None, None, 1, None, None, None) == 1
    big = _dims(T=4096, N=1, H=16, HV=32, K=128, V=128)
    assert lib.kda_recurrent_fwd_conv_workspace_bytes(ctypes.byref(big), 1) > kda.NOALLOC_SCRATCH_BYTES
    taps = kda.KdaShortConv(q_weight=FAKE[10].value, k_weight=FAKE[11].value, v_weight=FAKE[12].value,
                            q_bias=None, k_bias=None, v_bias=None, width=4)
    rc = lib.kda_recurrent_fwd_conv_noalloc(ctypes.byref(big), 1, FAKE[0], FAKE[1], FAKE[2],
                                            ctypes.byref(taps), None, None, FAKE[3], 2, None, 1,
                                            FAKE[4], None, FAKE[8], 1, FAKE[5], FAKE[6], None)
    assert rc == 6  # KDA_ERR_WORKSPACE


def test_training_forward_and_saved_backward_reject_bad_arguments():
    lib = kda.load()
    d = _dims(K=128, V=128)
    need_b = lib.kda_chunk_bwd_workspace_bytes(ctypes.byref(d), 1, 64)
    need_f = lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(d), 1, 64)
    assert need_b > need_f > 0

    def fwd(dims, dt=1, ws_bytes=1 << 40, ws=FAKE[7]):
        return lib.kda_chunk_fwd_train(ctypes.byref(dims), dt, FAKE[0], FAKE[1], FAKE[2], FAKE[3],
                                       FAKE[4], None, None, 64, 1, FAKE[5], FAKE[6], ws, ws_bytes, None)

    assert fwd(d, ws_bytes=need_f) == 6          # the backward's workspace is larger
    assert fwd(d, ws=None) == 6
    assert fwd(_dims(K=128, V=64), dt=0) == 4     # FP32 backward needs K = 64
    assert fwd(_dims(H=2, HV=3)) == 2
    assert fwd(d, ws=FAKE[5]) == 5                # workspace over o

    def bwd(dims, ws=FAKE[9], ws_bytes=1 << 40):
        return lib.kda_chunk_bwd_saved(ctypes.byref(dims), 1, FAKE[0], FAKE[1], FAKE[2], FAKE[3],
                                       FAKE[4], None, None, 64, FAKE[5], None, FAKE[6], FAKE[7],
                                       FAKE[8], FAKE[10], FAKE[11], FAKE[12], ws, ws_bytes, None)

    assert bwd(d, ws=None) == 6
    assert bwd(d, ws_bytes=need_b - 1) == 6
    assert bwd(_dims(K=96)) == 4


def test_prefill_and_step_ops_fake_shapes_on_meta_tensors():
    import torch

    import gated_delta_rule_69_amd.torch_ops  # noqa: F401

    m = dict(device="meta")
    q = torch.empty(1, 50, 2, 64, dtype=torch.bfloat16, **m)
    v = torch.empty(1, 50, 4, 32, dtype=torch.bfloat16, **m)
    x = torch.empty(1, 50, 4, 64, **m)
    beta = torch.empty(1, 50, 4, dtype=torch.bfloat16, **m)
    cu = torch.empty(4, dtype=torch.int32, **m)
    wq, wv = torch.empty(128, 4, **m), torch.empty(128, 4, **m)
    o, ht, hist = torch.ops.kda.chunk_kda_prefill(q, q, v, x, beta, None, None, cu, True,
                                                  wq, wq, wv, None, None, None)
    assert o.shape == v.shape and ht.shape == (3, 4, 64, 32) and hist.shape == (3, 3, 384)
    assert hist.dtype == torch.bfloat16
    st = torch.empty(3, 4, 64, 32, **m)
    o = torch.ops.kda.recurrent_kda_step(q, q, v, x, beta, None, st, hist, cu, True,
                                         wq, wq, wv, None, None, None)
    assert o.shape == v.shape


def test_gate_kind_entry_points_reject_bad_arguments():
    """kda_chunk_bwd_ex / kda_chunk_fwd_train_ex: a gate kind outside
    kda_gate_kind or an A_log with a kind other than KDA_GATE_RAW is
    KDA_ERR_SHAPE; an A_log overlapping an output is KDA_ERR_ALIAS."""
    lib = kda.load()
    d = _dims()

    def bwd(kind, A_log, dq=None):
        return lib.kda_chunk_bwd_ex(ctypes.byref(d), 1, FAKE[0], FAKE[1], FAKE[2], FAKE[3], kind, A_log,
                                    FAKE[4], None, None, 64, FAKE[5], None,
                                    dq if dq is not None else FAKE[6], FAKE[7], FAKE[8], FAKE[9],
                                    FAKE[10], FAKE[11], 0, FAKE[12], 1 << 40, None)

    def train(kind, A_log):
        return lib.kda_chunk_fwd_train_ex(ctypes.byref(d), 1, FAKE[0], FAKE[1], FAKE[2], FAKE[3], kind,
                                          A_log, FAKE[4], None, None, 64, 1, FAKE[5], FAKE[6],
                                          FAKE[7], 1 << 40, None)

    assert bwd(3, None) == 2 and bwd(-1, None) == 2
    assert bwd(kda.KDA_GATE_LOG2, FAKE[13]) == 2 and bwd(kda.KDA_GATE_NAT, FAKE[13]) == 2
    assert bwd(kda.KDA_GATE_RAW, FAKE[13], dq=FAKE[13]) == 5  # A_log inside dq
    assert train(3, None) == 2
    assert train(kda.KDA_GATE_NAT, FAKE[13]) == 2
