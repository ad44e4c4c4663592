"""torch.library registration of the KDA entry points (argument marshalling
only; every step runs in libkda's kernels).

  torch.ops.kda.chunk_kda_train(q, k, v, x, beta, A_log, dt_bias,
                                initial_state, cu_seqlens) -> (o, final_state)
      The chunked forward from the raw gate input x, differentiable in q, k,
      v, x, beta, A_log, dt_bias and initial_state. Without dt_bias the gate
      step runs inside the kernels (kda_chunk_fwd_fused_gate forward,
      kda_chunk_bwd_ex backward); with it, kda_gate_cumsum_biased forms the
      chunk-local log2 gate for kda_chunk_fwd and kda_chunk_bwd. Then
      kda_gate_bwd on the backward's dg.
  torch.ops.kda.recurrent_kda(q, k, v, x, beta, A_log, initial_state,
                              cu_seqlens) -> (o, final_state)
      Token-sequential forward with the gate activated in the scan kernel
      (kda_recurrent_fwd_fused_gate); inference only (no autograd formula).

  torch.ops.kda.chunk_kda_prefill(q, k, v, x, beta, A_log, initial_state,
                                  cu_seqlens, qk_l2norm, conv taps and biases)
                                  -> (o, final_state, conv_state)
      Inference prefill from raw projections (short convolution + SiLU and
      q/k L2 norm fused into the chunked forward) with the convolution history
      for the decode that follows.
  torch.ops.kda.recurrent_kda_step(q, k, v, x, beta, A_log, state, conv_state,
                                   cu_seqlens, qk_l2norm, conv taps and biases) -> o
      One decode step from raw projections; mutates state and conv_state.

All have fake (meta) implementations, so they trace under torch.compile and
FakeTensor. Shapes: q, k [B, T, H, K]; v [B, T, HV, V]; x [B, T, HV, K] FP32;
beta [B, T, HV]; A_log [HV] FP32; dt_bias [HV, K] FP32; initial_state
[N, HV, K, V] FP32; cu_seqlens [N + 1] int32 (varlen, B == 1).
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch
from torch import Tensor

from . import (chunk_kda, chunk_kda_bwd, conv_state_shape, gate_bwd, gate_cumsum, recurrent_kda,
               short_conv)

_CHUNK = 64


def _n_states(q: Tensor, cu_seqlens: Optional[Tensor]) -> int:
    return q.shape[0] if cu_seqlens is None else cu_seqlens.shape[0] - 1


@torch.library.custom_op("kda::chunk_kda_train", mutates_args=(), device_types="cuda")
def chunk_kda_train(q: Tensor, k: Tensor, v: Tensor, x: Tensor, beta: Tensor,
                    A_log: Optional[Tensor], dt_bias: Optional[Tensor],
                    initial_state: Optional[Tensor],
                    cu_seqlens: Optional[Tensor]) -> Tuple[Tensor, Tensor]:
    if dt_bias is None:  # gate step inside the chunk kernel (bit-identical to the two calls)
        return chunk_kda(q, k, v, x, beta, initial_state, cu_seqlens=cu_seqlens,
                         output_final_state=True, chunk_size=_CHUNK, use_gate_in_kernel=True,
                         A_log=A_log)
    G = gate_cumsum(x, A_log, cu_seqlens, _CHUNK, dt_bias=dt_bias)
    o, ht = chunk_kda(q, k, v, G, beta, initial_state, cu_seqlens=cu_seqlens,
                      output_final_state=True, chunk_size=_CHUNK)
    return o, ht


@chunk_kda_train.register_fake
def _chunk_kda_train_fake(q, k, v, x, beta, A_log, dt_bias, initial_state, cu_seqlens):
    N = _n_states(q, cu_seqlens)
    return torch.empty_like(v), q.new_empty((N, v.shape[2], q.shape[3], v.shape[3]),
                                            dtype=torch.float32)


def _chunk_setup(ctx, inputs, output):
    ctx.save_for_backward(*inputs)


def _chunk_backward(ctx, do, dht):
    q, k, v, x, beta, A_log, dt_bias, h0, cu = ctx.saved_tensors
    if dt_bias is None:  # gate step inside the backward's kernels (kda_chunk_bwd_ex)
        r = chunk_kda_bwd(q, k, v, x, beta, h0, do.contiguous(), dht.contiguous(), cu_seqlens=cu,
                          chunk_size=_CHUNK, use_gate_in_kernel=True, A_log=A_log)
    else:
        G = gate_cumsum(x, A_log, cu, _CHUNK, dt_bias=dt_bias)
        r = chunk_kda_bwd(q, k, v, G, beta, h0, do.contiguous(), dht.contiguous(), cu_seqlens=cu,
                          chunk_size=_CHUNK)
    dx, dA, db = gate_bwd(x, r["dg"], A_log, dt_bias, cu, dx=r["dg"])
    return (r["dq"], r["dk"], r["dv"], dx, r["dbeta"], dA, db,
            r["dh0"] if h0 is not None else None, None)


chunk_kda_train.register_autograd(_chunk_backward, setup_context=_chunk_setup)


@torch.library.custom_op("kda::recurrent_kda", mutates_args=(), device_types="cuda")
def recurrent_kda_op(q: Tensor, k: Tensor, v: Tensor, x: Tensor, beta: Tensor,
                     A_log: Optional[Tensor], initial_state: Optional[Tensor],
                     cu_seqlens: Optional[Tensor]) -> Tuple[Tensor, Tensor]:
    return recurrent_kda(q, k, v, x, beta, initial_state, cu_seqlens=cu_seqlens,
                         output_final_state=True, use_gate_in_kernel=True, A_log=A_log)


@recurrent_kda_op.register_fake
def _recurrent_kda_fake(q, k, v, x, beta, A_log, initial_state, cu_seqlens):
    N = _n_states(q, cu_seqlens)
    return torch.empty_like(v), q.new_empty((N, v.shape[2], q.shape[3], v.shape[3]),
                                            dtype=torch.float32)


def _taps(wq, wk, wv, bq, bk, bv):
    return None if wq is None else ((wq, bq), (wk, bk), (wv, bv))


@torch.library.custom_op("kda::chunk_kda_prefill", mutates_args=(), device_types="cuda")
def chunk_kda_prefill(q: Tensor, k: Tensor, v: Tensor, x: Tensor, beta: Tensor,
                      A_log: Optional[Tensor], initial_state: Optional[Tensor],
                      cu_seqlens: Optional[Tensor], qk_l2norm: bool,
                      conv_q_weight: Optional[Tensor], conv_k_weight: Optional[Tensor],
                      conv_v_weight: Optional[Tensor], conv_q_bias: Optional[Tensor],
                      conv_k_bias: Optional[Tensor],
                      conv_v_bias: Optional[Tensor]) -> Tuple[Tensor, Tensor, Tensor]:
    """Inference prefill from raw projections: the short convolution + SiLU of
    q, k, v (when the taps are given) and the q/k L2 norm fused into the
    chunked forward (kda_chunk_fwd_conv / kda_chunk_fwd_ex), gate activated in
    the kernel. Returns (o, final_state, conv_state): the convolution history
    [N, W - 1, 2HK + HV V] that decode continues from ([N, 0, ...] without taps)."""
    taps = _taps(conv_q_weight, conv_k_weight, conv_v_weight, conv_q_bias, conv_k_bias, conv_v_bias)
    o, ht = chunk_kda(q, k, v, x, beta, initial_state, cu_seqlens=cu_seqlens,
                      output_final_state=True, chunk_size=_CHUNK, use_gate_in_kernel=True,
                      A_log=A_log, qk_l2norm=qk_l2norm, short_conv=taps)
    W = 1 if taps is None else conv_q_weight.shape[-1]
    hist = q.new_zeros(conv_state_shape(q, v, cu_seqlens, W))
    if taps is not None and W > 1:
        short_conv(q, k, v, taps, cu_seqlens=cu_seqlens, conv_state_out=hist, outputs=False)
    return o, ht, hist


@chunk_kda_prefill.register_fake
def _chunk_kda_prefill_fake(q, k, v, x, beta, A_log, initial_state, cu_seqlens, qk_l2norm,
                            conv_q_weight, conv_k_weight, conv_v_weight, conv_q_bias, conv_k_bias,
                            conv_v_bias):
    N = _n_states(q, cu_seqlens)
    W = 1 if conv_q_weight is None else conv_q_weight.shape[-1]
    D = 2 * q.shape[2] * q.shape[3] + v.shape[2] * v.shape[3]
    return (torch.empty_like(v),
            q.new_empty((N, v.shape[2], q.shape[3], v.shape[3]), dtype=torch.float32),
            q.new_empty((N, W - 1, D)))


@torch.library.custom_op("kda::recurrent_kda_step", mutates_args=("state", "conv_state"),
                         device_types="cuda")
def recurrent_kda_step(q: Tensor, k: Tensor, v: Tensor, x: Tensor, beta: Tensor,
                       A_log: Optional[Tensor], state: Tensor, conv_state: Optional[Tensor],
                       cu_seqlens: Optional[Tensor], qk_l2norm: bool,
                       conv_q_weight: Optional[Tensor], conv_k_weight: Optional[Tensor],
                       conv_v_weight: Optional[Tensor], conv_q_bias: Optional[Tensor],
                       conv_k_bias: Optional[Tensor], conv_v_bias: Optional[Tensor]) -> Tensor:
    """Decode step from raw projections with the recurrent state [N, HV, K, V]
    and the convolution history updated in place (kda_recurrent_fwd_conv, or
    kda_recurrent_fwd_ex without taps). Returns o."""
    taps = _taps(conv_q_weight, conv_k_weight, conv_v_weight, conv_q_bias, conv_k_bias, conv_v_bias)
    o, _ = recurrent_kda(q, k, v, x, beta, state, cu_seqlens=cu_seqlens, output_final_state=True,
                         final_state=state, use_gate_in_kernel=True, A_log=A_log,
                         qk_l2norm=qk_l2norm, short_conv=taps, conv_state=conv_state,
                         conv_state_out=conv_state)
    return o


@recurrent_kda_step.register_fake
def _recurrent_kda_step_fake(q, k, v, x, beta, A_log, state, conv_state, cu_seqlens, qk_l2norm,
                             conv_q_weight, conv_k_weight, conv_v_weight, conv_q_bias, conv_k_bias,
                             conv_v_bias):
    return torch.empty_like(v)
