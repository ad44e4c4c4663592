// C ABI of libkda: argument validation, then kernel launches on the caller's stream.
#include <stdint.h>

#include <mutex>

#include "kda_common.h"

// Scratch of kda_recurrent_fwd_conv_noalloc: device memory the library owns, so
// that callers that cannot allocate (graph capture, serving loops) need not
// pass a workspace. Every GPU the library runs on holds its own copy until the
// process ends. In host code `scratch` names a host-side stand-in, never a
// device address: its address on a device comes from hipGetSymbolAddress,
// taken once per device with that device current (scratch_on_current_device).
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

bool valid_dtype(kda_dtype dt) { return dt == KDA_FP32 || dt == KDA_BF16; }
size_t esize(kda_dtype dt) { return dt == KDA_BF16 ? 2 : 4; }

// [a, a + na) and [b, b + nb) overlap (byte ranges; empty ranges never overlap)
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

kda_status check_dims(const kda_dims* d, const int32_t* cu) {
  if (!d) return KDA_ERR_NULL;
  if (d->B < 0 || d->T < 0 || d->N < 0 || d->H <= 0 || d->HV <= 0 || d->K <= 0 || d->V <= 0)
    return KDA_ERR_SHAPE;
  if (d->HV % d->H != 0) return KDA_ERR_SHAPE;
  if (cu) {
    if (d->B != 1) return KDA_ERR_SHAPE;
  } else {
    if (d->N != d->B) return KDA_ERR_SHAPE;
  }
  return KDA_OK;
}

struct Sizes {
  size_t qk, v, beta, gate, state;
};

Sizes sizes(const kda_dims* d, kda_dtype dt) {
  const size_t tok = (size_t)d->B * d->T;
  Sizes s;
  s.qk = tok * d->H * d->K * esize(dt);
  s.v = tok * d->HV * d->V * esize(dt);
  s.beta = tok * d->HV * esize(dt);
  s.gate = tok * d->HV * d->K * sizeof(float);
  s.state = (size_t)d->N * d->HV * d->K * d->V * sizeof(float);
  return s;
}

// Shared checks of the two scan entry points.
kda_status check_scan(const kda_dims* d, kda_dtype dt, const void* q, const void* k,
                      const void* v, const float* gate, const void* beta,
                      const float* h0, const int32_t* cu, int32_t write_final, const void* o,
                      const float* ht) {
  kda_status st = check_dims(d, cu);
  if (st != KDA_OK) return st;
  if (!valid_dtype(dt)) return KDA_ERR_DTYPE;
  const bool has_tokens = (size_t)d->B * d->T > 0;
  if (has_tokens && (!q || !k || !v || !gate || !beta || !o)) return KDA_ERR_NULL;
  if (write_final && !ht && d->N > 0) return KDA_ERR_NULL;
  const Sizes s = sizes(d, dt);
  // final_state may equal initial_state exactly; no other overlap
  if (h0 && ht && h0 != (const float*)ht && overlaps(h0, s.state, ht, s.state)) return KDA_ERR_ALIAS;
  const void* ins[] = {q, k, v, gate, beta, h0};
  const size_t ins_n[] = {s.qk, s.qk, s.v, s.gate, s.beta, s.state};
  for (int i = 0; i < 6; ++i) {
    if (overlaps(o, s.v, ins[i], ins_n[i])) return KDA_ERR_ALIAS;
    if (ht && ins[i] != h0 && overlaps(ht, s.state, ins[i], ins_n[i])) return KDA_ERR_ALIAS;
  }
  if (ht && overlaps(o, s.v, ht, s.state)) return KDA_ERR_ALIAS;
  return KDA_OK;
}

kda_status chunk_fwd_impl(const kda_dims* d, kda_dtype dt, const void* q, const void* k,
                          const void* v, const float* gate, int gate_mode, const float* A_log,
                          int qk_norm, const kda_short_conv* conv, const void* beta,
                          const float* h0, const int32_t* cu, int32_t chunk_size,
                          int32_t write_final, void* o, float* ht, void* workspace,
                          size_t workspace_bytes, hipStream_t stream, int save = 0) {
  kda_status st = check_scan(d, dt, q, k, v, gate, beta, h0, cu, write_final, o, ht);
  if (st != KDA_OK) return st;
  if (chunk_size != 64) return KDA_ERR_UNSUPPORTED;
  if (!((d->K == 64 || d->K == 128) && (d->V == 64 || d->V == 128))) return KDA_ERR_UNSUPPORTED;
  // a training forward fills the backward's workspace: only sizes the backward supports
  if (save && dt == KDA_FP32 && d->K != 64) return KDA_ERR_UNSUPPORTED;
  const Sizes s = sizes(d, dt);
  if (A_log && (overlaps(A_log, (size_t)d->HV * 4, o, s.v) ||
                overlaps(A_log, (size_t)d->HV * 4, ht, s.state)))
    return KDA_ERR_ALIAS;
  if (d->N == 0) return KDA_OK;
  // 16-byte vector loads of q, k, v and the gate, vector stores of o;
  // 256-byte aligned workspace
  if ((((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)gate | (uintptr_t)o) & 15) ||
      ((uintptr_t)workspace & 255))
    return KDA_ERR_UNSUPPORTED;
  const size_t need = save ? kda_host::chunk_bwd_workspace_bytes(*d, dt, chunk_size)
                           : kda_host::chunk_workspace_bytes(*d, dt, chunk_size);
  if (!workspace || workspace_bytes < need) return KDA_ERR_WORKSPACE;
  if (overlaps(workspace, need, o, s.v) || overlaps(workspace, need, ht, s.state) ||
      overlaps(workspace, need, h0, s.state) || overlaps(workspace, need, q, s.qk) ||
      overlaps(workspace, need, k, s.qk) || overlaps(workspace, need, v, s.v) ||
      overlaps(workspace, need, gate, s.gate) || overlaps(workspace, need, beta, s.beta) ||
      overlaps(workspace, need, A_log, A_log ? (size_t)d->HV * 4 : 0))
    return KDA_ERR_ALIAS;
  if (conv) {
    const size_t nqk = (size_t)d->H * d->K, nv = (size_t)d->HV * d->V, W = (size_t)conv->width;
    const void* bufs[] = {conv->q_weight, conv->k_weight, conv->v_weight,
                          conv->q_bias, conv->k_bias, conv->v_bias};
    const size_t lens[] = {nqk * W * 4, nqk * W * 4, nv * W * 4, nqk * 4, nqk * 4, nv * 4};
    for (int i = 0; i < 6; ++i)
      if (overlaps(bufs[i], lens[i], o, s.v) || overlaps(bufs[i], lens[i], ht, s.state) ||
          overlaps(bufs[i], lens[i], workspace, need))
        return KDA_ERR_ALIAS;
  }
  return kda_host::launch_chunk_fwd(*d, dt, q, k, v, gate, gate_mode, A_log, qk_norm ? 1 : 0,
                                    conv, beta, h0, cu,
                                    write_final ? 1 : 0, o, ht, workspace, workspace_bytes, save,
                                    stream) == hipSuccess
             ? KDA_OK
             : KDA_ERR_LAUNCH;
}

kda_status recurrent_impl(const kda_dims* d, kda_dtype dt, const void* q, const void* k,
                          const void* v, const float* gate, int gate_mode, const float* A_log,
                          int qk_norm, const void* beta, const float* h0, const int32_t* cu,
                          int32_t write_final, void* o, float* ht, hipStream_t stream) {
  kda_status st = check_scan(d, dt, q, k, v, gate, beta, h0, cu, write_final, o, ht);
  if (st != KDA_OK) return st;
  if (d->K > 256 || d->V > 256) return KDA_ERR_UNSUPPORTED;
  const Sizes s = sizes(d, dt);
  if (A_log && (overlaps(A_log, (size_t)d->HV * 4, o, s.v) ||
                overlaps(A_log, (size_t)d->HV * 4, ht, s.state)))
    return KDA_ERR_ALIAS;
  if (d->N == 0) return KDA_OK;
  return kda_host::launch_recurrent(*d, dt, q, k, v, gate, gate_mode, A_log, qk_norm ? 1 : 0,
                                    beta, h0, cu,
                                    write_final ? 1 : 0, o, ht, stream) == hipSuccess
             ? KDA_OK
             : KDA_ERR_LAUNCH;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Checks shared by the short-convolution entry points (no launch on failure).
kda_status check_conv(const kda_dims* d, kda_dtype dt, const void* q, const void* k,
                      const void* v, const kda_short_conv* conv, const int32_t* cu) {
  kda_status st = check_dims(d, cu);
  if (st != KDA_OK) return st;
  if (!valid_dtype(dt)) return KDA_ERR_DTYPE;
  if (!conv || !conv->q_weight || !conv->k_weight || !conv->v_weight) return KDA_ERR_NULL;
  if (conv->width < 1 || conv->width > kda::kConvMaxWidth) return KDA_ERR_UNSUPPORTED;
  const size_t epu = 16 / esize(dt);
  if (d->K % epu || d->V % epu) return KDA_ERR_UNSUPPORTED;  // 16-byte channel units
  if ((size_t)d->B * d->T > 0 && (!q || !k || !v)) return KDA_ERR_NULL;
  return KDA_OK;
}

size_t conv_state_bytes(const kda_dims* d, kda_dtype dt, int W) {
  return (size_t)d->N * (W - 1) * (2 * (size_t)d->H * d->K + (size_t)d->HV * d->V) * esize(dt);
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "required pointer is NULL";
    case KDA_ERR_SHAPE: return "inconsistent sizes";
    case KDA_ERR_DTYPE: return "unknown dtype";
    case KDA_ERR_UNSUPPORTED: return "unsupported size or chunk_size";
    case KDA_ERR_ALIAS: return "forbidden buffer overlap";
    case KDA_ERR_WORKSPACE: return "workspace missing or too small";
    case KDA_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

kda_status kda_gate_cumsum(const kda_dims* d, const float* gate_in, int32_t gate_in_is_raw,
                           const float* A_log, const int32_t* cu, int32_t chunk_size,
                           float* gate_out, hipStream_t stream) {
  kda_status st = check_dims(d, cu);
  if (st != KDA_OK) return st;
  if (chunk_size < 1 || chunk_size > 64) return KDA_ERR_UNSUPPORTED;
  if (!gate_in_is_raw && A_log) return KDA_ERR_SHAPE;
  const size_t n = (size_t)d->B * d->T * d->HV * d->K;
  if (n == 0) return KDA_OK;
  if (!gate_in || !gate_out) return KDA_ERR_NULL;
  // in place only for per-token output (a chunk may start inside another tile)
  if (overlaps(gate_in, n * 4, gate_out, n * 4) && !(chunk_size == 1 && gate_in == gate_out))
    return KDA_ERR_ALIAS;
  if (A_log && overlaps(A_log, (size_t)d->HV * 4, gate_out, n * 4)) return KDA_ERR_ALIAS;
  return kda_host::launch_gate(*d, gate_in, gate_in_is_raw ? 1 : 0, A_log, nullptr, cu,
                               chunk_size, gate_out, stream) == hipSuccess
             ? KDA_OK
             : KDA_ERR_LAUNCH;
}

kda_status kda_gate_cumsum_biased(const kda_dims* d, const float* x, const float* A_log,
                                  const float* dt_bias, const int32_t* cu, int32_t chunk_size,
                                  float* gate_out, hipStream_t stream) {
  kda_status st = check_dims(d, cu);
  if (st != KDA_OK) return st;
  if (chunk_size < 1 || chunk_size > 64) return KDA_ERR_UNSUPPORTED;
  const size_t n = (size_t)d->B * d->T * d->HV * d->K;
  if (n == 0) return KDA_OK;
  if (!x || !gate_out) return KDA_ERR_NULL;
  const size_t nb = (size_t)d->HV * d->K * 4;
  if (overlaps(x, n * 4, gate_out, n * 4) && !(chunk_size == 1 && x == gate_out)) return KDA_ERR_ALIAS;
  if (overlaps(A_log, (size_t)d->HV * 4, gate_out, n * 4) || overlaps(dt_bias, nb, gate_out, n * 4))
    return KDA_ERR_ALIAS;
  return kda_host::launch_gate(*d, x, 1, A_log, dt_bias, cu, chunk_size, gate_out, stream) ==
                 hipSuccess
             ? KDA_OK
             : KDA_ERR_LAUNCH;
}

size_t kda_gate_bwd_workspace_bytes(const kda_dims* d) {
  if (!d || d->B < 0 || d->T < 0 || d->HV <= 0 || d->K <= 0) return 0;
  return kda_host::gate_bwd_ws_bytes(*d);
}

kda_status kda_gate_bwd(const kda_dims* d, const float* x, const float* A_log,
                        const float* dt_bias, const float* dg, const int32_t* cu, float* dx,
                        float* dA_log, float* d_dt_bias, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  kda_status st = check_dims(d, cu);
  if (st != KDA_OK) return st;
  if (d->K > 4096) return KDA_ERR_UNSUPPORTED;
  // a parameter's gradient is produced exactly when the parameter is given
  if ((A_log == nullptr) != (dA_log == nullptr) || (dt_bias == nullptr) != (d_dt_bias == nullptr))
    return KDA_ERR_SHAPE;
  const size_t n = (size_t)d->B * d->T * d->HV * d->K * 4;
  const size_t na = (size_t)d->HV * 4, nb = (size_t)d->HV * d->K * 4;
  if (n > 0 && (!x || !dg || !dx)) return KDA_ERR_NULL;
  const bool reduce = dA_log || d_dt_bias;
  const size_t need = kda_host::gate_bwd_ws_bytes(*d);
  if (reduce && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;
  if (reduce && ((uintptr_t)workspace & 15)) return KDA_ERR_UNSUPPORTED;
  // dx may be dg itself (in place); no other overlap between outputs and anything else
  if (overlaps(dx, n, dg, n) && dx != dg) return KDA_ERR_ALIAS;
  const void* outs[] = {dx, dA_log, d_dt_bias, reduce ? workspace : nullptr};
  const size_t outs_n[] = {n, na, nb, reduce ? need : 0};
  const void* ins[] = {x, A_log, dt_bias, dg, cu};
  const size_t ins_n[] = {n, na, nb, n, cu ? (size_t)(d->N + 1) * 4 : 0};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 5; ++j)
      if (!(i == 0 && j == 3) && overlaps(outs[i], outs_n[i], ins[j], ins_n[j])) return KDA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], outs_n[i], outs[j], outs_n[j])) return KDA_ERR_ALIAS;
  }
  return kda_host::launch_gate_bwd(*d, x, A_log, dt_bias, dg, cu, dx, dA_log, d_dt_bias,
                                   workspace, stream) == hipSuccess
             ? KDA_OK
             : KDA_ERR_LAUNCH;
}

size_t kda_chunk_fwd_workspace_bytes(const kda_dims* d, kda_dtype dt, int32_t chunk_size) {
  if (!d || !valid_dtype(dt) || chunk_size != 64) return 0;
  if (!((d->K == 64 || d->K == 128) && (d->V == 64 || d->V == 128))) return 0;
  if (d->N < 0 || d->T < 0 || d->B < 0 || d->HV <= 0) return 0;
  return kda_host::chunk_workspace_bytes(*d, dt, chunk_size);
}

kda_status kda_chunk_fwd(const kda_dims* d, kda_dtype dt, const void* q, const void* k,
                         const void* v, const float* gate, const void* beta,
                         const float* h0, const int32_t* cu, int32_t chunk_size,
                         int32_t write_final, void* o, float* ht, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  return chunk_fwd_impl(d, dt, q, k, v, gate, kda::kGateLog2, nullptr, 0, nullptr, beta, h0, cu,
                        chunk_size, write_final, o, ht, workspace, workspace_bytes, stream);
}

kda_status kda_chunk_fwd_fused_gate(const kda_dims* d, kda_dtype dt, const void* q,
                                    const void* k, const void* v, const float* gate_in,
                                    int32_t gate_in_is_raw, const float* A_log, const void* beta,
                                    const float* h0, const int32_t* cu, int32_t chunk_size,
                                    int32_t write_final, void* o, float* ht, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  if (!gate_in_is_raw && A_log) return KDA_ERR_SHAPE;
  return chunk_fwd_impl(d, dt, q, k, v, gate_in, gate_in_is_raw ? kda::kGateRaw : kda::kGateLog,
                        A_log, 0, nullptr, beta, h0, cu, chunk_size, write_final, o, ht,
                        workspace, workspace_bytes, stream);
}

kda_status kda_chunk_fwd_ex(const kda_dims* d, kda_dtype dt, const void* q, const void* k,
                            const void* v, const float* gate, int32_t gate_kind,
                            const float* A_log, int32_t qk_l2norm, const void* beta,
                            const float* h0, const int32_t* cu, int32_t chunk_size,
                            int32_t write_final, void* o, float* ht, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if (gate_kind < KDA_GATE_LOG2 || gate_kind > KDA_GATE_RAW) return KDA_ERR_SHAPE;
  if (gate_kind != KDA_GATE_RAW && A_log) return KDA_ERR_SHAPE;
  return chunk_fwd_impl(d, dt, q, k, v, gate, (int)gate_kind, A_log, qk_l2norm != 0, nullptr, beta,
                        h0, cu, chunk_size, write_final, o, ht, workspace, workspace_bytes, stream);
}

kda_status kda_chunk_fwd_conv(const kda_dims* d, kda_dtype dt, const void* q, const void* k,
                              const void* v, const kda_short_conv* conv, const float* gate,
                              int32_t gate_kind, const float* A_log, int32_t qk_l2norm,
                              const void* beta, const float* h0, const int32_t* cu,
                              int32_t chunk_size, int32_t write_final, void* o, float* ht,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (gate_kind < KDA_GATE_LOG2 || gate_kind > KDA_GATE_RAW) return KDA_ERR_SHAPE;
  if (gate_kind != KDA_GATE_RAW && A_log) return KDA_ERR_SHAPE;
  if (!conv || !conv->q_weight || !conv->k_weight || !conv->v_weight) return KDA_ERR_NULL;
  if (conv->width < 1 || conv->width > kda::kConvMaxWidth) return KDA_ERR_UNSUPPORTED;
  return chunk_fwd_impl(d, dt, q, k, v, gate, (int)gate_kind, A_log, qk_l2norm != 0, conv, beta,
                        h0, cu, chunk_size, write_final, o, ht, workspace, workspace_bytes, stream);
}

size_t kda_chunk_bwd_workspace_bytes(const kda_dims* d, kda_dtype dt, int32_t chunk_size) {
  if (!d || !valid_dtype(dt) || chunk_size != 64) return 0;
  if (!((d->K == 64 || d->K == 128) && (d->V == 64 || d->V == 128))) return 0;
  if (dt == KDA_FP32 && d->K != 64) return 0;
  if (d->N < 0 || d->T < 0 || d->B < 0 || d->HV <= 0 || d->H <= 0) return 0;
  return kda_host::chunk_bwd_workspace_bytes(*d, dt, chunk_size);
}

}  // extern "C"

namespace {

kda_status chunk_bwd_impl(const kda_dims* d, kda_dtype dt, const void* q, const void* k,
                          const void* v, const float* gate, int gate_kind, const float* A_log,
                          const void* beta, const float* h0,
                          const int32_t* cu, int32_t chunk_size, const void* do_,
                          const float* dht, void* dq, void* dk, void* dv, float* dg, void* dbeta,
                          float* dh0, void* workspace, size_t workspace_bytes, int saved,
                          hipStream_t stream) {
  kda_status st = check_dims(d, cu);
  if (st != KDA_OK) return st;
  if (!valid_dtype(dt)) return KDA_ERR_DTYPE;
  if (gate_kind < KDA_GATE_LOG2 || gate_kind > KDA_GATE_RAW) return KDA_ERR_SHAPE;
  if (gate_kind != KDA_GATE_RAW && A_log) return KDA_ERR_SHAPE;
  const bool has_tokens = (size_t)d->B * d->T > 0;
  if (has_tokens && (!q || !k || !v || !gate || !beta || !do_ || !dq || !dk || !dv || !dg || !dbeta))
    return KDA_ERR_NULL;
  if (d->N > 0 && !dh0) return KDA_ERR_NULL;
  if (chunk_size != 64) return KDA_ERR_UNSUPPORTED;
  if (!((d->K == 64 || d->K == 128) && (d->V == 64 || d->V == 128))) return KDA_ERR_UNSUPPORTED;
  if (dt == KDA_FP32 && d->K != 64) return KDA_ERR_UNSUPPORTED;  // FP32 staging exceeds LDS
  const Sizes s = sizes(d, dt);
  const void* ins[] = {q, k, v, gate, beta, h0, do_, dht, A_log};
  const size_t ins_n[] = {s.qk, s.qk, s.v, s.gate, s.beta, s.state, s.v, s.state,
                          A_log ? (size_t)d->HV * sizeof(float) : 0};
  constexpr int NIN = 9;
  const void* outs[] = {dq, dk, dv, dg, dbeta, dh0};
  const size_t outs_n[] = {s.qk, s.qk, s.v, s.gate, s.beta, s.state};
  for (int i = 0; i < 6; ++i) {
    for (int j = 0; j < NIN; ++j)
      if (overlaps(outs[i], outs_n[i], ins[j], ins_n[j])) return KDA_ERR_ALIAS;
    for (int j = i + 1; j < 6; ++j)
      if (overlaps(outs[i], outs_n[i], outs[j], outs_n[j])) return KDA_ERR_ALIAS;
  }
  if (d->N == 0) return KDA_OK;
  if ((((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)gate | (uintptr_t)do_) & 15) ||
      ((uintptr_t)workspace & 255))
    return KDA_ERR_UNSUPPORTED;
  const size_t need = kda_host::chunk_bwd_workspace_bytes(*d, dt, chunk_size);
  if (!workspace || workspace_bytes < need) return KDA_ERR_WORKSPACE;
  for (int i = 0; i < 6; ++i)
    if (overlaps(workspace, need, outs[i], outs_n[i])) return KDA_ERR_ALIAS;
  for (int j = 0; j < NIN; ++j)
    if (overlaps(workspace, need, ins[j], ins_n[j])) return KDA_ERR_ALIAS;
  return kda_host::launch_chunk_bwd(*d, dt, q, k, v, gate, gate_kind, A_log, beta, h0, cu, do_,
                                    dht, dq, dk, dv, dg, dbeta, dh0, workspace, saved,
                                    stream) == hipSuccess
             ? KDA_OK
             : KDA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

kda_status kda_chunk_bwd(const kda_dims* d, kda_dtype dt, const void* q, const void* k,
                         const void* v, const float* gate, const void* beta, const float* h0,
                         const int32_t* cu, int32_t chunk_size, const void* do_,
                         const float* dht, void* dq, void* dk, void* dv, float* dg, void* dbeta,
                         float* dh0, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return chunk_bwd_impl(d, dt, q, k, v, gate, KDA_GATE_LOG2, nullptr, beta, h0, cu, chunk_size, do_,
                        dht, dq, dk, dv, dg, dbeta, dh0, workspace, workspace_bytes, 0, stream);
}

kda_status kda_chunk_fwd_train(const kda_dims* d, kda_dtype dt, const void* q, const void* k,
                               const void* v, const float* gate, const void* beta,
                               const float* h0, const int32_t* cu, int32_t chunk_size,
                               int32_t write_final, void* o, float* ht, void* bwd_workspace,
                               size_t bwd_workspace_bytes, hipStream_t stream) {
  return chunk_fwd_impl(d, dt, q, k, v, gate, kda::kGateLog2, nullptr, 0, nullptr, beta, h0, cu,
                        chunk_size, write_final, o, ht, bwd_workspace, bwd_workspace_bytes, stream,
                        1);
}

kda_status kda_chunk_bwd_saved(const kda_dims* d, kda_dtype dt, const void* q, const void* k,
                               const void* v, const float* gate, const void* beta,
                               const float* h0, const int32_t* cu, int32_t chunk_size,
                               const void* do_, const float* dht, void* dq, void* dk, void* dv,
                               float* dg, void* dbeta, float* dh0, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  return chunk_bwd_impl(d, dt, q, k, v, gate, KDA_GATE_LOG2, nullptr, beta, h0, cu, chunk_size, do_,
                        dht, dq, dk, dv, dg, dbeta, dh0, workspace, workspace_bytes, 1, stream);
}

kda_status kda_chunk_fwd_train_ex(const kda_dims* d, kda_dtype dt, const void* q, const void* k,
                                  const void* v, const float* gate, int32_t gate_kind,
                                  const float* A_log, const void* beta, const float* h0,
                                  const int32_t* cu, int32_t chunk_size, int32_t write_final,
                                  void* o, float* ht, void* bwd_workspace,
                                  size_t bwd_workspace_bytes, hipStream_t stream) {
  if (gate_kind < KDA_GATE_LOG2 || gate_kind > KDA_GATE_RAW) return KDA_ERR_SHAPE;
  if (gate_kind != KDA_GATE_RAW && A_log) return KDA_ERR_SHAPE;
  return chunk_fwd_impl(d, dt, q, k, v, gate, (int)gate_kind, A_log, 0, nullptr, beta, h0, cu,
                        chunk_size, write_final, o, ht, bwd_workspace, bwd_workspace_bytes, stream,
                        1);
}

kda_status kda_chunk_bwd_ex(const kda_dims* d, kda_dtype dt, const void* q, const void* k,
                            const void* v, const float* gate, int32_t gate_kind, const float* A_log,
                            const void* beta, const float* h0, const int32_t* cu,
                            int32_t chunk_size, const void* do_, const float* dht, void* dq,
                            void* dk, void* dv, float* dg, void* dbeta, float* dh0,
                            int32_t saved, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  return chunk_bwd_impl(d, dt, q, k, v, gate, (int)gate_kind, A_log, beta, h0, cu, chunk_size, do_,
                        dht, dq, dk, dv, dg, dbeta, dh0, workspace, workspace_bytes, saved ? 1 : 0,
                        stream);
}

kda_status kda_recurrent_fwd(const kda_dims* d, kda_dtype dt, const void* q, const void* k,
                             const void* v, const float* gate, const void* beta,
                             const float* h0, const int32_t* cu, int32_t write_final, void* o,
                             float* ht, hipStream_t stream) {
  return recurrent_impl(d, dt, q, k, v, gate, kda::kGateLog2, nullptr, 0, beta, h0, cu,
                        write_final, o, ht, stream);
}

kda_status kda_recurrent_fwd_fused_gate(const kda_dims* d, kda_dtype dt, const void* q,
                                        const void* k, const void* v, const float* gate_in,
                                        int32_t gate_in_is_raw, const float* A_log,
                                        const void* beta, const float* h0, const int32_t* cu,
                                        int32_t write_final, void* o, float* ht,
                                        hipStream_t stream) {
  if (!gate_in_is_raw && A_log) return KDA_ERR_SHAPE;
  return recurrent_impl(d, dt, q, k, v, gate_in, gate_in_is_raw ? kda::kGateRaw : kda::kGateLog,
                        A_log, 0, beta, h0, cu, write_final, o, ht, stream);
}

kda_status kda_short_conv_fwd(const kda_dims* d, kda_dtype dt, const void* q, const void* k,
                              const void* v, const kda_short_conv* conv, const int32_t* cu,
                              const void* st_in, void* st_out, void* q_out, void* k_out,
                              void* v_out, hipStream_t stream) {
  kda_status st = check_conv(d, dt, q, k, v, conv, cu);
  if (st != KDA_OK) return st;
  const bool out = q_out || k_out || v_out;
  if (out && (!q_out || !k_out || !v_out)) return KDA_ERR_NULL;
  const Sizes s = sizes(d, dt);
  const size_t sb = conv_state_bytes(d, dt, conv->width);
  // outputs equal their own input or overlap nothing; the history may be updated in place
  const void* ins[] = {q, k, v, st_in};
  const size_t ins_n[] = {s.qk, s.qk, s.v, st_in ? sb : 0};
  void* outs[] = {q_out, k_out, v_out, st_out};
  const size_t outs_n[] = {s.qk, s.qk, s.v, st_out ? sb : 0};
  for (int i = 0; i < 4; ++i) {
    if (!outs[i]) continue;
    for (int j = 0; j < 4; ++j) {
      const bool own_input = i == j && outs[i] == ins[j];  // in place
      if (!own_input && overlaps(outs[i], outs_n[i], ins[j], ins_n[j])) return KDA_ERR_ALIAS;
    }
    for (int j = i + 1; j < 4; ++j)
      if (outs[j] && overlaps(outs[i], outs_n[i], outs[j], outs_n[j])) return KDA_ERR_ALIAS;
  }
  const size_t nqk = (size_t)d->H * d->K, nv = (size_t)d->HV * d->V, W = (size_t)conv->width;
  const void* taps[] = {conv->q_weight, conv->k_weight, conv->v_weight,
                        conv->q_bias, conv->k_bias, conv->v_bias};
  const size_t taps_n[] = {nqk * W * 4, nqk * W * 4, nv * W * 4, nqk * 4, nqk * 4, nv * 4};
  for (int i = 0; i < 6; ++i)
    for (int j = 0; j < 4; ++j)
      if (outs[j] && overlaps(taps[i], taps_n[i], outs[j], outs_n[j])) return KDA_ERR_ALIAS;
  if ((((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)st_in | (uintptr_t)st_out |
        (uintptr_t)q_out | (uintptr_t)k_out | (uintptr_t)v_out) & 15))
    return KDA_ERR_UNSUPPORTED;
  if (d->N == 0) return KDA_OK;
  return kda_host::launch_short_conv(*d, dt, q, k, v, *conv, cu, st_in, st_out, q_out, k_out, v_out,
                                     stream) == hipSuccess
             ? KDA_OK
             : KDA_ERR_LAUNCH;
}

size_t kda_recurrent_fwd_conv_workspace_bytes(const kda_dims* d, kda_dtype dt) {
  if (!d || !valid_dtype(dt) || d->B < 0 || d->T < 0 || d->H <= 0 || d->HV <= 0 || d->K <= 0 ||
      d->V <= 0)
    return 0;
  const Sizes s = sizes(d, dt);
  return 2 * align256(s.qk) + align256(s.v);
}

kda_status kda_recurrent_fwd_conv(const kda_dims* d, kda_dtype dt, const void* q, const void* k,
                                  const void* v, const kda_short_conv* conv, const void* st_in,
                                  void* st_out, const float* gate, int32_t gate_kind,
                                  const float* A_log, int32_t qk_l2norm, const void* beta,
                                  const float* h0, const int32_t* cu, int32_t write_final, void* o,
                                  float* ht, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  if (gate_kind < KDA_GATE_LOG2 || gate_kind > KDA_GATE_RAW) return KDA_ERR_SHAPE;
  if (gate_kind != KDA_GATE_RAW && A_log) return KDA_ERR_SHAPE;
  kda_status st = check_conv(d, dt, q, k, v, conv, cu);
  if (st != KDA_OK) return st;
  st = check_scan(d, dt, q, k, v, gate, beta, h0, cu, write_final, o, ht);
  if (st != KDA_OK) return st;
  if (d->K > 256 || d->V > 256) return KDA_ERR_UNSUPPORTED;
  const Sizes s = sizes(d, dt);
  const size_t need = kda_recurrent_fwd_conv_workspace_bytes(d, dt);
  if (!workspace || workspace_bytes < need) return KDA_ERR_WORKSPACE;
  if ((uintptr_t)workspace & 255) return KDA_ERR_UNSUPPORTED;
  const size_t sb = conv_state_bytes(d, dt, conv->width);
  const void* others[] = {q, k, v, gate, beta, h0, o, ht, st_in, st_out, A_log};
  const size_t others_n[] = {s.qk, s.qk, s.v, s.gate, s.beta, s.state, s.v, s.state,
                             st_in ? sb : 0, st_out ? sb : 0, A_log ? (size_t)d->HV * 4 : 0};
  for (int i = 0; i < 11; ++i)
    if (overlaps(workspace, need, others[i], others_n[i])) return KDA_ERR_ALIAS;
  // the convolution writes the new history before the scan reads its inputs:
  // the history may overlap nothing the scan reads or writes
  if (st_out) {
    const size_t nqk = (size_t)d->H * d->K, nv = (size_t)d->HV * d->V, W = (size_t)conv->width;
    const void* scan_bufs[] = {o, ht, q, k, v, h0, gate, beta, A_log,
                               conv->q_weight, conv->k_weight, conv->v_weight,
                               conv->q_bias, conv->k_bias, conv->v_bias};
    const size_t scan_n[] = {s.v, s.state, s.qk, s.qk, s.v, s.state, s.gate, s.beta,
                             A_log ? (size_t)d->HV * 4 : 0, nqk * W * 4, nqk * W * 4, nv * W * 4,
                             nqk * 4, nqk * 4, nv * 4};
    for (int i = 0; i < 15; ++i)
      if (overlaps(st_out, sb, scan_bufs[i], scan_n[i])) return KDA_ERR_ALIAS;
  }
  if (A_log && (overlaps(A_log, (size_t)d->HV * 4, o, s.v) ||
                overlaps(A_log, (size_t)d->HV * 4, ht, s.state)))
    return KDA_ERR_ALIAS;
  if (d->N == 0) return KDA_OK;
  char* p = reinterpret_cast<char*>(workspace);
  void* qc = p;
  void* kc = p + align256(s.qk);
  void* vc = p + 2 * align256(s.qk);
  st = kda_short_conv_fwd(d, dt, q, k, v, conv, cu, st_in, st_out, qc, kc, vc, stream);
  if (st != KDA_OK) return st;
  return recurrent_impl(d, dt, qc, kc, vc, gate, (int)gate_kind, A_log, qk_l2norm != 0, beta, h0,
                        cu, write_final, o, ht, stream);
}

}  // extern "C"

namespace {

// Device address of `scratch` on the calling thread's current device, looked
// up on the first call for that device and kept.
kda_status scratch_on_current_device(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return KDA_ERR_LAUNCH;
  if (dev >= kMaxDevices) return KDA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KDA_ERR_LAUNCH;
    addr[dev] = p;
  }
  *out = addr[dev];
  return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_recurrent_fwd_conv_noalloc(const kda_dims* d, kda_dtype dt, const void* q,
                                          const void* k, const void* v, const kda_short_conv* conv,
                                          const void* conv_state_in, void* conv_state_out,
                                          const float* gate, int32_t gate_kind, const float* A_log,
                                          int32_t qk_l2norm, const void* beta, const float* h0,
                                          const int32_t* cu, int32_t write_final, void* o,
                                          float* ht, hipStream_t stream) {
  if (!d) return KDA_ERR_NULL;
  const size_t need = kda_recurrent_fwd_conv_workspace_bytes(d, dt);
  if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_WORKSPACE;
  void* ws = nullptr;
  const kda_status st = scratch_on_current_device(&ws);
  if (st != KDA_OK) return st;
  // every byte of the scratch the call uses is written before it is read
  // (the convolved q, k, v), so nothing needs clearing between calls
  return kda_recurrent_fwd_conv(d, dt, q, k, v, conv, conv_state_in, conv_state_out, gate,
                                gate_kind, A_log, qk_l2norm, beta, h0, cu, write_final, o, ht, ws,
                                (size_t)KDA_NOALLOC_SCRATCH_BYTES, stream);
}

kda_status kda_recurrent_fwd_ex(const kda_dims* d, kda_dtype dt, const void* q, const void* k,
                                const void* v, const float* gate, int32_t gate_kind,
                                const float* A_log, int32_t qk_l2norm, const void* beta,
                                const float* h0, const int32_t* cu, int32_t write_final, void* o,
                                float* ht, hipStream_t stream) {
  if (gate_kind < KDA_GATE_LOG2 || gate_kind > KDA_GATE_RAW) return KDA_ERR_SHAPE;
  if (gate_kind != KDA_GATE_RAW && A_log) return KDA_ERR_SHAPE;
  return recurrent_impl(d, dt, q, k, v, gate, (int)gate_kind, A_log, qk_l2norm != 0, beta, h0, cu,
                        write_final, o, ht, stream);
}

}  // extern "C"
