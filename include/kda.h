/*
 * kda.h -- C ABI of libkda, the MI355X (gfx950) Kimi Delta Attention scan.
 *
 * The operation (per value head hv of a sequence, with qk head h = hv / (HV/H)):
 *   S_t = (I - beta_t k_t k_t^T) Diag(2^{gate_t}) S_{t-1} + beta_t k_t v_t^T
 *   o_t = S_t^T (q_t / sqrt(K))
 * with S_t a K x V FP32 state. This is the gated delta rule with a
 * per-channel decay (KDA). Sources on the pages:
 *   - "kda in torchtitan (training)", pytorch/torchtitan PR #4164, the quoted
 *     attention-gym description of `recurrent_kda`: the argument contract
 *     (q, k, v, gate, beta, initial_state, cu_seqlens, output_final_state),
 *     device-resident int32 cu_seqlens, repeated offsets as empty slots whose
 *     state passes through bitwise, a capacity tail outside the contract, FP32
 *     states with one leading entry per logical sequence, the gate as a
 *     per-token log2 decay (chunk-local cumulative for the chunked op), the
 *     internal 1/sqrt(K) query scale, FP32 compute for any input dtype.
 *   - "[Fix] Use unit KDA gate scale when A_log is omitted", fla-org
 *     flash-linear-attention PR #1294, Summary and Breaking changes: decay
 *     scale exp(A_log), omitted A_log = unit scale = explicit zero A_log.
 *   - same page, squashed commit bodies: the chunked pipeline steps (kkt,
 *     solve_tril, recompute_w_u, fwd_h, fwd_o) of the sibling gated delta
 *     rule op, which kda_chunk_fwd follows for a per-channel gate.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers to contiguous row-major arrays.
 *     Dense layout: q, k [B, T, H, K]; v, o [B, T, HV, V]; gate [B, T, HV, K]
 *     FP32; beta [B, T, HV] (same dtype as q); states [N, HV, K, V] FP32.
 *   - Dense mode: cu_seqlens == NULL and N == B; batch row b is one sequence.
 *     Varlen mode: cu_seqlens is a device int32 array of N+1 non-decreasing
 *     offsets with cu_seqlens[0] == 0 and cu_seqlens[N] <= T; B must be 1.
 *     Sequence n covers tokens [cu_seqlens[n], cu_seqlens[n+1]); an empty
 *     range is an empty slot. Tokens in [cu_seqlens[N], T) (the capacity
 *     tail) are neither read nor written. The offsets are NOT validated
 *     (reading them would force a host sync); violating the preconditions is
 *     undefined behaviour.
 *   - Empty slot: no output row; if output_final_state, final_state[n] is a
 *     bitwise copy of initial_state[n] (or +0.0 when initial_state is NULL).
 *   - final_state may equal initial_state (in-place update); any other
 *     overlap between them, or between o and an input, is KDA_ERR_ALIAS.
 *   - The caller owns every buffer. The library allocates nothing, keeps no
 *     global state and never synchronises: each call only enqueues work on
 *     `stream`, and results are valid once that stream has been synchronised.
 *     The one exception is kda_recurrent_fwd_conv_noalloc, which uses a static
 *     device scratch of the library's own instead of a caller's workspace.
 *   - Host-checkable errors return before anything is enqueued. A failed
 *     kernel launch returns KDA_ERR_LAUNCH.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL = 1,        /* a required pointer is NULL */
  KDA_ERR_SHAPE = 2,       /* inconsistent sizes (HV % H != 0, N != B dense, B != 1 varlen, ...) */
  KDA_ERR_DTYPE = 3,       /* unknown dtype code */
  KDA_ERR_UNSUPPORTED = 4, /* valid but not implemented (K, V, chunk_size) */
  KDA_ERR_ALIAS = 5,       /* forbidden overlap between buffers */
  KDA_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required */
  KDA_ERR_LAUNCH = 7       /* the HIP runtime refused a launch */
} kda_status;

/* Element type of q, k, v, beta and o. States and gates are always FP32. */
typedef enum { KDA_FP32 = 0, KDA_BF16 = 1 } kda_dtype;

/* What the gate operand of kda_chunk_fwd_ex / kda_recurrent_fwd_ex holds:
 *   KDA_GATE_LOG2  the prepared log2 gate (kda_gate_cumsum output: chunk-local
 *                  cumsum for the chunked op, chunk_size 1 for the recurrent one);
 *   KDA_GATE_NAT   the per-token natural-log gate g (cumsum formed in the kernel);
 *   KDA_GATE_RAW   the raw activation input x, g = -exp(A_log) * softplus(x). */
typedef enum { KDA_GATE_LOG2 = 0, KDA_GATE_NAT = 1, KDA_GATE_RAW = 2 } kda_gate_kind;

/* Short causal convolution + SiLU applied to q, k and v before the scan (the
 * ShortConvolution / causal_conv1d_silu pre-processing step the pages import
 * next to the KDA op, "kda in torchtitan (training)" and the Paddle
 * compatibility page; no formula is printed there). Per channel c of a
 * sequence, with x taken as zero before the sequence's first token:
 *   z[t, c] = bias[c] + sum_{j < width} weight[c, j] * x[t - width + 1 + j, c]
 *   y[t, c] = z * sigmoid(z)                          (SiLU)
 * i.e. a depthwise Conv1d cross-correlation with width - 1 zeros of history
 * per sequence; weight[c, width - 1] multiplies the current token.
 * Caller-owned device buffers, FP32, contiguous:
 *   q_weight, k_weight [H*K, width], v_weight [HV*V, width] (channel = head * K
 *   + k, the flattening of [H, K]); q_bias, k_bias [H*K], v_bias [HV*V] or NULL
 *   (no bias). width in [1, 4]. */
typedef struct {
  const float* q_weight;
  const float* k_weight;
  const float* v_weight;
  const float* q_bias;
  const float* k_bias;
  const float* v_bias;
  int32_t width;
} kda_short_conv;

/* Problem sizes. T is the physical token extent per batch row (the capacity
 * in varlen mode); N is the number of state entries (B dense, len(cu)-1 varlen). */
typedef struct {
  int32_t B, T, N, H, HV, K, V;
} kda_dims;

/* Human-readable name of a status code (static storage). */
const char* kda_status_string(kda_status s);

/*
 * kda_gate_cumsum -- step A1: gate activation and chunk-local cumsum.
 * Pages: "[Fix] Use unit KDA gate scale when A_log is omitted", Summary and
 * Breaking changes (decay scale exp(A_log), an omitted A_log is the unit
 * scale); "kda in torchtitan (training)", quoted attention-gym description
 * (the gate as a per-token log2 decay, chunk-local cumulative for the chunked
 * op, produced by the gate cumsum with chunk_size 1 or the chunk size).
 *   gate_in  [B, T, HV, K] FP32. If gate_in_is_raw != 0 it holds the raw
 *            activation input x and the per-token natural-log decay is
 *            g = -exp(A_log[hv]) * softplus(x), softplus(x) = ln(1 + e^x)
 *            (x itself for x > 20); A_log [HV] FP32 or NULL for unit scale,
 *            bitwise identical to an all-zero A_log. If gate_in_is_raw == 0,
 *            gate_in already holds the natural-log g and A_log must be NULL.
 *   gate_out [B, T, HV, K] FP32: log2(e) * inclusive cumsum of g inside each
 *            chunk, chunks tiling every sequence from its own first token
 *            (the last chunk may be partial). chunk_size == 1 gives the
 *            per-token log2 decay consumed by kda_recurrent_fwd; chunk_size
 *            == 64 gives the input of kda_chunk_fwd. gate_out may equal gate_in
 *            only when chunk_size == 1 (else KDA_ERR_ALIAS).
 *            Summation order (FP32): within a chunk, blocks of 8 tokens from
 *            the chunk's first token; a token's sum is (C + P) where P adds
 *            its block's tokens up to it in order and C adds the earlier
 *            blocks' totals in order.
 *   Supports chunk_size in [1, 64] (ordinarily 1 or 64), any K, HV.
 */
kda_status kda_gate_cumsum(const kda_dims* dims, const float* gate_in, int32_t gate_in_is_raw,
                           const float* A_log, const int32_t* cu_seqlens, int32_t chunk_size,
                           float* gate_out, hipStream_t stream);

/*
 * kda_gate_cumsum_biased -- step A1 with a gate bias: as kda_gate_cumsum with a
 * raw input, g = -exp(A_log[hv]) * softplus(x + dt_bias[hv * K + c]). The
 * pages ("[Fix] Use unit KDA gate scale when A_log is omitted", commit list:
 * gate bias gradients reduced in FP32 before downcasting) name a gate bias
 * without printing where it enters; it is added to the raw input here.
 *   x        [B, T, HV, K] FP32 raw gate input.
 *   A_log    [HV] FP32 or NULL (unit scale).
 *   dt_bias  [HV, K] FP32 or NULL (no bias; bitwise identical to kda_gate_cumsum).
 *   gate_out as kda_gate_cumsum (same summation order, same in-place rule).
 * Errors as kda_gate_cumsum; dt_bias or A_log overlapping gate_out -> KDA_ERR_ALIAS.
 */
kda_status kda_gate_cumsum_biased(const kda_dims* dims, const float* x, const float* A_log,
                                  const float* dt_bias, const int32_t* cu_seqlens,
                                  int32_t chunk_size, float* gate_out, hipStream_t stream);

/* Workspace bytes kda_gate_bwd needs when it reduces dA_log or d_dt_bias. */
size_t kda_gate_bwd_workspace_bytes(const kda_dims* dims);

/*
 * kda_gate_bwd -- reverse of the raw gate activation of kda_gate_cumsum_biased
 * (and of kda_gate_cumsum with a raw input, dt_bias = NULL), for the gradient dg
 * of the per-token natural-log gate g (what kda_chunk_bwd returns as dg):
 *   dx[t, hv, c]   = -exp(A_log[hv]) * sigmoid(x + dt_bias[hv, c]) * dg[t, hv, c]
 *                    (sigmoid = 1 above 20, where softplus returns its argument)
 *   dA_log[hv]     = sum over tokens inside a sequence and channels of dg * g
 *   d_dt_bias[hv, c] = sum over tokens inside a sequence of dx[t, hv, c]
 *   x, dg    [B, T, HV, K] FP32; dx [B, T, HV, K] FP32 (may be dg itself; rows
 *            of tokens outside every sequence are untouched).
 *   A_log, dt_bias as in kda_gate_cumsum_biased; dA_log [HV] and d_dt_bias
 *            [HV, K] FP32 are written exactly when A_log, resp. dt_bias, is
 *            given (else KDA_ERR_SHAPE).
 *   Reductions: each block of 256 tokens sums its tokens in order into an FP32
 *            partial per element (in `workspace`); the partials are summed over
 *            blocks in order, and for dA_log then over channels in order, so
 *            results are run-to-run deterministic.
 *   workspace: at least kda_gate_bwd_workspace_bytes(), 16-byte aligned,
 *            required only when dA_log or d_dt_bias is requested (else may be
 *            NULL); scratch on entry and return.
 *   Supports any B, T, HV and K <= 4096. Errors: NULL inputs/outputs with
 *   tokens present -> KDA_ERR_NULL; missing or small workspace ->
 *   KDA_ERR_WORKSPACE; overlaps other than dx == dg -> KDA_ERR_ALIAS.
 */
kda_status kda_gate_bwd(const kda_dims* dims, const float* x, const float* A_log,
                        const float* dt_bias, const float* dg, const int32_t* cu_seqlens,
                        float* dx, float* dA_log, float* d_dt_bias, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes kda_chunk_fwd needs for these sizes (0 on unsupported input). */
size_t kda_chunk_fwd_workspace_bytes(const kda_dims* dims, kda_dtype dtype, int32_t chunk_size);

/*
 * kda_chunk_fwd -- steps A2..A6: the chunked scan (chunk_kda forward).
 * Pages: "[Fix] Use unit KDA gate scale when A_log is omitted", squashed
 * commit bodies (the chunked pipeline kkt, solve_tril, recompute_w_u, fwd_h,
 * fwd_o of the sibling gated delta rule op, here with a per-channel gate);
 * "kda in torchtitan (training)", quoted attention-gym description (the
 * chunk_kda argument contract and packed-sequence layout).
 *   gate   [B, T, HV, K] FP32 chunk-local cumulative log2 gate, i.e. the
 *          output of kda_gate_cumsum with the same chunk_size and cu_seqlens.
 *   initial_state [N, HV, K, V] FP32 or NULL (zeros).
 *   o      [B, T, HV, V] in `dtype`; rows outside every sequence untouched.
 *   final_state [N, HV, K, V] FP32, required iff output_final_state != 0
 *          (may equal initial_state).
 *   workspace: device scratch of at least kda_chunk_fwd_workspace_bytes();
 *          its contents are scratch on entry and on return.
 *   Supported: K, V in {64, 128}; chunk_size == 64; FP32 or BF16; q, k, v,
 *   gate and o 16-byte aligned, workspace 256-byte aligned (else
 *   KDA_ERR_UNSUPPORTED).
 *   Arithmetic: FP32 accumulation and FP32 state; for BF16 inputs the
 *   matrix products take bf16 operands on the matrix cores.
 */
kda_status kda_chunk_fwd(const kda_dims* dims, kda_dtype dtype, const void* q, const void* k,
                         const void* v, const float* gate, const void* beta,
                         const float* initial_state, const int32_t* cu_seqlens,
                         int32_t chunk_size, int32_t output_final_state, void* o,
                         float* final_state, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * kda_chunk_fwd_fused_gate -- steps A1..A6 in one call: kda_chunk_fwd with
 * the gate step done inside the intra-chunk kernel (the fused-gate chunk KDA
 * path, `use_gate_in_kernel`, of "[Fix] Use unit KDA gate scale when A_log is
 * omitted", Summary).
 *   gate_in, gate_in_is_raw, A_log: as kda_gate_cumsum (raw x with
 *          g = -exp(A_log[hv]) softplus(x), A_log NULL = unit scale; or the
 *          natural-log g itself, A_log NULL). The chunk-local log2 cumsum is
 *          formed in the kernel with the gate kernel's float operations, so o
 *          and final_state are bit-identical to kda_gate_cumsum(chunk_size)
 *          followed by kda_chunk_fwd, without materialising the log2 gate.
 *   Other arguments, workspace size, support and alignment as kda_chunk_fwd
 *   (gate_in in place of gate).
 */
kda_status kda_chunk_fwd_fused_gate(const kda_dims* dims, kda_dtype dtype, const void* q,
                                    const void* k, const void* v, const float* gate_in,
                                    int32_t gate_in_is_raw, const float* A_log, const void* beta,
                                    const float* initial_state, const int32_t* cu_seqlens,
                                    int32_t chunk_size, int32_t output_final_state, void* o,
                                    float* final_state, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/*
 * kda_chunk_fwd_ex -- kda_chunk_fwd / kda_chunk_fwd_fused_gate with the gate
 * kind as an argument and optional q/k L2 normalisation (the pages' l2norm
 * pre-processing step, "kda in torchtitan (training)", fused into the loads):
 *   gate_kind  kda_gate_kind; A_log only with KDA_GATE_RAW (else KDA_ERR_SHAPE).
 *   qk_l2norm  nonzero: q and k are used as x / sqrt(sum over K of x^2 + 1e-6)
 *              per (token, qk head), computed in FP32 from the input (bf16
 *              inputs: the normalised rows are rounded to bf16 before the
 *              matrix products, as a separate normalisation pass would store them).
 * With qk_l2norm == 0 the results are bit-identical to kda_chunk_fwd
 * (KDA_GATE_LOG2) and kda_chunk_fwd_fused_gate (the other kinds). No backward
 * counterpart: kda_chunk_bwd expects normalised inputs.
 */
kda_status kda_chunk_fwd_ex(const kda_dims* dims, kda_dtype dtype, const void* q, const void* k,
                            const void* v, const float* gate, int32_t gate_kind,
                            const float* A_log, int32_t qk_l2norm, const void* beta,
                            const float* initial_state, const int32_t* cu_seqlens,
                            int32_t chunk_size, int32_t output_final_state, void* o,
                            float* final_state, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * kda_chunk_fwd_conv -- kda_chunk_fwd_ex with the short convolution + SiLU of
 * q, k and v fused into the loads (pre-processing step of the KDA layer; the
 * torchtitan training page and the Paddle compatibility page import it):
 *   q, k, v  the raw projections ([B, T, H, K] / [B, T, HV, V] in `dtype`);
 *            the scan sees y = SiLU(conv(x)) of each (kda_short_conv), rounded
 *            to `dtype` as a separate convolution pass would store it.
 *   conv     taps and biases (kda_short_conv); NULL, a NULL weight or a width
 *            outside [1, 4] is an error (KDA_ERR_NULL / KDA_ERR_UNSUPPORTED).
 *   qk_l2norm  as kda_chunk_fwd_ex, applied to the convolution's output.
 * Every sequence starts from zero convolution history (no carried-over
 * convolution state). Other arguments, sizes, workspace and errors as
 * kda_chunk_fwd_ex; the conv buffers must not overlap o, final_state or the
 * workspace (KDA_ERR_ALIAS). No backward counterpart.
 */
kda_status kda_chunk_fwd_conv(const kda_dims* dims, kda_dtype dtype, const void* q, const void* k,
                              const void* v, const kda_short_conv* conv, const float* gate,
                              int32_t gate_kind, const float* A_log, int32_t qk_l2norm,
                              const void* beta, const float* initial_state,
                              const int32_t* cu_seqlens, int32_t chunk_size,
                              int32_t output_final_state, void* o, float* final_state,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_short_conv_fwd -- the short convolution + SiLU on its own, with a carried
 * per-sequence history (decode continues a sequence's filter; a prefill hands
 * its history over):
 *   q, k, v    raw projections [B, T, H, K], [B, T, H, K], [B, T, HV, V] in `dtype`.
 *   conv       taps and biases (kda_short_conv), as kda_chunk_fwd_conv.
 *   conv_state_in  [N, W - 1, 2*H*K + HV*V] in `dtype`, or NULL (zero history):
 *              per sequence the W - 1 raw inputs before its first token, oldest
 *              row first, channels in the order q (H*K), k (H*K), v (HV*V).
 *   conv_state_out same layout, or NULL: receives the last W - 1 raw inputs of
 *              each sequence, reaching back into conv_state_in (or zeros) for a
 *              sequence shorter than W - 1; an empty slot gets conv_state_in
 *              bitwise (or zeros). May equal conv_state_in (updated in place).
 *   q_out, k_out, v_out  outputs SiLU(conv(x)) (layout of the inputs, rounded to
 *              `dtype`), or all three NULL to compute the history only (reads
 *              only the last W - 1 tokens of each sequence). Each may equal its
 *              own input (in place); no other overlap (KDA_ERR_ALIAS).
 * Rows outside every sequence are neither read nor written. Needs K and V
 * multiples of 16 bytes' worth of elements and 16-byte aligned buffers
 * (KDA_ERR_UNSUPPORTED). Each thread walks one sequence's tokens in order:
 * meant for decode and short segments; long prefills use kda_chunk_fwd_conv.
 */
kda_status kda_short_conv_fwd(const kda_dims* dims, kda_dtype dtype, const void* q, const void* k,
                              const void* v, const kda_short_conv* conv,
                              const int32_t* cu_seqlens, const void* conv_state_in,
                              void* conv_state_out, void* q_out, void* k_out, void* v_out,
                              hipStream_t stream);

/* Workspace bytes kda_recurrent_fwd_conv needs (the convolved q, k, v; 0 on
 * invalid dims). */
size_t kda_recurrent_fwd_conv_workspace_bytes(const kda_dims* dims, kda_dtype dtype);

/*
 * kda_recurrent_fwd_conv -- decode from raw projections: kda_short_conv_fwd
 * (carried history conv_state_in -> conv_state_out, convolved q, k, v into the
 * workspace) then kda_recurrent_fwd_ex on them (gate kind, A_log and q/k L2
 * normalisation as there). Arguments as those two entry points; the workspace
 * (256-byte aligned, kda_recurrent_fwd_conv_workspace_bytes) must not overlap
 * any other buffer. All arguments are checked before the first launch.
 */
kda_status kda_recurrent_fwd_conv(const kda_dims* dims, kda_dtype dtype, const void* q,
                                  const void* k, const void* v, const kda_short_conv* conv,
                                  const void* conv_state_in, void* conv_state_out,
                                  const float* gate, int32_t gate_kind, const float* A_log,
                                  int32_t qk_l2norm, const void* beta, const float* initial_state,
                                  const int32_t* cu_seqlens, int32_t output_final_state, void* o,
                                  float* final_state, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* Size of the library's own device scratch used by
 * kda_recurrent_fwd_conv_noalloc (16 MiB per GPU, held until the process ends). */
#define KDA_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * kda_recurrent_fwd_conv_noalloc -- kda_recurrent_fwd_conv without a workspace
 * argument, for callers that cannot allocate device memory (HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc). Same arguments,
 * results (bit-identical) and errors as kda_recurrent_fwd_conv, minus
 * workspace / workspace_bytes: the convolved q, k, v live in a static device
 * scratch of KDA_NOALLOC_SCRATCH_BYTES that the library owns (one per GPU).
 *   Limit: kda_recurrent_fwd_conv_workspace_bytes(dims, dtype) must be at most
 *          KDA_NOALLOC_SCRATCH_BYTES (else KDA_ERR_WORKSPACE, nothing enqueued);
 *          e.g. 2 * T * H * K + T * HV * V bf16 elements = 4 MiB for 256 decode
 *          tokens at H = 16, HV = 32, K = V = 128.
 *   Allocates nothing: no hipMalloc / hipFree. The first call on a device
 *          looks up that device's scratch address (hipGetSymbolAddress).
 *   Concurrency: every call on a GPU shares that GPU's scratch; calls that
 *          overlap on one GPU (different streams, or host threads without
 *          ordering) race and must be serialised by the caller. The scratch
 *          keeps the last call's contents; each call writes all it reads.
 */
kda_status kda_recurrent_fwd_conv_noalloc(const kda_dims* dims, kda_dtype dtype, const void* q,
                                          const void* k, const void* v, const kda_short_conv* conv,
                                          const void* conv_state_in, void* conv_state_out,
                                          const float* gate, int32_t gate_kind, const float* A_log,
                                          int32_t qk_l2norm, const void* beta,
                                          const float* initial_state, const int32_t* cu_seqlens,
                                          int32_t output_final_state, void* o, float* final_state,
                                          hipStream_t stream);

/* Workspace bytes kda_chunk_bwd needs for these sizes (0 on unsupported input). */
size_t kda_chunk_bwd_workspace_bytes(const kda_dims* dims, kda_dtype dtype, int32_t chunk_size);

/*
 * kda_chunk_bwd -- steps B1..B3: gradients of kda_chunk_fwd.
 * Pages: "[KDA] Add Paddle training compatibility", Summary (dense and
 * variable-length chunk_kda forward/backward with gate, beta, state and GVA
 * gradients); "[Fix] Use unit KDA gate scale when A_log is omitted",
 * squashed commit bodies (the sibling op's backward kernels: bwd_dhu for the
 * reverse state-gradient recurrence, chunk_bwd_dqkwg and chunk_bwd_dv_local
 * for the local gradients, prepare_wy_repr_bwd for the UT transform's).
 *   Forward arguments as kda_chunk_fwd (gate = chunk-local log2 cumsum).
 *   do_    [B, T, HV, V] in `dtype`: gradient of o.
 *   dht    [N, HV, K, V] FP32 gradient of the final state, or NULL (zero).
 *   dq, dk [B, T, H, K] in `dtype` (summed over the HV/H value heads of each
 *          qk head); dv [B, T, HV, V] and dbeta [B, T, HV] in `dtype`;
 *   dg     [B, T, HV, K] FP32, gradient w.r.t. the per-token natural-log gate
 *          g (dg_t = sum over t' >= t in the chunk of dL/dG_t', G the
 *          natural-log cumulative gate);
 *   dh0    [N, HV, K, V] FP32 gradient of the initial state (for an empty
 *          slot a bitwise copy of dht, or +0.0).
 *   Rows outside every sequence are left untouched. The forward intra-chunk
 *   terms and chunk start states are recomputed, not taken from a forward
 *   call. Supported sizes and alignment as kda_chunk_fwd, except that FP32
 *   inputs need K == 64 (KDA_ERR_UNSUPPORTED otherwise).
 */
kda_status kda_chunk_bwd(const kda_dims* dims, kda_dtype dtype, const void* q, const void* k,
                         const void* v, const float* gate, const void* beta,
                         const float* initial_state, const int32_t* cu_seqlens,
                         int32_t chunk_size, const void* do_, const float* dht, void* dq,
                         void* dk, void* dv, float* dg, void* dbeta, float* dh0,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_chunk_fwd_train -- kda_chunk_fwd for training: the same outputs (o and
 * final_state bit-identical to kda_chunk_fwd), and on the way the backward
 * pass's workspace is filled with what the backward would otherwise form
 * again: every chunk's start state and Delta = U - W S0 (the backward's
 * forward recurrence, steps B1 and B2 of the chunked pipeline's backward,
 * fwd_h / bwd_dhu in the squashed commit bodies of "[Fix] Use unit KDA gate
 * scale when A_log is omitted") and the intra-chunk matrices the backward
 * reads (its recompute of the intra-chunk terms), so that kda_chunk_bwd_saved
 * skips both.
 *   Arguments as kda_chunk_fwd, except the workspace:
 *   bwd_workspace  at least kda_chunk_bwd_workspace_bytes() for the same
 *          dims, dtype and chunk_size, 256-byte aligned; to be handed,
 *          unmodified, to kda_chunk_bwd_saved with the same inputs (q, k, v,
 *          gate, beta, initial_state, cu_seqlens). The caller owns it.
 *   Supported sizes as kda_chunk_bwd (FP32 needs K == 64). Errors as
 *   kda_chunk_fwd (KDA_ERR_WORKSPACE if the workspace is smaller than the
 *   backward's).
 */
kda_status kda_chunk_fwd_train(const kda_dims* dims, kda_dtype dtype, const void* q, const void* k,
                               const void* v, const float* gate, const void* beta,
                               const float* initial_state, const int32_t* cu_seqlens,
                               int32_t chunk_size, int32_t output_final_state, void* o,
                               float* final_state, void* bwd_workspace, size_t bwd_workspace_bytes,
                               hipStream_t stream);

/*
 * kda_chunk_bwd_saved -- kda_chunk_bwd after kda_chunk_fwd_train: takes the
 * chunk start states, Deltas and intra-chunk matrices that the training
 * forward stored in `workspace` instead of forming them again (no forward
 * recurrence, no intra-chunk recompute); the remaining steps as kda_chunk_bwd,
 * and every gradient bit-identical to it.
 *   Arguments, sizes and errors as kda_chunk_bwd. Precondition (not
 *   checkable on the host): `workspace` holds the output of
 *   kda_chunk_fwd_train on the same dims, dtype, chunk_size and inputs, and has
 *   not been written since; otherwise the results are undefined.
 */
kda_status kda_chunk_bwd_saved(const kda_dims* dims, kda_dtype dtype, const void* q, const void* k,
                               const void* v, const float* gate, const void* beta,
                               const float* initial_state, const int32_t* cu_seqlens,
                               int32_t chunk_size, const void* do_, const float* dht, void* dq,
                               void* dk, void* dv, float* dg, void* dbeta, float* dh0,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_chunk_fwd_train_ex, kda_chunk_bwd_ex -- the training forward and the
 * backward with the gate kind as an argument, as kda_chunk_fwd_ex takes it:
 * with KDA_GATE_RAW (g = -exp(A_log[hv]) softplus(x), A_log NULL = unit
 * scale) or KDA_GATE_NAT the gate step (the fused-gate chunk KDA path,
 * `use_gate_in_kernel`, of "[Fix] Use unit KDA gate scale when A_log is
 * omitted", Summary) runs inside the kernels that read the gate, so a
 * training step never materialises the chunk-local log2 gate. The kernels use
 * the gate kernel's float operations and summation order: every result is
 * bit-identical to kda_gate_cumsum(chunk_size) followed by the KDA_GATE_LOG2
 * call.
 *   kda_chunk_fwd_train_ex  as kda_chunk_fwd_train, gate in `gate_kind`.
 *   kda_chunk_bwd_ex        as kda_chunk_bwd (saved == 0) or
 *          kda_chunk_bwd_saved (saved != 0: `workspace` filled by
 *          kda_chunk_fwd_train(_ex) on the same inputs and gate kind). dg is
 *          the gradient w.r.t. the per-token natural-log gate g in every kind
 *          (kda_gate_bwd takes it back to the raw input).
 *   gate_kind outside kda_gate_kind, or A_log with a kind other than
 *   KDA_GATE_RAW: KDA_ERR_SHAPE; A_log [HV] FP32 overlapping an output or
 *   the workspace: KDA_ERR_ALIAS. Everything else as the KDA_GATE_LOG2 entry
 *   points (with KDA_GATE_LOG2 they are those calls).
 */
kda_status kda_chunk_fwd_train_ex(const kda_dims* dims, kda_dtype dtype, const void* q,
                                  const void* k, const void* v, const float* gate,
                                  int32_t gate_kind, const float* A_log, const void* beta,
                                  const float* initial_state, const int32_t* cu_seqlens,
                                  int32_t chunk_size, int32_t output_final_state, void* o,
                                  float* final_state, void* bwd_workspace,
                                  size_t bwd_workspace_bytes, hipStream_t stream);
kda_status kda_chunk_bwd_ex(const kda_dims* dims, kda_dtype dtype, const void* q, const void* k,
                            const void* v, const float* gate, int32_t gate_kind,
                            const float* A_log, const void* beta, const float* initial_state,
                            const int32_t* cu_seqlens, int32_t chunk_size, const void* do_,
                            const float* dht, void* dq, void* dk, void* dv, float* dg,
                            void* dbeta, float* dh0, int32_t saved, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * kda_recurrent_fwd -- step A7: the token-sequential scan (recurrent_kda).
 * Page: "kda in torchtitan (training)", quoted attention-gym description of
 * recurrent_kda (signature and packed contract of chunk_kda, per-token log2
 * gate, 1/sqrt(K) query scale, FP32 state and compute).
 *   gate   [B, T, HV, K] FP32 per-token log2 decay (kda_gate_cumsum with
 *          chunk_size == 1).
 *   Other arguments as kda_chunk_fwd. Computes in FP32 for any input dtype.
 *   Supported: 1 <= K, V <= 256 (any value, not only powers of two).
 *   Decode is the T-per-sequence == 1 case; final_state == initial_state
 *   updates the states in place.
 */
kda_status kda_recurrent_fwd(const kda_dims* dims, kda_dtype dtype, const void* q, const void* k,
                             const void* v, const float* gate, const void* beta,
                             const float* initial_state, const int32_t* cu_seqlens,
                             int32_t output_final_state, void* o, float* final_state,
                             hipStream_t stream);

/*
 * kda_recurrent_fwd_fused_gate -- steps A1 + A7 in one call: kda_recurrent_fwd
 * with the per-token gate activation done in the scan kernel (the fused-gate
 * recurrent path of the same page).
 *   gate_in, gate_in_is_raw, A_log: as kda_gate_cumsum. Results are
 *   bit-identical to kda_gate_cumsum(chunk_size = 1) followed by
 *   kda_recurrent_fwd. Other arguments and support as kda_recurrent_fwd.
 */
kda_status kda_recurrent_fwd_fused_gate(const kda_dims* dims, kda_dtype dtype, const void* q,
                                        const void* k, const void* v, const float* gate_in,
                                        int32_t gate_in_is_raw, const float* A_log,
                                        const void* beta, const float* initial_state,
                                        const int32_t* cu_seqlens, int32_t output_final_state,
                                        void* o, float* final_state, hipStream_t stream);

/*
 * kda_recurrent_fwd_ex -- kda_recurrent_fwd / kda_recurrent_fwd_fused_gate with
 * the gate kind as an argument and optional q/k L2 normalisation, as
 * kda_chunk_fwd_ex (normalisation in FP32, reduced with the scan's own
 * reductions). With qk_l2norm == 0 bit-identical to those entry points.
 */
kda_status kda_recurrent_fwd_ex(const kda_dims* dims, kda_dtype dtype, const void* q,
                                const void* k, const void* v, const float* gate,
                                int32_t gate_kind, const float* A_log, int32_t qk_l2norm,
                                const void* beta, const float* initial_state,
                                const int32_t* cu_seqlens, int32_t output_final_state, void* o,
                                float* final_state, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
