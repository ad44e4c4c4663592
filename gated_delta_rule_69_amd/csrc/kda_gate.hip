// Step A1: KDA gate activation and chunk-local cumulative sum (log2 units).
//
// g = -exp(A_log[hv]) * softplus(x) (unit scale when A_log is omitted, per
// "[Fix] Use unit KDA gate scale when A_log is omitted", Summary), then the
// inclusive cumsum of g inside each chunk times log2(e) (the per-token or
// chunk-local cumulative log2 gate of the `recurrent_kda` / `chunk_kda`
// contract in "kda in torchtitan (training)").
//
// An optional per-(head, channel) bias is added to the raw input before the
// activation (the pages name a gate bias and its FP32-reduced gradient:
// "[Fix] Use unit KDA gate scale when A_log is omitted", commit list).
//
// The gate backward (gate_bwd_kernel, gate_bwd_reduce_kernel) turns the
// gradient of the per-token natural-log gate into dx = -exp(A_log) *
// sigmoid(x + dt_bias) * dg, d_dt_bias = sum over tokens of dx and dA_log =
// sum over tokens and channels of dg * g, with FP32 partials per block of
// tokens summed in a fixed order.
//
// HBM-bound elementwise + segmented scan. Each thread owns VEC consecutive
// floats of a token row (HV*K floats) and walks TILE tokens in order, so a
// wave reads 64*VEC*4 contiguous bytes per token. Chunks tile each sequence
// from its own first token, so a tile may start inside a chunk: the thread
// then first sums the chunk's earlier tokens (at most chunk-1 of them). The
// sums follow the blocked order of kGateBlock.
#include "kda_common.h"

namespace kda {

constexpr int kGateThreads = 256;
// TILE tokens per workgroup (64 for chunked output so any chunk start is
// reachable within one carry-in pass; 16 for per-token output).
template <int VEC, int TILE>
__global__ void __launch_bounds__(kGateThreads)
gate_cumsum_kernel(const float* __restrict__ in, int is_raw, const float* __restrict__ A_log,
                   const float* __restrict__ bias, const int32_t* __restrict__ cu, int N, int T,
                   int64_t n_tok, int HV, int K, int chunk, float* out) {
  __shared__ int64_t s_cstart[TILE];  // chunk start of each tile token (-1: outside)
  const int64_t t_a = (int64_t)blockIdx.x * TILE;
  const int row = HV * K;
  // per-token chunk start (sequence lookup: dense rows or binary search of cu)
  if (threadIdx.x < TILE) {
    const int64_t t = t_a + threadIdx.x;
    int64_t cs = -1;
    if (chunk == 1) {
      const int64_t lim = cu ? (int64_t)cu[N] : n_tok;
      cs = t < lim ? t : -1;
    } else if (t < n_tok) {
      int64_t bos = -1;
      if (cu == nullptr) {
        bos = (t / T) * (int64_t)T;
      } else if (t < cu[N]) {
        int lo = 0, hi = N - 1;  // last n with cu[n] <= t and cu[n+1] > t
        while (lo < hi) {
          int mid = (lo + hi + 1) >> 1;
          if (cu[mid] <= t) lo = mid; else hi = mid - 1;
        }
        bos = cu[lo];
      }
      if (bos >= 0) cs = bos + ((t - bos) / chunk) * chunk;
    }
    s_cstart[threadIdx.x] = cs;
  }
  __syncthreads();
  const int f0 = (blockIdx.y * kGateThreads + threadIdx.x) * VEC;
  if (f0 >= row) return;
  float scale[VEC], bv[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    int hv = (f0 + e) / K;
    scale[e] = (is_raw && A_log) ? expf(A_log[hv]) : 1.f;
    bv[e] = bias ? bias[f0 + e] : 0.f;
  }
  auto load = [&](int64_t t, float* x) {
    const float* p = in + t * row + f0;
    if constexpr (VEC == 4) {
      float4 v = *reinterpret_cast<const float4*>(p);
      x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    } else if constexpr (VEC == 2) {
      float2 v = *reinterpret_cast<const float2*>(p);
      x[0] = v.x; x[1] = v.y;
    } else {
      x[0] = *p;
    }
  };
  auto act = [&](float* x) {
#pragma unroll
    for (int e = 0; e < VEC; ++e)
      x[e] = gate_nat(bias ? x[e] + bv[e] : x[e], is_raw ? kGateRaw : kGateLog, scale[e]);
  };
  // blocked running sum (see kGateBlock): carry C of finished blocks, P of
  // the current block
  float C[VEC], P[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) C[e] = P[e] = 0.f;
  auto accumulate = [&](int64_t pos, const float* g) {
    const bool fresh = pos == 0, bstart = (pos % kGateBlock) == 0;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      C[e] = fresh ? 0.f : (bstart ? C[e] + P[e] : C[e]);
      P[e] = (bstart ? 0.f : P[e]) + g[e];
    }
  };
  // carry-in: the tile starts inside a chunk that began earlier
  if (chunk > 1) {
    const int64_t cs = s_cstart[0];
    if (cs >= 0 && cs < t_a) {
      for (int64_t t = cs; t < t_a; ++t) {
        float g[VEC];
        load(t, g);
        act(g);
        accumulate(t - cs, g);
      }
    }
  }
  // main pass: BATCH loads in flight (tokens outside the contract load token 0
  // and are discarded), then the scan and the stores. A thread only touches its
  // own elements, so in-place per-token use is safe.
  constexpr int BATCH = TILE < 16 ? TILE : 16;
  for (int i0 = 0; i0 < TILE; i0 += BATCH) {
    float g[BATCH][VEC];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int64_t t = t_a + i0 + b;
      load(s_cstart[i0 + b] >= 0 ? t : 0, g[b]);
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      act(g[b]);
      const int64_t t = t_a + i0 + b;
      const int64_t cs = s_cstart[i0 + b];
      accumulate(cs >= 0 ? t - cs : 0, g[b]);
      float r[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) r[e] = (C[e] + P[e]) * kLog2e;
      if (cs >= 0) {
        float* p = out + t * row + f0;
        if constexpr (VEC == 4) {
          *reinterpret_cast<float4*>(p) = make_float4(r[0], r[1], r[2], r[3]);
        } else if constexpr (VEC == 2) {
          *reinterpret_cast<float2*>(p) = make_float2(r[0], r[1]);
        } else {
          *p = r[0];
        }
      }
    }
  }
}

constexpr int kGateBwdTok = 256;  // tokens per workgroup of gate_bwd_kernel (one partial row)

// dx for the tokens [t_a, t_a + kGateBwdTok) inside a sequence, and this
// block's partial sums (in token order) of dx and dg * g per row element.
// Tokens outside every sequence are skipped (dx untouched, no contribution).
template <int VEC>
__global__ void __launch_bounds__(kGateThreads)
gate_bwd_kernel(const float* __restrict__ x, const float* __restrict__ A_log,
                const float* __restrict__ bias, const float* dg, const int32_t* __restrict__ cu,
                int N, int64_t n_tok, int HV, int K, float* dx, float* __restrict__ part_db,
                float* __restrict__ part_da) {
  const int row = HV * K;
  const int f0 = (blockIdx.y * kGateThreads + threadIdx.x) * VEC;
  if (f0 >= row) return;
  const int64_t lim = cu ? (int64_t)cu[N] : n_tok;
  const int64_t t_a = (int64_t)blockIdx.x * kGateBwdTok;
  const int64_t t_b = t_a + kGateBwdTok < lim ? t_a + kGateBwdTok : lim;
  float scale[VEC], bv[VEC], adb[VEC], ada[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    scale[e] = A_log ? expf(A_log[(f0 + e) / K]) : 1.f;
    bv[e] = bias ? bias[f0 + e] : 0.f;
    adb[e] = ada[e] = 0.f;
  }
  auto ld = [&](const float* base, int64_t t, float* v) {
    const float* p = base + t * row + f0;
    if constexpr (VEC == 4) {
      const float4 u = *reinterpret_cast<const float4*>(p);
      v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
    } else if constexpr (VEC == 2) {
      const float2 u = *reinterpret_cast<const float2*>(p);
      v[0] = u.x; v[1] = u.y;
    } else {
      v[0] = *p;
    }
  };
  constexpr int BATCH = 8;
  for (int64_t t0 = t_a; t0 < t_b; t0 += BATCH) {
    float xv[BATCH][VEC], gv[BATCH][VEC];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {  // tokens past t_b load t_a (inside) and are discarded
      const int64_t t = t0 + b < t_b ? t0 + b : t_a;
      ld(x, t, xv[b]);
      ld(dg, t, gv[b]);
    }
    // every loaded token is used (the partial sums select, only the store is
    // guarded): a token whose use sits behind a branch has its load sunk into
    // that branch, where it is issued just before it is needed
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const bool in = t0 + b < t_b;
      float r[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
#pragma clang fp contract(off)
        const float u = bias ? xv[b][e] + bv[e] : xv[b][e];
        const float g = -scale[e] * softplus_f32(u);
        r[e] = -scale[e] * sigmoid_f32(u) * gv[b][e];
        adb[e] = in ? adb[e] + r[e] : adb[e];
        ada[e] = in ? ada[e] + gv[b][e] * g : ada[e];
      }
      if (!in) continue;
      float* p = dx + (t0 + b) * row + f0;
      if constexpr (VEC == 4) {
        *reinterpret_cast<float4*>(p) = make_float4(r[0], r[1], r[2], r[3]);
      } else if constexpr (VEC == 2) {
        *reinterpret_cast<float2*>(p) = make_float2(r[0], r[1]);
      } else {
        *p = r[0];
      }
    }
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    if (part_db) part_db[(int64_t)blockIdx.x * row + f0 + e] = adb[e];
    if (part_da) part_da[(int64_t)blockIdx.x * row + f0 + e] = ada[e];
  }
}

// One workgroup per head: d_dt_bias[hv, c] = sum over blocks (in order) of
// the dx partials; dA_log[hv] = sum over channels c (in order) of the block
// sums (in order) of the dg * g partials. K floats of dynamic LDS.
__global__ void __launch_bounds__(kGateThreads)
gate_bwd_reduce_kernel(const float* __restrict__ part_db, const float* __restrict__ part_da,
                       int nblk, int HV, int K, float* __restrict__ d_bias,
                       float* __restrict__ dA) {
  extern __shared__ float s_ch[];
  const int hv = blockIdx.x, row = HV * K;
  constexpr int R = 16;  // partials in flight per thread; the sums still run in block order
  for (int c = threadIdx.x; c < K; c += blockDim.x) {
    float sb = 0.f, sa = 0.f;
    const int64_t base = (int64_t)hv * K + c;
    for (int b0 = 0; b0 < nblk; b0 += R) {
      float vb[R], va[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t o = (int64_t)(b0 + r < nblk ? b0 + r : 0) * row + base;
        vb[r] = d_bias ? part_db[o] : 0.f;
        va[r] = dA ? part_da[o] : 0.f;
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (b0 + r < nblk) {
          sb += vb[r];
          sa += va[r];
        }
      }
    }
    if (d_bias) d_bias[hv * K + c] = sb;
    s_ch[c] = sa;
  }
  __syncthreads();
  if (dA && threadIdx.x == 0) {
    float s = 0.f;
    for (int c = 0; c < K; ++c) s += s_ch[c];
    dA[hv] = s;
  }
}

}  // namespace kda

namespace kda_host {

hipError_t launch_gate(const kda_dims& d, const float* in, int is_raw, const float* A_log,
                       const float* dt_bias, const int32_t* cu, int chunk, float* out,
                       hipStream_t s) {
  const int64_t n_tok = (int64_t)d.B * d.T;
  if (n_tok == 0) return hipSuccess;
  const int row = d.HV * d.K;
  int vec = 1;
  if (row % 4 == 0 && ((uintptr_t)in % 16 == 0) && ((uintptr_t)out % 16 == 0)) vec = 4;
  else if (row % 2 == 0 && ((uintptr_t)in % 8 == 0) && ((uintptr_t)out % 8 == 0)) vec = 2;
  const int tile = chunk == 1 ? 16 : 64;
  dim3 grid((unsigned)((n_tok + tile - 1) / tile),
            (unsigned)((row / vec + kda::kGateThreads - 1) / kda::kGateThreads));
  dim3 block(kda::kGateThreads);
#define KDA_GATE_LAUNCH(V_, TL_)                                                              \
  hipLaunchKernelGGL((kda::gate_cumsum_kernel<V_, TL_>), grid, block, 0, s, in, is_raw, A_log, \
                     dt_bias, cu, d.N, d.T, n_tok, d.HV, d.K, chunk, out)
  if (tile == 16) {
    if (vec == 4) KDA_GATE_LAUNCH(4, 16);
    else if (vec == 2) KDA_GATE_LAUNCH(2, 16);
    else KDA_GATE_LAUNCH(1, 16);
  } else {
    if (vec == 4) KDA_GATE_LAUNCH(4, 64);
    else if (vec == 2) KDA_GATE_LAUNCH(2, 64);
    else KDA_GATE_LAUNCH(1, 64);
  }
#undef KDA_GATE_LAUNCH
  return hipGetLastError();
}

size_t gate_bwd_ws_bytes(const kda_dims& d) {
  const int64_t n_tok = (int64_t)d.B * d.T;
  const int64_t nblk = (n_tok + kda::kGateBwdTok - 1) / kda::kGateBwdTok;
  const size_t one = ((size_t)nblk * d.HV * d.K * sizeof(float) + 255) & ~(size_t)255;
  return 2 * one;
}

hipError_t launch_gate_bwd(const kda_dims& d, const float* x, const float* A_log,
                           const float* dt_bias, const float* dg, const int32_t* cu, float* dx,
                           float* dA_log, float* d_dt_bias, void* ws, hipStream_t s) {
  const int64_t n_tok = (int64_t)d.B * d.T;
  const int row = d.HV * d.K;
  const int64_t nblk = (n_tok + kda::kGateBwdTok - 1) / kda::kGateBwdTok;
  const size_t one = gate_bwd_ws_bytes(d) / 2;
  float* part_db = d_dt_bias ? reinterpret_cast<float*>(ws) : nullptr;
  float* part_da = dA_log ? reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + one) : nullptr;
  if (nblk > 0) {
    int vec = 1;
    const uintptr_t al = (uintptr_t)x | (uintptr_t)dg | (uintptr_t)dx;
    if (row % 4 == 0 && al % 16 == 0) vec = 4;
    else if (row % 2 == 0 && al % 8 == 0) vec = 2;
    dim3 grid((unsigned)nblk, (unsigned)((row / vec + kda::kGateThreads - 1) / kda::kGateThreads));
#define KDA_GATE_BWD(V_)                                                                       \
  hipLaunchKernelGGL((kda::gate_bwd_kernel<V_>), grid, dim3(kda::kGateThreads), 0, s, x, A_log, \
                     dt_bias, dg, cu, d.N, n_tok, d.HV, d.K, dx, part_db, part_da)
    if (vec == 4) KDA_GATE_BWD(4);
    else if (vec == 2) KDA_GATE_BWD(2);
    else KDA_GATE_BWD(1);
#undef KDA_GATE_BWD
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (dA_log || d_dt_bias) {
    hipLaunchKernelGGL(kda::gate_bwd_reduce_kernel, dim3((unsigned)d.HV), dim3(kda::kGateThreads),
                       (size_t)d.K * sizeof(float), s, part_db, part_da, (int)nblk, d.HV, d.K,
                       d_dt_bias, dA_log);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace kda_host
