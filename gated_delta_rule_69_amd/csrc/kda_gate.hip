// Step A1: KDA gate activation and chunk-local cumulative sum (log2 units).
//
// g = -exp(A_log[hv]) * softplus(x) (unit scale when A_log is omitted, per
// "[Fix] Use unit KDA gate scale when A_log is omitted", Summary), then the
// inclusive cumsum of g inside each chunk times log2(e) (the per-token or
// chunk-local cumulative log2 gate of the `recurrent_kda` / `chunk_kda`
// contract in "kda in torchtitan (training)").
//
// HBM-bound elementwise + segmented scan. Each thread owns VEC consecutive
// floats of a token row (HV*K floats) and walks TILE tokens in order, so a
// wave reads 64*VEC*4 contiguous bytes per token. Chunks tile each sequence
// from its own first token, so a tile may start inside a chunk: the thread
// then first sums the chunk's earlier tokens (at most chunk-1 of them).
#include "kda_common.h"

namespace kda {

constexpr int kGateTile = 64;
constexpr int kGateThreads = 256;

constexpr float kLn2 = 0.6931471805599453f;

// softplus(x) = ln(1 + e^x) = max(x, 0) + ln(1 + z), z = e^{-|x|} in (0, 1],
// on the transcendental unit. ln(1 + z) uses the classic correction
// ln(u) * z / (u - 1) with u = 1 + z (u - 1 is exact), which keeps full
// relative accuracy for small z. Above 20 the result is x itself.
__device__ __forceinline__ float softplus_f32(float x) {
  if (x > 20.f) return x;
  const float z = __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e);
  const float u = 1.f + z;
  const float l = (u == 1.f) ? z : __builtin_amdgcn_logf(u) * kLn2 * (z / (u - 1.f));
  return fmaxf(x, 0.f) + l;
}

template <int VEC>
__global__ void __launch_bounds__(kGateThreads)
gate_cumsum_kernel(const float* __restrict__ in, int is_raw, const float* __restrict__ A_log,
                   const int32_t* __restrict__ cu, int N, int T, int64_t n_tok, int HV, int K,
                   int chunk, float* out) {
  __shared__ int64_t s_cstart[kGateTile];  // chunk start of each tile token (-1: outside)
  const int64_t t_a = (int64_t)blockIdx.x * kGateTile;
  const int row = HV * K;
  // per-token chunk start (sequence lookup: dense rows or binary search of cu)
  if (threadIdx.x < kGateTile) {
    int64_t t = t_a + threadIdx.x;
    int64_t cs = -1;
    if (t < n_tok) {
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
  float scale[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    int hv = (f0 + e) / K;
    scale[e] = (is_raw && A_log) ? expf(A_log[hv]) : 1.f;
  }
  auto gate_of = [&](int64_t t, float* g) {
    const float* p = in + t * row + f0;
    float x[VEC];
    if constexpr (VEC == 4) {
      float4 v = *reinterpret_cast<const float4*>(p);
      x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    } else if constexpr (VEC == 2) {
      float2 v = *reinterpret_cast<const float2*>(p);
      x[0] = v.x; x[1] = v.y;
    } else {
      x[0] = *p;
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) g[e] = is_raw ? -scale[e] * softplus_f32(x[e]) : x[e];
  };
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  // carry-in: the tile starts inside a chunk that began earlier
  {
    int64_t cs = s_cstart[0];
    if (cs >= 0 && cs < t_a) {
      for (int64_t t = cs; t < t_a; ++t) {
        float g[VEC];
        gate_of(t, g);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] += g[e];
      }
    }
  }
  // main pass: BATCH tokens of loads in flight, then the scan and the stores
  // (a thread only ever touches its own elements, so in-place per-token use is safe)
  constexpr int BATCH = 16;
  for (int i0 = 0; i0 < kGateTile; i0 += BATCH) {
    float g[BATCH][VEC];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      if (s_cstart[i0 + b] >= 0) gate_of(t_a + i0 + b, g[b]);
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int64_t t = t_a + i0 + b;
      const int64_t cs = s_cstart[i0 + b];
      if (cs < 0) continue;  // outside the tensor or in the capacity tail
      if (cs == t) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
      }
      float r[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        acc[e] += g[b][e];
        r[e] = acc[e] * kLog2e;
      }
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

}  // namespace kda

namespace kda_host {

hipError_t launch_gate(const kda_dims& d, const float* in, int is_raw, const float* A_log,
                       const int32_t* cu, int chunk, float* out, hipStream_t s) {
  const int64_t n_tok = (int64_t)d.B * d.T;
  if (n_tok == 0) return hipSuccess;
  const int row = d.HV * d.K;
  int vec = 1;
  if (row % 4 == 0 && ((uintptr_t)in % 16 == 0) && ((uintptr_t)out % 16 == 0)) vec = 4;
  else if (row % 2 == 0 && ((uintptr_t)in % 8 == 0) && ((uintptr_t)out % 8 == 0)) vec = 2;
  dim3 grid((unsigned)((n_tok + kda::kGateTile - 1) / kda::kGateTile),
            (unsigned)((row / vec + kda::kGateThreads - 1) / kda::kGateThreads));
  dim3 block(kda::kGateThreads);
  if (vec == 4)
    hipLaunchKernelGGL(kda::gate_cumsum_kernel<4>, grid, block, 0, s, in, is_raw, A_log, cu, d.N,
                       d.T, n_tok, d.HV, d.K, chunk, out);
  else if (vec == 2)
    hipLaunchKernelGGL(kda::gate_cumsum_kernel<2>, grid, block, 0, s, in, is_raw, A_log, cu, d.N,
                       d.T, n_tok, d.HV, d.K, chunk, out);
  else
    hipLaunchKernelGGL(kda::gate_cumsum_kernel<1>, grid, block, 0, s, in, is_raw, A_log, cu, d.N,
                       d.T, n_tok, d.HV, d.K, chunk, out);
  return hipGetLastError();
}

}  // namespace kda_host
