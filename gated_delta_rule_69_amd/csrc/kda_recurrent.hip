// Step A7: token-sequential KDA scan (recurrent_kda), FP32 compute.
//
// Per token, with the per-token log2 gate (the `recurrent_kda` gate contract
// in "kda in torchtitan (training)", quoted attention-gym description):
//   S' = Diag(2^gate) S;  u = S'^T k;  w = S'^T q~;  delta = beta (v - u)
//   o  = w + delta (k . q~);  S = S' + k delta^T
// which is S_t = (I - beta k k^T) Diag(2^gate) S_{t-1} + beta k v^T and
// o_t = S_t^T q~ with q~ = q / sqrt(K), evaluated in one pass over S.
//
// One workgroup per (sequence, value head, V block). The K x BV block of S
// lives in registers: a thread owns VEC adjacent columns of ROWS rows
// (rows rg, rg + RG, ...), so every wave touches whole contiguous row
// segments of the state (coalesced 16-byte accesses for VEC = 4). The state
// is read once and written once; for decode (one token per sequence) the
// kernel is HBM-bound on those two passes. The reductions over K (u, w and
// k . q~) go through LDS.
#include "kda_common.h"

namespace kda {

constexpr int kRecThreads = 256;

template <int VEC>
struct VecF;
template <>
struct VecF<4> {
  static __device__ __forceinline__ void ld(const float* p, float* x) {
    float4 v = *reinterpret_cast<const float4*>(p);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  }
  static __device__ __forceinline__ void st(float* p, const float* x) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  }
};
template <>
struct VecF<2> {
  static __device__ __forceinline__ void ld(const float* p, float* x) {
    float2 v = *reinterpret_cast<const float2*>(p);
    x[0] = v.x; x[1] = v.y;
  }
  static __device__ __forceinline__ void st(float* p, const float* x) {
    *reinterpret_cast<float2*>(p) = make_float2(x[0], x[1]);
  }
};
template <>
struct VecF<1> {
  static __device__ __forceinline__ void ld(const float* p, float* x) { x[0] = *p; }
  static __device__ __forceinline__ void st(float* p, const float* x) { *p = x[0]; }
};

template <typename T, int VEC, int ROWS>
__global__ void __launch_bounds__(kRecThreads)
recurrent_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                 const float* __restrict__ gate, const T* __restrict__ beta,
                 const float* h0, const int32_t* __restrict__ cu, int Tlen, int H, int HV, int K,
                 int V, int BV, float scale, int write_final, T* __restrict__ o, float* ht) {
  extern __shared__ float smem[];
  // LDS: k[K], q~[K], decay[K], then partials [RG][TPR][2*VEC+1], then delta/final [BV]
  float* s_k = smem;
  float* s_q = s_k + K;
  float* s_d = s_q + K;
  float* s_part = s_d + K;

  const int TPR = BV / VEC;
  const int RG = kRecThreads / TPR;
  const int tid = threadIdx.x;
  const int cg = tid % TPR;
  const int rg = tid / TPR;
  const bool active = rg < RG;
  const int n = blockIdx.x / HV;
  const int hv = blockIdx.x % HV;
  const int h = hv / (HV / H);
  const int col0 = blockIdx.y * BV + cg * VEC;
  const bool col_ok = active && col0 < V;  // V % VEC == 0, so the whole vector is in range
  float* s_fin = s_part + (size_t)RG * TPR * (2 * VEC + 1);

  int64_t bos;
  int len;
  seq_range(cu, n, Tlen, &bos, &len);
  const size_t st_base = ((size_t)n * HV + hv) * (size_t)K * V;

  if (len == 0) {
    // empty slot: bitwise passthrough of the state (or +0.0 without one)
    if (!write_final || (h0 == ht && h0 != nullptr)) return;
    const int64_t KV = (int64_t)K * V;
    const int64_t c0 = (int64_t)blockIdx.y * BV;
    for (int64_t e = tid; e < (int64_t)K * BV; e += kRecThreads) {
      int64_t r = e / BV, c = c0 + e % BV;
      if (c >= V) continue;
      const int64_t off = r * V + c;
      uint32_t bits = h0 ? reinterpret_cast<const uint32_t*>(h0 + st_base)[off] : 0u;
      reinterpret_cast<uint32_t*>(ht + st_base)[off] = bits;
    }
    (void)KV;
    return;
  }

  float s[ROWS][VEC];
#pragma unroll
  for (int i = 0; i < ROWS; ++i) {
    const int r = rg + RG * i;
#pragma unroll
    for (int e = 0; e < VEC; ++e) s[i][e] = 0.f;
    if (h0 && col_ok && r < K) VecF<VEC>::ld(h0 + st_base + (size_t)r * V + col0, s[i]);
  }

  for (int it = 0; it < len; ++it) {
    const int64_t t = bos + it;
    __syncthreads();  // previous token's LDS reads are done
    for (int c = tid; c < K; c += kRecThreads) {
      s_k[c] = to_f32(k[(t * H + h) * K + c]);
      s_q[c] = to_f32(q[(t * H + h) * K + c]) * scale;
      s_d[c] = exp2f(gate[(t * HV + hv) * K + c]);
    }
    __syncthreads();
    float pu[VEC], pw[VEC], pkq = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) pu[e] = pw[e] = 0.f;
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
      const int r = rg + RG * i;
      if (r < K) {
        const float d = s_d[r], kr = s_k[r], qr = s_q[r];
        pkq += kr * qr;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          s[i][e] *= d;
          pu[e] += s[i][e] * kr;
          pw[e] += s[i][e] * qr;
        }
      }
    }
    if (active) {
      float* p = s_part + ((size_t)rg * TPR + cg) * (2 * VEC + 1);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        p[e] = pu[e];
        p[VEC + e] = pw[e];
      }
      p[2 * VEC] = pkq;
    }
    __syncthreads();
    if (tid < TPR && col0 < V) {
      float u[VEC], w[VEC], kq = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) u[e] = w[e] = 0.f;
      for (int g = 0; g < RG; ++g) {
        const float* p = s_part + ((size_t)g * TPR + cg) * (2 * VEC + 1);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          u[e] += p[e];
          w[e] += p[VEC + e];
        }
        kq += p[2 * VEC];
      }
      const float b = to_f32(beta[t * HV + hv]);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float vv = to_f32(v[(t * HV + hv) * V + col0 + e]);
        const float dl = b * (vv - u[e]);
        s_fin[cg * VEC + e] = dl;
        o[(t * HV + hv) * V + col0 + e] = from_f32<T>(w[e] + dl * kq);
      }
    }
    __syncthreads();
    if (col_ok) {
      float dl[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) dl[e] = s_fin[cg * VEC + e];
#pragma unroll
      for (int i = 0; i < ROWS; ++i) {
        const int r = rg + RG * i;
        if (r < K) {
          const float kr = s_k[r];
#pragma unroll
          for (int e = 0; e < VEC; ++e) s[i][e] += kr * dl[e];
        }
      }
    }
  }
  if (write_final && col_ok) {
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
      const int r = rg + RG * i;
      if (r < K) VecF<VEC>::st(ht + st_base + (size_t)r * V + col0, s[i]);
    }
  }
}

template <typename T, int VEC, int ROWS>
static hipError_t launch_rec_t(const kda_dims& d, const void* q, const void* k, const void* v,
                               const float* gate, const void* beta, const float* h0,
                               const int32_t* cu, int write_final, void* o, float* ht, int BV,
                               hipStream_t s) {
  const int TPR = BV / VEC, RG = kRecThreads / TPR;
  size_t lds = sizeof(float) * (3 * (size_t)d.K + (size_t)RG * TPR * (2 * VEC + 1) + BV);
  dim3 grid((unsigned)(d.N * d.HV), (unsigned)((d.V + BV - 1) / BV));
  hipLaunchKernelGGL((recurrent_kernel<T, VEC, ROWS>), grid, dim3(kRecThreads), lds, s,
                     (const T*)q, (const T*)k, (const T*)v, gate, (const T*)beta, h0, cu, d.T,
                     d.H, d.HV, d.K, d.V, BV, 1.0f / sqrtf((float)d.K), write_final, (T*)o, ht);
  return hipGetLastError();
}

template <typename T, int VEC>
static hipError_t launch_rec_v(const kda_dims& d, const void* q, const void* k, const void* v,
                               const float* gate, const void* beta, const float* h0,
                               const int32_t* cu, int write_final, void* o, float* ht,
                               hipStream_t s) {
  // columns per workgroup: 32 threads per row segment, at most 128 columns
  int BV = 32 * VEC;
  if (BV > d.V) BV = ((d.V + VEC - 1) / VEC) * VEC;
  const int TPR = BV / VEC, RG = kRecThreads / TPR;
  const int rows = (d.K + RG - 1) / RG;
  if (rows <= 4) return launch_rec_t<T, VEC, 4>(d, q, k, v, gate, beta, h0, cu, write_final, o, ht, BV, s);
  if (rows <= 8) return launch_rec_t<T, VEC, 8>(d, q, k, v, gate, beta, h0, cu, write_final, o, ht, BV, s);
  if (rows <= 16) return launch_rec_t<T, VEC, 16>(d, q, k, v, gate, beta, h0, cu, write_final, o, ht, BV, s);
  return launch_rec_t<T, VEC, 32>(d, q, k, v, gate, beta, h0, cu, write_final, o, ht, BV, s);
}

}  // namespace kda

namespace kda_host {

hipError_t launch_recurrent(const kda_dims& d, kda_dtype dt, const void* q, const void* k,
                            const void* v, const float* gate, const void* beta,
                            const float* h0, const int32_t* cu, int write_final, void* o,
                            float* ht, hipStream_t s) {
  if (d.N == 0) return hipSuccess;
  const bool st_al16 = ((uintptr_t)h0 % 16 == 0) && ((uintptr_t)ht % 16 == 0);
  const int vec = (d.V % 4 == 0 && st_al16) ? 4 : (d.V % 2 == 0 ? 2 : 1);
  if (dt == KDA_BF16) {
    if (vec == 4) return kda::launch_rec_v<kda::bf16, 4>(d, q, k, v, gate, beta, h0, cu, write_final, o, ht, s);
    if (vec == 2) return kda::launch_rec_v<kda::bf16, 2>(d, q, k, v, gate, beta, h0, cu, write_final, o, ht, s);
    return kda::launch_rec_v<kda::bf16, 1>(d, q, k, v, gate, beta, h0, cu, write_final, o, ht, s);
  }
  if (vec == 4) return kda::launch_rec_v<float, 4>(d, q, k, v, gate, beta, h0, cu, write_final, o, ht, s);
  if (vec == 2) return kda::launch_rec_v<float, 2>(d, q, k, v, gate, beta, h0, cu, write_final, o, ht, s);
  return kda::launch_rec_v<float, 1>(d, q, k, v, gate, beta, h0, cu, write_final, o, ht, s);
}

}  // namespace kda_host
