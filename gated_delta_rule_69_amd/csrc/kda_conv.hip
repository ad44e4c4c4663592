// Standalone short causal convolution + SiLU of q, k and v with a carried
// per-sequence history (the pre-processing step the pages import next to the
// KDA op as ShortConvolution / causal_conv1d_silu; no formula is printed
// there). Decode continues each sequence's filter from the last W - 1 raw
// inputs of its previous segment; a prefill hands that history over.
//
// One thread per (sequence, 16-byte channel unit) of the concatenated channel
// space [q (H*K) | k (H*K) | v (HV*V)]: it walks the sequence's tokens in order
// with the last W - 1 raw rows in registers, so the history it reads at the
// start and writes at the end is its own (in-place update is race-free).
#include "kda_common.h"

namespace kda {
namespace {

constexpr int kConvThreads = 256;

// Element e of a 16-byte unit of T values, as float.
template <typename T>
__device__ __forceinline__ float elem(const uint4& u, int e) {
  return to_f32(reinterpret_cast<const T*>(&u)[e]);
}

template <typename T, bool OUT>
__global__ void __launch_bounds__(kConvThreads)
short_conv_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                  kda_short_conv conv, const int32_t* __restrict__ cu, int N, int T_, int H, int HV,
                  int K, int V, const T* st_in, T* st_out, T* __restrict__ qo, T* __restrict__ ko,
                  T* __restrict__ vo) {
  constexpr int EPU = 16 / (int)sizeof(T), MW = kConvMaxWidth;
  const int HK = H * K, D = 2 * HK + HV * V, units = D / EPU;
  const int64_t gid = (int64_t)blockIdx.x * kConvThreads + threadIdx.x;
  if (gid >= (int64_t)N * units) return;
  const int n = (int)(gid / units), c0 = (int)(gid % units) * EPU;
  const int W = conv.width;

  // which tensor the unit belongs to, its channel there and its row stride
  const T* src;
  T* dst;
  const float* w;
  const float* b;
  int cc, stride;
  if (c0 < HK) {
    src = q; dst = qo; w = conv.q_weight; b = conv.q_bias; cc = c0; stride = HK;
  } else if (c0 < 2 * HK) {
    src = k; dst = ko; w = conv.k_weight; b = conv.k_bias; cc = c0 - HK; stride = HK;
  } else {
    src = v; dst = vo; w = conv.v_weight; b = conv.v_bias; cc = c0 - 2 * HK; stride = HV * V;
  }

  int64_t bos;
  int len;
  seq_range(cu, n, T_, &bos, &len);

  // hx[s - 1]: raw row s positions back (history rows are oldest first)
  uint4 hx[MW - 1];
  const size_t st_row = (size_t)D, st_base = (size_t)n * (W - 1) * st_row + c0;
#pragma unroll
  for (int s = 1; s < MW; ++s) {
    hx[s - 1] = make_uint4(0, 0, 0, 0);
    if (s < W && st_in)
      hx[s - 1] = *reinterpret_cast<const uint4*>(st_in + st_base + (size_t)(W - 1 - s) * st_row);
  }

  if (OUT) {
    // taps by distance (zero beyond W) and the bias of the unit's channels
    float ws[EPU][MW], bb[EPU];
    const float* wc = w + (size_t)cc * W;  // the unit's EPU x W taps are contiguous
    if (W == MW && ((uintptr_t)wc & 15) == 0) {
#pragma unroll
      for (int e = 0; e < EPU; ++e) {
        const float4 t = *reinterpret_cast<const float4*>(wc + e * MW);
        ws[e][0] = t.w;
        ws[e][1] = t.z;
        ws[e][2] = t.y;
        ws[e][3] = t.x;
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPU; ++e)
#pragma unroll
        for (int s = 0; s < MW; ++s) ws[e][s] = s < W ? wc[e * W + (W - 1 - s)] : 0.f;
    }
    if (b && ((uintptr_t)(b + cc) & 15) == 0) {
#pragma unroll
      for (int e = 0; e < EPU; e += 4) {
        const float4 t = *reinterpret_cast<const float4*>(b + cc + e);
        bb[e] = t.x;
        bb[e + 1] = t.y;
        bb[e + 2] = t.z;
        bb[e + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPU; ++e) bb[e] = b ? b[cc + e] : 0.f;
    }
    for (int i = 0; i < len; ++i) {
      const int64_t t = bos + i;
      const uint4 x = *reinterpret_cast<const uint4*>(src + t * stride + cc);
      union {
        T t[EPU];
        uint4 u;
      } y;
#pragma unroll
      for (int e = 0; e < EPU; ++e) {
        // oldest tap first, from the bias, as the chunked kernel sums
        float z = bb[e];
#pragma unroll
        for (int s = MW - 1; s >= 1; --s) z = fmaf(ws[e][s], elem<T>(hx[s - 1], e), z);
        z = fmaf(ws[e][0], elem<T>(x, e), z);
        y.t[e] = from_f32<T>(z * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-z * kLog2e)));
      }
      *reinterpret_cast<uint4*>(dst + t * stride + cc) = y.u;
#pragma unroll
      for (int s = MW - 1; s >= 2; --s) hx[s - 1] = hx[s - 2];
      hx[0] = x;
    }
  } else {
    // history only: the last W - 1 inputs, reaching back into the carried rows
    const int i0 = len > W - 1 ? len - (W - 1) : 0;
    for (int i = i0; i < len; ++i) {
      const uint4 x = *reinterpret_cast<const uint4*>(src + (bos + i) * stride + cc);
#pragma unroll
      for (int s = MW - 1; s >= 2; --s) hx[s - 1] = hx[s - 2];
      hx[0] = x;
    }
  }

  if (st_out) {
#pragma unroll
    for (int s = 1; s < MW; ++s)
      if (s < W)
        *reinterpret_cast<uint4*>(st_out + st_base + (size_t)(W - 1 - s) * st_row) = hx[s - 1];
  }
}

template <typename T>
hipError_t launch_t(const kda_dims& d, const void* q, const void* k, const void* v,
                    const kda_short_conv& conv, const int32_t* cu, const void* st_in, void* st_out,
                    void* qo, void* ko, void* vo, hipStream_t s) {
  constexpr int EPU = 16 / (int)sizeof(T);
  const int64_t units = (int64_t)(2 * d.H * d.K + d.HV * d.V) / EPU;
  const int64_t threads = (int64_t)d.N * units;
  if (threads == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((threads + kConvThreads - 1) / kConvThreads);
  if (qo) {
    hipLaunchKernelGGL((short_conv_kernel<T, true>), dim3(blocks), dim3(kConvThreads), 0, s,
                       (const T*)q, (const T*)k, (const T*)v, conv, cu, d.N, d.T, d.H, d.HV, d.K,
                       d.V, (const T*)st_in, (T*)st_out, (T*)qo, (T*)ko, (T*)vo);
  } else {
    hipLaunchKernelGGL((short_conv_kernel<T, false>), dim3(blocks), dim3(kConvThreads), 0, s,
                       (const T*)q, (const T*)k, (const T*)v, conv, cu, d.N, d.T, d.H, d.HV, d.K,
                       d.V, (const T*)st_in, (T*)st_out, (T*)nullptr, (T*)nullptr, (T*)nullptr);
  }
  return hipGetLastError();
}

}  // namespace
}  // namespace kda

namespace kda_host {

hipError_t launch_short_conv(const kda_dims& d, kda_dtype dt, const void* q, const void* k,
                             const void* v, const kda_short_conv& conv, const int32_t* cu,
                             const void* st_in, void* st_out, void* qo, void* ko, void* vo,
                             hipStream_t s) {
  if (dt == KDA_BF16)
    return kda::launch_t<kda::bf16>(d, q, k, v, conv, cu, st_in, st_out, qo, ko, vo, s);
  return kda::launch_t<float>(d, q, k, v, conv, cu, st_in, st_out, qo, ko, vo, s);
}

}  // namespace kda_host
