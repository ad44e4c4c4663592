// Shared device helpers for the libkda kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Matrix-core tile traits for a 16x16 output tile with FP32 accumulation.
//
// Fragment layout (checked on gfx950): for a step of KSTEP contraction
// indices, lane l (g = l / 16) feeds row (A) or column (B) l % 16 with PER
// consecutive slots; the accumulator lane l holds rows 4g + i (i = 0..3) of
// column l % 16.
//
// The contraction index carried by slot j of lane group g in step ks is
// kidx(ks, g, j). It is permuted on purpose: with this order the accumulator
// of a product X^T (two stacked 16-row tiles for bf16, one tile for FP32) is
// already the A fragment of X, so results feed the next product without an
// LDS round trip. Both operands of one product always use the same order.
template <typename T>
struct MF;

template <>
struct MF<bf16> {
  static constexpr int KSTEP = 32;
  static constexpr int PER = 8;
  typedef bf16x8 frag;
  static __device__ __forceinline__ int kidx(int ks, int g, int j) {
    return 32 * ks + (j < 4 ? 4 * g + j : 12 + 4 * g + j);
  }
  static __device__ __forceinline__ f32x4 mma(const frag& a, const frag& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ void set(frag& f, int j, float x) { f[j] = (bf16)x; }
  static __device__ __forceinline__ float get(const frag& f, int j) { return (float)f[j]; }
};

struct f32x1 {
  float v;
};

template <>
struct MF<float> {
  static constexpr int KSTEP = 4;
  static constexpr int PER = 1;
  typedef f32x1 frag;
  static __device__ __forceinline__ int kidx(int ks, int g, int /*j*/) {
    return 16 * (ks >> 2) + 4 * g + (ks & 3);
  }
  static __device__ __forceinline__ f32x4 mma(const frag& a, const frag& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a.v, b.v, c, 0, 0, 0);
  }
  static __device__ __forceinline__ void set(frag& f, int, float x) { f.v = x; }
  static __device__ __forceinline__ float get(const frag& f, int) { return f.v; }
};

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

constexpr float kLn2 = 0.6931471805599453f;

// softplus(x) = ln(1 + e^x) = max(x, 0) + ln(1 + z), z = e^{-|x|} in (0, 1],
// on the transcendental unit. With u = 1 + z rounded, c = z - (u - 1) is the
// exact rounding error of that sum (Dekker's Fast2Sum, since 1 >= z), so
// 1 + z = u + c exactly and ln(1 + z) = ln(u) + ln(1 + c / u); as |c| <= 2^-24,
// the second term is c to within |c| (u - 1) / u, a relative 2^-24 of the
// result. This keeps full relative accuracy for small z (where u rounds to 1,
// the result is z itself) with one logarithm and no division. Above 20 the
// result is x itself (z is below half an ulp of x). Branch-free, so loads
// around it can stay batched. No FMA contraction, so every kernel that inlines
// it rounds the same way.
__device__ __forceinline__ float softplus_f32(float x) {
#pragma clang fp contract(off)
  const float z = __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e);
  const float u = 1.f + z;
  const float l = __builtin_amdgcn_logf(u) * kLn2 + (z - (u - 1.f));
  return fmaxf(x, 0.f) + l;
}

// d softplus_f32 / dx = 1 / (1 + e^-x), exactly 1 above 20 (where softplus_f32 is x)
__device__ __forceinline__ float sigmoid_f32(float x) {
#pragma clang fp contract(off)
  const float z = __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e);
  const float r = (x >= 0.f ? 1.f : z) / (1.f + z);
  return x > 20.f ? 1.f : r;
}

// Widest short convolution the fused pre-processing accepts (taps per channel).
constexpr int kConvMaxWidth = 4;

// Optional q/k normalisation: x / sqrt(sum over K of x^2 + kL2NormEps) per
// (token, qk head), before any use of q and k.
constexpr float kL2NormEps = 1e-6f;
__device__ __forceinline__ float l2norm_inv(float sum_sq) {
#pragma clang fp contract(off)
  return 1.f / sqrtf(sum_sq + kL2NormEps);
}

// What a scan kernel's gate operand holds:
//   kGateLog2: the log2 gate already prepared (per token for the recurrent
//              scan, chunk-local inclusive cumsum G2 for the chunked scan);
//   kGateLog:  the per-token natural-log gate g;
//   kGateRaw:  the pre-activation x, with g = -exp(A_log[hv]) softplus(x)
//              (unit scale without A_log).
// The two last modes fuse the gate step into the scan; the arithmetic is the
// one of the gate kernel, so fused and two-step results agree bit for bit.
enum GateMode : int { kGateLog2 = 0, kGateLog = 1, kGateRaw = 2 };

// Summation order of the chunk-local cumsum (shared by the gate kernel and the
// fused-gate chunk kernel, so both round identically): inside a chunk, tokens
// form blocks of kGateBlock from the chunk's first token; token t at position
// m of block b gets (C_b + P_m) * log2(e), where P_m sums the block's tokens
// 0..m in order and C_b sums the totals of blocks 0..b-1 in order (C_0 = 0).
constexpr int kGateBlock = 8;

__device__ __forceinline__ float gate_head_scale(int mode, const float* A_log, int hv) {
  return (mode == kGateRaw && A_log) ? expf(A_log[hv]) : 1.f;
}
// natural-log gate g of one element (modes kGateLog and kGateRaw)
__device__ __forceinline__ float gate_nat(float x, int mode, float scale) {
#pragma clang fp contract(off)
  return mode == kGateRaw ? -scale * softplus_f32(x) : x;
}
// per-token log2 gate of one element, as the gate kernel writes it with chunk 1
__device__ __forceinline__ float gate_log2_token(float x, int mode, float scale) {
#pragma clang fp contract(off)
  return mode == kGateLog2 ? x : (0.f + gate_nat(x, mode, scale)) * kLog2e;
}

// Flat offset of the first token of dense/varlen sequence n, and its length.
__device__ __forceinline__ void seq_range(const int32_t* cu, int n, int T, int64_t* bos, int* len) {
  if (cu) {
    int a = cu[n], b = cu[n + 1];
    *bos = a;
    *len = b - a;
  } else {
    *bos = (int64_t)n * T;
    *len = T;
  }
}

}  // namespace kda

// Host-side launchers (defined in the .hip files, called by the C ABI).
namespace kda_host {
// Compute units of the calling thread's current device (256 on MI355X), for
// launch shapes that must give every compute unit a workgroup.
inline int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}
hipError_t launch_gate(const kda_dims& d, const float* in, int is_raw, const float* A_log,
                       const float* dt_bias, const int32_t* cu, int chunk, float* out,
                       hipStream_t s);
// Gate backward: dx and, when dA_log / d_dt_bias are requested, FP32 partials
// per token block in `ws` reduced in a fixed order.
size_t gate_bwd_ws_bytes(const kda_dims& d);
hipError_t launch_gate_bwd(const kda_dims& d, const float* x, const float* A_log,
                           const float* dt_bias, const float* dg, const int32_t* cu, float* dx,
                           float* dA_log, float* d_dt_bias, void* ws, hipStream_t s);
hipError_t launch_recurrent(const kda_dims& d, kda_dtype dt, const void* q, const void* k,
                            const void* v, const float* gate, int gate_mode, const float* A_log,
                            int qk_norm, const void* beta, const float* h0, const int32_t* cu,
                            int write_final, void* o, float* ht, hipStream_t s);
hipError_t launch_short_conv(const kda_dims& d, kda_dtype dt, const void* q, const void* k,
                             const void* v, const kda_short_conv& conv, const int32_t* cu,
                             const void* st_in, void* st_out, void* qo, void* ko, void* vo,
                             hipStream_t s);
size_t chunk_workspace_bytes(const kda_dims& d, kda_dtype dt, int chunk);
hipError_t launch_chunk_fwd(const kda_dims& d, kda_dtype dt, const void* q, const void* k,
                            const void* v, const float* gate, int gate_mode, const float* A_log,
                            int qk_norm, const kda_short_conv* conv, const void* beta,
                            const float* h0, const int32_t* cu, int write_final, void* o,
                            float* ht, void* ws, size_t ws_bytes, int save, hipStream_t s);
size_t chunk_bwd_workspace_bytes(const kda_dims& d, kda_dtype dt, int chunk);
hipError_t launch_chunk_bwd(const kda_dims& d, kda_dtype dt, const void* q, const void* k,
                            const void* v, const float* gate, int gate_mode, const float* A_log,
                            const void* beta, const float* h0,
                            const int32_t* cu, const void* dO, const float* dht, void* dq,
                            void* dk, void* dv, float* dg, void* dbeta, float* dh0, void* ws,
                            int saved, hipStream_t s);
}  // namespace kda_host
