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
#include <type_traits>

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
                 const float* __restrict__ gate, int gate_mode, const float* __restrict__ A_log,
                 int qk_norm, const T* __restrict__ beta,
                 const float* h0, const int32_t* __restrict__ cu, int Tlen, int H, int HV, int K,
                 int V, int BV, float scale, int write_final, T* __restrict__ o, float* ht) {
  extern __shared__ float smem[];
  // LDS: k[K], q~[K], decay[K], then partials [RG][TPR][PW], then delta/final [BV]
  constexpr int PW = 2 * VEC + 3;  // u, w, k.q~, |k|^2, |q~|^2
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
  float* s_fin = s_part + (size_t)RG * TPR * PW;

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

  const float gscale = gate_head_scale(gate_mode, A_log, hv);
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
      s_d[c] = exp2f(gate_log2_token(gate[(t * HV + hv) * K + c], gate_mode, gscale));
    }
    __syncthreads();
    float pu[VEC], pw[VEC], pkq = 0.f, pkk = 0.f, pqq = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) pu[e] = pw[e] = 0.f;
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
      const int r = rg + RG * i;
      if (r < K) {
        const float d = s_d[r], kr = s_k[r], qr = s_q[r];
        pkq += kr * qr;
        pkk += kr * kr;  // row norms: one thread per row group counts them (cg == 0)
        pqq += qr * qr;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          s[i][e] *= d;
          pu[e] += s[i][e] * kr;
          pw[e] += s[i][e] * qr;
        }
      }
    }
    if (active) {
      float* p = s_part + ((size_t)rg * TPR + cg) * PW;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        p[e] = pu[e];
        p[VEC + e] = pw[e];
      }
      p[2 * VEC] = pkq;
      p[2 * VEC + 1] = pkk;
      p[2 * VEC + 2] = pqq;
    }
    __syncthreads();
    if (tid < TPR && col0 < V) {
      float u[VEC], w[VEC], kq = 0.f, kk = 0.f, qq = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) u[e] = w[e] = 0.f;
      for (int g = 0; g < RG; ++g) {
        const float* p = s_part + ((size_t)g * TPR + cg) * PW;
        const float* p0 = s_part + ((size_t)g * TPR) * PW;  // column group 0 of the row group
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          u[e] += p[e];
          w[e] += p[VEC + e];
        }
        kq += p[2 * VEC];
        kk += p0[2 * VEC + 1];
        qq += p0[2 * VEC + 2];
      }
      // optional q/k normalisation (q~ = q * scale, so |q|^2 = |q~|^2 / scale^2)
      float rk = 1.f;
      if (qk_norm) {
        rk = l2norm_inv(kk);
        const float rq = l2norm_inv(qq / (scale * scale));
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          u[e] *= rk;
          w[e] *= rq;
        }
        kq *= rk * rq;
      }
      const float b = to_f32(beta[t * HV + hv]);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float vv = to_f32(v[(t * HV + hv) * V + col0 + e]);
        const float dl = b * (vv - u[e]);
        s_fin[cg * VEC + e] = dl * rk;  // the update takes the normalised k
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

// Wave-per-column-block form for K in {64, 128, 256}, V % 4 == 0 and 16-byte
// aligned operands (the common case, and the decode hot path).
//
// Each 64-lane wave owns all K rows of a CW-column block of one (sequence,
// value head) state; a lane holds RPL rows of CPL consecutive columns. The
// reductions over K are RPL-term partial sums followed by a sum over the RL
// lanes holding the other rows of the same columns, so every lane ends with
// u, w and k . q~ of its columns and computes delta redundantly: no LDS and no
// barrier. Waves are independent. Two layouts:
//   MANY (many chains, e.g. decode): RPL = 16, CPL = 4, lane = rl * CL + cl;
//     the row sums are a butterfly of lane shuffles (xor CL, 2 CL, ..., 32),
//     and the 16 decays of a row group are split over its CL lanes (NPL each,
//     activation included for a fused gate) and gathered with shuffles. The
//     next token's inputs are loaded while the current one is processed (two
//     register sets). Fewest redundant k / q loads for a bandwidth-bound pass.
//   FEW (fewer waves than SIMDs): RPL = 2 (4 for K = 256), CPL = 1, RL = K / RPL
//     consecutive row lanes, lane = cl * RL + rl, 2 / 1 / 1 columns per wave
//     for K = 64 / 128 / 256; the row sums are lane_group_sum, and every lane
//     activates its own RPL decays. A token costs a lane 2 (4) state updates
//     and three row sums (u, w, k . q~) instead of 64 updates, and a chain
//     spreads over 32 to 128 times as many waves: the shortest sequential chain
//     per token. Measured against 4 columns per lane: 50 -> 36 us on the tiny
//     FP32 case, 3.49 -> 2.49 ms on one 4096-token bf16 sequence with 16 heads
//     (2 columns: 42 us, 2.68 ms); 2 rows per lane beat 4 by 10% at 4 columns.
constexpr int kFewCols = 1;  // state columns per lane in the FEW form

template <int K, bool FEW>
struct WaveGeo {
  static constexpr int RPL = FEW ? K / 64 : 16;  // state rows per lane
  static constexpr int CPL = FEW ? kFewCols : 4;  // state columns per lane
  static constexpr int RL = K / RPL;             // row lanes
  static constexpr int CL = 64 / RL;             // column lanes (CPL columns each)
  static constexpr int CW = CPL * CL;            // columns per wave
  static constexpr int NPL = RPL / CL;           // decays activated per lane (MANY)
  static_assert(RL * CL == 64 && (FEW || (NPL >= 1 && RPL % CL == 0)), "wave geometry");
};

// Sum of x over aligned groups of RL consecutive lanes (RL = 16, 32 or 64),
// left in every lane of the group: four rotations inside each 16-lane row (DPP
// row_ror 1, 2, 4, 8), then for RL >= 32 the row-pair swap and for RL = 64 the
// half-wave swap (v_permlane16_swap / v_permlane32_swap, which exchange rows
// between two registers holding copies of x: their sum is x plus the value of
// the lane 16, resp. 32, lanes away). All VALU: no LDS round trip per step, as
// a shuffle through ds_bpermute would take. The swaps are written out because
// the compiler's two-result form of them loses the second result; the s_nop
// pairs give the two wait states a VALU result needs before a permlane reads
// it, and the same after.
template <int M>
__device__ __forceinline__ float add_row_ror(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                 0, __builtin_bit_cast(int, x), 0x120 + M, 0xF, 0xF, false));
}
__device__ __forceinline__ float add_swap16(float x) {
  unsigned a = __builtin_bit_cast(unsigned, x), b = a;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}
__device__ __forceinline__ float add_swap32(float x) {
  unsigned a = __builtin_bit_cast(unsigned, x), b = a;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}
template <int RL>
__device__ __forceinline__ float lane_group_sum(float x) {
  static_assert(RL == 16 || RL == 32 || RL == 64, "row lanes");
  x = add_row_ror<1>(x);
  x = add_row_ror<2>(x);
  x = add_row_ror<4>(x);
  x = add_row_ror<8>(x);
  if constexpr (RL >= 32) x = add_swap16(x);
  if constexpr (RL == 64) x = add_swap32(x);
  return x;
}

template <int NPL>
struct GVec;  // the NPL gate values of one lane
template <>
struct GVec<1> { float x[1]; };
template <>
struct GVec<2> { float2 v; };
template <>
struct GVec<4> { float4 v; };
template <>
struct GVec<8> { float4 v[2]; };
template <>
struct GVec<16> { float4 v[4]; };

// RPL consecutive elements of T as one or more vector loads of exactly BYTES
// bytes in all (4, 8 or a multiple of 16)
template <int BYTES>
struct RowVec {
  static_assert(BYTES == 2 || BYTES == 4 || BYTES == 8 || BYTES % 16 == 0, "row vector size");
  static constexpr int N = BYTES >= 16 ? BYTES / 16 : 1;
  typedef typename std::conditional<
      BYTES >= 16, uint4,
      typename std::conditional<BYTES == 8, uint2,
                                typename std::conditional<BYTES == 4, uint32_t, uint16_t>::type>::type>::type U;
  U u[N];
};

// CPL consecutive FP32 state elements as one vector (one 4-, 8- or 16-byte access)
template <int CPL>
struct StVec;
template <>
struct StVec<1> { typedef float type; typedef uint32_t bits; };
template <>
struct StVec<2> { typedef float __attribute__((ext_vector_type(2))) type; typedef uint32_t __attribute__((ext_vector_type(2))) bits; };
template <>
struct StVec<4> { typedef f32x4 type; typedef u32x4 bits; };
template <int CPL>
__device__ __forceinline__ float st_get(const typename StVec<CPL>::type& x, int e) {
  if constexpr (CPL == 1) return x;
  else return x[e];
}
template <int CPL>
__device__ __forceinline__ typename StVec<CPL>::type st_make(const float* r) {
  typename StVec<CPL>::type x;
  if constexpr (CPL == 1) {
    x = r[0];
  } else {
#pragma unroll
    for (int e = 0; e < CPL; ++e) x[e] = r[e];
  }
  return x;
}

template <typename T, int NPL, int RPL, int CPL>
struct WTok {  // one token's inputs for one lane (RPL rows of k and q, NPL gates, CPL of v)
  RowVec<RPL * (int)sizeof(T)> k, q;
  GVec<NPL> g;
  RowVec<CPL * (int)sizeof(T)> v;
  T b;
};

template <typename T, int NPL, int RPL, int CPL>
__device__ __forceinline__ void unpack_rows(const WTok<T, NPL, RPL, CPL>& x, float* kf, float* qf) {
  const T* kk = reinterpret_cast<const T*>(x.k.u);
  const T* qq = reinterpret_cast<const T*>(x.q.u);
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    kf[i] = to_f32(kk[i]);
    qf[i] = to_f32(qq[i]);
  }
}
template <typename T, int NPL, int RPL, int CPL>
__device__ __forceinline__ void unpack_v(const WTok<T, NPL, RPL, CPL>& x, float* vf) {
  const T* vv = reinterpret_cast<const T*>(x.v.u);
#pragma unroll
  for (int e = 0; e < CPL; ++e) vf[e] = to_f32(vv[e]);
}
// CPL output values as one store
template <int CPL>
__device__ __forceinline__ void store_o(bf16* p, const float* r) {
  if constexpr (CPL == 4) {
    bf16x4 t = {(bf16)r[0], (bf16)r[1], (bf16)r[2], (bf16)r[3]};
    *reinterpret_cast<bf16x4*>(p) = t;
  } else if constexpr (CPL == 2) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 t = {(bf16)r[0], (bf16)r[1]};
    *reinterpret_cast<bf16x2*>(p) = t;
  } else {
    *p = (bf16)r[0];
  }
}
template <int CPL>
__device__ __forceinline__ void store_o(float* p, const float* r) {
  *reinterpret_cast<typename StVec<CPL>::type*>(p) = st_make<CPL>(r);
}

template <typename T, int K, bool FEW>
__global__ void __launch_bounds__(kRecThreads)
recurrent_wave_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                      const float* __restrict__ gate, int gate_mode,
                      const float* __restrict__ A_log, int qk_norm, const T* __restrict__ beta,
                      const float* h0, const int32_t* __restrict__ cu, int Tlen, int H, int HV,
                      int V, int n_cb, int64_t n_tasks, float scale, int write_final,
                      T* __restrict__ o, float* ht) {
  using G = WaveGeo<K, FEW>;
  constexpr int RPL = G::RPL, CL = G::CL, CW = G::CW, NPL = G::NPL, CPL = G::CPL;
  constexpr int GPL = FEW ? RPL : NPL;  // gate values loaded (and activated) per lane
  using Tok = WTok<T, GPL, RPL, CPL>;
  using SV = typename StVec<CPL>::type;
  using SB = typename StVec<CPL>::bits;
  const int64_t task = (int64_t)blockIdx.x * (kRecThreads / 64) + (threadIdx.x >> 6);
  if (task >= n_tasks) return;  // whole wave
  const int lane = threadIdx.x & 63;
  const int cb = (int)(task % n_cb);
  const int64_t nh = task / n_cb;
  const int n = (int)(nh / HV), hv = (int)(nh % HV);
  const int h = hv / (HV / H);
  const int rl = FEW ? lane % G::RL : lane / CL, cl = FEW ? lane / G::RL : lane % CL;
  const int r0 = rl * RPL;
  const int col = cb * CW + cl * CPL;
  const bool col_ok = col < V;

  int64_t bos;
  int len;
  seq_range(cu, n, Tlen, &bos, &len);
  const size_t st_base = (size_t)nh * K * V + (size_t)r0 * V + col;

  if (len == 0) {
    // empty slot: bitwise passthrough of the state (or +0.0 without one)
    if (!write_final || (h0 == ht && h0 != nullptr) || !col_ok) return;
    SB bits[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i)
      bits[i] = h0 ? __builtin_nontemporal_load(
                         reinterpret_cast<const SB*>(h0 + st_base + (size_t)i * V))
                   : SB(0u);
#pragma unroll
    for (int i = 0; i < RPL; ++i)
      __builtin_nontemporal_store(bits[i], reinterpret_cast<SB*>(ht + st_base + (size_t)i * V));
    return;
  }

  // The state streams through once: non-temporal loads and stores keep it
  // from evicting the small per-token inputs from the caches.
  float s[RPL][CPL];
  if (h0 && col_ok) {
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const SV x =
          __builtin_nontemporal_load(reinterpret_cast<const SV*>(h0 + st_base + (size_t)i * V));
#pragma unroll
      for (int e = 0; e < CPL; ++e) s[i][e] = st_get<CPL>(x, e);
    }
  } else {
#pragma unroll
    for (int i = 0; i < RPL; ++i)
#pragma unroll
      for (int e = 0; e < CPL; ++e) s[i][e] = 0.f;
  }

  const float gscale = gate_head_scale(gate_mode, A_log, hv);
  const int colc = col_ok ? col : 0;  // lanes past V read column 0 and discard it
  auto load_tok = [&](int64_t t, Tok& x) {
    typedef typename decltype(x.k)::U U;
    const U* kp = reinterpret_cast<const U*>(k + (t * H + h) * K + r0);
    const U* qp = reinterpret_cast<const U*>(q + (t * H + h) * K + r0);
#pragma unroll
    for (int j = 0; j < decltype(x.k)::N; ++j) {
      x.k.u[j] = kp[j];
      x.q.u[j] = qp[j];
    }
    x.g = *reinterpret_cast<const GVec<GPL>*>(gate + (t * HV + hv) * K + r0 + (FEW ? 0 : cl * NPL));
    x.v.u[0] = *reinterpret_cast<const typename decltype(x.v)::U*>(v + (t * HV + hv) * V + colc);
    x.b = beta[t * HV + hv];
  };
  auto step = [&](const Tok& x, int64_t t) {
    float kf[RPL], qf[RPL], vf[CPL];
    unpack_rows(x, kf, qf);
    unpack_v(x, vf);
    // this lane's NPL decays (rows r0 + cl * NPL + m), then the row group's 16
    const float* gf = reinterpret_cast<const float*>(&x.g);
    float dloc[GPL];
#pragma unroll
    for (int m = 0; m < GPL; ++m) dloc[m] = exp2f(gate_log2_token(gf[m], gate_mode, gscale));
    float u[CPL], w[CPL], kq = 0.f, kk = 0.f, qq = 0.f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) u[e] = w[e] = 0.f;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const float d = FEW ? dloc[FEW ? i : 0] : __shfl(dloc[i % GPL], rl * CL + i / NPL);
      kk += kf[i] * kf[i];
      qq += qf[i] * qf[i];
      qf[i] *= scale;
      kq += kf[i] * qf[i];
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        s[i][e] *= d;
        u[e] += s[i][e] * kf[i];
        w[e] += s[i][e] * qf[i];
      }
    }
    if constexpr (FEW) {
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        u[e] = lane_group_sum<G::RL>(u[e]);
        w[e] = lane_group_sum<G::RL>(w[e]);
      }
      kq = lane_group_sum<G::RL>(kq);
      if (qk_norm) {
        kk = lane_group_sum<G::RL>(kk);
        qq = lane_group_sum<G::RL>(qq);
      }
    } else {
#pragma unroll
      for (int m = CL; m < 64; m <<= 1) {
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          u[e] += __shfl_xor(u[e], m);
          w[e] += __shfl_xor(w[e], m);
        }
        kq += __shfl_xor(kq, m);
        if (qk_norm) {
          kk += __shfl_xor(kk, m);
          qq += __shfl_xor(qq, m);
        }
      }
    }
    // optional q/k normalisation, applied to the reduced terms (u and the update
    // are linear in k, w in q, k.q~ in both)
    float rk = 1.f;
    if (qk_norm) {
      rk = l2norm_inv(kk);
      const float rq = l2norm_inv(qq);
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        u[e] *= rk;
        w[e] *= rq;
      }
      kq *= rk * rq;
    }
    const float b = to_f32(x.b);
    float dl[CPL], r[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      dl[e] = b * (vf[e] - u[e]);
      r[e] = w[e] + dl[e] * kq;
      dl[e] *= rk;
    }
    if (rl == 0 && col_ok) store_o<CPL>(o + (t * HV + hv) * V + col, r);
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
#pragma unroll
      for (int e = 0; e < CPL; ++e) s[i][e] += kf[i] * dl[e];
    }
  };

  if constexpr (FEW) {
    // a ring of RING token input sets: a token's inputs are requested RING - 1
    // steps before its step (the short per-token chain of this form would
    // otherwise wait on each load); loads past the end re-read the last token
    constexpr int RING = 4;
    Tok ring[RING];
#pragma unroll
    for (int j = 0; j < RING; ++j) load_tok(bos + min(j, len - 1), ring[j]);
    for (int it = 0; it < len; it += RING) {
#pragma unroll
      for (int j = 0; j < RING; ++j) {
        if (it + j < len) step(ring[j], bos + it + j);
        load_tok(bos + min(it + j + RING, len - 1), ring[j]);
      }
    }
  } else {
    Tok A, B;
    load_tok(bos, A);
    for (int it = 0; it < len; it += 2) {
      load_tok(bos + min(it + 1, len - 1), B);
      step(A, bos + it);
      if (it + 1 >= len) break;
      load_tok(bos + min(it + 2, len - 1), A);
      step(B, bos + it + 1);
    }
  }

  if (write_final && col_ok) {
#pragma unroll
    for (int i = 0; i < RPL; ++i)
      __builtin_nontemporal_store(st_make<CPL>(s[i]),
                                  reinterpret_cast<SV*>(ht + st_base + (size_t)i * V));
  }
}

template <typename T, int K, bool FEW>
static hipError_t launch_rec_wave_form(const kda_dims& d, const void* q, const void* k, const void* v,
                                      const float* gate, int gm, const float* A_log, int qn,
                                      const void* beta, const float* h0, const int32_t* cu,
                                      int write_final, void* o, float* ht, hipStream_t s) {
  const int n_cb = (d.V + WaveGeo<K, FEW>::CW - 1) / WaveGeo<K, FEW>::CW;
  const int64_t n_tasks = (int64_t)d.N * d.HV * n_cb;
  const int wpb = kRecThreads / 64;
  dim3 grid((unsigned)((n_tasks + wpb - 1) / wpb));
  hipLaunchKernelGGL((recurrent_wave_kernel<T, K, FEW>), grid, dim3(kRecThreads), 0, s, (const T*)q,
                     (const T*)k, (const T*)v, gate, gm, A_log, qn, (const T*)beta, h0, cu, d.T, d.H,
                     d.HV, d.V, n_cb, n_tasks, 1.0f / sqrtf((float)d.K), write_final, (T*)o, ht);
  return hipGetLastError();
}

// Layout: MANY when its (sequence, value head, column block) waves already give
// every SIMD of the device one wave, else FEW (more waves, shorter per-token
// chain).
template <typename T, int K>
static hipError_t launch_rec_wave(const kda_dims& d, const void* q, const void* k, const void* v,
                                  const float* gate, int gm, const float* A_log, int qn, const void* beta,
                                  const float* h0, const int32_t* cu, int write_final, void* o,
                                  float* ht, hipStream_t s) {
  const int64_t many = (int64_t)d.N * d.HV * ((d.V + WaveGeo<K, false>::CW - 1) / WaveGeo<K, false>::CW);
  if (many >= 4 * (int64_t)kda_host::device_cus())
    return launch_rec_wave_form<T, K, false>(d, q, k, v, gate, gm, A_log, qn, beta, h0, cu, write_final, o, ht, s);
  return launch_rec_wave_form<T, K, true>(d, q, k, v, gate, gm, A_log, qn, beta, h0, cu, write_final, o, ht, s);
}

template <typename T, int VEC, int ROWS>
static hipError_t launch_rec_t(const kda_dims& d, const void* q, const void* k, const void* v,
                               const float* gate, int gm, const float* A_log, int qn, const void* beta,
                               const float* h0,
                               const int32_t* cu, int write_final, void* o, float* ht, int BV,
                               hipStream_t s) {
  const int TPR = BV / VEC, RG = kRecThreads / TPR;
  size_t lds = sizeof(float) * (3 * (size_t)d.K + (size_t)RG * TPR * (2 * VEC + 3) + BV);
  dim3 grid((unsigned)(d.N * d.HV), (unsigned)((d.V + BV - 1) / BV));
  hipLaunchKernelGGL((recurrent_kernel<T, VEC, ROWS>), grid, dim3(kRecThreads), lds, s,
                     (const T*)q, (const T*)k, (const T*)v, gate, gm, A_log, qn, (const T*)beta, h0, cu,
                     d.T,
                     d.H, d.HV, d.K, d.V, BV, 1.0f / sqrtf((float)d.K), write_final, (T*)o, ht);
  return hipGetLastError();
}

template <typename T, int VEC>
static hipError_t launch_rec_v(const kda_dims& d, const void* q, const void* k, const void* v,
                               const float* gate, int gm, const float* A_log, int qn, const void* beta,
                               const float* h0,
                               const int32_t* cu, int write_final, void* o, float* ht,
                               hipStream_t s) {
  // columns per workgroup: 32 threads per row segment, at most 128 columns
  int BV = 32 * VEC;
  if (BV > d.V) BV = ((d.V + VEC - 1) / VEC) * VEC;
  const int TPR = BV / VEC, RG = kRecThreads / TPR;
  const int rows = (d.K + RG - 1) / RG;
  if (rows <= 4) return launch_rec_t<T, VEC, 4>(d, q, k, v, gate, gm, A_log, qn, beta, h0, cu, write_final, o, ht, BV, s);
  if (rows <= 8) return launch_rec_t<T, VEC, 8>(d, q, k, v, gate, gm, A_log, qn, beta, h0, cu, write_final, o, ht, BV, s);
  if (rows <= 16) return launch_rec_t<T, VEC, 16>(d, q, k, v, gate, gm, A_log, qn, beta, h0, cu, write_final, o, ht, BV, s);
  return launch_rec_t<T, VEC, 32>(d, q, k, v, gate, gm, A_log, qn, beta, h0, cu, write_final, o, ht, BV, s);
}

}  // namespace kda

namespace kda_host {

hipError_t launch_recurrent(const kda_dims& d, kda_dtype dt, const void* q, const void* k,
                            const void* v, const float* gate, int gm, const float* A_log,
                            int qn, const void* beta, const float* h0, const int32_t* cu,
                            int write_final, void* o, float* ht, hipStream_t s) {
  if (d.N == 0) return hipSuccess;
  auto al = [](const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; };
  const size_t esz = dt == KDA_BF16 ? 2 : 4;
  const bool wave_ok = (d.K == 64 || d.K == 128 || d.K == 256) && d.V % 4 == 0 && al(q, 16) &&
                       al(k, 16) && al(gate, 16) && al(v, 4 * esz) && al(o, 4 * esz) &&
                       al(h0, 16) && al(ht, 16);
  if (wave_ok) {
#define KDA_REC_WAVE(T_)                                                                     \
  switch (d.K) {                                                                             \
    case 64: return kda::launch_rec_wave<T_, 64>(d, q, k, v, gate, gm, A_log, qn, beta, h0, cu, write_final, o, ht, s);   \
    case 128: return kda::launch_rec_wave<T_, 128>(d, q, k, v, gate, gm, A_log, qn, beta, h0, cu, write_final, o, ht, s); \
    default: return kda::launch_rec_wave<T_, 256>(d, q, k, v, gate, gm, A_log, qn, beta, h0, cu, write_final, o, ht, s);  \
  }
    if (dt == KDA_BF16) {
      KDA_REC_WAVE(kda::bf16)
    } else {
      KDA_REC_WAVE(float)
    }
#undef KDA_REC_WAVE
  }
  const bool st_al16 = ((uintptr_t)h0 % 16 == 0) && ((uintptr_t)ht % 16 == 0);
  const int vec = (d.V % 4 == 0 && st_al16) ? 4 : (d.V % 2 == 0 ? 2 : 1);
  if (dt == KDA_BF16) {
    if (vec == 4) return kda::launch_rec_v<kda::bf16, 4>(d, q, k, v, gate, gm, A_log, qn, beta, h0, cu, write_final, o, ht, s);
    if (vec == 2) return kda::launch_rec_v<kda::bf16, 2>(d, q, k, v, gate, gm, A_log, qn, beta, h0, cu, write_final, o, ht, s);
    return kda::launch_rec_v<kda::bf16, 1>(d, q, k, v, gate, gm, A_log, qn, beta, h0, cu, write_final, o, ht, s);
  }
  if (vec == 4) return kda::launch_rec_v<float, 4>(d, q, k, v, gate, gm, A_log, qn, beta, h0, cu, write_final, o, ht, s);
  if (vec == 2) return kda::launch_rec_v<float, 2>(d, q, k, v, gate, gm, A_log, qn, beta, h0, cu, write_final, o, ht, s);
  return kda::launch_rec_v<float, 1>(d, q, k, v, gate, gm, A_log, qn, beta, h0, cu, write_final, o, ht, s);
}

}  // namespace kda_host
