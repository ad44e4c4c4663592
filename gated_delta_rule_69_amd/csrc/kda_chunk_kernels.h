#pragma once
// Steps A2..A6: the chunked KDA scan (chunk_kda forward) on gfx950.
//
// Per chunk of C = 64 tokens with start state S0, natural-log cumulative gate
// G (here log2 units, G2) and Gamma = 2^G2, the chunk form of the per-channel
// gated delta rule is
//   A_ij  = b_i sum_c k_ic k_jc 2^(G2_ic - G2_jc)   (i > j)         [kkt]
//   T     = (I + A)^-1                                              [solve_tril]
//   W     = T diag(b) (K * Gamma),  U = T diag(b) V                 [recompute_w_u]
//   Delta = U - W S0;  S_end = Diag(Gamma_last) S0 + Khat^T Delta   [fwd_h]
//   O     = (Q~ * Gamma) S0 + (P o M) Delta                         [fwd_o]
// with Khat = K * 2^(G2_last - G2), P_ij = sum_c q~_ic k_jc 2^(G2_ic - G2_jc)
// (j <= i) and q~ = q / sqrt(K). The step names in brackets are those the
// "[Fix] Use unit KDA gate scale when A_log is omitted" page lists for the
// sibling gated-delta-rule op (squashed commit bodies); the per-channel
// factors are written out for KDA here.
//
// Kernels (all on the caller's stream, no host synchronisation):
//   chunk_table_kernel  varlen only: chunks per sequence -> chunk table.
//   chunk_intra_kernel  one workgroup per (chunk, value head), fully parallel:
//                       A and P on the matrix cores, the FP32 solve, then W,
//                       U, Q~*Gamma, Khat^T, P and Gamma_last written to the
//                       workspace already in matrix-core fragment order.
//   chunk_scan_kernel   one workgroup per (sequence, value head, V block):
//                       the sequential inter-chunk recurrence with S held in
//                       FP32 matrix-core accumulators, fused with the output.
//
// Overflow-free decay products. 2^(G2_i - G2_j) for j < i is factored as
// 2^(G2_i - G2_r) * 2^(G2_r - G2_j) with a reference token j < r <= i, so
// both factors are <= 1 and a product of them can only underflow (harmless:
// the true value is then below FP32 range too). Off-diagonal 16x16 tiles use
// r = first token of the row tile. Inside a diagonal tile the reference is
// the middle token of a segment, halving segments until every factor is
// within 2^-+112 (pairs straddling a middle are exact at any range), plus
// the exact diagonal i == j when single tokens decay further. This keeps
// unbounded gates (chunk-local cumsums far below -126 in log2 units) exact.
#include <algorithm>
#include <type_traits>

#include "kda_common.h"

namespace kda {


constexpr int kC = 64;          // chunk size
constexpr int kThreads = 256;   // 4 waves

// ------------------------------------------------------------------ workspace layout
template <typename T, int K, int V>
struct Ws {
  // per (chunk, value head), in elements of T unless noted
  static constexpr size_t W = (size_t)kC * K;    // W fragments   [4][K/KSTEP][64][PER]
  static constexpr size_t QG = (size_t)kC * K;   // Q~*Gamma      [4][K/KSTEP][64][PER]
  static constexpr size_t KH = (size_t)K * kC;   // Khat^T        [K/16][C/KSTEP][64][PER]
  static constexpr size_t P = (size_t)kC * kC;   // P             [4][C/KSTEP][64][PER]
  // bf16: P - bf16(P) (same fragment order), so the output's intra-chunk
  // product P Delta sees P to about 16 mantissa bits; FP32 P is exact
  static constexpr size_t PL = sizeof(T) == 2 ? (size_t)kC * kC : 0;
  static constexpr size_t U = (size_t)kC * V;    // U accum order [4][V/16][64][4]
  static constexpr size_t elems = W + QG + KH + P + PL + U;
  static constexpr size_t bytes_T = elems * sizeof(T);
  static constexpr size_t bytes_GL = (size_t)K * sizeof(float);  // Gamma_last (FP32)
};

// Extra per-(chunk, value head) workspace of the backward pass.
template <typename T, int K, int V>
struct WsB {
  // elements of T
  static constexpr size_t PT = (size_t)kC * kC;   // P^T fragments     [4][C/KSTEP][64][PER]
  static constexpr size_t KHn = (size_t)kC * K;   // Khat fragments    [4][K/KSTEP][64][PER]
  static constexpr size_t QGT = (size_t)K * kC;   // (Q~ Gamma)^T frags [K/16][C/KSTEP][64][PER]
  static constexpr size_t WT = (size_t)K * kC;    // W^T fragments     [K/16][C/KSTEP][64][PER]
  // the next four are R x V matrices with their rows interleaved by four
  // (il4: element (r, c) at ((r / 4) V + c) 4 + r % 4), as the scans hold them
  static constexpr size_t S0 = (size_t)K * V;     // chunk start state [K][V]
  static constexpr size_t DL = (size_t)kC * V;    // Delta [C][V]
  static constexpr size_t DS = (size_t)K * V;     // dS at the chunk end [K][V]
  static constexpr size_t DDL = (size_t)kC * V;   // dDelta [C][V]
  static constexpr size_t elems = PT + KHn + QGT + WT + S0 + DL + DS + DDL;
  // FP32
  static constexpr size_t TM = (size_t)kC * kC;   // T = (I + A)^-1, row-major [C][C]
  static constexpr size_t AB = (size_t)kC * kC;   // Abar (A without beta), row-major [C][C]
  static constexpr size_t elems_f = TM + AB;
  // offsets inside one chunk-head block
  static constexpr size_t oPT = 0, oKHn = PT, oQGT = oKHn + KHn, oWT = oQGT + QGT,
                          oS0 = oWT + WT, oDL = oS0 + S0, oDS = oDL + DL, oDDL = oDS + DS;
};

// Offset of element (r, c) of an R x V matrix with rows interleaved by four:
// the four rows 4g .. 4g + 3 of one column that an accumulator lane holds are
// four consecutive elements, written with one 8-byte (bf16) or 16-byte (FP32)
// store instead of four 2- or 4-byte ones.
__device__ __forceinline__ size_t il4(int r, int c, int V) {
  return ((size_t)(r >> 2) * V + c) * 4 + (r & 3);
}
// Store 4 FP32 values as consecutive elements of T (16-byte aligned for FP32,
// 8-byte for bf16).
template <typename T>
__device__ __forceinline__ void store4(T* p, const float v0, const float v1, const float v2,
                                       const float v3) {
  // non-temporal: these are read back by a later kernel, long after the
  // caches could hold them, and would otherwise evict the operands the other
  // workgroups of the chain are about to read (saving, keeping and reverse
  // scans 3% faster)
  if constexpr (sizeof(T) == 2) {
    bf16x4 x = {(bf16)v0, (bf16)v1, (bf16)v2, (bf16)v3};
    typedef unsigned int u32x2_ __attribute__((ext_vector_type(2)));
    __builtin_nontemporal_store(__builtin_bit_cast(u32x2_, x), reinterpret_cast<u32x2_*>(p));
  } else {
    __builtin_nontemporal_store(f32x4{v0, v1, v2, v3}, reinterpret_cast<f32x4*>(p));
  }
}

// Non-temporal store of a 4-, 8- or 16-byte value: the chunk workspace is
// read back by a later kernel, long after the caches could hold it. Used for
// the intra kernel's whole-line workspace writes (a wave's fragment store
// covers 1 KB): the scan that reads them runs 131 -> 121 us on the dense
// workload (no dirty lines of the intra kernel left to evict). The stores
// that cover half a fragment or scattered 16-byte pieces stay ordinary:
// non-temporal they made the training forward's intra kernel 5% slower.
template <typename V_>
__device__ __forceinline__ void st_nt(V_* p, const V_& v) {
  static_assert(sizeof(V_) == 4 || sizeof(V_) == 8 || sizeof(V_) == 16, "store size");
  if constexpr (sizeof(V_) == 16) {
    typedef unsigned u4_ __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(__builtin_bit_cast(u4_, v), reinterpret_cast<u4_*>(p));
  } else if constexpr (sizeof(V_) == 8) {
    typedef unsigned u2_ __attribute__((ext_vector_type(2)));
    __builtin_nontemporal_store(__builtin_bit_cast(u2_, v), reinterpret_cast<u2_*>(p));
  } else {
    __builtin_nontemporal_store(__builtin_bit_cast(unsigned, v), reinterpret_cast<unsigned*>(p));
  }
}

// Non-temporal 16-byte load, for data a kernel reads exactly once (the
// backward local kernel's saved states and matrices, its q, k, gate, dO and v
// rows: 3613 -> 3486 us).
__device__ __forceinline__ uint4 ldg_nt(const uint4* p) {
  typedef unsigned u4_ __attribute__((ext_vector_type(4)));
  const u4_ r = __builtin_nontemporal_load(reinterpret_cast<const u4_*>(p));
  return make_uint4(r[0], r[1], r[2], r[3]);
}
__device__ __forceinline__ float4 ldg_nt(const float4* p) {
  const f32x4 r = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(r[0], r[1], r[2], r[3]);
}

struct ChunkGeo {
  int ok;        // 0: no such chunk (grid over-provisioned)
  int n;         // sequence
  int64_t t0;    // flat index of the chunk's first token
  int L;         // tokens in the chunk (1..64)
  int c;         // chunk index inside its sequence (0: the sequence's first)
};

__device__ __forceinline__ ChunkGeo chunk_geo(int j, const int32_t* cu, const int* ws_int, int N,
                                              int T) {
  ChunkGeo r{0, 0, 0, 0, 0};
  if (cu == nullptr) {
    const int nc = (T + kC - 1) / kC;
    const int n = j / nc, c = j % nc;
    if (n >= N) return r;
    r.ok = 1;
    r.n = n;
    r.t0 = (int64_t)n * T + (int64_t)c * kC;
    r.L = min(kC, T - c * kC);
    r.c = c;
  } else {
    if (j >= ws_int[0]) return r;
    const int n = ws_int[2 + 2 * N + j];
    const int c = j - ws_int[1 + n];
    const int bos = cu[n], len = cu[n + 1] - bos;
    r.ok = 1;
    r.n = n;
    r.t0 = bos + (int64_t)c * kC;
    r.L = min(kC, len - c * kC);
    r.c = c;
  }
  return r;
}

// ------------------------------------------------------------------ intra-chunk kernel
template <typename T, int K, int V>
struct IntraLds {
  static constexpr int TP = 16 / (int)sizeof(T);  // 16-byte row pad, in elements
  static constexpr int GS = K + 4;                // G2 row stride (floats)
  static constexpr int KSTR = K + TP;             // k / q row stride
  static constexpr int AS = kC + 4;               // A / T row stride (floats)
  static constexpr int VSTR = V + TP;             // b v row stride
  static constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t R1 = cmax((size_t)kC * GS * 4, (size_t)kC * VSTR * sizeof(T));
  static constexpr size_t R2 = (size_t)kC * KSTR * sizeof(T);
  static constexpr size_t R3 = cmax((size_t)kC * KSTR * sizeof(T), (size_t)kC * AS * 4);
  static constexpr size_t RB = (size_t)kC * 4;                    // beta
  static constexpr size_t RT = (size_t)(kC / kGateBlock) * K * 4;  // gate block totals
  static constexpr size_t total = R1 + R2 + R3 + RB + RT;
  // short convolution: taps by distance [kConvMaxWidth][D] then the bias [D],
  // for k, q (D = K) and v (D = V) of the workgroup's heads
  static constexpr size_t RC = (size_t)(kConvMaxWidth + 1) * (2 * K + V) * 4;
  static constexpr size_t total_conv = total + RC;
};

// 2^x on the transcendental unit (v_exp_f32). Results below 2^-126 flush to
// zero, which only drops decay products that are below FP32 range anyway.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Four consecutive LDS elements as floats (one 16- or 8-byte LDS read).
__device__ __forceinline__ void lds4(const float* p, float o[4]) {
  const float4 x = *reinterpret_cast<const float4*>(p);
  o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
}
__device__ __forceinline__ void lds4(const bf16* p, float o[4]) {
  const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
  o[0] = (float)x[0]; o[1] = (float)x[1]; o[2] = (float)x[2]; o[3] = (float)x[3];
}

// Element e of a 16-byte unit holding T values, as float.
template <typename T>
__device__ __forceinline__ float unit_elem(const uint4& u, int e) {
  const uint32_t w = (e >> (sizeof(T) == 2 ? 1 : 0)) == 0 ? u.x
                   : (e >> (sizeof(T) == 2 ? 1 : 0)) == 1 ? u.y
                   : (e >> (sizeof(T) == 2 ? 1 : 0)) == 2 ? u.z : u.w;
  if constexpr (sizeof(T) == 2) return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
  else return __uint_as_float(w);
}

// A 16-byte unit of T values, each multiplied by s (rounded back to T).
template <typename T>
__device__ __forceinline__ uint4 unit_scaled(const uint4& u, float s) {
  uint4 r = u;
  if constexpr (sizeof(T) == 2) {
    bf16* x = reinterpret_cast<bf16*>(&r);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (bf16)((float)x[e] * s);
  } else {
    float* x = reinterpret_cast<float*>(&r);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] *= s;
  }
  return r;
}

// Short causal convolution + SiLU (depthwise, taps on tokens t - W + 1 .. t,
// the last tap on t) of NU consecutive rows r0 .. r0 + NU - 1 of one head's
// [C][D] tile, channels ch .. ch + EPU - 1, in two steps so that the global
// reads of q, k and v can all be in flight before any of the arithmetic:
//   conv_halo   reads the W - 1 rows above r0 (the sequence's earlier tokens:
//               inside the chunk, or before it only when the chunk is not the
//               sequence's first, hist; else zero); hx[s - 1] = row r0 - s;
//   conv_apply  turns the raw rows x (zero past the chunk's L tokens) into
//               SiLU(z) rounded to T; rows past L stay zero. The taps come
//               from LDS, sw = [kConvMaxWidth][D] by distance (tap on token
//               t - s in row s, zero for s >= W) then the bias row, at channel ch.
//   src   row pointer of token 0 at channel ch; token t at src + t * tok_stride
// z is summed in FP32 from the bias, oldest tap first.
// The loads are unconditional (a halo row that is not used loads a valid row
// of the chunk instead) and conv_halo_mask zeroes the unused ones later: a
// load under a lane-dependent branch makes the compiler wait for every load
// issued before it at the branch join.
__device__ __forceinline__ bool conv_halo_used(int s, int r0, int L, bool hist, int W) {
  return r0 < L && s < W && (r0 - s >= 0 || hist);
}
template <typename T>
__device__ __forceinline__ void conv_halo(uint4 (&hx)[kConvMaxWidth - 1], const T* __restrict__ src,
                                          int64_t t0, int r0, int L, bool hist, int64_t tok_stride,
                                          int W) {
#pragma unroll
  for (int s = 1; s < kConvMaxWidth; ++s) {
    const int rr = conv_halo_used(s, r0, L, hist, W) ? r0 - s : (r0 < L ? r0 : L - 1);
    hx[s - 1] = *reinterpret_cast<const uint4*>(src + (t0 + rr) * tok_stride);
  }
}
__device__ __forceinline__ void conv_halo_mask(uint4 (&hx)[kConvMaxWidth - 1], int r0, int L,
                                               bool hist, int W) {
#pragma unroll
  for (int s = 1; s < kConvMaxWidth; ++s)
    if (!conv_halo_used(s, r0, L, hist, W)) hx[s - 1] = make_uint4(0, 0, 0, 0);
}

// SiLU z / (1 + e^-z) with the hardware reciprocal (1 ulp); e^-z = +inf for
// z below about -88 gives -0.
__device__ __forceinline__ float silu_f32(float z) {
  return z * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

template <typename T, int NU>
__device__ __forceinline__ void conv_apply(uint4 (&x)[NU], const uint4 (&hx)[kConvMaxWidth - 1],
                                           const float* sw, int D, int r0, int L) {
  constexpr int EPU = 16 / (int)sizeof(T), MW = kConvMaxWidth;
  if (r0 >= L) return;
  // z[u][e] for the NU rows at once, tap by tap (oldest first), so each tap
  // pair read from LDS is used at once. All kConvMaxWidth taps run: the staged
  // taps beyond W are zero and the rows they meet are finite, so those terms
  // add exactly zero.
  float z[NU][EPU];
#pragma unroll
  for (int e4 = 0; e4 < EPU; e4 += 4) {
    float b[4];
    lds4(sw + MW * D + e4, b);
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) z[u][e4 + e] = b[e];
  }
#pragma unroll
  for (int s = MW - 1; s >= 0; --s) {
#pragma unroll
    for (int e4 = 0; e4 < EPU; e4 += 4) {
      float ws[4];
      lds4(sw + s * D + e4, ws);
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float xv = s <= u ? unit_elem<T>(x[s <= u ? u - s : 0], e4 + e)
                                  : unit_elem<T>(hx[s > u ? s - u - 1 : 0], e4 + e);
          z[u][e4 + e] = fmaf(ws[e], xv, z[u][e4 + e]);
        }
    }
  }
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if (r0 + u < L) {
      union {
        T t[EPU];
        uint4 v;
      } out;
#pragma unroll
      for (int e = 0; e < EPU; ++e) out.t[e] = from_f32<T>(silu_f32(z[u][e]));
      x[u] = out.v;
    }
  }
}

// Quad p of a contraction dimension holds indices 16p + 4g + e (e = 0..3) for
// lane group g. With the kidx() order of MF<>, quad p is slots 4(p&1)..+3 of
// bf16 fragment p/2, or FP32 fragments 4p..4p+3.
template <typename M>
__device__ __forceinline__ void put_quad(typename M::frag* fr, int p, const float v[4]) {
  if constexpr (M::KSTEP == 32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) M::set(fr[p >> 1], 4 * (p & 1) + e, v[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) M::set(fr[4 * p + e], 0, v[e]);
  }
}

// A fragment carried as an unevaluated sum hi + lo of two bf16 values (about
// 16 mantissa bits): hi = bf16(x), lo = bf16(x - hi), where x - hi is exact in
// FP32. Products of such operands take three matrix-core steps (hi hi, hi lo,
// lo hi; lo lo is below FP32 accumulation noise). For FP32 fragments the
// value is exact already and lo does not exist.
template <typename M>
struct Frag2 {
  typename M::frag hi;
  typename M::frag lo;
};
template <>
struct Frag2<MF<float>> {
  typename MF<float>::frag hi;
};
template <typename M>
__device__ __forceinline__ void put_quad2(Frag2<M>* fr, int p, const float v[4]) {
  if constexpr (M::KSTEP == 32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bf16 h = (bf16)v[e];
      fr[p >> 1].hi[4 * (p & 1) + e] = h;
      fr[p >> 1].lo[4 * (p & 1) + e] = (bf16)(v[e] - (float)h);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) M::set(fr[4 * p + e].hi, 0, v[e]);
  }
}
// c + a b with both operands split
template <typename M>
__device__ __forceinline__ f32x4 mma3(const Frag2<M>& a, const Frag2<M>& b, f32x4 c) {
  c = M::mma(a.hi, b.hi, c);
  if constexpr (M::KSTEP == 32) {
    c = M::mma(a.hi, b.lo, c);
    c = M::mma(a.lo, b.hi, c);
  }
  return c;
}
// c + a b with only b split (a exact in bf16), resp. only a split
template <typename M>
__device__ __forceinline__ f32x4 mma2(const typename M::frag& a, const Frag2<M>& b, f32x4 c) {
  c = M::mma(a, b.hi, c);
  if constexpr (M::KSTEP == 32) c = M::mma(a, b.lo, c);
  return c;
}
template <typename M>
__device__ __forceinline__ f32x4 mma2(const Frag2<M>& a, const typename M::frag& b, f32x4 c) {
  c = M::mma(a.hi, b, c);
  if constexpr (M::KSTEP == 32) c = M::mma(a.lo, b, c);
  return c;
}

// Fragment of contraction step ks built from accumulator tiles of the
// transposed product (see MF<>): element jj comes from tile tile_of(ks, jj).
template <typename M>
__device__ __forceinline__ int acc_tile(int ks, int jj) {
  return (M::KSTEP == 32) ? (2 * ks + (jj >> 2)) : (ks >> 2);
}
template <typename M>
__device__ __forceinline__ int acc_elem(int ks, int jj) {
  return (M::KSTEP == 32) ? (jj & 3) : (ks & 3);
}

// Max exponent range (log2 units) that a single reference token may span in a
// diagonal tile: factors up to 2^112 and sums of 128 such products stay
// finite in FP32 and bf16.
constexpr float kFastRange = 112.f;

// BWD: also write what the backward pass needs (P^T, Khat, (Q~ Gamma)^T and
// W^T fragments, Abar and T) into ws_B / ws_Bf.  QN: L2-normalise the q and k
// rows as they are loaded (a template flag: the runtime branch alone cost the
// plain path a few percent in registers and scheduling).  CONV: q, k and v
// are raw projections; the short convolution + SiLU (taps in `conv`) runs on
// them first, and each thread then holds consecutive rows so that a row's
// window above it is its own rows plus W - 1 rows read again from L2.
// TRAIN (with BWD): the training forward -- the forward pass's entries (P and
// Q~ Gamma as well) and the backward's, so that the backward after it needs
// no intra-chunk recompute.
template <typename T, int K, int V, bool BWD, bool QN, bool CONV, bool TRAIN = false>
__global__ void __launch_bounds__(kThreads, 2)
chunk_intra_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                   const float* __restrict__ gate, int gate_mode,
                   const float* __restrict__ A_log, const T* __restrict__ beta,
                   const int32_t* __restrict__ cu, const int* __restrict__ ws_int, int N, int T_,
                   int H, int HV, float scale, T* __restrict__ ws_T, float* __restrict__ ws_GL,
                   T* __restrict__ ws_B, float* __restrict__ ws_Bf, kda_short_conv conv,
                   int head_fast) {
  using M = MF<T>;
  using F = typename M::frag;
  using Lds = IntraLds<T, K, V>;
  using WsL = Ws<T, K, V>;
  constexpr int KS_K = K / M::KSTEP;
  constexpr int KS_C = kC / M::KSTEP;
  constexpr int QK = K / 16;   // quads over channels
  constexpr int QC = kC / 16;  // quads over tokens
  constexpr int GS = Lds::GS, KSTR = Lds::KSTR, AS = Lds::AS;
  constexpr int EPU = 16 / (int)sizeof(T);      // elements of T per 16-byte unit
  constexpr int GU = kC * K / 4 / kThreads;     // float4 units of G2 per thread
  constexpr int KU = kC * K / EPU / kThreads;   // 16-byte units of k (and of q) per thread
  constexpr int VU = kC * V / EPU / kThreads;   // 16-byte units of v per thread
  static_assert(GU >= 1 && KU >= 1 && VU >= 1, "tile shape");
  constexpr int TK = K / EPU, TV = V / EPU;    // threads per row of k (q) and of v
  static_assert(kThreads % TK == 0 && kThreads % TV == 0, "row split");
  // row of a thread's 16-byte unit u (its column unit is tid % TK, resp. tid % TV)
  auto krow = [](int t, int u) { return CONV ? (t / TK) * KU + u : (t + u * kThreads) / TK; };
  auto vrow = [](int t, int u) { return CONV ? (t / TV) * VU + u : (t + u * kThreads) / TV; };

  extern __shared__ __align__(16) char smem[];
  float* sG = reinterpret_cast<float*>(smem);                       // R1: G2 [C][GS], later b v
  T* sK = reinterpret_cast<T*>(smem + Lds::R1);                     // R2: k [C][KSTR]
  T* sQ = reinterpret_cast<T*>(smem + Lds::R1 + Lds::R2);           // R3: q [C][KSTR]
  float* sA = reinterpret_cast<float*>(smem + Lds::R1 + Lds::R2);   // R3 later: A, then T [C][AS]
  float* sBeta = reinterpret_cast<float*>(smem + Lds::R1 + Lds::R2 + Lds::R3);
  float* sTot = reinterpret_cast<float*>(smem + Lds::R1 + Lds::R2 + Lds::R3 + Lds::RB);

  // 1-D grid over (chunk, value head). head_fast != 0 takes the value head
  // fastest: the workgroups in flight together read whole token rows of q, k,
  // v and the gate (all heads of a few chunks) instead of one head's 256-byte
  // pieces of many chunks, with the head rotated by the chunk index
  // (workgroups are dealt to the XCDs in turn; without the rotation every chunk
  // of head hv would land on XCD hv % 8).
  const unsigned nch = gridDim.x / (unsigned)HV;
  const bool hf = BWD || head_fast;
  const int chunk = hf ? (int)(blockIdx.x / (unsigned)HV) : (int)(blockIdx.x % nch);
  const int hv = hf ? (int)((blockIdx.x % (unsigned)HV + (unsigned)chunk) % (unsigned)HV)
                    : (int)(blockIdx.x / nch);
  const ChunkGeo geo = chunk_geo(chunk, cu, ws_int, N, T_);
  if (!geo.ok) return;
  const int h = hv / (HV / H);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int L = geo.L;
  const int64_t t0 = geo.t0;
  const size_t ch = (size_t)chunk * HV + hv;

  // ---- 1. global loads first (16-byte units), then LDS stores. With the
  // convolution its taps come first: their LDS staging then waits for them
  // alone (the load counter drains in issue order).
  constexpr int NCW = (kConvMaxWidth + 1) * (2 * K + V);  // k, q, v taps + biases
  constexpr int NCWT = CONV ? (NCW + kThreads - 1) / kThreads : 1;
  float cwr[NCWT];
  if constexpr (CONV) {
    // thread's staged values: taps of this workgroup's heads ordered by
    // distance ([kConvMaxWidth][D], zero at distances >= W), then the bias row
    constexpr int MW = kConvMaxWidth;
    const int W = conv.width;
#pragma unroll
    for (int j = 0; j < NCWT; ++j) {
      const int i = tid + j * kThreads;
      cwr[j] = 0.f;
      if (i < NCW) {
        const int t = i < (MW + 1) * K ? 0 : i < 2 * (MW + 1) * K ? 1 : 2;
        const int D = t < 2 ? K : V;
        const int rem = i - t * (MW + 1) * K, s = rem / D;
        const int c = (t < 2 ? h * K : hv * V) + rem % D;
        const float* w = t == 0 ? conv.k_weight : t == 1 ? conv.q_weight : conv.v_weight;
        const float* b = t == 0 ? conv.k_bias : t == 1 ? conv.q_bias : conv.v_bias;
        if (s < MW) {
          if (s < W) cwr[j] = w[(size_t)c * W + (W - 1 - s)];
        } else if (b) {
          cwr[j] = b[c];
        }
      }
    }
  }
  // Gate rows. When a thread's GU units make up one whole cumsum block
  // (GU == kGateBlock, K = 128), thread (block rb, channel group cg) loads
  // rows 8 rb .. 8 rb + 7 of channels 4 cg .. 4 cg + 3, and the in-block part
  // of a fused gate's cumsum runs in its registers; otherwise unit u is row
  // (tid + u * threads) / (K / 4) and the cumsum reads the rows back from LDS.
  constexpr bool GREG = GU == kGateBlock;
  auto grow = [&](int u) { return GREG ? kGateBlock * (tid / (K / 4)) + u : (tid + u * kThreads) / (K / 4); };
  auto gc4 = [&](int u) { return GREG ? tid % (K / 4) : (tid + u * kThreads) % (K / 4); };
  float4 gr[GU];
  uint4 kr[KU], qr[KU], vr[VU];
#pragma unroll
  for (int u = 0; u < GU; ++u) {
    const int row = grow(u), c4 = gc4(u);
    const int rr = row < L ? row : L - 1;  // pad rows repeat the last gate row
    gr[u] = *reinterpret_cast<const float4*>(gate + ((t0 + rr) * HV + hv) * K + 4 * c4);
  }
  // Pad rows of a short last chunk load the last valid row, like the gate, and
  // are zeroed where the values are first used: no load sits in a lane-
  // dependent branch, whose join would make the compiler wait for every load
  // issued so far before the remaining ones.
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const int row = krow(tid, u), cu_ = tid % TK;
    const int rr = row < L ? row : L - 1;
    kr[u] = *reinterpret_cast<const uint4*>(k + ((t0 + rr) * H + h) * K + EPU * cu_);
    qr[u] = *reinterpret_cast<const uint4*>(q + ((t0 + rr) * H + h) * K + EPU * cu_);
  }
  // v is first used by U, the last phase: without the convolution its loads
  // are issued after the A/P tiles, so the workgroup's first load batch (the
  // one every phase waits for) is a fifth smaller
  auto load_v = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int row = vrow(tid, u), cu_ = tid % TV;
      const int rr = row < L ? row : L - 1;
      vr[u] = *reinterpret_cast<const uint4*>(v + ((t0 + rr) * HV + hv) * V + EPU * cu_);
    }
  };
  if constexpr (CONV) load_v();
  const int brow = tid % kC < L ? tid % kC : L - 1;
  const T braw = beta[(t0 + brow) * HV + hv];  // every thread loads; threads < kC store
  auto zero_v_pad = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < VU; ++u)
      if (vrow(tid, u) >= L) vr[u] = make_uint4(0, 0, 0, 0);
  };
  auto zero_pad_rows = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < KU; ++u)
      if (krow(tid, u) >= L) kr[u] = qr[u] = make_uint4(0, 0, 0, 0);
    if constexpr (CONV) zero_v_pad();
  };
  if constexpr (CONV) {
    constexpr int MW = kConvMaxWidth;
    const bool hist = geo.c > 0;
    const int W = conv.width;
    const int ck = EPU * (tid % TK), cv = EPU * (tid % TV);
    const int rk = krow(tid, 0), rv = vrow(tid, 0);
    uint4 hk[MW - 1], hq[MW - 1], hvv[MW - 1];
    conv_halo<T>(hk, k + h * K + ck, t0, rk, L, hist, (int64_t)H * K, W);
    conv_halo<T>(hq, q + h * K + ck, t0, rk, L, hist, (int64_t)H * K, W);
    conv_halo<T>(hvv, v + hv * V + cv, t0, rv, L, hist, (int64_t)HV * V, W);
    float* sCw = reinterpret_cast<float*>(smem + Lds::total);
#pragma unroll
    for (int j = 0; j < NCWT; ++j) {
      const int i = tid + j * kThreads;
      if (i < NCW) sCw[i] = cwr[j];
    }
    __syncthreads();
    zero_pad_rows();
    conv_halo_mask(hk, rk, L, hist, W);
    conv_halo_mask(hq, rk, L, hist, W);
    conv_halo_mask(hvv, rv, L, hist, W);
    // one tensor at a time: interleaving the three raises register pressure
    // past the budget of two workgroups per compute unit
    conv_apply<T, KU>(kr, hk, sCw + ck, K, rk, L);
    __builtin_amdgcn_sched_barrier(0);
    conv_apply<T, KU>(qr, hq, sCw + (MW + 1) * K + ck, K, rk, L);
    __builtin_amdgcn_sched_barrier(0);
    conv_apply<T, VU>(vr, hvv, sCw + 2 * (MW + 1) * K + cv, V, rv, L);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (!CONV) zero_pad_rows();
  if (tid < kC) sBeta[tid] = tid < L ? to_f32(braw) : 0.f;
  if constexpr (QN) {
    // the K / EPU threads holding a row of q and k are consecutive lanes
    constexpr int TPR = K / EPU;
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      float sk = 0.f, sq = 0.f;
#pragma unroll
      for (int e = 0; e < EPU; ++e) {
        const float a = unit_elem<T>(kr[u], e), b = unit_elem<T>(qr[u], e);
        sk += a * a;
        sq += b * b;
      }
#pragma unroll
      for (int m = 1; m < TPR; m <<= 1) {
        sk += __shfl_xor(sk, m);
        sq += __shfl_xor(sq, m);
      }
      kr[u] = unit_scaled<T>(kr[u], l2norm_inv(sk));
      qr[u] = unit_scaled<T>(qr[u], l2norm_inv(sq));
    }
  }
  if (gate_mode != kGateLog2) {
    // fused gate step: per-token natural-log gate first (cumsum below)
    const float sc = gate_head_scale(gate_mode, A_log, hv);
#pragma unroll
    for (int u = 0; u < GU; ++u) {
      gr[u].x = gate_nat(gr[u].x, gate_mode, sc);
      gr[u].y = gate_nat(gr[u].y, gate_mode, sc);
      gr[u].z = gate_nat(gr[u].z, gate_mode, sc);
      gr[u].w = gate_nat(gr[u].w, gate_mode, sc);
    }
  }
  // fused gate with register blocks: in-block inclusive sums in registers
  // (pad rows keep the last token's value), block totals to LDS
  const bool greg_sum = GREG && gate_mode != kGateLog2;
  if (greg_sum) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < GU; ++u) {
      float ge[4] = {gr[u].x, gr[u].y, gr[u].z, gr[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (grow(u) < L) acc[e] = acc[e] + ge[e];
        ge[e] = acc[e];
      }
      gr[u] = make_float4(ge[0], ge[1], ge[2], ge[3]);
    }
    *reinterpret_cast<float4*>(sTot + (tid / (K / 4)) * K + 4 * gc4(0)) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  } else {
#pragma unroll
    for (int u = 0; u < GU; ++u)
      *reinterpret_cast<float4*>(sG + grow(u) * GS + 4 * gc4(u)) = gr[u];
  }
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const int row = krow(tid, u), cu_ = tid % TK;
    *reinterpret_cast<uint4*>(sK + row * KSTR + EPU * cu_) = kr[u];
    *reinterpret_cast<uint4*>(sQ + row * KSTR + EPU * cu_) = qr[u];
  }
  __syncthreads();
  if (greg_sum) {
    // block offsets C_b (totals of the earlier blocks, in order), then
    // G2 = (C_b + in-block sum) * log2(e): the gate kernel's order
    const int rb = tid / (K / 4), cg = gc4(0);
    float c[4] = {0.f, 0.f, 0.f, 0.f};
    for (int b = 0; b < rb; ++b) {
      float t4[4];
      lds4(sTot + b * K + 4 * cg, t4);
#pragma unroll
      for (int e = 0; e < 4; ++e) c[e] = c[e] + t4[e];
    }
#pragma unroll
    for (int u = 0; u < GU; ++u)
      *reinterpret_cast<float4*>(sG + grow(u) * GS + 4 * cg) =
          make_float4((c[0] + gr[u].x) * kLog2e, (c[1] + gr[u].y) * kLog2e, (c[2] + gr[u].z) * kLog2e,
                      (c[3] + gr[u].w) * kLog2e);
    __syncthreads();
  } else if (gate_mode != kGateLog2) {
    // chunk-local inclusive cumsum times log2(e) in the blocked order of
    // kGateBlock (the gate kernel's order, so G2 is bit-identical to its
    // output). Thread (cg, rb) owns channels 4cg..4cg+3 of token block rb.
    // Pad rows keep the last token's value.
    constexpr int NCG = K / 4, NB = kC / kGateBlock;
    const int cg = tid % NCG, rb = tid / NCG;
    float pm[kGateBlock][4];
    if (rb < NB) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < kGateBlock; ++m) {
        const int rr = rb * kGateBlock + m;
        lds4(sG + rr * GS + 4 * cg, pm[m]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (rr < L) acc[e] = acc[e] + pm[m][e];
          pm[m][e] = acc[e];
        }
      }
      *reinterpret_cast<float4*>(sTot + rb * K + 4 * cg) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
    __syncthreads();
    if (rb < NB) {
      float c[4] = {0.f, 0.f, 0.f, 0.f};
      for (int b = 0; b < rb; ++b) {
        float t4[4];
        lds4(sTot + b * K + 4 * cg, t4);
#pragma unroll
        for (int e = 0; e < 4; ++e) c[e] = c[e] + t4[e];
      }
#pragma unroll
      for (int m = 0; m < kGateBlock; ++m) {
        const int rr = rb * kGateBlock + m;
        *reinterpret_cast<float4*>(sG + rr * GS + 4 * cg) =
            make_float4((c[0] + pm[m][0]) * kLog2e, (c[1] + pm[m][1]) * kLog2e,
                        (c[2] + pm[m][2]) * kLog2e, (c[3] + pm[m][3]) * kLog2e);
      }
    }
    __syncthreads();
  }

  // ---- 2. A^T and P^T tiles: column tile I = wave (tokens i), row tiles J <= I (tokens j)
  const int I = wave;
  const int icol = 16 * I + l16;
  const int jl = l16, il = l16;
  const int jrow = 16 * I + jl;
  int lstar = 3;
  bool need_diag = false;
  {
    // 15 (level, segment) items on lanes l16 < 15; channels split over g
    const int lv = l16 < 1 ? 0 : l16 < 3 ? 1 : l16 < 7 ? 2 : 3;
    const int S = 16 >> lv, seg = l16 - ((1 << lv) - 1);
    const int ta = 16 * I + seg * S, tm = ta + S / 2, tb = ta + S - 1;
    float rng = 0.f;
    if (l16 < 15) {
#pragma unroll
      for (int p = 0; p < QK; ++p) {
        const int c0 = 16 * p + 4 * g;
        float ga[4], gm[4], gb[4];
        lds4(sG + ta * GS + c0, ga);
        lds4(sG + tm * GS + c0, gm);
        lds4(sG + tb * GS + c0, gb);
#pragma unroll
        for (int e = 0; e < 4; ++e) rng = fmaxf(rng, fmaxf(ga[e] - gm[e], gm[e] - gb[e]));
      }
    }
    rng = fmaxf(rng, __shfl_xor(rng, 16));
    rng = fmaxf(rng, __shfl_xor(rng, 32));
    const uint64_t okb = __ballot(rng <= kFastRange);  // bit l16 (lanes 0..15)
    if ((okb & 0x1ull) == 0x1ull) lstar = 0;
    else if ((okb & 0x6ull) == 0x6ull) lstar = 1;
    else if ((okb & 0x78ull) == 0x78ull) lstar = 2;
    else if ((okb & 0x7F80ull) == 0x7F80ull) lstar = 3;
    else need_diag = true;
  }
  // Reference token of column tile I. When the diagonal tile passes the
  // one-pass test (every factor of its middle token within 2^-+kFastRange),
  // the middle token r = 16I + 8 serves the whole column: left factors
  // 2^(G2_i - G2_r) stay below 2^kFastRange, right factors of earlier tiles
  // are <= 1, and the diagonal tile needs only its row factors. Otherwise
  // r = 16I keeps every off-diagonal factor <= 1 and the diagonal tile takes
  // the recursive passes below.
  const bool mid = (lstar == 0) && !need_diag;
  const int r = 16 * I + (mid ? 8 : 0);
  // The decay-scaled operands of A and P are not exact in bf16, and their
  // rounding, amplified by the cancellation in the channel sums, would
  // otherwise be the largest error of the bf16 forward: every one of them is
  // split hi + lo (Frag2, three matrix-core steps per product). To keep the
  // split operands within the register budget the channel sums run over
  // halves of K (64 channels each), building one half's operands at a time.
  constexpr int NHF = K >= 128 ? 2 : 1;  // channel halves
  constexpr int QH = QK / NHF;           // quads per half
  constexpr int FH = KS_K / NHF;         // fragments per half
  f32x4 accA[3], accP[3];            // tiles J < I
  f32x4 dA = zero4(), dP = zero4();  // tile J == I
  f32x4 pT[3], dPT = zero4();        // BWD: P tiles (rows i, cols j), J < I and J == I
#pragma unroll
  for (int J = 0; J < 3; ++J) accA[J] = accP[J] = pT[J] = zero4();
  f32x4 xa = zero4(), xp = zero4(), xt = zero4();  // diagonal tile, one-pass reference
#pragma unroll
  for (int hf = 0; hf < NHF; ++hf) {
    // column factors k_i 2^(G2_i - G2_r), q~_i 2^(G2_i - G2_r) of this half
    Frag2<M> lkf[FH], lqf[FH];
#pragma unroll
    for (int pp = 0; pp < QH; ++pp) {
      const int c0 = 16 * (QH * hf + pp) + 4 * g;
      float gi[4], g0[4], ki[4], qi[4], vk[4], vq[4];
      lds4(sG + icol * GS + c0, gi);
      lds4(sG + r * GS + c0, g0);
      lds4(sK + icol * KSTR + c0, ki);
      lds4(sQ + icol * KSTR + c0, qi);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = ex2(gi[e] - g0[e]);
        vk[e] = ki[e] * x;
        vq[e] = qi[e] * scale * x;
      }
      put_quad2<M>(lkf, pp, vk);
      put_quad2<M>(lqf, pp, vq);
    }
#pragma unroll
    for (int J = 0; J < 3; ++J) {
      if (J < I) {
        const int jrow = 16 * J + l16;
        Frag2<M> rf[FH];  // row factors k_j 2^(G2_r - G2_j) (<= 1: j < 16I <= r)
#pragma unroll
        for (int pp = 0; pp < QH; ++pp) {
          const int c0 = 16 * (QH * hf + pp) + 4 * g;
          float gj[4], g0[4], kj[4], vv[4];
          lds4(sG + jrow * GS + c0, gj);
          lds4(sG + r * GS + c0, g0);
          lds4(sK + jrow * KSTR + c0, kj);
#pragma unroll
          for (int e = 0; e < 4; ++e) vv[e] = kj[e] * ex2(g0[e] - gj[e]);
          put_quad2<M>(rf, pp, vv);
        }
#pragma unroll
        for (int ks = 0; ks < FH; ++ks) {
          accA[J] = mma3<M>(rf[ks], lkf[ks], accA[J]);
          accP[J] = mma3<M>(rf[ks], lqf[ks], accP[J]);
          if constexpr (BWD) pT[J] = mma3<M>(lqf[ks], rf[ks], pT[J]);
        }
      }
    }
    if (mid) {
      Frag2<M> ra[FH];  // k_j 2^(G2_r - G2_j), within 2^-+kFastRange
#pragma unroll
      for (int pp = 0; pp < QH; ++pp) {
        const int c0 = 16 * (QH * hf + pp) + 4 * g;
        float gj[4], g0[4], kj[4], vv[4];
        lds4(sG + jrow * GS + c0, gj);
        lds4(sG + r * GS + c0, g0);
        lds4(sK + jrow * KSTR + c0, kj);
#pragma unroll
        for (int e = 0; e < 4; ++e) vv[e] = kj[e] * ex2(g0[e] - gj[e]);
        put_quad2<M>(ra, pp, vv);
      }
#pragma unroll
      for (int ks = 0; ks < FH; ++ks) {
        xa = mma3<M>(ra[ks], lkf[ks], xa);
        xp = mma3<M>(ra[ks], lqf[ks], xp);
        if constexpr (BWD) xt = mma3<M>(lqf[ks], ra[ks], xt);
      }
    }
  }
  if (mid) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int jr = 4 * g + e;
      dA[e] = (il > jr) ? xa[e] : 0.f;
      dP[e] = (il >= jr) ? xp[e] : 0.f;
      dPT[e] = (jr >= l16) ? xt[e] : 0.f;  // P tile: row i = 4g + e, column j = l16
    }
  }
  // Diagonal tile, recursive mid-point references. Pass `lev` (0..3) splits
  // the tile into segments of S = 16 >> lev tokens and uses each segment's
  // middle token m as the reference of its rows and columns:
  // 2^(G2_i - G2_j) = 2^(G2_i - G2_m) 2^(G2_m - G2_j). Pairs that straddle the
  // middle (j < m <= i) get two factors <= 1 and are exact at any gate range;
  // the remaining same-segment pairs are exact when every factor stays within
  // 2^-+kFastRange, i.e. when the segment's gate range on each side of m is
  // at most kFastRange. The passes stop at the first level where that holds
  // for all segments (one pass for moderate gates); if even single tokens
  // exceed it, a last pass adds the diagonal i == j (decay factor 1).
  for (int lev = 0; !mid && lev <= lstar; ++lev) {
    const int S = 16 >> lev;
    const bool final_pass = (lev == lstar) && !need_diag;
    const int mj = 16 * I + (jl / S) * S + S / 2;  // reference of row j
    const int mi = 16 * I + (il / S) * S + S / 2;  // reference of column i
    f32x4 ya = zero4(), yp = zero4(), yt = zero4();
#pragma unroll
    for (int hf = 0; hf < NHF; ++hf) {
      Frag2<M> ra[FH], lk[FH], lq[FH];
#pragma unroll
      for (int pp = 0; pp < QH; ++pp) {
        const int c0 = 16 * (QH * hf + pp) + 4 * g;
        float kj[4], ki[4], qi[4], gj[4], gmj[4], gi[4], gmi[4], va[4], vk[4], vq[4];
        lds4(sK + jrow * KSTR + c0, kj);
        lds4(sK + icol * KSTR + c0, ki);
        lds4(sQ + icol * KSTR + c0, qi);
        lds4(sG + jrow * GS + c0, gj);
        lds4(sG + mj * GS + c0, gmj);
        lds4(sG + icol * GS + c0, gi);
        lds4(sG + mi * GS + c0, gmi);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          va[e] = kj[e] * ex2(gmj[e] - gj[e]);
          const float x = ex2(gi[e] - gmi[e]);
          vk[e] = ki[e] * x;
          vq[e] = qi[e] * scale * x;
        }
        put_quad2<M>(ra, pp, va);
        put_quad2<M>(lk, pp, vk);
        put_quad2<M>(lq, pp, vq);
      }
#pragma unroll
      for (int ks = 0; ks < FH; ++ks) {
        ya = mma3<M>(ra[ks], lk[ks], ya);
        yp = mma3<M>(ra[ks], lq[ks], yp);
        if constexpr (BWD) yt = mma3<M>(lq[ks], ra[ks], yt);
      }
    }
    // pair (row a, column b) belongs to this pass: same segment, and either
    // the last pass or straddling the segment's middle
    auto take = [&](int a, int b) {
      return (a / S == b / S) && (final_pass || ((a / (S / 2)) != (b / (S / 2))));
    };
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int jr = 4 * g + e;  // local row j of this accumulator element, column i = il
      if (take(jr, il)) {
        if (il > jr) dA[e] += ya[e];
        if (il >= jr) dP[e] += yp[e];
      }
      if constexpr (BWD) {
        // transposed tile: row i = 4g + e, column j = l16
        if (take(l16, jr) && jr >= l16) dPT[e] += yt[e];
      }
    }
  }
  if (!mid && need_diag) {
    // i == j: P_ii = q~_i . k_i (no decay; k is exact in its dtype, q~ is split)
    f32x4 yp = zero4(), yt = zero4();
#pragma unroll
    for (int hf = 0; hf < NHF; ++hf) {
      F ra[FH];
      Frag2<M> lq[FH];
#pragma unroll
      for (int pp = 0; pp < QH; ++pp) {
        const int c0 = 16 * (QH * hf + pp) + 4 * g;
        float kj[4], qi[4], vq[4];
        lds4(sK + jrow * KSTR + c0, kj);
        lds4(sQ + icol * KSTR + c0, qi);
#pragma unroll
        for (int e = 0; e < 4; ++e) vq[e] = qi[e] * scale;
        put_quad<M>(ra, pp, kj);
        put_quad2<M>(lq, pp, vq);
      }
#pragma unroll
      for (int ks = 0; ks < FH; ++ks) {
        yp = mma2<M>(ra[ks], lq[ks], yp);
        if constexpr (BWD) yt = mma2<M>(lq[ks], ra[ks], yt);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int jr = 4 * g + e;
      if (jr == il) dP[e] += yp[e];
      if constexpr (BWD) {
        if (jr == l16) dPT[e] += yt[e];
      }
    }
  }

  if constexpr (!CONV) load_v();
  T* wsW = ws_T + ch * WsL::elems;
  T* wsQG = wsW + WsL::W;
  T* wsKH = wsQG + WsL::QG;
  T* wsP = wsKH + WsL::KH;
  T* wsPL = wsP + WsL::P;
  T* wsU = wsPL + WsL::PL;
  float* wsGL = ws_GL + ch * K;

  // ---- 3. P fragments (rows i of tile I, contraction over j): accumulators of P^T
  // (P and Q~ Gamma in ws_T feed only the forward output; the backward's
  // recurrence forms no output and reads neither)
  if constexpr (!BWD || TRAIN) {
#pragma unroll
    for (int ks = 0; ks < KS_C; ++ks) {
      F f, fl;
#pragma unroll
      for (int jj = 0; jj < M::PER; ++jj) {
        const int tile = acc_tile<M>(ks, jj), el = acc_elem<M>(ks, jj);
        float x = 0.f;
#pragma unroll
        for (int J = 0; J < 4; ++J)
          if (J == tile) x = (J < I) ? accP[J < 3 ? J : 0][el] : (J == I ? dP[el] : 0.f);
        M::set(f, jj, x);
        if constexpr (WsL::PL > 0) M::set(fl, jj, x - M::get(f, jj));
      }
      st_nt(&reinterpret_cast<F*>(wsP)[((size_t)I * KS_C + ks) * 64 + lane], f);
      if constexpr (WsL::PL > 0) st_nt(&reinterpret_cast<F*>(wsPL)[((size_t)I * KS_C + ks) * 64 + lane], fl);
    }
  }
  if constexpr (BWD) {
    // P^T fragments (rows j, contraction over i): the P tile (I, J) accumulators
    // are half of fragment (J, I/2) (bf16) or fragments (J, 4I..4I+3) (FP32).
    T* wsPT = ws_B + ch * WsB<T, K, V>::elems + WsB<T, K, V>::oPT;
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      f32x4 x = zero4();
#pragma unroll
      for (int jj = 0; jj < 3; ++jj)
        if (jj == J && J < I) x = pT[jj];
      if (J == I) x = dPT;
      if constexpr (M::KSTEP == 32) {
        bf16x4 hx;
#pragma unroll
        for (int e = 0; e < 4; ++e) hx[e] = (bf16)x[e];
        *reinterpret_cast<bf16x4*>(wsPT + (((size_t)J * KS_C + (I >> 1)) * 64 + lane) * 8 + 4 * (I & 1)) = hx;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) wsPT[((size_t)J * KS_C + 4 * I + e) * 64 + lane] = from_f32<T>(x[e]);
      }
    }
    // Khat fragments (rows tokens i of tile I, contraction over channels)
    T* wsKHn = ws_B + ch * WsB<T, K, V>::elems + WsB<T, K, V>::oKHn;
    {
      F f[KS_K];
#pragma unroll
      for (int p = 0; p < QK; ++p) {
        const int c0 = 16 * p + 4 * g;
        float ki[4], gi[4], gl[4], vv[4];
        lds4(sK + icol * KSTR + c0, ki);
        lds4(sG + icol * GS + c0, gi);
        lds4(sG + (L - 1) * GS + c0, gl);
#pragma unroll
        for (int e = 0; e < 4; ++e) vv[e] = ki[e] * ex2(gl[e] - gi[e]);
        put_quad<M>(f, p, vv);
      }
#pragma unroll
      for (int ks = 0; ks < KS_K; ++ks) st_nt(&reinterpret_cast<F*>(wsKHn)[((size_t)I * KS_K + ks) * 64 + lane], f[ks]);
    }
    // (Q~ Gamma)^T fragments (rows channels, contraction over tokens), channel
    // tiles on waves 0..2 only, as the Khat^T ones below
    T* wsQGT = ws_B + ch * WsB<T, K, V>::elems + WsB<T, K, V>::oQGT;
#pragma unroll
    for (int rt0 = 0; rt0 < K / 16; rt0 += 3) {
      const int rt = rt0 + wave;
      if (wave == 3 || rt >= K / 16) continue;
      const int c = 16 * rt + l16;
      F f[KS_C];
#pragma unroll
      for (int p = 0; p < QC; ++p) {
        float vv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 16 * p + 4 * g + e;
          vv[e] = to_f32(sQ[j * KSTR + c]) * scale * ex2(sG[j * GS + c]);
        }
        put_quad<M>(f, p, vv);
      }
#pragma unroll
      for (int ks = 0; ks < KS_C; ++ks) st_nt(&reinterpret_cast<F*>(wsQGT)[((size_t)rt * KS_C + ks) * 64 + lane], f[ks]);
    }
  }
  // ---- 4. Q~ * Gamma fragments (rows i of tile I, contraction over channels)
  if constexpr (!BWD || TRAIN) {
    F f[KS_K];
#pragma unroll
    for (int p = 0; p < QK; ++p) {
      const int c0 = 16 * p + 4 * g;
      float qi[4], gi[4], vv[4];
      lds4(sQ + icol * KSTR + c0, qi);
      lds4(sG + icol * GS + c0, gi);
#pragma unroll
      for (int e = 0; e < 4; ++e) vv[e] = qi[e] * scale * ex2(gi[e]);
      put_quad<M>(f, p, vv);
    }
#pragma unroll
    for (int ks = 0; ks < KS_K; ++ks) st_nt(&reinterpret_cast<F*>(wsQG)[((size_t)I * KS_K + ks) * 64 + lane], f[ks]);
  }
  // ---- 5. Khat^T fragments (rows = channels, contraction over tokens j).
  // The channel tiles go to waves 0..2 only: wave 3 built the row factors of
  // three off-diagonal A/P tiles above and wave 0 of none, and the barrier
  // below waits for the last of them (bit-identical results; long-context
  // forward 1200 -> 1150 us, fused dense 188-201 -> 186-194 us on two boxes)
#pragma unroll
  for (int rt0 = 0; rt0 < K / 16; rt0 += 3) {
    const int rt = rt0 + wave;
    if (wave == 3 || rt >= K / 16) continue;
    const int c = 16 * rt + l16;
    const float gl = sG[(L - 1) * GS + c];
    F f[KS_C];
#pragma unroll
    for (int p = 0; p < QC; ++p) {
      float vv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 16 * p + 4 * g + e;
        vv[e] = to_f32(sK[j * KSTR + c]) * ex2(gl - sG[j * GS + c]);
      }
      put_quad<M>(f, p, vv);
    }
#pragma unroll
    for (int ks = 0; ks < KS_C; ++ks) st_nt(&reinterpret_cast<F*>(wsKH)[((size_t)rt * KS_C + ks) * 64 + lane], f[ks]);
  }
  if (tid < K) wsGL[tid] = ex2(sG[(L - 1) * GS + tid]);
  __syncthreads();  // q is dead: R3 <- A

  // ---- 6. A = b_i (A^T accumulators)^T into LDS (zero above the diagonal tiles)
  {
    const float b = sBeta[icol];
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (J < I) {
        const f32x4 a = accA[J < 3 ? J : 0];
        x = make_float4(b * a[0], b * a[1], b * a[2], b * a[3]);
      } else if (J == I) {
        x = make_float4(b * dA[0], b * dA[1], b * dA[2], b * dA[3]);
      }
      *reinterpret_cast<float4*>(&sA[icol * AS + 16 * J + 4 * g]) = x;
      if constexpr (BWD) {
        float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
        if (J < I) {
          const f32x4 a = accA[J < 3 ? J : 0];
          y = make_float4(a[0], a[1], a[2], a[3]);
        } else if (J == I) {
          y = make_float4(dA[0], dA[1], dA[2], dA[3]);
        }
        float* wsAB = ws_Bf + ch * WsB<T, K, V>::elems_f + WsB<T, K, V>::TM;
        *reinterpret_cast<float4*>(wsAB + icol * kC + 16 * J + 4 * g) = y;
      }
    }
  }
  __syncthreads();

  // ---- 7. T = (I + A)^-1 in FP32, in place
  // 7a. diagonal 16x16 blocks by forward substitution (wave d, lane = column)
  if (lane < 16) {
    const int d = wave, jj = lane;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float arow[16];
#pragma unroll
      for (int m4 = 0; m4 < 4; ++m4) lds4(sA + (16 * d + i) * AS + 16 * d + 4 * m4, arow + 4 * m4);
      float s = (i == jj) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m) s -= arow[m] * x[m];
      x[i] = s;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sA[(16 * d + i) * AS + 16 * d + jj] = x[i];
  }
  __syncthreads();
  // 7b. block rows T_IJ = -T_II sum_{M=J}^{I-1} A_IM T_MJ on the FP32 matrix
  // cores. Wave J owns block column J: its T_MJ stay in registers, since an
  // FP32 16x16 accumulator (lane: column l16, rows 4g..4g+3) is exactly the B
  // operand of the next product over those rows. A_IM and T_II are A operands
  // read as rows from LDS. The blocks are stored after every wave has read A.
  {
    f32x4 tcol[4];  // T_MJ of this wave's block column J, in B-operand layout
#pragma unroll
    for (int m = 0; m < 4; ++m) tcol[m] = zero4();
#pragma unroll
    for (int J = 0; J < 3; ++J) {  // compile-time J: register indices stay static
      if (J != wave) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) tcol[J][i] = sA[(16 * J + 4 * g + i) * AS + 16 * J + l16];
#pragma unroll
      for (int Ib = J + 1; Ib < 4; ++Ib) {
        f32x4 x = zero4();
#pragma unroll
        for (int Mb = J; Mb < Ib; ++Mb) {
          float a4[4];
          lds4(sA + (16 * Ib + l16) * AS + 16 * Mb + 4 * g, a4);
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            x = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[ks], tcol[Mb][ks], x, 0, 0, 0);
        }
        float t4[4];
        lds4(sA + (16 * Ib + l16) * AS + 16 * Ib + 4 * g, t4);
        f32x4 y = zero4();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          y = __builtin_amdgcn_mfma_f32_16x16x4f32(t4[ks], x[ks], y, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) tcol[Ib][i] = -y[i];
      }
    }
    __syncthreads();  // every read of A is done
#pragma unroll
    for (int J = 0; J < 3; ++J) {
      if (J != wave) continue;
#pragma unroll
      for (int Ib = J + 1; Ib < 4; ++Ib)
#pragma unroll
        for (int i = 0; i < 4; ++i) sA[(16 * Ib + 4 * g + i) * AS + 16 * J + l16] = tcol[Ib][i];
    }
    __syncthreads();
  }

  if constexpr (BWD) {
    float* wsTM = ws_Bf + ch * WsB<T, K, V>::elems_f;
#pragma unroll
    for (int u = 0; u < kC * kC / 4 / kThreads; ++u) {
      const int f = tid + u * kThreads, i = f / (kC / 4), c4 = f % (kC / 4);
      st_nt(reinterpret_cast<float4*>(wsTM + i * kC + 4 * c4), *reinterpret_cast<const float4*>(sA + i * AS + 4 * c4));
    }
  }
  // ---- 8. W^T = B^T T^T with B_mc = b_m k_mc 2^G2_mc built on the fly.
  // Wave split: a pair of 16-row tiles of the output dimension (= one bf16
  // contraction step of the consumer) times NI token tiles, so every wave
  // writes whole fragments.
  {
    constexpr int NP = K / 32;  // tile pairs over channels
    const int pw = wave % NP, I0 = (wave / NP) * NP;
    F tfr[NP][KS_C];  // T rows i of token tiles I0..I0+NP-1, over m
#pragma unroll
    for (int ii = 0; ii < NP; ++ii)
#pragma unroll
      for (int p = 0; p < QC; ++p) {
        float t4[4];
        lds4(sA + (16 * (I0 + ii) + l16) * AS + 16 * p + 4 * g, t4);
        put_quad<M>(tfr[ii], p, t4);
      }
    f32x4 accW[2][NP];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int c = 16 * (2 * pw + h2) + l16;
      F ba[KS_C];
#pragma unroll
      for (int p = 0; p < QC; ++p) {
        float b4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = 16 * p + 4 * g + e;
          b4[e] = sBeta[m] * to_f32(sK[m * KSTR + c]) * ex2(sG[m * GS + c]);
        }
        put_quad<M>(ba, p, b4);
      }
#pragma unroll
      for (int ii = 0; ii < NP; ++ii) {
        accW[h2][ii] = zero4();
#pragma unroll
        for (int ks = 0; ks < KS_C; ++ks) accW[h2][ii] = M::mma(ba[ks], tfr[ii][ks], accW[h2][ii]);
        if constexpr (BWD) {
          // W tile (rows i of token tile I0+ii, columns c of channel tile 2pw+h2):
          // half of the W^T fragment (channel tile, (I0+ii)/2)
          f32x4 wt = zero4();
#pragma unroll
          for (int ks = 0; ks < KS_C; ++ks) wt = M::mma(tfr[ii][ks], ba[ks], wt);
          T* wsWT = ws_B + ch * WsB<T, K, V>::elems + WsB<T, K, V>::oWT;
          const int ctile = 2 * pw + h2, It = I0 + ii;
          if constexpr (M::KSTEP == 32) {
            bf16x4 hx;
#pragma unroll
            for (int e = 0; e < 4; ++e) hx[e] = (bf16)wt[e];
            *reinterpret_cast<bf16x4*>(wsWT + (((size_t)ctile * KS_C + (It >> 1)) * 64 + lane) * 8 + 4 * (It & 1)) = hx;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) wsWT[((size_t)ctile * KS_C + 4 * It + e) * 64 + lane] = from_f32<T>(wt[e]);
          }
        }
      }
    }
    // channel tiles 2pw, 2pw+1 are contraction steps {pw} (bf16) or {8pw..8pw+7} (FP32)
#pragma unroll
    for (int ii = 0; ii < NP; ++ii) {
      if constexpr (M::KSTEP == 32) {
        F f;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) M::set(f, jj, accW[jj >> 2][ii][jj & 3]);
        st_nt(&reinterpret_cast<F*>(wsW)[((size_t)(I0 + ii) * KS_K + pw) * 64 + lane], f);
      } else {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            F f;
            M::set(f, 0, accW[h2][ii][e]);
            st_nt(&reinterpret_cast<F*>(wsW)[((size_t)(I0 + ii) * KS_K + 4 * (2 * pw + h2) + e) * 64 + lane], f);
          }
      }
    }
  }
  __syncthreads();  // G2 and k are dead: R1 <- V (row-major)
  constexpr int VSTR = Lds::VSTR;
  T* sV = reinterpret_cast<T*>(smem);  // R1: v [C][VSTR]
  if constexpr (!CONV) zero_v_pad();
#pragma unroll
  for (int u = 0; u < VU; ++u) {
    const int m = vrow(tid, u), cu_ = tid % TV;
    *reinterpret_cast<uint4*>(sV + m * VSTR + EPU * cu_) = vr[u];
  }
  __syncthreads();

  // ---- 9. U = (T diag(b)) V, same wave split over value tiles; accumulator
  // order. b scales T's columns, so V enters the product exactly as loaded
  // (rounding b v to bf16 instead costs about as much accuracy as rounding
  // the output).
  {
    constexpr int NP = V / 32;
    const int pw = wave % NP, I0 = (wave / NP) * NP;
    // the wave's two value tiles of V as B fragments (column gathers from
    // LDS), built once and shared by its NP row tiles of T
    F vb[2][KS_C];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int c = 16 * (2 * pw + h2) + l16;
#pragma unroll
      for (int p = 0; p < QC; ++p) {
        float v4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = to_f32(sV[(16 * p + 4 * g + e) * VSTR + c]);
        put_quad<M>(vb[h2], p, v4);
      }
    }
#pragma unroll
    for (int ii = 0; ii < NP; ++ii) {
      F ta[KS_C];
#pragma unroll
      for (int p = 0; p < QC; ++p) {
        float t4[4], b4[4];
        lds4(sA + (16 * (I0 + ii) + l16) * AS + 16 * p + 4 * g, t4);
        lds4(sBeta + 16 * p + 4 * g, b4);
#pragma unroll
        for (int e = 0; e < 4; ++e) t4[e] *= b4[e];
        put_quad<M>(ta, p, t4);
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int vt = 2 * pw + h2;
        f32x4 acc = zero4();
#pragma unroll
        for (int ks = 0; ks < KS_C; ++ks) acc = M::mma(ta[ks], vb[h2][ks], acc);
        T* dst = wsU + (((size_t)(I0 + ii) * (V / 16) + vt) * 64 + lane) * 4;
        if constexpr (sizeof(T) == 2) {
          bf16x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = (bf16)acc[e];
          st_nt(reinterpret_cast<bf16x4*>(dst), x);
        } else {
          st_nt(reinterpret_cast<float4*>(dst), make_float4(acc[0], acc[1], acc[2], acc[3]));
        }
      }
    }
  }
}

// ------------------------------------------------------------------ inter-chunk scan + output
// Raw 4-element vector of T (U in accumulator order).
template <typename T>
struct Raw4;
template <>
struct Raw4<bf16> {
  typedef uint2 type;
  static __device__ __forceinline__ float get(const uint2& r, int e) {
    const uint32_t w = e < 2 ? r.x : r.y;
    return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
  }
};
template <>
struct Raw4<float> {
  typedef float4 type;
  static __device__ __forceinline__ float get(const float4& r, int e) {
    return e == 0 ? r.x : e == 1 ? r.y : e == 2 ? r.z : r.w;
  }
};

// KEEP: store every chunk's start state S0 and Delta into ws_B for the
// backward pass instead of forming outputs (Q~ Gamma and P are not read);
// the forward instantiation has none of it. SAVE: the forward (outputs formed)
// that also stores S0 and Delta, bit for bit what KEEP stores, so that a
// backward pass that follows need not run the recurrence again.
// NW waves per workgroup (4 or 8). Work of one chunk: the Delta and output
// tiles (token tile x value tile) are split over the waves, NW / 4 waves per
// token tile; the state tiles (channel tile x value tile) by channel tile.
// With 8 waves every SIMD holds two waves of the chain, which hides part of
// the LDS, matrix-core and barrier latency of the sequential recurrence.
template <typename T, int K, int V, int BV, bool KEEP, int NW, bool SAVE = false>
__global__ void __launch_bounds__(NW * 64)
chunk_scan_kernel(const T* __restrict__ ws_T, const float* __restrict__ ws_GL,
                  const int* __restrict__ ws_int, const int32_t* __restrict__ cu,
                  const float* h0, int N, int T_, int HV, int write_final, T* __restrict__ o,
                  float* ht, T* __restrict__ ws_B) {
  using M = MF<T>;
  using F = typename M::frag;
  using WsL = Ws<T, K, V>;
  using R4 = Raw4<T>;
  static_assert(!(KEEP && SAVE), "SAVE is a forward mode");
  constexpr bool STORE = KEEP || SAVE;  // S0 and Delta of every chunk into ws_B
  typedef typename R4::type raw4;
  constexpr int KS_K = K / M::KSTEP;
  constexpr int KS_C = kC / M::KSTEP;
  constexpr int NTH = NW * 64;
  constexpr int NTT = kC / 16;       // token tiles
  constexpr int WPT = NW / NTT;      // waves per token tile
  constexpr int RTW = K / 16 / NW;   // state row (channel) tiles per wave
  constexpr int CTB = BV / 16;       // column tiles per block
  constexpr int CPW = CTB / WPT;     // column tiles per wave for Delta and the output
  static_assert(RTW >= 1 && CTB >= 1 && CPW >= 1 && CTB % WPT == 0 && NW % NTT == 0, "tile shape");

  __shared__ F sS[2][KS_K][CTB][64];  // S as B fragments (contraction over channels), 2 buffers
  __shared__ F sD[2][KS_C][CTB][64];  // Delta as B fragments (contraction over tokens), 2 buffers

  // 1-D grid (scan_grid): groups of 8 chains x all V blocks, block vb of chain
  // c being workgroup (c / 8) * 8 * NVB + vb * 8 + c % 8, so that every block
  // of a chain lands on the same XCD (workgroups are dealt to the 8 XCDs in
  // turn) and all of them are dispatched together
  constexpr int NVB = V / BV;
  const int grp = (int)blockIdx.x / (8 * NVB), rem = (int)blockIdx.x % (8 * NVB);
  const int cl = grp * 8 + rem % 8;
  if (cl >= N * HV) return;
  // packed batches: sequences in the chunk table's scan order (longest first)
  const int n = cu ? ws_int[2 + N + cl / HV] : cl / HV, hv = cl % HV, vb = rem / 8;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  // token tile and first value tile of this wave's Delta / output tiles
  const int tt = wave % NTT, ct0 = WPT == 1 ? 0 : (wave / NTT) * CPW;
  int64_t bos;
  int len;
  seq_range(cu, n, T_, &bos, &len);
  int cbeg, cend;
  if (cu == nullptr) {
    const int nc = (T_ + kC - 1) / kC;
    cbeg = n * nc;
    cend = cbeg + nc;
  } else {
    cbeg = ws_int[1 + n];
    cend = ws_int[2 + n];
  }
  const size_t st_base = ((size_t)n * HV + hv) * (size_t)K * V;
  const int col_base = vb * BV;

  if (len == 0) {
    if (!write_final || (h0 == ht && h0 != nullptr)) return;
    for (int e = tid; e < K * BV; e += NTH) {
      const int r = e / BV, c = col_base + e % BV;
      const size_t off = st_base + (size_t)r * V + c;
      uint32_t bits = h0 ? reinterpret_cast<const uint32_t*>(h0)[off] : 0u;
      reinterpret_cast<uint32_t*>(ht)[off] = bits;
    }
    return;
  }

  // per-chunk operands of this wave, loaded one chunk ahead
  constexpr int NPL = WsL::PL > 0 ? KS_C : 1;  // P low parts (bf16 only)
  struct Ops {
    F w[KS_K], qg[KS_K], p[KS_C], pl[NPL], kh[RTW][KS_C];
    raw4 u[CPW];
    float4 gl[RTW];
  };
  // part < 0: every operand; else one of four batches (W; Q~Gamma; P; Khat^T,
  // gate row, U), issued at four points of the previous chunk's step
  auto load_ops = [&](int cj, Ops& op, int part = -1) __attribute__((always_inline)) {
    const size_t ch = (size_t)cj * HV + hv;
    const T* wsW = ws_T + ch * WsL::elems;
    const F* fW = reinterpret_cast<const F*>(wsW);
    const F* fQG = reinterpret_cast<const F*>(wsW + WsL::W);
    const F* fKH = reinterpret_cast<const F*>(wsW + WsL::W + WsL::QG);
    const F* fP = reinterpret_cast<const F*>(wsW + WsL::W + WsL::QG + WsL::KH);
    const F* fPL = reinterpret_cast<const F*>(wsW + WsL::W + WsL::QG + WsL::KH + WsL::P);
    const T* wsU = wsW + WsL::W + WsL::QG + WsL::KH + WsL::P + WsL::PL;
    if (part < 0 || part == 0) {
#pragma unroll
      for (int ks = 0; ks < KS_K; ++ks) op.w[ks] = fW[((size_t)tt * KS_K + ks) * 64 + lane];
    }
    if constexpr (!KEEP) {
      if (part < 0 || part == 1) {
#pragma unroll
        for (int ks = 0; ks < KS_K; ++ks) op.qg[ks] = fQG[((size_t)tt * KS_K + ks) * 64 + lane];
      }
      if (part < 0 || part == 2) {
#pragma unroll
        for (int ks = 0; ks < KS_C; ++ks) {
          op.p[ks] = fP[((size_t)tt * KS_C + ks) * 64 + lane];
          if constexpr (WsL::PL > 0) op.pl[ks] = fPL[((size_t)tt * KS_C + ks) * 64 + lane];
        }
      }
    }
    if (part < 0 || part == 3) {
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt) {
#pragma unroll
        for (int ks = 0; ks < KS_C; ++ks)
          op.kh[rt][ks] = fKH[((size_t)(RTW * wave + rt) * KS_C + ks) * 64 + lane];
        op.gl[rt] = *reinterpret_cast<const float4*>(ws_GL + ch * K + 16 * (RTW * wave + rt) + 4 * g);
      }
#pragma unroll
      for (int cc = 0; cc < CPW; ++cc) {
        const int vt = (col_base >> 4) + ct0 + cc;
        op.u[cc] = *reinterpret_cast<const raw4*>(wsU + (((size_t)tt * (V / 16) + vt) * 64 + lane) * 4);
      }
    }
  };

  // S accumulators: wave owns channel tiles RTW*wave .. RTW*wave+RTW-1
  f32x4 S[RTW][CTB];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
    for (int ct = 0; ct < CTB; ++ct) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 16 * (RTW * wave + rt) + 4 * g + e;
        const int col = col_base + 16 * ct + l16;
        S[rt][ct][e] = h0 ? h0[st_base + (size_t)c * V + col] : 0.f;
      }
    }

  // Output rows of token tile tt of a chunk whose S0 and Delta sit in LDS
  // buffer `buf`: O = (Q~ Gamma) S0 + P Delta, formed transposed
  // (O^T = S0^T (Q~ Gamma)^T + Delta^T P^T): the B fragments of S0 and Delta are
  // the A fragments of their transposes and vice versa, and the O^T
  // accumulator gives each lane 4 consecutive value columns of one token,
  // written as one 8- or 16-byte store. It runs one chunk late, next to the
  // following chunk's W S products, so it stays off the recurrence's path.
  // What the deferred output needs is kept in registers: Q~ Gamma and P of
  // the chunk and, for bf16 with up to 32 value columns (CACHE), the S0 /
  // Delta fragments its step already read from LDS; otherwise they would not
  // fit the register file and are read again from the chunk's LDS buffers
  // (intact until the step after next).
  constexpr bool CACHE = !KEEP && sizeof(T) == 2 && CTB <= 2;
  struct OutOps {
    F qg[KS_K], p[KS_C], pl[NPL];
    F sf[CACHE ? KS_K : 1][CACHE ? CPW : 1];  // S0 fragments (value tiles ct0..)
    F df[CACHE ? KS_C : 1][CACHE ? CPW : 1];  // Delta fragments (value tiles ct0..)
  };
  auto output_mma = [&](const OutOps& op, const int buf, f32x4* OT) __attribute__((always_inline)) {
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc) OT[cc] = zero4();
#pragma unroll
    for (int ks = 0; ks < KS_K; ++ks)
#pragma unroll
      for (int cc = 0; cc < CPW; ++cc) {
        if constexpr (CACHE) OT[cc] = M::mma(op.sf[ks][cc], op.qg[ks], OT[cc]);
        else OT[cc] = M::mma(sS[buf][ks][ct0 + cc][lane], op.qg[ks], OT[cc]);
      }
#pragma unroll
    for (int ks = 0; ks < KS_C; ++ks)
#pragma unroll
      for (int cc = 0; cc < CPW; ++cc) {
        F dfr;
        if constexpr (CACHE) dfr = op.df[ks][cc];
        else dfr = sD[buf][ks][ct0 + cc][lane];
        OT[cc] = M::mma(dfr, op.p[ks], OT[cc]);
        if constexpr (WsL::PL > 0) OT[cc] = M::mma(dfr, op.pl[ks], OT[cc]);
      }
  };
  auto store_out = [&](const f32x4* OT, const int cj) __attribute__((always_inline)) {
    const int cidx = cj - cbeg;
    const int64_t t0 = bos + (int64_t)cidx * kC;
    const int L = min(kC, len - cidx * kC);
    const int i = 16 * tt + l16;
    if (i < L && o) {
      T* orow = o + ((t0 + i) * HV + hv) * V + col_base + 16 * ct0 + 4 * g;
#pragma unroll
      for (int cc = 0; cc < CPW; ++cc) {
        if constexpr (sizeof(T) == 2) {
          bf16x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = (bf16)OT[cc][e];
          *reinterpret_cast<bf16x4*>(orow + 16 * cc) = x;
        } else {
          *reinterpret_cast<float4*>(orow + 16 * cc) = make_float4(OT[cc][0], OT[cc][1], OT[cc][2], OT[cc][3]);
        }
      }
    }
  };
  auto output = [&](const OutOps& op, const int cj, const int buf) __attribute__((always_inline)) {
    if constexpr (KEEP) return;  // the backward's recurrence forms no output
    f32x4 OT[CPW];
    output_mma(op, buf, OT);
    store_out(OT, cj);
  };
  // one chunk of the recurrence with operands `cur`, LDS buffer `buf`; the
  // previous chunk's output (registers `prv`) is formed after the first
  // barrier, and this chunk's output registers are collected in `mine`
  // The next chunk's operands (chunk cn into `nxt`): with an output and 32 or
  // more value columns, requested in four batches spread over the step (a wave
  // stalls when it issues more loads than the compute unit's memory path has
  // room for, and a stall between phases leaves the phases running:
  // 138 -> 131 us dense, 651 -> 578 us varlen); the short steps of narrower
  // blocks and of the backward's recurrence need every operand a whole step
  // ahead and take them at once.
  constexpr bool SPLIT = !KEEP && BV >= 32;
  auto step = [&](const Ops& cur, const int cj, const int buf, OutOps& mine,
                  const OutOps& prv, const int cn, Ops& nxt) __attribute__((always_inline)) {
    const int cidx = cj - cbeg;
    const int64_t t0 = bos + (int64_t)cidx * kC;
    const int L = min(kC, len - cidx * kC);
    load_ops(cn, nxt, SPLIT ? 0 : -1);
    __builtin_amdgcn_sched_barrier(0);

    // backward support: keep the chunk's start state and Delta. With up to 32
    // columns the stores wait until after the second barrier (copies in
    // registers), so that they queue behind the step's loads, not in front of them
    constexpr bool LATE = STORE && BV <= 32;
    f32x4 s0c[LATE ? RTW : 1][LATE ? CTB : 1];
    f32x4 dc[LATE ? CPW : 1];
    if constexpr (LATE) {
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
        for (int ct = 0; ct < CTB; ++ct) s0c[rt][ct] = S[rt][ct];
    } else if constexpr (STORE) {
      T* st = ws_B + ((size_t)cj * HV + hv) * WsB<T, K, V>::elems + WsB<T, K, V>::oS0;
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
        for (int ct = 0; ct < CTB; ++ct)
          store4<T>(st + il4(16 * (RTW * wave + rt) + 4 * g, col_base + 16 * ct + l16, V),
                    S[rt][ct][0], S[rt][ct][1], S[rt][ct][2], S[rt][ct][3]);
    }
    // (1) publish S as B fragments: k-step ks is owned by the wave holding its channels
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const int tileK = RTW * wave + rt;  // channel tile
#pragma unroll
      for (int ct = 0; ct < CTB; ++ct) {
        if constexpr (M::KSTEP == 32) {
          // channel tile pair (2ks, 2ks+1) -> k-step ks; this tile fills half a fragment
          const int ks = tileK >> 1, half = tileK & 1;
          bf16x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = (bf16)S[rt][ct][e];
          *(reinterpret_cast<bf16x4*>(&sS[buf][ks][ct][lane]) + half) = x;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            F f;
            M::set(f, 0, S[rt][ct][e]);
            sS[buf][4 * tileK + e][ct][lane] = f;
          }
        }
      }
    }
    __syncthreads();

    if constexpr (SPLIT) {
      load_ops(cn, nxt, 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // 32-column blocks: the deferred output's stores wait until after the
    // second barrier, behind the step's loads (dense scan 120 -> 112 us; with 16
    // and 64 columns measured slower and not used)
    constexpr bool LATE_OUT = !KEEP && BV == 32;
    f32x4 OTd[CPW];
    if constexpr (LATE_OUT) {
      if (cj > cbeg) output_mma(prv, buf ^ 1, OTd);
    } else {
      if (cj > cbeg) output(prv, cj - 1, buf ^ 1);
    }
    if constexpr (SPLIT) {
      __builtin_amdgcn_sched_barrier(0);
      load_ops(cn, nxt, 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    // (2) Delta = U - W S for token tile tt, value tiles ct0..ct0+CPW-1
    f32x4 D[CPW];
    {
      f32x4 ws_[CPW];
#pragma unroll
      for (int cc = 0; cc < CPW; ++cc) ws_[cc] = zero4();
#pragma unroll
      for (int ks = 0; ks < KS_K; ++ks) {
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc) {
          const F sfr = sS[buf][ks][ct0 + cc][lane];
          if constexpr (CACHE) mine.sf[ks][cc] = sfr;
          ws_[cc] = M::mma(cur.w[ks], sfr, ws_[cc]);
        }
      }
#pragma unroll
      for (int cc = 0; cc < CPW; ++cc)
#pragma unroll
        for (int e = 0; e < 4; ++e) D[cc][e] = R4::get(cur.u[cc], e) - ws_[cc][e];
    }
    if constexpr (LATE) {
#pragma unroll
      for (int cc = 0; cc < CPW; ++cc) dc[cc] = D[cc];
    } else if constexpr (STORE) {  // backward support: keep Delta
      T* dl = ws_B + ((size_t)cj * HV + hv) * WsB<T, K, V>::elems + WsB<T, K, V>::oDL;
#pragma unroll
      for (int cc = 0; cc < CPW; ++cc)
        store4<T>(dl + il4(16 * tt + 4 * g, col_base + 16 * (ct0 + cc) + l16, V), D[cc][0], D[cc][1],
                  D[cc][2], D[cc][3]);
    }
    // publish Delta as B fragments (contraction over tokens)
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc) {
      const int ct = ct0 + cc;
      if constexpr (M::KSTEP == 32) {
        const int ks = tt >> 1, half = tt & 1;
        bf16x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (bf16)D[cc][e];
        *(reinterpret_cast<bf16x4*>(&sD[buf][ks][ct][lane]) + half) = x;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          F f;
          M::set(f, 0, D[cc][e]);
          sD[buf][4 * tt + e][ct][lane] = f;
        }
      }
    }
    __syncthreads();
    if constexpr (SPLIT) {
      load_ops(cn, nxt, 3);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (LATE_OUT) {
      if (cj > cbeg) store_out(OTd, cj - 1);
    }
    F dall[KS_C][CTB];
#pragma unroll
    for (int ks = 0; ks < KS_C; ++ks) {
#pragma unroll
      for (int ct = 0; ct < CTB; ++ct) dall[ks][ct] = sD[buf][ks][ct][lane];
#pragma unroll
      for (int cc = 0; cc < CPW; ++cc) {
        if constexpr (!CACHE) {
        } else if constexpr (WPT == 1) {
          mine.df[ks][cc] = dall[ks][cc];
        } else {  // select (no register-array indexing by a run-time value)
          F x = dall[ks][0];
#pragma unroll
          for (int ct = 1; ct < CTB; ++ct)
            if (ct == ct0 + cc) x = dall[ks][ct];
          mine.df[ks][cc] = x;
        }
      }
    }

    if constexpr (LATE) {
      T* st = ws_B + ((size_t)cj * HV + hv) * WsB<T, K, V>::elems + WsB<T, K, V>::oS0;
      T* dl = ws_B + ((size_t)cj * HV + hv) * WsB<T, K, V>::elems + WsB<T, K, V>::oDL;
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
        for (int ct = 0; ct < CTB; ++ct)
          store4<T>(st + il4(16 * (RTW * wave + rt) + 4 * g, col_base + 16 * ct + l16, V),
                    s0c[rt][ct][0], s0c[rt][ct][1], s0c[rt][ct][2], s0c[rt][ct][3]);
#pragma unroll
      for (int cc = 0; cc < CPW; ++cc)
        store4<T>(dl + il4(16 * tt + 4 * g, col_base + 16 * (ct0 + cc) + l16, V), dc[cc][0], dc[cc][1],
                  dc[cc][2], dc[cc][3]);
    }
    // (3) S = Diag(Gamma_last) S + Khat^T Delta for the wave's channel tiles
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const float gl[4] = {cur.gl[rt].x, cur.gl[rt].y, cur.gl[rt].z, cur.gl[rt].w};
#pragma unroll
      for (int ct = 0; ct < CTB; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[rt][ct][e] *= gl[e];
#pragma unroll
      for (int ks = 0; ks < KS_C; ++ks)
#pragma unroll
        for (int ct = 0; ct < CTB; ++ct) S[rt][ct] = M::mma(cur.kh[rt][ks], dall[ks][ct], S[rt][ct]);
    }
    if constexpr (!KEEP) {
#pragma unroll
      for (int ks = 0; ks < KS_K; ++ks) mine.qg[ks] = cur.qg[ks];
#pragma unroll
      for (int ks = 0; ks < KS_C; ++ks) {
        mine.p[ks] = cur.p[ks];
        if constexpr (WsL::PL > 0) mine.pl[ks] = cur.pl[ks];
      }
    }
  };

  // two operand sets, unrolled by two so the next chunk's loads stay in flight
  // (loads are unconditional -- the last chunk is simply fetched again -- so
  // the number of loads in flight is the same on every path); two output
  // register sets alternate the same way
  Ops opA, opB;
  OutOps oA, oB;
  load_ops(cbeg, opA);
  for (int cj = cbeg;; cj += 2) {
    step(opA, cj, 0, oA, oB, min(cj + 1, cend - 1), opB);
    if (cj + 1 >= cend) {
      output(oA, cj, 0);
      break;
    }
    step(opB, cj + 1, 1, oB, oA, min(cj + 2, cend - 1), opA);
    if (cj + 2 >= cend) {
      output(oB, cj + 1, 1);
      break;
    }
  }

  if (write_final) {
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int ct = 0; ct < CTB; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = 16 * (RTW * wave + rt) + 4 * g + e;
          const int col = col_base + 16 * ct + l16;
          ht[st_base + (size_t)c * V + col] = S[rt][ct][e];
        }
  }
}

// ------------------------------------------------------------------ host side
inline int64_t max_chunks(const kda_dims& d, bool varlen) {
  const int64_t per = (d.T + kC - 1) / kC;
  return varlen ? per + d.N : per * d.B;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workgroups of a scan over `chains` chains in V blocks of bv columns (the
// 1-D grid of chunk_scan_kernel and chunk_rev_scan_kernel: groups of 8 chains
// times V / bv blocks).
inline unsigned scan_grid(int64_t chains, int V, int bv) {
  return (unsigned)(((chains + 7) / 8) * 8 * (V / bv));
}

inline int scan_block_v(int64_t chains, int V, int cus) {
  int bv = 64;
  while (bv > 16 && chains * (V / bv) < cus) bv >>= 1;
  return bv > V ? V : bv;
}

// Chunk table of a varlen batch (chunk_table_kernel), enqueued on `s`.
hipError_t launch_chunk_table(const int32_t* cu, int N, int* ws_int, int max_chunks, hipStream_t s);

}  // namespace kda
