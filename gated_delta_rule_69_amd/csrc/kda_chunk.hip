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
// r = first token of the row tile. Inside a diagonal tile the pairs are split
// by the highest bit in which the local indices differ (levels 3..0, each
// with its own reference), plus the exact diagonal i == j. This keeps
// unbounded gates (chunk-local cumsums far below -126 in log2 units) exact.
#include <algorithm>

#include "kda_common.h"

namespace kda {

constexpr int kC = 64;          // chunk size
constexpr int kThreads = 256;   // 4 waves

// ------------------------------------------------------------------ chunk table
// ws_int layout: [0] total chunks, [1 .. N+1] first chunk of each sequence
// (seq_off, N+1 entries), then chunk_seq[max_chunks].
__global__ void __launch_bounds__(1024)
chunk_table_kernel(const int32_t* __restrict__ cu, int N, int* __restrict__ ws_int,
                   int max_chunks) {
  __shared__ int s_scan[1024];
  int* total = ws_int;
  int* seq_off = ws_int + 1;
  int* chunk_seq = ws_int + 2 + N;
  int carry = 0;
  for (int base = 0; base < N; base += 1024) {
    const int n = base + threadIdx.x;
    int cnt = 0;
    if (n < N) {
      const int len = cu[n + 1] - cu[n];
      cnt = len > 0 ? (len + kC - 1) / kC : 0;
    }
    s_scan[threadIdx.x] = cnt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      int x = threadIdx.x >= off ? s_scan[threadIdx.x - off] : 0;
      __syncthreads();
      s_scan[threadIdx.x] += x;
      __syncthreads();
    }
    const int incl = s_scan[threadIdx.x];
    const int excl = incl - cnt;
    if (n < N) {
      seq_off[n] = carry + excl;
      for (int c = 0; c < cnt; ++c) {
        const int j = carry + excl + c;
        if (j < max_chunks) chunk_seq[j] = n;
      }
    }
    carry += s_scan[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    seq_off[N] = carry;
    total[0] = carry;
  }
}

// ------------------------------------------------------------------ workspace layout
template <typename T, int K, int V>
struct Ws {
  // per (chunk, value head), in elements of T unless noted
  static constexpr size_t W = (size_t)kC * K;    // W fragments   [4][K/KSTEP][64][PER]
  static constexpr size_t QG = (size_t)kC * K;   // Q~*Gamma      [4][K/KSTEP][64][PER]
  static constexpr size_t KH = (size_t)K * kC;   // Khat^T        [K/16][C/KSTEP][64][PER]
  static constexpr size_t P = (size_t)kC * kC;   // P             [4][C/KSTEP][64][PER]
  static constexpr size_t U = (size_t)kC * V;    // U accum order [4][V/16][64][4]
  static constexpr size_t elems = W + QG + KH + P + U;
  static constexpr size_t bytes_T = elems * sizeof(T);
  static constexpr size_t bytes_GL = (size_t)K * sizeof(float);  // Gamma_last (FP32)
};

struct ChunkGeo {
  int ok;        // 0: no such chunk (grid over-provisioned)
  int n;         // sequence
  int64_t t0;    // flat index of the chunk's first token
  int L;         // tokens in the chunk (1..64)
};

__device__ __forceinline__ ChunkGeo chunk_geo(int j, const int32_t* cu, const int* ws_int, int N,
                                              int T) {
  ChunkGeo r{0, 0, 0, 0};
  if (cu == nullptr) {
    const int nc = (T + kC - 1) / kC;
    const int n = j / nc, c = j % nc;
    if (n >= N) return r;
    r.ok = 1;
    r.n = n;
    r.t0 = (int64_t)n * T + (int64_t)c * kC;
    r.L = min(kC, T - c * kC);
  } else {
    if (j >= ws_int[0]) return r;
    const int n = ws_int[2 + N + j];
    const int c = j - ws_int[1 + n];
    const int bos = cu[n], len = cu[n + 1] - bos;
    r.ok = 1;
    r.n = n;
    r.t0 = bos + (int64_t)c * kC;
    r.L = min(kC, len - c * kC);
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
  static constexpr int BTS = kC + TP;             // B^T and (bV)^T row stride
  static constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t R1 = cmax((size_t)kC * GS * 4, (size_t)V * BTS * sizeof(T));
  static constexpr size_t R2 = cmax((size_t)kC * KSTR * sizeof(T), (size_t)K * BTS * sizeof(T));
  static constexpr size_t R3 = cmax((size_t)kC * KSTR * sizeof(T), (size_t)kC * AS * 4);
  static constexpr size_t total = R1 + R2 + R3 + kC * 4;
};

template <typename T, int K, int V>
__global__ void __launch_bounds__(kThreads, 2)
chunk_intra_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                   const float* __restrict__ gate, const T* __restrict__ beta,
                   const int32_t* __restrict__ cu, const int* __restrict__ ws_int, int N, int T_,
                   int H, int HV, float scale, T* __restrict__ ws_T, float* __restrict__ ws_GL) {
  using M = MF<T>;
  using F = typename M::frag;
  using Lds = IntraLds<T, K, V>;
  using WsL = Ws<T, K, V>;
  constexpr int KS_K = K / M::KSTEP;
  constexpr int KS_C = kC / M::KSTEP;
  constexpr int GS = Lds::GS, KSTR = Lds::KSTR, AS = Lds::AS, BTS = Lds::BTS;

  extern __shared__ __align__(16) char smem[];
  float* sG = reinterpret_cast<float*>(smem);                       // R1: G2 [C][GS]
  T* sVT = reinterpret_cast<T*>(smem);                              // R1 later: (b v)^T [V][BTS]
  T* sK = reinterpret_cast<T*>(smem + Lds::R1);                     // R2: k [C][KSTR]
  T* sBT = reinterpret_cast<T*>(smem + Lds::R1);                    // R2 later: B^T [K][BTS]
  T* sQ = reinterpret_cast<T*>(smem + Lds::R1 + Lds::R2);           // R3: q [C][KSTR]
  float* sA = reinterpret_cast<float*>(smem + Lds::R1 + Lds::R2);   // R3 later: A, then T [C][AS]
  float* sBeta = reinterpret_cast<float*>(smem + Lds::R1 + Lds::R2 + Lds::R3);

  const ChunkGeo geo = chunk_geo(blockIdx.x, cu, ws_int, N, T_);
  if (!geo.ok) return;
  const int hv = blockIdx.y;
  const int h = hv / (HV / H);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int L = geo.L;
  const int64_t t0 = geo.t0;
  const size_t ch = (size_t)blockIdx.x * HV + hv;

  // ---- 1. stage G2, k, q, beta; prefetch v into registers
  for (int e = tid; e < kC * K; e += kThreads) {
    const int i = e / K, c = e - i * K;
    const int ii = i < L ? i : L - 1;  // pad rows repeat the last gate row
    sG[i * GS + c] = gate[((t0 + ii) * HV + hv) * K + c];
    T kv = from_f32<T>(0.f), qv = from_f32<T>(0.f);
    if (i < L) {
      kv = k[((t0 + i) * H + h) * K + c];
      qv = q[((t0 + i) * H + h) * K + c];
    }
    sK[i * KSTR + c] = kv;
    sQ[i * KSTR + c] = qv;
  }
  if (tid < kC) sBeta[tid] = tid < L ? to_f32(beta[(t0 + tid) * HV + hv]) : 0.f;
  constexpr int VPT = kC * V / kThreads;  // v elements per thread
  float vreg[VPT];
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int e = tid + u * kThreads;
    const int i = e / V, c = e - i * V;
    vreg[u] = i < L ? to_f32(v[((t0 + i) * HV + hv) * V + c]) : 0.f;
  }
  __syncthreads();

  // ---- 2. A^T and P^T tiles (column tile I = wave; row tiles J <= I)
  const int I = wave;
  f32x4 accA[4], accP[4];  // tiles J < I (off-diagonal)
  f32x4 dA = zero4(), dP = zero4();  // tile J == I
#pragma unroll
  for (int J = 0; J < 4; ++J) accA[J] = accP[J] = zero4();
  {
    const int icol = 16 * I + l16;  // B operand column (token i)
    // off-diagonal tiles: reference token r = 16 I
    const int r = 16 * I;
#pragma unroll
    for (int J = 0; J < 3; ++J) {
      if (J >= I) break;
      const int jrow = 16 * J + l16;  // A operand row (token j)
#pragma unroll
      for (int ks = 0; ks < KS_K; ++ks) {
        F ra, lk, lq;
#pragma unroll
        for (int jj = 0; jj < M::PER; ++jj) {
          const int c = M::kidx(ks, g, jj);
          const float gr = sG[r * GS + c];
          M::set(ra, jj, to_f32(sK[jrow * KSTR + c]) * exp2f(gr - sG[jrow * GS + c]));
          const float e = exp2f(sG[icol * GS + c] - gr);
          M::set(lk, jj, to_f32(sK[icol * KSTR + c]) * e);
          M::set(lq, jj, to_f32(sQ[icol * KSTR + c]) * scale * e);
        }
        accA[J] = M::mma(ra, lk, accA[J]);
        accP[J] = M::mma(ra, lq, accP[J]);
      }
    }
    // diagonal tile (I, I): levels 3..0 then the exact diagonal
    const int jl = l16, il = l16;
    const int jrow = 16 * I + jl;
#pragma unroll
    for (int lev = 3; lev >= -1; --lev) {
      f32x4 xa = zero4(), xp = zero4();
      const bool rowOn = lev < 0 || ((jl >> lev) & 1) == 0;
      const bool colOn = lev < 0 || ((il >> lev) & 1) == 1;
      const int rr = lev < 0 ? 0 : 16 * I + ((((jl >> lev) | 1)) << lev);  // ref for row j
      const int rc = lev < 0 ? 0 : 16 * I + ((il >> lev) << lev);          // ref for col i
#pragma unroll
      for (int ks = 0; ks < KS_K; ++ks) {
        F ra, lk, lq;
#pragma unroll
        for (int jj = 0; jj < M::PER; ++jj) {
          const int c = M::kidx(ks, g, jj);
          float a = 0.f, bk = 0.f, bq = 0.f;
          if (lev < 0) {
            a = to_f32(sK[jrow * KSTR + c]);
            bq = to_f32(sQ[icol * KSTR + c]) * scale;
          } else {
            if (rowOn) a = to_f32(sK[jrow * KSTR + c]) * exp2f(sG[rr * GS + c] - sG[jrow * GS + c]);
            if (colOn) {
              const float e = exp2f(sG[icol * GS + c] - sG[rc * GS + c]);
              bk = to_f32(sK[icol * KSTR + c]) * e;
              bq = to_f32(sQ[icol * KSTR + c]) * scale * e;
            }
          }
          M::set(ra, jj, a);
          M::set(lk, jj, bk);
          M::set(lq, jj, bq);
        }
        if (lev >= 0) xa = M::mma(ra, lk, xa);
        xp = M::mma(ra, lq, xp);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int jr = 4 * g + e;  // local row j of this accumulator element
        bool valid;
        if (lev < 0) valid = (jr == il);
        else valid = ((il >> (lev + 1)) == (jr >> (lev + 1))) && ((il >> lev) & 1) && !((jr >> lev) & 1);
        if (valid) {
          dA[e] += xa[e];
          dP[e] += xp[e];
        }
      }
    }
  }

  T* wsW = ws_T + ch * WsL::elems;
  T* wsQG = wsW + WsL::W;
  T* wsKH = wsQG + WsL::QG;
  T* wsP = wsKH + WsL::KH;
  T* wsU = wsP + WsL::P;
  float* wsGL = ws_GL + ch * K;

  // ---- 3. P fragments (rows i of tile I, contraction over j): accumulators of P^T
#pragma unroll
  for (int ks = 0; ks < KS_C; ++ks) {
    F f;
#pragma unroll
    for (int jj = 0; jj < M::PER; ++jj) {
      const int tile = (M::KSTEP == 32) ? (2 * ks + (jj >> 2)) : (ks >> 2);
      const int el = (M::KSTEP == 32) ? (jj & 3) : (ks & 3);
      float x = 0.f;
#pragma unroll
      for (int J = 0; J < 4; ++J)
        if (J == tile) x = (J < I) ? accP[J][el] : (J == I ? dP[el] : 0.f);
      M::set(f, jj, x);
    }
    reinterpret_cast<F*>(wsP)[((size_t)I * KS_C + ks) * 64 + lane] = f;
  }
  // ---- 4. Q~ * Gamma fragments (rows i of tile I, contraction over channels)
  {
    const int i = 16 * I + l16;
#pragma unroll
    for (int ks = 0; ks < KS_K; ++ks) {
      F f;
#pragma unroll
      for (int jj = 0; jj < M::PER; ++jj) {
        const int c = M::kidx(ks, g, jj);
        M::set(f, jj, to_f32(sQ[i * KSTR + c]) * scale * exp2f(sG[i * GS + c]));
      }
      reinterpret_cast<F*>(wsQG)[((size_t)I * KS_K + ks) * 64 + lane] = f;
    }
  }
  // ---- 5. Khat^T fragments (rows = channels, contraction over tokens j)
  for (int rt = wave; rt < K / 16; rt += 4) {
    const int c = 16 * rt + l16;
    const float gl = sG[(L - 1) * GS + c];
#pragma unroll
    for (int ks = 0; ks < KS_C; ++ks) {
      F f;
#pragma unroll
      for (int jj = 0; jj < M::PER; ++jj) {
        const int j = M::kidx(ks, g, jj);
        M::set(f, jj, to_f32(sK[j * KSTR + c]) * exp2f(gl - sG[j * GS + c]));
      }
      reinterpret_cast<F*>(wsKH)[((size_t)rt * KS_C + ks) * 64 + lane] = f;
    }
  }
  if (tid < K) wsGL[tid] = exp2f(sG[(L - 1) * GS + tid]);
  __syncthreads();  // q is dead: R3 becomes A

  // ---- 6. A = beta_i * (A^T accumulators)^T into LDS, zero elsewhere
  {
    const int i = 16 * I + l16;
    const float b = sBeta[i];
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (J < I) x = make_float4(b * accA[J][0], b * accA[J][1], b * accA[J][2], b * accA[J][3]);
      else if (J == I) x = make_float4(b * dA[0], b * dA[1], b * dA[2], b * dA[3]);
      *reinterpret_cast<float4*>(&sA[i * AS + 16 * J + 4 * g]) = x;
    }
  }
  // B^T = (b_m k_mc 2^G2_mc)^T and (b v)^T values into registers (G2 and k still live)
  constexpr int BPT = kC * K / kThreads;
  float breg[BPT];
#pragma unroll
  for (int u = 0; u < BPT; ++u) {
    const int e = tid + u * kThreads;
    const int m = e / K, c = e - m * K;
    breg[u] = sBeta[m] * to_f32(sK[m * KSTR + c]) * exp2f(sG[m * GS + c]);
  }
  __syncthreads();  // G2 and k are dead: R1 becomes (b v)^T, R2 becomes B^T
#pragma unroll
  for (int u = 0; u < BPT; ++u) {
    const int e = tid + u * kThreads;
    const int m = e / K, c = e - m * K;
    sBT[c * BTS + m] = from_f32<T>(breg[u]);
  }
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int e = tid + u * kThreads;
    const int m = e / V, c = e - m * V;
    sVT[c * BTS + m] = from_f32<T>(sBeta[m] * vreg[u]);
  }

  // ---- 7. T = (I + A)^-1 in FP32, in place
  // 7a. diagonal 16x16 blocks by forward substitution (wave d, lane = column)
  if (lane < 16) {
    const int d = wave, jj = lane;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = (i == jj) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m) s -= sA[(16 * d + i) * AS + 16 * d + m] * x[m];
      x[i] = s;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sA[(16 * d + i) * AS + 16 * d + jj] = x[i];
  }
  __syncthreads();
  // 7b. block rows: T_IJ = -T_II * sum_{M=J}^{I-1} A_IM T_MJ, scratch in the upper block (J, I)
  for (int Ib = 1; Ib < 4; ++Ib) {
    const int Jb = wave;
    const int a = l16, b0 = 4 * g;  // lane owns row a, columns b0..b0+3 of the block
    if (Jb < Ib) {
      float xs[4] = {0.f, 0.f, 0.f, 0.f};
      for (int Mb = Jb; Mb < Ib; ++Mb) {
#pragma unroll
        for (int p = 0; p < 16; ++p) {
          const float aim = sA[(16 * Ib + a) * AS + 16 * Mb + p];
#pragma unroll
          for (int e = 0; e < 4; ++e) xs[e] += aim * sA[(16 * Mb + p) * AS + 16 * Jb + b0 + e];
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sA[(16 * Jb + a) * AS + 16 * Ib + b0 + e] = xs[e];
    }
    __syncthreads();
    if (Jb < Ib) {
      float ts[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < 16; ++p) {
        const float tii = sA[(16 * Ib + a) * AS + 16 * Ib + p];
#pragma unroll
        for (int e = 0; e < 4; ++e) ts[e] -= tii * sA[(16 * Jb + p) * AS + 16 * Ib + b0 + e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sA[(16 * Ib + a) * AS + 16 * Jb + b0 + e] = ts[e];
    }
    __syncthreads();
    if (Jb < Ib) {
#pragma unroll
      for (int e = 0; e < 4; ++e) sA[(16 * Jb + a) * AS + 16 * Ib + b0 + e] = 0.f;
    }
    __syncthreads();
  }

  // ---- 8. W^T = B^T T^T (rows channels, cols tokens of tile I) -> W fragments of row tile I
  {
    const int i = 16 * I + l16;
    f32x4 accW[K / 16];
#pragma unroll
    for (int ct = 0; ct < K / 16; ++ct) accW[ct] = zero4();
#pragma unroll
    for (int ks = 0; ks < KS_C; ++ks) {
      F tb;
#pragma unroll
      for (int jj = 0; jj < M::PER; ++jj) M::set(tb, jj, sA[i * AS + M::kidx(ks, g, jj)]);
#pragma unroll
      for (int ct = 0; ct < K / 16; ++ct) {
        const int c = 16 * ct + l16;
        F ba;
#pragma unroll
        for (int jj = 0; jj < M::PER; ++jj) M::set(ba, jj, to_f32(sBT[c * BTS + M::kidx(ks, g, jj)]));
        accW[ct] = M::mma(ba, tb, accW[ct]);
      }
    }
#pragma unroll
    for (int ks = 0; ks < KS_K; ++ks) {
      F f;
#pragma unroll
      for (int jj = 0; jj < M::PER; ++jj) {
        const int tile = (M::KSTEP == 32) ? (2 * ks + (jj >> 2)) : (ks >> 2);
        const int el = (M::KSTEP == 32) ? (jj & 3) : (ks & 3);
        M::set(f, jj, accW[tile][el]);
      }
      reinterpret_cast<F*>(wsW)[((size_t)I * KS_K + ks) * 64 + lane] = f;
    }
  }
  // ---- 9. U = T (b V) (rows tokens of tile I), stored in accumulator order
  {
    const int i = 16 * I + l16;
    f32x4 accU[V / 16];
#pragma unroll
    for (int vt = 0; vt < V / 16; ++vt) accU[vt] = zero4();
#pragma unroll
    for (int ks = 0; ks < KS_C; ++ks) {
      F ta;
#pragma unroll
      for (int jj = 0; jj < M::PER; ++jj) M::set(ta, jj, sA[i * AS + M::kidx(ks, g, jj)]);
#pragma unroll
      for (int vt = 0; vt < V / 16; ++vt) {
        const int c = 16 * vt + l16;
        F vb;
#pragma unroll
        for (int jj = 0; jj < M::PER; ++jj) M::set(vb, jj, to_f32(sVT[c * BTS + M::kidx(ks, g, jj)]));
        accU[vt] = M::mma(ta, vb, accU[vt]);
      }
    }
#pragma unroll
    for (int vt = 0; vt < V / 16; ++vt) {
      T* dst = wsU + (((size_t)I * (V / 16) + vt) * 64 + lane) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = from_f32<T>(accU[vt][e]);
    }
  }
}

// ------------------------------------------------------------------ inter-chunk scan + output
template <typename T, int K, int V, int BV>
__global__ void __launch_bounds__(kThreads)
chunk_scan_kernel(const T* __restrict__ ws_T, const float* __restrict__ ws_GL,
                  const int* __restrict__ ws_int, const int32_t* __restrict__ cu,
                  const float* h0, int N, int T_, int HV, int write_final, T* __restrict__ o,
                  float* ht) {
  using M = MF<T>;
  using F = typename M::frag;
  using WsL = Ws<T, K, V>;
  constexpr int KS_K = K / M::KSTEP;
  constexpr int KS_C = kC / M::KSTEP;
  constexpr int RTW = K / 64;   // state row tiles per wave
  constexpr int CTB = BV / 16;  // column tiles per block
  static_assert(RTW >= 1 && CTB >= 1, "tile shape");

  __shared__ F sS[2][KS_K][CTB][64];  // S as B fragments (contraction over channels), 2 buffers
  __shared__ F sD[KS_C][CTB][64];     // Delta as B fragments (contraction over tokens)

  const int n = blockIdx.x / HV, hv = blockIdx.x % HV, vb = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
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
    for (int e = tid; e < K * BV; e += kThreads) {
      const int r = e / BV, c = col_base + e % BV;
      const size_t off = st_base + (size_t)r * V + c;
      uint32_t bits = h0 ? reinterpret_cast<const uint32_t*>(h0)[off] : 0u;
      reinterpret_cast<uint32_t*>(ht)[off] = bits;
    }
    return;
  }

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

  int buf = 0;
  for (int cj = cbeg; cj < cend; ++cj) {
    const int cidx = cj - cbeg;
    const int64_t t0 = bos + (int64_t)cidx * kC;
    const int L = min(kC, len - cidx * kC);
    const size_t ch = (size_t)cj * HV + hv;
    const T* wsW = ws_T + ch * WsL::elems;
    const T* wsQG = wsW + WsL::W;
    const T* wsKH = wsQG + WsL::QG;
    const T* wsP = wsKH + WsL::KH;
    const T* wsU = wsP + WsL::P;
    const float* wsGL = ws_GL + ch * K;

    // (1) publish S as B fragments: k-step ks is owned by the wave holding its channels
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const int tileK = RTW * wave + rt;  // channel tile
#pragma unroll
      for (int ct = 0; ct < CTB; ++ct) {
        if constexpr (M::KSTEP == 32) {
          // channel tile pair (2ks, 2ks+1) -> k-step ks; this tile fills half a fragment
          const int ks = tileK >> 1, half = tileK & 1;
          bf16* dst = reinterpret_cast<bf16*>(&sS[buf][ks][ct][lane]) + 4 * half;
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[e] = (bf16)S[rt][ct][e];
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

    // (2) Delta = U - W S for token tile `wave`
    f32x4 D[CTB];
    {
      f32x4 ws_[CTB];
#pragma unroll
      for (int ct = 0; ct < CTB; ++ct) ws_[ct] = zero4();
#pragma unroll
      for (int ks = 0; ks < KS_K; ++ks) {
        const F a = reinterpret_cast<const F*>(wsW)[((size_t)wave * KS_K + ks) * 64 + lane];
#pragma unroll
        for (int ct = 0; ct < CTB; ++ct) ws_[ct] = M::mma(a, sS[buf][ks][ct][lane], ws_[ct]);
      }
#pragma unroll
      for (int ct = 0; ct < CTB; ++ct) {
        const int vt = (col_base >> 4) + ct;
        const T* u = wsU + (((size_t)wave * (V / 16) + vt) * 64 + lane) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) D[ct][e] = to_f32(u[e]) - ws_[ct][e];
      }
    }
    // publish Delta as B fragments (contraction over tokens)
#pragma unroll
    for (int ct = 0; ct < CTB; ++ct) {
      if constexpr (M::KSTEP == 32) {
        const int ks = wave >> 1, half = wave & 1;
        bf16* dst = reinterpret_cast<bf16*>(&sD[ks][ct][lane]) + 4 * half;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[e] = (bf16)D[ct][e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          F f;
          M::set(f, 0, D[ct][e]);
          sD[4 * wave + e][ct][lane] = f;
        }
      }
    }
    __syncthreads();

    // (3) output rows of token tile `wave`: O = (Q~ Gamma) S0 + P Delta
    {
      f32x4 O[CTB];
#pragma unroll
      for (int ct = 0; ct < CTB; ++ct) O[ct] = zero4();
#pragma unroll
      for (int ks = 0; ks < KS_K; ++ks) {
        const F a = reinterpret_cast<const F*>(wsQG)[((size_t)wave * KS_K + ks) * 64 + lane];
#pragma unroll
        for (int ct = 0; ct < CTB; ++ct) O[ct] = M::mma(a, sS[buf][ks][ct][lane], O[ct]);
      }
#pragma unroll
      for (int ks = 0; ks < KS_C; ++ks) {
        const F a = reinterpret_cast<const F*>(wsP)[((size_t)wave * KS_C + ks) * 64 + lane];
#pragma unroll
        for (int ct = 0; ct < CTB; ++ct) O[ct] = M::mma(a, sD[ks][ct][lane], O[ct]);
      }
#pragma unroll
      for (int ct = 0; ct < CTB; ++ct) {
        const int col = col_base + 16 * ct + l16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * wave + 4 * g + e;
          if (i < L) o[((t0 + i) * HV + hv) * V + col] = from_f32<T>(O[ct][e]);
        }
      }
    }
    // (4) S = Diag(Gamma_last) S + Khat^T Delta for the wave's channel tiles
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const int tileK = RTW * wave + rt;
      float gl[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) gl[e] = wsGL[16 * tileK + 4 * g + e];
#pragma unroll
      for (int ct = 0; ct < CTB; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[rt][ct][e] *= gl[e];
#pragma unroll
      for (int ks = 0; ks < KS_C; ++ks) {
        const F a = reinterpret_cast<const F*>(wsKH)[((size_t)tileK * KS_C + ks) * 64 + lane];
#pragma unroll
        for (int ct = 0; ct < CTB; ++ct) S[rt][ct] = M::mma(a, sD[ks][ct][lane], S[rt][ct]);
      }
    }
    buf ^= 1;
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

template <typename T, int K, int V>
size_t ws_bytes_t(const kda_dims& d, bool varlen) {
  const int64_t mc = max_chunks(d, varlen);
  size_t b = align256(sizeof(int) * (size_t)(2 + d.N + mc));
  b += align256((size_t)mc * d.HV * Ws<T, K, V>::bytes_T);
  b += align256((size_t)mc * d.HV * Ws<T, K, V>::bytes_GL);
  return b;
}

template <typename T, int K, int V>
hipError_t chunk_fwd_t(const kda_dims& d, const void* q, const void* k, const void* v,
                       const float* gate, const void* beta, const float* h0, const int32_t* cu,
                       int write_final, void* o, float* ht, void* ws, hipStream_t s) {
  const bool varlen = cu != nullptr;
  const int64_t mc = max_chunks(d, varlen);
  char* p = reinterpret_cast<char*>(ws);
  int* ws_int = reinterpret_cast<int*>(p);
  p += align256(sizeof(int) * (size_t)(2 + d.N + mc));
  T* ws_T = reinterpret_cast<T*>(p);
  p += align256((size_t)mc * d.HV * Ws<T, K, V>::bytes_T);
  float* ws_GL = reinterpret_cast<float*>(p);
  if (varlen) {
    hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(1024), 0, s, cu, d.N, ws_int, (int)mc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (mc > 0) {
    const size_t lds = IntraLds<T, K, V>::total;
    hipLaunchKernelGGL((chunk_intra_kernel<T, K, V>), dim3((unsigned)mc, (unsigned)d.HV),
                       dim3(kThreads), lds, s, (const T*)q, (const T*)k, (const T*)v, gate,
                       (const T*)beta, cu, ws_int, d.N, d.T, d.H, d.HV,
                       1.0f / sqrtf((float)K), ws_T, ws_GL);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  constexpr int BV = (V >= 128) ? 32 : 16;
  hipLaunchKernelGGL((chunk_scan_kernel<T, K, V, BV>), dim3((unsigned)(d.N * d.HV), V / BV),
                     dim3(kThreads), 0, s, (const T*)ws_T, (const float*)ws_GL,
                     (const int*)ws_int, cu, h0, d.N, d.T, d.HV, write_final, (T*)o, ht);
  return hipGetLastError();
}

}  // namespace kda

namespace kda_host {

template <typename T>
static size_t ws_bytes_dispatch(const kda_dims& d) {
  auto both = [&](auto f_dense, auto f_var) { return std::max(f_dense, f_var); };
  if (d.K == 64 && d.V == 64) return both(kda::ws_bytes_t<T, 64, 64>(d, false), kda::ws_bytes_t<T, 64, 64>(d, true));
  if (d.K == 64 && d.V == 128) return both(kda::ws_bytes_t<T, 64, 128>(d, false), kda::ws_bytes_t<T, 64, 128>(d, true));
  if (d.K == 128 && d.V == 64) return both(kda::ws_bytes_t<T, 128, 64>(d, false), kda::ws_bytes_t<T, 128, 64>(d, true));
  if (d.K == 128 && d.V == 128) return both(kda::ws_bytes_t<T, 128, 128>(d, false), kda::ws_bytes_t<T, 128, 128>(d, true));
  return 0;
}

size_t chunk_workspace_bytes(const kda_dims& d, kda_dtype dt, int chunk) {
  if (chunk != kda::kC) return 0;
  return dt == KDA_BF16 ? ws_bytes_dispatch<kda::bf16>(d) : ws_bytes_dispatch<float>(d);
}

template <typename T, int K, int V>
static hipError_t run_kv(const kda_dims& d, const void* q, const void* k, const void* v,
                         const float* gate, const void* beta, const float* h0,
                         const int32_t* cu, int write_final, void* o, float* ht, void* ws,
                         hipStream_t s) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kda::chunk_intra_kernel<T, K, V>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)kda::IntraLds<T, K, V>::total);
  if (e != hipSuccess) return e;
  return kda::chunk_fwd_t<T, K, V>(d, q, k, v, gate, beta, h0, cu, write_final, o, ht, ws, s);
}

template <typename T>
static hipError_t run_t(const kda_dims& d, const void* q, const void* k, const void* v,
                        const float* gate, const void* beta, const float* h0, const int32_t* cu,
                        int write_final, void* o, float* ht, void* ws, hipStream_t s) {
  if (d.K == 64 && d.V == 64) return run_kv<T, 64, 64>(d, q, k, v, gate, beta, h0, cu, write_final, o, ht, ws, s);
  if (d.K == 64 && d.V == 128) return run_kv<T, 64, 128>(d, q, k, v, gate, beta, h0, cu, write_final, o, ht, ws, s);
  if (d.K == 128 && d.V == 64) return run_kv<T, 128, 64>(d, q, k, v, gate, beta, h0, cu, write_final, o, ht, ws, s);
  if (d.K == 128 && d.V == 128) return run_kv<T, 128, 128>(d, q, k, v, gate, beta, h0, cu, write_final, o, ht, ws, s);
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_fwd(const kda_dims& d, kda_dtype dt, const void* q, const void* k,
                            const void* v, const float* gate, const void* beta,
                            const float* h0, const int32_t* cu, int write_final, void* o,
                            float* ht, void* ws, size_t /*ws_bytes*/, hipStream_t s) {
  if (dt == KDA_BF16) return run_t<kda::bf16>(d, q, k, v, gate, beta, h0, cu, write_final, o, ht, ws, s);
  return run_t<float>(d, q, k, v, gate, beta, h0, cu, write_final, o, ht, ws, s);
}

}  // namespace kda_host
