// Steps B1..B3: backward of the chunked KDA scan (chunk_kda backward).
//
// Per chunk, with the forward chunk form of kda_chunk_kernels.h, start state
// S0, upstream dO and dS1 (gradient of the chunk's end state):
//   dDelta = P^T dO + Khat dS1
//   dS0    = (Q~ Gamma)^T dO + Diag(gamma) dS1 - W^T dDelta          [reverse scan]
//   dP = tril(dO Delta^T), d(Q~Gamma) = dO S0^T, dKhat = Delta dS1^T,
//   dgamma = rowsum(dS1 * S0), dW = -dDelta S0^T,
//   dT = dDelta (bV)^T + dW (b Kg)^T, dv = b * T^T dDelta, dKg = b * T^T dW,
//   dA = tril(-T^T dT T^T, -1), dAbar = b * dA,
//   then the decay-weighted products
//     X1_ic = sum_j dAbar_ij k_jc 2^(G2_ic - G2_jc),  X2_jc = sum_i dAbar_ij k_ic 2^(G2_ic - G2_jc)
//     Y1_ic = sum_j dP_ij    k_jc 2^(G2_ic - G2_jc),  Y2_jc = sum_i dP_ij    q~_ic 2^(G2_ic - G2_jc)
//   give dk = X1 + X2 + Y2 + dKhat * e_L + dKg * Gamma, dq~ = Y1 + d(Q~Gamma) * Gamma and the
//   gradient of the natural-log cumulative gate, dG = k (X1 - X2) + q~ Y1 - k Y2 + d(Q~Gamma) Q~Gamma
//   - dKhat Khat + dKg Kg (+ the last row's colsum(dKhat Khat) + dgamma gamma); dg is its reverse
//   cumsum inside the chunk. This is the reverse of the gated-delta-rule chunk
//   pipeline the "[Fix] Use unit KDA gate scale when A_log is omitted" page
//   lists (chunk_gated_delta_rule_bwd_dhu, chunk_bwd_dv_local, chunk_bwd_dqkwg,
//   prepare_wy_repr_bwd), written out here for the per-channel gate.
//
// Kernels (one stream, no host synchronisation):
//   chunk_intra_kernel<..., BWD=true>  forward intra-chunk terms + P^T, Khat,
//                                      (Q~Gamma)^T, W^T fragments, Abar, T.
//   chunk_scan_kernel (ws_B != null)   forward recurrence keeping S0, Delta.
//   chunk_rev_scan_kernel              reverse recurrence of dS per chain;
//                                      keeps dS1 and dDelta per chunk; dh0.
//   chunk_bwd_local_kernel             one workgroup per (chunk, value head):
//                                      every local gradient above.
//   gva_reduce_kernel                  dq, dk summed over the value heads
//                                      sharing a qk head (fixed order).
#include "kda_chunk_kernels.h"

namespace kda {

// ------------------------------------------------------------------ reverse scan
template <typename T, int K, int V, int BV>
__global__ void __launch_bounds__(kThreads)
chunk_rev_scan_kernel(const T* __restrict__ ws_T, const float* __restrict__ ws_GL,
                      T* __restrict__ ws_B, const int* __restrict__ ws_int,
                      const int32_t* __restrict__ cu, const T* __restrict__ dO,
                      const float* __restrict__ dht, int N, int T_, int HV,
                      float* __restrict__ dh0) {
  using M = MF<T>;
  using F = typename M::frag;
  using WB = WsB<T, K, V>;
  constexpr int KS_K = K / M::KSTEP;
  constexpr int KS_C = kC / M::KSTEP;
  constexpr int QC = kC / 16;
  constexpr int RTW = K / 64;
  constexpr int CTB = BV / 16;
  constexpr int TP = 16 / (int)sizeof(T);
  constexpr int DS = BV + TP;  // dO staging row stride

  // double buffered by chunk parity: two barriers per chunk suffice
  __shared__ F sS[2][KS_K][CTB][64];  // dS1 as B fragments (contraction over channels)
  __shared__ F sD[2][KS_C][CTB][64];  // dDelta as B fragments (contraction over tokens)
  __shared__ __align__(16) T sdO[2][kC * DS];  // dO block of the chunk, row-major, staged a chunk ahead

  // 1-D grid, the forward scan's mapping (scan_grid)
  constexpr int NVB = V / BV;
  const int grp = (int)blockIdx.x / (8 * NVB), rem = (int)blockIdx.x % (8 * NVB);
  const int cl = grp * 8 + rem % 8;
  if (cl >= N * HV) return;
  // packed batches: sequences in the chunk table's scan order (longest first)
  const int n = cu ? ws_int[2 + N + cl / HV] : cl / HV, hv = cl % HV, vb = rem / 8;
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

  if (len == 0) {  // empty slot: dh0 = dht
    for (int e = tid; e < K * BV; e += kThreads) {
      const int r = e / BV, c = col_base + e % BV;
      const size_t off = st_base + (size_t)r * V + c;
      uint32_t bits = dht ? reinterpret_cast<const uint32_t*>(dht)[off] : 0u;
      reinterpret_cast<uint32_t*>(dh0)[off] = bits;
    }
    return;
  }

  f32x4 S[RTW][CTB];  // dS: wave owns channel tiles RTW*wave ..
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
    for (int ct = 0; ct < CTB; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 16 * (RTW * wave + rt) + 4 * g + e;
        const int col = col_base + 16 * ct + l16;
        S[rt][ct][e] = dht ? dht[st_base + (size_t)c * V + col] : 0.f;
      }

  // Per-chunk operands of this wave, loaded one chunk ahead, and one 16-byte
  // unit per thread of the dO block of the chunk after it in the reverse order
  // (staged into LDS during this chunk's step, read in the next one).
  constexpr int UPR = BV * (int)sizeof(T) / 16;               // 16-byte units per dO row
  constexpr int DOU = (kC * UPR + kThreads - 1) / kThreads;  // units per thread
  struct ROps {
    F khn[KS_K], pt[KS_C], qgt[RTW][KS_C], wt[RTW][KS_C];
    float4 gl[RTW];
    uint4 dob[DOU];  // dO of chunk cj - 1 (clamped to cbeg)
  };
  // dO block of chunk cj: rows >= L read row 0 of the chunk and are zeroed when staged
  auto load_dob = [&](int cj, uint4* dob) {
    const int cidx = cj - cbeg;
    const int64_t t0 = bos + (int64_t)cidx * kC;
    const int L = min(kC, len - cidx * kC);
#pragma unroll
    for (int d = 0; d < DOU; ++d) {
      const int u = tid + d * kThreads;
      const int row = (u / UPR) < L ? (u / UPR) : 0, cu_ = u % UPR;
      dob[d] = u < kC * UPR
                   ? *reinterpret_cast<const uint4*>(dO + ((t0 + row) * HV + hv) * V + col_base + cu_ * (16 / sizeof(T)))
                   : make_uint4(0, 0, 0, 0);
    }
  };
  auto stage_dob = [&](int cj, const uint4* dob, T* dst) {
    const int L = min(kC, len - (cj - cbeg) * kC);
#pragma unroll
    for (int d = 0; d < DOU; ++d) {
      const int u = tid + d * kThreads;
      if (u < kC * UPR) {
        const int row = u / UPR, cu_ = u % UPR;
        *reinterpret_cast<uint4*>(dst + row * DS + cu_ * (16 / sizeof(T))) =
            row < L ? dob[d] : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto load_ops = [&](int cj, ROps& op) {
    const size_t ch = (size_t)cj * HV + hv;
    const T* wb = ws_B + ch * WB::elems;
    const F* fPT = reinterpret_cast<const F*>(wb + WB::oPT);
    const F* fKHn = reinterpret_cast<const F*>(wb + WB::oKHn);
    const F* fQGT = reinterpret_cast<const F*>(wb + WB::oQGT);
    const F* fWT = reinterpret_cast<const F*>(wb + WB::oWT);
#pragma unroll
    for (int ks = 0; ks < KS_K; ++ks) op.khn[ks] = fKHn[((size_t)wave * KS_K + ks) * 64 + lane];
#pragma unroll
    for (int ks = 0; ks < KS_C; ++ks) op.pt[ks] = fPT[((size_t)wave * KS_C + ks) * 64 + lane];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const int tileK = RTW * wave + rt;
#pragma unroll
      for (int ks = 0; ks < KS_C; ++ks) {
        op.qgt[rt][ks] = fQGT[((size_t)tileK * KS_C + ks) * 64 + lane];
        op.wt[rt][ks] = fWT[((size_t)tileK * KS_C + ks) * 64 + lane];
      }
      op.gl[rt] = *reinterpret_cast<const float4*>(ws_GL + ch * K + 16 * tileK + 4 * g);
    }
    load_dob(max(cj - 1, cbeg), op.dob);
  };

  // One chunk with LDS buffer set `buf`. Its dO block is already in sdO[buf]
  // (staged during the previous step, visible since that step's second
  // barrier), so P^T dO and (Q~Gamma)^T dO, which do not depend on dS, are
  // formed before the first barrier. Buffer reuse: every read of a buffer set
  // happens before the first barrier of the following step, and the set is
  // written again only after that barrier, two steps later.
  auto step = [&](const ROps& op, const int cj, const int buf) __attribute__((always_inline)) {
    const size_t ch = (size_t)cj * HV + hv;
    T* wb = ws_B + ch * WB::elems;

    // dO as B fragments (contraction over tokens)
    F bdo[CTB][KS_C];
#pragma unroll
    for (int ct = 0; ct < CTB; ++ct)
#pragma unroll
      for (int p = 0; p < QC; ++p) {
        float x4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x4[e] = to_f32(sdO[buf][(16 * p + 4 * g + e) * DS + 16 * ct + l16]);
        put_quad<M>(bdo[ct], p, x4);
      }
    // input terms: P^T dO (token tile `wave`) and (Q~Gamma)^T dO (the wave's channel tiles)
    f32x4 D[CTB], Sin[RTW][CTB];
#pragma unroll
    for (int ct = 0; ct < CTB; ++ct) {
      D[ct] = zero4();
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt) Sin[rt][ct] = zero4();
    }
#pragma unroll
    for (int ks = 0; ks < KS_C; ++ks)
#pragma unroll
      for (int ct = 0; ct < CTB; ++ct) {
        D[ct] = M::mma(op.pt[ks], bdo[ct][ks], D[ct]);
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) Sin[rt][ct] = M::mma(op.qgt[rt][ks], bdo[ct][ks], Sin[rt][ct]);
      }

    // keep dS1 of this chunk for the local kernel; publish it as B fragments.
    // With up to 32 columns the stores of dS1 and dDelta wait until after the
    // second barrier (a copy of dS1 in registers), behind the step's loads
    // rather than in front of them
    constexpr bool LATE = BV <= 32;
    T* dsl = wb + WB::oDS;
    f32x4 s1c[LATE ? RTW : 1][LATE ? CTB : 1];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const int tileK = RTW * wave + rt;
#pragma unroll
      for (int ct = 0; ct < CTB; ++ct) {
        if constexpr (LATE)
          s1c[rt][ct] = S[rt][ct];
        else
          store4<T>(dsl + il4(16 * tileK + 4 * g, col_base + 16 * ct + l16, V), S[rt][ct][0],
                    S[rt][ct][1], S[rt][ct][2], S[rt][ct][3]);
        if constexpr (M::KSTEP == 32) {
          bf16x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = (bf16)S[rt][ct][e];
          *(reinterpret_cast<bf16x4*>(&sS[buf][tileK >> 1][ct][lane]) + (tileK & 1)) = x;
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

    // dDelta for token tile `wave`: P^T dO + Khat dS1
#pragma unroll
    for (int ks = 0; ks < KS_K; ++ks) {
#pragma unroll
      for (int ct = 0; ct < CTB; ++ct) D[ct] = M::mma(op.khn[ks], sS[buf][ks][ct][lane], D[ct]);
    }
    T* ddl = wb + WB::oDDL;
#pragma unroll
    for (int ct = 0; ct < CTB; ++ct) {
      if constexpr (!LATE)
        store4<T>(ddl + il4(16 * wave + 4 * g, col_base + 16 * ct + l16, V), D[ct][0], D[ct][1],
                  D[ct][2], D[ct][3]);
      if constexpr (M::KSTEP == 32) {
        bf16x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (bf16)D[ct][e];
        *(reinterpret_cast<bf16x4*>(&sD[buf][wave >> 1][ct][lane]) + (wave & 1)) = x;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          F f;
          M::set(f, 0, D[ct][e]);
          sD[buf][4 * wave + e][ct][lane] = f;
        }
      }
    }
    // the dO block of the next chunk in the reverse order
    stage_dob(max(cj - 1, cbeg), op.dob, sdO[buf ^ 1]);
    __syncthreads();
    if constexpr (LATE) {
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
        for (int ct = 0; ct < CTB; ++ct)
          store4<T>(dsl + il4(16 * (RTW * wave + rt) + 4 * g, col_base + 16 * ct + l16, V),
                    s1c[rt][ct][0], s1c[rt][ct][1], s1c[rt][ct][2], s1c[rt][ct][3]);
#pragma unroll
      for (int ct = 0; ct < CTB; ++ct)
        store4<T>(ddl + il4(16 * wave + 4 * g, col_base + 16 * ct + l16, V), D[ct][0], D[ct][1],
                  D[ct][2], D[ct][3]);
    }

    // dS0 = Diag(gamma) dS1 + (Q~Gamma)^T dO - W^T dDelta
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const float ga[4] = {op.gl[rt].x, op.gl[rt].y, op.gl[rt].z, op.gl[rt].w};
      f32x4 neg[CTB];
#pragma unroll
      for (int ct = 0; ct < CTB; ++ct) neg[ct] = zero4();
#pragma unroll
      for (int ks = 0; ks < KS_C; ++ks) {
#pragma unroll
        for (int ct = 0; ct < CTB; ++ct) neg[ct] = M::mma(op.wt[rt][ks], sD[buf][ks][ct][lane], neg[ct]);
      }
#pragma unroll
      for (int ct = 0; ct < CTB; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[rt][ct][e] = S[rt][ct][e] * ga[e] + Sin[rt][ct][e] - neg[ct][e];
    }
  };

  // chunks in reverse; two operand sets, unrolled by two (the first chunk is
  // fetched again near the end so every path has the same loads in flight)
  ROps opA, opB;
  {
    uint4 d0[DOU];
    load_dob(cend - 1, d0);
    load_ops(cend - 1, opA);
    stage_dob(cend - 1, d0, sdO[0]);
  }
  __syncthreads();
  for (int cj = cend - 1;; cj -= 2) {
    load_ops(max(cj - 1, cbeg), opB);
    step(opA, cj, 0);
    if (cj - 1 < cbeg) break;
    load_ops(max(cj - 2, cbeg), opA);
    step(opB, cj - 1, 1);
    if (cj - 2 < cbeg) break;
  }
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
    for (int ct = 0; ct < CTB; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 16 * (RTW * wave + rt) + 4 * g + e;
        const int col = col_base + 16 * ct + l16;
        dh0[st_base + (size_t)c * V + col] = S[rt][ct][e];
      }
}

// ------------------------------------------------------------------ local gradients
template <typename T, int K, int V>
struct BwdLds {
  static constexpr int TP = 16 / (int)sizeof(T);
  // V columns per phase-1 block: 64 for bf16 (128-byte row pieces), 32 for FP32
  static constexpr int VB = sizeof(T) == 2 ? 64 : 32;
  static constexpr int GS = K + 4;          // G2 (floats)
  static constexpr int KSTR = K + TP;       // k, q, dW, b*Kg (elements of T)
  static constexpr int TS = kC + 4;         // T (floats)
  static constexpr int CS = kC + TP;        // C x C matrices and transposed C x K (elements of T)
  static constexpr int BS = VB + 4;         // phase-1 blocks (8-byte aligned rows)
  static constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t szG = (size_t)kC * GS * 4;
  static constexpr size_t szK = (size_t)kC * KSTR * sizeof(T);
  static constexpr size_t szT = (size_t)kC * TS * 4;
  static constexpr size_t szQ = (size_t)kC * KSTR * sizeof(T);
  // phase 1: dO, Delta, dDelta, v blocks [C][BS]; S0, dS1 blocks [K][BS]
  static constexpr size_t p1 = (4 * (size_t)kC + 2 * (size_t)K) * BS * sizeof(T);
  // from the end of phase 1 to the end: dP, dP^T [C][CS]; behind them the phase-2 area
  static constexpr size_t pP = 2 * (size_t)kC * CS * sizeof(T);
  // phase 2: dW^T [K][CS] + b*Kg [C][KSTR] + dW [C][KSTR]; later three [C][CS] slots:
  // dT^T then dAbar, Xm, dAbar^T
  static constexpr size_t p2a = (size_t)K * CS * sizeof(T) + 2 * (size_t)kC * KSTR * sizeof(T);
  static constexpr size_t p2b = 3 * (size_t)kC * CS * sizeof(T);
  // decay products (one-reference mode, bf16): kd, ke, qd fragments (hi and
  // lo) of one channel tile per half, behind the three phase-2 slots; FP32
  // builds them per wave (no room left in LDS)
  static constexpr bool share_ops = sizeof(T) == 2;
  static constexpr size_t pOp = share_ops ? 2 * 3 * 2 * (size_t)kC * 16 * sizeof(T) : 0;
  static constexpr size_t szX = cmax(p1, pP + cmax(p2a, p2b + pOp));
  // small arrays: per-token-tile column sums [4][K], dgamma [K], row sums [C] x 3 parts x 2 halves
  static constexpr size_t szSmall = (4 * (size_t)K + K + 6 * (size_t)kC) * 4;
  static constexpr size_t oG = 0, oK = oG + szG, oT = oK + szK, oQ = oT + szT, oX = oQ + szQ,
                          oSm = oX + szX, total = oSm + szSmall;
};

// A fragments of a row-major LDS matrix: rows `row`, contraction along the row.
// bf16 sources feed bf16 fragments bit for bit (quad p is half p & 1 of fragment p / 2).
template <typename M, typename E, int NQ>
__device__ __forceinline__ void frag_rows(typename M::frag* f, const E* base, int row, int stride,
                                          int g) {
#pragma unroll
  for (int p = 0; p < NQ; ++p) {
    if constexpr (M::KSTEP == 32 && sizeof(E) == 2) {
      *(reinterpret_cast<bf16x4*>(&f[p >> 1]) + (p & 1)) =
          *reinterpret_cast<const bf16x4*>(base + row * stride + 16 * p + 4 * g);
    } else {
      float v[4];
      lds4(base + row * stride + 16 * p + 4 * g, v);
      put_quad<M>(f, p, v);
    }
  }
}
// Fragments whose contraction runs down a column of a row-major LDS matrix.
template <typename M, typename E, int NQ>
__device__ __forceinline__ void frag_cols(typename M::frag* f, const E* base, int col, int stride,
                                          int g) {
#pragma unroll
  for (int p = 0; p < NQ; ++p) {
    if constexpr (M::KSTEP == 32 && sizeof(E) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) f[p >> 1][4 * (p & 1) + e] = base[(16 * p + 4 * g + e) * stride + col];
    } else {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = to_f32(base[(16 * p + 4 * g + e) * stride + col]);
      put_quad<M>(f, p, v);
    }
  }
}

// Quad p of a hi/lo operand pair: hi = bf16(v), lo = bf16(v - hi), so that
// hi*a + lo*a carries about 16 mantissa bits of v (FP32 fragments: lo = 0).
template <typename M>
__device__ __forceinline__ void put_quad_split(typename M::frag* hi, typename M::frag* lo, int p,
                                               const float v[4]) {
  float h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (M::KSTEP == 32) {
      h[e] = (float)(bf16)v[e];
      l[e] = v[e] - h[e];
    } else {
      h[e] = v[e];
      l[e] = 0.f;
    }
  }
  put_quad<M>(hi, p, h);
  put_quad<M>(lo, p, l);
}

// Materialise a running sum where it stands: keeps the compiler from sinking
// an accumulation chain towards its last use with every addend kept alive.
__device__ __forceinline__ void pin(f32x4& x) { asm volatile("" : "+v"(x)); }

// One workgroup per (chunk, value head), 8 waves: wave w takes token tile
// tt = w % 4 (16 rows of the chunk) and half hh = w / 4 of the column tiles
// (channel tiles hh*NCT/2 .. of the C x K products, column tiles 2hh, 2hh+1 of
// the C x C products), so every SIMD holds two waves of the workgroup.
constexpr int kBwdThreads = 512;

// GF: the gate arrives raw or natural-log (gate_mode) and its step runs in the
// prologue; otherwise it is the chunk-local log2 cumsum. Two instantiations, so
// that the log2-gate kernel carries nothing of the gate step.
template <typename T, int K, int V, bool GF = false>
__global__ void __launch_bounds__(kBwdThreads, 1)
chunk_bwd_local_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                       const float* __restrict__ gate, int gate_mode, const float* __restrict__ A_log,
                       const T* __restrict__ beta,
                       const T* __restrict__ dO, const int32_t* __restrict__ cu,
                       const int* __restrict__ ws_int, const T* __restrict__ ws_B,
                       const float* __restrict__ ws_Bf, int N, int T_, int H, int HV, float scale,
                       T* __restrict__ dq_out, T* __restrict__ dk_out, float* __restrict__ dq_part,
                       float* __restrict__ dk_part, T* __restrict__ dv, float* __restrict__ dg,
                       T* __restrict__ dbeta) {
  using M = MF<T>;
  using F = typename M::frag;
  using Lds = BwdLds<T, K, V>;
  using WB = WsB<T, K, V>;
  constexpr int NT = kBwdThreads;
  constexpr int KS_C = kC / M::KSTEP;
  constexpr int QK = K / 16, QC = kC / 16, NCT = K / 16;
  constexpr int NCH = NCT / 2;  // channel tiles per wave
  constexpr int JH = QC / 2;    // C x C column tiles per wave
  constexpr int GS = Lds::GS, KSTR = Lds::KSTR, TS = Lds::TS, CS = Lds::CS, BS = Lds::BS;
  constexpr int VB = Lds::VB;
  constexpr int EPU = 16 / (int)sizeof(T);
  constexpr int VTH = VB / 32;  // value tiles of a block per half
  static_assert(VTH * 32 == VB && V % VB == 0, "V blocks");

  extern __shared__ __align__(16) char smem[];
  float* sG = reinterpret_cast<float*>(smem + Lds::oG);
  T* sK = reinterpret_cast<T*>(smem + Lds::oK);
  float* sT = reinterpret_cast<float*>(smem + Lds::oT);
  T* sQ = reinterpret_cast<T*>(smem + Lds::oQ);
  char* X = smem + Lds::oX;
  T* XT = reinterpret_cast<T*>(X);  // dP, dP^T from the end of phase 1 on
  T* XP = XT + 2 * kC * CS;         // phase-2 area behind them
  float* sColP = reinterpret_cast<float*>(smem + Lds::oSm);  // [4][K] per-token-tile column sums
  float* sDgam = sColP + 4 * K;                               // [K]
  float* sRow = sDgam + K;                                    // [3 parts][2 halves][C] dbeta parts

  // 1-D grid, value head fastest and rotated by the chunk index (the order of
  // the backward's intra-chunk recompute): 2% faster than chunk fastest here
  const int chunk = (int)(blockIdx.x / (unsigned)HV);
  const int hv = (int)((blockIdx.x % (unsigned)HV + (unsigned)chunk) % (unsigned)HV);
  const ChunkGeo geo = chunk_geo(chunk, cu, ws_int, N, T_);
  if (!geo.ok) return;
  const int h = hv / (HV / H);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int tt = w & 3, hh = w >> 2;
  const int cb = NCH * hh;  // first channel tile of the wave
  const int L = geo.L;
  const int64_t t0 = geo.t0;
  const size_t ch = (size_t)chunk * HV + hv;
  const T* wb = ws_B + ch * WB::elems;
  const float* wTm = ws_Bf + ch * WB::elems_f;
  const float* wAb = wTm + WB::TM;

  // phase-1 blocks of VB value columns: dO, Delta, dDelta, v [C][BS]; S0, dS1 [K][BS],
  // staged through registers one block ahead
  T* bdO = XT;
  T* bDl = bdO + kC * BS;
  T* bdDl = bDl + kC * BS;
  T* bV = bdDl + kC * BS;
  T* bS0 = bV + kC * BS;
  T* bdS = bS0 + K * BS;
  constexpr int UPR = VB / EPU;  // 16-byte units per block row
  constexpr int NUC = (kC * UPR + NT - 1) / NT, NUK = (K * UPR + NT - 1) / NT;
  // S0, Delta, dS1, dDelta are stored with rows interleaved by four (il4): a
  // 16-byte unit holds CPU columns x 4 rows, unit i of row group rg covering
  // columns CPU i .. CPU i + CPU - 1 of the block; the same number of units per
  // block as the row-major inputs
  constexpr int CPU = EPU / 4;   // columns per interleaved unit
  constexpr int UPG = VB / CPU;  // interleaved units per row group
  struct Blk {
    uint4 a[NUC], b[NUC], c[NUC], d[NUC], s0[NUK], ds[NUK];
  };
  auto il_unit = [&](size_t off, int u, int c0) {
    return ldg_nt(reinterpret_cast<const uint4*>(wb + off + il4(4 * (u / UPG), c0 + CPU * (u % UPG), V)));
  };
  auto load_blk = [&](int vb, Blk& x) {
    const int c0 = vb * VB;
#pragma unroll
    for (int i = 0; i < NUC; ++i) {
      const int u = tid + i * NT;
      const int row = u / UPR < kC ? u / UPR : 0, cu_ = u % UPR;
      const int rr = row < L ? row : 0;
      const int ui = u < kC * UPR ? u : 0;
      x.a[i] = ldg_nt(reinterpret_cast<const uint4*>(dO + ((t0 + rr) * HV + hv) * V + c0 + EPU * cu_));
      x.d[i] = ldg_nt(reinterpret_cast<const uint4*>(v + ((t0 + rr) * HV + hv) * V + c0 + EPU * cu_));
      x.b[i] = il_unit(WB::oDL, ui, c0);
      x.c[i] = il_unit(WB::oDDL, ui, c0);
    }
#pragma unroll
    for (int i = 0; i < NUK; ++i) {
      const int u = tid + i * NT;
      const int ui = u < K * UPR ? u : 0;
      x.s0[i] = il_unit(WB::oS0, ui, c0);
      x.ds[i] = il_unit(WB::oDS, ui, c0);
    }
  };
  auto put16 = [](T* dst, const uint4& x) {  // block rows are 8-byte aligned
    reinterpret_cast<uint2*>(dst)[0] = make_uint2(x.x, x.y);
    reinterpret_cast<uint2*>(dst)[1] = make_uint2(x.z, x.w);
  };
  // an interleaved unit into the row-major [R][BS] block: row 4 rg + j takes
  // element j of each of the unit's CPU columns (4-byte LDS writes)
  auto put_il = [&](T* base, int u, const uint4& x) {
    const int r0 = 4 * (u / UPG), c = CPU * (u % UPG);
    if constexpr (sizeof(T) == 2) {
      const uint32_t w[4] = {(x.x & 0xFFFFu) | (x.z << 16), (x.x >> 16) | (x.z & 0xFFFF0000u),
                             (x.y & 0xFFFFu) | (x.w << 16), (x.y >> 16) | (x.w & 0xFFFF0000u)};
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<uint32_t*>(base + (r0 + j) * BS + c) = w[j];
    } else {
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<uint32_t*>(base + (r0 + j) * BS + c) = w[j];
    }
  };
  auto store_blk = [&](const Blk& x) {
#pragma unroll
    for (int i = 0; i < NUC; ++i) {
      const int u = tid + i * NT;
      if (u < kC * UPR) {
        const int row = u / UPR, cu_ = u % UPR;
        uint4 av = x.a[i], dv_ = x.d[i];
        if (row >= L) av = dv_ = make_uint4(0, 0, 0, 0);
        put16(bdO + row * BS + EPU * cu_, av);
        put_il(bDl, u, x.b[i]);
        put_il(bdDl, u, x.c[i]);
        put16(bV + row * BS + EPU * cu_, dv_);
      }
    }
#pragma unroll
    for (int i = 0; i < NUK; ++i) {
      const int u = tid + i * NT;
      if (u < K * UPR) {
        put_il(bS0, u, x.s0[i]);
        put_il(bdS, u, x.ds[i]);
      }
    }
  };
  Blk pf;

  // ---- stage G2, k, q, T and the first phase-1 block (all loads of a thread
  // issued before its stores); zero the small arrays.
  // Gate rows. With the gate step (GF), thread (group gg, channel group gcg)
  // holds rows NG gg .. NG gg + NG - 1 of channels 4 gcg .. 4 gcg + 3, i.e.
  // segment gg % GSEG of cumsum block gg / GSEG (the lanes of one block's
  // segments sit NCG apart in a wave); otherwise unit i of a thread is row
  // (tid + i NT) / NCG.
  constexpr int NG = kC * K / 4 / NT, NCG = K / 4, GSEG = kGateBlock / NG;
  static_assert(NG * GSEG == kGateBlock && (NT / NCG) * NG == kC && GSEG * NCG <= 64, "gate rows");
  const int gg = tid / NCG, gcg = tid % NCG;
  auto grow = [&](int i) { return GF ? NG * gg + i : (tid + i * NT) / NCG; };
  auto gcol = [&](int i) { return GF ? gcg : (tid + i * NT) % NCG; };
  float4 gx[NG];
  {
    constexpr int NKQ = kC * K / EPU / NT, NTm = kC * kC / 4 / NT;
    static_assert(NG * NT == kC * K / 4 && NKQ * NT == kC * K / EPU && NTm * NT == kC * kC / 4, "stage");
    float4 tx[NTm];
    uint4 kx[NKQ], qx[NKQ];
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int row = grow(i);
      const int rr = row < L ? row : L - 1;
      gx[i] = ldg_nt(reinterpret_cast<const float4*>(gate + ((t0 + rr) * HV + hv) * K + 4 * gcol(i)));
    }
#pragma unroll
    for (int i = 0; i < NKQ; ++i) {
      const int f = tid + i * NT, row = f / (K / EPU), cu_ = f % (K / EPU);
      const int rr = row < L ? row : 0;
      kx[i] = ldg_nt(reinterpret_cast<const uint4*>(k + ((t0 + rr) * H + h) * K + EPU * cu_));
      qx[i] = ldg_nt(reinterpret_cast<const uint4*>(q + ((t0 + rr) * H + h) * K + EPU * cu_));
    }
#pragma unroll
    for (int i = 0; i < NTm; ++i) {
      const int f = tid + i * NT, row = f / (kC / 4), c4 = f % (kC / 4);
      tx[i] = ldg_nt(reinterpret_cast<const float4*>(wTm + row * kC + 4 * c4));
    }
    // beta of the chunk's rows (row tid % C; pad rows load the last valid row):
    // unconditional, in the same batch as the other loads
    const int brow = tid % kC < L ? tid % kC : L - 1;
    const T braw = beta[(t0 + brow) * HV + hv];
    load_blk(0, pf);
    if constexpr (GF) {
      // fused gate step: the per-token natural-log gate, then the in-block part
      // of the chunk-local cumsum in the kernel's blocked order (segments of a
      // block take turns, each continuing from the previous one's last sum;
      // pad rows keep the last token's value); block totals to the small arrays
      const float sc = gate_head_scale(gate_mode, A_log, hv);
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        gx[i].x = gate_nat(gx[i].x, gate_mode, sc);
        gx[i].y = gate_nat(gx[i].y, gate_mode, sc);
        gx[i].z = gate_nat(gx[i].z, gate_mode, sc);
        gx[i].w = gate_nat(gx[i].w, gate_mode, sc);
      }
      const int seg = gg % GSEG;
      float st[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < GSEG; ++r) {
        if (seg == r) {
#pragma unroll
          for (int i = 0; i < NG; ++i) {
            float ge[4] = {gx[i].x, gx[i].y, gx[i].z, gx[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (NG * gg + i < L) st[e] = st[e] + ge[e];
              ge[e] = st[e];
            }
            gx[i] = make_float4(ge[0], ge[1], ge[2], ge[3]);
          }
        }
        if (r + 1 < GSEG) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float nx = __shfl_up(st[e], NCG);
            if (seg == r + 1) st[e] = nx;
          }
        }
      }
      if (seg == GSEG - 1)
        *reinterpret_cast<float4*>(sColP + (gg / GSEG) * K + 4 * gcg) = make_float4(st[0], st[1], st[2], st[3]);
    } else {
#pragma unroll
      for (int i = 0; i < NG; ++i)
        *reinterpret_cast<float4*>(sG + grow(i) * GS + 4 * gcol(i)) = gx[i];
    }
#pragma unroll
    for (int i = 0; i < NKQ; ++i) {
      const int f = tid + i * NT, row = f / (K / EPU), cu_ = f % (K / EPU);
      uint4 kv = kx[i], qv = qx[i];
      if (row >= L) kv = qv = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(sK + row * KSTR + EPU * cu_) = kv;
      *reinterpret_cast<uint4*>(sQ + row * KSTR + EPU * cu_) = qv;
    }
#pragma unroll
    for (int i = 0; i < NTm; ++i) {
      const int f = tid + i * NT, row = f / (kC / 4), c4 = f % (kC / 4);
      *reinterpret_cast<float4*>(sT + row * TS + 4 * c4) = tx[i];
    }
    // beta lives in the first pad column of the G2 rows (never written otherwise);
    // zero past the chunk's last token
    if (tid < kC) sG[tid * GS + K] = tid < L ? to_f32(braw) : 0.f;
    store_blk(pf);
    if (V / VB > 1) load_blk(1, pf);
  }
  if constexpr (GF) {
    // G2 = (C_b + in-block sum) * log2(e), C_b the totals of the earlier
    // blocks in order: the gate kernel's order, so G2 is bit-identical to its
    // output. The totals sat in the small arrays, cleared after this.
    static_assert(kC / kGateBlock * K <= 4 * K + K + 6 * kC, "block totals");
    __syncthreads();
    float c[4] = {0.f, 0.f, 0.f, 0.f};
    for (int b = 0; b < gg / GSEG; ++b) {
      float t4[4];
      lds4(sColP + b * K + 4 * gcg, t4);
#pragma unroll
      for (int e = 0; e < 4; ++e) c[e] = c[e] + t4[e];
    }
#pragma unroll
    for (int i = 0; i < NG; ++i)
      *reinterpret_cast<float4*>(sG + (NG * gg + i) * GS + 4 * gcg) =
          make_float4((c[0] + gx[i].x) * kLog2e, (c[1] + gx[i].y) * kLog2e, (c[2] + gx[i].z) * kLog2e,
                      (c[3] + gx[i].w) * kLog2e);
    __syncthreads();
  }
  for (int f = tid; f < 4 * K + K + 6 * kC; f += NT) sColP[f] = 0.f;
  // outputs of this chunk: uniform base pointers, 32-bit element offsets per lane
  T* const dvb = dv + (t0 * HV + hv) * (int64_t)V;
  float* const dgb = dg + (t0 * HV + hv) * (int64_t)K;
  float* const dqpb = dq_part ? dq_part + (t0 * HV + hv) * (int64_t)K : nullptr;
  float* const dkpb = dk_part ? dk_part + (t0 * HV + hv) * (int64_t)K : nullptr;
  T* const dqb = dq_out + (t0 * H + h) * (int64_t)K;
  T* const dkb = dk_out + (t0 * H + h) * (int64_t)K;
  __syncthreads();
  float bet[4];  // beta of the rows 16tt + 4g + e this lane's accumulators cover (0 past L)
#pragma unroll
  for (int e = 0; e < 4; ++e) bet[e] = sG[(16 * tt + 4 * g + e) * GS + K];

  // T^T fragments for rows j of token tile tt (T[i][j] down i), used three times
  F aTt[KS_C];
  frag_cols<M, float, QC>(aTt, sT, 16 * tt + l16, TS, g);

  // ---- phase 1: contractions over V, in blocks of VB columns
  f32x4 dP[JH], dQG[NCH], dW[NCH], dKH[NCH], dT1[JH];
#pragma unroll
  for (int jj = 0; jj < JH; ++jj) dP[jj] = dT1[jj] = zero4();
#pragma unroll
  for (int cc = 0; cc < NCH; ++cc) dQG[cc] = dW[cc] = dKH[cc] = zero4();
  float dbU[4] = {0.f, 0.f, 0.f, 0.f};
  float dgam_acc = 0.f;  // thread-partial of rowsum(dS1 * S0) for channel tid % K
  {
    constexpr int NVB = V / VB;
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) {
      const int c0 = vb * VB;
      constexpr int QV = VB / 16;
      constexpr int KSV = VB / M::KSTEP;
      F aO[KSV], aDl[KSV], adDl[KSV];
      frag_rows<M, T, QV>(aO, bdO, 16 * tt + l16, BS, g);
      frag_rows<M, T, QV>(aDl, bDl, 16 * tt + l16, BS, g);
      frag_rows<M, T, QV>(adDl, bdDl, 16 * tt + l16, BS, g);
#pragma unroll
      for (int jj = 0; jj < JH; ++jj) {
        const int J = JH * hh + jj;
        F bD[KSV], bVv[KSV];
        frag_rows<M, T, QV>(bD, bDl, 16 * J + l16, BS, g);   // Delta^T: column j, contraction over v
        frag_rows<M, T, QV>(bVv, bV, 16 * J + l16, BS, g);   // v^T
#pragma unroll
        for (int ks = 0; ks < KSV; ++ks) {
          dP[jj] = M::mma(aO[ks], bD[ks], dP[jj]);
          dT1[jj] = M::mma(adDl[ks], bVv[ks], dT1[jj]);
        }
      }
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc) {
        const int ct = cb + cc;
        F bS[KSV], bdS_[KSV];
        frag_rows<M, T, QV>(bS, bS0, 16 * ct + l16, BS, g);
        frag_rows<M, T, QV>(bdS_, bdS, 16 * ct + l16, BS, g);
#pragma unroll
        for (int ks = 0; ks < KSV; ++ks) {
          dQG[cc] = M::mma(aO[ks], bS[ks], dQG[cc]);
          dW[cc] = M::mma(adDl[ks], bS[ks], dW[cc]);
          dKH[cc] = M::mma(aDl[ks], bdS_[ks], dKH[cc]);
        }
      }
      // T^T dDelta for token tile tt (rows j), value tiles of half hh of the block -> dv, v part of dbeta
#pragma unroll
      for (int vv = 0; vv < VTH; ++vv) {
        const int vt = VTH * hh + vv;
        F bdd[KS_C];
        frag_cols<M, T, QC>(bdd, bdDl, 16 * vt + l16, BS, g);  // dDelta down i
        f32x4 acc = zero4();
#pragma unroll
        for (int ks = 0; ks < KS_C; ++ks) acc = M::mma(aTt[ks], bdd[ks], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 16 * tt + 4 * g + e;
          const int col = c0 + 16 * vt + l16;
          if (j < L) dvb[j * HV * V + col] = from_f32<T>(bet[e] * acc[e]);
          dbU[e] += to_f32(bV[j * BS + 16 * vt + l16]) * acc[e];
        }
      }
      // dgamma partial: rowsum(dS1 * S0) over this block
      {
        const int c = tid % K;
        constexpr int parts = NT / K;  // threads per channel
        const int pidx = tid / K;
        float s = 0.f;
#pragma unroll
        for (int x = 0; x < VB / parts; ++x)
          s += to_f32(bdS[c * BS + pidx + parts * x]) * to_f32(bS0[c * BS + pidx + parts * x]);
        dgam_acc += s;
      }
      __syncthreads();  // every read of block vb done
      if (vb + 1 < NVB) {
        store_blk(pf);
        if (vb + 2 < NVB) load_blk(vb + 2, pf);
        __syncthreads();
      }
    }
  }
  // Reference token of the one-reference decay products, and whether every
  // gate value of the chunk is within 2^-+kFastRange of it (pad rows repeat row L-1)
  const int mref = (L - 1) >> 1;
  int bad = 0;
  {
    const int c = tid % K;
    const float gm = sG[mref * GS + c];
#pragma unroll
    for (int x = 0; x < kC * K / NT; ++x) {
      const int j = tid / K + (NT / K) * x;
      bad |= !(fabsf(sG[j * GS + c] - gm) <= kFastRange);
    }
  }
  bool fastC;
  // dgamma: reduce the thread partials per channel (fixed order)
  {
    float* sRed = reinterpret_cast<float*>(X);
    sRed[tid] = dgam_acc;
    fastC = __syncthreads_or(bad) == 0;
    if (tid < K) {
      float s = 0.f;
#pragma unroll
      for (int p = 0; p < NT / K; ++p) s += sRed[tid + p * K];
      sDgam[tid] = s;
    }
    __syncthreads();
  }
  // row sums over the 16 lanes of each lane group, into dbeta part `part`
  auto row_part = [&](float x4[4], int part) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x = x4[e];
      x += __shfl_xor(x, 1);
      x += __shfl_xor(x, 2);
      x += __shfl_xor(x, 4);
      x += __shfl_xor(x, 8);
      x4[e] = x;
    }
    if (l16 == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) sRow[(2 * part + hh) * kC + 16 * tt + 4 * g + e] = x4[e];
    }
  };
  row_part(dbU, 0);

  // accumulators for token tile tt, channel tiles cb..: dq~, dk, dG (natural-log
  // cumulative gate), started from d(Q~Gamma) and dKhat; keep per-token-tile
  // column sums of dKhat * Khat
  f32x4 aq[NCH], ak[NCH], aG[NCH];
#pragma unroll
  for (int cc = 0; cc < NCH; ++cc) {
    const int c = 16 * (cb + cc) + l16;
    const float glast = sG[(L - 1) * GS + c];
    float cs = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * tt + 4 * g + e;
      const float gi = sG[i * GS + c];
      const float Gam = ex2(gi);
      const float qs = to_f32(sQ[i * KSTR + c]) * scale;
      const float kk = to_f32(sK[i * KSTR + c]);
      const float eL = ex2(glast - gi);
      aq[cc][e] = dQG[cc][e] * Gam;
      ak[cc][e] = dKH[cc][e] * eL;
      const float t = dKH[cc][e] * kk * eL;
      aG[cc][e] = dQG[cc][e] * qs * Gam - t;
      cs += t;
    }
    cs += __shfl_xor(cs, 16);
    cs += __shfl_xor(cs, 32);
    if (g == 0) sColP[tt * K + c] = cs;
    pin(aq[cc]);
    pin(ak[cc]);
    pin(aG[cc]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // dT1 = dDelta (b v)^T: scale column j by beta_j
#pragma unroll
  for (int jj = 0; jj < JH; ++jj) {
    const int j = 16 * (JH * hh + jj) + l16;
    const float bj = sG[j * GS + K];  // 0 past L
#pragma unroll
    for (int e = 0; e < 4; ++e) dT1[jj][e] *= bj;
  }
  // dP (lower, inclusive) into LDS, both orientations
  {
    T* sdP = reinterpret_cast<T*>(X);
    T* sdPT = sdP + kC * CS;
#pragma unroll
    for (int jj = 0; jj < JH; ++jj)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * tt + 4 * g + e, j = 16 * (JH * hh + jj) + l16;
        const T x = from_f32<T>((j <= i) ? dP[jj][e] : 0.f);
        sdP[i * CS + j] = x;
        sdPT[j * CS + i] = x;
      }
  }
  __syncthreads();

  // ---- phase 2: dT, T^T dW, dA
  {
    // Abar entries of this lane's dA elements, requested now and used at the
    // end of the phase (a load at the use would stall the wave on its latency)
    float abv[JH][4];
#pragma unroll
    for (int jj = 0; jj < JH; ++jj)
#pragma unroll
      for (int e = 0; e < 4; ++e) abv[jj][e] = wAb[(16 * tt + 4 * g + e) * kC + 16 * (JH * hh + jj) + l16];
    T* sdWT = XP;                                 // [K][CS]
    T* sBKg = sdWT + K * CS;                      // [C][KSTR] b * k * Gamma
    T* sdW = sBKg + kC * KSTR;                    // [C][KSTR] row-major dW
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * tt + 4 * g + e, c = 16 * (cb + cc) + l16;
        const T x = from_f32<T>(-dW[cc][e]);
        sdW[i * KSTR + c] = x;
        sdWT[c * CS + i] = x;
      }
#pragma unroll
    for (int it = 0; it < kC * K / 4 / NT; ++it) {
      const int f = tid + it * NT;
      const int m = f / (K / 4), c4 = f % (K / 4);
      float km[4], gm[4];
      lds4(sK + m * KSTR + 4 * c4, km);
      lds4(sG + m * GS + 4 * c4, gm);
      const float bm = sG[m * GS + K];  // 0 past L
#pragma unroll
      for (int e = 0; e < 4; ++e) sBKg[m * KSTR + 4 * c4 + e] = from_f32<T>(bm * km[e] * ex2(gm[e]));
    }
    __syncthreads();
    // dT = dT1 + dW (b Kg)^T, rows i of tile tt, column tiles of the half
    f32x4 dT[JH];
    {
      F adw[K / M::KSTEP];
      frag_rows<M, T, QK>(adw, sdW, 16 * tt + l16, KSTR, g);
#pragma unroll
      for (int jj = 0; jj < JH; ++jj) {
        F bk[K / M::KSTEP];
        frag_rows<M, T, QK>(bk, sBKg, 16 * (JH * hh + jj) + l16, KSTR, g);
        dT[jj] = dT1[jj];
#pragma unroll
        for (int ks = 0; ks < K / M::KSTEP; ++ks) dT[jj] = M::mma(adw[ks], bk[ks], dT[jj]);
      }
    }
    // T^T dW, rows j of tile tt -> dKg = b_j (T^T dW)
    {
      float dbw[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc) {
        const int ct = cb + cc;
        F bw[KS_C];
        frag_rows<M, T, QC>(bw, sdWT, 16 * ct + l16, CS, g);
        f32x4 acc = zero4();
#pragma unroll
        for (int ks = 0; ks < KS_C; ++ks) acc = M::mma(aTt[ks], bw[ks], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 16 * tt + 4 * g + e, c = 16 * ct + l16;
          const float Gam = ex2(sG[j * GS + c]);
          const float kg = to_f32(sK[j * KSTR + c]) * Gam;
          const float dkg = bet[e] * acc[e];
          ak[cc][e] += dkg * Gam;
          aG[cc][e] += dkg * kg;
          dbw[e] += kg * acc[e];
        }
        pin(ak[cc]);
        pin(aG[cc]);
        __builtin_amdgcn_sched_barrier(0);
      }
      row_part(dbw, 1);
    }
    __syncthreads();  // dW, dW^T, b Kg dead
    T* sdTT = XP;  // dT transposed [j][i]
#pragma unroll
    for (int jj = 0; jj < JH; ++jj)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sdTT[(16 * (JH * hh + jj) + l16) * CS + 16 * tt + 4 * g + e] = from_f32<T>(dT[jj][e]);
    __syncthreads();
    // Xm = T^T dT, rows a of tile tt
    T* sXm = sdTT + kC * CS;
#pragma unroll
    for (int jj = 0; jj < JH; ++jj) {
      const int J = JH * hh + jj;
      F bt[KS_C];
      frag_rows<M, T, QC>(bt, sdTT, 16 * J + l16, CS, g);
      f32x4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < KS_C; ++ks) acc = M::mma(aTt[ks], bt[ks], acc);
#pragma unroll
      for (int e = 0; e < 4; ++e) sXm[(16 * tt + 4 * g + e) * CS + 16 * J + l16] = from_f32<T>(acc[e]);
    }
    __syncthreads();
    // dA = -Xm T^T (strictly lower), dAbar = b dA; Abar part of dbeta
    T* sdAb = sdTT;  // dT^T is dead once Xm is in
    T* sdAbT = sXm + kC * CS;
    {
      F ax[KS_C];
      frag_rows<M, T, QC>(ax, sXm, 16 * tt + l16, CS, g);
      float dba[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < JH; ++jj) {
        const int J = JH * hh + jj;
        F bt[KS_C];
        frag_rows<M, float, QC>(bt, sT, 16 * J + l16, TS, g);  // T^T column c = T row c
        f32x4 acc = zero4();
#pragma unroll
        for (int ks = 0; ks < KS_C; ++ks) acc = M::mma(ax[ks], bt[ks], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int a = 16 * tt + 4 * g + e, c = 16 * J + l16;
          const float da = (c < a) ? -acc[e] : 0.f;
          dba[e] += abv[jj][e] * da;
          const T x = from_f32<T>(bet[e] * da);
          sdAb[a * CS + c] = x;
          sdAbT[c * CS + a] = x;
        }
      }
      row_part(dba, 2);
    }
    __syncthreads();
  }

  // ---- decay-weighted products Y1, Y2 (with dP) and X1, X2 (with dAbar)
  //   Y1_ic = sum_j dP_ij    k_jc 2^(G2_ic - G2_jc) = 2^(G2_ic - G2_rc)  sum_j dP_ij    [k_jc 2^(G2_rc - G2_jc)]
  //   X1_ic = sum_j dAbar_ij k_jc 2^(G2_ic - G2_jc) = 2^(G2_ic - G2_rc)  sum_j dAbar_ij [k_jc 2^(G2_rc - G2_jc)]
  //   Y2_jc = sum_i dP_ij    q~_ic 2^(G2_ic - G2_jc) = 2^(G2_r'c - G2_jc) sum_i dP_ij  [q~_ic 2^(G2_ic - G2_r'c)]
  //   X2_jc = sum_i dAbar_ij k_ic 2^(G2_ic - G2_jc) = 2^(G2_r'c - G2_jc) sum_i dAbar_ij [k_ic 2^(G2_ic - G2_r'c)]
  // for rows i (resp. j) of token tile tt. Each lane builds the three bracketed
  // operands of its channel column over all 64 tokens and feeds four products.
  // References: the chunk's middle token m for r and r' when every gate value
  // of the chunk is within 2^-+kFastRange of it (all factors bounded; the row
  // factors of the tile are then the operand exponentials of its own rows);
  // otherwise r = 16tt and r' = 16tt + 15, which keep every factor of an
  // earlier (later) tile <= 1, and the diagonal tile enters the products only
  // when its own gate range is within kFastRange, else it is summed exactly
  // element by element.
  {
    const T* sdP = XT;
    const T* sdPT = sdP + kC * CS;
    const T* sdAb = XP;
    const T* sdAbT = XP + 2 * kC * CS;
    bool tfast = true;  // gate range of tile tt within kFastRange (per-tile mode)
    if (!fastC) {
      float rng = 0.f;
#pragma unroll
      for (int p = 0; p < QK; ++p) {
        float a0[4], a1[4];
        lds4(sG + (16 * tt) * GS + 16 * p + 4 * g, a0);
        lds4(sG + (16 * tt + 15) * GS + 16 * p + 4 * g, a1);
#pragma unroll
        for (int e = 0; e < 4; ++e) rng = fmaxf(rng, a0[e] - a1[e]);
      }
      rng = fmaxf(rng, __shfl_xor(rng, 16));
      rng = fmaxf(rng, __shfl_xor(rng, 32));
      tfast = rng <= kFastRange;
    }
    const int rz = fastC ? mref : 16 * tt;        // reference of the Y1 / X1 operands
    const int rzt = fastC ? mref : 16 * tt + 15;  // reference of the Y2 / X2 operands
    // operand rows that enter the products: Z pattern j <= jmax, Z' pattern i >= imin
    const int jmax = fastC ? kC - 1 : (tfast ? 16 * tt + 15 : 16 * tt - 1);
    const int imin = fastC ? 0 : (tfast ? 16 * tt : 16 * tt + 16);
    // shared operand fragments of the one-reference mode, behind dP, dP^T and
    // the three phase-2 slots: [half][operand kd, ke, qd][hi, lo][k-step][lane]
    char* const sOp = X + Lds::pP + Lds::p2b;
    auto op_slot = [&](int op, int hl, int ks) {
      return sOp + ((((size_t)hh * 3 + op) * 2 + hl) * KS_C + ks) * 64 * sizeof(F) + lane * sizeof(F);
    };
    F aP[KS_C], aPT[KS_C], aAb[KS_C], aAbT[KS_C];
    frag_rows<M, T, QC>(aP, sdP, 16 * tt + l16, CS, g);
    frag_rows<M, T, QC>(aPT, sdPT, 16 * tt + l16, CS, g);
    frag_rows<M, T, QC>(aAb, sdAb, 16 * tt + l16, CS, g);
    frag_rows<M, T, QC>(aAbT, sdAbT, 16 * tt + l16, CS, g);
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
      const int c = 16 * (cb + cc) + l16;
      const float gz = sG[rz * GS + c], gzt = sG[rzt * GS + c];
      F kdh[KS_C], kdl[KS_C], keh[KS_C], kel[KS_C], qdh[KS_C], qdl[KS_C];
      float ed_t[4], eu_t[4], q_t[4], k_t[4], g_t[4];  // rows 16tt + 4g + e
      if (Lds::share_ops && fastC) {
        // One reference for the whole chunk: the operands of a channel tile are
        // the same for the four waves of a half, so wave tt builds token quad tt
        // (its own rows) and the quads meet in LDS.
        float kd[4], ke[4], qd[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 16 * tt + 4 * g + e;
          const float gj = sG[j * GS + c];
          const float kj = to_f32(sK[j * KSTR + c]), qj = to_f32(sQ[j * KSTR + c]);
          const float ed = ex2(gz - gj), eu = ex2(gj - gzt);
          kd[e] = kj * ed;
          ke[e] = kj * eu;
          qd[e] = qj * scale * eu;
          ed_t[e] = ed;
          eu_t[e] = eu;
          q_t[e] = qj;
          k_t[e] = kj;
          g_t[e] = gj;
        }
        __syncthreads();  // the previous channel tile's operands are read
        const float* src[3] = {kd, ke, qd};
#pragma unroll
        for (int op = 0; op < 3; ++op) {
          bf16x4 hi, lo;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            hi[e] = (bf16)src[op][e];
            lo[e] = (bf16)(src[op][e] - (float)hi[e]);
          }
          // quad tt is slots 4 (tt & 1) .. + 3 of fragment tt / 2
          *reinterpret_cast<bf16x4*>(op_slot(op, 0, tt >> 1) + 8 * (tt & 1)) = hi;
          *reinterpret_cast<bf16x4*>(op_slot(op, 1, tt >> 1) + 8 * (tt & 1)) = lo;
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < KS_C; ++ks) {
          kdh[ks] = *reinterpret_cast<const F*>(op_slot(0, 0, ks));
          keh[ks] = *reinterpret_cast<const F*>(op_slot(1, 0, ks));
          qdh[ks] = *reinterpret_cast<const F*>(op_slot(2, 0, ks));
          kdl[ks] = *reinterpret_cast<const F*>(op_slot(0, 1, ks));
          kel[ks] = *reinterpret_cast<const F*>(op_slot(1, 1, ks));
          qdl[ks] = *reinterpret_cast<const F*>(op_slot(2, 1, ks));
        }
      } else {
#pragma unroll
        for (int p = 0; p < QC; ++p) {
          float kd[4], ke[4], qd[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = 16 * p + 4 * g + e;
            const float gj = sG[j * GS + c];
            const float kj = to_f32(sK[j * KSTR + c]), qj = to_f32(sQ[j * KSTR + c]);
            const float ed = ex2(gz - gj), eu = ex2(gj - gzt);
            kd[e] = j <= jmax ? kj * ed : 0.f;
            ke[e] = j >= imin ? kj * eu : 0.f;
            qd[e] = j >= imin ? qj * scale * eu : 0.f;
            if (p == tt) {
              ed_t[e] = ed;
              eu_t[e] = eu;
              q_t[e] = qj;
              k_t[e] = kj;
              g_t[e] = gj;
            }
          }
          put_quad_split<M>(kdh, kdl, p, kd);
          put_quad_split<M>(keh, kel, p, ke);
          put_quad_split<M>(qdh, qdl, p, qd);
        }
      }
      f32x4 y1 = zero4(), x1 = zero4(), y2 = zero4(), x2 = zero4();
#pragma unroll
      for (int ks = 0; ks < KS_C; ++ks) {
        y1 = M::mma(aP[ks], kdh[ks], y1);
        x1 = M::mma(aAb[ks], kdh[ks], x1);
        y2 = M::mma(aPT[ks], qdh[ks], y2);
        x2 = M::mma(aAbT[ks], keh[ks], x2);
        if constexpr (M::KSTEP == 32) {
          y1 = M::mma(aP[ks], kdl[ks], y1);
          x1 = M::mma(aAb[ks], kdl[ks], x1);
          y2 = M::mma(aPT[ks], qdl[ks], y2);
          x2 = M::mma(aAbT[ks], kel[ks], x2);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * tt + 4 * g + e;
        // row factors 2^(G2_i - G2_r) and 2^(G2_r' - G2_i); with one reference
        // they are the operand exponentials of row i
        const float fz = fastC ? eu_t[e] : ex2(g_t[e] - gz);
        const float fzt = fastC ? ed_t[e] : ex2(gzt - g_t[e]);
        float Y1 = y1[e] * fz, X1 = x1[e] * fz, Y2 = y2[e] * fzt, X2 = x2[e] * fzt;
        if (!tfast) {  // diagonal tile, exact elementwise (per-tile mode only)
          for (int j = 16 * tt; j <= i; ++j) {
            const float f = to_f32(sK[j * KSTR + c]) * ex2(g_t[e] - sG[j * GS + c]);
            Y1 += to_f32(sdP[i * CS + j]) * f;
            X1 += to_f32(sdAb[i * CS + j]) * f;
          }
          for (int j = i; j <= 16 * tt + 15; ++j) {
            const float f = ex2(sG[j * GS + c] - g_t[e]);
            Y2 += to_f32(sdPT[i * CS + j]) * to_f32(sQ[j * KSTR + c]) * scale * f;
            X2 += to_f32(sdAbT[i * CS + j]) * to_f32(sK[j * KSTR + c]) * f;
          }
        }
        if (i < L) {  // dq complete (per value head; summed over the GVA group later when HV > H)
          const float dqv = (aq[cc][e] + Y1) * scale;
          if (dqpb) dqpb[i * HV * K + c] = dqv;
          else dqb[i * H * K + c] = from_f32<T>(dqv);
        }
        aG[cc][e] += q_t[e] * scale * Y1 + k_t[e] * X1 - k_t[e] * Y2 - k_t[e] * X2;
        ak[cc][e] += X1 + Y2 + X2;
      }
      pin(ak[cc]);
      pin(aG[cc]);
      // one channel tile at a time: hoisting the next tile's LDS reads evicts the accumulators
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- last row: colsum(dKhat * Khat) + dgamma * gamma; reverse cumsum; outputs
  __syncthreads();
  {
    float* sTile = reinterpret_cast<float*>(X);  // per-token-tile column totals [4][K]
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
      const int c = 16 * (cb + cc) + l16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * tt + 4 * g + e;
        if (i == L - 1) {
          const float cs = sColP[c] + sColP[K + c] + sColP[2 * K + c] + sColP[3 * K + c];
          aG[cc][e] += cs + sDgam[c] * ex2(sG[(L - 1) * GS + c]);
        }
      }
      float tot = aG[cc][0] + aG[cc][1] + aG[cc][2] + aG[cc][3];
      tot += __shfl_xor(tot, 16);
      tot += __shfl_xor(tot, 32);
      if (g == 0) sTile[tt * K + c] = tot;
    }
    __syncthreads();
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
      const int c = 16 * (cb + cc) + l16;
      float later = 0.f;  // rows of the later tiles
      for (int t2 = tt + 1; t2 < 4; ++t2) later += sTile[t2 * K + c];
      // suffix sums inside the tile: rows 4g..4g+3 in lanes of group g
      float s3 = aG[cc][3], s2 = s3 + aG[cc][2], s1 = s2 + aG[cc][1], s0 = s1 + aG[cc][0];
      float after = 0.f;
      const float g1 = __shfl_xor(s0, 16), g2 = __shfl_xor(s0, 32), g3 = __shfl_xor(s0, 48);
      // lane group g receives the totals of groups g^1, g^2, g^3; add those with a larger index
      if ((g ^ 1) > g) after += g1;
      if ((g ^ 2) > g) after += g2;
      if ((g ^ 3) > g) after += g3;
      const float base = later + after;
      const float sfx[4] = {s0 + base, s1 + base, s2 + base, s3 + base};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * tt + 4 * g + e;
        if (i < L) dgb[i * HV * K + c] = sfx[e];
      }
    }
  }
  // dk (per value head; summed over the GVA group later when HV > H), dbeta
#pragma unroll
  for (int cc = 0; cc < NCH; ++cc) {
    const int c = 16 * (cb + cc) + l16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * tt + 4 * g + e;
      if (i >= L) continue;
      if (dkpb) dkpb[i * HV * K + c] = ak[cc][e];
      else dkb[i * H * K + c] = from_f32<T>(ak[cc][e]);
    }
  }
  if (tid < kC && tid < L) {
    float db = 0.f;
#pragma unroll
    for (int p = 0; p < 6; ++p) db += sRow[p * kC + tid];
    dbeta[(t0 + tid) * HV + hv] = from_f32<T>(db);
  }
}

// dq, dk of a qk head = sum over its HV/H value heads, in head order.
template <typename T>
__global__ void gva_reduce_kernel(const float* __restrict__ dq_part, const float* __restrict__ dk_part,
                                  const int32_t* __restrict__ cu, int N, int64_t n_tok, int H, int HV,
                                  int K, T* __restrict__ dq, T* __restrict__ dk) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_tok = (int64_t)H * K;
  if (idx >= n_tok * per_tok) return;
  const int64_t t = idx / per_tok;
  if (cu && t >= cu[N]) return;
  const int h = (int)((idx % per_tok) / K), c = (int)(idx % K);
  const int G = HV / H;
  float a = 0.f, b = 0.f;
  for (int j = 0; j < G; ++j) {
    const int64_t o = (t * HV + h * G + j) * K + c;
    a += dq_part[o];
    b += dk_part[o];
  }
  dq[idx] = from_f32<T>(a);
  dk[idx] = from_f32<T>(b);
}

// ------------------------------------------------------------------ host side
template <typename T, int K, int V>
size_t bwd_ws_bytes_t(const kda_dims& d, bool varlen) {
  const int64_t mc = max_chunks(d, varlen);
  size_t b = align256(sizeof(int) * (size_t)(2 + 2 * (size_t)d.N + mc));
  b += align256((size_t)mc * d.HV * Ws<T, K, V>::bytes_T);
  b += align256((size_t)mc * d.HV * Ws<T, K, V>::bytes_GL);
  b += align256((size_t)mc * d.HV * WsB<T, K, V>::elems * sizeof(T));
  b += align256((size_t)mc * d.HV * WsB<T, K, V>::elems_f * sizeof(float));
  if (d.HV != d.H) b += 2 * align256((size_t)d.B * d.T * d.HV * K * sizeof(float));
  return b;
}

template <typename T, int K, int V>
hipError_t chunk_bwd_t(const kda_dims& d, const void* q, const void* k, const void* v,
                       const float* gate, int gate_mode, const float* A_log, const void* beta,
                       const float* h0, const int32_t* cu,
                       const void* dO, const float* dht, void* dq, void* dk, void* dv, float* dg,
                       void* dbeta, float* dh0, void* ws, int saved, hipStream_t s) {
  const bool varlen = cu != nullptr;
  const int64_t mc = max_chunks(d, varlen);
  char* p = reinterpret_cast<char*>(ws);
  int* ws_int = reinterpret_cast<int*>(p);
  p += align256(sizeof(int) * (size_t)(2 + 2 * (size_t)d.N + mc));
  T* ws_T = reinterpret_cast<T*>(p);
  p += align256((size_t)mc * d.HV * Ws<T, K, V>::bytes_T);
  float* ws_GL = reinterpret_cast<float*>(p);
  p += align256((size_t)mc * d.HV * Ws<T, K, V>::bytes_GL);
  T* ws_B = reinterpret_cast<T*>(p);
  p += align256((size_t)mc * d.HV * WsB<T, K, V>::elems * sizeof(T));
  float* ws_Bf = reinterpret_cast<float*>(p);
  p += align256((size_t)mc * d.HV * WsB<T, K, V>::elems_f * sizeof(float));
  float* dq_part = nullptr;
  float* dk_part = nullptr;
  if (d.HV != d.H) {
    dq_part = reinterpret_cast<float*>(p);
    p += align256((size_t)d.B * d.T * d.HV * K * sizeof(float));
    dk_part = reinterpret_cast<float*>(p);
  }
  hipError_t e;
  if (varlen) {
    e = launch_chunk_table(cu, d.N, ws_int, (int)mc, s);
    if (e != hipSuccess) return e;
  }
  const float scale = 1.0f / sqrtf((float)K);
  if (mc > 0) {
    // after a training forward (saved) every intra-chunk entry is in place
    if (!saved) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_intra_kernel<T, K, V, true, false, false>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)IntraLds<T, K, V>::total);
      if (e != hipSuccess) return e;
      const size_t lds_intra = IntraLds<T, K, V>::total;
      hipLaunchKernelGGL((chunk_intra_kernel<T, K, V, true, false, false>), dim3((unsigned)(mc * d.HV)),
                         dim3(kThreads), lds_intra, s, (const T*)q, (const T*)k,
                         (const T*)v, gate, gate_mode, A_log, (const T*)beta,
                         cu, ws_int, d.N, d.T, d.H, d.HV, scale,
                         ws_T, ws_GL, ws_B, ws_Bf, kda_short_conv{}, 1);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t chains = (int64_t)d.N * d.HV;
  // both recurrences are latency chains: 16-column V blocks when 32-column
  // blocks would leave compute units without a workgroup
  auto launch_scans = [&](auto bvc) -> hipError_t {
    constexpr int BVC = decltype(bvc)::value;
    // forward recurrence keeping S0 and Delta (no outputs), unless a training
    // forward (kda_chunk_fwd_train) already stored them in this workspace
    if (!saved) {
      hipLaunchKernelGGL((chunk_scan_kernel<T, K, V, BVC, true, 4>), dim3(scan_grid(chains, V, BVC)),
                         dim3(kThreads), 0, s, (const T*)ws_T, (const float*)ws_GL, (const int*)ws_int,
                         cu, h0, d.N, d.T, d.HV, 0, (T*)nullptr, (float*)nullptr, ws_B);
      hipError_t e2 = hipGetLastError();
      if (e2 != hipSuccess) return e2;
    }
    hipLaunchKernelGGL((chunk_rev_scan_kernel<T, K, V, BVC>), dim3(scan_grid(chains, V, BVC)),
                       dim3(kThreads), 0, s, (const T*)ws_T, (const float*)ws_GL, ws_B,
                       (const int*)ws_int, cu, (const T*)dO, dht, d.N, d.T, d.HV, dh0);
    return hipGetLastError();
  };
  e = chains * (V / 32) < kda_host::device_cus() ? launch_scans(std::integral_constant<int, 16>())
                                : launch_scans(std::integral_constant<int, 32>());
  if (e != hipSuccess) return e;
  // the instantiations the entry point accepts (bf16; FP32 with K = 64) stay within 158 KiB of
  // LDS (a workgroup asking for the full 160 KiB of the CU does not launch)
  static_assert(!(sizeof(T) == 2 || K == 64) || BwdLds<T, K, V>::total <= 158 * 1024, "LDS budget");
  if (mc > 0) {
    auto launch_local = [&](auto gfc) -> hipError_t {
      constexpr bool GF = decltype(gfc)::value;
      hipError_t e2 = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_bwd_local_kernel<T, K, V, GF>),
                                          hipFuncAttributeMaxDynamicSharedMemorySize,
                                          (int)BwdLds<T, K, V>::total);
      if (e2 != hipSuccess) return e2;
      const size_t lds_local = BwdLds<T, K, V>::total;
      hipLaunchKernelGGL((chunk_bwd_local_kernel<T, K, V, GF>), dim3((unsigned)(mc * d.HV)),
                         dim3(kBwdThreads), lds_local, s, (const T*)q, (const T*)k,
                         (const T*)v, gate, gate_mode, A_log, (const T*)beta, (const T*)dO, cu,
                         (const int*)ws_int,
                         (const T*)ws_B, (const float*)ws_Bf, d.N, d.T, d.H, d.HV, scale, (T*)dq,
                         (T*)dk, dq_part, dk_part, (T*)dv, dg, (T*)dbeta);
      return hipGetLastError();
    };
    e = gate_mode != kGateLog2 ? launch_local(std::true_type()) : launch_local(std::false_type());
    if (e != hipSuccess) return e;
  }
  const int64_t n_tok = (int64_t)d.B * d.T;
  if (d.HV != d.H && n_tok > 0) {  // no tokens: nothing to reduce (and no empty grid)
    const int64_t total = n_tok * d.H * K;
    hipLaunchKernelGGL(gva_reduce_kernel<T>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       dq_part, dk_part, cu, d.N, n_tok, d.H, d.HV, K, (T*)dq, (T*)dk);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kda

namespace kda_host {

template <typename T>
static size_t bwd_ws_dispatch(const kda_dims& d) {
  auto both = [](size_t a, size_t b) { return std::max(a, b); };
  if (d.K == 64 && d.V == 64) return both(kda::bwd_ws_bytes_t<T, 64, 64>(d, false), kda::bwd_ws_bytes_t<T, 64, 64>(d, true));
  if (d.K == 64 && d.V == 128) return both(kda::bwd_ws_bytes_t<T, 64, 128>(d, false), kda::bwd_ws_bytes_t<T, 64, 128>(d, true));
  if (d.K == 128 && d.V == 64) return both(kda::bwd_ws_bytes_t<T, 128, 64>(d, false), kda::bwd_ws_bytes_t<T, 128, 64>(d, true));
  if (d.K == 128 && d.V == 128) return both(kda::bwd_ws_bytes_t<T, 128, 128>(d, false), kda::bwd_ws_bytes_t<T, 128, 128>(d, true));
  return 0;
}

size_t chunk_bwd_workspace_bytes(const kda_dims& d, kda_dtype dt, int chunk) {
  if (chunk != kda::kC) return 0;
  return dt == KDA_BF16 ? bwd_ws_dispatch<kda::bf16>(d) : bwd_ws_dispatch<float>(d);
}

template <typename T>
static hipError_t bwd_t(const kda_dims& d, const void* q, const void* k, const void* v,
                        const float* gate, int gate_mode, const float* A_log, const void* beta,
                        const float* h0, const int32_t* cu,
                        const void* dO, const float* dht, void* dq, void* dk, void* dv, float* dg,
                        void* dbeta, float* dh0, void* ws, int saved, hipStream_t s) {
#define KDA_BWD_CASE(KK, VV)                                                                    \
  if (d.K == KK && d.V == VV)                                                                   \
    return kda::chunk_bwd_t<T, KK, VV>(d, q, k, v, gate, gate_mode, A_log, beta, h0, cu, dO, dht, \
                                       dq, dk, dv, dg, dbeta, dh0, ws, saved, s);
  KDA_BWD_CASE(64, 64)
  KDA_BWD_CASE(64, 128)
  KDA_BWD_CASE(128, 64)
  KDA_BWD_CASE(128, 128)
#undef KDA_BWD_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_bwd(const kda_dims& d, kda_dtype dt, const void* q, const void* k,
                            const void* v, const float* gate, int gate_mode, const float* A_log,
                            const void* beta, const float* h0,
                            const int32_t* cu, const void* dO, const float* dht, void* dq,
                            void* dk, void* dv, float* dg, void* dbeta, float* dh0, void* ws,
                            int saved, hipStream_t s) {
  if (dt == KDA_BF16)
    return bwd_t<kda::bf16>(d, q, k, v, gate, gate_mode, A_log, beta, h0, cu, dO, dht, dq, dk, dv,
                            dg, dbeta, dh0, ws, saved, s);
  return bwd_t<float>(d, q, k, v, gate, gate_mode, A_log, beta, h0, cu, dO, dht, dq, dk, dv, dg,
                      dbeta, dh0, ws, saved, s);
}

}  // namespace kda_host
