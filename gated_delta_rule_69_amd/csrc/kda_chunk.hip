// Steps A2..A6: host side of the chunked forward (chunk_kda) and the varlen
// chunk table. The kernels and the chunk-form derivation are in
// kda_chunk_kernels.h.
#include "kda_chunk_kernels.h"

namespace kda {

// ------------------------------------------------------------------ chunk table
// ws_int layout: [0] total chunks, [1 .. N+1] first chunk of each sequence
// (seq_off, N+1 entries), [N+2 .. 2N+2) the order in which the scans take the
// sequences (scan_seq), then chunk_seq[max_chunks].
__global__ void __launch_bounds__(1024)
chunk_table_kernel(const int32_t* __restrict__ cu, int N, int* __restrict__ ws_int,
                   int max_chunks) {
  __shared__ int s_scan[1024];
  int* total = ws_int;
  int* seq_off = ws_int + 1;
  int* scan_seq = ws_int + 2 + N;
  int* chunk_seq = ws_int + 2 + 2 * N;
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
    if (n < N) seq_off[n] = carry + excl;
    // chunks of this group of sequences, all threads together: chunk carry + j
    // belongs to the first sequence whose inclusive count exceeds j (binary
    // search over the counts in LDS)
    const int group = s_scan[1023];
    for (int j = threadIdx.x; j < group; j += 1024) {
      int lo = 0, hi = 1023;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_scan[mid] > j) hi = mid;
        else lo = mid + 1;
      }
      if (carry + j < max_chunks) chunk_seq[carry + j] = base + lo;
    }
    carry += group;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    seq_off[N] = carry;
    total[0] = carry;
  }
  // scan order: longest sequence first (ties in index order), so that the
  // longest chains, which bound a scan's time, start when the launch does
  // rather than behind workgroups of shorter ones; above 1024 sequences the
  // index order (each sequence is then a small share of the batch)
  if (N <= 1024) {
    const int n = threadIdx.x;
    const int len = n < N ? cu[n + 1] - cu[n] : 0;
    s_scan[n] = len;
    __syncthreads();
    if (n < N) {
      int r = 0;
      for (int j = 0; j < N; ++j) {
        const int lj = s_scan[j];
        r += (lj > len || (lj == len && j < n)) ? 1 : 0;
      }
      scan_seq[r] = n;
    }
  } else {
    for (int n = threadIdx.x; n < N; n += 1024) scan_seq[n] = n;
  }
}

hipError_t launch_chunk_table(const int32_t* cu, int N, int* ws_int, int max_chunks, hipStream_t s) {
  hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(1024), 0, s, cu, N, ws_int, max_chunks);
  return hipGetLastError();
}

template <typename T, int K, int V>
size_t ws_bytes_t(const kda_dims& d, bool varlen) {
  const int64_t mc = max_chunks(d, varlen);
  size_t b = align256(sizeof(int) * (size_t)(2 + 2 * (size_t)d.N + mc));
  b += align256((size_t)mc * d.HV * Ws<T, K, V>::bytes_T);
  b += align256((size_t)mc * d.HV * Ws<T, K, V>::bytes_GL);
  return b;
}

template <typename T, int K, int V>
hipError_t chunk_fwd_t(const kda_dims& d, const void* q, const void* k, const void* v,
                       const float* gate, int gate_mode, const float* A_log, int qn,
                       const kda_short_conv* conv, const void* beta, const float* h0,
                       const int32_t* cu, int write_final, void* o, float* ht, void* ws,
                       int save, hipStream_t s) {
  const bool varlen = cu != nullptr;
  const int64_t mc = max_chunks(d, varlen);
  char* p = reinterpret_cast<char*>(ws);
  int* ws_int = reinterpret_cast<int*>(p);
  p += align256(sizeof(int) * (size_t)(2 + 2 * (size_t)d.N + mc));
  T* ws_T = reinterpret_cast<T*>(p);
  p += align256((size_t)mc * d.HV * Ws<T, K, V>::bytes_T);
  float* ws_GL = reinterpret_cast<float*>(p);
  p += align256((size_t)mc * d.HV * Ws<T, K, V>::bytes_GL);
  // save != 0: `ws` is the backward pass's workspace, whose first regions have
  // the forward's layout and whose per-chunk areas (T-typed, then FP32) follow
  T* ws_save = save ? reinterpret_cast<T*>(p) : nullptr;
  float* ws_save_f =
      save ? reinterpret_cast<float*>(p + align256((size_t)mc * d.HV * WsB<T, K, V>::elems * sizeof(T)))
           : nullptr;
  // the training forward takes no pre-processing (its backward has none)
  if (save && (qn || conv)) return hipErrorInvalidValue;
  if (varlen) {
    hipError_t e = launch_chunk_table(cu, d.N, ws_int, (int)mc, s);
    if (e != hipSuccess) return e;
  }
  if (mc > 0) {
    const size_t lds = conv ? IntraLds<T, K, V>::total_conv : IntraLds<T, K, V>::total;
    const kda_short_conv taps = conv ? *conv : kda_short_conv{};
    // workgroup order (see chunk_intra_kernel): value head fastest from 32 value
    // heads on, chunk fastest below. Measured, head-fastest against
    // chunk-fastest: T = 65536 with 32 heads 1261 -> 1182 us, the 32-head varlen
    // batch 799 -> 778 us; B = 4, T = 4096 with 16 heads 209 -> 217 us (gate in
    // the kernel), 187 -> 187 us (precomputed gate), 273 -> 283 us (convolution)
    const int head_fast = d.HV >= 32 ? 1 : 0;
    auto launch_intra = [&](auto qnc, auto cvc) {
      constexpr bool QN = decltype(qnc)::value, CV = decltype(cvc)::value;
      hipLaunchKernelGGL((chunk_intra_kernel<T, K, V, false, QN, CV>), dim3((unsigned)(mc * d.HV)),
                         dim3(kThreads), lds, s, (const T*)q, (const T*)k, (const T*)v, gate,
                         gate_mode, A_log, (const T*)beta, cu, ws_int, d.N, d.T, d.H, d.HV,
                         1.0f / sqrtf((float)K), ws_T, ws_GL, (T*)nullptr, (float*)nullptr, taps,
                         head_fast);
    };
    if (save) {
      // training forward: the intra kernel also forms the backward's entries
      // (so the backward after it runs no intra-chunk recompute)
      hipLaunchKernelGGL((chunk_intra_kernel<T, K, V, true, false, false, true>),
                         dim3((unsigned)(mc * d.HV)), dim3(kThreads), lds, s, (const T*)q,
                         (const T*)k, (const T*)v, gate, gate_mode, A_log, (const T*)beta, cu,
                         ws_int, d.N, d.T, d.H, d.HV, 1.0f / sqrtf((float)K), ws_T, ws_GL, ws_save,
                         ws_save_f, taps, 1);
    } else if (conv) {
      if (qn) launch_intra(std::true_type(), std::true_type());
      else launch_intra(std::false_type(), std::true_type());
    } else {
      if (qn) launch_intra(std::true_type(), std::false_type());
      else launch_intra(std::false_type(), std::false_type());
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // V-block width of the scan: every V block of a chain re-reads the chain's
  // W, Q~Gamma, Khat and P from L2, so blocks are as wide as possible while
  // the grid still has a workgroup for every compute unit.
  const int64_t chains = (int64_t)d.N * d.HV;
  const int bv = scan_block_v(chains, V, kda_host::device_cus());
  // 4 waves per workgroup (8, with half the tiles per wave, measured slower:
  // more LDS traffic and wider barriers for the same chain latency)
  // ws_save: the backward pass's per-chunk area (kda_chunk_fwd_train), which
  // receives every chunk's start state and Delta as the scan forms them
  auto launch_scan = [&](auto bvc) {
    constexpr int BVC = decltype(bvc)::value;
    if (ws_save)
      hipLaunchKernelGGL((chunk_scan_kernel<T, K, V, BVC, false, 4, true>),
                         dim3(scan_grid(chains, V, BVC)), dim3(kThreads), 0, s, (const T*)ws_T,
                         (const float*)ws_GL, (const int*)ws_int, cu, h0, d.N, d.T, d.HV,
                         write_final, (T*)o, ht, ws_save);
    else
      hipLaunchKernelGGL((chunk_scan_kernel<T, K, V, BVC, false, 4>), dim3(scan_grid(chains, V, BVC)),
                         dim3(kThreads), 0, s, (const T*)ws_T, (const float*)ws_GL,
                         (const int*)ws_int, cu, h0, d.N, d.T, d.HV, write_final, (T*)o, ht,
                         (T*)nullptr);
  };
  // FP32 with K = 128 stays at 32 columns: the 64-column tile set does not
  // fit the register file
  constexpr bool kWide = !(sizeof(T) == 4 && K == 128);
  if (bv >= 64) {
    if constexpr (kWide) launch_scan(std::integral_constant<int, 64>());
    else launch_scan(std::integral_constant<int, 32>());
  } else if (bv == 32) {
    launch_scan(std::integral_constant<int, 32>());
  } else {
    launch_scan(std::integral_constant<int, 16>());
  }
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
                         const float* gate, int gm, const float* A_log, int qn,
                         const kda_short_conv* conv, const void* beta, const float* h0,
                         const int32_t* cu, int write_final, void* o, float* ht, void* ws,
                         int save, hipStream_t s) {
  using Lds = kda::IntraLds<T, K, V>;
  static_assert(sizeof(T) == 4 && K == 128 ? true : 2 * Lds::total_conv <= 158 * 1024,
                "two workgroups per compute unit, also with the convolution taps");
  const void* fns[] = {reinterpret_cast<const void*>(&kda::chunk_intra_kernel<T, K, V, false, false, false>),
                       reinterpret_cast<const void*>(&kda::chunk_intra_kernel<T, K, V, false, true, false>),
                       reinterpret_cast<const void*>(&kda::chunk_intra_kernel<T, K, V, false, false, true>),
                       reinterpret_cast<const void*>(&kda::chunk_intra_kernel<T, K, V, false, true, true>),
                       reinterpret_cast<const void*>(&kda::chunk_intra_kernel<T, K, V, true, false, false, true>)};
  for (int i = 0; i < 5; ++i) {
    const int lds = (int)(i == 2 || i == 3 ? Lds::total_conv : Lds::total);
    hipError_t e = hipFuncSetAttribute(fns[i], hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
  }
  return kda::chunk_fwd_t<T, K, V>(d, q, k, v, gate, gm, A_log, qn, conv, beta, h0, cu, write_final,
                                   o, ht, ws, save, s);
}

template <typename T>
static hipError_t run_t(const kda_dims& d, const void* q, const void* k, const void* v,
                        const float* gate, int gm, const float* A_log, int qn,
                        const kda_short_conv* conv, const void* beta,
                        const float* h0, const int32_t* cu, int write_final, void* o, float* ht,
                        void* ws, int save, hipStream_t s) {
  if (d.K == 64 && d.V == 64) return run_kv<T, 64, 64>(d, q, k, v, gate, gm, A_log, qn, conv, beta, h0, cu, write_final, o, ht, ws, save, s);
  if (d.K == 64 && d.V == 128) return run_kv<T, 64, 128>(d, q, k, v, gate, gm, A_log, qn, conv, beta, h0, cu, write_final, o, ht, ws, save, s);
  if (d.K == 128 && d.V == 64) return run_kv<T, 128, 64>(d, q, k, v, gate, gm, A_log, qn, conv, beta, h0, cu, write_final, o, ht, ws, save, s);
  if (d.K == 128 && d.V == 128) return run_kv<T, 128, 128>(d, q, k, v, gate, gm, A_log, qn, conv, beta, h0, cu, write_final, o, ht, ws, save, s);
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_fwd(const kda_dims& d, kda_dtype dt, const void* q, const void* k,
                            const void* v, const float* gate, int gm, const float* A_log,
                            int qn, const kda_short_conv* conv, const void* beta,
                            const float* h0, const int32_t* cu, int write_final, void* o,
                            float* ht, void* ws, size_t /*ws_bytes*/, int save, hipStream_t s) {
  if (dt == KDA_BF16) return run_t<kda::bf16>(d, q, k, v, gate, gm, A_log, qn, conv, beta, h0, cu, write_final, o, ht, ws, save, s);
  return run_t<float>(d, q, k, v, gate, gm, A_log, qn, conv, beta, h0, cu, write_final, o, ht, ws, save, s);
}

}  // namespace kda_host
