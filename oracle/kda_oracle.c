/*
 * CPU oracle for the Kimi Delta Attention (KDA) scan -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, FP64, token by token. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library. It shares no code
 * with the GPU library.
 *
 * What it computes (per value head hv of a sequence, qk head h = hv / (HV/H)):
 *   S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
 *   o_t = S_t^T (q_t * scale),  scale = 1/sqrt(K)
 * This is the gated delta rule with a per-channel (per key dimension) decay,
 * i.e. the KDA recurrence behind `recurrent_kda` and `chunk_kda`
 * ("kda in torchtitan (training)", quoted attention-gym description of
 * `recurrent_kda`: FP32 states with one leading entry per logical sequence,
 * repeated offsets as empty slots whose state passes through bitwise, queries
 * scaled by 1/sqrt(K) internally).
 *
 * It is evaluated in the algebraically identical rank-1 order
 *   S' = Diag(exp g_t) S_{t-1};  u = S'^T k_t;  S_t = S' + beta_t k_t (v_t - u)^T
 * which the tests pin against the explicit (I - beta k k^T) product form.
 *
 * Inputs are flat, token-major FP64 arrays over Ttot tokens:
 *   q, k  [Ttot][H][K]     v, o [Ttot][HV][V]     g [Ttot][HV][K] (natural log)
 *   beta  [Ttot][HV]       h0, ht [N][HV][K][V]
 * Sequence n covers tokens [bos[n], eos[n]); bos == eos is an empty slot.
 * Empty slots: ht[n] is a byte copy of h0[n] (or +0.0 when h0 is NULL) and
 * no row of o is written.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int kda_oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void kda_oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Forward recurrence. Returns 0 on success, -1 on bad arguments. */
int kda_oracle_fwd(int64_t N, const int64_t* bos, const int64_t* eos, int64_t H, int64_t HV,
                   int64_t K, int64_t V, double scale, const double* q, const double* k,
                   const double* v, const double* g, const double* beta, const double* h0,
                   double* o, double* ht) {
  if (N < 0 || H <= 0 || HV <= 0 || K <= 0 || V <= 0 || HV % H != 0) return -1;
  const int64_t G = HV / H;
  const int64_t KV = K * V;
  int64_t njobs = N * HV;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t job = 0; job < njobs; ++job) {
    const int64_t n = job / HV, hv = job % HV, h = hv / G;
    double* S = ht + (n * HV + hv) * KV;
    const int64_t t0 = bos[n], t1 = eos[n];
    if (t1 < t0) { err = 1; continue; }
    if (t1 == t0) {
      /* empty slot: bitwise passthrough */
      if (h0) memcpy(S, h0 + (n * HV + hv) * KV, (size_t)KV * sizeof(double));
      else memset(S, 0, (size_t)KV * sizeof(double));
      continue;
    }
    if (h0) memcpy(S, h0 + (n * HV + hv) * KV, (size_t)KV * sizeof(double));
    else memset(S, 0, (size_t)KV * sizeof(double));
    double* u = (double*)malloc((size_t)V * sizeof(double));
    for (int64_t t = t0; t < t1; ++t) {
      const double* kt = k + (t * H + h) * K;
      const double* qt = q + (t * H + h) * K;
      const double* vt = v + (t * HV + hv) * V;
      const double* gt = g + (t * HV + hv) * K;
      const double bt = beta[t * HV + hv];
      /* S' = Diag(exp g) S */
      for (int64_t c = 0; c < K; ++c) {
        const double d = exp(gt[c]);
        for (int64_t j = 0; j < V; ++j) S[c * V + j] *= d;
      }
      /* u = S'^T k */
      for (int64_t j = 0; j < V; ++j) u[j] = 0.0;
      for (int64_t c = 0; c < K; ++c)
        for (int64_t j = 0; j < V; ++j) u[j] += S[c * V + j] * kt[c];
      /* S = S' + beta k (v - u)^T */
      for (int64_t c = 0; c < K; ++c) {
        const double bk = bt * kt[c];
        for (int64_t j = 0; j < V; ++j) S[c * V + j] += bk * (vt[j] - u[j]);
      }
      /* o = S^T (q * scale) */
      double* ot = o + (t * HV + hv) * V;
      for (int64_t j = 0; j < V; ++j) ot[j] = 0.0;
      for (int64_t c = 0; c < K; ++c) {
        const double qs = qt[c] * scale;
        for (int64_t j = 0; j < V; ++j) ot[j] += S[c * V + j] * qs;
      }
    }
    free(u);
  }
  return err ? -1 : 0;
}

/*
 * Backward of the same recurrence (reverse-mode, written out by hand).
 * Given dL/do (do_, layout of o) and dL/dS_final (dht, or NULL for zero),
 * produces dq, dk [Ttot][H][K] (summed over the HV/H value heads sharing a qk
 * head), dv [Ttot][HV][V], dg [Ttot][HV][K] (w.r.t. the natural-log g),
 * dbeta [Ttot][HV] and dh0 [N][HV][K][V].
 *
 * Per token, going backwards, with S' = Diag(exp g) S_{t-1}, r = v - S'^T k and
 * dS holding dL/dS_t:
 *   dS  += q~ do^T            dq = scale * S_t do
 *   dv   = beta dS^T k        dbeta = k^T dS r
 *   dk   = beta (dS r - S' dS^T k)
 *   dS'  = dS - beta k (k^T dS)
 *   dg   = rowsum(dS' (.) S')  dS <- Diag(exp g) dS'
 * and dh0 = dS after the first token. Empty slots: dh0 = dht.
 * The tests pin this against central finite differences of kda_oracle_fwd.
 */
int kda_oracle_bwd(int64_t N, const int64_t* bos, const int64_t* eos, int64_t H, int64_t HV,
                   int64_t K, int64_t V, double scale, const double* q, const double* k,
                   const double* v, const double* g, const double* beta, const double* h0,
                   const double* do_, const double* dht, double* dq, double* dk, double* dv,
                   double* dg, double* dbeta, double* dh0) {
  if (N < 0 || H <= 0 || HV <= 0 || K <= 0 || V <= 0 || HV % H != 0) return -1;
  const int64_t G = HV / H;
  const int64_t KV = K * V;
  int64_t Ttot = 0;
  for (int64_t n = 0; n < N; ++n) if (eos[n] > Ttot) Ttot = eos[n];
  /* dq/dk are shared by G value heads: accumulate per value head, then reduce. */
  double* dq_hv = (double*)calloc((size_t)(Ttot * HV * K > 0 ? Ttot * HV * K : 1), sizeof(double));
  double* dk_hv = (double*)calloc((size_t)(Ttot * HV * K > 0 ? Ttot * HV * K : 1), sizeof(double));
  int64_t njobs = N * HV;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t job = 0; job < njobs; ++job) {
    const int64_t n = job / HV, hv = job % HV, h = hv / G;
    const int64_t t0 = bos[n], t1 = eos[n], L = t1 - t0;
    double* dS = dh0 + (n * HV + hv) * KV;
    if (dht) memcpy(dS, dht + (n * HV + hv) * KV, (size_t)KV * sizeof(double));
    else memset(dS, 0, (size_t)KV * sizeof(double));
    if (L <= 0) continue;
    /* forward pass, keeping every S_t (t = 0..L, S_0 = initial) */
    double* Ss = (double*)malloc((size_t)(L + 1) * KV * sizeof(double));
    double* Sp = (double*)malloc((size_t)KV * sizeof(double));
    double* tmpV = (double*)malloc((size_t)V * sizeof(double));
    double* r = (double*)malloc((size_t)V * sizeof(double));
    double* kdS = (double*)malloc((size_t)V * sizeof(double));
    if (!Ss || !Sp || !tmpV || !r || !kdS) { err = 1; free(Ss); free(Sp); free(tmpV); free(r); free(kdS); continue; }
    if (h0) memcpy(Ss, h0 + (n * HV + hv) * KV, (size_t)KV * sizeof(double));
    else memset(Ss, 0, (size_t)KV * sizeof(double));
    for (int64_t i = 0; i < L; ++i) {
      const int64_t t = t0 + i;
      const double* kt = k + (t * H + h) * K;
      const double* vt = v + (t * HV + hv) * V;
      const double* gt = g + (t * HV + hv) * K;
      const double bt = beta[t * HV + hv];
      const double* Sprev = Ss + i * KV;
      double* Snext = Ss + (i + 1) * KV;
      for (int64_t c = 0; c < K; ++c) {
        const double d = exp(gt[c]);
        for (int64_t j = 0; j < V; ++j) Snext[c * V + j] = d * Sprev[c * V + j];
      }
      for (int64_t j = 0; j < V; ++j) tmpV[j] = 0.0;
      for (int64_t c = 0; c < K; ++c)
        for (int64_t j = 0; j < V; ++j) tmpV[j] += Snext[c * V + j] * kt[c];
      for (int64_t c = 0; c < K; ++c)
        for (int64_t j = 0; j < V; ++j) Snext[c * V + j] += bt * kt[c] * (vt[j] - tmpV[j]);
    }
    /* reverse pass */
    for (int64_t i = L - 1; i >= 0; --i) {
      const int64_t t = t0 + i;
      const double* qt = q + (t * H + h) * K;
      const double* kt = k + (t * H + h) * K;
      const double* vt = v + (t * HV + hv) * V;
      const double* gt = g + (t * HV + hv) * K;
      const double* dot = do_ + (t * HV + hv) * V;
      const double bt = beta[t * HV + hv];
      const double* St = Ss + (i + 1) * KV;
      const double* Sprev = Ss + i * KV;
      /* output: o = S_t^T q~ */
      double* dqt = dq_hv + (t * HV + hv) * K;
      for (int64_t c = 0; c < K; ++c) {
        double acc = 0.0;
        for (int64_t j = 0; j < V; ++j) acc += St[c * V + j] * dot[j];
        dqt[c] = scale * acc;
        const double qs = qt[c] * scale;
        for (int64_t j = 0; j < V; ++j) dS[c * V + j] += qs * dot[j];
      }
      /* S' and r = v - S'^T k */
      for (int64_t c = 0; c < K; ++c) {
        const double d = exp(gt[c]);
        for (int64_t j = 0; j < V; ++j) Sp[c * V + j] = d * Sprev[c * V + j];
      }
      for (int64_t j = 0; j < V; ++j) tmpV[j] = 0.0;
      for (int64_t c = 0; c < K; ++c)
        for (int64_t j = 0; j < V; ++j) tmpV[j] += Sp[c * V + j] * kt[c];
      for (int64_t j = 0; j < V; ++j) r[j] = vt[j] - tmpV[j];
      /* kdS = dS^T k */
      for (int64_t j = 0; j < V; ++j) kdS[j] = 0.0;
      for (int64_t c = 0; c < K; ++c)
        for (int64_t j = 0; j < V; ++j) kdS[j] += kt[c] * dS[c * V + j];
      double* dvt = dv + (t * HV + hv) * V;
      for (int64_t j = 0; j < V; ++j) dvt[j] = bt * kdS[j];
      double db = 0.0;
      double* dkt = dk_hv + (t * HV + hv) * K;
      for (int64_t c = 0; c < K; ++c) {
        double dSr = 0.0, SpkdS = 0.0;
        for (int64_t j = 0; j < V; ++j) {
          dSr += dS[c * V + j] * r[j];
          SpkdS += Sp[c * V + j] * kdS[j];
        }
        db += kt[c] * dSr;
        dkt[c] = bt * (dSr - SpkdS);
      }
      dbeta[t * HV + hv] = db;
      /* dS' = dS - beta k kdS^T ; dg = rowsum(dS' * S') ; dS = Diag(exp g) dS' */
      double* dgt = dg + (t * HV + hv) * K;
      for (int64_t c = 0; c < K; ++c) {
        const double d = exp(gt[c]);
        double acc = 0.0;
        for (int64_t j = 0; j < V; ++j) {
          const double dsp = dS[c * V + j] - bt * kt[c] * kdS[j];
          acc += dsp * Sp[c * V + j];
          dS[c * V + j] = d * dsp;
        }
        dgt[c] = acc;
      }
    }
    free(Ss); free(Sp); free(tmpV); free(r); free(kdS);
  }
  /* GVA reduction of dq, dk over the value heads of each qk head */
  for (int64_t t = 0; t < Ttot; ++t)
    for (int64_t h = 0; h < H; ++h)
      for (int64_t c = 0; c < K; ++c) {
        double aq = 0.0, ak = 0.0;
        for (int64_t j = 0; j < G; ++j) {
          aq += dq_hv[(t * HV + h * G + j) * K + c];
          ak += dk_hv[(t * HV + h * G + j) * K + c];
        }
        dq[(t * H + h) * K + c] = aq;
        dk[(t * H + h) * K + c] = ak;
      }
  free(dq_hv); free(dk_hv);
  return err ? -1 : 0;
}
