/*
 * gdr_oracle.c -- plain fp64 CPU oracle for the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The GPU product
 * path never links, calls or falls back to it.  It shares no code, header or
 * constant with the HIP library.
 *
 * What it computes (one function, the definition itself):
 *
 *   For every sequence n and head h, starting from S = S_init (or 0), for each
 *   token t of the sequence in order
 *       alpha = exp(g_t)
 *       S     = alpha * S (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *       o_t   = S q_t                  (the state after the update)
 *   and S_out = S after the last token.
 *
 * This is the gated delta rule recurrence with a per-head state S of shape
 * dv x dk (row i of S is the dk-vector s_i; dk is the contiguous index).  The
 * fixup passage of the FlashInfer PR #3866 page ("CP delta-rule precompute
 * optimisation for ultra-low parallelism", code changes, section 2,
 * accumulate_state_fragment) fixes the orientation S_next = S * M: the state
 * multiplies transfer matrices from the left, i.e. row by row, which is the
 * orientation used here.
 *
 * Row i of the update written out:
 *       s_i <- alpha * (s_i - beta (s_i . k) k) + beta v_i k
 *
 * Optionally the state at the end of every chunk of `chunk` tokens (chunks
 * restart at each sequence start) is recorded, in the packed chunk order
 * given by chunk_offsets: slot chunk_offsets[n] + j holds the state after the
 * last token of chunk j of sequence n.  These are the "fixed" chunk states.
 *
 * Everything is double precision.  Inputs q, k, v may be given as bf16 bit
 * patterns (uint16), float32 or float64; bf16 -> double is exact (the bits are
 * the upper half of a float32).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_BF16 = 0, ORC_F32 = 1, ORC_F64 = 2 };

/* bf16 bit pattern -> double: place the 16 bits in the high half of an
 * IEEE binary32 word.  Exact. */
static double orc_bf16_to_double(uint16_t bits) {
  uint32_t w = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

static double orc_load(const void* base, int dtype, size_t idx) {
  switch (dtype) {
    case ORC_BF16: return orc_bf16_to_double(((const uint16_t*)base)[idx]);
    case ORC_F32: return (double)((const float*)base)[idx];
    default: return ((const double*)base)[idx];
  }
}

/*
 * oracle_recurrent
 *   q, k      [T_total, H, dk]  (dtype qkv_dtype)
 *   v         [T_total, H, dv]  (dtype qkv_dtype)
 *   g, beta   [T_total, H]      double; alpha = exp(g)
 *   cu        [N+1]             int64 token offsets of the packed sequences
 *   state_in  [N, H, dv, dk]    double, or NULL for a zero initial state
 *   state_out [N, H, dv, dk]    double (may alias state_in)
 *   o         [T_total, H, dv]  double
 *   pairs     [n_pairs, 2]      (n, h) pairs to compute, or NULL for all N*H
 *   chunk, chunk_offsets, chunk_states: optional recording of end-of-chunk
 *             states into chunk_states[chunk_offsets[n] + j, h, dv, dk]
 *             (chunk_states == NULL disables it)
 *   n_threads OpenMP threads (<= 0: library default)
 * Returns 0, or -1 when an allocation fails.
 */
int oracle_recurrent(const void* q, const void* k, const void* v, int qkv_dtype,
                     const double* g, const double* beta, const int64_t* cu, int N,
                     const double* state_in, double* state_out, double* o,
                     int H, int dk, int dv,
                     const int64_t* pairs, int n_pairs,
                     int chunk, const int64_t* chunk_offsets, double* chunk_states,
                     int n_threads) {
  int total = pairs ? n_pairs : N * H;
  int failed = 0;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif

#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
  for (int p = 0; p < total; ++p) {
    int n = pairs ? (int)pairs[2 * p] : p / H;
    int h = pairs ? (int)pairs[2 * p + 1] : p % H;
    double* S = (double*)malloc(sizeof(double) * (size_t)dv * dk);
    double* kk = (double*)malloc(sizeof(double) * (size_t)dk);
    double* qq = (double*)malloc(sizeof(double) * (size_t)dk);
    if (!S || !kk || !qq) {
      free(S); free(kk); free(qq);
      failed |= 1;
      continue;
    }
    size_t sbase = ((size_t)n * H + h) * (size_t)dv * dk;
    for (size_t e = 0; e < (size_t)dv * dk; ++e) S[e] = state_in ? state_in[sbase + e] : 0.0;

    int64_t t0 = cu[n], t1 = cu[n + 1];
    for (int64_t t = t0; t < t1; ++t) {
      size_t th = (size_t)t * H + h;
      double alpha = exp(g[th]);
      double b = beta[th];
      for (int j = 0; j < dk; ++j) {
        kk[j] = orc_load(k, qkv_dtype, th * dk + j);
        qq[j] = orc_load(q, qkv_dtype, th * dk + j);
      }
      for (int i = 0; i < dv; ++i) {
        double* s = S + (size_t)i * dk;
        double vi = orc_load(v, qkv_dtype, th * dv + i);
        double sk = 0.0;
        for (int j = 0; j < dk; ++j) sk += s[j] * kk[j];
        /* s <- alpha (s - beta (s.k) k) + beta v_i k */
        for (int j = 0; j < dk; ++j) s[j] = alpha * (s[j] - b * sk * kk[j]) + b * vi * kk[j];
        double oi = 0.0;
        for (int j = 0; j < dk; ++j) oi += s[j] * qq[j];
        o[th * dv + i] = oi;
      }
      if (chunk_states && chunk > 0) {
        int64_t local = t - t0;
        if ((local + 1) % chunk == 0 || t + 1 == t1) {
          int64_t slot = chunk_offsets[n] + local / chunk;
          double* dst = chunk_states + ((size_t)slot * H + h) * (size_t)dv * dk;
          memcpy(dst, S, sizeof(double) * (size_t)dv * dk);
        }
      }
    }
    memcpy(state_out + sbase, S, sizeof(double) * (size_t)dv * dk);
    free(S); free(kk); free(qq);
  }
  return failed ? -1 : 0;
}

/* Threads the OpenMP runtime would use by default (for reporting). */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
