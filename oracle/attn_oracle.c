/*
 * attn_oracle.c -- plain, slow fp64 CPU oracle for exact attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only tests/, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no code, header or constant with the HIP library.
 *
 * What it computes (per head, all tensors row-major [N][d], fp64):
 *
 *   S = s * Q K^T,  P = softmax(S) row-wise,  O = P V,  L_i = m_i + ln(l_i)
 *
 * following the standard-attention definition and the softmax decomposition
 * (m, f, l) in the FLASH-ATTN page (taking-lying-flat), FlashAttention paper
 * summary, sections "Background" (standard attention) and "Tiling and
 * Recomputation" (definitions of m(x), f(x), l(x), softmax(x)); the LSE
 * statistic L = m + log(l) is from the same page's FlashAttention-2 section.
 * The causal mask (S_ij = -inf for j > i) is from the FlashAttention-2 section
 * of that page.  The softmax scale s and the sliding window are not written in
 * the pages' formulas; s multiplies Q K^T, and a window W > 0 keeps key j for
 * query i when i - j < W (causal) or |i - j| < W (non-causal).
 *
 * The backward follows the chain rule listed in the FlashAttention-2 section
 * "Background" of the FLASH-ATTN page: dV = P^T dO, dP = dO V^T,
 * dS = dsoftmax(dP), dQ = dS K, dK = dS^T Q, with dsoftmax written out as the
 * softmax Jacobian dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik) and the scale s
 * carried through the chain rule into dQ and dK.
 *
 * Dropout (named by the FLASH-ATTN page as a supported variant, and in the
 * FlashAttention-2 "Background" paragraph as an elementwise operation on P):
 * the pages fix no random-number contract, so the reading taken here is
 * inverted dropout on the normalised probabilities, P~ = P o Z / q with
 * keep indicators Z drawn by the counter-based generator Philox-4x32-10
 * (oracle_philox), keep probability q = (256 - t) / 256 for the integer
 * threshold t = round(256 p), and L the log-sum-exp of the undropped scores.
 * The backward applies the same Z: dV = P~^T dO, dP = (dO V^T) o Z / q,
 * D_i = sum_j P_ij dP_ij, dS = P o (dP - D), dQ = s dS K, dK = s dS^T Q.
 *
 * Every quantity is an explicit fp64 array: one full score row per query in
 * the forward, and the full N x N matrices P and dS of one head in the
 * backward.  No blocking, no fused recurrence: the online (block-by-block)
 * recurrences live in oracle_online_fwd only, which exists to check the
 * plain definition against the pages' decomposition identities.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

/* ---- number formats: decoding only (the inputs arrive already encoded) ---- */

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
double oracle_bf16_to_f64(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

void oracle_bf16_decode(const uint16_t* src, double* dst, long n) {
  for (long i = 0; i < n; ++i) dst[i] = oracle_bf16_to_f64(src[i]);
}

/* OCP FP8 E4M3 ("fn" variant): 1 sign, 4 exponent bits (bias 7), 3 mantissa
 * bits; exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN; there is
 * no infinity, so the largest finite value is 1.75 * 2^8 = 448. */
double oracle_e4m3_to_f64(uint8_t c) {
  int sign = (c >> 7) & 1;
  int e = (c >> 3) & 0xF;
  int m = c & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

/* x = code_value * descale */
void oracle_e4m3_decode(const uint8_t* src, double descale, double* dst, long n) {
  for (long i = 0; i < n; ++i) dst[i] = oracle_e4m3_to_f64(src[i]) * descale;
}

/* Block-quantised tensor [heads][rows][d]: row r of head h is code value *
 * descales[h * nblk + r / block_rows] (FLASH-ATTN page, FlashAttention-3
 * summary, block quantisation: one scale per block of rows). */
void oracle_e4m3_decode_blocks(const uint8_t* src, long heads, long rows, int d,
                               int block_rows, const double* descales, double* dst) {
  const long nblk = (rows + block_rows - 1) / block_rows;
  for (long hh = 0; hh < heads; ++hh)
    for (long r = 0; r < rows; ++r) {
      const double ds = descales[hh * nblk + r / block_rows];
      const long off = (hh * rows + r) * d;
      for (int c = 0; c < d; ++c) dst[off + c] = oracle_e4m3_to_f64(src[off + c]) * ds;
    }
}

/* ---- visibility: which keys a query may attend to ---- */
int oracle_visible(long i, long j, int causal, long window) {
  if (causal && j > i) return 0;
  if (window > 0) {
    long diff = i - j;
    if (diff < 0) diff = -diff;
    if (diff >= window) return 0;
  }
  return 1;
}

static double dot(const double* a, const double* b, int d) {
  double acc = 0.0;
  for (int k = 0; k < d; ++k) acc += a[k] * b[k];
  return acc;
}

/* One query row qi, at position i among the N keys of one head: explicit
 * score row S_i, its max m_i, the sum l_i = sum_j exp(S_ij - m_i), the
 * probability row P_i, O_i = P_i V and L_i = m_i + ln(l_i).  srow and prow
 * are caller scratch of length N. */
static void query_row(int N, int d, double scale, int causal, long window,
                      const double* qi, long i, const double* k, const double* v,
                      double* srow, double* prow, double* o_row, double* lse_out) {
  double m = -INFINITY;
  for (long j = 0; j < N; ++j) {
    if (oracle_visible(i, j, causal, window)) {
      srow[j] = scale * dot(qi, k + j * (long)d, d);
      if (srow[j] > m) m = srow[j];
    } else {
      srow[j] = -INFINITY;
    }
  }
  double l = 0.0;
  for (long j = 0; j < N; ++j) {
    prow[j] = (srow[j] == -INFINITY) ? 0.0 : exp(srow[j] - m);
    l += prow[j];
  }
  for (long j = 0; j < N; ++j) prow[j] /= l;
  for (int c = 0; c < d; ++c) o_row[c] = 0.0;
  for (long j = 0; j < N; ++j) {
    if (prow[j] == 0.0) continue;
    const double* vj = v + j * (long)d;
    for (int c = 0; c < d; ++c) o_row[c] += prow[j] * vj[c];
  }
  if (lse_out) *lse_out = m + log(l);
}

/* Row i of one head whose queries and keys are the same N positions. */
static void fwd_row(int N, int d, double scale, int causal, long window,
                    const double* q, const double* k, const double* v, long i,
                    double* srow, double* prow, double* o_row, double* lse_out) {
  query_row(N, d, scale, causal, window, q + (long)i * d, i, k, v, srow, prow, o_row,
            lse_out);
}

/* Forward over BH heads, every row.  q,k,v,o: [BH][N][d]; lse: [BH][N]
 * (may be NULL).  Rows are independent, so they are spread over threads. */
void oracle_fwd(int BH, int N, int d, double scale, int causal, long window,
                const double* q, const double* k, const double* v, double* o,
                double* lse, int nthreads) {
  if (nthreads > 0) omp_set_num_threads(nthreads);
  long total = (long)BH * N;
#pragma omp parallel
  {
    double* srow = (double*)malloc(sizeof(double) * (size_t)N);
    double* prow = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 16)
    for (long r = 0; r < total; ++r) {
      long h = r / N, i = r % N;
      long off = h * (long)N * d;
      fwd_row(N, d, scale, causal, window, q + off, k + off, v + off, i, srow,
              prow, o + r * d, lse ? lse + r : NULL);
    }
    free(srow);
    free(prow);
  }
}

/* Forward for selected rows of one head (rows[t] in [0,N)); o_rows: [nrows][d]. */
void oracle_fwd_rows(int N, int d, double scale, int causal, long window,
                     const double* q, const double* k, const double* v,
                     const long* rows, int nrows, double* o_rows,
                     double* lse_rows, int nthreads) {
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
  {
    double* srow = (double*)malloc(sizeof(double) * (size_t)N);
    double* prow = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
    for (int t = 0; t < nrows; ++t)
      fwd_row(N, d, scale, causal, window, q, k, v, rows[t], srow, prow,
              o_rows + (long)t * d, lse_rows ? lse_rows + t : NULL);
    free(srow);
    free(prow);
  }
}

/* The probability row P_i of one head (for the row-sum and closed-form pins). */
void oracle_probs_row(int N, int d, double scale, int causal, long window,
                      const double* q, const double* k, const double* v, long i,
                      double* prow) {
  double* srow = (double*)malloc(sizeof(double) * (size_t)N);
  double* o_row = (double*)malloc(sizeof(double) * (size_t)d);
  fwd_row(N, d, scale, causal, window, q, k, v, i, srow, prow, o_row, NULL);
  free(srow);
  free(o_row);
}

/* Multi-query and grouped-query attention (FLASH-ATTN page, FlashAttention-2
 * section, the paragraph on MQA and GQA): H query heads share Hkv key/value
 * heads, H a multiple of Hkv.  Query head h of batch element b reads key and
 * value head b*Hkv + h/(H/Hkv) through its index; nothing is copied.  (The
 * page does not say which query heads share a head; consecutive ones do
 * here.)  Layouts: q, o [B][H][N][d]; k, v [B][Hkv][N][d]; lse [B][H][N]. */
static long kv_head_of(long bh, int H, int Hkv) {
  return (bh / H) * Hkv + (bh % H) / (H / Hkv);
}

void oracle_fwd_gqa(int B, int H, int Hkv, int N, int d, double scale, int causal,
                    long window, const double* q, const double* k, const double* v,
                    double* o, double* lse, int nthreads) {
  if (nthreads > 0) omp_set_num_threads(nthreads);
  long total = (long)B * H * N;
#pragma omp parallel
  {
    double* srow = (double*)malloc(sizeof(double) * (size_t)N);
    double* prow = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 16)
    for (long r = 0; r < total; ++r) {
      long bh = r / N, i = r % N;
      long qoff = bh * (long)N * d, kvoff = kv_head_of(bh, H, Hkv) * (long)N * d;
      fwd_row(N, d, scale, causal, window, q + qoff, k + kvoff, v + kvoff, i, srow,
              prow, o + r * d, lse ? lse + r : NULL);
    }
    free(srow);
    free(prow);
  }
}

/* A short block of Nq queries against Nk keys (decode: the FlashAttention-3
 * page's point on inference, one new query per step against every cached
 * key).  The block is the last Nq positions of the sequence: query row i sits
 * at key position Nk - Nq + i and the masks of the ordinary forward apply to
 * that position (causal: j <= Nk - Nq + i).  The pages fix no alignment for
 * Nq < Nk; this one reduces to the ordinary forward when Nq = Nk.  Shared
 * key/value heads as in oracle_fwd_gqa.
 * q, o [B][H][Nq][d]; k, v [B][Hkv][Nk][d]; lse [B][H][Nq]. */
void oracle_fwd_decode(int B, int H, int Hkv, int Nq, int Nk, int d, double scale,
                       int causal, long window, const double* q, const double* k,
                       const double* v, double* o, double* lse, int nthreads) {
  if (nthreads > 0) omp_set_num_threads(nthreads);
  long total = (long)B * H * Nq;
#pragma omp parallel
  {
    double* srow = (double*)malloc(sizeof(double) * (size_t)Nk);
    double* prow = (double*)malloc(sizeof(double) * (size_t)Nk);
#pragma omp for schedule(dynamic, 4)
    for (long r = 0; r < total; ++r) {
      long bh = r / Nq, i = r % Nq;
      long kvoff = kv_head_of(bh, H, Hkv) * (long)Nk * d;
      query_row(Nk, d, scale, causal, window, q + r * d, (long)(Nk - Nq) + i, k + kvoff,
                v + kvoff, srow, prow, o + r * d, lse ? lse + r : NULL);
    }
    free(srow);
    free(prow);
  }
}

/* Backward over BH heads.  Inputs q,k,v,dout: [BH][N][d].  Outputs dq,dk,dv:
 * [BH][N][d]; Dvec: [BH][N] receives D_i = sum_j P_ij dP_ij (may be NULL).
 * Per head: pass 1 builds the explicit rows of P and dS (and dQ) one query
 * at a time; pass 2 forms dV_j = sum_i P_ij dO_i and dK_j = s sum_i dS_ij Q_i
 * one key at a time from the stored matrices. */
void oracle_bwd(int BH, int N, int d, double scale, int causal, long window,
                const double* q, const double* k, const double* v,
                const double* dout, double* dq, double* dk, double* dv,
                double* Dvec, int nthreads) {
  if (nthreads > 0) omp_set_num_threads(nthreads);
  double* P = (double*)malloc(sizeof(double) * (size_t)N * (size_t)N);
  double* dS = (double*)malloc(sizeof(double) * (size_t)N * (size_t)N);
  for (int h = 0; h < BH; ++h) {
    long off = (long)h * N * d;
    const double *qh = q + off, *kh = k + off, *vh = v + off, *doh = dout + off;
#pragma omp parallel
    {
      double* srow = (double*)malloc(sizeof(double) * (size_t)N);
      double* dprow = (double*)malloc(sizeof(double) * (size_t)N);
      double* o_row = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 8)
      for (long i = 0; i < N; ++i) {
        double* prow = P + i * (long)N;
        double* dsrow = dS + i * (long)N;
        fwd_row(N, d, scale, causal, window, qh, kh, vh, i, srow, prow, o_row, NULL);
        /* dP_i = dO_i V^T */
        for (long j = 0; j < N; ++j)
          dprow[j] = oracle_visible(i, j, causal, window)
                         ? dot(doh + i * (long)d, vh + j * (long)d, d)
                         : 0.0;
        /* D_i = sum_j P_ij dP_ij ; dS_ij = P_ij (dP_ij - D_i) */
        double Di = 0.0;
        for (long j = 0; j < N; ++j) Di += prow[j] * dprow[j];
        for (long j = 0; j < N; ++j) dsrow[j] = prow[j] * (dprow[j] - Di);
        if (Dvec) Dvec[(long)h * N + i] = Di;
        /* dQ_i = s sum_j dS_ij K_j */
        double* dqi = dq + off + i * (long)d;
        for (int c = 0; c < d; ++c) dqi[c] = 0.0;
        for (long j = 0; j < N; ++j) {
          if (dsrow[j] == 0.0) continue;
          const double* kj = kh + j * (long)d;
          for (int c = 0; c < d; ++c) dqi[c] += dsrow[j] * kj[c];
        }
        for (int c = 0; c < d; ++c) dqi[c] *= scale;
      }
      free(srow);
      free(dprow);
      free(o_row);
    }
#pragma omp parallel for schedule(dynamic, 8)
    for (long j = 0; j < N; ++j) {
      double* dvj = dv + off + j * (long)d;
      double* dkj = dk + off + j * (long)d;
      for (int c = 0; c < d; ++c) dvj[c] = dkj[c] = 0.0;
      for (long i = 0; i < N; ++i) {
        double p = P[i * (long)N + j], ds = dS[i * (long)N + j];
        const double* doi = doh + i * (long)d;
        const double* qi = qh + i * (long)d;
        if (p != 0.0)
          for (int c = 0; c < d; ++c) dvj[c] += p * doi[c];
        if (ds != 0.0)
          for (int c = 0; c < d; ++c) dkj[c] += ds * qi[c];
      }
      for (int c = 0; c < d; ++c) dkj[c] *= scale;
    }
  }
  free(P);
  free(dS);
}

/* Block-by-block recurrences over a partition of the keys of one head, for
 * cross-checking oracle_fwd against the decomposition identities of the
 * FLASH-ATTN page.  bounds[0]=0 < bounds[1] < ... < bounds[nparts]=N.
 *   form 1: the FlashAttention online softmax, where the output is kept
 *           normalised after every block, O <- diag(l_old/l_new * e^{m_old-m_new}) O
 *           + diag(l_new)^{-1} e^{S_blk - m_new} V_blk ("Tiling and Recomputation"
 *           and the two-block online-softmax equations of the FlashAttention-2
 *           section);
 *   form 2: the FlashAttention-2 form with an unnormalised accumulator,
 *           O~ <- diag(e^{m_old-m_new}) O~ + e^{S_blk - m_new} V_blk, divided by
 *           l once at the end (FlashAttention-2 section).
 * Rows whose visible set is still empty keep m = -inf, l = 0, O = 0. */
void oracle_online_fwd(int N, int d, double scale, int causal, long window,
                       const double* q, const double* k, const double* v,
                       const long* bounds, int nparts, int form, double* o,
                       double* lse) {
  double* sblk = (double*)malloc(sizeof(double) * (size_t)N);
  for (long i = 0; i < N; ++i) {
    const double* qi = q + i * (long)d;
    double* oi = o + i * (long)d;
    double m = -INFINITY, l = 0.0;
    for (int c = 0; c < d; ++c) oi[c] = 0.0;
    for (int b = 0; b < nparts; ++b) {
      long j0 = bounds[b], j1 = bounds[b + 1];
      double mb = -INFINITY;
      for (long j = j0; j < j1; ++j) {
        sblk[j - j0] = oracle_visible(i, j, causal, window)
                           ? scale * dot(qi, k + j * (long)d, d)
                           : -INFINITY;
        if (sblk[j - j0] > mb) mb = sblk[j - j0];
      }
      double m_new = (mb > m) ? mb : m;
      if (m_new == -INFINITY) continue; /* nothing visible yet */
      double alpha = (m == -INFINITY) ? 0.0 : exp(m - m_new);
      double lb = 0.0;
      for (long j = j0; j < j1; ++j)
        lb += (sblk[j - j0] == -INFINITY) ? 0.0 : exp(sblk[j - j0] - m_new);
      double l_new = alpha * l + lb;
      if (form == 1) {
        double keep = (l_new > 0.0) ? alpha * l / l_new : 0.0;
        for (int c = 0; c < d; ++c) oi[c] *= keep;
        for (long j = j0; j < j1; ++j) {
          if (sblk[j - j0] == -INFINITY) continue;
          double p = exp(sblk[j - j0] - m_new) / l_new;
          const double* vj = v + j * (long)d;
          for (int c = 0; c < d; ++c) oi[c] += p * vj[c];
        }
      } else {
        for (int c = 0; c < d; ++c) oi[c] *= alpha;
        for (long j = j0; j < j1; ++j) {
          if (sblk[j - j0] == -INFINITY) continue;
          double p = exp(sblk[j - j0] - m_new);
          const double* vj = v + j * (long)d;
          for (int c = 0; c < d; ++c) oi[c] += p * vj[c];
        }
      }
      m = m_new;
      l = l_new;
    }
    if (form != 1)
      for (int c = 0; c < d; ++c) oi[c] /= l;
    if (lse) lse[i] = m + log(l);
  }
  free(sblk);
}

/* Backward of the grouped-query forward above (same passage): every query
 * head's gradients are those of one ordinary head reading its key/value
 * head (oracle_bwd), and the dK, dV of a shared head are the sums of the dK,
 * dV its query heads produce, added in increasing query-head order.
 * q, dout, dq [B][H][N][d]; k, v, dk, dv [B][Hkv][N][d]; Dvec [B][H][N]. */
void oracle_bwd_gqa(int B, int H, int Hkv, int N, int d, double scale, int causal,
                    long window, const double* q, const double* k, const double* v,
                    const double* dout, double* dq, double* dk, double* dv,
                    double* Dvec, int nthreads) {
  const long hs = (long)N * d;
  double* dk1 = (double*)malloc(sizeof(double) * (size_t)hs);
  double* dv1 = (double*)malloc(sizeof(double) * (size_t)hs);
  for (long x = 0; x < (long)B * Hkv * hs; ++x) dk[x] = dv[x] = 0.0;
  for (long bh = 0; bh < (long)B * H; ++bh) {
    const long kv = kv_head_of(bh, H, Hkv);
    oracle_bwd(1, N, d, scale, causal, window, q + bh * hs, k + kv * hs, v + kv * hs,
               dout + bh * hs, dq + bh * hs, dk1, dv1, Dvec ? Dvec + bh * N : NULL,
               nthreads);
    for (long x = 0; x < hs; ++x) {
      dk[kv * hs + x] += dk1[x];
      dv[kv * hs + x] += dv1[x];
    }
  }
  free(dk1);
  free(dv1);
}

/* ---- dropout: counter-based random numbers and the keep rule ---- */

/* Philox-4xW-R (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
 * easy as 1, 2, 3", SC 2011): a 4-word counter and a 2-word key; each of R
 * rounds multiplies counter words 0 and 2 by the constants M0, M1 into
 * double-width products, and the new counter is
 *   (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0));
 * between rounds the key words grow by the Weyl constants W0, W1.  One
 * routine serves both word widths, W = 32 and W = 64 (all words are held in
 * uint64_t; at W = 32 only their low halves are used). */
static const uint64_t PHILOX_M[2][2] = {{0xD2511F53ull, 0xCD9E8D57ull},
                                        {0xD2E7470EE14C6C93ull, 0xCA5A826395121157ull}};
static const uint64_t PHILOX_WEYL[2][2] = {{0x9E3779B9ull, 0xBB67AE85ull},
                                           {0x9E3779B97F4A7C15ull, 0xBB67AE8584CAA73Bull}};

static void mulhilo(int W, uint64_t a, uint64_t b, uint64_t* hi, uint64_t* lo) {
  if (W == 32) {
    const uint64_t p = a * b; /* both < 2^32: exact in 64 bits */
    *hi = p >> 32;
    *lo = p & 0xFFFFFFFFull;
  } else {
    const unsigned __int128 p = (unsigned __int128)a * b;
    *hi = (uint64_t)(p >> 64);
    *lo = (uint64_t)p;
  }
}

/* W in {32, 64}; R >= 1 rounds. */
void oracle_philox(int W, int R, const uint64_t ctr_in[4], const uint64_t key_in[2],
                   uint64_t out[4]) {
  const int wi = (W == 64);
  const uint64_t mask = wi ? ~0ull : 0xFFFFFFFFull;
  uint64_t c[4], k[2];
  for (int x = 0; x < 4; ++x) c[x] = ctr_in[x] & mask;
  for (int x = 0; x < 2; ++x) k[x] = key_in[x] & mask;
  for (int r = 0; r < R; ++r) {
    if (r > 0) {
      k[0] = (k[0] + PHILOX_WEYL[wi][0]) & mask;
      k[1] = (k[1] + PHILOX_WEYL[wi][1]) & mask;
    }
    uint64_t hi0, lo0, hi1, lo1;
    mulhilo(W, PHILOX_M[wi][0], c[0], &hi0, &lo0);
    mulhilo(W, PHILOX_M[wi][1], c[2], &hi1, &lo1);
    const uint64_t n0 = hi1 ^ c[1] ^ k[0], n2 = hi0 ^ c[3] ^ k[1];
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
  for (int x = 0; x < 4; ++x) out[x] = c[x];
}

void oracle_philox_constants(int W, uint64_t out[4]) {
  const int wi = (W == 64);
  out[0] = PHILOX_M[wi][0];
  out[1] = PHILOX_M[wi][1];
  out[2] = PHILOX_WEYL[wi][0];
  out[3] = PHILOX_WEYL[wi][1];
}

/* Threshold t = round(256 p) (halves up) of a dropout probability p. */
int oracle_dropout_threshold(double p) { return (int)floor(p * 256.0 + 0.5); }

/* The random byte of (query head bh, query i, key j): the score matrix of a
 * head is cut into 4 x 4 sub-blocks; sub-block (i/4, j/4) draws one
 * Philox-4x32-10 output with counter (j/4, i/4, bh, offset) and key (low,
 * high 32 bits of seed); word i%4 belongs to query i, and byte j%4 of that
 * word (least significant first) to key j. */
int oracle_dropout_byte(uint64_t seed, uint32_t offset, long bh, long i, long j) {
  const uint64_t ctr[4] = {(uint64_t)(j >> 2), (uint64_t)(i >> 2), (uint64_t)bh, offset};
  const uint64_t key[2] = {seed & 0xFFFFFFFFull, seed >> 32};
  uint64_t out[4];
  oracle_philox(32, 10, ctr, key, out);
  return (int)((out[i & 3] >> (8 * (j & 3))) & 0xFF);
}

/* Z_ij: the element is kept iff its byte is at least the threshold. */
int oracle_dropout_keep(uint64_t seed, uint32_t offset, int t, long bh, long i, long j) {
  return oracle_dropout_byte(seed, offset, bh, i, j) >= t;
}

/* Keep indicators of one head, [rows][cols] from (i0, j0). */
void oracle_dropout_mask(uint64_t seed, uint32_t offset, int t, long bh, long i0, long j0,
                         long rows, long cols, uint8_t* z) {
#pragma omp parallel for schedule(static)
  for (long a = 0; a < rows; ++a)
    for (long b = 0; b < cols; ++b)
      z[a * cols + b] = (uint8_t)oracle_dropout_keep(seed, offset, t, bh, i0 + a, j0 + b);
}

/* Forward with dropout for q [B][H][N][d], k, v [B][Hkv][N][d]: O_i =
 * sum_j P_ij Z_ij / keep V_j, L_i the log-sum-exp of the undropped scores.
 * The query heads given are heads bh0, bh0 + 1, ... of the generator's
 * numbering (bh0 = 0 for a whole tensor; a slice of heads passes its first
 * head's index). */
void oracle_fwd_dropout(int B, int H, int Hkv, int N, int d, double scale, int causal,
                        long window, double p, uint64_t seed, uint32_t offset, long bh0,
                        const double* q, const double* k, const double* v, double* o,
                        double* lse, int nthreads) {
  if (nthreads > 0) omp_set_num_threads(nthreads);
  const int t = oracle_dropout_threshold(p);
  const double keep = (256.0 - t) / 256.0;
  const long hs = (long)N * d, total = (long)B * H * N;
#pragma omp parallel
  {
    double* srow = (double*)malloc(sizeof(double) * (size_t)N);
    double* prow = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 16)
    for (long r = 0; r < total; ++r) {
      const long bh = r / N, i = r % N, kv = kv_head_of(bh, H, Hkv);
      double* o_row = o + r * d;
      query_row(N, d, scale, causal, window, q + bh * hs + i * d, i, k + kv * hs,
                v + kv * hs, srow, prow, o_row, lse ? lse + r : NULL);
      for (int c = 0; c < d; ++c) o_row[c] = 0.0;
      for (long j = 0; j < N; ++j) {
        if (prow[j] == 0.0 || !oracle_dropout_keep(seed, offset, t, bh0 + bh, i, j)) continue;
        const double w = prow[j] / keep;
        const double* vj = v + kv * hs + j * (long)d;
        for (int c = 0; c < d; ++c) o_row[c] += w * vj[c];
      }
    }
    free(srow);
    free(prow);
  }
}

/* Backward with dropout, same shapes and head numbering; dk, dv [B][Hkv][N][d]
 * are summed over the query heads of each group.  Dvec [B][H][N] receives D_i. */
void oracle_bwd_dropout(int B, int H, int Hkv, int N, int d, double scale, int causal,
                        long window, double p, uint64_t seed, uint32_t offset, long bh0,
                        const double* q, const double* k, const double* v,
                        const double* dout, double* dq, double* dk, double* dv,
                        double* Dvec, int nthreads) {
  if (nthreads > 0) omp_set_num_threads(nthreads);
  const int t = oracle_dropout_threshold(p);
  const double keep = (256.0 - t) / 256.0;
  const long hs = (long)N * d;
  double* P = (double*)malloc(sizeof(double) * (size_t)N * (size_t)N);
  double* Pd = (double*)malloc(sizeof(double) * (size_t)N * (size_t)N);
  double* dS = (double*)malloc(sizeof(double) * (size_t)N * (size_t)N);
  for (long x = 0; x < (long)B * Hkv * hs; ++x) dk[x] = dv[x] = 0.0;
  for (long bh = 0; bh < (long)B * H; ++bh) {
    const long kv = kv_head_of(bh, H, Hkv);
    const double *qh = q + bh * hs, *kh = k + kv * hs, *vh = v + kv * hs;
    const double* doh = dout + bh * hs;
#pragma omp parallel
    {
      double* srow = (double*)malloc(sizeof(double) * (size_t)N);
      double* dprow = (double*)malloc(sizeof(double) * (size_t)N);
      double* o_row = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 8)
      for (long i = 0; i < N; ++i) {
        double* prow = P + i * (long)N;
        double* pdrow = Pd + i * (long)N;
        double* dsrow = dS + i * (long)N;
        query_row(N, d, scale, causal, window, qh + i * (long)d, i, kh, vh, srow, prow,
                  o_row, NULL);
        /* Z_ij / keep, dP_ij = (dO_i . V_j) Z_ij / keep, and P~_ij = P_ij Z_ij / keep */
        for (long j = 0; j < N; ++j) {
          const double z = (prow[j] != 0.0 && oracle_dropout_keep(seed, offset, t, bh0 + bh, i, j))
                               ? 1.0 / keep
                               : 0.0;
          dprow[j] = z * dot(doh + i * (long)d, vh + j * (long)d, d);
          pdrow[j] = prow[j] * z;
        }
        double Di = 0.0;
        for (long j = 0; j < N; ++j) Di += prow[j] * dprow[j];
        for (long j = 0; j < N; ++j) dsrow[j] = prow[j] * (dprow[j] - Di);
        if (Dvec) Dvec[bh * N + i] = Di;
        double* dqi = dq + bh * hs + i * (long)d;
        for (int c = 0; c < d; ++c) dqi[c] = 0.0;
        for (long j = 0; j < N; ++j) {
          if (dsrow[j] == 0.0) continue;
          const double* kj = kh + j * (long)d;
          for (int c = 0; c < d; ++c) dqi[c] += dsrow[j] * kj[c];
        }
        for (int c = 0; c < d; ++c) dqi[c] *= scale;
      }
      free(srow);
      free(dprow);
      free(o_row);
    }
#pragma omp parallel for schedule(dynamic, 8)
    for (long j = 0; j < N; ++j) {
      double* dvj = dv + kv * hs + j * (long)d;
      double* dkj = dk + kv * hs + j * (long)d;
      for (long i = 0; i < N; ++i) {
        const double pd = Pd[i * (long)N + j], ds = dS[i * (long)N + j];
        const double* doi = doh + i * (long)d;
        const double* qi = qh + i * (long)d;
        if (pd != 0.0)
          for (int c = 0; c < d; ++c) dvj[c] += pd * doi[c];
        if (ds != 0.0)
          for (int c = 0; c < d; ++c) dkj[c] += scale * ds * qi[c];
      }
    }
  }
  free(P);
  free(Pd);
  free(dS);
}
