/* Exercises every entry point of the oracle (oracle/attn_oracle.c) on small
 * shapes and edge cases, for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer: any out-of-bounds access, leak, overflow or
 * other undefined behaviour aborts the program with a report.  Also checks
 * that every output is finite and that the two forward forms agree. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_bf16_decode(const uint16_t* src, double* dst, long n);
void oracle_e4m3_decode(const uint8_t* src, double descale, double* dst, long n);
void oracle_e4m3_decode_blocks(const uint8_t* src, long heads, long rows, int d, int block_rows,
                               const double* descales, double* dst);
void oracle_fwd(int BH, int N, int d, double scale, int causal, long window, const double* q,
                const double* k, const double* v, double* o, double* lse, int nthreads);
void oracle_fwd_rows(int N, int d, double scale, int causal, long window, const double* q,
                     const double* k, const double* v, const long* rows, int nrows,
                     double* o_rows, double* lse_rows, int nthreads);
void oracle_fwd_gqa(int B, int H, int Hkv, int N, int d, double scale, int causal, long window,
                    const double* q, const double* k, const double* v, double* o, double* lse,
                    int nthreads);
void oracle_fwd_decode(int B, int H, int Hkv, int Nq, int Nk, int d, double scale, int causal,
                       long window, const double* q, const double* k, const double* v, double* o,
                       double* lse, int nthreads);
void oracle_bwd(int BH, int N, int d, double scale, int causal, long window, const double* q,
                const double* k, const double* v, const double* dout, double* dq, double* dk,
                double* dv, double* Dvec, int nthreads);
void oracle_bwd_gqa(int B, int H, int Hkv, int N, int d, double scale, int causal, long window,
                    const double* q, const double* k, const double* v, const double* dout,
                    double* dq, double* dk, double* dv, double* Dvec, int nthreads);
void oracle_online_fwd(int N, int d, double scale, int causal, long window, const double* q,
                       const double* k, const double* v, const long* bounds, int nparts,
                       int form, double* o, double* lse);
void oracle_philox(int W, int R, const uint64_t ctr_in[4], const uint64_t key_in[2],
                   uint64_t out[4]);
void oracle_dropout_mask(uint64_t seed, uint32_t offset, int t, long bh, long i0, long j0,
                         long rows, long cols, uint8_t* z);
void oracle_fwd_dropout(int B, int H, int Hkv, int N, int d, double scale, int causal,
                        long window, double p, uint64_t seed, uint32_t offset, long bh0,
                        const double* q, const double* k, const double* v, double* o,
                        double* lse, int nthreads);
void oracle_bwd_dropout(int B, int H, int Hkv, int N, int d, double scale, int causal,
                        long window, double p, uint64_t seed, uint32_t offset, long bh0,
                        const double* q, const double* k, const double* v, const double* dout,
                        double* dq, double* dk, double* dv, double* Dvec, int nthreads);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double uniform(void) { /* xorshift64*, in (-1, 1) */
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return (double)((rng * 0x2545F4914F6CDD1Dull) >> 11) / 4503599627370496.0 - 1.0;
}
static double* arr(long n) {
  double* a = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (long i = 0; i < n; ++i) a[i] = uniform();
  return a;
}
static int failures = 0;
static void finite(const char* what, const double* a, long n) {
  for (long i = 0; i < n; ++i)
    if (!isfinite(a[i])) {
      printf("%s: element %ld not finite\n", what, i);
      ++failures;
      return;
    }
}

int main(void) {
  const int Ns[] = {1, 2, 7, 33};
  const int ds[] = {4, 8};
  const long wins[] = {0, 1, 3, 1000};
  for (int a = 0; a < 4; ++a)
    for (int b = 0; b < 2; ++b)
      for (int c = 0; c < 2; ++c)
        for (int w = 0; w < 4; ++w) {
          const int N = Ns[a], d = ds[b], causal = c, BH = 2, B = 1, H = 2, Hkv = 1;
          const long win = wins[w];
          const long n = (long)BH * N * d;
          double *q = arr(n), *k = arr(n), *v = arr(n), *dout = arr(n);
          double *o = arr(n), *lse = arr(BH * N), *o2 = arr(n), *lse2 = arr(BH * N);
          double *dq = arr(n), *dk = arr(n), *dv = arr(n), *D = arr(BH * N);
          oracle_fwd(BH, N, d, 0.5, causal, win, q, k, v, o, lse, 2);
          finite("fwd O", o, n);
          finite("fwd L", lse, BH * N);
          long bounds[3] = {0, N / 2, N};
          for (int form = 0; form < 2; ++form) {
            oracle_online_fwd(N, d, 0.5, causal, win, q, k, v, bounds, 2, form, o2, lse2);
            for (long i = 0; i < (long)N * d; ++i)
              if (fabs(o2[i] - o[i]) > 1e-12) {
                printf("online form %d differs at N=%d\n", form, N);
                ++failures;
                break;
              }
          }
          long rows[2] = {0, N - 1};
          oracle_fwd_rows(N, d, 0.5, causal, win, q, k, v, rows, 2, o2, lse2, 2);
          finite("fwd rows", o2, 2 * d);
          oracle_bwd(BH, N, d, 0.5, causal, win, q, k, v, dout, dq, dk, dv, D, 2);
          finite("bwd dQ", dq, n);
          finite("bwd dK", dk, n);
          finite("bwd dV", dv, n);
          oracle_fwd_gqa(B, H, Hkv, N, d, 0.5, causal, win, q, k, v, o2, lse2, 2);
          finite("gqa O", o2, n);
          oracle_bwd_gqa(B, H, Hkv, N, d, 0.5, causal, win, q, k, v, dout, dq, dk, dv, D, 2);
          finite("gqa dQ", dq, n);
          oracle_fwd_dropout(B, H, Hkv, N, d, 0.5, causal, win, 0.25, 7, 3, 0, q, k, v, o2, lse2, 2);
          finite("dropout O", o2, n);
          oracle_bwd_dropout(B, H, Hkv, N, d, 0.5, causal, win, 0.25, 7, 3, 0, q, k, v, dout, dq, dk,
                             dv, D, 2);
          finite("dropout dK", dk, (long)B * Hkv * N * d);
          const int Nq = N > 1 ? N / 2 : 1;
          oracle_fwd_decode(B, H, Hkv, Nq, N, d, 0.5, causal, win, q, k, v, o2, lse2, 2);
          finite("decode O", o2, (long)B * H * Nq * d);
          free(q); free(k); free(v); free(dout); free(o); free(lse); free(o2); free(lse2);
          free(dq); free(dk); free(dv); free(D);
        }
  /* decoders over every code, generator, keep masks */
  uint16_t b16[65536];
  uint8_t c8[256];
  double* x = arr(65536);
  for (int i = 0; i < 65536; ++i) b16[i] = (uint16_t)i;
  for (int i = 0; i < 256; ++i) c8[i] = (uint8_t)i;
  oracle_bf16_decode(b16, x, 65536);
  oracle_e4m3_decode(c8, 0.5, x, 256);
  double descales[8] = {1.0, 0.5, 2.0, 0.25, 1.5, 3.0, 0.125, 1.0}; /* 2 heads x 4 blocks */
  oracle_e4m3_decode_blocks(c8, 2, 16, 8, 5, descales, x);
  uint64_t ctr[4] = {~0ull, 1, 2, 3}, key[2] = {~0ull, 5}, out[4];
  oracle_philox(32, 10, ctr, key, out);
  oracle_philox(64, 10, ctr, key, out);
  uint8_t z[9 * 13];
  oracle_dropout_mask(~0ull, ~0u, 255, 3, 5, 7, 9, 13, z);
  free(x);
  printf("oracle under sanitizers: %s\n", failures ? "FAILED" : "ok");
  return failures ? 1 : 0;
}
