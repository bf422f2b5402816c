/* Test infrastructure: drives every entry point of the oracle (oracle/mla_oracle.c)
 * once on tiny ragged inputs, for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitizers.py).  Inputs are
 * float64 (storage code 2) from a fixed-seed generator; the outputs are only
 * checked for being produced -- correctness is the pin tests' business.  A
 * sanitizer report aborts the process with a non-zero status. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

/* The oracle's C entry points (definitions in oracle/mla_oracle.c). */
double mla_oracle_scale(int d_nope, int d_rope);
void mla_oracle_absorb(int H, int d_nope, int d_rope, int kv_rank, int64_t n_tok, const void* q_nope,
                       const void* q_pe, int q_dt, const void* w_uk, int w_dt, double* q_abs);
void mla_oracle_decompress(int H, int d_v, int kv_rank, int64_t n_tok, const void* o_lat, int o_dt,
                           const void* w_uv, int w_dt, double* out);
int64_t mla_oracle_decode(int method, int H, int kv_rank, int d_rope, int batch, int t_q, const void* q_abs,
                          int q_dt, const void* kv, int kv_dt, int64_t num_blocks, int block_size,
                          const int32_t* block_table, int max_blocks, const int32_t* seq_lens, double scale,
                          const int32_t* sel, int64_t n_sel, double* o_lat, double* lse);
int64_t mla_oracle_decode_share(int world, int rank, int interleave, int H, int kv_rank, int d_rope, int batch,
                                int t_q, const void* q_abs, int q_dt, const void* kv, int kv_dt, int64_t num_blocks,
                                int block_size, const int32_t* block_table, int max_blocks, const int32_t* seq_lens,
                                double scale, const int32_t* sel, int64_t n_sel, double* o_lat, double* lse);
int64_t mla_oracle_attend_absorbed(int H, int d_nope, int d_rope, int d_v, int kv_rank, int batch, int t_q,
                                   const void* q_nope, const void* q_pe, int q_dt, const void* w_uk,
                                   const void* w_uv, int w_dt, const void* kv, int kv_dt, int64_t num_blocks,
                                   int block_size, const int32_t* block_table, int max_blocks,
                                   const int32_t* seq_lens, double scale, const int32_t* sel, int64_t n_sel,
                                   double* out, double* o_lat, double* lse);
int64_t mla_oracle_attend_naive(int H, int d_nope, int d_rope, int d_v, int kv_rank, int batch, int t_q,
                                const void* q_nope, const void* q_pe, int q_dt, const void* w_uk, const void* w_uv,
                                int w_dt, const void* kv, int kv_dt, int64_t num_blocks, int block_size,
                                const int32_t* block_table, int max_blocks, const int32_t* seq_lens, double scale,
                                const int32_t* sel, int64_t n_sel, double* out, double* lse);
void mla_oracle_rope_interleaved(double* x, int n_dims, double pos, double base);
void mla_oracle_rope_neox(double* x, int n_dims, double pos, double base);
void mla_oracle_norm_to_neox_perm(int n_dims, int32_t* perm);
void mla_oracle_rmsnorm(const void* x, int x_dt, int64_t n_rows, int width, const void* gamma, int g_dt, double eps,
                        double* y);
void mla_oracle_rope_rows(const void* x, int x_dt, int64_t n_rows, int n_heads, int n_dims, const int32_t* pos,
                          double base, int style, double* y);
int64_t mla_oracle_cache_append(int kv_rank, int d_rope, int64_t n_tok, const void* c_kv, const void* k_pe, int in_dt,
                                const void* gamma, int g_dt, double eps, const int32_t* pos, double base, int style,
                                const int64_t* slots, double* cache, int64_t num_slots);

enum { F64 = 2 };

static uint64_t rng_state = 0x2545F4914F6CDD1DULL;
static double urand(void) { /* xorshift64*, uniform in [-1, 1) */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (double)((rng_state * 0x2545F4914F6CDD1DULL) >> 11) / 4503599627370496.0 - 1.0;
}
static double* fill(size_t n) {
  double* p = (double*)malloc(sizeof(double) * (n ? n : 1));
  for (size_t i = 0; i < n; ++i) p[i] = urand();
  return p;
}
static double* zeros(size_t n) { return (double*)calloc(n ? n : 1, sizeof(double)); }

int main(void) {
  /* Tiny geometry: rope width 8, a value width other than the key width. */
  const int H = 3, DN = 16, DR = 8, DV = 12, KR = 32, D = KR + DR;
  const int B = 4, T = 3, BS = 16, MB = 4, NB = 13;
  /* Lengths: empty, short, ragged over three blocks, below t_q (invalid). */
  const int32_t lens[4] = {0, 5, 37, 2};
  int32_t table[4 * 4];
  for (int i = 0; i < B * MB; ++i) table[i] = (int32_t)((i * 5 + 3) % NB); /* scattered ids */
  const int64_t n_tok = (int64_t)B * T, n_items = n_tok * H;
  double *q_nope = fill(n_tok * H * DN), *q_pe = fill(n_tok * H * DR), *w_uk = fill((size_t)H * DN * KR),
         *w_uv = fill((size_t)H * DV * KR), *kv = fill((size_t)NB * BS * D);
  const double scale = mla_oracle_scale(DN, DR);
  double* q_abs = zeros(n_tok * H * D);
  mla_oracle_absorb(H, DN, DR, KR, n_tok, q_nope, q_pe, F64, w_uk, F64, q_abs);
  double *o_lat = zeros(n_items * KR), *lse = zeros(n_items), *out = zeros(n_items * DV);
  int64_t bad = 0;
  for (int method = 0; method < 2; ++method)
    bad += mla_oracle_decode(method, H, KR, DR, B, T, q_abs, F64, kv, F64, NB, BS, table, MB, lens, scale, NULL, 0,
                             o_lat, lse);
  mla_oracle_decompress(H, DV, KR, n_tok, o_lat, F64, w_uv, F64, out);
  for (int rank = 0; rank < 3; ++rank)
    bad += mla_oracle_decode_share(3, rank, 2, H, KR, DR, B, T, q_abs, F64, kv, F64, NB, BS, table, MB, lens, scale,
                                   NULL, 0, o_lat, lse);
  bad += mla_oracle_attend_absorbed(H, DN, DR, DV, KR, B, T, q_nope, q_pe, F64, w_uk, w_uv, F64, kv, F64, NB, BS, table,
                                    MB, lens, scale, NULL, 0, out, o_lat, lse);
  bad += mla_oracle_attend_naive(H, DN, DR, DV, KR, B, T, q_nope, q_pe, F64, w_uk, w_uv, F64, kv, F64, NB, BS, table,
                                 MB, lens, scale, NULL, 0, out, lse);
  /* Selected items: (request, query, head) triples, last item of the last request first. */
  const int32_t sel[3 * 3] = {3, 2, 2, 2, 0, 1, 0, 1, 0};
  bad += mla_oracle_attend_naive(H, DN, DR, DV, KR, B, T, q_nope, q_pe, F64, w_uk, w_uv, F64, kv, F64, NB, BS, table,
                                 MB, lens, scale, sel, 3, out, lse);
  bad += mla_oracle_decode(1, H, KR, DR, B, T, q_abs, F64, kv, F64, NB, BS, table, MB, lens, scale, sel, 3, o_lat, lse);

  /* Prolog pieces: norms, rope rows in both pairings, the rope permutation,
   * and the slot-mapped cache append with a padding slot and one past the end. */
  double *x = fill(7 * KR), *gamma = fill(KR), *y = zeros(7 * KR);
  mla_oracle_rmsnorm(x, F64, 7, KR, gamma, F64, 1e-6, y);
  mla_oracle_rmsnorm(x, F64, 7, KR, NULL, F64, 1e-6, y);
  int32_t pos[7] = {0, 1, 17, 4096, 1000000, 3, 9};
  double *xr = fill(7 * H * DR), *yr = zeros(7 * H * DR);
  mla_oracle_rope_rows(xr, F64, 7, H, DR, pos, 8e6, 0, yr);
  mla_oracle_rope_rows(xr, F64, 7, H, DR, pos, 8e6, 1, yr);
  double* one = fill(DR);
  mla_oracle_rope_neox(one, DR, 5.0, 1e4);
  mla_oracle_rope_interleaved(one, DR, 5.0, 1e4);
  int32_t perm[8];
  mla_oracle_norm_to_neox_perm(DR, perm);
  const int64_t slots[7] = {0, -1, 63, 5, 64, 31, 2};
  double *c_kv = fill(7 * KR), *k_pe = fill(7 * DR), *cache = zeros(64 * D);
  const int64_t skipped =
      mla_oracle_cache_append(KR, DR, 7, c_kv, k_pe, F64, gamma, F64, 1e-6, pos, 8e6, 0, slots, cache, 64);

  double acc = 0.0;
  for (int64_t i = 0; i < n_items * DV; ++i) acc += isfinite(out[i]) ? fabs(out[i]) : 0.0;
  printf("invalid items %lld, skipped slots %lld, checksum %.6f\n", (long long)bad, (long long)skipped, acc);
  free(q_nope); free(q_pe); free(w_uk); free(w_uv); free(kv); free(q_abs); free(o_lat); free(lse); free(out);
  free(x); free(gamma); free(y); free(xr); free(yr); free(one); free(c_kv); free(k_pe); free(cache);
  return skipped == 1 ? 0 : 3;
}
