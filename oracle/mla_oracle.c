/*
 * mla_oracle.c -- plain CPU reference ("the oracle") for multi-head latent
 * attention (MLA) decode over a paged latent cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or constant with
 * the HIP library; its only common ground with that library is the seeded
 * input generator that feeds both.
 *
 * Every function computes in IEEE double precision from inputs stored as
 * float32, bfloat16 bit patterns or float64 (bfloat16 -> double is exact).
 * The loops are written straight from the definitions on the pages; there is
 * no blocking, fusion or reordering beyond what those definitions state.
 * The only parallelism is an OpenMP loop over independent output items.
 *
 * Pages cited (by title and section):
 *   [mla.rs]   memra-engine 0.124.0 source page "mla.rs" (docs.rs): MlaDims,
 *              MlaDims::scale, MlaInputs, softmax, mla_attend_naive,
 *              mla_attend_absorbed, rope_interleaved, rope_neox,
 *              norm_to_neox_perm, and its unit tests.
 *   [mla mod]  memra-engine 0.70.0 module page "Module mla" (docs.rs).
 *   [vt cpu]   vllm.cpp source page "cpu_mla_attn.cpp": header comment and
 *              MlaDecodeAttentionKernel.
 *   [vllm cpu] vLLM API page "vllm.v1.attention.backends.mla.cpu_mla":
 *              CPUMLABackend, CPUMLAImpl.forward_mqa, do_kv_cache_update.
 *   [prolog]   Huawei CANN operator page "aclnnMlaProlog": the RmsNorm formula
 *              and the c^KV / k^R cache formulas.
 *   [vllm cpu] also CPUMLAImpl construction: the context-parallel settings
 *              dcp_world_size and cp_kv_cache_interleave_size.
 *
 * Pins (what each function is checked against, outside itself) are listed in
 * the test file that exercises it; every function below is pinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Storage codes for inputs. */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2 };

/* Widen one stored element to double.  bfloat16 is the upper half of an
 * IEEE float32, so the widening is exact. */
static double ld(const void* p, int dt, int64_t i) {
  if (dt == ORC_F32) return (double)((const float*)p)[i];
  if (dt == ORC_BF16) {
    uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  return ((const double*)p)[i];
}

int mla_oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void mla_oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* [mla.rs] MlaDims::scale: the softmax scale is one over the square root of
 * the ORIGINAL query-key head width d_nope + d_rope, never of the absorbed
 * width kv_rank + d_rope. */
double mla_oracle_scale(int d_nope, int d_rope) {
  return 1.0 / sqrt((double)(d_nope + d_rope));
}

/* [mla.rs] mla_attend_absorbed, absorb step; [vllm cpu] forward_mqa, query
 * concatenation.  For each token n and head h:
 *   q_abs[n][h][l]          = sum_p q_nope[n][h][p] * w_uk[h][p][l]   (l < kv_rank)
 *   q_abs[n][h][kv_rank+r]  = q_pe[n][h][r]                            (r < d_rope)
 * Layouts (row-major): q_nope [n_tok][H][d_nope], q_pe [n_tok][H][d_rope],
 * w_uk [H][d_nope][kv_rank], q_abs [n_tok][H][kv_rank+d_rope] (double). */
void mla_oracle_absorb(int H, int d_nope, int d_rope, int kv_rank, int64_t n_tok,
                       const void* q_nope, const void* q_pe, int q_dt,
                       const void* w_uk, int w_dt, double* q_abs) {
  const int D = kv_rank + d_rope;
#pragma omp parallel for schedule(static)
  for (int64_t nh = 0; nh < n_tok * H; ++nh) {
    const int h = (int)(nh % H);
    double* dst = q_abs + nh * D;
    for (int l = 0; l < kv_rank; ++l) {
      double acc = 0.0;
      for (int p = 0; p < d_nope; ++p)
        acc += ld(q_nope, q_dt, nh * d_nope + p) *
               ld(w_uk, w_dt, ((int64_t)h * d_nope + p) * kv_rank + l);
      dst[l] = acc;
    }
    for (int r = 0; r < d_rope; ++r) dst[kv_rank + r] = ld(q_pe, q_dt, nh * d_rope + r);
  }
}

/* [mla.rs] mla_attend_absorbed, decompress step: out[n][h][j] =
 * sum_l w_uv[h][j][l] * o_lat[n][h][l].  o_lat [n_tok][H][kv_rank] (storage
 * code o_dt), w_uv [H][d_v][kv_rank], out [n_tok][H][d_v] (double). */
void mla_oracle_decompress(int H, int d_v, int kv_rank, int64_t n_tok,
                           const void* o_lat, int o_dt, const void* w_uv, int w_dt,
                           double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t nh = 0; nh < n_tok * H; ++nh) {
    const int h = (int)(nh % H);
    for (int j = 0; j < d_v; ++j) {
      double acc = 0.0;
      for (int l = 0; l < kv_rank; ++l)
        acc += ld(w_uv, w_dt, ((int64_t)h * d_v + j) * kv_rank + l) *
               ld(o_lat, o_dt, nh * kv_rank + l);
      out[nh * d_v + j] = acc;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Paged cache access.                                                       */
/*                                                                            */
/* [vt cpu] MlaDecodeAttentionKernel: cache row j of request b lives in the   */
/* physical block block_table[b][j / block_size], at slot j % block_size.    */
/* [vllm cpu] do_kv_cache_update: each row is [c_kv (kv_rank) | k_pe (d_rope)]*/
/* so the row width is D = kv_rank + d_rope.                                  */
/* ------------------------------------------------------------------------ */
typedef struct {
  int H, kv_rank, d_rope, D;
  int batch, t_q;
  const void* kv;
  int kv_dt;
  int64_t num_blocks;
  int block_size;
  const int32_t* block_table;
  int max_blocks;
  const int32_t* seq_lens;
} paged;

/* Request-level validity.  The pages fix: seq_len >= 0 ([vt cpu] header);
 * the block-table row must cover seq_len ([vt cpu] kernel check); queries
 * are a suffix of the cache, so t_q <= seq_len unless the request is empty
 * ([mla.rs] check_shapes).  A block id must name an existing block. */
static int request_valid(const paged* c, int b) {
  const int64_t L = c->seq_lens[b];
  if (L < 0) return 0;
  if (L == 0) return 1;
  if (L > (int64_t)c->max_blocks * c->block_size) return 0;
  if (L < c->t_q) return 0;
  const int64_t nblk = (L + c->block_size - 1) / c->block_size;
  for (int64_t k = 0; k < nblk; ++k) {
    const int64_t id = c->block_table[(int64_t)b * c->max_blocks + k];
    if (id < 0 || id >= c->num_blocks) return 0;
  }
  return 1;
}

/* Flat element index of column 0 of cache row j of request b. */
static int64_t row_base(const paged* c, int b, int64_t j) {
  const int64_t id = c->block_table[(int64_t)b * c->max_blocks + j / c->block_size];
  return (id * c->block_size + j % c->block_size) * (int64_t)c->D;
}

/* [mla.rs] MlaInputs: queries occupy the LAST t_q positions of the cache and
 * query i sees rows 0 ..= t_kv - t_q + i, i.e. this many rows. */
static int64_t horizon(int64_t L, int t_q, int i) { return L - t_q + i + 1; }

/* Score of one query against one cache row: scale * <q, row> over all D
 * columns ([vt cpu] kernel: the dot spans the full row; [mla.rs]
 * mla_attend_absorbed: latent part plus rope part). */
static double score(const paged* c, const void* q, int q_dt, int64_t q_off,
                    int64_t rb, double scale) {
  double s = 0.0;
  for (int d = 0; d < c->D; ++d) s += ld(q, q_dt, q_off + d) * ld(c->kv, c->kv_dt, rb + d);
  return s * scale;
}

static void fill(double* p, int n, double v) {
  for (int k = 0; k < n; ++k) p[k] = v;
}

/* Selected output items: sel[3*k .. 3*k+2] = (b, i, h); NULL means every
 * (b, i, h) in row-major order. */
static void item(const int32_t* sel, int64_t k, const paged* c, int* b, int* i, int* h) {
  if (sel) {
    *b = sel[3 * k];
    *i = sel[3 * k + 1];
    *h = sel[3 * k + 2];
  } else {
    *h = (int)(k % c->H);
    *i = (int)((k / c->H) % c->t_q);
    *b = (int)(k / ((int64_t)c->H * c->t_q));
  }
}

/* Two-pass softmax attention of one absorbed query over the paged cache
 * ([mla.rs] softmax + mla_attend_absorbed scores and latent-space AV):
 *   s_j = scale * <q_abs, row_j>            j < horizon
 *   m = max_j s_j,  Z = sum_j exp(s_j - m)
 *   o_lat = sum_j exp(s_j - m) / Z * row_j[0:kv_rank]   (V = leading kv_rank
 *           columns of the same row, [vt cpu] header)
 *   lse = m + ln Z   (natural log of the scaled logits, [vt cpu] kernel)
 * An empty request gives o_lat = 0 and lse = -inf ([vt cpu] header).
 * Returns 0 on success, 1 for an invalid request (outputs NaN). */
static int attend_twopass(const paged* c, const void* q, int q_dt, int64_t q_off,
                          int b, int i, double scale, double* s_buf,
                          double* o_lat, double* lse) {
  if (!request_valid(c, b)) {
    fill(o_lat, c->kv_rank, NAN);
    *lse = NAN;
    return 1;
  }
  const int64_t L = c->seq_lens[b];
  if (L == 0) {
    fill(o_lat, c->kv_rank, 0.0);
    *lse = -INFINITY;
    return 0;
  }
  const int64_t n = horizon(L, c->t_q, i);
  double m = -INFINITY;
  for (int64_t j = 0; j < n; ++j) {
    s_buf[j] = score(c, q, q_dt, q_off, row_base(c, b, j), scale);
    if (s_buf[j] > m) m = s_buf[j];
  }
  double Z = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    s_buf[j] = exp(s_buf[j] - m);
    Z += s_buf[j];
  }
  fill(o_lat, c->kv_rank, 0.0);
  for (int64_t j = 0; j < n; ++j) {
    const double p = s_buf[j] / Z;
    const int64_t rb = row_base(c, b, j);
    for (int l = 0; l < c->kv_rank; ++l) o_lat[l] += p * ld(c->kv, c->kv_dt, rb + l);
  }
  *lse = m + log(Z);
  return 0;
}

/* Single-pass online softmax of one absorbed query over the paged cache,
 * following the running-max recurrence of [vt cpu] MlaDecodeAttentionKernel:
 * keep a running max m, running sum l and an accumulator over the leading
 * kv_rank columns; on each row rescale both by exp(m_old - m_new) (zero while
 * m_old is -inf); finish with acc / l (zeros when l == 0) and lse = m + ln l
 * (-inf when l == 0). */
static int attend_online(const paged* c, const void* q, int q_dt, int64_t q_off,
                         int b, int i, double scale, double* o_lat, double* lse) {
  if (!request_valid(c, b)) {
    fill(o_lat, c->kv_rank, NAN);
    *lse = NAN;
    return 1;
  }
  const int64_t L = c->seq_lens[b];
  const int64_t n = L == 0 ? 0 : horizon(L, c->t_q, i);
  double m = -INFINITY, l = 0.0;
  fill(o_lat, c->kv_rank, 0.0);
  for (int64_t j = 0; j < n; ++j) {
    const int64_t rb = row_base(c, b, j);
    const double s = score(c, q, q_dt, q_off, rb, scale);
    const double m_new = s > m ? s : m;
    const double rescale = isinf(m) ? 0.0 : exp(m - m_new);
    const double p = exp(s - m_new);
    for (int d = 0; d < c->kv_rank; ++d)
      o_lat[d] = o_lat[d] * rescale + p * ld(c->kv, c->kv_dt, rb + d);
    l = l * rescale + p;
    m = m_new;
  }
  const double inv = l > 0.0 ? 1.0 / l : 0.0;
  for (int d = 0; d < c->kv_rank; ++d) o_lat[d] *= inv;
  *lse = l > 0.0 ? m + log(l) : -INFINITY;
  return 0;
}

static paged make_paged(int H, int kv_rank, int d_rope, int batch, int t_q,
                        const void* kv, int kv_dt, int64_t num_blocks, int block_size,
                        const int32_t* block_table, int max_blocks, const int32_t* seq_lens) {
  paged c;
  c.H = H;
  c.kv_rank = kv_rank;
  c.d_rope = d_rope;
  c.D = kv_rank + d_rope;
  c.batch = batch;
  c.t_q = t_q;
  c.kv = kv;
  c.kv_dt = kv_dt;
  c.num_blocks = num_blocks;
  c.block_size = block_size;
  c.block_table = block_table;
  c.max_blocks = max_blocks;
  c.seq_lens = seq_lens;
  return c;
}

/* Longest valid request (score buffers are sized by it; an over-long
 * seq_len makes its request invalid, so it never needs a buffer). */
static int64_t max_len(const paged* c) {
  const int64_t cap = (int64_t)c->max_blocks * c->block_size;
  int64_t m = 1;
  for (int b = 0; b < c->batch; ++b)
    if (c->seq_lens[b] > m && c->seq_lens[b] <= cap) m = c->seq_lens[b];
  return m;
}

/* Decode attention of given absorbed queries q_abs [B][t_q][H][D] against the
 * paged cache.  method 0 = two-pass (the plain definition), 1 = single-pass
 * online recurrence.  Outputs for item k: o_lat[k][kv_rank], lse[k].
 * Returns the number of items whose request is invalid (outputs NaN). */
int64_t mla_oracle_decode(int method, int H, int kv_rank, int d_rope, int batch, int t_q,
                          const void* q_abs, int q_dt, const void* kv, int kv_dt,
                          int64_t num_blocks, int block_size, const int32_t* block_table,
                          int max_blocks, const int32_t* seq_lens, double scale,
                          const int32_t* sel, int64_t n_sel, double* o_lat, double* lse) {
  paged c = make_paged(H, kv_rank, d_rope, batch, t_q, kv, kv_dt, num_blocks, block_size,
                       block_table, max_blocks, seq_lens);
  const int64_t n_items = sel ? n_sel : (int64_t)batch * t_q * H;
  const int64_t Lmax = max_len(&c);
  int64_t bad = 0;
#pragma omp parallel reduction(+ : bad)
  {
    double* s_buf = (double*)malloc(sizeof(double) * (size_t)Lmax);
#pragma omp for schedule(dynamic, 1)
    for (int64_t k = 0; k < n_items; ++k) {
      int b, i, h;
      item(sel, k, &c, &b, &i, &h);
      const int64_t q_off = (((int64_t)b * t_q + i) * H + h) * c.D;
      if (method == 0)
        bad += attend_twopass(&c, q_abs, q_dt, q_off, b, i, scale, s_buf,
                              o_lat + k * kv_rank, lse + k);
      else
        bad += attend_online(&c, q_abs, q_dt, q_off, b, i, scale, o_lat + k * kv_rank, lse + k);
    }
    free(s_buf);
  }
  return bad;
}

/* One rank's share of decode context parallelism ([vllm cpu] CPUMLAImpl
 * construction: dcp_world_size and cp_kv_cache_interleave_size).  The cache
 * rows of a request are dealt to `world` ranks in runs of `interleave` rows:
 * row j lives on rank (j / interleave) % world.  Rank `rank`'s share of one
 * query is the two-pass attention of mla_oracle_decode restricted to the
 * visible rows it holds:
 *   o_r = sum over its rows of exp(s_j - m_r) row_j / Z_r,  lse_r = m_r + ln Z_r,
 * with zeros and -inf when it holds none of them.  Combining the shares of all
 * ranks with the split merge gives the full decode.  Reads the request's
 * whole (global) paged cache; validity is the request's, as in decode.
 * Returns the number of invalid items (outputs NaN). */
static int attend_share(const paged* c, const void* q, int q_dt, int64_t q_off, int b, int i,
                        double scale, int world, int rank, int interleave, double* s_buf,
                        double* o_lat, double* lse) {
  if (!request_valid(c, b)) {
    fill(o_lat, c->kv_rank, NAN);
    *lse = NAN;
    return 1;
  }
  fill(o_lat, c->kv_rank, 0.0);
  *lse = -INFINITY;
  const int64_t L = c->seq_lens[b];
  if (L == 0) return 0;
  const int64_t n = horizon(L, c->t_q, i);
  double m = -INFINITY;
  int64_t held = 0;
  for (int64_t j = 0; j < n; ++j) {
    if ((j / interleave) % world != rank) continue;
    s_buf[j] = score(c, q, q_dt, q_off, row_base(c, b, j), scale);
    if (s_buf[j] > m) m = s_buf[j];
    ++held;
  }
  if (held == 0) return 0;
  double Z = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    if ((j / interleave) % world != rank) continue;
    s_buf[j] = exp(s_buf[j] - m);
    Z += s_buf[j];
  }
  for (int64_t j = 0; j < n; ++j) {
    if ((j / interleave) % world != rank) continue;
    const double p = s_buf[j] / Z;
    const int64_t rb = row_base(c, b, j);
    for (int l = 0; l < c->kv_rank; ++l) o_lat[l] += p * ld(c->kv, c->kv_dt, rb + l);
  }
  *lse = m + log(Z);
  return 0;
}

int64_t mla_oracle_decode_share(int world, int rank, int interleave, int H, int kv_rank, int d_rope,
                                int batch, int t_q, const void* q_abs, int q_dt, const void* kv,
                                int kv_dt, int64_t num_blocks, int block_size,
                                const int32_t* block_table, int max_blocks, const int32_t* seq_lens,
                                double scale, const int32_t* sel, int64_t n_sel, double* o_lat,
                                double* lse) {
  paged c = make_paged(H, kv_rank, d_rope, batch, t_q, kv, kv_dt, num_blocks, block_size,
                       block_table, max_blocks, seq_lens);
  const int64_t n_items = sel ? n_sel : (int64_t)batch * t_q * H;
  const int64_t Lmax = max_len(&c);
  int64_t bad = 0;
#pragma omp parallel reduction(+ : bad)
  {
    double* s_buf = (double*)malloc(sizeof(double) * (size_t)(Lmax > 0 ? Lmax : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t k = 0; k < n_items; ++k) {
      int b, i, h;
      item(sel, k, &c, &b, &i, &h);
      const int64_t q_off = (((int64_t)b * t_q + i) * H + h) * c.D;
      bad += attend_share(&c, q_abs, q_dt, q_off, b, i, scale, world, rank, interleave, s_buf,
                          o_lat + k * kv_rank, lse + k);
    }
    free(s_buf);
  }
  return bad;
}

/* Full absorbed form for selected items ([mla.rs] mla_attend_absorbed;
 * [mla mod] the absorbed form is exact by associativity and linearity):
 * absorb the query through W_UK, attend in latent space (two-pass), then
 * decompress once through W_UV.  Inputs as in mla_oracle_absorb with the
 * token index n = b * t_q + i.  Outputs out[k][d_v], o_lat[k][kv_rank],
 * lse[k].  Returns the number of invalid items. */
int64_t mla_oracle_attend_absorbed(int H, int d_nope, int d_rope, int d_v, int kv_rank,
                                   int batch, int t_q, const void* q_nope, const void* q_pe,
                                   int q_dt, const void* w_uk, const void* w_uv, int w_dt,
                                   const void* kv, int kv_dt, int64_t num_blocks,
                                   int block_size, const int32_t* block_table, int max_blocks,
                                   const int32_t* seq_lens, double scale, const int32_t* sel,
                                   int64_t n_sel, double* out, double* o_lat, double* lse) {
  paged c = make_paged(H, kv_rank, d_rope, batch, t_q, kv, kv_dt, num_blocks, block_size,
                       block_table, max_blocks, seq_lens);
  const int64_t n_items = sel ? n_sel : (int64_t)batch * t_q * H;
  const int64_t Lmax = max_len(&c);
  const int D = kv_rank + d_rope;
  int64_t bad = 0;
#pragma omp parallel reduction(+ : bad)
  {
    double* s_buf = (double*)malloc(sizeof(double) * (size_t)Lmax);
    double* qa = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
    for (int64_t k = 0; k < n_items; ++k) {
      int b, i, h;
      item(sel, k, &c, &b, &i, &h);
      const int64_t nh = ((int64_t)b * t_q + i) * H + h;
      /* absorb: qa[l] = sum_p q_nope[p] * w_uk[h][p][l]; then append q_pe */
      for (int l = 0; l < kv_rank; ++l) {
        double acc = 0.0;
        for (int p = 0; p < d_nope; ++p)
          acc += ld(q_nope, q_dt, nh * d_nope + p) *
                 ld(w_uk, w_dt, ((int64_t)h * d_nope + p) * kv_rank + l);
        qa[l] = acc;
      }
      for (int r = 0; r < d_rope; ++r) qa[kv_rank + r] = ld(q_pe, q_dt, nh * d_rope + r);
      double* ol = o_lat + k * kv_rank;
      bad += attend_twopass(&c, qa, ORC_F64, 0, b, i, scale, s_buf, ol, lse + k);
      /* decompress: out[j] = sum_l w_uv[h][j][l] * o_lat[l] */
      for (int j = 0; j < d_v; ++j) {
        double acc = 0.0;
        for (int l = 0; l < kv_rank; ++l)
          acc += ld(w_uv, w_dt, ((int64_t)h * d_v + j) * kv_rank + l) * ol[l];
        out[k * d_v + j] = acc;
      }
    }
    free(qa);
    free(s_buf);
  }
  return bad;
}

/* Naive form for selected items ([mla.rs] mla_attend_naive): decompress the
 * cache per head, k_nope_j = W_UK[h] c_kv_j (d_nope wide) and
 * v_j = W_UV[h] c_kv_j (d_v wide), score at query-key width d_nope + d_rope,
 *   s_j = scale * (<q_nope, k_nope_j> + <q_pe, k_pe_j>),
 * two-pass softmax, out = sum_j p_j v_j.  Also reports lse = m + ln Z.
 * Outputs out[k][d_v], lse[k].  Returns the number of invalid items. */
int64_t mla_oracle_attend_naive(int H, int d_nope, int d_rope, int d_v, int kv_rank,
                                int batch, int t_q, const void* q_nope, const void* q_pe,
                                int q_dt, const void* w_uk, const void* w_uv, int w_dt,
                                const void* kv, int kv_dt, int64_t num_blocks, int block_size,
                                const int32_t* block_table, int max_blocks,
                                const int32_t* seq_lens, double scale, const int32_t* sel,
                                int64_t n_sel, double* out, double* lse) {
  paged c = make_paged(H, kv_rank, d_rope, batch, t_q, kv, kv_dt, num_blocks, block_size,
                       block_table, max_blocks, seq_lens);
  const int64_t n_items = sel ? n_sel : (int64_t)batch * t_q * H;
  const int64_t Lmax = max_len(&c);
  int64_t bad = 0;
#pragma omp parallel reduction(+ : bad)
  {
    double* s_buf = (double*)malloc(sizeof(double) * (size_t)Lmax);
    double* kn = (double*)malloc(sizeof(double) * (size_t)(d_nope > 0 ? d_nope : 1));
    double* v = (double*)malloc(sizeof(double) * (size_t)d_v);
#pragma omp for schedule(dynamic, 1)
    for (int64_t k = 0; k < n_items; ++k) {
      int b, i, h;
      item(sel, k, &c, &b, &i, &h);
      double* o = out + k * d_v;
      if (!request_valid(&c, b)) {
        fill(o, d_v, NAN);
        lse[k] = NAN;
        bad += 1;
        continue;
      }
      const int64_t L = seq_lens[b];
      if (L == 0) {
        fill(o, d_v, 0.0);
        lse[k] = -INFINITY;
        continue;
      }
      const int64_t nh = ((int64_t)b * t_q + i) * H + h;
      const int64_t n = horizon(L, t_q, i);
      double m = -INFINITY;
      for (int64_t j = 0; j < n; ++j) {
        const int64_t rb = row_base(&c, b, j);
        for (int p = 0; p < d_nope; ++p) { /* k_nope = W_UK[h] . c_kv_j */
          double acc = 0.0;
          for (int l = 0; l < kv_rank; ++l)
            acc += ld(w_uk, w_dt, ((int64_t)h * d_nope + p) * kv_rank + l) * ld(kv, kv_dt, rb + l);
          kn[p] = acc;
        }
        double s = 0.0;
        for (int p = 0; p < d_nope; ++p) s += ld(q_nope, q_dt, nh * d_nope + p) * kn[p];
        for (int r = 0; r < d_rope; ++r)
          s += ld(q_pe, q_dt, nh * d_rope + r) * ld(kv, kv_dt, rb + kv_rank + r);
        s_buf[j] = s * scale;
        if (s_buf[j] > m) m = s_buf[j];
      }
      double Z = 0.0;
      for (int64_t j = 0; j < n; ++j) {
        s_buf[j] = exp(s_buf[j] - m);
        Z += s_buf[j];
      }
      fill(o, d_v, 0.0);
      for (int64_t j = 0; j < n; ++j) {
        const int64_t rb = row_base(&c, b, j);
        for (int jv = 0; jv < d_v; ++jv) { /* v = W_UV[h] . c_kv_j */
          double acc = 0.0;
          for (int l = 0; l < kv_rank; ++l)
            acc += ld(w_uv, w_dt, ((int64_t)h * d_v + jv) * kv_rank + l) * ld(kv, kv_dt, rb + l);
          v[jv] = acc;
        }
        const double p = s_buf[j] / Z;
        for (int jv = 0; jv < d_v; ++jv) o[jv] += p * v[jv];
      }
      lse[k] = m + log(Z);
    }
    free(v);
    free(kn);
    free(s_buf);
  }
  return bad;
}

/* ------------------------------------------------------------------------ */
/* RoPE pairings and the load-time permutation ([mla.rs] rope_interleaved,   */
/* rope_neox, norm_to_neox_perm).  These feed the cache-append prolog, which */
/* sits upstream of the decode path; they are here so that the permutation  */
/* identity is a pinned fact.                                                 */
/* ------------------------------------------------------------------------ */

/* Interleaved ("NORM") pairing: pair (x[2j], x[2j+1]) is rotated by
 * theta_j = pos * base^(-2j/n_dims), for j < n_dims/2. */
void mla_oracle_rope_interleaved(double* x, int n_dims, double pos, double base) {
  for (int j = 0; j < n_dims / 2; ++j) {
    const double th = pos * pow(base, -2.0 * j / n_dims);
    const double a = x[2 * j], b = x[2 * j + 1];
    x[2 * j] = a * cos(th) - b * sin(th);
    x[2 * j + 1] = a * sin(th) + b * cos(th);
  }
}

/* NEOX pairing: pair (x[j], x[j + n_dims/2]) rotated by the same theta_j. */
void mla_oracle_rope_neox(double* x, int n_dims, double pos, double base) {
  const int half = n_dims / 2;
  for (int j = 0; j < half; ++j) {
    const double th = pos * pow(base, -2.0 * j / n_dims);
    const double a = x[j], b = x[j + half];
    x[j] = a * cos(th) - b * sin(th);
    x[j + half] = a * sin(th) + b * cos(th);
  }
}

/* Source (interleaved) index -> NEOX index: pi(2j) = j, pi(2j+1) = j + n/2. */
void mla_oracle_norm_to_neox_perm(int n_dims, int32_t* perm) {
  const int half = n_dims / 2;
  for (int j = 0; j < half; ++j) {
    perm[2 * j] = j;
    perm[2 * j + 1] = j + half;
  }
}

/* ------------------------------------------------------------------------ */
/* Cache-append prolog: RmsNorm of the latent rows, rope of the rope rows,   */
/* slot-mapped write into the paged cache.                                   */
/* ------------------------------------------------------------------------ */

/* [prolog] RmsNorm formula: y_i = gamma_i * x_i / RMS(x), with
 * RMS(x) = sqrt(mean_i x_i^2 + eps) (eps inside the root).  x [n_rows][width];
 * gamma [width] or NULL for all ones; y [n_rows][width] (double). */
void mla_oracle_rmsnorm(const void* x, int x_dt, int64_t n_rows, int width, const void* gamma, int g_dt,
                        double eps, double* y) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; ++r) {
    double ss = 0.0;
    for (int i = 0; i < width; ++i) {
      const double v = ld(x, x_dt, r * width + i);
      ss += v * v;
    }
    const double rms = sqrt(ss / width + eps);
    for (int i = 0; i < width; ++i) {
      const double gi = gamma ? ld(gamma, g_dt, i) : 1.0;
      y[r * width + i] = gi * ld(x, x_dt, r * width + i) / rms;
    }
  }
}

/* Rope of rows x [n_rows][n_heads][n_dims], every head of row r at position
 * pos[r] ([mla.rs] rope_neox for style 0, rope_interleaved for style 1), into
 * y (double, same layout). */
void mla_oracle_rope_rows(const void* x, int x_dt, int64_t n_rows, int n_heads, int n_dims, const int32_t* pos,
                          double base, int style, double* y) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; ++r) {
    for (int h = 0; h < n_heads; ++h) {
      double* row = y + (r * n_heads + h) * n_dims;
      for (int i = 0; i < n_dims; ++i) row[i] = ld(x, x_dt, (r * n_heads + h) * n_dims + i);
      if (style == 0) mla_oracle_rope_neox(row, n_dims, (double)pos[r], base);
      else mla_oracle_rope_interleaved(row, n_dims, (double)pos[r], base);
    }
  }
}

/* [vllm cpu] do_kv_cache_update, fed by the prolog's RmsNorm and rope
 * ([prolog] c^KV and k^R formulas): for each new token n with
 * slots[n] >= 0, cache row slots[n] (a flat row index block * block_size +
 * offset) becomes [RmsNorm(c_kv[n]) | rope(k_pe[n], pos[n])].  Tokens with a
 * negative slot are skipped; slots at or past num_slots are skipped and
 * counted (the return value).  cache is [num_slots][kv_rank + d_rope] double,
 * updated in place. */
int64_t mla_oracle_cache_append(int kv_rank, int d_rope, int64_t n_tok, const void* c_kv, const void* k_pe,
                                int in_dt, const void* gamma, int g_dt, double eps, const int32_t* pos,
                                double base, int style, const int64_t* slots, double* cache, int64_t num_slots) {
  const int D = kv_rank + d_rope;
  int64_t bad = 0;
  double* c = (double*)malloc(sizeof(double) * (size_t)(kv_rank > 0 ? kv_rank : 1));
  double* k = (double*)malloc(sizeof(double) * (size_t)(d_rope > 0 ? d_rope : 1));
  for (int64_t n = 0; n < n_tok; ++n) {
    const int64_t slot = slots[n];
    if (slot < 0) continue;
    if (slot >= num_slots) {
      ++bad;
      continue;
    }
    double ss = 0.0;
    for (int i = 0; i < kv_rank; ++i) {
      const double v = ld(c_kv, in_dt, n * kv_rank + i);
      ss += v * v;
    }
    const double rms = sqrt(ss / kv_rank + eps);
    for (int i = 0; i < kv_rank; ++i)
      c[i] = (gamma ? ld(gamma, g_dt, i) : 1.0) * ld(c_kv, in_dt, n * kv_rank + i) / rms;
    for (int i = 0; i < d_rope; ++i) k[i] = ld(k_pe, in_dt, n * d_rope + i);
    if (d_rope > 0) {
      if (style == 0) mla_oracle_rope_neox(k, d_rope, (double)pos[n], base);
      else mla_oracle_rope_interleaved(k, d_rope, (double)pos[n], base);
    }
    double* dst = cache + slot * D;
    for (int i = 0; i < kv_rank; ++i) dst[i] = c[i];
    for (int i = 0; i < d_rope; ++i) dst[kv_rank + i] = k[i];
  }
  free(c);
  free(k);
  return bad;
}
