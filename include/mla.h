/*
 * mla.h -- C ABI of the MI355X (gfx950) MLA latent-cache decode library.
 *
 * Multi-head latent attention decode in the absorbed ("MQA") form:
 *
 *   1. mla_absorb_q          q_abs[n][h] = [ W_UK[h]^T q_nope[n][h] | q_pe[n][h] ]
 *   2. mla_decode_attention  split-KV attention of every absorbed query over the
 *                            shared paged latent cache rows [c_kv | k_pe], values
 *                            = the leading kv_rank columns of the same rows, then
 *                            an LSE-weighted merge of the splits
 *   3. mla_decompress_v      out[n][h] = W_UV[h] o_lat[n][h]
 *
 * and, upstream of step 2, the cache-append prolog mla_cache_append (RmsNorm
 * of the new latent rows, rope of their k_pe and of the query rope part, and
 * the slot-mapped write into the paged cache), and the whole fused prolog
 * mla_prolog (hidden states to absorbed queries and cache rows).  For prefill
 * and chunked prefill, mla_prefill_attention runs the naive (multi-head) form
 * over the same paged cache.  For context-parallel decode,
 * mla_decode_attention_dcp runs one rank's share and mla_lse_combine merges
 * the ranks' shares.
 *
 * Pages this interface follows (cited by title and section):
 *   memra-engine 0.124.0 source page "mla.rs": MlaDims (geometry), MlaDims::scale,
 *     MlaInputs (layouts and the causal suffix rule), mla_attend_absorbed.
 *   vllm.cpp source page "cpu_mla_attn.cpp": MlaDecodeAttentionKernel (argument
 *     list, paged addressing, LSE definition, zeros for an empty request).
 *   vLLM API page "vllm.v1.attention.backends.mla.cpu_mla": CPUMLABackend (head
 *     size 576 = 512 + 64, block size 16), CPUMLAImpl.forward_mqa (decode call),
 *     do_kv_cache_update (slot-mapped cache write, padding slots skipped).
 *   CANN page "aclnnMlaProlog": two-phase call (workspace size, then execute);
 *     the RmsNorm formula and the c^KV / k^R / q^R formulas.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is DEVICE memory owned by the caller; the library
 *     never allocates, frees or keeps a tensor.  Layouts are contiguous,
 *     row-major, exactly as stated per argument.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue
 *     work and return; buffers must stay valid and unmodified until the stream
 *     reaches that point.
 *   - Outputs are fully overwritten (no pre-zeroing needed).  Outputs and the
 *     workspace must not alias each other or any input.
 *   - Every function returns an mla_status; nothing aborts or throws.  A
 *     host-detected error returns before anything is enqueued and leaves all
 *     outputs untouched.
 *   - mla_dtype gives the storage type of a tensor: IEEE float32 or bfloat16.
 */
#ifndef MLA_LATENT_CACHE_AMD_MLA_H
#define MLA_LATENT_CACHE_AMD_MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Head geometry (memra mla.rs, struct MlaDims): n_head query heads, query-key
 * width d_nope (no rope) + d_rope (rope), decompressed value width d_v, latent
 * rank kv_rank.  A latent cache row is kv_rank + d_rope wide.
 * GLM-5.2: {64, 192, 64, 256, 512}; NoPE geometry: {64, 256, 0, 256, 512}. */
typedef struct mla_dims {
  int32_t n_head;
  int32_t d_nope;
  int32_t d_rope;
  int32_t d_v;
  int32_t kv_rank;
} mla_dims;

/* The enums below are 32-bit integers at the boundary.  Callers may pass any
 * value; the library rejects codes it does not know (MLA_ERR_ARG).  Under C++
 * they carry int32_t as their underlying type, so every such value is a valid
 * enum value there too. */
#ifdef __cplusplus
#define MLA_ENUM(name) enum name : int32_t
#else
#define MLA_ENUM(name) enum name
#endif

typedef MLA_ENUM(mla_dtype) { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

typedef MLA_ENUM(mla_status) {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,        /* a required pointer is NULL                   */
  MLA_ERR_DIMS = 2,        /* a geometry field is out of range             */
  MLA_ERR_SHAPE = 3,       /* a size argument is out of range              */
  MLA_ERR_UNSUPPORTED = 4, /* valid request this library does not handle   */
  MLA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required   */
  MLA_ERR_HIP = 6,         /* the HIP runtime reported an error            */
  MLA_ERR_ARG = 7          /* other invalid argument (scale, dtype code)   */
} mla_status;

/* Bits of the device-detected data-error word (mla_decode_status).  A request
 * that trips one gets NaN in every output element and LSE of that request. */
#define MLA_DATA_NEG_LEN 0x1u        /* seq_lens[b] < 0                            */
#define MLA_DATA_LEN_OVER_TABLE 0x2u /* seq_lens[b] > max_blocks * block_size      */
#define MLA_DATA_LEN_BELOW_TQ 0x4u   /* 0 < seq_lens[b] < t_q                      */
#define MLA_DATA_BAD_BLOCK 0x8u      /* a needed block id is outside [0,num_blocks) */

/* Softmax scale of the geometry: 1 / sqrt(d_nope + d_rope), the original
 * query-key head width, not the absorbed width (memra mla.rs, MlaDims::scale).
 * Returns NaN for a NULL pointer or d_nope + d_rope < 1. */
float mla_default_scale(const mla_dims* dims);

/* Step 1: absorb the query through W_UK (memra mla.rs, mla_attend_absorbed,
 * absorb step; CANN aclnnMlaProlog, the q^N = q^C W^UK formula) and append
 * the rope part (vLLM cpu_mla, forward_mqa concatenation):
 *   q_abs[n][h][l]           = sum_p q_nope[n][h][p] * w_uk[h][p][l]   l < kv_rank
 *   q_abs[n][h][kv_rank + r] = q_pe[n][h][r]                            r < d_rope
 * q_nope [n_tok][n_head][d_nope], q_pe [n_tok][n_head][d_rope] (may be NULL
 * when d_rope == 0), w_uk [n_head][d_nope][kv_rank]: all of type in_dt.
 * q_abs  [n_tok][n_head][kv_rank + d_rope] of type out_dt.
 * Products accumulate in float32.  n_tok == 0 is a no-op.  Every tensor
 * pointer must be 16-byte aligned.
 * Errors: MLA_ERR_NULL, MLA_ERR_DIMS (n_head, d_nope, kv_rank < 1 or d_rope < 0),
 * MLA_ERR_SHAPE (n_tok < 0), MLA_ERR_ARG (bad dtype code, misaligned pointer),
 * MLA_ERR_HIP. */
mla_status mla_absorb_q(const mla_dims* dims, int64_t n_tok, const void* q_nope,
                        const void* q_pe, const void* w_uk, mla_dtype in_dt, void* q_abs,
                        mla_dtype out_dt, void* stream);

/* Phase one of decode (CANN two-phase convention): bytes of device workspace
 * that mla_decode_attention needs for these sizes.  num_splits sets how the
 * cache rows are cut into ranges that run in parallel (0 = choose
 * automatically for the current device):
 *   - bf16, kv_rank 512, d_rope 0 or 64, and t_q * n_head >= 128: the 32-row
 *     tiles of all requests, in request order, are cut into batch * num_splits
 *     ranges of equal tile count (a length-balanced schedule built on the
 *     device from seq_lens; a request may span several ranges or share one);
 *   - otherwise: every request's rows are cut into num_splits ranges of whole
 *     cache blocks (ranges sized from max_blocks).
 * Errors: MLA_ERR_NULL, MLA_ERR_DIMS, MLA_ERR_SHAPE, MLA_ERR_UNSUPPORTED
 * (block_size != 16), MLA_ERR_HIP (device query failed, auto mode only). */
mla_status mla_decode_workspace_size(const mla_dims* dims, int32_t batch, int32_t t_q,
                                     int32_t max_blocks, int32_t block_size,
                                     int32_t num_splits, size_t* bytes);

/* The total number of KV ranges mla_decode_attention will use for these sizes
 * with bf16 storage (resolves num_splits == 0; see mla_decode_workspace_size).
 * Returns 0 on invalid arguments. */
int32_t mla_decode_resolve_splits(const mla_dims* dims, int32_t batch, int32_t t_q,
                                  int32_t max_blocks, int32_t num_splits);

/* Step 2: paged decode attention over the latent cache (vllm.cpp
 * cpu_mla_attn.cpp, MlaDecodeAttentionKernel; memra mla.rs, MlaInputs causal
 * rule), computed as split-KV partial attention plus an LSE-weighted merge.
 *
 * Semantics, per request b, query i < t_q, head h:
 *   L = seq_lens[b] counts every cache row of the request INCLUDING its t_q
 *   query rows; query i sees rows 0 .. L - t_q + i (for t_q == 1: all L rows).
 *   Row j of request b is kv_cache[block_table[b][j / 16]][j % 16][0 .. D),
 *   D = kv_rank + d_rope, laid out [c_kv | k_pe].
 *   s_j   = scale * <q_abs[b][i][h], row_j>           (all D columns)
 *   o_lat = sum_j softmax(s)_j * row_j[0 .. kv_rank)  (values = leading kv_rank)
 *   lse   = natural log of sum_j exp(s_j)              (scaled logits)
 *   L == 0: o_lat = 0 and lse = -inf for every query and head.
 *
 * q_abs     [batch][t_q][n_head][D], type dt
 * kv_cache  [num_blocks][block_size][D], type dt (d_nope and d_v are unused)
 * block_table int32 [batch][max_blocks]; entries past a request's last block
 *           are never read
 * seq_lens  int32 [batch]
 * out_lat   [batch][t_q][n_head][kv_rank], type out_dt
 * lse       float32 [batch][t_q][n_head], or NULL
 * workspace device buffer of at least mla_decode_workspace_size() bytes for
 *           the same (dims, batch, t_q, max_blocks, block_size, num_splits);
 *           it also holds the data-error word read by mla_decode_status.
 * Results do not depend on the block labels; for a fixed num_splits they are
 * bitwise reproducible run to run.  Accumulation is float32 (bf16 products).
 * Alignment: q_abs, kv_cache and out_lat 16 bytes; block_table, seq_lens and
 * lse 4 bytes; workspace 256 bytes (allocations from hipMalloc satisfy all).
 * Errors: MLA_ERR_NULL, MLA_ERR_DIMS, MLA_ERR_SHAPE (batch < 0, t_q < 1,
 * max_blocks < 1, num_blocks < 1, num_splits < 0, or counts beyond the
 * device's 32-bit indices), MLA_ERR_UNSUPPORTED (block_size != 16),
 * MLA_ERR_ARG (scale not finite or <= 0, bad dtype code, misaligned pointer),
 * MLA_ERR_WORKSPACE, MLA_ERR_HIP.  Data errors found on the device (see the
 * MLA_DATA_* bits) do not fail the call: they poison that request's outputs
 * with NaN and are reported by mla_decode_status. */
mla_status mla_decode_attention(const mla_dims* dims, float scale, int32_t batch, int32_t t_q,
                                const void* q_abs, const void* kv_cache, mla_dtype dt,
                                int64_t num_blocks, int32_t block_size,
                                const int32_t* block_table, int32_t max_blocks,
                                const int32_t* seq_lens, void* out_lat, mla_dtype out_dt,
                                float* lse, void* workspace, size_t workspace_bytes,
                                int32_t num_splits, void* stream);

/* mla_decode_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops, harnesses that forbid allocation):
 * the same arguments without the workspace, the same results bit for bit.
 * The workspace is a library-owned scratch array of 160 MiB in device memory,
 * one copy per GPU, held until the process ends; the call allocates nothing
 * (no hipMalloc, no allocating library routine).  Every call on one GPU uses
 * that GPU's copy: calls that overlap on one GPU (concurrent streams, or
 * threads) race and give undefined results; calls in one stream order are
 * safe.  The device status words live in that scratch and are not readable
 * through mla_decode_status; data errors still poison the affected requests'
 * outputs with NaN.
 * Errors: as mla_decode_attention, plus MLA_ERR_WORKSPACE when the call would
 * need more than 160 MiB (mla_decode_workspace_size for the same arguments
 * gives the need), MLA_ERR_HIP when the scratch address cannot be obtained. */
mla_status mla_decode_attention_noalloc(const mla_dims* dims, float scale, int32_t batch, int32_t t_q,
                                        const void* q_abs, const void* kv_cache, mla_dtype dt,
                                        int64_t num_blocks, int32_t block_size,
                                        const int32_t* block_table, int32_t max_blocks,
                                        const int32_t* seq_lens, void* out_lat, mla_dtype out_dt,
                                        float* lse, int32_t num_splits, void* stream);

/* One rank's share of decode context parallelism (the vLLM CPU MLA backend
 * page, CPUMLAImpl construction, names the settings dcp_world_size and
 * cp_kv_cache_interleave_size; the pages print no distributed kernel, so the
 * layout is the plain reading of those two settings).
 *
 * The rows of every request are dealt to dcp_world ranks in runs of
 * dcp_interleave rows: global row j lives on rank (j / dcp_interleave) %
 * dcp_world.  This call runs on rank dcp_rank: kv_cache and block_table hold
 * ONLY that rank's rows, in increasing global order, as the rank's own paged
 * request (its local row k is kv_cache[block_table[b][k / 16]][k % 16]).
 * seq_lens are the GLOBAL lengths (all ranks' rows, queries included); query i
 * sees the rows this rank holds among global rows 0 .. L - t_q + i.  Outputs
 * are this rank's partial result over those rows: out_lat (normalised over
 * them) and lse, both as in mla_decode_attention; a rank that holds none of a
 * query's rows gives zeros and -inf.  Combining the shares of all ranks with
 * mla_lse_combine gives mla_decode_attention's result.  Float32 out_lat keeps
 * the combine exact to float32; bf16 is accepted.
 *
 * Arguments and errors as mla_decode_attention (max_blocks and the workspace
 * size refer to the rank's own table), plus MLA_ERR_ARG for dcp_world < 1,
 * dcp_rank outside [0, dcp_world) or dcp_interleave < 1, and MLA_ERR_NULL for
 * a NULL lse (required: a share without its LSE cannot be combined).  The data
 * errors are judged on the rank's view: a length beyond the rank's table is
 * MLA_DATA_LEN_OVER_TABLE.  dcp_world == 1 is mla_decode_attention. */
mla_status mla_decode_attention_dcp(const mla_dims* dims, float scale, int32_t batch, int32_t t_q,
                                    const void* q_abs, const void* kv_cache, mla_dtype dt,
                                    int64_t num_blocks, int32_t block_size,
                                    const int32_t* block_table, int32_t max_blocks,
                                    const int32_t* seq_lens, int32_t dcp_world, int32_t dcp_rank,
                                    int32_t dcp_interleave, void* out_lat, mla_dtype out_dt,
                                    float* lse, void* workspace, size_t workspace_bytes,
                                    int32_t num_splits, void* stream);

/* LSE combine of n_parts partial attention results over disjoint row sets
 * (the split merge of step 2, here across context-parallel ranks after the
 * all-gather of their shares):
 *   M = max_p lse[p][r],  w_p = exp(lse[p][r] - M),
 *   out[r] = sum_p w_p o[p][r] / sum_p w_p,  lse_out[r] = M + ln sum_p w_p.
 * Parts with lse = -inf carry no weight (their vectors are not read); all
 * parts -inf gives zeros and -inf; a NaN lse in any part gives NaN.
 * o_parts float32 [n_parts][n_rows][width], lse_parts float32
 * [n_parts][n_rows], out [n_rows][width] type out_dt, lse_out float32
 * [n_rows] or NULL.  Float32 arithmetic, parts added in index order
 * (deterministic).  Asynchronous on `stream`.
 * Errors: MLA_ERR_SHAPE (width < 1, n_rows < 0, n_parts < 1), MLA_ERR_ARG
 * (bad dtype code), MLA_ERR_NULL, MLA_ERR_HIP. */
mla_status mla_lse_combine(int32_t width, int64_t n_rows, int32_t n_parts, const float* o_parts,
                           const float* lse_parts, void* out, mla_dtype out_dt, float* lse_out,
                           void* stream);

/* Step 3: decompress the latent output once through W_UV (memra mla.rs,
 * mla_attend_absorbed, decompress step):
 *   out[n][h][j] = sum_l w_uv[h][j][l] * o_lat[n][h][l]
 * o_lat [n_tok][n_head][kv_rank] type o_dt, w_uv [n_head][d_v][kv_rank] type
 * w_dt, out [n_tok][n_head][d_v] type out_dt.  Float32 accumulation; with
 * bf16 weights, float32 o_lat values are rounded to bf16 (nearest even) before
 * the products.  Every tensor pointer must be 16-byte aligned.
 * Errors: MLA_ERR_NULL, MLA_ERR_DIMS (n_head, d_v, kv_rank < 1), MLA_ERR_SHAPE
 * (n_tok < 0), MLA_ERR_ARG (bad dtype code, misaligned pointer), MLA_ERR_HIP. */
mla_status mla_decompress_v(const mla_dims* dims, int64_t n_tok, const void* o_lat,
                            mla_dtype o_dt, const void* w_uv, mla_dtype w_dt, void* out,
                            mla_dtype out_dt, void* stream);

/* Rope pairing (memra mla.rs, rope_neox and rope_interleaved): NEOX rotates
 * the pair (x[j], x[j + d/2]), interleaved ("NORM") the pair (x[2j], x[2j+1]),
 * both by the angle pos * base^(-2j/d), d = d_rope, j < d/2.  A model whose
 * weights expect interleaved rope can run NEOX after permuting the rope rows
 * of its projection weights once at load time (mla.rs, norm_to_neox_perm):
 * query-key dot products are unchanged. */
typedef MLA_ENUM(mla_rope_style) { MLA_ROPE_NEOX = 0, MLA_ROPE_INTERLEAVED = 1 } mla_rope_style;

/* Data-error bit of mla_cache_append. */
#define MLA_DATA_BAD_SLOT 0x10u /* a slot_mapping entry >= num_blocks * block_size */

/* Cache-append prolog: write the new tokens' latent rows into the paged cache
 * and rotate their query rope part (vLLM cpu_mla, do_kv_cache_update; CANN
 * aclnnMlaProlog, the formulas c^KV = RmsNorm(x W^DKV), k^C = Cache(c^KV),
 * k^R = Cache(ROPE(x W^KR)) and q^R = ROPE(.), applied to the projections the
 * caller passes in).  For each token n < n_tok with s = slot_mapping[n]:
 *   s >= 0:  cache row s (= kv_cache[s / 16][s % 16], all D = kv_rank + d_rope
 *            columns) becomes
 *              [ gamma * c_kv[n] / sqrt(mean(c_kv[n]^2) + eps) | rope(k_pe[n], p) ]
 *            with p = positions[n] and the pairing rope_style;
 *   s < 0:   padding token, no cache write;
 *   s >= num_blocks * 16: no cache write, MLA_DATA_BAD_SLOT is ORed into
 *            *data_err (when data_err is not NULL).
 *   q_pe[n][h] = rope(q_pe[n][h], p) for every head h, whatever s is.
 * c_kv   [n_tok][kv_rank], before RmsNorm, type in_dt
 * k_pe   [n_tok][d_rope], before rope, type in_dt (NULL allowed when d_rope == 0)
 * gamma  [kv_rank] type in_dt, or NULL for all ones
 * positions int32 [n_tok] (NULL allowed when d_rope == 0)
 * q_pe   [n_tok][n_head][d_rope] type in_dt, rotated in place, or NULL to
 *        leave the queries alone
 * slot_mapping int64 [n_tok]: flat cache row block * 16 + offset, or -1
 * kv_cache [num_blocks][block_size][D] type kv_dt; rows not named by a
 *        valid slot are not touched
 * data_err device uint32, or NULL; never cleared by the library
 * Arithmetic: float32 for the norm and the rotation; each angle is formed in
 * double and reduced to [-pi, pi] before the float sine and cosine.  Two
 * tokens naming the same slot leave that row in an unspecified mix of both.
 * Errors: MLA_ERR_NULL, MLA_ERR_DIMS (kv_rank < 1, d_rope < 0 or odd, n_head
 * < 1 with q_pe), MLA_ERR_SHAPE (n_tok < 0, num_blocks < 1), MLA_ERR_UNSUPPORTED
 * (block_size != 16, d_rope > 256), MLA_ERR_ARG (eps negative or not finite,
 * rope_base not finite or <= 0 when d_rope > 0, bad rope_style or dtype
 * code), MLA_ERR_HIP. */
mla_status mla_cache_append(const mla_dims* dims, int64_t n_tok, const void* c_kv, const void* k_pe,
                            const void* gamma, mla_dtype in_dt, float eps, const int32_t* positions,
                            double rope_base, int32_t rope_style, void* q_pe,
                            const int64_t* slot_mapping, void* kv_cache, mla_dtype kv_dt,
                            int64_t num_blocks, int32_t block_size, uint32_t* data_err,
                            void* stream);

/* Widths of the fused prolog's projections: the hidden state and the query
 * latent (the CANN aclnnMlaProlog page's x and c^Q; its tables, which would
 * give their sizes, are unreadable). */
typedef struct mla_prolog_dims {
  int32_t hidden;  /* width of x */
  int32_t q_rank;  /* width of c^Q */
} mla_prolog_dims;

/* Workspace bytes mla_prolog needs for n_tok tokens.  Errors: MLA_ERR_NULL,
 * MLA_ERR_DIMS, MLA_ERR_SHAPE (n_tok < 0), MLA_ERR_UNSUPPORTED (see
 * mla_prolog). */
mla_status mla_prolog_workspace_size(const mla_dims* dims, const mla_prolog_dims* pd, int64_t n_tok,
                                     size_t* bytes);

/* The fused MLA prolog (CANN aclnnMlaProlog: its four paths and formulas),
 * from the hidden states of n_tok new tokens to their absorbed queries and
 * their cache rows:
 *   c^Q  = RmsNorm(x W^DQ)            RmsNorm(y) = gamma * y / sqrt(mean(y^2) + eps)
 *   q^N  = (c^Q W^UQ) W^UK            per head (W^UK: the absorb step's)
 *   q^R  = ROPE(c^Q W^QR)             at positions[n]
 *   q_abs[n][h] = [q^N | q^R]          (what mla_decode_attention reads)
 *   cache row slot_mapping[n] <- [RmsNorm(x W^DKV) | ROPE(x W^KR)]
 * The cache write is mla_cache_append's (slots, padding -1, out-of-range
 * slots reported in *data_err); the last step is mla_absorb_q's.
 *
 * x [n_tok][hidden]; weights stored [out][in]: w_dq [q_rank][hidden],
 * w_dkv [kv_rank][hidden], w_kr [d_rope][hidden], w_uq [n_head d_nope][q_rank]
 * and w_qr [n_head d_rope][q_rank] (output feature h * width + j), w_uk
 * [n_head][d_nope][kv_rank]; gamma_q [q_rank], gamma_kv [kv_rank] or NULL
 * (ones); all of type dt, which must be MLA_BF16.  x and the projection
 * weights must be 16-byte aligned.  positions int32 [n_tok], slot_mapping
 * int64 [n_tok], kv_cache [num_blocks][16][kv_rank + d_rope] type kv_dt,
 * q_abs [n_tok][n_head][kv_rank + d_rope] type q_dt, data_err as in
 * mla_cache_append (NULL to ignore).  Intermediates (c^Q, the cache
 * inputs, q^C, q^R) are bf16 in the workspace; products and norms
 * accumulate in float32.  c^Q is stored as gamma_q (x W^DQ), before its
 * per-token 1 / RMS, which scales the float32 sums of the second product
 * instead (the products are linear in c^Q; equal up to rounding).  Asynchronous on `stream`; the workspace must not
 * be shared with a concurrent call.
 * Errors: those of mla_prolog_workspace_size, MLA_ERR_UNSUPPORTED (dt not
 * bf16, hidden or q_rank not a multiple of 32, q_rank > 4096, kv_rank,
 * d_rope, n_head d_nope or n_head d_rope not a multiple of 16, d_nope not a
 * multiple of 8, block_size != 16, d_rope > 256), MLA_ERR_ARG (eps, rope
 * base or style, dtype codes, misaligned x or weights), MLA_ERR_SHAPE
 * (num_blocks < 1, n_tok > 65535), MLA_ERR_WORKSPACE, MLA_ERR_HIP. */
mla_status mla_prolog(const mla_dims* dims, const mla_prolog_dims* pd, int64_t n_tok, const void* x,
                      const void* w_dq, const void* w_uq, const void* w_qr, const void* w_uk,
                      const void* w_dkv, const void* w_kr, const void* gamma_q, const void* gamma_kv,
                      mla_dtype dt, float eps_q, float eps_kv, const int32_t* positions,
                      double rope_base, int32_t rope_style, const int64_t* slot_mapping,
                      void* kv_cache, mla_dtype kv_dt, int64_t num_blocks, int32_t block_size,
                      void* q_abs, mla_dtype q_dt, uint32_t* data_err, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Naive-form (multi-head) attention for prefill and chunked prefill over the
 * paged latent cache (memra mla.rs, mla_attend_naive, and the MlaInputs causal
 * rule).  For request b, new query i < t_q and head h, with L = seq_lens[b]
 * counting every cache row of the request including its t_q new ones:
 *   k_nope_j = W_UK[h] c_kv_j (d_nope wide),  v_j = W_UV[h] c_kv_j (d_v wide),
 *   s_j = scale * (<q_nope[b][i][h], k_nope_j> + <q_pe[b][i][h], k_pe_j>),
 *   out[b][i][h] = sum_j softmax(s)_j v_j  over rows j = 0 .. L - t_q + i,
 *   lse[b][i][h] = natural log of sum_j exp(s_j);  L == 0: zeros and -inf.
 * Rows are read through the block table as in mla_decode_attention.  The
 * cache rows are first decompressed per head into the workspace (one GEMM
 * per request), then attended at query-key width d_nope + d_rope.
 * q_nope [batch][t_q][n_head][d_nope], q_pe [batch][t_q][n_head][d_rope] (NULL
 * allowed when d_rope == 0), w_uk [n_head][d_nope][kv_rank], w_uv
 * [n_head][d_v][kv_rank], kv_cache [num_blocks][block_size][kv_rank + d_rope]:
 * all bfloat16.  out [batch][t_q][n_head][d_v] of type out_dt; lse float32
 * [batch][t_q][n_head] or NULL.  workspace: at least
 * mla_prefill_workspace_size() bytes for the same (dims, batch, max_blocks);
 * it also holds the data-error word read by mla_decode_status.
 * Supported geometry: kv_rank 512, d_v 256, d_nope + d_rope = 256 with d_rope
 * 64 or 0, n_head * d_nope a multiple of 128 (GLM-5.2 and its NoPE variant).
 * Errors: MLA_ERR_NULL, MLA_ERR_DIMS, MLA_ERR_SHAPE (batch < 0, t_q < 1,
 * max_blocks < 1, num_blocks < 1), MLA_ERR_UNSUPPORTED (block_size != 16,
 * float32 inputs, another geometry), MLA_ERR_ARG (scale not finite or <= 0,
 * bad dtype code), MLA_ERR_WORKSPACE, MLA_ERR_HIP.  Data errors found on the
 * device (the MLA_DATA_* bits) do not fail the call: they poison that
 * request's outputs with NaN and are reported by mla_decode_status. */
mla_status mla_prefill_workspace_size(const mla_dims* dims, int32_t batch, int32_t max_blocks,
                                      int32_t block_size, size_t* bytes);
mla_status mla_prefill_attention(const mla_dims* dims, float scale, int32_t batch, int32_t t_q,
                                 const void* q_nope, const void* q_pe, const void* w_uk,
                                 const void* w_uv, const void* kv_cache, mla_dtype dt,
                                 int64_t num_blocks, int32_t block_size, const int32_t* block_table,
                                 int32_t max_blocks, const int32_t* seq_lens, void* out,
                                 mla_dtype out_dt, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Waits for `stream`, then ORs the MLA_DATA_* bits that the most recent
 * mla_decode_attention or mla_prefill_attention call on this workspace recorded into *flags (0 = no
 * data error).  Errors: MLA_ERR_NULL, MLA_ERR_WORKSPACE (the workspace holds
 * no completed decode), MLA_ERR_HIP. */
mla_status mla_decode_status(const void* workspace, uint32_t* flags, void* stream);

/* Static description of a status code (never NULL). */
const char* mla_status_string(mla_status status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_LATENT_CACHE_AMD_MLA_H */
