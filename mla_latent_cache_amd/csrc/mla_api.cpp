// C ABI of the MLA latent-cache decode library: argument validation, the
// split plan, kernel selection and launches.  Declarations and the contract
// of every entry point are in include/mla.h.
#include "mla.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "kernels.hpp"

#include <mutex>

namespace {

// Device scratch of mla_decode_attention_noalloc: one copy per GPU, held until
// the process ends.  Host code never uses the array's name as an address; the
// address of the current device's copy comes from hipGetSymbolAddress, once
// per device, and every later use goes through that pointer.
constexpr size_t kNoAllocScratchBytes = (size_t)160 << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mutex;

// The current device's scratch address, or null on failure.
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

bool dt_ok(mla_dtype d) { return d == MLA_F32 || d == MLA_BF16; }

// The kernels read and write tensors in 16-byte vectors (and stage cache
// blocks with 16-byte buffer loads), index arrays and LSE as 4-byte words, and
// lay the workspace out in 256-byte sections.
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Compute units of the current device (cached per device id).
int device_cus(int* out) {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (dev >= 0 && dev < 64 && cache[dev] > 0) {
    *out = cache[dev];
    return 0;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) return -1;
  if (dev >= 0 && dev < 64) cache[dev] = n;
  *out = n;
  return 0;
}

mla_status check_decode_dims(const mla_dims* d) {
  if (!d) return MLA_ERR_NULL;
  if (d->n_head < 1 || d->kv_rank < 1 || d->d_rope < 0) return MLA_ERR_DIMS;
  return MLA_OK;
}

// Automatic split count: enough (request, range, query tile) workgroups to give
// every compute unit one (the MFMA kernel's LDS use allows one workgroup per
// compute unit, and every extra split adds a partial to write and merge), or
// two per compute unit for the small generic workgroups; ranges of at most
// kMaxRangeBlocks cache blocks, so that with ragged lengths no single
// workgroup owns a whole long request; no range shorter than 8 cache blocks.
constexpr int kMaxRangeBlocks = 256;

int auto_splits(int n_head, int batch, int t_q, int max_blocks, int cus, bool mfma) {
  const int n_q = t_q * n_head;
  const int m_tiles = mfma ? (n_q + mla::kQRowsPerWG - 1) / mla::kQRowsPerWG : n_q;
  const long base = (long)(batch > 0 ? batch : 1) * m_tiles;
  const long target = mfma ? (long)cus : 2L * cus;
  long want = (target + base - 1) / base;
  const long by_length = (max_blocks + kMaxRangeBlocks - 1) / kMaxRangeBlocks;
  if (want < by_length) want = by_length;
  const long cap = (max_blocks + 7) / 8;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  if (want > mla::kMaxSplits) want = mla::kMaxSplits;
  return (int)want;
}

bool mfma_path(const mla_dims* d, bool bf16) {
  return bf16 && d->kv_rank == 512 && (d->d_rope == 0 || d->d_rope == 64);
}

// The length-balanced kernel (128 query rows per workgroup) from 128 query
// rows per request on; below that the per-request split kernel, whose
// workgroups hold 64 query rows.
bool flat_path(const mla_dims* d, int t_q, bool bf16) {
  return mla::flat_supported(d->kv_rank, d->d_rope, bf16) && (int64_t)t_q * d->n_head >= 128;
}

mla_status resolve(const mla_dims* d, int batch, int t_q, int max_blocks, int num_splits, bool bf16,
                   int* splits) {
  if (num_splits > 0) {
    *splits = num_splits;
    return MLA_OK;
  }
  int cus = 0;
  if (device_cus(&cus) != 0) return MLA_ERR_HIP;
  *splits = auto_splits(d->n_head, batch, t_q, max_blocks, cus, mfma_path(d, bf16));
  return MLA_OK;
}

}  // namespace

extern "C" {

float mla_default_scale(const mla_dims* dims) {
  if (!dims || dims->d_nope + dims->d_rope < 1) return NAN;
  return 1.0f / sqrtf((float)(dims->d_nope + dims->d_rope));
}

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "a required pointer is NULL";
    case MLA_ERR_DIMS: return "geometry field out of range";
    case MLA_ERR_SHAPE: return "size argument out of range";
    case MLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_HIP: return "HIP runtime error";
    case MLA_ERR_ARG: return "invalid argument";
  }
  return "unknown status";
}

mla_status mla_absorb_q(const mla_dims* dims, int64_t n_tok, const void* q_nope, const void* q_pe,
                        const void* w_uk, mla_dtype in_dt, void* q_abs, mla_dtype out_dt, void* stream) {
  if (!dims) return MLA_ERR_NULL;
  if (dims->n_head < 1 || dims->d_nope < 1 || dims->kv_rank < 1 || dims->d_rope < 0) return MLA_ERR_DIMS;
  if (n_tok < 0) return MLA_ERR_SHAPE;
  if (!dt_ok(in_dt) || !dt_ok(out_dt)) return MLA_ERR_ARG;
  if (n_tok == 0) return MLA_OK;
  if (!q_nope || !w_uk || !q_abs || (dims->d_rope > 0 && !q_pe)) return MLA_ERR_NULL;
  if (!aligned(q_nope, 16) || !aligned(w_uk, 16) || !aligned(q_abs, 16) || (q_pe && !aligned(q_pe, 16)))
    return MLA_ERR_ARG;
  const hipError_t e = mla::launch_absorb(dims->n_head, dims->d_nope, dims->d_rope, dims->kv_rank, n_tok, q_nope,
                                          q_pe, w_uk, in_dt == MLA_BF16, q_abs, out_dt == MLA_BF16,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

// Tile ranges of the length-balanced path: num_splits ranges per request on
// average (batch * num_splits in all), or one workgroup per compute unit.
static mla_status flat_ranges(const mla_dims* d, int batch, int t_q, int max_blocks, int num_splits, int64_t* G) {
  if (num_splits > 0) {
    *G = (int64_t)(batch > 0 ? batch : 1) * num_splits;
    return MLA_OK;
  }
  int cus = 0;
  if (device_cus(&cus) != 0) return MLA_ERR_HIP;
  *G = mla::flat_auto_ranges(d->n_head, batch, t_q, max_blocks, cus);
  return MLA_OK;
}

int32_t mla_decode_resolve_splits(const mla_dims* dims, int32_t batch, int32_t t_q, int32_t max_blocks,
                                  int32_t num_splits) {
  if (check_decode_dims(dims) != MLA_OK || batch < 0 || t_q < 1 || max_blocks < 1 || num_splits < 0) return 0;
  if (flat_path(dims, t_q, true)) {
    int64_t G = 0;
    if (flat_ranges(dims, batch, t_q, max_blocks, num_splits, &G) != MLA_OK) return 0;
    const mla::FlatPlan f = mla::flat_plan(dims->n_head, dims->d_rope, batch, t_q, max_blocks, G);
    return f.ok ? f.G : 0;
  }
  int splits = 0;
  if (resolve(dims, batch, t_q, max_blocks, num_splits, true, &splits) != MLA_OK) return 0;
  const mla::Plan p = mla::decode_plan(dims->n_head, dims->kv_rank, dims->d_rope, batch, t_q, max_blocks, splits,
                                       true);
  return p.ok && (int64_t)batch * p.splits <= INT32_MAX ? batch * p.splits : 0;
}

mla_status mla_decode_workspace_size(const mla_dims* dims, int32_t batch, int32_t t_q, int32_t max_blocks,
                                     int32_t block_size, int32_t num_splits, size_t* bytes) {
  const mla_status st = check_decode_dims(dims);
  if (st != MLA_OK) return st;
  if (!bytes) return MLA_ERR_NULL;
  if (batch < 0 || t_q < 1 || max_blocks < 1 || num_splits < 0) return MLA_ERR_SHAPE;
  if (block_size != 16) return MLA_ERR_UNSUPPORTED;
  // The float32 and bfloat16 calls of one geometry may take different paths;
  // size for the larger.
  size_t need = 0;
  for (const bool bf16 : {false, true}) {
    if (bf16 && flat_path(dims, t_q, true)) continue;
    int splits = 0;
    const mla_status r = resolve(dims, batch, t_q, max_blocks, num_splits, bf16, &splits);
    if (r != MLA_OK) return r;
    const mla::Plan p = mla::decode_plan(dims->n_head, dims->kv_rank, dims->d_rope, batch, t_q, max_blocks, splits,
                                         mfma_path(dims, bf16));
    if (!p.ok) return MLA_ERR_SHAPE;
    if (p.bytes > need) need = p.bytes;
  }
  if (flat_path(dims, t_q, true)) {
    int64_t G = 0;
    const mla_status rf = flat_ranges(dims, batch, t_q, max_blocks, num_splits, &G);
    if (rf != MLA_OK) return rf;
    const mla::FlatPlan f = mla::flat_plan(dims->n_head, dims->d_rope, batch, t_q, max_blocks, G);
    if (!f.ok) return MLA_ERR_SHAPE;
    if (f.bytes > need) need = f.bytes;
  }
  *bytes = need;
  return MLA_OK;
}

static mla_status decode_impl(const mla_dims* dims, float scale, int32_t batch, int32_t t_q, const void* q_abs,
                              const void* kv_cache, mla_dtype dt, int64_t num_blocks, int32_t block_size,
                              const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
                              int32_t dcp_world, int32_t dcp_rank, int32_t dcp_interleave, void* out_lat,
                              mla_dtype out_dt, float* lse, void* workspace, size_t workspace_bytes,
                              int32_t num_splits, void* stream) {
  const mla_status st = check_decode_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0 || t_q < 1 || max_blocks < 1 || num_blocks < 1 || num_splits < 0) return MLA_ERR_SHAPE;
  if (block_size != 16) return MLA_ERR_UNSUPPORTED;
  if (!dt_ok(dt) || !dt_ok(out_dt)) return MLA_ERR_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return MLA_ERR_ARG;
  if (!workspace) return MLA_ERR_NULL;
  if (batch > 0 && (!q_abs || !kv_cache || !block_table || !seq_lens || !out_lat)) return MLA_ERR_NULL;
  if (!aligned(q_abs, 16) || !aligned(kv_cache, 16) || !aligned(out_lat, 16) || !aligned(block_table, 4) ||
      !aligned(seq_lens, 4) || !aligned(lse, 4) || !aligned(workspace, 256))
    return MLA_ERR_ARG;
  const bool bf16 = dt == MLA_BF16;
  const bool mfma = mfma_path(dims, bf16);
  if (!mfma && dims->kv_rank > 1024) return MLA_ERR_UNSUPPORTED;
  if ((int64_t)batch * t_q * dims->n_head > 2147483647LL) return MLA_ERR_SHAPE;

  size_t need = 0;
  const mla_status ws = mla_decode_workspace_size(dims, batch, t_q, max_blocks, block_size, num_splits, &need);
  if (ws != MLA_OK) return ws;
  if (workspace_bytes < need) return MLA_ERR_WORKSPACE;
  char* wsb = static_cast<char*>(workspace);

  if (flat_path(dims, t_q, bf16)) {
    int64_t G = 0;
    const mla_status rf = flat_ranges(dims, batch, t_q, max_blocks, num_splits, &G);
    if (rf != MLA_OK) return rf;
    const mla::FlatPlan f = mla::flat_plan(dims->n_head, dims->d_rope, batch, t_q, max_blocks, G);
    if (!f.ok) return MLA_ERR_SHAPE;
    mla::FlatArgs a;
    memset(&a, 0, sizeof a);
    a.q = q_abs;
    a.kv = kv_cache;
    a.bt = block_table;
    a.seq_lens = seq_lens;
    a.out = out_lat;
    a.lse = lse;
    a.header = reinterpret_cast<uint32_t*>(wsb);
    a.status = reinterpret_cast<uint32_t*>(wsb + mla::kHeaderBytes);
    a.req = reinterpret_cast<int32_t*>(wsb + f.req_off);
    a.lse_part = reinterpret_cast<float*>(wsb + f.lse_off);
    a.o_part = reinterpret_cast<float*>(wsb + f.o_off);
    a.num_blocks = num_blocks;
    a.batch = batch;
    a.t_q = t_q;
    a.n_head = dims->n_head;
    a.max_blocks = max_blocks;
    a.n_q = t_q * dims->n_head;
    a.G = f.G;
    a.m_tiles = f.m_tiles;
    a.qt = f.qt;
    a.scale = scale;
    a.out_bf16 = out_dt == MLA_BF16;
    a.dcp_world = dcp_world;
    a.dcp_rank = dcp_rank;
    a.dcp_interleave = dcp_interleave;
    const hipError_t e = mla::launch_decode_flat(a, dims->d_rope, f.qb, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
  }

  int splits = 0;
  const mla_status r = resolve(dims, batch, t_q, max_blocks, num_splits, bf16, &splits);
  if (r != MLA_OK) return r;
  const mla::Plan p = mla::decode_plan(dims->n_head, dims->kv_rank, dims->d_rope, batch, t_q, max_blocks, splits, bf16);
  if (!p.ok) return MLA_ERR_SHAPE;
  if (workspace_bytes < p.bytes) return MLA_ERR_WORKSPACE;

  mla::DecodeArgs a;
  memset(&a, 0, sizeof a);
  a.q = q_abs;
  a.kv = kv_cache;
  a.bt = block_table;
  a.seq_lens = seq_lens;
  a.out = out_lat;
  a.lse = lse;
  a.header = reinterpret_cast<uint32_t*>(wsb);
  a.status = reinterpret_cast<uint32_t*>(wsb + mla::kHeaderBytes);
  a.lse_part = reinterpret_cast<float*>(wsb + p.lse_off);
  a.o_part = reinterpret_cast<float*>(wsb + p.o_off);
  a.num_blocks = num_blocks;
  a.batch = batch;
  a.t_q = t_q;
  a.n_head = dims->n_head;
  a.kv_rank = dims->kv_rank;
  a.d_rope = dims->d_rope;
  a.max_blocks = max_blocks;
  a.n_q = t_q * dims->n_head;
  a.splits = p.splits;
  a.chunk_blocks = p.chunk_blocks;
  a.m_tiles = p.m_tiles;
  a.n_pairs = p.n_pairs;
  a.n_items = p.n_items;
  a.scale = scale;
  a.out_bf16 = out_dt == MLA_BF16;
  a.direct = p.splits == 1;
  a.dcp_world = dcp_world;
  a.dcp_rank = dcp_rank;
  a.dcp_interleave = dcp_interleave;
  const hipError_t e = mla::launch_decode(a, mfma, bf16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_decode_attention(const mla_dims* dims, float scale, int32_t batch, int32_t t_q, const void* q_abs,
                                const void* kv_cache, mla_dtype dt, int64_t num_blocks, int32_t block_size,
                                const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
                                void* out_lat, mla_dtype out_dt, float* lse, void* workspace,
                                size_t workspace_bytes, int32_t num_splits, void* stream) {
  return decode_impl(dims, scale, batch, t_q, q_abs, kv_cache, dt, num_blocks, block_size, block_table, max_blocks,
                     seq_lens, 1, 0, 1, out_lat, out_dt, lse, workspace, workspace_bytes, num_splits, stream);
}

mla_status mla_decode_attention_noalloc(const mla_dims* dims, float scale, int32_t batch, int32_t t_q,
                                        const void* q_abs, const void* kv_cache, mla_dtype dt, int64_t num_blocks,
                                        int32_t block_size, const int32_t* block_table, int32_t max_blocks,
                                        const int32_t* seq_lens, void* out_lat, mla_dtype out_dt, float* lse,
                                        int32_t num_splits, void* stream) {
  size_t need = 0;
  const mla_status ws = mla_decode_workspace_size(dims, batch, t_q, max_blocks, block_size, num_splits, &need);
  if (ws != MLA_OK) return ws;
  if (need > kNoAllocScratchBytes) return MLA_ERR_WORKSPACE;
  void* ptr = device_scratch();
  if (!ptr) return MLA_ERR_HIP;
  return decode_impl(dims, scale, batch, t_q, q_abs, kv_cache, dt, num_blocks, block_size, block_table, max_blocks,
                     seq_lens, 1, 0, 1, out_lat, out_dt, lse, ptr, kNoAllocScratchBytes, num_splits, stream);
}

mla_status mla_decode_attention_dcp(const mla_dims* dims, float scale, int32_t batch, int32_t t_q, const void* q_abs,
                                    const void* kv_cache, mla_dtype dt, int64_t num_blocks, int32_t block_size,
                                    const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
                                    int32_t dcp_world, int32_t dcp_rank, int32_t dcp_interleave, void* out_lat,
                                    mla_dtype out_dt, float* lse, void* workspace, size_t workspace_bytes,
                                    int32_t num_splits, void* stream) {
  if (dcp_world < 1 || dcp_rank < 0 || dcp_rank >= dcp_world || dcp_interleave < 1) return MLA_ERR_ARG;
  if (!lse && batch > 0) return MLA_ERR_NULL;  // a share is only usable with its LSE
  return decode_impl(dims, scale, batch, t_q, q_abs, kv_cache, dt, num_blocks, block_size, block_table, max_blocks,
                     seq_lens, dcp_world, dcp_rank, dcp_interleave, out_lat, out_dt, lse, workspace,
                     workspace_bytes, num_splits, stream);
}

mla_status mla_lse_combine(int32_t width, int64_t n_rows, int32_t n_parts, const float* o_parts,
                           const float* lse_parts, void* out, mla_dtype out_dt, float* lse, void* stream) {
  if (width < 1 || n_rows < 0 || n_parts < 1) return MLA_ERR_SHAPE;
  if (!dt_ok(out_dt)) return MLA_ERR_ARG;
  if (n_rows == 0) return MLA_OK;
  if (!o_parts || !lse_parts || !out) return MLA_ERR_NULL;
  const hipError_t e = mla::launch_lse_combine(n_rows, n_parts, width, o_parts, lse_parts, out, out_dt == MLA_BF16,
                                               lse, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_decompress_v(const mla_dims* dims, int64_t n_tok, const void* o_lat, mla_dtype o_dt,
                            const void* w_uv, mla_dtype w_dt, void* out, mla_dtype out_dt, void* stream) {
  if (!dims) return MLA_ERR_NULL;
  if (dims->n_head < 1 || dims->d_v < 1 || dims->kv_rank < 1) return MLA_ERR_DIMS;
  if (n_tok < 0) return MLA_ERR_SHAPE;
  if (!dt_ok(o_dt) || !dt_ok(w_dt) || !dt_ok(out_dt)) return MLA_ERR_ARG;
  if (n_tok == 0) return MLA_OK;
  if (!o_lat || !w_uv || !out) return MLA_ERR_NULL;
  if (!aligned(o_lat, 16) || !aligned(w_uv, 16) || !aligned(out, 16)) return MLA_ERR_ARG;
  const hipError_t e = mla::launch_decompress(dims->n_head, dims->d_v, dims->kv_rank, n_tok, o_lat, o_dt == MLA_BF16,
                                              w_uv, w_dt == MLA_BF16, out, out_dt == MLA_BF16,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_cache_append(const mla_dims* dims, int64_t n_tok, const void* c_kv, const void* k_pe,
                            const void* gamma, mla_dtype in_dt, float eps, const int32_t* positions,
                            double rope_base, int32_t rope_style, void* q_pe, const int64_t* slot_mapping,
                            void* kv_cache, mla_dtype kv_dt, int64_t num_blocks, int32_t block_size,
                            uint32_t* data_err, void* stream) {
  if (!dims) return MLA_ERR_NULL;
  if (dims->kv_rank < 1 || dims->d_rope < 0 || dims->d_rope % 2 != 0 || (q_pe && dims->n_head < 1))
    return MLA_ERR_DIMS;
  if (n_tok < 0 || num_blocks < 1) return MLA_ERR_SHAPE;
  if (block_size != 16) return MLA_ERR_UNSUPPORTED;
  if (dims->d_rope > 2 * mla::kRopeTableMax) return MLA_ERR_UNSUPPORTED;
  if (!dt_ok(in_dt) || !dt_ok(kv_dt)) return MLA_ERR_ARG;
  if (!(eps >= 0.f) || !isfinite(eps)) return MLA_ERR_ARG;
  if (rope_style != MLA_ROPE_NEOX && rope_style != MLA_ROPE_INTERLEAVED) return MLA_ERR_ARG;
  if (dims->d_rope > 0 && (!(rope_base > 0.0) || !isfinite(rope_base))) return MLA_ERR_ARG;
  if (num_blocks > INT64_MAX / block_size) return MLA_ERR_SHAPE;
  if (n_tok == 0) return MLA_OK;
  if (!c_kv || !slot_mapping || !kv_cache) return MLA_ERR_NULL;
  if (dims->d_rope > 0 && (!k_pe || !positions)) return MLA_ERR_NULL;
  mla::CacheAppend c = {};
  c.c_kv = c_kv;
  c.k_pe = k_pe;
  c.gamma = gamma;
  c.q_pe = dims->d_rope > 0 ? q_pe : nullptr;
  c.positions = positions;
  c.slots = slot_mapping;
  c.cache = kv_cache;
  c.err = data_err;
  c.n_tok = n_tok;
  c.num_slots = num_blocks * block_size;
  c.kv_rank = dims->kv_rank;
  c.d_rope = dims->d_rope;
  c.n_head = dims->n_head;
  c.eps = eps;
  c.rope_base = rope_base;
  c.in_bf16 = in_dt == MLA_BF16;
  c.cache_bf16 = kv_dt == MLA_BF16;
  c.interleaved = rope_style == MLA_ROPE_INTERLEAVED;
  const hipError_t e = mla::launch_cache_append(c, static_cast<hipStream_t>(stream));
  if (e == hipErrorInvalidValue) return MLA_ERR_SHAPE;
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_prefill_workspace_size(const mla_dims* dims, int32_t batch, int32_t max_blocks, int32_t block_size,
                                      size_t* bytes) {
  if (!dims || !bytes) return MLA_ERR_NULL;
  if (dims->n_head < 1 || dims->d_nope < 1 || dims->d_rope < 0 || dims->d_v < 1 || dims->kv_rank < 1)
    return MLA_ERR_DIMS;
  if (batch < 0 || max_blocks < 1) return MLA_ERR_SHAPE;
  if (block_size != 16) return MLA_ERR_UNSUPPORTED;
  if (!mla::prefill_supported(dims->n_head, dims->d_nope, dims->d_rope, dims->d_v, dims->kv_rank))
    return MLA_ERR_UNSUPPORTED;
  if ((int64_t)max_blocks * 16 > INT32_MAX) return MLA_ERR_SHAPE;
  *bytes = mla::prefill_plan(dims->n_head, dims->d_nope, dims->d_rope, dims->d_v, dims->kv_rank, batch, max_blocks)
               .bytes;
  return MLA_OK;
}

mla_status mla_prefill_attention(const mla_dims* dims, float scale, int32_t batch, int32_t t_q, const void* q_nope,
                                 const void* q_pe, const void* w_uk, const void* w_uv, const void* kv_cache,
                                 mla_dtype dt, int64_t num_blocks, int32_t block_size, const int32_t* block_table,
                                 int32_t max_blocks, const int32_t* seq_lens, void* out, mla_dtype out_dt, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  size_t need = 0;
  const mla_status ws = mla_prefill_workspace_size(dims, batch, max_blocks, block_size, &need);
  if (ws != MLA_OK) return ws;
  if (t_q < 1 || num_blocks < 1) return MLA_ERR_SHAPE;
  if (!dt_ok(dt) || !dt_ok(out_dt)) return MLA_ERR_ARG;
  if (dt != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !isfinite(scale)) return MLA_ERR_ARG;
  if (!workspace) return MLA_ERR_NULL;
  if (workspace_bytes < need) return MLA_ERR_WORKSPACE;
  if (batch == 0) return MLA_OK;
  if (!q_nope || !w_uk || !w_uv || !kv_cache || !block_table || !seq_lens || !out || (dims->d_rope > 0 && !q_pe))
    return MLA_ERR_NULL;
  const mla::PrefillPlan p = mla::prefill_plan(dims->n_head, dims->d_nope, dims->d_rope, dims->d_v, dims->kv_rank,
                                               batch, max_blocks);
  char* wsb = static_cast<char*>(workspace);
  mla::PrefillArgs a = {};
  a.q_nope = q_nope;
  a.q_pe = q_pe;
  a.w_uk = w_uk;
  a.w_uv = w_uv;
  a.kv = kv_cache;
  a.bt = block_table;
  a.seq_lens = seq_lens;
  a.out = out;
  a.lse = lse;
  a.kw = reinterpret_cast<uint16_t*>(wsb + p.kw_off);
  a.vw = reinterpret_cast<uint16_t*>(wsb + p.vw_off);
  a.header = reinterpret_cast<uint32_t*>(wsb);
  a.status = reinterpret_cast<uint32_t*>(wsb + p.status_off);
  a.num_blocks = num_blocks;
  a.batch = batch;
  a.t_q = t_q;
  a.n_head = dims->n_head;
  a.max_blocks = max_blocks;
  a.max_rows = p.max_rows;
  a.scale = scale;
  a.out_bf16 = out_dt == MLA_BF16;
  const hipError_t e = mla::launch_prefill(a, dims->d_rope, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_decode_status(const void* workspace, uint32_t* flags, void* stream) {
  if (!workspace || !flags) return MLA_ERR_NULL;
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return MLA_ERR_HIP;
  uint32_t head[4];
  if (hipMemcpy(head, workspace, sizeof head, hipMemcpyDeviceToHost) != hipSuccess) return MLA_ERR_HIP;
  if (head[0] != mla::kWorkspaceMagic) return MLA_ERR_WORKSPACE;
  uint32_t acc = 0;
  const uint32_t n = head[1];
  const char* slots = static_cast<const char*>(workspace) + mla::kHeaderBytes;
  uint32_t buf[1024];
  for (uint32_t done = 0; done < n;) {
    const uint32_t k = n - done < 1024u ? n - done : 1024u;
    if (hipMemcpy(buf, slots + (size_t)done * 4, (size_t)k * 4, hipMemcpyDeviceToHost) != hipSuccess)
      return MLA_ERR_HIP;
    for (uint32_t i = 0; i < k; ++i) acc |= buf[i];
    done += k;
  }
  *flags = acc;
  return MLA_OK;
}

}  // extern "C"

extern "C" {

mla_status mla_prolog_workspace_size(const mla_dims* dims, const mla_prolog_dims* pd, int64_t n_tok, size_t* bytes) {
  if (!dims || !pd || !bytes) return MLA_ERR_NULL;
  if (dims->n_head < 1 || dims->d_nope < 1 || dims->d_rope < 0 || dims->d_rope % 2 != 0 || dims->kv_rank < 1 ||
      pd->hidden < 1 || pd->q_rank < 1)
    return MLA_ERR_DIMS;
  if (n_tok < 0) return MLA_ERR_SHAPE;
  if (!mla::prolog_supported(dims->n_head, dims->d_nope, dims->d_rope, dims->kv_rank, pd->hidden, pd->q_rank))
    return MLA_ERR_UNSUPPORTED;
  *bytes = mla::prolog_plan(dims->n_head, dims->d_nope, dims->d_rope, dims->kv_rank, pd->hidden, pd->q_rank, n_tok)
               .bytes;
  return MLA_OK;
}

mla_status mla_prolog(const mla_dims* dims, const mla_prolog_dims* pd, int64_t n_tok, const void* x, const void* w_dq,
                      const void* w_uq, const void* w_qr, const void* w_uk, const void* w_dkv, const void* w_kr,
                      const void* gamma_q, const void* gamma_kv, mla_dtype dt, float eps_q, float eps_kv,
                      const int32_t* positions, double rope_base, int32_t rope_style, const int64_t* slot_mapping,
                      void* kv_cache, mla_dtype kv_dt, int64_t num_blocks, int32_t block_size, void* q_abs,
                      mla_dtype q_dt, uint32_t* data_err, void* workspace, size_t workspace_bytes, void* stream) {
  size_t need = 0;
  const mla_status ws = mla_prolog_workspace_size(dims, pd, n_tok, &need);
  if (ws != MLA_OK) return ws;
  if (num_blocks < 1) return MLA_ERR_SHAPE;
  if (block_size != 16) return MLA_ERR_UNSUPPORTED;
  if (dims->d_rope > 2 * mla::kRopeTableMax) return MLA_ERR_UNSUPPORTED;
  if (!dt_ok(dt) || !dt_ok(kv_dt) || !dt_ok(q_dt)) return MLA_ERR_ARG;
  if (dt != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  if (!(eps_q >= 0.f) || !isfinite(eps_q) || !(eps_kv >= 0.f) || !isfinite(eps_kv)) return MLA_ERR_ARG;
  if (rope_style != MLA_ROPE_NEOX && rope_style != MLA_ROPE_INTERLEAVED) return MLA_ERR_ARG;
  if (dims->d_rope > 0 && (!(rope_base > 0.0) || !isfinite(rope_base))) return MLA_ERR_ARG;
  if (num_blocks > INT64_MAX / block_size) return MLA_ERR_SHAPE;
  if (!workspace) return MLA_ERR_NULL;
  if (workspace_bytes < need) return MLA_ERR_WORKSPACE;
  if (n_tok == 0) return MLA_OK;
  if (!x || !w_dq || !w_uq || !w_uk || !w_dkv || !slot_mapping || !kv_cache || !q_abs) return MLA_ERR_NULL;
  if (dims->d_rope > 0 && (!w_qr || !w_kr || !positions)) return MLA_ERR_NULL;
  // the products read 16-byte runs of x and of every weight row
  for (const void* ptr : {x, w_dq, w_uq, w_qr, w_dkv, w_kr})
    if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0) return MLA_ERR_ARG;
  const mla::PrologPlan p =
      mla::prolog_plan(dims->n_head, dims->d_nope, dims->d_rope, dims->kv_rank, pd->hidden, pd->q_rank, n_tok);
  char* wsb = static_cast<char*>(workspace);
  mla::PrologArgs a = {};
  a.x = x;
  a.w_dq = w_dq;
  a.w_uq = w_uq;
  a.w_qr = w_qr;
  a.w_uk = w_uk;
  a.w_dkv = w_dkv;
  a.w_kr = w_kr;
  a.gamma_q = gamma_q;
  a.gamma_kv = gamma_kv;
  a.eps_q = eps_q;
  a.eps_kv = eps_kv;
  a.positions = positions;
  a.rope_base = rope_base;
  a.interleaved = rope_style == MLA_ROPE_INTERLEAVED;
  a.cache_bf16 = kv_dt == MLA_BF16;
  a.q_bf16 = q_dt == MLA_BF16;
  a.slots = slot_mapping;
  a.cache = kv_cache;
  a.num_slots = num_blocks * block_size;
  a.err = data_err;
  a.q_abs = q_abs;
  a.n_tok = n_tok;
  a.hidden = pd->hidden;
  a.q_rank = pd->q_rank;
  a.n_head = dims->n_head;
  a.d_nope = dims->d_nope;
  a.d_rope = dims->d_rope;
  a.kv_rank = dims->kv_rank;
  a.splits1 = p.splits1;
  a.splits2 = p.splits2;
  a.part = reinterpret_cast<float*>(wsb + p.part_off);
  a.cq = reinterpret_cast<uint16_t*>(wsb + p.cq_off);
  a.ckv = reinterpret_cast<uint16_t*>(wsb + p.ckv_off);
  a.kpe = reinterpret_cast<uint16_t*>(wsb + p.kpe_off);
  a.qn = reinterpret_cast<uint16_t*>(wsb + p.qn_off);
  a.qp = reinterpret_cast<uint16_t*>(wsb + p.qp_off);
  a.yq = reinterpret_cast<float*>(wsb + p.yq_off);
  const hipError_t e = mla::launch_prolog(a, static_cast<hipStream_t>(stream));
  if (e == hipErrorInvalidValue) return MLA_ERR_SHAPE;
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"
