// Host-side launch interface between the C ABI (mla_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

// Workspace of one decode call:
//   [0, 256)            header: magic, number of status slots, splits, batch
//   [256, 256 + S4)     one uint32 data-error word per split workgroup
//   then (256-aligned)  lse partials  f32 [batch][splits][t_q * n_head]
//   then (256-aligned)  o partials    f32 [batch][splits][t_q * n_head][kv_rank]
constexpr uint32_t kWorkspaceMagic = 0x314C4D41u;  // "AML1"
constexpr size_t kHeaderBytes = 256;
constexpr int kMaxSplits = 1024;
constexpr int kQRowsPerWG = 64;     // query rows (query index x head) per MFMA workgroup
constexpr int kGenericQRows = 1;    // query rows per generic workgroup

struct DecodeArgs {
  const void* q;           // [B][t_q][H][D]
  const void* kv;          // [num_blocks][16][D]
  const int32_t* bt;       // [B][max_blocks]
  const int32_t* seq_lens; // [B]
  void* out;               // [B][t_q][H][kv_rank]      (written when splits == 1)
  float* lse;              // [B][t_q][H] or null       (written when splits == 1)
  float* lse_part;         // [B][splits][n_q]
  float* o_part;           // [B][splits][n_q][kv_rank]
  uint32_t* header;        // workspace header
  uint32_t* status;        // [n_items]
  int64_t num_blocks;
  int batch, t_q, n_head, kv_rank, d_rope, max_blocks;
  int n_q;                 // t_q * n_head
  int splits;              // KV splits per request
  int chunk_blocks;        // cache blocks per split
  int m_tiles;             // query-row tiles per (request, split)
  int n_pairs;             // batch * splits
  int n_items;             // status slots = n_pairs * m_tiles
  float scale;             // softmax scale
  int out_bf16;            // out dtype is bfloat16
  int direct;              // splits == 1: write final outputs, no merge
};

struct Plan {
  int splits, chunk_blocks, m_tiles, n_pairs, n_items;
  bool mfma;
  size_t lse_off, o_off, bytes;
};

// Kernel selection and workspace layout for a decode call.
Plan decode_plan(int n_head, int kv_rank, int d_rope, int batch, int t_q, int max_blocks,
                 int splits, bool bf16);

hipError_t launch_decode(const DecodeArgs& a, bool mfma, bool bf16, hipStream_t stream);

hipError_t launch_absorb(int n_head, int d_nope, int d_rope, int kv_rank, int64_t n_tok,
                         const void* q_nope, const void* q_pe, const void* w_uk, bool in_bf16,
                         void* q_abs, bool out_bf16, hipStream_t stream);

hipError_t launch_decompress(int n_head, int d_v, int kv_rank, int64_t n_tok, const void* o_lat,
                             bool o_bf16, const void* w_uv, bool w_bf16, void* out, bool out_bf16,
                             hipStream_t stream);

// One cache-append prolog call (RmsNorm of c_kv, rope of k_pe and q_pe,
// slot-mapped cache write).  Rope bases are tabulated per launch, so d_rope is
// at most 2 * kRopeTableMax.
constexpr int kRopeTableMax = 128;

struct CacheAppend {
  const void* c_kv;          // [n_tok][kv_rank]
  const void* k_pe;          // [n_tok][d_rope]
  const void* gamma;         // [kv_rank] or null
  void* q_pe;                // [n_tok][n_head][d_rope] or null
  const int32_t* positions;  // [n_tok]
  const int64_t* slots;      // [n_tok]
  void* cache;               // [num_slots][kv_rank + d_rope]
  uint32_t* err;             // data-error word or null
  int64_t n_tok, num_slots;
  int kv_rank, d_rope, n_head;
  float eps;
  double rope_base;
  bool in_bf16, cache_bf16, interleaved;
};

hipError_t launch_cache_append(const CacheAppend& c, hipStream_t stream);

}  // namespace mla
