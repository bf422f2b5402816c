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
  int dcp_world, dcp_rank, dcp_interleave;  // context-parallel share (1, 0, 1: all rows)
};

struct Plan {
  int splits, chunk_blocks, m_tiles, n_pairs, n_items;
  bool mfma;
  bool ok;  // counts fit the device's 32-bit indices
  size_t lse_off, o_off, bytes;
};

// Length-balanced decode (bf16, kv_rank 512, rope width 0 or 64).  The
// 32-row tiles of all requests, in request order, form one sequence of T
// tiles per query tile; range g of G covers tiles [g T / G, (g + 1) T / G),
// so every workgroup streams the same number of tiles whatever the lengths.
// A request that falls in one range is finished by its workgroup; the pieces
// of a request cut by range ends are merged by decode_flat_merge.
// Workspace:
//   [0, 256)           header: magic, number of status slots, ranges, batch
//   [256, ...)         one uint32 data-error word per workgroup (G * m_tiles)
//   then (256-aligned) int32x4 per request: first and last range holding it,
//                      partial slot of the first piece
//   then (256-aligned) lse partials f32 [G][m_tiles][2][qt]
//   then (256-aligned) o partials   [G][m_tiles][2][qt][512], bf16 when the output is bf16, else f32
struct FlatArgs {
  const void* q;           // [B][t_q][H][D]
  const void* kv;          // [num_blocks][16][D]
  const int32_t* bt;       // [B][max_blocks]
  const int32_t* seq_lens; // [B]
  void* out;               // [B][t_q][H][512]
  float* lse;              // [B][t_q][H] or null
  float* lse_part;
  float* o_part;
  int32_t* req;            // [B][4]
  uint32_t* header;
  uint32_t* status;        // [G * m_tiles]
  int64_t num_blocks;
  int batch, t_q, n_head, max_blocks, n_q;
  int G;                   // ranges per query tile
  int m_tiles, qt;         // query tiles per request, query rows per tile
  float scale;
  int out_bf16;
  int dcp_world, dcp_rank, dcp_interleave;
};

struct FlatPlan {
  int G, m_tiles, qt, qb;  // ranges, query tiles, rows per tile, waves per workgroup
  bool ok;
  size_t req_off, lse_off, o_off, bytes;
};

bool flat_supported(int kv_rank, int d_rope, bool bf16);
FlatPlan flat_plan(int n_head, int d_rope, int batch, int t_q, int max_blocks, int64_t ranges);
// Ranges that give one workgroup per compute unit (at most one per tile).
int64_t flat_auto_ranges(int n_head, int batch, int t_q, int max_blocks, int cus);
hipError_t launch_decode_flat(const FlatArgs& a, int d_rope, int qb, hipStream_t stream);

// Kernel selection and workspace layout for a decode call.
Plan decode_plan(int n_head, int kv_rank, int d_rope, int batch, int t_q, int max_blocks,
                 int splits, bool bf16);

hipError_t launch_decode(const DecodeArgs& a, bool mfma, bool bf16, hipStream_t stream);

hipError_t launch_lse_combine(int64_t n_rows, int n_parts, int width, const float* o_parts, const float* lse_parts,
                              void* out, bool out_bf16, float* lse_out, hipStream_t stream);

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

// The fused prolog.  Skinny GEMM: part[split][n][o] over the rows o of up to
// four concatenated weight segments (each [rows][K], rows a multiple of 16).
struct GemmSeg {
  const uint16_t* w;
  int rows;
};
struct SkinnyGemm {
  const uint16_t* x;  // [n_tok][K]
  GemmSeg seg[4];
  int n_seg, K, N;    // N = total rows
  int64_t n_tok;
  int splits, kper;   // K splits requested / k per split (set by the launcher)
  float* part;        // [splits][n_tok][N]
};
struct PrologArgs {
  const void *x, *w_dq, *w_uq, *w_qr, *w_uk, *w_dkv, *w_kr, *gamma_q, *gamma_kv;
  float eps_q, eps_kv;
  const int32_t* positions;
  double rope_base;
  bool interleaved, cache_bf16, q_bf16;
  const int64_t* slots;
  void* cache;
  int64_t num_slots;
  uint32_t* err;
  void* q_abs;
  int64_t n_tok;
  int hidden, q_rank, n_head, d_nope, d_rope, kv_rank;
  int splits1, splits2;
  float* part;                      // workspace: split partials
  uint16_t *cq, *ckv, *kpe, *qn, *qp;  // workspace: bf16 intermediates
  float* yq;                        // workspace: x W^DQ before its norm
};
struct PrologPlan {
  int splits1, splits2;
  size_t part_off, cq_off, ckv_off, kpe_off, qn_off, qp_off, yq_off, bytes;
};
PrologPlan prolog_plan(int n_head, int d_nope, int d_rope, int kv_rank, int hidden, int q_rank, int64_t n_tok);
bool prolog_supported(int n_head, int d_nope, int d_rope, int kv_rank, int hidden, int q_rank);
hipError_t launch_prolog(const PrologArgs& a, hipStream_t stream);

// One naive-form prefill call.  Workspace: the 256-byte header, one status
// word per request, then K_nope [B][H][max_rows][d_nope] and V
// [B][H][max_rows][d_v] (bf16), each 256-byte aligned.
struct PrefillArgs {
  const void* q_nope;        // [B][t_q][H][d_nope]
  const void* q_pe;          // [B][t_q][H][d_rope]
  const void* w_uk;          // [H][d_nope][kv_rank]
  const void* w_uv;          // [H][d_v][kv_rank]
  const void* kv;            // [num_blocks][16][kv_rank + d_rope]
  const int32_t* bt;         // [B][max_blocks]
  const int32_t* seq_lens;   // [B]
  void* out;                 // [B][t_q][H][d_v]
  float* lse;                // [B][t_q][H] or null
  uint16_t* kw;              // workspace K_nope
  uint16_t* vw;              // workspace V
  uint32_t* header;          // workspace header
  uint32_t* status;          // [B]
  int64_t num_blocks;
  int batch, t_q, n_head, max_blocks, max_rows;
  float scale;
  int out_bf16;
  // Launch geometry, filled by launch_prefill.
  int n_wtiles;  // 128-row tiles of the stacked [W_UK; W_UV]
  int n_mtiles;  // 128-row tiles of a request's cache rows
  int wgroup;    // weight tiles one XCD keeps in L2 while the cache tiles stream
};

struct PrefillPlan {
  int max_rows;
  size_t status_off, kw_off, vw_off, bytes;
};

PrefillPlan prefill_plan(int n_head, int d_nope, int d_rope, int d_v, int kv_rank, int batch, int max_blocks);
bool prefill_supported(int n_head, int d_nope, int d_rope, int d_v, int kv_rank);
hipError_t launch_prefill(const PrefillArgs& a, int d_rope, hipStream_t stream);

}  // namespace mla
