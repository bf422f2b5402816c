// Length-balanced split-KV paged MLA decode for gfx950: bf16 queries and cache,
// kv_rank 512, rope width 0 or 64, and the merge of the pieces it leaves.
//
// What is computed (vllm.cpp "cpu_mla_attn.cpp", MlaDecodeAttentionKernel;
// memra-engine "mla.rs", MlaInputs causal rule): for request b, query i and
// head h, scores s_j = scale * <q_abs, row_j> over the full latent row
// [c_kv | k_pe], softmax over the visible rows j < L - t_q + i + 1, output the
// softmax-weighted sum of the leading 512 columns of the same rows, and
// lse = log sum_j exp(s_j).  L == 0 gives zeros and -inf.
//
// Work split.  A request of L rows has ceil(L / 32) tiles of 32 rows (two
// 16-row cache blocks).  The tiles of all requests, in request order, form one
// sequence of T tiles; range g of G covers tiles [g T / G, (g + 1) T / G), so
// every workgroup streams the same number of tiles whatever the lengths (the
// sequence is rebuilt on the device from seq_lens by every workgroup: one
// load and a wave scan per 64 requests).  Each query tile (qt = 128 query
// rows x heads of one request) has its own G workgroups, placed so that the
// query tiles of one range share an XCD and read the cache through one L2.
// A request inside one range is finished there (final output and LSE);
// a request cut by a range end leaves (o, lse) pieces, at most two per
// workgroup (its first and its last request; o in the output's type, bf16 or
// float32, lse in float32), which decode_flat_merge combines:
//   M = max lse_k, w_k = exp(lse_k - M), o = sum w_k o_k / sum w_k,
//   lse = M + log sum w_k  (all -inf: zeros and -inf).
//
// Workgroup: four waves, one per SIMD; wave w owns query rows [32 w, 32 w + 32)
// of the tile over the full row width, so the scores, the softmax and the
// probabilities never leave its registers:
//   * tiles go HBM -> LDS directly (buffer_load ... lds) through a ring of four
//     tile images, three tiles in flight while one is consumed; one buffer
//     resource per cache block, sized to the request's valid rows (rows past
//     the end read as zeros; no address outside a real block is formed);
//   * S^T = K Q^T with 32x32x16 bf16 MFMA: the 32 tile rows as the A operand
//     (one 16-byte LDS read per lane and product), the wave's 32 queries as
//     B operands held in registers for the request;
//   * softmax against a fixed reference per row (the maximum of its first
//     visible tile; later tiles may exceed it by up to kLimit in log2 units,
//     and a piece that goes further is streamed a second time with its true
//     maximum), so the output accumulators change only through the matrix
//     products and stay in the matrix-core registers;
//   * the probabilities, packed to bf16, are already the B operand of
//     O^T = V^T P^T (the 32x32 output layout of S^T holds, per lane, the rows
//     that the B operand's k-slots take, and the transposing reads of V^T use
//     the same row order), so P^T stays in registers;
//   * V^T comes from the same LDS tile with ds_read_b64_tr_b16, two reads per
//     16 rows of a 32-column tile.
// One barrier per tile: after it tile k is resident for every wave and the
// slot of tile k - 1 is free for tile k + 3.  A wave issues one instruction
// at a time, so the tile step is kept short: per-lane load offsets computed
// once, 32-bit tile positions, LDS waits two reads at a time, the producer's
// scalar work among the first products, masking only on tiles that reach
// past a query's horizon.
#include "decode_common.hpp"
#include "kernels.hpp"

#include <math.h>
#include <utility>

namespace mla {
namespace {

constexpr int kWaves = 4;   // per workgroup, one per SIMD
constexpr int kRing = 4;    // tile images in LDS
constexpr int kKAhead = 6;  // K reads in flight ahead of their products
constexpr int kVAhead = 2;  // 32-column V^T tiles in flight ahead of their products
constexpr float kLimit = 64.f;  // log2 headroom of the fixed softmax reference

// LDS image of one 32-row tile (two 16-row cache blocks) of latent rows of
// width D = 512 + D_ROPE, filled by 1 KB wave-loads (64 lanes x 16 bytes).
// Every row takes 72 16-byte chunk slots (1152 bytes: the whole row at
// D = 576, the row and 8 empty slots at D = 512), and logical chunk c of row r
// sits in slot c ^ (r & 7).  The second block's image starts 128 bytes after
// the end of the first, so that the 16-byte K reads of one product (32 rows,
// both blocks, one chunk column) and the transposing V^T reads (4 rows x 64
// bytes per 32 lanes, rows chosen as below) are free of LDS bank conflicts on
// gfx950 (measured; without the 128-byte gap the K reads conflict two-way).
template <int D_ROPE>
struct FlatTile {
  static constexpr int D = 512 + D_ROPE;
  static constexpr int CH = D / 8;                 // 16-byte chunks of data per row
  static constexpr int STRIDE = 72;                // chunk slots per row
  static constexpr int BLK_POS = 16 * STRIDE;      // chunk slots of one block image
  static constexpr int BLK_LOADS = BLK_POS / 64;   // 1 KB wave-loads per block
  static constexpr int BLK1 = BLK_POS * 16 + 128;  // byte offset of the second block's image
  static constexpr int IMG_BYTES = BLK1 + BLK_POS * 16;  // one 32-row tile image
  static constexpr int TILE_LOADS = 2 * BLK_LOADS;
  static constexpr int KSTEPS = D / 16;            // 16-wide k-steps of q.k
  static_assert(CH <= STRIDE && BLK_POS % 64 == 0 && TILE_LOADS % 4 == 0 && IMG_BYTES % 16 == 0, "tile geometry");
};

typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 32x32x16 products whose accumulator lives in vector registers (the output
// accumulators fill the matrix-core registers, and the softmax reads the scores
// with vector instructions).  Written as assembly, so the compiler does not
// move the accumulator into matrix-core registers; it also does not know the
// products' latency, so a chain ends with mfma_vacc_drain() before anything
// else reads the accumulator.  Each product of a chain accumulates into the
// registers the previous one wrote, which the hardware forwards back to back.
__device__ __forceinline__ void mfma_vacc_first(f32x16& c, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_vacc(f32x16& c, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
// 20 wait states: more than any matrix product needs before a vector
// instruction may read its result.
__device__ __forceinline__ void mfma_vacc_drain(f32x16& c) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(c));
}

// Position within the tile (block * 16 + row) of the tile row that output row
// i of S^T = K Q^T stands for.  The products see the 32 rows in this order;
// it makes every group of 4 rows that one transposing V^T read covers
// {b, b + 1, b + 4, b + 5} (b = 8 e + 2 h), whose 64-byte pieces sit in
// different LDS banks.  Output element v of the 32x32 product in lane half h
// is row i = 8 (v / 4) + 4 h + v % 4, i.e. position 8 (v / 4) + 2 h +
// {0, 1, 4, 5}[v % 4].
__host__ __device__ constexpr int tile_pos(int i) {
  return 8 * (i >> 3) + 2 * ((i >> 2) & 1) + ((i & 1) | ((i & 2) << 1));
}

typedef __attribute__((address_space(4))) const int32_t const_i32;

// 16-byte / transposing 8-byte LDS reads at a compile-time offset; the result
// is not ready until a matching lgkm wait.  (Written as assembly so that the
// waits can be exact: the compiler would wait for every read before its use.)
template <int OFF>
__device__ __forceinline__ void lds_b128(uint32_t addr, u32x4& v) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
}
template <int OFF>
__device__ __forceinline__ void lds_tr_b64(uint32_t addr, uint2& v) {
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
}
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x4& x, u32x4& y) {
  static_assert(N >= 0 && N < 16, "lgkmcnt is four bits");
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(x), "+v"(y) : "i"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void lgkm_wait(uint2& x, uint2& y, uint2& z, uint2& u) {
  static_assert(N >= 0 && N < 16, "lgkmcnt is four bits");
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(x), "+v"(y), "+v"(z), "+v"(u) : "i"(N) : "memory");
}

// Tiles of a request of global length Lg (L rows held here), 0 for an empty or
// invalid request; f receives its data-error bits.
__device__ __forceinline__ int req_tiles(const FlatArgs& a, int64_t Lg, int64_t& L, uint32_t& f) {
  L = held_rows(Lg, a.dcp_world, a.dcp_rank, a.dcp_interleave);
  f = request_flags(Lg, L, a.t_q, a.max_blocks);
  return (f || L <= 0) ? 0 : (int)((L + 31) >> 5);
}

__device__ __forceinline__ int64_t wave_sum64(int64_t v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// The workgroup's place in the tile sequence, computed identically by every
// wave: T (total tiles), the range [t0, t1) of range g, and the first request
// this workgroup handles with the index of its first tile.  That request is
// the first one not entirely before t0, where an empty request whose position
// is exactly t0 counts as this range's (an empty request belongs to the range
// holding its position; empty requests at position T belong to the last range).
struct FlatRange {
  int T, t0, t1, p_first;
  int b_first;
};

__device__ FlatRange flat_range(const FlatArgs& a, int g) {
  const int lane = threadIdx.x & 63;
  int64_t acc = 0;
  for (int base = 0; base < a.batch; base += 64) {
    const int b = base + lane;
    if (b < a.batch) {
      int64_t L;
      uint32_t f;
      acc += req_tiles(a, a.seq_lens[b], L, f);
    }
  }
  FlatRange r;
  r.T = (int)uniform64(wave_sum64(acc));
  r.t0 = (int)((int64_t)g * r.T / a.G);
  r.t1 = (int)((int64_t)(g + 1) * r.T / a.G);
  r.b_first = a.batch;
  r.p_first = r.T;
  int64_t run = 0;
  for (int base = 0; base < a.batch; base += 64) {
    const int b = base + lane;
    int64_t n = 0;
    if (b < a.batch) {
      int64_t L;
      uint32_t f;
      n = req_tiles(a, a.seq_lens[b], L, f);
    }
    int64_t incl = n;
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    incl += run;
    const int64_t excl = incl - n;
    const bool before = b < a.batch && incl <= r.t0 && (n > 0 || excl < r.t0);
    const int cnt = __popcll(__ballot(before));
    if (cnt < 64) {
      r.b_first = __builtin_amdgcn_readfirstlane(base + cnt);
      r.p_first = (int)uniform64(__shfl(excl, cnt, 64));
      break;
    }
    run = __shfl(incl, 63, 64);
  }
  return r;
}

// The range holding tile t (t < T): the largest g with g T / G <= t.
__device__ __forceinline__ int range_of(int64_t t, int64_t T, int G) { return (int)(((t + 1) * G - 1) / T); }

// A request cursor: request b starts at tile p of the sequence and has n tiles
// and L rows here (L <= Lg, a 32-bit length); row is its block-table row.
struct Cursor {
  int b, n, p;
  int L, Lg;
  uint32_t f;
  const const_i32* row;
};

__device__ __forceinline__ void cursor_load(const FlatArgs& a, Cursor& c) {
  const const_i32* sl = (const const_i32*)a.seq_lens;
  c.Lg = sl[c.b];
  int64_t L;
  c.n = req_tiles(a, c.Lg, L, c.f);
  c.L = (int)L;
  c.row = (const const_i32*)a.bt + (int64_t)c.b * a.max_blocks;
}

// Four waves (one per SIMD), 128 query rows per workgroup: wave w owns query
// rows [32 w, 32 w + 32) of the workgroup's query tile over the full row
// width and all 512 value columns, as the 32 columns of 32x32x16 bf16 matrix
// products.  A request's 128 query rows x heads share every tile image, so
// its cache rows go HBM -> LDS once, and every 16-byte K read and every pair
// of transposing V^T reads from LDS feeds one 32-row product.  The queries
// (144 registers) and the output accumulators (256) fill most of a SIMD's
// register file, hence one wave per SIMD: its latencies are covered by reads
// issued several products ahead.
template <int D_ROPE>
__global__ __launch_bounds__(64 * kWaves, 1) void decode_flat_mfma(const FlatArgs a) {
  using T = FlatTile<D_ROPE>;
  constexpr int D = T::D, CH = T::CH, STRIDE = T::STRIDE, KS = T::KSTEPS;
  constexpr int QT = 32 * kWaves;  // query rows per workgroup
  constexpr int NCT = 16;          // 32-column output tiles of the 512 value columns
  __shared__ __attribute__((aligned(16))) u32x4 ring[kRing * T::IMG_BYTES / 16];
  __shared__ int vote[kWaves];

  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.header[0] = kWorkspaceMagic;
    a.header[1] = (uint32_t)(a.G * a.m_tiles);
    a.header[2] = (uint32_t)a.G;
    a.header[3] = (uint32_t)a.batch;
  }
  // Workgroup i runs on XCD i % 8: the query tiles of range g all land on XCD g % 8.
  const int lin = blockIdx.x;
  const int rest = lin >> 3;
  const int mt = rest % a.m_tiles;
  const int g = (rest / a.m_tiles) * 8 + (lin & 7);
  if (g >= a.G) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j32 = lane & 31, h = lane >> 5;  // query column of the products, lane half
  const int l16 = lane & 15;

  const FlatRange R = flat_range(a, g);
  const int t0 = R.t0, t1 = R.t1;
  const bool last_range = g == a.G - 1;
  if (t0 == t1 && !last_range) {
    // No tiles and no request here; the merge may still walk over this range
    // (ranges outnumber tiles), so its first slot reads as an empty piece.
    const int64_t pidx = ((int64_t)g * a.m_tiles + mt) * 2;
    for (int i = tid; i < QT; i += 64 * kWaves) a.lse_part[pidx * QT + i] = -INFINITY;
    if (tid == 0) a.status[(int64_t)g * a.m_tiles + mt] = 0u;
    return;
  }

  const uint16_t* kv = static_cast<const uint16_t*>(a.kv);
  const uint32_t nb32 = a.num_blocks < (int64_t)INT32_MAX ? (uint32_t)a.num_blocks : (uint32_t)INT32_MAX;

  // Tile loads: wave w loads half w % 2 of block my_hb = w / 2 of a tile
  // image, the 1 KB wave-loads u = LJ (w % 2) + j of that block, load u
  // covering chunk slots [64 u, 64 u + 64) of the block image.  vo[j]: global
  // byte offset (within the block) of this lane's 16 bytes of load j; padding
  // slots get an offset past any block (they read zeros).
  constexpr int LJ = T::BLK_LOADS / 2;  // loads per wave per tile
  static_assert(kWaves == 4 && T::BLK_LOADS % 2 == 0 && 2 * LJ * 2 == T::TILE_LOADS, "two waves per block");
  const int my_hb = w >> 1;
  uint32_t vo[LJ];
#pragma unroll
  for (int j = 0; j < LJ; ++j) {
    const int pos = (LJ * (w & 1) + j) * 64 + lane;
    const int rl = pos / STRIDE;
    const int c = (pos - rl * STRIDE) ^ (rl & 7);
    vo[j] = c < CH ? (uint32_t)(rl * D + c * 8) * 2u : 0x7ffffff0u;
  }
  const uint32_t ring_base = lds_addr(ring);
  // This wave's part of a tile image: its block's image, then its half.
  const uint32_t wave_img = (my_hb ? (uint32_t)T::BLK1 : 0u) + (uint32_t)(LJ * (w & 1)) * 1024u;

  // Producer: fetch(k) finds the request holding tile k, issues the scalar
  // loads of its two block ids and notes how many rows of each block are
  // valid; it runs one tile step ahead of launch(k), which forms the buffer
  // resource of this wave's block (sized to its valid rows), picks the
  // tile's ring slot and records in slot_bad whether a block id of the tile
  // was outside the cache.  The S step then issues this wave's 1 KB loads one
  // at a time (dma_part), so that the memory pipeline takes them while the
  // matrix cores work.  Every tile step launches one tile: past the range's
  // last tile the resource is empty, so the loads deliver zeros into the free
  // image, and every wait counts the same loads.
  Cursor prod;
  prod.b = R.b_first;
  prod.p = R.p_first;
  if (prod.b < a.batch) cursor_load(a, prod);
  int32_t pid[2] = {-1, -1};
  int pnv[2] = {0, 0};
  uint32_t slot_bad = 0;
  auto fetch = [&](int k) {
    while (k >= prod.p + prod.n) {  // k < T, so a request holding it follows
      prod.p += prod.n;
      ++prod.b;
      cursor_load(a, prod);
    }
    const int pkl = k - prod.p;
    const int left = prod.L - 32 * pkl;  // rows of the request from this tile on (> 0)
    const const_i32* row = prod.row + 2 * pkl;
    pid[0] = row[0];
    pnv[0] = left >= 16 ? 16 : left;
    pnv[1] = left >= 32 ? 16 : (left > 16 ? left - 16 : 0);
    pid[1] = pnv[1] > 0 ? row[1] : -1;
  };
  i32x4 lrs;
  uint32_t lbase = 0;
  auto dma_part = [&](int j) { dma16(lrs, lbase + (uint32_t)j * 1024u, vo[j]); };
  auto launch = [&](int k) {
    const bool real = k < t1;
    const bool bad0 = pnv[0] > 0 && (uint32_t)pid[0] >= nb32, bad1 = pnv[1] > 0 && (uint32_t)pid[1] >= nb32;
    const uint32_t badbit = real && (bad0 || bad1) ? 1u : 0u;
    const int32_t id = my_hb ? pid[1] : pid[0];
    const int nv = my_hb ? pnv[1] : pnv[0];
    const bool ok = real && (uint32_t)id < nb32;
    lrs = raw_rsrc(kv + (ok ? (int64_t)(uint32_t)id * (16 * D) : 0), ok ? (uint32_t)(nv * D * 2) : 0u);
    const uint32_t slot = (uint32_t)(k - t0) & (kRing - 1);
    slot_bad = (slot_bad & ~(1u << slot)) | (badbit << slot);
    // Scalar: the M0 base of this wave's loads.
    lbase = __builtin_amdgcn_readfirstlane(ring_base + slot * (uint32_t)T::IMG_BYTES + wave_img);
  };
  // The first kRing - 1 tiles in flight, and the block ids of the next.
  int k_next = t0;
  auto prologue = [&]() {
    for (int s = 0; s < kRing - 1; ++s) {
      if (k_next < t1) fetch(k_next);
      launch(k_next++);
#pragma unroll
      for (int j = 0; j < LJ; ++j) dma_part(j);
    }
    if (k_next < t1) fetch(k_next);
  };
  prologue();

  // Per-lane LDS offsets within a tile image (the swizzle only permutes
  // chunks within aligned groups of 8, so a lane's offset depends on the
  // k-step or column tile modulo a small period plus whole groups).
  // K (A operand of S^T), k-step s: tile row tile_pos(j32), chunk 2 s + h.
  uint32_t k_off[4];
  {
    const int p = tile_pos(j32), r = p & 15;
    const uint32_t blk = (p >> 4) ? (uint32_t)T::BLK1 : 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) k_off[e] = blk + (uint32_t)((r * STRIDE + ((2 * e + h) ^ (r & 7))) * 16);
  }
  // V^T (A operand of O^T), 32-column tile ct, rows of read e in block kh:
  // lane supplies row 8 e + 2 h + {0, 1, 4, 5}[l16 / 4] and the 8 bytes of
  // columns 32 ct + 16 (j32 / 16) + 4 (l16 % 4) .. + 3, and receives column
  // 32 ct + j32 of the four rows.
  uint32_t v_off[2][2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int r = 8 * e + 2 * h + (((l16 >> 2) & 1) | (((l16 >> 2) & 2) << 1));
#pragma unroll
    for (int cp = 0; cp < 2; ++cp) {
      const int chunk = 4 * cp + 2 * (j32 >> 4) + ((l16 & 3) >> 1);
      v_off[e][cp] = (uint32_t)((r * STRIDE + (chunk ^ (r & 7))) * 16 + (l16 & 1) * 8);
    }
  }

  const float sl2 = a.scale * kLog2e;
  uint32_t wflags = 0;
  // This lane's query row, within the workgroup's tile and within the request.
  const int ql = 32 * w + j32;
  const int qr = mt * QT + ql;
  const bool q_ok = qr < a.n_q;

  bf16x8 qf[KS];
  f32x16 acc[NCT];

  // Writes the lane's query row of request b: its value columns
  // 32 ct + 8 (v / 4) + 4 h + v % 4 (acc times inv, or fill_v everywhere) and
  // the LSE, to the final output or to partial slot `pidx` (-1: final).
  auto write_row = [&](int b, float inv, float lse_v, bool fill, float fill_v, int64_t pidx) {
    if (!q_ok) return;
    auto val = [&](int ct, int q) {
      return fill ? f32x4{fill_v, fill_v, fill_v, fill_v}
                  : f32x4{acc[ct][4 * q], acc[ct][4 * q + 1], acc[ct][4 * q + 2], acc[ct][4 * q + 3]} * inv;
    };
    if (pidx < 0) {
      const int64_t orow = (int64_t)b * a.n_q + qr;
      if (a.out_bf16) {
        uint16_t* o = static_cast<uint16_t*>(a.out) + orow * 512 + 4 * h;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 v = val(ct, q);
            *reinterpret_cast<uint2*>(o + 32 * ct + 8 * q) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          }
      } else {
        float* o = static_cast<float*>(a.out) + orow * 512 + 4 * h;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int q = 0; q < 4; ++q) *reinterpret_cast<f32x4*>(o + 32 * ct + 8 * q) = val(ct, q);
      }
      if (h == 0 && a.lse) a.lse[orow] = lse_v;
    } else {
      // A piece is stored in the output's type: bf16 when the final output is
      // bf16 (it is rounded to bf16 anyway), else float32.
      if (a.out_bf16) {
        uint16_t* o = reinterpret_cast<uint16_t*>(a.o_part) + (pidx * QT + ql) * 512 + 4 * h;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 v = val(ct, q);
            *reinterpret_cast<uint2*>(o + 32 * ct + 8 * q) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          }
      } else {
        float* o = a.o_part + (pidx * QT + ql) * 512 + 4 * h;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int q = 0; q < 4; ++q) *reinterpret_cast<f32x4*>(o + 32 * ct + 8 * q) = val(ct, q);
      }
      if (h == 0) a.lse_part[pidx * QT + ql] = lse_v;
    }
  };

  Cursor cons;
  cons.b = R.b_first;
  cons.p = R.p_first;
  for (; cons.b < a.batch; ++cons.b) {
    cursor_load(a, cons);
    if (cons.p >= t1 && !last_range) break;
    const int b = cons.b;
    if (cons.n == 0) {  // empty or invalid request, owned by this range
      write_row(b, 0.f, cons.f ? NAN : -INFINITY, true, cons.f ? NAN : 0.f, -1);
      wflags |= cons.f;
      if (mt == 0 && tid == 0) *reinterpret_cast<i32x4*>(a.req + 4 * (int64_t)b) = i32x4{-1, -1, 0, 0};
      continue;
    }
    const int ka = cons.p > t0 ? cons.p : t0;
    const int ke = cons.p + cons.n < t1 ? cons.p + cons.n : t1;
    const bool first_piece = ka == cons.p;
    const bool whole = first_piece && ke == cons.p + cons.n;
    if (first_piece && mt == 0 && tid == 0) {
      const int g1 = whole ? g : range_of(cons.p + cons.n - 1, R.T, a.G);
      *reinterpret_cast<i32x4*>(a.req + 4 * (int64_t)b) = i32x4{g, g1, cons.p == t0 ? 0 : 1, 0};
    }

    // The lane's query as B operands of S^T: columns 16 s + 8 h .. + 7 of
    // query row qr (zero past n_q); the rows of this request visible to it
    // (its causal horizon), and the fewest any of the wave's valid rows sees:
    // tiles below that need no mask.
    {
      const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.q) +
                                                         ((int64_t)b * a.n_q + (q_ok ? qr : 0)) * D + 8 * h);
#pragma unroll
      for (int s = 0; s < KS; ++s) qf[s] = as_bf16x8(q_ok ? src[2 * s] : u32x4{0u, 0u, 0u, 0u});
    }
    int hz;
    {
      const int64_t hh = q_ok ? held_rows(cons.Lg - a.t_q + qr / a.n_head + 1, a.dcp_world, a.dcp_rank,
                                          a.dcp_interleave)
                              : 0;
      hz = (int)(hh < cons.L ? hh : cons.L);
    }
    int hz_min = q_ok ? hz : INT32_MAX;
    for (int off = 32; off > 0; off >>= 1) {
      const int o = __shfl_xor(hz_min, off, 64);
      hz_min = o < hz_min ? o : hz_min;
    }
    hz_min = __builtin_amdgcn_readfirstlane(hz_min);
    // The query loads are the only vector-memory loads the compiler tracks in
    // this loop: wait for them here (with every tile load issued so far), so it
    // does not put a full wait before every tile's first product.
    wait_vmcnt<0>();

    // Softmax with a fixed reference per pass (log2 units): m_ref is the
    // maximum of the first tile with a visible row, and later tiles may exceed
    // it by up to kLimit (probabilities up to 2^kLimit: bf16 and float32 share
    // the exponent range, so nothing overflows and relative precision is
    // unchanged).  The accumulators are then touched by the matrix products
    // alone.  If a tile goes past the limit, the workgroup streams the piece a
    // second time with the piece's true maximum as the reference.
    float m_ref = -INFINITY, m_hi = -INFINITY, lsum = 0.f;
    bool bad = false;
    for (int pass = 0;; ++pass) {
      lsum = 0.f;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) acc[ct] = f32x16{};
      bool over = false;

      for (int k = ka; k < ke; ++k) {
        // Tile k resident: this wave's loads of it are done once at most the
        // loads of the two tiles issued after it are outstanding (the first
        // tile of a pass was waited for before the loop).
        if (k != ka) wait_vmcnt<2 * LJ>();
        barrier_keep_loads();  // tile k visible to all waves; tile k - 1 no longer read
        const int kl = k - cons.p;
        const uint32_t slot = (uint32_t)(k - t0) & (kRing - 1);
        if ((slot_bad >> slot) & 1u) bad = true;
        const uint32_t img = ring_base + slot * (uint32_t)T::IMG_BYTES;

        // S^T of the tile (32 rows x the wave's 32 queries), one product per
        // 16-wide k-step s, K read kAhead steps ahead and waited for two at a
        // time.  The scalar work of the producer runs among the first
        // products (launch of tile k + 3 in step 0, the block ids of the tile
        // after it in step 2), and this wave's loads of tile k + 3 go out one
        // per odd step (zero-size past the range's last tile).
        f32x16 sacc;
        {
          constexpr int kAhead = kKAhead;
          constexpr int DSTEP = KS / 2 / LJ;  // two-read steps between two tile loads
          static_assert(kAhead % 2 == 0 && KS % 2 == 0 && DSTEP >= 1 && LJ * DSTEP <= KS / 2, "S step plan");
          // k-step s: chunk 2 s + h, i.e. lane offset k_off[s % 4] plus 128 (s / 4) bytes.
          const uint32_t kaddr[4] = {img + k_off[0], img + k_off[1], img + k_off[2], img + k_off[3]};
          u32x4 kr[KS];
          [&]<int... I>(std::integer_sequence<int, I...>) {
            (lds_b128<128 * (I / 4)>(kaddr[I % 4], kr[I]), ...);
          }(std::make_integer_sequence<int, kAhead>{});
          [&]<int... J>(std::integer_sequence<int, J...>) {
            (([&] {
               constexpr int I = 2 * J;
               constexpr int issued = I + kAhead < KS ? I + kAhead : KS;
               lgkm_wait<issued - 2 - I>(kr[I], kr[I + 1]);
               if constexpr (I == 0)
                 mfma_vacc_first(sacc, as_bf16x8(kr[I]), qf[I]);
               else
                 mfma_vacc(sacc, as_bf16x8(kr[I]), qf[I]);
               mfma_vacc(sacc, as_bf16x8(kr[I + 1]), qf[I + 1]);
               if constexpr (I + kAhead < KS) {
                 constexpr int P = I + kAhead;
                 lds_b128<128 * (P / 4)>(kaddr[P % 4], kr[P]);
                 lds_b128<128 * ((P + 1) / 4)>(kaddr[(P + 1) % 4], kr[P + 1]);
               }
               if constexpr (J == 0) launch(k_next++);
               if constexpr (J == 2) {
                 if (k_next < t1) fetch(k_next);  // block ids of the tile the next step issues
               }
               if constexpr (J % DSTEP == DSTEP / 2 && J / DSTEP < LJ) dma_part(J / DSTEP);
               __builtin_amdgcn_sched_barrier(0);
             }()),
             ...);
          }(std::make_integer_sequence<int, KS / 2>{});
        }

        mfma_vacc_drain(sacc);

        // Softmax of the lane's query over its 16 tile rows (element v is tile
        // position 8 (v / 4) + 2 h + {0, 1, 4, 5}[v % 4]; the other 16 rows sit
        // in lane ^ 32).  Rows past a query's horizon are masked, on the tiles
        // that reach past the wave's smallest horizon only.
        if (32 * kl + 32 > hz_min) {
          const int base = 32 * kl + 2 * h;
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (base + 8 * (v >> 2) + ((v & 1) | ((v & 2) << 1)) >= hz) sacc[v] = -INFINITY;
        }
        bf16x8 pB[2];
        {
          float tmax = sacc[0];
#pragma unroll
          for (int v = 1; v < 16; ++v) tmax = fmaxf(tmax, sacc[v]);
          {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
            tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
          }
          tmax *= sl2;
          m_hi = fmaxf(m_hi, tmax);
          if (m_ref == -INFINITY) m_ref = tmax;
          over |= tmax > m_ref + kLimit;
          const float nm = m_ref == -INFINITY ? 0.f : -m_ref;
          float pr[16];
#pragma unroll
          for (int v = 0; v < 16; ++v) pr[v] = __builtin_amdgcn_exp2f(fmaf(sacc[v], sl2, nm));
          float ps = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) ps += (pr[4 * q] + pr[4 * q + 1]) + (pr[4 * q + 2] + pr[4 * q + 3]);
          lsum += ps;
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
            pB[kh] = as_bf16x8(u32x4{pack_bf16x2(pr[8 * kh], pr[8 * kh + 1]), pack_bf16x2(pr[8 * kh + 2], pr[8 * kh + 3]),
                                     pack_bf16x2(pr[8 * kh + 4], pr[8 * kh + 5]), pack_bf16x2(pr[8 * kh + 6], pr[8 * kh + 7])});
        }

        // O^T += V^T P^T over the two 16-row halves (blocks) of the tile: the
        // k-slots 8 h + t of half kh are tile positions 16 kh + 8 (t / 4) + 2 h +
        // {0, 1, 4, 5}[t % 4], the rows of the two transposing reads e = t / 4.
        // V^T read kAhead column tiles ahead and waited for one column tile
        // (four reads) at a time.
        {
          constexpr int kAhead = kVAhead;
          uint2 vr[NCT][2][2];  // [ct][kh][e]
          auto vread = [&]<int CT>(std::integral_constant<int, CT>) {
            constexpr uint32_t cofs = 128u * (CT / 2);
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
              for (int e = 0; e < 2; ++e) {
                if (kh == 0)
                  lds_tr_b64<cofs>(img + v_off[e][CT % 2], vr[CT][kh][e]);
                else
                  lds_tr_b64<cofs + T::BLK1>(img + v_off[e][CT % 2], vr[CT][kh][e]);
              }
          };
          [&]<int... I>(std::integer_sequence<int, I...>) {
            (vread(std::integral_constant<int, I>{}), ...);
          }(std::make_integer_sequence<int, kAhead>{});
          [&]<int... I>(std::integer_sequence<int, I...>) {
            (([&] {
               constexpr int issued = I + kAhead < NCT ? I + kAhead : NCT;
               lgkm_wait<4 * (issued - 1 - I)>(vr[I][0][0], vr[I][0][1], vr[I][1][0], vr[I][1][1]);
#pragma unroll
               for (int kh = 0; kh < 2; ++kh) {
                 const bf16x8 vA = as_bf16x8(u32x4{vr[I][kh][0].x, vr[I][kh][0].y, vr[I][kh][1].x, vr[I][kh][1].y});
                 acc[I] = mfma32x32x16(vA, pB[kh], acc[I]);
               }
               if constexpr (I + kAhead < NCT) vread(std::integral_constant<int, I + kAhead>{});
               __builtin_amdgcn_sched_barrier(0);
             }()),
             ...);
          }(std::make_integer_sequence<int, NCT>{});
        }
      }

      // Every wave votes; a second pass if any query row of the workgroup
      // needs one (the tile loads are shared, so all waves go again).
      if (pass > 0) break;
      {
        // The ballot with every lane active (inside the lane-0 branch it
        // would see lane 0 alone).
        const int any_over = __ballot(over) != 0 ? 1 : 0;
        if (lane == 0) vote[w] = any_over;
      }
      barrier_keep_loads();
      int redo = 0;
#pragma unroll
      for (int i = 0; i < kWaves; ++i) redo |= vote[i];
      if (!redo) break;
      // Rewind the producer to the piece's first tile: drain the loads in
      // flight, wait until no wave reads the ring, and issue the first tiles
      // again; the second pass uses each row's maximum over the piece.
      wait_vmcnt<0>();
      barrier_keep_loads();
      prod.b = cons.b;
      prod.p = cons.p;
      cursor_load(a, prod);
      k_next = ka;
      prologue();
      wait_vmcnt<2 * LJ>();
      m_ref = m_hi;
    }

    // Finish the piece: 1 / l and the LSE of the lane's query (l summed over
    // its two lanes), then the final output or a partial slot.
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
      const float l = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const float lse_v = bad ? NAN : (l > 0.f ? (m_ref + __log2f(l)) * kLn2 : -INFINITY);
      if (bad) wflags |= kBadBlock;
      const int64_t pidx = whole ? -1 : ((int64_t)g * a.m_tiles + mt) * 2 + (cons.p <= t0 ? 0 : 1);
      write_row(b, inv, lse_v, bad, NAN, pidx);
    }
    cons.p += cons.n;
  }
  if (tid == 0) a.status[(int64_t)g * a.m_tiles + mt] = wflags;
}

// ---------------------------------------------------------------------------
// Merge of the pieces of the requests cut by range ends.  W waves per query
// row (one row per workgroup when W > 1, else kMergeRows rows of one wave):
// wave v sums the contiguous pieces [v P / W, (v + 1) P / W) of the row's P
// pieces, and the wave sums are added in wave order through LDS, so the result
// does not depend on timing.  Lane l owns value columns 4 l .. + 3 and
// 256 + 4 l .. + 3.  Pieces are read eight at a time.
// ---------------------------------------------------------------------------
constexpr int kMergeRows = 4;

// Four bf16 values (two packed pairs, low half first) widened to float32.
__device__ __forceinline__ f32x4 bf16x4_to_f32(uint2 v) {
  return f32x4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
               __uint_as_float(v.y & 0xffff0000u)};
}

__device__ __forceinline__ float wmax(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wsum(float v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int W>
__global__ __launch_bounds__(64 * (W > 1 ? W : kMergeRows)) void decode_flat_merge(const FlatArgs a) {
  __shared__ float red[W > 1 ? W : 1][2];
  __shared__ __attribute__((aligned(16))) f32x4 part[W > 1 ? W : 1][2][64];
  const int lane = threadIdx.x & 63, v = threadIdx.x >> 6;
  const int64_t qrow = W > 1 ? (int64_t)blockIdx.x : (int64_t)blockIdx.x * kMergeRows + v;
  if (qrow >= (int64_t)a.batch * a.n_q) return;
  const int b = (int)(qrow / a.n_q);
  const int q = (int)(qrow - (int64_t)b * a.n_q);
  const i32x4 info = *reinterpret_cast<const i32x4*>(a.req + 4 * (int64_t)b);
  const int g0 = info[0], g1 = info[1], s0 = info[2];
  if (g0 < 0 || g0 == g1) return;  // written by the split kernel
  const int mt = q / a.qt, ql = q - mt * a.qt;
  const int P = g1 - g0 + 1;
  auto pidx = [&](int k) { return ((int64_t)(g0 + k) * a.m_tiles + mt) * 2 + (k == 0 ? s0 : 0); };
  auto lse_of = [&](int k) { return a.lse_part[pidx(k) * a.qt + ql]; };

  if (W == 1 && P <= 8) {
    // Up to eight pieces: every load (the pieces' LSEs, one per lane, and
    // their outputs, lane l owning columns 8 l .. 8 l + 7) goes out at once,
    // then the weights.  Pieces are added in index order.
    const float ls = lane < P ? lse_of(lane) : -INFINITY;
    f32x4 xa[8], xb[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      xa[u] = xb[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (u < P) {
        const int64_t base = (pidx(u) * a.qt + ql) * 512 + 8 * lane;
        if (a.out_bf16) {
          const uint4 r = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.o_part) + base);
          xa[u] = bf16x4_to_f32(uint2{r.x, r.y});
          xb[u] = bf16x4_to_f32(uint2{r.z, r.w});
        } else {
          xa[u] = *reinterpret_cast<const f32x4*>(a.o_part + base);
          xb[u] = *reinterpret_cast<const f32x4*>(a.o_part + base + 4);
        }
      }
    }
    const float M = wmax(ls);
    const bool any_nan = __ballot(isnan(ls)) != 0;
    float wtot = 0.f;
    f32x4 oa = {0.f, 0.f, 0.f, 0.f}, ob = oa;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float lu = __shfl(ls, u, 64);
      const bool live = u < P && lu != -INFINITY && M != -INFINITY;  // an empty piece may hold anything
      const float wgt = live ? __expf(lu - M) : 0.f;
      wtot += wgt;
      oa += wgt * (live ? xa[u] : f32x4{0.f, 0.f, 0.f, 0.f});
      ob += wgt * (live ? xb[u] : f32x4{0.f, 0.f, 0.f, 0.f});
    }
    const float inv = wtot > 0.f ? 1.f / wtot : 0.f;
    const f32x4 nan4 = {NAN, NAN, NAN, NAN};
    const f32x4 ra = any_nan ? nan4 : oa * inv, rb = any_nan ? nan4 : ob * inv;
    if (a.out_bf16) {
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + qrow * 512 + 8 * lane) =
          uint4{pack_bf16x2(ra[0], ra[1]), pack_bf16x2(ra[2], ra[3]), pack_bf16x2(rb[0], rb[1]), pack_bf16x2(rb[2], rb[3])};
    } else {
      float* o = static_cast<float*>(a.out) + qrow * 512 + 8 * lane;
      *reinterpret_cast<f32x4*>(o) = ra;
      *reinterpret_cast<f32x4*>(o + 4) = rb;
    }
    if (lane == 0 && a.lse) a.lse[qrow] = any_nan ? NAN : (M == -INFINITY ? -INFINITY : M + __logf(wtot));
    return;
  }

  const int wv = W > 1 ? v : 0;
  const int k0 = (int)((int64_t)P * wv / W), k1 = (int)((int64_t)P * (wv + 1) / W);
  // Maximum LSE and NaN over all pieces (every wave scans all of them).
  float mx = -INFINITY;
  bool nan_seen = false;
  for (int k = lane; k < P; k += 64) {
    const float x = lse_of(k);
    nan_seen |= isnan(x);
    mx = fmaxf(mx, x);
  }
  const float M = wmax(mx);
  const bool any_nan = __ballot(nan_seen) != 0;
  float wp = 0.f;
  if (M != -INFINITY)
    for (int k = lane; k < P; k += 64) {
      const float x = lse_of(k);
      wp += x == -INFINITY ? 0.f : __expf(x - M);
    }
  const float wtot = wsum(wp);
  const float inv = wtot > 0.f ? 1.f / wtot : 0.f;

  f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = o0;
  if (M != -INFINITY) {
    for (int k = k0; k < k1; k += 8) {
      float wk[8];
      f32x4 x0[8], x1[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int kk = k + u < k1 ? k + u : k1 - 1;
        const int64_t base = (pidx(kk) * a.qt + ql) * 512;
        wk[u] = lse_of(kk);
        if (a.out_bf16) {
          const uint16_t* op = reinterpret_cast<const uint16_t*>(a.o_part) + base;
          x0[u] = bf16x4_to_f32(*reinterpret_cast<const uint2*>(op + 4 * lane));
          x1[u] = bf16x4_to_f32(*reinterpret_cast<const uint2*>(op + 256 + 4 * lane));
        } else {
          x0[u] = *reinterpret_cast<const f32x4*>(a.o_part + base + 4 * lane);
          x1[u] = *reinterpret_cast<const f32x4*>(a.o_part + base + 256 + 4 * lane);
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool live = k + u < k1 && wk[u] != -INFINITY;  // an empty piece may hold anything
        const float wgt = live ? __expf(wk[u] - M) : 0.f;
        o0 += wgt * (live ? x0[u] : f32x4{0.f, 0.f, 0.f, 0.f});
        o1 += wgt * (live ? x1[u] : f32x4{0.f, 0.f, 0.f, 0.f});
      }
    }
  }
  if constexpr (W > 1) {
    part[v][0][lane] = o0;
    part[v][1][lane] = o1;
    __syncthreads();
    if (v != 0) return;
    o0 = o1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < W; ++i) {
      o0 += part[i][0][lane];
      o1 += part[i][1][lane];
    }
  }
  const f32x4 nan4 = {NAN, NAN, NAN, NAN};
  const f32x4 r0 = any_nan ? nan4 : o0 * inv, r1 = any_nan ? nan4 : o1 * inv;
  if (a.out_bf16) {
    uint16_t* o = static_cast<uint16_t*>(a.out) + qrow * 512;
    *reinterpret_cast<uint2*>(o + 4 * lane) = uint2{pack_bf16x2(r0[0], r0[1]), pack_bf16x2(r0[2], r0[3])};
    *reinterpret_cast<uint2*>(o + 256 + 4 * lane) = uint2{pack_bf16x2(r1[0], r1[1]), pack_bf16x2(r1[2], r1[3])};
  } else {
    float* o = static_cast<float*>(a.out) + qrow * 512;
    *reinterpret_cast<f32x4*>(o + 4 * lane) = r0;
    *reinterpret_cast<f32x4*>(o + 256 + 4 * lane) = r1;
  }
  if (lane == 0 && a.lse) a.lse[qrow] = any_nan ? NAN : (M == -INFINITY ? -INFINITY : M + __logf(wtot));
  (void)red;
}

}  // namespace

bool flat_supported(int kv_rank, int d_rope, bool bf16) { return bf16 && kv_rank == 512 && (d_rope == 0 || d_rope == 64); }

int64_t flat_auto_ranges(int n_head, int batch, int t_q, int max_blocks, int cus) {
  const int n_q = t_q * n_head;
  const int m_tiles = (n_q + 127) / 128;
  int64_t G = cus / m_tiles;
  if (G < 1) G = 1;
  const int64_t max_tiles = (int64_t)(batch > 0 ? batch : 1) * ((max_blocks + 1) / 2);
  return G < max_tiles ? G : max_tiles;
}

FlatPlan flat_plan(int n_head, int d_rope, int batch, int t_q, int max_blocks, int64_t ranges) {
  (void)d_rope;
  FlatPlan p = {};
  const int64_t n_q = (int64_t)t_q * n_head;
  // 128 query rows per workgroup (four waves of 32); the query tiles of one
  // range share an XCD, so a cache tile is fetched from HBM once and from L2
  // by the rest.
  p.qb = kWaves;  // waves per workgroup
  p.qt = 32 * kWaves;
  p.m_tiles = (int)((n_q + p.qt - 1) / p.qt);
  const int64_t G = ranges < 1 ? 1 : ranges;
  // Device arithmetic: tile positions t < T <= batch * ceil(max_blocks / 2) in
  // 32 bits ((t + 1) * G in 64), and workgroup and slot counts in 32 bits.
  const int64_t max_tiles = (int64_t)(batch > 0 ? batch : 1) * ((max_blocks + 1) / 2);
  const int64_t wgs = (G + 7) / 8 * 8 * p.m_tiles;
  p.ok = G <= (1 << 24) && max_tiles <= (int64_t)(INT32_MAX / 2) && wgs <= INT32_MAX;
  if (!p.ok) return p;
  p.G = (int)G;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t n_status = (size_t)G * p.m_tiles;
  p.req_off = al(kHeaderBytes + n_status * 4);
  p.lse_off = al(p.req_off + (size_t)(batch > 0 ? batch : 1) * 16);
  const size_t slots = (size_t)G * p.m_tiles * 2 * p.qt;
  p.o_off = al(p.lse_off + slots * 4);
  p.bytes = al(p.o_off + slots * 512 * 4);
  return p;
}

hipError_t launch_decode_flat(const FlatArgs& a, int d_rope, int qb, hipStream_t stream) {
  const int grid = (a.G + 7) / 8 * 8 * a.m_tiles;
  if (qb != kWaves) return hipErrorInvalidValue;
  if (d_rope == 64)
    hipLaunchKernelGGL(decode_flat_mfma<64>, dim3(grid), dim3(64 * kWaves), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_flat_mfma<0>, dim3(grid), dim3(64 * kWaves), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.batch == 0 || a.G == 1) return e;
  const int64_t rows = (int64_t)a.batch * a.n_q;
  if (rows > INT32_MAX) return hipErrorInvalidConfiguration;
  // Many pieces per request on average: one 16-wave workgroup per row.
  if ((int64_t)a.G >= 32 * (int64_t)a.batch) {
    hipLaunchKernelGGL(decode_flat_merge<16>, dim3((unsigned)rows), dim3(64 * 16), 0, stream, a);
  } else {
    hipLaunchKernelGGL(decode_flat_merge<1>, dim3((unsigned)((rows + kMergeRows - 1) / kMergeRows)),
                       dim3(64 * kMergeRows), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace mla
