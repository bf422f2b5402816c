// Split-KV paged MLA decode attention and the LSE-weighted merge, for gfx950.
//
// What is computed (vllm.cpp "cpu_mla_attn.cpp", MlaDecodeAttentionKernel;
// memra-engine "mla.rs", MlaInputs causal rule): for request b, query i and
// head h, scores s_j = scale * <q_abs, row_j> over the full latent row
// [c_kv | k_pe], softmax over the visible rows j < L - t_q + i + 1, output the
// softmax-weighted sum of the leading kv_rank columns of the same rows, and
// lse = log sum_j exp(s_j).
//
// Schedule.  The rows of a request are cut into `splits` ranges of whole cache
// blocks.  One workgroup of eight waves handles one (request, range, tile of 64
// query rows) and walks its range 32 rows (two 16-row cache blocks) at a time:
//   * blocks go HBM -> LDS directly (buffer_load ... lds), one buffer resource
//     per block, so rows past the request's end read as zeros and no address
//     outside a real block is formed; a ring of three tile buffers keeps the
//     next tile loading while one is consumed;
//   * wave (qh, dq) computes the partial S^T = K Q^T of query rows
//     [32 qh, 32 qh + 32) over its quarter dq of the row width with 16x16x32
//     bf16 MFMA, the K operand read as two 8-byte LDS reads per lane;
//   * the partials are summed through LDS so that each wave owns eight query
//     rows for the online softmax; it publishes bf16 P^T, already in the
//     B-operand layout of O^T = V^T P^T, and the per-query rescale factor;
//   * wave (qh, dq) then accumulates output columns [128 dq, 128 dq + 128) of
//     its 32 query rows, reading V^T from the same LDS tile with the
//     transposing ds_read_b64_tr_b16; this PV step of tile t runs in the same
//     phase as the softmax of tile t + 1 (P^T and the rescale factors are
//     double-buffered by tile parity).
// Two waves share each SIMD, so one wave's LDS reads overlap the other's MFMAs.
// With one range per request the workgroup writes the final output and LSE;
// otherwise it writes (o, lse) partials and decode_merge combines them:
//   M = max_s lse_s, w_s = exp(lse_s - M), o = sum w_s o_s / sum w_s,
//   lse = M + log sum w_s  (all -inf: zeros and -inf).
#include "decode_common.hpp"
#include "kernels.hpp"

#include <math.h>
#include <type_traits>
#include <utility>

namespace mla {
namespace {

// XCD-aware decode of the linear workgroup id (workgroup i runs on XCD i % 8,
// each XCD with its own L2).  With a batch that is a multiple of 8, every
// workgroup of request b -- all its ranges and query tiles -- lands on XCD
// b % 8: the request's queries are fetched into one L2 only, and its split
// partials are written to the L2 the merge of request b reads them from.
// Otherwise the m-tiles that share one (request, range), and so read the same
// cache blocks, land on the same XCD.
__device__ __forceinline__ bool decode_item(const DecodeArgs& a, int& b, int& s, int& mt, int& item) {
  const int lin = blockIdx.x;
  const int p_lo = lin & 7;
  const int rest = lin >> 3;
  if (a.batch % 8 == 0) {
    const int per_b = a.splits * a.m_tiles;
    const int bg = rest / per_b;
    const int r2 = rest - bg * per_b;
    b = bg * 8 + p_lo;
    s = r2 / a.m_tiles;
    mt = r2 - s * a.m_tiles;
    if (b >= a.batch) return false;
    item = (b * a.splits + s) * a.m_tiles + mt;
    return true;
  }
  mt = rest % a.m_tiles;
  const int pair = (rest / a.m_tiles) * 8 + p_lo;
  if (pair >= a.n_pairs) return false;
  b = pair / a.splits;
  s = pair - b * a.splits;
  item = pair * a.m_tiles + mt;
  return true;
}

__device__ __forceinline__ void write_header(const DecodeArgs& a) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.header[0] = kWorkspaceMagic;
    a.header[1] = (uint32_t)a.n_items;
    a.header[2] = (uint32_t)a.splits;
    a.header[3] = (uint32_t)a.batch;
  }
}




// Two 8-byte LDS reads at lds_addr + OFF and + OFF + 32, as separate
// ds_read_b64 instructions (the compiler would pair them into one
// ds_read2_b64, which this access pattern serves markedly slower).  The
// results are not ready until a matching lgkm_wait.
template <int OFF>
__device__ __forceinline__ void lds_read_b64x2(uint32_t lds_addr, uint2& lo, uint2& hi) {
  asm volatile("ds_read_b64 %0, %2 offset:%3\n\tds_read_b64 %1, %2 offset:%4"
               : "=v"(lo), "=v"(hi)
               : "v"(lds_addr), "i"(OFF), "i"(OFF + 32)
               : "memory");
}
// Wait until at most N (< 16) of this wave's LDS operations are outstanding;
// the two registers are tied to the wait so their uses cannot move above it.
template <int N>
__device__ __forceinline__ void lgkm_wait(uint2& a, uint2& b) {
  static_assert(N >= 0 && N < 16, "lgkmcnt is four bits");
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "i"(N) : "memory");
}

// ---------------------------------------------------------------------------
// MFMA split kernel: bf16 queries and cache, kv_rank 512, rope width D_ROPE.
// ---------------------------------------------------------------------------
template <int D_ROPE>
struct Tile {
  static constexpr int KV = 512;
  static constexpr int D = KV + D_ROPE;
  static constexpr int CH = D / 8;                         // 16-byte chunks per row
  static constexpr int STRIDE = CH + 2;                    // LDS row pitch in chunks: 8 * odd dwords
  static constexpr int BLK_POS = 16 * STRIDE;              // chunk slots of one block image
  static constexpr int BLK_IMG = (BLK_POS + 63) / 64 * 64; // whole wave-loads per block
  static constexpr int BLK_LOADS = BLK_IMG / 64;
  static constexpr int IMG = 2 * BLK_IMG;                  // one 32-row tile
  static constexpr int TILE_LOADS = 2 * BLK_LOADS;         // 1 KB wave-loads per tile
  static constexpr int LOADER_LOADS = (TILE_LOADS + 3) / 4;  // per loading wave and tile (at most)
  static constexpr int KSTEPS = D / 32;                    // 32-wide k-steps of S
  static constexpr int KQ = (KSTEPS + 3) / 4;              // k-steps of the largest D quarter
  static constexpr int CT = 8;                             // 16-column output tiles per quarter
  static_assert((STRIDE * 4) % 16 == 8, "row pitch must be 8 * odd dwords");
  static_assert(KSTEPS >= 16 && KSTEPS <= 20, "four k-steps per quarter plus a partial fifth");
};

template <int D_ROPE>
__global__ __launch_bounds__(512, 1) void decode_split_mfma(const DecodeArgs a) {
  using T = Tile<D_ROPE>;
  constexpr int D = T::D, CH = T::CH, STRIDE = T::STRIDE, KQ = T::KQ, CT = T::CT;
  // Exchange planes are 64 lanes x 8 bytes, padded to 576 bytes so that the
  // softmax-layout reads (8 lanes per 64-byte run, runs 128 bytes apart,
  // consecutive planes) spread over all banks.
  constexpr int PLANE = 72;  // plane pitch in 8-byte units
  __shared__ __attribute__((aligned(16))) u32x4 ring[3 * T::IMG];  // three tile buffers
  __shared__ __attribute__((aligned(16))) uint2 xs[8][2][4][PLANE];  // S partials [wave][half][n * 2 + rt][lane]
  __shared__ __attribute__((aligned(16))) uint2 pb[2][2][2][2][PLANE];  // bf16 P^T [parity][qh][n][rt][lane]
  __shared__ float al[2][64];                                          // per-query rescale [parity][query]
  __shared__ float fin[64];                                          // per-query 1 / l at the end
  __shared__ uint32_t wflags[8];                                     // data-error bits seen by each wave

  write_header(a);
  int b, s, mt, item;
  if (!decode_item(a, b, s, mt, item)) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  // Query half and D / column quarter.  Waves 0-3 (one per SIMD) take the two
  // quarters with one k-step fewer and issue every tile load; their SIMD
  // partners 4-7 take the longer quarters and start on the matrix work at
  // once, so one wave's wait on the load address unit overlaps the other's
  // MFMAs.
  const int qh = w & 1, dq = ((w >> 1) + 2) & 3;
  auto wave_of = [](int h, int d) { return h + 2 * ((d + 2) & 3); };  // wave holding (qh, dq)
  const int l16 = lane & 15, g = lane >> 4;

  // Lengths count global rows; L and the query horizons count the rows this
  // rank holds (all of them on a single rank).
  const int64_t Lg = a.seq_lens[b];
  const int64_t L = held_rows(Lg, a.dcp_world, a.dcp_rank, a.dcp_interleave);
  uint32_t flags = request_flags(Lg, L, a.t_q, a.max_blocks);
  const int64_t r_begin = (int64_t)s * a.chunk_blocks * 16;
  int64_t r_end = r_begin + (int64_t)a.chunk_blocks * 16;
  if (flags || r_end > L) r_end = flags ? r_begin : L;
  const int n_tiles = r_end > r_begin ? (int)((r_end - r_begin + 31) / 32) : 0;

  // Matrix layout: lane (l16, g) of query tile n works on query row
  // 32 qh + 16 n + l16 of the workgroup's 64.
  int q_row[2];
  bool q_ok[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    q_row[n] = mt * kQRowsPerWG + 32 * qh + 16 * n + l16;
    q_ok[n] = q_row[n] < a.n_q;
  }
  // Softmax layout: lane (qi, rt, g) = bits (0..2, 3, 4..5) owns query row
  // fq = 32 qh + 16 (dq / 2) + 8 (dq % 2) + qi and tile rows 16 rt + 4 g + i.
  const int qi = lane & 7, rt_f = (lane >> 3) & 1, g_f = lane >> 4;
  const int nf = dq >> 1, hf = dq & 1;
  const int fq = 32 * qh + 16 * nf + 8 * hf + qi;
  const int src_lane = g_f * 16 + 8 * hf + qi;  // same query and rows in the matrix layout
  int vis_lim;
  {
    const int qr = mt * kQRowsPerWG + fq;
    const bool ok = qr < a.n_q;
    const int64_t horizon =
        held_rows(Lg - a.t_q + (ok ? qr / a.n_head : 0) + 1, a.dcp_world, a.dcp_rank, a.dcp_interleave);
    const int64_t vis_end = horizon < r_end ? horizon : r_end;
    vis_lim = !ok || vis_end <= r_begin ? 0 : (int)(vis_end - r_begin);
  }

  // B operand of S^T for this wave's k-steps kk = dq + 4 j.  The lane's eight
  // k slots are columns 32 kk + 4 g + {0..3} and 32 kk + 16 + 4 g + {0..3}: the
  // K operand is then two 8-byte LDS reads per lane, 32 bytes apart.
  const int nk = (T::KSTEPS - dq + 3) / 4;
  bf16x8 qf[2][KQ];
  const float sl2 = a.scale * kLog2e;

  f32x4 acc[CT][2];
#pragma unroll
  for (int c = 0; c < CT; ++c) acc[c][0] = acc[c][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m2 = -INFINITY, lsum = 0.f;  // softmax state of query fq (log2 units)

  const uint16_t* kv = static_cast<const uint16_t*>(a.kv);
  const int32_t* bt_row = a.bt + (int64_t)b * a.max_blocks;

  // Block ids come from the table through scalar loads (which do not touch
  // the vector-memory counter the tile waits use), fetched one phase before
  // they are needed.  Tile t uses range-relative slots 2t and 2t + 1.
  const int slot0 = s * a.chunk_blocks;
  const int nslots = (int)((r_end - r_begin + 15) / 16);
  // (The table is read-only for the whole call, so the scalar cache may hold it.)
  typedef __attribute__((address_space(4))) const int32_t const_i32;
  const_i32* bt_s = (const_i32*)(bt_row + slot0);
  auto tile_ids = [&](int t, int32_t* ids) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int rel = 2 * t + hb;
      ids[hb] = rel < nslots ? bt_s[rel] : -1;
    }
  };

  // The 1 KB wave-loads of a tile image are issued by waves 0-3: load
  // u = w + 4 j covers chunk slots [64 u, 64 u + 64) of the image, i.e. block
  // u / BLK_LOADS.  Rows 8..15 of a block swap the two 16-byte chunks of each
  // 32-byte pair (bank spreading); slots past a row's end are padding.
  const bool loader = w < 4;
  auto tile_voff = [&](int u) {  // global byte offset (within its block) of this lane's slot of load u
    const int hb = u / T::BLK_LOADS;
    const int pos = (u - hb * T::BLK_LOADS) * 64 + lane;
    const int rl = pos / STRIDE;
    const int cp = pos - rl * STRIDE;
    return (rl < 16 && cp < CH) ? (uint32_t)(rl * D + ((cp ^ ((rl >> 3) & 1)) * 8)) * 2u : 0x7ffffff0u;
  };
  uint32_t voffs[T::LOADER_LOADS];
#pragma unroll
  for (int j = 0; j < T::LOADER_LOADS; ++j) voffs[j] = tile_voff(w + 4 * j);
  int c_w = 0;  // this wave's loads of a prologue tile (for the vmcnt waits)
#pragma unroll
  for (int j = 0; j < (T::TILE_LOADS + 7) / 8; ++j) c_w += w + 8 * j < T::TILE_LOADS ? 1 : 0;

  // Issue the loads of tile t (block ids `ids`) into `dst`.  All bounds are
  // 32-bit scalar arithmetic (a range never holds 2^31 rows, a cache never
  // 2^31 blocks), and which block a load belongs to is known at compile time
  // except for the one load that straddles the two blocks.
  const int range_rows = (int)(r_end - r_begin);
  const uint32_t nb32 = a.num_blocks < (int64_t)INT32_MAX ? (uint32_t)a.num_blocks : (uint32_t)INT32_MAX;
  // In the loop only waves 0-3 issue tile loads (u = w + 4 j, offsets voffs);
  // the two tiles of the prologue are split over all eight waves
  // (u = w + 8 j, offsets computed on the spot), so that they go out at once.
  auto issue_tile = [&](int t, const int32_t* ids, u32x4* dst, auto all8) {
    constexpr bool ALL8 = decltype(all8)::value;
    if (!ALL8 && !loader) return;
    i32x4 rs[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int32_t id = ids[hb];
      const int left = range_rows - 32 * t - 16 * hb;
      const int nvalid = left <= 0 ? 0 : (left >= 16 ? 16 : left);
      const bool ok = (uint32_t)id < nb32;
      if (nvalid > 0 && !ok) flags |= kBadBlock;
      rs[hb] = raw_rsrc(kv + (int64_t)(ok ? id : 0) * (16 * D), ok ? (uint32_t)(nvalid * D * 2) : 0u);
    }
    const uint32_t lbase = lds_addr(dst);
    if constexpr (ALL8) {
#pragma unroll
      for (int j = 0; j < (T::TILE_LOADS + 7) / 8; ++j) {
        const int u = w + 8 * j;
        if (u < T::TILE_LOADS) dma16(u < T::BLK_LOADS ? rs[0] : rs[1], lbase + (uint32_t)u * 1024u, tile_voff(u));
      }
    } else {
#pragma unroll
      for (int j = 0; j < T::LOADER_LOADS; ++j) {
        const int u = w + 4 * j;
        const bool in_tile = 4 * j + 3 < T::TILE_LOADS || u < T::TILE_LOADS;
        const bool blk0 = 4 * j + 3 < T::BLK_LOADS || (4 * j < T::BLK_LOADS && u < T::BLK_LOADS);
        if (in_tile) dma16(blk0 ? rs[0] : rs[1], lbase + (uint32_t)u * 1024u, voffs[j]);
      }
    }
  };
  using all_waves = std::true_type;
  using loader_waves = std::false_type;

  // Per-lane LDS byte offsets within a tile image.  Tile row r, chunk c lives
  // at chunk slot (r / 16) * BLK_IMG + (r % 16) * STRIDE + (c ^ sw) with
  // sw = ((r % 16) >> 3) & 1, which only flips bit 0 of the chunk.
  // K (A operand of S^T), k-step kk, block rt: row l16, bytes 64 kk + 8 g and +32.
  const int sw_k = (l16 >> 3) & 1;
  const int k_off = (l16 * STRIDE + ((g >> 1) ^ sw_k)) * 16 + (g & 1) * 8 + 64 * dq;
  // V^T (A operand of O^T) for column tile ct of quarter dq: rows rr and 16 + rr,
  // columns 128 dq + 16 ct + 4 (l16 % 4) .. + 3.
  const int rr = 4 * g + (l16 >> 2);
  const int sw_v = (rr >> 3) & 1;
  const int v_off = (rr * STRIDE + ((16 * dq + ((l16 & 3) >> 1)) ^ sw_v)) * 16 + (l16 & 1) * 8;

  // O^T += V^T P^T for tile image `img`, after rescaling by the factors the
  // softmax step published with P.  The rescale (a rare, uniform branch) is a
  // step of its own so that the products can share a basic block with the
  // next softmax and interleave with it.
  auto pv_rescale = [&](int par) {
    const float al0 = al[par][32 * qh + l16], al1 = al[par][32 * qh + 16 + l16];
    if (__ballot(al0 != 1.f || al1 != 1.f)) {
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        acc[c][0] *= al0;
        acc[c][1] *= al1;
      }
    }
  };
  auto pv_mma = [&](const u32x4* img, int par) {
    const uint2 p00 = pb[par][qh][0][0][lane], p01 = pb[par][qh][0][1][lane];
    const uint2 p10 = pb[par][qh][1][0][lane], p11 = pb[par][qh][1][1][lane];
    const bf16x8 pB0 = as_bf16x8(u32x4{p00.x, p00.y, p01.x, p01.y});
    const bf16x8 pB1 = as_bf16x8(u32x4{p10.x, p10.y, p11.x, p11.y});
    const char* vb = reinterpret_cast<const char*>(img) + v_off;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const s16x4 v0 = lds_read_tr16(vb + ct * 32);
      const s16x4 v1 = lds_read_tr16(vb + T::BLK_IMG * 16 + ct * 32);
      const bf16x8 vA = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[ct][0] = mfma16x16x32(vA, pB0, acc[ct][0]);
      acc[ct][1] = mfma16x16x32(vA, pB1, acc[ct][1]);
    }
  };

  // Partial S^T of tile image `img` over this wave's k-steps, to xs[w].  The
  // K reads run kAhead (k-step, block) pairs ahead of the MFMAs, so at most
  // 2 kAhead reads are outstanding and every wait count is exact.  (A fifth
  // k-step that this wave does not own reads padding and neighbouring-row
  // columns inside the tile image, all finite, and is not used.)
  auto s_part = [&](const u32x4* img) {
    constexpr int NP = 2 * KQ;  // (k-step, block) pairs
    constexpr int kAhead = 7;
    static_assert(NP > kAhead && 2 * kAhead < 16, "read-ahead must fit the LDS counter");
    const uint32_t ka = lds_addr(reinterpret_cast<const char*>(img) + k_off);
    uint2 kr[KQ][2][2];
    [&]<int... I>(std::integer_sequence<int, I...>) {
      (lds_read_b64x2<(I % 2) * T::BLK_IMG * 16 + 256 * (I / 2)>(ka, kr[I / 2][I % 2][0], kr[I / 2][I % 2][1]), ...);
    }(std::make_integer_sequence<int, kAhead>{});
    f32x4 sp[2][2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) sp[rt][0] = sp[rt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    [&]<int... I>(std::integer_sequence<int, I...>) {
      (([&] {
         constexpr int j = I / 2, rt = I % 2;
         // pairs issued so far: min(I + kAhead, NP); those after pair I are outstanding
         constexpr int issued = I + kAhead < NP ? I + kAhead : NP;
         lgkm_wait<2 * (issued - 1 - I)>(kr[j][rt][0], kr[j][rt][1]);
         if (j < 4 || j < nk) {
           const bf16x8 kA = as_bf16x8(u32x4{kr[j][rt][0].x, kr[j][rt][0].y, kr[j][rt][1].x, kr[j][rt][1].y});
           sp[rt][0] = mfma16x16x32(kA, qf[0][j], sp[rt][0]);
           sp[rt][1] = mfma16x16x32(kA, qf[1][j], sp[rt][1]);
         }
         if constexpr (I + kAhead < NP) {
           constexpr int P = I + kAhead;
           lds_read_b64x2<(P % 2) * T::BLK_IMG * 16 + 256 * (P / 2)>(ka, kr[P / 2][P % 2][0], kr[P / 2][P % 2][1]);
         }
         // Keep this step's MFMAs between its wait and the next step's wait:
         // the scheduler would otherwise sink them below all the waits and
         // serialise the reads and the matrix work.
         __builtin_amdgcn_sched_barrier(0);
       }()),
       ...);
    }(std::make_integer_sequence<int, NP>{});
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        xs[w][0][n * 2 + rt][lane] = uint2{__float_as_uint(sp[rt][n][0]), __float_as_uint(sp[rt][n][1])};
        xs[w][1][n * 2 + rt][lane] = uint2{__float_as_uint(sp[rt][n][2]), __float_as_uint(sp[rt][n][3])};
      }
  };

  // Full scores of tile t for this lane's query and rows (sum of the four
  // quarter partials), online softmax, and P^T / rescale factors published to
  // LDS for the PV step.  The exponent reference m2 moves only when a tile max
  // exceeds it by more than kSlack (log2 units): probabilities stay below
  // 2^kSlack, the output is rescaled rarely, and acc / l and lse = m2 + log2(l)
  // do not depend on the reference.
  auto softmax = [&](int t) {
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint2 lo = xs[wave_of(qh, d)][0][nf * 2 + rt_f][src_lane];
      const uint2 hi = xs[wave_of(qh, d)][1][nf * 2 + rt_f][src_lane];
      sc += f32x4{__uint_as_float(lo.x), __uint_as_float(lo.y), __uint_as_float(hi.x), __uint_as_float(hi.y)};
    }
    const int j0 = t * 32 + 16 * rt_f + 4 * g_f;
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = j0 + i < vis_lim ? sc[i] * sl2 : -INFINITY;
      tmax = fmaxf(tmax, sc[i]);
    }
    tmax = fmaxf(tmax, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                     0, __builtin_bit_cast(int, tmax), 0x128, 0xf, 0xf, false)));
    tmax = max4rows(tmax);
    const bool grow = tmax > m2 + kSlack;
    const float alpha = grow && m2 > -INFINITY ? __builtin_amdgcn_exp2f(m2 - tmax) : 1.f;
    if (grow) m2 = tmax;
    const float m_use = m2 == -INFINITY ? 0.f : m2;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sc[i] - m_use);
    lsum = lsum * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    const uint2 pk = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
    pb[t & 1][qh][nf][rt_f][src_lane] = pk;
    al[t & 1][fq] = alpha;  // every lane of query fq holds the same factor
  };

  auto q_swizzle = [](int r) { return CH % 16 == 0 ? (r & 15) : ((r >> 1) & 7); };
  // Prologue: tile 0's loads go out first, then the workgroup's 64 query rows,
  // then tile 1; the wait leaves only tile 1 in flight.  The query rows go
  // HBM -> LDS with the same 1 KB coalesced loads as the tiles -- rows 0..31
  // into the third ring buffer (first used by tile 2), rows 32..63 into the
  // partial-exchange planes (first written by the S step of tile 0) -- and each
  // wave then reads its B operands from there; rows past n_q read as zeros.
  // (Loading the operands straight from global memory, 8 scattered bytes per
  // lane, costs several times the address work of a tile.)
  int32_t ids[2];
  if (n_tiles > 0) {
    tile_ids(0, ids);
    issue_tile(0, ids, ring, all_waves{});
    constexpr int Q_LOADS = 64 * D * 2 / 1024;  // 1 KB wave-loads of 64 query rows
    constexpr int Q_HALF = Q_LOADS / 2;
    static_assert(Q_LOADS % 8 == 0 && Q_HALF * 1024 == 32 * D * 2, "query rows split evenly over eight waves and two halves");
    static_assert(Q_HALF * 1024 <= T::IMG * 16 && Q_HALF * 1024 <= (int)sizeof(xs), "query staging fits");
    const int q_valid = a.n_q - mt * kQRowsPerWG < kQRowsPerWG ? a.n_q - mt * kQRowsPerWG : kQRowsPerWG;
    const i32x4 qrs = raw_rsrc(static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.n_q + (int64_t)mt * kQRowsPerWG) * D,
                               (uint32_t)(q_valid * D * 2));
    const uint32_t q_lds0 = lds_addr(ring + 2 * T::IMG), q_lds1 = lds_addr(xs);
    static_assert(CH % 16 == 0 || CH % 16 == 8, "staged query rows need a 1024- or 1152-byte-class pitch");
    // Staged row r (of a half) keeps its 16-byte chunk c at position c ^ sw(r),
    // so that the 16 rows read at one column fall on different banks: with a
    // 1152-byte pitch (rope width 64) rows already alternate between two bank
    // halves and sw(r) = (r >> 1) & 7; with a 1024-byte pitch every row starts
    // on the same bank and sw(r) = r & 15.
#pragma unroll
    for (int i = 0; i < Q_LOADS / 8; ++i) {
      const int u = w + 8 * i;
      const int hq = u < Q_HALF ? 0 : 1;
      const int unit = (u - hq * Q_HALF) * 64 + lane;  // 16-byte position within the half
      const int r = unit / CH, pc = unit - r * CH;
      const uint32_t voff = (uint32_t)((32 * hq + r) * D * 2 + (pc ^ q_swizzle(r)) * 16);
      dma16(qrs, (hq == 0 ? q_lds0 : q_lds1) + (uint32_t)(u - hq * Q_HALF) * 1024u, voff);
    }
  }
  if (n_tiles > 1) {
    tile_ids(1, ids);
    issue_tile(1, ids, ring + T::IMG, all_waves{});
    switch (c_w) {  // tile 1 stays in flight
      case 5: wait_vmcnt<5>(); break;
      case 4: wait_vmcnt<4>(); break;
      default: wait_vmcnt<0>(); break;
    }
  } else {
    wait_vmcnt<0>();
  }
  if (n_tiles > 0) {
    barrier_keep_loads();  // tile 0 and the query rows resident
    // Queries: B operand of S^T for this wave's k-steps (see qf).
    const char* qsrc = reinterpret_cast<const char*>(qh == 0 ? (const void*)(ring + 2 * T::IMG) : (const void*)xs);
    const int qsw = q_swizzle(l16);  // chunk swizzle of rows 16 n + l16 (same for both n)
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const char* qp = qsrc + (16 * n + l16) * D * 2 + (g & 1) * 8;
#pragma unroll
      for (int j = 0; j < KQ; ++j) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (j < nk) {
          const int c = 4 * (dq + 4 * j) + (g >> 1);  // chunk of columns 32 kk + 4 g
          const uint2 lo = *reinterpret_cast<const uint2*>(qp + (c ^ qsw) * 16);
          const uint2 hi = *reinterpret_cast<const uint2*>(qp + ((c + 2) ^ qsw) * 16);
          v = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
        qf[n][j] = as_bf16x8(v);
      }
    }
    barrier_keep_loads();  // staging areas free again
  }
  int cur = 0;  // ring slot of tile t
  // Phase 1 of tile t: partial S^T of tile t.  Phase 2: softmax of tile t and
  // PV of tile t - 1 (its P^T was published one phase earlier), so the matrix
  // cores have work while the softmax waits on LDS.  Tile t + 2 is issued once
  // tile t - 1 is no longer read, after the second barrier.
  for (int t = 0; t < n_tiles; ++t) {
    const int prev = cur == 0 ? 2 : cur - 1;  // tile t - 1's slot, reused by tile t + 2
    const bool more = t + 2 < n_tiles;
    if (more) tile_ids(t + 2, ids);  // scalar loads, complete by the barriers below
    s_part(ring + cur * T::IMG);
    barrier_keep_loads();  // partials visible
    if (t > 0) pv_rescale((t - 1) & 1);
    softmax(t);
    if (t > 0) pv_mma(ring + prev * T::IMG, (t - 1) & 1);
    if (t + 1 < n_tiles) wait_vmcnt<0>();
    barrier_keep_loads();  // P^T visible; tile t + 1 resident; tile t - 1 no longer read
    if (more) issue_tile(t + 2, ids, ring + prev * T::IMG, loader_waves{});
    cur = cur == 2 ? 0 : cur + 1;
  }
  if (n_tiles > 0) {
    pv_rescale((n_tiles - 1) & 1);
    pv_mma(ring + (cur == 0 ? 2 : cur - 1) * T::IMG, (n_tiles - 1) & 1);
  }

  // Final normalisation: the owner lanes of each query sum their partial l,
  // publish 1 / l, and write the LSE.  Block-id errors are seen only by the
  // loading waves: every wave takes the union.
  if (lane == 0) wflags[w] = flags;
  __syncthreads();
  flags = wflags[0] | wflags[1] | wflags[2] | wflags[3] | wflags[4] | wflags[5] | wflags[6] | wflags[7];
  const bool bad = flags != 0;
  lsum += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, lsum), 0x128, 0xf, 0xf, false));
  lsum = sum4rows(lsum);
  if (lane < 8) {
    fin[fq] = lsum > 0.f ? 1.f / lsum : 0.f;
    const int qr = mt * kQRowsPerWG + fq;
    if (qr < a.n_q) {
      const float lse_v = bad ? NAN : (lsum > 0.f ? (m2 + __log2f(lsum)) * kLn2 : -INFINITY);
      if (a.direct) {
        if (a.lse) a.lse[(int64_t)b * a.n_q + qr] = lse_v;
      } else {
        a.lse_part[((int64_t)b * a.splits + s) * a.n_q + qr] = lse_v;
      }
    }
  }
  __syncthreads();
  const f32x4 nan4 = {NAN, NAN, NAN, NAN};
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    if (!q_ok[n]) continue;
    const float inv = fin[32 * qh + 16 * n + l16];
    const int col0 = 128 * dq + 4 * g;
    if (a.direct) {
      const int64_t qrow = (int64_t)b * a.n_q + q_row[n];
      if (a.out_bf16) {
        uint16_t* o = static_cast<uint16_t*>(a.out) + qrow * T::KV + col0;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const f32x4 v = bad ? nan4 : acc[ct][n] * inv;
          const uint2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *reinterpret_cast<uint2*>(o + 16 * ct) = pk;
        }
      } else {
        float* o = static_cast<float*>(a.out) + qrow * T::KV + col0;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) *reinterpret_cast<f32x4*>(o + 16 * ct) = bad ? nan4 : acc[ct][n] * inv;
      }
    } else if (n_tiles > 0 || bad) {  // an empty range leaves its partial unwritten (lse -inf: merge skips it)
      const int64_t prow = ((int64_t)b * a.splits + s) * a.n_q + q_row[n];
      float* o = a.o_part + prow * T::KV + col0;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) *reinterpret_cast<f32x4*>(o + 16 * ct) = bad ? nan4 : acc[ct][n] * inv;
    }
  }
  if (tid == 0) a.status[item] = flags;
}

// ---------------------------------------------------------------------------
// Generic split kernel: any geometry, float32 or bfloat16 storage.  One
// workgroup of 128 threads per (request, range, query row); plain single-pass
// online softmax, one row at a time.  Used for shapes the MFMA kernel does
// not cover (and for float32 inputs).
// ---------------------------------------------------------------------------
template <typename TS>
__global__ __launch_bounds__(128) void decode_split_generic(const DecodeArgs a) {
  __shared__ float red[4];
  __shared__ int32_t blk_id;
  write_header(a);
  int b, s, mt, item;
  if (!decode_item(a, b, s, mt, item)) return;
  const int q = mt;  // one query row per workgroup
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int D = a.kv_rank + a.d_rope, R = a.kv_rank;

  const int64_t Lg = a.seq_lens[b];
  const int64_t L = held_rows(Lg, a.dcp_world, a.dcp_rank, a.dcp_interleave);
  uint32_t flags = request_flags(Lg, L, a.t_q, a.max_blocks);
  const int64_t r_begin = (int64_t)s * a.chunk_blocks * 16;
  int64_t r_end = r_begin + (int64_t)a.chunk_blocks * 16;
  if (flags || r_end > L) r_end = flags ? r_begin : L;
  const int64_t horizon = held_rows(Lg - a.t_q + q / a.n_head + 1, a.dcp_world, a.dcp_rank, a.dcp_interleave);
  if (r_end > horizon) r_end = horizon > r_begin ? horizon : r_begin;

  const TS* qp = static_cast<const TS*>(a.q) + ((int64_t)b * a.n_q + q) * D;
  const TS* kv = static_cast<const TS*>(a.kv);
  constexpr int MAXC = 8;  // up to 8 * 128 = 1024 value columns per thread block
  float acc[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) acc[c] = 0.f;
  float m = -INFINITY, l = 0.f;

  for (int64_t j = r_begin; j < r_end; ++j) {
    if ((j & 15) == 0 || j == r_begin) {
      __syncthreads();
      if (tid == 0) blk_id = a.bt[(int64_t)b * a.max_blocks + (j >> 4)];
      __syncthreads();
    }
    const int32_t id = blk_id;
    if (id < 0 || (int64_t)id >= a.num_blocks) {
      flags |= kBadBlock;
      break;
    }
    const TS* row = kv + ((int64_t)id * 16 + (j & 15)) * D;
    float part = 0.f;
    for (int d = tid; d < D; d += 128)
      part += Storage<TS>::load(qp, d) * Storage<TS>::load(row, d);
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
    __syncthreads();
    if (lane == 0) red[w] = part;
    __syncthreads();
    const float sj = (red[0] + red[1]) * a.scale;
    const float m_new = fmaxf(m, sj);
    const float rescale = m == -INFINITY ? 0.f : expf(m - m_new);
    const float p = expf(sj - m_new);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int col = tid + 128 * c;
      if (col < R) acc[c] = acc[c] * rescale + p * Storage<TS>::load(row, col);
    }
    l = l * rescale + p;
    m = m_new;
  }
  const bool bad = flags != 0;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float lse_v = l > 0.f ? m + logf(l) : -INFINITY;
  if (bad) lse_v = NAN;
  const int64_t qrow = (int64_t)b * a.n_q + q;
  for (int c = 0; c < MAXC; ++c) {
    const int col = tid + 128 * c;
    if (col >= R) break;
    const float v = bad ? NAN : acc[c] * inv;
    if (a.direct) {
      if (a.out_bf16) static_cast<uint16_t*>(a.out)[qrow * R + col] = f32_to_bf16(v);
      else static_cast<float*>(a.out)[qrow * R + col] = v;
    } else {
      a.o_part[(((int64_t)b * a.splits + s) * a.n_q + q) * R + col] = v;
    }
  }
  if (tid == 0) {
    if (a.direct) {
      if (a.lse) a.lse[qrow] = lse_v;
    } else {
      a.lse_part[((int64_t)b * a.splits + s) * a.n_q + q] = lse_v;
    }
    a.status[item] = flags;
  }
}

// ---------------------------------------------------------------------------
// Merge of the split partials: one wave per query row, four rows per workgroup.
// Lane l owns output columns 4 l + 256 j; the split loop is unrolled by eight
// so each lane has up to sixteen 16-byte partial loads in flight.
// ---------------------------------------------------------------------------
constexpr int kMergeRows = 4;
constexpr int kMergeRegSplits = 16;  // register-resident merge up to this many splits

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Workgroups per request in the merge (kMergeRows query rows each).
__device__ __host__ inline int merge_wg_per_request(int n_q) { return (n_q + kMergeRows - 1) / kMergeRows; }

// Register-resident merge of one query row over S <= KR splits: every LSE and
// partial vector of the row is loaded at once (one memory latency); lane l owns
// columns 4 l .. + 3 and 256 + 4 l .. + 3 of a 512-wide row.  Loads past the
// last split repeat it and are masked out.
template <int KR>
__device__ __forceinline__ void merge_row_reg(const DecodeArgs& a, int64_t qrow, const float* lp, const float* op,
                                              int64_t sstride, int S, int R, int lane) {
  float lk[KR];
  f32x4 v0[KR], v1[KR];
#pragma unroll
  for (int k = 0; k < KR; ++k) {
    const int kk = k < S ? k : S - 1;
    lk[k] = lp[(int64_t)kk * a.n_q];
    v0[k] = *reinterpret_cast<const f32x4*>(op + kk * sstride + 4 * lane);
    v1[k] = *reinterpret_cast<const f32x4*>(op + kk * sstride + 256 + 4 * lane);
  }
  float M = -INFINITY;
  bool any_nan = false;
#pragma unroll
  for (int k = 0; k < KR; ++k) {
    if (k < S) {
      any_nan |= isnan(lk[k]);
      M = fmaxf(M, lk[k]);
    }
  }
  float wsum = 0.f;
  f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = o0;
#pragma unroll
  for (int k = 0; k < KR; ++k) {
    const bool live = k < S && lk[k] != -INFINITY && M != -INFINITY;  // empty splits may be unwritten
    const float wk = live ? __expf(lk[k] - M) : 0.f;
    wsum += wk;
    o0 += wk * (live ? v0[k] : f32x4{0.f, 0.f, 0.f, 0.f});
    o1 += wk * (live ? v1[k] : f32x4{0.f, 0.f, 0.f, 0.f});
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const f32x4 nan4 = {NAN, NAN, NAN, NAN};
  const f32x4 r0 = any_nan ? nan4 : o0 * inv, r1 = any_nan ? nan4 : o1 * inv;
  if (a.out_bf16) {
    uint16_t* o = static_cast<uint16_t*>(a.out) + qrow * R;
    *reinterpret_cast<uint2*>(o + 4 * lane) = uint2{pack_bf16x2(r0[0], r0[1]), pack_bf16x2(r0[2], r0[3])};
    *reinterpret_cast<uint2*>(o + 256 + 4 * lane) = uint2{pack_bf16x2(r1[0], r1[1]), pack_bf16x2(r1[2], r1[3])};
  } else {
    float* o = static_cast<float*>(a.out) + qrow * R;
    *reinterpret_cast<f32x4*>(o + 4 * lane) = r0;
    *reinterpret_cast<f32x4*>(o + 256 + 4 * lane) = r1;
  }
  if (lane == 0 && a.lse) a.lse[qrow] = any_nan ? NAN : (M == -INFINITY ? -INFINITY : M + __logf(wsum));
}

__global__ __launch_bounds__(64 * kMergeRows) void decode_merge(const DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  int64_t qrow;  // b * n_q + q
  if (a.batch % 8 == 0) {  // request b on XCD b % 8, where its partials were written
    const int per_b = merge_wg_per_request(a.n_q);
    const int rest = blockIdx.x >> 3;
    const int bg = rest / per_b;
    const int b_ = bg * 8 + (blockIdx.x & 7);
    const int q_ = (rest - bg * per_b) * kMergeRows + (threadIdx.x >> 6);
    if (q_ >= a.n_q) return;
    qrow = (int64_t)b_ * a.n_q + q_;
  } else {
    qrow = (int64_t)blockIdx.x * kMergeRows + (threadIdx.x >> 6);
  }
  if (qrow >= (int64_t)a.batch * a.n_q) return;
  const int b = (int)(qrow / a.n_q);
  const int q = (int)(qrow - (int64_t)b * a.n_q);
  const int S = a.splits, R = a.kv_rank;
  const float* lp = a.lse_part + (int64_t)b * S * a.n_q + q;  // split k at lp[k * n_q]
  const float* op = a.o_part + ((int64_t)b * S * a.n_q + q) * R;
  const int64_t sstride = (int64_t)a.n_q * R;

  if (R == 2 * 256 && S <= 8) {
    merge_row_reg<8>(a, qrow, lp, op, sstride, S, R, lane);
    return;
  }
  if (R == 2 * 256 && S <= kMergeRegSplits) {
    merge_row_reg<kMergeRegSplits>(a, qrow, lp, op, sstride, S, R, lane);
    return;
  }

  float mx = -INFINITY;
  bool nan_seen = false;
  for (int k = lane; k < S; k += 64) {
    const float v = lp[(int64_t)k * a.n_q];
    nan_seen |= isnan(v);
    mx = fmaxf(mx, v);
  }
  const float M = wave_max(mx);
  const bool any_nan = __ballot(nan_seen) != 0;
  float wpart = 0.f;
  if (M != -INFINITY)
    for (int k = lane; k < S; k += 64) wpart += __expf(lp[(int64_t)k * a.n_q] - M);
  const float wsum = wave_sum(wpart);
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;

  for (int c0 = 4 * lane; c0 < R; c0 += 256) {
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
      if (R - c0 >= 4) {
        // Splits with lse -inf (empty ranges) contribute nothing and their
        // partials may be unwritten: the loads (always inside the workspace)
        // are issued regardless, and their values discarded by a select.
        int k = 0;
        for (; k + 8 <= S; k += 8) {
          f32x4 v[8];
          float wk[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            wk[u] = lp[(int64_t)(k + u) * a.n_q];
            v[u] = *reinterpret_cast<const f32x4*>(op + (k + u) * sstride + c0);
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const bool live = wk[u] != -INFINITY;
            const float wgt = live ? __expf(wk[u] - M) : 0.f;
            const f32x4 vv = live ? v[u] : f32x4{0.f, 0.f, 0.f, 0.f};
            o += wgt * vv;
          }
        }
        for (; k < S; ++k) {
          const float wk = lp[(int64_t)k * a.n_q];
          if (wk != -INFINITY) o += __expf(wk - M) * *reinterpret_cast<const f32x4*>(op + k * sstride + c0);
        }
      } else {
        for (int k = 0; k < S; ++k) {
          const float lk = lp[(int64_t)k * a.n_q];
          if (lk == -INFINITY) continue;
          const float wk = __expf(lk - M);
          for (int e = 0; c0 + e < R; ++e) o[e] += wk * op[k * sstride + c0 + e];
        }
      }
    }
    for (int e = 0; e < 4 && c0 + e < R; ++e) {
      const float v = any_nan ? NAN : o[e] * inv;
      if (a.out_bf16) static_cast<uint16_t*>(a.out)[qrow * R + c0 + e] = f32_to_bf16(v);
      else static_cast<float*>(a.out)[qrow * R + c0 + e] = v;
    }
  }
  if (lane == 0 && a.lse) a.lse[qrow] = any_nan ? NAN : (M == -INFINITY ? -INFINITY : M + __logf(wsum));
}

// ---------------------------------------------------------------------------
// Merge for many splits per request (few query rows, long requests): one
// workgroup of kWideWaves waves per query row.  Wave v sums the contiguous
// splits [v S / W, (v + 1) S / W); the per-wave sums are then added in wave
// order through LDS, so the result does not depend on timing.
// ---------------------------------------------------------------------------
constexpr int kWideWaves = 16;
constexpr int kWideMinSplits = 64;  // decode_merge_wide from this many splits on

__global__ __launch_bounds__(64 * kWideWaves) void decode_merge_wide(const DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) float wsum_lds[];  // [kWideWaves][kv_rank], then scratch
  float* red = wsum_lds + kWideWaves * a.kv_rank;                  // [kWideWaves] reductions
  const int tid = threadIdx.x, lane = tid & 63, v = tid >> 6;
  int64_t qrow;
  if (a.batch % 8 == 0) {  // request b on XCD b % 8, as in decode_merge
    const int rest = blockIdx.x >> 3;
    const int bg = rest / a.n_q;
    qrow = (int64_t)(bg * 8 + (blockIdx.x & 7)) * a.n_q + (rest - bg * a.n_q);
  } else {
    qrow = blockIdx.x;
  }
  const int b = (int)(qrow / a.n_q);
  const int q = (int)(qrow - (int64_t)b * a.n_q);
  const int S = a.splits, R = a.kv_rank;
  const float* lp = a.lse_part + (int64_t)b * S * a.n_q + q;

  float mx = -INFINITY;
  bool nan_seen = false;
  for (int k = tid; k < S; k += 64 * kWideWaves) {
    const float x = lp[(int64_t)k * a.n_q];
    nan_seen |= isnan(x);
    mx = fmaxf(mx, x);
  }
  mx = wave_max(mx);
  const int any_nan = __syncthreads_or(nan_seen ? 1 : 0);
  if (lane == 0) red[v] = mx;
  __syncthreads();
  float M = -INFINITY;
  for (int i = 0; i < kWideWaves; ++i) M = fmaxf(M, red[i]);
  __syncthreads();
  float wpart = 0.f;
  if (M != -INFINITY)
    for (int k = tid; k < S; k += 64 * kWideWaves) wpart += __expf(lp[(int64_t)k * a.n_q] - M);
  wpart = wave_sum(wpart);
  if (lane == 0) red[v] = wpart;
  __syncthreads();
  float wsum = 0.f;
  for (int i = 0; i < kWideWaves; ++i) wsum += red[i];
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;

  const int k0 = (int)((int64_t)S * v / kWideWaves), k1 = (int)((int64_t)S * (v + 1) / kWideWaves);
  const float* op = a.o_part + ((int64_t)b * S * a.n_q + q) * R;
  const int64_t sstride = (int64_t)a.n_q * R;
  for (int c0 = 4 * lane; c0 < R; c0 += 256) {
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
      if (R - c0 >= 4) {
        int k = k0;
        for (; k + 4 <= k1; k += 4) {
          f32x4 x[4];
          float wk[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            wk[u] = lp[(int64_t)(k + u) * a.n_q];
            x[u] = *reinterpret_cast<const f32x4*>(op + (k + u) * sstride + c0);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const bool live = wk[u] != -INFINITY;
            o += (live ? __expf(wk[u] - M) : 0.f) * (live ? x[u] : f32x4{0.f, 0.f, 0.f, 0.f});
          }
        }
        for (; k < k1; ++k) {
          const float wk = lp[(int64_t)k * a.n_q];
          if (wk != -INFINITY) o += __expf(wk - M) * *reinterpret_cast<const f32x4*>(op + k * sstride + c0);
        }
      } else {
        for (int k = k0; k < k1; ++k) {
          const float lk = lp[(int64_t)k * a.n_q];
          if (lk == -INFINITY) continue;
          const float wk = __expf(lk - M);
          for (int e = 0; c0 + e < R; ++e) o[e] += wk * op[k * sstride + c0 + e];
        }
      }
    }
    for (int e = 0; e < 4 && c0 + e < R; ++e) wsum_lds[v * R + c0 + e] = o[e];
  }
  __syncthreads();
  for (int c = tid; c < R; c += 64 * kWideWaves) {
    float acc = 0.f;
    for (int i = 0; i < kWideWaves; ++i) acc += wsum_lds[i * R + c];
    const float val = any_nan ? NAN : acc * inv;
    if (a.out_bf16) static_cast<uint16_t*>(a.out)[qrow * R + c] = f32_to_bf16(val);
    else static_cast<float*>(a.out)[qrow * R + c] = val;
  }
  if (tid == 0 && a.lse) a.lse[qrow] = any_nan ? NAN : (M == -INFINITY ? -INFINITY : M + __logf(wsum));
}

// The same merge for kv_rank 512, with each row's columns split over
// kWideCols workgroups (128 columns each), so that a few long rows still
// spread their partials over every compute unit.  Wave v sums the splits
// [v S / W, (v + 1) S / W): lanes 0-31 take the even splits of that run and
// lanes 32-63 the odd ones, four columns per lane, and the two halves are
// added before the per-wave sums are added in wave order through LDS.
// Workgroup i handles column chunk i / rows of row i % rows (rows = batch x
// query rows), so with a row count that is a multiple of 8 a row's chunks run
// on the XCD the row's other workgroups use.
constexpr int kWideCols = 4;

__global__ __launch_bounds__(64 * kWideWaves) void decode_merge_wide512(const DecodeArgs a) {
  constexpr int R = 512, CW = R / kWideCols;
  static_assert(CW == 128, "32 lanes x 4 columns per chunk");
  __shared__ __attribute__((aligned(16))) f32x4 wsum_lds[kWideWaves][CW / 4];
  __shared__ float red[kWideWaves];
  const int tid = threadIdx.x, lane = tid & 63, v = tid >> 6;
  const int64_t rows = (int64_t)a.batch * a.n_q;
  const int chunk = (int)(blockIdx.x / rows);
  const int64_t rid = blockIdx.x - (int64_t)chunk * rows;
  int64_t qrow;
  if (a.batch % 8 == 0) {  // request b on XCD b % 8, as in decode_merge
    const int64_t rest = rid >> 3;
    const int64_t bg = rest / a.n_q;
    qrow = (bg * 8 + (rid & 7)) * a.n_q + (rest - bg * a.n_q);
  } else {
    qrow = rid;
  }
  const int b = (int)(qrow / a.n_q);
  const int q = (int)(qrow - (int64_t)b * a.n_q);
  const int S = a.splits;
  const float* lp = a.lse_part + (int64_t)b * S * a.n_q + q;

  float mx = -INFINITY;
  bool nan_seen = false;
  for (int k = tid; k < S; k += 64 * kWideWaves) {
    const float x = lp[(int64_t)k * a.n_q];
    nan_seen |= isnan(x);
    mx = fmaxf(mx, x);
  }
  mx = wave_max(mx);
  const int any_nan = __syncthreads_or(nan_seen ? 1 : 0);
  if (lane == 0) red[v] = mx;
  __syncthreads();
  float M = -INFINITY;
  for (int i = 0; i < kWideWaves; ++i) M = fmaxf(M, red[i]);
  __syncthreads();
  float wpart = 0.f;
  if (M != -INFINITY)
    for (int k = tid; k < S; k += 64 * kWideWaves) wpart += __expf(lp[(int64_t)k * a.n_q] - M);
  wpart = wave_sum(wpart);
  if (lane == 0) red[v] = wpart;
  __syncthreads();
  float wsum = 0.f;
  for (int i = 0; i < kWideWaves; ++i) wsum += red[i];
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;

  const int k0 = (int)((int64_t)S * v / kWideWaves), k1 = (int)((int64_t)S * (v + 1) / kWideWaves);
  const int hl = lane >> 5;                              // split parity of this lane half
  const int c0 = chunk * CW + 4 * (lane & 31);           // this lane's four columns
  const float* op = a.o_part + ((int64_t)b * S * a.n_q + q) * R + c0;
  const int64_t sstride = (int64_t)a.n_q * R;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
    // Splits k0 + hl, k0 + hl + 2, ...: four at a time per lane half.
    int k = k0 + hl;
    for (; k + 6 < k1; k += 8) {
      f32x4 x[4];
      float wk[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        wk[u] = lp[(int64_t)(k + 2 * u) * a.n_q];
        x[u] = *reinterpret_cast<const f32x4*>(op + (k + 2 * u) * sstride);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool live = wk[u] != -INFINITY;  // an empty split may be unwritten
        o += (live ? __expf(wk[u] - M) : 0.f) * (live ? x[u] : f32x4{0.f, 0.f, 0.f, 0.f});
      }
    }
    for (; k < k1; k += 2) {
      const float wk = lp[(int64_t)k * a.n_q];
      if (wk != -INFINITY) o += __expf(wk - M) * *reinterpret_cast<const f32x4*>(op + k * sstride);
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] += __shfl_xor(o[e], 32, 64);
  if (hl == 0) wsum_lds[v][lane] = o;
  __syncthreads();
  if (v == 0 && hl == 0) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < kWideWaves; ++i) acc += wsum_lds[i][lane];
    const f32x4 nan4 = {NAN, NAN, NAN, NAN};
    const f32x4 val = any_nan ? nan4 : acc * inv;
    if (a.out_bf16) {
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + qrow * R + c0) =
          uint2{pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3])};
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + qrow * R + c0) = val;
    }
  }
  if (chunk == 0 && tid == 0 && a.lse) a.lse[qrow] = any_nan ? NAN : (M == -INFINITY ? -INFINITY : M + __logf(wsum));
}

// LSE combine of P partial results over disjoint row sets (the split merge,
// here across context-parallel ranks): one wave per row.  With M the largest
// part LSE and w_p = exp(lse_p - M), o = sum_p w_p o_p / sum_p w_p and
// lse = M + ln sum_p w_p; parts with lse -inf carry no weight and their
// vectors are not read; all -inf gives zeros and -inf; a NaN LSE in any part
// gives NaN.  Deterministic: parts are added in index order.  Lane l owns
// columns 4 l .. + 3 of every 256-column chunk; the weights of 64 parts at a
// time are formed once (lane p holds part p's) and broadcast, and the part
// vectors go out eight at a time before they are summed, so the row costs a
// few memory latencies rather than one per part.
constexpr int kCombineRows = 4;  // rows (waves) per workgroup
__global__ __launch_bounds__(64 * kCombineRows) void lse_combine_kernel(int64_t n_rows, int n_parts, int width,
                                                                        const float* __restrict__ o_parts,
                                                                        const float* __restrict__ lse_parts,
                                                                        void* out, int out_bf16, float* lse_out,
                                                                        int vec) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kCombineRows + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  float M = -INFINITY;
  bool nan_seen = false;
  for (int p = lane; p < n_parts; p += 64) {
    const float v = lse_parts[(int64_t)p * n_rows + row];
    nan_seen |= isnan(v);
    M = fmaxf(M, v);
  }
  M = wave_max(M);
  const bool any_nan = __ballot(nan_seen) != 0;
  auto weight = [&](int p) {  // weight of part p (0 past the last part or for an empty part)
    if (p >= n_parts || M == -INFINITY) return 0.f;
    const float v = lse_parts[(int64_t)p * n_rows + row];
    return v == -INFINITY ? 0.f : __expf(v - M);
  };
  float wsum = 0.f;
  for (int p = lane; p < n_parts; p += 64) wsum += weight(p);
  wsum = wave_sum(wsum);
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const float* orow = o_parts + row * width;
  const int64_t pstride = n_rows * width;
  for (int c0 = 0; c0 < width; c0 += 256) {
    const int c = c0 + 4 * lane;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int p0 = 0; p0 < n_parts; p0 += 64) {
      const float wl = weight(p0 + lane);  // lane k: weight of part p0 + k
      const int np = n_parts - p0 < 64 ? n_parts - p0 : 64;
      for (int k0 = 0; k0 < np; k0 += 8) {
        f32x4 v[8];
        float wk[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          wk[k] = __shfl(wl, k0 + k, 64);
          v[k] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (k0 + k < np && wk[k] != 0.f && c < width) {
            const float* src = orow + (int64_t)(p0 + k0 + k) * pstride + c;
            if (vec) {
              v[k] = *reinterpret_cast<const f32x4*>(src);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) v[k][e] = c + e < width ? src[e] : 0.f;
            }
          }
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) acc += wk[k] * v[k];
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (c + e >= width) break;
      const float r = any_nan ? NAN : acc[e] * inv;
      if (out_bf16) static_cast<uint16_t*>(out)[row * width + c + e] = f32_to_bf16(r);
      else static_cast<float*>(out)[row * width + c + e] = r;
    }
  }
  if (lane == 0 && lse_out) lse_out[row] = any_nan ? NAN : (M == -INFINITY ? -INFINITY : M + __logf(wsum));
}

}  // namespace

hipError_t launch_lse_combine(int64_t n_rows, int n_parts, int width, const float* o_parts, const float* lse_parts,
                              void* out, bool out_bf16, float* lse_out, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  const int64_t grid = (n_rows + kCombineRows - 1) / kCombineRows;
  if (grid > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(lse_combine_kernel, dim3((unsigned)grid), dim3(64 * kCombineRows), 0, stream, n_rows, n_parts,
                     width, o_parts, lse_parts, out, (int)out_bf16, lse_out,
                     (int)((width & 3) == 0 && (reinterpret_cast<uintptr_t>(o_parts) & 15) == 0));
  return hipGetLastError();
}

Plan decode_plan(int n_head, int kv_rank, int d_rope, int batch, int t_q, int max_blocks,
                 int splits, bool bf16) {
  Plan p;
  p.mfma = bf16 && kv_rank == 512 && (d_rope == 0 || d_rope == 64);
  const int n_q = t_q * n_head;
  p.splits = splits < 1 ? 1 : (splits > max_blocks ? max_blocks : splits);
  if (p.splits > kMaxSplits) p.splits = kMaxSplits;
  p.chunk_blocks = (max_blocks + p.splits - 1) / p.splits;
  p.splits = (max_blocks + p.chunk_blocks - 1) / p.chunk_blocks;  // no empty tail ranges
  p.m_tiles = p.mfma ? (n_q + kQRowsPerWG - 1) / kQRowsPerWG : n_q;
  // Workgroup and status-slot counts are 32-bit on the device (and the grid
  // rounds the pairs up to a multiple of 8): larger plans are refused.
  const int64_t pairs = (int64_t)batch * p.splits;
  const int64_t rounded = (pairs + 7) / 8 * 8;
  p.ok = p.m_tiles >= 1 && rounded <= (int64_t)INT32_MAX / p.m_tiles;
  p.n_pairs = p.ok ? (int)pairs : 0;
  p.n_items = p.ok ? (int)(pairs * p.m_tiles) : 0;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t status_bytes = al((size_t)(p.n_items > 0 ? p.n_items : 1) * 4);
  p.lse_off = kHeaderBytes + status_bytes;
  const size_t parts = (size_t)batch * p.splits * n_q;
  p.o_off = al(p.lse_off + parts * 4);
  p.bytes = p.splits > 1 ? al(p.o_off + parts * (size_t)kv_rank * 4) : p.lse_off;
  return p;
}

hipError_t launch_decode(const DecodeArgs& a, bool mfma, bool bf16, hipStream_t stream) {
  int grid;
  if (a.batch % 8 == 0 && a.batch > 0) {
    grid = a.batch * a.splits * a.m_tiles;  // = (batch / 8) * 8 * splits * m_tiles
  } else {
    const int groups = (a.n_pairs + 7) / 8;
    grid = (groups > 0 ? groups : 1) * 8 * a.m_tiles;
  }
  if (mfma) {
    if (a.d_rope == 64)
      hipLaunchKernelGGL(decode_split_mfma<64>, dim3(grid), dim3(512), 0, stream, a);
    else
      hipLaunchKernelGGL(decode_split_mfma<0>, dim3(grid), dim3(512), 0, stream, a);
  } else if (bf16) {
    hipLaunchKernelGGL(decode_split_generic<uint16_t>, dim3(grid), dim3(128), 0, stream, a);
  } else {
    hipLaunchKernelGGL(decode_split_generic<float>, dim3(grid), dim3(128), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.direct || a.batch == 0) return e;
  const int64_t rows = (int64_t)a.batch * a.n_q;
  if (a.splits >= kWideMinSplits && a.kv_rank == 512) {
    if (rows * kWideCols > INT32_MAX) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(decode_merge_wide512, dim3((unsigned)(rows * kWideCols)), dim3(64 * kWideWaves), 0, stream, a);
    return hipGetLastError();
  }
  if (a.splits >= kWideMinSplits) {
    const size_t lds = ((size_t)kWideWaves * a.kv_rank + kWideWaves) * sizeof(float);
    hipLaunchKernelGGL(decode_merge_wide, dim3((unsigned)rows), dim3(64 * kWideWaves), lds, stream, a);
    return hipGetLastError();
  }
  const int64_t mgrid = a.batch % 8 == 0 ? (int64_t)a.batch * merge_wg_per_request(a.n_q)
                                         : (rows + kMergeRows - 1) / kMergeRows;
  hipLaunchKernelGGL(decode_merge, dim3((unsigned)mgrid), dim3(64 * kMergeRows), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
