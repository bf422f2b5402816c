// Naive-form (multi-head) MLA attention for prefill and chunked prefill, for
// gfx950.
//
// What is computed (memra-engine "mla.rs", mla_attend_naive; MlaInputs
// causal rule): per request b, head h and new query i < t_q,
//   k_nope_j = W_UK[h] c_kv_j (d_nope wide), v_j = W_UV[h] c_kv_j (d_v wide),
//   s_j = scale * (<q_nope, k_nope_j> + <q_pe, k_pe_j>),
//   out = sum_j softmax(s)_j v_j over the visible rows j <= L - t_q + i,
// with L = seq_lens[b] counting the t_q new rows.  This is the form whose
// attention runs at query-key width d_nope + d_rope and value width d_v
// instead of the absorbed kv_rank + d_rope / kv_rank, at the price of
// decompressing the cache rows first.
//
// Two kernels:
//   * prefill_decompress: one GEMM per request, the cache rows (gathered
//     through the block table) times [W_UK; W_UV]^T, written per head as
//     K_nope [H][rows][d_nope] and V [H][rows][d_v] (bf16) into the workspace.
//     Tiles of 128 weight rows x 128 cache rows, k-chunks of 64 staged in LDS
//     by LDS-DMA with an XOR swizzle, 16x16x32 bf16 MFMA with the weights as
//     the A operand so each lane stores four consecutive output columns.
//   * prefill_attend: flash attention per (request, head, 128 queries); eight
//     waves of 16 queries (two per SIMD; a four-wave form of 32 queries per
//     wave is kept as a template instance).  Tiles of 32 rows -- K_nope and V
//     from the workspace, k_pe straight from the paged cache (shared by all
//     heads) -- go HBM -> LDS by LDS-DMA through a four-stage ring, three
//     tiles in flight.  S^T = K Q^T with the queries
//     in registers, online softmax with a delayed reference maximum, P^T kept
//     in registers in the B-operand layout of O^T = V^T P^T, V^T read with the
//     transposing ds_read_b64_tr_b16.  One barrier per tile: every wave owns
//     complete query rows, so nothing is exchanged.
#include <math.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace mla {
namespace {

constexpr uint32_t kNegLen = 0x1u, kLenOverTable = 0x2u, kLenBelowTq = 0x4u, kBadBlock = 0x8u;
constexpr float kSlackP = 8.f;  // log2 headroom before the softmax reference moves

template <int DR>
struct PGeom {
  static constexpr int KR = 512;       // latent rank
  static constexpr int DN = 256 - DR;  // query-key width without rope
  static constexpr int DV = 256;       // value width
  static constexpr int D = KR + DR;    // cache row width
};

__device__ __forceinline__ uint32_t prefill_flags(int64_t L, int t_q, int max_blocks) {
  if (L < 0) return kNegLen;
  if (L > (int64_t)max_blocks * 16) return kLenOverTable;
  if (L > 0 && L < t_q) return kLenBelowTq;
  return 0u;
}

// 16-byte chunk swizzle of a staged row whose pitch is `pitch_chunks` chunks,
// so that 16 consecutive rows read at one chunk fall on 16 different bank
// groups (64 banks = 16 chunks).
template <int PITCH>
__device__ __forceinline__ int row_swizzle(int r) {
  static_assert(PITCH % 16 == 0 || PITCH % 16 == 8, "pitch of 8 or 16 chunks modulo 16");
  return PITCH % 16 == 0 ? (r & 15) : ((r >> 1) & 7);
}

// ---------------------------------------------------------------------------
// Decompression GEMM
// ---------------------------------------------------------------------------
constexpr int kGN = 128, kGM = 128, kGK = 64;  // weight rows, cache rows, k per chunk
constexpr int kGChunks = kGK / 8;              // 16-byte chunks per staged row (8)
constexpr int kWeightGroup = 14;               // weight tiles per XCD group (1.75 MB of bf16)

template <int DR>
__global__ __launch_bounds__(256, 2) void prefill_decompress(const PrefillArgs a) {
  using G = PGeom<DR>;
  constexpr int KR = G::KR, D = G::D;
  __shared__ __attribute__((aligned(16))) u32x4 sw[2][kGN * kGChunks];  // weight rows [128][64]
  __shared__ __attribute__((aligned(16))) u32x4 sc[2][kGM * kGChunks];  // cache rows [128][64]

  // Workgroup i runs on XCD i % 8.  Each XCD takes whole groups of
  // a.wgroup weight tiles (group g on XCD g % 8) and, per group, walks every
  // cache-row tile with the group's weight tiles innermost, so the group's
  // weights stay in that XCD's L2 while the cache tiles stream past.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int per_group = a.batch * a.n_mtiles * a.wgroup;
  const int grp = (slot / per_group) * 8 + xcd;
  const int rem = slot - (slot / per_group) * per_group;
  const int ct = rem / a.wgroup, wt = grp * a.wgroup + (rem - ct * a.wgroup);
  if (wt >= a.n_wtiles) return;  // whole workgroup
  const int b = ct / a.n_mtiles;
  const int m0 = (ct - b * a.n_mtiles) * kGM, n0 = wt * kGN;
  const int64_t L = a.seq_lens[b];
  if (prefill_flags(L, a.t_q, a.max_blocks) != 0 || (int64_t)m0 >= L) return;  // whole workgroup
  const int rows = L - m0 < kGM ? (int)(L - m0) : kGM;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = w & 1, wm = w >> 1;  // 64-row quarter of the tile: weights wn, cache rows wm
  const int l16 = lane & 15, g = lane >> 4;

  const int NK = a.n_head * G::DN;  // rows of W_UK in the [W_UK; W_UV] stack
  const bool is_k = n0 < NK;
  const uint16_t* wrows = is_k ? static_cast<const uint16_t*>(a.w_uk) + (int64_t)n0 * KR
                               : static_cast<const uint16_t*>(a.w_uv) + (int64_t)(n0 - NK) * KR;
  const i32x4 rs_w = raw_rsrc(wrows, (uint32_t)(kGN * KR * 2));

  // Each wave stages weight rows [32 w, 32 w + 32) and cache rows
  // [32 w, 32 w + 32) of the tile: four 1 KB loads each (8 rows x 128 bytes).
  // The cache rows of one load lie in one 16-row block.
  const uint16_t* kv = static_cast<const uint16_t*>(a.kv);
  const int32_t* bt_row = a.bt + (int64_t)b * a.max_blocks;
  const uint32_t nb32 = a.num_blocks < (int64_t)INT32_MAX ? (uint32_t)a.num_blocks : (uint32_t)INT32_MAX;
  uint32_t flags = 0;
  i32x4 rs_c[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int r0 = 32 * w + 16 * k;  // first tile row of this block
    const int nval = rows - r0 <= 0 ? 0 : (rows - r0 >= 16 ? 16 : rows - r0);
    int32_t id = -1;
    if (nval > 0) id = __builtin_amdgcn_readfirstlane(bt_row[(m0 + r0) >> 4]);
    const bool ok = (uint32_t)id < nb32;
    if (nval > 0 && !ok) flags |= kBadBlock;
    rs_c[k] = raw_rsrc(kv + (int64_t)(ok ? id : 0) * (16 * D), ok ? (uint32_t)(nval * D * 2) : 0u);
  }
  // Lane slot of a load: row 8 i + lane / 8 of the wave's 32, chunk position
  // p = lane % 8 holding global chunk p ^ swizzle(row).
  const int lr = lane >> 3, lp = lane & 7;
  auto issue_chunk = [&](int c, int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 32 * w + 8 * i + lr;  // tile row
      const int gc = lp ^ row_swizzle<kGChunks>(r);
      dma16(rs_w, lds_addr(&sw[buf][(32 * w + 8 * i) * kGChunks]), (uint32_t)(r * KR * 2 + c * kGK * 2 + gc * 16));
      dma16(rs_c[i >> 1], lds_addr(&sc[buf][(32 * w + 8 * i) * kGChunks]),
            (uint32_t)(((8 * i + lr) & 15) * D * 2 + c * kGK * 2 + gc * 16));
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int NCH = KR / kGK;
  issue_chunk(0, 0);
  for (int c = 0; c < NCH; ++c) {
    const int buf = c & 1;
    if (c + 1 < NCH) {
      issue_chunk(c + 1, buf ^ 1);
      wait_vmcnt<8>();  // this wave's loads of chunk c are done
    } else {
      wait_vmcnt<0>();
    }
    barrier_keep_loads();  // every wave's loads of chunk c are visible
    const char* pw = reinterpret_cast<const char*>(sw[buf]);
    const char* pc = reinterpret_cast<const char*>(sc[buf]);
#pragma unroll
    for (int ks = 0; ks < kGK / 32; ++ks) {
      bf16x8 fa[4], fb[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int rw = 64 * wn + 16 * t + l16, rc = 64 * wm + 16 * t + l16;
        const int ch = 4 * ks + g;
        fa[t] = as_bf16x8(*reinterpret_cast<const u32x4*>(pw + (rw * kGChunks + (ch ^ row_swizzle<kGChunks>(rw))) * 16));
        fb[t] = as_bf16x8(*reinterpret_cast<const u32x4*>(pc + (rc * kGChunks + (ch ^ row_swizzle<kGChunks>(rc))) * 16));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(fa[i], fb[j], acc[i][j]);
    }
    barrier_keep_loads();  // buffer `buf` is refilled in the next iteration
  }

  // out[n][m]: lane (l16, g) holds cache row m = 64 wm + 16 j + l16 and weight
  // rows n = 64 wn + 16 i + 4 g .. + 3, four consecutive columns of one head.
  const int DW = is_k ? G::DN : G::DV;
  uint16_t* dst_base = is_k ? a.kw : a.vw;
  const int nb = is_k ? n0 : n0 - NK;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = 64 * wm + 16 * j + l16;
    if (m >= rows) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = nb + 64 * wn + 16 * i + 4 * g;
      const int h = n / DW, col = n - h * DW;
      uint16_t* dst = dst_base + (((int64_t)b * a.n_head + h) * a.max_rows + m0 + m) * DW + col;
      *reinterpret_cast<uint2*>(dst) = uint2{pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3])};
    }
  }
  if (flags && tid == 0) atomicOr(&a.status[b], flags);
}

// ---------------------------------------------------------------------------
// Causal flash attention over the decompressed rows
// ---------------------------------------------------------------------------
constexpr int kAQ = 128;     // queries per workgroup (16 per wave)
constexpr int kAW = 8;       // waves per attention workgroup
constexpr int kAT = 32;      // cache rows per tile
constexpr int kAStages = 4;  // tile ring: three tiles in flight while one is used

template <int DR>
struct ATile {
  using G = PGeom<DR>;
  static constexpr int DN = G::DN, DV = G::DV;
  static constexpr int KN_CH = DN / 8, KP_CH = DR / 8, V_CH = DV / 8;  // 16-byte chunks of data per row
  // Staged rows.  K_nope and k_pe rows keep their width, with the 16-byte
  // chunks of row r permuted by an XOR with row_swizzle(r); V rows take two
  // pad chunks (34 chunks = 544 bytes, a 32-byte bank shift per row).  Both
  // keep the operand reads free of bank conflicts (measured), and both leave
  // every operand address a lane base plus a constant: the XOR only touches
  // the low 3 (K_nope at 24 chunks, k_pe) or 4 (K_nope at 32 chunks) chunk
  // bits, so each residue of the k-step modulo KB gets a base of its own.
  // V's pad chunks are filled with zeros and never read.
  static constexpr int KN_P = KN_CH, KP_P = KP_CH, V_P = V_CH + 2;
  static constexpr int KB = KN_CH % 16 == 0 ? 4 : 2;          // K_nope lane bases (k-steps per swizzle group)
  static constexpr int KN_LOADS = (kAT * KN_P + 63) / 64;    // 1 KB loads of the K_nope rows
  static constexpr int KP_HALF = (16 * KP_P + 63) / 64;       // loads per 16-row block of k_pe
  static constexpr int KP_LOADS = DR > 0 ? 2 * KP_HALF : 0;
  static constexpr int V_LOADS = (kAT * V_P + 63) / 64;
  static constexpr int USED = KN_LOADS + KP_LOADS + V_LOADS;
  static constexpr int STAGE = USED * 64;                      // chunks per stage
  static constexpr int KP0 = KN_LOADS * 64, V0 = (KN_LOADS + KP_LOADS) * 64;  // region starts (chunks)
  static constexpr int KSTEPS = (DN + DR) / 32, KN_STEPS = DN / 32;
  static_assert(DN % 32 == 0 && DR % 32 == 0, "k-steps of 32 dims");
  // Loads u = w + kAW j: the k_pe loads (fewer than the waves) fall on distinct
  // waves, so a wave needs the block id of one k_pe block at most.
  static_assert(KP_LOADS <= kAW, "one k_pe load per wave at most");
  static_assert(16 * (V0 + 16 * V_P) + 32 * (DV / 16) < 65536, "LDS offsets fit the instruction");
};

// LDS operand reads with a constant offset; the result is not ready until a
// matching lgkm_wait (the compiler does not track these).
template <int OFF>
__device__ __forceinline__ void lds_read_b128(uint32_t addr, u32x4& v) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
}
template <int OFF>
__device__ __forceinline__ void lds_read_tr(uint32_t addr, uint2& v) {
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
}
// Wait until at most N (< 16) LDS operations of this wave are outstanding;
// the registers are tied to the wait so their uses cannot move above it.
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x4& v) {
  static_assert(N >= 0 && N < 16, "lgkmcnt is four bits");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(v) : "i"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void lgkm_wait(uint2& x, uint2& y) {
  static_assert(N >= 0 && N < 16, "lgkmcnt is four bits");
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(x), "+v"(y) : "i"(N) : "memory");
}

// Eight waves per workgroup, 16 queries each, two waves per SIMD: one wave's
// softmax and LDS waits overlap the other's matrix products (256 registers per
// wave at most).  (A four-wave form with 32 queries per wave and one wave per
// SIMD measured the same.)  Query-tile loops run over NQT = 1 tile per wave.
template <int DR>
__global__ __launch_bounds__(64 * kAW, 1) void prefill_attend(const PrefillArgs a) {
  using T = ATile<DR>;
  using G = PGeom<DR>;
  constexpr int NW = kAW;
  constexpr int DN = T::DN, DV = T::DV, D = G::D;
  constexpr int QPW = kAQ / NW, NQT = QPW / 16;  // queries and 16-query tiles per wave
  static_assert(NQT == 1 && kAQ % 16 == 0, "one query tile per wave");
  __shared__ __attribute__((aligned(16))) u32x4 stage[kAStages][T::STAGE];
  __shared__ uint32_t wflags[NW];

  // Workgroup i runs on XCD i % 8: the query tiles of one (request, head)
  // take consecutive slots of one XCD, so they stream the same decompressed
  // rows through one L2 at about the same time; the tiles that see the most
  // rows go first.
  const int n_qt = (a.t_q + kAQ - 1) / kAQ;
  const int slot = blockIdx.x >> 3;
  const int pair = (slot / n_qt) * 8 + (blockIdx.x & 7);
  if (pair >= a.batch * a.n_head) return;  // whole workgroup
  const int b = pair / a.n_head, h = pair - b * a.n_head;
  const int i0 = (n_qt - 1 - (slot - (slot / n_qt) * n_qt)) * kAQ;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int H = a.n_head, t_q = a.t_q;

  const int64_t L = a.seq_lens[b];
  // Length errors, and block-id errors the decompression found for this request.
  uint32_t flags = prefill_flags(L, t_q, a.max_blocks) | a.status[b];
  // Rows the queries of this workgroup may see: [0, vis_end).
  const int i_last = i0 + kAQ - 1 < t_q - 1 ? i0 + kAQ - 1 : t_q - 1;
  const int64_t vis_end = flags ? 0 : L - t_q + i_last + 1;
  const int n_tiles = vis_end > 0 ? (int)((vis_end + kAT - 1) / kAT) : 0;

  // Queries: B operand of S^T = K Q^T.  Lane (l16, g) of query tile n holds
  // query i = i0 + QPW w + 16 n + l16, dims 32 ks + 8 g .. + 7.
  bf16x8 qf[NQT][T::KSTEPS];
  int qi[NQT];
#pragma unroll
  for (int n = 0; n < NQT; ++n) {
    qi[n] = i0 + QPW * w + 16 * n + l16;
    const bool ok = qi[n] < t_q;
    const int64_t row = ((int64_t)b * t_q + (ok ? qi[n] : 0)) * H + h;
#pragma unroll
    for (int ks = 0; ks < T::KSTEPS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ok) {
        const int d = 32 * ks + 8 * g;
        const uint16_t* src = d < DN ? static_cast<const uint16_t*>(a.q_nope) + row * DN + d
                                     : static_cast<const uint16_t*>(a.q_pe) + row * DR + (d - DN);
        v = *reinterpret_cast<const u32x4*>(src);
      }
      qf[n][ks] = as_bf16x8(v);
    }
  }

  // Tile loads.  Load u of a stage fills chunks [64 u, 64 u + 64): loads
  // [0, KN_LOADS) the K_nope rows (pitch KN_P), then KP_HALF loads per 16-row
  // block of k_pe (pitch KP_P), then the V rows (pitch V_P).  Each wave loads
  // from one source, so it builds one buffer resource per tile (the k_pe wave
  // two, one per block): waves 0-3 take the 16 loads of K_nope and k_pe, four
  // consecutive each (k_pe, when present, is wave 3's); waves 4-7 take the V
  // loads u = 16 + (w - 4) + 4 j, wave 4 one more than the others.  The lane
  // offsets do not depend on the tile.
  static_assert(T::KN_LOADS + T::KP_LOADS == 16 && T::KN_LOADS % 4 == 0 && (DR == 0 || T::KP_HALF == 2),
                "four K-side loads per wave of waves 0-3, k_pe (two blocks) on wave 3 only");
  static_assert(T::V_LOADS > 16 && T::V_LOADS <= 20, "V loads: four per wave of waves 4-7, plus at most four");
  constexpr int NLD = 5;                                    // loads of the busiest wave
  const bool kside = w < 4, kpe_w = DR > 0 && w == 3;
  const int nld_w = kside ? 4 : (w - 4 < T::V_LOADS - 16 ? 5 : 4);  // this wave's loads per tile
  auto load_u = [&](int j) { return kside ? 4 * w + j : 16 + (w - 4) + 4 * j; };
  const uint16_t* kw = a.kw + ((int64_t)b * H + h) * a.max_rows * DN;
  const uint16_t* vw = a.vw + ((int64_t)b * H + h) * a.max_rows * DV;
  const uint16_t* kv = static_cast<const uint16_t*>(a.kv);
  constexpr uint32_t kOut = 0x40000000u;  // beyond any buffer range: loads zeros
  uint32_t voffs[NLD];
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    const int u = load_u(j), q = 64 * u + lane;
    uint32_t v = kOut;
    if (j >= nld_w) {
    } else if (u < T::KN_LOADS) {
      const int r = q / T::KN_P, p = q - r * T::KN_P;  // slot p of row r holds chunk p ^ swizzle(r)
      if (r < kAT) v = (uint32_t)(r * DN * 2 + (p ^ row_swizzle<T::KN_CH>(r)) * 16);
    } else if (u < T::KN_LOADS + T::KP_LOADS) {
      if constexpr (DR > 0) {  // (no k_pe loads without a rope part)
        const int ql = q - T::KP0 - ((u - T::KN_LOADS) / T::KP_HALF) * T::KP_HALF * 64;
        const int r = ql / T::KP_P, p = ql - r * T::KP_P;
        if (r < 16) v = (uint32_t)(r * D * 2 + (p ^ row_swizzle<T::KP_CH>(r)) * 16);
      }
    } else if (u < T::USED) {
      const int qv = q - T::V0;
      const int r = qv / T::V_P, p = qv - r * T::V_P;
      if (r < kAT && p < T::V_CH) v = (uint32_t)(r * DV * 2 + p * 16);
    }
    voffs[j] = v;
  }
  // Block ids through scalar loads (the table is read-only for the call), so
  // the vector-memory counter only tracks tile loads.
  typedef __attribute__((address_space(4))) const int32_t const_i32;
  const_i32* bt_s = (const_i32*)(a.bt + (int64_t)b * a.max_blocks);
  const uint32_t nb32 = a.num_blocks < (int64_t)INT32_MAX ? (uint32_t)a.num_blocks : (uint32_t)INT32_MAX;
  // Block ids of tile t (scalar loads), -1 where the tile has no rows there.
  auto load_ids = [&](int t, int32_t (&id)[2]) {
    id[0] = id[1] = -1;
    if constexpr (DR > 0) {
      const int j0 = t * kAT;
      id[0] = bt_s[j0 >> 4];
      if (L - j0 > 16) id[1] = bt_s[(j0 >> 4) + 1];
    }
  };
  auto issue_tile = [&](int t, int buf, const int32_t (&id)[2]) {
    const int j0 = t * kAT;
    const int nval = L - j0 >= kAT ? kAT : (int)(L - j0);  // rows that exist (>= 1)
    const uint32_t base = lds_addr(stage[buf]);
    if (kpe_w) {
      if constexpr (DR > 0) {
        // k_pe of the tile's two blocks (loads 12, 13: block 0; 14, 15: block
        // 1); row r of a block at byte r * D * 2 from its column 512.  This
        // wave checks the ids: the flags of all waves are merged at the end.
        if ((uint32_t)id[0] >= nb32 || (nval > 16 && (uint32_t)id[1] >= nb32)) flags |= kBadBlock;
        i32x4 rs[2];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const int nv = nval - 16 * hb <= 0 ? 0 : (nval - 16 * hb >= 16 ? 16 : nval - 16 * hb);
          const int32_t bid = id[hb];
          const bool ok = (uint32_t)bid < nb32;
          rs[hb] = raw_rsrc(kv + (int64_t)(ok ? bid : 0) * (16 * D) + G::KR,
                            ok && nv > 0 ? (uint32_t)((nv - 1) * D * 2 + DR * 2) : 0u);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) dma16(rs[j / 2], base + 1024u * (uint32_t)(12 + j), voffs[j]);
      }
    } else if (kside) {
      const i32x4 rs_k = raw_rsrc(kw + (int64_t)j0 * DN, (uint32_t)(nval * DN * 2));
#pragma unroll
      for (int j = 0; j < 4; ++j) dma16(rs_k, base + 1024u * (uint32_t)(4 * w + j), voffs[j]);
    } else {
      const i32x4 rs_v = raw_rsrc(vw + (int64_t)j0 * DV, (uint32_t)(nval * DV * 2));
      const uint32_t vbase = base + 1024u * (uint32_t)(16 + (w - 4));
#pragma unroll
      for (int j = 0; j < 4; ++j) dma16(rs_v, vbase + 4096u * (uint32_t)j, voffs[j]);
      if (nld_w > 4) dma16(rs_v, vbase + 4096u * 4u, voffs[4]);
    }
  };
  // Wait until at most K tiles' loads of this wave are outstanding.
  auto wait_tiles = [&](auto k_tiles) {
    constexpr int K = decltype(k_tiles)::value;
    if (nld_w > 4) wait_vmcnt<K * 5>();
    else wait_vmcnt<K * 4>();
  };
  using tiles0 = std::integral_constant<int, 0>;
  using tiles1 = std::integral_constant<int, 1>;
  using tiles2 = std::integral_constant<int, 2>;

  f32x4 acc[DV / 16][NQT];
#pragma unroll
  for (int c = 0; c < DV / 16; ++c)
#pragma unroll
    for (int n = 0; n < NQT; ++n) acc[c][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m2[NQT], lsum[NQT];
#pragma unroll
  for (int n = 0; n < NQT; ++n) m2[n] = -INFINITY, lsum[n] = 0.f;
  const float sl2 = a.scale * kLog2e;
  int horizon[NQT];  // last visible row of each query (inclusive)
#pragma unroll
  for (int n = 0; n < NQT; ++n) horizon[n] = qi[n] < t_q ? (int)(L - t_q + qi[n]) : -1;

  // Lane bases of the operand reads within a stage (bytes).
  //   K (A of S^T), rows 16 kt + l16, dims 32 ks + 8 g: K_nope for
  //   ks < KN_STEPS, then k_pe (block kt).
  //   V^T (A of O^T) for columns 16 dt .. + 15: tile rows 4 g + e and
  //   16 + 4 g + e (the lane's k slots), read transposed.  Provider lane a of
  //   a 16-lane group gives row 4 g + a / 4 (+ 16), columns 16 dt + 4 (a % 4).
  //   Rows 16 kt + l16 share l16's swizzle, so kt is a constant offset.
  uint32_t bk[T::KB], bp[2];
#pragma unroll
  for (int q = 0; q < T::KB; ++q) bk[q] = 16u * (uint32_t)(l16 * T::KN_P + ((4 * q + g) ^ row_swizzle<T::KN_CH>(l16)));
#pragma unroll
  for (int q = 0; q < 2; ++q) bp[q] = DR > 0 ? 16u * (uint32_t)(l16 * T::KP_P + ((4 * q + g) ^ row_swizzle<8>(l16))) : 0u;
  const int vr = 4 * g + (l16 >> 2);
  const uint32_t bv = 16u * (uint32_t)(vr * T::V_P + ((l16 & 3) >> 1)) + 8u * (uint32_t)(l16 & 1);

  // S^T of one tile into sp: the 2 x KSTEPS (k-step, row half) reads run kA
  // steps ahead of the MFMAs, with exact waits.
  constexpr int NS = 2 * T::KSTEPS, kA = 8;
  static_assert(NS > kA && kA < 16, "read-ahead must fit the LDS counter");
  // The S step I also runs piece I of the caller's work (the softmax of the
  // previous tile), so that the vector ALU works while the matrix cores do.
  auto s_tile = [&](uint32_t sb, f32x4 (&sp)[2][NQT], auto&& piece) {
    u32x4 kr[NS];
    auto rd = [&]<int I>() {
      constexpr int ks = I / 2, kt = I % 2;
      if constexpr (ks < T::KN_STEPS)
        lds_read_b128<16 * 16 * T::KN_P * kt + 16 * 4 * T::KB * (ks / T::KB)>(sb + bk[ks % T::KB], kr[I]);
      else
        lds_read_b128<16 * (T::KP0 + kt * T::KP_HALF * 64)>(sb + bp[ks - T::KN_STEPS], kr[I]);
    };
    [&]<int... I>(std::integer_sequence<int, I...>) { (rd.template operator()<I>(), ...); }(
        std::make_integer_sequence<int, kA>{});
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int n = 0; n < NQT; ++n) sp[kt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    [&]<int... I>(std::integer_sequence<int, I...>) {
      (([&] {
         constexpr int ks = I / 2, kt = I % 2;
         constexpr int issued = I + kA < NS ? I + kA : NS;
         lgkm_wait<issued - 1 - I>(kr[I]);
         const bf16x8 kA_ = as_bf16x8(kr[I]);
#pragma unroll
         for (int n = 0; n < NQT; ++n) sp[kt][n] = mfma16x16x32(kA_, qf[n][ks], sp[kt][n]);
         if constexpr (I + kA < NS) rd.template operator()<I + kA>();
         piece.template operator()<I>();
         __builtin_amdgcn_sched_barrier(0);
       }()),
       ...);
    }(std::make_integer_sequence<int, NS>{});
  };
  auto no_piece = []<int I>() {};

  // Software pipeline: the S products of tile t + 1 are independent of the
  // softmax and PV products of tile t.  Ring of kAStages tiles: t (V read by
  // PV), t + 1 (K read by S), t + 2 in flight, t + 3 issued into the buffer
  // tile t - 1 released.
  constexpr int ND = DV / 16, kAV = 6;  // PV column tiles; reads (two each) run kAV tiles ahead
  static_assert(ND > kAV && 2 * kAV < 16, "read-ahead must fit the LDS counter");
  int32_t nid[2];  // block ids of the next tile to issue, loaded one iteration ahead
#pragma unroll
  for (int k = 0; k < kAStages - 1; ++k)
    if (k < n_tiles) {
      load_ids(k, nid);
      issue_tile(k, k, nid);
    }
  if (kAStages - 1 < n_tiles) load_ids(kAStages - 1, nid);
  f32x4 spc[2][NQT];  // raw scores of the current tile
  if (n_tiles > 0) {
    if (n_tiles >= 3) wait_tiles(tiles2{});
    else if (n_tiles == 2) wait_tiles(tiles1{});
    else wait_tiles(tiles0{});
    barrier_keep_loads();  // tile 0 visible
    s_tile(lds_addr(stage[0]), spc, no_piece);
  }
  for (int t = 0; t < n_tiles; ++t) {
    // Tile t + 1 resident: at most the loads of tile t + 2 still outstanding.
    if (t + 2 < n_tiles) wait_tiles(tiles1{});
    else wait_tiles(tiles0{});
    barrier_keep_loads();  // tile t + 1 visible; every wave is past PV of tile t - 1
    if (t + kAStages - 1 < n_tiles) issue_tile(t + kAStages - 1, (t + kAStages - 1) % kAStages, nid);

    // Online softmax of tile t per query (lane column): element e = 4 kt + i
    // is row 16 kt + 4 g + i of the tile.  Eight pieces per query tile, run
    // beside the sixteen S steps (two query tiles: steps 8 n .. 8 n + 7; one:
    // the even steps): pieces 0-3 scale and mask two elements each and keep
    // a running maximum, piece 4 takes the maximum over the four lane rows
    // and moves the reference (delayed by kSlackP), pieces 5-7 form the
    // probabilities, their sum and the packed P^T operand.
    int lim[NQT];  // element e of query tile n is visible when 16 kt + i <= lim[n]
#pragma unroll
    for (int n = 0; n < NQT; ++n) lim[n] = horizon[n] - t * kAT - 4 * g;
    float sc[NQT][8], tmx[NQT], alpha[NQT], m_use[NQT], pr[NQT][8];
    bf16x8 pB[NQT];
    auto sm_piece = [&]<int I>() {
      constexpr int n = NQT == 2 ? I / 8 : 0, k = NQT == 2 ? I % 8 : I / 2;
      if constexpr (NQT == 1 && I % 2 == 1) {
      } else if constexpr (k < 4) {
#pragma unroll
        for (int e = 2 * k; e < 2 * k + 2; ++e) {
          sc[n][e] = 16 * (e / 4) + (e % 4) <= lim[n] ? spc[e / 4][n][e % 4] * sl2 : -INFINITY;
          tmx[n] = e == 0 ? sc[n][0] : fmaxf(tmx[n], sc[n][e]);
        }
      } else if constexpr (k == 4) {
        const float tm = max4rows(tmx[n]);
        const bool grow = tm > m2[n] + kSlackP;
        alpha[n] = grow && m2[n] > -INFINITY ? __builtin_amdgcn_exp2f(m2[n] - tm) : 1.f;
        if (grow) m2[n] = tm;
        m_use[n] = m2[n] == -INFINITY ? 0.f : m2[n];
      } else {
        constexpr int e0 = k == 5 ? 0 : (k == 6 ? 3 : 6), e1 = k == 5 ? 3 : (k == 6 ? 6 : 8);
#pragma unroll
        for (int e = e0; e < e1; ++e) {
          pr[n][e] = __builtin_amdgcn_exp2f(sc[n][e] - m_use[n]);
          asm volatile("" : "+v"(pr[n][e]));  // computed here, not sunk to its use after a branch
        }
        if constexpr (k == 7) {
          const float* q = pr[n];
          lsum[n] = lsum[n] * alpha[n] + (((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7])));
          u32x4 pk = {pack_bf16x2(q[0], q[1]), pack_bf16x2(q[2], q[3]), pack_bf16x2(q[4], q[5]), pack_bf16x2(q[6], q[7])};
          asm volatile("" : "+v"(pk), "+v"(lsum[n]));
          pB[n] = as_bf16x8(pk);
        }
      }
    };

    // S of tile t + 1 beside the softmax of tile t (on the last tile the S
    // products read a stale buffer that no load targets; they are not used).
    f32x4 spn[2][NQT];
    s_tile(lds_addr(stage[(t + 1) % kAStages]), spn, sm_piece);
    // The ids of the tile issued next iteration; the next barrier's wait
    // covers their latency.
    if (t + kAStages < n_tiles) load_ids(t + kAStages, nid);

    const uint32_t vb = lds_addr(stage[t % kAStages]) + bv;
    uint2 vv[ND][2];
    auto rdv = [&]<int DT>() {
      lds_read_tr<16 * T::V0 + 32 * DT>(vb, vv[DT][0]);
      lds_read_tr<16 * (T::V0 + 16 * T::V_P) + 32 * DT>(vb, vv[DT][1]);
    };
    [&]<int... I>(std::integer_sequence<int, I...>) { (rdv.template operator()<I>(), ...); }(
        std::make_integer_sequence<int, kAV>{});
    bool moved = false;
#pragma unroll
    for (int n = 0; n < NQT; ++n) moved |= alpha[n] != 1.f;
    if (__ballot(moved)) {  // rare, uniform
#pragma unroll
      for (int c = 0; c < ND; ++c)
#pragma unroll
        for (int n = 0; n < NQT; ++n) acc[c][n] *= alpha[n];
    }
    [&]<int... I>(std::integer_sequence<int, I...>) {
      (([&] {
         constexpr int issued = I + kAV < ND ? I + kAV : ND;
         lgkm_wait<2 * (issued - 1 - I)>(vv[I][0], vv[I][1]);
         const bf16x8 vA = __builtin_bit_cast(bf16x8, u32x4{vv[I][0].x, vv[I][0].y, vv[I][1].x, vv[I][1].y});
#pragma unroll
         for (int n = 0; n < NQT; ++n) acc[I][n] = mfma16x16x32(vA, pB[n], acc[I][n]);
         if constexpr (I + kAV < ND) rdv.template operator()<I + kAV>();
         __builtin_amdgcn_sched_barrier(0);
       }()),
       ...);
    }(std::make_integer_sequence<int, ND>{});
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int n = 0; n < NQT; ++n) spc[kt][n] = spn[kt][n];
  }

  // Block-id errors are seen by the waves that issued the loads: share them.
  if (lane == 0) wflags[w] = flags;
  __syncthreads();
  flags = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) flags |= wflags[v];
  const bool bad = flags != 0;
  if (tid == 0 && (flags & kBadBlock)) atomicOr(&a.status[b], kBadBlock);

  const f32x4 nan4 = {NAN, NAN, NAN, NAN};
#pragma unroll
  for (int n = 0; n < NQT; ++n) {
    const float l = sum4rows(lsum[n]);
    if (qi[n] >= t_q) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t orow = ((int64_t)b * t_q + qi[n]) * H + h;
    if (g == 0 && a.lse) a.lse[orow] = bad ? NAN : (l > 0.f ? (m2[n] + __log2f(l)) * kLn2 : -INFINITY);
    if (a.out_bf16) {
      uint16_t* o = static_cast<uint16_t*>(a.out) + orow * DV + 4 * g;
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt) {
        const f32x4 v = bad ? nan4 : acc[dt][n] * inv;
        *reinterpret_cast<uint2*>(o + 16 * dt) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    } else {
      float* o = static_cast<float*>(a.out) + orow * DV + 4 * g;
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt) *reinterpret_cast<f32x4*>(o + 16 * dt) = bad ? nan4 : acc[dt][n] * inv;
    }
  }
}

__global__ void prefill_header(const PrefillArgs a) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) {
    a.header[0] = kWorkspaceMagic;
    a.header[1] = (uint32_t)a.batch;
    a.header[2] = 1u;
    a.header[3] = (uint32_t)a.batch;
  }
  if (i < a.batch) a.status[i] = prefill_flags(a.seq_lens[i], a.t_q, a.max_blocks);
}

}  // namespace

PrefillPlan prefill_plan(int n_head, int d_nope, int d_rope, int d_v, int kv_rank, int batch, int max_blocks) {
  PrefillPlan p;
  p.max_rows = max_blocks * 16;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  p.status_off = kHeaderBytes;
  p.kw_off = al(p.status_off + (size_t)(batch > 0 ? batch : 1) * 4);
  const size_t per = (size_t)batch * n_head * p.max_rows;
  p.vw_off = al(p.kw_off + per * (size_t)d_nope * 2);
  p.bytes = al(p.vw_off + per * (size_t)d_v * 2);
  (void)kv_rank;
  (void)d_rope;
  return p;
}

bool prefill_supported(int n_head, int d_nope, int d_rope, int d_v, int kv_rank) {
  return kv_rank == 512 && d_v == 256 && (d_rope == 64 || d_rope == 0) && d_nope + d_rope == 256 &&
         ((int64_t)n_head * d_nope) % kGN == 0 && ((int64_t)n_head * d_v) % kGN == 0;
}

hipError_t launch_prefill(const PrefillArgs& a, int d_rope, hipStream_t stream) {
  hipLaunchKernelGGL(prefill_header, dim3((a.batch + 255) / 256 > 0 ? (a.batch + 255) / 256 : 1), dim3(256), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.batch == 0 || a.t_q == 0) return e;
  PrefillArgs g = a;
  const int n_cols = a.n_head * ((d_rope == 64 ? 192 : 256) + 256);
  g.n_wtiles = n_cols / kGN;
  g.n_mtiles = (a.max_rows + kGM - 1) / kGM;
  g.wgroup = g.n_wtiles < kWeightGroup ? g.n_wtiles : kWeightGroup;
  const int64_t groups = (g.n_wtiles + g.wgroup - 1) / g.wgroup;
  const int64_t n1 = 8 * ((groups + 7) / 8) * (int64_t)a.batch * g.n_mtiles * g.wgroup;
  const int64_t n2 = 8 * (((int64_t)a.batch * a.n_head + 7) / 8) * ((a.t_q + kAQ - 1) / kAQ);
  if (n1 > INT32_MAX || n2 > INT32_MAX) return hipErrorInvalidConfiguration;
  if (d_rope == 64) {
    hipLaunchKernelGGL(prefill_decompress<64>, dim3((unsigned)n1), dim3(256), 0, stream, g);
    hipLaunchKernelGGL(prefill_attend<64>, dim3((unsigned)n2), dim3(64 * kAW), 0, stream, g);
  } else {
    hipLaunchKernelGGL(prefill_decompress<0>, dim3((unsigned)n1), dim3(256), 0, stream, g);
    hipLaunchKernelGGL(prefill_attend<0>, dim3((unsigned)n2), dim3(64 * kAW), 0, stream, g);
  }
  return hipGetLastError();
}

}  // namespace mla
