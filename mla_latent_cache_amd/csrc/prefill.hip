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
//   * prefill_attend: flash attention per (request, head, 128 queries); four
//     waves of 32 queries each.  Tiles of 32 rows -- K_nope and V from the
//     workspace, k_pe straight from the paged cache (shared by all heads) --
//     go HBM -> LDS by LDS-DMA, double-buffered.  S^T = K Q^T with the queries
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

template <int DR>
__global__ __launch_bounds__(256, 2) void prefill_decompress(const PrefillArgs a) {
  using G = PGeom<DR>;
  constexpr int KR = G::KR, D = G::D;
  __shared__ __attribute__((aligned(16))) u32x4 sw[2][kGN * kGChunks];  // weight rows [128][64]
  __shared__ __attribute__((aligned(16))) u32x4 sc[2][kGM * kGChunks];  // cache rows [128][64]

  const int b = blockIdx.z;
  const int m0 = blockIdx.y * kGM, n0 = blockIdx.x * kGN;
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
constexpr int kAQ = 128;  // queries per workgroup (32 per wave)
constexpr int kAT = 32;   // cache rows per tile

template <int DR>
struct ATile {
  using G = PGeom<DR>;
  static constexpr int DN = G::DN, DV = G::DV;
  static constexpr int KN_CH = DN / 8, KP_CH = DR / 8, V_CH = DV / 8;  // 16-byte chunks per row
  static constexpr int KN = kAT * KN_CH, KP = kAT * KP_CH, VV = kAT * V_CH;  // chunks per tile
  static constexpr int STAGE = KN + KP + VV;                                    // chunks per stage
  static constexpr int LOADS = STAGE / 64;                                      // 1 KB loads per stage
  static_assert(KN % 64 == 0 && KP % 64 == 0 && VV % 64 == 0 && LOADS % 4 == 0, "whole loads per wave");
  static constexpr int KSTEPS = (DN + DR) / 32;
};

template <int DR>
__global__ __launch_bounds__(256, 1) void prefill_attend(const PrefillArgs a) {
  using T = ATile<DR>;
  using G = PGeom<DR>;
  constexpr int DN = T::DN, DV = T::DV, D = G::D;
  __shared__ __attribute__((aligned(16))) u32x4 stage[2][T::STAGE];
  __shared__ uint32_t wflags[4];

  const int b = blockIdx.z, h = blockIdx.y, i0 = blockIdx.x * kAQ;
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
  // query i = i0 + 32 w + 16 n + l16, dims 32 ks + 8 g .. + 7.
  bf16x8 qf[2][T::KSTEPS];
  int qi[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    qi[n] = i0 + 32 * w + 16 * n + l16;
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

  // Tile loads.  Stage layout (16-byte chunks): K_nope rows [0, KN), k_pe rows
  // [KN, KN + KP), V rows [KN + KP, STAGE).  Load u (of LOADS) covers chunks
  // [64 u, 64 u + 64); wave w issues loads u = w + 4 j.
  const uint16_t* kw = a.kw + ((int64_t)b * H + h) * a.max_rows * DN;
  const uint16_t* vw = a.vw + ((int64_t)b * H + h) * a.max_rows * DV;
  const uint16_t* kv = static_cast<const uint16_t*>(a.kv);
  // Block ids through scalar loads (the table is read-only for the call), so
  // the vector-memory counter only tracks tile loads.
  typedef __attribute__((address_space(4))) const int32_t const_i32;
  const_i32* bt_s = (const_i32*)(a.bt + (int64_t)b * a.max_blocks);
  const uint32_t nb32 = a.num_blocks < (int64_t)INT32_MAX ? (uint32_t)a.num_blocks : (uint32_t)INT32_MAX;
  auto issue_tile = [&](int t, int buf) {
    const int j0 = t * kAT;
    const int nval = L - j0 >= kAT ? kAT : (int)(L - j0);  // rows that exist (>= 1)
    const i32x4 rs_k = raw_rsrc(kw + (int64_t)j0 * DN, (uint32_t)(nval * DN * 2));
    const i32x4 rs_v = raw_rsrc(vw + (int64_t)j0 * DV, (uint32_t)(nval * DV * 2));
    i32x4 rs_p[2];
    if constexpr (DR > 0) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int nv = nval - 16 * hb <= 0 ? 0 : (nval - 16 * hb >= 16 ? 16 : nval - 16 * hb);
        int32_t id = -1;
        if (nv > 0) id = bt_s[(j0 >> 4) + hb];
        const bool ok = (uint32_t)id < nb32;
        if (nv > 0 && !ok) flags |= kBadBlock;
        // k_pe of row r of the block at byte r * D * 2 from the block's column 512
        rs_p[hb] = raw_rsrc(kv + (int64_t)(ok ? id : 0) * (16 * D) + G::KR,
                            ok && nv > 0 ? (uint32_t)((nv - 1) * D * 2 + DR * 2) : 0u);
      }
    }
    const uint32_t base = lds_addr(stage[buf]);
#pragma unroll
    for (int j = 0; j < T::LOADS / 4; ++j) {
      const int u = w + 4 * j;
      const int unit = 64 * u + lane;  // chunk of the stage
      uint32_t voff;
      if (u * 64 < T::KN) {
        const int r = unit / T::KN_CH, p = unit - r * T::KN_CH;
        voff = (uint32_t)(r * DN * 2 + (p ^ row_swizzle<T::KN_CH>(r)) * 16);
        dma16(rs_k, base + 1024u * u, voff);
      } else if (DR > 0 && u * 64 < T::KN + T::KP) {
        if constexpr (DR > 0) {
          const int pu = unit - T::KN;
          const int r = pu / T::KP_CH, p = pu - r * T::KP_CH;
          voff = (uint32_t)((r & 15) * D * 2 + (p ^ row_swizzle<T::KP_CH>(r)) * 16);
          // the 8 rows of one load lie in one block
          const int blk = ((u * 64 - T::KN) / T::KP_CH) >> 4;
          dma16(blk ? rs_p[1] : rs_p[0], base + 1024u * u, voff);
        }
      } else {
        const int vu = unit - T::KN - T::KP;
        const int r = vu / T::V_CH, p = vu - r * T::V_CH;
        voff = (uint32_t)(r * DV * 2 + (p ^ (2 * (r & 7))) * 16);
        dma16(rs_v, base + 1024u * u, voff);
      }
    }
  };

  f32x4 acc[DV / 16][2];
#pragma unroll
  for (int c = 0; c < DV / 16; ++c) acc[c][0] = acc[c][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m2[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};
  const float sl2 = a.scale * kLog2e;
  int horizon[2];  // last visible row of each query (inclusive)
#pragma unroll
  for (int n = 0; n < 2; ++n) horizon[n] = qi[n] < t_q ? (int)(L - t_q + qi[n]) : -1;

  // K operand (A of S^T): row 16 kt + l16 of the tile, dims 32 ks + 8 g.
  auto k_frag = [&](const char* st, int kt, int ks) {
    const int r = 16 * kt + l16;
    const int ch = 4 * ks + g;
    if (32 * ks < DN) {
      return as_bf16x8(*reinterpret_cast<const u32x4*>(st + (r * T::KN_CH + (ch ^ row_swizzle<T::KN_CH>(r))) * 16));
    } else {
      const int cp = ch - T::KN_CH;
      return as_bf16x8(*reinterpret_cast<const u32x4*>(st + (T::KN + r * T::KP_CH + (cp ^ row_swizzle<T::KP_CH>(r))) * 16));
    }
  };
  // V^T (A of O^T) for value columns 16 dt .. + 15: tile rows 4 g + e and
  // 16 + 4 g + e (the lane's k slots), read transposed.  Provider lane a of a
  // 16-lane group gives row 4 g + a / 4 (+ 16), columns 16 dt + 4 (a % 4).
  const int vr = 4 * g + (l16 >> 2);
  auto v_frag = [&](const char* st, int dt) {
    const char* vb = st + (T::KN + T::KP) * 16;
    const int c = 2 * dt + ((l16 & 3) >> 1);  // chunk of columns 16 dt + 4 (l16 % 4)
    const s16x4 v0 = lds_read_tr16(vb + (vr * T::V_CH + (c ^ (2 * (vr & 7)))) * 16 + (l16 & 1) * 8);
    const int vr1 = vr + 16;
    const s16x4 v1 = lds_read_tr16(vb + (vr1 * T::V_CH + (c ^ (2 * (vr1 & 7)))) * 16 + (l16 & 1) * 8);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  if (n_tiles > 0) issue_tile(0, 0);
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    wait_vmcnt<0>();       // this wave's loads of tile t are done
    barrier_keep_loads();  // tile t visible; every wave is past tile t - 1
    // Buffer buf ^ 1 held tile t - 1, which no wave reads any more.
    if (t + 1 < n_tiles) issue_tile(t + 1, buf ^ 1);
    const char* st = reinterpret_cast<const char*>(stage[buf]);

    // S^T for the tile's two 16-row halves and this wave's two query tiles.
    f32x4 sp[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) sp[kt][0] = sp[kt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < T::KSTEPS; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 kA = k_frag(st, kt, ks);
        sp[kt][0] = mfma16x16x32(kA, qf[0][ks], sp[kt][0]);
        sp[kt][1] = mfma16x16x32(kA, qf[1][ks], sp[kt][1]);
      }
      // bound how far operand reads are hoisted (register budget of two waves per SIMD)
      if (ks % 2 == 1) __builtin_amdgcn_sched_barrier(0);
    }

    // Online softmax per query (lane column), rows 16 kt + 4 g + i.
    bf16x8 pB[2];
    float alpha[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      float tmax = -INFINITY;
      float sc[2][4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = t * kAT + 16 * kt + 4 * g + i;
          sc[kt][i] = j <= horizon[n] ? sp[kt][n][i] * sl2 : -INFINITY;
          tmax = fmaxf(tmax, sc[kt][i]);
        }
      tmax = max4rows(tmax);
      const bool grow = tmax > m2[n] + kSlackP;
      alpha[n] = grow && m2[n] > -INFINITY ? __builtin_amdgcn_exp2f(m2[n] - tmax) : 1.f;
      if (grow) m2[n] = tmax;
      const float m_use = m2[n] == -INFINITY ? 0.f : m2[n];
      float p[2][4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[kt][i] = __builtin_amdgcn_exp2f(sc[kt][i] - m_use);
      lsum[n] = lsum[n] * alpha[n] + (((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) + ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3])));
      pB[n] = as_bf16x8(u32x4{pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                              pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3])});
    }
    if (__ballot(alpha[0] != 1.f || alpha[1] != 1.f)) {
#pragma unroll
      for (int c = 0; c < DV / 16; ++c) {
        acc[c][0] *= alpha[0];
        acc[c][1] *= alpha[1];
      }
    }
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) {
      const bf16x8 vA = v_frag(st, dt);
      acc[dt][0] = mfma16x16x32(vA, pB[0], acc[dt][0]);
      acc[dt][1] = mfma16x16x32(vA, pB[1], acc[dt][1]);
      if (dt % 4 == 3) __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Block-id errors are seen by the waves that issued the loads: share them.
  if (lane == 0) wflags[w] = flags;
  __syncthreads();
  flags = wflags[0] | wflags[1] | wflags[2] | wflags[3];
  const bool bad = flags != 0;
  if (tid == 0 && (flags & kBadBlock)) atomicOr(&a.status[b], kBadBlock);

  const f32x4 nan4 = {NAN, NAN, NAN, NAN};
#pragma unroll
  for (int n = 0; n < 2; ++n) {
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
  const int n_cols = a.n_head * ((d_rope == 64 ? 192 : 256) + 256);
  const dim3 g1(n_cols / kGN, (a.max_rows + kGM - 1) / kGM, a.batch);
  const dim3 g2((a.t_q + kAQ - 1) / kAQ, a.n_head, a.batch);
  if (d_rope == 64) {
    hipLaunchKernelGGL(prefill_decompress<64>, g1, dim3(256), 0, stream, a);
    hipLaunchKernelGGL(prefill_attend<64>, g2, dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(prefill_decompress<0>, g1, dim3(256), 0, stream, a);
    hipLaunchKernelGGL(prefill_attend<0>, g2, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace mla
