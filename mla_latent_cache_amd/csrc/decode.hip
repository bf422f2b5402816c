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
// blocks.  One workgroup handles one (request, range, tile of 64 query rows)
// and walks its range 32 rows (two 16-row cache blocks) at a time:
//   * blocks go HBM -> LDS directly (buffer_load ... lds), one buffer resource
//     per block, so rows past the request's end read as zeros and no address
//     outside a real block is formed; a ring of three tile buffers keeps two
//     tiles in flight while one is consumed;
//   * wave (qh, dh) owns query rows [32 qh, 32 qh + 32) of the tile and half
//     dh of the row width: it computes the partial S^T = K Q^T over its half
//     of D with 16x16x32 bf16 MFMA (every K read from LDS feeds two MFMAs),
//     trades partials with its partner wave through LDS, and both partners
//     then hold the same full scores and run the same online softmax;
//   * P^T is already in the B-operand layout of O^T = V^T P^T; wave (qh, dh)
//     accumulates output columns [256 dh, 256 dh + 256) for its 32 query rows,
//     reading V^T from the same LDS tile with the transposing ds_read_b64_tr_b16
//     (again one read per two MFMAs).
// With one range per request the workgroup writes the final output and LSE;
// otherwise it writes (o, lse) partials and decode_merge combines them:
//   M = max_s lse_s, w_s = exp(lse_s - M), o = sum w_s o_s / sum w_s,
//   lse = M + log sum w_s  (all -inf: zeros and -inf).
#include "device_common.hpp"
#include "kernels.hpp"

#include <math.h>

namespace mla {
namespace {

constexpr uint32_t kNegLen = 0x1u, kLenOverTable = 0x2u, kLenBelowTq = 0x4u, kBadBlock = 0x8u;

__device__ __forceinline__ uint32_t request_flags(int64_t L, int t_q, int max_blocks) {
  if (L < 0) return kNegLen;
  if (L > (int64_t)max_blocks * 16) return kLenOverTable;
  if (L > 0 && L < t_q) return kLenBelowTq;
  return 0u;
}

// XCD-aware decode of the linear workgroup id: the m-tiles that share one
// (request, range) -- and so read the same cache blocks -- get the same id
// modulo 8, i.e. land on the same XCD and share its L2.
__device__ __forceinline__ bool decode_item(const DecodeArgs& a, int& b, int& s, int& mt, int& item) {
  const int lin = blockIdx.x;
  const int p_lo = lin & 7;
  const int rest = lin >> 3;
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

// s_waitcnt with vmcnt <= N and no constraint on the other counters.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

// Workgroup barrier that keeps vector-memory loads in flight: it waits only
// for this wave's LDS accesses, unlike __syncthreads(), whose release fence
// also waits for every outstanding global load.  The empty asm statements
// keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_keep_loads() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

constexpr int kIdWindow = 512;  // cache-block ids of a range staged in LDS at a time
constexpr float kSlack = 8.f;   // log2 headroom before the softmax reference moves

// ---------------------------------------------------------------------------
// MFMA split kernel: bf16 queries and cache, kv_rank 512, rope width D_ROPE.
// ---------------------------------------------------------------------------
template <int D_ROPE>
struct Tile {
  static constexpr int KV = 512;
  static constexpr int D = KV + D_ROPE;
  static constexpr int CH = D / 8;                         // 16-byte chunks per row
  static constexpr int STRIDE = CH + 2;                    // LDS row stride: 8 * odd dwords
  static constexpr int BLK_POS = 16 * STRIDE;              // chunk slots of one block image
  static constexpr int BLK_IMG = (BLK_POS + 63) / 64 * 64; // whole wave-loads per block
  static constexpr int BLK_LOADS = BLK_IMG / 64;
  static constexpr int IMG = 2 * BLK_IMG;                  // one 32-row tile
  static constexpr int KSTEPS = D / 32;                    // 32-wide k-steps of S
  static constexpr int KH = KSTEPS / 2;                    // k-steps per half of D
  static constexpr int CTH = KV / 32;                      // 16-column output tiles per half
  static_assert((STRIDE * 4) % 16 == 8, "row stride must be 8 * odd dwords");
  static_assert(KSTEPS % 2 == 0, "D must split into two halves of whole k-steps");
};

template <int D_ROPE>
__global__ __launch_bounds__(256, 1) void decode_split_mfma(const DecodeArgs a) {
  using T = Tile<D_ROPE>;
  constexpr int D = T::D, CH = T::CH, STRIDE = T::STRIDE, KH = T::KH, CTH = T::CTH;
  __shared__ __attribute__((aligned(16))) u32x4 lds0[T::IMG];
  __shared__ __attribute__((aligned(16))) u32x4 lds1[T::IMG];
  __shared__ __attribute__((aligned(16))) u32x4 lds2[T::IMG];
  __shared__ __attribute__((aligned(16))) f32x4 xch[4][4][64];  // S partials: [wave][rt * 2 + n][lane]
  __shared__ int32_t id_lds[kIdWindow];

  write_header(a);
  int b, s, mt, item;
  if (!decode_item(a, b, s, mt, item)) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int qh = w >> 1, dh = w & 1;
  const int l16 = lane & 15, g = lane >> 4;

  const int64_t L = a.seq_lens[b];
  uint32_t flags = request_flags(L, a.t_q, a.max_blocks);
  const int64_t r_begin = (int64_t)s * a.chunk_blocks * 16;
  int64_t r_end = r_begin + (int64_t)a.chunk_blocks * 16;
  if (flags || r_end > L) r_end = flags ? r_begin : L;
  const int n_tiles = r_end > r_begin ? (int)((r_end - r_begin + 31) / 32) : 0;

  // The lane's query rows in the wave's two 16-row tiles n = 0, 1, and how
  // many rows of the range each of them sees (range end and causal horizon).
  int q_row[2], vis_lim[2];
  bool q_ok[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    q_row[n] = mt * kQRowsPerWG + 32 * qh + 16 * n + l16;
    q_ok[n] = q_row[n] < a.n_q;
    const int64_t horizon = L - a.t_q + (q_ok[n] ? q_row[n] / a.n_head : 0) + 1;
    const int64_t vis_end = horizon < r_end ? horizon : r_end;
    vis_lim[n] = !q_ok[n] || vis_end <= r_begin ? 0 : (int)(vis_end - r_begin);
  }

  // B operand of S^T: absorbed queries of both tiles over this wave's half of D.
  bf16x8 qf[2][KH];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.n_q + q_row[n]) * D +
                         32 * KH * dh + 8 * g;
#pragma unroll
    for (int kk = 0; kk < KH; ++kk)
      qf[n][kk] = q_ok[n] ? *reinterpret_cast<const bf16x8*>(qp + 32 * kk) : zero_bf16x8();
  }
  wait_vmcnt<0>();  // queries resident before the tile loop (keeps its waits exact)
  const float sl2 = a.scale * kLog2e;

  f32x4 acc[CTH][2];
#pragma unroll
  for (int c = 0; c < CTH; ++c) acc[c][0] = acc[c][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m2[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};

  const uint16_t* kv = static_cast<const uint16_t*>(a.kv);
  const int32_t* bt_row = a.bt + (int64_t)b * a.max_blocks;

  // Block ids of the range are staged in LDS, kIdWindow at a time, so the loop
  // reads them without a vector-memory wait (which would also wait for the
  // tiles in flight).  Tile t uses range-relative slots 2t and 2t + 1.
  const int slot0 = s * a.chunk_blocks;
  const int nslots = (int)((r_end - r_begin + 15) / 16);
  auto load_ids = [&](int win0) {
    for (int i = tid; i < kIdWindow; i += 256) {
      const int rel = win0 + i;
      id_lds[i] = rel < nslots ? bt_row[slot0 + rel] : -1;
    }
  };
  auto tile_ids = [&](int t, int win0, int32_t* ids) {
    ids[0] = __builtin_amdgcn_readfirstlane(id_lds[2 * t - win0]);
    ids[1] = __builtin_amdgcn_readfirstlane(id_lds[2 * t + 1 - win0]);
  };

  // This wave's share of the 64-chunk wave-loads of one block image, as byte
  // offsets into the block (the same for every block).  Rows 8..15 of a block
  // swap the two 16-byte chunks of each 32-byte pair (bank spreading).
  constexpr int WAVE_LOADS = (T::BLK_LOADS + 3) / 4;
  uint32_t voffs[WAVE_LOADS];
#pragma unroll
  for (int u = 0; u < WAVE_LOADS; ++u) {
    const int pos = (w + 4 * u) * 64 + lane;
    const int rl = pos / STRIDE;
    const int cp = pos - rl * STRIDE;
    voffs[u] = (rl < 16 && cp < CH) ? (uint32_t)(rl * D + ((cp ^ ((rl >> 3) & 1)) * 8)) * 2u : 0x7ffffff0u;
  }
  int c_w = 0;  // this wave's buffer loads per tile (for the vmcnt waits)
#pragma unroll
  for (int u = 0; u < WAVE_LOADS; ++u) c_w += (w + 4 * u < T::BLK_LOADS) ? 2 : 0;

  // Issue the loads of block hb (0 or 1) of tile t (block ids `ids`) into buffer `dst`.
  auto issue_block = [&](int t, int hb, const int32_t* ids, u32x4* dst) {
    const int64_t r0 = r_begin + (int64_t)t * 32;
    {
      const int64_t left = r_end - (r0 + hb * 16);
      const int nvalid = left <= 0 ? 0 : (left >= 16 ? 16 : (int)left);
      const int32_t id = ids[hb];
      const bool ok = id >= 0 && (int64_t)id < a.num_blocks;
      if (nvalid > 0 && !ok) flags |= kBadBlock;
      const uint16_t* base = ok ? kv + (int64_t)id * 16 * D : kv;
      const i32x4 rs = raw_rsrc(base, ok ? (uint32_t)(nvalid * D * 2) : 0u);
      const uint32_t lbase = lds_addr(dst + hb * T::BLK_IMG);
#pragma unroll
      for (int u = 0; u < WAVE_LOADS; ++u) {
        if (w + 4 * u < T::BLK_LOADS) dma16(rs, lbase + (uint32_t)((w + 4 * u) * 64 * 16), voffs[u]);
      }
    }
  };

  // Per-lane LDS offsets.  Tile row r, chunk c lives at chunk slot
  // (r / 16) * BLK_IMG + (r % 16) * STRIDE + (c ^ sw), sw = ((r % 16) >> 3) & 1;
  // sw only flips bit 0, so every address below is a lane base plus a constant.
  // K (A operand of S^T) for k-step kk of half dh: row l16 (+16 rt), chunk 4 (KH dh + kk) + g.
  const int sw_k = (l16 >> 3) & 1;
  const int k_base = l16 * STRIDE + ((4 * KH * dh + g) ^ sw_k);
  // V^T (A operand of O^T) for column tile ct of half dh: rows rr and 16 + rr,
  // columns 256 dh + 16 ct + 4 (l16 % 4) .. + 3.
  const int rr = 4 * g + (l16 >> 2);
  const int sw_v = (rr >> 3) & 1;
  const int v_base = (rr * STRIDE + ((32 * dh + ((l16 & 3) >> 1)) ^ sw_v)) * 16 + (l16 & 1) * 8;  // bytes

  auto consume = [&](const u32x4* src, int t, bool more, const int32_t* nids, u32x4* nxt) {
    // Partial S^T over this wave's half of D: sp[rt][n] for row half rt and
    // query tile n.  K reads run one group of KG k-steps ahead of the MFMAs.
    constexpr int KG = KH % 3 == 0 ? 3 : 4;
    constexpr int NKG = KH / KG;
    static_assert(KH % KG == 0, "k-step groups must tile half of D");
    f32x4 sp[2][2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) sp[rt][0] = sp[rt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 kk[2][2][KG];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int u = 0; u < KG; ++u) kk[0][rt][u] = src[rt * T::BLK_IMG + k_base + 4 * u];
#pragma unroll
    for (int kg = 0; kg < NKG; ++kg) {
      if (kg + 1 < NKG) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int u = 0; u < KG; ++u)
            kk[(kg + 1) & 1][rt][u] = src[rt * T::BLK_IMG + k_base + 4 * ((kg + 1) * KG + u)];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < KG; ++u)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int n = 0; n < 2; ++n)
            sp[rt][n] = mfma16x16x32(as_bf16x8(kk[kg & 1][rt][u]), qf[n][kg * KG + u], sp[rt][n]);
      // The next tile's loads go out between MFMA groups, so a stall on the
      // memory queue overlaps the MFMAs already issued.
      if (more && kg < 2) issue_block(t + 2, kg, nids, nxt);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Trade partials with the partner wave (other half of D).  Both partners
    // form partial(0) + partial(1) with one commutative add, so they hold
    // bitwise identical scores.
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int n = 0; n < 2; ++n) xch[w][rt * 2 + n][lane] = sp[rt][n];
    barrier_keep_loads();
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int n = 0; n < 2; ++n) sp[rt][n] += xch[w ^ 1][rt * 2 + n][lane];

    // Online softmax per query tile.  The exponent reference m2 moves only when
    // a tile max exceeds it by more than kSlack (log2 units): probabilities stay
    // below 2^kSlack, the accumulator is rescaled rarely, and acc / l and
    // lse = m2 + log2(l) do not depend on the reference.
    u32x4 pp[2];
    float alpha[2];
    bool any_rescale = false;
    // Masking is needed only where some query of the wave sees part of the tile.
    const bool partial = __ballot(t * 32 + 32 > (vis_lim[0] < vis_lim[1] ? vis_lim[0] : vis_lim[1])) != 0;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      float sc[2][4];
      float tmax = -INFINITY;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = t * 32 + rt * 16 + 4 * g + i;
          sc[rt][i] = sp[rt][n][i] * sl2;
          if (partial && j >= vis_lim[n]) sc[rt][i] = -INFINITY;
          tmax = fmaxf(tmax, sc[rt][i]);
        }
      tmax = max4rows(tmax);
      const bool grow = tmax > m2[n] + kSlack;
      const bool rescale = grow && m2[n] > -INFINITY;
      alpha[n] = rescale ? __builtin_amdgcn_exp2f(m2[n] - tmax) : 1.f;
      any_rescale |= rescale;
      if (grow) m2[n] = tmax;
      const float m_use = m2[n] == -INFINITY ? 0.f : m2[n];
      float p[2][4];
      float psum = 0.f;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[rt][i] = __builtin_amdgcn_exp2f(sc[rt][i] - m_use);
          psum += p[rt][i];
        }
      lsum[n] = lsum[n] * alpha[n] + psum;
      pp[n] = u32x4{pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                    pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3])};
    }
    if (__ballot(any_rescale)) {
#pragma unroll
      for (int c = 0; c < CTH; ++c) {
        acc[c][0] *= alpha[0];
        acc[c][1] *= alpha[1];
      }
    }
    const bf16x8 pB0 = as_bf16x8(pp[0]), pB1 = as_bf16x8(pp[1]);

    // O^T += V^T P^T for this wave's 16 column tiles; one transposed V read
    // pair feeds the MFMAs of both query tiles.
    const char* vb = reinterpret_cast<const char*>(src) + v_base;
    constexpr int CG = 4;  // column tiles per read group
    s16x4 vv[2][CG][2];
#pragma unroll
    for (int u = 0; u < CG; ++u) {
      vv[0][u][0] = lds_read_tr16(vb + u * 32);
      vv[0][u][1] = lds_read_tr16(vb + T::BLK_IMG * 16 + u * 32);
    }
#pragma unroll
    for (int cg = 0; cg < CTH / CG; ++cg) {
      if (cg + 1 < CTH / CG) {
#pragma unroll
        for (int u = 0; u < CG; ++u) {
          const int ct = (cg + 1) * CG + u;
          vv[(cg + 1) & 1][u][0] = lds_read_tr16(vb + ct * 32);
          vv[(cg + 1) & 1][u][1] = lds_read_tr16(vb + T::BLK_IMG * 16 + ct * 32);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < CG; ++u) {
        const bf16x8 vA = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(vv[cg & 1][u][0], vv[cg & 1][u][1], 0, 1, 2, 3, 4, 5, 6, 7));
        acc[cg * CG + u][0] = mfma16x16x32(vA, pB0, acc[cg * CG + u][0]);
        acc[cg * CG + u][1] = mfma16x16x32(vA, pB1, acc[cg * CG + u][1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Wait until at most k tiles issued after the current one are still loading.
  auto wait_tiles = [&](int k) {
    switch (k * c_w) {
      case 10: wait_vmcnt<10>(); break;
      case 9: wait_vmcnt<9>(); break;
      case 8: wait_vmcnt<8>(); break;
      default: wait_vmcnt<0>(); break;
    }
  };

  int win0 = 0;
  if (n_tiles > 0) {
    load_ids(0);
    __syncthreads();
  }
  int32_t ids[2];
  if (n_tiles > 0) {
    tile_ids(0, win0, ids);
    issue_block(0, 0, ids, lds0);
    issue_block(0, 1, ids, lds0);
  }
  if (n_tiles > 1) {
    tile_ids(1, win0, ids);
    issue_block(1, 0, ids, lds1);
    issue_block(1, 1, ids, lds1);
  }
  // One pipeline step: tile t is consumed from `cur` while tile t + 2 is issued into `nxt`.
  auto step = [&](int t, const u32x4* cur, u32x4* nxt) {
    wait_tiles(n_tiles - 1 - t > 0 ? 1 : 0);
    barrier_keep_loads();
    const bool more = t + 2 < n_tiles;
    if (more) {
      if (2 * (t + 2) + 1 >= win0 + kIdWindow) {  // next window of block ids (drains the loads in flight)
        win0 = 2 * (t + 2);
        load_ids(win0);
        __syncthreads();
      }
      tile_ids(t + 2, win0, ids);
    }
    consume(cur, t, more, ids, nxt);
  };
  for (int t = 0; t < n_tiles; t += 3) {
    step(t, lds0, lds2);
    if (t + 1 < n_tiles) step(t + 1, lds1, lds0);
    if (t + 2 < n_tiles) step(t + 2, lds2, lds1);
  }

  const bool bad = flags != 0;
  float inv[2], lse_v[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    lsum[n] = sum4rows(lsum[n]);
    inv[n] = lsum[n] > 0.f ? 1.f / lsum[n] : 0.f;
    lse_v[n] = bad ? NAN : (lsum[n] > 0.f ? (m2[n] + __log2f(lsum[n])) * kLn2 : -INFINITY);
  }
  const f32x4 nan4 = {NAN, NAN, NAN, NAN};
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    if (!q_ok[n]) continue;
    const int64_t qrow = (int64_t)b * a.n_q + q_row[n];
    const int col0 = 256 * dh + 4 * g;
    if (a.direct) {
      if (a.out_bf16) {
        uint16_t* o = static_cast<uint16_t*>(a.out) + qrow * T::KV + col0;
#pragma unroll
        for (int ct = 0; ct < CTH; ++ct) {
          const f32x4 v = bad ? nan4 : acc[ct][n] * inv[n];
          const uint2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *reinterpret_cast<uint2*>(o + 16 * ct) = pk;
        }
      } else {
        float* o = static_cast<float*>(a.out) + qrow * T::KV + col0;
#pragma unroll
        for (int ct = 0; ct < CTH; ++ct) *reinterpret_cast<f32x4*>(o + 16 * ct) = bad ? nan4 : acc[ct][n] * inv[n];
      }
      if (a.lse && dh == 0 && g == 0) a.lse[qrow] = lse_v[n];
    } else {
      const int64_t prow = ((int64_t)b * a.splits + s) * a.n_q + q_row[n];
      float* o = a.o_part + prow * T::KV + col0;
#pragma unroll
      for (int ct = 0; ct < CTH; ++ct) *reinterpret_cast<f32x4*>(o + 16 * ct) = bad ? nan4 : acc[ct][n] * inv[n];
      if (dh == 0 && g == 0) a.lse_part[prow] = lse_v[n];
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

  const int64_t L = a.seq_lens[b];
  uint32_t flags = request_flags(L, a.t_q, a.max_blocks);
  const int64_t r_begin = (int64_t)s * a.chunk_blocks * 16;
  int64_t r_end = r_begin + (int64_t)a.chunk_blocks * 16;
  if (flags || r_end > L) r_end = flags ? r_begin : L;
  const int64_t horizon = L - a.t_q + q / a.n_head + 1;
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
// Merge of the split partials: one workgroup of 128 threads per query row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void decode_merge(const DecodeArgs a) {
  __shared__ float wts[kMaxSplits];
  __shared__ float red[2];
  const int64_t qrow = blockIdx.x;  // b * n_q + q
  const int b = (int)(qrow / a.n_q);
  const int q = (int)(qrow - (int64_t)b * a.n_q);
  const int tid = threadIdx.x;
  const int S = a.splits, R = a.kv_rank;
  const float* lp = a.lse_part + (int64_t)b * S * a.n_q + q;

  float mx = -INFINITY;
  bool nan_seen = false;
  for (int k = tid; k < S; k += 128) {
    const float v = lp[(int64_t)k * a.n_q];
    nan_seen |= isnan(v);
    mx = fmaxf(mx, v);
  }
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  const int any_nan = __syncthreads_or(nan_seen ? 1 : 0);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  const float M = fmaxf(red[0], red[1]);
  __syncthreads();

  float wsum_part = 0.f;
  for (int k = tid; k < S; k += 128) {
    const float wk = M == -INFINITY ? 0.f : expf(lp[(int64_t)k * a.n_q] - M);
    wts[k] = wk;
    wsum_part += wk;
  }
  for (int off = 32; off > 0; off >>= 1) wsum_part += __shfl_xor(wsum_part, off, 64);
  if ((tid & 63) == 0) red[tid >> 6] = wsum_part;
  __syncthreads();
  const float wsum = red[0] + red[1];
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;

  const float* op = a.o_part + ((int64_t)b * S * a.n_q + q) * R;
  const int64_t sstride = (int64_t)a.n_q * R;
  for (int c0 = tid * 4; c0 < R; c0 += 128 * 4) {
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    if (R - c0 >= 4) {
      for (int k = 0; k < S; ++k) {
        const float wk = wts[k];
        if (wk != 0.f) o += wk * *reinterpret_cast<const f32x4*>(op + k * sstride + c0);
      }
    } else {
      for (int k = 0; k < S; ++k)
        for (int e = 0; c0 + e < R; ++e) o[e] += wts[k] * op[k * sstride + c0 + e];
    }
    for (int e = 0; e < 4 && c0 + e < R; ++e) {
      const float v = any_nan ? NAN : o[e] * inv;
      if (a.out_bf16) static_cast<uint16_t*>(a.out)[qrow * R + c0 + e] = f32_to_bf16(v);
      else static_cast<float*>(a.out)[qrow * R + c0 + e] = v;
    }
  }
  if (tid == 0 && a.lse) a.lse[qrow] = any_nan ? NAN : (M == -INFINITY ? -INFINITY : M + logf(wsum));
}

}  // namespace

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
  p.n_pairs = batch * p.splits;
  p.n_items = p.n_pairs * p.m_tiles;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t status_bytes = al((size_t)(p.n_items > 0 ? p.n_items : 1) * 4);
  p.lse_off = kHeaderBytes + status_bytes;
  const size_t parts = (size_t)batch * p.splits * n_q;
  p.o_off = al(p.lse_off + parts * 4);
  p.bytes = p.splits > 1 ? al(p.o_off + parts * (size_t)kv_rank * 4) : p.lse_off;
  return p;
}

hipError_t launch_decode(const DecodeArgs& a, bool mfma, bool bf16, hipStream_t stream) {
  const int groups = (a.n_pairs + 7) / 8;
  const int grid = (groups > 0 ? groups : 1) * 8 * a.m_tiles;
  if (mfma) {
    if (a.d_rope == 64)
      hipLaunchKernelGGL(decode_split_mfma<64>, dim3(grid), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(decode_split_mfma<0>, dim3(grid), dim3(256), 0, stream, a);
  } else if (bf16) {
    hipLaunchKernelGGL(decode_split_generic<uint16_t>, dim3(grid), dim3(128), 0, stream, a);
  } else {
    hipLaunchKernelGGL(decode_split_generic<float>, dim3(grid), dim3(128), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.direct || a.batch == 0) return e;
  hipLaunchKernelGGL(decode_merge, dim3((unsigned)((int64_t)a.batch * a.n_q)), dim3(128), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
