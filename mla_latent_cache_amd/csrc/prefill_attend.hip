// Causal flash attention of the naive-form MLA prefill over the decompressed
// rows, for gfx950 (memra-engine "mla.rs", mla_attend_naive; MlaInputs
// causal rule): per request b, head h and new query i < t_q,
//   s_j = scale * (<q_nope, k_nope_j> + <q_pe, k_pe_j>),
//   out = sum_j softmax(s)_j v_j over the visible rows j <= L - t_q + i,
// with k_nope_j and v_j the rows prefill_decompress wrote into the workspace
// and k_pe_j read straight from the paged cache (shared by all heads).
//
// Workgroup: one (request, head) and 256 queries, eight waves of 32 queries,
// two per SIMD.  Tiles of 32 rows go HBM -> LDS by LDS-DMA (36 copies of 1 KB
// per tile, dealt over the waves) through a ring of four images, three tiles
// in flight.  S^T = K Q^T and O^T = V^T P^T are 32x32x16 bf16 products with
// the wave's 32 queries as N: the queries stay in registers, each 16-byte K
// read and each pair of transposing V^T reads feeds all 32 queries, and the
// probabilities leave S^T already in the B layout of O^T.  Online softmax
// with a delayed reference maximum.  One barrier per tile: every wave owns
// whole queries, so nothing is exchanged.
#include <math.h>

#include "prefill_common.hpp"

namespace mla {
namespace {

using namespace prefill;

constexpr float kSlackP = 8.f;  // log2 headroom before the softmax reference moves

// ---------------------------------------------------------------------------
// Causal flash attention over the decompressed rows
// ---------------------------------------------------------------------------
constexpr int kQW = 32;          // queries per wave (the 32 columns of the products)
constexpr int kAW = 8;           // waves per attention workgroup, two per SIMD
constexpr int kAQ = kQW * kAW;   // queries per workgroup
constexpr int kAT = 32;          // cache rows per tile
constexpr int kRingT = 4;        // tile ring: three tiles in flight while one is used
constexpr int kCopies = 36;      // 1 KB tile copies per tile: waves 0-3 take five, waves 4-7 four
constexpr int kCopiesMax = 5;

// LDS image of one 32-row tile, filled by 36 copies of 1 KB (five or four per wave):
// the K_nope rows at a pitch of one 16-byte chunk more than the row (25 or
// 33 chunks), then the k_pe rows of the tile's two cache blocks (pitch 9, three
// copies per block; two idle copies without a rope part), then the V rows
// (pitch 33).  An odd pitch puts one chunk of any 16 rows on 16 distinct bank
// groups, which the operand reads below rely on.  Padding slots read zeros.
template <int DR>
struct PTile {
  static constexpr int DN = 256 - DR, DV = 256;
  static constexpr int KC = DN / 8, KP = KC + 1;     // K_nope chunks per row, pitch
  static constexpr int IK = (kAT * KP + 63) / 64;     // K_nope copies
  static constexpr int IP = DR ? 6 : 2;               // k_pe copies (or idle ones)
  static constexpr int VP = DV / 8 + 1;               // V pitch
  static constexpr int IV = (kAT * VP + 63) / 64;     // V copies
  static constexpr int PE0 = 64 * IK, V0 = 64 * (IK + IP);  // region starts (chunks)
  static constexpr int SLOTS = 64 * (IK + IP + IV);  // chunks per image
  static constexpr int KSN = DN / 16;                 // k-steps of q.k over K_nope (16 in all)
  static_assert(IK + IP + IV == kCopies, "36 copies per tile");
  static_assert(DR == 0 || DR == 64, "rope width");
  // Source of copy u: 0 K_nope, 1 / 2 k_pe of block 0 / 1, 3 V, 4 idle.
  static constexpr int source(int u) {
    return u < IK ? 0 : (u < IK + IP ? (DR ? 1 + (u - IK) / 3 : 4) : 3);
  }
  // The source of copy j of every wave that has one (u = w + 8 j < 36), or -1 where the waves differ.
  static constexpr int common_source(int j) {
    const int last = 8 * j + 7 < kCopies ? 8 * j + 7 : kCopies - 1;
    for (int u = 8 * j; u <= last; ++u)
      if (source(u) != source(8 * j)) return -1;
    return source(8 * j);
  }
};

// Tile row that output row i (0..31) of S^T = K Q^T stands for.  Output rows
// 4a .. 4a + 3 (the rows a transposing V^T read covers in one k-slot group)
// map to rows 4 b + a % 4 + 16 (a / 4), b = 0..3, which the odd pitches place
// on four distinct groups of four banks.
__host__ __device__ constexpr int out_row_pos(int i) { return 16 * (i >> 4) + 4 * (i & 3) + ((i >> 2) & 3); }

// Eight waves of 32 queries per (request, head, 256 queries), two per SIMD.
// Wave w owns queries i0 + 32 w .. + 31 over the full width: S^T = K Q^T and
// O^T = V^T P^T are 32x32x16 bf16 products with the tile rows / value
// columns as the M dimension and the wave's queries as N, so every 16-byte K
// read and every pair of transposing V^T reads feeds one 32-query product,
// the queries (B of S^T) stay in registers, and the probabilities leave S^T
// already in the B layout of O^T (the k order of each 16-row step follows the
// output rows a lane holds).  Online softmax per query against a reference
// that moves only when a tile's maximum exceeds it by more than kSlackP.
template <int DR>
__global__ __launch_bounds__(64 * kAW, 1) void prefill_attend(const PrefillArgs a) {
  using T = PTile<DR>;
  using G = PGeom<DR>;
  constexpr int DN = T::DN, DV = T::DV, D = G::D, KP = T::KP, VP = T::VP;
  constexpr int NCT = DV / 32;  // 32-column output tiles
  __shared__ __attribute__((aligned(16))) u32x4 ring[kRingT][T::SLOTS];

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
  const int j32 = lane & 31, hl = lane >> 5, l16 = lane & 15;
  const int H = a.n_head, t_q = a.t_q;

  const int64_t L = a.seq_lens[b];
  // Length errors, and block-id errors the decompression found for this request.
  uint32_t flags = prefill_flags(L, t_q, a.max_blocks) | a.status[b];
  const int i_last = i0 + kAQ - 1 < t_q - 1 ? i0 + kAQ - 1 : t_q - 1;
  const int64_t vis_end = flags ? 0 : L - t_q + i_last + 1;  // rows [0, vis_end) are seen
  const int n_tiles = vis_end > 0 ? (int)((vis_end + kAT - 1) / kAT) : 0;

  // Tile copies u = w + 8 j of this wave (five for waves 0-3, four for
  // waves 4-7): global byte offset of the lane's 16 bytes within the copy's
  // source.  Padding slots get an offset past any source.
  constexpr uint32_t kOut = 0x7ffffff0u;
  const int n_copies = w < kCopies - 32 ? 5 : 4;
  uint32_t vo[kCopiesMax];
#pragma unroll
  for (int j = 0; j < kCopiesMax; ++j) {
    const int u = w + 8 * j, pos = 64 * u + lane;
    uint32_t v = kOut;
    if (u < T::IK) {
      const int r = pos / KP, c = pos - r * KP;
      if (c < T::KC && r < kAT) v = (uint32_t)(r * DN * 2 + c * 16);
    } else if (u < T::IK + T::IP) {
      if constexpr (DR > 0) {
        const int blk = (u - T::IK) / 3, p = pos - T::PE0 - 192 * blk;
        const int r = p / 9, c = p - r * 9;
        if (c < 8 && r < 16) v = (uint32_t)(r * D * 2 + c * 16);
      }
    } else {
      const int p = pos - T::V0, r = p / VP, c = p - r * VP;
      if (c < DV / 8 && r < kAT) v = (uint32_t)(r * DV * 2 + c * 16);
    }
    vo[j] = v;
  }
  const uint16_t* kw = a.kw + ((int64_t)b * H + h) * a.max_rows * DN;
  const uint16_t* vw = a.vw + ((int64_t)b * H + h) * a.max_rows * DV;
  const uint16_t* kv = static_cast<const uint16_t*>(a.kv);
  typedef __attribute__((address_space(4))) const int32_t const_i32;
  const_i32* bt_s = (const_i32*)(a.bt + (int64_t)b * a.max_blocks);
  const uint32_t nb32 = a.num_blocks < (int64_t)INT32_MAX ? (uint32_t)a.num_blocks : (uint32_t)INT32_MAX;
  const uint32_t ring_base = lds_addr(ring);

  // Block ids of tile t (scalar loads, -1 where the tile has no rows there),
  // read one tile step before the tile is issued.
  int32_t nid[2] = {-1, -1};
  auto load_ids = [&](int t) {
    nid[0] = nid[1] = -1;
    if constexpr (DR > 0) {
      if (t < n_tiles) {
        const int j0 = t * kAT;
        nid[0] = bt_s[j0 >> 4];
        if (vis_end - j0 > 16) nid[1] = bt_s[(j0 >> 4) + 1];
      }
    }
  };
  // Issue tile t into ring slot t % 4; past the last tile the sources are
  // empty and the copies deliver zeros, so every tile step issues the same copies
  // per wave and the waits stay exact.
  auto issue = [&](int t) {
    const int j0 = t * kAT;
    const int nval = t < n_tiles ? (vis_end - j0 >= kAT ? kAT : (int)(vis_end - j0)) : 0;
    const i32x4 rk = raw_rsrc(kw + (int64_t)j0 * DN, (uint32_t)(nval * DN * 2));
    const i32x4 rv = raw_rsrc(vw + (int64_t)j0 * DV, (uint32_t)(nval * DV * 2));
    i32x4 rp[2] = {rk, rk};
    if constexpr (DR > 0) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int nv = nval - 16 * blk <= 0 ? 0 : (nval - 16 * blk >= 16 ? 16 : nval - 16 * blk);
        const int32_t id = nid[blk];
        const bool ok = nv > 0 && (uint32_t)id < nb32;
        if (nv > 0 && !ok) flags |= kBadBlock;
        rp[blk] = raw_rsrc(kv + (int64_t)(ok ? id : 0) * (16 * D) + G::KR,
                           ok ? (uint32_t)((nv - 1) * D * 2 + DR * 2) : 0u);
      }
    }
    const uint32_t base = ring_base + (uint32_t)(t & (kRingT - 1)) * (uint32_t)(T::SLOTS * 16);
    const i32x4 r_idle = raw_rsrc(kv, 0u);
    auto pick = [&](int sr) { return sr == 0 ? rk : (sr == 1 ? rp[0] : (sr == 2 ? rp[1] : (sr == 3 ? rv : r_idle))); };
    static_for<kCopiesMax>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      constexpr int cs = T::common_source(j);
      if (j < 4 || n_copies > 4) {
        const i32x4 rs = cs >= 0 ? pick(cs) : pick(T::source(w + 8 * j));
        dma16(rs, base + 1024u * (uint32_t)(w + 8 * j), vo[j]);
      }
    });
  };

  // Tile 0 and the queries, then tiles 1 and 2 in flight.
  load_ids(0);
  issue(0);
  // The lane's query as B operands of S^T: dims 16 s + 8 hl .. + 7 (q_nope,
  // then q_pe), zero for queries past t_q.
  const int qi = i0 + kQW * w + j32;
  const bool q_ok = qi < t_q;
  bf16x8 qf[16];
  {
    const int64_t row = ((int64_t)b * t_q + (q_ok ? qi : 0)) * H + h;
    const u32x4* qn = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.q_nope) + row * DN + 8 * hl);
#pragma unroll
    for (int s = 0; s < T::KSN; ++s) qf[s] = as_bf16x8(q_ok ? qn[2 * s] : u32x4{0u, 0u, 0u, 0u});
    if constexpr (DR > 0) {
      const u32x4* qp = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.q_pe) + row * DR + 8 * hl);
#pragma unroll
      for (int s = T::KSN; s < 16; ++s) qf[s] = as_bf16x8(q_ok ? qp[2 * (s - T::KSN)] : u32x4{0u, 0u, 0u, 0u});
    }
  }
  wait_vmcnt<0>();
  load_ids(1);
  issue(1);
  load_ids(2);
  issue(2);
  load_ids(3);

  // Per-lane LDS byte offsets within an image.
  //   K (A of S^T), k-step s: output row j32 stands for tile row pr; K_nope
  //   chunk 2 s + hl of it, or k_pe chunk 2 (s - KSN) + hl in its block.
  //   V^T (A of O^T), 32-column tile ct, 16-row step kk, read q: provider lane
  //   l16 addresses tile row 16 kk + 4 (l16 / 4) + 2 q + hl (the output rows
  //   16 kk + 8 q + 4 hl + e, e = l16 / 4) and the 8 bytes of columns
  //   32 ct + 16 (j32 / 16) + 4 (l16 % 4) .. + 3; lane l16 receives column
  //   32 ct + j32 of the four rows.
  const int pr = out_row_pos(j32);
  const uint32_t k_off = (uint32_t)((pr * KP + hl) * 16);
  const uint32_t p_off = (uint32_t)((T::PE0 + 192 * (pr >> 4) + 9 * (pr & 15) + hl) * 16);
  const uint32_t v_off = (uint32_t)((T::V0 + (4 * (l16 >> 2) + hl) * VP + 2 * (j32 >> 4) + ((l16 & 3) >> 1)) * 16 +
                                    (l16 & 1) * 8);

  typedef float f32x16 __attribute__((ext_vector_type(16)));
  f32x16 acc[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = 0.f;
  float m2 = -INFINITY, lsum = 0.f;  // running reference (log2 units) and partial sum of this lane's rows
  const float sl2 = a.scale * kLog2e;
  const int hz = q_ok ? (int)(L - t_q + qi) : -1;  // last visible row of this lane's query

  // K operand k-step s of this lane from the tile image at img.
  auto k_at = [&](const char* img, int s) {
    return s < T::KSN ? *reinterpret_cast<const bf16x8*>(img + k_off + 32 * s)
                      : *reinterpret_cast<const bf16x8*>(img + p_off + 32 * (s - T::KSN));
  };
  constexpr int kKA = 4;  // K reads in flight ahead of their products

  // Step t: tile t resident, t + 1 and t + 2 in flight, t + 3 issued into
  // the slot tile t - 1 released.  S^T (one dependent chain of 16 products,
  // K reads four ahead), the softmax, then O^T with the V^T reads two column
  // tiles ahead.  The other wave of the SIMD fills the gaps of this one.
  for (int t = 0; t < n_tiles; ++t) {
    if (t > 0) {  // tile t resident: tiles t + 1, t + 2 may be in flight
      if (n_copies > 4) wait_vmcnt<10>();
      else wait_vmcnt<8>();
    }
    barrier_keep_loads();  // every wave's copies of tile t visible; every wave is past step t - 1
    issue(t + 3);
    load_ids(t + 4);
    const char* img = reinterpret_cast<const char*>(ring[t & (kRingT - 1)]);

    f32x16 sc;
#pragma unroll
    for (int v = 0; v < 16; ++v) sc[v] = 0.f;
    bf16x8 kr[16];
#pragma unroll
    for (int s = 0; s < kKA; ++s) kr[s] = k_at(img, s);
    static_for<16>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[i], qf[i], sc, 0, 0, 0);
      if constexpr (i + kKA < 16) kr[i + kKA] = k_at(img, i + kKA);
      __builtin_amdgcn_sched_barrier(0);
    });
    s16x4 vr[NCT][2][2];
    auto rd_v = [&](int ct, int kk) {
      vr[ct][kk][0] = lds_read_tr16(img + v_off + (16 * kk * VP + 4 * ct) * 16);
      vr[ct][kk][1] = lds_read_tr16(img + v_off + (16 * kk * VP + 2 * VP + 4 * ct) * 16);
    };
    rd_v(0, 0), rd_v(0, 1), rd_v(1, 0), rd_v(1, 1);

    // Softmax of tile t.  Element v is output row 8 (v / 4) + 4 hl + v % 4,
    // tile row 16 (v / 8) + 4 (v % 4) + 2 ((v / 4) % 2) + hl.
    const int lim = hz - t * kAT - hl;  // element v is visible when its tile row less hl is at most lim
    float x[16], tm = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = 16 * (v >> 3) + 4 * (v & 3) + 2 * ((v >> 2) & 1);
      x[v] = r <= lim ? sc[v] * sl2 : -INFINITY;
      tm = fmaxf(tm, x[v]);
    }
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tm), __float_as_uint(tm), false, false);
      tm = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));  // both lane halves of the query's 32 rows
    }
    const bool grow = tm > m2 + kSlackP;
    const float alpha = grow && m2 > -INFINITY ? __builtin_amdgcn_exp2f(m2 - tm) : 1.f;
    m2 = grow ? tm : m2;
    const float m_use = m2 == -INFINITY ? 0.f : m2;
#pragma unroll
    for (int v = 0; v < 16; ++v) x[v] = __builtin_amdgcn_exp2f(x[v] - m_use);
    const float ps = (((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]))) +
                     (((x[8] + x[9]) + (x[10] + x[11])) + ((x[12] + x[13]) + (x[14] + x[15])));
    lsum = lsum * alpha + ps;
    bf16x8 pB[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const u32x4 pk = {pack_bf16x2(x[8 * kk], x[8 * kk + 1]), pack_bf16x2(x[8 * kk + 2], x[8 * kk + 3]),
                        pack_bf16x2(x[8 * kk + 4], x[8 * kk + 5]), pack_bf16x2(x[8 * kk + 6], x[8 * kk + 7])};
      pB[kk] = as_bf16x8(pk);
    }
    if (__ballot(alpha != 1.f)) {  // rare, uniform
#pragma unroll
      for (int c = 0; c < NCT; ++c) acc[c] *= alpha;
    }

    // O^T += V^T P^T, the V^T reads of column tile ct + 2 issued behind the
    // products of column tile ct.
    static_for<NCT>([&](auto cc) {
      constexpr int ct = decltype(cc)::value;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 vA =
            __builtin_bit_cast(bf16x8, __builtin_shufflevector(vr[ct][kk][0], vr[ct][kk][1], 0, 1, 2, 3, 4, 5, 6, 7));
        acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vA, pB[kk], acc[ct], 0, 0, 0);
      }
      if constexpr (ct + 2 < NCT) rd_v(ct + 2, 0), rd_v(ct + 2, 1);
      __builtin_amdgcn_sched_barrier(0);
    });
  }
  // Drain the copies of the tiles past the end before the workgroup exits.
  wait_vmcnt<0>();

  // Every wave checked every block id it used; merge the flags of the workgroup.
  const uint32_t wf = __builtin_amdgcn_readfirstlane(flags);
  __shared__ uint32_t wflags[kAW];
  if (lane == 0) wflags[w] = wf;
  __syncthreads();
  uint32_t all = 0;
#pragma unroll
  for (int v = 0; v < kAW; ++v) all |= wflags[v];
  const bool bad = all != 0;
  if (tid == 0 && (all & kBadBlock)) atomicOr(&a.status[b], kBadBlock);

  const float l = lsum + __shfl_xor(lsum, 32, 64);
  if (!q_ok) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int64_t orow = ((int64_t)b * t_q + qi) * H + h;
  if (hl == 0 && a.lse) a.lse[orow] = bad ? NAN : (l > 0.f ? (m2 + __log2f(l)) * kLn2 : -INFINITY);
  // Lane (j32, hl) holds, in acc[ct][4 q + i], value column 32 ct + 8 q + 4 hl + i.
  const f32x4 nan4 = {NAN, NAN, NAN, NAN};
  if (a.out_bf16) {
    uint16_t* o = static_cast<uint16_t*>(a.out) + orow * DV + 4 * hl;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = bad ? nan4 : f32x4{acc[ct][4 * q], acc[ct][4 * q + 1], acc[ct][4 * q + 2], acc[ct][4 * q + 3]} * inv;
        *reinterpret_cast<uint2*>(o + 32 * ct + 8 * q) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
  } else {
    float* o = static_cast<float*>(a.out) + orow * DV + 4 * hl;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(o + 32 * ct + 8 * q) =
            bad ? nan4 : f32x4{acc[ct][4 * q], acc[ct][4 * q + 1], acc[ct][4 * q + 2], acc[ct][4 * q + 3]} * inv;
  }
}


}  // namespace

hipError_t launch_prefill_attend(const PrefillArgs& a, int d_rope, hipStream_t stream) {
  // Workgroups: (request, head) pairs rounded up to whole groups of eight (one
  // per XCD) times the query tiles of a request.
  const int64_t grid = 8 * (((int64_t)a.batch * a.n_head + 7) / 8) * ((a.t_q + kAQ - 1) / kAQ);
  if (grid > INT32_MAX) return hipErrorInvalidConfiguration;
  if (d_rope == 64)
    hipLaunchKernelGGL(prefill_attend<64>, dim3((unsigned)grid), dim3(64 * kAW), 0, stream, a);
  else
    hipLaunchKernelGGL(prefill_attend<0>, dim3((unsigned)grid), dim3(64 * kAW), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
