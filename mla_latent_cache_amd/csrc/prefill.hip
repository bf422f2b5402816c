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
//   * prefill_attend (prefill_attend.hip): causal flash attention per
//     (request, head, 256 queries) over these rows and the cache's k_pe.
#include <math.h>

#include "prefill_common.hpp"

namespace mla {
namespace {

using namespace prefill;

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
  // Chunk buffers (weight rows [2][128][64], cache rows [2][128][64]), reused
  // after the k loop as the output stage [128 cache rows][128 + 8 values].
  constexpr int kStagePitch = kGN + 8;  // bf16 values per staged output row (16 bytes of padding)
  constexpr int kLdsChunks = (kGM * kStagePitch * 2 / 16) > 4 * kGN * kGChunks ? kGM * kStagePitch * 2 / 16
                                                                              : 4 * kGN * kGChunks;
  __shared__ __attribute__((aligned(16))) u32x4 lds[kLdsChunks];
  u32x4(*sw)[kGN * kGChunks] = reinterpret_cast<u32x4(*)[kGN * kGChunks]>(lds);
  u32x4(*sc)[kGM * kGChunks] = reinterpret_cast<u32x4(*)[kGM * kGChunks]>(lds + 2 * kGN * kGChunks);

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
  // rows n = 64 wn + 16 i + 4 g .. + 3 in acc[i][j].  They go through LDS as
  // rows m of 128 values n (the padding spreads the rows of one write over the
  // banks), and leave as 16-byte pieces of eight consecutive columns of one
  // head, whole lines of each (head, row) segment.
  uint16_t* st = reinterpret_cast<uint16_t*>(lds);
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 64 * wm + 16 * j + l16, n = 64 * wn + 16 * i + 4 * g;
      *reinterpret_cast<uint2*>(st + m * kStagePitch + n) =
          uint2{pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3])};
    }
  barrier_keep_loads();
  const int DW = is_k ? G::DN : G::DV;
  uint16_t* dst_base = is_k ? a.kw : a.vw;
  const int nb = is_k ? n0 : n0 - NK;
  for (int idx = tid; idx < rows * (kGN / 8); idx += 256) {
    const int m = idx / (kGN / 8), c = idx - m * (kGN / 8);
    const int n = nb + 8 * c;
    const int h = n / DW, col = n - h * DW;
    uint16_t* dst = dst_base + (((int64_t)b * a.n_head + h) * a.max_rows + m0 + m) * DW + col;
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(st + m * kStagePitch + 8 * c);
  }
  if (flags && tid == 0) atomicOr(&a.status[b], flags);
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
  if (n1 > INT32_MAX) return hipErrorInvalidConfiguration;
  if (d_rope == 64) {
    hipLaunchKernelGGL(prefill_decompress<64>, dim3((unsigned)n1), dim3(256), 0, stream, g);
  } else {
    hipLaunchKernelGGL(prefill_decompress<0>, dim3((unsigned)n1), dim3(256), 0, stream, g);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_prefill_attend(g, d_rope, stream);
}

}  // namespace mla
