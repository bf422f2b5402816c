// Per-head batched GEMMs around the latent attention, for gfx950.
//
// Absorb (memra-engine "mla.rs", mla_attend_absorbed absorb step; CANN
// "aclnnMlaProlog", the q^N = q^C W^UK formula; vLLM "cpu_mla",
// forward_mqa query concatenation):
//   q_abs[n][h][l] = sum_p q_nope[n][h][p] * W_UK[h][p][l],  q_abs[n][h][kv_rank:] = q_pe[n][h]
// Decompress (memra-engine "mla.rs", mla_attend_absorbed decompress step):
//   out[n][h][j] = sum_l W_UV[h][j][l] * o_lat[n][h][l]
//
// Both are weight-read bound at decode batch sizes (a few to a few hundred
// tokens against 12-17 MB of weights), and at the smallest of them bound by
// latency: a workgroup issues every load it needs at once (one memory round
// trip; it never waits twice) and runs 16x16x32 bf16 MFMA tiles from
// registers and LDS.  Operands reach LDS through the buffer unit as whole
// rows (whole cache lines), at a pitch of one 16-byte chunk more than the row
// so that 16 rows' same chunk falls on 16 distinct bank groups; results leave
// through an LDS stage as whole rows.
//   * Absorb: one workgroup per head and 64-column slice of W_UK, with the
//     64-token groups spread over grid z only as far as those workgroups
//     leave compute units idle.  W_UK is contiguous along the output index,
//     so its slice is read back from LDS with the transposing
//     ds_read_b64_tr_b16.  absorb_mfma serves one group per workgroup in a
//     single pass; absorb_loop serves several, with the slice read once and
//     the next group's rows copied while the current one computes.
//   * Decompress: one workgroup per head and 64-row slice of W_UV (rows
//     contiguous along the contraction), whose rows each wave then keeps in
//     registers while it loops over 64-token groups, the next group's o_lat
//     rows copied while the current one computes.
#include <algorithm>
#include <type_traits>
#include "device_common.hpp"
#include "kernels.hpp"

namespace mla {
namespace {

constexpr int kCols = 64;  // weight columns (absorb) or rows (decompress) per workgroup, 16 per wave
constexpr int kMaxKS = 16; // contraction length up to 512 (32 per k-step)

template <typename TO>
__device__ __forceinline__ void store_c(TO* out, int64_t idx, float v) { Storage<TO>::store(out, idx, v); }

// Four consecutive outputs at out[idx .. idx + 3] (idx a multiple of 4).
__device__ __forceinline__ void store4(float* out, int64_t idx, f32x4 v) { *reinterpret_cast<f32x4*>(out + idx) = v; }
__device__ __forceinline__ void store4(uint16_t* out, int64_t idx, f32x4 v) {
  *reinterpret_cast<uint2*>(out + idx) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

// Run f with the number of live 16-token tiles of a group (1..MAXT) as a
// compile-time constant, so that the tiles' accumulations are independent
// chains the matrix cores overlap.
template <int MAXT, typename F>
__device__ __forceinline__ void dispatch_tiles(int live, F&& f) {
  if constexpr (MAXT >= 4) { if (live >= 4) { f(std::integral_constant<int, 4>{}); return; } }
  if constexpr (MAXT >= 3) { if (live == 3) { f(std::integral_constant<int, 3>{}); return; } }
  if (live >= 2) f(std::integral_constant<int, 2>{});
  else if (live == 1) f(std::integral_constant<int, 1>{});
}

// acc[j] += A[t] . B(j, t) over the k-steps t of NT token tiles, with B read
// from token rows staged in LDS at a pitch of P 16-byte chunks: `rows` points
// at this lane's first operand (row l16, chunk g), and B(j, t) is chunk 4 t of
// row 16 j from there.  The reads of a pass (k-steps T0 .. T0 + KC - 1, at
// most 32 operands) are all issued before its products, so the LDS latency is
// paid once per pass rather than once per product.
template <int NT, int KS, int P, int T0 = 0>
__device__ __forceinline__ void tile_products(f32x4 (&acc)[NT], const bf16x8 (&A)[KS], const u32x4* rows) {
  constexpr int KC = (32 / NT) < (KS - T0) ? (32 / NT) : (KS - T0);
  bf16x8 B[NT][KC];
#pragma unroll
  for (int t = 0; t < KC; ++t)
#pragma unroll
    for (int j = 0; j < NT; ++j) B[j][t] = as_bf16x8(rows[16 * j * P + 4 * (T0 + t)]);
#pragma unroll
  for (int t = 0; t < KC; ++t)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = mfma16x16x32(A[T0 + t], B[j][t], acc[j]);
  // Keep the pass's LDS reads ahead of its products (the scheduler would
  // otherwise pair each read with its product to save registers).
  __builtin_amdgcn_sched_group_barrier(0x100, NT * KC, 0);  // LDS reads
  __builtin_amdgcn_sched_group_barrier(0x008, NT * KC, 0);  // matrix-core products
  if constexpr (T0 + KC < KS) tile_products<NT, KS, P, T0 + KC>(acc, A, rows);
}

// Tokens per workgroup: four 16-token tiles, two when the contraction is
// longer than 256 (the absorb weight slice then takes most of the LDS).
template <int KS>
constexpr int absorb_tiles() { return KS <= 8 ? 4 : 2; }
constexpr int kDecompTiles = 4;

// Copy `rows` rows of CPR 16-byte chunks (row r at byte offset r * pitch in
// the resource) into LDS with a row pitch of CPR + 1 chunks.  Copy i fills
// slots 64 i .. 64 i + 63 (slot s: row s / (CPR + 1), chunk s % (CPR + 1)), so
// each copy reads whole rows' consecutive bytes, and the odd pitch puts the
// same chunk of any 16 consecutive rows on 16 distinct bank groups.  Padding
// slots and rows at or past `rows` read as zeros.  Copies are dealt
// round-robin to the four waves.
template <int CPR>
__device__ __forceinline__ void copy_rows(i32x4 rs, uint32_t lbase, int rows, uint32_t pitch, int w, int lane) {
  constexpr int P = CPR + 1;
  const int copies = (rows * P + 63) / 64;
  for (int i = w; i < copies; i += 4) {
    const int s = 64 * i + lane;
    const int r = s / P, c = s - r * P;
    const uint32_t off = (c < CPR && r < rows) ? (uint32_t)r * pitch + 16u * (uint32_t)c : 0xFFFFFFF0u;
    dma16(rs, lbase + 1024u * i, off);
  }
}

// Output staging: a workgroup's results as token rows of 64 values, at a
// pitch of one 16-byte chunk more than the row, so that rows leave the
// workgroup as whole 16-byte pieces (whole cache lines per row) rather than
// as each lane's four values.
template <typename TO>
constexpr int stage_pitch() { return 64 * (int)sizeof(TO) / 16 + 1; }

// Lane (l16, g) of wave w holds, in acc[j], the values of columns 16 w + 4 g
// .. + 3 of token row 16 j + l16.
template <typename TO, int NT>
__device__ __forceinline__ void stage_tiles(u32x4* stage, const f32x4 (&acc)[NT], int w, int l16, int g) {
  constexpr int SP = stage_pitch<TO>();
  char* base = reinterpret_cast<char*>(stage);
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    char* dst = base + (16 * j + l16) * SP * 16 + (16 * w + 4 * g) * (int)sizeof(TO);
    if constexpr (sizeof(TO) == 2)
      *reinterpret_cast<uint2*>(dst) = uint2{pack_bf16x2(acc[j][0], acc[j][1]), pack_bf16x2(acc[j][2], acc[j][3])};
    else
      *reinterpret_cast<f32x4*>(dst) = acc[j];
  }
}

// Store staged rows 0 .. cnt - 1 to row_base(r) .. + 63, of which the first
// `valid` values (a multiple of 4) exist: 16-byte pieces where st16 (bf16
// rows whose stride is a multiple of 8 values), else 4-value pieces.
template <typename TO, typename F>
__device__ __forceinline__ void store_rows(const u32x4* stage, int cnt, int valid, bool st16, F&& row_base, int tid) {
  constexpr int SP = stage_pitch<TO>();
  if (sizeof(TO) == 2 && st16) {
    for (int idx = tid; idx < cnt * 8; idx += 256) {
      const int r = idx >> 3, c = idx & 7;
      if (8 * c >= valid) continue;
      const u32x4 v = stage[r * SP + c];
      TO* dst = row_base(r) + 8 * c;
      if (8 * c + 8 <= valid) *reinterpret_cast<u32x4*>(dst) = v;
      else *reinterpret_cast<uint2*>(dst) = uint2{v[0], v[1]};
    }
  } else {
    const char* base = reinterpret_cast<const char*>(stage);
    for (int idx = tid; idx < cnt * 16; idx += 256) {
      const int r = idx >> 4, p = idx & 15;
      if (4 * p >= valid) continue;
      TO* dst = row_base(r) + 4 * p;
      const char* src = base + r * SP * 16 + p * 4 * (int)sizeof(TO);
      if constexpr (sizeof(TO) == 2) *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(src);
      else *reinterpret_cast<f32x4*>(dst) = *reinterpret_cast<const f32x4*>(src);
    }
  }
}

// 16-byte chunk swizzle of the LDS weight slice of absorb (rows of 128
// bytes): a half-wave's transposing reads touch rows r0 + {0..3} and
// r0 + 8 + {0..3} (r0 a multiple of 16), two chunks each; rows of equal parity
// would share banks, and the XOR spreads them over distinct chunk pairs.
__device__ __forceinline__ int chunk_swz(int row) { return ((row >> 1) & 1) * 2 + ((row >> 3) & 1) * 4; }

// ---------------------------------------------------------------------------
// Absorb, bf16 in.  Grid (n_head, kv_rank / 64, token groups); 256 threads;
// d_nope = 32 KS.  q_abs^T = W_UK^T q_nope^T: the weight columns are the M
// dimension (read transposed from LDS), tokens the N dimension.  The rope
// tail q_abs[n][h][kv_rank:] = q_pe[n][h] is copied by the column-slice
// workgroups of the token group, 16 bytes per thread.
// ---------------------------------------------------------------------------
template <typename TO, int KS>
__global__ __launch_bounds__(256) void absorb_mfma(int H, int R, int kv_rank, int n_tok,
                                                   const uint16_t* __restrict__ q_nope,
                                                   const uint16_t* __restrict__ q_pe,
                                                   const uint16_t* __restrict__ w_uk,
                                                   TO* __restrict__ q_abs) {
  constexpr int DN = 32 * KS, NTW = absorb_tiles<KS>(), P = 4 * KS + 1;
  constexpr int kTokSlots = (16 * NTW * P + 63) / 64 * 64;
  __shared__ __attribute__((aligned(16))) u32x4 wl[DN * 8];      // DN rows x 8 chunks, swizzled
  __shared__ __attribute__((aligned(16))) u32x4 tl[kTokSlots];   // token rows, pitch P chunks
  __shared__ __attribute__((aligned(16))) u32x4 ol[16 * NTW * stage_pitch<TO>()];
  const int h = blockIdx.x, c0 = blockIdx.y * kCols, m0 = blockIdx.z * (16 * NTW);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, g = lane >> 4;
  const int D = kv_rank + R;
  const int cnt = min(16 * NTW, n_tok - m0);  // tokens of this group
  const int nt = (cnt + 15) / 16;

  // Weight slice W_UK[h][0:DN][c0:c0+64] into LDS: eight rows (1 KB) per copy, copy i by wave i % 4.
  const i32x4 wrs = raw_rsrc(w_uk + (int64_t)h * DN * kv_rank, (uint32_t)(DN * kv_rank * 2));
  const uint32_t wbase = lds_addr(wl);
#pragma unroll
  for (int u = 0; u < KS; ++u) {
    const int i = w + 4 * u;
    const int row = 8 * i + (lane >> 3);
    dma16(wrs, wbase + 1024u * i, (uint32_t)(row * kv_rank + c0 + 8 * ((lane & 7) ^ chunk_swz(row))) * 2u);
  }
  // The group's q_nope rows.
  const uint32_t qpitch = (uint32_t)(H * DN * 2);
  copy_rows<4 * KS>(raw_rsrc(q_nope + ((int64_t)m0 * H + h) * DN, (uint32_t)(cnt - 1) * qpitch + DN * 2),
                    lds_addr(tl), cnt, qpitch, w, lane);

  // Rope tail: this thread's first 16-byte piece travels with the copies above.
  const int r8 = R >> 3;
  const int qchunks = (R & 7) == 0 ? cnt * r8 : 0;
  const int q_step = 256 * (int)gridDim.y;
  int qi = (int)blockIdx.y * 256 + tid;
  u32x4 qv = {0u, 0u, 0u, 0u};
  if (qi < qchunks) {
    const int n = qi / r8, r = qi - n * r8;
    qv = *reinterpret_cast<const u32x4*>(q_pe + ((int64_t)(m0 + n) * H + h) * R + 8 * r);
  }
  wait_vmcnt<0>();
  if (qi < qchunks) {
    const int n = qi / r8, r = qi - n * r8;
    TO* dst = q_abs + ((int64_t)(m0 + n) * H + h) * D + kv_rank + 8 * r;
    if constexpr (sizeof(TO) == 2) {
      *reinterpret_cast<u32x4*>(dst) = qv;
    } else {
      const bf16x8 b = as_bf16x8(qv);
      *reinterpret_cast<f32x4*>(dst) = f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{(float)b[4], (float)b[5], (float)b[6], (float)b[7]};
    }
  }
  barrier_keep_loads();

  // This wave's 16 weight columns as the A operand: lane (l16, g) of k-step t
  // holds column 16 w + l16, rows 32 t + 8 g .. + 7 (two transposing reads).
  const char* wlb = reinterpret_cast<const char*>(wl);
  bf16x8 A[KS];
#pragma unroll
  for (int t = 0; t < KS; ++t) {
    const int prow = 32 * t + 8 * g + (l16 >> 2);
    const int chunk = 2 * w + ((l16 & 3) >> 1), half = 8 * (l16 & 1);
    const s16x4 b0 = lds_read_tr16(wlb + prow * 128 + (chunk ^ chunk_swz(prow)) * 16 + half);
    const s16x4 b1 = lds_read_tr16(wlb + (prow + 4) * 128 + (chunk ^ chunk_swz(prow + 4)) * 16 + half);
    A[t] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
  }
  dispatch_tiles<NTW>(nt, [&](auto nt_c) {
    constexpr int NT = decltype(nt_c)::value;
    f32x4 acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    tile_products<NT, KS, P>(acc, A, tl + l16 * P + g);
    stage_tiles<TO, NT>(ol, acc, w, l16, g);
  });
  barrier_keep_loads();
  store_rows<TO>(ol, cnt, kCols, D % 8 == 0, [&](int r) { return q_abs + ((int64_t)(m0 + r) * H + h) * D + c0; },
                 tid);

  // Rope pieces beyond the first per thread (more than 256 x slices of them per group).
  for (qi += q_step; qi < qchunks; qi += q_step) {
    const int n = qi / r8, r = qi - n * r8;
    const u32x4 v = *reinterpret_cast<const u32x4*>(q_pe + ((int64_t)(m0 + n) * H + h) * R + 8 * r);
    TO* dst = q_abs + ((int64_t)(m0 + n) * H + h) * D + kv_rank + 8 * r;
    if constexpr (sizeof(TO) == 2) {
      *reinterpret_cast<u32x4*>(dst) = v;
    } else {
      const bf16x8 b = as_bf16x8(v);
      *reinterpret_cast<f32x4*>(dst) = f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{(float)b[4], (float)b[5], (float)b[6], (float)b[7]};
    }
  }
  // A rope width that is not a multiple of 8 is copied element by element.
  if ((R & 7) != 0) {
    for (int idx = (int)blockIdx.y * 256 + tid; idx < cnt * R; idx += q_step) {
      const int n = idx / R, r = idx - n * R;
      store_c(q_abs, ((int64_t)(m0 + n) * H + h) * D + kv_rank + r,
              bf16_to_f32(q_pe[((int64_t)(m0 + n) * H + h) * R + r]));
    }
  }
}

// Absorb for workgroups that serve several token groups of one (head,
// column slice): the weight slice is copied once and kept as the A operand
// in registers, its LDS buffer then takes token rows, and each group's
// q_nope rows are copied into one of two buffers while the previous group
// computes.  (With one group per workgroup the single-pass kernel above is
// faster by a few tenths of a microsecond.)
template <typename TO, int KS>
__global__ __launch_bounds__(256) void absorb_loop(int H, int R, int kv_rank, int n_tok,
                                                   const uint16_t* __restrict__ q_nope,
                                                   const uint16_t* __restrict__ q_pe,
                                                   const uint16_t* __restrict__ w_uk,
                                                   TO* __restrict__ q_abs) {
  constexpr int DN = 32 * KS, NTW = absorb_tiles<KS>(), P = 4 * KS + 1, G = 16 * NTW;
  constexpr int kTokSlots = (G * P + 63) / 64 * 64;
  constexpr int kBuf1 = kTokSlots > DN * 8 ? kTokSlots : DN * 8;
  __shared__ __attribute__((aligned(16))) u32x4 buf0[kTokSlots];  // token rows, pitch P chunks
  __shared__ __attribute__((aligned(16))) u32x4 buf1[kBuf1];      // the weight slice (swizzled), then token rows
  __shared__ __attribute__((aligned(16))) u32x4 ol[G * stage_pitch<TO>()];
  const int h = blockIdx.x, c0 = blockIdx.y * kCols, zs = (int)gridDim.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, g = lane >> 4;
  const int D = kv_rank + R;
  const int ngroups = (n_tok + G - 1) / G;
  const uint32_t qpitch = (uint32_t)(H * DN * 2);

  // The q_nope rows of group gi into LDS buffer b.
  auto copy_group = [&](int gi, int b) {
    const int m0 = gi * G, cnt = min(G, n_tok - m0);
    copy_rows<4 * KS>(raw_rsrc(q_nope + ((int64_t)m0 * H + h) * DN, (uint32_t)(cnt - 1) * qpitch + DN * 2),
                      lds_addr(b ? buf1 : buf0), cnt, qpitch, w, lane);
  };
  // Weight slice W_UK[h][0:DN][c0:c0+64] into buffer 1: eight rows (1 KB) per copy, copy i by wave i % 4.
  const i32x4 wrs = raw_rsrc(w_uk + (int64_t)h * DN * kv_rank, (uint32_t)(DN * kv_rank * 2));
  const uint32_t wbase = lds_addr(buf1);
#pragma unroll
  for (int u = 0; u < KS; ++u) {
    const int i = w + 4 * u;
    const int row = 8 * i + (lane >> 3);
    dma16(wrs, wbase + 1024u * i, (uint32_t)(row * kv_rank + c0 + 8 * ((lane & 7) ^ chunk_swz(row))) * 2u);
  }
  int gi = (int)blockIdx.z;  // < ngroups: the launch has at most ngroups z-slices
  copy_group(gi, 0);

  // Rope columns, dealt over the head's column slices in 16-byte pieces (or
  // element by element for a rope width that is not a multiple of 8): this
  // thread's first piece of a group is loaded with the group's copies and
  // stored as soon as they have landed.
  const int r8 = R >> 3;
  const int q_step = 256 * (int)gridDim.y, q_first = (int)blockIdx.y * 256 + tid;
  auto rope_src = [&](int m0, int qi) { return q_pe + ((int64_t)(m0 + qi / r8) * H + h) * R + 8 * (qi % r8); };
  auto rope_put = [&](int m0, int qi, u32x4 v) {
    TO* dst = q_abs + ((int64_t)(m0 + qi / r8) * H + h) * D + kv_rank + 8 * (qi % r8);
    if constexpr (sizeof(TO) == 2) {
      *reinterpret_cast<u32x4*>(dst) = v;
    } else {
      const bf16x8 x = as_bf16x8(v);
      *reinterpret_cast<f32x4*>(dst) = f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{(float)x[4], (float)x[5], (float)x[6], (float)x[7]};
    }
  };
  auto rope_pieces = [&](int gi) { return (R & 7) == 0 ? min(G, n_tok - gi * G) * r8 : 0; };
  u32x4 qv = {0u, 0u, 0u, 0u};
  if (q_first < rope_pieces(gi)) qv = *reinterpret_cast<const u32x4*>(rope_src(gi * G, q_first));
  wait_vmcnt<0>();
  if (q_first < rope_pieces(gi)) rope_put(gi * G, q_first, qv);
  barrier_keep_loads();

  // This wave's 16 weight columns as the A operand: lane (l16, g) of k-step t
  // holds column 16 w + l16, rows 32 t + 8 g .. + 7 (two transposing reads).
  const char* wlb = reinterpret_cast<const char*>(buf1);
  bf16x8 A[KS];
#pragma unroll
  for (int t = 0; t < KS; ++t) {
    const int prow = 32 * t + 8 * g + (l16 >> 2);
    const int chunk = 2 * w + ((l16 & 3) >> 1), half = 8 * (l16 & 1);
    const s16x4 b0 = lds_read_tr16(wlb + prow * 128 + (chunk ^ chunk_swz(prow)) * 16 + half);
    const s16x4 b1 = lds_read_tr16(wlb + (prow + 4) * 128 + (chunk ^ chunk_swz(prow + 4)) * 16 + half);
    A[t] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
  }
  if (gi + zs < ngroups) barrier_keep_loads();  // every wave holds its weights: buffer 1 is free

  for (int b = 0; gi < ngroups; gi += zs, b ^= 1) {
    const int m0 = gi * G, cnt = min(G, n_tok - m0);
    const int nt = (cnt + 15) / 16;
    const bool more = gi + zs < ngroups;
    const bool next_piece = more && q_first < rope_pieces(gi + zs);
    if (more) copy_group(gi + zs, b ^ 1);
    if (next_piece) qv = *reinterpret_cast<const u32x4*>(rope_src((gi + zs) * G, q_first));
    dispatch_tiles<NTW>(nt, [&](auto nt_c) {
      constexpr int NT = decltype(nt_c)::value;
      f32x4 acc[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      tile_products<NT, KS, P>(acc, A, (b ? buf1 : buf0) + l16 * P + g);
      stage_tiles<TO, NT>(ol, acc, w, l16, g);
    });
    if (more) wait_vmcnt<0>();  // the next group's rows (and this wave's earlier stores)
    if (next_piece) rope_put((gi + zs) * G, q_first, qv);
    barrier_keep_loads();  // stage complete; the next group's rows visible; buffer b free
    store_rows<TO>(ol, cnt, kCols, D % 8 == 0,
                   [&](int r) { return q_abs + ((int64_t)(m0 + r) * H + h) * D + c0; }, tid);

    const int pieces = rope_pieces(gi);
    for (int qi = q_first + q_step; qi < pieces; qi += q_step)
      rope_put(m0, qi, *reinterpret_cast<const u32x4*>(rope_src(m0, qi)));
    if ((R & 7) != 0) {
      for (int idx = q_first; idx < cnt * R; idx += q_step) {
        const int n = idx / R, r = idx - n * R;
        store_c(q_abs, ((int64_t)(m0 + n) * H + h) * D + kv_rank + r,
                bf16_to_f32(q_pe[((int64_t)(m0 + n) * H + h) * R + r]));
      }
    }
    if (more) barrier_keep_loads();  // the stage is read out before the next group writes it
  }
}

// ---------------------------------------------------------------------------
// Decompress, bf16 weights.  Grid (n_head, ceil(d_v / 64), zs); 256 threads;
// kv_rank = 32 KS.  The workgroup copies its 64 rows of W_UV[h] (rows past
// d_v read as zeros) into LDS as whole rows, and each wave keeps 16 of them
// in registers as the A operand of out^T = W_UV o_lat^T.  Workgroup z then
// takes the 64-token groups z, z + zs, ...: each group's o_lat rows (bf16)
// are copied into one of two LDS buffers while the previous group computes
// (the weight buffer becomes the second token buffer once the weights are in
// registers); float32 o_lat is read straight from global memory and rounded
// to bf16.  Results leave through the LDS stage as whole rows.
// ---------------------------------------------------------------------------
template <typename TI, typename TO, int KS>
__global__ __launch_bounds__(256) void decompress_mfma(int H, int DV, int n_tok, const TI* __restrict__ o_lat,
                                                       const uint16_t* __restrict__ w_uv,
                                                       TO* __restrict__ out) {
  constexpr int KR = 32 * KS, P = 4 * KS + 1, G = 16 * kDecompTiles;
  constexpr bool kStage = sizeof(TI) == 2;
  __shared__ __attribute__((aligned(16))) u32x4 buf[2][kCols * P];  // [1]: weights, then tokens; [0]: tokens
  __shared__ __attribute__((aligned(16))) u32x4 ol[G * stage_pitch<TO>()];
  const int h = blockIdx.x, j0 = blockIdx.y * kCols, zs = (int)gridDim.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, g = lane >> 4;
  const int nrows = min(kCols, DV - j0);  // weight rows (output columns) of this slice
  const int ngroups = (n_tok + G - 1) / G;
  const uint32_t opitch = (uint32_t)(H * KR * sizeof(TI));

  // The o_lat rows of group gi into LDS buffer b (bf16 only).
  auto copy_group = [&](int gi, int b) {
    const int m0 = gi * G, cnt = min(G, n_tok - m0);
    copy_rows<4 * KS>(raw_rsrc(o_lat + ((int64_t)m0 * H + h) * KR, (uint32_t)(cnt - 1) * opitch + KR * 2),
                      lds_addr(buf[b]), cnt, opitch, w, lane);
  };
  copy_rows<4 * KS>(raw_rsrc(w_uv + ((int64_t)h * DV + j0) * KR, (uint32_t)(nrows * KR * 2)), lds_addr(buf[1]),
                    nrows, KR * 2, w, lane);
  int gi = (int)blockIdx.z;
  if constexpr (kStage)
    if (gi < ngroups) copy_group(gi, 0);
  wait_vmcnt<0>();
  barrier_keep_loads();
  bf16x8 A[KS];
  const u32x4* arow = buf[1] + (16 * w + l16) * P + g;
#pragma unroll
  for (int t = 0; t < KS; ++t) A[t] = as_bf16x8(arow[4 * t]);
  if (gi + zs < ngroups) barrier_keep_loads();  // every wave holds its weights: buffer 1 is free

  for (int b = 0; gi < ngroups; gi += zs, b ^= 1) {
    const int m0 = gi * G, cnt = min(G, n_tok - m0);
    const int nt = (cnt + 15) / 16;
    if constexpr (kStage) {
      if (gi + zs < ngroups) copy_group(gi + zs, b ^ 1);
      dispatch_tiles<kDecompTiles>(nt, [&](auto nt_c) {
        constexpr int NT = decltype(nt_c)::value;
        f32x4 acc[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        tile_products<NT, KS, P>(acc, A, buf[b] + l16 * P + g);
        stage_tiles<TO, NT>(ol, acc, w, l16, g);
      });
      wait_vmcnt<0>();  // the next group's rows (and this wave's earlier stores)
    } else {
      // Float32 activations: two 16-byte loads per k-step, rounded to bf16; tokens past the group read as zeros.
      const __amdgpu_buffer_rsrc_t ors =
          make_rsrc(o_lat + ((int64_t)m0 * H + h) * KR, (uint32_t)(cnt - 1) * opitch + KR * 4);
      for (int j = 0; j < nt; ++j) {
        const uint32_t roff = (uint32_t)(16 * j + l16) * opitch + 32u * g;
        f32x4 acc[1] = {{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int t = 0; t < KS; ++t) {
          const f32x4 x = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ors, roff + 128u * t, 0, 0));
          const f32x4 y =
              __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ors, roff + 128u * t + 16u, 0, 0));
          const u32x4 v = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(y[0], y[1]),
                           pack_bf16x2(y[2], y[3])};
          acc[0] = mfma16x16x32(A[t], as_bf16x8(v), acc[0]);
        }
        stage_tiles<TO, 1>(ol + 16 * j * stage_pitch<TO>(), acc, w, l16, g);
      }
    }
    barrier_keep_loads();  // stage complete; the next group's rows visible; buffer b free
    store_rows<TO>(ol, cnt, nrows, DV % 8 == 0,
                   [&](int r) { return out + ((int64_t)(m0 + r) * H + h) * DV + j0; }, tid);
    if (gi + zs < ngroups) barrier_keep_loads();  // the stage is read out before the next group writes it
  }
}

// ---------------------------------------------------------------------------
// Generic fallbacks (any sizes, float32 or bf16 storage): one thread per output.
// ---------------------------------------------------------------------------
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void absorb_generic(int H, int DN, int R, int KR, int64_t n_tok,
                                                      const TI* q_nope, const TI* q_pe, const TI* w_uk,
                                                      TO* q_abs) {
  const int D = KR + R;
  const int64_t total = n_tok * H * D;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const int64_t nh = idx / D;
    const int c = (int)(idx - nh * D);
    const int h = (int)(nh % H);
    float v;
    if (c < KR) {
      v = 0.f;
      for (int p = 0; p < DN; ++p)
        v += Storage<TI>::load(q_nope, nh * DN + p) * Storage<TI>::load(w_uk, ((int64_t)h * DN + p) * KR + c);
    } else {
      v = Storage<TI>::load(q_pe, nh * R + (c - KR));
    }
    store_c(q_abs, idx, v);
  }
}

template <typename TI, typename TW, typename TO>
__global__ __launch_bounds__(256) void decompress_generic(int H, int DV, int KR, int64_t n_tok,
                                                          const TI* o_lat, const TW* w_uv, TO* out) {
  const int64_t total = n_tok * H * DV;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const int64_t nh = idx / DV;
    const int j = (int)(idx - nh * DV);
    const int h = (int)(nh % H);
    float v = 0.f;
    for (int l = 0; l < KR; ++l)
      v += Storage<TW>::load(w_uv, ((int64_t)h * DV + j) * KR + l) * Storage<TI>::load(o_lat, nh * KR + l);
    store_c(out, idx, v);
  }
}

unsigned generic_grid(int64_t total) {
  int64_t g = (total + 255) / 256;
  if (g > 65536) g = 65536;
  return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

// Run f with the contraction length in k-steps of 32 (1..16) as a compile-time constant.
template <typename F>
void with_ksteps(int ks, F&& f) {
  switch (ks) {
#define MLA_KS(n) \
  case n: f(std::integral_constant<int, n>{}); break;
    MLA_KS(1) MLA_KS(2) MLA_KS(3) MLA_KS(4) MLA_KS(5) MLA_KS(6) MLA_KS(7) MLA_KS(8)
    MLA_KS(9) MLA_KS(10) MLA_KS(11) MLA_KS(12) MLA_KS(13) MLA_KS(14) MLA_KS(15) MLA_KS(16)
#undef MLA_KS
    default: break;
  }
}

// 32-bit buffer offsets of the MFMA paths: a token group's rows and a head's
// weight matrix must each span less than 2 GiB.
bool fits_u31(int64_t bytes) { return bytes < ((int64_t)1 << 31); }

hipError_t launch_absorb(int H, int DN, int R, int KR, int64_t n_tok, const void* q_nope, const void* q_pe,
                         const void* w_uk, bool in_bf16, void* q_abs, bool out_bf16, hipStream_t stream) {
  if (n_tok == 0) return hipSuccess;
  // (Four-column output stores need rows of a multiple of 4 elements.)
  const bool mfma = in_bf16 && DN % 32 == 0 && DN / 32 <= kMaxKS && KR % kCols == 0 && R % 4 == 0 &&
                    n_tok <= INT32_MAX && fits_u31((int64_t)64 * H * DN * 2) && fits_u31((int64_t)DN * KR * 2);
  if (mfma) {
    const uint16_t *qn = static_cast<const uint16_t*>(q_nope), *qp = static_cast<const uint16_t*>(q_pe),
                   *wk = static_cast<const uint16_t*>(w_uk);
    with_ksteps(DN / 32, [&](auto ks_c) {
      constexpr int KS = decltype(ks_c)::value;
      // Token groups are spread over grid z only as far as the (head, column
      // slice) workgroups leave compute units idle; where a workgroup is left
      // with several groups it loops over them and reads its weight slice into
      // LDS once.
      const int per = 16 * absorb_tiles<KS>();
      const int64_t groups = (n_tok + per - 1) / per, slices = (int64_t)H * (KR / kCols);
      const int64_t zs = std::max<int64_t>(1, std::min<int64_t>(groups, 256 / std::max<int64_t>(1, slices)));
      const dim3 grid(H, KR / kCols, (unsigned)zs);
      if (zs == groups) {
        if (out_bf16)
          hipLaunchKernelGGL((absorb_mfma<uint16_t, KS>), grid, dim3(256), 0, stream, H, R, KR, (int)n_tok, qn, qp,
                             wk, static_cast<uint16_t*>(q_abs));
        else
          hipLaunchKernelGGL((absorb_mfma<float, KS>), grid, dim3(256), 0, stream, H, R, KR, (int)n_tok, qn, qp,
                             wk, static_cast<float*>(q_abs));
      } else {
        if (out_bf16)
          hipLaunchKernelGGL((absorb_loop<uint16_t, KS>), grid, dim3(256), 0, stream, H, R, KR, (int)n_tok, qn, qp,
                             wk, static_cast<uint16_t*>(q_abs));
        else
          hipLaunchKernelGGL((absorb_loop<float, KS>), grid, dim3(256), 0, stream, H, R, KR, (int)n_tok, qn, qp,
                             wk, static_cast<float*>(q_abs));
      }
    });
    return hipGetLastError();
  }
  const unsigned grid = generic_grid(n_tok * H * (KR + R));
  if (in_bf16) {
    const uint16_t *qn = static_cast<const uint16_t*>(q_nope), *qp = static_cast<const uint16_t*>(q_pe),
                   *wk = static_cast<const uint16_t*>(w_uk);
    if (out_bf16)
      hipLaunchKernelGGL((absorb_generic<uint16_t, uint16_t>), dim3(grid), dim3(256), 0, stream, H, DN, R, KR,
                         n_tok, qn, qp, wk, static_cast<uint16_t*>(q_abs));
    else
      hipLaunchKernelGGL((absorb_generic<uint16_t, float>), dim3(grid), dim3(256), 0, stream, H, DN, R, KR,
                         n_tok, qn, qp, wk, static_cast<float*>(q_abs));
  } else {
    const float *qn = static_cast<const float*>(q_nope), *qp = static_cast<const float*>(q_pe),
                *wk = static_cast<const float*>(w_uk);
    if (out_bf16)
      hipLaunchKernelGGL((absorb_generic<float, uint16_t>), dim3(grid), dim3(256), 0, stream, H, DN, R, KR,
                         n_tok, qn, qp, wk, static_cast<uint16_t*>(q_abs));
    else
      hipLaunchKernelGGL((absorb_generic<float, float>), dim3(grid), dim3(256), 0, stream, H, DN, R, KR, n_tok,
                         qn, qp, wk, static_cast<float*>(q_abs));
  }
  return hipGetLastError();
}

hipError_t launch_decompress(int H, int DV, int KR, int64_t n_tok, const void* o_lat, bool o_bf16,
                             const void* w_uv, bool w_bf16, void* out, bool out_bf16, hipStream_t stream) {
  if (n_tok == 0) return hipSuccess;
  const int64_t osz = o_bf16 ? 2 : 4;
  const bool mfma = w_bf16 && KR % 32 == 0 && KR / 32 <= kMaxKS && DV % 4 == 0 && n_tok <= INT32_MAX &&
                    fits_u31((int64_t)64 * H * KR * osz) && fits_u31((int64_t)(DV + kCols) * KR * 2);
  if (mfma) {
    // Token groups are split over grid z only as far as the (head, slice)
    // workgroups leave compute units idle; each workgroup loops over the rest.
    const int64_t slices = (int64_t)H * ((DV + kCols - 1) / kCols);
    const int64_t groups = (n_tok + 16 * kDecompTiles - 1) / (16 * kDecompTiles);
    const int64_t zs = std::max<int64_t>(1, std::min<int64_t>(groups, 256 / std::max<int64_t>(1, slices)));
    const dim3 grid(H, (DV + kCols - 1) / kCols, (unsigned)zs);
    const uint16_t* wv = static_cast<const uint16_t*>(w_uv);
    with_ksteps(KR / 32, [&](auto ks_c) {
      constexpr int KS = decltype(ks_c)::value;
#define MLA_DECOMP(TI, TO)                                                                                      \
  hipLaunchKernelGGL((decompress_mfma<TI, TO, KS>), grid, dim3(256), 0, stream, H, DV, (int)n_tok,             \
                     static_cast<const TI*>(o_lat), wv, static_cast<TO*>(out))
      if (o_bf16 && out_bf16) MLA_DECOMP(uint16_t, uint16_t);
      else if (o_bf16) MLA_DECOMP(uint16_t, float);
      else if (out_bf16) MLA_DECOMP(float, uint16_t);
      else MLA_DECOMP(float, float);
#undef MLA_DECOMP
    });
    return hipGetLastError();
  }
  const unsigned grid = generic_grid(n_tok * H * DV);
#define MLA_DECOMP_G(TI, TW, TO)                                                                          \
  hipLaunchKernelGGL((decompress_generic<TI, TW, TO>), dim3(grid), dim3(256), 0, stream, H, DV, KR, n_tok, \
                     static_cast<const TI*>(o_lat), static_cast<const TW*>(w_uv), static_cast<TO*>(out))
  if (o_bf16) {
    if (w_bf16) { if (out_bf16) MLA_DECOMP_G(uint16_t, uint16_t, uint16_t); else MLA_DECOMP_G(uint16_t, uint16_t, float); }
    else { if (out_bf16) MLA_DECOMP_G(uint16_t, float, uint16_t); else MLA_DECOMP_G(uint16_t, float, float); }
  } else {
    if (w_bf16) { if (out_bf16) MLA_DECOMP_G(float, uint16_t, uint16_t); else MLA_DECOMP_G(float, uint16_t, float); }
    else { if (out_bf16) MLA_DECOMP_G(float, float, uint16_t); else MLA_DECOMP_G(float, float, float); }
  }
#undef MLA_DECOMP_G
  return hipGetLastError();
}

}  // namespace mla
