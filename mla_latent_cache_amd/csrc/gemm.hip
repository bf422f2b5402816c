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
// tokens against 12-17 MB of weights), so each weight element is read from
// HBM exactly once: one workgroup owns one head and a 64-column slice of the
// weight, keeps that slice on chip, and sweeps every token past it with
// 16x16x32 bf16 MFMA.  W_UV rows are contiguous along the contraction index,
// so its B operand is loaded straight into VGPRs; W_UK is contiguous along the
// output index, so its slice is staged in LDS and read back with the
// transposing ds_read_b64_tr_b16.
#include <type_traits>
#include "device_common.hpp"
#include "kernels.hpp"

namespace mla {
namespace {

constexpr int kCols = 64;  // weight columns per workgroup (16 per wave)

// Load 8 consecutive activations starting at p as bf16 MFMA operand lanes.
__device__ __forceinline__ bf16x8 load8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ bf16x8 load8(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  const u32x4 v = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                   pack_bf16x2(b[2], b[3])};
  return as_bf16x8(v);
}

template <typename TO>
__device__ __forceinline__ void store_c(TO* out, int64_t idx, float v) { Storage<TO>::store(out, idx, v); }

// Four consecutive outputs at out[idx .. idx + 3] (idx a multiple of 4).
__device__ __forceinline__ void store4(float* out, int64_t idx, f32x4 v) { *reinterpret_cast<f32x4*>(out + idx) = v; }
__device__ __forceinline__ void store4(uint16_t* out, int64_t idx, f32x4 v) {
  *reinterpret_cast<uint2*>(out + idx) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

constexpr int kMaxK = 16;   // contraction length up to 512 (32 per k-step)
constexpr int kTC = 64;     // tokens staged in LDS at a time

// Stage activations act[m0 + i][h][0:K] (i < kTC, rows past n_tok as zeros)
// into LDS as bf16 rows of pitch K + 8 elements (16 bytes of padding: the
// 16-byte operand reads of 16 consecutive rows then cover all 64 banks).
// Every thread issues all of its global loads before its first LDS write.
constexpr int kStagePer = kTC * 512 / 8 / 256;  // most 8-element chunks per thread (K <= 512)

template <typename TI>
__device__ __forceinline__ void load_tokens(bf16x8 (&v)[kStagePer], const TI* act, int64_t row_stride, int64_t m0,
                                            int64_t n_tok, int K, int tid) {
  const int c8n = K / 8;  // 8-element chunks per row
#pragma unroll
  for (int i = 0; i < kStagePer; ++i) {
    const int idx = tid + 256 * i;
    const int r = idx / c8n, c8 = idx - r * c8n;
    v[i] = (r < kTC && m0 + r < n_tok) ? load8(act + (m0 + r) * row_stride + 8 * c8) : zero_bf16x8();
  }
}

__device__ __forceinline__ void store_tokens(uint16_t* lds, const bf16x8 (&v)[kStagePer], int K, int tid) {
  const int c8n = K / 8;
#pragma unroll
  for (int i = 0; i < kStagePer; ++i) {
    const int idx = tid + 256 * i;
    const int r = idx / c8n, c8 = idx - r * c8n;
    if (r < kTC) *reinterpret_cast<bf16x8*>(lds + r * (K + 8) + 8 * c8) = v[i];
  }
}

// Run f with the number of 16-token tiles of a staged chunk (1..4, kTC = 64)
// as a compile-time constant, so that the tiles' accumulations are
// independent chains the matrix cores overlap.
template <typename F>
__device__ __forceinline__ void dispatch_tiles(int live, F&& f) {
  static_assert(kTC == 64, "four 16-token tiles per chunk");
  if (live >= 4) f(std::integral_constant<int, 4>{});
  else if (live == 3) f(std::integral_constant<int, 3>{});
  else if (live == 2) f(std::integral_constant<int, 2>{});
  else if (live == 1) f(std::integral_constant<int, 1>{});
}

// B operand (tokens as the N dimension) of k-step t for token row `row` of
// the staged chunk: contraction elements 32 t + 8 g .. + 7.
__device__ __forceinline__ bf16x8 token_operand(const uint16_t* lds, int row, int K, int t, int g) {
  return *reinterpret_cast<const bf16x8*>(lds + row * (K + 8) + 32 * t + 8 * g);
}

// ---------------------------------------------------------------------------
// Absorb, bf16 in.  Grid (n_head, kv_rank / 64); 256 threads.  DN = d_nope (multiple of 32).
// LDS: W_UK[h][0:DN][c0:c0+64] with a 160-byte row pitch (40 dwords = 8 * odd),
// then kTC staged q_nope rows.  q_abs^T = W_UK^T q_nope^T: the weight columns
// are the M dimension (read transposed from LDS), tokens the N dimension, so
// each lane ends with four consecutive columns of one token.
// ---------------------------------------------------------------------------
// WIDE (many tokens): the token tiles of a chunk accumulate as independent
// chains; otherwise one tile after another (faster at decode-step sizes, where
// a chunk holds one or two tiles).  Both give the same bits.
template <typename TO, bool WIDE>
__global__ __launch_bounds__(256) void absorb_mfma(int H, int DN, int R, int kv_rank, int64_t n_tok,
                                                   const uint16_t* __restrict__ q_nope,
                                                   const uint16_t* __restrict__ q_pe,
                                                   const uint16_t* __restrict__ w_uk,
                                                   TO* __restrict__ q_abs) {
  constexpr int PITCH = 80;  // elements per weight row in LDS (64 used)
  extern __shared__ __attribute__((aligned(16))) uint16_t wl[];  // [DN][PITCH], then [kTC][DN + 8]
  uint16_t* al = wl + DN * PITCH;
  const int h = blockIdx.x, c0 = blockIdx.y * kCols;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, g = lane >> 4;
  const int D = kv_rank + R;
  const int ksteps = DN / 32;
  const uint16_t* qbase = q_nope + (int64_t)h * DN;  // token n at qbase + n * H * DN
  const int64_t qstride = (int64_t)H * DN;

  // Weight slice: thread tid stages 16 bytes of rows p = tid / 8 + 32 i; its
  // loads go out together with the first token chunk's.
  const uint16_t* wsrc = w_uk + (int64_t)h * DN * kv_rank + c0;
  {
    const int pr = tid >> 3, c = (tid & 7) * 8;
    u32x4 st[kMaxK];
#pragma unroll
    for (int i = 0; i < kMaxK; ++i)
      if (i < ksteps) st[i] = *reinterpret_cast<const u32x4*>(wsrc + (int64_t)(pr + 32 * i) * kv_rank + c);
    bf16x8 v[kStagePer];
    load_tokens(v, qbase, qstride, 0, n_tok, DN, tid);
#pragma unroll
    for (int i = 0; i < kMaxK; ++i)
      if (i < ksteps) *reinterpret_cast<u32x4*>(wl + (pr + 32 * i) * PITCH + c) = st[i];
    store_tokens(al, v, DN, tid);
  }

  // The rope tail q_abs[n][h][kv_rank:] = q_pe[n][h] is copied by the first
  // column slice, eight elements per thread and step.
  if (blockIdx.y == 0) {
    const int r8 = R / 8;
    if (R % 8 == 0) {
      for (int64_t idx = tid; idx < n_tok * r8; idx += 256) {
        const int64_t n = idx / r8;
        const int r = (int)(idx - n * r8) * 8;
        const u32x4 v = *reinterpret_cast<const u32x4*>(q_pe + (n * H + h) * R + r);
        TO* dst = q_abs + (n * H + h) * D + kv_rank + r;
        if constexpr (sizeof(TO) == 2) {
          *reinterpret_cast<u32x4*>(dst) = v;
        } else {
          const bf16x8 b = as_bf16x8(v);
          *reinterpret_cast<f32x4*>(dst) = f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
          *reinterpret_cast<f32x4*>(dst + 4) = f32x4{(float)b[4], (float)b[5], (float)b[6], (float)b[7]};
        }
      }
    } else {
      for (int64_t idx = tid; idx < n_tok * R; idx += 256) {
        const int64_t n = idx / R;
        const int r = (int)(idx - n * R);
        store_c(q_abs, (n * H + h) * D + kv_rank + r, bf16_to_f32(q_pe[(n * H + h) * R + r]));
      }
    }
  }
  __syncthreads();

  // This wave's 16 weight columns as the A operand (rows p read transposed from LDS).
  const int cw = w * 16;
  bf16x8 B[kMaxK];
#pragma unroll
  for (int t = 0; t < kMaxK; ++t) {
    if (t < ksteps) {
      const int prow = 32 * t + 8 * g + (l16 >> 2);
      const int col = cw + 4 * (l16 & 3);
      const s16x4 b0 = lds_read_tr16(wl + prow * PITCH + col);
      const s16x4 b1 = lds_read_tr16(wl + (prow + 4) * PITCH + col);
      B[t] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      B[t] = zero_bf16x8();
    }
  }
  for (int64_t m0 = 0; m0 < n_tok; m0 += kTC) {
    if (m0 > 0) {
      __syncthreads();  // every wave is done with the previous chunk
      bf16x8 v[kStagePer];
      load_tokens(v, qbase, qstride, m0, n_tok, DN, tid);
      store_tokens(al, v, DN, tid);
      __syncthreads();
    }
    if constexpr (WIDE) {
      const int live = (int)(((n_tok - m0 < kTC ? n_tok - m0 : kTC) + 15) / 16);  // token tiles in the chunk
      dispatch_tiles(live, [&](auto nt_c) {
        constexpr int NT = decltype(nt_c)::value;
        f32x4 acc[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < kMaxK; ++t)
          if (t < ksteps) {
#pragma unroll
            for (int j = 0; j < NT; ++j) acc[j] = mfma16x16x32(B[t], token_operand(al, 16 * j + l16, DN, t, g), acc[j]);
          }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int64_t n = m0 + 16 * j + l16;
          if (n < n_tok) store4(q_abs, (n * H + h) * D + c0 + cw + 4 * g, acc[j]);
        }
      });
    } else {
      for (int s16 = 0; s16 < kTC && m0 + s16 < n_tok; s16 += 16) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < kMaxK; ++t)
          if (t < ksteps) acc = mfma16x16x32(B[t], token_operand(al, s16 + l16, DN, t, g), acc);
        const int64_t n = m0 + s16 + l16;
        if (n < n_tok) store4(q_abs, (n * H + h) * D + c0 + cw + 4 * g, acc);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Decompress, bf16 weights.  Grid (n_head, d_v / 64); 256 threads; kv_rank = KR
// (multiple of 32, at most 512).  Each wave keeps its 16 weight rows in VGPRs
// (the A operand of out^T = W_UV o_lat^T); o_lat rows are staged in LDS kTC
// tokens at a time and read as the N-dimension operand, so each lane ends with
// output columns j4 .. j4 + 3 of one token.
// ---------------------------------------------------------------------------
template <typename TI, typename TO, bool WIDE>
__global__ __launch_bounds__(256) void decompress_mfma(int H, int DV, int KR, int64_t n_tok,
                                                       const TI* __restrict__ o_lat,
                                                       const uint16_t* __restrict__ w_uv,
                                                       TO* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) uint16_t ol[];  // [kTC][KR + 8]
  const int h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, g = lane >> 4;
  const int j_b = blockIdx.y * kCols + w * 16 + l16;  // weight row (output index) of this lane's A operand
  const int ksteps = KR / 32;
  const TI* obase = o_lat + (int64_t)h * KR;  // token n at obase + n * H * KR
  const int64_t ostride = (int64_t)H * KR;
  bf16x8 Bk[kMaxK];
  const uint16_t* wrow = w_uv + ((int64_t)h * DV + j_b) * KR + 8 * g;
#pragma unroll
  for (int t = 0; t < kMaxK; ++t)
    Bk[t] = (t < ksteps && j_b < DV) ? load8(wrow + 32 * t) : zero_bf16x8();
  const int j4 = blockIdx.y * kCols + w * 16 + 4 * g;
  for (int64_t m0 = 0; m0 < n_tok; m0 += kTC) {
    if (m0 > 0) __syncthreads();  // every wave is done with the previous chunk
    {
      bf16x8 v[kStagePer];
      load_tokens(v, obase, ostride, m0, n_tok, KR, tid);
      store_tokens(ol, v, KR, tid);
    }
    __syncthreads();
    if constexpr (WIDE) {
      const int live = (int)(((n_tok - m0 < kTC ? n_tok - m0 : kTC) + 15) / 16);  // token tiles in the chunk
      dispatch_tiles(live, [&](auto nt_c) {
        constexpr int NT = decltype(nt_c)::value;
        f32x4 acc[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < kMaxK; ++t)
          if (t < ksteps) {
#pragma unroll
            for (int j = 0; j < NT; ++j) acc[j] = mfma16x16x32(Bk[t], token_operand(ol, 16 * j + l16, KR, t, g), acc[j]);
          }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int64_t n = m0 + 16 * j + l16;
          if (n < n_tok && j4 < DV) store4(out, (n * H + h) * DV + j4, acc[j]);
        }
      });
    } else {
      for (int s16 = 0; s16 < kTC && m0 + s16 < n_tok; s16 += 16) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < kMaxK; ++t)
          if (t < ksteps) acc = mfma16x16x32(Bk[t], token_operand(ol, s16 + l16, KR, t, g), acc);
        const int64_t n = m0 + s16 + l16;
        if (n < n_tok && j4 < DV) store4(out, (n * H + h) * DV + j4, acc);
      }
    }
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

hipError_t launch_absorb(int H, int DN, int R, int KR, int64_t n_tok, const void* q_nope, const void* q_pe,
                         const void* w_uk, bool in_bf16, void* q_abs, bool out_bf16, hipStream_t stream) {
  if (n_tok == 0) return hipSuccess;
  // (Four-column output stores need rows of a multiple of 4 elements.)
  const bool mfma = in_bf16 && DN % 32 == 0 && KR % kCols == 0 && DN <= 512 && R % 4 == 0;
  if (mfma) {
    const dim3 grid(H, KR / kCols);
    const size_t lds = (size_t)DN * 80 * 2 + (size_t)kTC * (DN + 8) * 2;
    const uint16_t *qn = static_cast<const uint16_t*>(q_nope), *qp = static_cast<const uint16_t*>(q_pe),
                   *wk = static_cast<const uint16_t*>(w_uk);
    // Independent tile chains from two chunks on (measured: slower for one chunk).
    const bool wide = n_tok > kTC;
    if (out_bf16) {
      auto k = wide ? absorb_mfma<uint16_t, true> : absorb_mfma<uint16_t, false>;
      hipLaunchKernelGGL(k, grid, dim3(256), lds, stream, H, DN, R, KR, n_tok, qn, qp, wk, static_cast<uint16_t*>(q_abs));
    } else {
      auto k = wide ? absorb_mfma<float, true> : absorb_mfma<float, false>;
      hipLaunchKernelGGL(k, grid, dim3(256), lds, stream, H, DN, R, KR, n_tok, qn, qp, wk, static_cast<float*>(q_abs));
    }
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
  const bool mfma = w_bf16 && KR % 32 == 0 && KR <= 512 && DV % 4 == 0;
  if (mfma) {
    const dim3 grid(H, (DV + kCols - 1) / kCols);
    const uint16_t* wv = static_cast<const uint16_t*>(w_uv);
    const size_t lds = (size_t)kTC * (KR + 8) * 2;
    // Independent tile chains from 33 tokens on (measured: slower at 32).
    const bool wide = n_tok > 32;
#define MLA_DECOMP(TI, TO)                                                                                 \
  hipLaunchKernelGGL((wide ? decompress_mfma<TI, TO, true> : decompress_mfma<TI, TO, false>), grid, dim3(256), \
                     lds, stream, H, DV, KR, n_tok, static_cast<const TI*>(o_lat), wv, static_cast<TO*>(out))
    if (o_bf16 && out_bf16) MLA_DECOMP(uint16_t, uint16_t);
    else if (o_bf16) MLA_DECOMP(uint16_t, float);
    else if (out_bf16) MLA_DECOMP(float, uint16_t);
    else MLA_DECOMP(float, float);
#undef MLA_DECOMP
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
