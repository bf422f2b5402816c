// The fused MLA prolog (CANN operator page "aclnnMlaProlog": the four paths
// from the hidden states x to the absorbed queries and the cache rows), for
// gfx950:
//   c^Q  = RmsNorm(x W^DQ)                  -> gemm 1, finish 1 (gain), finish 2 (1 / RMS)
//   q^C  = c^Q W^UQ,  q^R' = c^Q W^QR        -> gemm 2, finish 2
//   cache row <- [RmsNorm(x W^DKV) | ROPE(x W^KR)], q^R = ROPE(q^R')
//                                           -> the cache-append kernel
//   q_abs = [q^C W^UK | q^R]                 -> the absorb kernel
// x W^DQ, x W^DKV and x W^KR are one GEMM over the three weight matrices (x
// read once per output tile); so are c^Q W^UQ and c^Q W^QR.  Weights are
// stored [out][in], so both MFMA operands are 16-byte runs along K straight
// from global memory: at decode sizes (tens of tokens) the products are
// bound by the weight reads, and the K dimension is split over workgroups to
// put every compute unit on them.  Intermediates are bf16, as the inputs;
// every product and the norms accumulate in float32.
#include <math.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace mla {
namespace {

constexpr int kTokTile = 64;  // tokens per workgroup pass (four MFMA column tiles)
constexpr int kKBatch = 4;    // k-steps of 32 per batch of activation loads
constexpr int kKChunk = 16;   // k-steps of 32 per chunk: weight loads in flight and LDS-staged activations

// part[split][n][o] = sum over this split's k of x[n][k] * W[o][k], for the
// rows o of the concatenated segments.  Each wave takes 16 rows (one
// segment) and the workgroup's tokens, NT tiles of 16 (registers sized to the
// tiles in use).  Per chunk of kKChunk k-steps the wave's weight loads go out
// first (HBM); meanwhile the workgroup stages its tokens' activations for
// the chunk in LDS once (rows XOR-swizzled by row % 16 in 16-byte units, so
// the operand reads are free of bank conflicts) instead of every wave
// reading them from L2.
template <int NT>
__global__ __launch_bounds__(256) void skinny_gemm(const SkinnyGemm g) {
  constexpr int CH = 4 * kKChunk;  // 16-byte chunks of a staged row (kKChunk k-steps of 32)
  __shared__ __attribute__((aligned(16))) u32x4 xs[16 * NT][CH];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, grp = lane >> 4;
  const int o0 = blockIdx.x * 64 + 16 * w;  // first output row of the wave
  const bool active = o0 < g.N;             // (the workgroup's barriers need every wave)
  int si = 0, base = 0;
  while (si + 1 < g.n_seg && o0 >= base + g.seg[si].rows) base += g.seg[si++].rows;
  const uint16_t* wrow = g.seg[si].w + (int64_t)((active ? o0 - base : 0) + l16) * g.K + 8 * grp;
  const int k0 = blockIdx.y * g.kper;
  const int k1 = k0 + g.kper < g.K ? k0 + g.kper : g.K;
  const int64_t t0 = (int64_t)blockIdx.z * kTokTile;
  const int nt = g.n_tok - t0 >= 16 * NT ? NT : (int)((g.n_tok - t0 + 15) / 16);  // token tiles in use
  f32x4 acc[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kc = k0; kc < k1; kc += 32 * kKChunk) {
    u32x4 a[kKChunk];
#pragma unroll
    for (int u = 0; u < kKChunk; ++u)
      a[u] = active && kc + 32 * u < k1 ? *reinterpret_cast<const u32x4*>(wrow + kc + 32 * u)
                                        : u32x4{0u, 0u, 0u, 0u};
    // Stage x[t0 + r][kc + 8 c .. + 7] at xs[r][c ^ (r % 16)] (zeros past the
    // tokens or the split).
    for (int i = tid; i < 16 * NT * CH; i += 256) {
      const int r = i / CH, c = i - r * CH;
      const int64_t tok = t0 + r;
      const int k = kc + 8 * c;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (tok < g.n_tok && k < k1) v = *reinterpret_cast<const u32x4*>(g.x + tok * g.K + k);
      xs[r][c ^ (r & 15)] = v;
    }
    __syncthreads();
    if (active) {
#pragma unroll
      for (int u = 0; u < kKChunk; ++u) {
        if (kc + 32 * u >= k1) break;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          if (tt >= nt) continue;
          const int r = 16 * tt + l16;
          const u32x4 b = xs[r][(4 * u + grp) ^ (r & 15)];
          acc[tt] = mfma16x16x32(as_bf16x8(a[u]), as_bf16x8(b), acc[tt]);
        }
      }
    }
    __syncthreads();  // the staging area is refilled for the next chunk
  }
  if (!active) return;
  // Lane (l16, grp) holds token column l16 of each tile and rows 4 grp .. + 3.
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int64_t tok = t0 + 16 * tt + l16;
    if (tt < nt && tok < g.n_tok)
      *reinterpret_cast<f32x4*>(g.part + ((int64_t)blockIdx.y * g.n_tok + tok) * g.N + o0 + 4 * grp) = acc[tt];
  }
}

__device__ __forceinline__ float load_gain(const void* gamma, bool bf16, int i) {
  if (!gamma) return 1.f;
  return bf16 ? bf16_to_f32(static_cast<const uint16_t*>(gamma)[i]) : static_cast<const float*>(gamma)[i];
}

// Sum over the split partials of one output column (the splits in order,
// loads eight at a time so the row costs a few memory latencies).
__device__ __forceinline__ float sum_splits(const float* p, int64_t sstride, int splits) {
  float v = 0.f;
  int s = 0;
  for (; s + 8 <= splits; s += 8) {
    float t[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) t[k] = p[(s + k) * sstride];
#pragma unroll
    for (int k = 0; k < 8; ++k) v += t[k];
  }
  for (; s < splits; ++s) v += p[s * sstride];
  return v;
}

// Finish 1, one thread per (token, column): the sums of x W^DQ go to the
// float32 row the norm reads and, times gamma_q, to the bf16 c^Q the second
// product reads (RmsNorm's per-token 1 / RMS is a scale of the row, so it is
// applied after that product, in finish 2); those of x W^DKV and x W^KR go to
// the cache append as they are (bf16).
constexpr int kFinishPerThread = 16;  // q_rank <= 256 * 16
__global__ __launch_bounds__(256) void prolog_finish1(const PrologArgs a) {
  const int64_t n = blockIdx.y;
  const int N = a.q_rank + a.kv_rank + a.d_rope;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= N) return;
  const float v = sum_splits(a.part + n * N + c, a.n_tok * (int64_t)N, a.splits1);
  if (c < a.q_rank) {
    a.yq[n * a.q_rank + c] = v;
    a.cq[n * a.q_rank + c] = f32_to_bf16(load_gain(a.gamma_q, true, c) * v);
  } else if (c < a.q_rank + a.kv_rank) {
    a.ckv[n * a.kv_rank + (c - a.q_rank)] = f32_to_bf16(v);
  } else {
    a.kpe[n * a.d_rope + (c - a.q_rank - a.kv_rank)] = f32_to_bf16(v);
  }
}

// Finish 2: the token's 1 / RMS(x W^DQ) (eps_q inside the root; float32, in
// a fixed order), then the split partials of (gamma c) W^UQ and (gamma c)
// W^QR summed and scaled by it into q^C [n][H][d_nope] and the unrotated q^R
// [n][H][d_rope] (bf16).
__global__ __launch_bounds__(256) void prolog_finish2(const PrologArgs a) {
  const int64_t n = blockIdx.y;
  const int tid = threadIdx.x;
  const float* y = a.yq + n * a.q_rank;
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kFinishPerThread; ++j) {
    const int c = tid + 256 * j;
    const float v = c < a.q_rank ? y[c] : 0.f;
    ss += v * v;
  }
  __shared__ float red[4];
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float inv = 1.f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)a.q_rank + a.eps_q);
  const int NQ = a.n_head * a.d_nope, N = NQ + a.n_head * a.d_rope;
  const int c = blockIdx.x * 256 + tid;
  if (c >= N) return;
  const float v = sum_splits(a.part + n * N + c, a.n_tok * (int64_t)N, a.splits2) * inv;
  if (c < NQ) a.qn[n * NQ + c] = f32_to_bf16(v);
  else a.qp[n * (N - NQ) + (c - NQ)] = f32_to_bf16(v);
}

int pick_splits(int K, int64_t n_tok, int n_tiles) {
  // Enough workgroups for about four per compute unit, split K in whole
  // batches of k-steps, and keep the float32 partials under a quarter of the
  // weight bytes (splits <= K / (8 n_tok)).
  const int kb = 32 * kKBatch;
  int s = (1024 + n_tiles - 1) / n_tiles;
  const int by_k = K / kb > 0 ? K / kb : 1;
  const int64_t by_part = K / (8 * (n_tok > 0 ? n_tok : 1));
  if (s > by_k) s = by_k;
  if (s > by_part) s = (int)(by_part > 0 ? by_part : 1);
  return s < 1 ? 1 : s;
}

hipError_t launch_skinny(const SkinnyGemm& g0, hipStream_t stream) {
  SkinnyGemm g = g0;
  const int kb = 32 * kKBatch;
  g.kper = ((g.K + g.splits - 1) / g.splits + kb - 1) / kb * kb;
  const dim3 grid((g.N + 63) / 64, (g.K + g.kper - 1) / g.kper, (unsigned)((g.n_tok + kTokTile - 1) / kTokTile));
  // token tiles per pass: all four once a pass is full, else just those in use
  const int64_t t = g.n_tok >= kTokTile ? 4 : (g.n_tok + 15) / 16;
  if (t <= 1) hipLaunchKernelGGL(skinny_gemm<1>, grid, dim3(256), 0, stream, g);
  else if (t == 2) hipLaunchKernelGGL(skinny_gemm<2>, grid, dim3(256), 0, stream, g);
  else hipLaunchKernelGGL(skinny_gemm<4>, grid, dim3(256), 0, stream, g);
  return hipGetLastError();
}

}  // namespace

PrologPlan prolog_plan(int n_head, int d_nope, int d_rope, int kv_rank, int hidden, int q_rank, int64_t n_tok) {
  PrologPlan p;
  const int N1 = q_rank + kv_rank + d_rope, N2 = n_head * (d_nope + d_rope);
  p.splits1 = pick_splits(hidden, n_tok, (N1 + 63) / 64);
  p.splits2 = pick_splits(q_rank, n_tok, (N2 + 63) / 64);
  // the split counts the launches will realise (k per split rounded up to whole batches)
  const int kb = 32 * kKBatch;
  auto real = [&](int K, int s) { const int kper = ((K + s - 1) / s + kb - 1) / kb * kb; return (K + kper - 1) / kper; };
  p.splits1 = real(hidden, p.splits1);
  p.splits2 = real(q_rank, p.splits2);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t part1 = (size_t)p.splits1 * n_tok * N1 * 4, part2 = (size_t)p.splits2 * n_tok * N2 * 4;
  p.part_off = 0;
  p.cq_off = al(part1 > part2 ? part1 : part2);
  p.ckv_off = al(p.cq_off + (size_t)n_tok * q_rank * 2);
  p.kpe_off = al(p.ckv_off + (size_t)n_tok * kv_rank * 2);
  p.qn_off = al(p.kpe_off + (size_t)n_tok * d_rope * 2);
  p.qp_off = al(p.qn_off + (size_t)n_tok * n_head * d_nope * 2);
  p.yq_off = al(p.qp_off + (size_t)n_tok * n_head * d_rope * 2);
  p.bytes = al(p.yq_off + (size_t)n_tok * q_rank * 4);
  if (p.bytes == 0) p.bytes = 256;
  return p;
}

bool prolog_supported(int n_head, int d_nope, int d_rope, int kv_rank, int hidden, int q_rank) {
  return hidden % 32 == 0 && q_rank % 32 == 0 && q_rank <= 256 * kFinishPerThread && kv_rank % 16 == 0 &&
         d_rope % 16 == 0 && (n_head * d_nope) % 16 == 0 && (n_head * d_rope) % 16 == 0 && d_nope % 8 == 0;
}

hipError_t launch_prolog(const PrologArgs& a, hipStream_t stream) {
  if (a.n_tok == 0) return hipSuccess;
  if (a.n_tok > 65535) return hipErrorInvalidValue;  // grid rows of the finish kernels
  // 1: x [W^DQ; W^DKV; W^KR]^T
  SkinnyGemm g1 = {};
  g1.x = static_cast<const uint16_t*>(a.x);
  g1.seg[0] = {static_cast<const uint16_t*>(a.w_dq), a.q_rank};
  g1.seg[1] = {static_cast<const uint16_t*>(a.w_dkv), a.kv_rank};
  g1.seg[2] = {static_cast<const uint16_t*>(a.w_kr), a.d_rope};
  g1.n_seg = a.d_rope > 0 ? 3 : 2;
  g1.K = a.hidden;
  g1.N = a.q_rank + a.kv_rank + a.d_rope;
  g1.n_tok = a.n_tok;
  g1.splits = a.splits1;
  g1.part = a.part;
  hipError_t e = launch_skinny(g1, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prolog_finish1, dim3((unsigned)((g1.N + 255) / 256), (unsigned)a.n_tok), dim3(256), 0, stream,
                     a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 2: c^Q [W^UQ; W^QR]^T
  SkinnyGemm g2 = {};
  g2.x = a.cq;
  g2.seg[0] = {static_cast<const uint16_t*>(a.w_uq), a.n_head * a.d_nope};
  g2.seg[1] = {static_cast<const uint16_t*>(a.w_qr), a.n_head * a.d_rope};
  g2.n_seg = a.d_rope > 0 ? 2 : 1;
  g2.K = a.q_rank;
  g2.N = a.n_head * (a.d_nope + a.d_rope);
  g2.n_tok = a.n_tok;
  g2.splits = a.splits2;
  g2.part = a.part;
  if ((e = launch_skinny(g2, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(prolog_finish2, dim3((unsigned)((g2.N + 255) / 256), (unsigned)a.n_tok), dim3(256), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 3: cache rows [RmsNorm(c^KV) | ROPE(k^R)], q^R rotated in place
  CacheAppend c = {};
  c.c_kv = a.ckv;
  c.k_pe = a.kpe;
  c.gamma = a.gamma_kv;
  c.q_pe = a.d_rope > 0 ? a.qp : nullptr;
  c.positions = a.positions;
  c.slots = a.slots;
  c.cache = a.cache;
  c.err = a.err;
  c.n_tok = a.n_tok;
  c.num_slots = a.num_slots;
  c.kv_rank = a.kv_rank;
  c.d_rope = a.d_rope;
  c.n_head = a.n_head;
  c.eps = a.eps_kv;
  c.rope_base = a.rope_base;
  c.in_bf16 = true;
  c.cache_bf16 = a.cache_bf16;
  c.interleaved = a.interleaved;
  if ((e = launch_cache_append(c, stream)) != hipSuccess) return e;
  // 4: q_abs = [q^C W^UK | q^R]
  return launch_absorb(a.n_head, a.d_nope, a.d_rope, a.kv_rank, a.n_tok, a.qn, a.d_rope > 0 ? a.qp : nullptr, a.w_uk,
                       true, a.q_abs, a.q_bf16, stream);
}

}  // namespace mla
