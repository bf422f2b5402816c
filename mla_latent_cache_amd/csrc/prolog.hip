// Cache-append prolog of MLA decode, for gfx950.
//
// For each new token n (vLLM cpu_mla page, do_kv_cache_update; CANN
// aclnnMlaProlog page, the c^KV = RmsNorm(.) and k^R = ROPE(.) formulas):
//   cache row slots[n]  <-  [ RmsNorm(c_kv[n]) | rope(k_pe[n], pos[n]) ]
//   q_pe[n][h]          <-  rope(q_pe[n][h], pos[n])          (in place)
// RmsNorm is gamma * x / sqrt(mean(x^2) + eps); rope rotates pairs by
// pos * base^(-2j/d_rope) (memra mla.rs page, rope_neox / rope_interleaved).
//
// The work is HBM-bound and tiny per token, so the kernel is laid out for
// coalesced 16-byte accesses and short latency chains, not for arithmetic.
// One workgroup of 256 threads per token:
//   - threads j < d_rope/2 each form one angle pos * base^(-2j/d_rope) (in
//     double, reduced to [-pi, pi]) and its float cosine and sine, into LDS;
//   - wave 0 normalises the latent row (8 consecutive elements per lane, so
//     kv_rank 512 is one 16-byte load per lane; the sum of squares is a wave
//     reduction) and writes it to the cache row;
//   - threads 64 .. 64 + d_rope/16 rotate 16-element chunks of k_pe into the
//     cache row, and every thread rotates (head, chunk) items of q_pe in place.
// The latent row and the first q_pe item are loaded before the barrier that
// publishes the angle table, so their memory latency overlaps the angle math.
#include <math.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace mla {
namespace {

constexpr int kAppendThreads = 256;
constexpr uint32_t kBadSlot = 0x10u;  // a slot at or past the end of the cache
constexpr int kNeox = 0;
constexpr double kTwoPi = 6.283185307179586;
constexpr double kInvTwoPi = 0.15915494309189535;

struct AppendArgs {
  const void* c_kv;       // [n_tok][kv_rank]
  const void* k_pe;       // [n_tok][d_rope]
  const void* gamma;      // [kv_rank] or null
  void* q_pe;             // [n_tok][n_head][d_rope] or null
  const int32_t* pos;     // [n_tok]
  const int64_t* slots;   // [n_tok]
  void* cache;            // [num_slots][kv_rank + d_rope]
  uint32_t* err;          // data-error word or null
  int64_t n_tok, num_slots;
  int kv_rank, d_rope, n_head;
  float eps;
  double inv_freq[kRopeTableMax];  // base^(-2j/d_rope), j < d_rope/2
};

// ---- P consecutive elements of a storage type, as floats ----
template <int P>
__device__ __forceinline__ void loadn(const uint16_t* p, float* v) {
  if constexpr (P == 8) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int k = 0; k < P; ++k) v[k] = bf16_to_f32(p[k]);
  }
}
template <int P>
__device__ __forceinline__ void loadn(const float* p, float* v) {
  if constexpr (P == 8) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = a[k];
      v[4 + k] = b[k];
    }
  } else {
#pragma unroll
    for (int k = 0; k < P; ++k) v[k] = p[k];
  }
}
template <int P>
__device__ __forceinline__ void storen(uint16_t* p, const float* v) {
  if constexpr (P == 8) {
    const u32x4 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                     pack_bf16x2(v[6], v[7])};
    *reinterpret_cast<u32x4*>(p) = w;
  } else {
#pragma unroll
    for (int k = 0; k < P; ++k) p[k] = f32_to_bf16(v[k]);
  }
}
template <int P>
__device__ __forceinline__ void storen(float* p, const float* v) {
  if constexpr (P == 8) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
  } else {
#pragma unroll
    for (int k = 0; k < P; ++k) p[k] = v[k];
  }
}

// Element offsets (within one rope row) of the two P-element runs of chunk c,
// and the pair layout inside them.  NEOX: pair k of the chunk is
// (x[cP + k], x[half + cP + k]).  Interleaved: the chunk is the 2P elements
// x[2cP ..], pair k is (x[2j], x[2j + 1]) with j = cP + k.  In both, pair k
// rotates by angle index j = cP + k.
template <int STYLE, int P>
__device__ __forceinline__ void chunk_offsets(int half, int c, int* o0, int* o1) {
  if constexpr (STYLE == kNeox) {
    *o0 = c * P;
    *o1 = half + c * P;
  } else {
    *o0 = 2 * c * P;
    *o1 = 2 * c * P + P;
  }
}
template <int STYLE, int P>
__device__ __forceinline__ void rotate(float* x0, float* x1, const float* cs, const float* sn) {
  if constexpr (STYLE == kNeox || P == 1) {
#pragma unroll
    for (int k = 0; k < P; ++k) {
      const float u = x0[k], v = x1[k];
      x0[k] = u * cs[k] - v * sn[k];
      x1[k] = u * sn[k] + v * cs[k];
    }
  } else {
#pragma unroll
    for (int k = 0; k < P; ++k) {
      float* e = k < P / 2 ? x0 : x1;
      const int i = 2 * (k % (P / 2));
      const float u = e[i], v = e[i + 1];
      e[i] = u * cs[k] - v * sn[k];
      e[i + 1] = u * sn[k] + v * cs[k];
    }
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// RmsNorm of one latent row into the cache row by one wave, element by
// element (any kv_rank); the second pass re-reads the row from cache.
template <typename TI, typename TC>
__device__ __forceinline__ void norm_row_elementwise(const AppendArgs& a, const TI* src, TC* dst, int lane) {
  const TI* g = static_cast<const TI*>(a.gamma);
  const int R = a.kv_rank;
  float ss = 0.f;
  for (int i = lane; i < R; i += 64) {
    float x;
    loadn<1>(src + i, &x);
    ss += x * x;
  }
  ss = wave_sum(ss);
  const float rinv = 1.0f / sqrtf(ss / (float)R + a.eps);
  for (int i = lane; i < R; i += 64) {
    float x, gv = 1.f;
    loadn<1>(src + i, &x);
    if (g) loadn<1>(g + i, &gv);
    x = x * rinv * gv;
    storen<1>(dst + i, &x);
  }
}

template <typename TI, typename TC, int STYLE, int P>
__global__ __launch_bounds__(kAppendThreads) void cache_append_kernel(const AppendArgs a) {
  __shared__ float2 ang[kRopeTableMax];  // (cos, sin) of angle index j
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t n = blockIdx.x;
  const int half = a.d_rope >> 1;
  const int cpr = half / P;  // rope chunks per rope row
  const int64_t slot = a.slots[n];
  const bool write_row = slot >= 0 && slot < a.num_slots;
  if (tid == 0 && slot >= a.num_slots && a.err) atomicOr(a.err, kBadSlot);
  TC* row = static_cast<TC*>(a.cache) + (write_row ? slot : 0) * (int64_t)(a.kv_rank + a.d_rope);

  // Loads that do not need the angles: the latent row (wave 0) and the first
  // q_pe item of every thread.
  const TI* g = static_cast<const TI*>(a.gamma);
  const TI* src = static_cast<const TI*>(a.c_kv) + n * a.kv_rank;
  float x[2][8];
  float rinv = 0.f;
  const int nv = a.kv_rank / 8;
  if constexpr (P == 8) {
    if (w == 0 && write_row) {
      float ss = 0.f;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int v = lane + 64 * r;
        if (v < nv) {
          loadn<8>(src + 8 * v, x[r]);
#pragma unroll
          for (int k = 0; k < 8; ++k) ss += x[r][k] * x[r][k];
        }
      }
      ss = wave_sum(ss);
      rinv = 1.0f / sqrtf(ss / (float)a.kv_rank + a.eps);
    }
  }
  const int items = a.q_pe ? a.n_head * cpr : 0;
  TI* qrow = static_cast<TI*>(a.q_pe) + n * (int64_t)a.n_head * a.d_rope;
  float q0[P], q1[P];
  int qo0 = 0, qo1 = 0;
  if (tid < items) {
    const int h = tid / cpr, c = tid - h * cpr;
    chunk_offsets<STYLE, P>(half, c, &qo0, &qo1);
    qo0 += h * a.d_rope;
    qo1 += h * a.d_rope;
    loadn<P>(qrow + qo0, q0);
    loadn<P>(qrow + qo1, q1);
  }

  if (half > 0) {
    const int pos = a.pos[n];
    for (int j = tid; j < half; j += kAppendThreads) {
      const double th = (double)pos * a.inv_freq[j];
      const double turns = rint(th * kInvTwoPi);
      const float r = (float)fma(-turns, kTwoPi, th);
      float sv, cv;
      sincosf(r, &sv, &cv);
      ang[j] = make_float2(cv, sv);
    }
  }
  __syncthreads();

  if (write_row) {
    if (w == 0) {
      if constexpr (P == 8) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int v = lane + 64 * r;
          if (v < nv) {
            float gv[8];
            if (g) {
              loadn<8>(g + 8 * v, gv);
            } else {
#pragma unroll
              for (int k = 0; k < 8; ++k) gv[k] = 1.f;
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) x[r][k] = x[r][k] * rinv * gv[k];
            storen<8>(row + 8 * v, x[r]);
          }
        }
      } else {
        norm_row_elementwise<TI, TC>(a, src, row, lane);
      }
    } else if (tid >= 64 && tid - 64 < cpr) {
      const int c = tid - 64;
      float cs[P], sn[P];
#pragma unroll
      for (int k = 0; k < P; ++k) {
        const float2 e = ang[c * P + k];
        cs[k] = e.x;
        sn[k] = e.y;
      }
      int o0, o1;
      chunk_offsets<STYLE, P>(half, c, &o0, &o1);
      const TI* kp = static_cast<const TI*>(a.k_pe) + n * a.d_rope;
      float k0[P], k1[P];
      loadn<P>(kp + o0, k0);
      loadn<P>(kp + o1, k1);
      rotate<STYLE, P>(k0, k1, cs, sn);
      storen<P>(row + a.kv_rank + o0, k0);
      storen<P>(row + a.kv_rank + o1, k1);
    }
  }

  for (int it = tid; it < items; it += kAppendThreads) {
    const int h = it / cpr, c = it - h * cpr;
    if (it != tid) {
      chunk_offsets<STYLE, P>(half, c, &qo0, &qo1);
      qo0 += h * a.d_rope;
      qo1 += h * a.d_rope;
      loadn<P>(qrow + qo0, q0);
      loadn<P>(qrow + qo1, q1);
    }
    float cs[P], sn[P];
#pragma unroll
    for (int k = 0; k < P; ++k) {
      const float2 e = ang[c * P + k];
      cs[k] = e.x;
      sn[k] = e.y;
    }
    rotate<STYLE, P>(q0, q1, cs, sn);
    storen<P>(qrow + qo0, q0);
    storen<P>(qrow + qo1, q1);
  }
}

template <typename TI, typename TC, int STYLE>
hipError_t launch_typed(const AppendArgs& a, bool fast, int64_t grid, hipStream_t stream) {
  if (fast)
    hipLaunchKernelGGL((cache_append_kernel<TI, TC, STYLE, 8>), dim3((unsigned)grid), dim3(kAppendThreads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((cache_append_kernel<TI, TC, STYLE, 1>), dim3((unsigned)grid), dim3(kAppendThreads), 0,
                       stream, a);
  return hipGetLastError();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

hipError_t launch_cache_append(const CacheAppend& c, hipStream_t stream) {
  AppendArgs a = {};
  a.c_kv = c.c_kv;
  a.k_pe = c.k_pe;
  a.gamma = c.gamma;
  a.q_pe = c.q_pe;
  a.pos = c.positions;
  a.slots = c.slots;
  a.cache = c.cache;
  a.err = c.err;
  a.n_tok = c.n_tok;
  a.num_slots = c.num_slots;
  a.kv_rank = c.kv_rank;
  a.d_rope = c.d_rope;
  a.n_head = c.n_head;
  a.eps = c.eps;
  const int half = c.d_rope / 2;
  for (int j = 0; j < half; ++j) a.inv_freq[j] = pow(c.rope_base, -2.0 * j / c.d_rope);

  const bool fast = c.kv_rank % 8 == 0 && c.kv_rank <= 1024 && c.d_rope % 16 == 0 && aligned16(c.c_kv) &&
                    aligned16(c.k_pe) && aligned16(c.gamma) && aligned16(c.q_pe) && aligned16(c.cache);
  // One workgroup per token.
  if (c.n_tok > 0x7fffffff) return hipErrorInvalidValue;
  const int64_t grid = c.n_tok;
  if (grid == 0) return hipSuccess;
  if (c.in_bf16) {
    if (c.cache_bf16)
      return c.interleaved ? launch_typed<uint16_t, uint16_t, 1>(a, fast, grid, stream)
                           : launch_typed<uint16_t, uint16_t, kNeox>(a, fast, grid, stream);
    return c.interleaved ? launch_typed<uint16_t, float, 1>(a, fast, grid, stream)
                         : launch_typed<uint16_t, float, kNeox>(a, fast, grid, stream);
  }
  if (c.cache_bf16)
    return c.interleaved ? launch_typed<float, uint16_t, 1>(a, fast, grid, stream)
                         : launch_typed<float, uint16_t, kNeox>(a, fast, grid, stream);
  return c.interleaved ? launch_typed<float, float, 1>(a, fast, grid, stream)
                       : launch_typed<float, float, kNeox>(a, fast, grid, stream);
}

}  // namespace mla
