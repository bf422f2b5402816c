// Device-side helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Buffer-resource word 3 for raw (unswizzled, untyped) 32-bit-indexed access.
constexpr int kRsrcWord3 = 0x00020000;

// bfloat16 bits -> float (exact widening).
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed pair of bfloat16 in one dword, lo = a: one hardware
// conversion (round to nearest even, NaN stays NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Reinterpret four dwords as eight bfloat16 MFMA operand lanes.
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, z);
}

template <typename T>
struct Storage;

template <>
struct Storage<float> {
  __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, int64_t i, float v) { p[i] = v; }
};

template <>
struct Storage<uint16_t> {
  __device__ __forceinline__ static float load(const uint16_t* p, int64_t i) {
    return bf16_to_f32(p[i]);
  }
  __device__ __forceinline__ static void store(uint16_t* p, int64_t i, float v) {
    p[i] = f32_to_bf16(v);
  }
};

// 16 x 16 x 32 bf16 matrix-core product, float32 accumulate.
// Lane l: A row l%16, k = 8*(l/16)..+7; B column l%16, same k; C rows 4*(l/16)+i, column l%16.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read: within each 16-lane group, lane j receives, as element e,
// the 16-bit word (j % 4) of the 8 bytes addressed by lane 4*e + j/4 of its group.
__device__ __forceinline__ s16x4 lds_read_tr16(const void* lds_byte_addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_byte_addr));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRsrcWord3);
}

// 16 bytes from buffer offset `voff` straight into LDS at (wave base + 16 * lane).
// Offsets at or beyond the buffer size deliver zeros.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rsrc, void* lds_wave_base,
                                                  uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds_wave_base), 16, voff, 0, 0, 0);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource (base, size in bytes) as four scalar words.  The words
// are taken from the first lane: a resource is wave-uniform, and the inline
// assembly that consumes it needs scalar registers even where the compiler has
// computed a uniform value in vector registers.
__device__ __forceinline__ i32x4 raw_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r = {__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
             __builtin_amdgcn_readfirstlane((int)(uint32_t)((a >> 32) & 0xffffu)),
             __builtin_amdgcn_readfirstlane((int)bytes), kRsrcWord3};
  return r;
}

// LDS byte address of a __shared__ object (32-bit local address space).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) void*)(p));
}

// Asynchronous 16-byte copy per lane, buffer offset `voff` -> LDS (wave base + 16 * lane);
// offsets at or past the resource size deliver zeros.  Issued as inline assembly so the
// compiler does not track it: the caller orders it with explicit vmcnt waits.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_wave_base, uint32_t voff) {
  // The LDS base is wave-uniform; take it from the first lane so it is a scalar operand.
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_wave_base);
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(base), "v"(voff), "s"(rsrc)
      : "memory", "m0");
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

// Max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the four 16-lane rows
// holding one MFMA output column), with the row-swapping permlane instructions.
__device__ __forceinline__ float max4rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float sum4rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

}  // namespace mla
