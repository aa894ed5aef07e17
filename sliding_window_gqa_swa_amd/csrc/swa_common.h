// swa_common.h -- small device helpers shared by the libswa kernels.
// gfx950 (CDNA4) only: 64-lane wavefronts, MFMA matrix cores, 160 KB LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/swa.h"

namespace swa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Non-negative remainder for any int64 numerator (m > 0).
__device__ __forceinline__ int64_t pos_mod(int64_t x, int64_t m) {
  int64_t r = x % m;
  return r < 0 ? r + m : r;
}

// bf16 bit pattern <-> fp32 (exact widening).
__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) {
  return __uint_as_float(h << 16);
}

// fp32 -> bf16 bit pattern, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu)) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Unpack 8 bf16 held in a 16-byte vector into fp32.
__device__ __forceinline__ void unpack8(const u32x4 w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Raw buffer loads (MUBUF): a 128-bit descriptor {base, num_records bytes,
// config}; a load whose offset is >= num_records returns zeros and makes no
// memory access, which gives branch-free predication of HBM reads.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
__device__ u32x4 llvm_raw_buffer_load_v4i32(i32x4 rsrc, int32_t voffset, int32_t soffset,
                                             int32_t aux) __asm("llvm.amdgcn.raw.buffer.load.v4i32");

struct __attribute__((packed)) BufferDesc {
  const void* base;
  uint32_t num_records;
  uint32_t config;
};
constexpr uint32_t kBufferConfigGfx9 = 0x00020000u;  // raw 32-bit dword access
constexpr int32_t kBufferOob = 0x7fffffff;           // an offset that is always out of range

__device__ __forceinline__ i32x4 make_buffer_rsrc(const void* base, uint32_t bytes) {
  BufferDesc d{base, bytes, kBufferConfigGfx9};
  return __builtin_bit_cast(i32x4, d);
}
__device__ __forceinline__ u32x4 buffer_load16(i32x4 rsrc, int32_t byte_offset) {
  return llvm_raw_buffer_load_v4i32(rsrc, byte_offset, 0, 0);
}

// Butterfly sum / max over groups of `width` consecutive lanes (power of 2).
template <int width>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}
template <int width>
__device__ __forceinline__ float group_max(float x) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
  return x;
}

}  // namespace swa
