// swa_common.h -- small device helpers shared by the libswa kernels.
// gfx950 (CDNA4) only: 64-lane wavefronts, MFMA matrix cores, 160 KB LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

// Sum over groups of `width` consecutive lanes (power of 2, at most 64),
// the same value in every lane of a group, without LDS: DPP within rows of
// 16 lanes (neighbour in the quad, the other lane pair of the quad, the
// mirrored half-row, the mirrored row; each step adds two values that are
// already uniform over their halves, so every lane adds the same two
// numbers), then the gfx950 row swaps for lanes l ^ 16 and l ^ 32.
template <int width>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(width >= 1 && width <= 64 && (width & (width - 1)) == 0, "power of 2");
  auto dpp = [](float v, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value,
                                                      0xf, 0xf, false));
  };
  if constexpr (width >= 2) x += dpp(x, std::integral_constant<int, 0xb1>{});   // quad_perm 1,0,3,2
  if constexpr (width >= 4) x += dpp(x, std::integral_constant<int, 0x4e>{});   // quad_perm 2,3,0,1
  if constexpr (width >= 8) x += dpp(x, std::integral_constant<int, 0x141>{});  // row_half_mirror
  if constexpr (width >= 16) x += dpp(x, std::integral_constant<int, 0x140>{}); // row_mirror
  if constexpr (width >= 32) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  }
  if constexpr (width >= 64) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  }
  return x;
}

// x of lane l ^ o (o = 8, 16 or 32), without LDS.
template <int o>
__device__ __forceinline__ float lane_xor(float x) {
  static_assert(o == 8 || o == 16 || o == 32, "lane distance");
  if constexpr (o == 8) {
    // l ^ 8 is l + 8 mod 16 within a row of 16: row_ror:8
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
  } else {
    // the row swaps return (x of the lower row, x of the upper row) in every
    // lane of the pair of rows
    const auto a = o == 16
                       ? __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false)
                       : __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const bool upper = (__lane_id() & o) != 0;
    return __uint_as_float(upper ? a[0] : a[1]);
  }
}

}  // namespace swa
