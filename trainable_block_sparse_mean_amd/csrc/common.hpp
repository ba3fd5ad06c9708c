// Device helpers shared by the gfx950 kernels of the InfLLM-V2 sparse path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace infv2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;        // head dim supported on the GPU
constexpr int kBS = 64;        // key block size supported on the GPU
constexpr int kMaxG = 16;      // heads per GQA group (MFMA N dimension)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D = A(16x32) * B(32x16) + C on the matrix cores, bf16 in, fp32 accumulate.
// Operand layout (wave64): lane l feeds row (A) / column (B) l % 16 with the
// eight k-slots 8*(l/16) .. 8*(l/16)+7; the 16x16 result gives lane l column
// l % 16 and rows 4*(l/16) .. 4*(l/16)+3.
__device__ __forceinline__ floatx4 mfma_16x16x32(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void store16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(f)));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// fp64 -> bf16 bit pattern, round to nearest even, without an intermediate
// fp32 rounding.  Normal range: add the rounding bias at the last kept
// mantissa bit of the double and truncate; results below 2^-126 (bf16
// subnormals) are rounded on the fixed 2^-133 grid.
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double x) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  const uint32_t sign = static_cast<uint32_t>(u >> 48) & 0x8000u;
  const uint64_t a = u & 0x7fffffffffffffffull;
  if (a > 0x7ff0000000000000ull) return sign | 0x7fc0u;           // NaN
  const double ax = __longlong_as_double(static_cast<long long>(a));
  if (ax < 1.1754943508222875e-38) {                               // < 2^-126
    const double r = rint(ax * 0x1p133);                           // integer count of 2^-133
    return sign | static_cast<uint32_t>(r);                        // 0..128 (128 = 2^-126)
  }
  const uint64_t lsb = (a >> 45) & 1ull;                           // last kept bit (7 mantissa bits)
  const uint64_t rounded = (a + 0x0000100000000000ull - 1ull + lsb) & ~((1ull << 45) - 1ull);
  const double rv = __longlong_as_double(static_cast<long long>(rounded));
  if (rv >= 0x1p128) return sign | 0x7f80u;                        // overflow -> inf
  return sign | (__float_as_uint(static_cast<float>(rv)) >> 16);   // exact conversion
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// number of set bits of `mask` in lanes below the calling lane
__device__ __forceinline__ int mask_rank(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

}  // namespace infv2
