// Device helpers shared by the gfx950 kernels of the InfLLM-V2 sparse path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace infv2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

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
// Two floats to a bf16 pair (round to nearest even), lo in the low half: one
// v_cvt_pk_bf16_f32 (converting the halves separately costs four instructions).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{lo, hi}, bf16x2));
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

// Slot of 16-byte chunk c in LDS row r: c ^ swz(r), with swz a linear map of
// the row's low 4 bits (bit0 = r0, bit1 = r1, bit2 = r0^r2, bit3 = r0^r1^r3).
// It is chosen so that every fragment read below is free of bank conflicts
// whether the LDS serves 8 or 16 lanes of a 16-byte read, or 16 or 32 lanes
// of an 8-byte transposing read, per cycle: any 8 aligned rows have distinct
// low 3 slot bits, any 4 aligned rows distinct slot bits 1-2 and 2-3, and
// any 8 aligned rows distinct slot bits 1-3.
__device__ __forceinline__ int swz(int r) {
  return (r & 3) | (((r ^ (r >> 2)) & 1) << 2) | (((r ^ (r >> 1) ^ (r >> 3)) & 1) << 3);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(p)));
}

// reductions over lanes l, l^16 (the two rows of a row pair) and l, l^32
// (the two wave halves): v_permlane{16,32}_swap of a value with itself
// returns both partners' values
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One direct-to-LDS load: 64 lanes x 16 bytes land contiguously at LDS byte
// address `lds` (M0), read from the scalar base address plus each lane's
// 32-bit byte offset.  Issued from asm so the compiler does not serialise the
// later LDS reads behind it; completion is awaited explicitly (wait_dma)
// before the workgroup barrier that publishes the block.  No output registers.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  // the base must be wave-uniform; readfirstlane keeps it in SGPRs.  The
  // builtin returns int: both halves go through uint32_t so that the low
  // half is zero-extended, not sign-extended, into the 64-bit address.
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32)));
  const uint64_t sbase = (static_cast<uint64_t>(hi) << 32) | lo;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(sbase) : "memory", "m0");
}

// One direct-to-LDS load of 4 bytes per active lane (lane l writes LDS byte
// address lds + 4 l).  Same contract as dma16.
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32)));
  const uint64_t sbase = (static_cast<uint64_t>(hi) << 32) | lo;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(sbase) : "memory", "m0");
}

// Wait until at most N of this wave's vector memory loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Wait for register values produced by global loads here, once, on every
// path: afterwards they count as written by this (empty) asm, so no later
// instruction inherits a wait on those loads -- which would also wait on the
// block prefetches issued after them.
__device__ __forceinline__ float settle_f(float x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ bf16x8 settle(bf16x8 x) {
  u32x4 w = as_u32x4(x);
  asm volatile("" : "+v"(w));
  return as_bf16x8(w);
}

}  // namespace infv2
