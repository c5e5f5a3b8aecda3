// Cross-lane helpers of the matrix-core attention kernels (wave64, DPP
// and permlane swaps on gfx950) and the exact fp16 split of an fp32 value
// into two MFMA operand halves.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace lynx {
namespace lanes {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// ---- cross-lane helpers -----------------------------------------------------
// value of lane n ^ 8 within each row of 16 lanes (DPP row rotate by 8);
// the masked forms write only lanes n >= 8 (banks 2, 3 of each row) or only
// lanes n < 8 (banks 0, 1) and leave `keep` in the others
__device__ __forceinline__ float ror8_to_hi(float keep, float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      __builtin_bit_cast(int, keep), __builtin_bit_cast(int, x), 0x128, 0xF, 0xC, false));
}
__device__ __forceinline__ float ror8_to_lo(float keep, float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      __builtin_bit_cast(int, keep), __builtin_bit_cast(int, x), 0x128, 0xF, 0x3, false));
}
// (a rotation within the row reads a valid lane for every lane, so the
// destination needs no previous value)
template <int kCtrl>
__device__ __forceinline__ int dpp_all(int x) {
  return __builtin_amdgcn_mov_dpp(x, kCtrl, 0xF, 0xF, true);
}
__device__ __forceinline__ float ror8(float x) {
  return __builtin_bit_cast(float, dpp_all<0x128>(__builtin_bit_cast(int, x)));
}
__device__ __forceinline__ double ror8(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const int lo = dpp_all<0x128>(static_cast<int>(u));
  const int hi = dpp_all<0x128>(static_cast<int>(u >> 32));
  return __builtin_bit_cast(double, static_cast<uint64_t>(static_cast<uint32_t>(lo)) |
                                        (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32));
}
// op over lanes l, l ^ 16, l ^ 32, l ^ 48 (v_permlane16_swap / v_permlane32_swap
// of a value with itself return the values of the two rows being paired)
template <typename Op>
__device__ __forceinline__ float xrows(float v, Op op) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ double xrows_sum(double v) {
#pragma unroll
  for (int step = 0; step < 2; ++step) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = static_cast<uint32_t>(u), hi = static_cast<uint32_t>(u >> 32);
    const auto l = step == 0 ? __builtin_amdgcn_permlane16_swap(lo, lo, false, false)
                             : __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto h = step == 0 ? __builtin_amdgcn_permlane16_swap(hi, hi, false, false)
                             : __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    v = __builtin_bit_cast(double, static_cast<uint64_t>(l[0]) | (static_cast<uint64_t>(h[0]) << 32)) +
        __builtin_bit_cast(double, static_cast<uint64_t>(l[1]) | (static_cast<uint64_t>(h[1]) << 32));
  }
  return v;
}
struct MaxOp { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };
struct SumOp { __device__ float operator()(float a, float b) const { return a + b; } };

// max over all 64 lanes
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, dpp_all<0xB1>(__builtin_bit_cast(int, v))));
  v = fmaxf(v, __builtin_bit_cast(float, dpp_all<0x4E>(__builtin_bit_cast(int, v))));
  v = fmaxf(v, __builtin_bit_cast(float, dpp_all<0x124>(__builtin_bit_cast(int, v))));
  v = fmaxf(v, ror8(v));
  return xrows(v, MaxOp());
}

// x split for a column half: the high half keeps fp16(trunc x) (the
// truncation is the f32 bit pattern with the low 13 mantissa bits cleared),
// the low half the remainder; both land in the two k slots of one element.
__device__ __forceinline__ uint32_t split_dup(float x, uint32_t keep_mask) {
  const float y = x - __uint_as_float(__float_as_uint(x) & keep_mask);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(y, y));
}

}  // namespace lanes
}  // namespace lynx
