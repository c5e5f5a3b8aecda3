// Re-cut of one unit of 32 elements from 4 + 4 nibble planes into
// b + (8 - b) bit streams (device code shared by the packer and the
// encoder's cut variants).
//
// Page "Lynx: the KV cache does not have to arrive whole", section 3 cuts
// the 8-bit code 4 + 4; section 7 names other cuts as untried.  A b-bit
// anchor is the top b bits of the two's-complement code (an arithmetic
// shift), the residual its low 8 - b bits.  Element k of a unit is nibble
// k of the unit's 16 plane bytes (word k / 8, nibble k % 8); in a stream
// it occupies bits k*b .. k*b + b - 1, least significant first, so a unit
// is exactly b words of the anchor stream and 8 - b of the residual.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lynx {
namespace cut {

// Code of element k, from the 4 words of each nibble plane.
__device__ __forceinline__ int code_of(const uint32_t *a4, const uint32_t *r4, int k) {
  const uint32_t an = (a4[k >> 3] >> (4 * (k & 7))) & 15u;
  const uint32_t rn = (r4[k >> 3] >> (4 * (k & 7))) & 15u;
  return static_cast<int8_t>(static_cast<uint8_t>((an << 4) | rn));
}

// Pack 32 values of B bits (low bits of v[k]) into B words, least
// significant first.
template <int B>
__device__ __forceinline__ void pack32(const uint32_t *v, uint32_t *w) {
  uint64_t acc = 0;
  int nb = 0, wi = 0;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    acc |= static_cast<uint64_t>(v[k] & ((1u << B) - 1u)) << nb;
    nb += B;
    if (nb >= 32) {
      w[wi++] = static_cast<uint32_t>(acc);
      acc >>= 32;
      nb -= 32;
    }
  }
}

// The B anchor words and 8 - B residual words of a unit.
template <int B>
__device__ __forceinline__ void unit(const uint32_t (&a4)[4], const uint32_t (&r4)[4],
                                     uint32_t (&wa)[B], uint32_t (&wr)[8 - B]) {
  constexpr int RB = 8 - B;
  uint32_t va[32], vr[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const int q = code_of(a4, r4, k);
    va[k] = static_cast<uint32_t>(q >> RB);  // arithmetic: the signed anchor
    vr[k] = static_cast<uint32_t>(q) & ((1u << RB) - 1u);
  }
  pack32<B>(va, wa);
  pack32<RB>(vr, wr);
}

}  // namespace cut
}  // namespace lynx
