// Host-side constant tables of liblynx, built once per process.
//
// Code map (page "Lynx: the KV cache does not have to arrive whole",
// section 3, non-linear transform): the magnitude level of u = |y| in [0,1]
// is m = round-half-up(127 ln(1 + alpha u) / ln(1 + alpha)), alpha = 255.
// The encoder takes m exactly as the number of thresholds T[k] <= u, where
// T[k] is found by bisection over fp32 bit patterns with the level evaluated
// in double precision.  The bucket table (level at the start of each
// 5-mantissa-bit bucket of u) lets the encoder find the level with one table
// read and one comparison.
//
// Decode (same section, the cut; section 4 for draft vs full): the 8-bit
// code q gives m = q >= 0 ? q : ~q and yhat = sign ((1 + alpha)^(m/127) - 1)
// / alpha, tabulated for all 256 codes; the draft of anchor a is the code
// 16 a + 7.
#include <cmath>
#include <cstring>
#include <mutex>

#include "lynx_internal.h"

namespace lynx {
namespace {

double level_of(float u) {
  return static_cast<double>(kLevels) * std::log1p(kAlpha * static_cast<double>(u)) /
         std::log1p(kAlpha);
}

float float_from_bits(uint32_t b) {
  float f;
  std::memcpy(&f, &b, sizeof f);
  return f;
}

CodeTable build_code_table() {
  CodeTable t;
  t.t[0] = 0.0f;
  const uint32_t one = 0x3F800000u;  // bits of 1.0f
  for (int k = 1; k <= kLevels; ++k) {
    const double target = k - 0.5;
    // smallest bit pattern b in [0, one] with level(b) >= target
    uint32_t lo = 0, hi = one;
    while (lo < hi) {
      const uint32_t mid = lo + (hi - lo) / 2;
      if (level_of(float_from_bits(mid)) >= target)
        hi = mid;
      else
        lo = mid + 1;
    }
    t.t[k] = float_from_bits(lo);
  }
  return t;
}

// number of thresholds T[1..127] not above u
int count_thresholds(const CodeTable &t, float u) {
  int m = 0;
  for (int k = 1; k <= kLevels; ++k) m += t.t[k] <= u ? 1 : 0;
  return m;
}

BucketTable build_bucket_table(const CodeTable &t) {
  BucketTable b;
  b.ok = t.t[1] > float_from_bits(kBucketFirstKey << kBucketShift);
  b.base[0] = 0;
  for (int i = 1; i < kBuckets - 1; ++i) {
    const uint32_t key = kBucketFirstKey + static_cast<uint32_t>(i) - 1u;
    const int lo = count_thresholds(t, float_from_bits(key << kBucketShift));
    const int hi = count_thresholds(t, float_from_bits(((key + 1u) << kBucketShift) - 1u));
    b.base[i] = static_cast<uint8_t>(lo);
    if (hi > lo + 1) b.ok = false;
  }
  b.base[kBuckets - 1] = static_cast<uint8_t>(kLevels);
  return b;
}

double yhat_of_code(int q) {
  const int m = q >= 0 ? q : -q - 1;
  const double g = (std::pow(1.0 + kAlpha, static_cast<double>(m) / kLevels) - 1.0) / kAlpha;
  return q >= 0 ? g : -g;
}

DecodeTable build_decode_table() {
  DecodeTable d;
  for (int q = -128; q < 128; ++q) d.y[q + 128] = static_cast<float>(yhat_of_code(q));
  return d;
}

DraftTable build_draft_table() {
  DraftTable d;
  for (int nib = 0; nib < 16; ++nib) {
    const int a = nib >= 8 ? nib - 16 : nib;  // two's complement int4
    d.y[nib] = static_cast<float>(yhat_of_code(16 * a + 7));
  }
  return d;
}

FixedDecodeTable build_fixed_table() {
  FixedDecodeTable d;
  for (int q = -128; q < 128; ++q)
    d.y[q + 128] = static_cast<int32_t>(std::llround(std::ldexp(yhat_of_code(q), kFixedYBits)));
  for (int nib = 0; nib < 16; ++nib) {
    const int a = nib >= 8 ? nib - 16 : nib;
    d.draft[nib] = static_cast<int32_t>(std::llround(std::ldexp(yhat_of_code(16 * a + 7), kFixedYBits)));
  }
  return d;
}

std::once_flag g_once;
CodeTable g_code;
DecodeTable g_decode;
DraftTable g_draft;
FixedDecodeTable g_fixed;
BucketTable g_bucket;

void init_tables() {
  g_code = build_code_table();
  g_bucket = build_bucket_table(g_code);
  g_decode = build_decode_table();
  g_draft = build_draft_table();
  g_fixed = build_fixed_table();
}

}  // namespace

const CodeTable &code_table() {
  std::call_once(g_once, init_tables);
  return g_code;
}

const DecodeTable &decode_table() {
  std::call_once(g_once, init_tables);
  return g_decode;
}

const DraftTable &draft_table() {
  std::call_once(g_once, init_tables);
  return g_draft;
}

const FixedDecodeTable &fixed_decode_table() {
  std::call_once(g_once, init_tables);
  return g_fixed;
}

const BucketTable &bucket_table() {
  std::call_once(g_once, init_tables);
  return g_bucket;
}

}  // namespace lynx
