// Fused-dequant single-query GQA decode attention on MFMA (GQA group <= 8).
//
// Page "Lynx: the KV cache does not have to arrive whole", section 4 (draft
// on the anchor stream, refinement on anchor + residual); page "LLM KV cache
// quantization", sections "The architecture" and "End-to-end flow" (read the
// compact cache, expand it only in registers, attention unchanged).
//
// Algebra.  With khat = c0 + c1*yhat and vhat = c0v + c1v*yhat per chunk
// and channel (c0 = mn + rg*mu, c1 = rg*s), a score is
//   sum_d q_d c0_d  +  sum_d (q_d c1_d) yhat_td
// and a 32-token chunk needs two dense products:
//   S^T[16 tok][16 col]  = Yk[16 tok][k] * W[k][16 col]   (v_mfma_i32_16x16x64_i8)
//   O^T[16 ch ][16 col] += Yv^T[16 ch][k] * P[k][16 col]  (v_mfma_f32_16x16x32_f16)
// Scores are exact integer products.  With 100x outlier channels a score
// reaches a few hundred and the output moves with a few fp32 ulps of it, so
// no part of a score is accumulated in fp32: yhat is held in fixed point,
// Y = round(yhat 2^30), and w = q c1 (bf16 query times the fp64 scale
// product) as W = floor(w 2^S), S per chunk so that |W| < 2^30.  Both are
// split into 4 signed bytes (Y = sum_i Y_i 2^(8i), likewise W), a table word
// holds the 4 bytes of one element's Y, so k = 4*element + i.  Column n of
// the 16 holds query head n % 8 at level L (the byte products Y_i W_j with
// i + j = L, weight 2^(8L)): its W operand for element d is the byte string
// (W_L, W_(L-1), W_(L-2), W_(L-3)) of that element (0 outside 0..3), one
// v_perm.  Three products per step take levels (6, 5), (4, 3) and (2, 1) for
// columns n < 8 and n >= 8; int32 accumulation is exact, and the dropped
// level 0 (Y_0 W_0) weighs 2^-48 of the largest term.  The six level sums of
// a (token, head) are combined in fp64 and scaled by 2^-(S + 22).  The chunk
// bias sum_d q_d c0_d is summed in fp64, and only the small difference of a
// score to the running maximum is rounded before exp2.
// For the value product yhat is an fp16 pair (hi, lo) with 22 significant
// bits in two consecutive k slots (k = 2*element + {0: hi, 1: lo}), and the
// 16 columns are [hi part | lo part] of the probabilities of the 8 query
// heads: a probability p is split into a truncated fp16 high part and the
// fp16 remainder, so the product sums (hi + lo) * p.
//
// Lane l of a wave: n = l % 16 (MFMA row / column), r = l / 16 (k group).
// Keys are token-major: lane (n, r) of K tile t reads the 16 bytes of
// channels 32r .. 32r+31 of token 16t + n and feeds channels 32r + 4st + i
// (i < 4) in step st.  Values are channel-major with the chunk's tokens
// permuted so that word r of channel 16ct + n holds exactly the 8 tokens
// whose probabilities lane (n, r) provides: tokens 4r..4r+3 (step 0) and
// 16+4r..16+4r+3 (step 1).
//
// Work split: one workgroup of 16 waves (8 K/V wave pairs, one workgroup per
// CU) per (request, KV head, run of pages); each pair streams a contiguous
// part of the run, the K wave scoring chunk c while the V wave sums the
// values of chunk c - 1, each with its next chunk's codes and scales in
// flight.  Between chunks the K wave stages the next chunk's W words and
// c0 in LDS, so that a score step only reads its four W words.  The block
// merges its pairs through LDS and writes the output itself when one run
// covers the request; otherwise it writes a partial (base-2 max m, sum l,
// unnormalised o) and a second, small kernel merges the runs exactly.
//
// Other cuts of the code (page "Lynx: the KV cache does not have to arrive
// whole", section 7 names 6 + 2, 2 + 6 and 5 + 3): the kernel reads a
// b-bit anchor stream (and an (8 - b)-bit residual stream), where a unit of
// 32 elements -- the 16 bytes of a 4-bit plane -- is b words with the
// fields least significant first.  A key lane reads its whole unit; a value
// lane reads the 2 or 3 words that hold its 8 fields and aligns them with
// v_alignbyte.  The fields become one table index byte per element: the
// code byte (a << (8 - b) | r) for the full code, which indexes the same
// table as the 4 + 4 code, or the anchor field for the draft, whose table
// row holds the draft value of the anchor's round-half-down centre.
#include <math.h>

#include <type_traits>

#include "lynx_internal.h"
#include "lynx_lanes.h"

namespace lynx {
namespace {

using namespace lanes;

constexpr int kHeads = 8;  // MFMA columns per part
constexpr float kSlack = 8.0f;  // log2 of the largest probability before rescaling

// LDS map in bytes.  The tables: 256 rows of 256 bytes, one row per code
// byte; a row's first 128 bytes hold the key table word (Y), its last 128
// the value table word (fp16 pair).  Full code and cuts: 32 copies of the
// word, copy l % 32 for lane l; 4 + 4 draft (row = two anchor nibbles,
// element 2j in the low one): 16 copies of the pair of words, copy l % 16.
// A wave's 4-byte reads are served 32 lanes (128 bytes) per pass, so no two
// lanes of a pass share a bank.  Its 8-byte reads are served 32 lanes per
// pass over 64 banks: lanes l and l + 16 read the same copy, which costs a
// second pass when their rows differ (32 copies of the pairs would avoid
// it at twice the table space).  The lane bits of a value read carry the
// 128-byte offset.
constexpr int kValueHalf = 128;
constexpr int kTableBytes = 256 * 256;
// The W words of a chunk's score products: [8 heads][32 units of 4
// channels + 1 pad unit] x 16 B (the pad turns each head's row by 4 banks,
// so the 8 heads of one read pass meet different banks).
constexpr int kWRowBytes = 33 * 16;
constexpr int kWBytes = kHeads * kWRowBytes;
// q as f64 [8 heads][130]: rows padded by 16 bytes, which turns each head's
// row by 4 banks, so the lanes of one LDS pass, which read the same
// channels of different heads, meet different banks
constexpr int kQStride = kDim + 2;
// Merge staging of the waves' value sums: rows of 128 floats padded to 132,
// so that the 8 lanes of each 128-byte pass of a 16-byte store (8 rows, one
// per lane) fall on 8 different 4-bank groups.
constexpr int kORow = kDim + 4;

struct MfmaTables {
  uint32_t full[256];   // code byte (a << 4 | r) -> fp16 hi | fp16 lo << 16 of yhat
  uint32_t draft[16];   // anchor nibble -> fp16 hi | fp16 lo << 16 of the draft yhat
  uint32_t kfull[256];  // code byte -> the 4 signed bytes of round(yhat 2^30)
  uint32_t kdraft[16];  // anchor nibble -> the same for the draft yhat
};

using Partials = AttnPartials;

__device__ __forceinline__ Partials partials_of(void *ws, const AttnShape &s) {
  return attn_partials(ws, s);
}

// ---- operand construction ---------------------------------------------------
// 8 nibble-pair codes of one anchor word a and residual word r (element k in
// nibble k): byte j of e is the code byte (a << 4 | r) of element 2j, byte j
// of o that of element 2j+1.
__device__ __forceinline__ void code_bytes(uint32_t a, uint32_t r, uint32_t &e, uint32_t &o) {
  e = ((a << 4) & 0xF0F0F0F0u) | (r & 0x0F0F0F0Fu);
  o = (a & 0xF0F0F0F0u) | ((r >> 4) & 0x0F0F0F0Fu);
}

// LDS byte address of table row x.byte[j]: byte 0 the lane's copy offset
// and table half (byte 0 of lb), byte 1 the row.
template <int J>
__device__ __forceinline__ uint32_t lut_addr(uint32_t x, uint32_t lb) {
  return __builtin_amdgcn_perm(x, lb, 0x0C0C0000u | ((4u + J) << 8));
}

// Table words of elements 4s .. 4s+3 of a code word pair (key table or
// value table by the lane bits): an i8 key operand (4 bytes per element) or
// an f16 value operand (hi, lo of each in consecutive k slots).
template <int S>
__device__ __forceinline__ u32x4 operand_full(uint32_t e, uint32_t o, uint32_t lb, const char *lut) {
  u32x4 w;
  w[0] = *reinterpret_cast<const uint32_t *>(lut + lut_addr<2 * S>(e, lb));
  w[1] = *reinterpret_cast<const uint32_t *>(lut + lut_addr<2 * S>(o, lb));
  w[2] = *reinterpret_cast<const uint32_t *>(lut + lut_addr<2 * S + 1>(e, lb));
  w[3] = *reinterpret_cast<const uint32_t *>(lut + lut_addr<2 * S + 1>(o, lb));
  return w;
}
template <int S>
__device__ __forceinline__ u32x4 operand_draft(uint32_t a, uint32_t lb, const char *lut) {
  const uint2 p0 = *reinterpret_cast<const uint2 *>(lut + lut_addr<2 * S>(a, lb));
  const uint2 p1 = *reinterpret_cast<const uint2 *>(lut + lut_addr<2 * S + 1>(a, lb));
  u32x4 w;
  w[0] = p0.x;
  w[1] = p0.y;
  w[2] = p1.x;
  w[3] = p1.y;
  return w;
}

// ---- b + (8 - b) cut streams --------------------------------------------------
// Words of a b-bit stream that hold the 8 fields of value lane r (fields
// 8r .. 8r + 7 of a unit, bytes r*b .. r*b + b - 1), over the 4 lanes r.
constexpr int cut_window_words(int b) {
  int n = 1;
  for (int r = 0; r < 4; ++r) {
    const int span = ((r * b + b - 1) >> 2) - ((r * b) >> 2) + 1;
    n = span > n ? span : n;
  }
  return n;
}

// Field k of B bits (least significant first) of a little-endian word array.
template <int B, int N>
__device__ __forceinline__ uint32_t cut_field(const uint32_t (&w)[N], int k) {
  const int p = k * B, i = p >> 5, o = p & 31;
  constexpr uint32_t kMask = (1u << B) - 1u;
  if (o + B <= 32) return (w[i] >> o) & kMask;
  return __builtin_amdgcn_alignbit(w[i + 1], w[i], static_cast<uint32_t>(o)) & kMask;
}

// Fields k0 .. k0 + 3 as the bytes of one word.
template <int B, int N>
__device__ __forceinline__ uint32_t cut_bytes(const uint32_t (&w)[N], int k0) {
  return cut_field<B>(w, k0) | (cut_field<B>(w, k0 + 1) << 8) | (cut_field<B>(w, k0 + 2) << 16) |
         (cut_field<B>(w, k0 + 3) << 24);
}

// 64 bits of a value lane's window starting at its first byte (shift in
// bytes, 0 .. 3).
template <int NW>
__device__ __forceinline__ void cut_align(const uint32_t (&w)[NW], uint32_t shift, uint32_t (&o)[2]) {
  const uint32_t w1 = NW > 1 ? w[NW > 1 ? 1 : 0] : 0u;
  const uint32_t w2 = NW > 2 ? w[NW > 2 ? 2 : 0] : 0u;
  o[0] = __builtin_amdgcn_alignbyte(w1, w[0], shift);
  o[1] = __builtin_amdgcn_alignbyte(w2, w1, shift);
}

// Table words of the 4 elements whose table index bytes are x.
__device__ __forceinline__ u32x4 operand_bytes(uint32_t x, uint32_t lb, const char *lut) {
  u32x4 w;
  w[0] = *reinterpret_cast<const uint32_t *>(lut + lut_addr<0>(x, lb));
  w[1] = *reinterpret_cast<const uint32_t *>(lut + lut_addr<1>(x, lb));
  w[2] = *reinterpret_cast<const uint32_t *>(lut + lut_addr<2>(x, lb));
  w[3] = *reinterpret_cast<const uint32_t *>(lut + lut_addr<3>(x, lb));
  return w;
}

// ---- streamed chunk data ----------------------------------------------------
__device__ __forceinline__ u32x4 load_nt(const u32x4 *p) {
  return __builtin_nontemporal_load(p);
}
__device__ __forceinline__ uint32_t load_nt(const uint32_t *p) {
  return __builtin_nontemporal_load(p);
}

// W word of one (channel, head) for the level products: the floor of
// w * 2^S (here w * 2^S + 0x80808080, so the truncating conversion is a
// floor and every byte carries a +128 bias), with the bias of each byte
// flipped back, is the 4-byte signed split (byte j = W_j); each product
// then takes the bytes its column's level needs.
__device__ __forceinline__ uint32_t w_bytes(double q, double c1s) {
  constexpr double kBias = 2155905152.0;  // 0x80808080
  return static_cast<uint32_t>(__builtin_fma(q, c1s, kBias)) ^ 0x80808080u;
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct LaneConst {
  int n, r, lane;
  uint32_t koff, voff, soff;  // lane byte offsets in a K chunk, a V chunk, a scale row
  bool lo;
  uint32_t lbk, lbv;   // lane bits of key and value table addresses
  uint32_t keep_mask;  // 0 for the high column half, ~0x1FFF for the low one
  uint32_t lvl[3];     // v_perm selectors of this column's W bytes in the 3 level products
  double sm2;          // sm_scale * log2(e)
  // cut streams: byte offsets of the lane's K unit within a chunk of the
  // anchor / residual stream, of its V window words (channel n, chunk
  // start), and the window's byte shift
  uint32_t kca, kcr;
  uint32_t vwa[3], vwr[3];
  uint32_t vsa, vsr;
};

// Lane offsets into b-bit and (8 - b)-bit streams.
template <int B>
__device__ __forceinline__ void cut_lane_offsets(LaneConst &lc) {
  constexpr int RB = 8 - B;
  lc.kca = static_cast<uint32_t>((4 * lc.n + lc.r) * 4 * B);
  lc.kcr = static_cast<uint32_t>((4 * lc.n + lc.r) * 4 * RB);
  const int ia = (lc.r * B) >> 2, ir = (lc.r * RB) >> 2;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    // a window word past the unit is never needed: read the unit's last word
    lc.vwa[j] = static_cast<uint32_t>(lc.n * 4 * B + 4 * (ia + j < B ? ia + j : B - 1));
    lc.vwr[j] = static_cast<uint32_t>(lc.n * 4 * RB + 4 * (ir + j < RB ? ir + j : RB - 1));
  }
  lc.vsa = static_cast<uint32_t>((lc.r * B) & 3);
  lc.vsr = static_cast<uint32_t>((lc.r * RB) & 3);
}

// ---- K/V wave pairs -----------------------------------------------------------
// The roles of a chunk are split between two waves, so that each holds half
// the registers of the whole chunk and a CU runs 16 waves (4 per SIMD).
// Wave p < 8 (the K wave of pair p) streams the key codes and scales of its
// run of chunks and computes each chunk's scores, running maximum and
// probabilities; wave p + 8 (the V wave) streams the value codes and scales
// of the same run and accumulates the value sums one chunk behind.  The K
// wave hands each chunk's probabilities, rescale factor and probability sum
// to its V wave through LDS (two buffers per pair); the block steps in
// lockstep, one barrier per chunk step.
constexpr int kPairs = 8;
constexpr int kPThreads = 128 * kPairs;
constexpr int kKSlotBytes = kWBytes + 1024;  // W words | c0k f64[128]
constexpr int kVSlotBytes = 512 + 512;       // c1v f32[128] | c0v f32[128]
// probabilities [tile][r][head][4 tokens] f32 (lane (n, r) of the K wave
// holds tokens 16 tile + 4r .. + 3 of head n % 8, tile = n / 8), then the
// rescale factor and the probability sum of the 8 heads
constexpr int kHandBytes = 1024 + 32 + 32;
constexpr int kPKSlotOff = kTableBytes;
constexpr int kPVSlotOff = kPKSlotOff + kPairs * kKSlotBytes;
constexpr int kPHandOff = kPVSlotOff + kPairs * kVSlotBytes;
constexpr int kPQOff = kPHandOff + kPairs * 2 * kHandBytes;
constexpr int kPLdsBytes = kPQOff + kHeads * kQStride * 8;
// after the chunk loop: o of every pair [pair][16 col][128 ch] f32 over the
// table space, then m, l of every pair's 8 heads
constexpr int kPMlOff = kPairs * 16 * kORow * 4;
static_assert(kPMlOff + kPairs * 2 * kHeads * 4 <= kPQOff, "merge area must fit below q");
static_assert(kKSlotBytes % 16 == 0 && kHandBytes % 16 == 0 && kPLdsBytes <= 160 * 1024,
              "LDS budget of one workgroup");

// Codes of a chunk.  4 + 4 planes: K tile t, anchor / residual of channels
// 32r .. of token 16t + n; V word r of channel 16ct + n.  b + (8 - b)
// streams (b != 4): the lane's K unit words of each tile, and the window
// words of its V fields in channel 16ct + n (residual words for the full
// code only).
template <int kBits>
struct KCodes {
  uint32_t ka[2][kBits], kr[2][8 - kBits];
};
template <>
struct KCodes<4> {
  u32x4 ka[2], kr[2];
};
template <int kBits>
struct VCodes {
  uint32_t va[8][cut_window_words(kBits)], vr[8][cut_window_words(8 - kBits)];
};
template <>
struct VCodes<4> {
  uint32_t va[8], vr[8];
};
struct KScales {
  float2 mnk, rgk, muk, sk;  // channels 2l, 2l+1
};
struct VScales {
  float2 mnv, rgv, muv, sv;
};

template <bool kFull, int kBits>
__device__ __forceinline__ void load_kcodes(KCodes<kBits> &cd, const PlanesArg &kp, size_t tile, int c,
                                            const LaneConst &lc) {
  if constexpr (kBits != 4) {
    // a tile is 1024 units of 4 * b bytes, a chunk 128 of them
    const size_t unit0 = tile * 1024 + static_cast<size_t>(c) * 128;
    const char *ka = reinterpret_cast<const char *>(kp.anchor) + unit0 * (4 * kBits);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < kBits; ++i)
        cd.ka[t][i] = load_nt(reinterpret_cast<const uint32_t *>(ka + lc.kca + t * 256 * kBits + 4 * i));
    if (kFull) {
      constexpr int RB = 8 - kBits;
      const char *kr = reinterpret_cast<const char *>(kp.residual) + unit0 * (4 * RB);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < RB; ++i)
          cd.kr[t][i] = load_nt(reinterpret_cast<const uint32_t *>(kr + lc.kcr + t * 256 * RB + 4 * i));
    }
    return;
  } else {
  const uint32_t koff = lc.koff;
  const size_t cbytes = tile * kPlaneTileBytes + static_cast<size_t>(c) * (kChunk * kDim / 2);
  const char *ka = reinterpret_cast<const char *>(kp.anchor) + cbytes;
  cd.ka[0] = load_nt(reinterpret_cast<const u32x4 *>(ka + koff));
  cd.ka[1] = load_nt(reinterpret_cast<const u32x4 *>(ka + koff + 1024));
  if (kFull) {
    const char *kr = reinterpret_cast<const char *>(kp.residual) + cbytes;
    cd.kr[0] = load_nt(reinterpret_cast<const u32x4 *>(kr + koff));
    cd.kr[1] = load_nt(reinterpret_cast<const u32x4 *>(kr + koff + 1024));
  }
  }
}

template <bool kFull, int kBits>
__device__ __forceinline__ void load_vcodes(VCodes<kBits> &cd, const PlanesArg &vp, size_t tile, int c,
                                            const LaneConst &lc) {
  if constexpr (kBits != 4) {
    const size_t unit0 = tile * 1024 + static_cast<size_t>(c) * 128;
    const char *va = reinterpret_cast<const char *>(vp.anchor) + unit0 * (4 * kBits);
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int j = 0; j < cut_window_words(kBits); ++j)
        cd.va[ct][j] = load_nt(reinterpret_cast<const uint32_t *>(va + ct * 64 * kBits + lc.vwa[j]));
    if (kFull) {
      constexpr int RB = 8 - kBits;
      const char *vr = reinterpret_cast<const char *>(vp.residual) + unit0 * (4 * RB);
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int j = 0; j < cut_window_words(RB); ++j)
          cd.vr[ct][j] = load_nt(reinterpret_cast<const uint32_t *>(vr + ct * 64 * RB + lc.vwr[j]));
    }
    return;
  } else {
  const uint32_t voff = lc.voff;
  const size_t cbytes = tile * kPlaneTileBytes + static_cast<size_t>(c) * (kChunk * kDim / 2);
  const char *va = reinterpret_cast<const char *>(vp.anchor) + cbytes;
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) cd.va[ct] = load_nt(reinterpret_cast<const uint32_t *>(va + voff + ct * 256));
  if (kFull) {
    const char *vr = reinterpret_cast<const char *>(vp.residual) + cbytes;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) cd.vr[ct] = load_nt(reinterpret_cast<const uint32_t *>(vr + voff + ct * 256));
  }
  }
}

__device__ __forceinline__ float2 scale_pair(const float *base, size_t off, uint32_t soff) {
  return *reinterpret_cast<const float2 *>(reinterpret_cast<const char *>(base) + off + soff);
}

__device__ __forceinline__ void load_kscales(KScales &sc, const PlanesArg &kp, size_t tile, int c,
                                             uint32_t soff) {
  const size_t pb = tile * kDim * 4;
  const size_t cb = (tile * kChunks + c) * kDim * 4;
  sc.muk = scale_pair(kp.chunk_mean, cb, soff);
  sc.sk = scale_pair(kp.chunk_maxabs, cb, soff);
  sc.mnk = scale_pair(kp.page_min, pb, soff);
  sc.rgk = scale_pair(kp.page_range, pb, soff);
}

__device__ __forceinline__ void load_vscales(VScales &sc, const PlanesArg &vp, size_t tile, int c,
                                             uint32_t soff) {
  const size_t pb = tile * kDim * 4;
  const size_t cb = (tile * kChunks + c) * kDim * 4;
  sc.muv = scale_pair(vp.chunk_mean, cb, soff);
  sc.sv = scale_pair(vp.chunk_maxabs, cb, soff);
  sc.mnv = scale_pair(vp.page_min, pb, soff);
  sc.rgv = scale_pair(vp.page_range, pb, soff);
}

// Chunk constants of the K wave's next chunk into its LDS slot: the W words
// and c0k.  c1k = rg * s is formed in fp64 (exact) and scaled by 2^S,
// S = 29 - e with e the exponent of qmax * max c1k (qmax = largest |q| of
// the group), so every |q * c1k * 2^S| stays below 2^30 (the fp32 maximum
// can undercut the fp64 one by an ulp, which still leaves it below
// 2^31 - 2^24, the range of a 4-byte signed split).  Lane l forms the W
// words of channels 2l, 2l + 1 for the 8 heads (q from the block's f64
// copy) and c0k of its two channels; returns 2^-(S + 22), the weight of the
// level sums assembled in score_chunk.
__device__ __forceinline__ double stage_kslot(const KScales &sc, char *slot, int lane, float qmax,
                                              const double *q64) {
  const float c1a = sc.rgk.x * sc.sk.x, c1b = sc.rgk.y * sc.sk.y;  // bound only
  const float bound = qmax * wave_max(fmaxf(c1a, c1b));
  int S = 0;
  const uint32_t eb = (__float_as_uint(bound) >> 23) & 0xFFu;
  if (bound > 0.0f && eb != 0xFFu) {
    const int e = eb != 0u ? static_cast<int>(eb) - 127
                           : -127 - __builtin_clz(__float_as_uint(bound)) + 9;
    S = 29 - e;
  }
  const double ks = __builtin_bit_cast(double, static_cast<uint64_t>(1023 + S) << 52);
  const double inv = __builtin_bit_cast(double, static_cast<uint64_t>(1023 - S - 22) << 52);
  const double c1x = static_cast<double>(sc.rgk.x) * sc.sk.x * ks;
  const double c1y = static_cast<double>(sc.rgk.y) * sc.sk.y * ks;
  char *wdst = slot + (lane >> 1) * 16 + (lane & 1) * 8;
  const double *qsrc = q64 + 2 * lane;
#pragma unroll
  for (int hh = 0; hh < kHeads; ++hh) {
    const double2 qq = *reinterpret_cast<const double2 *>(qsrc + hh * kQStride);
    *reinterpret_cast<uint2 *>(wdst + hh * kWRowBytes) = make_uint2(w_bytes(qq.x, c1x), w_bytes(qq.y, c1y));
  }
  double *c0k = reinterpret_cast<double *>(slot + kWBytes);
  reinterpret_cast<double2 *>(c0k)[lane] =
      make_double2(static_cast<double>(sc.mnk.x) + static_cast<double>(sc.rgk.x) * sc.muk.x,
                   static_cast<double>(sc.mnk.y) + static_cast<double>(sc.rgk.y) * sc.muk.y);
  return inv;
}

// Chunk bias sum_d q_d c0k_d in fp64 of the lane's head: lane (n, r) takes
// channels 32r + 16 (n >= 8) .. + 15, then lanes n, n ^ 8 and the 4 rows
// are summed.
__device__ __forceinline__ double chunk_bias(const char *slot, const double *q64, const LaneConst &lc) {
  const double *c0k = reinterpret_cast<const double *>(slot + kWBytes);
  const int d0 = 32 * lc.r + (lc.lo ? 16 : 0);
  const double *qh = q64 + (lc.n & 7) * kQStride + d0;
  double a0 = 0.0, a1 = 0.0;
#pragma unroll
  for (int k = 0; k < 16; k += 2) {
    const double2 qq = *reinterpret_cast<const double2 *>(qh + k);
    const double2 cc = *reinterpret_cast<const double2 *>(c0k + d0 + k);
    a0 = fma(qq.x, cc.x, a0);
    a1 = fma(qq.y, cc.y, a1);
  }
  double bias = a0 + a1;
  bias += ror8(bias);
  return xrows_sum(bias);
}

// Table index bytes of a K chunk: 4 + 4 code bytes of even / odd elements
// (full) or the anchor words (draft), per tile and word; drafts from a
// b-bit stream: the anchor fields of elements 8w .. 8w + 3 (e) and
// 8w + 4 .. 8w + 7 (o), one byte each.
template <bool kFull, int kBits>
__device__ __forceinline__ void key_bytes(const KCodes<kBits> &cd, uint32_t (&e)[2][4], uint32_t (&o)[2][4]) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if constexpr (kBits != 4) {
        e[t][w] = cut_bytes<kBits>(cd.ka[t], 8 * w);
        o[t][w] = cut_bytes<kBits>(cd.ka[t], 8 * w + 4);
        if (kFull) {
          e[t][w] = (e[t][w] << (8 - kBits)) | cut_bytes<8 - kBits>(cd.kr[t], 8 * w);
          o[t][w] = (o[t][w] << (8 - kBits)) | cut_bytes<8 - kBits>(cd.kr[t], 8 * w + 4);
        }
      } else if (kFull) {
        code_bytes(cd.ka[t][w], cd.kr[t][w], e[t][w], o[t][w]);
      } else {
        e[t][w] = cd.ka[t][w];
        o[t][w] = 0u;
      }
    }
}

// Chunk constants of the V wave's next chunk: c1v and c0v.
__device__ __forceinline__ void stage_vslot(const VScales &sc, char *slot, int lane) {
  float *c1v = reinterpret_cast<float *>(slot);
  float *c0v = c1v + kDim;
  reinterpret_cast<float2 *>(c1v)[lane] = make_float2(sc.rgv.x * sc.sv.x, sc.rgv.y * sc.sv.y);
  reinterpret_cast<float2 *>(c0v)[lane] =
      make_float2(__builtin_fmaf(sc.rgv.x, sc.muv.x, sc.mnv.x), __builtin_fmaf(sc.rgv.y, sc.muv.y, sc.mnv.y));
}

// K wave, one chunk: scores, online softmax (base 2); the probabilities, the
// rescale factor and the probability sum go to the hand-off buffer.
template <bool kFull, int kBits>
__device__ __forceinline__ void score_chunk(const uint32_t (&e)[2][4], const uint32_t (&o)[2][4],
                                            const char *slot, double inv_s, double bias,
                                            const LaneConst &lc, const char *lut,
                                            float &m_run, float &l_run, float *srow, char *hand) {
  const int n = lc.n, r = lc.r;

  // ---- scores: S^T = Yk * W, three level products per tile (exact int32) ----
  i32x4 sa0 = {0, 0, 0, 0}, sb0 = {0, 0, 0, 0}, sc0 = {0, 0, 0, 0};
  i32x4 sa1 = {0, 0, 0, 0}, sb1 = {0, 0, 0, 0}, sc1 = {0, 0, 0, 0};
  {
    const char *wrow = slot + (n & 7) * kWRowBytes + r * 128;
#pragma unroll
    for (int stp = 0; stp < 8; ++stp) {
      const u32x4 wv = *reinterpret_cast<const u32x4 *>(wrow + stp * 16);
      i32x4 ba, bb, bc;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ba[i] = static_cast<int>(__builtin_amdgcn_perm(wv[i], wv[i], lc.lvl[0]));
        bb[i] = static_cast<int>(__builtin_amdgcn_perm(wv[i], wv[i], lc.lvl[1]));
        bc[i] = static_cast<int>(__builtin_amdgcn_perm(wv[i], wv[i], lc.lvl[2]));
      }
      u32x4 a0, a1;
      const int w = stp >> 1;
      if constexpr (kBits != 4) {
        a0 = operand_bytes((stp & 1) ? o[0][w] : e[0][w], lc.lbk, lut);
        a1 = operand_bytes((stp & 1) ? o[1][w] : e[1][w], lc.lbk, lut);
      } else if (kFull) {
        if (stp & 1) {
          a0 = operand_full<1>(e[0][w], o[0][w], lc.lbk, lut);
          a1 = operand_full<1>(e[1][w], o[1][w], lc.lbk, lut);
        } else {
          a0 = operand_full<0>(e[0][w], o[0][w], lc.lbk, lut);
          a1 = operand_full<0>(e[1][w], o[1][w], lc.lbk, lut);
        }
      } else {
        if (stp & 1) {
          a0 = operand_draft<1>(e[0][w], lc.lbk, lut);
          a1 = operand_draft<1>(e[1][w], lc.lbk, lut);
        } else {
          a0 = operand_draft<0>(e[0][w], lc.lbk, lut);
          a1 = operand_draft<0>(e[1][w], lc.lbk, lut);
        }
      }
      const i32x4 y0 = __builtin_bit_cast(i32x4, a0), y1 = __builtin_bit_cast(i32x4, a1);
      sa0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(y0, ba, sa0, 0, 0, 0);
      sa1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(y1, ba, sa1, 0, 0, 0);
      sb0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(y0, bb, sb0, 0, 0, 0);
      sb1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(y1, bb, sb1, 0, 0, 0);
      sc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(y0, bc, sc0, 0, 0, 0);
      sc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(y1, bc, sc1, 0, 0, 0);
    }
  }

  // ---- assemble: lanes n < 8 take tile 0, lanes n >= 8 tile 1 (tokens 16t + 4r + i) ----
  const double scale2 = lc.sm2 * inv_s;
  const double bias2 = bias * lc.sm2;
  double sc2[4];
  float cmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    auto hi = [](int t0, int t1) {
      return __builtin_bit_cast(int, ror8_to_hi(__builtin_bit_cast(float, t0), __builtin_bit_cast(float, t1)));
    };
    auto lo = [](int t1, int t0) {
      return __builtin_bit_cast(int, ror8_to_lo(__builtin_bit_cast(float, t1), __builtin_bit_cast(float, t0)));
    };
    const int l6 = hi(sa0[i], sa1[i]), l5 = lo(sa1[i], sa0[i]);
    const int l4 = hi(sb0[i], sb1[i]), l3 = lo(sb1[i], sb0[i]);
    const int l2 = hi(sc0[i], sc1[i]), l1 = lo(sc1[i], sc0[i]);
    const int a = l6 * 256 + l5, b2 = l4 * 256 + l3, c2 = l2 * 256 + l1;
    const double t = fma(fma(static_cast<double>(a), 65536.0, static_cast<double>(b2)), 65536.0,
                         static_cast<double>(c2));
    sc2[i] = fma(t, scale2, bias2);
    cmax = fmaxf(cmax, static_cast<float>(sc2[i]));
  }
  cmax = fmaxf(cmax, ror8(cmax));
  cmax = xrows(cmax, MaxOp());
  const bool rescale = __builtin_amdgcn_ballot_w64(cmax > m_run + kSlack) != 0;
  float alpha = 1.0f;
  if (rescale) {
    const float m_new = fmaxf(m_run, cmax);
    alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
  }
  float p[4];
  float psum = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[i] = __builtin_amdgcn_exp2f(static_cast<float>(sc2[i] - static_cast<double>(m_run)));
    psum += p[i];
  }
  psum += ror8(psum);
  psum = xrows(psum, SumOp());
  l_run = l_run * alpha + psum;
  if (srow != nullptr) {
    constexpr double kLn2 = 0.69314718055994530942;
    *reinterpret_cast<float4 *>(srow + (lc.lo ? 16 : 0) + 4 * r) =
        make_float4(static_cast<float>(sc2[0] * kLn2), static_cast<float>(sc2[1] * kLn2),
                    static_cast<float>(sc2[2] * kLn2), static_cast<float>(sc2[3] * kLn2));
  }
  *reinterpret_cast<float4 *>(hand + (lc.lo ? 512 : 0) + r * 128 + (n & 7) * 16) =
      make_float4(p[0], p[1], p[2], p[3]);
  if (r == 0 && !lc.lo) {
    reinterpret_cast<float *>(hand + 1024)[n] = alpha;
    reinterpret_cast<float *>(hand + 1056)[n] = psum;
  }
}

// V wave, one chunk: O^T += Yv^T * P with the K wave's probabilities, then
// the chunk's affine map; acc is rescaled first when the K wave moved its
// running maximum.
template <bool kFull, int kBits>
__device__ __forceinline__ void value_chunk(const VCodes<kBits> &cd, const char *slot, const LaneConst &lc,
                                            const char *lut, floatx4 (&acc)[8], const char *hand) {
  const int n = lc.n, r = lc.r;
  const float *c1v = reinterpret_cast<const float *>(slot);
  const float *c0v = c1v + kDim;
  const float alpha = reinterpret_cast<const float *>(hand + 1024)[n & 7];
  const float psum = reinterpret_cast<const float *>(hand + 1056)[n & 7];
  const float4 p0 = *reinterpret_cast<const float4 *>(hand + r * 128 + (n & 7) * 16);
  const float4 p1 = *reinterpret_cast<const float4 *>(hand + 512 + r * 128 + (n & 7) * 16);
  if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) acc[ct] *= alpha;
  }
  // ---- P operands: step h holds tokens 16h + 4r + i of column n ----
  half8 pa0, pa1;
  {
    u32x4 w0, w1;
    w0[0] = split_dup(p0.x, lc.keep_mask);
    w0[1] = split_dup(p0.y, lc.keep_mask);
    w0[2] = split_dup(p0.z, lc.keep_mask);
    w0[3] = split_dup(p0.w, lc.keep_mask);
    w1[0] = split_dup(p1.x, lc.keep_mask);
    w1[1] = split_dup(p1.y, lc.keep_mask);
    w1[2] = split_dup(p1.z, lc.keep_mask);
    w1[3] = split_dup(p1.w, lc.keep_mask);
    pa0 = __builtin_bit_cast(half8, w0);
    pa1 = __builtin_bit_cast(half8, w1);
  }
  const float pc0 = lc.lo ? 0.0f : psum;  // the c0v term once per head (high half)
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) {
    half8 y0, y1;
    if constexpr (kBits != 4) {
      uint32_t win[2];
      cut_align<cut_window_words(kBits)>(cd.va[ct], lc.vsa, win);
      uint32_t xa = cut_bytes<kBits>(win, 0), xb = cut_bytes<kBits>(win, 4);
      if (kFull) {
        uint32_t wr[2];
        cut_align<cut_window_words(8 - kBits)>(cd.vr[ct], lc.vsr, wr);
        xa = (xa << (8 - kBits)) | cut_bytes<8 - kBits>(wr, 0);
        xb = (xb << (8 - kBits)) | cut_bytes<8 - kBits>(wr, 4);
      }
      y0 = __builtin_bit_cast(half8, operand_bytes(xa, lc.lbv, lut));
      y1 = __builtin_bit_cast(half8, operand_bytes(xb, lc.lbv, lut));
    } else if (kFull) {
      uint32_t e, o;
      code_bytes(cd.va[ct], cd.vr[ct], e, o);
      y0 = __builtin_bit_cast(half8, operand_full<0>(e, o, lc.lbv, lut));
      y1 = __builtin_bit_cast(half8, operand_full<1>(e, o, lc.lbv, lut));
    } else {
      y0 = __builtin_bit_cast(half8, operand_draft<0>(cd.va[ct], lc.lbv, lut));
      y1 = __builtin_bit_cast(half8, operand_draft<1>(cd.va[ct], lc.lbv, lut));
    }
    floatx4 ov = {0.0f, 0.0f, 0.0f, 0.0f};
    ov = __builtin_amdgcn_mfma_f32_16x16x32_f16(y0, pa0, ov, 0, 0, 0);
    ov = __builtin_amdgcn_mfma_f32_16x16x32_f16(y1, pa1, ov, 0, 0, 0);
    const float4 a1 = *reinterpret_cast<const float4 *>(c1v + 16 * ct + 4 * r);
    const float4 a0 = *reinterpret_cast<const float4 *>(c0v + 16 * ct + 4 * r);
    acc[ct][0] = __builtin_fmaf(a1.x, ov[0], __builtin_fmaf(a0.x, pc0, acc[ct][0]));
    acc[ct][1] = __builtin_fmaf(a1.y, ov[1], __builtin_fmaf(a0.y, pc0, acc[ct][1]));
    acc[ct][2] = __builtin_fmaf(a1.z, ov[2], __builtin_fmaf(a0.z, pc0, acc[ct][2]));
    acc[ct][3] = __builtin_fmaf(a1.w, ov[3], __builtin_fmaf(a0.w, pc0, acc[ct][3]));
  }
}

template <bool kFull, int kBits>
__global__ __launch_bounds__(kPThreads) void attn_pair_kernel(
    const uint16_t *__restrict__ q, PlanesArg kp, PlanesArg vp,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens,
    AttnShape s, float sm_scale, float *__restrict__ out, float *__restrict__ scores, void *ws,
    MfmaTables tab) {
  __shared__ __align__(16) char smem[kPLdsBytes];
  char *lut = smem;
  double *q64 = reinterpret_cast<double *>(smem + kPQOff);
  float *s_ml = reinterpret_cast<float *>(smem + kPMlOff);

  const unsigned nblk = gridDim.x;
  unsigned lb_idx = blockIdx.x;
  if ((nblk & 7u) == 0u) lb_idx = (blockIdx.x & 7u) * (nblk >> 3) + (blockIdx.x >> 3);
  const int split = static_cast<int>(lb_idx % static_cast<unsigned>(s.splits));
  const int bh = static_cast<int>(lb_idx / static_cast<unsigned>(s.splits));
  const int h = bh % s.heads;
  const int b = bh / s.heads;  // query row
  const int req = b / s.tq;     // its request
  const int g = s.group;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index: uniform
  const bool kwave = w < kPairs;
  const int pr = kwave ? w : w - kPairs;  // pair

  LaneConst lc;
  lc.lane = tid & 63;
  lc.n = lc.lane & 15;
  lc.r = lc.lane >> 4;
  lc.lo = lc.n >= 8;
  lc.koff = static_cast<uint32_t>(lc.n * 64 + lc.r * 16);
  lc.voff = static_cast<uint32_t>(lc.n * 16 + lc.r * 4);
  lc.soff = static_cast<uint32_t>(lc.lane * 8);
  lc.keep_mask = lc.lo ? 0xFFFFE000u : 0u;
  constexpr bool kWordTable = kFull || kBits != 4;
  lc.lbk = kWordTable ? static_cast<uint32_t>((lc.lane & 31) * 4) : static_cast<uint32_t>((lc.lane & 15) * 8);
  lc.lbv = lc.lbk | static_cast<uint32_t>(kValueHalf);
  lc.lvl[0] = lc.lo ? 0x02030C0Cu : 0x030C0C0Cu;
  lc.lvl[1] = lc.lo ? 0x00010203u : 0x0102030Cu;
  lc.lvl[2] = lc.lo ? 0x0C0C0001u : 0x0C000102u;
  if constexpr (kBits != 4) cut_lane_offsets<kBits>(lc);
  lc.sm2 = static_cast<double>(sm_scale) * 1.4426950408889634074;

  // ---- this pair's run of chunks ----
  const __attribute__((address_space(4))) int32_t *bt_c =
      (const __attribute__((address_space(4))) int32_t *)block_table;
  const __attribute__((address_space(4))) int32_t *sl_c =
      (const __attribute__((address_space(4))) int32_t *)seq_lens;
  int npages = s.max_pages;
  if (seq_lens) {
    npages = sl_c[req] / kPage;
    npages = npages < 0 ? 0 : (npages > s.max_pages ? s.max_pages : npages);
  }
  const int pps = s.pages_per_split;
  const int p0 = split * pps;
  int p1 = p0 + pps;
  p1 = p1 > npages ? npages : p1;
  auto run_of = [&](int pp, int &rb, int &re) {
    rb = p0 * kChunks + pp * pps;
    re = rb + pps;
    if (re > p1 * kChunks) re = p1 * kChunks;
    if (rb > re) rb = re;
  };
  int cb, ce, cb0, ce0;
  run_of(pr, cb, ce);
  run_of(0, cb0, ce0);
  const int nrun = ce - cb;
  const int nsteps = ce0 - cb0 + 1;  // pair 0 has the longest run; the V waves lag one step

  auto page_of = [&](int ci) -> long long {
    const int lp = ci >> 3;
    const long long pg = block_table ? bt_c[static_cast<size_t>(req) * s.max_pages + lp]
                                     : static_cast<long long>(req) * s.max_pages + lp;
    return (pg < 0 || pg >= s.pool_pages) ? -1 : pg;
  };
  auto page_in_run = [&](int c) -> long long { return c < ce ? page_of(c) : -1; };
  auto tile_of = [&](long long pg) { return pg >= 0 ? static_cast<size_t>(pg) * s.heads + h : 0; };
  auto chunk_of = [&](long long pg, int c) { return pg >= 0 ? (c & 7) : 0; };

  // ---- set-up, run by each role after it has requested its first chunks
  // (their latency overlaps it): the tables (1024 threads, 64 bytes each),
  // and in the K waves the query group in LDS as f64 (zero rows for heads
  // >= g; K wave w writes head w's row from the lanes n = w and n = w + 8),
  // which returns the group's largest |q| ----
  auto setup_tables = [&]() {
    const int trow = (tid >> 1) & 255;
    const bool tval = tid >= 512;
    uint32_t tw0, tw1;  // this thread's table words
    if constexpr (kFull) {
      // row = the 8-bit code, for the planes and every cut
      tw0 = tval ? tab.full[trow] : tab.kfull[trow];
      tw1 = tw0;
    } else if constexpr (kBits != 4) {
      // row f: the draft of anchor field f (sign-extended), the code
      // a * 2^(8-b) + 2^(7-b) - 1
      constexpr int RB = 8 - kBits;
      const int f = trow & ((1 << kBits) - 1);
      const int a = f >= (1 << (kBits - 1)) ? f - (1 << kBits) : f;
      const int code = (a * (1 << RB) + (1 << (RB - 1)) - 1) & 255;
      tw0 = tval ? tab.full[code] : tab.kfull[code];
      tw1 = tw0;
    } else {
      tw0 = tval ? tab.draft[trow & 15] : tab.kdraft[trow & 15];
      tw1 = tval ? tab.draft[trow >> 4] : tab.kdraft[trow >> 4];
    }
    const u32x4 v = kWordTable ? u32x4{tw0, tw0, tw0, tw0} : u32x4{tw0, tw1, tw0, tw1};
    u32x4 *dst = reinterpret_cast<u32x4 *>(lut + trow * 256 + (tval ? kValueHalf : 0) + (tid & 1) * 64);
#pragma unroll
    for (int k = 0; k < 4; ++k) dst[k] = v;
  };
  auto setup_query = [&]() -> float {
    const uint16_t *qg = q + (static_cast<size_t>(b) * s.q_heads + static_cast<size_t>(h) * g) * kDim;
    const int jq = lc.n & 7;
    const bool qvalid = jq < g;
    uint4 qraw[4];
    const uint4 *qrow = reinterpret_cast<const uint4 *>(qg + (qvalid ? jq : 0) * kDim + 32 * lc.r);
#pragma unroll
    for (int k = 0; k < 4; ++k) qraw[k] = qrow[k];
    setup_tables();
    float qv[32];
    float qmax = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t u[4] = {qraw[k].x, qraw[k].y, qraw[k].z, qraw[k].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qv[8 * k + 2 * e] = qvalid ? __uint_as_float(u[e] << 16) : 0.0f;
        qv[8 * k + 2 * e + 1] = qvalid ? __uint_as_float(u[e] & 0xFFFF0000u) : 0.0f;
      }
    }
#pragma unroll
    for (int k = 0; k < 32; ++k) qmax = fmaxf(qmax, fabsf(qv[k]));
    qmax = wave_max(qmax);
    if (jq == w) {
      const bool second = lc.n >= 8;
      const int d0 = 32 * lc.r + (second ? 16 : 0);
#pragma unroll
      for (int k = 0; k < 16; ++k) q64[w * kQStride + d0 + k] = static_cast<double>(second ? qv[16 + k] : qv[k]);
    }
    return qmax;
  };

  const size_t T = static_cast<size_t>(s.max_pages) * kPage;
  float m_run = -INFINITY, l_run = 0.0f;
  floatx4 acc[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) acc[ct] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  char *hand0 = smem + kPHandOff + pr * 2 * kHandBytes;

  if (kwave) {
    char *kslot = smem + kPKSlotOff + pr * kKSlotBytes;
    float *srow_base = nullptr;
    if (scores != nullptr && (lc.n & 7) < g)
      srow_base = scores + (static_cast<size_t>(b) * s.q_heads + static_cast<size_t>(h) * g + (lc.n & 7)) * T;
    // One buffer each: a step turns its chunk's codes into table index
    // bytes before it requests the next chunk's codes into the same
    // registers, and stages the next chunk's constants before it requests
    // the scales of the chunk after that.
    KCodes<kBits> kc;
    KScales ks;
    long long pg_c = page_in_run(cb);      // page of the chunk whose codes kc holds
    long long pg_s = page_in_run(cb + 1);  // page of the chunk whose scales ks holds next
    load_kscales(ks, kp, tile_of(pg_c), chunk_of(pg_c, cb), lc.soff);
    load_kcodes<kFull, kBits>(kc, kp, tile_of(pg_c), chunk_of(pg_c, cb), lc);
    const float qmax = setup_query();
    __syncthreads();  // tables and q
    double inv = stage_kslot(ks, kslot, lc.lane, qmax, q64);
    wave_lds_sync();
    double bias = chunk_bias(kslot, q64, lc);
    load_kscales(ks, kp, tile_of(pg_s), chunk_of(pg_s, cb + 1), lc.soff);
    // the run's steps, then barrier-only steps up to the block's count (two
    // loops, so the code registers need no copies at a join)
    int si = 0;
    for (; si < nrun; ++si) {
      const int c = cb + si;
      const long long cur = pg_c;
      uint32_t e[2][4], o[2][4];
      key_bytes<kFull, kBits>(kc, e, o);
      pg_c = pg_s;
      load_kcodes<kFull, kBits>(kc, kp, tile_of(pg_c), chunk_of(pg_c, c + 1), lc);
      if (cur >= 0)
        score_chunk<kFull, kBits>(e, o, kslot, inv, bias, lc, lut, m_run, l_run,
                           srow_base ? srow_base + static_cast<size_t>(c) * kChunk : nullptr,
                           hand0 + (si & 1) * kHandBytes);
      wave_lds_sync();
      inv = stage_kslot(ks, kslot, lc.lane, qmax, q64);  // constants of chunk c + 1
      wave_lds_sync();
      bias = chunk_bias(kslot, q64, lc);
      pg_s = page_in_run(c + 2);
      load_kscales(ks, kp, tile_of(pg_s), chunk_of(pg_s, c + 2), lc.soff);
      __syncthreads();
    }
    for (; si < nsteps; ++si) __syncthreads();
  } else {
    char *vslot = smem + kPVSlotOff + pr * kVSlotBytes;
    // codes of chunk c in buffer (c - cb) % 2; one scale buffer, refilled
    // after the next chunk's constants are staged
    // the full code of a cut holds up to twice the code words of the
    // planes: one buffer, refilled after its chunk's products
    constexpr int kVBuf = (kFull && kBits != 4) ? 1 : 2;
    VCodes<kBits> vc[kVBuf];
    VScales vs;
    long long pg[2];
    pg[0] = page_in_run(cb);
    pg[1] = page_in_run(cb + 1);
    // the first codes are needed one step later than the scales: requested
    // after the table fill, they leave the K waves' first requests less
    // traffic to queue behind
    load_vscales(vs, vp, tile_of(pg[0]), chunk_of(pg[0], cb), lc.soff);
    setup_tables();
    __syncthreads();  // tables and q
    load_vcodes<kFull, kBits>(vc[0], vp, tile_of(pg[0]), chunk_of(pg[0], cb), lc);
    stage_vslot(vs, vslot, lc.lane);
    load_vscales(vs, vp, tile_of(pg[1]), chunk_of(pg[1], cb + 1), lc.soff);
    __syncthreads();  // step 0: the K waves score the first chunks
    // step si >= 1 takes chunk c = cb + si - 1, whose probabilities the K
    // wave left in buffer (si - 1) & 1
    auto step = [&](auto jc, int si) {
      constexpr int J = decltype(jc)::value;
      const int c = cb + si - 1;
      if (si - 1 < nrun) {
        const long long cur = pg[J];
        pg[J] = page_in_run(c + 2);
        if constexpr (kVBuf == 2) {
          load_vcodes<kFull, kBits>(vc[J ^ 1], vp, tile_of(pg[J ^ 1]), chunk_of(pg[J ^ 1], c + 1), lc);
          if (cur >= 0)
            value_chunk<kFull, kBits>(vc[J], vslot, lc, lut, acc, hand0 + ((si - 1) & 1) * kHandBytes);
        } else {
          if (cur >= 0)
            value_chunk<kFull, kBits>(vc[0], vslot, lc, lut, acc, hand0 + ((si - 1) & 1) * kHandBytes);
          load_vcodes<kFull, kBits>(vc[0], vp, tile_of(pg[J ^ 1]), chunk_of(pg[J ^ 1], c + 1), lc);
        }
        wave_lds_sync();
        stage_vslot(vs, vslot, lc.lane);  // constants of chunk c + 1
        load_vscales(vs, vp, tile_of(pg[J]), chunk_of(pg[J], c + 2), lc.soff);
      }
      __syncthreads();
    };
    for (int si = 1; si < nsteps; si += 2) {
      step(std::integral_constant<int, 0>(), si);
      if (si + 1 >= nsteps) break;
      step(std::integral_constant<int, 1>(), si + 1);
    }
  }

  // ---- merge the 8 pairs of the block ----
  __syncthreads();  // every wave is done with the tables: reuse their space
  float *s_o = reinterpret_cast<float *>(lut);  // [pair][16 col][128 ch, padded to kORow]
  if (kwave) {
    if (lc.r == 0 && lc.n < 8) {
      s_ml[(pr * 2 + 0) * kHeads + lc.n] = m_run;
      s_ml[(pr * 2 + 1) * kHeads + lc.n] = l_run;
    }
  } else {
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
      *reinterpret_cast<float4 *>(s_o + (pr * 16 + lc.n) * kORow + 16 * ct + 4 * lc.r) =
          make_float4(acc[ct][0], acc[ct][1], acc[ct][2], acc[ct][3]);
  }
  __syncthreads();

  if (tid < g * (kDim / 4)) {
    const int j = tid >> 5, c = tid & 31;
    float M = -INFINITY;
#pragma unroll
    for (int pp = 0; pp < kPairs; ++pp) M = fmaxf(M, s_ml[(pp * 2) * kHeads + j]);
    float L = 0.0f;
    float4 O = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int pp = 0; pp < kPairs; ++pp) {
      const float mw = s_ml[(pp * 2) * kHeads + j];
      const float f = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
      L += f * s_ml[(pp * 2 + 1) * kHeads + j];
      const float4 hi = reinterpret_cast<const float4 *>(s_o + (pp * 16 + j) * kORow)[c];
      const float4 lo = reinterpret_cast<const float4 *>(s_o + (pp * 16 + 8 + j) * kORow)[c];
      O.x += f * (hi.x + lo.x);
      O.y += f * (hi.y + lo.y);
      O.z += f * (hi.z + lo.z);
      O.w += f * (hi.w + lo.w);
    }
    if (s.parts == 1) {
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
      reinterpret_cast<float4 *>(
          out + (static_cast<size_t>(b) * s.q_heads + static_cast<size_t>(h) * g + j) * kDim)[c] =
          make_float4(O.x * inv, O.y * inv, O.z * inv, O.w * inv);
    } else {
      Partials pt = partials_of(ws, s);
      const size_t row = (static_cast<size_t>(bh) * s.parts + split) * g + j;
      reinterpret_cast<float4 *>(pt.o + row * kDim)[c] = O;
      if (c == 0) {
        pt.m[row] = static_cast<double>(M);
        pt.l[row] = L;
      }
    }
  }
}

// Merge of the split partials (base-2 maxima) of one (request, KV head)
// into the output.  Block = (request, KV head, 16 channels).  The global
// loads of a thread are issued up front; the per-head maximum and sum over
// the splits are wave reductions (32 lanes per head).
constexpr int kCombThreads = 256;
constexpr int kCombChannels = 16;
constexpr int kCombMaxSplits = 288;  // attention_shape makes at most 256 splits, the tail one more part

// op over the 32 lanes of each half of a wave
template <typename Op>
__device__ __forceinline__ float half_wave_reduce(float v, Op op) {
  v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
  v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
  v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false)));
  v = op(v, ror8(v));
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(a[0]), __uint_as_float(a[1]));
}

__global__ __launch_bounds__(kCombThreads) void attn_mfma_combine_kernel(AttnShape s, const void *ws,
                                                                         float *__restrict__ out) {
  const int per_bh = kDim / kCombChannels;
  const int bh = blockIdx.x / per_bh;
  const int cq = blockIdx.x % per_bh;
  const int b = bh / s.heads, h = bh % s.heads;
  const int g = s.group;
  const int ns = s.parts;
  const int tid = threadIdx.x;
  Partials pt = partials_of(const_cast<void *>(ws), s);
  const size_t first = static_cast<size_t>(bh) * ns * g;  // rows of split 0
  const int units = g * (kCombChannels / 4);               // (head, float4) columns
  const int nsg = kCombThreads / units;                    // split groups
  __shared__ float c_w[kCombMaxSplits * kHeads];           // [split][head] weights
  __shared__ float c_L[kHeads];
  __shared__ float4 c_o[kCombThreads];

  // o rows of this thread's first 8 splits
  const int col = tid % units, sg = tid / units;
  const int j = col / (kCombChannels / 4);
  const int c4 = cq * (kCombChannels / 4) + col % (kCombChannels / 4);
  const bool active = sg < nsg;
  float4 v[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int sp = sg + u * nsg;
    v[u] = active && sp < ns
               ? reinterpret_cast<const float4 *>(pt.o + (first + static_cast<size_t>(sp) * g + j) * kDim)[c4]
               : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
  // per head: 32 lanes over the splits
  {
    const int jh = tid >> 5, i = tid & 31;
    const bool valid = jh < g;
    float mloc[kCombMaxSplits / 32], lloc[kCombMaxSplits / 32];
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kCombMaxSplits / 32; ++k) {
      const int sp = i + 32 * k;
      const bool ok = valid && sp < ns;
      mloc[k] = ok ? static_cast<float>(pt.m[first + static_cast<size_t>(sp) * g + jh]) : -INFINITY;
      lloc[k] = ok ? pt.l[first + static_cast<size_t>(sp) * g + jh] : 0.0f;
      M = fmaxf(M, mloc[k]);
    }
    M = half_wave_reduce(M, MaxOp());
    float L = 0.0f;
#pragma unroll
    for (int k = 0; k < kCombMaxSplits / 32; ++k) {
      const int sp = i + 32 * k;
      const float wgt = mloc[k] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mloc[k] - M);
      L += wgt * lloc[k];
      if (valid && sp < ns) c_w[sp * kHeads + jh] = wgt;
    }
    L = half_wave_reduce(L, SumOp());
    if (valid && i == 0) c_L[jh] = L;
  }
  __syncthreads();
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (active) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sp = sg + u * nsg;
      const float wgt = sp < ns ? c_w[sp * kHeads + j] : 0.0f;
      acc.x += wgt * v[u].x;
      acc.y += wgt * v[u].y;
      acc.z += wgt * v[u].z;
      acc.w += wgt * v[u].w;
    }
    for (int sp = sg + 8 * nsg; sp < ns; sp += nsg) {
      const float4 x = reinterpret_cast<const float4 *>(
          pt.o + (first + static_cast<size_t>(sp) * g + j) * kDim)[c4];
      const float wgt = c_w[sp * kHeads + j];
      acc.x += wgt * x.x;
      acc.y += wgt * x.y;
      acc.z += wgt * x.z;
      acc.w += wgt * x.w;
    }
  }
  c_o[tid] = acc;
  __syncthreads();
  if (tid < units) {
    float4 o = c_o[tid];
    for (int k = 1; k < nsg; ++k) {
      const float4 x = c_o[k * units + tid];
      o.x += x.x;
      o.y += x.y;
      o.z += x.z;
      o.w += x.w;
    }
    const float Lj = c_L[j];
    const float inv = Lj > 0.0f ? 1.0f / Lj : 0.0f;
    reinterpret_cast<float4 *>(
        out + (static_cast<size_t>(b) * s.q_heads + static_cast<size_t>(h) * g + j) * kDim)[c4] =
        make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
  }
}

// The same merge with one block per (query row, KV head), for launches with
// many of them (the verify pass's rows): the block computes the part
// weights once for all 128 channels and reads every partial row whole;
// thread t takes head j = t / 32 and channels 4(t % 32) .. + 3.  The o rows
// of the first kRowCombPre parts are requested before the weights.
constexpr int kRowCombPre = 16;
constexpr int kRowCombMinPairs = 128;  // (row, KV head) pairs from which this kernel runs

__global__ __launch_bounds__(kCombThreads) void attn_mfma_combine_rows_kernel(AttnShape s, const void *ws,
                                                                              float *__restrict__ out) {
  const int bh = blockIdx.x;
  const int b = bh / s.heads, h = bh % s.heads;
  const int g = s.group;
  const int ns = s.parts;
  const int tid = threadIdx.x, j = tid >> 5, i = tid & 31;
  const bool valid = j < g;
  Partials pt = partials_of(const_cast<void *>(ws), s);
  const size_t first = static_cast<size_t>(bh) * ns * g;  // rows of part 0
  __shared__ float c_w[kCombMaxSplits * kHeads];           // [part][head] weights
  auto orow = [&](int sp) {
    return reinterpret_cast<const float4 *>(pt.o + (first + static_cast<size_t>(sp) * g + j) * kDim) + i;
  };
  float4 v[kRowCombPre];
#pragma unroll
  for (int u = 0; u < kRowCombPre; ++u)
    v[u] = valid && u < ns ? *orow(u) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  // part weights of head j: its 32 lanes over the parts
  float L;
  {
    float mloc[kCombMaxSplits / 32], lloc[kCombMaxSplits / 32];
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kCombMaxSplits / 32; ++k) {
      const int sp = i + 32 * k;
      const bool ok = valid && sp < ns;
      mloc[k] = ok ? static_cast<float>(pt.m[first + static_cast<size_t>(sp) * g + j]) : -INFINITY;
      lloc[k] = ok ? pt.l[first + static_cast<size_t>(sp) * g + j] : 0.0f;
      M = fmaxf(M, mloc[k]);
    }
    M = half_wave_reduce(M, MaxOp());
    L = 0.0f;
#pragma unroll
    for (int k = 0; k < kCombMaxSplits / 32; ++k) {
      const int sp = i + 32 * k;
      const float wgt = mloc[k] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mloc[k] - M);
      L += wgt * lloc[k];
      if (valid && sp < ns) c_w[sp * kHeads + j] = wgt;
    }
    L = half_wave_reduce(L, SumOp());
  }
  __syncthreads();
  if (!valid) return;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  auto add = [&](float wgt, const float4 &x) {
    acc.x += wgt * x.x;
    acc.y += wgt * x.y;
    acc.z += wgt * x.z;
    acc.w += wgt * x.w;
  };
#pragma unroll
  for (int u = 0; u < kRowCombPre; ++u)
    if (u < ns) add(c_w[u * kHeads + j], v[u]);
  int sp = kRowCombPre;
  for (; sp + 4 <= ns; sp += 4) {
    float4 x[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = *orow(sp + k);
#pragma unroll
    for (int k = 0; k < 4; ++k) add(c_w[(sp + k) * kHeads + j], x[k]);
  }
  for (; sp < ns; ++sp) add(c_w[sp * kHeads + j], *orow(sp));
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  reinterpret_cast<float4 *>(out + (static_cast<size_t>(b) * s.q_heads + static_cast<size_t>(h) * g + j) *
                                       kDim)[i] = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

// Output of requests whose every page is skipped (an empty pool): zeros.
__global__ __launch_bounds__(256) void attn_zero_kernel(float *__restrict__ out, size_t n) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) out[i] = 0.0f;
}

MfmaTables build_mfma_tables() {
  MfmaTables t;
  const DecodeTable &dt = decode_table();
  const DraftTable &df = draft_table();
  auto pair = [](float y) {
    const _Float16 hi = static_cast<_Float16>(y);
    const _Float16 lo = static_cast<_Float16>(y - static_cast<float>(hi));
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) << 16);
  };
  for (int byte = 0; byte < 256; ++byte) {
    // the byte is the code read as int8: (a << 4 | r)
    const int code = byte >= 128 ? byte - 256 : byte;
    t.full[byte] = pair(dt.y[code + 128]);
  }
  for (int nib = 0; nib < 16; ++nib) t.draft[nib] = pair(df.y[nib]);
  // fixed-point yhat as 4 signed bytes: Y + 0x80808080 puts a +128 bias on
  // every byte, and flipping each byte's top bit removes it again, so byte j
  // holds Y_j in -128 .. 127 with sum_j Y_j 2^(8j) = Y (|Y| <= 2^30)
  const FixedDecodeTable &fx = fixed_decode_table();
  auto bytes = [](int32_t y) { return (static_cast<uint32_t>(y) + 0x80808080u) ^ 0x80808080u; };
  for (int byte = 0; byte < 256; ++byte) {
    const int code = byte >= 128 ? byte - 256 : byte;
    t.kfull[byte] = bytes(fx.y[code + 128]);
  }
  for (int nib = 0; nib < 16; ++nib) t.kdraft[nib] = bytes(fx.draft[nib]);
  return t;
}

template <bool kFull, int kBits>
void launch_mfma_kernel(dim3 grid, hipStream_t stream, const uint16_t *q, const PlanesArg &k,
                        const PlanesArg &v, const int32_t *block_table, const int32_t *seq_lens,
                        const AttnShape &s, float sm_scale, float *out, float *scores,
                        void *workspace, const MfmaTables &tables) {
  hipLaunchKernelGGL((attn_pair_kernel<kFull, kBits>), grid, dim3(kPThreads), 0, stream, q, k, v,
                     block_table, seq_lens, s, sm_scale, out, scores, workspace, tables);
}

template <int kBits>
void launch_mfma_bits(bool full, dim3 grid, hipStream_t stream, const uint16_t *q,
                      const PlanesArg &k, const PlanesArg &v, const int32_t *block_table,
                      const int32_t *seq_lens, const AttnShape &s, float sm_scale, float *out,
                      float *scores, void *workspace, const MfmaTables &tables) {
  if (full)
    launch_mfma_kernel<true, kBits>(grid, stream, q, k, v, block_table, seq_lens, s, sm_scale, out,
                                    scores, workspace, tables);
  else
    launch_mfma_kernel<false, kBits>(grid, stream, q, k, v, block_table, seq_lens, s, sm_scale,
                                     out, scores, workspace, tables);
}

}  // namespace

bool attention_mfma_supported(int group) { return group >= 1 && group <= kHeads; }

int attention_mfma_target_blocks() { return 256; }

hipError_t launch_attention_mfma(const uint16_t *q, const PlanesArg &k, const PlanesArg &v,
                                 const int32_t *block_table, const int32_t *seq_lens,
                                 const AttnShape &s, float sm_scale, bool full, float *out,
                                 float *scores, void *workspace, bool merge, hipStream_t stream,
                                 int anchor_bits) {
  static const MfmaTables tables = build_mfma_tables();
  if (s.parts > kCombMaxSplits || anchor_bits < 1 || anchor_bits > 7) return hipErrorInvalidValue;
  if (s.pool_pages <= 0) {
    // no page can be read: every request's context is empty
    const size_t n = static_cast<size_t>(s.batch) * s.q_heads * kDim;
    hipLaunchKernelGGL(attn_zero_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                       stream, out, n);
    return hipGetLastError();
  }
  const dim3 grid(static_cast<unsigned>(static_cast<long long>(s.batch) * s.heads * s.splits));
  auto go = [&](auto bits) {
    launch_mfma_bits<decltype(bits)::value>(full, grid, stream, q, k, v, block_table, seq_lens, s,
                                            sm_scale, out, scores, workspace, tables);
  };
  switch (anchor_bits) {
    case 1: go(std::integral_constant<int, 1>()); break;
    case 2: go(std::integral_constant<int, 2>()); break;
    case 3: go(std::integral_constant<int, 3>()); break;
    case 5: go(std::integral_constant<int, 5>()); break;
    case 6: go(std::integral_constant<int, 6>()); break;
    case 7: go(std::integral_constant<int, 7>()); break;
    default: go(std::integral_constant<int, 4>()); break;
  }
  if (s.parts == 1 || !merge) return hipGetLastError();  // output or partials written
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attention_mfma_combine(s, workspace, out, stream);
}

hipError_t launch_attention_mfma_combine(const AttnShape &s, const void *workspace, float *out,
                                         hipStream_t stream) {
  if (s.parts > kCombMaxSplits) return hipErrorInvalidValue;
  const long long pairs = static_cast<long long>(s.batch) * s.heads;
  if (pairs >= kRowCombMinPairs) {
    hipLaunchKernelGGL(attn_mfma_combine_rows_kernel, dim3(static_cast<unsigned>(pairs)),
                       dim3(kCombThreads), 0, stream, s, workspace, out);
    return hipGetLastError();
  }
  const dim3 cgrid(static_cast<unsigned>(pairs * (kDim / kCombChannels)));
  hipLaunchKernelGGL(attn_mfma_combine_kernel, cgrid, dim3(kCombThreads), 0, stream, s, workspace,
                     out);
  return hipGetLastError();
}

}  // namespace lynx
