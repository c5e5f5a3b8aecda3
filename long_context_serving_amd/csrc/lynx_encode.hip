// Lynx page encoder and nibble-plane packer for gfx950.
//
// Page "Lynx: the KV cache does not have to arrive whole", section 3 "The
// quantizer": per page of 256 tokens and per channel, page min/range
// normalisation; per chunk of C = 32 tokens, centring by the chunk mean and
// scaling by the chunk's largest deviation; a sign-aware alpha-law map onto
// 127 magnitude levels; and the cut of each 8-bit code into an anchor
// (high nibble) and a residual (low nibble) plane.
//
// One workgroup encodes one (page, KV head) tile of 256 tokens x 128
// channels with 8 waves, one wave per 32-token chunk, so every chunk
// statistic is a reduction inside one wave.  Lane (cg, r) of a wave owns
// channels 8cg..8cg+7 of the 8 tokens {4r..4r+3, 16+4r..16+4r+3} of the
// chunk: bf16 rows are read as 16-byte pieces (4 token rows of 256 B per
// wave load), and the same register tile yields both plane layouts with
// 32-bit stores -- a token's 8 channel nibbles (keys) or a channel's 8 token
// nibbles (values).  Page min/max crosses the 8 waves once through LDS.
//
// Numeric contract (shared with the C ABI header): the statistics are fp32
// IEEE operations without contraction (this file is built with
// -ffp-contract=off), reciprocals are correctly rounded, the chunk sum is
// exact in fp64 (whenever every nonzero normalised value of the chunk is at
// least 2^-24, see the header), the page range and chunk max-abs are the
// plain fp32 values, and the level m is exactly #{k >= 1 : u >= T[k]}.
#include "lynx_cut.h"
#include "lynx_internal.h"

namespace lynx {
namespace {

constexpr int kEncThreads = 512;

// Kernel-argument copy of the host tables: thresholds T[0..127] and the level
// at the start of each u bucket (see BucketTable).
struct EncodeTables {
  float t[128];
  uint8_t base[(kBuckets + 3) & ~3];
};

__device__ __forceinline__ int chunk_token(int r, int j) {
  return j < 4 ? 4 * r + j : 16 + 4 * r + (j - 4);
}

// Exact level: number of thresholds T[1..127] not above u (T increasing).
__device__ __forceinline__ int level_exact(float u, const float *T) {
  int m = 0;
#pragma unroll
  for (int step = 64; step >= 1; step >>= 1) {
    const int k = m + step;
    if (k <= 127 && u >= T[k]) m = k;
  }
  return m;
}

// LDS bucket entry: (bits of the first threshold above the bucket start,
// level at the bucket start); every bucket holds at most one threshold, so
// for u in the bucket the level is base + (bits(u) >= next threshold):
// positive floats order like their bit patterns.
__device__ __forceinline__ void fill_level_table(uint2 *lvl, const EncodeTables &tab) {
  for (int i = threadIdx.x; i < kBuckets; i += blockDim.x) {
    const int m = tab.base[i];
    lvl[i] = make_uint2(m < 127 ? __float_as_uint(tab.t[m + 1]) : 0xFFFFFFFFu,
                        static_cast<uint32_t>(m));
  }
}

// Streaming accesses: the input is read once and the outputs are not read
// back by this kernel, so both bypass cache retention (non-temporal).  The
// non-temporal stores are whole 16-byte units, contiguous across a wave:
// narrower ones could not be merged into full lines.
__device__ __forceinline__ uint4 load_stream(const char *p) {
  const uint32_t *q = reinterpret_cast<const uint32_t *>(p);
  return make_uint4(__builtin_nontemporal_load(q), __builtin_nontemporal_load(q + 1),
                    __builtin_nontemporal_load(q + 2), __builtin_nontemporal_load(q + 3));
}
__device__ __forceinline__ void store_stream(char *p, uint4 v) {
  uint32_t *q = reinterpret_cast<uint32_t *>(p);
  __builtin_nontemporal_store(v.x, q);
  __builtin_nontemporal_store(v.y, q + 1);
  __builtin_nontemporal_store(v.z, q + 2);
  __builtin_nontemporal_store(v.w, q + 3);
}
__device__ __forceinline__ void store_stream(float *p, float4 v) {
  __builtin_nontemporal_store(v.x, p);
  __builtin_nontemporal_store(v.y, p + 1);
  __builtin_nontemporal_store(v.z, p + 2);
  __builtin_nontemporal_store(v.w, p + 3);
}

// Reductions over the 4 lanes of a quad (lanes 4j .. 4j+3 share their
// channels): two DPP quad permutations, which fold into the reducing op.  A
// quad permutation reads a lane of the same quad for every lane, so the
// destination needs no previous value.
template <int kCtrl>
__device__ __forceinline__ float quad_perm(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kCtrl,
                                                            0xF, 0xF, true));
}
template <int kCtrl>
__device__ __forceinline__ double quad_perm(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(u), kCtrl, 0xF, 0xF, true));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(u >> 32), kCtrl, 0xF, 0xF, true));
  return __builtin_bit_cast(double, static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32));
}
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2, 3, 0, 1]
template <typename Op>
__device__ __forceinline__ float xreduce_f32(float v, Op op) {
  v = op(v, quad_perm<kQuadXor1>(v));
  return op(v, quad_perm<kQuadXor2>(v));
}
__device__ __forceinline__ double xsum_f64(double v) {
  v = v + quad_perm<kQuadXor1>(v);
  return v + quad_perm<kQuadXor2>(v);
}
struct MinOp { __device__ float operator()(float a, float b) const { return fminf(a, b); } };
struct MaxOp { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };

// low bytes of a, b, c, d -> bytes 0..3 of one word
__device__ __forceinline__ uint32_t pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);
  const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0c0c0400u);
  return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

// The cut of 8 codes (element k in nibble k): anchor = code >> 4 and
// residual = code & 15 per element.  we / wo hold the even / odd elements'
// code bytes.
__device__ __forceinline__ uint32_t anchor_word(uint32_t we, uint32_t wo) {
  return ((we >> 4) & 0x0F0F0F0Fu) | (wo & 0xF0F0F0F0u);
}
__device__ __forceinline__ uint32_t residual_word(uint32_t we, uint32_t wo) {
  return (we & 0x0F0F0F0Fu) | ((wo << 4) & 0xF0F0F0F0u);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Level of u >= 0 from its bits: the key bits(u) >> 18 is clamped into the
// bucket range (u below 2^-14 -> bucket 0, u >= 1 -> bucket 449, which also
// keeps any u from non-finite input inside the table), then one table read
// and one comparison.
__device__ __forceinline__ uint32_t level_of(float u, const uint2 *lvl) {
  const uint32_t ubits = __float_as_uint(u);
  uint32_t key = ubits >> kBucketShift;
  key = key < kBucketFirstKey - 1u ? kBucketFirstKey - 1u : key;
  key = key > kBucketLastKey ? kBucketLastKey : key;
  const uint2 e = lvl[key - (kBucketFirstKey - 1u)];
  return e.y + (ubits >= e.x ? 1u : 0u);
}

// sign masks: byte k = 0xFF where element k is negative (v_perm selectors
// 9 and 11 replicate bit 31 of the low and the high source)
__device__ __forceinline__ uint32_t signs4(float a, float b, float c, float d) {
  const uint32_t ab = __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x0c0c0b09u);
  const uint32_t cd = __builtin_amdgcn_perm(__float_as_uint(d), __float_as_uint(c), 0x0b090c0cu);
  return ab | cd;
}

// Sign-aware code bytes of 4 centred values: m for d >= 0, ~m for d < 0 (d
// is never -0: x' - mu rounds an exact zero to +0).
__device__ __forceinline__ uint32_t codes4(float d0, float d1, float d2, float d3,
                                           float i0, float i1, float i2, float i3,
                                           const uint2 *lvl) {
  const uint32_t m = pack4(level_of(fabsf(d0) * i0, lvl), level_of(fabsf(d1) * i1, lvl),
                           level_of(fabsf(d2) * i2, lvl), level_of(fabsf(d3) * i3, lvl));
  return m ^ signs4(d0, d1, d2, d3);
}

// One workgroup of 8 waves per (page, head) tile; wave c owns chunk c; lane
// (cg, r) holds channels 8cg..8cg+7 of the 8 tokens chunk_token(r, 0..7).
// Two workgroups fit on a CU (at most 128 VGPRs), so that one streams its
// tile in while the other computes.  Addresses are a wave-uniform base plus
// 32-bit lane offsets.  kBits = 4 writes the 4-bit planes; other values
// write the b + (8 - b) streams of the same codes (out.anchor: b bits per
// element, out.residual: 8 - b), re-cut from the staged planes.
// Workgroup storage of one tile.  The planes are staged in LDS and written
// out as contiguous 16-byte units.  K rows of 16 words are padded to 20 and
// V's 16-byte units are XOR-swizzled (unit ^ (unit >> 3 & 7)), which spreads
// a wave's word writes over the banks and keeps every 16-byte unit
// contiguous.
struct EncodeSmem {
  uint2 lvl[kBuckets];
  float min[kChunks][kDim];
  float max[kChunks][kDim];
  float mn[kDim];
  float inv[kDim];
  __align__(16) uint32_t pl[2][kPage * 20];
};

template <int kRole, int kBits>
__device__ __forceinline__ void encode_tile(EncodeSmem &sm, const uint16_t *__restrict__ kv,
                                            int heads, int tile, const PlanesArg &out,
                                            const EncodeTables &tab) {
  const int c = threadIdx.x >> 6;  // chunk = wave
  const int lane = threadIdx.x & 63;
  const int cg = lane >> 2;  // channel group: channels 8cg .. 8cg+7
  const int r = lane & 3;    // token group (the 4 lanes of a quad share channels)
  uint2 *const s_lvl = sm.lvl;
  float (*const s_min)[kDim] = sm.min;
  float (*const s_max)[kDim] = sm.max;
  float *const s_mn = sm.mn;
  float *const s_inv = sm.inv;
  uint32_t (*const s_pl)[kPage * 20] = sm.pl;

  // tile = page * heads + head
  fill_level_table(s_lvl, tab);  // published by the first __syncthreads below

  // ---- load the lane's 8 tokens x 8 channels (bf16 -> fp32 is exact) ----
  float x[8][8];
  {
    const int p = tile / heads;
    const int h = tile - p * heads;
    const uint32_t row_bytes = static_cast<uint32_t>(heads) * kDim * 2;
    const char *page = reinterpret_cast<const char *>(kv) +
                       static_cast<size_t>(p) * kPage * row_bytes + static_cast<size_t>(h) * kDim * 2;
    const uint32_t lane_off = static_cast<uint32_t>(c * kChunk) * row_bytes + cg * 16;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t off = lane_off + static_cast<uint32_t>(chunk_token(r, j)) * row_bytes;
      const uint4 v = load_stream(page + off);
      x[j][0] = bf16_lo(v.x); x[j][1] = bf16_hi(v.x);
      x[j][2] = bf16_lo(v.y); x[j][3] = bf16_hi(v.y);
      x[j][4] = bf16_lo(v.z); x[j][5] = bf16_hi(v.z);
      x[j][6] = bf16_lo(v.w); x[j][7] = bf16_hi(v.w);
    }
  }
  {
    // ---- page-level normalisation: per-channel min and max ----
    {
      float mn[8], mx[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        mn[i] = fminf(fminf(fminf(x[0][i], x[1][i]), fminf(x[2][i], x[3][i])),
                      fminf(fminf(x[4][i], x[5][i]), fminf(x[6][i], x[7][i])));
        mx[i] = fmaxf(fmaxf(fmaxf(x[0][i], x[1][i]), fmaxf(x[2][i], x[3][i])),
                      fmaxf(fmaxf(x[4][i], x[5][i]), fmaxf(x[6][i], x[7][i])));
        mn[i] = xreduce_f32(mn[i], MinOp());
        mx[i] = xreduce_f32(mx[i], MaxOp());
      }
      if (r == 0) {
        reinterpret_cast<float4 *>(&s_min[c][cg * 8])[0] = make_float4(mn[0], mn[1], mn[2], mn[3]);
        reinterpret_cast<float4 *>(&s_min[c][cg * 8])[1] = make_float4(mn[4], mn[5], mn[6], mn[7]);
        reinterpret_cast<float4 *>(&s_max[c][cg * 8])[0] = make_float4(mx[0], mx[1], mx[2], mx[3]);
        reinterpret_cast<float4 *>(&s_max[c][cg * 8])[1] = make_float4(mx[4], mx[5], mx[6], mx[7]);
      }
    }
    __syncthreads();
    if (threadIdx.x < kDim) {
      const int d = threadIdx.x;
      float a = s_min[0][d], b = s_max[0][d];
#pragma unroll
      for (int cc = 1; cc < kChunks; ++cc) {
        a = fminf(a, s_min[cc][d]);
        b = fmaxf(b, s_max[cc][d]);
      }
      const float rg = b - a;  // fp32
      // correctly rounded fp32 reciprocal (fp64 quotient, one rounding)
      const float inv = rg > 0.0f ? static_cast<float>(1.0 / static_cast<double>(rg)) : 0.0f;
      s_mn[d] = a;
      s_inv[d] = inv;
      __builtin_nontemporal_store(a, out.page_min + static_cast<size_t>(tile) * kDim + d);
      __builtin_nontemporal_store(rg, out.page_range + static_cast<size_t>(tile) * kDim + d);
    }
    __syncthreads();

    // ---- x' = (x - mn) * inv_rg, and the exact chunk sum in fp64 ----
    float mu[8];
    {
      const float4 mn0 = reinterpret_cast<const float4 *>(&s_mn[cg * 8])[0];
      const float4 mn1 = reinterpret_cast<const float4 *>(&s_mn[cg * 8])[1];
      const float4 iv0 = reinterpret_cast<const float4 *>(&s_inv[cg * 8])[0];
      const float4 iv1 = reinterpret_cast<const float4 *>(&s_inv[cg * 8])[1];
      const float mn[8] = {mn0.x, mn0.y, mn0.z, mn0.w, mn1.x, mn1.y, mn1.z, mn1.w};
      const float inv_rg[8] = {iv0.x, iv0.y, iv0.z, iv0.w, iv1.x, iv1.y, iv1.z, iv1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x[0][i] = (x[0][i] - mn[i]) * inv_rg[i];
        double sum = static_cast<double>(x[0][i]);  // (x' >= 0: no signed zero to keep)
#pragma unroll
        for (int j = 1; j < 8; ++j) {
          x[j][i] = (x[j][i] - mn[i]) * inv_rg[i];
          sum += static_cast<double>(x[j][i]);
        }
        sum = xsum_f64(sum);
        mu[i] = static_cast<float>(sum * (1.0 / kChunk));
      }
    }

    // ---- chunk centring and max-abs ----
    float sabs[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j][i] = x[j][i] - mu[i];
      sabs[i] = fmaxf(fmaxf(fmaxf(fabsf(x[0][i]), fabsf(x[1][i])),
                            fmaxf(fabsf(x[2][i]), fabsf(x[3][i]))),
                      fmaxf(fmaxf(fabsf(x[4][i]), fabsf(x[5][i])),
                            fmaxf(fabsf(x[6][i]), fabsf(x[7][i]))));
      sabs[i] = xreduce_f32(sabs[i], MaxOp());
    }
    if (r == 0) {
      const size_t cidx = (static_cast<size_t>(tile) * kChunks + c) * kDim + cg * 8;
      store_stream(out.chunk_mean + cidx, make_float4(mu[0], mu[1], mu[2], mu[3]));
      store_stream(out.chunk_mean + cidx + 4, make_float4(mu[4], mu[5], mu[6], mu[7]));
      store_stream(out.chunk_maxabs + cidx, make_float4(sabs[0], sabs[1], sabs[2], sabs[3]));
      store_stream(out.chunk_maxabs + cidx + 4, make_float4(sabs[4], sabs[5], sabs[6], sabs[7]));
    }
    // correctly rounded reciprocals: each of the 4 lanes sharing these
    // channels computes 2 of the 8, the rest are gathered from the other lanes
    float inv_s[8];
    {
      float my_inv[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float s = r == 0 ? sabs[k] : r == 1 ? sabs[2 + k] : r == 2 ? sabs[4 + k] : sabs[6 + k];
        my_inv[k] = s > 0.0f ? static_cast<float>(1.0 / static_cast<double>(s)) : 0.0f;
      }
      // channel i's reciprocal is in lane r = i / 2 of the quad (DPP quad broadcast)
      inv_s[0] = quad_perm<0x00>(my_inv[0]);
      inv_s[1] = quad_perm<0x00>(my_inv[1]);
      inv_s[2] = quad_perm<0x55>(my_inv[0]);
      inv_s[3] = quad_perm<0x55>(my_inv[1]);
      inv_s[4] = quad_perm<0xAA>(my_inv[0]);
      inv_s[5] = quad_perm<0xAA>(my_inv[1]);
      inv_s[6] = quad_perm<0xFF>(my_inv[0]);
      inv_s[7] = quad_perm<0xFF>(my_inv[1]);
    }

    // ---- sign-aware alpha-law codes and the cut into nibble planes ----
    if (kRole == LYNX_ROLE_KEY) {
      // token-major [256 tokens][64 B]: one word = 8 channels of one token
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t we = codes4(x[j][0], x[j][2], x[j][4], x[j][6],
                                   inv_s[0], inv_s[2], inv_s[4], inv_s[6], s_lvl);
        const uint32_t wo = codes4(x[j][1], x[j][3], x[j][5], x[j][7],
                                   inv_s[1], inv_s[3], inv_s[5], inv_s[7], s_lvl);
        const int widx = (c * kChunk + chunk_token(r, j)) * 20 + cg;
        s_pl[0][widx] = anchor_word(we, wo);
        s_pl[1][widx] = residual_word(we, wo);
      }
    } else {
      // channel-major [8 chunks][128 channels][16 B]: one word = the lane's
      // 8 tokens of one channel
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float is = inv_s[i];
        const uint32_t we = codes4(x[0][i], x[2][i], x[4][i], x[6][i], is, is, is, is, s_lvl);
        const uint32_t wo = codes4(x[1][i], x[3][i], x[5][i], x[7][i], is, is, is, is, s_lvl);
        const int unit = c * kDim + cg * 8 + i;
        const int widx = (unit ^ ((unit >> 3) & 7)) * 4 + r;
        s_pl[0][widx] = anchor_word(we, wo);
        s_pl[1][widx] = residual_word(we, wo);
      }
    }
    __syncthreads();
    // write-out: 1024 units of 16 B per plane, two per thread, contiguous
    // (or, for a cut, b and 8 - b words per unit)
    constexpr int kUnits = kPlaneTileBytes / 16;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int unit = k * kEncThreads + threadIdx.x;
      const int widx = kRole == LYNX_ROLE_KEY ? (unit >> 2) * 20 + (unit & 3) * 4
                                              : (unit ^ ((unit >> 3) & 7)) * 4;
      const uint4 a = *reinterpret_cast<const uint4 *>(&s_pl[0][widx]);
      const uint4 rr = *reinterpret_cast<const uint4 *>(&s_pl[1][widx]);
      if constexpr (kBits == 4) {
        char *an = reinterpret_cast<char *>(out.anchor) + static_cast<size_t>(tile) * kPlaneTileBytes;
        char *re = reinterpret_cast<char *>(out.residual) + static_cast<size_t>(tile) * kPlaneTileBytes;
        store_stream(an + unit * 16, a);
        store_stream(re + unit * 16, rr);
      } else {
        constexpr int RB = 8 - kBits;
        const uint32_t a4[4] = {a.x, a.y, a.z, a.w};
        const uint32_t r4[4] = {rr.x, rr.y, rr.z, rr.w};
        uint32_t wa[kBits], wr[RB];
        cut::unit<kBits>(a4, r4, wa, wr);
        uint32_t *an = reinterpret_cast<uint32_t *>(out.anchor) +
                       (static_cast<size_t>(tile) * kUnits + unit) * kBits;
        uint32_t *re = reinterpret_cast<uint32_t *>(out.residual) +
                       (static_cast<size_t>(tile) * kUnits + unit) * RB;
#pragma unroll
        for (int i = 0; i < kBits; ++i) __builtin_nontemporal_store(wa[i], an + i);
#pragma unroll
        for (int i = 0; i < RB; ++i) __builtin_nontemporal_store(wr[i], re + i);
      }
    }
  }
}

template <int kRole, int kBits>
__global__ __launch_bounds__(kEncThreads) __attribute__((amdgpu_waves_per_eu(4)))
void encode_kernel(const uint16_t *__restrict__ kv, int heads, PlanesArg out, EncodeTables tab) {
  __shared__ EncodeSmem sm;
  encode_tile<kRole, kBits>(sm, kv, heads, static_cast<int>(blockIdx.x), out, tab);
}

// K and V of one layer in one launch: block 2t encodes K tile t and block
// 2t + 1 V tile t, so that no launch boundary separates the two tensors and
// blocks of the two roles (whose compute and store patterns differ) share
// the chip throughout.
__global__ __launch_bounds__(kEncThreads) __attribute__((amdgpu_waves_per_eu(4)))
void encode_kv_kernel(const uint16_t *__restrict__ k, const uint16_t *__restrict__ v, int heads,
                      int ntiles, PlanesArg kout, PlanesArg vout, EncodeTables tab) {
  __shared__ EncodeSmem sm;
  const int t = static_cast<int>(blockIdx.x);
  if ((t & 1) == 0)
    encode_tile<LYNX_ROLE_KEY, 4>(sm, k, heads, t >> 1, kout, tab);
  else
    encode_tile<LYNX_ROLE_VALUE, 4>(sm, v, heads, t >> 1, vout, tab);
}

// Exhaustive check of the encoder's level path (the bucket table) against
// the exact threshold count over fp32 bit patterns [begin, end) (values in
// [0, 2); above 1 the expected level is that of the clamped u, 127).
__global__ __launch_bounds__(256) void code_map_check_kernel(uint32_t begin, uint32_t end,
                                                             unsigned long long *mismatches,
                                                             EncodeTables tab) {
  __shared__ float s_T[128];
  __shared__ uint2 s_lvl[kBuckets];
  if (threadIdx.x < 128) s_T[threadIdx.x] = tab.t[threadIdx.x];
  fill_level_table(s_lvl, tab);
  __syncthreads();
  unsigned long long bad = 0;
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t b = begin + blockIdx.x * blockDim.x + threadIdx.x; b < end && b >= begin;
       b += stride) {
    const float u = __uint_as_float(b);
    bad += static_cast<int>(level_of(u, s_lvl)) != level_exact(fminf(u, 1.0f), s_T);
  }
  if (bad) atomicAdd(mismatches, bad);
}

EncodeTables encode_tables() {
  EncodeTables tab = {};
  const CodeTable &ct = code_table();
  const BucketTable &bt = bucket_table();
  for (int k = 0; k < 128; ++k) tab.t[k] = ct.t[k];
  for (int i = 0; i < kBuckets; ++i) tab.base[i] = bt.base[i];
  return tab;
}

}  // namespace

hipError_t launch_code_map_check(uint32_t begin, uint32_t end, unsigned long long *mismatches,
                                 hipStream_t stream) {
  if (end <= begin) return hipSuccess;
  EncodeTables tab = encode_tables();
  hipLaunchKernelGGL(code_map_check_kernel, dim3(4096), dim3(256), 0, stream, begin, end,
                     mismatches, tab);
  return hipGetLastError();
}

namespace {
template <int kBits>
void launch_encode_bits(const uint16_t *kv, unsigned blocks, int heads, int role,
                        const PlanesArg &out, const EncodeTables &tab, hipStream_t stream) {
  if (role == LYNX_ROLE_KEY)
    hipLaunchKernelGGL((encode_kernel<LYNX_ROLE_KEY, kBits>), dim3(blocks), dim3(kEncThreads), 0,
                       stream, kv, heads, out, tab);
  else
    hipLaunchKernelGGL((encode_kernel<LYNX_ROLE_VALUE, kBits>), dim3(blocks), dim3(kEncThreads), 0,
                       stream, kv, heads, out, tab);
}
}  // namespace

hipError_t launch_encode_kv(const uint16_t *k, const uint16_t *v, int64_t num_pages, int heads,
                            const PlanesArg &kout, const PlanesArg &vout, hipStream_t stream) {
  if (num_pages == 0) return hipSuccess;
  if (!bucket_table().ok || 2 * num_pages * heads > INT32_MAX) return hipErrorInvalidValue;
  EncodeTables tab = encode_tables();
  const int ntiles = static_cast<int>(num_pages * heads);
  hipLaunchKernelGGL(encode_kv_kernel, dim3(static_cast<unsigned>(2 * ntiles)), dim3(kEncThreads), 0,
                     stream, k, v, heads, ntiles, kout, vout, tab);
  return hipGetLastError();
}

hipError_t launch_encode(const uint16_t *kv, int64_t num_pages, int heads,
                         int role, const PlanesArg &out, hipStream_t stream, int anchor_bits) {
  if (num_pages == 0) return hipSuccess;
  if (!bucket_table().ok || anchor_bits < 1 || anchor_bits > 7) return hipErrorInvalidValue;
  EncodeTables tab = encode_tables();
  const unsigned blocks = static_cast<unsigned>(num_pages * heads);
  switch (anchor_bits) {
    case 1: launch_encode_bits<1>(kv, blocks, heads, role, out, tab, stream); break;
    case 2: launch_encode_bits<2>(kv, blocks, heads, role, out, tab, stream); break;
    case 3: launch_encode_bits<3>(kv, blocks, heads, role, out, tab, stream); break;
    case 5: launch_encode_bits<5>(kv, blocks, heads, role, out, tab, stream); break;
    case 6: launch_encode_bits<6>(kv, blocks, heads, role, out, tab, stream); break;
    case 7: launch_encode_bits<7>(kv, blocks, heads, role, out, tab, stream); break;
    default: launch_encode_bits<4>(kv, blocks, heads, role, out, tab, stream); break;
  }
  return hipGetLastError();
}

}  // namespace lynx
