// Other cuts of the 8-bit code: a b + (8 - b) split into an anchor stream of
// b bits and a residual stream of 8 - b bits per element; and the
// dequantizers of every cut, the 4 + 4 planes included.
//
// Page "Lynx: the KV cache does not have to arrive whole", section 3 cuts
// the code 4 + 4 (the anchor names a geometric interval, the residual a
// position in it), section 4 decodes a draft from the anchor alone and the
// refined cache from both, and section 7 names 6 + 2, 2 + 6 and 5 + 3 as
// untried.  A
// cut keeps the top b bits of the code as the anchor and the low 8 - b bits
// as the residual; the draft code of anchor a is a * 2^(8-b) + 2^(7-b) - 1,
// the round-half-down centre of the anchor's codes.
//
// Streams: element k of a (page, head) tile -- the k-th nibble of the
// tile's 4-bit planes, in their role-dependent order -- occupies bits
// k*b .. k*b + b - 1 (least significant first) of the tile's anchor
// stream (b * 4096 bytes) and bits k*(8-b) .. of its residual stream.  A
// unit of 32 elements (16 bytes of each 4-bit plane) is exactly b words of
// the anchor stream and 8 - b words of the residual stream, so every
// thread here reads and writes whole words of its own units.
#include "lynx_cut.h"
#include "lynx_internal.h"

namespace lynx {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSplitThreads = 256;
constexpr int kUnitsPerTile = kPage * kDim / 32;  // 1024

struct YTable {
  float y[256];
};

// Field k of B bits of a unit's words (B <= 7, so a field spans at most
// two words), sign-extended or not.
template <int B, bool kSigned>
__device__ __forceinline__ int field(const uint32_t *w, int k) {
  const int o = k * B;
  const uint32_t lo = w[o >> 5];
  const uint32_t hi = ((o & 31) + B > 32) ? w[(o >> 5) + 1] : 0u;
  const uint32_t x = static_cast<uint32_t>(((static_cast<uint64_t>(hi) << 32) | lo) >> (o & 31));
  return kSigned ? __builtin_amdgcn_sbfe(static_cast<int>(x), 0, B)
                 : static_cast<int>(__builtin_amdgcn_ubfe(x, 0, B));
}

// Thread t of a block packs unit u0 + t.  The block's 256 units are b KiB
// of the anchor stream and 8 - b KiB of the residual stream, each
// contiguous, so the words are staged in LDS and written as 512 pieces of
// 16 B (pieces p < 64b the anchor stream's): every store instruction of a
// wave writes 1 KiB contiguous.  The launch covers whole tiles, a multiple
// of the block.
template <int B>
__global__ __launch_bounds__(kSplitThreads) void split_planes_kernel(
    const u32x4 *__restrict__ a4, const u32x4 *__restrict__ r4, uint32_t *__restrict__ aout,
    uint32_t *__restrict__ rout) {
  constexpr int RB = 8 - B;
  __shared__ __align__(16) uint32_t s_w[kSplitThreads * 8];  // anchor words, then residual words
  const size_t u0 = static_cast<size_t>(blockIdx.x) * kSplitThreads;
  const size_t u = u0 + threadIdx.x;
  const u32x4 av = __builtin_nontemporal_load(a4 + u);
  const u32x4 rv = __builtin_nontemporal_load(r4 + u);
  const uint32_t aw[4] = {av[0], av[1], av[2], av[3]};
  const uint32_t rw[4] = {rv[0], rv[1], rv[2], rv[3]};
  uint32_t wa[B], wr[RB];
  cut::unit<B>(aw, rw, wa, wr);
#pragma unroll
  for (int i = 0; i < B; ++i) s_w[threadIdx.x * B + i] = wa[i];
#pragma unroll
  for (int i = 0; i < RB; ++i) s_w[kSplitThreads * B + threadIdx.x * RB + i] = wr[i];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int p = static_cast<int>(threadIdx.x) + k * kSplitThreads;
    const u32x4 x = reinterpret_cast<const u32x4 *>(s_w)[p];
    u32x4 *dst = p < 64 * B ? reinterpret_cast<u32x4 *>(aout + u0 * B) + p
                            : reinterpret_cast<u32x4 *>(rout + u0 * RB) + (p - 64 * B);
    __builtin_nontemporal_store(x, dst);
  }
}

// xhat = mn + rg * (mu + s * yhat(code)) in fp32, written in the encoder's
// input layout [P][256][H][128].  The full code is the same 8-bit code at
// every cut, so a full reconstruction does not depend on b.  Every 16-byte
// store holds 4 channels of one token, and every store instruction of a
// wave writes two whole 512-byte token rows (splitting a row between store
// instructions, or writing half rows, measured a quarter to a third slower).
//
// A block takes one (page, head) tile.  Keys (a unit is 32 channels of one
// token): lane t unpacks the 4 units of token t into an LDS tile of 256
// tokens x 128 table indices; then lane l of wave v stores channels
// 4q .. 4q+3 (q = l % 32) of tokens 64v + 2m + g (g = l / 32, m < 32), one
// LDS word per token.  Values (a unit is the 32 tokens of one channel of a
// chunk): lane l of wave v loads the 4 adjacent units of channels 4q .. 4q+3
// of chunk 2v + g and stores its 32 tokens.
template <int B, int kRole, bool kFull>
__global__ __launch_bounds__(kSplitThreads) void dequant_split_kernel(
    const uint32_t *__restrict__ astream, const uint32_t *__restrict__ rstream, PlanesArg sc,
    int heads, float *__restrict__ out, YTable tab) {
  constexpr int RB = 8 - B;
  constexpr int kMid = RB > 0 ? (1 << (RB - 1)) - 1 : 0;
  __shared__ float s_y[256];
  s_y[threadIdx.x] = tab.y[threadIdx.x];
  const int q = threadIdx.x & 31;
  const int g = (threadIdx.x >> 5) & 1;
  const int v = threadIdx.x >> 6;
  const size_t row = static_cast<size_t>(heads) * kDim;
  float mn[4], rg[4], mu[4], s[4];
  auto load4 = [](float (&x)[4], const float *src) {
    const float4 f = *reinterpret_cast<const float4 *>(src);
    x[0] = f.x; x[1] = f.y; x[2] = f.z; x[3] = f.w;
  };
  const size_t tile = blockIdx.x;
  const size_t p = tile / static_cast<size_t>(heads);
  const int h = static_cast<int>(tile % static_cast<size_t>(heads));
  if constexpr (kRole == LYNX_ROLE_KEY) {
    // [token][128 table indices]; the 16-byte group j of token t's row sits
    // at group j ^ ((t >> 1) & 7), so that 16 lanes writing groups of 16
    // rows hit 64 distinct banks.
    __shared__ u32x4 s_code[kPage * kDim / 16];
    const int t = threadIdx.x;
    // the 4 units of token t (128 channels), B or 8 - B words each, are
    // contiguous and 16-byte aligned
    const size_t unit0 = tile * kUnitsPerTile + 4 * static_cast<size_t>(t);
    uint32_t wa[4 * B], wr[RB > 0 ? 4 * RB : 1];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const u32x4 x = reinterpret_cast<const u32x4 *>(astream + unit0 * B)[i];
      wa[4 * i] = x[0]; wa[4 * i + 1] = x[1]; wa[4 * i + 2] = x[2]; wa[4 * i + 3] = x[3];
    }
    if (kFull) {
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const u32x4 x = reinterpret_cast<const u32x4 *>(rstream + unit0 * RB)[i];
        wr[4 * i] = x[0]; wr[4 * i + 1] = x[1]; wr[4 * i + 2] = x[2]; wr[4 * i + 3] = x[3];
      }
    }
    // lane (q, g) of wave v: tokens 64v + 2m + g, chunk 2v (m < 16) or 2v + 1
    const int c0 = 2 * v;
    float mu1[4], s1[4];
    load4(mn, sc.page_min + tile * kDim + 4 * q);
    load4(rg, sc.page_range + tile * kDim + 4 * q);
    load4(mu, sc.chunk_mean + (tile * kChunks + c0) * kDim + 4 * q);
    load4(s, sc.chunk_maxabs + (tile * kChunks + c0) * kDim + 4 * q);
    load4(mu1, sc.chunk_mean + (tile * kChunks + c0 + 1) * kDim + 4 * q);
    load4(s1, sc.chunk_maxabs + (tile * kChunks + c0 + 1) * kDim + 4 * q);
#pragma unroll
    for (int j = 0; j < kDim / 16; ++j) {  // 16 channels: half of unit j / 2
      u32x4 x;
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) {
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = 16 * (j & 1) + 4 * w4 + e;  // field of unit j / 2
          const int a = field<B, true>(wa + (j >> 1) * B, k);
          const int r = kFull ? field<RB, false>(wr + (j >> 1) * RB, k) : kMid;
          word |= static_cast<uint32_t>(a * (1 << RB) + r + 128) << (8 * e);
        }
        x[w4] = word;
      }
      s_code[t * (kDim / 16) + (j ^ ((t >> 1) & 7))] = x;
    }
    __syncthreads();
    const uint32_t *codes = reinterpret_cast<const uint32_t *>(s_code);
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const int tk = 64 * v + 2 * m + g;
      const uint32_t w = codes[tk * (kDim / 4) + 4 * ((q >> 2) ^ ((tk >> 1) & 7)) + (q & 3)];
      const float *cm = m < 16 ? mu : mu1;
      const float *cs = m < 16 ? s : s1;
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = __builtin_fmaf(rg[i], __builtin_fmaf(cs[i], s_y[(w >> (8 * i)) & 255u], cm[i]), mn[i]);
      float *dst = out + (p * kPage + static_cast<size_t>(tk)) * row + static_cast<size_t>(h) * kDim;
      reinterpret_cast<float4 *>(dst)[q] = make_float4(o[0], o[1], o[2], o[3]);
    }
  } else {
    const int c = 2 * v + g;
    const size_t unit0 = tile * kUnitsPerTile + static_cast<size_t>(c) * kDim + 4 * q;
    // the 4 units' words are contiguous and 16-byte aligned (unit0 % 4 == 0)
    uint32_t wa[4 * B], wr[RB > 0 ? 4 * RB : 1];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const u32x4 x = reinterpret_cast<const u32x4 *>(astream + unit0 * B)[i];
      wa[4 * i] = x[0]; wa[4 * i + 1] = x[1]; wa[4 * i + 2] = x[2]; wa[4 * i + 3] = x[3];
    }
    if (kFull) {
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const u32x4 x = reinterpret_cast<const u32x4 *>(rstream + unit0 * RB)[i];
        wr[4 * i] = x[0]; wr[4 * i + 1] = x[1]; wr[4 * i + 2] = x[2]; wr[4 * i + 3] = x[3];
      }
    }
    load4(mn, sc.page_min + tile * kDim + 4 * q);
    load4(rg, sc.page_range + tile * kDim + 4 * q);
    load4(mu, sc.chunk_mean + (tile * kChunks + c) * kDim + 4 * q);
    load4(s, sc.chunk_maxabs + (tile * kChunks + c) * kDim + 4 * q);
    __syncthreads();  // the table
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int a = field<B, true>(wa + i * B, k);
        const int r = kFull ? field<RB, false>(wr + i * RB, k) : kMid;
        o[i] = __builtin_fmaf(rg[i], __builtin_fmaf(s[i], s_y[a * (1 << RB) + r + 128], mu[i]), mn[i]);
      }
      // field k is token 4 fw + fj (fj < 4) or 16 + 4 fw + fj - 4 of the
      // chunk, fw = k / 8, fj = k % 8
      const int fw = k >> 3, fj = k & 7;
      const int t = c * kChunk + (fj < 4 ? 4 * fw + fj : 16 + 4 * fw + (fj - 4));
      float *dst = out + (p * kPage + static_cast<size_t>(t)) * row + static_cast<size_t>(h) * kDim;
      reinterpret_cast<float4 *>(dst)[q] = make_float4(o[0], o[1], o[2], o[3]);
    }
  }
}

template <int B>
hipError_t launch_split_b(const PlanesArg &in, size_t units, uint8_t *aout, uint8_t *rout,
                          hipStream_t stream) {
  static_assert(kUnitsPerTile % kSplitThreads == 0, "blocks cover whole tiles");
  const dim3 grid(static_cast<unsigned>(units / kSplitThreads));
  hipLaunchKernelGGL(split_planes_kernel<B>, grid, dim3(kSplitThreads), 0, stream,
                     reinterpret_cast<const u32x4 *>(in.anchor),
                     reinterpret_cast<const u32x4 *>(in.residual), reinterpret_cast<uint32_t *>(aout),
                     reinterpret_cast<uint32_t *>(rout));
  return hipGetLastError();
}

template <int B, int kRole, bool kFull>
hipError_t launch_dq_split(const uint8_t *a, const uint8_t *r, const PlanesArg &sc, int heads,
                           size_t units, float *out, hipStream_t stream) {
  YTable tab;
  const DecodeTable &dt = decode_table();
  for (int i = 0; i < 256; ++i) tab.y[i] = dt.y[i];
  static_assert(kSplitThreads == kPage && kChunks == 2 * kSplitThreads / 64,
                "a block's lanes cover a tile's tokens, its waves the tile's chunks");
  const dim3 grid(static_cast<unsigned>(units / kUnitsPerTile));  // one tile per block
  hipLaunchKernelGGL((dequant_split_kernel<B, kRole, kFull>), grid, dim3(kSplitThreads), 0, stream,
                     reinterpret_cast<const uint32_t *>(a), reinterpret_cast<const uint32_t *>(r), sc,
                     heads, out, tab);
  return hipGetLastError();
}

template <int B>
hipError_t launch_dq_b(const uint8_t *a, const uint8_t *r, const PlanesArg &sc, int heads,
                       int role, size_t units, float *out, hipStream_t stream) {
  if (role == LYNX_ROLE_KEY)
    return r ? launch_dq_split<B, LYNX_ROLE_KEY, true>(a, r, sc, heads, units, out, stream)
             : launch_dq_split<B, LYNX_ROLE_KEY, false>(a, r, sc, heads, units, out, stream);
  return r ? launch_dq_split<B, LYNX_ROLE_VALUE, true>(a, r, sc, heads, units, out, stream)
           : launch_dq_split<B, LYNX_ROLE_VALUE, false>(a, r, sc, heads, units, out, stream);
}

}  // namespace

hipError_t launch_split_planes(const PlanesArg &in, int64_t num_pages, int heads, int anchor_bits,
                               uint8_t *anchor_out, uint8_t *residual_out, hipStream_t stream) {
  const size_t units = static_cast<size_t>(num_pages) * heads * kUnitsPerTile;
  if (units == 0) return hipSuccess;
  switch (anchor_bits) {
    case 1: return launch_split_b<1>(in, units, anchor_out, residual_out, stream);
    case 2: return launch_split_b<2>(in, units, anchor_out, residual_out, stream);
    case 3: return launch_split_b<3>(in, units, anchor_out, residual_out, stream);
    case 4: return launch_split_b<4>(in, units, anchor_out, residual_out, stream);
    case 5: return launch_split_b<5>(in, units, anchor_out, residual_out, stream);
    case 6: return launch_split_b<6>(in, units, anchor_out, residual_out, stream);
    case 7: return launch_split_b<7>(in, units, anchor_out, residual_out, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_dequant_split(const uint8_t *anchor, const uint8_t *residual, int anchor_bits,
                                const PlanesArg &scales, int64_t num_pages, int heads, int role,
                                float *out, hipStream_t stream) {
  const size_t units = static_cast<size_t>(num_pages) * heads * kUnitsPerTile;
  if (units == 0) return hipSuccess;
  switch (anchor_bits) {
    case 1: return launch_dq_b<1>(anchor, residual, scales, heads, role, units, out, stream);
    case 2: return launch_dq_b<2>(anchor, residual, scales, heads, role, units, out, stream);
    case 3: return launch_dq_b<3>(anchor, residual, scales, heads, role, units, out, stream);
    case 4: return launch_dq_b<4>(anchor, residual, scales, heads, role, units, out, stream);
    case 5: return launch_dq_b<5>(anchor, residual, scales, heads, role, units, out, stream);
    case 6: return launch_dq_b<6>(anchor, residual, scales, heads, role, units, out, stream);
    case 7: return launch_dq_b<7>(anchor, residual, scales, heads, role, units, out, stream);
    default: return hipErrorInvalidValue;
  }
}

// The 4 + 4 planes are the b = 4 streams (element k of a tile is nibble k of
// its planes) and 16a + 7 is the b = 4 round-half-down centre, so the 4 + 4
// dequantizers are the b = 4 kernel.
hipError_t launch_dequant(const PlanesArg &in, int64_t num_pages, int heads, int role, bool full,
                          float *out, hipStream_t stream) {
  return launch_dequant_split(in.anchor, full ? in.residual : nullptr, 4, in, num_pages, heads,
                              role, out, stream);
}

}  // namespace lynx
