// Other cuts of the 8-bit code: a b + (8 - b) split into an anchor stream of
// b bits and a residual stream of 8 - b bits per element.
//
// Page "Lynx: the KV cache does not have to arrive whole", section 3 cuts
// the code 4 + 4 (the anchor names a geometric interval, the residual a
// position in it); section 7 names 6 + 2, 2 + 6 and 5 + 3 as untried.  A
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
// thread here reads and writes whole words of its own unit.
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

template <int B>
__global__ __launch_bounds__(kSplitThreads) void split_planes_kernel(
    const u32x4 *__restrict__ a4, const u32x4 *__restrict__ r4, uint32_t *__restrict__ aout,
    uint32_t *__restrict__ rout, size_t units) {
  constexpr int RB = 8 - B;
  const size_t u = static_cast<size_t>(blockIdx.x) * kSplitThreads + threadIdx.x;
  if (u >= units) return;
  const u32x4 av = __builtin_nontemporal_load(a4 + u);
  const u32x4 rv = __builtin_nontemporal_load(r4 + u);
  const uint32_t aw[4] = {av[0], av[1], av[2], av[3]};
  const uint32_t rw[4] = {rv[0], rv[1], rv[2], rv[3]};
  uint32_t wa[B], wr[RB];
  cut::unit<B>(aw, rw, wa, wr);
#pragma unroll
  for (int i = 0; i < B; ++i) __builtin_nontemporal_store(wa[i], aout + u * B + i);
#pragma unroll
  for (int i = 0; i < RB; ++i) __builtin_nontemporal_store(wr[i], rout + u * RB + i);
}

// xhat = mn + rg * (mu + s * yhat(code)), the arithmetic of the 4 + 4
// dequantizers (so a full reconstruction is bit-identical to theirs).  A
// block takes 256 units of one tile.  Values: a unit is the 32 tokens of
// one channel of a chunk, and consecutive lanes hold consecutive channels,
// so each lane keeps its channel's four scales and every store instruction
// is contiguous.  Keys: a unit is 32 channels of one token; the block's 256
// units are 64 whole tokens, so each lane first unpacks its unit's codes
// into an LDS tile of 64 tokens x 128 channels, then takes one channel of
// one chunk (32 tokens) as for the values.
template <int B, int kRole, bool kFull>
__global__ __launch_bounds__(kSplitThreads) void dequant_split_kernel(
    const uint32_t *__restrict__ astream, const uint32_t *__restrict__ rstream, PlanesArg sc,
    int heads, float *__restrict__ out, YTable tab) {
  constexpr int RB = 8 - B;
  constexpr int kMid = RB > 0 ? (1 << (RB - 1)) - 1 : 0;
  __shared__ float s_y[256];
  __shared__ uint32_t s_code[kRole == LYNX_ROLE_KEY ? 64 * kDim / 4 : 1];  // [token][128 codes]
  s_y[threadIdx.x] = tab.y[threadIdx.x];
  // the launch covers whole tiles: kUnitsPerTile is a multiple of the block
  const size_t u = static_cast<size_t>(blockIdx.x) * kSplitThreads + threadIdx.x;
  uint32_t wa[B], wr[RB > 0 ? RB : 1];
#pragma unroll
  for (int i = 0; i < B; ++i) wa[i] = astream[u * B + i];
  if (kFull) {
#pragma unroll
    for (int i = 0; i < RB; ++i) wr[i] = rstream[u * RB + i];
  }
  // table index (code + 128) of field k of this lane's unit
  auto index = [&](int k) {
    const int a = field<B, true>(wa, k);
    const int r = kFull ? field<RB, false>(wr, k) : kMid;
    return static_cast<uint32_t>(a * (1 << RB) + r + 128);
  };
  const size_t tile = u / kUnitsPerTile;
  const size_t p = tile / static_cast<size_t>(heads);
  const int h = static_cast<int>(tile % static_cast<size_t>(heads));
  const size_t row = static_cast<size_t>(heads) * kDim;
  const int ub = static_cast<int>((static_cast<size_t>(blockIdx.x) * kSplitThreads) % kUnitsPerTile);
  int d, c, t0;  // this lane's channel, chunk and first token in the tile
  uint32_t idx[32];
  if (kRole == LYNX_ROLE_KEY) {
    // unit ub + i: token (ub + i) / 4, channels ((ub + i) % 4) * 32 ..
#pragma unroll
    for (int w4 = 0; w4 < 8; ++w4)
      s_code[threadIdx.x * 8 + w4] = index(4 * w4) | (index(4 * w4 + 1) << 8) |
                                      (index(4 * w4 + 2) << 16) | (index(4 * w4 + 3) << 24);
    __syncthreads();
    d = threadIdx.x & 127;
    const int half = threadIdx.x >> 7;  // tokens 32 half .. of the block's 64
    t0 = ub / 4 + 32 * half;
    c = t0 / kChunk;
    const uint8_t *codes = reinterpret_cast<const uint8_t *>(s_code);
#pragma unroll
    for (int k = 0; k < 32; ++k) idx[k] = codes[(32 * half + k) * kDim + d];
  } else {
    const int uu = ub + static_cast<int>(threadIdx.x);
    c = uu >> 7;
    d = uu & 127;
    t0 = c * kChunk;
#pragma unroll
    for (int k = 0; k < 32; ++k) idx[k] = index(k);
    __syncthreads();  // the table
  }
  const float mn = sc.page_min[tile * kDim + d];
  const float rg = sc.page_range[tile * kDim + d];
  const float mu = sc.chunk_mean[(tile * kChunks + c) * kDim + d];
  const float s = sc.chunk_maxabs[(tile * kChunks + c) * kDim + d];
  float *dst = out + (p * kPage + static_cast<size_t>(t0)) * row + static_cast<size_t>(h) * kDim + d;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    // keys: token k of the lane's 32; values: field k is token 4w + i
    // (i < 4) or 16 + 4w + i - 4 of the chunk, w = k / 8, i = k % 8
    const int w = k >> 3, i = k & 7;
    const int t = kRole == LYNX_ROLE_KEY ? k : (i < 4 ? 4 * w + i : 16 + 4 * w + (i - 4));
    dst[static_cast<size_t>(t) * row] = __builtin_fmaf(rg, __builtin_fmaf(s, s_y[idx[k]], mu), mn);
  }
}

template <int B>
hipError_t launch_split_b(const PlanesArg &in, size_t units, uint8_t *aout, uint8_t *rout,
                          hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((units + kSplitThreads - 1) / kSplitThreads));
  hipLaunchKernelGGL(split_planes_kernel<B>, grid, dim3(kSplitThreads), 0, stream,
                     reinterpret_cast<const u32x4 *>(in.anchor),
                     reinterpret_cast<const u32x4 *>(in.residual), reinterpret_cast<uint32_t *>(aout),
                     reinterpret_cast<uint32_t *>(rout), units);
  return hipGetLastError();
}

template <int B, int kRole, bool kFull>
hipError_t launch_dq_split(const uint8_t *a, const uint8_t *r, const PlanesArg &sc, int heads,
                           size_t units, float *out, hipStream_t stream) {
  YTable tab;
  const DecodeTable &dt = decode_table();
  for (int i = 0; i < 256; ++i) tab.y[i] = dt.y[i];
  static_assert(kUnitsPerTile % kSplitThreads == 0, "blocks cover whole tiles");
  const dim3 grid(static_cast<unsigned>(units / kSplitThreads));
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

}  // namespace lynx
