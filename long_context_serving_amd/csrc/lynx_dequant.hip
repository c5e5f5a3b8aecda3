// Standalone dequantizers: anchor-only (draft) and anchor + residual (full).
//
// Page "Lynx: the KV cache does not have to arrive whole", section 3 (the
// cut: the anchor fixes a geometric interval, the residual a position inside
// it) and section 4 (the draft decodes from the anchor stream alone; the
// refined cache from both).  The draft code of anchor a is 16a + 7, the
// round-half-down centre of the anchor's 16 codes.
//
// xhat = mn + rg * (mu + s * yhat(code)), written as fp32 in the encoder's
// input layout [P][256][H][128].  One workgroup per (page, head) tile; the
// 256-entry yhat table sits in LDS.  Lanes run along channels so that every
// store instruction writes contiguous 256-byte rows.
#include "lynx_internal.h"

namespace lynx {
namespace {

constexpr int kDqThreads = 256;

struct YTable {
  float y[256];
};

__device__ __forceinline__ int chunk_token(int w, int j) {
  return j < 4 ? 4 * w + j : 16 + 4 * w + (j - 4);
}

// Table index of the code from its anchor nibble (two's complement int4)
// and residual nibble: (a << 4 | r) read as int8, plus 128.
__device__ __forceinline__ int table_index(uint32_t a_nib, uint32_t r_nib) {
  return static_cast<int>(((a_nib << 4) | r_nib) ^ 0x80u);
}

template <bool kFull>
__global__ __launch_bounds__(kDqThreads) void dequant_key_kernel(
    PlanesArg in, int heads, float *__restrict__ out, YTable tab) {
  const int tile = blockIdx.x;
  const int p = tile / heads;
  const int h = tile - p * heads;
  __shared__ float s_y[256];
  s_y[threadIdx.x] = tab.y[threadIdx.x];
  __syncthreads();
  const uint32_t *an = reinterpret_cast<const uint32_t *>(in.anchor);
  const uint32_t *re = reinterpret_cast<const uint32_t *>(in.residual);
  const size_t row = static_cast<size_t>(heads) * kDim;
  // 256 tokens x 16 channel groups of 8; lanes walk the channel groups
  for (int it = 0; it < kPage * 16 / kDqThreads; ++it) {
    const int item = it * kDqThreads + threadIdx.x;
    const int t = item >> 4;
    const int cg = item & 15;
    const int c = t / kChunk;
    const size_t w = (static_cast<size_t>(tile) * kPage + t) * 16 + cg;
    const uint32_t a = an[w];
    const uint32_t q = kFull ? re[w] : 0x77777777u;
    const float *pm = in.page_min + static_cast<size_t>(tile) * kDim + cg * 8;
    const float *pr = in.page_range + static_cast<size_t>(tile) * kDim + cg * 8;
    const size_t cidx = (static_cast<size_t>(tile) * kChunks + c) * kDim + cg * 8;
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float y = s_y[table_index((a >> (4 * i)) & 15u, (q >> (4 * i)) & 15u)];
      const float inner = __builtin_fmaf(in.chunk_maxabs[cidx + i], y, in.chunk_mean[cidx + i]);
      o[i] = __builtin_fmaf(pr[i], inner, pm[i]);
    }
    float *dst = out + (static_cast<size_t>(p) * kPage + t) * row + static_cast<size_t>(h) * kDim + cg * 8;
    reinterpret_cast<float4 *>(dst)[0] = make_float4(o[0], o[1], o[2], o[3]);
    reinterpret_cast<float4 *>(dst)[1] = make_float4(o[4], o[5], o[6], o[7]);
  }
}

template <bool kFull>
__global__ __launch_bounds__(kDqThreads) void dequant_value_kernel(
    PlanesArg in, int heads, float *__restrict__ out, YTable tab) {
  const int tile = blockIdx.x;
  const int p = tile / heads;
  const int h = tile - p * heads;
  __shared__ float s_y[256];
  s_y[threadIdx.x] = tab.y[threadIdx.x];
  __syncthreads();
  const uint32_t *an = reinterpret_cast<const uint32_t *>(in.anchor);
  const uint32_t *re = reinterpret_cast<const uint32_t *>(in.residual);
  const size_t row = static_cast<size_t>(heads) * kDim;
  // 8 chunks x 4 words x 128 channels; lanes walk the channels
  for (int it = 0; it < kChunks * 4 * kDim / kDqThreads; ++it) {
    const int item = it * kDqThreads + threadIdx.x;
    const int d = item & (kDim - 1);
    const int wd = (item >> 7) & 3;
    const int c = item >> 9;
    const size_t w = ((static_cast<size_t>(tile) * kChunks + c) * kDim + d) * 4 + wd;
    const uint32_t a = an[w];
    const uint32_t q = kFull ? re[w] : 0x77777777u;
    const float mn = in.page_min[static_cast<size_t>(tile) * kDim + d];
    const float rg = in.page_range[static_cast<size_t>(tile) * kDim + d];
    const size_t cidx = (static_cast<size_t>(tile) * kChunks + c) * kDim + d;
    const float mu = in.chunk_mean[cidx];
    const float s = in.chunk_maxabs[cidx];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float y = s_y[table_index((a >> (4 * j)) & 15u, (q >> (4 * j)) & 15u)];
      const int t = c * kChunk + chunk_token(wd, j);
      out[(static_cast<size_t>(p) * kPage + t) * row + static_cast<size_t>(h) * kDim + d] =
          __builtin_fmaf(rg, __builtin_fmaf(s, y, mu), mn);
    }
  }
}

}  // namespace

hipError_t launch_dequant(const PlanesArg &in, int64_t num_pages, int heads,
                          int role, bool full, float *out,
                          hipStream_t stream) {
  if (num_pages == 0) return hipSuccess;
  YTable tab;
  const DecodeTable &dt = decode_table();
  for (int k = 0; k < 256; ++k) tab.y[k] = dt.y[k];
  const dim3 grid(static_cast<unsigned>(num_pages * heads));
  if (role == LYNX_ROLE_KEY) {
    if (full)
      hipLaunchKernelGGL(dequant_key_kernel<true>, grid, dim3(kDqThreads), 0, stream, in, heads, out, tab);
    else
      hipLaunchKernelGGL(dequant_key_kernel<false>, grid, dim3(kDqThreads), 0, stream, in, heads, out, tab);
  } else {
    if (full)
      hipLaunchKernelGGL(dequant_value_kernel<true>, grid, dim3(kDqThreads), 0, stream, in, heads, out, tab);
    else
      hipLaunchKernelGGL(dequant_value_kernel<false>, grid, dim3(kDqThreads), 0, stream, in, heads, out, tab);
  }
  return hipGetLastError();
}

}  // namespace lynx
