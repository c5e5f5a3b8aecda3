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
// 256-entry yhat table sits in LDS.  A lane writes 4 channels of a token as
// one 16-byte store, half a wave covering a 512-byte token row, so each store
// instruction of a wave writes two whole rows (splitting a row over two store
// instructions, or writing half rows, measured about a quarter slower).  A
// wave takes 2 of a tile's 8 chunks and requests both chunks' codes and
// scales before its first store.
#include "lynx_internal.h"

namespace lynx {
namespace {

constexpr int kDqThreads = 256;
constexpr int kWaveChunks = kChunks / (kDqThreads / 64);  // chunks per wave

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
  // Wave v takes chunks v, v + 4; lane l of it channels 4q .. 4q+3 (q =
  // l % 32) of the chunk's tokens 2k + g (g = l / 32), so every 16-byte store
  // of a wave writes two adjacent whole 512-byte token rows.  The 4 channels
  // are nibbles 4(q % 2) .. 4(q % 2) + 3 of the token's code word q / 2.
  const int q = threadIdx.x & 31;
  const int g = (threadIdx.x >> 5) & 1;
  const int sh = (q & 1) * 16;
  float mn[4], rg[4];
  {
    const float4 m = reinterpret_cast<const float4 *>(in.page_min + static_cast<size_t>(tile) * kDim)[q];
    const float4 r = reinterpret_cast<const float4 *>(in.page_range + static_cast<size_t>(tile) * kDim)[q];
    mn[0] = m.x; mn[1] = m.y; mn[2] = m.z; mn[3] = m.w;
    rg[0] = r.x; rg[1] = r.y; rg[2] = r.z; rg[3] = r.w;
  }
  // Both chunks' scales and codes are requested before the first store.
  float4 u[kWaveChunks], sv[kWaveChunks];
  uint32_t a[kWaveChunks][kChunk / 2], r[kWaveChunks][kChunk / 2];
#pragma unroll
  for (int n = 0; n < kWaveChunks; ++n) {
    const int c = (threadIdx.x >> 6) + n * (kDqThreads / 64);
    const size_t cidx = (static_cast<size_t>(tile) * kChunks + c) * kDim;
    u[n] = reinterpret_cast<const float4 *>(in.chunk_mean + cidx)[q];
    sv[n] = reinterpret_cast<const float4 *>(in.chunk_maxabs + cidx)[q];
#pragma unroll
    for (int k = 0; k < kChunk / 2; ++k) {
      const size_t w = (static_cast<size_t>(tile) * kPage + c * kChunk + 2 * k + g) * 16 + (q >> 1);
      a[n][k] = an[w] >> sh;
      r[n][k] = kFull ? re[w] >> sh : 0x7777u;
    }
  }
  // Keep every load ahead of the stores: the memory counter the waits use
  // counts stores too, so a load placed after a store waits for that store.
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int n = 0; n < kWaveChunks; ++n) {
    const int c = (threadIdx.x >> 6) + n * (kDqThreads / 64);
    const float mu[4] = {u[n].x, u[n].y, u[n].z, u[n].w};
    const float sc[4] = {sv[n].x, sv[n].y, sv[n].z, sv[n].w};
#pragma unroll
    for (int k = 0; k < kChunk / 2; ++k) {
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float y = s_y[table_index((a[n][k] >> (4 * i)) & 15u, (r[n][k] >> (4 * i)) & 15u)];
        o[i] = __builtin_fmaf(rg[i], __builtin_fmaf(sc[i], y, mu[i]), mn[i]);
      }
      const int t = c * kChunk + 2 * k + g;
      float *dst = out + (static_cast<size_t>(p) * kPage + t) * row + static_cast<size_t>(h) * kDim;
      reinterpret_cast<float4 *>(dst)[q] = make_float4(o[0], o[1], o[2], o[3]);
    }
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
  // Wave v takes chunks v, v + 4; lane l of it channels 4q .. 4q+3 (q =
  // l % 32) and the 16 tokens in words 2g, 2g + 1 (g = l / 32) of each
  // channel's 4 code words, so every 16-byte store of a wave covers two whole
  // 512-byte token rows (tokens t and t + 8).
  const int q = threadIdx.x & 31;
  const int g = (threadIdx.x >> 5) & 1;
  float mn[4], rg[4];
  {
    const float4 m = reinterpret_cast<const float4 *>(in.page_min + static_cast<size_t>(tile) * kDim)[q];
    const float4 r = reinterpret_cast<const float4 *>(in.page_range + static_cast<size_t>(tile) * kDim)[q];
    mn[0] = m.x; mn[1] = m.y; mn[2] = m.z; mn[3] = m.w;
    rg[0] = r.x; rg[1] = r.y; rg[2] = r.z; rg[3] = r.w;
  }
  // Both chunks' scales and codes are requested before the first store.
  float4 u[kWaveChunks], sv[kWaveChunks];
  uint2 a[kWaveChunks][4], r[kWaveChunks][4];
#pragma unroll
  for (int n = 0; n < kWaveChunks; ++n) {
    const int c = (threadIdx.x >> 6) + n * (kDqThreads / 64);
    const size_t cidx = (static_cast<size_t>(tile) * kChunks + c) * kDim;
    u[n] = reinterpret_cast<const float4 *>(in.chunk_mean + cidx)[q];
    sv[n] = reinterpret_cast<const float4 *>(in.chunk_maxabs + cidx)[q];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t w = (cidx + 4 * q + i) * 4 + 2 * g;
      a[n][i] = *reinterpret_cast<const uint2 *>(an + w);
      r[n][i] = kFull ? *reinterpret_cast<const uint2 *>(re + w) : make_uint2(0x77777777u, 0x77777777u);
    }
  }
  // Keep every load ahead of the stores: the memory counter the waits use
  // counts stores too, so a load placed after a store waits for that store.
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int n = 0; n < kWaveChunks; ++n) {
    const int c = (threadIdx.x >> 6) + n * (kDqThreads / 64);
    const float mu[4] = {u[n].x, u[n].y, u[n].z, u[n].w};
    const float sc[4] = {sv[n].x, sv[n].y, sv[n].z, sv[n].w};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t aw = k ? a[n][i].y : a[n][i].x;
          const uint32_t rw = k ? r[n][i].y : r[n][i].x;
          const float y = s_y[table_index((aw >> (4 * j)) & 15u, (rw >> (4 * j)) & 15u)];
          o[i] = __builtin_fmaf(rg[i], __builtin_fmaf(sc[i], y, mu[i]), mn[i]);
        }
        const int t = c * kChunk + chunk_token(2 * g + k, j);
        float *dst = out + (static_cast<size_t>(p) * kPage + t) * row + static_cast<size_t>(h) * kDim;
        reinterpret_cast<float4 *>(dst)[q] = make_float4(o[0], o[1], o[2], o[3]);
      }
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
