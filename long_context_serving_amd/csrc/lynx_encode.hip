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
// exact in fp64, the page range and chunk max-abs keep 7 significant bits
// (rounded up), and the level m is exactly #{k >= 1 : u >= T[k]}.
#include "lynx_internal.h"

namespace lynx {
namespace {

constexpr int kEncThreads = 512;

// Level window of the fast path: if 127 F(u) computed with v_log_f32 lies
// within this many levels of a rounding boundary, the level is recomputed
// exactly from the threshold table.  The fast path's error is far smaller
// (it is checked exhaustively over every fp32 u in [0, 1] by the tests).
constexpr float kNearWindow = 1.0f / 4096.0f;

struct EncodeTables {
  float t[128];
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

// Level of u in [0, 1]: 127 ln(1 + 255u)/ln 256 = 15.875 log2(1 + 255u),
// rounded half up.
__device__ __forceinline__ int level_of(float u, const float *T) {
  const float w = __builtin_fmaf(u, 255.0f, 1.0f);
  const float l2 = __builtin_amdgcn_logf(w);
  const float t = __builtin_fmaf(l2, 15.875f, 0.5f);
  int m = static_cast<int>(t);
  const float f = t - static_cast<float>(m);
  m = m > 127 ? 127 : m;
  if (f < kNearWindow || f > 1.0f - kNearWindow) m = level_exact(u, T);
  return m;
}

// Keep 7 significant bits, rounding towards +infinity (x >= 0, finite).
__device__ __forceinline__ float round_up_7bits(float x) {
  uint32_t b = __float_as_uint(x);
  if (b & 0x1FFFFu) b = (b + 0x1FFFFu) & ~0x1FFFFu;
  return __uint_as_float(b);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__global__ __launch_bounds__(kEncThreads) void encode_kernel(
    const uint16_t *__restrict__ kv, int heads, int role, PlanesArg out,
    EncodeTables tab) {
  const int tile = blockIdx.x;  // page * heads + head
  const int p = tile / heads;
  const int h = tile - p * heads;
  const int c = threadIdx.x >> 6;  // chunk = wave
  const int lane = threadIdx.x & 63;
  const int cg = lane & 15;
  const int r = lane >> 4;

  __shared__ float s_T[128];
  __shared__ float s_min[kChunks][kDim];
  __shared__ float s_max[kChunks][kDim];
  __shared__ float s_mn[kDim];
  __shared__ float s_inv[kDim];

  if (threadIdx.x < 128) s_T[threadIdx.x] = tab.t[threadIdx.x];

  // ---- load the lane's 8 tokens x 8 channels (bf16 -> fp32 is exact) ----
  const size_t row = static_cast<size_t>(heads) * kDim;
  const uint16_t *base = kv + static_cast<size_t>(p) * kPage * row +
                         static_cast<size_t>(h) * kDim + cg * 8;
  float x[8][8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int t = c * kChunk + chunk_token(r, j);
    const uint4 v = *reinterpret_cast<const uint4 *>(base + static_cast<size_t>(t) * row);
    x[j][0] = bf16_lo(v.x); x[j][1] = bf16_hi(v.x);
    x[j][2] = bf16_lo(v.y); x[j][3] = bf16_hi(v.y);
    x[j][4] = bf16_lo(v.z); x[j][5] = bf16_hi(v.z);
    x[j][6] = bf16_lo(v.w); x[j][7] = bf16_hi(v.w);
  }

  // ---- page-level normalisation: per-channel min and max ----
  float mn[8], mx[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    mn[i] = x[0][i];
    mx[i] = x[0][i];
#pragma unroll
    for (int j = 1; j < 8; ++j) {
      mn[i] = fminf(mn[i], x[j][i]);
      mx[i] = fmaxf(mx[i], x[j][i]);
    }
    mn[i] = fminf(mn[i], __shfl_xor(mn[i], 16));
    mx[i] = fmaxf(mx[i], __shfl_xor(mx[i], 16));
    mn[i] = fminf(mn[i], __shfl_xor(mn[i], 32));
    mx[i] = fmaxf(mx[i], __shfl_xor(mx[i], 32));
  }
  if (r == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      s_min[c][cg * 8 + i] = mn[i];
      s_max[c][cg * 8 + i] = mx[i];
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
    // the range is kept with 7 significant bits (rounded up), which makes
    // every scale product exact in the decoder's fp16 operand halves
    const float rg = round_up_7bits(b - a);
    // correctly rounded fp32 reciprocal (fp64 quotient, one rounding)
    const float inv = rg > 0.0f ? static_cast<float>(1.0 / static_cast<double>(rg)) : 0.0f;
    s_mn[d] = a;
    s_inv[d] = inv;
    const size_t sidx = static_cast<size_t>(tile) * kDim + d;
    out.page_min[sidx] = a;
    out.page_range[sidx] = rg;
  }
  __syncthreads();

  float inv_rg[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    mn[i] = s_mn[cg * 8 + i];
    inv_rg[i] = s_inv[cg * 8 + i];
  }

  // ---- x' = (x - mn) * inv_rg, and the exact chunk sum in fp64 ----
  double sum[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sum[i] = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float diff = x[j][i] - mn[i];
      x[j][i] = diff * inv_rg[i];
      sum[i] += static_cast<double>(x[j][i]);
    }
  }
  float mu[8], sabs[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    sum[i] += __shfl_xor(sum[i], 16);
    sum[i] += __shfl_xor(sum[i], 32);
    mu[i] = static_cast<float>(sum[i] * (1.0 / kChunk));
    sabs[i] = 0.0f;
  }

  // ---- chunk centring and max-abs ----
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[j][i] = x[j][i] - mu[i];
      sabs[i] = fmaxf(sabs[i], fabsf(x[j][i]));
    }
  }
  float inv_s[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    sabs[i] = fmaxf(sabs[i], __shfl_xor(sabs[i], 16));
    sabs[i] = fmaxf(sabs[i], __shfl_xor(sabs[i], 32));
    sabs[i] = round_up_7bits(sabs[i]);
  }
  // each of the 4 lanes sharing these channels computes 2 of the 8
  // reciprocals; the rest are gathered from the other lanes
  float my_inv[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float s = sabs[2 * r + k];
    my_inv[k] = s > 0.0f ? static_cast<float>(1.0 / static_cast<double>(s)) : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int src = cg + 16 * (i >> 1);  // lane holding channel i's reciprocal
    const float v0 = __shfl(my_inv[0], src);
    const float v1 = __shfl(my_inv[1], src);
    inv_s[i] = (i & 1) ? v1 : v0;
  }
  if (r == 0) {
    float *mean_out = out.chunk_mean + (static_cast<size_t>(tile) * kChunks + c) * kDim + cg * 8;
    float *maxabs_out = out.chunk_maxabs + (static_cast<size_t>(tile) * kChunks + c) * kDim + cg * 8;
    reinterpret_cast<float4 *>(mean_out)[0] = make_float4(mu[0], mu[1], mu[2], mu[3]);
    reinterpret_cast<float4 *>(mean_out)[1] = make_float4(mu[4], mu[5], mu[6], mu[7]);
    reinterpret_cast<float4 *>(maxabs_out)[0] = make_float4(sabs[0], sabs[1], sabs[2], sabs[3]);
    reinterpret_cast<float4 *>(maxabs_out)[1] = make_float4(sabs[4], sabs[5], sabs[6], sabs[7]);
  }

  // ---- sign-aware alpha-law code ----
  int code[8][8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float u = fabsf(x[j][i]) * inv_s[i];
      u = fminf(u, 1.0f);
      const int m = level_of(u, s_T);
      code[j][i] = x[j][i] < 0.0f ? ~m : m;
    }
  }

  // ---- the cut: anchor = code >> 4, residual = code & 15; pack nibbles ----
  if (role == LYNX_ROLE_KEY) {
    uint32_t *an = reinterpret_cast<uint32_t *>(out.anchor);
    uint32_t *re = reinterpret_cast<uint32_t *>(out.residual);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t a = 0, q = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        a |= static_cast<uint32_t>((code[j][i] >> 4) & 15) << (4 * i);
        q |= static_cast<uint32_t>(code[j][i] & 15) << (4 * i);
      }
      const int t = c * kChunk + chunk_token(r, j);
      const size_t w = (static_cast<size_t>(tile) * kPage + t) * (kDim / 8) + cg;
      an[w] = a;
      re[w] = q;
    }
  } else {
    uint32_t *an = reinterpret_cast<uint32_t *>(out.anchor);
    uint32_t *re = reinterpret_cast<uint32_t *>(out.residual);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t a = 0, q = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        a |= static_cast<uint32_t>((code[j][i] >> 4) & 15) << (4 * j);
        q |= static_cast<uint32_t>(code[j][i] & 15) << (4 * j);
      }
      const size_t w = ((static_cast<size_t>(tile) * kChunks + c) * kDim + cg * 8 + i) * 4 + r;
      an[w] = a;
      re[w] = q;
    }
  }
}

// Exhaustive check of the fast level path against the exact threshold count
// over fp32 bit patterns [begin, end) (values in [0, 1]).
__global__ __launch_bounds__(256) void code_map_check_kernel(uint32_t begin, uint32_t end,
                                                             unsigned long long *mismatches,
                                                             EncodeTables tab) {
  __shared__ float s_T[128];
  if (threadIdx.x < 128) s_T[threadIdx.x] = tab.t[threadIdx.x];
  __syncthreads();
  unsigned long long bad = 0;
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t b = begin + blockIdx.x * blockDim.x + threadIdx.x; b < end && b >= begin;
       b += stride) {
    const float u = __uint_as_float(b);
    bad += level_of(u, s_T) != level_exact(u, s_T);
  }
  if (bad) atomicAdd(mismatches, bad);
}

}  // namespace

hipError_t launch_code_map_check(uint32_t begin, uint32_t end, unsigned long long *mismatches,
                                 hipStream_t stream) {
  if (end <= begin) return hipSuccess;
  EncodeTables tab;
  const CodeTable &ct = code_table();
  for (int k = 0; k < 128; ++k) tab.t[k] = ct.t[k];
  hipLaunchKernelGGL(code_map_check_kernel, dim3(4096), dim3(256), 0, stream, begin, end,
                     mismatches, tab);
  return hipGetLastError();
}

hipError_t launch_encode(const uint16_t *kv, int64_t num_pages, int heads,
                         int role, const PlanesArg &out, hipStream_t stream) {
  if (num_pages == 0) return hipSuccess;
  EncodeTables tab;
  const CodeTable &ct = code_table();
  for (int k = 0; k < 128; ++k) tab.t[k] = ct.t[k];
  const unsigned blocks = static_cast<unsigned>(num_pages * heads);
  hipLaunchKernelGGL(encode_kernel, dim3(blocks), dim3(kEncThreads), 0, stream, kv,
                     heads, role, out, tab);
  return hipGetLastError();
}

}  // namespace lynx
