// Attention over the bf16 tail page of each request.
//
// Pages are quantized whole (page "Lynx: the KV cache does not have to
// arrive whole", section 3: the page of 256 tokens is the unit of the
// quantizer), so the newest tokens of a request -- fewer than a page, plus
// the speculative tokens a verify pass scores (section 4: drafts run on the
// anchor stream, the refined cache verifies them) -- stay in bf16 until
// their page fills.  This kernel reduces the tail of every (query row, KV
// head) to one (m, l, o) partial that the split combine merges with the
// partials of the quantized pages; query token i of a request sees tail
// tokens 0 .. tail_len - tq + i (itself and everything before it).
//
// The tail holds at most LYNX_TAIL_TOKENS tokens per request, so a block of
// 256 threads keeps every score of its row group in LDS.  Products of bf16
// values are exact in fp64 and the sums run in fp64, so the only roundings
// are those of the fp64 sums and of storing l and o as fp32 partials.
#include <math.h>

#include "lynx_internal.h"

namespace lynx {
namespace {

constexpr int kTailThreads = 256;
constexpr int kTailCap = LYNX_TAIL_TOKENS;
constexpr int kMaxG = LYNX_MAX_GROUP;

// (m, l, o) partial rows, laid out as the page kernels lay them out:
// m fp64 [n], l fp32 [n], o fp32 [n][128], n = rows * H * parts * group
using TailPartials = AttnPartials;

__device__ __forceinline__ TailPartials tail_partials_of(void *ws, const AttnShape &s) {
  return attn_partials(ws, s);
}

__device__ __forceinline__ double bf16_to_double(uint32_t bits16) {
  return static_cast<double>(__uint_as_float(bits16 << 16));
}

// Block = (query row b, KV head h).
__global__ __launch_bounds__(kTailThreads) void attn_tail_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ tail_k,
    const uint16_t *__restrict__ tail_v, const int32_t *__restrict__ tail_len, AttnShape s,
    int tail_cap, double score_scale, bool base2, void *ws) {
  const int bh = blockIdx.x;
  const int h = bh % s.heads;
  const int b = bh / s.heads;
  const int req = b / s.tq;
  const int i = b % s.tq;  // query token within the request
  const int g = s.group;
  const int tid = threadIdx.x;

  __shared__ double s_q[kMaxG][kDim];
  __shared__ double s_p[kTailCap][kMaxG];  // scores, then probabilities
  __shared__ double s_m[kMaxG], s_l[kMaxG];

  int n = tail_len[req];
  n = n < 0 ? 0 : (n > tail_cap ? tail_cap : n);
  int vis = n - s.tq + i + 1;  // tail tokens this query token sees
  vis = vis < 0 ? 0 : (vis > n ? n : vis);

  for (int e = tid; e < g * kDim; e += kTailThreads) {
    const int j = e / kDim, d = e % kDim;
    s_q[j][d] = bf16_to_double(q[(static_cast<size_t>(b) * s.q_heads + h * g + j) * kDim + d]);
  }
  __syncthreads();

  // ---- scores: thread t takes tail token t (and t + 256) for every head ----
  const size_t row_stride = static_cast<size_t>(s.heads) * kDim;  // one token of the tail
  const uint16_t *kbase = tail_k + (static_cast<size_t>(req) * tail_cap * s.heads + h) * kDim;
  for (int t = tid; t < vis; t += kTailThreads) {
    double acc[kMaxG];
#pragma unroll
    for (int j = 0; j < kMaxG; ++j) acc[j] = 0.0;
    const uint4 *krow = reinterpret_cast<const uint4 *>(kbase + t * row_stride);
    for (int d8 = 0; d8 < kDim / 8; ++d8) {
      const uint4 w = krow[d8];
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double k0 = bf16_to_double(u[e] & 0xFFFFu), k1 = bf16_to_double(u[e] >> 16);
        const int d = 8 * d8 + 2 * e;
#pragma unroll
        for (int j = 0; j < kMaxG; ++j)
          if (j < g) acc[j] = fma(s_q[j][d + 1], k1, fma(s_q[j][d], k0, acc[j]));
      }
    }
#pragma unroll
    for (int j = 0; j < kMaxG; ++j)
      if (j < g) s_p[t][j] = acc[j] * score_scale;
  }
  __syncthreads();

  // ---- per head: maximum, probabilities, their sum (16 lanes per head) ----
  {
    const int j = tid >> 4, l16 = tid & 15;
    double mx = -INFINITY;
    if (j < g)
      for (int t = l16; t < vis; t += 16) mx = fmax(mx, s_p[t][j]);
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) mx = fmax(mx, __shfl_xor(mx, off, 16));
    double sum = 0.0;
    if (j < g)
      for (int t = l16; t < vis; t += 16) {
        const double x = s_p[t][j] - mx;
        const double p = base2 ? exp2(x) : exp(x);
        s_p[t][j] = p;
        sum += p;
      }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 16);
    if (j < g && l16 == 0) {
      s_m[j] = mx;
      s_l[j] = sum;
    }
  }
  __syncthreads();

  // ---- values: thread (channel d, heads 8*half .. 8*half + 7) ----
  const int d = tid & (kDim - 1);
  const int half = tid >> 7;
  double o[8];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) o[jj] = 0.0;
  const uint16_t *vbase = tail_v + (static_cast<size_t>(req) * tail_cap * s.heads + h) * kDim + d;
  for (int t = 0; t < vis; ++t) {
    const double v = bf16_to_double(vbase[t * row_stride]);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = 8 * half + jj;
      if (j < g) o[jj] = fma(s_p[t][j], v, o[jj]);
    }
  }

  TailPartials pt = tail_partials_of(ws, s);
  const size_t row0 = (static_cast<size_t>(bh) * s.parts + s.splits) * g;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int j = 8 * half + jj;
    if (j < g) pt.o[(row0 + j) * kDim + d] = static_cast<float>(o[jj]);
  }
  if (tid < g) {
    pt.m[row0 + tid] = s_m[tid];  // -inf when the token sees no tail token
    pt.l[row0 + tid] = static_cast<float>(s_l[tid]);
  }
}

}  // namespace

hipError_t launch_attention_tail_part(const uint16_t *q, const uint16_t *tail_k,
                                      const uint16_t *tail_v, const int32_t *tail_len,
                                      int tail_cap, const AttnShape &s, float sm_scale, bool base2,
                                      void *workspace, hipStream_t stream) {
  if (s.batch == 0) return hipSuccess;
  if (tail_cap < 1 || tail_cap > kTailCap || s.group > kMaxG) return hipErrorInvalidValue;
  const double scale = base2 ? static_cast<double>(sm_scale) * 1.4426950408889634074
                             : static_cast<double>(sm_scale);
  const dim3 grid(static_cast<unsigned>(static_cast<long long>(s.batch) * s.heads));
  hipLaunchKernelGGL(attn_tail_kernel, grid, dim3(kTailThreads), 0, stream, q, tail_k, tail_v,
                     tail_len, s, tail_cap, scale, base2, workspace);
  return hipGetLastError();
}

}  // namespace lynx
