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

// Tail tokens staged in LDS per pass: 64 tokens x 128 bf16, rows padded by
// 16 bytes so that lanes reading different tokens at one channel hit
// different banks.
constexpr int kSlab = 64;
constexpr int kSlabRow = kDim + 8;
// q rows in LDS are padded by 16 bytes, so lanes reading different heads'
// rows at one channel hit different banks.
constexpr int kQStride = kDim + 2;

// Block = (query row b, KV head h).  The visible tail tokens pass through
// LDS in slabs of 64 (K for the scores, then V for the values), each slab
// loaded by the whole block with 16-byte loads at once.
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

  __shared__ double s_q[kMaxG * kQStride];
  __shared__ double s_p[kTailCap][kMaxG];  // scores, then probabilities
  __shared__ double s_m[kMaxG], s_l[kMaxG];
  __shared__ __align__(16) uint16_t s_slab[kSlab * kSlabRow];

  int n = tail_len[req];
  n = n < 0 ? 0 : (n > tail_cap ? tail_cap : n);
  int vis = n - s.tq + i + 1;  // tail tokens this query token sees
  vis = vis < 0 ? 0 : (vis > n ? n : vis);

  for (int e = tid; e < g * kDim; e += kTailThreads) {
    const int j = e / kDim, d = e % kDim;
    s_q[j * kQStride + d] =
        bf16_to_double(q[(static_cast<size_t>(b) * s.q_heads + h * g + j) * kDim + d]);
  }

  const size_t row_stride = static_cast<size_t>(s.heads) * kDim;  // one token of the tail
  const size_t tail0 = (static_cast<size_t>(req) * tail_cap * s.heads + h) * kDim;
  // slab of tokens t0 .. t0 + 63 (< vis) of one tail tensor into s_slab:
  // thread tid loads 16-byte pieces tid, tid + 256, ... (16 per token)
  auto stage = [&](const uint16_t *tail, int t0) {
    const int cnt = vis - t0 < kSlab ? vis - t0 : kSlab;
    uint4 piece[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = tid + k * kTailThreads;  // piece e: token e / 16, channels 8 (e % 16) ..
      const int tk = e >> 4;
      piece[k] = tk < cnt ? *reinterpret_cast<const uint4 *>(
                                tail + tail0 + static_cast<size_t>(t0 + tk) * row_stride + (e & 15) * 8)
                          : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = tid + k * kTailThreads;
      *reinterpret_cast<uint4 *>(s_slab + (e >> 4) * kSlabRow + (e & 15) * 8) = piece[k];
    }
    return cnt;
  };

  // ---- scores: 4 tail tokens of one head per thread and pass (each q
  // value read from LDS serves 4 products) ----
  for (int t0 = 0; t0 < vis; t0 += kSlab) {
    __syncthreads();  // q staged / the previous slab consumed
    const int cnt = stage(tail_k, t0);
    __syncthreads();
    const int groups = (cnt + 3) >> 2;  // tokens past cnt are zero in the slab
    for (int item = tid; item < groups * g; item += kTailThreads) {
      const int tg = item / g, j = item - tg * g;
      const double *qj = s_q + j * kQStride;
      const uint16_t *k0 = s_slab + 4 * tg * kSlabRow;
      double a[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 2
      for (int d8 = 0; d8 < kDim / 8; ++d8) {
        uint32_t u[4][4];
#pragma unroll
        for (int tk = 0; tk < 4; ++tk) {
          const uint4 w = *reinterpret_cast<const uint4 *>(k0 + tk * kSlabRow + 8 * d8);
          u[tk][0] = w.x;
          u[tk][1] = w.y;
          u[tk][2] = w.z;
          u[tk][3] = w.w;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const double q0 = qj[8 * d8 + 2 * e], q1 = qj[8 * d8 + 2 * e + 1];
#pragma unroll
          for (int tk = 0; tk < 4; ++tk) {
            a[tk] = fma(q0, bf16_to_double(u[tk][e] & 0xFFFFu), a[tk]);
            a[tk] = fma(q1, bf16_to_double(u[tk][e] >> 16), a[tk]);
          }
        }
      }
#pragma unroll
      for (int tk = 0; tk < 4; ++tk)
        if (4 * tg + tk < cnt) s_p[t0 + 4 * tg + tk][j] = a[tk] * score_scale;
    }
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

  // ---- values: thread (channel d, heads half, half + 2, ...) ----
  const int d = tid & (kDim - 1);
  const int half = tid >> 7;
  double o[kMaxG / 2];
#pragma unroll
  for (int jj = 0; jj < kMaxG / 2; ++jj) o[jj] = 0.0;
  for (int t0 = 0; t0 < vis; t0 += kSlab) {
    __syncthreads();  // probabilities written / the previous slab consumed
    const int cnt = stage(tail_v, t0);
    __syncthreads();
    for (int tk = 0; tk < cnt; ++tk) {
      const double v = bf16_to_double(s_slab[tk * kSlabRow + d]);
#pragma unroll
      for (int jj = 0; jj < kMaxG / 2; ++jj) {
        const int j = half + 2 * jj;
        if (j < g) o[jj] = fma(s_p[t0 + tk][j], v, o[jj]);
      }
    }
  }
  __syncthreads();  // s_m, s_l of a row that sees no tail token

  TailPartials pt = tail_partials_of(ws, s);
  const size_t row0 = (static_cast<size_t>(bh) * s.parts + s.splits) * g;
#pragma unroll
  for (int jj = 0; jj < kMaxG / 2; ++jj) {
    const int j = half + 2 * jj;
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
