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
// Products of bf16 values are exact in fp64 and the score sums run in fp64,
// as does the running maximum.  The exponentials (of fp64 differences
// rounded to fp32), the probability sums and the value sums run in fp32:
// their rounding reaches the output only through the softmax weights, a
// convex combination (the page kernels' value operands keep 22 bits).
#include <math.h>

#include "lynx_internal.h"

namespace lynx {
namespace {

constexpr int kTailThreads = 512;
constexpr int kTailCap = LYNX_TAIL_TOKENS;
constexpr int kMaxG = LYNX_MAX_GROUP;
static_assert(kMaxG <= 4 * (kTailThreads / 64), "four heads per wave at most");

// (m, l, o) partial rows, laid out as the page kernels lay them out:
// m fp64 [n], l fp32 [n], o fp32 [n][128], n = rows * H * parts * group
using TailPartials = AttnPartials;

__device__ __forceinline__ TailPartials tail_partials_of(void *ws, const AttnShape &s) {
  return attn_partials(ws, s);
}

__device__ __forceinline__ double bf16_to_double(uint32_t bits16) {
  return static_cast<double>(__uint_as_float(bits16 << 16));
}

// Tail tokens staged in LDS per pass: 64 tokens x 128 bf16.  K rows are
// padded by 16 bytes so that lanes reading different tokens at one channel
// hit different banks; every lane reads the same V row at once, so V rows
// are not padded.
constexpr int kSlab = 64;
constexpr int kKRow = kDim + 8;
constexpr int kWaves = kTailThreads / 64;

__device__ __forceinline__ double wave_max_d(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Block = (query row b, KV head h), eight waves; wave w owns the query heads
// w, w + 8, ... of the group (kHpw of them).  Per slab of 64 visible tail
// tokens the whole block stages K and V in LDS with one round of 16-byte
// loads (q with the first slab), then each wave works alone: lane t scores
// token t against its heads, the wave reduces the maximum and the sum of the
// exponentials (an online softmax across slabs), and lane c accumulates
// channels 2c, 2c + 1 of the value sums, reading each token's probability
// from the lane that holds it.
template <int kHpw>
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
  const int lane = tid & 63;
  const int wave = tid >> 6;

  __shared__ double s_q[kWaves * kHpw][kDim];  // head j at row j (zero past g)
  __shared__ __align__(16) uint16_t s_k[kSlab * kKRow];
  __shared__ __align__(16) uint16_t s_v[kSlab * kDim];

  // q: 16-byte pieces e = tid, tid + 512, ... (16 per head, heads of the
  // group contiguous in the row)
  constexpr int kQPieces = kWaves * kHpw * (kDim / 8);
  constexpr int kQPer = (kQPieces + kTailThreads - 1) / kTailThreads;
  const uint16_t *qrow = q + (static_cast<size_t>(b) * s.q_heads + static_cast<size_t>(h) * g) * kDim;
  uint4 qp[kQPer];
#pragma unroll
  for (int k = 0; k < kQPer; ++k) {
    const int e = tid + k * kTailThreads;
    qp[k] = e < kQPieces && (e >> 4) < g ? *reinterpret_cast<const uint4 *>(qrow + 8 * e)
                                         : make_uint4(0u, 0u, 0u, 0u);
  }

  const size_t row_stride = static_cast<size_t>(s.heads) * kDim;  // one token of the tail
  const size_t tail0 = (static_cast<size_t>(req) * tail_cap * s.heads + h) * kDim;

  // K and V pieces e = tid + 512 k of a slab: token e / 16, channels
  // 8 (e % 16) .. 8 (e % 16) + 7; rows from `rows` on are zero
  constexpr int kPer = kSlab * (kDim / 8) / kTailThreads;
  uint4 kp[kPer], vp[kPer];
  auto load_slab = [&](int t0, int rows) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int e = tid + k * kTailThreads;
      const int tk = e >> 4;
      const size_t at = tail0 + static_cast<size_t>(t0 + tk) * row_stride + (e & 15) * 8;
      kp[k] = tk < rows ? *reinterpret_cast<const uint4 *>(tail_k + at) : make_uint4(0u, 0u, 0u, 0u);
      vp[k] = tk < rows ? *reinterpret_cast<const uint4 *>(tail_v + at) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  // The first slab is requested before the tail length is known: its rows
  // below min(64, tail_cap) lie in this request's tail, and rows past the
  // visible count are never used (their scores are replaced by -inf and
  // their values are not read).
  load_slab(0, tail_cap < kSlab ? tail_cap : kSlab);

  int n = tail_len[req];
  n = n < 0 ? 0 : (n > tail_cap ? tail_cap : n);
  int vis = n - s.tq + i + 1;  // tail tokens this query token sees
  vis = vis < 0 ? 0 : (vis > n ? n : vis);

  double m_run[kHpw];
  float l_run[kHpw], o[kHpw][2];
#pragma unroll
  for (int hh = 0; hh < kHpw; ++hh) {
    m_run[hh] = -INFINITY;
    l_run[hh] = 0.0f;
    o[hh][0] = o[hh][1] = 0.0f;
  }

  for (int t0 = 0; t0 < vis; t0 += kSlab) {
    const int cnt = vis - t0 < kSlab ? vis - t0 : kSlab;
    if (t0 > 0) {
      load_slab(t0, cnt);
      __syncthreads();  // the previous slab consumed
    } else {
#pragma unroll
      for (int k = 0; k < kQPer; ++k) {
        const int e = tid + k * kTailThreads;
        if (e < kQPieces) {
          const uint32_t w4[4] = {qp[k].x, qp[k].y, qp[k].z, qp[k].w};
          double *dst = &s_q[e >> 4][8 * (e & 15)];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            dst[2 * c] = bf16_to_double(w4[c] & 0xFFFFu);
            dst[2 * c + 1] = bf16_to_double(w4[c] >> 16);
          }
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int e = tid + k * kTailThreads;
      *reinterpret_cast<uint4 *>(s_k + (e >> 4) * kKRow + (e & 15) * 8) = kp[k];
      *reinterpret_cast<uint4 *>(s_v + (e >> 4) * kDim + (e & 15) * 8) = vp[k];
    }
    __syncthreads();
    if (wave >= g) continue;  // no head of the group in this wave (uniform)

    // ---- scores: lane t against token t (only lanes t < cnt count) ----
    double acc[kHpw][2];
#pragma unroll
    for (int hh = 0; hh < kHpw; ++hh) acc[hh][0] = acc[hh][1] = 0.0;
    const uint16_t *krow = s_k + lane * kKRow;
#pragma unroll 2
    for (int d8 = 0; d8 < kDim / 8; ++d8) {
      const uint4 w = *reinterpret_cast<const uint4 *>(krow + 8 * d8);
      const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
      double kv[8];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        kv[2 * c] = bf16_to_double(w4[c] & 0xFFFFu);
        kv[2 * c + 1] = bf16_to_double(w4[c] >> 16);
      }
#pragma unroll
      for (int hh = 0; hh < kHpw; ++hh) {
        const double *qj = &s_q[wave + kWaves * hh][8 * d8];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[hh][d8 & 1] = fma(qj[c], kv[c], acc[hh][d8 & 1]);
      }
    }

    // ---- online softmax over the slab, then the value sums ----
    // exponent in base 2: fp64 difference (times log2 e for natural-base
    // scores) rounded to fp32
    constexpr double kLog2e = 1.4426950408889634074;
    auto exp_of = [&](double d) {
      return __builtin_amdgcn_exp2f(static_cast<float>(base2 ? d : d * kLog2e));
    };
    float p[kHpw];
#pragma unroll
    for (int hh = 0; hh < kHpw; ++hh) {
      const double x = lane < cnt ? (acc[hh][0] + acc[hh][1]) * score_scale : -INFINITY;
      const double m_new = fmax(m_run[hh], wave_max_d(x));  // finite: cnt >= 1
      const float alpha = exp_of(m_run[hh] - m_new);          // 0 on the first slab
      p[hh] = lane < cnt ? exp_of(x - m_new) : 0.0f;
      l_run[hh] = l_run[hh] * alpha + wave_sum_f(p[hh]);
      m_run[hh] = m_new;
      o[hh][0] *= alpha;
      o[hh][1] *= alpha;
    }
    for (int t = 0; t < cnt; ++t) {
      const uint32_t v2 = *reinterpret_cast<const uint32_t *>(s_v + t * kDim + 2 * lane);
      const float v0 = __uint_as_float(v2 << 16), v1 = __uint_as_float(v2 & 0xFFFF0000u);
#pragma unroll
      for (int hh = 0; hh < kHpw; ++hh) {
        const float pt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p[hh]), t));
        o[hh][0] = __builtin_fmaf(pt, v0, o[hh][0]);
        o[hh][1] = __builtin_fmaf(pt, v1, o[hh][1]);
      }
    }
  }

  TailPartials pt = tail_partials_of(ws, s);
  const size_t row0 = (static_cast<size_t>(bh) * s.parts + s.splits) * g;
#pragma unroll
  for (int hh = 0; hh < kHpw; ++hh) {
    const int j = wave + kWaves * hh;
    if (j < g) {
      reinterpret_cast<float2 *>(pt.o + (row0 + j) * kDim)[lane] = make_float2(o[hh][0], o[hh][1]);
      if (lane == 0) {
        pt.m[row0 + j] = m_run[hh];  // -inf when the token sees no tail token
        pt.l[row0 + j] = l_run[hh];
      }
    }
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
  if (s.group <= kWaves)
    hipLaunchKernelGGL(attn_tail_kernel<1>, grid, dim3(kTailThreads), 0, stream, q, tail_k,
                       tail_v, tail_len, s, tail_cap, scale, base2, workspace);
  else if (s.group <= 2 * kWaves)
    hipLaunchKernelGGL(attn_tail_kernel<2>, grid, dim3(kTailThreads), 0, stream, q, tail_k,
                       tail_v, tail_len, s, tail_cap, scale, base2, workspace);
  else
    hipLaunchKernelGGL(attn_tail_kernel<4>, grid, dim3(kTailThreads), 0, stream, q, tail_k,
                       tail_v, tail_len, s, tail_cap, scale, base2, workspace);
  return hipGetLastError();
}

}  // namespace lynx
