// Fused-dequant single-query GQA decode attention over Lynx planes.
//
// Page "Lynx: the KV cache does not have to arrive whole", section 4: the
// draft runs on the anchor stream alone, the refined pass on anchor and
// residual.  Page "LLM KV cache quantization", sections "The architecture"
// and "End-to-end flow": the compact cache is read in its stored form and
// expanded only in registers right before the score dot products and the
// value sum; attention itself is unchanged (scaled q.k, softmax, weighted
// sum of v).
//
// Algebra used so that no dequantized element is ever materialised:
//   khat_td = c0_cd + c1_cd * yhat_td,  c0 = mn + rg*mu, c1 = rg*s  (per
//   chunk c, channel d), hence for query head j
//   score_tj = sum_d (sm*q_jd*c1_cd) yhat_td + sum_d sm*q_jd*c0_cd
//            = dot(q'_cj, yhat_t) + bias_cj
//   and o_jd = sum_c [c1v_cd * sum_{t in c} p_tj yhat_td + c0v_cd * sum_{t in c} p_tj].
// q' = q * rg * s is formed in fp64 (bf16 q times the fp32 scales), the dot
// product with the fp32 yhat runs in fp64, and the bias and the softmax
// scale are applied in fp64, so no score is rounded to fp32 at its full
// magnitude (with 100x outlier channels scores reach a few hundred).
//
// Split-K: each workgroup reduces a contiguous run of pages of one (request,
// KV head) to (m, l, o) partials; a combine kernel merges them exactly.
#include <math.h>

#include "lynx_internal.h"

namespace lynx {
namespace {

constexpr int kAttnThreads = 256;
constexpr int kMaxG = LYNX_MAX_GROUP;
constexpr int kTargetBlocks = 2048;  // VALU kernel (group > 8)
// splits per (request, KV head) never exceed the block target (see
// attention_shape), which bounds the combine kernel's weight array
constexpr int kMaxSplits = kTargetBlocks;
constexpr int kCombineThreads = 256;
constexpr int kCombineParts = 4;  // the combine splits the head dimension into 4 x 32 channels

struct YTable {
  float y[256];
};

__device__ __forceinline__ int chunk_token(int w, int j) {
  return j < 4 ? 4 * w + j : 16 + 4 * w + (j - 4);
}

__device__ __forceinline__ int table_index(uint32_t a_nib, uint32_t r_nib) {
  return static_cast<int>(((a_nib << 4) | r_nib) ^ 0x80u);
}

using Partials = AttnPartials;

__device__ __forceinline__ Partials partials_of(void *ws, const AttnShape &s) {
  return attn_partials(ws, s);
}

template <bool kFull>
__global__ __launch_bounds__(kAttnThreads) void attn_split_kernel(
    const uint16_t *__restrict__ q, PlanesArg kp, PlanesArg vp,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens,
    AttnShape s, float sm_scale, float *__restrict__ scores, void *ws,
    YTable tab) {
  const int split = blockIdx.x % s.splits;
  const int bh = blockIdx.x / s.splits;
  const int h = bh % s.heads;
  const int b = bh / s.heads;  // query row
  const int req = b / s.tq;     // its request
  const int g = s.group;
  const int tid = threadIdx.x;

  int npages = s.max_pages;
  if (seq_lens) {
    npages = seq_lens[req] / kPage;
    npages = npages < 0 ? 0 : (npages > s.max_pages ? s.max_pages : npages);
  }
  const int p0 = split * s.pages_per_split;
  int p1 = p0 + s.pages_per_split;
  p1 = p1 > npages ? npages : p1;

  __shared__ double s_q[kMaxG][kDim];     // q (exact bf16 values)
  __shared__ double s_qp[kMaxG][kDim];    // q' = q * c1 (per chunk, fp64)
  __shared__ double s_c0k[kDim], s_c1k[kDim];
  __shared__ double s_c0v[kDim], s_c1v[kDim];
  __shared__ double s_bias[kMaxG];
  __shared__ double s_score[kChunk][kMaxG];
  __shared__ float s_p[kChunk][kMaxG];
  __shared__ float s_part[2][kMaxG][kDim];
  __shared__ double s_m[kMaxG];
  __shared__ float s_l[kMaxG], s_scale[kMaxG], s_psum[kMaxG];
  __shared__ float s_y[256];

  s_y[tid] = tab.y[tid];
  for (int e = tid; e < g * kDim; e += kAttnThreads) {
    const int j = e / kDim, d = e % kDim;
    const uint16_t bits = q[(static_cast<size_t>(b) * s.q_heads + h * g + j) * kDim + d];
    s_q[j][d] = static_cast<double>(__uint_as_float(static_cast<uint32_t>(bits) << 16));
  }
  if (tid < kMaxG) {
    s_m[tid] = -INFINITY;
    s_l[tid] = 0.0f;
  }
  // value accumulators: thread (d, half) owns heads 8*half .. 8*half+7
  const int vd = tid & (kDim - 1);
  const int vhalf = tid >> 7;
  double acc[8];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) acc[jj] = 0.0;
  __syncthreads();

  const size_t T = static_cast<size_t>(s.max_pages) * kPage;
  for (int lp = p0; lp < p1; ++lp) {
    const long long pg = block_table ? block_table[static_cast<size_t>(req) * s.max_pages + lp]
                                     : static_cast<long long>(req) * s.max_pages + lp;
    if (pg < 0 || pg >= s.pool_pages) continue;  // invalid entry: page skipped
    const size_t tile = static_cast<size_t>(pg) * s.heads + h;
    for (int c = 0; c < kChunks; ++c) {
      // ---- per-chunk affine constants ----
      if (tid < kDim) {
        const int d = tid;
        const double mn = kp.page_min[tile * kDim + d];
        const double rg = kp.page_range[tile * kDim + d];
        const double mu = kp.chunk_mean[(tile * kChunks + c) * kDim + d];
        const double sc = kp.chunk_maxabs[(tile * kChunks + c) * kDim + d];
        s_c0k[d] = mn + rg * mu;
        s_c1k[d] = rg * sc;
      } else {
        const int d = tid - kDim;
        const double mn = vp.page_min[tile * kDim + d];
        const double rg = vp.page_range[tile * kDim + d];
        const double mu = vp.chunk_mean[(tile * kChunks + c) * kDim + d];
        const double sc = vp.chunk_maxabs[(tile * kChunks + c) * kDim + d];
        s_c0v[d] = mn + rg * mu;
        s_c1v[d] = rg * sc;
      }
      __syncthreads();
      for (int e = tid; e < g * kDim; e += kAttnThreads) {
        const int j = e / kDim, d = e % kDim;
        s_qp[j][d] = s_q[j][d] * s_c1k[d];
      }
      {
        const int j = tid >> 4, part = tid & 15;
        double bsum = 0.0;
        if (j < g) {
#pragma unroll
          for (int k = 0; k < 8; ++k) bsum += s_q[j][part * 8 + k] * s_c0k[part * 8 + k];
        }
        bsum += __shfl_xor(bsum, 1);
        bsum += __shfl_xor(bsum, 2);
        bsum += __shfl_xor(bsum, 4);
        bsum += __shfl_xor(bsum, 8);
        if (j < g && part == 0) s_bias[j] = bsum;
      }
      __syncthreads();

      // ---- scores: thread (token t, 16 channels) ----
      {
        const int t = tid >> 3;
        const int cg = tid & 7;
        const size_t w = (tile * kPage + c * kChunk + t) * 16 + cg * 2;
        const uint2 a2 = reinterpret_cast<const uint2 *>(kp.anchor)[w / 2];
        const uint2 r2 = kFull ? reinterpret_cast<const uint2 *>(kp.residual)[w / 2]
                               : make_uint2(0x77777777u, 0x77777777u);
        float y[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          y[i] = s_y[table_index((a2.x >> (4 * i)) & 15u, (r2.x >> (4 * i)) & 15u)];
          y[8 + i] = s_y[table_index((a2.y >> (4 * i)) & 15u, (r2.y >> (4 * i)) & 15u)];
        }
        for (int j = 0; j < g; ++j) {
          // fp32 operands, fp64 accumulation: every product is exact and the
          // sum is never rounded at the score's magnitude in fp32
          double dot = 0.0;
#pragma unroll
          for (int i = 0; i < 16; ++i)
            dot = fma(s_qp[j][cg * 16 + i], static_cast<double>(y[i]), dot);
          dot += __shfl_xor(dot, 1);
          dot += __shfl_xor(dot, 2);
          dot += __shfl_xor(dot, 4);
          if (cg == 0) {
            const double sc = (dot + s_bias[j]) * static_cast<double>(sm_scale);
            s_score[t][j] = sc;
            if (scores)
              scores[(static_cast<size_t>(b) * s.q_heads + h * g + j) * T +
                     static_cast<size_t>(lp) * kPage + c * kChunk + t] = static_cast<float>(sc);
          }
        }
      }
      __syncthreads();

      // ---- online softmax ----
      if (tid < g) {
        const int j = tid;
        double cm = s_score[0][j];
        for (int t = 1; t < kChunk; ++t) cm = fmax(cm, s_score[t][j]);
        const double mold = s_m[j];
        const double mnew = fmax(mold, cm);
        s_scale[j] = static_cast<float>(exp(mold - mnew));
        s_m[j] = mnew;
      }
      __syncthreads();
      for (int e = tid; e < kChunk * g; e += kAttnThreads) {
        const int t = e / g, j = e % g;
        s_p[t][j] = expf(static_cast<float>(s_score[t][j] - s_m[j]));
      }
      __syncthreads();
      if (tid < g) {
        const int j = tid;
        float ps = 0.0f;
        for (int t = 0; t < kChunk; ++t) ps += s_p[t][j];
        s_psum[j] = ps;
        s_l[j] = s_l[j] * s_scale[j] + ps;
      }

      // ---- values: thread (channel d, 16 tokens) ----
      {
        const size_t w = ((tile * kChunks + c) * kDim + vd) * 4 + vhalf * 2;
        const uint2 a2 = reinterpret_cast<const uint2 *>(vp.anchor)[w / 2];
        const uint2 r2 = kFull ? reinterpret_cast<const uint2 *>(vp.residual)[w / 2]
                               : make_uint2(0x77777777u, 0x77777777u);
        float part[kMaxG];
#pragma unroll
        for (int j = 0; j < kMaxG; ++j) part[j] = 0.0f;
#pragma unroll
        for (int ww = 0; ww < 2; ++ww) {
          const uint32_t aw = ww ? a2.y : a2.x;
          const uint32_t rw = ww ? r2.y : r2.x;
#pragma unroll
          for (int jn = 0; jn < 8; ++jn) {
            const float y = s_y[table_index((aw >> (4 * jn)) & 15u, (rw >> (4 * jn)) & 15u)];
            const int t = chunk_token(vhalf * 2 + ww, jn);
#pragma unroll
            for (int j = 0; j < kMaxG; ++j)
              if (j < g) part[j] = __builtin_fmaf(s_p[t][j], y, part[j]);
          }
        }
#pragma unroll
        for (int j = 0; j < kMaxG; ++j)
          if (j < g) s_part[vhalf][j][vd] = part[j];
      }
      __syncthreads();
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int j = vhalf * 8 + jj;
        if (j < g) {
          const double tot = static_cast<double>(s_part[0][j][vd]) + s_part[1][j][vd];
          acc[jj] = acc[jj] * s_scale[j] + s_c1v[vd] * tot + s_c0v[vd] * static_cast<double>(s_psum[j]);
        }
      }
      __syncthreads();
    }
  }

  // ---- write (m, l, o) partials ----
  Partials pt = partials_of(ws, s);
  const size_t base = (static_cast<size_t>(bh) * s.parts + split) * g;
  if (tid < g) {
    pt.m[base + tid] = s_m[tid];
    pt.l[base + tid] = s_l[tid];
  }
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int j = vhalf * 8 + jj;
    if (j < g) pt.o[(base + j) * kDim + vd] = static_cast<float>(acc[jj]);
  }
}

// Exact merge of the (m, l, o) partials of every split of one (request, KV
// head), for one query head and 32 of its channels per block:
//   M = max m_s,  w_s = exp(m_s - M),  out = sum_s w_s o_s / sum_s w_s l_s.
// The weights are computed once into LDS; 32 groups of 8 threads then sum
// float4 slices of the o partials of every 32nd split (four loads in flight
// per thread), in fp64, and one last pass adds the 32 group sums.
__device__ __forceinline__ double block_reduce(double v, bool is_max, double *s_red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const double o = __shfl_xor(v, off);
    v = is_max ? fmax(v, o) : v + o;
  }
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_red[w] = v;
  __syncthreads();
  v = s_red[0];
#pragma unroll
  for (int k = 1; k < kCombineThreads / 64; ++k) v = is_max ? fmax(v, s_red[k]) : v + s_red[k];
  return v;
}

__global__ __launch_bounds__(kCombineThreads) void attn_combine_kernel(AttnShape s, const void *ws,
                                                                        float *__restrict__ out) {
  const int bj = blockIdx.x / kCombineParts;  // b * Hq + query head
  const int part = blockIdx.x % kCombineParts;
  const int b = bj / s.q_heads;
  const int jq = bj % s.q_heads;
  const int h = jq / s.group;
  const int j = jq % s.group;
  const int tid = threadIdx.x;
  Partials pt = partials_of(const_cast<void *>(ws), s);
  const size_t first = (static_cast<size_t>(b) * s.heads + h) * s.parts;
  __shared__ float s_w[kMaxSplits + 1];
  __shared__ double s_red[kCombineThreads / 64];
  __shared__ double s_o[32][33];

  double M = -INFINITY;
  for (int sp = tid; sp < s.parts; sp += kCombineThreads)
    M = fmax(M, pt.m[(first + sp) * s.group + j]);
  M = block_reduce(M, true, s_red);
  double L = 0.0;
  for (int sp = tid; sp < s.parts; sp += kCombineThreads) {
    const size_t r = (first + sp) * s.group + j;
    const double m = pt.m[r];
    const float wgt = m == -INFINITY ? 0.0f : static_cast<float>(exp(m - M));
    s_w[sp] = wgt;
    L += static_cast<double>(wgt) * pt.l[r];
  }
  L = block_reduce(L, false, s_red);  // its barriers also publish s_w

  const int c4 = tid & 7;   // float4 slice of the block's 32 channels
  const int sg = tid >> 3;  // split group 0..31
  const int d0 = part * 32 + 4 * c4;
  double o[4] = {0.0, 0.0, 0.0, 0.0};
  for (int sp0 = sg; sp0 < s.parts; sp0 += 4 * 32) {
    float4 v[4];
    float wk[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int sp = sp0 + 32 * u;
      const bool ok = sp < s.parts;
      wk[u] = ok ? s_w[sp] : 0.0f;
      v[u] = ok ? *reinterpret_cast<const float4 *>(pt.o + ((first + sp) * s.group + j) * kDim + d0)
                : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const double wd = wk[u];
      o[0] += wd * v[u].x;
      o[1] += wd * v[u].y;
      o[2] += wd * v[u].z;
      o[3] += wd * v[u].w;
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) s_o[sg][4 * c4 + e] = o[e];
  __syncthreads();
  if (tid < 32) {
    double O = 0.0;
#pragma unroll 8
    for (int g2 = 0; g2 < 32; ++g2) O += s_o[g2][tid];
    out[static_cast<size_t>(bj) * kDim + part * 32 + tid] = L > 0.0 ? static_cast<float>(O / L) : 0.0f;
  }
}

}  // namespace

// Pages per run: `units` work items (row and KV head, or row group) each
// split into runs so that at most `target` blocks cover the call whenever
// units <= target (a block per CU is one round: more blocks than that would
// start a second round for a few of them), and one run per unit beyond.
static long long run_pages(long long units, int max_pages, long long target) {
  if (max_pages < 1 || units < 1) return 1;
  const long long runs = units >= target ? 1 : target / units;  // >= 1
  long long pps = (max_pages + runs - 1) / runs;
  return pps < 1 ? 1 : (pps > max_pages ? max_pages : pps);
}

AttnShape attention_shape(int batch, int heads, int q_heads, int max_pages) {
  AttnShape s;
  s.batch = batch;
  s.tq = 1;
  s.heads = heads;
  s.q_heads = q_heads;
  s.group = heads > 0 ? q_heads / heads : 0;
  s.max_pages = max_pages;
  s.pool_pages = 0;
  const long long units = static_cast<long long>(batch) * heads;
  const long long target =
      attention_mfma_supported(s.group) ? attention_mfma_target_blocks() : kTargetBlocks;
  const long long pps = run_pages(units, max_pages, target);
  s.pages_per_split = static_cast<int>(pps);
  s.splits = max_pages > 0 ? static_cast<int>((max_pages + pps - 1) / pps) : 1;
  s.parts = s.splits;
  return s;
}

AttnShape attention_shape_tail(int requests, int tq, int heads, int q_heads, int max_pages) {
  AttnShape s = attention_shape(requests * tq, heads, q_heads, max_pages);
  s.tq = tq;
  if (verify_mfma_used(s.group, tq) && max_pages > 0) {
    // the verify kernel's blocks: (request, KV head, run, group of 16 or 32 rows)
    const long long units = static_cast<long long>(requests) * heads * verify_row_blocks(tq);
    const long long pps = run_pages(units, max_pages, attention_mfma_target_blocks());
    s.pages_per_split = static_cast<int>(pps);
    s.splits = static_cast<int>((max_pages + pps - 1) / pps);
  }
  s.parts = s.splits + 1;
  return s;
}

// Partials (m, l, o) of every split.
size_t attention_workspace_bytes(const AttnShape &s) {
  const size_t n = static_cast<size_t>(s.batch) * s.heads * s.parts * s.group;
  return ((n + 1) & ~static_cast<size_t>(1)) * sizeof(double) +
         ((n + 3) & ~static_cast<size_t>(3)) * sizeof(float) + n * kDim * sizeof(float);
}

hipError_t launch_attention(const uint16_t *q, const PlanesArg &k,
                            const PlanesArg &v, const int32_t *block_table,
                            const int32_t *seq_lens, const AttnShape &s,
                            float sm_scale, bool full, float *out,
                            float *scores, void *workspace,
                            hipStream_t stream, int anchor_bits) {
  if (s.batch == 0) return hipSuccess;
  if (attention_mfma_supported(s.group))
    return launch_attention_mfma(q, k, v, block_table, seq_lens, s, sm_scale, full, out, scores,
                                 workspace, true, stream, anchor_bits);
  if (anchor_bits != 4) return hipErrorInvalidValue;  // cut streams: matrix-core kernel only
  YTable tab;
  const DecodeTable &dt = decode_table();
  for (int i = 0; i < 256; ++i) tab.y[i] = dt.y[i];
  const dim3 grid(static_cast<unsigned>(static_cast<long long>(s.batch) * s.heads * s.splits));
  if (full)
    hipLaunchKernelGGL(attn_split_kernel<true>, grid, dim3(kAttnThreads), 0, stream, q, k, v,
                       block_table, seq_lens, s, sm_scale, scores, workspace, tab);
  else
    hipLaunchKernelGGL(attn_split_kernel<false>, grid, dim3(kAttnThreads), 0, stream, q, k, v,
                       block_table, seq_lens, s, sm_scale, scores, workspace, tab);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel,
                     dim3(static_cast<unsigned>(s.batch * s.q_heads * kCombineParts)),
                     dim3(kCombineThreads), 0, stream, s, static_cast<const void *>(workspace), out);
  return hipGetLastError();
}

hipError_t launch_attention_with_tail(const uint16_t *q, const PlanesArg &k, const PlanesArg &v,
                                      const int32_t *block_table, const int32_t *page_tokens,
                                      const uint16_t *tail_k, const uint16_t *tail_v,
                                      const int32_t *tail_len, int tail_cap, const AttnShape &s,
                                      float sm_scale, bool full, float *out, void *workspace,
                                      hipStream_t stream) {
  if (s.batch == 0) return hipSuccess;
  const bool mfma = attention_mfma_supported(s.group);
  AttnShape sp = s;
  hipError_t e;
  if (s.pool_pages <= 0) {
    // no page can be read: the tail is the whole context
    sp.splits = 0;
    sp.parts = 1;
  } else if (verify_mfma_used(s.group, s.tq)) {
    e = launch_verify_mfma(q, k, v, block_table, page_tokens, sp, sm_scale, full, workspace, stream);
    if (e != hipSuccess) return e;
  } else if (mfma) {
    e = launch_attention_mfma(q, k, v, block_table, page_tokens, sp, sm_scale, full, out, nullptr,
                              workspace, false, stream);
    if (e != hipSuccess) return e;
  } else {
    YTable tab;
    const DecodeTable &dt = decode_table();
    for (int i = 0; i < 256; ++i) tab.y[i] = dt.y[i];
    const dim3 grid(static_cast<unsigned>(static_cast<long long>(sp.batch) * sp.heads * sp.splits));
    if (full)
      hipLaunchKernelGGL(attn_split_kernel<true>, grid, dim3(kAttnThreads), 0, stream, q, k, v,
                         block_table, page_tokens, sp, sm_scale, nullptr, workspace, tab);
    else
      hipLaunchKernelGGL(attn_split_kernel<false>, grid, dim3(kAttnThreads), 0, stream, q, k, v,
                         block_table, page_tokens, sp, sm_scale, nullptr, workspace, tab);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  e = launch_attention_tail_part(q, tail_k, tail_v, tail_len, tail_cap, sp, sm_scale, mfma,
                                 workspace, stream);
  if (e != hipSuccess) return e;
  if (mfma) return launch_attention_mfma_combine(sp, workspace, out, stream);
  hipLaunchKernelGGL(attn_combine_kernel,
                     dim3(static_cast<unsigned>(sp.batch * sp.q_heads * kCombineParts)),
                     dim3(kCombineThreads), 0, stream, sp, static_cast<const void *>(workspace), out);
  return hipGetLastError();
}

}  // namespace lynx
