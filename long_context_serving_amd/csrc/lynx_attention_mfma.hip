// Fused-dequant single-query GQA decode attention on MFMA (GQA group <= 8).
//
// Page "Lynx: the KV cache does not have to arrive whole", section 4 (draft
// on the anchor stream, refinement on anchor + residual); page "LLM KV cache
// quantization", sections "The architecture" and "End-to-end flow" (read
// the compact cache, expand it only in registers, attention unchanged).
//
// Per (request, KV head), each wave streams 32-token chunks.  With
//   khat = c0 + c1*yhat, vhat = c0v + c1v*yhat   (c0 = mn + rg*mu, c1 = rg*s)
// a chunk needs two dense products that run on v_mfma_f32_16x16x32_f16:
//   S^T[16 tok][16 col] += Yk[16 tok][32 ch] * Q'[32 ch][16 col]  (4 K-steps)
//   O  [16 col][16 ch ] += P [16 col][32 tok] * Yv[32 tok][16 ch]
// yhat comes from a table as an fp16 pair hi + lo (22 bits).  The encoder
// keeps the page range and chunk max-abs with 7 significant bits, so
// q' = q * rg * s of a bf16 query has at most 22 bits and is split EXACTLY
// into two fp16 halves (after a per-chunk power-of-two scale that keeps it
// inside the fp16 range).  The 16 MFMA columns hold [Q'hi of the 8 heads |
// Q'lo of the 8 heads] (and likewise P), so running the Y side twice (hi,
// then lo, into separate accumulators) yields all four cross products.
// With 100x outlier channels scores reach a few hundred and the output is
// sensitive to one fp32 ulp of a score, so the score is never rounded to
// fp32 at its full magnitude: the large (hi x hi) part and the small parts,
// the fp64 chunk bias and the softmax shift are combined in fp64, and only
// the small difference to the running max is rounded before exp().
//
// Lane l of a wave: n = l % 16 (MFMA column / token / channel index), r = l /
// 16 (MFMA k-group).  Keys are token-major, so lane (n, r) of K-tile t reads
// the 16 bytes of channels 32r..32r+31 of token 16t + n; values are
// channel-major with the chunk's tokens permuted so that lane (n, r) reads
// the 4 bytes of word r of channel 16ct + n, which hold exactly the 8 tokens
// whose probabilities lane (n, r) produced on the score side.
#include <math.h>

#include "lynx_internal.h"

namespace lynx {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kLutCopies = 32;  // full table replicated per LDS bank

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

struct MfmaTables {
  uint32_t full[256];  // raw code byte (a << 4 | r) -> fp16 hi | fp16 lo << 16 of yhat
  uint32_t draft[16];  // anchor nibble -> fp16 hi | fp16 lo << 16 of the draft yhat
};

struct Partials {
  double *m;
  float *l;
  float *o;
};

__device__ __forceinline__ Partials partials_of(void *ws, const AttnShape &s) {
  const size_t n = static_cast<size_t>(s.batch) * s.heads * s.splits * s.group;
  Partials pt;
  pt.m = reinterpret_cast<double *>(ws);
  pt.l = reinterpret_cast<float *>(pt.m + ((n + 1) & ~static_cast<size_t>(1)));
  pt.o = pt.l + ((n + 3) & ~static_cast<size_t>(3));
  return pt;
}

// [a.lo16 | b.lo16 << 16] and [a.hi16 | b.hi16 << 16]
__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ half8 as_half8(const uint32_t (&u)[4]) {
  half8 h;
  __builtin_memcpy(&h, u, sizeof h);
  return h;
}

// 8 codes (nibble i of the anchor / residual words = element i) -> the hi and
// lo fp16 operand words of yhat for elements (2k, 2k+1) in word k.
__device__ __forceinline__ void decode8_full(uint32_t a, uint32_t r, const uint32_t *lut,
                                             uint32_t bank, uint32_t (&hi)[4],
                                             uint32_t (&lo)[4]) {
  const uint32_t even = ((a << 4) & 0xF0F0F0F0u) | (r & 0x0F0F0F0Fu);
  const uint32_t odd = (a & 0xF0F0F0F0u) | ((r >> 4) & 0x0F0F0F0Fu);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t e = lut[(((even >> (8 * k)) & 0xFFu) << 5) | bank];
    const uint32_t o = lut[(((odd >> (8 * k)) & 0xFFu) << 5) | bank];
    hi[k] = lo_halves(e, o);
    lo[k] = hi_halves(e, o);
  }
}

__device__ __forceinline__ void decode8_draft(uint32_t a, const uint2 *pairs, uint32_t (&hi)[4],
                                              uint32_t (&lo)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint2 v = pairs[(a >> (8 * k)) & 0xFFu];
    hi[k] = v.x;
    lo[k] = v.y;
  }
}

// fp16 bits of the hi part of x (round to nearest even) or of the remainder x - hi.
__device__ __forceinline__ uint32_t split_part(float x, bool want_lo) {
  const _Float16 h = static_cast<_Float16>(x);
  const float rem = x - static_cast<float>(h);
  const _Float16 l = static_cast<_Float16>(rem);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, want_lo ? l : h));
}

template <bool kFull>
__global__ __launch_bounds__(kThreads) void attn_mfma_kernel(
    const uint16_t *__restrict__ q, PlanesArg kp, PlanesArg vp,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens,
    AttnShape s, float sm_scale, float *__restrict__ scores, void *ws, MfmaTables tab) {
  const int split = blockIdx.x % s.splits;
  const int bh = blockIdx.x / s.splits;
  const int h = bh % s.heads;
  const int b = bh / s.heads;
  const int g = s.group;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 15;
  const int r = lane >> 4;
  const bool lo_col = n >= 8;
  const int head = n & 7;
  const uint32_t bank = static_cast<uint32_t>(lane & (kLutCopies - 1));

  // LDS: yhat tables (the full table is replicated once per bank so that a
  // wave's 32-lane halves never conflict), per-wave chunk scales, and the
  // end-of-block combine area (which reuses the table space).
  __shared__ __align__(16) uint32_t s_big[256 * kLutCopies];  // 32 KiB
  __shared__ __align__(16) uint2 s_pairs[256];
  __shared__ __align__(16) float s_sc[kWaves][3][kDim];      // c1k (scaled), c1v, c0v
  __shared__ __align__(16) double s_c0k[kWaves][kDim];       // c0k = mn + rg * mu (exact)
  __shared__ float s_ml[kWaves][2][8];

  if (kFull) {
    for (int i = tid; i < 256 * kLutCopies; i += kThreads) s_big[i] = tab.full[i >> 5];
  } else {
    const uint32_t lo = tab.draft[tid & 15], hi = tab.draft[tid >> 4];
    s_pairs[tid] = make_uint2(lo_halves(lo, hi), hi_halves(lo, hi));
  }

  int npages = s.max_pages;
  if (seq_lens) {
    npages = seq_lens[b] / kPage;
    npages = npages < 0 ? 0 : (npages > s.max_pages ? s.max_pages : npages);
  }
  const int p0 = split * s.pages_per_split;
  int p1 = p0 + s.pages_per_split;
  p1 = p1 > npages ? npages : p1;

  // q (exact bf16 values) for this lane's head, channels 32r .. 32r+31;
  // sm_scale is applied in fp64 when the score is assembled
  float qv[32];
  float qmax = 0.0f;
  {
    const bool valid = head < g;
    const uint16_t *qrow = q + (static_cast<size_t>(b) * s.q_heads + h * g + (valid ? head : 0)) * kDim + 32 * r;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint4 v = reinterpret_cast<const uint4 *>(qrow)[k];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qv[8 * k + 2 * e] = valid ? __uint_as_float(u[e] << 16) : 0.0f;
        qv[8 * k + 2 * e + 1] = valid ? __uint_as_float(u[e] & 0xFFFF0000u) : 0.0f;
      }
    }
#pragma unroll
    for (int k = 0; k < 32; ++k) qmax = fmaxf(qmax, fabsf(qv[k]));
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) qmax = fmaxf(qmax, __shfl_xor(qmax, off));
  }
  const double sm64 = static_cast<double>(sm_scale);

  float m_run = -INFINITY, l_run = 0.0f;
  floatx4 acc[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) acc[ct] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  __syncthreads();

  const size_t T = static_cast<size_t>(s.max_pages) * kPage;
  const int c_begin = p0 * kChunks, c_end = p1 * kChunks;
  float *sc = &s_sc[w][0][0];
  for (int ci = c_begin + w; ci < c_end; ci += kWaves) {
    const int lp = ci >> 3;
    const int c = ci & 7;
    const int pg = block_table ? block_table[static_cast<size_t>(b) * s.max_pages + lp]
                               : b * s.max_pages + lp;
    if (pg < 0 || pg >= s.pool_pages) continue;  // invalid entry: page skipped (wave-uniform)
    const size_t tile = static_cast<size_t>(pg) * s.heads + h;

    // ---- code loads (issued first) ----
    const uint4 *kan = reinterpret_cast<const uint4 *>(kp.anchor);
    const uint4 *kre = reinterpret_cast<const uint4 *>(kp.residual);
    uint4 ka[2], kr[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const size_t idx = (tile * kPage + c * kChunk + 16 * t + n) * 4 + r;
      ka[t] = kan[idx];
      kr[t] = kFull ? kre[idx] : make_uint4(0, 0, 0, 0);
    }
    const uint32_t *van = reinterpret_cast<const uint32_t *>(vp.anchor);
    const uint32_t *vre = reinterpret_cast<const uint32_t *>(vp.residual);
    uint32_t va[8], vr[8];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const size_t idx = ((tile * kChunks + c) * kDim + 16 * ct + n) * 4 + r;
      va[ct] = van[idx];
      vr[ct] = kFull ? vre[idx] : 0u;
    }

    // ---- chunk affine constants: lane handles channels 2l, 2l+1 ----
    // c1 = rg * s is exact (7 + 7 significant bits); it is scaled by a power
    // of two chosen so that every q * c1 stays inside the fp16 range.
    float kscale;
    {
      const size_t pidx = tile * (kDim / 2) + lane;
      const size_t cidx = (tile * kChunks + c) * (kDim / 2) + lane;
      const float2 mnk = reinterpret_cast<const float2 *>(kp.page_min)[pidx];
      const float2 rgk = reinterpret_cast<const float2 *>(kp.page_range)[pidx];
      const float2 muk = reinterpret_cast<const float2 *>(kp.chunk_mean)[cidx];
      const float2 sk = reinterpret_cast<const float2 *>(kp.chunk_maxabs)[cidx];
      const float2 mnv = reinterpret_cast<const float2 *>(vp.page_min)[pidx];
      const float2 rgv = reinterpret_cast<const float2 *>(vp.page_range)[pidx];
      const float2 muv = reinterpret_cast<const float2 *>(vp.chunk_mean)[cidx];
      const float2 sv = reinterpret_cast<const float2 *>(vp.chunk_maxabs)[cidx];
      const float c1a = rgk.x * sk.x, c1b = rgk.y * sk.y;
      float cmax = fmaxf(c1a, c1b);
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) cmax = fmaxf(cmax, __shfl_xor(cmax, off));
      // largest |q'| <= qmax * cmax; keep it below 2^15
      const float bound = qmax * cmax;
      kscale = 1.0f;
      if (bound >= 16384.0f) {
        const int e = static_cast<int>((__float_as_uint(bound) >> 23) & 0xFFu) - 127;  // >= 14
        kscale = __uint_as_float(static_cast<uint32_t>(127 + 13 - e) << 23);
      }
      reinterpret_cast<float2 *>(sc + 0 * kDim)[lane] = make_float2(c1a * kscale, c1b * kscale);
      reinterpret_cast<float2 *>(sc + 1 * kDim)[lane] = make_float2(rgv.x * sv.x, rgv.y * sv.y);
      reinterpret_cast<float2 *>(sc + 2 * kDim)[lane] =
          make_float2(__builtin_fmaf(rgv.x, muv.x, mnv.x), __builtin_fmaf(rgv.y, muv.y, mnv.y));
      reinterpret_cast<double2 *>(&s_c0k[w][0])[lane] =
          make_double2(static_cast<double>(mnk.x) + static_cast<double>(rgk.x) * muk.x,
                       static_cast<double>(mnk.y) + static_cast<double>(rgk.y) * muk.y);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- Q' operand (exact halves: hi in columns 0..7, lo in 8..15) ----
    half8 bq[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const float4 c1a = reinterpret_cast<const float4 *>(sc + 0 * kDim + 32 * r + 8 * st)[0];
      const float4 c1b = reinterpret_cast<const float4 *>(sc + 0 * kDim + 32 * r + 8 * st)[1];
      const float c1[8] = {c1a.x, c1a.y, c1a.z, c1a.w, c1b.x, c1b.y, c1b.z, c1b.w};
      uint32_t u[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float x0 = qv[8 * st + 2 * k] * c1[2 * k];
        const float x1 = qv[8 * st + 2 * k + 1] * c1[2 * k + 1];
        u[k] = split_part(x0, lo_col) | (split_part(x1, lo_col) << 16);
      }
      bq[st] = as_half8(u);
    }
    // ---- chunk bias sum_d q_d c0_d in fp64 (lanes n and n+8 take 16 channels each) ----
    double bias;
    {
      const double *c0 = &s_c0k[w][32 * r + (lo_col ? 16 : 0)];
      double acc0 = 0.0, acc1 = 0.0;
#pragma unroll
      for (int k = 0; k < 16; k += 2) {
        const double2 cc = reinterpret_cast<const double2 *>(c0)[k / 2];
        const float qa = lo_col ? qv[16 + k] : qv[k];
        const float qb = lo_col ? qv[17 + k] : qv[k + 1];
        acc0 = fma(static_cast<double>(qa), cc.x, acc0);
        acc1 = fma(static_cast<double>(qb), cc.y, acc1);
      }
      bias = acc0 + acc1;
      bias += __shfl_xor(bias, 8);
      bias += __shfl_xor(bias, 16);
      bias += __shfl_xor(bias, 32);
    }

    // ---- scores: S^T = Yk * Q' on MFMA (yhat hi and lo into separate accumulators) ----
    floatx4 shi[2], slo[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      shi[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
      slo[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
      const uint32_t aw[4] = {ka[t].x, ka[t].y, ka[t].z, ka[t].w};
      const uint32_t rw[4] = {kr[t].x, kr[t].y, kr[t].z, kr[t].w};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        uint32_t hi[4], lo[4];
        if (kFull)
          decode8_full(aw[st], rw[st], s_big, bank, hi, lo);
        else
          decode8_draft(aw[st], s_pairs, hi, lo);
        shi[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(hi), bq[st], shi[t], 0, 0, 0);
        slo[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(lo), bq[st], slo[t], 0, 0, 0);
      }
    }
    // Column n (< 8) holds yhat_hi * q'hi: the only large part.  Everything
    // else is small; it is summed in fp32, the large part joins in fp64.
    // tokens of this lane: 16t + 4r + i; every lane ends with its head's score.
    const double inv_k = 1.0 / static_cast<double>(kscale);
    const double scale64 = sm64 * inv_k;
    double sfull[8];
    float cmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = shi[t][i], bb = slo[t][i];
        const float a2 = __shfl_xor(a, 8), b2 = __shfl_xor(bb, 8);
        const float big = lo_col ? a2 : a;
        const float small = (lo_col ? a : a2) + bb + b2;
        const double sc64 = (static_cast<double>(big) + static_cast<double>(small) + bias * kscale) * scale64;
        sfull[4 * t + i] = sc64;
        cmax = fmaxf(cmax, static_cast<float>(sc64));
      }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = m_run == -INFINITY ? 0.0f : __expf(m_run - m_new);
    float p[8];
    float psum = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      p[k] = __expf(static_cast<float>(sfull[k] - static_cast<double>(m_new)));
      psum += p[k];
    }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (scores != nullptr && !lo_col && head < g) {
      float *srow = scores + (static_cast<size_t>(b) * s.q_heads + h * g + head) * T +
                    static_cast<size_t>(lp) * kPage + c * kChunk;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) srow[16 * t + 4 * r + i] = static_cast<float>(sfull[4 * t + i]);
    }

    // ---- P operand: this lane's 8 probabilities, hi or lo part by column ----
    half8 pop;
    {
      uint32_t u[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        u[k] = split_part(p[2 * k], lo_col) | (split_part(p[2 * k + 1], lo_col) << 16);
      pop = as_half8(u);
    }

    // ---- rescale the running output of columns 4r + i ----
    float acol[4], pcol[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int src = (4 * r + i) & 7;  // lane holding that head's values (r = 0 row)
      acol[i] = __shfl(alpha, src);
      pcol[i] = r < 2 ? __shfl(psum, src) : 0.0f;  // c0v term once, on the hi rows
    }
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[ct][i] *= acol[i];

    // ---- values: O += P * Yv on MFMA, then the chunk's affine map ----
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      uint32_t hi[4], lo[4];
      if (kFull)
        decode8_full(va[ct], vr[ct], s_big, bank, hi, lo);
      else
        decode8_draft(va[ct], s_pairs, hi, lo);
      floatx4 ov = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
      ov = __builtin_amdgcn_mfma_f32_16x16x32_f16(pop, as_half8(hi), ov, 0, 0, 0);
      ov = __builtin_amdgcn_mfma_f32_16x16x32_f16(pop, as_half8(lo), ov, 0, 0, 0);
      const float c1v = sc[1 * kDim + 16 * ct + n];
      const float c0v = sc[2 * kDim + 16 * ct + n];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[ct][i] = __builtin_fmaf(c1v, ov[i], __builtin_fmaf(c0v, pcol[i], acc[ct][i]));
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- combine the 4 waves of the block, write one (m, l, o) partial ----
  __syncthreads();  // every wave is done with the tables: reuse them
  float *s_o = reinterpret_cast<float *>(s_big);  // [wave][16 col][128 ch]
  if (r == 0 && n < 8) {
    s_ml[w][0][n] = m_run;
    s_ml[w][1][n] = l_run;
  }
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_o[(w * 16 + 4 * r + i) * kDim + 16 * ct + n] = acc[ct][i];
  __syncthreads();
  Partials pt = partials_of(ws, s);
  const size_t base = static_cast<size_t>(blockIdx.x) * g;
  for (int e = tid; e < g * kDim; e += kThreads) {
    const int j = e / kDim, d = e % kDim;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, s_ml[ww][0][j]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float mw = s_ml[ww][0][j];
      if (mw == -INFINITY) continue;
      const float f = __expf(mw - M);
      L += f * s_ml[ww][1][j];
      O += f * (s_o[(ww * 16 + j) * kDim + d] + s_o[(ww * 16 + 8 + j) * kDim + d]);
    }
    pt.o[(base + j) * kDim + d] = O;
    if (d == 0) {
      pt.m[base + j] = static_cast<double>(M);
      pt.l[base + j] = L;
    }
  }
}

MfmaTables build_mfma_tables() {
  MfmaTables t;
  const DecodeTable &dt = decode_table();
  const DraftTable &df = draft_table();
  auto pair = [](float y) {
    const _Float16 hi = static_cast<_Float16>(y);
    const _Float16 lo = static_cast<_Float16>(y - static_cast<float>(hi));
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) << 16);
  };
  for (int byte = 0; byte < 256; ++byte) {
    // the byte is the code read as int8: (a << 4 | r)
    const int code = byte >= 128 ? byte - 256 : byte;
    t.full[byte] = pair(dt.y[code + 128]);
  }
  for (int nib = 0; nib < 16; ++nib) t.draft[nib] = pair(df.y[nib]);
  return t;
}

}  // namespace

bool attention_mfma_supported(int group) { return group >= 1 && group <= 8; }

hipError_t launch_attention_mfma(const uint16_t *q, const PlanesArg &k, const PlanesArg &v,
                                 const int32_t *block_table, const int32_t *seq_lens,
                                 const AttnShape &s, float sm_scale, bool full, float *scores,
                                 void *workspace, hipStream_t stream) {
  static const MfmaTables tables = build_mfma_tables();
  const dim3 grid(static_cast<unsigned>(static_cast<long long>(s.batch) * s.heads * s.splits));
  if (full)
    hipLaunchKernelGGL(attn_mfma_kernel<true>, grid, dim3(kThreads), 0, stream, q, k, v,
                       block_table, seq_lens, s, sm_scale, scores, workspace, tables);
  else
    hipLaunchKernelGGL(attn_mfma_kernel<false>, grid, dim3(kThreads), 0, stream, q, k, v,
                       block_table, seq_lens, s, sm_scale, scores, workspace, tables);
  return hipGetLastError();
}

}  // namespace lynx
