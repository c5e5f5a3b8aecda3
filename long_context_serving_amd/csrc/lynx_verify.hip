// Verify-pass attention on matrix cores: the speculative tokens of a
// request attend to its compact pages (GQA group 8).
//
// Page "Lynx: the KV cache does not have to arrive whole", section 4: the
// drafted tokens are verified in one pass over the refined cache; section 3
// gives the reconstruction x = mn + rg * (mu + s * yhat).  The decode
// kernel serves one query token per row and rebuilds every chunk's operands
// per row; here up to 32 query rows of one request and KV head share a
// block, and each chunk's operands are built once per block in LDS:
//
//   K' = rg * mu + c1 * yhat = x - mn (c1 = rg * s), times a power of two
//        ks, so the score of a token is q . K' / ks + q . mn, the page bias
//        q . mn summed in fp64 once per page (the page minimum holds a
//        channel's offset, which may dwarf its range); q enters the product
//        unsplit (a bf16 value is an fp16 value after a power-of-two scale),
//        so one 16 x 16 x 32 product covers 16 tokens x (2 query rows x 8
//        heads) x 16 channels;
//   V  = the reconstructed values themselves, whose rounding error reaches
//        the output only through the softmax weights (a convex combination).
//
// K' and V are stored as fp16 (hi, lo) pairs (hi = the value truncated to
// 11 significant bits, lo = the rounded remainder), each pair in two
// consecutive k slots.  In the score product q repeats its value in both
// slots; in the value product every 16 tokens take two products into the
// same accumulator, one with the probabilities' hi parts repeated in both
// slots and one with their lo parts, so that a lane's value columns are its
// own score columns (row, head).  Scores are assembled in fp64 (MFMA sum
// times 1/ks, plus the fp64 page bias), the running maximum is base 2 and moves
// only when exceeded by 2^8, and each wave keeps its 4 rows' accumulators
// (two column groups of 2 rows x 8 heads) in the matrix-core C operand for
// the whole run, so a block's 32 rows share each chunk's build (one group
// of 2 rows, 16 per block, when the request has no more rows).  A block
// covers one run of pages; the runs' partials (m, l, o) are merged with the
// bf16 tail's by the split combine kernel.
#include <math.h>

#include "lynx_internal.h"
#include "lynx_lanes.h"

namespace lynx {
namespace {

using namespace lanes;

constexpr int kVW = 8;                      // waves per block
constexpr int kVT = 64 * kVW;
constexpr int kGroupRows = 2 * kVW;         // query rows per block and column group
constexpr int kG = 8;                       // query heads per KV head
constexpr float kVSlack = 8.0f;             // log2 of the largest probability before rescaling
constexpr int kKRowB = kDim * 4 + 16;       // one token of K': 128 (hi, lo) words + 16 B pad
constexpr int kKTileB = kChunk * kKRowB;
constexpr int kVRowB = kChunk * 4 + 16;     // one channel of V: 32 (hi, lo) words + 16 B pad
constexpr int kVTileB = kDim * kVRowB;
// c1 * ks f32[128] | rg * mu * ks f32[128] | mn f64[128] | 1/(ks qs) f64
constexpr int kSlotB = kDim * 16 + 16;
// LDS map: yhat table (256 codes x 64 copies, lane l reads copy l), two K'
// tiles, two V tiles, three scale slots, and the block's |q| maxima.
constexpr int kYOff = 0;
constexpr int kKOff = 256 * 256;
constexpr int kVOff = kKOff + 2 * kKTileB;
constexpr int kSOff = kVOff + 2 * kVTileB;
constexpr int kQmOff = kSOff + 3 * kSlotB;
constexpr int kVLds = kQmOff + kVW * 4;
static_assert(kVLds <= 160 * 1024, "LDS of one block");

struct VerifyTable {
  float y[256];  // code byte (the code read as int8) -> yhat
};

// Per-thread inputs of one chunk's build: the K word of token t / 16,
// channels 8 (t % 16) .. + 7, and the V word t % 4 of channel t / 4, with
// that channel's V scales.
struct BuildIn {
  uint32_t ka, kr, va, vr;
  float mnv, rgv, muv, sv;
};
// K scales of channels 2l, 2l + 1 (every wave loads all 128 channels).
struct KScale {
  float2 mnk, rgk, muk, sk;
};

__device__ __forceinline__ uint32_t ldg_nt(const uint8_t *base, size_t off) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(base + off));
}

// LDS byte address of table row x.byte[J], copy of lane bits lb.
template <int J>
__device__ __forceinline__ uint32_t yaddr(uint32_t x, uint32_t lb) {
  return __builtin_amdgcn_perm(x, lb, 0x0C0C0000u | ((4u + J) << 8));
}

// fp16 (hi, lo) pair of x: hi = x truncated to 11 significant bits, lo =
// the remainder rounded to fp16.
__device__ __forceinline__ uint32_t pair16(float x) {
  const float hi = __uint_as_float(__float_as_uint(x) & 0xFFFFE000u);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(hi, x - hi));
}

// 8 code bytes of a word pair: byte j of e = element 2j, of o = element
// 2j + 1 (element i is nibble i); the draft code is (a << 4) | 7.
template <bool kFull>
__device__ __forceinline__ void code_bytes8(uint32_t a, uint32_t r, uint32_t &e, uint32_t &o) {
  if (kFull) {
    e = ((a << 4) & 0xF0F0F0F0u) | (r & 0x0F0F0F0Fu);
    o = (a & 0xF0F0F0F0u) | ((r >> 4) & 0x0F0F0F0Fu);
  } else {
    e = ((a << 4) & 0xF0F0F0F0u) | 0x07070707u;
    o = (a & 0xF0F0F0F0u) | 0x07070707u;
  }
}

// yhat of the 8 elements (in element order) of a word pair.
template <bool kFull>
__device__ __forceinline__ void yhat8(uint32_t a, uint32_t r, uint32_t lb, const char *ytab,
                                      float (&y)[8]) {
  uint32_t e, o;
  code_bytes8<kFull>(a, r, e, o);
  auto rd = [&](uint32_t addr) { return *reinterpret_cast<const float *>(ytab + addr); };
  y[0] = rd(yaddr<0>(e, lb));
  y[1] = rd(yaddr<0>(o, lb));
  y[2] = rd(yaddr<1>(e, lb));
  y[3] = rd(yaddr<1>(o, lb));
  y[4] = rd(yaddr<2>(e, lb));
  y[5] = rd(yaddr<2>(o, lb));
  y[6] = rd(yaddr<3>(e, lb));
  y[7] = rd(yaddr<3>(o, lb));
}

template <bool kFull>
__device__ __forceinline__ void load_build(BuildIn &in, const PlanesArg &kp, const PlanesArg &vp,
                                           size_t tile, int c, int t) {
  const size_t cb = tile * kPlaneTileBytes + static_cast<size_t>(c) * (kChunk * kDim / 2);
  const size_t koff = cb + static_cast<size_t>((t >> 4) * 64 + (t & 15) * 4);
  const size_t voff = cb + static_cast<size_t>((t >> 2) * 16 + (t & 3) * 4);
  in.ka = ldg_nt(kp.anchor, koff);
  in.va = ldg_nt(vp.anchor, voff);
  if (kFull) {
    in.kr = ldg_nt(kp.residual, koff);
    in.vr = ldg_nt(vp.residual, voff);
  } else {
    in.kr = 0u;
    in.vr = 0u;
  }
  const int ch = t >> 2;
  const size_t pidx = tile * kDim + ch;
  const size_t cidx = (tile * kChunks + c) * kDim + ch;
  in.mnv = vp.page_min[pidx];
  in.rgv = vp.page_range[pidx];
  in.muv = vp.chunk_mean[cidx];
  in.sv = vp.chunk_maxabs[cidx];
}

__device__ __forceinline__ void load_kscale(KScale &ks, const PlanesArg &kp, size_t tile, int c,
                                            int lane) {
  const size_t pidx = tile * kDim + 2 * lane;
  const size_t cidx = (tile * kChunks + c) * kDim + 2 * lane;
  ks.mnk = *reinterpret_cast<const float2 *>(kp.page_min + pidx);
  ks.rgk = *reinterpret_cast<const float2 *>(kp.page_range + pidx);
  ks.muk = *reinterpret_cast<const float2 *>(kp.chunk_mean + cidx);
  ks.sk = *reinterpret_cast<const float2 *>(kp.chunk_maxabs + cidx);
}

// Scale slot of a chunk: c1 * ks, rg * mu * ks and mn for every channel
// (lane l writes channels 2l, 2l + 1), and 1 / (ks * qs) (lane 0).
// ks = 2^(14 - e), e the exponent of the largest rg * (mu + s) (|yhat| <= 1),
// keeps every K' below 2^15.  One wave (kStager) loads the K scales and
// stages every slot; the last wave has the fewest query rows.
constexpr int kStager = kVW - 1;
__device__ __forceinline__ void stage_slot(const KScale &k, char *slot, int lane, double inv_qs) {
  const float c1a = k.rgk.x * k.sk.x, c1b = k.rgk.y * k.sk.y;  // fp32
  const float c0a = k.rgk.x * k.muk.x, c0b = k.rgk.y * k.muk.y;
  const float top = wave_max(fmaxf(fabsf(c1a) + fabsf(c0a), fabsf(c1b) + fabsf(c0b)));
  float ks = 1.0f;
  double inv_ks = 1.0;
  const uint32_t eb = (__float_as_uint(top) >> 23) & 0xFFu;
  if (eb != 0u && eb != 0xFFu) {
    int ex = 127 + 14 + 127 - static_cast<int>(eb);
    ex = ex < 1 ? 1 : (ex > 254 ? 254 : ex);
    ks = __uint_as_float(static_cast<uint32_t>(ex) << 23);
    inv_ks = __builtin_bit_cast(double, static_cast<uint64_t>(1023 + 127 - ex) << 52);
  }
  reinterpret_cast<float2 *>(slot)[lane] = make_float2(c1a * ks, c1b * ks);
  reinterpret_cast<float2 *>(slot + kDim * 4)[lane] = make_float2(c0a * ks, c0b * ks);
  reinterpret_cast<double2 *>(slot + kDim * 8)[lane] =
      make_double2(static_cast<double>(k.mnk.x), static_cast<double>(k.mnk.y));
  if (lane == 0) *reinterpret_cast<double *>(slot + kDim * 16) = inv_ks * inv_qs;
}

// Build the K' and V tiles of one chunk from thread t's inputs.
template <bool kFull>
__device__ __forceinline__ void build_chunk(const BuildIn &in, const char *slot, char *ktile,
                                            char *vtile, const char *ytab, int t, uint32_t lb) {
  {
    // K': token t / 16, channels 8 (t % 16) .. + 7
    float y[8];
    yhat8<kFull>(in.ka, in.kr, lb, ytab, y);
    const int ch0 = (t & 15) * 8;
    const float4 ca = *reinterpret_cast<const float4 *>(slot + ch0 * 4);  // c1 * ks
    const float4 cb = *reinterpret_cast<const float4 *>(slot + ch0 * 4 + 16);
    const float4 da = *reinterpret_cast<const float4 *>(slot + kDim * 4 + ch0 * 4);  // rg * mu * ks
    const float4 db = *reinterpret_cast<const float4 *>(slot + kDim * 4 + ch0 * 4 + 16);
    u32x4 w0, w1;
    w0[0] = pair16(__builtin_fmaf(y[0], ca.x, da.x));
    w0[1] = pair16(__builtin_fmaf(y[1], ca.y, da.y));
    w0[2] = pair16(__builtin_fmaf(y[2], ca.z, da.z));
    w0[3] = pair16(__builtin_fmaf(y[3], ca.w, da.w));
    w1[0] = pair16(__builtin_fmaf(y[4], cb.x, db.x));
    w1[1] = pair16(__builtin_fmaf(y[5], cb.y, db.y));
    w1[2] = pair16(__builtin_fmaf(y[6], cb.z, db.z));
    w1[3] = pair16(__builtin_fmaf(y[7], cb.w, db.w));
    char *dst = ktile + (t >> 4) * kKRowB + ch0 * 4;
    *reinterpret_cast<u32x4 *>(dst) = w0;
    *reinterpret_cast<u32x4 *>(dst + 16) = w1;
  }
  {
    // V: channel t / 4, word t % 4 = tokens 4g .. 4g + 3 (elements 0..3)
    // and 16 + 4g .. (elements 4..7)
    float y[8];
    yhat8<kFull>(in.va, in.vr, lb, ytab, y);
    u32x4 w0, w1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w0[i] = pair16(__builtin_fmaf(in.rgv, __builtin_fmaf(in.sv, y[i], in.muv), in.mnv));
      w1[i] = pair16(__builtin_fmaf(in.rgv, __builtin_fmaf(in.sv, y[4 + i], in.muv), in.mnv));
    }
    const int g4 = (t & 3) * 4;
    char *dst = vtile + (t >> 2) * kVRowB;
    *reinterpret_cast<u32x4 *>(dst + g4 * 4) = w0;
    *reinterpret_cast<u32x4 *>(dst + (16 + g4) * 4) = w1;
  }
}

// Running state of a wave: lane (n, r) follows column n = (row n / 8,
// head n % 8) for the softmax and holds channels 16ct + 4r + i of that
// column's value sums.
struct VState {
  float m, l;
  floatx4 acc[8];
};

// kGroups column groups of 2 query rows x 8 heads per wave (1 or 2): a
// block serves 16 kGroups rows.
template <bool kFull, int kGroups>
__global__ __launch_bounds__(kVT) void verify_mfma_kernel(
    const uint16_t *__restrict__ q, PlanesArg kp, PlanesArg vp,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ page_tokens,
    AttnShape s, int row_blocks, float sm_scale, void *ws, VerifyTable tab) {
  __shared__ __align__(16) char smem[kVLds];
  const int t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int n = lane & 15, r = lane >> 4;
  const uint32_t lb = static_cast<uint32_t>(lane * 4);

  // blocks of one (request, KV head, run) are consecutive logical blocks
  // (their row groups share the run's pages); spread over the 8 XCDs in
  // contiguous groups
  const unsigned nblk = gridDim.x;
  unsigned lbi = blockIdx.x;
  if ((nblk & 7u) == 0u) lbi = (blockIdx.x & 7u) * (nblk >> 3) + (blockIdx.x >> 3);
  const int rb = static_cast<int>(lbi % static_cast<unsigned>(row_blocks));
  const unsigned rest = lbi / static_cast<unsigned>(row_blocks);
  const int split = static_cast<int>(rest % static_cast<unsigned>(s.splits));
  const int bh = static_cast<int>(rest / static_cast<unsigned>(s.splits));
  const int h = bh % s.heads;
  const int req = bh / s.heads;

  // ---- this wave's rows and its lanes' query values: in column group g,
  // lane (n, r) follows row row_a + 2g + n / 8, head n % 8 ----
  const int row_a = rb * kGroupRows * kGroups + 2 * kGroups * w;
  // a wave whose rows all lie past the request's tq builds and stages its
  // share of every chunk but computes nothing (wave-uniform)
  const bool wave_rows = row_a < s.tq;
  bool row_ok[kGroups];
  uint2 qraw[kGroups][8];  // channels 16st + 4r .. + 3
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    const int my_row = row_a + 2 * g + (n >> 3);
    row_ok[g] = my_row < s.tq;
    const size_t qrow = static_cast<size_t>(req) * s.tq + (row_ok[g] ? my_row : s.tq - 1);
    const uint16_t *qg = q + (qrow * s.q_heads + static_cast<size_t>(h) * kG + (n & 7)) * kDim;
#pragma unroll
    for (int st = 0; st < 8; ++st)
      qraw[g][st] = *reinterpret_cast<const uint2 *>(qg + 16 * st + 4 * r);
  }

  // ---- this block's run of chunks ----
  const __attribute__((address_space(4))) int32_t *bt_c =
      (const __attribute__((address_space(4))) int32_t *)block_table;
  const __attribute__((address_space(4))) int32_t *pt_c =
      (const __attribute__((address_space(4))) int32_t *)page_tokens;
  int npages = s.max_pages;
  if (page_tokens) {
    npages = pt_c[req] / kPage;
    npages = npages < 0 ? 0 : (npages > s.max_pages ? s.max_pages : npages);
  }
  const int p0 = split * s.pages_per_split;
  int p1 = p0 + s.pages_per_split;
  p1 = p1 > npages ? npages : p1;
  const int cb = p0 * kChunks;
  const int ce = p1 > p0 ? p1 * kChunks : cb;
  auto page_of = [&](int c) -> long long {
    if (c >= ce) return -1;
    const int lp = c >> 3;
    const long long pg = block_table ? bt_c[static_cast<size_t>(req) * s.max_pages + lp]
                                     : static_cast<long long>(req) * s.max_pages + lp;
    return (pg < 0 || pg >= s.pool_pages) ? -1 : pg;
  };
  auto tile_of = [&](long long pg) { return pg >= 0 ? static_cast<size_t>(pg) * s.heads + h : 0; };
  auto chunk_of = [&](long long pg, int c) { return pg >= 0 ? (c & 7) : 0; };

  // ---- first loads: inputs of chunk cb, K scales of cb and cb + 1 ----
  BuildIn bin;
  KScale ksa, ring;
  {
    const long long g0 = page_of(cb), g1 = page_of(cb + 1);
    if (w == kStager) {
      load_kscale(ksa, kp, tile_of(g0), chunk_of(g0, cb), lane);
      load_kscale(ring, kp, tile_of(g1), chunk_of(g1, cb + 1), lane);
    }
    load_build<kFull>(bin, kp, vp, tile_of(g0), chunk_of(g0, cb), t);
  }

  // ---- yhat table: 64 copies of each entry ----
  char *ytab = smem + kYOff;
  {
    const float yv = tab.y[t & 255];
    const uint32_t yb = __float_as_uint(yv);
    u32x4 *dst = reinterpret_cast<u32x4 *>(ytab + (t & 255) * 256 + (t >> 8) * 128);
#pragma unroll
    for (int k = 0; k < 8; ++k) dst[k] = u32x4{yb, yb, yb, yb};
  }

  // ---- the block-wide power of two qs that brings max |q| into
  // [2^14, 2^15): q * qs is then an exact fp16 value (bf16 has 8 significant
  // bits), which both the score product and the fp64 page bias use ----
  auto q_at = [&](int g, int st, int i) {  // bf16 q of channel 16st + 4r + i, 0 past the rows
    const uint32_t u = (i >> 1) ? qraw[g][st].y : qraw[g][st].x;
    const uint32_t bits = (i & 1) ? (u & 0xFFFF0000u) : (u << 16);
    return row_ok[g] ? __uint_as_float(bits) : 0.0f;
  };
  float qmax = 0.0f;
#pragma unroll
  for (int g = 0; g < kGroups; ++g)
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) qmax = fmaxf(qmax, fabsf(q_at(g, st, i)));
  qmax = wave_max(qmax);
  float *s_qm = reinterpret_cast<float *>(smem + kQmOff);
  if (lane == 0) s_qm[w] = qmax;
  __syncthreads();  // table and maxima
  qmax = s_qm[0];
#pragma unroll
  for (int k = 1; k < kVW; ++k) qmax = fmaxf(qmax, s_qm[k]);
  float qs = 1.0f;
  double inv_qs = 1.0;
  {
    const uint32_t eb = (__float_as_uint(qmax) >> 23) & 0xFFu;
    if (eb != 0u && eb != 0xFFu) {
      int ex = 127 + 14 + 127 - static_cast<int>(eb);
      ex = ex < 1 ? 1 : (ex > 254 ? 254 : ex);
      qs = __uint_as_float(static_cast<uint32_t>(ex) << 23);
      inv_qs = __builtin_bit_cast(double, static_cast<uint64_t>(1023 + 127 - ex) << 52);
    }
  }
  // B operand of step st: q * qs of channels 16st + 4r + i, in both k slots
  u32x4 qb[kGroups][8];
#pragma unroll
  for (int g = 0; g < kGroups; ++g)
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = q_at(g, st, i) * qs;
        qb[g][st][i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x, x));
      }

  char *ktiles = smem + kKOff;
  char *vtiles = smem + kVOff;
  char *slots = smem + kSOff;
  const double sm2 = static_cast<double>(sm_scale) * 1.4426950408889634074;
  const double bias_scale = sm2 * inv_qs;

  VState st[kGroups];
  double bias2[kGroups];  // the current page's bias, times sm2 / qs
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    bias2[g] = 0.0;
    st[g].m = -INFINITY;
    st[g].l = 0.0f;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) st[g].acc[ct] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  if (cb < ce) {
    if (w == kStager) {
      stage_slot(ksa, slots, lane, inv_qs);
      stage_slot(ring, slots + kSlotB, lane, inv_qs);
    }
    __syncthreads();
    build_chunk<kFull>(bin, slots, ktiles, vtiles, ytab, t, lb);
    __syncthreads();

    // step j: load the build inputs of chunk c + 1 and the K scales of
    // chunk c + 2, compute chunk c = cb + j from tiles j & 1 and slot j % 3,
    // then build chunk c + 1 and stage slot (j + 2) % 3 (the loads have had
    // the compute of chunk c to land)
    for (int j = 0; cb + j < ce; ++j) {
      const int c = cb + j;
      const int tb = j & 1;
      {
        const long long g1 = page_of(c + 1), g2 = page_of(c + 2);
        load_build<kFull>(bin, kp, vp, tile_of(g1), chunk_of(g1, c + 1), t);
        if (w == kStager) load_kscale(ring, kp, tile_of(g2), chunk_of(g2, c + 2), lane);
      }
      if (wave_rows && page_of(c) >= 0) {
        // (the q operands are redefined here so that the bias's conversions
        // of them stay inside the step: hoisted out of the loop, the fp64
        // values would take 128 registers)
#pragma unroll
        for (int g = 0; g < kGroups; ++g)
#pragma unroll
          for (int s8 = 0; s8 < 8; ++s8)
            asm volatile("" : "+v"(qb[g][s8][0]), "+v"(qb[g][s8][1]), "+v"(qb[g][s8][2]), "+v"(qb[g][s8][3]));
        const char *kt = ktiles + tb * kKTileB;
        const char *vt = vtiles + tb * kVTileB;
        const char *slot = slots + (j % 3) * kSlotB;
        // page bias sum_d (q_d qs) mn_d (fp64) of each group's column n over
        // channels 16st + 4r + i, times sm2 / qs, at the first chunk of a page
        if (j == 0 || (c & (kChunks - 1)) == 0) {
          const double *mnp = reinterpret_cast<const double *>(slot + kDim * 8);
          double a0[kGroups], a1[kGroups];
#pragma unroll
          for (int g = 0; g < kGroups; ++g) a0[g] = a1[g] = 0.0;
#pragma unroll
          for (int s8 = 0; s8 < 8; ++s8) {
            const double2 x0 = *reinterpret_cast<const double2 *>(mnp + 16 * s8 + 4 * r);
            const double2 x1 = *reinterpret_cast<const double2 *>(mnp + 16 * s8 + 4 * r + 2);
#pragma unroll
            for (int g = 0; g < kGroups; ++g) {
              auto qv = [&](int i) {
                return static_cast<double>(
                    static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(qb[g][s8][i]))));
              };
              a0[g] = fma(qv(0), x0.x, a0[g]);
              a1[g] = fma(qv(1), x0.y, a1[g]);
              a0[g] = fma(qv(2), x1.x, a0[g]);
              a1[g] = fma(qv(3), x1.y, a1[g]);
            }
          }
#pragma unroll
          for (int g = 0; g < kGroups; ++g) bias2[g] = xrows_sum(a0[g] + a1[g]) * bias_scale;
        }
        // scores S^T[16 tok][16 col] of both groups for tiles 0, 1 (each K'
        // operand read serves both groups)
        floatx4 s0[kGroups], s1[kGroups];
#pragma unroll
        for (int g = 0; g < kGroups; ++g) s0[g] = s1[g] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) {
          const half8 a0 = *reinterpret_cast<const half8 *>(kt + n * kKRowB + (16 * s8 + 4 * r) * 4);
          const half8 a1 =
              *reinterpret_cast<const half8 *>(kt + (16 + n) * kKRowB + (16 * s8 + 4 * r) * 4);
#pragma unroll
          for (int g = 0; g < kGroups; ++g) {
            const half8 b = __builtin_bit_cast(half8, qb[g][s8]);
            s0[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b, s0[g], 0, 0, 0);
            s1[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b, s1[g], 0, 0, 0);
          }
          // keep the operand reads of at most two steps in flight
          if (s8 & 1) __builtin_amdgcn_sched_barrier(0);
        }
        const double scale2 = sm2 * *reinterpret_cast<const double *>(slot + kDim * 16);
        // online softmax per group; P operands: the lane's own column n,
        // tokens 16tt + 4r + i (p[4tt + i]), each in the two k slots of its
        // V (hi, lo) pair: once the P hi part in both, once the P lo part
        half8 pk[kGroups][4];  // [2tt]: hi parts of tile tt, [2tt + 1]: lo parts
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
          double sc[8];
          float cmax = -INFINITY;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sc[i] = fma(static_cast<double>(s0[g][i]), scale2, bias2[g]);
            sc[4 + i] = fma(static_cast<double>(s1[g][i]), scale2, bias2[g]);
            cmax = fmaxf(cmax, fmaxf(static_cast<float>(sc[i]), static_cast<float>(sc[4 + i])));
          }
          cmax = xrows(cmax, MaxOp());
          const bool rescale = __builtin_amdgcn_ballot_w64(cmax > st[g].m + kVSlack) != 0;
          float alpha = 1.0f;
          if (rescale) {
            const float m_new = fmaxf(st[g].m, cmax);
            alpha = st[g].m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(st[g].m - m_new);
            st[g].m = m_new;
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) st[g].acc[ct] *= alpha;
          }
          float p[8];
          float psum = 0.0f;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            p[i] = __builtin_amdgcn_exp2f(static_cast<float>(sc[i] - static_cast<double>(st[g].m)));
            psum += p[i];
          }
          psum = xrows(psum, SumOp());
          st[g].l = st[g].l * alpha + psum;
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            u32x4 vh, vl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              vh[i] = split_dup(p[4 * tt + i], 0u);
              vl[i] = split_dup(p[4 * tt + i], 0xFFFFE000u);
            }
            pk[g][2 * tt] = __builtin_bit_cast(half8, vh);
            pk[g][2 * tt + 1] = __builtin_bit_cast(half8, vl);
          }
        }
        // values: O^T[16 ch][16 col] += V^T[16 ch][32 k] * P[32 k][16 col]
        // (each V operand read serves both groups)
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
          const char *vrow = vt + (16 * ct + n) * kVRowB;
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const half8 y = *reinterpret_cast<const half8 *>(vrow + (16 * tt + 4 * r) * 4);
#pragma unroll
            for (int g = 0; g < kGroups; ++g) {
              st[g].acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(y, pk[g][2 * tt], st[g].acc[ct], 0, 0, 0);
              st[g].acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(y, pk[g][2 * tt + 1], st[g].acc[ct], 0, 0, 0);
            }
          }
          if (ct & 1) __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (c + 1 < ce)
        build_chunk<kFull>(bin, slots + ((j + 1) % 3) * kSlotB, ktiles + (tb ^ 1) * kKTileB,
                           vtiles + (tb ^ 1) * kVTileB, ytab, t, lb);
      if (w == kStager) stage_slot(ring, slots + ((j + 2) % 3) * kSlotB, lane, inv_qs);
      __syncthreads();
    }
  }

  // ---- partials: lane (n, r) writes column n of each group ----
  {
    AttnPartials pt = attn_partials(ws, s);
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      const int row = row_a + 2 * g + (n >> 3);
      if (row < s.tq) {
        const size_t grow = static_cast<size_t>(req) * s.tq + row;
        const size_t prow = ((grow * s.heads + h) * s.parts + split) * kG + (n & 7);
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
          *reinterpret_cast<float4 *>(pt.o + prow * kDim + 16 * ct + 4 * r) =
              make_float4(st[g].acc[ct][0], st[g].acc[ct][1], st[g].acc[ct][2], st[g].acc[ct][3]);
        if (r == 0) {
          pt.m[prow] = static_cast<double>(st[g].m);
          pt.l[prow] = st[g].l;
        }
      }
    }
  }
}

VerifyTable build_verify_table() {
  VerifyTable t;
  const DecodeTable &dt = decode_table();
  for (int byte = 0; byte < 256; ++byte) {
    const int code = byte >= 128 ? byte - 256 : byte;
    t.y[byte] = dt.y[code + 128];
  }
  return t;
}

}  // namespace

// A block's cost per chunk does not depend on how many of its rows are
// used, so few query tokens per request are cheaper on the decode kernels
// (one row per query token); the crossover is measured.
constexpr int kVerifyMinTokens = 3;

bool verify_mfma_used(int group, int tq) { return group == kG && tq >= kVerifyMinTokens; }

// Two column groups per wave (32 rows per block) share each chunk's build
// over twice the rows, at twice a block's per-chunk products; one group is
// cheaper while all rows fit in 16.
int verify_groups(int tq) { return tq > kGroupRows ? 2 : 1; }

int verify_row_blocks(int tq) {
  const int rows = kGroupRows * verify_groups(tq);
  return (tq + rows - 1) / rows;
}

hipError_t launch_verify_mfma(const uint16_t *q, const PlanesArg &k, const PlanesArg &v,
                              const int32_t *block_table, const int32_t *page_tokens,
                              const AttnShape &s, float sm_scale, bool full, void *workspace,
                              hipStream_t stream) {
  static const VerifyTable table = build_verify_table();
  if (s.group != kG || s.tq < 1 || s.splits < 1 || s.pool_pages <= 0) return hipErrorInvalidValue;
  const int requests = s.batch / s.tq;
  const int rbs = verify_row_blocks(s.tq);
  const dim3 grid(static_cast<unsigned>(static_cast<long long>(requests) * s.heads * s.splits * rbs));
  const bool two = verify_groups(s.tq) == 2;
  if (full && two)
    hipLaunchKernelGGL((verify_mfma_kernel<true, 2>), grid, dim3(kVT), 0, stream, q, k, v, block_table,
                       page_tokens, s, rbs, sm_scale, workspace, table);
  else if (full)
    hipLaunchKernelGGL((verify_mfma_kernel<true, 1>), grid, dim3(kVT), 0, stream, q, k, v, block_table,
                       page_tokens, s, rbs, sm_scale, workspace, table);
  else if (two)
    hipLaunchKernelGGL((verify_mfma_kernel<false, 2>), grid, dim3(kVT), 0, stream, q, k, v, block_table,
                       page_tokens, s, rbs, sm_scale, workspace, table);
  else
    hipLaunchKernelGGL((verify_mfma_kernel<false, 1>), grid, dim3(kVT), 0, stream, q, k, v, block_table,
                       page_tokens, s, rbs, sm_scale, workspace, table);
  return hipGetLastError();
}

}  // namespace lynx
