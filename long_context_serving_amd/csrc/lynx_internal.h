// Internal declarations shared by the liblynx translation units.
//
// Everything here is product code: host-side constant tables, kernel
// argument structs and launcher prototypes.  The CPU oracle under oracle/
// shares nothing with it.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/lynx.h"

namespace lynx {

constexpr int kPage = LYNX_PAGE_TOKENS;      // 256 tokens per page
constexpr int kChunk = LYNX_CHUNK_TOKENS;    // C = 32
constexpr int kChunks = LYNX_CHUNKS_PER_PAGE;
constexpr int kDim = LYNX_HEAD_DIM;          // 128 channels per head
constexpr int kLevels = 127;                 // magnitude levels 0..127
constexpr double kAlpha = 255.0;             // alpha-law constant (a reading)

// Plane bytes per (page, head): 256 tokens x 128 channels x 4 bits.
constexpr int kPlaneTileBytes = kPage * kDim / 2;  // 16 KiB

// Code-map thresholds: T[0] = 0, T[k] = smallest fp32 u whose level
// 127 ln(1 + 255u)/ln 256 reaches k - 1/2 (k = 1..127).
struct CodeTable {
  float t[128];
};

// Decode table: yhat for every 8-bit code (index code + 128), fp32.
struct DecodeTable {
  float y[256];
};

const CodeTable &code_table();
const DecodeTable &decode_table();

// Level buckets.  An fp32 u in [0, 2) is bucketed by key = bits(u) >> 18
// (exponent and the top 5 mantissa bits).  Bucket 0 takes every u below
// 2^-14 (all of level 0: T[1] > 2^-14), buckets 1..448 split the binades
// 2^-14 .. 2^-1 into 32 parts each, and bucket 449 takes every u >= 1
// (level 127).  Consecutive thresholds are more than 4.4% apart while a
// bucket is at most 1/32 = 3.1% wide, so a bucket holds at most one
// threshold and the level is base[b] + (u >= T[base[b] + 1]).  The builder
// verifies this for every bucket (ok = false otherwise).
constexpr uint32_t kBucketShift = 18;
constexpr uint32_t kBucketFirstKey = 113u << 5;  // key of 2^-14
constexpr uint32_t kBucketLastKey = 127u << 5;   // key of 1.0
constexpr int kBuckets = static_cast<int>(kBucketLastKey - kBucketFirstKey) + 2;  // 450
struct BucketTable {
  uint8_t base[kBuckets];
  bool ok;
};
const BucketTable &bucket_table();

// Draft (anchor-only) values for the 16 anchor nibbles (index = nibble,
// i.e. a & 15): yhat(16a + 7).
struct DraftTable {
  float y[16];
};
const DraftTable &draft_table();

// yhat in fixed point for the exact integer score products: round(yhat *
// 2^30) of every 8-bit code (index code + 128) and of the 16 draft codes
// 16a + 7 (index = nibble).  |yhat| <= 1, so every value fits 31 bits.
constexpr int kFixedYBits = 30;
struct FixedDecodeTable {
  int32_t y[256];
  int32_t draft[16];
};
const FixedDecodeTable &fixed_decode_table();

// ---------------------------------------------------------------------------
// Launchers (return hipError_t of the launch; argument checking happens in
// the API layer).
// ---------------------------------------------------------------------------
struct PlanesArg {
  uint8_t *anchor;
  uint8_t *residual;
  float *page_min;
  float *page_range;
  float *chunk_mean;
  float *chunk_maxabs;
};

// anchor_bits 4 writes the 4-bit planes; 1 .. 7 the b + (8 - b) streams
// (out.anchor b * 4096 and out.residual (8 - b) * 4096 bytes per tile).
hipError_t launch_encode(const uint16_t *kv, int64_t num_pages, int heads,
                         int role, const PlanesArg &out, hipStream_t stream,
                         int anchor_bits = 4);

// K and V of one layer (4 + 4 planes) in one launch.
hipError_t launch_encode_kv(const uint16_t *k, const uint16_t *v, int64_t num_pages, int heads,
                            const PlanesArg &kout, const PlanesArg &vout, hipStream_t stream);

hipError_t launch_code_map_check(uint32_t begin, uint32_t end,
                                 unsigned long long *mismatches, hipStream_t stream);

hipError_t launch_dequant(const PlanesArg &in, int64_t num_pages, int heads,
                          int role, bool full, float *out,
                          hipStream_t stream);

// Query rows b = 0 .. batch-1 each hold Hq query heads; row b belongs to
// request b / tq (tq query tokens per request; 1 for decode).  The pages of
// a (row, KV head) are reduced in `splits` runs; `parts` partial rows are
// merged per (row, KV head): the splits, plus one for the bf16 tail page
// when there is one.
// b + (8 - b) cuts: re-cut 4 + 4 planes into a b-bit anchor stream and an
// (8 - b)-bit residual stream (b * 4096 and (8 - b) * 4096 bytes per tile),
// and dequantize from such streams (residual NULL: the draft).
hipError_t launch_split_planes(const PlanesArg &in, int64_t num_pages, int heads, int anchor_bits,
                               uint8_t *anchor_out, uint8_t *residual_out, hipStream_t stream);
hipError_t launch_dequant_split(const uint8_t *anchor, const uint8_t *residual, int anchor_bits,
                                const PlanesArg &scales, int64_t num_pages, int heads, int role,
                                float *out, hipStream_t stream);

struct AttnShape {
  int batch;         // query rows (requests * tq)
  int tq;            // query tokens per request
  int heads;         // KV heads H
  int q_heads;       // Hq
  int group;         // Hq / H
  int max_pages;     // per request
  int pages_per_split;
  int splits;
  int parts;         // partial rows merged per (row, KV head)
  long long pool_pages;  // pages in the k / v pools (block-table bound)
};

// Split partials in an attention workspace: n = batch * heads * parts *
// group rows of the running maximum m (double), the sum l and the
// unnormalised output o[128]; query head j of (row, head) and part p is
// row ((row * heads + head) * parts + p) * group + j.
struct AttnPartials {
  double *m;
  float *l;
  float *o;
};

__host__ __device__ inline AttnPartials attn_partials(void *ws, const AttnShape &s) {
  const size_t n = static_cast<size_t>(s.batch) * s.heads * s.parts * s.group;
  AttnPartials pt;
  pt.m = reinterpret_cast<double *>(ws);
  pt.l = reinterpret_cast<float *>(pt.m + ((n + 1) & ~static_cast<size_t>(1)));
  pt.o = pt.l + ((n + 3) & ~static_cast<size_t>(3));
  return pt;
}

AttnShape attention_shape(int batch, int heads, int q_heads, int max_pages);
// Shape of `requests` requests with tq query tokens each over their pages
// and a bf16 tail page.
AttnShape attention_shape_tail(int requests, int tq, int heads, int q_heads, int max_pages);
size_t attention_workspace_bytes(const AttnShape &s);

bool attention_mfma_supported(int group);
int attention_mfma_target_blocks();
// Page runs of every (row, KV head): writes `out` itself when parts == 1,
// else the split partials.  With merge set and parts > 1 the partials are
// merged into `out` inside the launch.  anchor_bits 4 reads the 4-bit
// planes; 1 .. 7 otherwise read b + (8 - b) streams (k.anchor, v.anchor:
// b bits per element; k.residual, v.residual: 8 - b).
hipError_t launch_attention_mfma(const uint16_t *q, const PlanesArg &k, const PlanesArg &v,
                                 const int32_t *block_table, const int32_t *seq_lens,
                                 const AttnShape &s, float sm_scale, bool full, float *out,
                                 float *scores, void *workspace, bool merge, hipStream_t stream,
                                 int anchor_bits = 4);
hipError_t launch_attention_mfma_combine(const AttnShape &s, const void *workspace, float *out,
                                         hipStream_t stream);

// Verify-pass page kernel (GQA group 8, 3 or more query tokens per
// request; fewer run on the decode kernels): up to 16 query rows of one
// request and KV head per block when tq <= 16, else up to 32; one block per
// (request, KV head, run of pages, group of rows); writes the split
// partials of its rows.
bool verify_mfma_used(int group, int tq);
int verify_row_blocks(int tq);
hipError_t launch_verify_mfma(const uint16_t *q, const PlanesArg &k, const PlanesArg &v,
                              const int32_t *block_table, const int32_t *page_tokens,
                              const AttnShape &s, float sm_scale, bool full, void *workspace,
                              hipStream_t stream);

// bf16 tail page of each request (tail_k / tail_v [requests][tail_cap][H][128],
// tail_len [requests] on the device): query token i of a request sees tail
// tokens 0 .. tail_len - tq + i.  Writes partial row `s.splits` of every
// (row, KV head); base2 selects the maxima convention of the page kernels
// (base-2 scores for the matrix-core kernel, natural ones otherwise).
hipError_t launch_attention_tail_part(const uint16_t *q, const uint16_t *tail_k,
                                      const uint16_t *tail_v, const int32_t *tail_len,
                                      int tail_cap, const AttnShape &s, float sm_scale, bool base2,
                                      void *workspace, hipStream_t stream);

// anchor_bits other than 4: b + (8 - b) streams, matrix-core groups only.
hipError_t launch_attention(const uint16_t *q, const PlanesArg &k,
                            const PlanesArg &v, const int32_t *block_table,
                            const int32_t *seq_lens, const AttnShape &s,
                            float sm_scale, bool full, float *out,
                            float *scores, void *workspace,
                            hipStream_t stream, int anchor_bits = 4);

// Pages plus the bf16 tail page, merged into out [batch][Hq][128]
// (s from attention_shape_tail).
hipError_t launch_attention_with_tail(const uint16_t *q, const PlanesArg &k, const PlanesArg &v,
                                      const int32_t *block_table, const int32_t *page_tokens,
                                      const uint16_t *tail_k, const uint16_t *tail_v,
                                      const int32_t *tail_len, int tail_cap, const AttnShape &s,
                                      float sm_scale, bool full, float *out, void *workspace,
                                      hipStream_t stream);

// Library-owned scratch (lynx_scratch.hip): capacity in bytes, and the
// scratch's device address on the current device (looked up on the first
// call per device).
size_t scratch_capacity();
hipError_t scratch_address(void **ptr);

}  // namespace lynx
