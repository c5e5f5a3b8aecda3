// liblynx C ABI: argument validation, device check and dispatch.
//
// See include/lynx.h for the contract of every entry point.  Nothing here
// allocates device memory or synchronizes; all work is enqueued on the
// caller's stream.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "lynx_internal.h"

namespace {

using lynx::PlanesArg;

constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
int g_dev_ok[kMaxDevices];
int g_dev_cus[kMaxDevices];

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks that the current device is a gfx950 and returns its compute-unit
// count through *cus (both cached per device).
int check_device(int *cus = nullptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LYNX_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return LYNX_ERR_DEVICE;
  std::call_once(g_dev_once[dev], [dev]() {
    hipDeviceProp_t prop;
    g_dev_ok[dev] = 0;
    g_dev_cus[dev] = 0;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) {
      g_dev_ok[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
      g_dev_cus[dev] = prop.multiProcessorCount;
    }
  });
  if (!g_dev_ok[dev] || g_dev_cus[dev] < 1) return LYNX_ERR_DEVICE;
  if (cus) *cus = g_dev_cus[dev];
  return LYNX_OK;
}

int check_planes(const lynx_planes *pl, bool need_residual) {
  if (!pl || !pl->anchor || !pl->page_min || !pl->page_range || !pl->chunk_mean ||
      !pl->chunk_maxabs || (need_residual && !pl->residual))
    return LYNX_ERR_NULL_ARG;
  if (!aligned16(pl->anchor) || !aligned16(pl->page_min) || !aligned16(pl->page_range) ||
      !aligned16(pl->chunk_mean) || !aligned16(pl->chunk_maxabs) ||
      (need_residual && !aligned16(pl->residual)))
    return LYNX_ERR_MISALIGNED;
  return LYNX_OK;
}

PlanesArg to_arg(const lynx_planes *pl) {
  PlanesArg a;
  a.anchor = pl->anchor;
  a.residual = pl->residual;
  a.page_min = pl->page_min;
  a.page_range = pl->page_range;
  a.chunk_mean = pl->chunk_mean;
  a.chunk_maxabs = pl->chunk_maxabs;
  return a;
}

int check_tile_shape(int64_t num_pages, int32_t heads, int32_t head_dim, int32_t role) {
  if (head_dim != LYNX_HEAD_DIM || heads < 1 || heads > LYNX_MAX_KV_HEADS || num_pages < 0)
    return LYNX_ERR_BAD_SHAPE;
  if (num_pages * static_cast<int64_t>(heads) > 0x7FFFFFFFLL) return LYNX_ERR_BAD_SHAPE;
  if (role != LYNX_ROLE_KEY && role != LYNX_ROLE_VALUE) return LYNX_ERR_BAD_ARG;
  return LYNX_OK;
}

int dequant_common(const lynx_planes *in, int64_t num_pages, int32_t heads, int32_t head_dim,
                   int32_t role, float *out, void *stream, bool full) {
  int rc = check_tile_shape(num_pages, heads, head_dim, role);
  if (rc) return rc;
  if (num_pages == 0) return LYNX_OK;
  if (!out) return LYNX_ERR_NULL_ARG;
  rc = check_planes(in, full);
  if (rc) return rc;
  if (!aligned16(out)) return LYNX_ERR_MISALIGNED;
  rc = check_device();
  if (rc) return rc;
  PlanesArg a = to_arg(in);
  if (!full) a.residual = nullptr;
  const hipError_t e = lynx::launch_dequant(a, num_pages, heads, role, full, out,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LYNX_OK : LYNX_ERR_HIP;
}

int attention_common(const uint16_t *q, const lynx_planes *k, const lynx_planes *v,
                     const int32_t *block_table, const int32_t *seq_lens, int32_t batch,
                     int32_t heads, int32_t q_heads, int32_t head_dim, int32_t max_pages,
                     int64_t pool_pages, float sm_scale, float *out, float *scores, void *workspace,
                     size_t workspace_bytes, void *stream, bool full, int anchor_bits = 4) {
  if (head_dim != LYNX_HEAD_DIM || batch < 0 || heads < 1 || q_heads < heads ||
      q_heads % heads != 0 || q_heads / heads > LYNX_MAX_GROUP || max_pages < 1)
    return LYNX_ERR_BAD_SHAPE;
  // cut streams are read by the matrix-core kernel (GQA groups up to 8)
  if (anchor_bits != 4 && !lynx::attention_mfma_supported(q_heads / heads)) return LYNX_ERR_BAD_SHAPE;
  // grid sizes: the combine launches 4 blocks per (request, query head)
  if (static_cast<int64_t>(batch) * q_heads * 4 > 0x7FFFFFFFLL) return LYNX_ERR_BAD_SHAPE;
  if (pool_pages < 0 || pool_pages * static_cast<int64_t>(heads) > 0x7FFFFFFFLL)
    return LYNX_ERR_BAD_SHAPE;
  if (!block_table && static_cast<int64_t>(batch) * max_pages > pool_pages)
    return LYNX_ERR_BAD_SHAPE;
  if (batch == 0) return LYNX_OK;
  if (!q || !out) return LYNX_ERR_NULL_ARG;
  int rc = check_planes(k, full);
  if (rc) return rc;
  rc = check_planes(v, full);
  if (rc) return rc;
  if (!aligned16(q) || !aligned16(out) || (scores && !aligned16(scores)) ||
      (block_table && !aligned16(block_table)) || (seq_lens && !aligned16(seq_lens)))
    return LYNX_ERR_MISALIGNED;
  lynx::AttnShape s = lynx::attention_shape(batch, heads, q_heads, max_pages);
  s.pool_pages = pool_pages;
  if (static_cast<int64_t>(batch) * heads * s.splits > 0x7FFFFFFFLL) return LYNX_ERR_BAD_SHAPE;
  const size_t need = lynx::attention_workspace_bytes(s);
  if (!workspace || workspace_bytes < need) return LYNX_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LYNX_ERR_MISALIGNED;
  rc = check_device();
  if (rc) return rc;
  PlanesArg ka = to_arg(k), va = to_arg(v);
  if (!full) {
    ka.residual = nullptr;
    va.residual = nullptr;
  }
  const hipError_t e = lynx::launch_attention(q, ka, va, block_table, seq_lens, s, sm_scale,
                                              full, out, scores, workspace,
                                              static_cast<hipStream_t>(stream), anchor_bits);
  return e == hipSuccess ? LYNX_OK : LYNX_ERR_HIP;
}

int tail_attention_common(const uint16_t *q, int32_t tq, const lynx_planes *k,
                          const lynx_planes *v, const int32_t *block_table,
                          const int32_t *page_tokens, const uint16_t *tail_k,
                          const uint16_t *tail_v, const int32_t *tail_len, int32_t batch,
                          int32_t heads, int32_t q_heads, int32_t head_dim, int32_t max_pages,
                          int64_t pool_pages, float sm_scale, float *out, void *workspace,
                          size_t workspace_bytes, void *stream, bool full) {
  if (head_dim != LYNX_HEAD_DIM || batch < 0 || tq < 1 || tq > LYNX_MAX_QUERY_TOKENS ||
      heads < 1 || q_heads < heads || q_heads % heads != 0 ||
      q_heads / heads > LYNX_MAX_GROUP || max_pages < 1)
    return LYNX_ERR_BAD_SHAPE;
  const int64_t rows = static_cast<int64_t>(batch) * tq;
  if (rows * q_heads * 4 > 0x7FFFFFFFLL) return LYNX_ERR_BAD_SHAPE;
  if (pool_pages < 0 || pool_pages * static_cast<int64_t>(heads) > 0x7FFFFFFFLL)
    return LYNX_ERR_BAD_SHAPE;
  if (!block_table && pool_pages > 0 && static_cast<int64_t>(batch) * max_pages > pool_pages)
    return LYNX_ERR_BAD_SHAPE;
  if (batch == 0) return LYNX_OK;
  if (!q || !out || !tail_k || !tail_v || !tail_len) return LYNX_ERR_NULL_ARG;
  if (pool_pages > 0) {
    int rc = check_planes(k, full);
    if (rc) return rc;
    rc = check_planes(v, full);
    if (rc) return rc;
  }
  if (!aligned16(q) || !aligned16(out) || !aligned16(tail_k) || !aligned16(tail_v) ||
      !aligned16(tail_len) || (block_table && !aligned16(block_table)) ||
      (page_tokens && !aligned16(page_tokens)))
    return LYNX_ERR_MISALIGNED;
  lynx::AttnShape s = lynx::attention_shape_tail(batch, tq, heads, q_heads, max_pages);
  s.pool_pages = pool_pages;
  if (rows * heads * s.splits > 0x7FFFFFFFLL) return LYNX_ERR_BAD_SHAPE;
  const size_t need = lynx::attention_workspace_bytes(s);
  if (!workspace || workspace_bytes < need) return LYNX_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LYNX_ERR_MISALIGNED;
  const int rc = check_device();
  if (rc) return rc;
  PlanesArg ka{}, va{};
  if (pool_pages > 0) {
    ka = to_arg(k);
    va = to_arg(v);
    if (!full) {
      ka.residual = nullptr;
      va.residual = nullptr;
    }
  }
  const hipError_t e = lynx::launch_attention_with_tail(
      q, ka, va, block_table, page_tokens, tail_k, tail_v, tail_len, LYNX_TAIL_TOKENS, s, sm_scale,
      full, out, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LYNX_OK : LYNX_ERR_HIP;
}

}  // namespace

extern "C" {

size_t lynx_plane_bytes(int64_t num_pages, int32_t num_kv_heads) {
  if (num_pages < 0 || num_kv_heads < 1) return 0;
  return static_cast<size_t>(num_pages) * num_kv_heads * lynx::kPlaneTileBytes;
}

size_t lynx_page_scale_bytes(int64_t num_pages, int32_t num_kv_heads) {
  if (num_pages < 0 || num_kv_heads < 1) return 0;
  return static_cast<size_t>(num_pages) * num_kv_heads * lynx::kDim * sizeof(float);
}

size_t lynx_chunk_scale_bytes(int64_t num_pages, int32_t num_kv_heads) {
  if (num_pages < 0 || num_kv_heads < 1) return 0;
  return static_cast<size_t>(num_pages) * num_kv_heads * lynx::kChunks * lynx::kDim *
         sizeof(float);
}

int lynx_quantize_pages(const uint16_t *kv, int64_t num_pages, int32_t num_kv_heads,
                        int32_t head_dim, int32_t role, const lynx_planes *out, void *stream) {
  int rc = check_tile_shape(num_pages, num_kv_heads, head_dim, role);
  if (rc) return rc;
  if (num_pages == 0) return LYNX_OK;
  if (!kv) return LYNX_ERR_NULL_ARG;
  rc = check_planes(out, true);
  if (rc) return rc;
  if (!aligned16(kv)) return LYNX_ERR_MISALIGNED;
  rc = check_device();
  if (rc) return rc;
  const hipError_t e = lynx::launch_encode(kv, num_pages, num_kv_heads, role, to_arg(out),
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LYNX_OK : LYNX_ERR_HIP;
}

int lynx_quantize_kv_pages(const uint16_t *k, const uint16_t *v, int64_t num_pages,
                           int32_t num_kv_heads, int32_t head_dim, const lynx_planes *k_out,
                           const lynx_planes *v_out, void *stream) {
  int rc = check_tile_shape(num_pages, num_kv_heads, head_dim, LYNX_ROLE_KEY);
  if (rc) return rc;
  if (2 * num_pages * static_cast<int64_t>(num_kv_heads) > 0x7FFFFFFFLL) return LYNX_ERR_BAD_SHAPE;
  if (num_pages == 0) return LYNX_OK;
  if (!k || !v) return LYNX_ERR_NULL_ARG;
  rc = check_planes(k_out, true);
  if (rc) return rc;
  rc = check_planes(v_out, true);
  if (rc) return rc;
  if (!aligned16(k) || !aligned16(v)) return LYNX_ERR_MISALIGNED;
  rc = check_device();
  if (rc) return rc;
  const hipError_t e = lynx::launch_encode_kv(k, v, num_pages, num_kv_heads, to_arg(k_out),
                                              to_arg(v_out), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LYNX_OK : LYNX_ERR_HIP;
}

int lynx_quantize_pages_split(const uint16_t *kv, int64_t num_pages, int32_t num_kv_heads,
                              int32_t head_dim, int32_t role, int32_t anchor_bits,
                              const lynx_planes *out, void *stream) {
  int rc = check_tile_shape(num_pages, num_kv_heads, head_dim, role);
  if (rc) return rc;
  if (anchor_bits < 1 || anchor_bits > 7) return LYNX_ERR_BAD_ARG;
  if (num_pages == 0) return LYNX_OK;
  if (!kv) return LYNX_ERR_NULL_ARG;
  rc = check_planes(out, true);
  if (rc) return rc;
  if (!aligned16(kv)) return LYNX_ERR_MISALIGNED;
  rc = check_device();
  if (rc) return rc;
  const hipError_t e = lynx::launch_encode(kv, num_pages, num_kv_heads, role, to_arg(out),
                                           static_cast<hipStream_t>(stream), anchor_bits);
  return e == hipSuccess ? LYNX_OK : LYNX_ERR_HIP;
}

int lynx_dequantize_anchor(const lynx_planes *in, int64_t num_pages, int32_t num_kv_heads,
                           int32_t head_dim, int32_t role, float *out, void *stream) {
  return dequant_common(in, num_pages, num_kv_heads, head_dim, role, out, stream, false);
}

int lynx_dequantize_full(const lynx_planes *in, int64_t num_pages, int32_t num_kv_heads,
                         int32_t head_dim, int32_t role, float *out, void *stream) {
  return dequant_common(in, num_pages, num_kv_heads, head_dim, role, out, stream, true);
}

size_t lynx_decode_attention_workspace_size(int32_t batch, int32_t num_kv_heads,
                                            int32_t num_q_heads, int32_t head_dim,
                                            int32_t max_pages_per_seq) {
  if (head_dim != LYNX_HEAD_DIM || batch < 0 || num_kv_heads < 1 ||
      num_q_heads < num_kv_heads || num_q_heads % num_kv_heads != 0 ||
      num_q_heads / num_kv_heads > LYNX_MAX_GROUP || max_pages_per_seq < 1)
    return 0;
  return lynx::attention_workspace_bytes(
      lynx::attention_shape(batch, num_kv_heads, num_q_heads, max_pages_per_seq));
}

int lynx_decode_attention_anchor(const uint16_t *q, const lynx_planes *k, const lynx_planes *v,
                                 const int32_t *block_table, const int32_t *seq_lens,
                                 int32_t batch, int32_t num_kv_heads, int32_t num_q_heads,
                                 int32_t head_dim, int32_t max_pages_per_seq,
                                 int64_t pool_pages, float sm_scale,
                                 float *out, float *scores, void *workspace,
                                 size_t workspace_bytes, void *stream) {
  return attention_common(q, k, v, block_table, seq_lens, batch, num_kv_heads, num_q_heads,
                          head_dim, max_pages_per_seq, pool_pages, sm_scale, out, scores,
                          workspace,
                          workspace_bytes, stream, false);
}

int lynx_decode_attention_full(const uint16_t *q, const lynx_planes *k, const lynx_planes *v,
                               const int32_t *block_table, const int32_t *seq_lens,
                               int32_t batch, int32_t num_kv_heads, int32_t num_q_heads,
                               int32_t head_dim, int32_t max_pages_per_seq,
                               int64_t pool_pages, float sm_scale,
                               float *out, float *scores, void *workspace,
                               size_t workspace_bytes, void *stream) {
  return attention_common(q, k, v, block_table, seq_lens, batch, num_kv_heads, num_q_heads,
                          head_dim, max_pages_per_seq, pool_pages, sm_scale, out, scores,
                          workspace,
                          workspace_bytes, stream, true);
}

int lynx_decode_attention_full_static(const uint16_t *q, const lynx_planes *k,
                                      const lynx_planes *v, const int32_t *block_table,
                                      const int32_t *seq_lens, int32_t batch,
                                      int32_t num_kv_heads, int32_t num_q_heads, int32_t head_dim,
                                      int32_t max_pages_per_seq, int64_t pool_pages,
                                      float sm_scale, float *out, float *scores, void *stream) {
  // shape errors first, with the same checks and codes as the workspace call
  if (head_dim != LYNX_HEAD_DIM || batch < 0 || num_kv_heads < 1 || num_q_heads < num_kv_heads ||
      num_q_heads % num_kv_heads != 0 || num_q_heads / num_kv_heads > LYNX_MAX_GROUP ||
      max_pages_per_seq < 1)
    return LYNX_ERR_BAD_SHAPE;
  if (batch == 0)
    return attention_common(q, k, v, block_table, seq_lens, batch, num_kv_heads, num_q_heads,
                            head_dim, max_pages_per_seq, pool_pages, sm_scale, out, scores,
                            nullptr, 0, stream, true);
  const size_t need = lynx::attention_workspace_bytes(
      lynx::attention_shape(batch, num_kv_heads, num_q_heads, max_pages_per_seq));
  if (need > lynx::scratch_capacity()) return LYNX_ERR_SCRATCH;
  int rc = check_device();
  if (rc) return rc;
  void *scratch = nullptr;
  if (lynx::scratch_address(&scratch) != hipSuccess) return LYNX_ERR_HIP;
  return attention_common(q, k, v, block_table, seq_lens, batch, num_kv_heads, num_q_heads,
                          head_dim, max_pages_per_seq, pool_pages, sm_scale, out, scores, scratch,
                          lynx::scratch_capacity(), stream, true);
}

size_t lynx_split_stream_bytes(int64_t num_pages, int32_t num_kv_heads, int32_t bits) {
  if (num_pages < 0 || num_kv_heads < 1 || bits < 1 || bits > 8) return 0;
  return static_cast<size_t>(num_pages) * num_kv_heads * static_cast<size_t>(bits) * 4096u;
}

int lynx_split_planes(const lynx_planes *in, int64_t num_pages, int32_t num_kv_heads,
                      int32_t head_dim, int32_t anchor_bits, uint8_t *anchor_out,
                      uint8_t *residual_out, void *stream) {
  int rc = check_tile_shape(num_pages, num_kv_heads, head_dim, LYNX_ROLE_KEY);
  if (rc) return rc;
  if (num_pages * static_cast<int64_t>(num_kv_heads) * 4 > 0x7FFFFFFFLL) return LYNX_ERR_BAD_SHAPE;
  if (anchor_bits < 1 || anchor_bits > 7) return LYNX_ERR_BAD_ARG;
  if (num_pages == 0) return LYNX_OK;
  if (!in || !in->anchor || !in->residual || !anchor_out || !residual_out) return LYNX_ERR_NULL_ARG;
  if (!aligned16(in->anchor) || !aligned16(in->residual) || !aligned16(anchor_out) ||
      !aligned16(residual_out))
    return LYNX_ERR_MISALIGNED;
  rc = check_device();
  if (rc) return rc;
  const hipError_t e = lynx::launch_split_planes(to_arg(in), num_pages, num_kv_heads, anchor_bits,
                                                 anchor_out, residual_out,
                                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LYNX_OK : LYNX_ERR_HIP;
}

int lynx_dequantize_split(const uint8_t *anchor, const uint8_t *residual, int32_t anchor_bits,
                          const lynx_planes *scales, int64_t num_pages, int32_t num_kv_heads,
                          int32_t head_dim, int32_t role, float *out, void *stream) {
  int rc = check_tile_shape(num_pages, num_kv_heads, head_dim, role);
  if (rc) return rc;
  if (num_pages * static_cast<int64_t>(num_kv_heads) * 4 > 0x7FFFFFFFLL) return LYNX_ERR_BAD_SHAPE;
  if (anchor_bits < 1 || anchor_bits > 7) return LYNX_ERR_BAD_ARG;
  if (num_pages == 0) return LYNX_OK;
  if (!anchor || !out || !scales || !scales->page_min || !scales->page_range ||
      !scales->chunk_mean || !scales->chunk_maxabs)
    return LYNX_ERR_NULL_ARG;
  if (!aligned16(anchor) || (residual && !aligned16(residual)) || !aligned16(out) ||
      !aligned16(scales->page_min) || !aligned16(scales->page_range) ||
      !aligned16(scales->chunk_mean) || !aligned16(scales->chunk_maxabs))
    return LYNX_ERR_MISALIGNED;
  rc = check_device();
  if (rc) return rc;
  PlanesArg sc{};
  sc.page_min = scales->page_min;
  sc.page_range = scales->page_range;
  sc.chunk_mean = scales->chunk_mean;
  sc.chunk_maxabs = scales->chunk_maxabs;
  const hipError_t e = lynx::launch_dequant_split(anchor, residual, anchor_bits, sc, num_pages,
                                                  num_kv_heads, role, out,
                                                  static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LYNX_OK : LYNX_ERR_HIP;
}

int lynx_decode_attention_split(const uint16_t *q, const lynx_planes *k, const lynx_planes *v,
                                int32_t anchor_bits, int32_t full, const int32_t *block_table,
                                const int32_t *seq_lens, int32_t batch, int32_t num_kv_heads,
                                int32_t num_q_heads, int32_t head_dim, int32_t max_pages_per_seq,
                                int64_t pool_pages, float sm_scale, float *out, float *scores,
                                void *workspace, size_t workspace_bytes, void *stream) {
  if (anchor_bits < 1 || anchor_bits > 7) return LYNX_ERR_BAD_ARG;
  return attention_common(q, k, v, block_table, seq_lens, batch, num_kv_heads, num_q_heads,
                          head_dim, max_pages_per_seq, pool_pages, sm_scale, out, scores,
                          workspace, workspace_bytes, stream, full != 0, anchor_bits);
}

size_t lynx_verify_attention_workspace_size(int32_t batch, int32_t tq, int32_t num_kv_heads,
                                            int32_t num_q_heads, int32_t head_dim,
                                            int32_t max_pages_per_seq) {
  if (head_dim != LYNX_HEAD_DIM || batch < 0 || tq < 1 || tq > LYNX_MAX_QUERY_TOKENS ||
      num_kv_heads < 1 || num_q_heads < num_kv_heads || num_q_heads % num_kv_heads != 0 ||
      num_q_heads / num_kv_heads > LYNX_MAX_GROUP || max_pages_per_seq < 1)
    return 0;
  return lynx::attention_workspace_bytes(
      lynx::attention_shape_tail(batch, tq, num_kv_heads, num_q_heads, max_pages_per_seq));
}

int lynx_verify_attention(const uint16_t *q, int32_t tq, const lynx_planes *k, const lynx_planes *v,
                          const int32_t *block_table, const int32_t *page_tokens,
                          const uint16_t *tail_k, const uint16_t *tail_v, const int32_t *tail_len,
                          int32_t batch, int32_t num_kv_heads, int32_t num_q_heads,
                          int32_t head_dim, int32_t max_pages_per_seq, int64_t pool_pages,
                          float sm_scale, float *out, void *workspace, size_t workspace_bytes,
                          void *stream) {
  return tail_attention_common(q, tq, k, v, block_table, page_tokens, tail_k, tail_v, tail_len,
                               batch, num_kv_heads, num_q_heads, head_dim, max_pages_per_seq,
                               pool_pages, sm_scale, out, workspace, workspace_bytes, stream, true);
}

int lynx_draft_attention(const uint16_t *q, int32_t tq, const lynx_planes *k, const lynx_planes *v,
                         const int32_t *block_table, const int32_t *page_tokens,
                         const uint16_t *tail_k, const uint16_t *tail_v, const int32_t *tail_len,
                         int32_t batch, int32_t num_kv_heads, int32_t num_q_heads,
                         int32_t head_dim, int32_t max_pages_per_seq, int64_t pool_pages,
                         float sm_scale, float *out, void *workspace, size_t workspace_bytes,
                         void *stream) {
  return tail_attention_common(q, tq, k, v, block_table, page_tokens, tail_k, tail_v, tail_len,
                               batch, num_kv_heads, num_q_heads, head_dim, max_pages_per_seq,
                               pool_pages, sm_scale, out, workspace, workspace_bytes, stream, false);
}

const char *lynx_status_string(int status) {
  switch (status) {
    case LYNX_OK: return "ok";
    case LYNX_ERR_NULL_ARG: return "a required pointer is NULL";
    case LYNX_ERR_BAD_SHAPE: return "unsupported shape";
    case LYNX_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case LYNX_ERR_WORKSPACE: return "workspace missing or too small";
    case LYNX_ERR_HIP: return "HIP runtime error";
    case LYNX_ERR_DEVICE: return "current device is not gfx950";
    case LYNX_ERR_BAD_ARG: return "invalid argument value";
    case LYNX_ERR_SCRATCH: return "shape needs more than the library's static scratch";
    default: return "unknown status";
  }
}

void lynx_code_thresholds(float *out128) {
  if (!out128) return;
  const lynx::CodeTable &t = lynx::code_table();
  for (int k = 0; k < 128; ++k) out128[k] = t.t[k];
}

void lynx_decode_table(float *out256) {
  if (!out256) return;
  const lynx::DecodeTable &t = lynx::decode_table();
  for (int k = 0; k < 256; ++k) out256[k] = t.y[k];
}

int lynx_selftest_code_map(uint32_t begin_bits, uint32_t end_bits,
                           unsigned long long *mismatches, void *stream) {
  if (!mismatches) return LYNX_ERR_NULL_ARG;
  if (end_bits > 0x40000000u || begin_bits > end_bits) return LYNX_ERR_BAD_ARG;
  if (begin_bits == end_bits) return LYNX_OK;
  const int rc = check_device();
  if (rc) return rc;
  const hipError_t e = lynx::launch_code_map_check(begin_bits, end_bits, mismatches,
                                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LYNX_OK : LYNX_ERR_HIP;
}

const char *lynx_version(void) { return "liblynx 0.1 (gfx950)"; }

}  // extern "C"
