/*
 * lynx.h -- C ABI of liblynx, the MI355X (gfx950) implementation of Lynx
 * progressive KV-cache quantization.
 *
 * What is computed (page "Lynx: the KV cache does not have to arrive whole",
 * section 3 "The quantizer", and section 4 "Speculation at the communication
 * boundary"):
 *
 *   encode, per page of 256 tokens, per KV head h, per channel d:
 *     mn = min_t x, rg = fl32(max_t x - mn), inv_rg = fl32(1/rg) (0 if 0)
 *     x'_t = fl32(fl32(x_t - mn) * inv_rg)                    (map to [0,1])
 *     per chunk c of C = 32 tokens:
 *       mu = fl32(exact_sum(x'_t) / 32), d_t = fl32(x'_t - mu)
 *       s  = max_t |d_t|,  inv_s = fl32(1/s) (0 if s = 0)
 *       u_t = min(1, fl32(|d_t| * inv_s))                     (y = sign(d) u)
 *     m_t = round_half_up(127 * ln(1 + 255 u_t) / ln 256)      (0..127)
 *     q_t = d_t < 0 ? -m_t - 1 : m_t                           (int8, sign-aware)
 *     anchor a_t = q_t >> 4 (int4, -8..7), residual r_t = q_t & 15 (uint4)
 *   decode:
 *     draft code 16 a + 7, full code 16 a + r;  m = code >= 0 ? code : ~code
 *     yhat = sign * (256^(m/127) - 1) / 255
 *     xhat = mn + rg * (mu + s * yhat)
 *   decode attention (page "LLM KV cache quantization", sections "The
 *   architecture" and "End-to-end flow"): one query token per request,
 *   scores = sm_scale * q . khat_t, softmax over all cached tokens, output =
 *   softmax-weighted sum of vhat_t; query head j reads KV head j / (Hq / H).
 *   The compact planes are expanded only in registers.
 *
 * fl32() is one IEEE binary32 operation rounded to nearest even (no fused
 * multiply-add).  exact_sum() is the exact sum, which the encoder forms in
 * binary64: that sum is exact whenever every nonzero x'_t of the chunk is at
 * least 2^-24 (the 32 terms then span at most 53 bits), so the scales and
 * codes are bit-exact under that condition.  A chunk that breaks it (a
 * value above the page minimum by less than 2^-24 of the page range) may
 * see its sum rounded once more: its mean is then
 * within one ulp of the exact one and its codes within one level.
 * alpha = 255, 127 levels, C = 32, fp32 scales and the +7 draft point are
 * the readings documented with the repository.
 *
 * Conventions for every entry point:
 *   - all pointers are DEVICE pointers unless stated otherwise; buffers are
 *     owned and allocated by the caller; the library never allocates device
 *     memory and never synchronizes;
 *   - every call is asynchronous on `stream` (a hipStream_t; NULL = default);
 *   - inputs must be finite; the output for NaN/Inf input is unspecified;
 *   - calls return LYNX_OK (0) or a negative lynx_status; argument errors are
 *     detected on the host before any launch; no exception crosses the ABI;
 *   - calls are reentrant; the library holds no mutable state after its
 *     one-time host-side table set-up.
 */
#ifndef LYNX_H
#define LYNX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LYNX_PAGE_TOKENS 256 /* tokens per page (section 3) */
#define LYNX_CHUNK_TOKENS 32 /* C, tokens per chunk (section 3) */
#define LYNX_CHUNKS_PER_PAGE 8
#define LYNX_HEAD_DIM 128    /* the only head_dim the library supports */
#define LYNX_MAX_GROUP 16    /* largest supported Hq / H */
#define LYNX_MAX_KV_HEADS 65535  /* largest H of an encoded tensor (a page of
                                    256 tokens stays below 4 GiB) */
#define LYNX_MAX_QUERY_TOKENS 64 /* largest number of speculative tokens a
                                    verify pass scores at once */
#define LYNX_TAIL_TOKENS 320     /* capacity of a request's bf16 tail: a page
                                    not yet full plus the speculative tokens */
#define LYNX_STATIC_SCRATCH_BYTES (32u << 20) /* library-owned scratch of
                                    lynx_decode_attention_full_static, per GPU */

typedef enum lynx_status {
    LYNX_OK = 0,
    LYNX_ERR_NULL_ARG = -1,      /* a required pointer is NULL */
    LYNX_ERR_BAD_SHAPE = -2,     /* head_dim != 128, H < 1 or > 65535, P < 0, Hq % H,
                                    Hq / H > 16, batch < 0, a grid beyond
                                    2^31 - 1 blocks (P*H tiles, 4*B*Hq, or
                                    B*H*splits), ... */
    LYNX_ERR_MISALIGNED = -3,    /* a pointer is not 16-byte aligned */
    LYNX_ERR_WORKSPACE = -4,     /* workspace NULL or smaller than required */
    LYNX_ERR_HIP = -5,           /* a HIP runtime call or launch failed */
    LYNX_ERR_DEVICE = -6,        /* current device is not gfx950 */
    LYNX_ERR_BAD_ARG = -7,       /* unknown role or other invalid value */
    LYNX_ERR_SCRATCH = -8        /* the shape needs more than the library's
                                    static scratch (LYNX_STATIC_SCRATCH_BYTES) */
} lynx_status;

/*
 * Plane roles.  Keys and values are quantized identically (the pages make no
 * distinction); only the byte layout of the two nibble planes differs, each
 * chosen so that decode attention reads its operand tiles with contiguous
 * 16-byte loads.
 *
 * LYNX_ROLE_KEY   anchor/residual: uint8 [P][H][256 tokens][64]
 *                 byte j of token row t holds channel 2j (low nibble) and
 *                 channel 2j+1 (high nibble).
 * LYNX_ROLE_VALUE anchor/residual: uint8 [P][H][8 chunks][128 channels][16]
 *                 the 16 bytes of (chunk c, channel d) hold that channel's 32
 *                 tokens of chunk c as 4 little-endian 32-bit words; word w
 *                 holds, in nibbles 0..7 (least significant first), the
 *                 tokens 4w, 4w+1, 4w+2, 4w+3, 16+4w, 16+4w+1, 16+4w+2,
 *                 16+4w+3 of the chunk.
 * Anchor nibbles are two's complement int4 (a & 15); residual nibbles are
 * uint4.  Both roles share the scale layout below.
 */
typedef enum lynx_role { LYNX_ROLE_KEY = 0, LYNX_ROLE_VALUE = 1 } lynx_role;

/* One encoded K or V tensor of one layer: P pages x H heads x 128 channels. */
typedef struct lynx_planes {
    uint8_t *anchor;     /* 0.5 B/element, layout by role (see above) */
    uint8_t *residual;   /* 0.5 B/element; may be NULL for anchor-only reads */
    float *page_min;     /* [P][H][128]    fp32 page minimum mn */
    float *page_range;   /* [P][H][128]    fp32 page range rg */
    float *chunk_mean;   /* [P][H][8][128] fp32 chunk mean mu (normalised) */
    float *chunk_maxabs; /* [P][H][8][128] fp32 chunk max-abs s (normalised) */
} lynx_planes;

/* Byte sizes of one plane and of the scale arrays for P pages, H heads. */
size_t lynx_plane_bytes(int64_t num_pages, int32_t num_kv_heads);
size_t lynx_page_scale_bytes(int64_t num_pages, int32_t num_kv_heads);
size_t lynx_chunk_scale_bytes(int64_t num_pages, int32_t num_kv_heads);

/*
 * Encoder (section 3, all four stages) and plane packer.
 *   kv    bf16 bit patterns [P][256][H][128] (a page is 256 tokens x KV heads
 *         x head_dim, in paged order), 16-byte aligned
 *   role  LYNX_ROLE_KEY or LYNX_ROLE_VALUE: plane layout to write
 *   out   every member non-NULL and 16-byte aligned; written completely
 * P = 0 is a no-op (no pointer is inspected).  Errors: NULL_ARG, BAD_SHAPE,
 * MISALIGNED, BAD_ARG, DEVICE, HIP.
 */
int lynx_quantize_pages(const uint16_t *kv, int64_t num_pages,
                        int32_t num_kv_heads, int32_t head_dim, int32_t role,
                        const lynx_planes *out, void *stream);

/*
 * The K and the V tensor of one layer in one call (section 3's quantizer on
 * both caches of a layer): the same planes, byte for byte, as
 * lynx_quantize_pages(k, ..., LYNX_ROLE_KEY, k_out) followed by
 * lynx_quantize_pages(v, ..., LYNX_ROLE_VALUE, v_out), from one kernel
 * launch, so that the V tiles start as the K tiles finish.
 *   k, v          bf16 bit patterns [P][256][H][128] each, 16-byte aligned
 *   k_out, v_out  planes as for one tensor (every member non-NULL, 16-byte
 *                 aligned); the four inputs and outputs must not overlap
 * 2 * P * H must not exceed 2^31 - 1.  P = 0 is a no-op.  Errors: NULL_ARG,
 * BAD_SHAPE, MISALIGNED, DEVICE, HIP.
 */
int lynx_quantize_kv_pages(const uint16_t *k, const uint16_t *v, int64_t num_pages,
                           int32_t num_kv_heads, int32_t head_dim,
                           const lynx_planes *k_out, const lynx_planes *v_out,
                           void *stream);

/*
 * Standalone dequantizers (section 4: the draft reads the anchor stream
 * alone; the refined cache reads anchor and residual).  `in` as written by
 * lynx_quantize_pages with the same role; the anchor variant never reads
 * in->residual (it may be NULL).  out: fp32 [P][256][H][128] (the input
 * layout of the encoder).  P = 0 is a no-op.  Errors as for the encoder.
 */
int lynx_dequantize_anchor(const lynx_planes *in, int64_t num_pages,
                           int32_t num_kv_heads, int32_t head_dim,
                           int32_t role, float *out, void *stream);
int lynx_dequantize_full(const lynx_planes *in, int64_t num_pages,
                         int32_t num_kv_heads, int32_t head_dim, int32_t role,
                         float *out, void *stream);

/*
 * Fused-dequant single-query GQA decode attention (anchor-only = draft, or
 * anchor + residual = Q_full).  K planes must have been written with
 * LYNX_ROLE_KEY and V planes with LYNX_ROLE_VALUE.
 *   q            bf16 bits [B][Hq][128]
 *   k, v         encoded pools of pages (any number of pages)
 *   block_table  int32 [B][max_pages_per_seq]: pool page index of each
 *                logical page of each request; NULL = request b owns pool
 *                pages b*max_pages_per_seq .. + n_b - 1 (then
 *                batch*max_pages_per_seq must not exceed pool_pages)
 *   pool_pages   number of pages in the k and v pools; a block-table entry
 *                outside [0, pool_pages) is skipped (its page contributes
 *                nothing), so no out-of-bounds read can happen
 *   seq_lens     int32 [B] tokens per request, a multiple of 256 in
 *                [256, 256*max_pages_per_seq]; NULL = every request is
 *                max_pages_per_seq pages long.  Device memory, read on device:
 *                values outside the range make the output unspecified (no
 *                out-of-bounds access happens: lengths are clamped).
 *   sm_scale     softmax scale applied to q . k (e.g. 1/sqrt(128))
 *   out          fp32 [B][Hq][128]
 *   scores       optional fp32 [B][Hq][256*max_pages_per_seq]: the scaled
 *                logits, for ranking comparisons; NULL = not written
 *   workspace    device scratch of at least
 *                lynx_decode_attention_workspace_size(...) bytes, 16-byte
 *                aligned; contents need not be initialised.  Calls that
 *                overlap in time must not share a workspace.
 * The anchor variant never reads k->residual or v->residual.  batch = 0 is
 * a no-op once the shape arguments are valid (no pointer is inspected).
 * Errors: NULL_ARG, BAD_SHAPE, MISALIGNED, WORKSPACE, DEVICE, HIP.
 */
size_t lynx_decode_attention_workspace_size(int32_t batch,
                                            int32_t num_kv_heads,
                                            int32_t num_q_heads,
                                            int32_t head_dim,
                                            int32_t max_pages_per_seq);
int lynx_decode_attention_anchor(const uint16_t *q, const lynx_planes *k,
                                 const lynx_planes *v,
                                 const int32_t *block_table,
                                 const int32_t *seq_lens, int32_t batch,
                                 int32_t num_kv_heads, int32_t num_q_heads,
                                 int32_t head_dim, int32_t max_pages_per_seq,
                                 int64_t pool_pages, float sm_scale,
                                 float *out, float *scores,
                                 void *workspace, size_t workspace_bytes,
                                 void *stream);
int lynx_decode_attention_full(const uint16_t *q, const lynx_planes *k,
                               const lynx_planes *v,
                               const int32_t *block_table,
                               const int32_t *seq_lens, int32_t batch,
                               int32_t num_kv_heads, int32_t num_q_heads,
                               int32_t head_dim, int32_t max_pages_per_seq,
                               int64_t pool_pages, float sm_scale,
                               float *out, float *scores,
                               void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * lynx_decode_attention_full without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The split partials go to a
 * library-owned static device array of LYNX_STATIC_SCRATCH_BYTES that every
 * GPU the library runs on holds until the process ends; the call allocates
 * nothing.  Arguments, layouts and results are those of
 * lynx_decode_attention_full (the same kernels), on the CURRENT device (the
 * stream must belong to it).
 *   returns LYNX_ERR_SCRATCH, before any launch, when
 *   lynx_decode_attention_workspace_size() of the shape exceeds
 *   LYNX_STATIC_SCRATCH_BYTES; LYNX_ERR_HIP if the scratch's device address
 *   cannot be looked up.
 * Every call on a GPU shares that GPU's scratch, whose contents persist
 * between calls: a call writes every partial it reads, so nothing needs
 * clearing, but calls that overlap on one GPU (concurrent streams, or
 * threads) race and must be serialized by the caller.
 */
int lynx_decode_attention_full_static(const uint16_t *q, const lynx_planes *k,
                                      const lynx_planes *v,
                                      const int32_t *block_table,
                                      const int32_t *seq_lens, int32_t batch,
                                      int32_t num_kv_heads, int32_t num_q_heads,
                                      int32_t head_dim, int32_t max_pages_per_seq,
                                      int64_t pool_pages, float sm_scale,
                                      float *out, float *scores, void *stream);

/*
 * Other cuts of the 8-bit code (page "Lynx: the KV cache does not have to
 * arrive whole", section 3 cuts it 4 + 4; section 7 names 6 + 2, 2 + 6 and
 * 5 + 3 as untried).  A b + (8 - b) cut keeps the top b bits of each code as
 * the anchor (two's complement, -2^(b-1) .. 2^(b-1) - 1) and the low 8 - b
 * bits as the residual; the draft code of anchor a is
 * a * 2^(8-b) + 2^(7-b) - 1, the round-half-down centre of its codes.
 * Streams: element k of a (page, head) tile -- the k-th nibble of the
 * tile's 4-bit planes, in their role-dependent order -- occupies bits
 * k*b .. k*b + b - 1 (least significant first) of the tile's anchor stream
 * and bits k*(8-b) .. of its residual stream; tiles follow each other
 * page-major as in the 4-bit planes.
 *   lynx_split_stream_bytes  bytes of one stream of `bits` bits per element
 *                           for P pages x H heads (bits * 4096 per tile);
 *                           0 for an invalid shape
 *   lynx_split_planes        re-cut planes written by lynx_quantize_pages
 *                           (anchor and residual read) into the two streams
 *   lynx_dequantize_split    fp32 [P][256][H][128] from the streams: full
 *                           (residual given; bit-identical to
 *                           lynx_dequantize_full) or draft (residual NULL);
 *                           only the four scale pointers of `scales` are read
 * anchor_bits: 1 .. 7.  Pointers are device pointers, 16-byte aligned.
 * P = 0 is a no-op.  Errors: NULL_ARG, BAD_SHAPE (also P*H*4 >= 2^31),
 * BAD_ARG (anchor_bits, role), MISALIGNED, DEVICE, HIP.
 */
size_t lynx_split_stream_bytes(int64_t num_pages, int32_t num_kv_heads, int32_t bits);
/*
 * lynx_quantize_pages_split: lynx_quantize_pages writing a b + (8 - b) cut
 * directly: out->anchor receives the anchor stream (anchor_bits * 4096
 * bytes per tile), out->residual the residual stream ((8 - anchor_bits) *
 * 4096), the scale pointers the scales; byte-identical to
 * lynx_quantize_pages followed by lynx_split_planes.  anchor_bits 1 .. 7
 * (4: the 4-bit planes).  Errors: as lynx_quantize_pages, plus BAD_ARG for
 * anchor_bits.
 */
int lynx_quantize_pages_split(const uint16_t *kv, int64_t num_pages,
                              int32_t num_kv_heads, int32_t head_dim,
                              int32_t role, int32_t anchor_bits,
                              const lynx_planes *out, void *stream);
int lynx_split_planes(const lynx_planes *in, int64_t num_pages,
                      int32_t num_kv_heads, int32_t head_dim,
                      int32_t anchor_bits, uint8_t *anchor_out,
                      uint8_t *residual_out, void *stream);
int lynx_dequantize_split(const uint8_t *anchor, const uint8_t *residual,
                          int32_t anchor_bits, const lynx_planes *scales,
                          int64_t num_pages, int32_t num_kv_heads,
                          int32_t head_dim, int32_t role, float *out,
                          void *stream);

/*
 * Fused-dequant decode attention over b + (8 - b) streams (page "Lynx: the
 * KV cache does not have to arrive whole", section 4: drafts on the anchor
 * stream alone, the full code on both; section 7: other cuts).  Arguments
 * as lynx_decode_attention_anchor / _full, except:
 *   k, v         k->anchor and v->anchor are anchor streams of anchor_bits
 *                bits per element, k->residual and v->residual residual
 *                streams of 8 - anchor_bits bits (read only when full),
 *                both as written by lynx_split_planes from K (role key) and
 *                V (role value) planes; the scale pointers are those of the
 *                planes they were cut from
 *   anchor_bits  1 .. 7 (4: the streams are the 4-bit planes themselves)
 *   full         0: the draft, the anchor's round-half-down centre code
 *                a * 2^(8-b) + 2^(7-b) - 1; otherwise the full code (equal
 *                to lynx_decode_attention_full over the uncut planes)
 * The workspace size is lynx_decode_attention_workspace_size's.  GQA groups
 * up to 8 only (BAD_SHAPE otherwise).  Errors: as the decode calls, plus
 * BAD_ARG for anchor_bits.
 */
int lynx_decode_attention_split(const uint16_t *q, const lynx_planes *k,
                                const lynx_planes *v, int32_t anchor_bits,
                                int32_t full, const int32_t *block_table,
                                const int32_t *seq_lens, int32_t batch,
                                int32_t num_kv_heads, int32_t num_q_heads,
                                int32_t head_dim, int32_t max_pages_per_seq,
                                int64_t pool_pages, float sm_scale,
                                float *out, float *scores,
                                void *workspace, size_t workspace_bytes,
                                void *stream);

/*
 * Attention of the tq newest tokens of each request over its compact pages
 * and its bf16 tail (page "Lynx: the KV cache does not have to arrive
 * whole", section 4: drafts run on the anchor stream alone, the refined
 * cache Q_full verifies them).  Pages are quantized whole (section 3), so
 * the tokens that have not filled a page yet -- including the speculative
 * tokens being scored -- stay in bf16 in the tail until their page fills.
 * lynx_verify_attention reads anchor and residual (the verify pass over
 * Q_full, tq up to 64); lynx_draft_attention reads the anchor plane alone
 * (a draft step, usually tq = 1).
 *   q            bf16 bits [B][tq][Hq][128]: row (b, i) is the i-th of the
 *                request's tq newest tokens
 *   tq           1 .. LYNX_MAX_QUERY_TOKENS
 *   k, v         encoded page pools as for the decode calls; a pool of 0
 *                pages is allowed (then only the tail is read)
 *   block_table  int32 [B][max_pages_per_seq] as for the decode calls
 *   page_tokens  int32 [B] tokens in quantized pages per request, a multiple
 *                of 256 in [0, 256*max_pages_per_seq]; NULL = every request
 *                has max_pages_per_seq pages.  Device memory; values outside
 *                the range are clamped (output unspecified).
 *   tail_k/v     bf16 bits [B][LYNX_TAIL_TOKENS][H][128]: the request's
 *                tokens after its pages, in order
 *   tail_len     int32 [B] tokens in the tail, in [tq, LYNX_TAIL_TOKENS]
 *                (device memory; clamped, output unspecified outside).  The
 *                last tq tail tokens are the query tokens: token i sees
 *                every page token and tail tokens 0 .. tail_len - tq + i.
 *   out          fp32 [B][tq][Hq][128]
 *   workspace    at least lynx_verify_attention_workspace_size(...) bytes,
 *                16-byte aligned, contents need not be initialised; calls
 *                that overlap in time must not share a workspace.
 * The draft variant never reads k->residual or v->residual.  batch = 0 is a
 * no-op once the shape arguments are valid.  Errors: NULL_ARG, BAD_SHAPE,
 * MISALIGNED, WORKSPACE, DEVICE, HIP.
 */
size_t lynx_verify_attention_workspace_size(int32_t batch, int32_t tq,
                                            int32_t num_kv_heads,
                                            int32_t num_q_heads,
                                            int32_t head_dim,
                                            int32_t max_pages_per_seq);
int lynx_verify_attention(const uint16_t *q, int32_t tq, const lynx_planes *k,
                          const lynx_planes *v, const int32_t *block_table,
                          const int32_t *page_tokens, const uint16_t *tail_k,
                          const uint16_t *tail_v, const int32_t *tail_len,
                          int32_t batch, int32_t num_kv_heads,
                          int32_t num_q_heads, int32_t head_dim,
                          int32_t max_pages_per_seq, int64_t pool_pages,
                          float sm_scale, float *out, void *workspace,
                          size_t workspace_bytes, void *stream);
int lynx_draft_attention(const uint16_t *q, int32_t tq, const lynx_planes *k,
                         const lynx_planes *v, const int32_t *block_table,
                         const int32_t *page_tokens, const uint16_t *tail_k,
                         const uint16_t *tail_v, const int32_t *tail_len,
                         int32_t batch, int32_t num_kv_heads,
                         int32_t num_q_heads, int32_t head_dim,
                         int32_t max_pages_per_seq, int64_t pool_pages,
                         float sm_scale, float *out, void *workspace,
                         size_t workspace_bytes, void *stream);

/* Static string for a status code (never NULL). */
const char *lynx_status_string(int status);

/*
 * Host-side introspection, for tests (no GPU needed):
 * lynx_code_thresholds writes the 128 fp32 thresholds T[0..127] the encoder
 * uses: T[0] = 0 and, for k >= 1, T[k] is the smallest fp32 u with
 * 127 ln(1 + 255 u)/ln 256 >= k - 1/2, so that m(u) = #{k >= 1 : u >= T[k]}.
 * lynx_decode_table writes the 256 fp32 values yhat(code) indexed by
 * code + 128, as used by the dequantizers.
 */
void lynx_code_thresholds(float *out128);

/*
 * Device self-test of the encoder's level computation: for every fp32 bit
 * pattern b in [begin_bits, end_bits) (end_bits <= 0x40000000, i.e. values
 * in [0, 2); the encoder meets u slightly above 1 through rounding and must
 * give it the level of 1), compares the encoder's fast level path with the
 * exact threshold count of min(u, 1) and adds the number of disagreements
 * to *mismatches (a device uint64 the caller zeroes).  Errors: NULL_ARG,
 * BAD_ARG, DEVICE, HIP.
 */
int lynx_selftest_code_map(uint32_t begin_bits, uint32_t end_bits,
                           unsigned long long *mismatches, void *stream);
void lynx_decode_table(float *out256);
const char *lynx_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LYNX_H */
