/*
 * kvq.h -- C ABI of a low-bit KV-cache library for decode attention on
 * AMD Instinct MI355X (gfx950).
 *
 * What it computes.  Keys and values appended to a decode cache are quantized
 * group-wise to 3, 4 or 8 bits (or to a 16-entry non-uniform codebook with
 * fp16 outliers), and decode attention reads the packed codes directly:
 * dequantization happens inside the score, online-softmax and value-product
 * pass, so every code byte is read from HBM exactly once per step.
 *
 * Sources.  The operations follow five web pages on KV-cache quantization:
 *   - "NIAH" page (www.cf-1.com/news/5482713): q8_0 KV cache in llama.cpp,
 *     quantizing only the appended row (sections 1.1, 1.2, 2.2).
 *   - "TurboQuant" page (www.dpshk.com/news/6341316): per-token cache size
 *     2*L*d*h*bytes (section 2.1); 3-bit dynamic asymmetric quantization with
 *     scale = absmax/(2^(b-1)-1) and a min offset (section 3.1).
 *   - "KVQuant" page (www.cf-1.com/news/2306543): per-channel pre-RoPE keys,
 *     non-uniform codebooks, dense-and-sparse fp16 outliers with a bounded
 *     count per token, quantize-on-append and fused dequantization
 *     (sections 2.1, 2.2, 3.3, 3.4).
 *   - "Survey" page (www.discosf.com/news/4854722): per-head, per-position
 *     groups with a scale and zero point per group (section 2.4); keeping
 *     scores, softmax and the value product on chip (section 2.3).
 *   - "Memory-killer" page (www.demingchina.com/news/57821): decode is bound
 *     by streaming the cache (sections 1.3, 4.2); group-wise scaling and
 *     dequantization fused into the attention product (section 2.3); the
 *     8B / 128K element count (section 1.2).
 *
 * Conventions for every call.
 *   - All pointers are device pointers unless stated; the caller owns every
 *     buffer.  The library never allocates or frees memory.
 *   - Device pointers must be 16-byte aligned.
 *   - Work is enqueued on the given HIP stream (a hipStream_t passed as
 *     void*, NULL = the default stream) and never synchronizes the host.
 *   - Every argument is checked on the host before anything is launched.  A
 *     non-OK status leaves all state unchanged and sets a message readable
 *     with kvq_last_error().  No C++ exception crosses this interface.
 *   - head_dim must be 128.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
typedef int32_t kvq_status;
#define KVQ_OK                    0
#define KVQ_ERR_INVALID_ARGUMENT (-1) /* NULL/misaligned pointer, bad size    */
#define KVQ_ERR_UNSUPPORTED      (-2) /* valid but not implemented here       */
#define KVQ_ERR_CAPACITY         (-3) /* append would exceed max_ctx          */
#define KVQ_ERR_DEVICE           (-4) /* a HIP launch reported an error       */

/* ---- element types ----------------------------------------------------- */
#define KVQ_F16   0
#define KVQ_BF16  1
#define KVQ_F32   2

/* ---- quantizers (per tensor) ------------------------------------------- */
/* NONE: raw fp16/bf16 storage (bits = 16).
 * ASYM_MINMAX: per group scale = f16((max-min)/(2^b-1)), zero = f16(min),
 *   code = clamp(rint((x-zero)/scale), 0, 2^b-1)  [Survey page 2.4,
 *   Memory-killer page 2.3].  bits 3, 4 or 8.
 * ASYM_ABSMAX_OFFSET: scale = f16(max|x|/(2^(b-1)-1)), offset = f16(min),
 *   code as above [TurboQuant page 3.1, fixed groups instead of sliding
 *   windows].  bits 3, 4 or 8.
 * SYM_Q8_0: scale = f16(max|x|/127), zero 0, code = clamp(rint(x/scale),
 *   -128, 127) [NIAH page 1.2].  bits 8, per-token groups of group_size.
 * CODEBOOK: 4-bit index of the nearest of 16 fp16 centroids of that
 *   (kv head, channel), ties to the lower index; optionally the
 *   ceil(outlier_frac * n_kv_heads * head_dim) entries of largest |x| of each
 *   token are kept in fp16 (CSR; n_kv_heads * head_dim <= 4096; with a
 *   per-tile index of the same entries grouped by KV head, which decode
 *   reads) and replace the dense value
 *   [KVQuant page 2.2, 3.3].  The int32 row pointers bound the capacity:
 *   (batch * Tcap + 1) * outliers per token must not exceed 2^31 - 1
 *   (KVQ_ERR_UNSUPPORTED otherwise).
 * FP8_E5M2: each element is the FP8 E5M2 byte (sign, 5 exponent bits, 2
 *   mantissa bits: the high byte of an fp16) of x / s_h, rounded to nearest
 *   even and saturated at +-57344, with one float32 scale s_h per KV head
 *   (kvq_cache.k_scale / v_scale; NULL = 1) [Survey page 3.4: vLLM's fp8
 *   KV cache, scale per head].  bits 8, PER_TOKEN, group_size 0.  Stored
 *   in the 8-bit key-row and value-tile layouts; no parameter region.
 * All arithmetic of the encoders is IEEE float32 with round-half-even;
 * scales and zeros are rounded to fp16 before codes are computed; a group
 * whose fp16 scale is 0 stores code 0 everywhere. */
#define KVQ_QUANT_NONE                0
#define KVQ_QUANT_ASYM_MINMAX         1
#define KVQ_QUANT_ASYM_ABSMAX_OFFSET  2
#define KVQ_QUANT_SYM_Q8_0            3
#define KVQ_QUANT_CODEBOOK            4
#define KVQ_QUANT_FP8_E5M2            5

/* ---- group layouts ----------------------------------------------------- */
/* PER_TOKEN: groups of group_size consecutive channels of one token
 *   (group_size in {32, 64, 128}).
 * PER_CHANNEL: keys only; groups of group_size consecutive tokens of one
 *   channel [KVQuant page 2.2 per-channel keys, Survey page 2.4 per-position
 *   groups]; group_size a multiple of 32, at most 256.  Tokens of the
 *   unfinished last group stay unquantized in an fp16/bf16 tail until the
 *   group fills. */
#define KVQ_LAYOUT_PER_TOKEN    0
#define KVQ_LAYOUT_PER_CHANNEL  1

/* ---- decode kernel selection ------------------------------------------- */
/* AUTO picks the matrix-core kernel when the formats allow it (uniform
 * quantizers or raw storage for both tensors, no RoPE, no codebook, at most
 * 8 query heads per KV head), the lookup-table kernel for 4-bit codebook
 * keys and values with one query head per KV head (with or without
 * outliers and RoPE), and the general vector-ALU kernel otherwise.  VALU,
 * MFMA and LUT force a kernel; MFMA or LUT on a configuration it cannot run
 * is KVQ_ERR_UNSUPPORTED.  All compute the same attention to rounding. */
#define KVQ_PATH_AUTO 0
#define KVQ_PATH_VALU 1
#define KVQ_PATH_MFMA 2
#define KVQ_PATH_LUT  3

/* ---- kvq_cache_bytes selectors ----------------------------------------- */
#define KVQ_BYTES_PAYLOAD 0   /* bytes that hold n_ctx tokens, x n_layers    */
#define KVQ_BYTES_ALLOC   1   /* one layer's allocation at max_ctx            */

typedef struct kvq_tensor_format {
  int32_t quantizer;      /* KVQ_QUANT_*                                     */
  int32_t bits;           /* 3, 4, 8 (16 for NONE)                           */
  int32_t group_size;     /* see the layouts; ignored by NONE and CODEBOOK   */
  int32_t layout;         /* KVQ_LAYOUT_*                                    */
  float   outlier_frac;   /* CODEBOOK only: 0 or a fraction in (0, 0.25]     */
  int32_t window_overlap; /* PER_CHANNEL keys with ASYM_MINMAX or
                             ASYM_ABSMAX_OFFSET: the scale and zero of the
                             group of tokens [g G, g G + G) come from the
                             window [g G - window_overlap, g G + G) (clipped
                             at the first quantized token): sliding windows
                             that advance by G and overlap by window_overlap
                             tokens [TurboQuant page 3.1: parameters from a
                             sliding window's extrema; 6, problem 1: a window
                             overlap of 64 tokens].  0 (none) or a multiple
                             of 32 up to 256; 0 for every other format.  The
                             key tail then keeps G + window_overlap rows.    */
  const int32_t* head_group_size; /* PER_TOKEN layouts of ASYM_MINMAX,
                             ASYM_ABSMAX_OFFSET or SYM_Q8_0: NULL (every KV
                             head uses group_size), or a host array of
                             n_kv_heads group sizes in {32, 64, 128}, one per
                             KV head [Memory-killer page 2.3 and 5.3: finer
                             groups for the heads that are sensitive to
                             quantization, coarser ones for stable heads].
                             Read during each call only; at most 64 KV heads. */
} kvq_tensor_format;

typedef struct kvq_config {
  int32_t batch;          /* sequences B                                     */
  int32_t n_q_heads;      /* query heads Hq; a multiple of n_kv_heads        */
  int32_t n_kv_heads;     /* KV heads Hkv; query head j reads KV head j/(Hq/Hkv) */
  int32_t head_dim;       /* d, must be 128                                  */
  int64_t max_ctx;        /* capacity in tokens per sequence                 */
  int32_t kv_dtype;       /* KVQ_F16 or KVQ_BF16: dtype of K, V and q        */
  int32_t rope;           /* 1: keys are stored pre-RoPE and both q and k are
                             rotated at decode time (rotate-half pairs
                             (i, i+d/2), theta_i = rope_base^(-2i/d)) [KVQuant
                             page 2.1-2.2]                                    */
  float   rope_base;      /* e.g. 10000                                      */
  int32_t decode_splits;  /* 0 = automatic; otherwise the maximum number of
                             token splits per (sequence, KV head)            */
  int32_t decode_path;    /* KVQ_PATH_AUTO, _VALU, _MFMA or _LUT             */
  kvq_tensor_format k;    /* key format                                      */
  kvq_tensor_format v;    /* value format (PER_TOKEN only)                   */
  int32_t sink_tokens;    /* attention sink [KVQuant page, Attention Sink]:
                             tokens [0, sink_tokens) of every sequence keep
                             their kv_dtype keys and values and are attended
                             exactly; the formats apply to the later tokens,
                             which form a quantized cache that starts at token
                             sink_tokens (per-channel key groups start there).
                             A position threshold (quantize only positions
                             >= N [NIAH page 5.2, its threshold parameter])
                             is this with sink_tokens = N.
                             0 .. 4096; 0 = none                              */
  int32_t page_pool;      /* paged cache [Survey page 3.4: vLLM's block-table
                             cache, --block-size 16]: 0 = one contiguous
                             stretch of max_ctx tokens per sequence; > 0 = a
                             pool of this many physical pages of 32 tokens
                             (two of vLLM's 16-token blocks: the value tile
                             of the decode kernels) shared by the sequences
                             through kvq_cache.page_table.  A page holds the
                             codes, per-token parameters and outlier rows of
                             its 32 tokens for every KV head; per-channel key
                             parameters, the key tail and the attention sink
                             stay per sequence.  0 .. 2^26                    */
} kvq_config;

typedef struct kvq_cache {
  void*       base;       /* device buffer of kvq_cache_bytes(KVQ_BYTES_ALLOC)
                             bytes, zero-filled before first use (all zero =
                             empty cache).  The decode call also uses a
                             workspace region inside it.                     */
  const void* k_codebook; /* CODEBOOK keys: fp16 [n_kv_heads, head_dim, 16],
                             ascending per (head, channel); else NULL         */
  const void* v_codebook; /* same for values                                 */
  int64_t     n_ctx;      /* tokens held per sequence (host state; advanced
                             by kvq_quantize_append on success)              */
  const float* k_scale;   /* FP8_E5M2 keys: device float32 [n_kv_heads]
                             scales (finite, > 0), or NULL for 1; ignored by
                             the other formats                               */
  const float* v_scale;   /* same for values                                 */
  const int32_t* page_table; /* page_pool > 0: device int32
                             [batch][pages_per_seq] (kvq_layout_info;
                             ceil(max_ctx / 32)): entry i of sequence b is
                             the physical page of its tokens [32 i, 32 i + 32).
                             Pages a call writes or reads must be distinct
                             across sequences and logical pages; entries not
                             yet in use are ignored.  Entries outside
                             [0, page_pool) are clamped into it (no access
                             leaves the allocation; the results are then
                             undefined).  NULL when page_pool is 0.  Owned by
                             the caller, who may update entries for pages
                             not yet written between calls.                   */
} kvq_cache;

/* Location of one array inside the cache allocation (bytes from base). */
typedef struct kvq_region {
  uint64_t offset;
  uint64_t bytes;
} kvq_region;

typedef struct kvq_tensor_regions {
  kvq_region codes;    /* packed codes (raw rows for NONE)                  */
  kvq_region params;   /* fp16 scale/zero pairs (q8_0: scales)              */
  kvq_region tail;     /* per-channel keys: fp16/bf16 [B, Hkv, G, d]        */
  kvq_region row_ptr;  /* outliers: int32 [B*Tcap + 1]                      */
  kvq_region col;      /* outliers: uint16, bits 0-11 column h*d + c, bits
                          12-15 the dense codebook index at that position  */
  kvq_region val;      /* outliers: fp16 value                              */
  kvq_region sink;     /* attention sink: kv_dtype [B, Hkv, sink_tokens, d] */
  kvq_region tile_off; /* outliers: uint16 [rows / 32][round_up(Hkv + 1, 8)]:
                          for the tile of 32 CSR rows (32 tokens; a page of
                          a paged cache), where KV head h's entries start in
                          the tile's block of tile_ent; [Hkv] the tile's
                          count; zero padding                             */
  kvq_region tile_ent; /* outliers: uint32 [rows / 32][32 * k]: the tile's
                          entries grouped by KV head, each head's in token
                          order (a token's in column order): bits 0-6
                          channel, 7-11 token in the tile, 12-15 the dense
                          index replaced, 16-31 the fp16 value            */
} kvq_tensor_regions;

typedef struct kvq_layout_info {
  kvq_tensor_regions k;
  kvq_tensor_regions v;
  kvq_region workspace;     /* split-K partial softmax states               */
  uint64_t   total_bytes;   /* == kvq_cache_bytes(..., KVQ_BYTES_ALLOC)     */
  int64_t    capacity;      /* Tcap = max_ctx rounded up to 1024 (a
                               multiple of the 32-token tile; the stride
                               between (sequence, head) streams stays a
                               multiple of 1024 tokens)                      */
  int32_t    max_splits;    /* split-K partial slots per (b, query head)   */
  int32_t    pages_per_seq; /* paged cache: entries per sequence of
                               kvq_cache.page_table (0 when not paged)      */
} kvq_layout_info;

/*
 * kvq_cache_bytes -- size of the cache.  Host only; touches no device.
 *   what = KVQ_BYTES_PAYLOAD: bytes that hold n_ctx tokens (packed codes,
 *     scale/zero parameters, the unquantized per-channel tail, outliers as
 *     the per-tile index that decode streams, codebooks), times n_layers.  With NONE for both tensors this is
 *     exactly 2 * n_layers * n_kv_heads * head_dim * 2 * n_ctx * batch, the
 *     per-token formula of the TurboQuant page (section 2.1), which gives
 *     327,680 bytes per token for Llama-2-70B (L = 80, h = 8, d = 128).
 *     With an attention sink, the first min(sink_tokens, n_ctx) tokens
 *     count their raw kv_dtype bytes and the formats the rest.
 *     This is also the number of bytes one decode step must read.
 *   what = KVQ_BYTES_ALLOC: size of one layer's allocation at max_ctx,
 *     including padding and the decode workspace (n_ctx, n_layers ignored).
 *   Errors: INVALID_ARGUMENT (NULL, negative sizes, bad config, unknown
 *   selector), UNSUPPORTED (head_dim != 128 or an unsupported format).
 */
kvq_status kvq_cache_bytes(const kvq_config* cfg, int64_t n_ctx, int64_t n_layers,
                           int32_t what, uint64_t* out_bytes);

/*
 * kvq_cache_layout -- offsets of every array inside one layer's allocation,
 * for callers that checkpoint or inspect the cache.  Host only.
 * Byte layouts (d = 128):
 *   segment of 32 codes u = 8m + e (block m, element e): 8-bit: byte u;
 *     4-bit: byte j = code 2j | code 2j+1 << 4; 3-bit: three little-endian
 *     dwords D0, D1, D2 -- for block m and r = 0..3 the pair (8m+r, 8m+r+4)
 *     keeps its low two bits at bits 2p and 16+2p of D[m/2], p = 4(m%2)+r,
 *     and its high bits at bits H and 16+H of D2, H = 8(m/2) + 2r + m%2.
 *   keys: a row of 16*bits bytes per token, segment q = 0..3 holding
 *     channels 32m + 8q + e; codes [B][Hkv][Tcap][row].
 *   values: tiles of 32 tokens, 64 lanes L = 16q + i of 8*bits bytes (two
 *     segments s); segment s, block m of lane L holds channel 16(4s+m) + i,
 *     element e is token 4q+e (e < 4) or 16+4q+e-4 of the tile.
 *   CODEBOOK values: tiles of 32 tokens (2048 bytes); byte 32l + tau holds
 *     channel l in its low nibble and channel l+64 in its high nibble of
 *     token tau (l = 0..63).
 *   params: per-token [B][Hkv][Tcap][d/G] of (scale, zero) fp16 pairs
 *     (q8_0: scales only); per-channel [B][Hkv][Tcap/G][d] pairs.
 *   NONE: raw rows [B][Hkv][Tcap][d] of kv_dtype for keys and values.
 *   Paged cache (page_pool P > 0): every array with one record per token
 *     and head (key rows, value tiles, per-token params, raw rows) holds
 *     [P][Hkv][32] token rows instead of [B][Hkv][Tcap]: token t of
 *     sequence b, head h is row (page_table[b][t / 32] * Hkv + h) * 32 +
 *     t % 32.  The outlier CSR has P * 32 rows (row page * 32 + t % 32;
 *     row_ptr [P * 32 + 1]) and the per-tile index one tile per page.  Per-channel params, tail and sink keep their
 *     per-sequence shapes.
 * Errors: as kvq_cache_bytes.
 */
kvq_status kvq_cache_layout(const kvq_config* cfg, kvq_layout_info* out);

/*
 * kvq_quantize_append -- quantize n_new new tokens of every sequence and
 * append them at position cache->n_ctx; on success n_ctx += n_new.
 * Only the new rows are encoded; existing codes are never re-quantized
 * (NIAH page 1.1 and 2.2: quantize just the appended row; KVQuant page 3.4:
 * new keys and values are quantized with fixed parameters and stored as
 * codes plus fp16 outliers).  Appending in several calls gives exactly the
 * bytes of one call with all tokens.
 *   k_new, v_new: device [B][n_new][Hkv][d] of kv_dtype, contiguous.
 *   n_new = 0 is a no-op.  Bulk prefill is one call with n_new = T.
 *   Tokens that fall below cfg->sink_tokens are copied raw to the sink;
 *   the others are quantized at their position in the quantized cache.
 * Errors: INVALID_ARGUMENT (NULL/misaligned pointers, n_new < 0, bad config,
 *   codebook pointer missing or present when the format says otherwise),
 *   UNSUPPORTED, CAPACITY (n_ctx + n_new > max_ctx; checked before any
 *   launch), DEVICE.
 */
kvq_status kvq_quantize_append(const kvq_config* cfg, kvq_cache* cache, const void* k_new,
                               const void* v_new, int32_t n_new, void* stream);

/*
 * kvq_decode_attention -- one decode step of attention over the cached
 * tokens [0, n_ctx) for every sequence and query head:
 *   out[b, j, :] = sum_t softmax_t(sm_scale * q'_j . k'_t) * v_t
 * with k, v the dequantized cache of KV head j / (Hq / Hkv) (outliers
 * replacing their dense values), q' = R(q_pos) q and k'_t = R(t) k_t when
 * rope is on (identity otherwise).  Dequantization is fused into the pass
 * (Memory-killer page 2.3; KVQuant page 3.4); the token axis is split over
 * the GPU and the partial softmax states are merged by log-sum-exp.
 *   q: device [B][Hq][d] of kv_dtype.  q_pos: device int32 [B] or NULL
 *   (= n_ctx - 1).  sm_scale <= 0 selects 1/sqrt(d).
 *   out: device [B][Hq][d] of out_dtype (KVQ_F32, KVQ_F16 or KVQ_BF16).
 * With an attention sink, its raw tokens are streamed as a raw cache of
 * their own whose partial softmax states (one per split of at least 256
 * tokens) join the merge, and positions stay absolute (token t of the
 * quantized cache is at position sink_tokens + t).
 * The call writes the workspace region of cache->base: decode calls on the
 * same cache must not overlap in time (same stream or synchronized).
 * Errors: INVALID_ARGUMENT (NULL/misaligned pointers, n_ctx == 0 or beyond
 *   max_ctx, bad out_dtype), UNSUPPORTED, DEVICE.
 */
kvq_status kvq_decode_attention(const kvq_config* cfg, const kvq_cache* cache, const void* q,
                                const int32_t* q_pos, float sm_scale, void* out,
                                int32_t out_dtype, void* stream);

/*
 * kvq_append_decode -- one serving step: append one token per sequence and
 * decode over the cache that now holds it.  Cache bytes, n_ctx and out are
 * those of kvq_quantize_append(cfg, cache, k_new, v_new, 1, stream)
 * followed by kvq_decode_attention(cfg, cache, q, q_pos, sm_scale, out,
 * out_dtype, stream): the same bytes, the same attention to rounding
 * (NIAH page 1.1 and 2.2: only the appended row is quantized; Memory-killer
 * page 1.3 and 4.2: each generated token streams the cache once).
 * Where kvq_append_decode_fused says so, the append takes no launch of its
 * own: the decode kernels stream the n_ctx tokens cached before the step,
 * and the launch that merges their split softmax states also encodes the
 * new token into the cache and adds its term (key and value as the codes
 * just written stand for them).  Otherwise the two calls run in turn.
 *   k_new, v_new: device [B][1][Hkv][d] of kv_dtype, contiguous.  q, q_pos,
 *   sm_scale, out, out_dtype: as kvq_decode_attention; q is the new
 *   token's query (position n_ctx before the call).  On success n_ctx
 *   grows by one.  Writes the workspace region of cache->base, as decode.
 * Errors: INVALID_ARGUMENT and UNSUPPORTED as the two calls, CAPACITY when
 *   n_ctx == max_ctx (before any launch), DEVICE.
 */
kvq_status kvq_append_decode(const kvq_config* cfg, kvq_cache* cache, const void* k_new,
                             const void* v_new, const void* q, const int32_t* q_pos,
                             float sm_scale, void* out, int32_t out_dtype, void* stream);

/*
 * kvq_append_decode_fused -- 1 when kvq_append_decode on a cache of n_ctx
 * tokens runs the fused step, 0 when it runs the two calls in turn.  Fused:
 * keys and values in ASYM_MINMAX, ASYM_ABSMAX_OFFSET, SYM_Q8_0, FP8_E5M2 or
 * raw storage (so no codebook or outliers), per-token keys or per-channel
 * keys whose current group stays open after the append (the token goes to
 * the unquantized tail), no RoPE, n_ctx >= sink_tokens, at most 128 query
 * heads per KV head.  Host only; a negative status for an invalid
 * configuration or n_ctx outside [0, max_ctx).
 */
int32_t kvq_append_decode_fused(const kvq_config* cfg, int64_t n_ctx);

/*
 * kvq_decode_attention_scratch -- kvq_decode_attention for callers that
 * cannot allocate device memory or write outside the buffers they pass
 * (code under HIP graph capture, serving loops and harnesses that forbid
 * allocation).  It computes the same attention with the same kernels, but
 * keeps the split-K partial softmax states in a static device array of the
 * library (KVQ_DECODE_SCRATCH_BYTES per GPU, held until the process ends)
 * instead of the workspace region of cache->base, which it leaves
 * untouched.  It allocates nothing.
 *   Arguments, layout and errors as kvq_decode_attention.  When the array
 *   holds fewer partial states per (sequence, query head) than the library
 *   would use, the token axis is split fewer times (same result up to
 *   rounding); UNSUPPORTED when it cannot hold one state per query head
 *   plus one per 256 sink tokens (batch * n_q_heads * (head_dim + 2) * 4
 *   bytes each).
 *   All calls on one GPU share its array and it keeps the last call's
 *   contents: calls that overlap in time on one GPU (other streams, other
 *   host threads) race and must be serialized by the caller.
 */
#define KVQ_DECODE_SCRATCH_BYTES (8u << 20)
kvq_status kvq_decode_attention_scratch(const kvq_config* cfg, const kvq_cache* cache,
                                        const void* q, const int32_t* q_pos, float sm_scale,
                                        void* out, int32_t out_dtype, void* stream);

/*
 * kvq_prefill_attention -- causal attention of the last n_q tokens of every
 * sequence over the cache: the attention of a prefill chunk (chunked
 * prefill) once its keys and values have been appended with
 * kvq_quantize_append [NIAH page 4.2: first-token latency is the prefill
 * pass; Survey page 2.3 and 5.3: QK^T, softmax and the value product of
 * prefill kept on chip].
 *   out[b, i, j, :] = sum_{t <= p_i} softmax_t(sm_scale * q'_{i,j} . k'_t) * v_t,
 *   p_i = n_ctx - n_q + i,
 * with k, v the cache exactly as kvq_decode_attention reads it (dequantized,
 * outliers, per-channel tail, raw attention-sink tokens) and the same RoPE
 * convention, the query of row i at position p_i.
 *   q: device [B][n_q][Hq][d] of kv_dtype (query i is that of token
 *   n_ctx - n_q + i).  1 <= n_q <= n_ctx.  sm_scale <= 0 selects 1/sqrt(d).
 *   out: device [B][n_q][Hq][d] of out_dtype (KVQ_F32, KVQ_F16 or KVQ_BF16).
 *   workspace: device scratch of workspace_bytes bytes (16-byte aligned) for
 *   the partial softmax states of a token axis split over several
 *   workgroups; the call splits the axis only as far as the workspace holds
 *   (kvq_prefill_workspace_bytes gives the size for the library's own
 *   choice); NULL / 0 = no split.  The caller owns it; calls that share it
 *   must not overlap in time.
 * Runs on the matrix cores for every cache format; the query heads per KV
 * head (Hq / Hkv) must divide 64.  Reads the cache only: it may overlap
 * with other reads of the same cache, not with appends to it.
 * Errors: INVALID_ARGUMENT (NULL/misaligned pointers, n_ctx == 0, n_q out
 *   of range, bad out_dtype), UNSUPPORTED (group size), DEVICE.
 */
kvq_status kvq_prefill_attention(const kvq_config* cfg, const kvq_cache* cache, const void* q,
                                 int32_t n_q, float sm_scale, void* out, int32_t out_dtype,
                                 void* workspace, uint64_t workspace_bytes, void* stream);

/*
 * kvq_prefill_workspace_bytes -- workspace size for the token-axis split
 * kvq_prefill_attention would choose for n_q queries over a cache of n_ctx
 * tokens (0 when it would not split).
 * Errors: INVALID_ARGUMENT (bad config, NULL out, n_q or n_ctx out of range).
 */
kvq_status kvq_prefill_workspace_bytes(const kvq_config* cfg, int32_t n_q, int64_t n_ctx,
                                       uint64_t* out_bytes);

/*
 * kvq_prefill_kernel -- which kernel kvq_prefill_attention runs for this
 * configuration: KVQ_PREFILL_CODES (the packed codes enter the matrix cores
 * as exact fp16 operands, the scales the query and probability operands;
 * 4-bit per-channel keys with 4-bit values in per-token groups of 128 or 32
 * channels and fp16 data, 3-bit keys and values in per-token groups of 64,
 * q8_0 keys and values in blocks of 32, and FP8 E5M2; no attention sink, no
 * RoPE, one group size for every KV head) or KVQ_PREFILL_STAGED (each
 * block dequantized into LDS as fp16 high and low parts: every format).
 * Host only.  Returns a negative status for an invalid configuration.
 */
#define KVQ_PREFILL_CODES  1
#define KVQ_PREFILL_STAGED 2
int32_t kvq_prefill_kernel(const kvq_config* cfg);

/*
 * kvq_decode_path -- which decode kernel kvq_decode_attention runs for this
 * configuration: KVQ_PATH_VALU, KVQ_PATH_MFMA or KVQ_PATH_LUT (what KVQ_PATH_AUTO resolves
 * to, or the forced path).  Host only.  Returns a negative status for an
 * invalid configuration or a forced path it cannot run.
 */
int32_t kvq_decode_path(const kvq_config* cfg);

/*
 * kvq_set_decode_events -- optional instrumentation for profiling.  With
 * start and stop non-NULL hipEvent_t handles (created by the caller, which
 * keeps ownership), the next kvq_decode_attention call on this host thread
 * has them recorded at the start and at the end of its token-streaming
 * kernel (hipExtLaunchKernel; the first and the last launch when a
 * configuration needs several), so that start..stop is that kernel's
 * execution alone: not the dispatch gap before it, the sink's kernel or the
 * split merge.  Without a streaming kernel (no quantized tokens) both are
 * recorded back to back.  The next call that passes validation and launches
 * uses them and clears them; NULL, NULL clears them without a launch.  Host only; returns KVQ_OK, or INVALID_ARGUMENT when exactly
 * one of the two is NULL.
 */
kvq_status kvq_set_decode_events(void* start, void* stop);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* kvq_last_error(void);

/* Version of this interface (major * 100 + minor); 101 since kvq_config
   gained sink_tokens and kvq_tensor_regions gained sink; 102 adds
   kvq_prefill_attention; 103 adds KVQ_QUANT_FP8_E5M2 and the kvq_cache
   scale pointers; 104 gives kvq_prefill_attention a workspace and adds
   kvq_prefill_workspace_bytes; 105 adds kvq_decode_attention_scratch;
   106 adds the paged cache (kvq_config.page_pool, kvq_cache.page_table,
   kvq_layout_info.pages_per_seq); 107 adds kvq_tensor_format.window_overlap
   and head_group_size; 108 adds the per-head outlier counts
   (kvq_tensor_regions.head_count); 109 replaces them by per-head end
   offsets (kvq_tensor_regions.head_end); 110 replaces those by the
   per-tile index (kvq_tensor_regions.tile_off, tile_ent); 111 adds
   kvq_prefill_kernel; 112 adds kvq_append_decode and
   kvq_append_decode_fused. */
int32_t kvq_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
