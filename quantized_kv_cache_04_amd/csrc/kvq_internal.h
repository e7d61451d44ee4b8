// Internal declarations shared by the host entry points and the kernel
// launchers of libkvq.  Not part of the public interface (include/kvq.h).
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "../../include/kvq.h"

namespace kvq {

constexpr int kHeadDim = 128;
constexpr int kTile = 32;          // tokens per value tile / decode block
constexpr int kCapAlign = 1024;    // token capacity granularity (a multiple of kTile)
constexpr int kMaxSink = 4096;     // attention-sink tokens kept raw per sequence
constexpr int kSinkSplitTokens = 256;   // a split of the sink spans at least this many tokens
constexpr int kMaxHeadsPH = 64;     // KV heads of a format with per-head group sizes
constexpr int kMaxAppendHeads = 128;   // query heads per KV head of the fused append step

// Host-side description of one cache tensor (keys or values) and where its
// arrays sit in the allocation.
struct TensorLayout {
  int quant = 0;        // KVQ_QUANT_*
  int bits = 16;
  int G = 0;            // group size (0 for NONE / CODEBOOK)
  int per_channel = 0;  // 1: groups along tokens (keys only)
  int row_bytes = 0;    // bytes of one token's codes (raw: d * 2)
  int ng = 0;           // groups per token (per-token layouts)
  int psize = 0;        // bytes per group parameter record (4: scale+zero, 2: scale)
  int k_out = 0;        // outliers kept per token (CODEBOOK)
  int overlap = 0;      // per-channel keys: tokens the statistics window reaches back
  // per-token groups with a size per KV head: groups per token of head h
  // and their prefix sums (ng_pre[Hkv] = groups per token over all heads)
  int per_head = 0;
  uint8_t ngh[kMaxHeadsPH] = {};
  uint16_t ng_pre[kMaxHeadsPH + 1] = {};
  uint64_t codes_off = 0, codes_bytes = 0;
  uint64_t params_off = 0, params_bytes = 0;
  uint64_t tail_off = 0, tail_bytes = 0;
  uint64_t rowptr_off = 0, rowptr_bytes = 0;
  uint64_t col_off = 0, col_bytes = 0;
  uint64_t val_off = 0, val_bytes = 0;
  uint64_t toff_off = 0, toff_bytes = 0;   // outliers: uint16 [tiles][round_up(Hkv + 1, 8)]
  uint64_t tent_off = 0, tent_bytes = 0;   // outliers: uint32 [tiles][32 k] grouped by head
  uint64_t sink_off = 0, sink_bytes = 0;   // attention sink: raw [B, Hkv, sink, d]
};

struct Layout {
  TensorLayout k, v;
  int64_t Tcap = 0;          // token capacity per sequence (multiple of 32)
  int n_pages = 0;           // paged cache: physical pages of kTile tokens (0: contiguous)
  int pages_per_seq = 0;     // paged cache: page-table entries per sequence
  int sink = 0;              // attention-sink tokens kept raw per sequence
  int S_max = 1;             // partial slots per (b, query head)
  uint64_t partial_off = 0;  // float [B][Hq][S_max][d + 2]
  uint64_t ws_off = 0, ws_bytes = 0;
  uint64_t total = 0;
};

// Device-side view of one tensor, passed by value to kernels.
struct DevTensor {
  int quant, bits, G, per_channel, row_bytes, ng, k_out;
  // per-channel keys: the window reaches ``overlap`` tokens back, and the
  // unquantized tail is a ring of tail_rows = G + overlap rows in which
  // token t sits at row t mod tail_rows
  int overlap, tail_rows;
  // per-token groups with a size per KV head (per_head = 1): head h has
  // ngh[h] groups of 128 / ngh[h] channels per token, and its parameter
  // records follow those of heads 0 .. h-1 (ng_pre[h] records per token
  // before it, ng_pre[Hkv] in all); G and ng are then unused
  int per_head;
  uint8_t ngh[kMaxHeadsPH];
  uint16_t ng_pre[kMaxHeadsPH + 1];
  uint8_t* codes;
  void* params;
  uint16_t* tail;
  int32_t* row_ptr;
  uint16_t* col;
  uint16_t* val;
  uint16_t* toff;             // outliers: per tile, where each KV head's entries start
  uint32_t* tent;             // outliers: per tile, the entries grouped by KV head
  const uint16_t* codebook;   // fp16 [Hkv][d][16]
  const float* hscale;        // FP8: float32 scale per KV head (null = 1)
};

struct DevShape {
  int B, Hq, Hkv, g, kv_bf16;
  int64_t Tcap;
  // appends: the input holds in_tok tokens per sequence; the call encodes
  // input tokens [in_off, in_off + n_new)
  int64_t in_tok = 0, in_off = 0;
  // paged cache: physical page (kTile tokens of every KV head) of logical
  // page i of sequence b is page_table[b * pages_per_seq + i]; null for a
  // contiguous cache
  const int32_t* page_table = nullptr;
  int pages_per_seq = 0;
  int n_pages = 0;
};

DevTensor make_dev_tensor(const TensorLayout& tl, void* base, const void* codebook,
                          const float* scale);

// ---- encode launchers (encode.hip) ----------------------------------------
hipError_t launch_encode_tensor(const DevShape& sh, const DevTensor& t, bool is_key,
                                const void* x_new, int64_t n_ctx, int n_new,
                                hipStream_t stream);
// keys and values of one append (a single launch for the common serving step)
hipError_t launch_encode_kv(const DevShape& sh, const DevTensor& kt, const DevTensor& vt,
                            const void* k_new, const void* v_new, int64_t n_ctx, int n_new,
                            hipStream_t stream);
// raw copy of input tokens [in_off, in_off + n) to sink rows [pos, pos + n)
hipError_t launch_encode_sink(const DevShape& sh, uint16_t* sink, int sink_cap, const void* x_new,
                              int64_t pos, int n, hipStream_t stream);

// ---- decode launchers ------------------------------------------------------
struct DecodeArgs {
  DevShape sh;
  DevTensor k, v;
  const void* q;
  const int32_t* q_pos;
  void* out;
  int out_dtype;
  float sm_scale;       // softmax scale (already resolved)
  int rope;
  float rope_base;
  int n_ctx;            // tokens this launch streams
  int pos0;             // absolute position of its token 0
  int q_last;           // absolute position of the sequence's last token (default query position)
  int splits;           // splits of the token axis this launch uses
  int blocks_per_split; // 32-token blocks per split
  int slot0;            // partial slot of split 0 (general kernel; the others start at 0)
  int direct;           // 1: the streaming kernel writes the output itself (one split, no sink)
  int n_partials;       // partial states the combine merges
  int S_max;
  float* partial;       // [B][Hq][S_max][d + 2]
  int kp_groups;        // matrix-core kernel: key groups staged in LDS per wave (0 = none)
  int head_class = 0;   // matrix-core kernel, per-head group sizes: only the KV heads
                        // whose values have this many groups per token (0 = all)
  // profiling (kvq_set_decode_events): recorded at the start and the end of
  // the streaming kernel (the first and the last of its launches)
  hipEvent_t ev_start = nullptr, ev_stop = nullptr;
};

// kvq_decode_attention with the split-K partial states in partial_ws
// (ws_bytes) instead of the cache's workspace region when partial_ws is set.
// With k_new and v_new (the fused step of kvq_append_decode), the decode
// streams the cache->n_ctx cached tokens and the merge launch appends one
// token per sequence and adds its term; the caller advances n_ctx.
kvq_status decode_attention_impl(const kvq_config* cfg, const kvq_cache* cache, const void* q,
                                 const int32_t* q_pos, float sm_scale, void* out,
                                 int32_t out_dtype, void* stream, float* partial_ws,
                                 uint64_t ws_bytes, const void* k_new = nullptr,
                                 const void* v_new = nullptr);
// the error message of the calling thread (kvq_last_error)
kvq_status set_error(kvq_status st, const char* msg);

hipError_t launch_decode_generic(const DecodeArgs& a, hipStream_t stream);
// merge of the split-K partials, the sink's included (when a.direct is 0)
hipError_t launch_combine(const DecodeArgs& a, hipStream_t stream);
// One serving step's new token (kvq_append_decode): encode it at position
// pos of the quantized cache and merge its attention term with the split
// partial states of a (a.direct is 0; a.n_partials may be 0).
hipError_t launch_append_merge(const DecodeArgs& a, const void* k_new, const void* v_new,
                               int64_t pos, hipStream_t stream);
// Whether the matrix-core kernel handles this configuration's formats.
bool mfma_config_supported(const kvq_config& c);
hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream);
// Whether the lookup-table kernel handles this configuration (4-bit codebook
// keys and values, one query head per KV head;
// k_out_*: outliers per token of keys and values).
bool lut_config_supported(const kvq_config& c, int k_out_k, int k_out_v);
// a.splits = token ranges per sequence, each of a.blocks_per_split 32-token chunks
hipError_t launch_decode_lut(const DecodeArgs& a, hipStream_t stream);

// ---- chunked-prefill launcher ------------------------------------------------
struct PrefillArgs {
  DevShape sh;
  DevTensor k, v;            // quantized cache: tokens [n_sink, n_total)
  const uint16_t* k_sink;    // raw [B][Hkv][sink_cap][d]: tokens [0, n_sink)
  const uint16_t* v_sink;
  int sink_cap, n_sink;
  int n_total;               // tokens in the cache, sink included
  int n_q;                   // queries: the last n_q tokens, positions n_total - n_q + i
  const void* q;             // [B][n_q][Hq][d], kv dtype
  void* out;                 // [B][n_q][Hq][d], out_dtype
  int out_dtype;
  float sm_scale;            // resolved
  int rope;
  float rope_base;
  int codes;                 // 1: the code-operand kernel (prefill_codes_supported)
  int splits;                // token-axis splits (grid z); > 1: partial states to partial
  int blocks_per_split;      // 32-token blocks per split
  float* partial;            // [B][n_q][Hq][splits][d + 2] (o, m, l) when splits > 1
};
// 64 query rows per workgroup: Hq / Hkv must divide 64
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
// Whether the code-operand prefill kernel serves this configuration (the
// staging kernel serves every other one).
bool prefill_codes_supported(const kvq_config& c);
// The code-operand prefill kernel (same grid, splits and partial records
// as the staging one); false, with nothing launched, for formats it is not
// compiled for.
bool launch_prefill_codes(const PrefillArgs& a, hipStream_t stream);

}  // namespace kvq
