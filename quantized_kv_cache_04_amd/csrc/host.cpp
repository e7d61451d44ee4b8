// Host side of libkvq: argument checks, cache layout, cache sizes and the
// dispatch of the HIP kernels.  Everything here runs before any launch, so
// a rejected call leaves the device and the cache untouched.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include <hip/hip_runtime_api.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

thread_local std::string g_last_error;
// events recorded around the next decode's streaming kernel (kvq_set_decode_events)
thread_local hipEvent_t g_ev_start = nullptr, g_ev_stop = nullptr;

kvq_status fail(kvq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

// partial slots the attention sink may need: one per kSinkSplitTokens
int64_t sink_slots(int64_t sink) { return (sink + kSinkSplitTokens - 1) / kSinkSplitTokens; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int outlier_count(float frac, int n) {
  if (!(frac > 0.0f)) return 0;
  return (int)ceil((double)frac * (double)n);
}

kvq_status check_format(const kvq_tensor_format& f, const kvq_config& c, bool is_key,
                        const char* name) {
  const int d = c.head_dim;
  if (f.quantizer != KVQ_QUANT_CODEBOOK && f.outlier_frac != 0.0f)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: outlier_frac is only valid for CODEBOOK", name);
  if (f.window_overlap != 0) {
    if (f.layout != KVQ_LAYOUT_PER_CHANNEL ||
        (f.quantizer != KVQ_QUANT_ASYM_MINMAX && f.quantizer != KVQ_QUANT_ASYM_ABSMAX_OFFSET))
      return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: window_overlap applies to per-channel keys "
                  "with ASYM_MINMAX or ASYM_ABSMAX_OFFSET only", name);
    if (f.window_overlap < 0 || f.window_overlap > 256 || f.window_overlap % kTile)
      return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: window_overlap must be a multiple of 32 in "
                  "[0, 256] (got %d)", name, f.window_overlap);
  }
  if (f.head_group_size) {
    if (f.layout != KVQ_LAYOUT_PER_TOKEN ||
        (f.quantizer != KVQ_QUANT_ASYM_MINMAX && f.quantizer != KVQ_QUANT_ASYM_ABSMAX_OFFSET &&
         f.quantizer != KVQ_QUANT_SYM_Q8_0))
      return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: head_group_size applies to per-token "
                  "ASYM_MINMAX, ASYM_ABSMAX_OFFSET or SYM_Q8_0 formats only", name);
    if (c.n_kv_heads > kMaxHeadsPH)
      return fail(KVQ_ERR_UNSUPPORTED, "%s: per-head group sizes need n_kv_heads <= %d", name,
                  kMaxHeadsPH);
    for (int h = 0; h < c.n_kv_heads; ++h) {
      const int g = f.head_group_size[h];
      if (g != 32 && g != 64 && g != 128)
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: head_group_size[%d] must be 32, 64 or 128 "
                    "(got %d)", name, h, g);
    }
  }
  if (f.layout != KVQ_LAYOUT_PER_TOKEN && f.layout != KVQ_LAYOUT_PER_CHANNEL)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: unknown layout %d", name, f.layout);
  switch (f.quantizer) {
    case KVQ_QUANT_NONE:
      if (f.bits != 16) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: NONE needs bits = 16", name);
      if (f.layout != KVQ_LAYOUT_PER_TOKEN)
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: NONE has no per-channel layout", name);
      return KVQ_OK;
    case KVQ_QUANT_ASYM_MINMAX:
    case KVQ_QUANT_ASYM_ABSMAX_OFFSET:
      if (f.bits != 3 && f.bits != 4 && f.bits != 8)
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: bits must be 3, 4 or 8 (got %d)", name, f.bits);
      break;
    case KVQ_QUANT_SYM_Q8_0:
      if (f.bits != 8) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: q8_0 needs bits = 8", name);
      if (f.layout != KVQ_LAYOUT_PER_TOKEN)
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: q8_0 blocks run along head_dim", name);
      break;
    case KVQ_QUANT_CODEBOOK:
      if (f.bits != 4) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: CODEBOOK needs bits = 4", name);
      if (f.layout != KVQ_LAYOUT_PER_TOKEN)
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: CODEBOOK uses per-(head, channel) codebooks "
                    "and the per-token layout", name);
      if (!(f.outlier_frac >= 0.0f && f.outlier_frac <= 0.25f))
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: outlier_frac must be in [0, 0.25]", name);
      if (f.outlier_frac > 0.0f && (int64_t)c.n_kv_heads * d > 4096)
        return fail(KVQ_ERR_UNSUPPORTED, "%s: outliers need n_kv_heads * head_dim <= 4096",
                    name);
      return KVQ_OK;
    case KVQ_QUANT_FP8_E5M2:
      if (f.bits != 8) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: FP8_E5M2 needs bits = 8", name);
      if (f.layout != KVQ_LAYOUT_PER_TOKEN || f.group_size != 0)
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: FP8_E5M2 takes the per-token layout and "
                    "group_size 0 (its scale is per KV head)", name);
      return KVQ_OK;
    default:
      return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: unknown quantizer %d", name, f.quantizer);
  }
  if (f.layout == KVQ_LAYOUT_PER_TOKEN) {
    if (f.head_group_size) return KVQ_OK;   // group_size is not used
    if (f.group_size != 32 && f.group_size != 64 && f.group_size != 128)
      return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: per-token group_size must be 32, 64 or 128 "
                  "(got %d)", name, f.group_size);
  } else {
    if (!is_key)
      return fail(KVQ_ERR_UNSUPPORTED, "%s: per-channel layout is supported for keys only", name);
    if (f.group_size < 32 || f.group_size > 256 || f.group_size % 32)
      return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: per-channel group_size must be a multiple of 32 "
                  "in [32, 256] (got %d)", name, f.group_size);
  }
  return KVQ_OK;
}

kvq_status check_config(const kvq_config* c) {
  if (!c) return fail(KVQ_ERR_INVALID_ARGUMENT, "config is NULL");
  if (c->batch < 1 || c->n_kv_heads < 1 || c->n_q_heads < 1)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "batch and head counts must be >= 1");
  if (c->n_q_heads % c->n_kv_heads)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)",
                c->n_q_heads, c->n_kv_heads);
  if (c->head_dim != kHeadDim)
    return fail(KVQ_ERR_UNSUPPORTED, "head_dim must be 128 (got %d)", c->head_dim);
  if (c->max_ctx < 1 || c->max_ctx > (int64_t)1 << 30)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "max_ctx must be in [1, 2^30] (got %lld)",
                (long long)c->max_ctx);
  if (c->kv_dtype != KVQ_F16 && c->kv_dtype != KVQ_BF16)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "kv_dtype must be KVQ_F16 or KVQ_BF16");
  if (c->rope != 0 && c->rope != 1) return fail(KVQ_ERR_INVALID_ARGUMENT, "rope must be 0 or 1");
  if (c->rope && !(c->rope_base > 1.0f))
    return fail(KVQ_ERR_INVALID_ARGUMENT, "rope_base must be > 1");
  if (c->decode_splits < 0) return fail(KVQ_ERR_INVALID_ARGUMENT, "decode_splits must be >= 0");
  if (c->decode_path < KVQ_PATH_AUTO || c->decode_path > KVQ_PATH_LUT)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "unknown decode_path %d", c->decode_path);
  if ((uint64_t)c->batch * (uint64_t)c->max_ctx > ((uint64_t)1 << 31))
    return fail(KVQ_ERR_INVALID_ARGUMENT, "batch * max_ctx must be <= 2^31");
  if (c->sink_tokens < 0 || c->sink_tokens > kMaxSink)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "sink_tokens must be in [0, %d] (got %d)", kMaxSink,
                c->sink_tokens);
  if (c->page_pool < 0 || c->page_pool > (1 << 26))
    return fail(KVQ_ERR_INVALID_ARGUMENT, "page_pool must be in [0, 2^26] (got %d)", c->page_pool);
  kvq_status st = check_format(c->k, *c, true, "k");
  if (st != KVQ_OK) return st;
  st = check_format(c->v, *c, false, "v");
  if (st != KVQ_OK) return st;
  // the CSR row pointers are int32 offsets k * r over every row r of the
  // capacity (B * Tcap rows): they must not wrap
  const uint64_t rows = (c->page_pool ? (uint64_t)c->page_pool * kTile
                                      : (uint64_t)c->batch * align_up((uint64_t)c->max_ctx, kCapAlign)) + 1;
  const kvq_tensor_format* fmts[2] = {&c->k, &c->v};
  for (int i = 0; i < 2; ++i) {
    if (fmts[i]->quantizer != KVQ_QUANT_CODEBOOK) continue;
    const uint64_t k = (uint64_t)outlier_count(fmts[i]->outlier_frac, c->n_kv_heads * c->head_dim);
    if (k && rows * k > (uint64_t)INT32_MAX)
      return fail(KVQ_ERR_UNSUPPORTED, "%s: %llu outliers per token over batch * capacity = %llu "
                  "rows overflow the int32 CSR row pointers", i ? "v" : "k",
                  (unsigned long long)k, (unsigned long long)(rows - 1));
  }
  return KVQ_OK;
}

// slots: token records per KV head of the per-token arrays (B * Tcap for a
// contiguous cache, n_pages * kTile for a paged one)
void fill_tensor(TensorLayout& t, const kvq_tensor_format& f, const kvq_config& c, int64_t Tcap,
                 uint64_t slots, uint64_t& off) {
  const uint64_t B = c.batch, H = c.n_kv_heads, d = c.head_dim;
  t.quant = f.quantizer;
  t.bits = f.quantizer == KVQ_QUANT_NONE ? 16 : f.bits;
  t.per_channel = f.layout == KVQ_LAYOUT_PER_CHANNEL;
  t.G = (f.quantizer == KVQ_QUANT_NONE || f.quantizer == KVQ_QUANT_CODEBOOK ||
         f.quantizer == KVQ_QUANT_FP8_E5M2) ? 0 : f.group_size;
  t.row_bytes = (int)(d * t.bits / 8);
  t.per_head = f.head_group_size != nullptr;
  if (t.per_head) {
    t.ng_pre[0] = 0;
    for (uint64_t h = 0; h < H; ++h) {
      t.ngh[h] = (uint8_t)(d / f.head_group_size[h]);
      t.ng_pre[h + 1] = (uint16_t)(t.ng_pre[h] + t.ngh[h]);
    }
    t.G = f.head_group_size[0];   // per-head formats read ngh / ng_pre instead
  }
  t.ng = (t.G && !t.per_channel) ? (int)(d / t.G) : 0;
  // parameter records per token over all heads
  const uint64_t ng_all = t.per_head ? t.ng_pre[H] : H * (uint64_t)t.ng;
  t.psize = f.quantizer == KVQ_QUANT_SYM_Q8_0 ? 2 : 4;
  t.k_out = f.quantizer == KVQ_QUANT_CODEBOOK ? outlier_count(f.outlier_frac, (int)(H * d)) : 0;
  auto put = [&](uint64_t& o, uint64_t& sz, uint64_t bytes) {
    o = off;
    sz = bytes;
    off = align_up(off + bytes, 256);
  };
  put(t.codes_off, t.codes_bytes, H * slots * t.row_bytes);
  if (t.G) {
    if (t.per_channel)
      put(t.params_off, t.params_bytes, B * H * (uint64_t)(Tcap / t.G) * d * 4);
    else
      put(t.params_off, t.params_bytes, slots * ng_all * t.psize);
  }
  t.overlap = t.per_channel ? f.window_overlap : 0;
  if (t.per_channel) put(t.tail_off, t.tail_bytes, B * H * (uint64_t)(t.G + t.overlap) * d * 2);
  if (t.k_out) {
    put(t.rowptr_off, t.rowptr_bytes, (slots + 1) * 4);
    put(t.col_off, t.col_bytes, slots * t.k_out * 2);
    put(t.val_off, t.val_bytes, slots * t.k_out * 2);
    // the per-tile index: offsets per head, entries grouped by head
    put(t.toff_off, t.toff_bytes, (slots / kTile) * ((H + 8) / 8 * 16));
    put(t.tent_off, t.tent_bytes, slots * t.k_out * 4);
  }
}

Layout make_layout(const kvq_config& c) {
  Layout L;
  // Capacity: max_ctx rounded up to 1024 tokens.  The decode kernels stream
  // B * Hkv rows of Tcap tokens side by side; with FP8 rows some strides of
  // 4 KB granularity (e.g. 66,016 and 66,080 tokens) ran 15 % slower on
  // MI355X than any multiple of 1024 tokens measured.
  L.Tcap = (int64_t)align_up((uint64_t)c.max_ctx, kCapAlign);
  L.n_pages = c.page_pool;
  L.pages_per_seq = c.page_pool ? (int)((c.max_ctx + kTile - 1) / kTile) : 0;
  const uint64_t slots = c.page_pool ? (uint64_t)c.page_pool * kTile : (uint64_t)c.batch * L.Tcap;
  uint64_t off = 0;
  fill_tensor(L.k, c.k, c, L.Tcap, slots, off);
  fill_tensor(L.v, c.v, c, L.Tcap, slots, off);
  L.sink = c.sink_tokens;
  if (L.sink) {
    const uint64_t sb = (uint64_t)c.batch * c.n_kv_heads * L.sink * c.head_dim * 2;
    L.k.sink_off = off;
    L.k.sink_bytes = sb;
    off = align_up(off + sb, 256);
    L.v.sink_off = off;
    L.v.sink_bytes = sb;
    off = align_up(off + sb, 256);
  }
  // partial slots: the splits of the quantized cache and those of the sink
  // (the merge reads at most 256)
  int64_t s = (L.Tcap + 63) / 64 + sink_slots(L.sink);
  L.S_max = (int)(s < 1 ? 1 : (s > 256 ? 256 : s));
  L.ws_off = off;
  L.partial_off = off;
  off = align_up(off + (uint64_t)c.batch * c.n_q_heads * L.S_max * (c.head_dim + 2) * 4, 256);
  L.ws_bytes = off - L.ws_off;
  L.total = off;
  return L;
}

uint64_t tensor_payload(const TensorLayout& t, const kvq_config& c, int64_t n) {
  const uint64_t B = c.batch, H = c.n_kv_heads, d = c.head_dim;
  if (t.quant == KVQ_QUANT_NONE) return B * H * (uint64_t)n * d * 2;
  // FP8: a byte per element and the per-head float32 scales decode reads
  if (t.quant == KVQ_QUANT_FP8_E5M2) return B * H * (uint64_t)n * d + H * 4;
  uint64_t total;
  if (t.quant == KVQ_QUANT_CODEBOOK) {
    total = B * H * (uint64_t)n * t.row_bytes + H * d * 16 * 2;
    // outliers: the per-tile index the decode kernels stream (entries of the
    // n tokens and the offsets of their tiles)
    if (t.k_out)
      total += B * ((uint64_t)n * 4 * t.k_out + (((uint64_t)n + kTile - 1) / kTile) * ((H + 8) / 8 * 16));
    return total;
  }
  if (t.per_channel) {
    uint64_t nf = (uint64_t)(n / t.G) * t.G;
    return B * H * (nf * t.row_bytes + (nf / t.G) * d * 4 + ((uint64_t)n - nf) * d * 2);
  }
  const uint64_t ng_all = t.per_head ? t.ng_pre[H] : H * (uint64_t)t.ng;
  return B * (uint64_t)n * (H * t.row_bytes + ng_all * t.psize);
}

void fill_regions(kvq_tensor_regions& r, const TensorLayout& t) {
  r.codes = {t.codes_off, t.codes_bytes};
  r.params = {t.params_off, t.params_bytes};
  r.tail = {t.tail_off, t.tail_bytes};
  r.row_ptr = {t.rowptr_off, t.rowptr_bytes};
  r.col = {t.col_off, t.col_bytes};
  r.val = {t.val_off, t.val_bytes};
  r.tile_off = {t.toff_off, t.toff_bytes};
  r.tile_ent = {t.tent_off, t.tent_bytes};
  r.sink = {t.sink_off, t.sink_bytes};
}

kvq_status check_codebooks(const kvq_config& c, const kvq_cache& cache) {
  const bool kc = c.k.quantizer == KVQ_QUANT_CODEBOOK, vc = c.v.quantizer == KVQ_QUANT_CODEBOOK;
  if (kc != (cache.k_codebook != nullptr))
    return fail(KVQ_ERR_INVALID_ARGUMENT, "k_codebook must be given iff keys use CODEBOOK");
  if (vc != (cache.v_codebook != nullptr))
    return fail(KVQ_ERR_INVALID_ARGUMENT, "v_codebook must be given iff values use CODEBOOK");
  if ((cache.k_codebook && !aligned16(cache.k_codebook)) ||
      (cache.v_codebook && !aligned16(cache.v_codebook)))
    return fail(KVQ_ERR_INVALID_ARGUMENT, "codebook pointers must be 16-byte aligned");
  if ((cache.k_scale && (reinterpret_cast<uintptr_t>(cache.k_scale) & 3u)) ||
      (cache.v_scale && (reinterpret_cast<uintptr_t>(cache.v_scale) & 3u)))
    return fail(KVQ_ERR_INVALID_ARGUMENT, "scale pointers must be 4-byte aligned");
  if ((c.page_pool > 0) != (cache.page_table != nullptr))
    return fail(KVQ_ERR_INVALID_ARGUMENT, "page_table must be given iff page_pool > 0");
  if (cache.page_table && (reinterpret_cast<uintptr_t>(cache.page_table) & 3u))
    return fail(KVQ_ERR_INVALID_ARGUMENT, "page_table must be 4-byte aligned");
  return KVQ_OK;
}

// the paged-cache fields of a kernel's shape
void set_paging(DevShape& sh, const Layout& L, const kvq_cache& cache) {
  sh.page_table = L.n_pages ? cache.page_table : nullptr;
  sh.pages_per_seq = L.pages_per_seq;
  sh.n_pages = L.n_pages;
}

kvq_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess)
    return fail(KVQ_ERR_DEVICE, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
  return KVQ_OK;
}

}  // namespace

kvq_status set_error(kvq_status st, const char* msg) {
  g_last_error = msg;
  return st;
}

DevTensor make_dev_tensor(const TensorLayout& tl, void* base, const void* codebook,
                          const float* scale) {
  uint8_t* b = static_cast<uint8_t*>(base);
  DevTensor t;
  t.quant = tl.quant;
  t.bits = tl.bits;
  t.G = tl.G;
  t.per_channel = tl.per_channel;
  t.row_bytes = tl.row_bytes;
  t.ng = tl.ng;
  t.k_out = tl.k_out;
  t.overlap = tl.overlap;
  t.tail_rows = tl.G + tl.overlap;
  t.per_head = tl.per_head;
  memcpy(t.ngh, tl.ngh, sizeof t.ngh);
  memcpy(t.ng_pre, tl.ng_pre, sizeof t.ng_pre);
  t.codes = b + tl.codes_off;
  t.params = tl.params_bytes ? b + tl.params_off : nullptr;
  t.tail = tl.tail_bytes ? reinterpret_cast<uint16_t*>(b + tl.tail_off) : nullptr;
  t.row_ptr = tl.rowptr_bytes ? reinterpret_cast<int32_t*>(b + tl.rowptr_off) : nullptr;
  t.col = tl.col_bytes ? reinterpret_cast<uint16_t*>(b + tl.col_off) : nullptr;
  t.val = tl.val_bytes ? reinterpret_cast<uint16_t*>(b + tl.val_off) : nullptr;
  t.toff = tl.toff_bytes ? reinterpret_cast<uint16_t*>(b + tl.toff_off) : nullptr;
  t.tent = tl.tent_bytes ? reinterpret_cast<uint32_t*>(b + tl.tent_off) : nullptr;
  t.codebook = static_cast<const uint16_t*>(codebook);
  t.hscale = tl.quant == KVQ_QUANT_FP8_E5M2 ? scale : nullptr;
  return t;
}

}  // namespace kvq

using namespace kvq;

extern "C" {

const char* kvq_last_error(void) { return g_last_error.c_str(); }

int32_t kvq_decode_path(const kvq_config* cfg) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  const bool ok = mfma_config_supported(*cfg);
  const Layout L = make_layout(*cfg);
  const bool lut = lut_config_supported(*cfg, L.k.k_out, L.v.k_out);
  if (cfg->decode_path == KVQ_PATH_MFMA && !ok)
    return fail(KVQ_ERR_UNSUPPORTED, "the matrix-core decode kernel needs uniform or raw formats "
                "for keys and values, no RoPE and at most 8 query heads per KV head");
  if (cfg->decode_path == KVQ_PATH_LUT && !lut)
    return fail(KVQ_ERR_UNSUPPORTED, "the lookup-table decode kernel needs 4-bit codebook keys "
                "and values and one query head per KV head");
  if (cfg->decode_path == KVQ_PATH_VALU) return KVQ_PATH_VALU;
  if (cfg->decode_path == KVQ_PATH_LUT || (cfg->decode_path == KVQ_PATH_AUTO && lut))
    return KVQ_PATH_LUT;
  return ok ? KVQ_PATH_MFMA : KVQ_PATH_VALU;
}

int32_t kvq_prefill_kernel(const kvq_config* cfg) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  return prefill_codes_supported(*cfg) ? KVQ_PREFILL_CODES : KVQ_PREFILL_STAGED;
}

int32_t kvq_abi_version(void) { return 112; }

kvq_status kvq_set_decode_events(void* start, void* stop) {
  if ((start == nullptr) != (stop == nullptr))
    return fail(KVQ_ERR_INVALID_ARGUMENT, "start and stop events must both be set or both NULL");
  g_ev_start = static_cast<hipEvent_t>(start);
  g_ev_stop = static_cast<hipEvent_t>(stop);
  return KVQ_OK;
}

kvq_status kvq_cache_bytes(const kvq_config* cfg, int64_t n_ctx, int64_t n_layers, int32_t what,
                           uint64_t* out_bytes) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (!out_bytes) return fail(KVQ_ERR_INVALID_ARGUMENT, "out_bytes is NULL");
  Layout L = make_layout(*cfg);
  if (what == KVQ_BYTES_ALLOC) {
    *out_bytes = L.total;
    return KVQ_OK;
  }
  if (what != KVQ_BYTES_PAYLOAD) return fail(KVQ_ERR_INVALID_ARGUMENT, "unknown selector %d", what);
  if (n_ctx < 0 || n_layers < 0)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "n_ctx and n_layers must be >= 0");
  // the attention sink holds min(sink, n_ctx) raw tokens; the formats apply to the rest
  const int64_t ns = n_ctx < L.sink ? n_ctx : L.sink;
  const uint64_t raw = (uint64_t)cfg->batch * cfg->n_kv_heads * ns * cfg->head_dim * 2;
  *out_bytes = (uint64_t)n_layers * (tensor_payload(L.k, *cfg, n_ctx - ns) +
                                     tensor_payload(L.v, *cfg, n_ctx - ns) + 2 * raw);
  return KVQ_OK;
}

kvq_status kvq_cache_layout(const kvq_config* cfg, kvq_layout_info* out) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (!out) return fail(KVQ_ERR_INVALID_ARGUMENT, "out is NULL");
  Layout L = make_layout(*cfg);
  memset(out, 0, sizeof *out);
  fill_regions(out->k, L.k);
  fill_regions(out->v, L.v);
  out->workspace = {L.ws_off, L.ws_bytes};
  out->total_bytes = L.total;
  out->capacity = L.Tcap;
  out->max_splits = L.S_max;
  out->pages_per_seq = L.pages_per_seq;
  return KVQ_OK;
}

kvq_status kvq_quantize_append(const kvq_config* cfg, kvq_cache* cache, const void* k_new,
                               const void* v_new, int32_t n_new, void* stream) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (!cache) return fail(KVQ_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (!cache->base || !aligned16(cache->base))
    return fail(KVQ_ERR_INVALID_ARGUMENT, "cache->base must be a 16-byte aligned device pointer");
  if (n_new < 0) return fail(KVQ_ERR_INVALID_ARGUMENT, "n_new must be >= 0");
  if (cache->n_ctx < 0 || cache->n_ctx > cfg->max_ctx)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "cache->n_ctx out of range");
  st = check_codebooks(*cfg, *cache);
  if (st != KVQ_OK) return st;
  if (n_new == 0) return KVQ_OK;
  if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new))
    return fail(KVQ_ERR_INVALID_ARGUMENT, "k_new and v_new must be 16-byte aligned device pointers");
  if (cache->n_ctx + n_new > cfg->max_ctx)
    return fail(KVQ_ERR_CAPACITY, "append of %d tokens at n_ctx %lld exceeds max_ctx %lld", n_new,
                (long long)cache->n_ctx, (long long)cfg->max_ctx);
  Layout L = make_layout(*cfg);
  DevShape sh{cfg->batch, cfg->n_q_heads, cfg->n_kv_heads, cfg->n_q_heads / cfg->n_kv_heads,
              cfg->kv_dtype == KVQ_BF16, L.Tcap};
  set_paging(sh, L, *cache);
  sh.in_tok = n_new;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // input tokens that fall below the sink length are copied raw; the rest
  // are quantized at their position in the quantized cache
  const int64_t n0 = cache->n_ctx;
  const int n_sink_new = n0 >= L.sink ? 0 : (int)(L.sink - n0 < n_new ? L.sink - n0 : n_new);
  const int n_q_new = n_new - n_sink_new;
  const int64_t n_q0 = n0 > L.sink ? n0 - L.sink : 0;
  if (n_sink_new > 0) {
    uint8_t* base = static_cast<uint8_t*>(cache->base);
    st = device_status(launch_encode_sink(sh, reinterpret_cast<uint16_t*>(base + L.k.sink_off),
                                          L.sink, k_new, n0, n_sink_new, s), "sink keys");
    if (st != KVQ_OK) return st;
    st = device_status(launch_encode_sink(sh, reinterpret_cast<uint16_t*>(base + L.v.sink_off),
                                          L.sink, v_new, n0, n_sink_new, s), "sink values");
    if (st != KVQ_OK) return st;
  }
  if (n_q_new > 0) {
    sh.in_off = n_sink_new;
    DevTensor kt = make_dev_tensor(L.k, cache->base, cache->k_codebook, cache->k_scale);
    DevTensor vt = make_dev_tensor(L.v, cache->base, cache->v_codebook, cache->v_scale);
    st = device_status(launch_encode_kv(sh, kt, vt, k_new, v_new, n_q0, n_q_new, s),
                       "encode keys and values");
    if (st != KVQ_OK) return st;
  }
  cache->n_ctx += n_new;
  return KVQ_OK;
}

kvq_status kvq_decode_attention(const kvq_config* cfg, const kvq_cache* cache, const void* q,
                                const int32_t* q_pos, float sm_scale, void* out,
                                int32_t out_dtype, void* stream) {
  return kvq::decode_attention_impl(cfg, cache, q, q_pos, sm_scale, out, out_dtype, stream,
                                    nullptr, 0);
}

namespace {
// uniform quantizers, FP8 and raw storage: the formats whose one-token
// append the merge launch encodes itself
bool append_merge_format(const kvq_tensor_format& f) {
  return f.quantizer == KVQ_QUANT_NONE || f.quantizer == KVQ_QUANT_ASYM_MINMAX ||
         f.quantizer == KVQ_QUANT_ASYM_ABSMAX_OFFSET || f.quantizer == KVQ_QUANT_SYM_Q8_0 ||
         f.quantizer == KVQ_QUANT_FP8_E5M2;
}
}  // namespace

int32_t kvq_append_decode_fused(const kvq_config* cfg, int64_t n_ctx) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (n_ctx < 0 || n_ctx >= cfg->max_ctx)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "n_ctx must be in [0, max_ctx) for an append of one "
                "token (got %lld)", (long long)n_ctx);
  if (cfg->rope || n_ctx < cfg->sink_tokens) return 0;
  if (!append_merge_format(cfg->k) || !append_merge_format(cfg->v)) return 0;
  if (cfg->n_q_heads / cfg->n_kv_heads > kvq::kMaxAppendHeads) return 0;
  if (cfg->k.layout == KVQ_LAYOUT_PER_CHANNEL) {
    // the key must go to the tail: its group stays open after the append
    const int64_t nq = n_ctx - cfg->sink_tokens, G = cfg->k.group_size;
    if (nq / G != (nq + 1) / G) return 0;
  }
  return 1;
}

kvq_status kvq_append_decode(const kvq_config* cfg, kvq_cache* cache, const void* k_new,
                             const void* v_new, const void* q, const int32_t* q_pos,
                             float sm_scale, void* out, int32_t out_dtype, void* stream) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (!cache) return fail(KVQ_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (cache->n_ctx < 0 || cache->n_ctx > cfg->max_ctx)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "cache->n_ctx out of range");
  if (cache->n_ctx + 1 > cfg->max_ctx)
    return fail(KVQ_ERR_CAPACITY, "append of 1 token at n_ctx %lld exceeds max_ctx %lld",
                (long long)cache->n_ctx, (long long)cfg->max_ctx);
  const int32_t fused = kvq_append_decode_fused(cfg, cache->n_ctx);
  if (fused < 0) return fused;
  if (!fused) {
    st = kvq_quantize_append(cfg, cache, k_new, v_new, 1, stream);
    if (st != KVQ_OK) return st;
    return kvq_decode_attention(cfg, cache, q, q_pos, sm_scale, out, out_dtype, stream);
  }
  if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new))
    return fail(KVQ_ERR_INVALID_ARGUMENT, "k_new and v_new must be 16-byte aligned device pointers");
  st = kvq::decode_attention_impl(cfg, cache, q, q_pos, sm_scale, out, out_dtype, stream, nullptr,
                                  0, k_new, v_new);
  if (st == KVQ_OK) cache->n_ctx += 1;
  return st;
}

}  // extern "C"

// One decode step (kvq_decode_attention).  partial_ws: the split-K partial
// states go there instead of the workspace region of the cache allocation,
// which then holds at most ws_bytes of them (fewer splits when needed).
kvq_status kvq::decode_attention_impl(const kvq_config* cfg, const kvq_cache* cache,
                                      const void* q, const int32_t* q_pos, float sm_scale,
                                      void* out, int32_t out_dtype, void* stream,
                                      float* partial_ws, uint64_t ws_bytes, const void* k_new,
                                      const void* v_new) {
  const bool fused = k_new != nullptr;
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (!cache) return fail(KVQ_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (!cache->base || !aligned16(cache->base))
    return fail(KVQ_ERR_INVALID_ARGUMENT, "cache->base must be a 16-byte aligned device pointer");
  if (cache->n_ctx < (fused ? 0 : 1) || cache->n_ctx > cfg->max_ctx - (fused ? 1 : 0))
    return fail(KVQ_ERR_INVALID_ARGUMENT, "n_ctx must be in [1, max_ctx] (got %lld): attention "
                "over an empty cache is undefined", (long long)cache->n_ctx);
  st = check_codebooks(*cfg, *cache);
  if (st != KVQ_OK) return st;
  if (!q || !out || !aligned16(q) || !aligned16(out))
    return fail(KVQ_ERR_INVALID_ARGUMENT, "q and out must be 16-byte aligned device pointers");
  if (q_pos && !aligned16(q_pos))
    return fail(KVQ_ERR_INVALID_ARGUMENT, "q_pos must be 16-byte aligned");
  if (out_dtype != KVQ_F32 && out_dtype != KVQ_F16 && out_dtype != KVQ_BF16)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "out_dtype must be KVQ_F32, KVQ_F16 or KVQ_BF16");
  if (!isfinite(sm_scale)) return fail(KVQ_ERR_INVALID_ARGUMENT, "sm_scale must be finite");

  Layout L = make_layout(*cfg);
  DecodeArgs a;
  a.sh = DevShape{cfg->batch, cfg->n_q_heads, cfg->n_kv_heads, cfg->n_q_heads / cfg->n_kv_heads,
                  cfg->kv_dtype == KVQ_BF16, L.Tcap};
  set_paging(a.sh, L, *cache);
  a.k = make_dev_tensor(L.k, cache->base, cache->k_codebook, cache->k_scale);
  a.v = make_dev_tensor(L.v, cache->base, cache->v_codebook, cache->v_scale);
  a.q = q;
  a.q_pos = q_pos;
  a.out = out;
  a.out_dtype = out_dtype;
  a.sm_scale = sm_scale > 0.0f ? sm_scale : (float)(1.0 / sqrt((double)cfg->head_dim));
  a.rope = cfg->rope;
  a.rope_base = cfg->rope_base;
  // the attention sink holds tokens [0, n_sink); the quantized cache the rest
  const int n_sink = (int)(cache->n_ctx < L.sink ? cache->n_ctx : L.sink);
  a.n_ctx = (int)(cache->n_ctx - n_sink);
  a.pos0 = n_sink;
  a.q_last = (int)cache->n_ctx - (fused ? 0 : 1);
  a.slot0 = 0;
  a.S_max = L.S_max;
  a.kp_groups = 0;
  a.partial = reinterpret_cast<float*>(static_cast<uint8_t*>(cache->base) + L.partial_off);
  if (partial_ws) {
    // as many partial slots per (sequence, query head) as the buffer holds
    const uint64_t per_slot = (uint64_t)cfg->batch * cfg->n_q_heads * (cfg->head_dim + 2) * 4;
    const uint64_t fit = ws_bytes / per_slot;
    if (fit < (uint64_t)a.S_max) a.S_max = (int)fit;
    if (a.S_max < 1 + sink_slots(L.sink))
      return fail(KVQ_ERR_UNSUPPORTED, "the %llu-byte scratch holds %llu partial states per "
                  "(sequence, query head); this batch of %d x %d query heads with %lld sink "
                  "tokens needs at least %lld", (unsigned long long)ws_bytes,
                  (unsigned long long)fit, cfg->batch, cfg->n_q_heads, (long long)L.sink,
                  (long long)(1 + sink_slots(L.sink)));
    a.partial = partial_ws;
  }
  // partial slots left for the quantized cache's splits
  const int64_t max_q_splits = a.S_max - sink_slots(L.sink);

  // Split the token axis so that the grid is about one resident round of
  // workgroups (256 CUs x 2 workgroups of 4 waves): fewer, longer
  // workgroups amortize each one's set-up and merge, and more rounds only
  // add a ragged tail.  Each split keeps at least 8 blocks of 32 tokens.
  const int32_t path = kvq_decode_path(cfg);
  if (path < 0) return path;
  a.splits = 0;
  a.blocks_per_split = 0;
  if (a.n_ctx > 0) {
    const int64_t nblocks = (a.n_ctx + kTile - 1) / kTile;
    const int64_t pairs = (int64_t)cfg->batch * cfg->n_kv_heads;
    constexpr int64_t kTargetWorkgroups = 512;
    int64_t want = (kTargetWorkgroups + pairs - 1) / pairs;
    int64_t by_len = nblocks / 8;
    if (want > by_len) want = by_len;
    if (cfg->decode_splits > 0 && want > cfg->decode_splits) want = cfg->decode_splits;
    if (want > max_q_splits) want = max_q_splits;
    if (want < 1) want = 1;
    a.blocks_per_split = (int)((nblocks + want - 1) / want);
    if (path == KVQ_PATH_MFMA && cfg->k.layout == KVQ_LAYOUT_PER_CHANNEL) {
      // the matrix-core kernel deals a split's blocks to its waves one key
      // group at a time: splits start on a group boundary
      const int gblk = cfg->k.group_size / kTile;
      a.blocks_per_split = (a.blocks_per_split + gblk - 1) / gblk * gblk;
    }
    a.splits = (int)((nblocks + a.blocks_per_split - 1) / a.blocks_per_split);
    if (path == KVQ_PATH_LUT) {
      // ranges of whole 32-token chunks; a workgroup serves 4 KV heads and
      // three of them fit on a CU, so about 768 workgroups take
      // 768 / (batch * ceil(Hkv / 4)) ranges per sequence, each at least 4
      // chunks long
      constexpr int64_t kLutWorkgroups = 768;
      const int64_t nchunks = nblocks;
      const int64_t units = (int64_t)cfg->batch * ((cfg->n_kv_heads + 3) / 4);
      int64_t r = (kLutWorkgroups + units - 1) / units;
      if (r > nchunks / 4) r = nchunks / 4;
      if (cfg->decode_splits > 0 && r > cfg->decode_splits) r = cfg->decode_splits;
      if (r > max_q_splits) r = max_q_splits;
      if (r < 1) r = 1;
      const int64_t per = (nchunks + r - 1) / r;
      a.blocks_per_split = (int)per;
      a.splits = (int)((nchunks + per - 1) / per);
    }
  }
  // The sink is a raw cache of its own, [B, Hkv, sink, d], streamed by the
  // general kernel with positions from 0; its partial states follow those
  // of the quantized cache.  Each of its splits spans at least
  // kSinkSplitTokens tokens.
  DecodeArgs sa = a;
  if (n_sink > 0) {
    uint8_t* base = static_cast<uint8_t*>(cache->base);
    for (int i = 0; i < 2; ++i) {
      DevTensor raw{};
      raw.quant = KVQ_QUANT_NONE;
      raw.bits = 16;
      raw.row_bytes = cfg->head_dim * 2;
      raw.codes = base + (i == 0 ? L.k.sink_off : L.v.sink_off);
      (i == 0 ? sa.k : sa.v) = raw;
    }
    sa.sh.Tcap = L.sink;
    sa.sh.page_table = nullptr;   // the sink stays per sequence
    sa.n_ctx = n_sink;
    sa.pos0 = 0;
    sa.slot0 = a.splits;
    const int64_t nblocks = (n_sink + kTile - 1) / kTile;
    const int64_t pairs = (int64_t)cfg->batch * cfg->n_kv_heads;
    int64_t want = (512 + pairs - 1) / pairs;
    const int64_t by_len = nblocks / (kSinkSplitTokens / kTile);
    if (want > by_len) want = by_len;
    if (want > sink_slots(L.sink)) want = sink_slots(L.sink);
    if (want < 1) want = 1;
    sa.blocks_per_split = (int)((nblocks + want - 1) / want);
    sa.splits = (int)((nblocks + sa.blocks_per_split - 1) / sa.blocks_per_split);
  } else {
    sa.splits = 0;
  }
  // a streaming kernel writes the output itself only when its one split
  // holds every token; otherwise the partial states are merged
  a.n_partials = sa.n_partials = a.splits + sa.splits;
  a.direct = sa.direct = a.n_partials == 1 && !fused ? 1 : 0;

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t ev0 = g_ev_start, ev1 = g_ev_stop;
  g_ev_start = g_ev_stop = nullptr;
  hipError_t e = hipSuccess;
  if (a.n_ctx > 0) {
    // the profiling events are recorded at the streaming kernel's own start
    // and end (the sink's kernel and the merge are not part of it)
    a.ev_start = ev0;
    a.ev_stop = ev1;
    e = path == KVQ_PATH_MFMA ? launch_decode_mfma(a, s)
        : path == KVQ_PATH_LUT ? launch_decode_lut(a, s)
                               : launch_decode_generic(a, s);
  } else if (ev0) {   // no streaming kernel: an empty interval
    e = hipEventRecord(ev0, s);
    if (e == hipSuccess) e = hipEventRecord(ev1, s);
  }
  if (e == hipSuccess && n_sink > 0) e = launch_decode_generic(sa, s);
  if (e == hipSuccess && fused)
    e = launch_append_merge(a, k_new, v_new, a.n_ctx, s);
  else if (e == hipSuccess && !a.direct)
    e = launch_combine(a, s);
  return device_status(e, fused ? "append and decode" : "decode attention");
}

extern "C" {

namespace {
// Token-axis split of prefill: about 512 workgroups (two per CU), at least
// 8 blocks of 32 tokens per split, at most 64 splits (and decode_splits,
// when set).
int prefill_splits(const kvq_config& c, int32_t n_q, int64_t n_ctx) {
  const int g = c.n_q_heads / c.n_kv_heads;
  const int64_t qt = 64 / g;
  const int64_t tiles = (n_q + qt - 1) / qt;
  const int64_t wgs = tiles * c.batch * c.n_kv_heads;
  const int64_t ns = n_ctx < c.sink_tokens ? n_ctx : c.sink_tokens;
  const int64_t nblk = (ns + kTile - 1) / kTile + (n_ctx - ns + kTile - 1) / kTile;
  int64_t want = (512 + wgs - 1) / wgs;
  if (want > nblk / 8) want = nblk / 8;
  if (want > 64) want = 64;
  if (c.decode_splits > 0 && want > c.decode_splits) want = c.decode_splits;
  if (want < 1) want = 1;
  return (int)want;
}

uint64_t prefill_ws_bytes(const kvq_config& c, int32_t n_q, int splits) {
  return splits > 1 ? (uint64_t)c.batch * n_q * c.n_q_heads * splits * (c.head_dim + 2) * 4 : 0;
}
}  // namespace

kvq_status kvq_prefill_workspace_bytes(const kvq_config* cfg, int32_t n_q, int64_t n_ctx,
                                       uint64_t* out_bytes) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (!out_bytes) return fail(KVQ_ERR_INVALID_ARGUMENT, "out_bytes is NULL");
  if (n_ctx < 1 || n_ctx > cfg->max_ctx || n_q < 1 || n_q > n_ctx)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "need 1 <= n_q <= n_ctx <= max_ctx");
  *out_bytes = prefill_ws_bytes(*cfg, n_q, prefill_splits(*cfg, n_q, n_ctx));
  return KVQ_OK;
}

kvq_status kvq_prefill_attention(const kvq_config* cfg, const kvq_cache* cache, const void* q,
                                 int32_t n_q, float sm_scale, void* out, int32_t out_dtype,
                                 void* workspace, uint64_t workspace_bytes, void* stream) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (!cache) return fail(KVQ_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (!cache->base || !aligned16(cache->base))
    return fail(KVQ_ERR_INVALID_ARGUMENT, "cache->base must be a 16-byte aligned device pointer");
  if (cache->n_ctx < 1 || cache->n_ctx > cfg->max_ctx)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "n_ctx must be in [1, max_ctx] (got %lld)",
                (long long)cache->n_ctx);
  if (n_q < 1 || n_q > cache->n_ctx)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "n_q must be in [1, n_ctx] (got %d, n_ctx %lld): the "
                "queries are those of the last n_q cached tokens", n_q, (long long)cache->n_ctx);
  const int g = cfg->n_q_heads / cfg->n_kv_heads;
  if (64 % g != 0)
    return fail(KVQ_ERR_UNSUPPORTED, "prefill needs n_q_heads / n_kv_heads to divide 64 (got %d)", g);
  st = check_codebooks(*cfg, *cache);
  if (st != KVQ_OK) return st;
  if (!q || !out || !aligned16(q) || !aligned16(out))
    return fail(KVQ_ERR_INVALID_ARGUMENT, "q and out must be 16-byte aligned device pointers");
  if (out_dtype != KVQ_F32 && out_dtype != KVQ_F16 && out_dtype != KVQ_BF16)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "out_dtype must be KVQ_F32, KVQ_F16 or KVQ_BF16");
  if (!isfinite(sm_scale)) return fail(KVQ_ERR_INVALID_ARGUMENT, "sm_scale must be finite");
  if (workspace && !aligned16(workspace))
    return fail(KVQ_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");

  Layout L = make_layout(*cfg);
  PrefillArgs a;
  a.sh = DevShape{cfg->batch, cfg->n_q_heads, cfg->n_kv_heads, g, cfg->kv_dtype == KVQ_BF16, L.Tcap};
  set_paging(a.sh, L, *cache);
  a.k = make_dev_tensor(L.k, cache->base, cache->k_codebook, cache->k_scale);
  a.v = make_dev_tensor(L.v, cache->base, cache->v_codebook, cache->v_scale);
  uint8_t* base = static_cast<uint8_t*>(cache->base);
  a.k_sink = L.sink ? reinterpret_cast<const uint16_t*>(base + L.k.sink_off) : nullptr;
  a.v_sink = L.sink ? reinterpret_cast<const uint16_t*>(base + L.v.sink_off) : nullptr;
  a.sink_cap = L.sink;
  a.n_sink = (int)(cache->n_ctx < L.sink ? cache->n_ctx : L.sink);
  a.n_total = (int)cache->n_ctx;
  a.n_q = n_q;
  a.q = q;
  a.out = out;
  a.out_dtype = out_dtype;
  a.sm_scale = sm_scale > 0.0f ? sm_scale : (float)(1.0 / sqrt((double)cfg->head_dim));
  a.rope = cfg->rope;
  a.rope_base = cfg->rope_base;
  a.codes = prefill_codes_supported(*cfg) ? 1 : 0;
  // the split, as far as the workspace holds it
  int splits = prefill_splits(*cfg, n_q, cache->n_ctx);
  const uint64_t per_split = prefill_ws_bytes(*cfg, n_q, 2) / 2;
  const uint64_t fit = workspace ? workspace_bytes / per_split : 0;
  if ((uint64_t)splits > fit) splits = fit > 1 ? (int)fit : 1;
  const int64_t nblk = (a.n_sink + kTile - 1) / kTile + (a.n_total - a.n_sink + kTile - 1) / kTile;
  a.blocks_per_split = (int)((nblk + splits - 1) / splits);
  a.splits = (int)((nblk + a.blocks_per_split - 1) / a.blocks_per_split);
  a.partial = a.splits > 1 ? static_cast<float*>(workspace) : nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_prefill(a, s);
  if (e == hipSuccess && a.splits > 1) {
    // merge the splits' partial states: rows (b, i) as sequences of Hq heads
    DecodeArgs c{};
    c.sh = a.sh;
    c.sh.B = cfg->batch * n_q;
    c.partial = a.partial;
    c.S_max = a.splits;
    c.n_partials = a.splits;
    c.out = out;
    c.out_dtype = out_dtype;
    e = launch_combine(c, s);
  }
  return device_status(e, "prefill attention");
}

}  // extern "C"
