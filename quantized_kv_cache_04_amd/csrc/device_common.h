// Device helpers shared by the libkvq kernels: element conversions and the
// addressing of the packed cache layouts (see include/kvq.h,
// kvq_cache_layout, for the layout contract).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {

__device__ __forceinline__ float h2f(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ float bf2f(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}
__device__ __forceinline__ float elem2f(uint16_t h, int is_bf16) {
  return is_bf16 ? bf2f(h) : h2f(h);
}
// Round-to-nearest-even conversions.
__device__ __forceinline__ uint16_t f2h_rn(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ uint16_t f2bf_rn(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---- token rows of the per-token arrays ---------------------------------------
// Entry lp of sequence b of a paged cache's table, read through the
// constant address space: the table does not change during a kernel, and
// with a wave-uniform index this is a scalar load, which a kernel can wait
// for without waiting for its vector loads in flight.
typedef __attribute__((address_space(4))) const int32_t const_i32;
__device__ __forceinline__ int table_entry(const DevShape& sh, int b, int64_t lp) {
  const const_i32* t = (const const_i32*)sh.page_table;
  return t[(int64_t)b * sh.pages_per_seq + lp];
}
// Physical page of a table entry.  Entries outside [0, n_pages) are clamped
// into it: a bad table gives wrong values, never an access outside the
// allocation.
__device__ __forceinline__ int64_t clamp_page(const DevShape& sh, int p) {
  return (int64_t)min(max(p, 0), sh.n_pages - 1);
}
__device__ __forceinline__ int64_t page_of(const DevShape& sh, int b, int64_t lp) {
  return clamp_page(sh, table_entry(sh, b, lp));
}
// Row of token 0 of (physical page p, KV head h): see tok_row.
__device__ __forceinline__ int64_t page_head_row(const DevShape& sh, int64_t p, int h) {
  return (p * sh.Hkv + h) * kTile;
}
// Row of token t of (sequence b, KV head h) in the arrays with one record
// per token and head (codes, per-token parameters; value tiles are 32 rows):
// [B][Hkv][Tcap] in a contiguous cache, [page][Hkv][kTile] in a paged one.
// The kTile tokens of one page and head are consecutive rows either way.
__device__ __forceinline__ int64_t tok_row(const DevShape& sh, int b, int h, int64_t t) {
  if (!sh.page_table) return ((int64_t)b * sh.Hkv + h) * sh.Tcap + t;
  return page_head_row(sh, page_of(sh, b, t / kTile), h) + (t % kTile);
}
// Index of the first parameter record of token t of (sequence b, KV head h)
// in a per-token parameter array (records of one token are consecutive):
// tok_row * ng for one group size; with a group size per head the heads'
// records of a sequence (or page) follow one another,
// [B][h][Tcap][ngh[h]] or [page][h][kTile][ngh[h]].
__device__ __forceinline__ int64_t prm_rec(const DevTensor& p, const DevShape& sh, int b, int h,
                                           int64_t t) {
  if (!p.per_head) return tok_row(sh, b, h, t) * p.ng;
  const int64_t tot = p.ng_pre[sh.Hkv], pre = p.ng_pre[h], nh = p.ngh[h];
  if (!sh.page_table) return sh.Tcap * ((int64_t)b * tot + pre) + t * nh;
  return (int64_t)kTile * (page_of(sh, b, t / kTile) * tot + pre) + (t % kTile) * nh;
}
// The tensor as head h sees it: its group size and groups per token.
__device__ __forceinline__ DevTensor head_view(const DevTensor& p, int h) {
  DevTensor v = p;
  if (p.per_head) {
    v.ng = p.ngh[h];
    v.G = kHeadDim / p.ngh[h];
  }
  return v;
}

// Row of token t of sequence b in the outlier CSR (one row per token, all
// heads): b * Tcap + t, or page * kTile + t mod kTile.
__device__ __forceinline__ int64_t csr_row(const DevShape& sh, int b, int64_t t) {
  if (!sh.page_table) return (int64_t)b * sh.Tcap + t;
  return page_of(sh, b, t / kTile) * kTile + (t % kTile);
}

// ---- segment of 32 codes (u = 8m + e) ---------------------------------------
// 8-bit: byte u.  4-bit: nibble u (low nibble = even u).  3-bit: see kvq.h.
__device__ __forceinline__ uint32_t seg_code(const uint8_t* seg, int bits, int u) {
  if (bits == 8) return seg[u];
  if (bits == 4) return (seg[u >> 1] >> ((u & 1) * 4)) & 15u;
  const int m = u >> 3, e = u & 7, r = e & 3, hi16 = (e >> 2) * 16;
  const int p = 4 * (m & 1) + r, H = 8 * (m >> 1) + 2 * r + (m & 1);
  const uint32_t* dw = reinterpret_cast<const uint32_t*>(seg);
  const uint32_t lo2 = (dw[m >> 1] >> (2 * p + hi16)) & 3u;
  const uint32_t hi1 = (dw[2] >> (H + hi16)) & 1u;
  return lo2 | (hi1 << 2);
}

// Key rows: segment q holds channels 32m + 8q + e.
__device__ __forceinline__ uint32_t k_row_code(const uint8_t* row, int bits, int c) {
  const int q = (c & 31) >> 3, u = ((c >> 5) << 3) | (c & 7);
  return seg_code(row + q * 4 * bits, bits, u);
}

// Value tiles: token tau of the tile and channel c.
__device__ __forceinline__ uint32_t v_tile_code(const uint8_t* tile, int bits, int tau, int c) {
  const int q = (tau & 15) >> 2, e = (tau & 3) + 4 * (tau >> 4);
  const int nb = c >> 4, i = c & 15;
  const int lane = 16 * q + i, s = nb >> 2, m = nb & 3;
  return seg_code(tile + lane * 8 * bits + s * 4 * bits, bits, 8 * m + e);
}

// Codebook value tiles: byte 32 l + tau holds channel l (low nibble) and
// channel l + 64 (high nibble) of token tau.
__device__ __forceinline__ uint32_t v_pair_code(const uint8_t* tile, int tau, int c) {
  return (tile[(c & 63) * 32 + tau] >> (4 * (c >> 6))) & 15u;
}

// Bit fields of dword j of a segment: calls f(u, shift, width, field) where
// ``field`` is 0 for the whole code, 1 for the low two bits, 2 for the high
// bit (3-bit packing).
template <typename F>
__device__ __forceinline__ void seg_dword_fields(int bits, int j, F&& f) {
  if (bits == 8) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f(4 * j + e, 8 * e, 8, 0);
  } else if (bits == 4) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f(8 * j + e, 4 * e, 4, 0);
  } else if (j < 2) {
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 2 * j + mm, p = 4 * mm + r;
        f(8 * m + r, 2 * p, 2, 1);
        f(8 * m + r + 4, 16 + 2 * p, 2, 1);
      }
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int H = 8 * (m >> 1) + 2 * r + (m & 1);
        f(8 * m + r, H, 1, 2);
        f(8 * m + r + 4, 16 + H, 1, 2);
      }
  }
}

__device__ __forceinline__ uint32_t field_value(uint32_t code, int field) {
  return field == 0 ? code : (field == 1 ? (code & 3u) : (code >> 2) & 1u);
}

// ---- FP8 E5M2 -----------------------------------------------------------------
// E5M2 is the high byte of an fp16: decoding is exact.
__device__ __forceinline__ float e5m2_to_f(uint32_t code) {
  return h2f((uint16_t)((code & 0xffu) << 8));
}
// float32 -> E5M2 byte, round to nearest even, magnitudes of 57344 and
// beyond saturate to 57344; the sign is kept (also for zero).  NaN inputs
// are outside the cache contract.
__device__ __forceinline__ uint32_t f_to_e5m2(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  const uint32_t sign = (u >> 24) & 0x80u, a = u & 0x7fffffffu;
  uint32_t r;
  if (a >= 0x47600000u) {
    r = 0x7bu;
  } else if (a >= 0x38800000u) {
    // normal: rebias the exponent (127 -> 15) and round the mantissa to 2 bits
    const uint32_t b = a - (112u << 23);
    r = (b + 0x000fffffu + ((b >> 21) & 1u)) >> 21;
  } else {
    // below 2^-14: multiples of 2^-16 (4 is the smallest normal)
    r = (uint32_t)rintf(__builtin_bit_cast(float, a) * 65536.0f);
  }
  return sign | r;
}

__device__ __forceinline__ float fp8_scale(const DevTensor& t, int h) {
  return t.hscale ? t.hscale[h] : 1.0f;
}

// ---- element-wise dequantization (general kernel, prefill staging) --------
__device__ __forceinline__ float deq_uniform(uint32_t code, int quant, const void* params,
                                             int64_t rec) {
  if (quant == KVQ_QUANT_SYM_Q8_0)
    return (float)(int8_t)code * h2f(static_cast<const uint16_t*>(params)[rec]);
  const uint32_t pz = static_cast<const uint32_t*>(params)[rec];
  return (float)code * h2f((uint16_t)(pz & 0xffff)) + h2f((uint16_t)(pz >> 16));
}

// Dense (codebook or uniform) value of key channel c of token t of KV head h
// (bh = b * Hkv + h); per-channel keys past n_full come from the tail.
__device__ inline float deq_key(const DevTensor& k, const DevShape& sh, int bh, int h, int64_t t,
                                int c, int64_t n_full) {
  const int64_t row = tok_row(sh, bh / sh.Hkv, h, t);
  if (k.quant == KVQ_QUANT_NONE)
    return elem2f(reinterpret_cast<const uint16_t*>(k.codes)[row * kHeadDim + c], sh.kv_bf16);
  if (k.per_channel && t >= n_full)
    return elem2f(k.tail[((int64_t)bh * k.tail_rows + t % k.tail_rows) * kHeadDim + c], sh.kv_bf16);
  const uint32_t code = k_row_code(k.codes + row * k.row_bytes, k.bits, c);
  if (k.quant == KVQ_QUANT_CODEBOOK) return h2f(k.codebook[((int64_t)h * kHeadDim + c) * 16 + code]);
  if (k.quant == KVQ_QUANT_FP8_E5M2) return e5m2_to_f(code) * fp8_scale(k, h);
  if (k.per_channel)
    return deq_uniform(code, k.quant, k.params,
                       ((int64_t)bh * (sh.Tcap / k.G) + t / k.G) * kHeadDim + c);
  return deq_uniform(code, k.quant, k.params,
                     prm_rec(k, sh, bh / sh.Hkv, h, t) + c / head_view(k, h).G);
}

// Dense value of value channel c of token t of KV head h.
__device__ inline float deq_value(const DevTensor& v, const DevShape& sh, int bh, int h, int64_t t,
                                  int c) {
  const int64_t row = tok_row(sh, bh / sh.Hkv, h, t);
  if (v.quant == KVQ_QUANT_NONE)
    return elem2f(reinterpret_cast<const uint16_t*>(v.codes)[row * kHeadDim + c], sh.kv_bf16);
  const uint8_t* tile = v.codes + (row - (t & (kTile - 1))) * v.row_bytes;
  if (v.quant == KVQ_QUANT_CODEBOOK) {
    const uint32_t code = v_pair_code(tile, (int)(t & (kTile - 1)), c);
    return h2f(v.codebook[((int64_t)h * kHeadDim + c) * 16 + code]);
  }
  const uint32_t code = v_tile_code(tile, v.bits, (int)(t & (kTile - 1)), c);
  if (v.quant == KVQ_QUANT_FP8_E5M2) return e5m2_to_f(code) * fp8_scale(v, h);
  return deq_uniform(code, v.quant, v.params,
                     prm_rec(v, sh, bh / sh.Hkv, h, t) + c / head_view(v, h).G);
}

// ---- cross-lane reductions (wave of 64 lanes) -----------------------------------
// x of lane l + k (row rotations within each row of 16 lanes, by DPP)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
// x of lane l ^ 16 and of lane l ^ 32, by the gfx950 row swaps: of the pair
// permlane{16,32}_swap returns for (x, x), one element is x[l] and the
// other the partner's
__device__ __forceinline__ float swap16(float x) {
  const int xi = __builtin_bit_cast(int, x);
  auto c = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
  return __builtin_bit_cast(float, (int)((__lane_id() & 16) ? c[0] : c[1]));
}
__device__ __forceinline__ float swap_halves(float x) {
  const int xi = __builtin_bit_cast(int, x);
  auto c = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return __builtin_bit_cast(float, (int)((__lane_id() & 32) ? c[0] : c[1]));
}
// maximum / sum over the 4 rows of 16 lanes (lanes l, l^16, l^32, l^48);
// both elements of a swap pair enter symmetrically, so every lane gets the
// same bits
__device__ __forceinline__ float rows_max(float x) {
  const int xi = __builtin_bit_cast(int, x);
  auto a = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
  x = fmaxf(__builtin_bit_cast(float, (int)a[0]), __builtin_bit_cast(float, (int)a[1]));
  const int yi = __builtin_bit_cast(int, x);
  auto c = __builtin_amdgcn_permlane32_swap(yi, yi, false, false);
  return fmaxf(__builtin_bit_cast(float, (int)c[0]), __builtin_bit_cast(float, (int)c[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  const int xi = __builtin_bit_cast(int, x);
  auto a = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
  x = __builtin_bit_cast(float, (int)a[0]) + __builtin_bit_cast(float, (int)a[1]);
  const int yi = __builtin_bit_cast(int, x);
  auto c = __builtin_amdgcn_permlane32_swap(yi, yi, false, false);
  return __builtin_bit_cast(float, (int)c[0]) + __builtin_bit_cast(float, (int)c[1]);
}
// maximum / sum over the whole wave: rotations within each row of 16, then
// across the rows
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<0x128>(x));   // row_ror:8
  x = fmaxf(x, dpp_f<0x124>(x));   // row_ror:4
  x = fmaxf(x, dpp_f<0x122>(x));   // row_ror:2
  x = fmaxf(x, dpp_f<0x121>(x));   // row_ror:1
  return rows_max(x);
}
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f<0x128>(x);
  x += dpp_f<0x124>(x);
  x += dpp_f<0x122>(x);
  x += dpp_f<0x121>(x);
  return rows_sum(x);
}

// ---- rotary embedding --------------------------------------------------------------
// (cos, sin) of the rotation by dt * theta.  The angle is formed and reduced
// to [-pi, pi] in float64, so that no error grows with the position, and
// only the reduced angle goes through the float32 sincosf.
__device__ __forceinline__ float2 rope_cs(double theta, int64_t dt) {
  const double ang = (double)dt * theta;
  const double two_pi = 6.283185307179586476925286766559;
  const double red = ang - two_pi * rint(ang / two_pi);
  float sn, cs;
  sincosf((float)red, &sn, &cs);
  return make_float2(cs, sn);
}

}  // namespace kvq
