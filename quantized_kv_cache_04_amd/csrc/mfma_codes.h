// Matrix-core operand helpers of libkvq, shared by the decode and the
// prefill kernels: packed codes unpacked into exact fp16 subnormal operands
// of v_mfma_f32_16x16x32_f16 (a code c in the low bits of an fp16 is
// c * 2^-24), fp32 values split into fp16 high and low parts, and the pair
// order both operands use.
#pragma once
#include <hip/hip_runtime.h>

#include "device_common.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half8 as_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(half8, v);
}

__device__ __forceinline__ f32x4 mfma16(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 2^e for integer e in [-126, 127]
__device__ __forceinline__ float pow2i(int e) {
  return __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
}
// smallest e with x <= 2^e, for x > 0 (x = 0 -> -126)
__device__ __forceinline__ int ceil_log2(float x) {
  if (!(x > 0.0f)) return -126;
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  int e = (int)((u >> 23) & 0xff) - 127;
  if (u & 0x7fffff) ++e;
  return e < -126 ? -126 : e;
}

// Two fp32 values rounded to the nearest fp16 (one v_cvt_pk_f16_f32)
__device__ __forceinline__ half2v cvt_pk_rn(float x0, float x1) {
  return __builtin_convertvector(f32x2{x0, x1}, half2v);
}

// Two fp32 values as the fp16 high parts (lo_mask = 0) or low parts
// (lo_mask = 1) of a high/low pair: hi = x rounded to the nearest fp16,
// lo = (x - hi) rounded to nearest.  Both roundings are unbiased, so the
// error of hi + lo does not pile up in one direction over long sums, even
// where lo (or hi) is an fp16 subnormal.
__device__ __forceinline__ uint32_t hilo2(float x0, float x1, float lo_mask) {
  const half2v h = cvt_pk_rn(x0, x1);
  const float y0 = x0 - lo_mask * (float)h[0];
  const float y1 = x1 - lo_mask * (float)h[1];
  return __builtin_bit_cast(uint32_t, cvt_pk_rn(y0, y1));
}

// hi/lo split of two fp32 values without scaling (see hilo2)
__device__ __forceinline__ uint32_t hilo_split(float x0, float x1, float lo_mask) {
  return hilo2(x0, x1, lo_mask);
}

// ---- code unpacking: block of 8 codes -> 4 dwords of subnormal fp16 pairs ---
// pair r holds elements (r, r + 4) of the block.  4-bit pairs 1 and 3 carry a
// factor 16 (the nibble sits 4 bits up), compensated in the other operand.
template <int BITS>
struct Unpack;

template <>
struct Unpack<4> {
  static constexpr float f[4] = {1.0f, 1.0f / 16.0f, 1.0f, 1.0f / 16.0f};
  template <bool FLIP>
  __device__ static __forceinline__ void run(uint32_t w, uint32_t out[4]) {
    const uint32_t w8 = w >> 8;
    out[0] = w & 0x000f000fu;
    out[1] = (FLIP ? ~w : w) & 0x00f000f0u;     // one v_bitop3 either way
    out[2] = w8 & 0x000f000fu;
    out[3] = (FLIP ? ~w8 : w8) & 0x00f000f0u;
  }
};

template <>
struct Unpack<3> {
  // Pair r as code * 4^r (the factor 4^-r sits in the other operand): its
  // low two bits come from dlo = D[m / 2] at bit 2r (+ 8 for odd m), its high
  // bit from d2, where it sits at H = 8 (m / 2) + 2r + (m % 2) and one shift
  // per block moves it to 2r + 2.  The two fields are disjoint, so one AND
  // and one AND-OR give the whole code.  FLIP complements the odd pairs:
  // their low and high bits both sit under the mask 0xcccc of each half.
  template <bool FLIP>
  __device__ static __forceinline__ void run(uint32_t dlo, uint32_t d2, int m, uint32_t out[4]) {
    if (FLIP) { dlo ^= 0xccccccccu; d2 ^= 0xccccccccu; }
    const uint32_t l = (m & 1) ? (dlo >> 8) : dlo;
    const int sh = 8 * (m >> 1) + (m & 1) - 2;
    const uint32_t h = sh >= 0 ? (d2 >> sh) : (d2 << (-sh));
#pragma unroll
    for (int r = 0; r < 4; ++r)
      out[r] = (l & (0x00030003u << (2 * r))) | (h & (0x00010001u << (2 * r + 2)));
  }
};

template <>
struct Unpack<8> {
  static constexpr float f[4] = {1.0f, 1.0f, 1.0f, 1.0f};
  // d0: elements 0-3, d1: elements 4-7 (already offset to unsigned)
  __device__ static __forceinline__ void run(uint32_t d0, uint32_t d1, uint32_t out[4]) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      out[r] = __builtin_amdgcn_perm(d1, d0, 0x0c000c00u | ((uint32_t)(4 + r) << 16) | (uint32_t)r);
  }
};

// codes of block m of a segment of BITS-bit codes held in ``seg`` dwords
// (3-bit codes: the 12-byte segment of 32 codes, low-bit dwords D[0..1] and
// the high-bit dword D[2]).  FLIP: the odd pairs hold the complemented codes
// (2^BITS - 1) - c (signed 8-bit: 127 - q, the complement of the offset code
// q + 128).
template <int BITS, bool SIGNED, bool FLIP = false>
__device__ __forceinline__ half8 seg_block(const uint32_t* seg, int m) {
  uint32_t o[4];
  if constexpr (BITS == 4) {
    Unpack<4>::run<FLIP>(seg[m], o);
  } else if constexpr (BITS == 3) {
    Unpack<3>::run<FLIP>(seg[m >> 1], seg[2], m, o);
  } else {
    // pair r takes byte r of both dwords: bytes 1 and 3 are the odd pairs
    constexpr uint32_t kFlipMask = SIGNED ? 0x7f807f80u : 0xff00ff00u;
    constexpr uint32_t kX = FLIP ? kFlipMask : (SIGNED ? 0x80808080u : 0u);
    const uint32_t d0 = seg[2 * m] ^ kX, d1 = seg[2 * m + 1] ^ kX;
    Unpack<8>::run(d0, d1, o);
  }
  return as_h8(o[0], o[1], o[2], o[3]);
}

// FP8 E5M2 block m of a segment of byte codes: the bytes become the high
// bytes of fp16 values (exact); pair r = (byte r of dword 2m, byte r of
// dword 2m + 1), the pair order of the byte unpack above.
__device__ __forceinline__ half8 fp8_block(const uint32_t* seg, int m) {
  const uint32_t d0 = seg[2 * m], d1 = seg[2 * m + 1];
  uint32_t o[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
    o[r] = __builtin_amdgcn_perm(d1, d0, ((uint32_t)(4 + r) << 24) | 0x000c0000u | ((uint32_t)r << 8) | 0x0cu);
  return as_h8(o[0], o[1], o[2], o[3]);
}

// operand of block m of a segment: FP8 E5M2 bytes (F8) or BITS-bit codes
template <int BITS, bool SIGNED, bool FLIP, bool F8>
__device__ __forceinline__ half8 code_block(const uint32_t* seg, int m) {
  if constexpr (F8)
    return fp8_block(seg, m);
  else
    return seg_block<BITS, SIGNED, FLIP>(seg, m);
}

// factor of pair r that the other operand of a code operand must carry
template <int BITS>
__device__ __forceinline__ float pair_factor(int r) {
  if constexpr (BITS == 4) return (r & 1) ? 1.0f / 16.0f : 1.0f;
  if constexpr (BITS == 3) return r == 0 ? 1.0f : (r == 1 ? 0.25f : (r == 2 ? 0.0625f : 0.015625f));
  return 1.0f;
}

// P operand pairs with the same factor share an exponent class: 4-bit values
// (odd pairs unpack 4 bits up: 2^-4) and 3-bit values (pair r: 4^-r)
template <int VB>
constexpr int kClasses = VB == 3 ? 4 : 2;
template <int VB>
__device__ __forceinline__ constexpr int pe_class(int r) { return VB == 3 ? r : (r & 1); }
template <int VB>
__device__ __forceinline__ constexpr int pe_exp(int cls) { return VB == 3 ? 2 * cls : (VB == 4 ? 4 * cls : 0); }

// Operand in "pair order" from 8 values x[e] (e = 0..7): pair r = (x[r],
// x[r + 4]) times sc and divided by the unpack factor of the other operand,
// as fp16 high and low parts.  The high part sits on a fixed grid: with
// |x * sc| <= 2^14 for every value the wave feeds, hi is
// x * sc * pair_factor rounded to a multiple of 16 * pair_factor (at most
// 1024 steps, exact in fp16), lo = the rest rounded to nearest.  Every
// high-part product with a code is then an integer multiple of 16 * 2^-24,
// and a sum of 32 of them is exact within the matrix cores' adder, which
// otherwise drops the low bits of products far below the largest one (the
// error that would leave grows with the spread of |q * scale| over the
// channels, and it does not cancel).
template <int BITS>
__device__ __forceinline__ void pair_operand_fixed(const float x[8], float sc, u32x4& hi, u32x4& lo) {
  uint32_t h[4], l[4];
  const float c16 = sc * 0.0625f;   // x * sc / 16: the grid index (all factors are powers of two)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float f = sc * pair_factor<BITS>(r);
    const float step = 16.0f * pair_factor<BITS>(r);
    const float ha = __builtin_rintf(x[r] * c16) * step, hb = __builtin_rintf(x[r + 4] * c16) * step;
    h[r] = __builtin_bit_cast(uint32_t, cvt_pk_rn(ha, hb));
    l[r] = __builtin_bit_cast(uint32_t, cvt_pk_rn(__builtin_fmaf(x[r], f, -ha), __builtin_fmaf(x[r + 4], f, -hb)));
  }
  hi = u32x4{h[0], h[1], h[2], h[3]};
  lo = u32x4{l[0], l[1], l[2], l[3]};
}

// Load ``N`` dwords from a 4-byte aligned address.
template <int N>
__device__ __forceinline__ void load_dw(const uint8_t* p, uint32_t* out) {
  const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(q + 4 * i);
      out[4 * i] = v.x; out[4 * i + 1] = v.y; out[4 * i + 2] = v.z; out[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = q[i];
  }
}

}  // namespace
}  // namespace kvq
