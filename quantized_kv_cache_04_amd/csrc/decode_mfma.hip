// Matrix-core decode kernel of libkvq for uniform formats (3/4/8-bit
// asymmetric or q8_0 codes, per-token or per-channel keys) and GQA groups of
// up to 8 query heads per KV head.
//
// Decode attention streams the whole cache once per step (Memory-killer
// page, sections 1.3 and 4.2); dequantization is fused into the two
// products (Memory-killer page, section 2.3; KVQuant page, section 3.4) and
// the softmax stays in registers (Survey page, section 2.3).  With a GQA
// group the scores of one KV head are a small dense contraction, so both
// products run on the gfx950 matrix cores (v_mfma_f32_16x16x32_f16):
//
//  * QK^T: rows = 16 tokens, columns n = j + 8*hl (query head j of the
//    group, hl = 0 for the high and 1 for the low fp16 part of the fp32
//    operand), K = 32 channels per instruction.  The packed codes are the A
//    operand as-is: a code placed in the low bits of an fp16 is the exact
//    subnormal code * 2^-24, so a nibble dword unpacks with a few masks.
//    The other operand (q for per-token keys, q * scale for per-channel
//    keys) is pre-scaled by a power of two and split into fp16 high and low
//    parts, which keeps the products exact to about 2^-22.
//  * P.V: rows n = j + 8*hl (high/low parts of p * value-scale), K = 32
//    tokens, columns = 16 channels.  The register layout of the QK^T result
//    (lane (q, n) holds tokens 4q + r and 16 + 4q + r) is exactly the A
//    operand the value tiles are packed for, so no data moves between the
//    two products.
//
// Zero points enter as per-group sums (sum_c q_c z_c for per-channel keys,
// z * sum_c q_c for per-token keys, sum_t p_t z_t for values).  q8_0 codes
// are fed as x + 128 (unsigned) and the 128 * sum term is removed.
//
// Grid: (splits, B * Hkv); 256 threads = 4 waves, each wave a contiguous run
// of 32-token blocks.  The four waves are merged in LDS and the split-K
// partials by the last block (splitk.h).
#include <hip/hip_runtime.h>

#include "splitk.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = kHeadDim;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ half8 as_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(half8, v);
}

__device__ __forceinline__ f32x4 mfma16(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// value of lane (lane + 8) mod 16 within each row of 16 lanes
__device__ __forceinline__ float dpp_ror8(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));
}

__device__ __forceinline__ float rows_max(float x) {  // over the 4 rows of 16 lanes
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  return fmaxf(x, __shfl_xor(x, 32, 64));
}
__device__ __forceinline__ float rows_sum(float x) {
  x += __shfl_xor(x, 16, 64);
  return x + __shfl_xor(x, 32, 64);
}
__device__ __forceinline__ float wave_max(float x) {
  for (int off = 1; off < 64; off <<= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
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

// fp16 high part (lo = false) or low part (lo = true) of x, as raw bits
__device__ __forceinline__ uint32_t split16(float x, bool lo) {
  const _Float16 h = (_Float16)x;
  const _Float16 r = lo ? (_Float16)(x - (float)h) : h;
  return (uint32_t)__builtin_bit_cast(uint16_t, r);
}

// ---- code unpacking: block of 8 codes -> 4 dwords of subnormal fp16 pairs ---
// pair r holds elements (r, r + 4) of the block.  4-bit pairs 1 and 3 carry a
// factor 16 (the nibble sits 4 bits up), compensated in the other operand.
template <int BITS>
struct Unpack;

template <>
struct Unpack<4> {
  static constexpr float f[4] = {1.0f, 1.0f / 16.0f, 1.0f, 1.0f / 16.0f};
  __device__ static __forceinline__ void run(uint32_t w, uint32_t out[4]) {
    const uint32_t w8 = w >> 8;
    out[0] = w & 0x000f000fu;
    out[1] = w & 0x00f000f0u;
    out[2] = w8 & 0x000f000fu;
    out[3] = w8 & 0x00f000f0u;
  }
};

template <>
struct Unpack<3> {
  static constexpr float f[4] = {1.0f, 1.0f, 1.0f, 1.0f};
  // dlo: dword with the low two bits of block m (D[m / 2]); d2: high bits
  __device__ static __forceinline__ void run(uint32_t dlo, uint32_t d2, int m, uint32_t out[4]) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int p = 4 * (m & 1) + r, P = 4 * m + r;
      const uint32_t lo2 = (dlo >> (2 * p)) & 0x00030003u;
      const uint32_t hi1 = (P >= 2 ? (d2 >> (P - 2)) : (d2 << (2 - P))) & 0x00040004u;
      out[r] = lo2 | hi1;
    }
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
template <int BITS, bool SIGNED>
__device__ __forceinline__ half8 seg_block(const uint32_t* seg, int m) {
  uint32_t o[4];
  if constexpr (BITS == 4) {
    Unpack<4>::run(seg[m], o);
  } else if constexpr (BITS == 3) {
    Unpack<3>::run(seg[m >> 1], seg[2], m, o);
  } else {
    uint32_t d0 = seg[2 * m], d1 = seg[2 * m + 1];
    if (SIGNED) { d0 ^= 0x80808080u; d1 ^= 0x80808080u; }
    Unpack<8>::run(d0, d1, o);
  }
  return as_h8(o[0], o[1], o[2], o[3]);
}

template <int BITS>
__device__ __forceinline__ float pair_factor(int r) {
  if constexpr (BITS == 4) return (r & 1) ? 1.0f / 16.0f : 1.0f;
  return 1.0f;
}

// Operand in "pair order" from 8 values x[e] (e = 0..7): pair r = (x[r], x[r + 4])
// each divided by the unpack factor of the other operand, scaled by ``sc`` and
// split into the high or low fp16 part.
template <int BITS>
__device__ __forceinline__ half8 pair_operand(const float x[8], float sc, bool lo) {
  uint32_t o[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float f = sc * pair_factor<BITS>(r);
    o[r] = split16(x[r] * f, lo) | (split16(x[r + 4] * f, lo) << 16);
  }
  return as_h8(o[0], o[1], o[2], o[3]);
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

// Parameters of this lane's 8 tokens (4q + r and 16 + 4q + r of the block):
// NG groups per token; scale (and zero unless Q8) as float.
template <bool Q8, int NG>
__device__ __forceinline__ void load_token_params(const void* params, int64_t rec0, int q4,
                                                  int valid_to, float s[2][4][NG],
                                                  float z[2][4][NG]) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int64_t t4 = rec0 + 16 * mb + 4 * q4;      // first of 4 consecutive tokens
    if constexpr (Q8) {
      // 4 * NG fp16 scales = 2 * NG dwords
      const uint16_t* p = static_cast<const uint16_t*>(params) + t4 * NG;
      uint32_t d[2 * NG];
      load_dw<2 * NG>(reinterpret_cast<const uint8_t*>(p), d);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          const int idx = r * NG + gi;
          s[mb][r][gi] = h2f((uint16_t)(d[idx >> 1] >> (16 * (idx & 1))));
          z[mb][r][gi] = 0.f;
        }
    } else {
      const uint32_t* p = static_cast<const uint32_t*>(params) + t4 * NG;
      uint32_t d[4 * NG];
      load_dw<4 * NG>(reinterpret_cast<const uint8_t*>(p), d);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          s[mb][r][gi] = h2f((uint16_t)(d[r * NG + gi] & 0xffff));
          z[mb][r][gi] = h2f((uint16_t)(d[r * NG + gi] >> 16));
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (16 * mb + 4 * q4 + r >= valid_to) {
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) { s[mb][r][gi] = 0.f; z[mb][r][gi] = 0.f; }
      }
  }
}

template <int KB, bool KCH, bool KQ8, int NGK, int VB, bool VQ8, int NGV>
__global__ __launch_bounds__(256) void dec_mfma_kernel(DecodeArgs a) {
  __shared__ float wm[4][8], wl[4][8];
  __shared__ float wo[4][8][kD];
  __shared__ float wb[4][8][NGV];   // per wave, head, value group: additive term
  __shared__ int flag;

  const int split = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.sh.Hkv, h = bh % a.sh.Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q4 = lane >> 4, n = lane & 15, j = n & 7;
  const bool lo_lane = n >= 8;
  const int g = a.sh.g;
  const int nctx = a.n_ctx;
  const int64_t Tcap = a.sh.Tcap;
  const DevTensor& K = a.k;
  const DevTensor& V = a.v;
  const int Gk = K.G;
  const int n_full = KCH ? (nctx / Gk) * Gk : nctx;
  const int64_t prow = (int64_t)bh * Tcap;   // token record of token 0 of (b, h)

  // ---- token range of this wave (whole 32-token blocks) ----------------------
  const int blk0 = split * a.blocks_per_split;
  const int nblk_total = (nctx + kTile - 1) / kTile;
  const int blk1 = min(nblk_total, blk0 + a.blocks_per_split);
  const int nb_split = blk1 - blk0;
  const int per_wave = (nb_split + 3) / 4;
  const int wb0 = blk0 + min(nb_split, wave * per_wave);
  const int wb1 = blk0 + min(nb_split, (wave + 1) * per_wave);

  // ---- query of this lane's column: head j, channels 32m + 8*q4 + e -------------
  const bool head_ok = j < g;
  float qv[4][8];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         ((int64_t)b * a.sh.Hq + h * g + (head_ok ? j : 0)) * kD;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qp + 32 * m + 8 * q4);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t bits = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        qv[m][e] = head_ok ? elem2f(bits, a.sh.kv_bf16) : 0.0f;
      }
    }
  }
  const float sm2 = a.sm_scale * kLog2e;

  // ---- per-token keys: fixed B operand, scaled by 2^Eq ---------------------------
  half8 bq[4];
  float qsum[NGK];   // per key group: sum of q (high lanes only), true units
  float qoff[NGK];   // q8_0: 128 * 2^-24 * sum of the fed operand (MFMA output units)
  float kq = 0.f;    // MFMA output units -> true units
  if constexpr (!KCH) {
    float mx = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(qv[m][e]));
    mx = wave_max(mx);
    int Eq = 14 - ceil_log2(mx);
    if (Eq > 100) Eq = 100;
    kq = pow2i(24 - Eq > 126 ? 126 : 24 - Eq);
    const float sc = pow2i(Eq);
#pragma unroll
    for (int gi = 0; gi < NGK; ++gi) { qsum[gi] = 0.f; qoff[gi] = 0.f; }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      bq[m] = pair_operand<KB>(qv[m], sc, lo_lane);
      const int grp = m * NGK / 4;
      float s = 0.f, so = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s += qv[m][e];
      if constexpr (KQ8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) so += (float)bq[m][e];
      }
      qsum[grp] += s;
      qoff[grp] += so;
    }
#pragma unroll
    for (int gi = 0; gi < NGK; ++gi) {
      qsum[gi] = lo_lane ? 0.f : rows_sum(qsum[gi]);
      qoff[gi] = 128.0f * 0x1p-24f * rows_sum(qoff[gi]);
    }
  }

  // ---- value scale exponent of this wave's range: p * scale * 2^(24-Ev) <= 2^14
  int Ev;
  {
    float mx = 0.f;
    const int t_lo = wb0 * kTile, t_hi = min(nctx, wb1 * kTile);
    for (int t = t_lo + lane; t < t_hi; t += 64) {
#pragma unroll
      for (int gi = 0; gi < NGV; ++gi) {
        float s;
        if (VQ8) s = h2f(static_cast<const uint16_t*>(V.params)[(prow + t) * NGV + gi]);
        else s = h2f((uint16_t)(static_cast<const uint32_t*>(V.params)[(prow + t) * NGV + gi] & 0xffff));
        mx = fmaxf(mx, s);
      }
    }
    mx = wave_max(mx);
    Ev = ceil_log2(mx) + 10;
  }
  const int pexp = 24 - Ev > 126 ? 126 : 24 - Ev;
  const float pscale = pow2i(pexp);           // fed P operand = p * scale * pscale
  const float vscale = pow2i(-pexp);          // fed units -> true units (with 2^-24 codes: x 2^24)

  // ---- running state -----------------------------------------------------------
  f32x4 oacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;   // per column head j (lanes n, n + 8 agree)
  float l_run = 0.f;         // partial over this lane's tokens
  float vbias[NGV];          // sum p * zero (values), true units
  float voff[NGV];           // q8_0: sum of the fed P operand
#pragma unroll
  for (int gi = 0; gi < NGV; ++gi) { vbias[gi] = 0.f; voff[gi] = 0.f; }

  // per-channel keys: B operand of the current key group
  half8 bk[4];
  float kbias = 0.f;
  float kscale = 0.f;
  int cur_group = -1;

  const uint8_t* kcodes = K.codes + prow * K.row_bytes;
  const uint8_t* vcodes = V.codes + prow * V.row_bytes;

  for (int blk = wb0; blk < wb1; ++blk) {
    const int t0 = blk * kTile;
    const int valid = nctx - t0;            // tokens of this block that exist
    // ---------------- loads ----------------
    uint32_t kseg[2][KB];
    uint32_t vlane[2 * VB];
    const bool tail_blk = KCH && t0 >= n_full;
    if (!tail_blk) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        load_dw<KB>(kcodes + (int64_t)(t0 + 16 * mb + n) * K.row_bytes + q4 * 4 * KB, kseg[mb]);
    }
    load_dw<2 * VB>(vcodes + (int64_t)t0 * V.row_bytes + lane * 8 * VB, vlane);
    float vs[2][4][NGV], vz[2][4][NGV];
    load_token_params<VQ8, NGV>(V.params, prow + t0, q4, valid, vs, vz);

    // ---------------- scores: QK^T ----------------
    float sc[2][4];
    if constexpr (KCH) {
      if (tail_blk) {
        // unquantized tail: A = fp16 keys, B = q (exact in fp16), natural order
        const uint16_t* tail = K.tail + ((int64_t)bh * Gk + (t0 - n_full)) * kD;
        half8 bt[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          uint32_t o[4];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            o[r] = split16(lo_lane ? 0.f : qv[m][2 * r], false) |
                   (split16(lo_lane ? 0.f : qv[m][2 * r + 1], false) << 16);
          bt[m] = as_h8(o[0], o[1], o[2], o[3]);
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          f32x4 c = {0.f, 0.f, 0.f, 0.f};
          const int tt = 16 * mb + n;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(tail + (int64_t)tt * kD + 32 * m + 8 * q4);
            c = mfma16(__builtin_bit_cast(half8, v), bt[m], c);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[mb][r] = c[r];
        }
      } else {
        const int grp = t0 / Gk;
        if (grp != cur_group) {
          cur_group = grp;
          // scale/zero of this lane's 32 channels for key group ``grp``
          const uint32_t* prm = static_cast<const uint32_t*>(K.params) +
                                ((int64_t)bh * (Tcap / Gk) + grp) * kD;
          float qs[4][8];
          float mx = 0.f, zb = 0.f;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const u32x4 p0 = *reinterpret_cast<const u32x4*>(prm + 32 * m + 8 * q4);
            const u32x4 p1 = *reinterpret_cast<const u32x4*>(prm + 32 * m + 8 * q4 + 4);
            const uint32_t pz[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float s = h2f((uint16_t)(pz[e] & 0xffff));
              const float z = h2f((uint16_t)(pz[e] >> 16));
              qs[m][e] = qv[m][e] * s;
              mx = fmaxf(mx, fabsf(qs[m][e]));
              zb += qv[m][e] * z;
            }
          }
          mx = wave_max(mx);
          int E = 14 - ceil_log2(mx);
          if (E > 100) E = 100;
          kscale = pow2i(24 - E > 126 ? 126 : 24 - E);
          const float s2 = pow2i(E);
#pragma unroll
          for (int m = 0; m < 4; ++m) bk[m] = pair_operand<KB>(qs[m], s2, lo_lane);
          kbias = lo_lane ? 0.f : rows_sum(zb);
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int m = 0; m < 4; ++m) c = mfma16(seg_block<KB, KQ8>(kseg[mb], m), bk[m], c);
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[mb][r] = c[r] * kscale + kbias;
        }
      }
    } else {
      // per-token keys: one accumulator per key group, then scale and zero
      float ks[2][4][NGK], kz[2][4][NGK];
      load_token_params<KQ8, NGK>(K.params, prow + t0, q4, valid, ks, kz);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int gi = 0; gi < NGK; ++gi) {
          f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int m = gi * 4 / NGK; m < (gi + 1) * 4 / NGK; ++m)
            c = mfma16(seg_block<KB, KQ8>(kseg[mb], m), bq[m], c);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float dot = (c[r] - (KQ8 ? qoff[gi] : 0.f)) * kq;
            acc[r] += ks[mb][r][gi] * dot + kz[mb][r][gi] * qsum[gi];
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[mb][r] = acc[r];
      }
    }

    // ---------------- online softmax ----------------
    float bmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float s = (sc[mb][r] + dpp_ror8(sc[mb][r])) * sm2;
        if (16 * mb + 4 * q4 + r >= valid) s = -INFINITY;
        sc[mb][r] = s;
        bmax = fmaxf(bmax, s);
      }
    bmax = rows_max(bmax);
    const float m_new = fmaxf(m_run, bmax);
    if (__any(m_new > m_run)) {
      // rescale when any head's maximum grew (wave-uniform branch)
      const float alpha = m_run == -INFINITY ? 0.f : exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int gi = 0; gi < NGV; ++gi) { vbias[gi] *= alpha; voff[gi] *= alpha; }
      // accumulator row r of this lane belongs to head (4 q4 + r) & 7
      float al[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        al[jj] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), jj));
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float f = (q4 & 1) ? al[4 + r] : al[r];
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) oacc[nb][r] *= f;
      }
      m_run = m_new;
    }
    float p[2][4];
    float lsum = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[mb][r] = exp2f(sc[mb][r] - m_run);
        lsum += p[mb][r];
      }
    l_run += lsum;

    // ---------------- P.V ----------------
    half8 pa[NGV];
#pragma unroll
    for (int gi = 0; gi < NGV; ++gi) {
      float x[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[r] = p[0][r] * vs[0][r][gi];
        x[r + 4] = p[1][r] * vs[1][r][gi];
        if constexpr (!VQ8) vbias[gi] += p[0][r] * vz[0][r][gi] + p[1][r] * vz[1][r][gi];
      }
      pa[gi] = pair_operand<VB>(x, pscale, lo_lane);
      if constexpr (VQ8) {
        float so = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) so += (float)pa[gi][e];
        voff[gi] += so;
      }
    }
#pragma unroll
    for (int nbk = 0; nbk < 8; ++nbk) {
      const uint32_t* seg = vlane + (nbk >> 2) * VB;
      oacc[nbk] = mfma16(pa[nbk * NGV / 8], seg_block<VB, VQ8>(seg, nbk & 3), oacc[nbk]);
    }
  }

  // ---- wave result -> LDS (true units) ------------------------------------------
  const float l_tot = rows_sum(l_run);
  // high + low rows: lanes q4 = 0, 1 hold the high parts of heads 4*q4 + r,
  // lanes q4 + 2 the low parts.
#pragma unroll
  for (int nbk = 0; nbk < 8; ++nbk)
#pragma unroll
    for (int r = 0; r < 4; ++r) oacc[nbk][r] += __shfl_xor(oacc[nbk][r], 32, 64);
  const float oscale = 0x1p24f * vscale;    // codes are fed as code * 2^-24
  if (q4 < 2) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int jj = 4 * q4 + r;
#pragma unroll
      for (int nbk = 0; nbk < 8; ++nbk) wo[wave][jj][16 * nbk + n] = oacc[nbk][r] * oscale;
    }
  }
  float vb_tot[NGV], vo_tot[NGV];
#pragma unroll
  for (int gi = 0; gi < NGV; ++gi) {
    vb_tot[gi] = rows_sum(vbias[gi]);
    vo_tot[gi] = rows_sum(voff[gi]);
    vo_tot[gi] += dpp_ror8(vo_tot[gi]);   // rows (j, hi) + (j, lo)
  }
  if (q4 == 0 && n < 8) {
    wm[wave][j] = m_run;
    wl[wave][j] = l_tot;
#pragma unroll
    for (int gi = 0; gi < NGV; ++gi)
      wb[wave][j][gi] = VQ8 ? -128.0f * vo_tot[gi] * vscale : vb_tot[gi];
  }
  __syncthreads();

  // ---- merge the four waves and write this block's partials ------------------------
  for (int idx = threadIdx.x; idx < g * kD; idx += blockDim.x) {
    const int jj = idx / kD, c = idx % kD;
    const int gi = c * NGV / kD;
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][jj]);
    float O = 0.f, L = 0.f;
    if (M > -INFINITY) {
      for (int w = 0; w < 4; ++w) {
        const float wt = wm[w][jj] == -INFINITY ? 0.f : exp2f(wm[w][jj] - M);
        O += wt * (wo[w][jj][c] + wb[w][jj][gi]);
        L += wt * wl[w][jj];
      }
    }
    float* rec = partial_rec(a, b, h * g + jj, split);
    rec[c] = O;
    if (c == 0) { rec[kD] = M; rec[kD + 1] = L; }
  }
  splitk_finish(a, b, h, &flag);
}

// ---- dispatch ---------------------------------------------------------------------
template <int KB, bool KCH, bool KQ8, int NGK, int VB, bool VQ8, int NGV>
void launch_t(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((dec_mfma_kernel<KB, KCH, KQ8, NGK, VB, VQ8, NGV>),
                     dim3(a.splits, a.sh.B * a.sh.Hkv), dim3(256), 0, s, a);
}

template <int KB, bool KCH, bool KQ8, int NGK, int NGV>
bool launch_vb(const DecodeArgs& a, hipStream_t s) {
  if (a.v.quant == KVQ_QUANT_SYM_Q8_0) { launch_t<KB, KCH, KQ8, NGK, 8, true, NGV>(a, s); return true; }
  switch (a.v.bits) {
    case 3: launch_t<KB, KCH, KQ8, NGK, 3, false, NGV>(a, s); return true;
    case 4: launch_t<KB, KCH, KQ8, NGK, 4, false, NGV>(a, s); return true;
    case 8: launch_t<KB, KCH, KQ8, NGK, 8, false, NGV>(a, s); return true;
  }
  return false;
}

// per-channel keys: any value grouping
template <int KB>
bool launch_kch(const DecodeArgs& a, hipStream_t s) {
  switch (a.v.ng) {
    case 1: return launch_vb<KB, true, false, 1, 1>(a, s);
    case 2: return launch_vb<KB, true, false, 1, 2>(a, s);
    case 4: return launch_vb<KB, true, false, 1, 4>(a, s);
  }
  return false;
}

// per-token keys: the same group size for keys and values
template <int KB, bool KQ8>
bool launch_ktok(const DecodeArgs& a, hipStream_t s) {
  if (a.k.ng != a.v.ng) return false;
  switch (a.k.ng) {
    case 1: return launch_vb<KB, false, KQ8, 1, 1>(a, s);
    case 2: return launch_vb<KB, false, KQ8, 2, 2>(a, s);
    case 4: return launch_vb<KB, false, KQ8, 4, 4>(a, s);
  }
  return false;
}

bool uniform(const kvq_tensor_format& f) {
  return f.quantizer == KVQ_QUANT_ASYM_MINMAX || f.quantizer == KVQ_QUANT_ASYM_ABSMAX_OFFSET ||
         f.quantizer == KVQ_QUANT_SYM_Q8_0;
}

}  // namespace

bool mfma_config_supported(const kvq_config& c) {
  if (!uniform(c.k) || !uniform(c.v) || c.rope) return false;
  if (c.n_q_heads / c.n_kv_heads > 8) return false;
  if (c.k.layout == KVQ_LAYOUT_PER_CHANNEL) return c.kv_dtype == KVQ_F16;
  return c.k.group_size == c.v.group_size;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t s) {
  bool ok = false;
  if (a.k.per_channel) {
    switch (a.k.bits) {
      case 3: ok = launch_kch<3>(a, s); break;
      case 4: ok = launch_kch<4>(a, s); break;
      case 8: ok = launch_kch<8>(a, s); break;
    }
  } else if (a.k.quant == KVQ_QUANT_SYM_Q8_0) {
    ok = launch_ktok<8, true>(a, s);
  } else {
    switch (a.k.bits) {
      case 3: ok = launch_ktok<3, false>(a, s); break;
      case 4: ok = launch_ktok<4, false>(a, s); break;
      case 8: ok = launch_ktok<8, false>(a, s); break;
    }
  }
  if (!ok) return hipErrorNotSupported;
  return hipGetLastError();
}

}  // namespace kvq
