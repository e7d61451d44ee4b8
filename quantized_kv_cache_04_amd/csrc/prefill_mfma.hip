// Chunked-prefill attention of libkvq: causal attention of the last n_q
// tokens of every sequence over the whole cache, on the gfx950 matrix cores.
//
// Prefill scores many queries against the same keys, so unlike decode it is
// a dense contraction: QK^T and P.V of a tile of query rows run as
// v_mfma_f32_16x16x32_f16 products with the scores, the online softmax and
// the value sums kept on chip (Survey page, sections 2.3 and 5.3: prefill
// latency is its QK^T, done on chip; NIAH page, section 4.2).  The cache is
// read in its quantized form and dequantized into LDS once per 32-token
// block for the whole tile (KVQuant page, section 3.4: dequantize where the
// product needs it).
//
// Workgroup: one (sequence, KV head) and 64 query rows, a row being one
// (query token, query head of the group): 64 / g consecutive query tokens
// times the g heads.  Four waves own 16 rows each.  Per block of 32 tokens:
//  * all 256 threads dequantize the block's keys and values (outliers
//    replacing their dense values, keys rotated at their own positions) and
//    store them in LDS as fp16 high and low parts (x ~ hi + lo to about
//    2^-22 relative);
//  * QK^T: A = keys (16 tokens x 32 channels), B = the query rows (fp16 high
//    and low parts of q * scale, rotated to the query position), three
//    products per pair (hi.hi + lo.hi + hi.lo);
//  * the score lane layout (row n = lane & 15, tokens 8 (lane >> 4) + j) is
//    the B operand of P.V as it stands: O^T (16 channels x 16 rows) +=
//    V^T (16 channels x 32 tokens) . P (32 tokens x 16 rows), again three
//    products, so each lane's output channels belong to its own row and the
//    softmax rescale needs no data movement.
// Keys are stored before the rotary embedding (KVQuant page, sections
// 2.1-2.2): a key is rotated at its position t, a query at p, and
// R(p) q . R(t) k = q . R(t - p) k.  Attention-sink tokens come from the raw
// sink region, the rest from the quantized cache (positions stay absolute).
#include <hip/hip_runtime.h>

#include "device_common.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = kHeadDim;
constexpr int kRows = 64;      // query rows per workgroup
constexpr int kBlk = 32;       // tokens per staged block
constexpr float kLog2e = 1.4426950408889634f;

// LDS: the block's keys in fp32 before RoPE ([token][channel]), then keys
// [token][channel] and values [channel][token] as fp16 high and low planes.
// 16-byte chunks of the planes are XOR-swizzled so that the operand reads of
// one instruction hit every bank once:
//  * key row r, chunk u (channels 8u..8u+7) sits at chunk u ^ kswz(r);
//  * value row c, chunk u (tokens 8u..8u+7) sits at chunk u ^ ((c >> 2) & 3).
struct PreLds {
  float kf[kBlk][kD + 4];                          // 16.5 KB
  uint4 khi[kBlk][kD / 8], klo[kBlk][kD / 8];     // 2 x 8 KB
  uint4 vhi[kD][kBlk / 8], vlo[kD][kBlk / 8];     // 2 x 8 KB
  uint16_t cbk[kD][16], cbv[kD][16];               // codebooks of the KV head
  double theta[kD / 2];
};

__device__ __forceinline__ int kswz(int r) { return (r & 3) | (((r >> 3) & 3) << 2); }

__device__ __forceinline__ f32x4 mfma16(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void split8(const float x[8], uint4& hi, uint4& lo) {
  half8 h, l;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = (_Float16)x[e];
    l[e] = (_Float16)(x[e] - (float)h[e]);
  }
  hi = __builtin_bit_cast(uint4, h);
  lo = __builtin_bit_cast(uint4, l);
}

__device__ __forceinline__ half8 as_h8(uint4 v) { return __builtin_bit_cast(half8, v); }

__device__ __forceinline__ void rope_cs(double theta, int64_t pos, float& cs, float& sn) {
  const double ang = (double)pos * theta;
  const double two_pi = 6.283185307179586476925286766559;
  sincosf((float)(ang - two_pi * rint(ang / two_pi)), &sn, &cs);
}

__device__ __forceinline__ void load8(const uint16_t* p, int bf16, float x[8]) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = elem2f((uint16_t)(w[e >> 1] >> (16 * (e & 1))), bf16);
}

// The 8 codes of block m (codes 8 m .. 8 m + 7) of the 32-code segment at p,
// in the packing of include/kvq.h: bytes (8-bit), nibbles (4-bit) or, for 3
// bits, the two low bits of pair (8m + r, 8m + r + 4) at bits 2p and
// 16 + 2p of D[m / 2] (p = 4 (m % 2) + r) and the high bits at bits P and
// 16 + P of D2 (P = 8 (m / 2) + 2r + m % 2).  Only the dwords holding block m
// are read.
template <int BITS>
__device__ __forceinline__ void block_codes(const uint8_t* p, int m, uint32_t c[8]) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(p);
  if (BITS == 8) {
    const uint2 v = reinterpret_cast<const uint2*>(p)[m];
#pragma unroll
    for (int e = 0; e < 8; ++e) c[e] = ((e < 4 ? v.x : v.y) >> (8 * (e & 3))) & 255u;
  } else if (BITS == 4) {
    const uint32_t v = w[m];
#pragma unroll
    for (int e = 0; e < 8; ++e) c[e] = (v >> (4 * e)) & 15u;
  } else {
    const uint32_t lo = w[m >> 1] >> (8 * (m & 1)), hi = w[2] >> (8 * (m >> 1) + (m & 1));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = 2 * (e & 3) + 16 * (e >> 2);
      c[e] = ((lo >> sh) & 3u) | (((hi >> sh) & 1u) << 2);
    }
  }
}

__device__ __forceinline__ int h_of(int bh, const DevShape& sh) { return bh % sh.Hkv; }

__device__ __forceinline__ float uniform_x(uint32_t code, uint32_t pz) {
  return fmaf((float)code, h2f((uint16_t)(pz & 0xffff)), h2f((uint16_t)(pz >> 16)));
}

// Keys of quantized token tq: channels 32 m + 8 sq + e of blocks m = 2 hm and
// 2 hm + 1 (one 32-code segment of the key row), dense values in fp32.
template <int BITS>
__device__ __forceinline__ void key_codes(const DevTensor& k, const DevShape& sh, const PreLds& S,
                                          int bh, int64_t tq, int sq, int hm, float x[2][8]) {
  const uint8_t* seg = k.codes + ((int64_t)bh * sh.Tcap + tq) * k.row_bytes + sq * 4 * BITS;
#pragma unroll
  for (int mm = 0; mm < 2; ++mm) {
    const int m = 2 * hm + mm, c0 = 32 * m + 8 * sq;
    uint32_t cd[8];
    block_codes<BITS>(seg, m, cd);
    if (k.quant == KVQ_QUANT_CODEBOOK) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[mm][e] = h2f(S.cbk[c0 + e][cd[e]]);
    } else if (k.quant == KVQ_QUANT_FP8_E5M2) {
      const float sc = fp8_scale(k, h_of(bh, sh));
#pragma unroll
      for (int e = 0; e < 8; ++e) x[mm][e] = e5m2_to_f(cd[e]) * sc;
    } else if (k.per_channel) {
      const uint4* pp = reinterpret_cast<const uint4*>(
          static_cast<const uint32_t*>(k.params) +
          ((int64_t)bh * (sh.Tcap / k.G) + tq / k.G) * kHeadDim + c0);
      const uint4 p0 = pp[0], p1 = pp[1];
      const uint32_t pz[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) x[mm][e] = uniform_x(cd[e], pz[e]);
    } else if (k.quant == KVQ_QUANT_SYM_Q8_0) {
      const float sc = h2f(static_cast<const uint16_t*>(k.params)[((int64_t)bh * sh.Tcap + tq) * k.ng + c0 / k.G]);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[mm][e] = (float)(int8_t)cd[e] * sc;
    } else {
      const uint32_t pz = static_cast<const uint32_t*>(k.params)[((int64_t)bh * sh.Tcap + tq) * k.ng + c0 / k.G];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[mm][e] = uniform_x(cd[e], pz);
    }
  }
}

// Values of channel c for tokens 16 hv + u (u < 16) of the 32-token value
// tile that starts at quantized token tq0; tokens at or past n_valid are 0.
// Token 4q + r (+16 hv) of channel c is code 8m + r + 4hv of segment c / 64
// of tile lane 16q + c % 16 (m = (c / 16) % 4).
template <int BITS>
__device__ __forceinline__ void value_codes(const DevTensor& v, const DevShape& sh, int bh,
                                            int64_t tq0, int c, int hv, int n_valid, float x[16]) {
  const uint8_t* tile = v.codes + ((int64_t)bh * sh.Tcap + tq0) * v.row_bytes;
  const int i = c & 15, sg = c >> 6, m = (c >> 4) & 3;
  uint32_t cd[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t blk[8];
    block_codes<BITS>(tile + (16 * q + i) * 8 * BITS + sg * 4 * BITS, m, blk);
#pragma unroll
    for (int r = 0; r < 4; ++r) cd[4 * q + r] = hv ? blk[4 + r] : blk[r];
  }
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int tk = 16 * hv + u;
    float y;
    if (v.quant == KVQ_QUANT_FP8_E5M2) {
      y = e5m2_to_f(cd[u]) * fp8_scale(v, h_of(bh, sh));
    } else {
      const int64_t rec = ((int64_t)bh * sh.Tcap + tq0 + tk) * v.ng + c / v.G;
      if (v.quant == KVQ_QUANT_SYM_Q8_0)
        y = (float)(int8_t)cd[u] * h2f(static_cast<const uint16_t*>(v.params)[rec]);
      else
        y = uniform_x(cd[u], static_cast<const uint32_t*>(v.params)[rec]);
    }
    x[u] = tk < n_valid ? y : 0.f;
  }
}

// Outliers replace their dense value in the staged tile (quantized tokens
// tq0 + tk, tk < n_valid): entry e of the CSR row of token tk (all heads of
// the token) per thread; entries of other heads are skipped.  Keys go to the
// fp32 stage (RoPE follows), values to the fp16 planes.
template <bool KEY>
__device__ __forceinline__ void stage_outliers(const DevTensor& ten, PreLds& S, int tid, int b,
                                               int h, int64_t tq0, int n_valid, int64_t Tcap) {
  const int ko = ten.k_out;
  for (int idx = tid; idx < n_valid * ko; idx += 256) {
    const int tk = idx / ko;
    const int64_t rr = (int64_t)b * Tcap + tq0 + tk;
    const int e = ten.row_ptr[rr] + idx % ko;
    if (e >= ten.row_ptr[rr + 1]) continue;
    const int cc = (ten.col[e] & 0xfff) - h * kD;
    if (cc < 0 || cc >= kD) continue;
    const float v = h2f(ten.val[e]);
    if (KEY) {
      S.kf[tk][cc] = v;
    } else {
      const _Float16 xh = (_Float16)v;
      const int at = 8 * ((tk >> 3) ^ ((cc >> 2) & 3)) + (tk & 7);
      reinterpret_cast<_Float16*>(&S.vhi[cc][0])[at] = xh;
      reinterpret_cast<_Float16*>(&S.vlo[cc][0])[at] = (_Float16)(v - (float)xh);
    }
  }
}

__global__ __launch_bounds__(256, 2) void pre_mfma_kernel(PrefillArgs a) {
  __shared__ PreLds S;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, q4 = lane >> 4;
  const int bh = blockIdx.y, b = bh / a.sh.Hkv, h = bh % a.sh.Hkv;
  const int g = a.sh.g, qt = kRows / g;
  // longest tiles (latest queries) first
  const int tile = gridDim.x - 1 - blockIdx.x;
  const int base = a.n_total - a.n_q;                 // position of query 0
  const int i_last = min(a.n_q - 1, tile * qt + qt - 1);
  const int p_max = base + i_last;                     // last position the tile sees
  const int n_qc = a.n_total - a.n_sink;               // quantized tokens
  const int64_t n_full = a.k.per_channel ? (int64_t)(n_qc / a.k.G) * a.k.G : n_qc;
  if (a.rope && tid < kD / 2) S.theta[tid] = pow((double)a.rope_base, -2.0 * tid / (double)kD);
  if (a.k.quant == KVQ_QUANT_CODEBOOK)
    for (int idx = tid; idx < kD * 16; idx += 256)
      S.cbk[idx >> 4][idx & 15] = a.k.codebook[(int64_t)h * kD * 16 + idx];
  if (a.v.quant == KVQ_QUANT_CODEBOOK)
    for (int idx = tid; idx < kD * 16; idx += 256)
      S.cbv[idx >> 4][idx & 15] = a.v.codebook[(int64_t)h * kD * 16 + idx];
  __syncthreads();

  // ---- this lane's query row ------------------------------------------------
  const int r = 16 * wave + n;
  const int qi = tile * qt + r / g, jh = h * g + r % g;
  const bool row_ok = qi < a.n_q;
  const int p_row = row_ok ? base + qi : -1;
  const int wave_first = tile * qt + (16 * wave) / g;  // first query token of the wave
  const int p_wave = min(base + tile * qt + (16 * wave + 15) / g, p_max);
  const bool wave_ok = wave_first < a.n_q;
  half8 qh[4], ql[4];
  {
    float x[4][8];
    if (row_ok) {
      const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                           (((int64_t)b * a.n_q + qi) * a.sh.Hq + jh) * kD;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) load8(qp + 32 * ks + 8 * q4, a.sh.kv_bf16, x[ks]);
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[ks][e] = 0.f;
    }
    if (a.rope && row_ok) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float cs, sn;
          rope_cs(S.theta[32 * ks + 8 * q4 + e], p_row, cs, sn);
          const float x0 = x[ks][e], x1 = x[ks + 2][e];
          x[ks][e] = x0 * cs - x1 * sn;
          x[ks + 2][e] = x1 * cs + x0 * sn;
        }
    }
    const float sc = a.sm_scale * kLog2e;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[ks][e] *= sc;
      uint4 hi, lo;
      split8(x[ks], hi, lo);
      qh[ks] = as_h8(hi);
      ql[ks] = as_h8(lo);
    }
  }

  f32x4 o[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) o[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // Blocks: the attention sink in 32-token blocks, then the quantized cache
  // in its own 32-token tiles (so that value tiles and per-channel key
  // groups stay aligned); positions stay absolute.
  const int n_sb = (a.n_sink + kBlk - 1) / kBlk;
  const int n_qb = p_max >= a.n_sink ? (p_max - a.n_sink) / kBlk + 1 : 0;
  const int64_t sink_row0 = (int64_t)bh * a.sink_cap;
  for (int blk = 0; blk < n_sb + n_qb; ++blk) {
    const bool sinkb = blk < n_sb;
    const int t0 = sinkb ? blk * kBlk : a.n_sink + (blk - n_sb) * kBlk;   // position of token 0
    const int64_t tq0 = sinkb ? 0 : (int64_t)(blk - n_sb) * kBlk;         // quantized index of token 0
    // tokens t0 + tk with tk < n_valid are in this block and visible to the tile
    const int n_valid = min(kBlk, (sinkb ? min(a.n_sink, p_max + 1) : p_max + 1) - t0);
    __syncthreads();   // the previous block's operand reads are done
    // ---- phase 1: dense keys to fp32 (token tk, channels 32 m + 8 sq + e of
    // blocks m = 2 hm, 2 hm + 1) and values to fp16 planes (channel c,
    // tokens 16 hv .. 16 hv + 15) --------------------------------------------
    {
      const int tk = tid >> 3, sq = (tid & 7) >> 1, hm = tid & 1;
      float x[2][8];
      const int64_t tq = tq0 + tk;
      if (tk >= n_valid) {
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
#pragma unroll
          for (int e = 0; e < 8; ++e) x[mm][e] = 0.f;
      } else if (sinkb || a.k.quant == KVQ_QUANT_NONE ||
                 (a.k.per_channel && tq >= n_full)) {
        // raw rows: the sink, a raw cache, or the per-channel tail
        const uint16_t* row =
            sinkb ? a.k_sink + (sink_row0 + t0 + tk) * kD
            : a.k.quant == KVQ_QUANT_NONE
                ? reinterpret_cast<const uint16_t*>(a.k.codes) + ((int64_t)bh * a.sh.Tcap + tq) * kD
                : a.k.tail + ((int64_t)bh * a.k.G + (tq - n_full)) * kD;
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) load8(row + 32 * (2 * hm + mm) + 8 * sq, a.sh.kv_bf16, x[mm]);
      } else if (a.k.bits == 4) {
        key_codes<4>(a.k, a.sh, S, bh, tq, sq, hm, x);
      } else if (a.k.bits == 3) {
        key_codes<3>(a.k, a.sh, S, bh, tq, sq, hm, x);
      } else {
        key_codes<8>(a.k, a.sh, S, bh, tq, sq, hm, x);
      }
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        float4* dst = reinterpret_cast<float4*>(&S.kf[tk][32 * (2 * hm + mm) + 8 * sq]);
        dst[0] = float4{x[mm][0], x[mm][1], x[mm][2], x[mm][3]};
        dst[1] = float4{x[mm][4], x[mm][5], x[mm][6], x[mm][7]};
      }
    }
    {
      const int c = tid >> 1, hv = tid & 1;
      float x[16];
      if (sinkb || a.v.quant == KVQ_QUANT_NONE) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int tk = 16 * hv + u;
          const uint16_t* row =
              sinkb ? a.v_sink + (sink_row0 + t0 + tk) * kD
                    : reinterpret_cast<const uint16_t*>(a.v.codes) + ((int64_t)bh * a.sh.Tcap + tq0 + tk) * kD;
          x[u] = tk < n_valid ? elem2f(row[c], a.sh.kv_bf16) : 0.f;
        }
      } else if (a.v.quant == KVQ_QUANT_CODEBOOK) {
        // pair tiles: byte 32 l + tau holds channels l (low nibble) and l + 64
        const uint4 w = *reinterpret_cast<const uint4*>(
            a.v.codes + ((int64_t)bh * a.sh.Tcap + tq0) * a.v.row_bytes + 32 * (c & 63) + 16 * hv);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const uint32_t code = (ww[u >> 2] >> (8 * (u & 3) + 4 * (c >> 6))) & 15u;
          x[u] = 16 * hv + u < n_valid ? h2f(S.cbv[c][code]) : 0.f;
        }
      } else if (a.v.bits == 4) {
        value_codes<4>(a.v, a.sh, bh, tq0, c, hv, n_valid, x);
      } else if (a.v.bits == 3) {
        value_codes<3>(a.v, a.sh, bh, tq0, c, hv, n_valid, x);
      } else {
        value_codes<8>(a.v, a.sh, bh, tq0, c, hv, n_valid, x);
      }
      const int sw = (c >> 2) & 3;
      uint4 hi, lo;
      split8(x, hi, lo);
      S.vhi[c][(2 * hv) ^ sw] = hi;
      S.vlo[c][(2 * hv) ^ sw] = lo;
      split8(x + 8, hi, lo);
      S.vhi[c][(2 * hv + 1) ^ sw] = hi;
      S.vlo[c][(2 * hv + 1) ^ sw] = lo;
    }
    // ---- phase 2: outliers replace their dense value -------------------------
    if (!sinkb && (a.k.k_out > 0 || a.v.k_out > 0)) {
      __syncthreads();
      if (a.k.k_out > 0) stage_outliers<true>(a.k, S, tid, b, h, tq0, n_valid, a.sh.Tcap);
      if (a.v.k_out > 0) stage_outliers<false>(a.v, S, tid, b, h, tq0, n_valid, a.sh.Tcap);
    }
    __syncthreads();
    // ---- phase 3: RoPE at the key's position, then fp16 planes (token tk,
    // channel pairs (i, i + 64) for i = 8 pb .. 8 pb + 7) ----------------------
    {
      const int tk = tid >> 3, pb = tid & 7, t = t0 + tk;
      float x0[8], x1[8];
      const float4* r0 = reinterpret_cast<const float4*>(&S.kf[tk][8 * pb]);
      const float4* r1 = reinterpret_cast<const float4*>(&S.kf[tk][64 + 8 * pb]);
      const float4 a0 = r0[0], a1 = r0[1], b0 = r1[0], b1 = r1[1];
      x0[0] = a0.x; x0[1] = a0.y; x0[2] = a0.z; x0[3] = a0.w;
      x0[4] = a1.x; x0[5] = a1.y; x0[6] = a1.z; x0[7] = a1.w;
      x1[0] = b0.x; x1[1] = b0.y; x1[2] = b0.z; x1[3] = b0.w;
      x1[4] = b1.x; x1[5] = b1.y; x1[6] = b1.z; x1[7] = b1.w;
      if (a.rope && tk < n_valid) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float cs, sn;
          rope_cs(S.theta[8 * pb + e], t, cs, sn);
          const float y0 = x0[e], y1 = x1[e];
          x0[e] = y0 * cs - y1 * sn;
          x1[e] = y1 * cs + y0 * sn;
        }
      }
      uint4 hi, lo;
      const int sw = kswz(tk);
      split8(x0, hi, lo);
      S.khi[tk][pb ^ sw] = hi;
      S.klo[tk][pb ^ sw] = lo;
      split8(x1, hi, lo);
      S.khi[tk][(pb + 8) ^ sw] = hi;
      S.klo[tk][(pb + 8) ^ sw] = lo;
    }
    __syncthreads();
    if (!wave_ok || t0 > p_wave) continue;   // nothing of this block is visible to the wave

    // ---- scores: tokens 8 q4 + 4T + i for T = 0, 1 --------------------------
    f32x4 acc[2];
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      acc[T] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int tok = 8 * (n >> 2) + 4 * T + (n & 3);
      const int sw = kswz(tok);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int ch = (4 * ks + q4) ^ sw;
        const half8 khi = as_h8(S.khi[tok][ch]), klo = as_h8(S.klo[tok][ch]);
        acc[T] = mfma16(khi, qh[ks], acc[T]);
        acc[T] = mfma16(klo, qh[ks], acc[T]);
        acc[T] = mfma16(khi, ql[ks], acc[T]);
      }
    }
    float s[8];
    float mloc = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tk = 8 * q4 + j;
      s[j] = tk < n_valid && t0 + tk <= p_row ? acc[j >> 2][j & 3] : -INFINITY;
      mloc = fmaxf(mloc, s[j]);
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float m_new = fmaxf(m_run, mloc);
    float pr[8];
    float alpha = 1.f;
    if (m_new == -INFINITY) {
#pragma unroll
      for (int j = 0; j < 8; ++j) pr[j] = 0.f;
    } else {
      alpha = exp2f(m_run - m_new);
#pragma unroll
      for (int j = 0; j < 8; ++j) pr[j] = exp2f(s[j] - m_new);
      m_run = m_new;
    }
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) psum += pr[j];
    l_run = l_run * alpha + psum;
    uint4 phi_u, plo_u;
    split8(pr, phi_u, plo_u);
    const half8 phi = as_h8(phi_u), plo = as_h8(plo_u);
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      o[ct] *= alpha;
      const int c = 16 * ct + n;
      const int ch = q4 ^ ((c >> 2) & 3);
      const half8 vhi = as_h8(S.vhi[c][ch]), vlo = as_h8(S.vlo[c][ch]);
      o[ct] = mfma16(vhi, phi, o[ct]);
      o[ct] = mfma16(vlo, phi, o[ct]);
      o[ct] = mfma16(vhi, plo, o[ct]);
    }
  }

  // ---- normalize and store: lane holds channels 16 ct + 4 q4 + i of row n ----
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (!row_ok) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int64_t orow = (((int64_t)b * a.n_q + qi) * a.sh.Hq + jh) * kD;
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = o[ct][i] * inv;
      const int64_t idx = orow + 16 * ct + 4 * q4 + i;
      if (a.out_dtype == KVQ_F32)
        static_cast<float*>(a.out)[idx] = v;
      else if (a.out_dtype == KVQ_F16)
        static_cast<uint16_t*>(a.out)[idx] = f2h_rn(v);
      else
        static_cast<uint16_t*>(a.out)[idx] = f2bf_rn(v);
    }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const int g = a.sh.g;
  if (g < 1 || kRows % g != 0 || a.n_q < 1 || a.n_q > a.n_total) return hipErrorInvalidValue;
  const int qt = kRows / g;
  const int tiles = (a.n_q + qt - 1) / qt;
  hipLaunchKernelGGL(pre_mfma_kernel, dim3((unsigned)tiles, (unsigned)(a.sh.B * a.sh.Hkv)),
                     dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
