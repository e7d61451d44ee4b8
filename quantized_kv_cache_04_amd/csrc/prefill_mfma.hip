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
  // RoPE of keys by angle addition: rt[tk][i] = (cos, sin) of tk * theta_i
  // for the 32 offsets of a block, rb[parity][i] = (cos, sin) of t0 * theta_i
  // for the block's first position (double-buffered by block parity)
  float2 rt[kBlk][kD / 2];
  float2 rb[2][kD / 2];
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

// rotation by the sum of two angles given as (cos, sin) pairs
__device__ __forceinline__ void rot_add(float2 a, float2 b, float& cs, float& sn) {
  cs = a.x * b.x - a.y * b.y;
  sn = a.y * b.x + a.x * b.y;
}

__device__ __forceinline__ void load8(const uint16_t* p, int bf16, float x[8]) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = elem2f((uint16_t)(w[e >> 1] >> (16 * (e & 1))), bf16);
}

// Cache formats the kernel is specialized for (F_ANY: read from the tensor
// at run time).  The two asymmetric quantizers dequantize alike (c * s + z).
enum : int { F_ANY = 0, F_PC4 = 1, F_U4 = 2, F_U3 = 3, F_Q8 = 4, F_CB = 5, F_F8 = 6 };
template <int F>
__device__ __forceinline__ int fmt_kind(const DevTensor& t) {
  if constexpr (F == F_ANY)
    return t.quant == KVQ_QUANT_ASYM_ABSMAX_OFFSET ? KVQ_QUANT_ASYM_MINMAX : t.quant;
  else if constexpr (F == F_Q8) return KVQ_QUANT_SYM_Q8_0;
  else if constexpr (F == F_CB) return KVQ_QUANT_CODEBOOK;
  else if constexpr (F == F_F8) return KVQ_QUANT_FP8_E5M2;
  else return KVQ_QUANT_ASYM_MINMAX;
}
template <int F>
__device__ __forceinline__ int fmt_bits(const DevTensor& t) {
  if constexpr (F == F_ANY) return t.bits;
  else if constexpr (F == F_U3) return 3;
  else if constexpr (F == F_Q8 || F == F_F8) return 8;
  else return 4;
}
template <int F>
__device__ __forceinline__ bool fmt_pc(const DevTensor& t) {
  if constexpr (F == F_ANY) return t.per_channel != 0;
  else return F == F_PC4;
}

__device__ __forceinline__ float uniform_x(uint32_t code, uint32_t pz) {
  return fmaf((float)code, h2f((uint16_t)(pz & 0xffff)), h2f((uint16_t)(pz >> 16)));
}

// The 8 codes of block m (codes 8 m .. 8 m + 7) of a 32-code segment, in the
// packing of include/kvq.h, from the dwords that hold the block: 8-bit: two
// dwords (bytes 8m .. 8m + 7); 4-bit: dword m (nibbles); 3-bit: lo = D[m/2]
// and hi = D2, the two low bits of pair (8m + r, 8m + r + 4) sitting at bits
// 2p and 16 + 2p of lo (p = 4 (m % 2) + r) and the high bits at bits P and
// 16 + P of hi (P = 8 (m / 2) + 2r + m % 2).
template <int BITS>
__device__ __forceinline__ void block_codes(uint32_t w0, uint32_t w1, int m, uint32_t c[8]) {
  if (BITS == 8) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c[e] = ((e < 4 ? w0 : w1) >> (8 * (e & 3))) & 255u;
  } else if (BITS == 4) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c[e] = (w0 >> (4 * e)) & 15u;
  } else {
    const uint32_t lo = w0 >> (8 * (m & 1)), hi = w1 >> (8 * (m >> 1) + (m & 1));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = 2 * (e & 3) + 16 * (e >> 2);
      c[e] = ((lo >> sh) & 3u) | (((hi >> sh) & 1u) << 2);
    }
  }
}

// Raw words of one 32-token block for one thread, fetched a block ahead so
// that their loads run under the previous block's matrix-core work.
//  keys (token tk, the 8-channel runs c0 = 32 mp + 8 sq and c0 + 64):
//    kc: the code dwords (4-bit: runs' dwords; 8-bit: two each; 3-bit: the
//        segment's D0, D1, D2), kq: per-channel (scale, zero) pairs of both
//        runs, or the raw rows of the sink / a raw cache / the per-channel
//        tail (kq[0], kq[1]), kpz: per-token parameters of both runs;
//  values (channel c, tokens 16 hv + u): vc: the code dwords of block m of
//    the four tile lanes 16q + c % 16 (two each for 8 and 3 bits; codebook
//    pair tiles: 16 bytes), vp: the per-token parameters, or raw elements.
struct Raw {
  uint32_t kc[4];
  uint4 kq[4];
  uint32_t kpz[2];
  uint32_t vc[8];
  uint32_t vp[16];
};

// fp32 keys of one 8-channel run (channels cr .. cr + 7; run 0 or 1 of the
// thread's two) from its codes
__device__ __forceinline__ void key_run(int kind, bool pc, const PreLds& S, const Raw& R,
                                        const uint32_t cd[8], int cr, int run, float h_scale,
                                        float x[8]) {
  if (kind == KVQ_QUANT_CODEBOOK) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = h2f(S.cbk[cr + e][cd[e]]);
  } else if (kind == KVQ_QUANT_FP8_E5M2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = e5m2_to_f(cd[e]) * h_scale;
  } else if (pc) {
    const uint4 p0 = run ? R.kq[2] : R.kq[0], p1 = run ? R.kq[3] : R.kq[1];
    const uint32_t pz[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = uniform_x(cd[e], pz[e]);
  } else if (kind == KVQ_QUANT_SYM_Q8_0) {
    const float sc = h2f((uint16_t)(run ? R.kpz[1] : R.kpz[0]));
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)(int8_t)cd[e] * sc;
  } else {
    const uint32_t pz = run ? R.kpz[1] : R.kpz[0];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = uniform_x(cd[e], pz);
  }
}

// fp32 keys of runs c0 and c0 + 64 of the token from its raw words
template <int BITS>
__device__ __forceinline__ void key_values(int kind, bool pc, const PreLds& S, const Raw& R,
                                           int mp, int sq, float h_scale, float x0[8], float x1[8]) {
  uint32_t cd[2][8];
  if (BITS == 3) {
    block_codes<3>(R.kc[0], R.kc[2], mp, cd[0]);
    block_codes<3>(R.kc[1], R.kc[2], mp + 2, cd[1]);
  } else if (BITS == 8) {
    block_codes<8>(R.kc[0], R.kc[1], mp, cd[0]);
    block_codes<8>(R.kc[2], R.kc[3], mp + 2, cd[1]);
  } else {
    block_codes<4>(R.kc[0], 0u, mp, cd[0]);
    block_codes<4>(R.kc[1], 0u, mp + 2, cd[1]);
  }
  const int c0 = 32 * mp + 8 * sq;
  key_run(kind, pc, S, R, cd[0], c0, 0, h_scale, x0);
  key_run(kind, pc, S, R, cd[1], c0 + 64, 1, h_scale, x1);
}

// fp32 values of channel c, tokens 16 hv + u, from the raw words
template <int BITS>
__device__ __forceinline__ void value_values(int kind, const Raw& R, int c, int hv,
                                             float h_scale, int n_valid, float x[16]) {
  const int m = (c >> 4) & 3;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t blk[8];
    if (BITS == 4)
      block_codes<4>(R.vc[q], 0u, m, blk);
    else
      block_codes<BITS>(R.vc[2 * q], R.vc[2 * q + 1], m, blk);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t code = hv ? blk[4 + r] : blk[r];
      const int u = 4 * q + r;
      float y;
      if (kind == KVQ_QUANT_FP8_E5M2)
        y = e5m2_to_f(code) * h_scale;
      else if (kind == KVQ_QUANT_SYM_Q8_0)
        y = (float)(int8_t)code * h2f((uint16_t)R.vp[u]);
      else
        y = uniform_x(code, R.vp[u]);
      x[u] = 16 * hv + u < n_valid ? y : 0.f;
    }
  }
}

// Outliers replace their dense value in the staged tile (quantized tokens
// tq0 + tk, tk < n_valid).  The tile's per-tile index lists the KV head's
// entries contiguously (off[h] .. off[h + 1] - 1 of the tile's block, one
// dword each: channel, token in the tile, the dense index replaced, fp16
// value), so one offset read and one load per entry find them, thread i
// taking entry i.  Keys go to the fp32 stage (RoPE follows), values to the
// fp16 planes.
template <bool KEY>
__device__ __forceinline__ void stage_outliers(const DevTensor& ten, PreLds& S, int tid, int b,
                                               int h, int64_t tq0, int n_valid, const DevShape& sh) {
  const int64_t tile = csr_row(sh, b, tq0) >> 5;   // the block is one tile (a page when paged)
  const int o_row = (sh.Hkv + 8) / 8 * 8;
  const uint16_t* off = ten.toff + tile * o_row;
  const int e0 = off[h], e1 = off[h + 1];
  const uint32_t* ent = ten.tent + tile * ((int64_t)kTile * ten.k_out);
  for (int i = e0 + tid; i < e1; i += 256) {
    const uint32_t en = ent[i];
    const int tk = (int)((en >> 7) & 31u), cc = (int)(en & (kD - 1));
    if (tk >= n_valid) continue;
    const float v = h2f((uint16_t)(en >> 16));
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

// KF, VF: key and value formats (F_ANY: any, read at run time).  The
// specialized kernels fetch a block's raw words one block ahead, under the
// previous block's products; the general one fetches them just in time.
template <int KF, int VF>
__global__ __launch_bounds__(256, 2) void pre_mfma_kernel(PrefillArgs a) {
  constexpr bool PIPE = KF != F_ANY && VF != F_ANY;
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
  if (a.rope) {
    __syncthreads();
    for (int idx = tid; idx < kBlk * (kD / 2); idx += 256) {
      S.rt[idx / (kD / 2)][idx % (kD / 2)] = rope_cs(S.theta[idx % (kD / 2)], idx / (kD / 2));
    }
  }
  if (fmt_kind<KF>(a.k) == KVQ_QUANT_CODEBOOK)
    for (int idx = tid; idx < kD * 16; idx += 256)
      S.cbk[idx >> 4][idx & 15] = a.k.codebook[(int64_t)h * kD * 16 + idx];
  if (fmt_kind<VF>(a.v) == KVQ_QUANT_CODEBOOK)
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
          const float2 r = rope_cs(S.theta[32 * ks + 8 * q4 + e], p_row);
          const float cs = r.x, sn = r.y;
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
  const int n_blk = n_sb + n_qb;
  const int64_t sink_row0 = (int64_t)bh * a.sink_cap;
  const int64_t Tcap = a.sh.Tcap;
  const int kkind = fmt_kind<KF>(a.k), vkind = fmt_kind<VF>(a.v);
  const int kbits = fmt_bits<KF>(a.k), vbits = fmt_bits<VF>(a.v);
  const bool kpc = fmt_pc<KF>(a.k);
  // group sizes and groups per token of this workgroup's head
  const int kG = head_view(a.k, h).G, vG = head_view(a.v, h).G, vng = head_view(a.v, h).ng;
  const bool kraw = kkind == KVQ_QUANT_NONE, vraw = vkind == KVQ_QUANT_NONE;
  const bool kstage = a.k.k_out > 0;   // keys go through the fp32 stage (outliers, then RoPE)
  const float ksc = fp8_scale(a.k, h), vsc = fp8_scale(a.v, h);
  // thread roles in staging: keys of token ktk, runs 32 kmp + 8 ksq (+64);
  // values of channel vch, tokens 16 vhv .. 16 vhv + 15
  const int ktk = tid >> 3, ksq = (tid >> 1) & 3, kmp = tid & 1;
  const int vch = tid >> 1, vhv = tid & 1;
  struct Desc { bool sinkb; int t0; int64_t tq0; int n_valid; };
  auto desc = [&](int blk) {
    Desc d;
    d.sinkb = blk < n_sb;
    d.t0 = d.sinkb ? blk * kBlk : a.n_sink + (blk - n_sb) * kBlk;   // position of token 0
    d.tq0 = d.sinkb ? 0 : (int64_t)(blk - n_sb) * kBlk;            // quantized index of token 0
    // tokens t0 + tk with tk < n_valid are in this block and visible to the tile
    d.n_valid = min(kBlk, (d.sinkb ? min(a.n_sink, p_max + 1) : p_max + 1) - d.t0);
    return d;
  };
  // issue the loads of block blk's raw words
  auto fetch = [&](int blk, Raw& R) {
    if (blk >= n_blk) return;
    const Desc d = desc(blk);
    // row of the quantized block's first token (its 32 tokens are
    // consecutive rows, one page of a paged cache)
    const int64_t qrow0 = d.sinkb ? 0 : tok_row(a.sh, b, h, d.tq0);
    if (ktk < d.n_valid) {
      const int64_t tq = d.tq0 + ktk;
      if (d.sinkb || kraw || (kpc && tq >= n_full)) {
        const uint16_t* row =
            d.sinkb ? a.k_sink + (sink_row0 + d.t0 + ktk) * kD
            : kraw  ? reinterpret_cast<const uint16_t*>(a.k.codes) + (qrow0 + ktk) * kD
                    : a.k.tail + ((int64_t)bh * a.k.tail_rows + tq % a.k.tail_rows) * kD;
        R.kq[0] = *reinterpret_cast<const uint4*>(row + 32 * kmp + 8 * ksq);
        R.kq[1] = *reinterpret_cast<const uint4*>(row + 64 + 32 * kmp + 8 * ksq);
      } else {
        const int bits = kbits;
        const uint8_t* seg = a.k.codes + (qrow0 + ktk) * a.k.row_bytes + ksq * 4 * bits;
        const uint32_t* w = reinterpret_cast<const uint32_t*>(seg);
        if (bits == 4) {
          R.kc[0] = w[kmp];
          R.kc[1] = w[kmp + 2];
        } else if (bits == 8) {
          const uint2 u0 = reinterpret_cast<const uint2*>(seg)[kmp];
          const uint2 u1 = reinterpret_cast<const uint2*>(seg)[kmp + 2];
          R.kc[0] = u0.x; R.kc[1] = u0.y; R.kc[2] = u1.x; R.kc[3] = u1.y;
        } else {
          R.kc[0] = w[0]; R.kc[1] = w[1]; R.kc[2] = w[2];
        }
        const int c0 = 32 * kmp + 8 * ksq;
        if (kpc) {
          const uint4* pp = reinterpret_cast<const uint4*>(
              static_cast<const uint32_t*>(a.k.params) + ((int64_t)bh * (Tcap / a.k.G) + tq / a.k.G) * kD + c0);
          R.kq[0] = pp[0]; R.kq[1] = pp[1]; R.kq[2] = pp[16]; R.kq[3] = pp[17];
        } else if (kkind == KVQ_QUANT_SYM_Q8_0) {
          const uint16_t* pp = static_cast<const uint16_t*>(a.k.params) + prm_rec(a.k, a.sh, b, h, tq);
          R.kpz[0] = pp[c0 / kG];
          R.kpz[1] = pp[(c0 + 64) / kG];
        } else if (kkind != KVQ_QUANT_CODEBOOK && kkind != KVQ_QUANT_FP8_E5M2) {
          const uint32_t* pp = static_cast<const uint32_t*>(a.k.params) + prm_rec(a.k, a.sh, b, h, tq);
          R.kpz[0] = pp[c0 / kG];
          R.kpz[1] = pp[(c0 + 64) / kG];
        }
      }
    }
    if (d.sinkb || vraw) {
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int tk = 16 * vhv + u;
        const uint16_t* row =
            d.sinkb ? a.v_sink + (sink_row0 + d.t0 + tk) * kD
                    : reinterpret_cast<const uint16_t*>(a.v.codes) + (qrow0 + tk) * kD;
        R.vp[u] = tk < d.n_valid ? row[vch] : 0u;
      }
    } else {
      const uint8_t* tile = a.v.codes + qrow0 * a.v.row_bytes;
      if (vkind == KVQ_QUANT_CODEBOOK) {
        // pair tiles: byte 32 l + tau holds channels l (low nibble) and l + 64
        const uint4 w = *reinterpret_cast<const uint4*>(tile + 32 * (vch & 63) + 16 * vhv);
        R.vc[0] = w.x; R.vc[1] = w.y; R.vc[2] = w.z; R.vc[3] = w.w;
      } else {
        const int bits = vbits, i = vch & 15, sg = vch >> 6, m = (vch >> 4) & 3;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint8_t* seg = tile + (16 * q + i) * 8 * bits + sg * 4 * bits;
          const uint32_t* w = reinterpret_cast<const uint32_t*>(seg);
          if (bits == 4) {
            R.vc[q] = w[m];
          } else if (bits == 8) {
            R.vc[2 * q] = w[2 * m];
            R.vc[2 * q + 1] = w[2 * m + 1];
          } else {
            R.vc[2 * q] = w[m >> 1];
            R.vc[2 * q + 1] = w[2];
          }
        }
        // the block's tokens are consecutive records of one (sequence, head)
        if (vkind == KVQ_QUANT_SYM_Q8_0) {
          const uint16_t* pp = static_cast<const uint16_t*>(a.v.params) +
                               prm_rec(a.v, a.sh, b, h, d.tq0 + 16 * vhv) + vch / vG;
#pragma unroll
          for (int u = 0; u < 16; ++u) R.vp[u] = pp[u * vng];
        } else if (vkind != KVQ_QUANT_FP8_E5M2) {
          const uint32_t* pp = static_cast<const uint32_t*>(a.v.params) +
                               prm_rec(a.v, a.sh, b, h, d.tq0 + 16 * vhv) + vch / vG;
#pragma unroll
          for (int u = 0; u < 16; ++u) R.vp[u] = pp[u * vng];
        }
      }
    }
  };

  // (cos, sin) of the first position of block blk into rb[blk & 1]
  auto base_rot = [&](int blk) {
    if (a.rope && blk < n_blk && tid < kD / 2) {
      S.rb[blk & 1][tid] = rope_cs(S.theta[tid], desc(blk).t0);
    }
  };
  // this workgroup's split of the blocks
  const int blk_lo = blockIdx.z * a.blocks_per_split;
  const int blk_hi = min(n_blk, blk_lo + a.blocks_per_split);
  base_rot(blk_lo);
  Raw R;
  if (PIPE) fetch(blk_lo, R);
  for (int blk = blk_lo; blk < blk_hi; ++blk) {
    const Desc d = desc(blk);
    const bool sinkb = d.sinkb;
    const int t0 = d.t0, n_valid = d.n_valid;
    const int64_t tq0 = d.tq0;
    __syncthreads();   // the previous block's operand reads are done
    if (!PIPE) fetch(blk, R);
    // ---- keys: decode, then RoPE at the key's position and fp16 planes ---------
    {
      float x0[8], x1[8];
      const int64_t tq = tq0 + ktk;
      if (ktk >= n_valid) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x0[e] = x1[e] = 0.f;
      } else if (sinkb || kraw || (kpc && tq >= n_full)) {
        const uint4 r0 = R.kq[0], r1 = R.kq[1];
        const uint32_t w0[4] = {r0.x, r0.y, r0.z, r0.w}, w1[4] = {r1.x, r1.y, r1.z, r1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x0[e] = elem2f((uint16_t)(w0[e >> 1] >> (16 * (e & 1))), a.sh.kv_bf16);
          x1[e] = elem2f((uint16_t)(w1[e >> 1] >> (16 * (e & 1))), a.sh.kv_bf16);
        }
      } else if (kbits == 4) {
        key_values<4>(kkind, kpc, S, R, kmp, ksq, ksc, x0, x1);
      } else if (kbits == 3) {
        key_values<3>(kkind, kpc, S, R, kmp, ksq, ksc, x0, x1);
      } else {
        key_values<8>(kkind, kpc, S, R, kmp, ksq, ksc, x0, x1);
      }
      const int c0 = 32 * kmp + 8 * ksq;
      if (kstage) {
        // outliers overwrite some of these before RoPE: stage in fp32
        float4* d0 = reinterpret_cast<float4*>(&S.kf[ktk][c0]);
        float4* d1 = reinterpret_cast<float4*>(&S.kf[ktk][c0 + 64]);
        d0[0] = float4{x0[0], x0[1], x0[2], x0[3]};
        d0[1] = float4{x0[4], x0[5], x0[6], x0[7]};
        d1[0] = float4{x1[0], x1[1], x1[2], x1[3]};
        d1[1] = float4{x1[4], x1[5], x1[6], x1[7]};
      } else {
        if (a.rope && ktk < n_valid) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float cs, sn;
            rot_add(S.rb[blk & 1][c0 + e], S.rt[ktk][c0 + e], cs, sn);
            const float y0 = x0[e], y1 = x1[e];
            x0[e] = y0 * cs - y1 * sn;
            x1[e] = y1 * cs + y0 * sn;
          }
        }
        uint4 hi, lo;
        const int sw = kswz(ktk);
        split8(x0, hi, lo);
        S.khi[ktk][(c0 >> 3) ^ sw] = hi;
        S.klo[ktk][(c0 >> 3) ^ sw] = lo;
        split8(x1, hi, lo);
        S.khi[ktk][((c0 >> 3) + 8) ^ sw] = hi;
        S.klo[ktk][((c0 >> 3) + 8) ^ sw] = lo;
      }
    }
    // ---- values: channel vch, tokens 16 vhv .. 16 vhv + 15 -------------------------
    {
      float x[16];
      if (sinkb || vraw) {
#pragma unroll
        for (int u = 0; u < 16; ++u) x[u] = elem2f((uint16_t)R.vp[u], a.sh.kv_bf16);
      } else if (vkind == KVQ_QUANT_CODEBOOK) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const uint32_t code = (R.vc[u >> 2] >> (8 * (u & 3) + 4 * (vch >> 6))) & 15u;
          x[u] = 16 * vhv + u < n_valid ? h2f(S.cbv[vch][code]) : 0.f;
        }
      } else if (vbits == 4) {
        value_values<4>(vkind, R, vch, vhv, vsc, n_valid, x);
      } else if (vbits == 3) {
        value_values<3>(vkind, R, vch, vhv, vsc, n_valid, x);
      } else {
        value_values<8>(vkind, R, vch, vhv, vsc, n_valid, x);
      }
      const int sw = (vch >> 2) & 3;
      uint4 hi, lo;
      split8(x, hi, lo);
      S.vhi[vch][(2 * vhv) ^ sw] = hi;
      S.vlo[vch][(2 * vhv) ^ sw] = lo;
      split8(x + 8, hi, lo);
      S.vhi[vch][(2 * vhv + 1) ^ sw] = hi;
      S.vlo[vch][(2 * vhv + 1) ^ sw] = lo;
    }
    // ---- outliers replace their dense value ------------------------------------
    if (!sinkb && (a.k.k_out > 0 || a.v.k_out > 0)) {
      __syncthreads();
      if (a.k.k_out > 0) stage_outliers<true>(a.k, S, tid, b, h, tq0, n_valid, a.sh);
      if (a.v.k_out > 0) stage_outliers<false>(a.v, S, tid, b, h, tq0, n_valid, a.sh);
    }
    if (kstage) {
      // RoPE at the key's position, then fp16 planes (token ktk, pairs (i, i + 64)
      // for i = 8 pb .. 8 pb + 7)
      __syncthreads();
      const int pb = tid & 7;
      float x0[8], x1[8];
      const float4* r0 = reinterpret_cast<const float4*>(&S.kf[ktk][8 * pb]);
      const float4* r1 = reinterpret_cast<const float4*>(&S.kf[ktk][64 + 8 * pb]);
      const float4 a0 = r0[0], a1 = r0[1], b0 = r1[0], b1 = r1[1];
      x0[0] = a0.x; x0[1] = a0.y; x0[2] = a0.z; x0[3] = a0.w;
      x0[4] = a1.x; x0[5] = a1.y; x0[6] = a1.z; x0[7] = a1.w;
      x1[0] = b0.x; x1[1] = b0.y; x1[2] = b0.z; x1[3] = b0.w;
      x1[4] = b1.x; x1[5] = b1.y; x1[6] = b1.z; x1[7] = b1.w;
      if (a.rope && ktk < n_valid) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float cs, sn;
          rot_add(S.rb[blk & 1][8 * pb + e], S.rt[ktk][8 * pb + e], cs, sn);
          const float y0 = x0[e], y1 = x1[e];
          x0[e] = y0 * cs - y1 * sn;
          x1[e] = y1 * cs + y0 * sn;
        }
      }
      uint4 hi, lo;
      const int sw = kswz(ktk);
      split8(x0, hi, lo);
      S.khi[ktk][pb ^ sw] = hi;
      S.klo[ktk][pb ^ sw] = lo;
      split8(x1, hi, lo);
      S.khi[ktk][(pb + 8) ^ sw] = hi;
      S.klo[ktk][(pb + 8) ^ sw] = lo;
    }
    __syncthreads();
    if (PIPE && blk + 1 < blk_hi) fetch(blk + 1, R);   // the next block's loads run under this block's products
    base_rot(blk + 1);             // read after the next block's first barrier
    if (!wave_ok || t0 > p_wave) continue;   // nothing of this block is visible to the wave

    // ---- scores: tokens 8 q4 + 4T + i for T = 0, 1 --------------------------
    // (the products run at raised wave priority, so that they issue while
    // the other workgroup of the CU stages its block)
    __builtin_amdgcn_s_setprio(1);
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
    __builtin_amdgcn_s_setprio(0);
  }

  // ---- normalize and store (or the split's partial state): lane holds
  // channels 16 ct + 4 q4 + i of row n ------------------------------------------
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (!row_ok) return;
  const int64_t rowi = ((int64_t)b * a.n_q + qi) * a.sh.Hq + jh;
  if (a.splits > 1) {
    float* rec = a.partial + (rowi * a.splits + blockIdx.z) * (kD + 2);
    // records are 8-byte aligned (d + 2 floats): scalar stores
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) rec[16 * ct + 4 * q4 + i] = o[ct][i];
    if (q4 == 0) {
      rec[kD] = m_run;
      rec[kD + 1] = l_tot;
    }
    return;
  }
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int64_t orow = rowi * kD;
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
  if (a.splits < 1 || (a.splits > 1 && !a.partial)) return hipErrorInvalidValue;
  if (a.codes) return launch_prefill_codes(a, stream) ? hipGetLastError() : hipErrorNotSupported;
  const dim3 grid((unsigned)tiles, (unsigned)(a.sh.B * a.sh.Hkv), (unsigned)a.splits);
  const DevTensor &k = a.k, &v = a.v;
  auto asym = [](const DevTensor& t, int bits) {
    return (t.quant == KVQ_QUANT_ASYM_MINMAX || t.quant == KVQ_QUANT_ASYM_ABSMAX_OFFSET) && t.bits == bits;
  };
  if (asym(k, 4) && k.per_channel && asym(v, 4))
    hipLaunchKernelGGL((pre_mfma_kernel<F_PC4, F_U4>), grid, dim3(256), 0, stream, a);
  else if (asym(k, 3) && !k.per_channel && asym(v, 3))
    hipLaunchKernelGGL((pre_mfma_kernel<F_U3, F_U3>), grid, dim3(256), 0, stream, a);
  else if (k.quant == KVQ_QUANT_SYM_Q8_0 && v.quant == KVQ_QUANT_SYM_Q8_0)
    hipLaunchKernelGGL((pre_mfma_kernel<F_Q8, F_Q8>), grid, dim3(256), 0, stream, a);
  else if (k.quant == KVQ_QUANT_CODEBOOK && v.quant == KVQ_QUANT_CODEBOOK)
    hipLaunchKernelGGL((pre_mfma_kernel<F_CB, F_CB>), grid, dim3(256), 0, stream, a);
  else if (k.quant == KVQ_QUANT_FP8_E5M2 && v.quant == KVQ_QUANT_FP8_E5M2)
    hipLaunchKernelGGL((pre_mfma_kernel<F_F8, F_F8>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((pre_mfma_kernel<F_ANY, F_ANY>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
