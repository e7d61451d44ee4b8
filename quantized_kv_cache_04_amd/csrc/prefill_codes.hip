// Chunked-prefill attention of libkvq for the uniform formats (3/4/8-bit
// asymmetric or q8_0 codes with per-token or per-channel keys, and FP8
// E5M2), with the packed codes themselves as matrix-core operands.
//
// Prefill scores many queries against the same cached keys, so both
// products are dense contractions (Survey page, sections 2.3 and 5.3;
// NIAH page, section 4.2), and dequantization is fused into them (KVQuant
// page, section 3.4).  The operand scheme is the decode kernel's: a code in
// the low bits of an fp16 is the exact subnormal code * 2^-24, so the
// packed codes unpack into MFMA operands with a few masks, and the scales go
// to the other operand.  Here that operand holds 16 query rows, a row being
// one (query token, query head of the group):
//  * QK^T (v_mfma_f32_16x16x32_f16): A = the codes of 16 tokens, 32
//    channels per instruction; B = the 16 rows' q (times the key scales of
//    the current group for per-channel keys), pre-scaled by a power of two
//    and split into fp16 high and low parts.  Zero points and per-token key
//    scales are applied to the score in fp32.
//  * P.V: A = the 16 rows' probabilities times the value scale of each
//    token, again as high and low parts; B = the value codes of the value
//    tile.  The QK^T result layout (lane (q, n): tokens 4q + r and
//    16 + 4q + r of row n) is that A operand as it stands.
// The high and low parts are two instructions into one accumulator, the low
// parts first.  The matrix cores keep only so many bits below the largest
// product of an instruction: the query operand's high part therefore sits
// on a fixed grid (pair_operand_fixed), which makes the high-part products
// of the scores add up exactly.
// Each wave owns 16 rows and streams every block of its range itself; the
// four waves of a workgroup read the same bytes at about the same time,
// which the vector cache serves.  Per 32-token block a wave spends 32
// matrix-core instructions on its rows, and its vector work is the code
// unpacking plus the softmax of 16 rows.
//
// The online softmax keeps the decode kernel's conventions: probabilities in
// "fed units" p' = 2^(s - m_run + pexp - pe_exp(class)), a lazily moved
// running maximum per row, a per-wave exponent pexp that keeps the fed value
// operand below 2^15, odd token pairs fed as -P against complemented codes
// (so that the products alternate in sign), and the accumulators moved into
// fp32 sums in LDS every 16 blocks.  Rows see the tokens at or before their
// own position (causal); the blocks a wave sees only in part are masked.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "mfma_codes.h"

namespace kvq {
namespace {

constexpr int kD = kHeadDim;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRowsWG = 64;   // query rows per workgroup, 16 per wave

template <int KB, bool KCH, bool KQ8, int NGK, int VB, bool VQ8, int NGV, bool F8>
__global__ __launch_bounds__(256, 2) void pre_codes_kernel(PrefillArgs a) {
  static_assert(!F8 || (KB == 8 && VB == 8 && !KCH && !KQ8 && !VQ8 && NGK == 1 && NGV == 1),
                "FP8 keys and values: one shape");
  // raw dwords of one 32-token block for this lane (the decode kernel's
  // register layout)
  constexpr int VPD = F8 ? 1 : (VQ8 ? 2 * NGV : 4 * NGV);            // value params of 4 tokens
  constexpr int KPD = (KCH || F8) ? 1 : (KQ8 ? 2 * NGK : 4 * NGK);   // key params of 4 tokens
  struct Buf {
    uint32_t k[2][KB];      // key codes, token 16 mb + n, segment q4
    uint32_t v[2 * VB];     // value tile, this lane's 8 VB bytes
    uint32_t vp[2][VPD];    // value scale(/zero) of tokens 16 mb + 4 q4 + r
    uint32_t kp[2][KPD];    // key scale(/zero) of the same tokens (per-token keys)
  };
  constexpr float kLazy = 8.0f;   // log2 headroom before a row's running max moves
  constexpr int kFedLog2 = 15;    // fed P operand entries stay below 2^kFedLog2
  constexpr int NC = kClasses<VB>;
  constexpr float kCmax = VQ8 ? 127.0f : (float)((1 << VB) - 1);
  constexpr int kFlush = 16;

  // byte codes (q8_0, FP8): the waves share the unpacking of the blocks that
  // every row of the workgroup sees whole.  (Shared 4-bit unpacking was
  // slower, 22.3 against 20.5 ms on the serving shape: there the barrier per
  // block and the LDS round trip cost more than the masks they save, and so
  // they did for 3-bit codes, 359 -> 340 TFLOP/s on the config-3 shape; for byte
  // codes the per-wave loads and byte permutes cost more: FP8 403 -> 519
  // TFLOP/s, q8_0 260 -> 278.)
  constexpr bool SHARE = KB == 8 && VB == 8;
  struct SBuf {               // one wave's share of a block, and the parameters
    uint32_t k[2 * KB / 4];   // key blocks m0, m0 + 1 of token 16 mb_s + n, segment q4
    uint32_t v[2 * VB / 4];   // value blocks nb0, nb0 + 1 of the lane's tile bytes
    uint32_t vp[2][VPD];
    uint32_t kp[2][KPD];
  };
  // MFMA operands of the block, by lane: [buffer][4 mb + m][lane] and [buffer][nb][lane]
  __shared__ u32x4 kop[SHARE ? 2 : 1][SHARE ? 8 : 1][64];
  __shared__ u32x4 vop[SHARE ? 2 : 1][SHARE ? 8 : 1][64];
  __shared__ float wo[4][16][kD];    // per wave and row: output sums (true units)
  __shared__ float wml[4][16][2];    // per wave and row: running max, sum of p

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int q4 = lane >> 4, n = lane & 15;
  const int bh = blockIdx.y, b = bh / a.sh.Hkv, h = bh % a.sh.Hkv;
  const int g = a.sh.g, qt = kRowsWG / g;
  const int tile = gridDim.x - 1 - blockIdx.x;   // longest tiles (latest queries) first
  const int base = a.n_total - a.n_q;            // position of query 0
  const DevTensor& K = a.k;
  const DevTensor& V = a.v;
  const int64_t Tcap = a.sh.Tcap;
  const int64_t prow = (int64_t)bh * Tcap;       // row of token 0 of (b, h), contiguous cache
  const float sm2 = a.sm_scale * kLog2e;
  const bool paged = a.sh.page_table != nullptr;

  // ---- rows: this lane's row 16 wave + n, and the wave's position range ----------
  const int rw = 16 * wave + n;
  const int qi = tile * qt + rw / g, jh = h * g + rw % g;
  const bool row_ok = qi < a.n_q;
  const int p_row = row_ok ? base + qi : -1;
  const int qi_w0 = tile * qt + (16 * wave) / g;                    // wave-uniform
  const int qi_w1 = min(a.n_q - 1, tile * qt + (16 * wave + 15) / g);
  const bool wave_ok = qi_w0 < a.n_q;
  const int p_wlo = base + qi_w0, p_whi = base + qi_w1;
  const int p_max = base + min(a.n_q - 1, tile * qt + qt - 1);     // the workgroup's last position

  // ---- blocks: this split's range, the wave's part of it --------------------------
  const int n_blk = p_max / kTile + 1;
  const int blk_lo = blockIdx.z * a.blocks_per_split;
  const int blk_hi = min(n_blk, blk_lo + a.blocks_per_split);
  const int wblk_hi = wave_ok ? min(blk_hi, p_whi / kTile + 1) : blk_lo;
  // per-channel keys: tokens below n_full have quantized keys, the others sit
  // in the unquantized tail (whole blocks: the group size is a multiple of 32)
  const int n_full = KCH ? (a.n_total / K.G) * K.G : a.n_total;
  const int qend = n_full / kTile;
  // blocks every row of the wave sees whole, with quantized keys: no masking
  const int f_end = max(blk_lo, min(min(wblk_hi, KCH ? qend : wblk_hi), (p_wlo + 1) / kTile));

  // ---- this lane's query: channels 32 m + 8 q4 + e -----------------------------------
  uint32_t qw[4][4];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (((int64_t)b * a.n_q + (row_ok ? qi : 0)) * a.sh.Hq + jh) * kD + 8 * q4;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qp + 32 * m);
      qw[m][0] = row_ok ? v.x : 0u;
      qw[m][1] = row_ok ? v.y : 0u;
      qw[m][2] = row_ok ? v.z : 0u;
      qw[m][3] = row_ok ? v.w : 0u;
    }
  }
  auto q_el = [&](int m, int e) {
    return elem2f((uint16_t)(qw[m][e >> 1] >> (16 * (e & 1))), a.sh.kv_bf16);
  };

  // ---- running state ---------------------------------------------------------------
  f32x4 oacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;   // row's reference maximum (the four lanes of a row agree)
  float mref = 0.f;          // m_run - pexp once the row has seen a token
  float thr = -INFINITY;     // move the maximum when t > thr
  float l_run[NC];
  float vbias[NGV][NC];      // sum of p' * zero (and the complement terms) per class
  float voff[NGV];           // q8_0 values: offset term of what was fed
#pragma unroll
  for (int c = 0; c < NC; ++c) l_run[c] = 0.f;
#pragma unroll
  for (int gi = 0; gi < NGV; ++gi) {
#pragma unroll
    for (int c = 0; c < NC; ++c) vbias[gi][c] = 0.f;
    voff[gi] = 0.f;
  }
  int pexp = 0;
  float sbound = 0.f;
  float kbias = 0.f;         // per-channel keys: sm2 * sum_c q_c z_c of the row
  float tbias[NC], kb2[NC];
  auto set_bias = [&]() {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      tbias[c] = -mref - (float)pe_exp<VB>(c);
      kb2[c] = kbias + tbias[c];
    }
  };
  set_bias();
  for (int i = lane; i < 16 * kD; i += 64) (&wo[wave][0][0])[i] = 0.f;

  // ---- per-token keys: fixed B operand of the rows, scaled by 2^Eq ------------------
  half8 bqh[4], bql[4];
  float qsum[NGK];   // per key group: sm2 * sum of the row's q
  float qoff[NGK];   // q8_0 keys: 128 * 2^-24 * sum of the fed operand
  float kq = 0.f;    // accumulator units -> sm2 * true units
  if constexpr (!KCH) {
    float qv[4][8];
    float mx = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qv[m][e] = q_el(m, e);
        mx = fmaxf(mx, fabsf(qv[m][e]));
      }
    mx = wave_max(mx);
    int Eq = 14 - ceil_log2(mx);
    if (Eq > 100) Eq = 100;
    kq = F8 ? pow2i(-Eq) * sm2 * fp8_scale(K, h) : pow2i(24 - Eq > 126 ? 126 : 24 - Eq) * sm2;
    const float sc = pow2i(Eq);
#pragma unroll
    for (int gi = 0; gi < NGK; ++gi) { qsum[gi] = 0.f; qoff[gi] = 0.f; }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float s = 0.f, so = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s += qv[m][e];
      u32x4 hi, lo;
      pair_operand_fixed<KB>(qv[m], sc, hi, lo);
      bqh[m] = __builtin_bit_cast(half8, hi);
      bql[m] = __builtin_bit_cast(half8, lo);
      if constexpr (KQ8) {
        const half8 hv = bqh[m], lv = bql[m];
#pragma unroll
        for (int e = 0; e < 8; ++e) so += (float)hv[e] + (float)lv[e];
      }
      qsum[m * NGK / 4] += s;
      qoff[m * NGK / 4] += so;
    }
#pragma unroll
    for (int gi = 0; gi < NGK; ++gi) {
      qsum[gi] = rows_sum(qsum[gi]) * sm2;
      qoff[gi] = 128.0f * 0x1p-24f * rows_sum(qoff[gi]);
    }
  }

  // ---- per-channel keys: B operand and zero term of key group grp ------------------
  // q * scale of the lane's 32 channels, scaled by a power of two common to
  // the wave, split into fp16 high and low parts in pair order.
  float kscale = 0.f;
  int grp_cur = -1;
  auto key_group = [&](int grp) {
    const uint32_t* prm = static_cast<const uint32_t*>(K.params) +
                          ((int64_t)bh * (Tcap / K.G) + grp) * kD + 8 * q4;
    float xs[4][8];
    float zb = 0.f, mx = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const u32x4 p0 = *reinterpret_cast<const u32x4*>(prm + 32 * m);
      const u32x4 p1 = *reinterpret_cast<const u32x4*>(prm + 32 * m + 4);
      const uint32_t pz[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const half2v sz = __builtin_bit_cast(half2v, pz[e]);   // (scale, zero)
        const float qe = h2f((uint16_t)(qw[m][e >> 1] >> (16 * (e & 1))));   // fp16 keys and queries
        xs[m][e] = qe * (float)sz[0];
        mx = fmaxf(mx, fabsf(xs[m][e]));
        zb = __builtin_fmaf(qe, (float)sz[1], zb);
      }
    }
    mx = wave_max(mx);
    int E = 14 - ceil_log2(mx);
    if (E > 100) E = 100;
    kscale = pow2i(24 - E > 126 ? 126 : 24 - E) * sm2;
    const float s2 = pow2i(E);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      u32x4 hi, lo;
      pair_operand_fixed<KB>(xs[m], s2, hi, lo);
      bqh[m] = __builtin_bit_cast(half8, hi);
      bql[m] = __builtin_bit_cast(half8, lo);
    }
    kbias = rows_sum(zb) * sm2;
#pragma unroll
    for (int c = 0; c < NC; ++c) kb2[c] = kbias + tbias[c];
  };
  auto group_for = [&](int blk) {
    if constexpr (KCH) {
      const int grp = blk * kTile / K.G;
      if (grp != grp_cur) {   // wave-uniform
        grp_cur = grp;
        key_group(grp);
      }
    }
  };

  // ---- loads --------------------------------------------------------------------------
  const uint32_t k_lane_off = (uint32_t)n * (16 * KB) + (uint32_t)q4 * (4 * KB);
  const uint32_t v_lane_off = (uint32_t)lane * (8 * VB);
  const uint32_t p_lane_tok = 4u * (uint32_t)q4;
  // row of the block's first token (its 32 tokens are consecutive rows: one
  // page of a paged cache)
  auto block_row = [&](int blk) -> int64_t {
    return paged ? page_head_row(a.sh, page_of(a.sh, b, blk), h) : prow + (int64_t)blk * kTile;
  };
  auto load_row = [&](Buf& B, int64_t r0) {
    const uint8_t* kcodes = K.codes + r0 * (4 * KB * 4);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      load_dw<KB>(kcodes + (16 * mb) * (16 * KB) + k_lane_off, B.k[mb]);
      const uint32_t tok = 16 * mb + p_lane_tok;
      if constexpr (F8) {
        B.vp[mb][0] = 0u;
        B.kp[mb][0] = 0u;
      } else {
        const uint8_t* vprm = static_cast<const uint8_t*>(V.params) + r0 * NGV * (VQ8 ? 2 : 4);
        load_dw<VPD>(vprm + tok * (NGV * (VQ8 ? 2 : 4)), B.vp[mb]);
        if constexpr (!KCH) {
          const uint8_t* kprm = static_cast<const uint8_t*>(K.params) + r0 * NGK * (KQ8 ? 2 : 4);
          load_dw<KPD>(kprm + tok * (NGK * (KQ8 ? 2 : 4)), B.kp[mb]);
        } else {
          B.kp[mb][0] = 0u;
        }
      }
    }
    load_dw<2 * VB>(V.codes + r0 * (4 * VB * 4) + v_lane_off, B.v);
  };

  // ---- shared unpacking (byte formats): wave w loads and unpacks key
  // blocks m = 2 (w & 1), +1 of tokens 16 (w >> 1) + (0..15) and value blocks
  // nb = 2 w, 2 w + 1, for every lane's slot of those operands ----------------------
  const int mb_s = wave >> 1, m0 = 2 * (wave & 1), nb0 = 2 * wave;
  auto load_share = [&](SBuf& S, int64_t r0) {
    const uint8_t* kcodes = K.codes + r0 * (4 * KB * 4);
    // a block of 8 codes is KB bytes of the lane's segment
    load_dw<2 * KB / 4>(kcodes + (16 * mb_s) * (16 * KB) + k_lane_off + m0 * KB, S.k);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const uint32_t tok = 16 * mb + p_lane_tok;
      if constexpr (F8) {
        S.vp[mb][0] = 0u;
        S.kp[mb][0] = 0u;
      } else {
        const uint8_t* vprm = static_cast<const uint8_t*>(V.params) + r0 * NGV * (VQ8 ? 2 : 4);
        load_dw<VPD>(vprm + tok * (NGV * (VQ8 ? 2 : 4)), S.vp[mb]);
        if constexpr (!KCH) {
          const uint8_t* kprm = static_cast<const uint8_t*>(K.params) + r0 * NGK * (KQ8 ? 2 : 4);
          load_dw<KPD>(kprm + tok * (NGK * (KQ8 ? 2 : 4)), S.kp[mb]);
        } else {
          S.kp[mb][0] = 0u;
        }
      }
    }
    load_dw<2 * VB / 4>(V.codes + r0 * (4 * VB * 4) + v_lane_off + nb0 * VB, S.v);
  };
  auto produce = [&](const SBuf& S, int buf) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      kop[buf][4 * mb_s + m0 + j][lane] = __builtin_bit_cast(u32x4, code_block<KB, KQ8, false, F8>(S.k, j));
#pragma unroll
    for (int j = 0; j < 2; ++j)
      vop[buf][nb0 + j][lane] = __builtin_bit_cast(u32x4, code_block<VB, VQ8, true, F8>(S.v, j));
  };

  // ---- scores of a block with quantized keys: sc = t + mref, per token pair
  // class (the class bias is in kb2 / tbias) -----------------------------------
  // kcode_of(mb, m): the key operand of tokens 16 mb + (0..15),
  // channels 32 m + (0..31); kp: the per-token key parameters
  auto scores_q = [&](const uint32_t (*kp)[KPD], auto&& kcode_of, float sc[2][4]) {
    if constexpr (KCH) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
        half8 kcode[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) kcode[m] = kcode_of(mb, m);
#pragma unroll
        for (int m = 0; m < 4; ++m) c = mfma16(kcode[m], bql[m], c);
#pragma unroll
        for (int m = 0; m < 4; ++m) c = mfma16(kcode[m], bqh[m], c);
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[mb][r] = c[r] * kscale + kb2[pe_class<VB>(r)];
      }
    } else {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        // score = kq * sum_g scale_g * dot_g + sum_g zero_g * qsum_g + bias
        float sd[4], zq[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) { sd[r] = 0.f; zq[r] = tbias[pe_class<VB>(r)]; }
#pragma unroll
        for (int gi = 0; gi < NGK; ++gi) {
          f32x4 c = {0.f, 0.f, 0.f, 0.f};
          half8 kcode[4];
#pragma unroll
          for (int m = gi * 4 / NGK; m < (gi + 1) * 4 / NGK; ++m) kcode[m] = kcode_of(mb, m);
#pragma unroll
          for (int m = gi * 4 / NGK; m < (gi + 1) * 4 / NGK; ++m) c = mfma16(kcode[m], bql[m], c);
#pragma unroll
          for (int m = gi * 4 / NGK; m < (gi + 1) * 4 / NGK; ++m) c = mfma16(kcode[m], bqh[m], c);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t* d = kp[mb];
            if constexpr (F8) {
              sd[r] += c[r];
            } else if constexpr (KQ8) {
              const int idx = r * NGK + gi;
              const half2v sv = __builtin_bit_cast(half2v, d[idx >> 1]);
              sd[r] = __builtin_fmaf((float)sv[idx & 1], c[r] - qoff[gi], sd[r]);
            } else {
              const half2v sz = __builtin_bit_cast(half2v, d[r * NGK + gi]);   // (scale, zero)
              sd[r] = __builtin_fmaf((float)sz[0], c[r], sd[r]);
              zq[r] = __builtin_fmaf((float)sz[1], qsum[gi], zq[r]);
            }
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[mb][r] = __builtin_fmaf(sd[r], kq, zq[r]);
      }
    }
  };

  // scores of a block of the per-channel keys' unquantized tail: the fp16
  // keys and the row's fp16 query are exact operands (one product)
  auto scores_tail = [&](int blk, float sc[2][4]) {
    const int t0 = blk * kTile;
    // 32 consecutive rows of the tail ring (its size is a multiple of 32)
    const uint16_t* tail = K.tail + ((int64_t)bh * K.tail_rows + t0 % K.tail_rows) * kD;
    half8 bt[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) bt[m] = as_h8(qw[m][0], qw[m][1], qw[m][2], qw[m][3]);
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
      for (int r = 0; r < 4; ++r) sc[mb][r] = c[r] * sm2 + tbias[pe_class<VB>(r)];
    }
  };

  // ---- softmax and P.V of one block (t0: its first token).  MASKED (an
  // integral_constant): the causal mask per row and the end of the cache
  // apply; the other blocks are seen whole by every row of the wave.
  // vp_in: value parameters of the lane's 8 tokens; vcode_of(nb): the
  // value operand of channels 16 nb + (0..15)
  auto softmax_pv = [&](auto masked, float sc[2][4], const uint32_t (*vp_in)[VPD], auto&& vcode_of,
                        int t0) {
    constexpr bool MASKED = decltype(masked)::value;
    auto vis = [&](int mb, int r) { return !MASKED || t0 + 16 * mb + 4 * q4 + r <= p_row; };
    auto present = [&](int mb, int r) { return !MASKED || t0 + 16 * mb + 4 * q4 + r < a.n_total; };
    float t[2][4];
    float bmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        t[mb][r] = vis(mb, r) ? sc[mb][r] : -INFINITY;
        bmax = fmaxf(bmax, t[mb][r]);
      }
    if (__any(bmax > thr)) {
      // move the rows' reference maxima (rare after the first blocks); a row
      // that has seen no token yet keeps m_run = -inf
      const float m_new = fmaxf(m_run, rows_max(bmax) + mref);
      const bool live = m_new > -INFINITY;
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int c = 0; c < NC; ++c) l_run[c] *= alpha;
#pragma unroll
      for (int gi = 0; gi < NGV; ++gi) {
#pragma unroll
        for (int c = 0; c < NC; ++c) vbias[gi][c] *= alpha;
        voff[gi] *= alpha;
      }
      // accumulator row r of this lane is row 4 q4 + r, whose factor sits in
      // lane 4 q4 + r
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float f = __shfl(alpha, 4 * q4 + r, 64);
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          oacc[nb][r] *= f;
          wo[wave][4 * q4 + r][16 * nb + n] *= f;
        }
      }
      m_run = m_new;
      const float mref_new = live ? m_run - (float)pexp : mref;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) t[mb][r] += mref - mref_new;
      mref = mref_new;
      thr = live ? kLazy + (float)pexp : -INFINITY;
      set_bias();
    }

    // value parameters of this lane's 8 tokens (zeroed past the cache)
    uint32_t vp[2][VPD];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int w = 0; w < VPD; ++w) {
        uint32_t d = vp_in[mb][w];
        if constexpr (MASKED) {
          if constexpr (VQ8) {   // two entries (token r = entry / NGV) per dword
            const uint32_t lo = present(mb, (2 * w) / NGV) ? 0x0000ffffu : 0u;
            const uint32_t hi = present(mb, (2 * w + 1) / NGV) ? 0xffff0000u : 0u;
            d &= lo | hi;
          } else {               // scale | zero << 16 of token r = w / NGV
            d = present(mb, w / NGV) ? d : 0u;
          }
        }
        vp[mb][w] = d;
      }
    // largest value scale of the block (scales are non-negative fp16)
    half2v smx = __builtin_bit_cast(half2v, vp[0][0]);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int w = 0; w < VPD; ++w) smx = __builtin_elementwise_max(smx, __builtin_bit_cast(half2v, vp[mb][w]));
    const float smax = F8 ? 1.0f : (VQ8 ? fmaxf((float)smx[0], (float)smx[1]) : (float)smx[0]);
    if (__any(smax > sbound)) {
      const float sm = rows_max(smax);         // the same tokens in every row
      int np = kFedLog2 - (int)kLazy - ceil_log2(sm);
      np = np < -60 ? -60 : (np > 60 ? 60 : np);
      const int e = np - pexp;                 // rescale what was fed so far
      const float f = pow2i(e);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[nb][r] *= f;
#pragma unroll
      for (int c = 0; c < NC; ++c) l_run[c] *= f;
#pragma unroll
      for (int gi = 0; gi < NGV; ++gi) {
#pragma unroll
        for (int c = 0; c < NC; ++c) vbias[gi][c] *= f;
        voff[gi] *= f;
      }
      pexp = np;
      sbound = pow2i(kFedLog2 - (int)kLazy - np);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) t[mb][r] += (float)e;
      mref -= (float)e;
      thr = m_run == -INFINITY ? -INFINITY : kLazy + (float)pexp;
      set_bias();
    }

    // probabilities in fed units
    float pr[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[mb][r] = __builtin_amdgcn_exp2f(t[mb][r]);
        l_run[pe_class<VB>(r)] += pr[mb][r];
      }
    // P operand of each value group: pair r = tokens (4 q4 + r, 16 + 4 q4 + r),
    // p' * scale as fp16 high and low parts; zero points enter through vbias
    half8 pah[NGV], pal[NGV];
#pragma unroll
    for (int gi = 0; gi < NGV; ++gi) {
      uint32_t oh[4], ol[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          if constexpr (F8) {
            x[mb] = pr[mb][r];   // signed values: no complement, no scale
          } else if constexpr (VQ8) {
            const int idx = r * NGV + gi;
            const half2v hv = __builtin_bit_cast(half2v, vp[mb][idx >> 1]);
            const float sc_h = (float)hv[idx & 1];
            x[mb] = __builtin_fmaf(pr[mb][r], (r & 1) ? -sc_h : sc_h, 0.f);
          } else {
            const half2v hv = __builtin_bit_cast(half2v, vp[mb][r * NGV + gi]);
            const float sc_h = (float)hv[0];
            x[mb] = __builtin_fmaf(pr[mb][r], (r & 1) ? -sc_h : sc_h, 0.f);
            // odd pairs: + cmax p' scale (x holds -p' scale there)
            const int cl = pe_class<VB>(r);
            const float vb = (r & 1) ? __builtin_fmaf(-kCmax, x[mb], vbias[gi][cl]) : vbias[gi][cl];
            vbias[gi][cl] = __builtin_fmaf(pr[mb][r], (float)hv[1], vb);
          }
        }
        const half2v hh = cvt_pk_rn(x[0], x[1]);
        const float h0 = (float)hh[0], h1 = (float)hh[1];
        const half2v ll = cvt_pk_rn(x[0] - h0, x[1] - h1);
        oh[r] = __builtin_bit_cast(uint32_t, hh);
        ol[r] = __builtin_bit_cast(uint32_t, ll);
        if constexpr (VQ8) {   // the offset term must cancel what was fed
          // even pairs: P (q + 128) -> -128 P; odd: -P (127 - q) -> +127 P
          const float fed = (h0 + (float)ll[0]) + (h1 + (float)ll[1]);
          voff[gi] = __builtin_fmaf(fed, (r & 1) ? -kCmax : -128.0f, voff[gi]);
        }
      }
      pah[gi] = as_h8(oh[0], oh[1], oh[2], oh[3]);
      pal[gi] = as_h8(ol[0], ol[1], ol[2], ol[3]);
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int nbk = 0; nbk < 8; ++nbk) {
      const half8 vcode = vcode_of(nbk);
      oacc[nbk] = mfma16(pal[nbk * NGV / 8], vcode, oacc[nbk]);
      oacc[nbk] = mfma16(pah[nbk * NGV / 8], vcode, oacc[nbk]);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Move the accumulators into the wave's LDS sums (true units) and restart
  // them: the code products times 2^24 (codes are fed as code * 2^-24) plus
  // the zero or offset term.  Doing this every kFlush blocks bounds the fp32
  // sums the matrix cores keep adding into.
  int since_flush = 0;
  const float ofac = F8 ? fp8_scale(V, h) : 0x1p24f;
  auto flush = [&]() {
    const float vscale = pow2i(-pexp);
    float vb_row[NGV][4];
#pragma unroll
    for (int gi = 0; gi < NGV; ++gi) {
      float vb = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) vb = __builtin_fmaf(vbias[gi][c], pow2i(pe_exp<VB>(c)), vb);
      const float tot = rows_sum(VQ8 ? voff[gi] : vb);   // the row's total, in all its lanes
#pragma unroll
      for (int r = 0; r < 4; ++r) vb_row[gi][r] = __shfl(tot, 4 * q4 + r, 64);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
        wo[wave][4 * q4 + r][16 * nb + n] += (oacc[nb][r] * ofac + vb_row[nb * NGV / 8][r]) * vscale;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) oacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gi = 0; gi < NGV; ++gi) {
#pragma unroll
      for (int c = 0; c < NC; ++c) vbias[gi][c] = 0.f;
      voff[gi] = 0.f;
    }
    since_flush = 0;
  };

  // operands straight from a block's registers
  auto kregs = [](const Buf& B) {
    return [&B](int mb, int m) { return code_block<KB, KQ8, false, F8>(B.k[mb], m); };
  };
  auto vregs = [](const Buf& B) {
    return [&B](int nb) { return code_block<VB, VQ8, true, F8>(B.v + (nb >> 2) * VB, nb & 3); };
  };
  // the next block to load, one load ahead of the block computed; a paged
  // cache's table entry of it is read one load ahead (a scalar load), and the
  // prefetch past the last block re-reads it
  int pf = blk_lo, cb = blk_lo, pf_end = blk_lo;
  int pf_page = 0;
  auto start_loads = [&](int end) {
    pf = cb = blk_lo;
    pf_end = end;
    if (paged) pf_page = table_entry(a.sh, b, pf);
  };
  auto next_row = [&]() {
    const int64_t r0 = paged ? page_head_row(a.sh, clamp_page(a.sh, pf_page), h) : prow + (int64_t)pf * kTile;
    if (pf + 1 < pf_end) ++pf;
    if (paged) pf_page = table_entry(a.sh, b, pf);
    return r0;
  };

  int w_from = f_end;   // first block of the wave's own masked loop
  if constexpr (SHARE) {
    // ---- blocks every row of the workgroup sees whole: the four waves unpack
    // a quarter of each block's codes into a double-buffered LDS operand area
    // (one barrier per block) and all read every operand from it ----------------
    const int p_wg = base + tile * qt;   // the workgroup's first (earliest) row
    const int fs_end = max(blk_lo, min(min(blk_hi, KCH ? qend : blk_hi), (p_wg + 1) / kTile));
    w_from = fs_end;
    const int ns = fs_end - blk_lo;   // uniform over the workgroup
    if (ns > 0) {
      start_loads(fs_end);
      auto compute = [&](const SBuf& S, int buf) {
        const int blk = cb++;
        float sc[2][4];
        __builtin_amdgcn_s_setprio(1);
        group_for(blk);
        scores_q(S.kp, [&](int mb, int m) { return __builtin_bit_cast(half8, kop[buf][4 * mb + m][lane]); }, sc);
        __builtin_amdgcn_s_setprio(0);
        softmax_pv(std::false_type{}, sc, S.vp,
                   [&](int nb) { return __builtin_bit_cast(half8, vop[buf][nb][lane]); }, blk * kTile);
        if (++since_flush == kFlush) flush();
      };
      // A wave writes buffer i & 1 for block i only after the barrier of
      // block i - 1, which every wave passes after computing block i - 2, the
      // last reader of that buffer.
      SBuf s0, s1;
      load_share(s0, next_row());
      for (int k = 0; k < ns; k += 2) {
        produce(s0, 0);
        __syncthreads();
        load_share(s1, next_row());
        compute(s0, 0);
        if (k + 1 >= ns) break;
        produce(s1, 1);
        __syncthreads();
        load_share(s0, next_row());
        compute(s1, 1);
      }
    }
  } else {
    // ---- blocks every row of the wave sees whole: register pipeline, one
    // block in flight while one is computed -----------------------------------------
    const int nf = f_end - blk_lo;
    if (nf > 0) {
      start_loads(f_end);
      auto compute = [&](const Buf& B) {
        const int blk = cb++;
        float sc[2][4];
        __builtin_amdgcn_s_setprio(1);
        group_for(blk);
        scores_q(B.kp, kregs(B), sc);
        __builtin_amdgcn_s_setprio(0);
        softmax_pv(std::false_type{}, sc, B.vp, vregs(B), blk * kTile);
        if (++since_flush == kFlush) flush();
      };
      Buf b0, b1;
      load_row(b0, next_row());
      for (int k = 0; k < nf; k += 2) {
        load_row(b1, next_row());
        compute(b0);
        if (k + 1 >= nf) break;
        load_row(b0, next_row());
        compute(b1);
      }
    }
  }
  // ---- the wave's other blocks: seen in part (causal mask), or keys in the
  // unquantized tail -----------------------------------------------------------------
  for (int blk = max(w_from, blk_lo); blk < wblk_hi; ++blk) {
    Buf B;
    load_row(B, block_row(blk));
    float sc[2][4];
    if (KCH && blk >= qend) {
      scores_tail(blk, sc);
    } else {
      group_for(blk);
      scores_q(B.kp, kregs(B), sc);
    }
    softmax_pv(std::true_type{}, sc, B.vp, vregs(B), blk * kTile);
    if (++since_flush == kFlush) flush();
  }
  if (since_flush > 0) flush();

  // ---- results of the wave's rows --------------------------------------------------
  float l_sum = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) l_sum = __builtin_fmaf(l_run[c], pow2i(pe_exp<VB>(c)), l_sum);
  const float l_tot = rows_sum(l_sum) * pow2i(-pexp);
  if (q4 == 0) {
    wml[wave][n][0] = m_run;
    wml[wave][n][1] = l_tot;
  }
  __syncthreads();
  for (int idx = lane; idx < 16 * kD; idx += 64) {
    const int rr = idx / kD, c = idx % kD;
    const int rwr = 16 * wave + rr;
    const int qr = tile * qt + rwr / g;
    if (qr >= a.n_q) continue;
    const int64_t rowi = ((int64_t)b * a.n_q + qr) * a.sh.Hq + h * g + rwr % g;
    const float O = wo[wave][rr][c];
    const float M = wml[wave][rr][0], L = wml[wave][rr][1];
    if (a.splits > 1) {
      float* rec = a.partial + (rowi * a.splits + blockIdx.z) * (kD + 2);
      rec[c] = O;
      if (c == 0) {
        rec[kD] = M;
        rec[kD + 1] = L;
      }
    } else {
      const float v = L > 0.f ? O / L : 0.f;
      const int64_t oi = rowi * kD + c;
      if (a.out_dtype == KVQ_F32)
        static_cast<float*>(a.out)[oi] = v;
      else if (a.out_dtype == KVQ_F16)
        static_cast<uint16_t*>(a.out)[oi] = f2h_rn(v);
      else
        static_cast<uint16_t*>(a.out)[oi] = f2bf_rn(v);
    }
  }
}

template <int KB, bool KCH, bool KQ8, int NGK, int VB, bool VQ8, int NGV, bool F8 = false>
void launch_t(const PrefillArgs& a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((pre_codes_kernel<KB, KCH, KQ8, NGK, VB, VQ8, NGV, F8>), grid, dim3(256), 0, s, a);
}

bool asym(const DevTensor& t, int bits) {
  return (t.quant == KVQ_QUANT_ASYM_MINMAX || t.quant == KVQ_QUANT_ASYM_ABSMAX_OFFSET) && t.bits == bits;
}

}  // namespace

// The formats the kernel is compiled for (launch_prefill_codes below), with
// no sink, no RoPE and one group size for every KV head.
bool prefill_codes_supported(const kvq_config& c) {
  if (c.sink_tokens > 0 || c.rope || c.k.head_group_size || c.v.head_group_size) return false;
  if (c.n_q_heads % c.n_kv_heads != 0 || kRowsWG % (c.n_q_heads / c.n_kv_heads) != 0) return false;
  const kvq_tensor_format &k = c.k, &v = c.v;
  auto asym = [](const kvq_tensor_format& f, int bits) {
    return (f.quantizer == KVQ_QUANT_ASYM_MINMAX || f.quantizer == KVQ_QUANT_ASYM_ABSMAX_OFFSET) &&
           f.bits == bits;
  };
  auto tok = [](const kvq_tensor_format& f, int G) {
    return f.layout == KVQ_LAYOUT_PER_TOKEN && f.group_size == G;
  };
  if (k.quantizer == KVQ_QUANT_FP8_E5M2 && v.quantizer == KVQ_QUANT_FP8_E5M2) return true;
  if (asym(k, 4) && k.layout == KVQ_LAYOUT_PER_CHANNEL && c.kv_dtype == KVQ_F16 && asym(v, 4) &&
      (tok(v, 128) || tok(v, 32)))
    return true;
  if (asym(k, 3) && tok(k, 64) && asym(v, 3) && tok(v, 64)) return true;
  return k.quantizer == KVQ_QUANT_SYM_Q8_0 && tok(k, 32) && v.quantizer == KVQ_QUANT_SYM_Q8_0 &&
         tok(v, 32);
}

bool launch_prefill_codes(const PrefillArgs& a, hipStream_t s) {
  const DevTensor &k = a.k, &v = a.v;
  const int g = a.sh.g;
  if (g < 1 || kRowsWG % g != 0) return false;
  const int qt = kRowsWG / g;
  const dim3 grid((unsigned)((a.n_q + qt - 1) / qt), (unsigned)(a.sh.B * a.sh.Hkv), (unsigned)a.splits);
  if (k.quant == KVQ_QUANT_FP8_E5M2 && v.quant == KVQ_QUANT_FP8_E5M2) {
    launch_t<8, false, false, 1, 8, false, 1, true>(a, grid, s);
    return true;
  }
  if (asym(k, 4) && k.per_channel && !a.sh.kv_bf16 && asym(v, 4) && !v.per_channel) {
    if (v.ng == 1) { launch_t<4, true, false, 1, 4, false, 1>(a, grid, s); return true; }
    if (v.ng == 4) { launch_t<4, true, false, 1, 4, false, 4>(a, grid, s); return true; }
    return false;
  }
  if (asym(k, 3) && !k.per_channel && asym(v, 3) && !v.per_channel && k.ng == 2 && v.ng == 2) {
    launch_t<3, false, false, 2, 3, false, 2>(a, grid, s);
    return true;
  }
  if (k.quant == KVQ_QUANT_SYM_Q8_0 && v.quant == KVQ_QUANT_SYM_Q8_0 && k.ng == 4 && v.ng == 4) {
    launch_t<8, false, true, 4, 8, true, 4>(a, grid, s);
    return true;
  }
  return false;
}

}  // namespace kvq
