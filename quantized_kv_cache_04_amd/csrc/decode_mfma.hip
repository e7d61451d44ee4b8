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
// Grid: (splits, B * Hkv); 256 threads = 4 waves, which take the split's
// 32-token blocks in turn, one key group (per-channel keys) or one block at a
// time.  The four waves are merged in LDS; the split-K partials are merged by
// dec_combine_kernel (splitk.h).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "mfma_codes.h"
#include "splitk.h"
#include "timed_launch.h"

namespace kvq {
namespace {

constexpr int kD = kHeadDim;
constexpr float kLog2e = 1.4426950408889634f;

// F8: keys and values are FP8 E5M2 (KB = VB = 8, one group, no per-token
// parameters): codes enter as fp16 values, the per-head scales multiply the
// scores and the value sums.
template <int KB, bool KCH, bool KQ8, int NGK, int VB, bool VQ8, int NGV, bool F8 = false>
__global__ __launch_bounds__(256) void dec_mfma_kernel(DecodeArgs a) {
  static_assert(!F8 || (KB == 8 && VB == 8 && !KCH && !KQ8 && !VQ8 && NGK == 1 && NGV == 1),
                "FP8 keys and values: one shape");
  // raw dwords of one 32-token block for this lane
  constexpr int VPD = F8 ? 1 : (VQ8 ? 2 * NGV : 4 * NGV);       // value params of 4 tokens
  constexpr int KPD = (KCH || F8) ? 1 : (KQ8 ? 2 * NGK : 4 * NGK);   // key params of 4 tokens
  struct Buf {
    uint32_t k[2][KB];      // key codes, rows 16*mb + n, segment q4
    uint32_t v[2 * VB];     // value tile, this lane's 8*VB bytes
    uint32_t vp[2][VPD];    // value scale(/zero) of tokens 16*mb + 4*q4 + r
    uint32_t kp[2][KPD];    // key scale(/zero) (per-token keys)
  };
  constexpr float kLazy = 8.0f;   // log2 headroom before the running max moves
  constexpr int kFedLog2 = 15;    // fed P operand entries stay below 2^kFedLog2
  // Register pipeline: two buffers, one block in flight while one is
  // computed.  (A third buffer, where the registers allowed it, was slower
  // once the waves of a workgroup interleave their blocks: 202.9 against
  // 200.8 us on the 4-bit serving workload, with 30 more registers.)

  __shared__ float wm[4][8], wl[4][8];
  __shared__ float wo[4][8][kD];
  __shared__ float wb[4][8][NGV];   // per wave, head, value group: additive term
  __shared__ float q_lds[8][kD + 4];   // the group's queries as fp32 (zero rows for j >= g)
  // per-channel keys: the B operand of each wave's current key group,
  // [wave][head][high/low part][8-channel block] in MFMA pair order, and the
  // zero-point sums sum_c q_c z_c of its heads
  __shared__ u32x4 kb_tab[KCH ? 4 : 1][8][2][16];
  __shared__ float zb_tab[4][8];
  extern __shared__ u32x4 kp_lds[];  // per-channel keys: [4 waves][a.kp_groups][32]

  const int split = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.sh.Hkv, h = bh % a.sh.Hkv;
  // per-head group sizes: this launch serves the KV heads whose values
  // (and per-token keys) have NGV groups per token
  if (a.head_class && a.v.ngh[h] != a.head_class) return;
  // the wave index is uniform: keep it (and all block bookkeeping) scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int q4 = lane >> 4, n = lane & 15, j = n & 7;
  const float lo_mask = n >= 8 ? 1.0f : 0.0f;   // 1 in the low-part columns/rows
  const bool hi_lane = n < 8;
  const int g = a.sh.g;
  const int nctx = a.n_ctx;
  const int64_t Tcap = a.sh.Tcap;
  const DevTensor& K = a.k;
  const DevTensor& V = a.v;
  const int Gk = K.G;
  const int n_full = KCH ? (nctx / Gk) * Gk : nctx;
  const int64_t prow = (int64_t)bh * Tcap;   // token record of token 0 of (b, h)
  const float sm2 = a.sm_scale * kLog2e;

  // ---- blocks of this wave ----------------------------------------------------
  // The split's 32-token blocks [blk0, blk1) are dealt out to the four waves
  // in units of U blocks (one key group for per-channel keys, else one block):
  // unit i goes to wave i mod 4.  The waves of a workgroup then stream
  // neighbouring pieces of the same key, value and parameter arrays at any
  // one time, which the memory system serves faster than four separate runs.
  // (The host makes blocks_per_split a multiple of U.)
  const int gblk = KCH ? Gk / kTile : 1;   // blocks per key group
  const int U = gblk;
  const int blk0 = split * a.blocks_per_split;
  const int nblk_total = (nctx + kTile - 1) / kTile;
  const int blk1 = min(nblk_total, blk0 + a.blocks_per_split);
  // k-th block of this wave
  auto wblock = [&](int k) { return blk0 + (wave + 4 * (k / U)) * U + k % U; };
  // number of this wave's blocks below block e (blk0 <= e)
  auto wcount = [&](int e) {
    const int nfu = (e - blk0) / U, rem = (e - blk0) % U;
    const int cf = nfu > wave ? (nfu - wave + 3) / 4 : 0;
    return cf * U + ((nfu & 3) == wave ? rem : 0);
  };
  // blocks [blk0, qend) have quantized keys (per-channel keys: [qend, blk1)
  // read the unquantized tail); [blk0, fend) hold 32 cached tokens each
  const int qend = KCH ? max(blk0, min(blk1, n_full / kTile)) : blk1;
  const int fend = KCH ? qend : max(blk0, min(blk1, nctx / kTile));
  const int nk_full = wcount(fend);

  // query of this lane's column: head j, channels 32m + 8*q4 + e
  const bool head_ok = j < g;
  const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                       ((int64_t)b * a.sh.Hq + h * g + (head_ok ? j : 0)) * kD + 8 * q4;
  {
    // 4 elements a thread (256 threads); every load is issued before the
    // first LDS write (rows j >= g read row g - 1 and store zeros)
    const uint16_t* qg = static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.sh.Hq + h * g) * kD;
    uint16_t qe[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int idx = threadIdx.x + 256 * k, jj = idx / kD, c = idx % kD;
      qe[k] = qg[min(jj, g - 1) * kD + c];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int idx = threadIdx.x + 256 * k, jj = idx / kD, c = idx % kD;
      q_lds[jj][c] = jj < g ? elem2f(qe[k], a.sh.kv_bf16) : 0.0f;
    }
  }
  __syncthreads();
  // the wave's running output sums (true units, relative to m_run)
  for (int i = lane; i < 8 * kD; i += 64) (&wo[wave][0][0])[i] = 0.f;
  auto load_q = [&](int m, float x[8]) {
    const f32x4 u = *reinterpret_cast<const f32x4*>(&q_lds[j][32 * m + 8 * q4]);
    const f32x4 v = *reinterpret_cast<const f32x4*>(&q_lds[j][32 * m + 8 * q4 + 4]);
    x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
    x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
  };

  // ---- per-token keys: fixed B operand, scaled by 2^Eq ---------------------------
  half8 bq[4];
  float qsum[NGK];   // per key group: sm2 * sum of q (high lanes only)
  float qoff[NGK];   // q8_0: 128 * 2^-24 * sum of the fed operand (MFMA output units)
  float kq = 0.f;    // MFMA output units -> sm2 * true units
  if constexpr (!KCH) {
    float qv[4][8];
    float mx = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      load_q(m, qv[m]);
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(qv[m][e]));
    }
    mx = wave_max(mx);
    int Eq = 14 - ceil_log2(mx);
    if (Eq > 100) Eq = 100;
    // FP8 values are fed as they are, integer codes as code * 2^-24
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
      bq[m] = __builtin_bit_cast(half8, hi_lane ? hi : lo);
      if constexpr (KQ8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) so += (float)bq[m][e];
      }
      qsum[m * NGK / 4] += s;
      qoff[m * NGK / 4] += so;
    }
#pragma unroll
    for (int gi = 0; gi < NGK; ++gi) {
      qsum[gi] = hi_lane ? rows_sum(qsum[gi]) * sm2 : 0.f;
      qoff[gi] = 128.0f * 0x1p-24f * rows_sum(qoff[gi]);
    }
  }

  // ---- per-channel keys: the wave's key-group parameters, staged in LDS ----------
  // A ring of a.kp_groups of the wave's groups (every fourth group of the
  // split), refilled by the wave alone when the next group lies past it.
  const int last_grp = (KCH && nk_full > 0) ? wblock(nk_full - 1) / gblk : 0;
  const uint32_t* kgrp_base = KCH ? static_cast<const uint32_t*>(K.params) +
                                        (int64_t)bh * (Tcap / Gk) * kD
                                  : nullptr;
  u32x4* const kp_w = kp_lds + wave * a.kp_groups * 32;
  int kp_lo = 0, kp_hi = 0;    // staged groups [kp_lo, kp_hi)
  auto stage_kp = [&](int g0) {
    // groups g0, g0 + 4, ..., up to the wave's last group
    const int ng = min(a.kp_groups, (last_grp - g0) / 4 + 1);
    const u32x4* src = reinterpret_cast<const u32x4*>(kgrp_base + (int64_t)g0 * kD);
    const int n4 = ng * 32;
    for (int c0 = 0; c0 < n4; c0 += 256) {
      // unconditional loads (indices clamped into the staged groups), so that
      // all four are in flight at once
      u32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = min(c0 + u * 64 + lane, n4 - 1);
        v[u] = src[(c >> 5) * 128 + (c & 31)];   // group g0 + 4 (c / 32)
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + u * 64 + lane;
        if (c < n4) kp_w[c] = v[u];
      }
    }
    kp_lo = g0;
    kp_hi = g0 + 4 * ng;
    // LDS accesses of one wave complete in order: the reads that follow see
    // these writes from every lane
    __builtin_amdgcn_wave_barrier();
  };

  // ---- running state -----------------------------------------------------------
  f32x4 oacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Probabilities are kept in "fed units": p' = 2^(s - m_run + pexp) times
  // 2^-pe_exp of the pair's class (4-bit values: the nibble of an odd pair
  // is unpacked 4 bits up; 3-bit values: pair r carries 4^r).  The bias
  // -(m_run - pexp) - pe_exp is folded into the key products of the high
  // columns, so one exp2 of t = s - mref - pe_exp yields p'.
  constexpr int NC = kClasses<VB>;
  // Value codes are unsigned, so without care every P.V product would be
  // positive, and the matrix cores drop the parts of products that sit far
  // below the largest product of a dot product: those losses would add up
  // in one direction over thousands of tokens.  Odd pairs therefore feed
  // -P against the complemented codes cmax - c (q8_0: 255 - (q + 128)):
  // their products are p c - cmax p, the signs alternate from token to
  // token, and the fixed part cmax p goes into the exact fp32 zero term.
  constexpr float kCmax = VQ8 ? 127.0f : (float)((1 << VB) - 1);
  float m_run = -INFINITY;   // reference maximum of head j (lanes n, n + 8 agree)
  float mref = 0.f;          // bias folded into t (m_run - pexp once m_run is set)
  float thr = -INFINITY;     // rescale when t > thr (= kLazy + m_run - mref)
  float l_run[NC];           // sum of p' over this lane's tokens of each class
  float vbias[NGV][NC];      // sum p' * zero over the tokens of each class (values)
  float voff[NGV];           // q8_0: offset term of the fp16 P operand parts this lane fed
#pragma unroll
  for (int c = 0; c < NC; ++c) l_run[c] = 0.f;
#pragma unroll
  for (int gi = 0; gi < NGV; ++gi) {
#pragma unroll
    for (int c = 0; c < NC; ++c) vbias[gi][c] = 0.f;
    voff[gi] = 0.f;
  }
  // value operand scale: fed P = p * scale * 2^pexp <= 2^kFedLog2 (p <= 2^kLazy);
  // pexp changes when a block brings a scale above sbound (the accumulators
  // are then rescaled by the exact power of two)
  int pexp = 0;
  float sbound = 0.f;

  // per-channel keys: B operand of the current key group
  half8 bk[4];
  float kbias = 0.f;         // sm2 * sum_c q_c z_c (high lanes)
  float tbias[NC];           // high lanes: -mref - pe_exp(class)
  float kb2[NC];             // kbias + tbias
  auto set_bias = [&]() {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      tbias[c] = hi_lane ? -mref - (float)pe_exp<VB>(c) : 0.f;
      kb2[c] = kbias + tbias[c];
    }
  };
  set_bias();
  float kscale = 0.f;        // sm2 * 2^(24 - E)
  int grp_end = -1;          // first block after the current key group

  const uint32_t k_lane_off = (uint32_t)n * (16 * KB) + (uint32_t)q4 * (4 * KB);
  const uint32_t v_lane_off = (uint32_t)lane * (8 * VB);
  const uint32_t p_lane_tok = 4u * (uint32_t)q4;
  const bool paged = a.sh.page_table != nullptr;

  // (a block's 32 tokens are consecutive rows from its first token's row:
  // one page of a paged cache)
  // first parameter record of a block (token t0, row r0, page of a paged
  // cache): r0 * NG, or the per-head record layout
  auto prec = [&](const DevTensor& T, int NG, int64_t r0, int64_t t0, int64_t page) -> int64_t {
    if (!T.per_head) return r0 * NG;
    const int64_t tot = T.ng_pre[a.sh.Hkv], pre = T.ng_pre[h];
    return paged ? (int64_t)kTile * (page * tot + pre) : a.sh.Tcap * ((int64_t)b * tot + pre) + t0 * NG;
  };
  auto load_row = [&](Buf& B, int64_t r0, int64_t t0, int64_t page) {
    const uint8_t* kcodes = K.codes + r0 * (4 * KB * 4);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      load_dw<KB>(kcodes + (16 * mb) * (16 * KB) + k_lane_off, B.k[mb]);
      const uint32_t tok = 16 * mb + p_lane_tok;
      if constexpr (F8) {
        B.vp[mb][0] = 0u;
        B.kp[mb][0] = 0u;
      } else {
        const uint8_t* vprm = static_cast<const uint8_t*>(V.params) +
                              prec(V, NGV, r0, t0, page) * (VQ8 ? 2 : 4);
        load_dw<VPD>(vprm + tok * (NGV * (VQ8 ? 2 : 4)), B.vp[mb]);
        if constexpr (!KCH) {
          const uint8_t* kprm = static_cast<const uint8_t*>(K.params) +
                                prec(K, NGK, r0, t0, page) * (KQ8 ? 2 : 4);
          load_dw<KPD>(kprm + tok * (NGK * (KQ8 ? 2 : 4)), B.kp[mb]);
        }
      }
    }
    load_dw<2 * VB>(V.codes + r0 * (4 * VB * 4) + v_lane_off, B.v);
  };
  auto load = [&](Buf& B, int blk) {
    const int64_t page = paged ? page_of(a.sh, b, blk) : 0;
    load_row(B, paged ? page_head_row(a.sh, page, h) : prow + (int64_t)blk * kTile,
             (int64_t)blk * kTile, page);
  };

  // per-channel keys: B operand and zero-point term of key group ``grp``
  // The g * 16 blocks of 8 channels of the group's heads are shared out over
  // the lanes (lane L takes blocks L and L + 64): each block's q * scale
  // products are split into fp16 high/low parts in pair order and written
  // to the wave's table, from which every lane reads its own operand.
  auto key_group = [&](int grp) {
    if (grp >= kp_hi) stage_kp(grp);   // wave-uniform
    const u32x4* prm4 = kp_w + ((grp - kp_lo) >> 2) * 32;
    const int nblocks = g * 16;
    float xs[2][8];
    float zb[2] = {0.f, 0.f};
    float mx = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int bi = lane + 64 * u;
#pragma unroll
      for (int e = 0; e < 8; ++e) xs[u][e] = 0.f;
      if (bi < nblocks) {
        const int hd = bi >> 4, cb = bi & 15;
        const f32x4 qa = *reinterpret_cast<const f32x4*>(&q_lds[hd][8 * cb]);
        const f32x4 qb = *reinterpret_cast<const f32x4*>(&q_lds[hd][8 * cb + 4]);
        const float qv[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
        const u32x4 p0 = prm4[2 * cb], p1 = prm4[2 * cb + 1];
        const uint32_t pz[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const half2v sz = __builtin_bit_cast(half2v, pz[e]);   // (scale, zero)
          xs[u][e] = __builtin_fmaf(qv[e], (float)sz[0], 0.f);
          mx = fmaxf(mx, fabsf(xs[u][e]));
          zb[u] = __builtin_fmaf(qv[e], (float)sz[1], zb[u]);
        }
      }
    }
    mx = wave_max(mx);
    int E = 14 - ceil_log2(mx);
    if (E > 100) E = 100;
    kscale = pow2i(24 - E > 126 ? 126 : 24 - E) * sm2;
    const float s2 = pow2i(E);
    // zero-point sums: the 16 lanes of a row hold the 16 blocks of one head
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float z = zb[u];
      z += dpp_f<0x128>(z);
      z += dpp_f<0x124>(z);
      z += dpp_f<0x122>(z);
      z += dpp_f<0x121>(z);
      const int bi = lane + 64 * u;
      if (bi < nblocks) {
        const int hd = bi >> 4, cb = bi & 15;
        if (cb == 0) zb_tab[wave][hd] = z;
        u32x4 hi, lo;
        pair_operand_fixed<KB>(xs[u], s2, hi, lo);
        kb_tab[wave][hd][0][cb] = hi;
        kb_tab[wave][hd][1][cb] = lo;
      }
    }
    // LDS accesses of one wave complete in order: the reads see the table
    __builtin_amdgcn_wave_barrier();
    const int hl = n >> 3;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      bk[m] = head_ok ? __builtin_bit_cast(half8, kb_tab[wave][j][hl][4 * m + q4])
                      : as_h8(0u, 0u, 0u, 0u);
    kbias = (hi_lane && head_ok) ? zb_tab[wave][j] * sm2 : 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) kb2[c] = kbias + tbias[c];
  };

  // Softmax and P.V for one block.  sc: per-column partial scores (the bias
  // tbias sits in the high columns), so that the sum of a lane's high and
  // low columns is t = s - mref - pe_exp.  RAGGED (an
  // integral_constant) is true only for a block with fewer than 32 cached
  // tokens: the others skip the masking.
  auto softmax_pv = [&](auto ragged, float sc[2][4], const uint32_t* vl,
                        const uint32_t (*vp_in)[VPD], int valid) {
    constexpr bool RAGGED = decltype(ragged)::value;
    auto tok_ok = [&](int mb, int r) { return !RAGGED || 16 * mb + 4 * q4 + r < valid; };
    float t[2][4];
    float bmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = sc[mb][r] + dpp_f<0x128>(sc[mb][r]);
        t[mb][r] = tok_ok(mb, r) ? x : -INFINITY;
        bmax = fmaxf(bmax, t[mb][r]);
      }
    if (__any(bmax > thr)) {
      // move the reference maximum (wave-uniform branch, rare after warm-up)
      const float m_new = fmaxf(m_run, rows_max(bmax) + mref);
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int c = 0; c < NC; ++c) l_run[c] *= alpha;
#pragma unroll
      for (int gi = 0; gi < NGV; ++gi) {
#pragma unroll
        for (int c = 0; c < NC; ++c) vbias[gi][c] *= alpha;
        voff[gi] *= alpha;
      }
      // accumulator row r of this lane belongs to head (4 q4 + r) & 7, whose
      // factor sits in lane (4 q4 + r) & 7 (a lane shuffle: a per-lane pick
      // from an array would go through scratch memory)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float f = __shfl(alpha, 4 * (q4 & 1) + r, 64);
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) oacc[nb][r] *= f;
        if (q4 < 2) {
#pragma unroll
          for (int nb = 0; nb < 8; ++nb) wo[wave][4 * q4 + r][16 * nb + n] *= f;
        }
      }
      m_run = m_new;
      const float mref_new = m_run - (float)pexp;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) t[mb][r] += mref - mref_new;
      mref = mref_new;
      thr = kLazy + (float)pexp;
      set_bias();
    }

    // value parameters of this lane's 8 tokens (zeroed past the context)
    uint32_t vp[2][VPD];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int w = 0; w < VPD; ++w) {
        uint32_t d = vp_in[mb][w];
        if constexpr (RAGGED) {
          if constexpr (VQ8) {   // two entries (token r = entry / NGV) per dword
            const uint32_t lo = tok_ok(mb, (2 * w) / NGV) ? 0x0000ffffu : 0u;
            const uint32_t hi = tok_ok(mb, (2 * w + 1) / NGV) ? 0xffff0000u : 0u;
            d &= lo | hi;
          } else {               // scale | zero << 16 of token r = w / NGV
            d = tok_ok(mb, w / NGV) ? d : 0u;
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
      const float sm = rows_max(smax);         // same tokens in every column
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
      thr = kLazy + (float)pexp;
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
    // P operand: pair r = tokens (4 q4 + r, 16 + 4 q4 + r), p' * scale split
    // into fp16 high / low parts; zero points enter through vbias
    half8 pa[NGV];
#pragma unroll
    for (int gi = 0; gi < NGV; ++gi) {
      uint32_t o[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          if constexpr (F8) {
            x[mb] = pr[mb][r];   // signed values: no complement, no scale
          } else if constexpr (VQ8) {
            const int idx = r * NGV + gi;
            const half2v h = __builtin_bit_cast(half2v, vp[mb][idx >> 1]);
            const float sc_h = (float)h[idx & 1];
            x[mb] = __builtin_fmaf(pr[mb][r], (r & 1) ? -sc_h : sc_h, 0.f);
          } else {
            const half2v h = __builtin_bit_cast(half2v, vp[mb][r * NGV + gi]);
            const float sc_h = (float)h[0];
            x[mb] = __builtin_fmaf(pr[mb][r], (r & 1) ? -sc_h : sc_h, 0.f);
            // odd pairs: + cmax p' scale (x holds -p' scale there)
            const int cl = pe_class<VB>(r);
            const float vb = (r & 1) ? __builtin_fmaf(-kCmax, x[mb], vbias[gi][cl]) : vbias[gi][cl];
            vbias[gi][cl] = __builtin_fmaf(pr[mb][r], (float)h[1], vb);
          }
        }
        o[r] = hilo_split(x[0], x[1], lo_mask);
        if constexpr (VQ8) {   // the offset term must cancel what was fed, not x
          // even pairs: P (q + 128) -> -128 P; odd: -P (127 - q) -> +127 P
          const half2v f = __builtin_bit_cast(half2v, o[r]);
          voff[gi] = __builtin_fmaf((float)f[0] + (float)f[1], (r & 1) ? -kCmax : -128.0f, voff[gi]);
        }
      }
      pa[gi] = as_h8(o[0], o[1], o[2], o[3]);
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int nbk = 0; nbk < 8; ++nbk) {
      const uint32_t* seg = vl + (nbk >> 2) * VB;
      oacc[nbk] = mfma16(pa[nbk * NGV / 8], code_block<VB, VQ8, true, F8>(seg, nbk & 3), oacc[nbk]);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Move the accumulators into the wave's LDS sums and restart them: the
  // high + low rows times 2^24 (codes are fed as code * 2^-24) plus the zero
  // or offset term, in true units.  The code products are much larger than
  // the attention output that remains once the zero term is added; settling
  // that difference every kFlush blocks bounds the size of the fp32 sums
  // the matrix cores keep adding into.
  constexpr int kFlush = 16;
  int since_flush = 0;
  // accumulator units -> true units: integer codes were fed as code * 2^-24,
  // FP8 values as they are (times the per-head value scale)
  const float ofac = F8 ? fp8_scale(V, h) : 0x1p24f;
  auto flush = [&]() {
    const float vscale = pow2i(-pexp);
    float vb_row[NGV][4];
#pragma unroll
    for (int gi = 0; gi < NGV; ++gi) {
      float vb = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) vb = __builtin_fmaf(vbias[gi][c], pow2i(pe_exp<VB>(c)), vb);
      const float tot = VQ8 ? rows_sum(voff[gi] + dpp_f<0x128>(voff[gi])) : rows_sum(vb);
#pragma unroll
      for (int r = 0; r < 4; ++r) vb_row[gi][r] = __shfl(tot, 4 * (q4 & 1) + r, 64);
    }
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) oacc[nb][r] += swap_halves(oacc[nb][r]);
    if (q4 < 2) {       // lanes q4 = 0, 1 now hold heads 4 q4 + r
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
          wo[wave][4 * q4 + r][16 * nb + n] +=
              (oacc[nb][r] * ofac + vb_row[nb * NGV / 8][r]) * vscale;
    }
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

  // one block with quantized keys
  auto compute = [&](auto ragged, const Buf& B, int blk) {
    const int valid = nctx - blk * kTile;
    float sc[2][4];
    // Waves in their matrix-core phases (key products here, value products
    // at the end of softmax_pv) run at raised priority, so that their
    // back-to-back products issue while the other wave of the SIMD does its
    // vector work (about 1 % on the 4-bit serving workload).
    __builtin_amdgcn_s_setprio(1);
    if constexpr (KCH) {
      if (blk >= grp_end) {     // wave-uniform: once per key group
        const int grp = blk / gblk;
        grp_end = (grp + 1) * gblk;
        key_group(grp);
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m) c = mfma16(seg_block<KB, KQ8>(B.k[mb], m), bk[m], c);
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[mb][r] = c[r] * kscale + kb2[pe_class<VB>(r)];
      }
    } else {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        // score = kq * sum_g scale_g * dot_g + sum_g zero_g * qsum_g + bias:
        // the fp16 scale and zero enter v_fma_mix straight from their halves
        float sd[4], zq[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) { sd[r] = 0.f; zq[r] = tbias[pe_class<VB>(r)]; }
#pragma unroll
        for (int gi = 0; gi < NGK; ++gi) {
          f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int m = gi * 4 / NGK; m < (gi + 1) * 4 / NGK; ++m)
            c = mfma16(code_block<KB, KQ8, false, F8>(B.k[mb], m), bq[m], c);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t* d = B.kp[mb];
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
    __builtin_amdgcn_s_setprio(0);
    softmax_pv(ragged, sc, B.v, B.vp, valid);
    if (++since_flush == kFlush) flush();
  };

  // ---- hot loop: register pipeline over the wave's blocks with 32 cached
  // tokens and quantized keys; one block is in flight while one is computed.
  // (Prefetches past the end re-read the last block.)
  if (nk_full > 0) {
    // iterator over wblock(0), wblock(1), ... (scalar): within a unit the
    // next block follows, after a unit's last block come 3 units of the
    // other waves
    struct BlockIter {
      int blk, u, k;
    };
    auto advance = [&](BlockIter& it) {
      if (it.k + 1 >= nk_full) return;   // stay on the last block
      ++it.k;
      if (++it.u == U) {
        it.u = 0;
        it.blk += 1 + 3 * U;
      } else {
        ++it.blk;
      }
    };
    BlockIter pf{wblock(0), 0, 0}, cb{wblock(0), 0, 0};
    // a paged cache's table entry of the next block to load is read one
    // load ahead (a scalar load), and used only when that block's loads
    // are issued
    int pf_page = paged ? table_entry(a.sh, b, pf.blk) : 0;
    auto next_load = [&](Buf& B) {
      const int64_t page = paged ? clamp_page(a.sh, pf_page) : 0;
      const int64_t t0 = (int64_t)pf.blk * kTile;
      const int64_t r = paged ? page_head_row(a.sh, page, h) : prow + t0;
      advance(pf);
      if (paged) pf_page = table_entry(a.sh, b, pf.blk);
      load_row(B, r, t0, page);
    };
    auto next_comp = [&]() { const int b = cb.blk; advance(cb); return b; };
    Buf b0, b1;
    next_load(b0);
    for (int k = 0; k < nk_full; k += 2) {
      next_load(b1);
      compute(std::false_type{}, b0, next_comp());
      if (k + 1 >= nk_full) break;
      next_load(b0);
      compute(std::false_type{}, b1, next_comp());
    }
  }
  // per-token keys: the ragged last block of the context, taken by the wave
  // its unit falls to
  if constexpr (!KCH) {
    if (blk1 > fend && ((fend - blk0) & 3) == wave) {
      Buf br;
      load(br, fend);
      compute(std::true_type{}, br, fend);
    }
  }

  // ---- per-channel keys: blocks of the unquantized tail ---------------------------
  if constexpr (KCH) {
    for (int blk = qend + wave; blk < blk1; blk += 4) {   // shared out over the waves
      const int t0 = blk * kTile;
      // 32 consecutive rows of the tail ring (its size is a multiple of 32)
      const uint16_t* tail = K.tail + ((int64_t)bh * K.tail_rows + t0 % K.tail_rows) * kD;
      half8 bt[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(qp + 32 * m);
        const bool z = !hi_lane || !head_ok;
        bt[m] = as_h8(z ? 0u : v.x, z ? 0u : v.y, z ? 0u : v.z, z ? 0u : v.w);
      }
      float sc[2][4];
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
      Buf B;
      load(B, blk);
      softmax_pv(std::true_type{}, sc, B.v, B.vp, nctx - t0);
      if (++since_flush == kFlush) flush();
    }
  }

  // ---- wave result -> LDS (true units) ------------------------------------------
  // (nothing to move when the last block ended a flush period)
  if (since_flush > 0) flush();
  float l_sum = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) l_sum = __builtin_fmaf(l_run[c], pow2i(pe_exp<VB>(c)), l_sum);
  const float l_tot = rows_sum(l_sum) * pow2i(-pexp);
  if (q4 == 0 && n < 8) {
    wm[wave][j] = m_run;
    wl[wave][j] = l_tot;
#pragma unroll
    for (int gi = 0; gi < NGV; ++gi) wb[wave][j][gi] = 0.f;   // the zero terms are in wo
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
    if (a.direct) {
      // the only partial state (one split, no sink): normalize and write the output
      store_out(a, ((int64_t)b * a.sh.Hq + h * g + jj) * kD + c, L > 0.f ? O / L : 0.f);
    } else {
      float* rec = partial_rec(a, b, h * g + jj, split);
      rec[c] = O;
      if (c == 0) { rec[kD] = M; rec[kD + 1] = L; }
    }
  }
}

// ---- dispatch ---------------------------------------------------------------------
template <int KB, bool KCH, bool KQ8, int NGK, int VB, bool VQ8, int NGV, bool F8 = false>
void launch_t(const DecodeArgs& a, hipStream_t s) {
  const size_t lds = KCH ? (size_t)4 * a.kp_groups * 32 * sizeof(u32x4) : 0;
  launch_timed(dec_mfma_kernel<KB, KCH, KQ8, NGK, VB, VQ8, NGV, F8>, dim3(a.splits, a.sh.B * a.sh.Hkv),
               dim3(256), (uint32_t)lds, s, a);
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

// group size of KV head h of a per-token format
int head_group(const kvq_tensor_format& f, int h) {
  return f.head_group_size ? f.head_group_size[h] : f.group_size;
}

bool mfma_config_supported(const kvq_config& c) {
  if (c.k.quantizer == KVQ_QUANT_FP8_E5M2 && c.v.quantizer == KVQ_QUANT_FP8_E5M2)
    return !c.rope && c.n_q_heads / c.n_kv_heads <= 8;
  if (!uniform(c.k) || !uniform(c.v) || c.rope) return false;
  if (c.n_q_heads / c.n_kv_heads > 8) return false;
  if (c.k.layout == KVQ_LAYOUT_PER_CHANNEL) return c.kv_dtype == KVQ_F16;
  // per-token keys: each KV head's key and value groups of one size
  for (int h = 0; h < c.n_kv_heads; ++h)
    if (head_group(c.k, h) != head_group(c.v, h)) return false;
  return true;
}

hipError_t launch_decode_mfma(const DecodeArgs& a_in, hipStream_t s) {
  DecodeArgs a = a_in;
  a.kp_groups = 0;
  if (a.k.per_channel) {
    // key groups one wave can touch (its blocks plus one partial group), up
    // to a ring of kMaxKpGroups per wave (32 KB of LDS for the 4 waves)
    constexpr int kMaxKpGroups = 16;
    const int per_wave = (a.blocks_per_split + 3) / 4;
    const int gblk = a.k.G / kTile;
    const int groups = (per_wave + gblk - 1) / gblk + 1;
    a.kp_groups = groups < kMaxKpGroups ? groups : kMaxKpGroups;
  }
  if (a.v.per_head || a.k.per_head) {
    // per-head group sizes: one launch per number of groups per token, over
    // the KV heads that have it (the other workgroups return at once)
    bool seen[5] = {false, false, false, false, false};
    for (int h = 0; h < a.sh.Hkv; ++h) seen[a.v.per_head ? a.v.ngh[h] : a.v.ng] = true;
    // launches: one per class (one in all for uniform values); the profiling
    // events go to the first and the last
    int last = 0, first = 0;
    for (int c : {4, 2, 1}) if (seen[c]) first = c;
    for (int c : {1, 2, 4}) if (seen[c]) last = c;
    if (!a.v.per_head) last = first;
    for (int c : {1, 2, 4}) {
      if (!seen[c]) continue;
      DecodeArgs ac = a;
      ac.ev_start = c == first ? a.ev_start : nullptr;
      ac.ev_stop = c == last ? a.ev_stop : nullptr;
      ac.head_class = c;
      ac.v.ng = c;
      if (!ac.k.per_channel) ac.k.ng = c;
      if (!ac.v.per_head) {   // uniform values with per-head keys: one class
        ac.head_class = 0;
      }
      bool ok = false;
      if (ac.k.per_channel) {
        switch (ac.k.bits) {
          case 3: ok = launch_kch<3>(ac, s); break;
          case 4: ok = launch_kch<4>(ac, s); break;
          case 8: ok = launch_kch<8>(ac, s); break;
        }
      } else if (ac.k.quant == KVQ_QUANT_SYM_Q8_0) {
        ok = launch_ktok<8, true>(ac, s);
      } else {
        switch (ac.k.bits) {
          case 3: ok = launch_ktok<3, false>(ac, s); break;
          case 4: ok = launch_ktok<4, false>(ac, s); break;
          case 8: ok = launch_ktok<8, false>(ac, s); break;
        }
      }
      if (!ok) return hipErrorNotSupported;
      if (!ac.head_class) break;
    }
    return hipGetLastError();
  }
  bool ok = false;
  if (a.k.quant == KVQ_QUANT_FP8_E5M2 && a.v.quant == KVQ_QUANT_FP8_E5M2) {
    launch_t<8, false, false, 1, 8, false, 1, true>(a, s);
    ok = true;
  } else if (a.k.per_channel) {
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
