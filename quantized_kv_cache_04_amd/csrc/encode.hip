// Encode kernels of libkvq: quantize appended K/V rows into the packed cache.
//
// Compiled with -ffp-contract=off: every step is one IEEE float32 operation
// with round-to-nearest-even -- (x - zero) then / scale, scale and zero
// rounded to fp16 before any code is computed -- so the packed bytes are
// reproducible bit for bit.
//
// Quantizers (include/kvq.h): group-wise asymmetric min/max (Survey page,
// section 2.4; Memory-killer page, section 2.3), TurboQuant's absmax scale
// with a min offset (TurboQuant page, section 3.1), q8_0 (NIAH page, section
// 1.2), and the KVQuant codebook with dense-and-sparse outliers (KVQuant
// page, section 2.2).  Only appended rows are encoded (NIAH page, sections
// 1.1 and 2.2; KVQuant page, section 3.4).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "splitk.h"

namespace kvq {
namespace {

constexpr int kD = kHeadDim;

// Codebook index of x: the number of midpoints between consecutive centroids
// that lie below x (nearest centroid, ties to the lower index).
// (The 16 centroids of a channel are 32 contiguous, 16-byte aligned bytes:
// two 16-byte loads.)
__device__ __forceinline__ uint32_t cb_code(const uint16_t* cb, float x) {
  const uint4 a = reinterpret_cast<const uint4*>(cb)[0], b = reinterpret_cast<const uint4*>(cb)[1];
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  float c[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    c[2 * i] = h2f((uint16_t)(w[i] & 0xffffu));
    c[2 * i + 1] = h2f((uint16_t)(w[i] >> 16));
  }
  uint32_t n = 0;
#pragma unroll
  for (int i = 0; i < 15; ++i) n += x > (c[i] + c[i + 1]) * 0.5f;
  return n;
}

// Quantize channels c0 .. c0 + 7 (c0 = 8 j8) of one row whose 128 channels
// are held by 16 lanes (j8 = lane % 16; the row segment is lane / 16).  For
// per-token uniform formats the group statistics are reduced over the G/8
// lanes of the group.  Writes the group's parameters (first lane of each
// group) at ``prm_row`` unless it is null, and returns the 8 codes as bytes
// (two's complement for q8_0).  ``dq`` (optional) receives the values the
// codes stand for, as the decode kernels reconstruct them.
__device__ __forceinline__ uint2 encode8(const DevTensor& t, int h, int j8, const float x[8],
                                         void* prm_row, float* dq = nullptr) {
  const int c0 = 8 * j8;
  uint32_t q[8];
  if (t.quant == KVQ_QUANT_CODEBOOK) {
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = cb_code(t.codebook + ((int64_t)h * kD + c0 + e) * 16, x[e]);
    if (dq) {
#pragma unroll
      for (int e = 0; e < 8; ++e) dq[e] = h2f(t.codebook[((int64_t)h * kD + c0 + e) * 16 + q[e]]);
    }
  } else if (t.quant == KVQ_QUANT_FP8_E5M2) {
    // one float32 division per element, as the format defines it
    const float s = fp8_scale(t, h);
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = f_to_e5m2(x[e] / s);
    if (dq) {
#pragma unroll
      for (int e = 0; e < 8; ++e) dq[e] = e5m2_to_f(q[e]) * s;
    }
  } else {
    float lo = x[0], hi = x[0], am = fabsf(x[0]);
#pragma unroll
    for (int e = 1; e < 8; ++e) {
      lo = fminf(lo, x[e]);
      hi = fmaxf(hi, x[e]);
      am = fmaxf(am, fabsf(x[e]));
    }
    const int gl = t.G >> 3;   // lanes of a group
    for (int off = 1; off < gl; off <<= 1) {
      lo = fminf(lo, __shfl_xor(lo, off, 64));
      hi = fmaxf(hi, __shfl_xor(hi, off, 64));
      am = fmaxf(am, __shfl_xor(am, off, 64));
    }
    const bool writer = prm_row != nullptr && (j8 & (gl - 1)) == 0;
    const int grp = c0 / t.G;
    if (t.quant == KVQ_QUANT_SYM_Q8_0) {
      const uint16_t sh = f2h_rn(am / 127.0f);
      const float s = h2f(sh);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = s == 0.0f ? 0.0f : rintf(x[e] / s);
        v = fminf(fmaxf(v, -128.0f), 127.0f);
        q[e] = (uint32_t)((int)v & 0xff);
        if (dq) dq[e] = v * s;
      }
      if (writer) static_cast<uint16_t*>(prm_row)[grp] = sh;
    } else {
      const float qmax = (float)((1 << t.bits) - 1);
      uint16_t sh;
      if (t.quant == KVQ_QUANT_ASYM_MINMAX)
        sh = f2h_rn((hi - lo) / qmax);
      else
        sh = f2h_rn(am / (float)((1 << (t.bits - 1)) - 1));
      const uint16_t zh = f2h_rn(lo);
      const float s = h2f(sh), z = h2f(zh);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = s == 0.0f ? 0.0f : rintf((x[e] - z) / s);
        q[e] = (uint32_t)fminf(fmaxf(v, 0.0f), qmax);
        if (dq) dq[e] = (float)q[e] * s + z;
      }
      if (writer) static_cast<uint32_t*>(prm_row)[grp] = (uint32_t)sh | ((uint32_t)zh << 16);
    }
  }
  return uint2{q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24),
               q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24)};
}

__device__ __forceinline__ void unpack8(uint4 v, int is_bf16, float x[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = elem2f((uint16_t)(w[e >> 1] >> (16 * (e & 1))), is_bf16);
}

// Dword W of a key row, assembled from the row's codes in LDS.
__device__ __forceinline__ uint32_t k_row_dword(const uint8_t* rowc, int bits, int W) {
  const int q = W / bits, j = W % bits;
  uint32_t dw = 0;
  seg_dword_fields(bits, j, [&](int u, int sh, int, int field) {
    const int c = 32 * (u >> 3) + 8 * q + (u & 7);
    dw |= field_value(rowc[c], field) << sh;
  });
  return dw;
}

// ---- per-token rows: keys (K-row layout) and raw rows for NONE --------------
// 16 lanes per row (b, new token, kv head), 8 channels a lane; 16 rows per
// 256-thread block.
__global__ __launch_bounds__(256) void enc_rows_kernel(DevShape sh, DevTensor t, const void* x_new,
                                                       int64_t n_ctx, int n_new) {
  __shared__ uint8_t rowc[16][kD];
  const int tid = threadIdx.x, rl = tid >> 4, j8 = tid & 15;
  const int64_t nrows = (int64_t)sh.B * n_new * sh.Hkv;
  auto row_of = [&](int64_t r, int& h) -> int64_t {   // cache row of block row r
    h = (int)(r % sh.Hkv);
    const int64_t bt = r / sh.Hkv;
    const int b = (int)(bt / n_new);
    return tok_row(sh, b, h, n_ctx + bt % n_new);
  };
  const int64_t r = (int64_t)blockIdx.x * 16 + rl;
  const bool active = r < nrows;
  uint4 v = uint4{0u, 0u, 0u, 0u};
  int h = 0;
  int64_t row = 0;
  if (active) {
    row = row_of(r, h);
    const int64_t bt = r / sh.Hkv;
    const int64_t rin = ((int64_t)(bt / n_new) * sh.in_tok + sh.in_off + bt % n_new) * sh.Hkv + h;
    v = reinterpret_cast<const uint4*>(x_new)[rin * (kD / 8) + j8];
  }
  if (t.quant == KVQ_QUANT_NONE) {
    if (active) reinterpret_cast<uint4*>(t.codes)[row * (kD / 8) + j8] = v;
    return;
  }
  float x[8];
  unpack8(v, sh.kv_bf16, x);
  void* prm = nullptr;
  if (active && t.params) {
    const int64_t bt = r / sh.Hkv;
    prm = static_cast<uint8_t*>(t.params) +
          prm_rec(t, sh, (int)(bt / n_new), h, n_ctx + bt % n_new) *
              (t.quant == KVQ_QUANT_SYM_Q8_0 ? 2 : 4);
  }
  const uint2 cq = encode8(head_view(t, h), h, j8, x, prm);
  *reinterpret_cast<uint2*>(&rowc[rl][8 * j8]) = cq;
  __syncthreads();
  const int dw_row = 4 * t.bits;
  for (int idx = tid; idx < 16 * dw_row; idx += 256) {
    const int r2 = idx / dw_row, W = idx % dw_row;
    const int64_t rr = (int64_t)blockIdx.x * 16 + r2;
    if (rr >= nrows) continue;
    int h2;
    const int64_t row2 = row_of(rr, h2);
    reinterpret_cast<uint32_t*>(t.codes + row2 * t.row_bytes)[W] = k_row_dword(rowc[r2], t.bits, W);
  }
}

// ---- value tiles --------------------------------------------------------------
// One block per (tile, b*Hkv + h) touched by the append.  New tokens of the
// tile are encoded into LDS, then every dword of the tile that holds a new
// code is rewritten; bits of older tokens are preserved.
// KeyTail (optional): keys of a per-channel key cache whose new tokens all
// go to the unquantized tail in this append (no key group completes).  The
// first block of each (b, h) then also copies those key rows to the tail,
// which saves the separate tail launch in the one-token serving step.
struct KeyTail {
  uint32_t* tail;      // the key tail ring, [B*Hkv][R][kD] 16-bit elements
  const void* k_new;   // the appended keys
  int R;               // ring rows per (b, h): token p sits at row p mod R
  int64_t p_first;     // first token position written to the tail
  int n_rows;          // tail rows written per (b, h); 0: no keys here
};

__global__ __launch_bounds__(256) void enc_vtile_kernel(DevShape sh, DevTensor t, const void* x_new,
                                                        int64_t n_ctx, int n_new, int64_t tile0,
                                                        KeyTail kt) {
  __shared__ uint8_t codes[kTile][kD];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int bh = blockIdx.y;
  const int b = bh / sh.Hkv, h = bh % sh.Hkv;
  if (kt.n_rows > 0 && blockIdx.x == 0) {
    // one thread per dword (two elements) of a tail row, as enc_kchan_tail_kernel
    for (int idx = threadIdx.x; idx < kt.n_rows * (kD / 2); idx += 256) {
      const int64_t p = kt.p_first + idx / (kD / 2);
      const int w = idx % (kD / 2);
      const int64_t rin = ((int64_t)b * sh.in_tok + sh.in_off + (p - n_ctx)) * sh.Hkv + h;
      kt.tail[((int64_t)bh * kt.R + p % kt.R) * (kD / 2) + w] =
          static_cast<const uint32_t*>(kt.k_new)[rin * (kD / 2) + w];
    }
  }
  const int64_t tile = tile0 + blockIdx.x;
  const int64_t t_begin = tile * kTile;
  const int64_t lo_new = n_ctx, hi_new = n_ctx + n_new;
  // 16 lanes per token, 8 channels a lane: the wave takes tokens
  // tau = 8 wave + 4 p + (lane / 16), p = 0, 1; both loads first
  const int sub = lane >> 4, j8 = lane & 15;
  uint4 xin[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int64_t tpos = t_begin + 8 * wave + 4 * p + sub;
    xin[p] = uint4{0u, 0u, 0u, 0u};
    if (tpos >= lo_new && tpos < hi_new) {
      const int64_t rin = (((int64_t)b * sh.in_tok + sh.in_off + (tpos - n_ctx)) * sh.Hkv + h);
      xin[p] = reinterpret_cast<const uint4*>(x_new)[rin * (kD / 8) + j8];
    }
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int tau = 8 * wave + 4 * p + sub;
    const int64_t tpos = t_begin + tau;
    const bool fresh = tpos >= lo_new && tpos < hi_new;
    float x[8];
    unpack8(xin[p], sh.kv_bf16, x);
    void* prm = nullptr;
    if (fresh && t.params)
      prm = static_cast<uint8_t*>(t.params) +
            prm_rec(t, sh, b, h, tpos) * (t.quant == KVQ_QUANT_SYM_Q8_0 ? 2 : 4);
    const uint2 cq = encode8(head_view(t, h), h, j8, x, prm);
    if (fresh) *reinterpret_cast<uint2*>(&codes[tau][8 * j8]) = cq;
  }
  __syncthreads();
  const int bits = t.bits;
  uint32_t* tile_dw = reinterpret_cast<uint32_t*>(t.codes + tok_row(sh, b, h, t_begin) * t.row_bytes);
  if (t.quant == KVQ_QUANT_CODEBOOK) {
    // pair tiles: byte 32 l + tau = code(tau, l) | code(tau, l + 64) << 4
    for (int W = threadIdx.x; W < 512; W += 256) {
      const int l = W >> 3, j = W & 7;
      uint32_t nb = 0, nm = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int tau = 4 * j + k;
        const int64_t tpos = t_begin + tau;
        if (tpos >= lo_new && tpos < hi_new) {
          nb |= (uint32_t)(codes[tau][l] | (codes[tau][l + 64] << 4)) << (8 * k);
          nm |= 0xffu << (8 * k);
        }
      }
      if (nm == 0) continue;
      if (nm != 0xffffffffu) nb |= tile_dw[W] & ~nm;
      tile_dw[W] = nb;
    }
    return;
  }
  for (int W = threadIdx.x; W < 128 * bits; W += 256) {
    const int L = W / (2 * bits), s = (W / bits) & 1, j = W % bits;
    const int q = L >> 4, i = L & 15;
    uint32_t nb = 0, nm = 0;
    seg_dword_fields(bits, j, [&](int u, int shf, int wd, int field) {
      const int m = u >> 3, e = u & 7;
      const int tau = e < 4 ? 4 * q + e : 16 + 4 * q + (e - 4);
      const int c = 16 * (4 * s + m) + i;
      const int64_t tpos = t_begin + tau;
      if (tpos >= lo_new && tpos < hi_new) {
        nb |= field_value(codes[tau][c], field) << shf;
        nm |= ((1u << wd) - 1u) << shf;
      }
    });
    if (nm == 0) continue;
    if (nm != 0xffffffffu) nb |= tile_dw[W] & ~nm;
    tile_dw[W] = nb;
  }
}

// ---- one serving step: the new token, appended and merged ------------------------
// One workgroup per (sequence b, KV head h), run after the decode kernels
// have streamed the tokens cached before the step into split partial
// states.  It encodes the step's token (position pos of the quantized
// cache) exactly as an append of it would -- wave 0 the value, wave 1 the
// key, 16 lanes of 8 channels each -- and merges, for the g query heads of
// h, the partial states with the new token's own term: score q_j . k (k and
// v as the codes just written stand for them), l = 1, o = v.  That is the
// log-sum-exp merge of the combine kernel with one more state, so the
// result is the decode over the cache that holds the token.
// 128 threads (one channel each) per query head, up to 8 heads at once
// (more heads take further passes).  Everything that does not wait for the
// new token -- the query channel, up to kU split states, the value-tile
// dwords the token shares with older tokens -- is loaded first, so that the
// step waits for memory about once.
struct NewToken {
  const void* k_new;   // [B][1][Hkv][d] of the cache dtype
  const void* v_new;
  int64_t pos;         // its position in the quantized cache
};

constexpr int kAppendPassHeads = 8;

__global__ __launch_bounds__(128 * kAppendPassHeads) void dec_append_merge_kernel(DecodeArgs a,
                                                                                  NewToken nt) {
  __shared__ uint8_t kcode[kD], vcode[kD];
  __shared__ float kdq[kD], vdq[kD];
  __shared__ float red[2 * kAppendPassHeads];
  const int tid = threadIdx.x, nthr = blockDim.x, wave = tid >> 6, lane = tid & 63;
  const DevShape& sh = a.sh;
  const int bh = blockIdx.x, b = bh / sh.Hkv, h = bh % sh.Hkv;
  const int64_t p = nt.pos;
  const int g = sh.g, hs = nthr >> 7, jj = tid >> 7, c = tid & (kD - 1);
  const int S = a.n_partials;
  const uint16_t* qg = static_cast<const uint16_t*>(a.q) + ((int64_t)b * sh.Hq + (int64_t)h * g) * kD;

  // ---- loads that do not wait for the new token ----------------------------------
  const uint4 raw = wave < 2 && lane < 16
      ? static_cast<const uint4*>(wave == 0 ? nt.v_new : nt.k_new)[(int64_t)bh * (kD / 8) + lane]
      : uint4{0u, 0u, 0u, 0u};
  float qv = elem2f(qg[(int64_t)jj * kD + c], sh.kv_bf16);
  constexpr int kU = 16;   // split states per round trip
  float m[kU], l[kU], o[kU];
  const float* rec = partial_rec(a, b, h * g + jj, 0);
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const bool ok = u < S;
    const float* pr = rec + (int64_t)(ok ? u : 0) * (kD + 2);
    m[u] = ok ? pr[kD] : -INFINITY;
    l[u] = ok ? pr[kD + 1] : 0.f;
    o[u] = ok ? pr[c] : 0.f;
  }
  // value tile: the 32 * bits dwords of the lanes 16 q + i (i < 16) that hold token tau
  const bool vtile = a.v.quant != KVQ_QUANT_NONE;
  const int vbits = a.v.bits, tau = (int)(p & (kTile - 1)), tq = (tau & 15) >> 2;
  uint32_t* tile_dw = reinterpret_cast<uint32_t*>(a.v.codes + tok_row(sh, b, h, p - tau) * a.v.row_bytes);
  int tw[2];
  uint32_t told[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int idx = tid + k * nthr;
    tw[k] = -1;
    told[k] = 0u;
    if (vtile && idx < 32 * vbits) {
      const int i = idx / (2 * vbits), rem = idx - i * 2 * vbits;
      tw[k] = (16 * tq + i) * (2 * vbits) + rem;
      told[k] = tile_dw[tw[k]];
    }
  }

  // ---- encode the token (waves 0 and 1), fold the first split states ----------------
  if (wave < 2 && lane < 16) {
    const bool val = wave == 0;
    const DevTensor& t = val ? a.v : a.k;
    const int j8 = lane;
    float x[8], dq[8];
    unpack8(raw, sh.kv_bf16, x);
    if (t.quant == KVQ_QUANT_NONE) {
      reinterpret_cast<uint4*>(t.codes)[tok_row(sh, b, h, p) * (kD / 8) + j8] = raw;
#pragma unroll
      for (int e = 0; e < 8; ++e) dq[e] = x[e];
    } else if (!val && t.per_channel) {
      // a per-channel key whose group stays open: the unquantized tail ring
      reinterpret_cast<uint4*>(t.tail)[((int64_t)bh * t.tail_rows + p % t.tail_rows) * (kD / 8) + j8] = raw;
#pragma unroll
      for (int e = 0; e < 8; ++e) dq[e] = x[e];
    } else {
      void* prm = t.params ? static_cast<uint8_t*>(t.params) +
                                 prm_rec(t, sh, b, h, p) * (t.quant == KVQ_QUANT_SYM_Q8_0 ? 2 : 4)
                           : nullptr;
      const uint2 cq = encode8(head_view(t, h), h, j8, x, prm, dq);
      *reinterpret_cast<uint2*>(&(val ? vcode : kcode)[8 * j8]) = cq;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) (val ? vdq : kdq)[8 * j8 + e] = dq[e];
  }
  float M = -INFINITY, L = 0.f, O = 0.f;   // merged split states of head jj
  auto fold = [&](const float* mu, const float* lu, const float* ou) {
    float mc = M;
#pragma unroll
    for (int u = 0; u < kU; ++u) mc = fmaxf(mc, mu[u]);
    if (mc == -INFINITY) return;
    const float r = M == -INFINITY ? 0.f : exp2f(M - mc);
    L *= r;
    O *= r;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float w = mu[u] == -INFINITY ? 0.f : exp2f(mu[u] - mc);
      L = __builtin_fmaf(w, lu[u], L);
      O = __builtin_fmaf(w, ou[u], O);
    }
    M = mc;
  };
  fold(m, l, o);
  __syncthreads();

  // ---- the token's codes into the cache layouts ------------------------------------
  if (a.k.quant != KVQ_QUANT_NONE && !a.k.per_channel) {
    uint32_t* row = reinterpret_cast<uint32_t*>(a.k.codes + tok_row(sh, b, h, p) * a.k.row_bytes);
    for (int W = tid; W < 4 * a.k.bits; W += nthr) row[W] = k_row_dword(kcode, a.k.bits, W);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    if (tw[k] < 0) continue;
    const int W = tw[k], Lw = W / (2 * vbits), sw = (W / vbits) & 1, j = W % vbits, i = Lw & 15;
    uint32_t nb = 0, nm = 0;
    seg_dword_fields(vbits, j, [&](int u, int shf, int wd, int field) {
      const int mm = u >> 3, e = u & 7;
      if ((e & 3) == (tau & 3) && (e >> 2) == (tau >> 4)) {   // token 4 tq + e or 16 + 4 tq + e - 4
        nb |= field_value(vcode[16 * (4 * sw + mm) + i], field) << shf;
        nm |= ((1u << wd) - 1u) << shf;
      }
    });
    if (nm != 0) tile_dw[W] = (told[k] & ~nm) | nb;
  }

  // ---- per pass of up to 8 heads: the token's score, then the merge -------------
  const float sm2 = a.sm_scale * 1.4426950408889634f;   // base-2 scores, as the decode kernels
  const float kc = kdq[c], vc = vdq[c];
  for (int j0 = 0; j0 < g; j0 += hs) {
    const int j = j0 + jj;
    const bool act = j < g;
    if (j0 > 0) {
      // a later pass: its query channel and split states
      qv = act ? elem2f(qg[(int64_t)j * kD + c], sh.kv_bf16) : 0.f;
      M = -INFINITY;
      L = O = 0.f;
      __syncthreads();   // the previous pass has read red
    }
    const float d = wave_sum(qv * kc);
    if (lane == 0) red[wave] = d;
    __syncthreads();
    if (!act) continue;
    const float* rj = partial_rec(a, b, h * g + j, 0);
    for (int s0 = j0 > 0 ? 0 : kU; s0 < S; s0 += kU) {   // states beyond those folded
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const bool ok = s0 + u < S;
        const float* pr = rj + (int64_t)(ok ? s0 + u : 0) * (kD + 2);
        m[u] = ok ? pr[kD] : -INFINITY;
        l[u] = ok ? pr[kD + 1] : 0.f;
        o[u] = ok ? pr[c] : 0.f;
      }
      fold(m, l, o);
    }
    // the new token: m = its score, l = 1, o = its value
    const float sn = (red[2 * jj] + red[2 * jj + 1]) * sm2;
    const float mc = fmaxf(M, sn);
    const float r = M == -INFINITY ? 0.f : exp2f(M - mc), wn = exp2f(sn - mc);
    store_out(a, ((int64_t)b * sh.Hq + h * g + j) * kD + c,
              __builtin_fmaf(wn, vc, O * r) / __builtin_fmaf(wn, 1.0f, L * r));
  }
}

// ---- per-channel keys ---------------------------------------------------------
// Quantize completed token groups: one block of 256 threads per (group,
// b*Hkv + h).  The group's G rows (tokens that arrived in earlier calls come
// from the fp16/bf16 tail) are staged in LDS with 16-byte loads; two threads
// per channel reduce min / max / absmax over half of the tokens each and
// encode them.
__global__ __launch_bounds__(256) void enc_kchan_flush_kernel(DevShape sh, DevTensor t,
                                                              const void* x_new, int64_t n_ctx,
                                                              int n_new, int64_t g0) {
  extern __shared__ uint4 kch_lds[];                      // raw [G][128] elements, codes [G][128]
  __shared__ float red[3][kD];
  const int G = t.G;
  uint16_t* raw = reinterpret_cast<uint16_t*>(kch_lds);
  uint8_t* gcodes = reinterpret_cast<uint8_t*>(raw + (int64_t)G * kD);
  const int tid = threadIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / sh.Hkv, h = bh % sh.Hkv;
  const int64_t gi = g0 + blockIdx.x;
  const int64_t p0 = gi * G;
  const int R = t.tail_rows;
  const uint16_t* tail = t.tail + (int64_t)bh * R * kD;   // ring: token p at row p mod R
  for (int idx = tid; idx < G * (kD / 8); idx += 256) {
    const int k = idx / (kD / 8), u = idx % (kD / 8);
    const int64_t p = p0 + k;
    const uint4* src;
    if (p < n_ctx) {
      src = reinterpret_cast<const uint4*>(tail + (p % R) * kD);
    } else {
      const int64_t rin = ((int64_t)b * sh.in_tok + sh.in_off + (p - n_ctx)) * sh.Hkv + h;
      src = reinterpret_cast<const uint4*>(x_new) + rin * (kD / 8);
    }
    kch_lds[idx] = src[u];
  }
  __syncthreads();
  const int c = tid & (kD - 1), half = tid >> 7;
  const int k0 = half * (G / 2), k1 = k0 + G / 2;
  float lo = INFINITY, hi = -INFINITY, am = 0.0f;
  for (int k = k0; k < k1; ++k) {
    const float x = elem2f(raw[k * kD + c], sh.kv_bf16);
    lo = fminf(lo, x);
    hi = fmaxf(hi, x);
    am = fmaxf(am, fabsf(x));
  }
  // the window reaches overlap tokens back, into the previous group (never
  // before token 0): from the tail ring, or from this append's input
  const int64_t w0 = p0 - t.overlap > 0 ? p0 - t.overlap : 0;
  const int64_t wn = p0 - w0, wk0 = half * (wn / 2), wk1 = half ? wn : wn / 2;
  for (int64_t k = wk0; k < wk1; ++k) {
    const int64_t p = w0 + k;
    uint16_t e;
    if (p < n_ctx) {
      e = tail[(p % R) * kD + c];
    } else {
      const int64_t rin = ((int64_t)b * sh.in_tok + sh.in_off + (p - n_ctx)) * sh.Hkv + h;
      e = static_cast<const uint16_t*>(x_new)[rin * kD + c];
    }
    const float x = elem2f(e, sh.kv_bf16);
    lo = fminf(lo, x);
    hi = fmaxf(hi, x);
    am = fmaxf(am, fabsf(x));
  }
  if (half) {
    red[0][c] = lo;
    red[1][c] = hi;
    red[2][c] = am;
  }
  __syncthreads();
  const float qmax = (float)((1 << t.bits) - 1);
  if (!half) {
    lo = fminf(lo, red[0][c]);
    hi = fmaxf(hi, red[1][c]);
    am = fmaxf(am, red[2][c]);
    uint16_t shh;
    if (t.quant == KVQ_QUANT_ASYM_MINMAX)
      shh = f2h_rn((hi - lo) / qmax);
    else
      shh = f2h_rn(am / (float)((1 << (t.bits - 1)) - 1));
    const uint16_t zh = f2h_rn(lo);
    static_cast<uint32_t*>(t.params)[((int64_t)bh * (sh.Tcap / G) + gi) * kD + c] =
        (uint32_t)shh | ((uint32_t)zh << 16);
    red[0][c] = h2f(shh);
    red[1][c] = h2f(zh);
  }
  __syncthreads();
  const float s = red[0][c], z = red[1][c];
  for (int k = k0; k < k1; ++k) {
    uint32_t q = 0;
    if (s != 0.0f) {
      const float v = rintf((elem2f(raw[k * kD + c], sh.kv_bf16) - z) / s);
      q = (uint32_t)fminf(fmaxf(v, 0.0f), qmax);
    }
    gcodes[k * kD + c] = (uint8_t)q;
  }
  __syncthreads();
  const int dw_per_row = 4 * t.bits;
  for (int idx = tid; idx < G * dw_per_row; idx += 256) {
    const int k = idx / dw_per_row, W = idx % dw_per_row;
    // a group spans G / 32 tiles, each on its own page in a paged cache
    reinterpret_cast<uint32_t*>(t.codes + tok_row(sh, b, h, p0 + k) * t.row_bytes)[W] =
        k_row_dword(gcodes + k * kD, t.bits, W);
  }
  // (the tail ring is brought up to date by enc_kchan_ring_kernel once
  // every group of the append is encoded)
}

// Rewrite the key tail ring after an append that completed groups: row s
// holds the latest token p < n1 with p = s mod R if p is still needed
// (p >= live_start: the next window's reach back and the unfinished
// group), copied from the input when it arrived in this append; other rows
// are cleared.  One block per (row, b * Hkv + h), a thread per dword.
__global__ __launch_bounds__(64) void enc_kchan_ring_kernel(DevShape sh, DevTensor t,
                                                            const void* x_new, int64_t n_ctx,
                                                            int n_new, int64_t live_start) {
  const int bh = blockIdx.y;
  const int b = bh / sh.Hkv, h = bh % sh.Hkv;
  const int R = t.tail_rows, s = blockIdx.x;
  const int64_t n1 = n_ctx + n_new;
  const int64_t back = ((n1 - 1 - s) % R + R) % R;
  const int64_t p = n1 - 1 - back;               // = s mod R, in [n1 - R, n1)
  uint32_t* dst = reinterpret_cast<uint32_t*>(t.tail + ((int64_t)bh * R + s) * kD) + threadIdx.x;
  if (p < 0 || p < live_start) {
    *dst = 0u;
  } else if (p >= n_ctx) {
    const int64_t rin = ((int64_t)b * sh.in_tok + sh.in_off + (p - n_ctx)) * sh.Hkv + h;
    *dst = static_cast<const uint32_t*>(x_new)[rin * (kD / 2) + threadIdx.x];
  }
}

// Copy new tokens of the unfinished last group into the tail ring (an
// append that completes no group).
__global__ __launch_bounds__(64) void enc_kchan_tail_kernel(DevShape sh, DevTensor t,
                                                            const void* x_new, int64_t n_ctx,
                                                            int n_new, int64_t p_first) {
  const int bh = blockIdx.y;
  const int b = bh / sh.Hkv, h = bh % sh.Hkv;
  const int64_t p = p_first + blockIdx.x;
  const int64_t rin = ((int64_t)b * sh.in_tok + sh.in_off + (p - n_ctx)) * sh.Hkv + h;
  const uint32_t pair = static_cast<const uint32_t*>(x_new)[rin * (kD / 2) + threadIdx.x];
  uint32_t* dst = reinterpret_cast<uint32_t*>(
      t.tail + ((int64_t)bh * t.tail_rows + p % t.tail_rows) * kD);
  dst[threadIdx.x] = pair;
}

// ---- dense-and-sparse outliers (CODEBOOK) ----------------------------------
// One block per (new token, b).  Keys (|x| bits << 16 | 0xffff - index) are
// unique, so the k-th largest key is found exactly by a radix select over
// four digits (bits 30-23, 22-15, 14-7, 6-0), each from LDS histograms (one
// per wave, to spread atomic contention); the k keys at or above it are then
// written in index order.
__global__ __launch_bounds__(256) void enc_outliers_kernel(DevShape sh, DevTensor t,
                                                           const void* x_new, int64_t n_ctx,
                                                           int n_new) {
  extern __shared__ uint32_t keys[];                      // [n]
  __shared__ uint32_t hist[4][256];
  __shared__ uint32_t sel[2];                             // digit, remaining rank
  __shared__ uint32_t wsum[4];
  const int n = sh.Hkv * kD;
  const int k = t.k_out;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int tn = blockIdx.x, b = blockIdx.y;
  const int64_t tpos = n_ctx + tn;
  const uint16_t* xr = static_cast<const uint16_t*>(x_new) + ((int64_t)b * sh.in_tok + sh.in_off + tn) * n;
  for (int i = tid; i < n; i += 256)
    keys[i] = ((uint32_t)(xr[i] & 0x7fffu) << 16) | (0xffffu - (uint32_t)i);
  uint32_t prefix = 0, mask = 0, kk = (uint32_t)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = pass < 3 ? 23 - 8 * pass : 0;
    const uint32_t dmask = pass < 3 ? 0xffu : 0x7fu;
    for (int i = tid; i < 4 * 256; i += 256) (&hist[0][0])[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += 256) {
      const uint32_t key = keys[i];
      if ((key & mask) == prefix) atomicAdd(&hist[wave][(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l holds bins 4l .. 4l + 3; suffix sums over the lanes find the
      // digit d with count(digit > d) < kk <= count(digit >= d)
      uint32_t c[4], tot = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int bin = 4 * lane + j;
        c[j] = hist[0][bin] + hist[1][bin] + hist[2][bin] + hist[3][bin];
        tot += c[j];
      }
      uint32_t suf = tot;                                  // sum over lanes >= this lane
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_down(suf, off, 64);
        if (lane + off < 64) suf += v;
      }
      const uint32_t above = suf - tot;                    // lanes > this lane
      if (above < kk && kk <= suf) {
        uint32_t run = above;
        for (int j = 3; j >= 0; --j) {
          if (run + c[j] >= kk) {
            sel[0] = (uint32_t)(4 * lane + j);
            sel[1] = kk - run;
            break;
          }
          run += c[j];
        }
      }
    }
    __syncthreads();
    prefix |= sel[0] << shift;
    mask |= dmask << shift;
    kk = sel[1];
    __syncthreads();
  }
  // prefix is now the k-th largest key: write the k keys >= prefix in index
  // order (thread tid owns indices per * tid .. per * tid + per - 1)
  const int per = (n + 255) / 256;
  const int i0 = tid * per, i1 = min(n, i0 + per);
  uint32_t mine = 0;
  for (int i = i0; i < i1; ++i) mine += keys[i] >= prefix;
  uint32_t incl = mine;
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t pos = incl - mine;
  for (int w = 0; w < wave; ++w) pos += wsum[w];
  const int64_t r = csr_row(sh, b, tpos);
  for (int i = i0; i < i1; ++i) {
    if (keys[i] >= prefix) {
      // column h*d + c in bits 0-11, the replaced dense index in bits 12-15
      const uint32_t dense = cb_code(t.codebook + (int64_t)i * 16, elem2f(xr[i], sh.kv_bf16));
      t.col[r * k + pos] = (uint16_t)(i | (dense << 12));
      // outliers are kept in fp16: a bf16 input is rounded to nearest-even
      t.val[r * k + pos] = sh.kv_bf16 ? f2h_rn(bf2f(xr[i])) : xr[i];
      ++pos;
    }
  }
  if (tid == 0) {
    // both ends of the row (every row pointer is k times its index, so
    // neighbouring tokens write equal values; in a paged cache the next
    // row may be the first of another page)
    t.row_ptr[r] = (int32_t)(k * r);
    t.row_ptr[r + 1] = (int32_t)(k * (r + 1));
  }
}

// ---- per-tile outlier index (CODEBOOK with outliers) ------------------------
// The decode kernels read a tile's outliers grouped by KV head: for the tile
// of 32 tokens and head h, the entries of its tokens in token order (each
// token's in column order), one dword each -- channel (bits 0-6), token in
// the tile (7-11), the dense index it replaces (12-15), fp16 value (16-31);
// off[h] is where head h's entries start in the tile's block of 32 k
// entries, off[Hkv] the tile's count.  One block per (tile that this append
// touches, sequence) rebuilds the tile from its tokens' CSR rows.
__global__ __launch_bounds__(256) void enc_otile_kernel(DevShape sh, DevTensor t, int64_t n_total,
                                                        int64_t tile0) {
  __shared__ uint32_t cnt[kTile][33];   // entries of (token, head); then their rank offsets
  __shared__ uint32_t pos[kTile][33];   // where (token, head)'s entries start in the head's list
  __shared__ uint32_t hoff[33];         // where each head's list starts in the tile's block
  const int tid = threadIdx.x;
  const int b = blockIdx.y;
  const int64_t t0 = (tile0 + blockIdx.x) * kTile;
  const int nt = (int)min((int64_t)kTile, n_total - t0);
  const int H = sh.Hkv, k = t.k_out;
  const int64_t r0 = csr_row(sh, b, t0);          // rows r0 .. r0 + nt - 1 (one page)
  const int64_t tile = r0 / kTile;
  const int o_row = (H + 8) / 8 * 8;
  for (int i = tid; i < kTile * 33; i += 256) (&cnt[0][0])[i] = 0u;
  __syncthreads();
  const int ne = nt * k;
  for (int i = tid; i < ne; i += 256)
    atomicAdd(&cnt[i / k][(t.col[r0 * k + i] & 0xfffu) >> 7], 1u);
  __syncthreads();
  // head h's list: its tokens in turn
  if (tid < H) {
    uint32_t acc = 0;
    for (int tau = 0; tau < kTile; ++tau) { pos[tau][tid] = acc; acc += cnt[tau][tid]; }
    hoff[tid] = acc;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t acc = 0;
    for (int h = 0; h < H; ++h) { const uint32_t c = hoff[h]; hoff[h] = acc; acc += c; }
    hoff[H] = acc;
  }
  // a token's row holds its entries in column order: the first of head h
  // in the row is the sum of its counts over the heads before
  if (tid < kTile) {
    uint32_t acc = 0;
    for (int h = 0; h < H; ++h) { const uint32_t c = cnt[tid][h]; cnt[tid][h] = acc; acc += c; }
  }
  __syncthreads();
  uint32_t* blk = t.tent + tile * ((int64_t)kTile * k);
  for (int i = tid; i < ne; i += 256) {
    const int tau = i / k, j = i - tau * k;
    const uint32_t col = t.col[r0 * k + i];
    const int h = (int)((col & 0xfffu) >> 7);
    const uint32_t dst = hoff[h] + pos[tau][h] + ((uint32_t)j - cnt[tau][h]);
    blk[dst] = (col & 0xf07fu) | ((uint32_t)tau << 7) | ((uint32_t)t.val[r0 * k + i] << 16);
  }
  for (int h = tid; h < o_row; h += 256) t.toff[tile * o_row + h] = h <= H ? (uint16_t)hoff[h] : 0;
}

}  // namespace

hipError_t launch_encode_tensor(const DevShape& sh, const DevTensor& t, bool is_key,
                                const void* x_new, int64_t n_ctx, int n_new,
                                hipStream_t stream) {
  const int64_t nrows = (int64_t)sh.B * n_new * sh.Hkv;
  if (t.quant == KVQ_QUANT_NONE || (is_key && !t.per_channel)) {
    const int64_t blocks = (nrows + 15) / 16;
    hipLaunchKernelGGL(enc_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, sh, t, x_new,
                       n_ctx, n_new);
  } else if (is_key) {
    const int G = t.G;
    const int64_t n1 = n_ctx + n_new;
    const int64_t g_first = n_ctx / G, g_end = n1 / G;   // groups [g_first, g_end) complete now
    if (g_end > g_first) {
      // encode the completed groups (their windows read the ring as it
      // was), then bring the ring up to date
      hipLaunchKernelGGL(enc_kchan_flush_kernel, dim3((unsigned)(g_end - g_first), sh.B * sh.Hkv),
                         dim3(256), (size_t)G * kD * 3, stream, sh, t, x_new, n_ctx, n_new, g_first);
      const int64_t live = g_end * G - t.overlap;
      hipLaunchKernelGGL(enc_kchan_ring_kernel, dim3((unsigned)t.tail_rows, sh.B * sh.Hkv),
                         dim3(64), 0, stream, sh, t, x_new, n_ctx, n_new, live > 0 ? live : 0);
    } else {
      hipLaunchKernelGGL(enc_kchan_tail_kernel, dim3((unsigned)n_new, sh.B * sh.Hkv),
                         dim3(64), 0, stream, sh, t, x_new, n_ctx, n_new, n_ctx);
    }
  } else {
    const int64_t tile0 = n_ctx / kTile, tile1 = (n_ctx + n_new - 1) / kTile;
    hipLaunchKernelGGL(enc_vtile_kernel, dim3((unsigned)(tile1 - tile0 + 1), sh.B * sh.Hkv),
                       dim3(256), 0, stream, sh, t, x_new, n_ctx, n_new, tile0, KeyTail{});
  }
  if (t.k_out > 0) {
    hipLaunchKernelGGL(enc_outliers_kernel, dim3(n_new, sh.B), dim3(256),
                       (size_t)sh.Hkv * kD * 4, stream, sh, t, x_new, n_ctx, n_new);
    const int64_t tile0 = n_ctx / kTile, tile1 = (n_ctx + n_new - 1) / kTile;
    hipLaunchKernelGGL(enc_otile_kernel, dim3((unsigned)(tile1 - tile0 + 1), sh.B), dim3(256), 0,
                       stream, sh, t, n_ctx + n_new, tile0);
  }
  return hipGetLastError();
}

// Keys and values of one append.  When the keys are per-channel groups and
// this append completes none of them (so every new key row goes to the
// tail), and the values are value tiles without outliers, one launch of
// enc_vtile_kernel encodes the values and copies the key rows; otherwise the
// two tensors are encoded one after the other.
hipError_t launch_encode_kv(const DevShape& sh, const DevTensor& kt, const DevTensor& vt,
                            const void* k_new, const void* v_new, int64_t n_ctx, int n_new,
                            hipStream_t stream) {
  const bool k_tail_only = kt.quant != KVQ_QUANT_NONE && kt.per_channel && kt.k_out == 0 &&
                           n_ctx / kt.G == (n_ctx + n_new) / kt.G;
  const bool v_tiles = vt.quant != KVQ_QUANT_NONE && vt.k_out == 0;
  if (!(k_tail_only && v_tiles)) {
    const hipError_t e = launch_encode_tensor(sh, kt, true, k_new, n_ctx, n_new, stream);
    if (e != hipSuccess) return e;
    return launch_encode_tensor(sh, vt, false, v_new, n_ctx, n_new, stream);
  }
  KeyTail tail;
  tail.tail = reinterpret_cast<uint32_t*>(kt.tail);
  tail.k_new = k_new;
  tail.R = kt.tail_rows;
  tail.p_first = n_ctx;
  tail.n_rows = n_new;
  const int64_t tile0 = n_ctx / kTile, tile1 = (n_ctx + n_new - 1) / kTile;
  hipLaunchKernelGGL(enc_vtile_kernel, dim3((unsigned)(tile1 - tile0 + 1), sh.B * sh.Hkv),
                     dim3(256), 0, stream, sh, vt, v_new, n_ctx, n_new, tile0, tail);
  return hipGetLastError();
}

hipError_t launch_append_merge(const DecodeArgs& a, const void* k_new, const void* v_new,
                               int64_t pos, hipStream_t stream) {
  const int heads = a.sh.g < kAppendPassHeads ? a.sh.g : kAppendPassHeads;
  hipLaunchKernelGGL(dec_append_merge_kernel, dim3((unsigned)(a.sh.B * a.sh.Hkv)),
                     dim3(128 * heads), 0, stream, a, NewToken{k_new, v_new, pos});
  return hipGetLastError();
}

// ---- attention sink: raw rows ----------------------------------------------
// One thread per 4 elements (8 bytes) of a row: input token in_off + i of
// sequence b, KV head h goes to sink row pos + i.
__global__ __launch_bounds__(256) void enc_sink_kernel(DevShape sh, uint16_t* sink, int sink_cap,
                                                       const void* x_new, int64_t pos, int n) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)sh.B * n * sh.Hkv * (kD / 4);
  if (idx >= total) return;
  const int c4 = (int)(idx % (kD / 4));
  const int64_t r = idx / (kD / 4);
  const int h = (int)(r % sh.Hkv);
  const int64_t bt = r / sh.Hkv;
  const int b = (int)(bt / n), i = (int)(bt % n);
  const int64_t rin = ((int64_t)b * sh.in_tok + sh.in_off + i) * sh.Hkv + h;
  const uint2 v = reinterpret_cast<const uint2*>(x_new)[rin * (kD / 4) + c4];
  const int64_t row = ((int64_t)b * sh.Hkv + h) * sink_cap + pos + i;
  reinterpret_cast<uint2*>(sink)[row * (kD / 4) + c4] = v;
}

hipError_t launch_encode_sink(const DevShape& sh, uint16_t* sink, int sink_cap, const void* x_new,
                              int64_t pos, int n, hipStream_t stream) {
  const int64_t total = (int64_t)sh.B * n * sh.Hkv * (kD / 4);
  hipLaunchKernelGGL(enc_sink_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                     sh, sink, sink_cap, x_new, pos, n);
  return hipGetLastError();
}

}  // namespace kvq
