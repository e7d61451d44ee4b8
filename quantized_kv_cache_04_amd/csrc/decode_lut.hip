// Lookup-table decode kernel of libkvq: codebook keys and values (4-bit
// indices into 16 fp16 centroids per KV head and channel), one query head
// per KV head, optional dense-and-sparse outliers and RoPE on the keys.
//
// The non-uniform codebooks and the sparse fp16 outliers follow the KVQuant
// page (sections 2.2 and 3.3), with keys quantized before the rotary
// embedding (sections 2.1-2.2) so that the rotation is applied at decode
// time; dequantization stays fused into the single pass over the cache
// (Memory-killer page, section 2.3).  Without a GQA group there is no dense
// contraction to give the matrix cores, so everything runs on the vector
// ALUs, and the lookups are LDS reads.  The kernel is latency-bound, so it
// is shaped to keep three workgroups (12 waves) on a CU: 54.5 KB of LDS and
// at most 168 registers per lane.
//
//  * workgroup = 4 waves = 4 KV heads over one range of tokens, walked in
//    chunks of 32 tokens (one value tile);
//  * keys: lanes tau and tau + 32 share token tau, each taking half of the
//    64 rotate-half pairs (a_i, b_i) = (k_i, k_{i+64}) (two 16-byte
//    segments of the key row); the score of token t is
//      sum_i a_i (X_i cos + Y_i sin) + b_i (Y_i cos - X_i sin)
//    with (cos, sin) of tau theta_i from a fixed table and (X_i, Y_i) the
//    query pair rotated by (t0 - q_pos) theta_i once per chunk, every angle
//    reduced in float64, so no rounding carries over from chunk to chunk.
//    All lanes of one half read the same channel's 16 centroids (one
//    32-byte row): a broadcast;
//  * values, lane = channel pair (l, l + 64): the codebook value tiles hold
//    both 4-bit indices of a lane in one byte per token, and one LDS dword
//    per (centroid, lane) holds both channels' centroids, so lane l always
//    reads bank l;
//  * outliers: every 32-token tile indexes its outliers by KV head (the
//    per-tile index next to the CSR rows); each wave reads its head's
//    entries of the chunk, one per lane, and adds (val - centroid)
//    corrections to the token's score for keys (through LDS per-token sums)
//    and, through the wave's LDS channel sums, to the value sums.  Waves of
//    a workgroup never wait for each other inside the token loop.
//
// Each wave leaves an (o, m, l) partial per split, or the output when the
// context is one split and there is no attention sink.
#include <hip/hip_runtime.h>

#include "splitk.h"
#include "timed_launch.h"

namespace kvq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

constexpr int kD = kHeadDim;
constexpr int kChunk = 32;      // tokens per chunk: one value tile
constexpr int kHeads = 4;       // KV heads per workgroup, one per wave
constexpr int kPairs = kD / 2;
constexpr int kResync = 32;     // chunks between exact evaluations of the query rotation
constexpr float kLog2e = 1.4426950408889634f;

struct __align__(16) LutLds {
  float2 e[kPairs][kChunk];        // (cos, sin) of tau * theta_i, fixed                 16 KB
  uint16_t kt[kHeads][kD][16];     // key centroids, fp16 [head][channel][index]         16 KB
  uint32_t vt[kHeads][16][64];     // value centroids: (index, l) -> C(l) | C(l+64) << 16 16 KB
  float2 qr[kHeads][kPairs];       // query pairs * sm_scale * log2(e), rotated to the chunk
  float p[kHeads][kChunk];         // probabilities of the chunk, one row per wave
  float vcorr[kHeads][kD];         // value outlier sums of the chunk, one row per wave
};
// three workgroups per CU: the 160 KB of LDS is allocated in units of 1280 bytes
static_assert(sizeof(LutLds) <= 42 * 1280, "three workgroups per CU");

__device__ __forceinline__ float half_lo(uint32_t w) {
  return (float)__builtin_bit_cast(half2v, w)[0];
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return (float)__builtin_bit_cast(half2v, w)[1];
}

template <bool ROPE, bool KOUT, bool VOUT>
__global__ __launch_bounds__(256, 3) void dec_lut_kernel(DecodeArgs a) {
  __shared__ LutLds S;
  const DevTensor& K = a.k;
  const DevTensor& V = a.v;
  const int Hkv = a.sh.Hkv;
  const int nhg = (Hkv + kHeads - 1) / kHeads;

  // workgroup -> (sequence and range r, head group hg): the head groups of
  // one range take consecutive ids of one residue mod 8, so that they run
  // close together on one chiplet and share its L2 for the outlier rows
  const int w = blockIdx.x;
  const int hg = (w % (8 * nhg)) / 8;
  const int r = (w / (8 * nhg)) * 8 + (w % 8);
  if (r >= a.sh.B * a.splits) return;            // padding workgroup (whole block)
  const int b = r / a.splits, split = r % a.splits;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tau = lane & 31, half = lane >> 5;   // key side: token, half of the pairs
  const int tid = threadIdx.x;
  const int h = hg * kHeads + wave;
  const bool head_ok = h < Hkv;                  // wave-uniform
  const int nctx = a.n_ctx;
  const int t_begin = split * a.blocks_per_split * kTile;
  const int t_end = min(nctx, t_begin + a.blocks_per_split * kTile);
  const int n_chunks = (t_end - t_begin + kChunk - 1) / kChunk;
  // positions are absolute: token t of this cache sits at a.pos0 + t
  const int qpos = a.q_pos ? a.q_pos[b] : a.q_last;
  const float sm2 = a.sm_scale * kLog2e;

  // ---- tables ------------------------------------------------------------------
  if (head_ok) {
    // key centroids: the head's [128][16] fp16 block (4 KB), four 16-byte
    // loads a lane, all issued before the first LDS write
    const u32x4* src = reinterpret_cast<const u32x4*>(K.codebook) + (int64_t)h * kD * 2;
    u32x4* dst = reinterpret_cast<u32x4*>(&S.kt[wave][0][0]);
    u32x4 kcb[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) kcb[k] = src[64 * k + lane];
#pragma unroll
    for (int k = 0; k < 4; ++k) dst[64 * k + lane] = kcb[k];
    // value centroids of channels lane and lane + 64 (32 bytes each, two
    // 16-byte loads), interleaved per index: dword e = C_lane[e] | C_lane+64[e] << 16
    const u32x4* vc = reinterpret_cast<const u32x4*>(V.codebook) + (int64_t)h * kD * 2;
    const u32x4 va[2] = {vc[2 * lane], vc[2 * lane + 1]};
    const u32x4 vb[2] = {vc[2 * (lane + 64)], vc[2 * (lane + 64) + 1]};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t x = va[k >> 2][k & 3], y = vb[k >> 2][k & 3];   // indices 2k, 2k + 1
      S.vt[wave][2 * k][lane] = __builtin_amdgcn_perm(y, x, 0x05040100u);
      S.vt[wave][2 * k + 1][lane] = __builtin_amdgcn_perm(y, x, 0x07060302u);
    }
  }
  // thread (head qw, pair qi) owns one query pair: q * sm_scale * log2(e)
  const int qw = tid >> 6, qi = tid & 63, qh = hg * kHeads + qw;
  float qx = 0.f, qy = 0.f;
  if (qh < Hkv) {
    const uint16_t* qg = static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.sh.Hq + qh) * kD;
    qx = elem2f(qg[qi], a.sh.kv_bf16) * sm2;
    qy = elem2f(qg[qi + kPairs], a.sh.kv_bf16) * sm2;
  }
  double theta = 0.0;                            // theta of pair qi
  if constexpr (ROPE) theta = pow((double)a.rope_base, -2.0 * (double)qi / (double)kD);
  // The query pair rotated by (t0 - q_pos) theta: then the key of token
  // t0 + tau needs only the rotation by tau theta from the fixed table.  The
  // rotation advances by one complex multiplication per chunk and is
  // evaluated exactly from a float64 angle every kResync chunks.
  float2 rot = make_float2(1.f, 0.f), rstep = make_float2(1.f, 0.f);
  if constexpr (ROPE) rstep = rope_cs(theta, kChunk);
  auto set_q = [&](int ci) {
    if constexpr (ROPE) {
      if (ci % kResync == 0) {
        rot = rope_cs(theta, (int64_t)a.pos0 + t_begin + (int64_t)ci * kChunk - qpos);
      } else {
        rot = make_float2(rot.x * rstep.x - rot.y * rstep.y, rot.x * rstep.y + rot.y * rstep.x);
      }
      S.qr[qw][qi] = make_float2(qx * rot.x + qy * rot.y, qy * rot.x - qx * rot.y);
    } else {
      S.qr[qw][qi] = make_float2(qx, qy);
    }
  };
  if constexpr (ROPE) {
    // wave w fills pairs 16w .. 16w + 15; lane (tau, half) two of them per step
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = 16 * wave + 2 * k + half;
      const double th = __shfl(theta, i, 64);
      S.e[i][tau] = rope_cs(th, tau);
    }
  }
  set_q(0);
  for (int i = tid; i < kHeads * kD; i += 256) (&S.vcorr[0][0])[i] = 0.f;
  __syncthreads();

  // ---- per-wave state ------------------------------------------------------------
  float m_run = -INFINITY, l_lane = 0.f;
  float acc0 = 0.f, acc1 = 0.f;                  // channels lane, lane + 64
  const int hr = head_ok ? h : 0;

  // Codes of one chunk: segments 2 half and 2 half + 1 (32 bytes) of the key
  // row of token tau, and the 32 value bytes of channel pair (lane).  Every
  // load is unconditional, with addresses clamped into the cache, so that
  // the compiler can count outstanding loads exactly: past the end, keys are
  // masked and values meet zero probabilities.  The key codes of chunk
  // ci + 1 load during the value phase of chunk ci; the value codes of a
  // chunk load at its start.
  const int last_tile = (nctx - 1) & ~31;
  // rows of the chunk at t0 (32 consecutive rows from its first token's,
  // also on a page of a paged cache); chunks past the end read the last one
  // (a paged cache's table is read one chunk ahead of the loads: chunk_row)
  auto chunk_row = [&](int t0) { return tok_row(a.sh, b, hr, min(t0, last_tile)); };
  // Addresses are a wave-uniform base plus a 32-bit lane offset, so that
  // the loads take their base from scalar registers; the empty asm keeps the
  // compiler from folding the lane offset into a per-lane 64-bit pointer
  // held across the loop.
  auto at = [](const uint8_t* base, uint32_t off) {
    asm volatile("" : "+v"(off));
    return base + off;
  };
  auto load_k = [&](int t0, int64_t rowc, u32x4* kk) {
    const int tk = min(t0 + tau, nctx - 1);
    const uint32_t off = (uint32_t)(tk - min(t0, last_tile)) * 64u + (uint32_t)half * 32u;
    const u32x4* kr = reinterpret_cast<const u32x4*>(at(K.codes + rowc * 64, off));
    kk[0] = kr[0];
    kk[1] = kr[1];
  };
  auto load_v = [&](int64_t rowc, u32x4* vv) {
    const u32x4* vr = reinterpret_cast<const u32x4*>(at(V.codes + rowc * 64, (uint32_t)lane * 32u));
    vv[0] = vr[0];
    vv[1] = vr[1];
  };
  u32x4 kc[2];
  int64_t row_c = chunk_row(t_begin);
  load_k(t_begin, row_c, kc);

  // ---- dense-and-sparse outliers ---------------------------------------------------------
  // A tile of 32 tokens (one chunk) indexes its outliers by KV head: the
  // wave's head h finds its entries of the chunk, in token order, at
  // off[h] .. off[h + 1] - 1 of the tile's block (offsets read with scalar
  // loads).  Lane j takes entry j; lists longer than 64 entries are taken
  // 64 at a time.  An entry is one dword: channel (bits 0-6), token in the
  // tile (7-11), the dense index it replaces (12-15) and its fp16 value
  // (16-31).  The key entries of a chunk load at its start, the value
  // entries after its key phase; no workgroup barrier is involved.
  typedef __attribute__((address_space(4))) const uint32_t const_u32;
  const int o_row = (Hkv + 8) / 8 * 8;           // offsets per tile: round_up(Hkv + 1, 8)
  struct Lst { uint32_t ent; int n; int64_t base, blk; };
  // entry base + i of the list (i < n; any other lane reads the tile's first)
  auto ent_at = [&](const DevTensor& T, const Lst& L, int i) -> uint32_t {
    const int64_t e = i < L.n ? L.base + i : L.blk;
    return T.tent[e];
  };
  auto make_list = [&](const DevTensor& T, int64_t row0, Lst& L) {
    const int64_t tile = row0 >> 5;
    const const_u32* o = (const const_u32*)(T.toff + tile * o_row);
    const uint32_t w0 = o[hr >> 1], w1 = o[(hr + 1) >> 1];
    const uint32_t a0 = (hr & 1) ? (w0 >> 16) : (w0 & 0xffffu);
    const uint32_t a1 = (hr & 1) ? (w1 & 0xffffu) : (w0 >> 16);
    L.n = head_ok ? (int)(a1 - a0) : 0;
    L.blk = tile * ((int64_t)kTile * T.k_out);
    L.base = L.blk + a0;
    L.ent = ent_at(T, L, lane);
  };
  // f(entry, valid) for every entry of the list, 64 at a time (every lane
  // takes part in each call)
  auto for_list = [&](const DevTensor& T, const Lst& L, auto&& f) {
    f(L.ent, lane < L.n);
    for (int i0 = 64; i0 < L.n; i0 += 64) f(ent_at(T, L, i0 + lane), i0 + lane < L.n);
  };

  for (int ci = 0; ci < n_chunks; ++ci) {
    const int t0 = t_begin + ci * kChunk;
    const int nt = min(kChunk, t_end - t0);      // tokens of this chunk
    const int64_t row0 = csr_row(a.sh, b, t0);   // CSR row of token t0
    const int64_t row_n = chunk_row(t0 + kChunk);

    // where this chunk's outlier entries of the head lie; its key entries
    // (the value entries load after the key phase)
    Lst kl, vl;
    if constexpr (KOUT) make_list(K, row0, kl);
    u32x4 vc[2], kn[2];
    load_v(row_c, vc);

    // ---- keys: lanes (tau, half), pairs i = 32m + 16 half + 8qq + e --------------------
    float s = 0.f;
    if (head_ok) {
      // segment 2 half + qq: dword 4qq + m' holds channel 32m' + 8(2 half + qq) + e
      const uint32_t kw[8] = {kc[0].x, kc[0].y, kc[0].z, kc[0].w, kc[1].x, kc[1].y, kc[1].z, kc[1].w};
      // Centroid lookups: the byte offset of S.kt[wave][c][code] is
      // c * 32 + wave * 4096 + code * 2, with c * 32 = (a constant of the
      // unrolled loop) + 512 half.  The codes of a dword are first spread as
      // code * 2 into the bytes of two words (even and odd nibbles); one byte
      // permute then joins a code byte with the lane's (wave, half) byte.
      const uint8_t* ktb = reinterpret_cast<const uint8_t*>(&S.kt[0][0][0]);
      const uint32_t wvb = (uint32_t)(16 * wave + 2 * half) << 8;
      const float2* qb = &S.qr[wave][16 * half];
      const float2* eb = &S.e[16 * half][tau];
      auto spread = [](uint32_t wd, uint32_t out[2]) {
        out[0] = (wd << 1) & 0x1e1e1e1eu;     // nibbles 0, 2, 4, 6
        out[1] = (wd >> 3) & 0x1e1e1e1eu;     // nibbles 1, 3, 5, 7
      };
      auto cent = [&](const uint32_t x[2], int e, int c) -> float {
        const uint32_t off = __builtin_amdgcn_perm(x[e & 1], wvb, 0x0c0c0100u | (uint32_t)(4 + (e >> 1)));
        return (float)*reinterpret_cast<const _Float16*>(ktb + c * 32 + off);
      };
#pragma unroll
      for (int qq = 0; qq < 2; ++qq)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          uint32_t xa[2], xb[2];
          spread(kw[4 * qq + m], xa);
          spread(kw[4 * qq + m + 2], xb);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int ic = 32 * m + 8 * qq + e;        // pair (ic + 16 half) less 16 half
            const float av = cent(xa, e, ic);
            const float bv = cent(xb, e, ic + kPairs);
            const float2 q2 = qb[ic];
            if constexpr (ROPE) {
              const float2 cs = eb[ic * kChunk];
              s = __builtin_fmaf(av, q2.x * cs.x + q2.y * cs.y, s);
              s = __builtin_fmaf(bv, q2.y * cs.x - q2.x * cs.y, s);
            } else {
              s = __builtin_fmaf(av, q2.x, s);
              s = __builtin_fmaf(bv, q2.y, s);
            }
          }
        }
      s += swap_halves(s);                           // both halves of token tau
      // key outliers: (value - centroid) * coefficient into the wave's
      // per-token sums (the first 32 of its channel sums, zero here)
      if constexpr (KOUT) {
        for_list(K, kl, [&](uint32_t ent, bool valid) {
          if (valid) {
            const int te = (int)((ent >> 7) & 31u), c = (int)(ent & (kD - 1));
            const float delta = h2f((uint16_t)(ent >> 16)) - h2f(S.kt[wave][c][(ent >> 12) & 15u]);
            const int i = c & (kPairs - 1);
            const float2 q2 = S.qr[wave][i];
            float coef;
            if constexpr (ROPE) {
              const float2 cs = S.e[i][te];
              coef = c < kPairs ? q2.x * cs.x + q2.y * cs.y : q2.y * cs.x - q2.x * cs.y;
            } else {
              coef = c < kPairs ? q2.x : q2.y;
            }
            atomicAdd(&S.vcorr[wave][te], delta * coef);
          }
        });
        // LDS accesses of one wave complete in order: the sums are complete
        __builtin_amdgcn_wave_barrier();
        s += S.vcorr[wave][tau];
        __builtin_amdgcn_wave_barrier();
        if (half == 0) S.vcorr[wave][tau] = 0.f;
      }
    }
    // the rotated queries of this chunk are consumed (each wave rotates its
    // own head's queries; LDS accesses of one wave complete in order)
    __builtin_amdgcn_wave_barrier();

    // this chunk's value entries; key codes, rotated queries and outlier
    // counts of the next chunk
    if constexpr (VOUT) make_list(V, row0, vl);
    load_k(t0 + kChunk, row_n, kn);
    row_c = row_n;
    if constexpr (ROPE) set_q(ci + 1);

    if (head_ok) {
      // ---- online softmax ----------------------------------------------------------
      if (tau >= nt) s = -INFINITY;
      const float m_new = fmaxf(m_run, wave_max(s));
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      const float pt = tau < nt ? __builtin_amdgcn_exp2f(s - m_new) : 0.f;
      l_lane = l_lane * alpha + (half == 0 ? pt : 0.f);
      m_run = m_new;
      if (half == 0) S.p[wave][tau] = pt;
      acc0 *= alpha;
      acc1 *= alpha;
      // LDS accesses of one wave complete in order: the reads below see p
      __builtin_amdgcn_wave_barrier();

      // ---- values: lane = channel pair ----------------------------------------------
      const uint32_t vw[8] = {vc[0].x, vc[0].y, vc[0].z, vc[0].w, vc[1].x, vc[1].y, vc[1].z, vc[1].w};
      // byte offset of S.vt[wave][code][lane] = lane * 4 + (16 wave + code) * 256:
      // the code bytes of a dword (16 wave added in every byte) are joined
      // with the lane's byte by one byte permute per lookup
      const uint8_t* vtb = reinterpret_cast<const uint8_t*>(&S.vt[0][0][0]);
      const uint32_t l4 = (uint32_t)lane << 2;
      const uint32_t wpat = (uint32_t)wave * 0x10101010u;
#pragma unroll
      for (int d4 = 0; d4 < 8; ++d4) {
        const f32x4 p4 = *reinterpret_cast<const f32x4*>(&S.p[wave][4 * d4]);
        const uint32_t wd = vw[d4];
        const uint32_t xlo = (wd & 0x0f0f0f0fu) | wpat;
        const uint32_t xhi = ((wd >> 4) & 0x0f0f0f0fu) | wpat;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t sel = 0x0c0c0000u | ((uint32_t)(4 + k) << 8);
          const uint32_t c0 = *reinterpret_cast<const uint32_t*>(vtb + __builtin_amdgcn_perm(xlo, l4, sel));
          const uint32_t c1 = *reinterpret_cast<const uint32_t*>(vtb + __builtin_amdgcn_perm(xhi, l4, sel));
          acc0 = __builtin_fmaf(p4[k], half_lo(c0), acc0);
          acc1 = __builtin_fmaf(p4[k], half_hi(c1), acc1);
        }
      }

      // ---- value outliers: p * (value - centroid) into the wave's channel sums ----------
      if constexpr (VOUT) {
        for_list(V, vl, [&](uint32_t ent, bool valid) {
          const float pe = __shfl(pt, (int)((ent >> 7) & 31u), 64);   // p of the entry's token
          if (valid) {
            const int c = (int)(ent & (kD - 1));
            const uint32_t cc = S.vt[wave][(ent >> 12) & 15u][c & (kPairs - 1)];
            const float dense = c < kPairs ? half_lo(cc) : half_hi(cc);
            atomicAdd(&S.vcorr[wave][c], pe * (h2f((uint16_t)(ent >> 16)) - dense));
          }
        });
        // LDS accesses of one wave complete in order: the sums are complete
        __builtin_amdgcn_wave_barrier();
        acc0 += S.vcorr[wave][lane];
        acc1 += S.vcorr[wave][lane + 64];
        S.vcorr[wave][lane] = 0.f;
        S.vcorr[wave][lane + 64] = 0.f;
        __builtin_amdgcn_wave_barrier();
      }
    }

#pragma unroll
    for (int i = 0; i < 2; ++i) kc[i] = kn[i];
  }

  // ---- partial of this split ---------------------------------------------------------
  if (!head_ok) return;
  const float L = wave_sum(l_lane);
  if (a.direct) {
    const int64_t o = ((int64_t)b * a.sh.Hq + h) * kD;
    store_out(a, o + lane, L > 0.f ? acc0 / L : 0.f);
    store_out(a, o + lane + 64, L > 0.f ? acc1 / L : 0.f);
  } else {
    float* rec = partial_rec(a, b, h, split);
    rec[lane] = acc0;
    rec[lane + 64] = acc1;
    if (lane == 0) { rec[kD] = m_run; rec[kD + 1] = L; }
  }
}

template <bool ROPE>
void launch_r(const DecodeArgs& a, unsigned grid, hipStream_t s) {
  const bool ko = a.k.k_out > 0, vo = a.v.k_out > 0;
  if (ko && vo) launch_timed(dec_lut_kernel<ROPE, true, true>, dim3(grid), dim3(256), 0u, s, a);
  else if (ko) launch_timed(dec_lut_kernel<ROPE, true, false>, dim3(grid), dim3(256), 0u, s, a);
  else if (vo) launch_timed(dec_lut_kernel<ROPE, false, true>, dim3(grid), dim3(256), 0u, s, a);
  else launch_timed(dec_lut_kernel<ROPE, false, false>, dim3(grid), dim3(256), 0u, s, a);
}

}  // namespace

bool lut_config_supported(const kvq_config& c, int, int) {
  return c.k.quantizer == KVQ_QUANT_CODEBOOK && c.v.quantizer == KVQ_QUANT_CODEBOOK &&
         c.k.bits == 4 && c.v.bits == 4 && c.n_q_heads == c.n_kv_heads &&
         c.k.layout == KVQ_LAYOUT_PER_TOKEN && c.v.layout == KVQ_LAYOUT_PER_TOKEN;
}

hipError_t launch_decode_lut(const DecodeArgs& a, hipStream_t s) {
  const int nhg = (a.sh.Hkv + kHeads - 1) / kHeads;
  const int64_t ranges = (int64_t)a.sh.B * a.splits;
  const unsigned grid = (unsigned)(((ranges + 7) / 8) * 8 * nhg);
  if (a.rope) launch_r<true>(a, grid, s);
  else launch_r<false>(a, grid, s);
  return hipGetLastError();
}

}  // namespace kvq
