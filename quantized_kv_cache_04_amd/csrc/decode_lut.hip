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
// ALUs; the kernel is shaped so that every centroid lookup is an LDS read
// without bank conflicts:
//
//  * workgroup = 4 waves = 4 KV heads over one range of tokens, walked in
//    chunks of 64 tokens;
//  * keys, lane = token: the score of token t is
//      sum_i a_i (x_i cos + y_i sin) + b_i (y_i cos - x_i sin)
//    over the rotate-half pairs (a_i, b_i) = (k_i, k_{i+64}) of the
//    dequantized key and (x_i, y_i) of the query, at the angle
//    (t - q_pos) theta_i.  All lanes of one lookup read the same channel, so
//    the 16 centroids (one 32-byte row) serve every lane by broadcast;
//  * values, lane = channel pair (l, l + 64): the codebook value tiles hold
//    both 4-bit indices of a lane in one byte per token, and one LDS dword
//    per (centroid, lane) holds both channels' centroids, so lane l always
//    reads bank l;
//  * the (cos, sin) table of a chunk (64 pairs x 64 tokens) is shared by the
//    4 heads and advanced by one complex multiplication per entry and chunk,
//    re-anchored from float64 angles every 32 chunks;
//  * outliers (CSR rows of one token over all heads) are filtered by the
//    whole workgroup and enter as (val - centroid) corrections: to the
//    chunk's scores for keys, to LDS channel sums for values.
//
// Each wave leaves an (o, m, l) partial per split, or the output when the
// context is one split.
#include <hip/hip_runtime.h>

#include "splitk.h"

namespace kvq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

constexpr int kD = kHeadDim;
constexpr int kChunk = 64;      // tokens per chunk: one per lane on the key side
constexpr int kHeads = 4;       // KV heads per workgroup, one per wave
constexpr int kPairs = kD / 2;
constexpr int kResync = 32;     // chunks between exact re-anchorings of the table
constexpr float kLog2e = 1.4426950408889634f;

struct __align__(16) LutLds {
  float2 e[kPairs][kChunk];        // (cos, sin) of (t0 + tau - p) theta_i       32 KB
  uint16_t kt[kHeads][kD][16];     // key centroids, fp16 [head][channel][index]   16 KB
  uint32_t vt[kHeads][16][64];     // value centroids: (index, l) -> C(l) | C(l+64) << 16
  float qs[kHeads][kD];            // query * sm_scale * log2(e)
  float scorr[kHeads][kChunk];     // key outlier corrections of the chunk's scores
  float p[kHeads][kChunk];         // probabilities of the chunk
  float vcorr[kHeads][kD];         // value outlier sums of the chunk
  float2 estep[kPairs];            // (cos, sin) of kChunk * theta_i
  double theta[kPairs];
  uint2 ring[kHeads][64];          // per wave: outlier entries of its head group, compacted
};

__device__ __forceinline__ float wave_max(float x) {
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// (cos, sin) of dt * theta, the angle formed and reduced in float64
__device__ __forceinline__ float2 rope_cs(double theta, int64_t dt) {
  const double ang = (double)dt * theta;
  const double two_pi = 6.283185307179586476925286766559;
  const double red = ang - two_pi * rint(ang / two_pi);
  float sn, cs;
  sincosf((float)red, &sn, &cs);
  return make_float2(cs, sn);
}

__device__ __forceinline__ float half_lo(uint32_t w) {
  return (float)__builtin_bit_cast(half2v, w)[0];
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return (float)__builtin_bit_cast(half2v, w)[1];
}

template <bool ROPE, bool KOUT, bool VOUT>
__global__ __launch_bounds__(256, 2) void dec_lut_kernel(DecodeArgs a) {
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
  const int tid = threadIdx.x;
  const int h = hg * kHeads + wave;
  const bool head_ok = h < Hkv;                  // wave-uniform
  const int nctx = a.n_ctx;
  const int64_t Tcap = a.sh.Tcap;
  const int t_begin = split * a.blocks_per_split * kTile;
  const int t_end = min(nctx, t_begin + a.blocks_per_split * kTile);
  const int n_chunks = (t_end - t_begin + kChunk - 1) / kChunk;
  const int qpos = a.q_pos ? a.q_pos[b] : nctx - 1;
  const float sm2 = a.sm_scale * kLog2e;

  // ---- tables ------------------------------------------------------------------
  if (head_ok) {
    // key centroids: the head's [128][16] fp16 block, copied as dwords
    const uint32_t* src = reinterpret_cast<const uint32_t*>(K.codebook) + (int64_t)h * kD * 8;
    uint32_t* dst = reinterpret_cast<uint32_t*>(&S.kt[wave][0][0]);
    for (int i = lane; i < kD * 8; i += 64) dst[i] = src[i];
    // value centroids of channels lane and lane + 64, interleaved per index
    const uint16_t* vc = V.codebook + (int64_t)h * kD * 16;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      S.vt[wave][e][lane] = (uint32_t)vc[lane * 16 + e] | ((uint32_t)vc[(lane + 64) * 16 + e] << 16);
    const uint16_t* qg = static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.sh.Hq + h) * kD;
    S.qs[wave][lane] = elem2f(qg[lane], a.sh.kv_bf16) * sm2;
    S.qs[wave][lane + 64] = elem2f(qg[lane + 64], a.sh.kv_bf16) * sm2;
  }
  if constexpr (ROPE) {
    if (tid < kPairs) S.theta[tid] = pow((double)a.rope_base, -2.0 * (double)tid / (double)kD);
  }
  for (int i = tid; i < kHeads * kChunk; i += 256) (&S.scorr[0][0])[i] = 0.f;
  for (int i = tid; i < kHeads * kD; i += 256) (&S.vcorr[0][0])[i] = 0.f;
  __syncthreads();
  auto anchor = [&](int t0) {   // exact (cos, sin) of the chunk starting at t0
    for (int idx = tid; idx < kPairs * kChunk; idx += 256) {
      const int i = idx / kChunk, tau = idx % kChunk;
      S.e[i][tau] = rope_cs(S.theta[i], (int64_t)t0 + tau - qpos);
    }
  };
  if constexpr (ROPE) {
    if (tid < kPairs) S.estep[tid] = rope_cs(S.theta[tid], kChunk);
    anchor(t_begin);
    __syncthreads();
  }

  // ---- per-wave state ------------------------------------------------------------
  float m_run = -INFINITY, l_lane = 0.f;
  float acc0 = 0.f, acc1 = 0.f;                  // channels lane, lane + 64
  const uint8_t* krows = K.codes + ((int64_t)b * Hkv + (head_ok ? h : 0)) * Tcap * 64;
  const uint8_t* vtiles = V.codes + ((int64_t)b * Hkv + (head_ok ? h : 0)) * Tcap * 64;

  // codes of one chunk: key row of token (lane), value bytes of channel pair (lane)
  u32x4 kc[4], vc[4];
  auto load_chunk = [&](int t0, u32x4* kk, u32x4* vv) {
    const int tk = min(t0 + lane, nctx - 1);          // clamp past the end (masked later)
    const u32x4* kr = reinterpret_cast<const u32x4*>(krows + (int64_t)tk * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) kk[i] = kr[i];
    // two tiles of 32 tokens; lane owns 32 bytes of each (a tile past the
    // range is not read: its probabilities are zero)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      if (t0 + 32 * tt < t_end) {
        const u32x4* vr = reinterpret_cast<const u32x4*>(vtiles + (int64_t)(t0 + 32 * tt) * 64 + lane * 32);
        vv[2 * tt] = vr[0];
        vv[2 * tt + 1] = vr[1];
      } else {
        vv[2 * tt] = u32x4{0u, 0u, 0u, 0u};
        vv[2 * tt + 1] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  if (head_ok && n_chunks > 0) load_chunk(t_begin, kc, vc);

  // Outlier entries of a chunk: the CSR rows of its tokens are contiguous
  // (k entries per token), read as 16-byte vectors of 8 entries.  Thread j
  // takes vectors j and j + 256; a vector may run up to 7 entries past the
  // chunk's rows (still inside the allocation: every outlier array is
  // followed by another region), and those entries are skipped.
  constexpr int kVec = 2;                        // vectors per thread and tensor
  struct OutVec { u32x4 col, val; };
  auto load_out = [&](const DevTensor& T, int64_t row0, int nt, OutVec* o) {
    const int64_t e0 = row0 * T.k_out;
    const int nv = (nt * T.k_out + 7) / 8;
    const u32x4* cv = reinterpret_cast<const u32x4*>(T.col + e0);
    const u32x4* vv = reinterpret_cast<const u32x4*>(T.val + e0);
#pragma unroll
    for (int u = 0; u < kVec; ++u) {
      const int vi = tid + 256 * u;
      if (vi < nv) {
        o[u].col = cv[vi];
        o[u].val = vv[vi];
      } else {
        o[u].col = u32x4{0u, 0u, 0u, 0u};
        o[u].val = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  // Calls f(ww, tau, c, dense index, value) for the entries of this
  // workgroup's heads.  Each wave compacts the matching entries among those
  // its threads loaded into its ring (ballot + lane count) and works through
  // the ring once it holds a wave's worth: about one entry in eight belongs
  // to the workgroup, so the per-entry work then runs on full waves.
  auto for_entries = [&](const DevTensor& T, int nt, const OutVec* o, auto&& f) {
    const int ko = T.k_out;
    const int n_ent = nt * ko;
    const float inv_k = 1.0f / (float)ko;
    int qn = 0;                                    // ring fill, wave-uniform
    auto drain = [&]() {
      __builtin_amdgcn_wave_barrier();             // ring writes of this wave land first
      if (lane < qn) {
        const uint2 r = S.ring[wave][lane];
        const uint32_t col = r.x & 0xffffu;
        const int e = (int)(r.x >> 16);
        // token of entry e: floor(e / k), exact in float for e < 2^16
        const int tau = (int)(((float)e + 0.5f) * inv_k);
        const int ww = (int)((col & 0xfffu) >> 7) - hg * kHeads;
        f(ww, tau, (int)(col & (kD - 1)), col >> 12, h2f((uint16_t)r.y));
      }
      __builtin_amdgcn_wave_barrier();             // reads done before the ring refills
      qn = 0;
    };
#pragma unroll
    for (int u = 0; u < kVec; ++u) {
      const uint32_t cw[4] = {o[u].col.x, o[u].col.y, o[u].col.z, o[u].col.w};
      const uint32_t vw[4] = {o[u].val.x, o[u].val.y, o[u].val.z, o[u].val.w};
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int e = 8 * (tid + 256 * u) + x;     // entry index within the chunk
        const uint32_t col = (cw[x >> 1] >> (16 * (x & 1))) & 0xffffu;
        // head of the flat index (col & 0xfff) >> 7; its group: bits 9-11
        const bool hit = e < n_ent && ((col >> 9) & 7u) == (uint32_t)hg;
        const uint64_t mask = __ballot(hit);
        const int cnt = __popcll(mask);
        if (qn + cnt > 64) drain();
        if (hit) {
          const int slot = qn + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                                __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
          S.ring[wave][slot] = make_uint2(col | ((uint32_t)e << 16), (vw[x >> 1] >> (16 * (x & 1))) & 0xffffu);
        }
        qn += cnt;
      }
    }
    if (qn > 0) drain();
  };

  for (int ci = 0; ci < n_chunks; ++ci) {
    const int t0 = t_begin + ci * kChunk;
    const int nt = min(kChunk, t_end - t0);      // tokens of this chunk
    const int64_t row0 = (int64_t)b * Tcap + t0; // CSR row of token t0

    OutVec ko_v[kVec], vo_v[kVec];
    if constexpr (KOUT) load_out(K, row0, nt, ko_v);
    if constexpr (VOUT) load_out(V, row0, nt, vo_v);
    u32x4 kn[4], vn[4];
    if (head_ok && ci + 1 < n_chunks) load_chunk(t0 + kChunk, kn, vn);

    // ---- keys: lane = token (dense part) ------------------------------------------
    float s = 0.f;
    if (head_ok) {
      const uint32_t kw[16] = {kc[0].x, kc[0].y, kc[0].z, kc[0].w, kc[1].x, kc[1].y, kc[1].z, kc[1].w,
                               kc[2].x, kc[2].y, kc[2].z, kc[2].w, kc[3].x, kc[3].y, kc[3].z, kc[3].w};
      // Centroid lookups: the byte offset of S.kt[wave][c][code] is
      // c * 32 (a constant of the unrolled loop) + wave * 4096 + code * 2.
      // The codes of a dword are first spread as code * 2 into the bytes of
      // two words (even and odd nibbles); one byte permute then joins a
      // code byte with the wave's byte into the offset.
      const uint8_t* ktb = reinterpret_cast<const uint8_t*>(&S.kt[0][0][0]);
      const uint32_t wvb = (uint32_t)wave << 12;
      auto spread = [](uint32_t wd, uint32_t out[2]) {
        out[0] = (wd << 1) & 0x1e1e1e1eu;     // nibbles 0, 2, 4, 6
        out[1] = (wd >> 3) & 0x1e1e1e1eu;     // nibbles 1, 3, 5, 7
      };
      auto cent = [&](const uint32_t x[2], int e, int c) -> float {
        const uint32_t off = __builtin_amdgcn_perm(x[e & 1], wvb, 0x0c0c0100u | (uint32_t)(4 + (e >> 1)));
        return (float)*reinterpret_cast<const _Float16*>(ktb + c * 32 + off);
      };
      // dword 4q + m of the row holds channels 32m + 8q + e (e = 0..7)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          uint32_t xa[2], xb[2];
          spread(kw[4 * q + m], xa);
          spread(kw[4 * q + m + 2], xb);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int i = 32 * m + 8 * q + e;          // pair (i, i + 64)
            const float av = cent(xa, e, i);
            const float bv = cent(xb, e, i + kPairs);
            const float x = S.qs[wave][i], y = S.qs[wave][i + kPairs];
            if constexpr (ROPE) {
              const float2 cs = S.e[i][lane];
              s = __builtin_fmaf(av, x * cs.x + y * cs.y, s);
              s = __builtin_fmaf(bv, y * cs.x - x * cs.y, s);
            } else {
              s = __builtin_fmaf(av, x, s);
              s = __builtin_fmaf(bv, y, s);
            }
          }
        }
    }

    // ---- key outliers: (value - centroid) * coefficient into the scores ----------------
    if constexpr (KOUT) {
      for_entries(K, nt, ko_v, [&](int ww, int tau, int c, uint32_t code, float val) {
        const float delta = val - h2f(S.kt[ww][c][code]);
        float coef;
        if constexpr (ROPE) {
          const int i = c & (kPairs - 1);
          const float2 cs = S.e[i][tau];
          const float x = S.qs[ww][i], y = S.qs[ww][i + kPairs];
          coef = c < kPairs ? x * cs.x + y * cs.y : y * cs.x - x * cs.y;
        } else {
          coef = S.qs[ww][c];
        }
        atomicAdd(&S.scorr[ww][tau], delta * coef);
      });
    }
    if constexpr (KOUT || VOUT || ROPE) __syncthreads();   // scores complete; e consumed

    // ---- next chunk's rotation table ---------------------------------------------------
    if constexpr (ROPE) {
      if (ci + 1 < n_chunks) {
        if ((ci + 1) % kResync == 0) {
          anchor(t0 + kChunk);
        } else {
          for (int idx = tid; idx < kPairs * kChunk; idx += 256) {
            const int i = idx / kChunk, tau = idx % kChunk;
            const float2 e0 = S.e[i][tau], st = S.estep[i];
            S.e[i][tau] = make_float2(e0.x * st.x - e0.y * st.y, e0.x * st.y + e0.y * st.x);
          }
        }
      }
    }

    if (head_ok) {
      // ---- online softmax ----------------------------------------------------------
      if constexpr (KOUT) {
        s += S.scorr[wave][lane];
        S.scorr[wave][lane] = 0.f;
      }
      if (lane >= nt) s = -INFINITY;
      const float m_new = fmaxf(m_run, wave_max(s));
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      const float pt = lane < nt ? __builtin_amdgcn_exp2f(s - m_new) : 0.f;
      l_lane = l_lane * alpha + pt;
      m_run = m_new;
      S.p[wave][lane] = pt;
      acc0 *= alpha;
      acc1 *= alpha;
      // LDS accesses of one wave complete in order: the reads below see p
      __builtin_amdgcn_wave_barrier();

      // ---- values: lane = channel pair ----------------------------------------------
      const uint32_t vw[16] = {vc[0].x, vc[0].y, vc[0].z, vc[0].w, vc[1].x, vc[1].y, vc[1].z, vc[1].w,
                               vc[2].x, vc[2].y, vc[2].z, vc[2].w, vc[3].x, vc[3].y, vc[3].z, vc[3].w};
      // byte offset of S.vt[wave][code][lane] = lane * 4 + (16 wave + code) * 256:
      // the code bytes of a dword (16 wave added in every byte) are joined
      // with the lane's byte by one byte permute per lookup
      const uint8_t* vtb = reinterpret_cast<const uint8_t*>(&S.vt[0][0][0]);
      const uint32_t l4 = (uint32_t)lane << 2;
      const uint32_t wpat = (uint32_t)wave * 0x10101010u;
#pragma unroll
      for (int d4 = 0; d4 < 16; ++d4) {
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
    }

    // ---- value outliers: p * (value - centroid) into LDS channel sums ------------------
    if constexpr (VOUT) {
      __syncthreads();                               // p of every head complete
      for_entries(V, nt, vo_v, [&](int ww, int tau, int c, uint32_t code, float val) {
        const uint32_t cc = S.vt[ww][code][c & (kPairs - 1)];
        const float dense = c < kPairs ? half_lo(cc) : half_hi(cc);
        atomicAdd(&S.vcorr[ww][c], S.p[ww][tau] * (val - dense));
      });
      __syncthreads();                               // sums complete
      if (head_ok) {
        acc0 += S.vcorr[wave][lane];
        acc1 += S.vcorr[wave][lane + 64];
        S.vcorr[wave][lane] = 0.f;
        S.vcorr[wave][lane + 64] = 0.f;
      }
    }
    // next table complete; score corrections read and cleared before the
    // next chunk adds to them (with value outliers, their barriers order this)
    if constexpr ((ROPE || KOUT) && !VOUT) __syncthreads();

    if (head_ok && ci + 1 < n_chunks) {
#pragma unroll
      for (int i = 0; i < 4; ++i) { kc[i] = kn[i]; vc[i] = vn[i]; }
    }
  }

  // ---- partial of this split ---------------------------------------------------------
  if (!head_ok) return;
  const float L = wave_sum(l_lane);
  if (a.splits == 1) {
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
  if (ko && vo) hipLaunchKernelGGL((dec_lut_kernel<ROPE, true, true>), dim3(grid), dim3(256), 0, s, a);
  else if (ko) hipLaunchKernelGGL((dec_lut_kernel<ROPE, true, false>), dim3(grid), dim3(256), 0, s, a);
  else if (vo) hipLaunchKernelGGL((dec_lut_kernel<ROPE, false, true>), dim3(grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((dec_lut_kernel<ROPE, false, false>), dim3(grid), dim3(256), 0, s, a);
}

}  // namespace

bool lut_config_supported(const kvq_config& c, int k_out_k, int k_out_v) {
  // a chunk's outlier rows are read as 2 vectors of 8 entries per thread:
  // at most 64 outliers per token
  return c.k.quantizer == KVQ_QUANT_CODEBOOK && c.v.quantizer == KVQ_QUANT_CODEBOOK &&
         c.k.bits == 4 && c.v.bits == 4 && c.n_q_heads == c.n_kv_heads &&
         c.k.layout == KVQ_LAYOUT_PER_TOKEN && c.v.layout == KVQ_LAYOUT_PER_TOKEN &&
         k_out_k <= 64 && k_out_v <= 64;
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
