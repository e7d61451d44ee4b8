// Generic decode kernel of libkvq: vector-ALU attention over any cache
// format (raw, uniform 3/4/8-bit, q8_0, codebook with CSR outliers), with
// or without RoPE, for any GQA group size.
//
// Dequantization is fused into the pass (Memory-killer page, section 2.3;
// KVQuant page, section 3.4): each lane dequantizes the codes it needs
// straight from the packed layout, scores them, and the online softmax and
// value product follow in registers (Survey page, section 2.3).  Keys are
// stored before the rotary embedding (KVQuant page, sections 2.1-2.2); the
// score uses q . R(t - p) k, whose angle is formed in float64.  Outliers
// replace their dense value (KVQuant page, section 2.2): the kernel adds
// (value - dense) times the score's derivative for keys, and p times
// (value - dense) for values.
//
// The same kernel streams the raw attention-sink prefix (KVQuant page,
// "Attention Sink"), launched over the sink region as a raw cache whose
// partial states follow those of the quantized cache.
//
// Grid: (splits, B * Hkv); 256 threads = 4 waves; each wave takes chunks of
// 64 tokens of the block's range.
#include <hip/hip_runtime.h>

#include "splitk.h"
#include "timed_launch.h"

namespace kvq {
namespace {

constexpr int kD = kHeadDim;
constexpr int JB = 8;   // query heads per pass
constexpr int CH = 64;  // tokens per wave chunk

// Dense (codebook or uniform) value of key channel c of token t.
__device__ __forceinline__ float deq_k(const DecodeArgs& a, int bh, int h, int t, int c, int n_full) {
  return deq_key(a.k, a.sh, bh, h, t, c, n_full);
}

__device__ __forceinline__ float deq_v(const DecodeArgs& a, int bh, int h, int t, int c) {
  return deq_value(a.v, a.sh, bh, h, t, c);
}

__global__ __launch_bounds__(256) void dec_generic_kernel(DecodeArgs a) {
  __shared__ float qs[JB][kD];
  __shared__ double theta[kD / 2];
  __shared__ float wm[4][JB], wl[4][JB];
  __shared__ float wo[4][JB][kD];
  const int split = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.sh.Hkv, h = bh % a.sh.Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = a.n_ctx;
  const int t_begin = split * a.blocks_per_split * kTile;
  const int t_end = min(n, t_begin + a.blocks_per_split * kTile);
  // positions are absolute: token t of this cache sits at a.pos0 + t
  const int p = a.q_pos ? a.q_pos[b] : a.q_last;
  const int g = a.sh.g;
  const int n_full = a.k.per_channel ? (n / a.k.G) * a.k.G : n;
  const float scale = a.sm_scale * 1.4426950408889634f;   // base-2 scores
  if (a.rope && threadIdx.x < kD / 2)
    theta[threadIdx.x] = pow((double)a.rope_base, -2.0 * (double)threadIdx.x / (double)kD);

  for (int j0 = 0; j0 < g; j0 += JB) {
    const int nj = min(JB, g - j0);
    for (int idx = threadIdx.x; idx < nj * kD; idx += blockDim.x) {
      const int jj = idx / kD, c = idx % kD;
      const int64_t qi = ((int64_t)b * a.sh.Hq + h * g + j0 + jj) * kD + c;
      qs[jj][c] = elem2f(static_cast<const uint16_t*>(a.q)[qi], a.sh.kv_bf16);
    }
    __syncthreads();
    float m[JB], l[JB], o0[JB], o1[JB];
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) { m[jj] = -INFINITY; l[jj] = 0.f; o0[jj] = 0.f; o1[jj] = 0.f; }

    for (int chunk = t_begin + wave * CH; chunk < t_end; chunk += 4 * CH) {
      const int t = chunk + lane;
      const bool valid = t < t_end;
      float sc[JB];
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) sc[jj] = 0.f;
      if (valid) {
        for (int i = 0; i < kD / 2; ++i) {
          const float k0 = deq_k(a, bh, h, t, i, n_full);
          const float k1 = deq_k(a, bh, h, t, i + kD / 2, n_full);
          if (a.rope) {
            const float2 r = rope_cs(theta[i], (int64_t)a.pos0 + t - p);
            const float cs = r.x, sn = r.y;
#pragma unroll
            for (int jj = 0; jj < JB; ++jj) {
              if (jj < nj) {
                const float qa = qs[jj][i], qb = qs[jj][i + kD / 2];
                sc[jj] += cs * (qa * k0 + qb * k1) + sn * (qb * k0 - qa * k1);
              }
            }
          } else {
#pragma unroll
            for (int jj = 0; jj < JB; ++jj)
              if (jj < nj) sc[jj] += qs[jj][i] * k0 + qs[jj][i + kD / 2] * k1;
          }
        }
        if (a.k.k_out) {
          const int64_t r = csr_row(a.sh, b, t);
          const int e0 = a.k.row_ptr[r], e1 = a.k.row_ptr[r + 1];
          for (int e = e0; e < e1; ++e) {
            const int col = (a.k.col[e] & 0xfff) - h * kD;
            if (col < 0 || col >= kD) continue;
            const float delta = h2f(a.k.val[e]) - deq_k(a, bh, h, t, col, n_full);
            const int i = col & (kD / 2 - 1);
            const bool upper = col >= kD / 2;
            float cs = 1.f, sn = 0.f;
            if (a.rope) { const float2 r = rope_cs(theta[i], (int64_t)a.pos0 + t - p); cs = r.x; sn = r.y; }
#pragma unroll
            for (int jj = 0; jj < JB; ++jj) {
              if (jj < nj) {
                const float qa = qs[jj][i], qb = qs[jj][i + kD / 2];
                const float grad = upper ? (cs * qb - sn * qa) : (cs * qa + sn * qb);
                sc[jj] += delta * grad;
              }
            }
          }
        }
      }
      float pv[JB];
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        pv[jj] = 0.f;
        if (jj < nj) {
          const float sv = valid ? sc[jj] * scale : -INFINITY;
          const float mn = fmaxf(m[jj], wave_max(sv));
          const float alpha = m[jj] == -INFINITY ? 0.f : exp2f(m[jj] - mn);
          pv[jj] = valid ? exp2f(sv - mn) : 0.f;
          l[jj] = l[jj] * alpha + wave_sum(pv[jj]);
          o0[jj] *= alpha;
          o1[jj] *= alpha;
          m[jj] = mn;
        }
      }
      const int cnt = min(CH, t_end - chunk);
      for (int tt = 0; tt < cnt; ++tt) {
        const int t2 = chunk + tt;
        const float v0 = deq_v(a, bh, h, t2, lane);
        const float v1 = deq_v(a, bh, h, t2, lane + 64);
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
          if (jj < nj) {
            const float pj = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pv[jj]), tt));
            o0[jj] += pj * v0;
            o1[jj] += pj * v1;
          }
        }
      }
      if (a.v.k_out) {
        for (int tt = 0; tt < cnt; ++tt) {
          const int t2 = chunk + tt;
          const int64_t r = csr_row(a.sh, b, t2);
          const int e0 = a.v.row_ptr[r], e1 = a.v.row_ptr[r + 1];
          for (int e = e0; e < e1; ++e) {
            const int col = (a.v.col[e] & 0xfff) - h * kD;
            if (col < 0 || col >= kD || (col & 63) != lane) continue;
            const float delta = h2f(a.v.val[e]) - deq_v(a, bh, h, t2, col);
#pragma unroll
            for (int jj = 0; jj < JB; ++jj) {
              if (jj < nj) {
                const float pj = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pv[jj]), tt));
                if (col < 64) o0[jj] += pj * delta; else o1[jj] += pj * delta;
              }
            }
          }
        }
      }
    }
    // merge the four waves of the block into one partial per query head
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
      if (jj < nj) {
        if (lane == 0) { wm[wave][jj] = m[jj]; wl[wave][jj] = l[jj]; }
        wo[wave][jj][lane] = o0[jj];
        wo[wave][jj][lane + 64] = o1[jj];
      }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < nj * kD; idx += blockDim.x) {
      const int jj = idx / kD, c = idx % kD;
      float M = -INFINITY;
      for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][jj]);
      float O = 0.f, L = 0.f;
      if (M > -INFINITY) {
        for (int w = 0; w < 4; ++w) {
          const float wt = wm[w][jj] == -INFINITY ? 0.f : exp2f(wm[w][jj] - M);
          O += wt * wo[w][jj][c];
          L += wt * wl[w][jj];
        }
      }
      if (a.direct) {
        // the only partial state (one split, no sink): normalize and write the output
        store_out(a, ((int64_t)b * a.sh.Hq + h * g + j0 + jj) * kD + c, L > 0.f ? O / L : 0.f);
      } else {
        float* rec = partial_rec(a, b, h * g + j0 + jj, a.slot0 + split);
        rec[c] = O;
        if (c == 0) { rec[kD] = M; rec[kD + 1] = L; }
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_decode_generic(const DecodeArgs& a, hipStream_t stream) {
  launch_timed(dec_generic_kernel, dim3(a.splits, a.sh.B * a.sh.Hkv), dim3(256), 0u, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
