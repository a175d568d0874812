// cce_device.h -- gfx950 kernels of libcce (the flash cut-cross-entropy head).
//
// What is computed follows page "mlx-bun 0.0.4 -> 0.0.6",
// src/train/flash-cce.ts: the vocab-parallel forward (per-block online-softmax
// partials, then a cross-block log-sum-exp merge) and the recompute-based
// backward (coefficient g*(onehot - softmax)*c', contracted with the head and
// summed over vocabulary blocks).  How it is computed is designed for CDNA4:
//
//  * Forward logits use bf16 MFMA on EXACT operands.  h is bf16 as given; the
//    integer codes q in [0, 255] are exact in bf16.  Per 64-wide quantization
//    group the MFMA yields A_g = sum_d h_d q_d in fp32 and the tile folds it as
//    acc += s[v,g] * A_g (the qdot factoring of the page's scalar forward
//    kernel, lifted onto the matrix cores).  The bias term sum_g b[v,g]*S[t,g]
//    (S = per-group sum of h) rides along as extra K columns: hi/lo bf16
//    splits S_hi*b_hi + S_lo*b_hi + S_hi*b_lo, accumulated directly.
//  * The backward contracts bf16 coefficients -g*p*c' with a bf16-dequantized
//    head tile (s*q + b rounded once, in LDS), fp32 accumulation.  The target
//    column's whole term g*(1 - p_t)*c'_t*w_t is kept out of that path and
//    added in fp32, with 1 - p_t = -expm1(y_t - lse): exact for a flat softmax
//    (where that term dominates) and for a peaked one (where it is a small
//    difference of large numbers).
//
// Tile roles: a workgroup is 4 waves (256 threads).  MFMA v_mfma_f32_16x16x32_bf16
// lane layout (verified on gfx950): operand lane l holds row l%16, K elements
// 8*(l/16)..+8; result lane l holds column l%16, rows 4*(l/16)+0..3.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cce {

typedef short bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int BM = 256;        // tokens per workgroup tile (4 waves x 64)
constexpr int BN = 128;        // vocabulary rows per tile
constexpr int KSTEP = 64;      // K per step = one quantization group
constexpr int NTHREADS = 256;
constexpr int WROW = KSTEP + 8;  // padded bf16 row stride of the LDS code tile
constexpr int DT = 128;        // dh columns per workgroup in the dh contraction
constexpr int MAX_G = 256;     // H <= 16384

// Per-token side data, one 16-byte record per compacted row.
struct TokRec {
  float lse;   // backward: lse of the token (0 for padding rows)
  float g;     // backward: cotangent (0 for padding rows)
  float tval;  // forward: softcapped target logit; backward: target coefficient
  int tgt;     // target id, -1 for padding rows
};

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two floats that are exact in bf16 (low 16 bits zero) -> one bf16 pair.
__device__ __forceinline__ uint32_t pack_exact(float lo, float hi) {
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

__device__ __forceinline__ uint32_t pack_rne(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

// 8 four-bit codes of one word -> 4 dwords of exact bf16 pairs, in element order.
__device__ __forceinline__ void unpack4(uint32_t w, uint32_t *o) {
  const uint32_t ev = w & 0x0F0F0F0Fu;         // codes 0,2,4,6 in bytes 0..3
  const uint32_t od = (w >> 4) & 0x0F0F0F0Fu;  // codes 1,3,5,7
#pragma unroll
  for (int k = 0; k < 4; ++k)
    o[k] = pack_exact((float)((ev >> (8 * k)) & 0xFFu), (float)((od >> (8 * k)) & 0xFFu));
}

// 4 eight-bit codes of one word -> 2 dwords of exact bf16 pairs.
__device__ __forceinline__ void unpack8(uint32_t w, uint32_t *o) {
  o[0] = pack_exact((float)(w & 0xFFu), (float)((w >> 8) & 0xFFu));
  o[1] = pack_exact((float)((w >> 16) & 0xFFu), (float)(w >> 24));
}

template <int BITS>
__device__ __forceinline__ uint32_t code_at(const uint32_t *row, int d) {
  constexpr int PER = 32 / BITS;
  return (row[d / PER] >> (BITS * (d % PER))) & ((1u << BITS) - 1u);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// ---------------------------------------------------------------------------
// Token compaction: idx[r] = t of the r-th supervised token, inv[t] = r or -1.
// One workgroup of 1024 threads scans the mask in order (ballot + popcount).
__global__ void __launch_bounds__(1024) k_compact(const uint8_t *mask, int M, int M_pad,
                                                   int *idx, int *inv, int *cnt) {
  __shared__ int wsum[16];
  __shared__ int base;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) base = 0;
  __syncthreads();
  for (int c0 = 0; c0 < M; c0 += 1024) {
    const int t = c0 + tid;
    const int f = (t < M) ? (mask ? (mask[t] != 0) : 1) : 0;
    const uint64_t b = __ballot(f);
    const int pre = __popcll(b & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wave] = __popcll(b);
    __syncthreads();
    int woff = 0, total = 0;
    for (int w = 0; w < 16; ++w) {
      woff += (w < wave) ? wsum[w] : 0;
      total += wsum[w];
    }
    const int r = base + woff + pre;
    if (t < M) {
      inv[t] = f ? r : -1;
      if (f) idx[r] = t;
    }
    __syncthreads();
    if (tid == 0) base += total;
    __syncthreads();
  }
  const int me = base;
  for (int r = me + tid; r < M_pad; r += 1024) idx[r] = -1;
  if (tid == 0) cnt[0] = me;
}

// ---------------------------------------------------------------------------
// Per compacted row: gather h, write the augmented row [bias block | h] and the
// token record.  Bias block column kk (part = kk / G, gi = kk % G):
// part 0 -> S_hi[gi], 1 -> S_lo[gi], 2 -> S_hi[gi], else 0.
__global__ void __launch_bounds__(256) k_prep(const uint16_t *h, int H, int G, int Kb, int Ka,
                                              const int *idx, const int32_t *targets,
                                              const float *lse, const float *g, TokRec *tok,
                                              uint16_t *haug) {
  __shared__ float sS[MAX_G];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int src = idx[r];
  uint16_t *dst = haug + (size_t)r * Ka;
  for (int gg = wave; gg < G; gg += 4) {
    const int d = gg * KSTEP + lane;
    const uint16_t x = (src >= 0) ? h[(size_t)src * H + d] : (uint16_t)0;
    dst[Kb + d] = x;
    const float s = wave_sum(bf16_to_f32(x));
    if (lane == 0) sS[gg] = s;
  }
  __syncthreads();
  for (int kk = tid; kk < Kb; kk += NTHREADS) {
    const int part = kk / G, gi = kk - part * G;
    uint32_t val = 0;
    if (part < 3) {
      const float S = sS[gi];
      const uint32_t hi = bf16_rne(S);
      val = (part == 1) ? bf16_rne(S - bf16_to_f32(hi)) : hi;
    }
    dst[kk] = (uint16_t)val;
  }
  if (tid == 0) {
    TokRec rec;
    rec.lse = (src >= 0 && lse) ? lse[src] : 0.0f;
    rec.g = (src >= 0) ? (g ? g[src] : 1.0f) : 0.0f;
    rec.tval = 0.0f;
    rec.tgt = (src >= 0) ? targets[src] : -1;
    tok[r] = rec;
  }
}

// ---------------------------------------------------------------------------
// Target logit of each compacted row, in fp32 straight from the packed row:
// z = sum_g (s * sum_{d in g} h_d q_d + b * S_g).  One wave per row.
// Forward: tval = c(z).  Backward: tval = g * (1 - exp(c(z) - lse)) * c'(z),
// the target column's coefficient.
template <int BITS>
__global__ void __launch_bounds__(256) k_target(const uint16_t *haug, int Ka, int Kb, int H, int G,
                                                const uint32_t *wq, int wpr, const float *scales,
                                                const float *biases, int64_t V, float cap,
                                                const int *cnt, TokRec *tok, int M_pad, int bwd) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= M_pad) return;
  const int tgt = tok[r].tgt;
  float out = 0.0f;
  if (r < cnt[0] && tgt >= 0 && (int64_t)tgt < V) {
    float part = 0.0f;
    const uint32_t *wrow = wq + (size_t)tgt * wpr;
    const uint16_t *hrow = haug + (size_t)r * Ka + Kb;
    for (int gg = lane; gg < G; gg += 64) {
      float A = 0.0f, S = 0.0f;
      for (int d = gg * KSTEP; d < gg * KSTEP + KSTEP; ++d) {
        const float x = bf16_to_f32(hrow[d]);
        A += x * (float)code_at<BITS>(wrow, d);
        S += x;
      }
      part += scales[(size_t)tgt * G + gg] * A + biases[(size_t)tgt * G + gg] * S;
    }
    const float z = wave_sum(part);
    float y = z, dc = 1.0f;
    if (cap > 0.0f) {
      const float th = tanhf(z / cap);
      y = cap * th;
      dc = 1.0f - th * th;
    }
    out = bwd ? tok[r].g * -expm1f(y - tok[r].lse) * dc : y;
  }
  if (lane == 0) tok[r].tval = out;
}

// ---------------------------------------------------------------------------
// The logit tile: 256 tokens x 128 vocabulary rows per workgroup, K = Ka
// (bias block, then H).  Wave w owns tokens [64w, 64w+64) of the tile; the
// code tile is shared through LDS (double buffered, one group per step), the
// token operand is loaded straight from the augmented rows.
struct TileArgs {
  const uint16_t *haug;  // [M_pad][Ka] bf16
  const uint32_t *wq;
  const float *scales;
  const float *biases;
  const int *cnt;
  const TokRec *tok;
  float *part;           // forward: [gridDim.y][M_pad] x (max, sumexp)
  uint16_t *coeff;       // backward: [M_pad][ld_coeff] bf16 coefficient chunk
  int64_t ld_coeff;
  int64_t V;
  int G, Ka, NB, wpr, M_pad;
  int range_tile0, range_tiles, tiles_per_wg;
  float cap;
};

template <int BITS>
struct Producer {
  // Thread tid stages row tid/2, K half tid%2 (32 codes) of each step.
  static constexpr int NW = BITS;  // words per thread per step (32 codes)
  uint32_t w[NW];
  float s;

  __device__ __forceinline__ void load(const TileArgs &a, int64_t v0, int step, int prow, int phalf) {
    const int64_t v = v0 + prow;
    const bool ok = v < a.V;
    if (step >= a.NB) {
      const int g = step - a.NB;
      const uint32_t *src = a.wq + (size_t)v * a.wpr + g * (2 * BITS) + phalf * BITS;
#pragma unroll
      for (int i = 0; i < NW; i += 4) {
        const u32x4_t x = ok ? *(const u32x4_t *)(src + i) : u32x4_t{0, 0, 0, 0};
        w[i] = x[0]; w[i + 1] = x[1]; w[i + 2] = x[2]; w[i + 3] = x[3];
      }
      s = (ok && phalf == 0) ? a.scales[(size_t)v * a.G + g] : 0.0f;
    }
  }

  __device__ __forceinline__ void store(const TileArgs &a, int64_t v0, int step, int prow, int phalf,
                                        uint16_t *sw, float *ss) {
    uint32_t o[16];
    if (step >= a.NB) {
      if (BITS == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) unpack4(w[i], o + 4 * i);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) unpack8(w[i], o + 2 * i);
      }
      if (phalf == 0) ss[prow] = s;
    } else {
      // bias block chunk: hi/lo splits of the fp32 biases (part 0,1 -> hi; 2 -> lo)
      const int64_t v = v0 + prow;
      const bool ok = v < a.V;
      const float *brow = a.biases + (size_t)v * a.G;
#pragma unroll 4
      for (int e = 0; e < 32; e += 2) {
        uint32_t pr[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int kk = step * KSTEP + phalf * 32 + e + u;
          const int part = kk / a.G, gi = kk - part * a.G;
          uint32_t val = 0;
          if (ok && part < 3) {
            const float b = brow[gi];
            const uint32_t hi = bf16_rne(b);
            val = (part == 2) ? bf16_rne(b - bf16_to_f32(hi)) : hi;
          }
          pr[u] = val;
        }
        o[e / 2] = pr[0] | (pr[1] << 16);
      }
    }
    uint16_t *dst = sw + prow * WROW + phalf * 32;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(u32x4_t *)(dst + 8 * i) = u32x4_t{o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
  }
};

template <int BITS, bool BWD>
__global__ void __launch_bounds__(NTHREADS, 1) k_tile(TileArgs a) {
  const int tt = blockIdx.x;
  if (tt * BM >= a.cnt[0]) return;
  const int wr = blockIdx.y;
  const int tile_begin = wr * a.tiles_per_wg;
  const int tile_end = min(tile_begin + a.tiles_per_wg, a.range_tiles);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int prow = tid >> 1, phalf = tid & 1;
  const int steps = a.NB + a.G;

  __shared__ __attribute__((aligned(16))) uint16_t sW[2][BN * WROW];
  __shared__ __attribute__((aligned(16))) float sS[2][BN];

  const int tok0 = tt * BM + wave * 64;
  const uint16_t *hp[4];
#pragma unroll
  for (int ti = 0; ti < 4; ++ti) hp[ti] = a.haug + (size_t)(tok0 + ti * 16 + l16) * a.Ka + lq * 8;

  float run_m[4], run_s[4];
  float lse_t[4], g_t[4];
  int64_t tgt_t[4];
#pragma unroll
  for (int ti = 0; ti < 4; ++ti) {
    run_m[ti] = -INFINITY;
    run_s[ti] = 0.0f;
    if (BWD) {
      const TokRec rec = a.tok[tok0 + ti * 16 + l16];
      lse_t[ti] = rec.lse;
      g_t[ti] = rec.g;
      tgt_t[ti] = rec.tgt;
    }
  }

  Producer<BITS> pr;
  for (int tile = tile_begin; tile < tile_end; ++tile) {
    const int64_t v0 = (int64_t)(a.range_tile0 + tile) * BN;
    f32x4_t acc[8][4];
#pragma unroll
    for (int vi = 0; vi < 8; ++vi)
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) acc[vi][ti] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    bf16x8_t bcur[4][2], bnext[4][2];
    pr.load(a, v0, 0, prow, phalf);
    pr.store(a, v0, 0, prow, phalf, sW[0], sS[0]);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) bcur[ti][ks] = *(const bf16x8_t *)(hp[ti] + ks * 32);
    __syncthreads();

    for (int st = 0; st < steps; ++st) {
      const int cb = st & 1;
      const bool more = st + 1 < steps;
      if (more) {
        pr.load(a, v0, st + 1, prow, phalf);
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            bnext[ti][ks] = *(const bf16x8_t *)(hp[ti] + (st + 1) * KSTEP + ks * 32);
      }
      const uint16_t *sw = sW[cb];
      if (st < a.NB) {
#pragma unroll
        for (int vi = 0; vi < 8; ++vi) {
          const bf16x8_t a0 = *(const bf16x8_t *)(sw + (vi * 16 + l16) * WROW + lq * 8);
          const bf16x8_t a1 = *(const bf16x8_t *)(sw + (vi * 16 + l16) * WROW + 32 + lq * 8);
#pragma unroll
          for (int ti = 0; ti < 4; ++ti) {
            acc[vi][ti] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bcur[ti][0], acc[vi][ti], 0, 0, 0);
            acc[vi][ti] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bcur[ti][1], acc[vi][ti], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int vi = 0; vi < 8; ++vi) {
          const bf16x8_t a0 = *(const bf16x8_t *)(sw + (vi * 16 + l16) * WROW + lq * 8);
          const bf16x8_t a1 = *(const bf16x8_t *)(sw + (vi * 16 + l16) * WROW + 32 + lq * 8);
          const f32x4_t sc = *(const f32x4_t *)(sS[cb] + vi * 16 + lq * 4);
#pragma unroll
          for (int ti = 0; ti < 4; ++ti) {
            f32x4_t t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bcur[ti][0], f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bcur[ti][1], t, 0, 0, 0);
            acc[vi][ti] += sc * t;
          }
        }
      }
      if (more) {
        pr.store(a, v0, st + 1, prow, phalf, sW[cb ^ 1], sS[cb ^ 1]);
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) bcur[ti][ks] = bnext[ti][ks];
      }
      __syncthreads();
    }

    // ---- epilogue: acc[vi][ti][j] is the logit of vocab row v0 + vi*16 + lq*4 + j
    //      and token tok0 + ti*16 + l16.
    const float cap = a.cap;
    if (!BWD) {
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        float tmax = -INFINITY;
#pragma unroll
        for (int vi = 0; vi < 8; ++vi)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int64_t v = v0 + vi * 16 + lq * 4 + j;
            float y = acc[vi][ti][j];
            if (cap > 0.0f) y = cap * tanhf(y / cap);
            y = (v < a.V) ? y : -INFINITY;
            acc[vi][ti][j] = y;
            tmax = fmaxf(tmax, y);
          }
        const float mnew = fmaxf(run_m[ti], tmax);
        if (mnew == -INFINITY) continue;
        float ssum = 0.0f;
#pragma unroll
        for (int vi = 0; vi < 8; ++vi)
#pragma unroll
          for (int j = 0; j < 4; ++j) ssum += __expf(acc[vi][ti][j] - mnew);
        run_s[ti] = run_s[ti] * __expf(run_m[ti] - mnew) + ssum;
        run_m[ti] = mnew;
      }
    } else {
      const int64_t col0 = (int64_t)tile * BN;  // chunk-local coefficient column of this tile
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        uint16_t *crow = a.coeff + (size_t)(tok0 + ti * 16 + l16) * a.ld_coeff + col0;
#pragma unroll
        for (int p2 = 0; p2 < 4; ++p2) {
          float c[8];
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int vi = 2 * p2 + h2;
              const int64_t v = v0 + vi * 16 + lq * 4 + j;
              const float z = acc[vi][ti][j];
              float y = z, dc = 1.0f;
              if (cap > 0.0f) {
                const float th = tanhf(z / cap);
                y = cap * th;
                dc = 1.0f - th * th;
              }
              // -g * softmax * c'; the target column is left out here and its
              // whole term g * (1 - p) * c' * w is added in fp32 by k_dh_reduce.
              const float val = -g_t[ti] * __expf(y - lse_t[ti]) * dc;
              c[h2 * 4 + j] = (v < a.V && v != tgt_t[ti]) ? val : 0.0f;
            }
          // packet (p2, lq): rows {32*p2 + 4*lq + 0..3} then {32*p2 + 16 + 4*lq + 0..3}
          *(u32x4_t *)(crow + (p2 * 4 + lq) * 8) =
              u32x4_t{pack_rne(c[0], c[1]), pack_rne(c[2], c[3]), pack_rne(c[4], c[5]), pack_rne(c[6], c[7])};
        }
      }
    }
  }

  if (!BWD) {
    // merge the 4 lanes (lq = 0..3) that share a token column
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      float m = run_m[ti], s = run_s[ti];
#pragma unroll
      for (int o = 16; o <= 32; o <<= 1) {
        const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
        const float mn = fmaxf(m, m2);
        if (mn != -INFINITY) {
          s = s * __expf(m - mn) + s2 * __expf(m2 - mn);
          m = mn;
        }
      }
      if (lq == 0) {
        float *dst = a.part + ((size_t)wr * a.M_pad + tok0 + ti * 16 + l16) * 2;
        dst[0] = m;
        dst[1] = s;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Cross-split merge (page "mlx-bun 0.0.4 -> 0.0.6", flashCceForward's host
// merge): lse = m* + log sum_s s_s exp(m_s - m*), logp = target logit - lse.
__global__ void __launch_bounds__(256) k_merge(const float *part, int nsplit, int M_pad, const int *inv,
                                               const TokRec *tok, int M, float *logp, float *lse) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= M) return;
  const int r = inv[t];
  if (r < 0) {
    logp[t] = 0.0f;
    lse[t] = 0.0f;
    return;
  }
  float mx = -INFINITY;
  for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, part[((size_t)s * M_pad + r) * 2]);
  float se = 0.0f;
  for (int s = 0; s < nsplit; ++s) {
    const float m = part[((size_t)s * M_pad + r) * 2];
    if (m != -INFINITY) se += part[((size_t)s * M_pad + r) * 2 + 1] * __expf(m - mx);
  }
  const float l = mx + logf(se);
  lse[t] = l;
  logp[t] = tok[r].tval - l;
}

// ---------------------------------------------------------------------------
// dh contraction: dh_part[k][t][d] (+)= sum_v coeff[t][v] * bf16(s*q + b)[v][d]
// over the vocabulary rows of split k of one coefficient chunk.  Workgroup:
// 256 tokens x 128 dh columns; wave w owns tokens [64w, 64w+64).  The head
// tile is dequantized once into LDS as [d][v] (v contiguous, in the packet
// order the coefficient producer writes), the coefficient operand is loaded
// straight from the chunk.
struct GemmArgs {
  const uint16_t *coeff;
  int64_t ld_coeff;
  const uint32_t *wq;
  const float *scales;
  const float *biases;
  const int *cnt;
  float *dh_part;        // [ksplit][M_pad][H]
  int64_t V;
  int H, G, wpr, M_pad;
  int chunk_tile0, chunk_tiles, tiles_per_split;
  int accumulate;
};

template <int BITS>
__global__ void __launch_bounds__(NTHREADS, 1) k_dh_gemm(GemmArgs a) {
  constexpr int KST = (BITS == 4) ? 128 : 64;   // vocabulary rows per K step
  constexpr int SPT = BN / KST;                  // K steps per vocab tile
  constexpr int BROW = KST + 8;                  // padded LDS row stride (bf16)
  constexpr int NPK = KST / 8;                   // packets per step
  constexpr int WC = NTHREADS / NPK;             // word columns staged per step
  constexpr int DPW = 32 / BITS;                 // dh columns per word

  const int tt = blockIdx.x;
  if (tt * BM >= a.cnt[0]) return;
  const int d0 = blockIdx.y * DT;
  const int ks_ = blockIdx.z;
  const int tile_begin = ks_ * a.tiles_per_split;
  const int tile_end = min(tile_begin + a.tiles_per_split, a.chunk_tiles);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;

  __shared__ __attribute__((aligned(16))) uint16_t sB[2][DT * BROW];

  const int tok0 = tt * BM + wave * 64;
  const uint16_t *cp[4];
#pragma unroll
  for (int ti = 0; ti < 4; ++ti) cp[ti] = a.coeff + (size_t)(tok0 + ti * 16 + l16) * a.ld_coeff + lq * 8;

  f32x4_t acc[4][8];
#pragma unroll
  for (int ti = 0; ti < 4; ++ti)
#pragma unroll
    for (int di = 0; di < 8; ++di) acc[ti][di] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // producer: packet pk (8 vocab rows), word column wc (DPW consecutive d)
  const int pk = tid / WC, wc = tid % WC;
  const int dcol = wc * DPW;                 // first local dh column of the word
  const bool dok = d0 + dcol < a.H;
  const int gq = (d0 + dcol) / KSTEP;        // quantization group of these columns

  const int nsteps = (tile_end - tile_begin) * SPT;
  uint32_t wv[8];
  float sv[8], bv[8];

  auto load_step = [&](int step) {
    const int tile = tile_begin + step / SPT, half = step % SPT;
    const int64_t vb = (int64_t)(a.chunk_tile0 + tile) * BN;
    const int P = half * NPK + pk;           // packet index within the vocab tile
    const int rowA = 32 * (P / 4) + 4 * (P % 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t v = vb + rowA + (e < 4 ? e : 12 + e);
      const bool ok = dok && v < a.V;
      wv[e] = ok ? a.wq[(size_t)v * a.wpr + (d0 + dcol) / DPW] : 0u;
      sv[e] = ok ? a.scales[(size_t)v * a.G + gq] : 0.0f;
      bv[e] = ok ? a.biases[(size_t)v * a.G + gq] : 0.0f;
    }
  };
  auto store_step = [&](uint16_t *sb) {
#pragma unroll
    for (int k = 0; k < DPW; ++k) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t q = (wv[e] >> (BITS * k)) & ((1u << BITS) - 1u);
        x[e] = sv[e] * (float)q + bv[e];
      }
      *(u32x4_t *)(sb + (dcol + k) * BROW + pk * 8) =
          u32x4_t{pack_rne(x[0], x[1]), pack_rne(x[2], x[3]), pack_rne(x[4], x[5]), pack_rne(x[6], x[7])};
    }
  };

  if (nsteps > 0) {
    bf16x8_t acur[4][KST / 32], anext[4][KST / 32];
    load_step(0);
    store_step(sB[0]);
    {
      const int64_t cc = (int64_t)tile_begin * BN;
#pragma unroll
      for (int ti = 0; ti < 4; ++ti)
#pragma unroll
        for (int ks = 0; ks < KST / 32; ++ks) acur[ti][ks] = *(const bf16x8_t *)(cp[ti] + cc + ks * 32);
    }
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
      const int cb = st & 1;
      const bool more = st + 1 < nsteps;
      if (more) {
        load_step(st + 1);
        const int64_t cc = (int64_t)tile_begin * BN + (int64_t)(st + 1) * KST;
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
          for (int ks = 0; ks < KST / 32; ++ks) anext[ti][ks] = *(const bf16x8_t *)(cp[ti] + cc + ks * 32);
      }
      const uint16_t *sb = sB[cb];
#pragma unroll
      for (int ks = 0; ks < KST / 32; ++ks) {
#pragma unroll
        for (int di = 0; di < 8; ++di) {
          const bf16x8_t b = *(const bf16x8_t *)(sb + (di * 16 + l16) * BROW + ks * 32 + lq * 8);
#pragma unroll
          for (int ti = 0; ti < 4; ++ti)
            acc[ti][di] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(acur[ti][ks], b, acc[ti][di], 0, 0, 0);
        }
      }
      if (more) {
        store_step(sB[cb ^ 1]);
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
          for (int ks = 0; ks < KST / 32; ++ks) acur[ti][ks] = anext[ti][ks];
      }
      __syncthreads();
    }
  } else if (a.accumulate) {
    return;
  }

  // result lane layout: column d0 + di*16 + l16, rows tok0 + ti*16 + lq*4 + j
#pragma unroll
  for (int ti = 0; ti < 4; ++ti)
#pragma unroll
    for (int di = 0; di < 8; ++di) {
      const int d = d0 + di * 16 + l16;
      if (d >= a.H) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float *dst = a.dh_part + ((size_t)ks_ * a.M_pad + tok0 + ti * 16 + lq * 4 + j) * a.H + d;
        *dst = a.accumulate ? (*dst + acc[ti][di][j]) : acc[ti][di][j];
      }
    }
}

// ---------------------------------------------------------------------------
// dh[t][:] = sum_k dh_part[k][r][:] + tval * w[target][:] (fp32 dequant),
// zero rows for masked tokens.
template <int BITS>
__global__ void __launch_bounds__(256) k_dh_reduce(const float *dh_part, int ksplit, int M_pad, int H, int G,
                                                   const int *inv, const TokRec *tok, const uint32_t *wq,
                                                   int wpr, const float *scales, const float *biases,
                                                   int64_t V, float *dh) {
  const int t = blockIdx.x;
  const int d = blockIdx.y * 256 + threadIdx.x;
  if (d >= H) return;
  const int r = inv[t];
  float acc = 0.0f;
  if (r >= 0) {
    for (int k = 0; k < ksplit; ++k) acc += dh_part[((size_t)k * M_pad + r) * H + d];
    const TokRec rec = tok[r];
    if (rec.tgt >= 0 && (int64_t)rec.tgt < V) {
      const size_t gi = (size_t)rec.tgt * G + d / KSTEP;
      const float q = (float)code_at<BITS>(wq + (size_t)rec.tgt * wpr, d);
      acc += rec.tval * (scales[gi] * q + biases[gi]);
    }
  }
  dh[(size_t)t * H + d] = acc;
}

}  // namespace cce
