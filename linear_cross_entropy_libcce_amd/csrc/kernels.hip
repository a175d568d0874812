// kernels.hip -- the small kernels of libcce (compaction, prep, target logit,
// merge, split reduce).
#include "cce_device.h"

namespace cce {

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
// Per compacted row r: gather h, write the augmented row [bias block | h] in
// fragment-major layout, and the token record.  Bias block column kk
// (part = kk / G, gi = kk % G): part 0 -> 256 S_hi[gi], 1 -> 256 S_lo[gi],
// 2 -> S_hi[gi], else 0, with S = per-group sum of h split into bf16 hi + lo
// (the head side holds the matching fixed-point digits of the biases).  h rows
// are 16-byte aligned.
__global__ void __launch_bounds__(256) k_prep(const uint16_t *h, int H, int G, int Kb, int Ka,
                                              const int *idx, const int32_t *targets,
                                              const float *lse, const float *g, TokRec *tok,
                                              uint16_t *haug) {
  __shared__ float sS[MAX_G];
  const int r = blockIdx.x, tid = threadIdx.x;
  const int src = idx[r];
  const int64_t ks16 = Ka / 16;
  const int nch = H / 8;  // 16-byte chunks of the h part; 8 per group
  for (int c = tid; c < nch; c += 256) {
    const u32x4_t x = (src >= 0) ? *(const u32x4_t *)(h + (size_t)src * H + 8 * c) : u32x4_t{0, 0, 0, 0};
    *(u32x4_t *)(haug + frag_slot(r, Kb / 8 + c, ks16)) = x;
    float part = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) part += bf16_to_f32(x[e] & 0xFFFFu) + bf16_to_f32(x[e] >> 16);
    // the 8 chunks of one group sit in 8 consecutive lanes
    part += __shfl_xor(part, 1, 8);
    part += __shfl_xor(part, 2, 8);
    part += __shfl_xor(part, 4, 8);
    if ((c & 7) == 0) sS[c >> 3] = part;
  }
  __syncthreads();
  for (int c = tid; c < Kb / 8; c += 256) {
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t pr2[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int kk = 8 * c + 2 * e + u;
        const int part = kk / G, gi = kk - part * G;
        uint32_t val = 0;
        if (part < 3) {
          const float S = sS[gi];
          const uint32_t hi = bf16_rne(S);
          const float x = (part == 1) ? 256.0f * (S - bf16_to_f32(hi)) : bf16_to_f32(hi) * (part == 0 ? 256.0f : 1.0f);
          val = bf16_rne(x);
        }
        pr2[u] = val;
      }
      o[e] = pr2[0] | (pr2[1] << 16);
    }
    *(u32x4_t *)(haug + frag_slot(r, c, ks16)) = u32x4_t{o[0], o[1], o[2], o[3]};
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
__global__ void __launch_bounds__(256) k_target(const uint16_t *h, const int *idx, int H, int G,
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
    const uint16_t *hrow = h + (size_t)idx[r] * H;
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
// Cross-split merge (page "mlx-bun 0.0.4 -> 0.0.6", flashCceForward's host
// merge): lse = m* + log sum_s s_s exp(m_s - m*), logp = target logit - lse.
__global__ void __launch_bounds__(256) k_merge(const float *part, int nblocks, int tiles, int max_splits,
                                               int M_pad, const int *inv, const int *cnt, const TokRec *tok,
                                               int M, float *logp, float *lse) {
  // two partials (vocabulary halves of the tile) per split of the forward
  const int nsplit = 2 * splits_for(nblocks, active_tiles(cnt), tiles, max_splits);
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
// Pair flags of the backward skips (page "mlx-bun 0.0.4 -> 0.0.6",
// src/train/flash-cce.ts, the block early exit of the backward kernels): the
// (token tile tt, vocabulary tile b) pair is needed unless, for every
// supervised token of the tile, block_max - lse < log(eps) and the target is
// outside the tile.  block_on = 0 marks every pair needed (filter only).
// Workgroup: one token tile x 64 vocabulary tiles; thread (b = tid % 64,
// quarter = tid / 64) scans every fourth token of the tile, the quarters are
// OR-ed through LDS.  Reads of block_max are 64 consecutive floats per wave.
__global__ void __launch_bounds__(256) k_warm(const int *cnt, const int *idx, const TokRec *tok, const float *bmx,
                                              int64_t nbv, int64_t tiles, float log_eps, int block_on, uint8_t *fl) {
  __shared__ int sW[4][64];
  const int64_t nbc = (tiles + 63) / 64;
  const int tt = (int)(blockIdx.x / nbc);
  const int n = cnt[0];
  if (tt * BM >= n) return;
  const int bl = threadIdx.x & 63, qt = threadIdx.x >> 6;
  const int64_t b = (int64_t)(blockIdx.x % nbc) * 64 + bl;
  int warm = block_on ? 0 : 1;
  if (block_on && b < tiles) {
    const int64_t lo = b * BNT;
    for (int j = qt; j < BM; j += 4) {
      const int r = tt * BM + j;
      if (r >= n) break;
      const TokRec rec = tok[r];
      const bool hot = bmx[(int64_t)idx[r] * nbv + b] - rec.lse >= log_eps;
      const bool holds = rec.tgt >= lo && rec.tgt < lo + BNT;
      if (hot || holds) {
        warm = 1;
        break;
      }
    }
  }
  sW[qt][bl] = warm;
  __syncthreads();
  if (qt == 0 && b < tiles)
    fl[(int64_t)tt * tiles + b] = (uint8_t)(sW[0][bl] | sW[1][bl] | sW[2][bl] | sW[3][bl]);
}

// block_max rows of masked tokens are 0.
__global__ void __launch_bounds__(256) k_bmx_mask(int64_t nbv, const int *inv, float *bmx) {
  const int64_t nbc = (nbv + 255) / 256;
  const int t = (int)(blockIdx.x / nbc);
  const int64_t b = (int64_t)(blockIdx.x % nbc) * 256 + threadIdx.x;
  if (b < nbv && inv[t] < 0) bmx[(int64_t)t * nbv + b] = 0.0f;
}

// ---------------------------------------------------------------------------
// dh[t][:] = sum_k dh_part[k][r][:] + tval * w[target][:] (fp32 dequant),
// zero rows for masked tokens.
template <int BITS>
__global__ void __launch_bounds__(256) k_dh_reduce(GemmArgs a, const int *inv, const TokRec *tok, float *dh) {
  const int t = blockIdx.x;
  const int d = blockIdx.y * 256 + threadIdx.x;
  const int H = a.H;
  if (d >= H) return;
  const int r = inv[t];
  float acc = 0.0f;
  if (r >= 0) {
    const int act = active_tiles(a.cnt);
    int ksd, steps_per;
    dh_split(a, act, ksd, steps_per);
    for (int k = 0; k < ksd; ++k) acc += a.dh_part[((size_t)k * act * BM + r) * H + d];
    const TokRec rec = tok[r];
    if (rec.tgt >= 0 && (int64_t)rec.tgt < a.V) {
      const size_t gi = (size_t)rec.tgt * a.G + d / KSTEP;
      const float q = (float)code_at<BITS>(a.wq + (size_t)rec.tgt * a.wpr, d);
      acc += rec.tval * (a.scales[gi] * q + a.biases[gi]);
    }
  }
  dh[(size_t)t * H + d] = acc;
}

void launch_compact(hipStream_t st, const uint8_t *mask, int M, int M_pad, int *idx, int *inv, int *cnt) {
  hipLaunchKernelGGL(k_compact, dim3(1), dim3(1024), 0, st, mask, M, M_pad, idx, inv, cnt);
}

void launch_prep(hipStream_t st, int M_pad, const uint16_t *h, int H, int G, int Kb, int Ka, const int *idx,
                 const int32_t *targets, const float *lse, const float *g, TokRec *tok, uint16_t *haug) {
  hipLaunchKernelGGL(k_prep, dim3((unsigned)M_pad), dim3(256), 0, st, h, H, G, Kb, Ka, idx, targets, lse, g, tok,
                     haug);
}

void launch_target(hipStream_t st, int bits, int M_pad, const uint16_t *h, const int *idx, int H, int G,
                   const uint32_t *wq, int wpr, const float *scales, const float *biases, int64_t V, float cap,
                   const int *cnt, TokRec *tok, int bwd) {
  const dim3 grid((unsigned)((M_pad + 3) / 4));
  if (bits == 4)
    hipLaunchKernelGGL(k_target<4>, grid, dim3(256), 0, st, h, idx, H, G, wq, wpr, scales, biases, V, cap,
                       cnt, tok, M_pad, bwd);
  else
    hipLaunchKernelGGL(k_target<8>, grid, dim3(256), 0, st, h, idx, H, G, wq, wpr, scales, biases, V, cap,
                       cnt, tok, M_pad, bwd);
}

void launch_merge(hipStream_t st, int M, const float *part, int nblocks, int tiles, int max_splits, int M_pad,
                  const int *inv, const int *cnt, const TokRec *tok, float *logp, float *lse) {
  hipLaunchKernelGGL(k_merge, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, st, part, nblocks, tiles, max_splits,
                     M_pad, inv, cnt, tok, M, logp, lse);
}

void launch_warm(hipStream_t st, int TT, int64_t tiles, const int *cnt, const int *idx, const TokRec *tok,
                 const float *bmx, int64_t nbv, float log_eps, int block_on, uint8_t *fl) {
  const dim3 grid((unsigned)(((tiles + 63) / 64) * TT));
  hipLaunchKernelGGL(k_warm, grid, dim3(256), 0, st, cnt, idx, tok, bmx, nbv, tiles, log_eps, block_on, fl);
}

void launch_bmx_mask(hipStream_t st, int M, int64_t nbv, const int *inv, float *bmx) {
  const dim3 grid((unsigned)(((nbv + 255) / 256) * M));
  hipLaunchKernelGGL(k_bmx_mask, grid, dim3(256), 0, st, nbv, inv, bmx);
}

void launch_dh_reduce(hipStream_t st, int bits, int M, const GemmArgs &ga, const int *inv, const TokRec *tok,
                      float *dh) {
  const dim3 grid((unsigned)M, (unsigned)((ga.H + 255) / 256));
  if (bits == 4)
    hipLaunchKernelGGL(k_dh_reduce<4>, grid, dim3(256), 0, st, ga, inv, tok, dh);
  else
    hipLaunchKernelGGL(k_dh_reduce<8>, grid, dim3(256), 0, st, ga, inv, tok, dh);
}

}  // namespace cce
