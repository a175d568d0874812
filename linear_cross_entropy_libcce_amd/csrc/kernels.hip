// kernels.hip -- the small kernels of libcce (compaction, prep, target logit,
// merge, split reduce) and the dh contraction.
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
// 256 tokens x 128 dh columns; wave w owns tokens [64w, 64w+64) as 2 x 4
// blocks of v_mfma_f32_32x32x16_bf16 (rows = tokens, columns = d).  The head
// tile is dequantized once per step into LDS as [d][v] (v contiguous); the
// coefficient operand is loaded straight from the chunk into registers.

template <int BITS>
__global__ void __launch_bounds__(NTHREADS, 2) k_dh_gemm(GemmArgs a) {
  constexpr int KST = 64;                        // vocabulary rows per K step
  constexpr int SPT = BN / KST;                  // K steps per 128-row vocab tile
  constexpr int BROW = KST + 8;                  // padded LDS row stride (bf16)
  constexpr int RPT = 4;                         // vocabulary rows staged per thread
  constexpr int NRG = KST / RPT;                 // row groups per step
  constexpr int WC = NTHREADS / NRG;             // 8-column groups of d staged per step
  constexpr int DPW = 32 / BITS;                 // dh columns per word
  constexpr int WPT = 8 / DPW;                   // words per row per thread (8 columns of d)
  constexpr int NKS = KST / 16;                  // MFMA k-steps per K step
  static_assert(WC * 8 == DT, "each thread stages 8 columns of the dh tile");

  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  if (bid >= a.nblocks) return;
  const int ks_ = bid % a.ksplit;
  const int dt = (bid / a.ksplit) % a.HT;
  const int tt = bid / (a.ksplit * a.HT);
  if (tt * BM >= a.cnt[0]) return;
  const int d0 = dt * DT;
  const int tile_begin = ks_ * a.tiles_per_split;
  const int tile_end = min(tile_begin + a.tiles_per_split, a.chunk_tiles);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, lh = lane >> 5;

  __shared__ __attribute__((aligned(16))) uint16_t sB[2][DT * BROW];

  const int tok0 = tt * BM + wave * 64;
  // fragment-major coefficient chunk: one 1 KiB block per (32 tokens, 16 vocab rows)
  const int64_t ksv = a.ld_coeff / 16;
  const uint16_t *cp0 = a.coeff + ((size_t)(tok0 >> 5) * ksv * 64 + lane) * 8 + (size_t)tile_begin * (BN / 16) * 512;
  const uint16_t *cp1 = cp0 + (size_t)ksv * 512;

  f32x16_t acc[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[rb][c][e] = 0.0f;

  // producer: RPT consecutive vocabulary rows x 8 columns of d (WPT words per
  // row).  The row group varies fastest across lanes so that the LDS writes of
  // neighbouring lanes land side by side in one [d] row.
  const int rg = tid % NRG, wc = tid / NRG;
  const int dcol = wc * 8;
  const bool dok = d0 + dcol < a.H;
  const int gq = (d0 + dcol) / KSTEP;
  const int64_t wcol = (d0 + dcol) / DPW;

  const int nsteps = (tile_end - tile_begin) * SPT;
  uint32_t wv[RPT][WPT];
  float sv[RPT], bv[RPT];

  auto load_step = [&](int step) {
    const int64_t vb = (int64_t)(a.chunk_tile0 + tile_begin) * BN + (int64_t)step * KST + rg * RPT;
#pragma unroll
    for (int e = 0; e < RPT; ++e) {
      const int64_t v = vb + e;
      const bool ok = dok && v < a.V;
#pragma unroll
      for (int u = 0; u < WPT; ++u) wv[e][u] = ok ? a.wq[(size_t)v * a.wpr + wcol + u] : 0u;
      sv[e] = ok ? a.scales[(size_t)v * a.G + gq] : 0.0f;
      bv[e] = ok ? a.biases[(size_t)v * a.G + gq] : 0.0f;
    }
  };
  auto store_step = [&](uint16_t *sb) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float x[RPT];
#pragma unroll
      for (int e = 0; e < RPT; ++e) {
        const uint32_t q = (wv[e][k / DPW] >> (BITS * (k % DPW))) & ((1u << BITS) - 1u);
        x[e] = sv[e] * (float)q + bv[e];
      }
      *(uint2 *)(sb + (dcol + k) * BROW + rg * RPT) = make_uint2(pack_rne(x[0], x[1]), pack_rne(x[2], x[3]));
    }
  };

  if (nsteps > 0) {
    bf16x8_t cA[2][NKS];
    load_step(0);
    store_step(sB[0]);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      cA[0][ks] = *(const bf16x8_t *)(cp0 + ks * 512);
      cA[1][ks] = *(const bf16x8_t *)(cp1 + ks * 512);
    }
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
      const int cb = st & 1;
      const bool more = st + 1 < nsteps;
      if (more) load_step(st + 1);
      const uint16_t *sb = sB[cb] + l32 * BROW + lh * 8;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        bf16x8_t bq[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) bq[c] = *(const bf16x8_t *)(sb + c * 32 * BROW + ks * 16);
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            acc[rb][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cA[rb][ks], bq[c], acc[rb][c], 0, 0, 0);
        if (more) {
          cA[0][ks] = *(const bf16x8_t *)(cp0 + (size_t)((st + 1) * NKS + ks) * 512);
          cA[1][ks] = *(const bf16x8_t *)(cp1 + (size_t)((st + 1) * NKS + ks) * 512);
        }
      }
      if (more) store_step(sB[cb ^ 1]);
      __syncthreads();
    }
  } else if (a.accumulate) {
    return;
  }

  // result lane layout: column d0 + c*32 + l32, rows tok0 + rb*32 + 8i + 4*lh + j
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int d = d0 + c * 32 + l32;
      if (d >= a.H) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float *dst = a.dh_part + ((size_t)ks_ * a.M_pad + tok0 + rb * 32 + 8 * i + 4 * lh + j) * a.H + d;
          const float v = acc[rb][c][4 * i + j];
          *dst = a.accumulate ? (*dst + v) : v;
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

void launch_merge(hipStream_t st, int M, const float *part, int nsplit, int M_pad, const int *inv,
                  const TokRec *tok, float *logp, float *lse) {
  hipLaunchKernelGGL(k_merge, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, st, part, nsplit, M_pad, inv, tok, M,
                     logp, lse);
}

void launch_dh_gemm(hipStream_t st, int bits, dim3 grid, const GemmArgs &a) {
  if (bits == 4)
    hipLaunchKernelGGL(k_dh_gemm<4>, grid, dim3(NTHREADS), 0, st, a);
  else
    hipLaunchKernelGGL(k_dh_gemm<8>, grid, dim3(NTHREADS), 0, st, a);
}

void launch_dh_reduce(hipStream_t st, int bits, int M, const float *dh_part, int ksplit, int M_pad, int H, int G,
                      const int *inv, const TokRec *tok, const uint32_t *wq, int wpr, const float *scales,
                      const float *biases, int64_t V, float *dh) {
  const dim3 grid((unsigned)M, (unsigned)((H + 255) / 256));
  if (bits == 4)
    hipLaunchKernelGGL(k_dh_reduce<4>, grid, dim3(256), 0, st, dh_part, ksplit, M_pad, H, G, inv, tok, wq, wpr,
                       scales, biases, V, dh);
  else
    hipLaunchKernelGGL(k_dh_reduce<8>, grid, dim3(256), 0, st, dh_part, ksplit, M_pad, H, G, inv, tok, wq, wpr,
                       scales, biases, V, dh);
}

}  // namespace cce
