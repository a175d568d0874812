// kernels.hip -- the small kernels of libcce (compaction, front: token rows
// and head preparation, merge, pair flags of the skips, split reduce).
#include "cce_device.h"

namespace cce {

// ---------------------------------------------------------------------------
// Token compaction: idx[r] = t of the r-th supervised token, inv[t] = r or -1.
// One workgroup of 1024 threads scans the mask in order (ballot + popcount).
__global__ void __launch_bounds__(1024) k_compact(const uint8_t *mask, int M, int M_pad,
                                                   int *idx, int *inv, int *cnt, float *out_logp,
                                                   float *out_lse) {
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
      if (!f && out_logp) {
        out_logp[t] = 0.0f;
        out_lse[t] = 0.0f;
      }
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
// The front of every call, one launch (after the compaction):
//
// Workgroups [0, M_pad): compacted row r.  Gather h, write the augmented row
// [bias block | h] in fragment-major layout, the row's sum over groups of
// |S_g| and its token record (target id, or -1 when the target is outside
// [0, V); tval 0 -- the tile that owns the target's column fills it in).
//
// The bias block carries sum_g b'[v][g] * S[t][g] (S = per-group sum of h)
// with b' = b + 128 s for 8-bit heads, whose codes the tile uses as q - 128,
// and b' = b + 8 s for 4-bit heads (codes used as q - 8): symmetric heads have
// b' = 0.  Row v holds b' in fixed point, b' ~= u_v * n with
// u_v = max_g |b'| / BIAS_NMAX and n = 65536 d2 + 256 d1 + d0 (balanced signed
// digits, exact in bf16, stored as two's-complement bytes); the token side holds
// S = S1 + S2 + S3 (three bf16 pieces, each the rounding of what the
// previous ones leave).  The products that matter are MFMA columns, in two
// halves of P columns each (part = column / Gq within the half, group gi =
// column % Gq, zero past 3 Gq):
//
//   half 0, refinement:  d2 * 65536 S3 | d1 * 256 S2 | d0 * S1
//   half 1, coarse:      d2 * 65536 S1 | d2 * 65536 S2 | d1 * 256 S1
//
// Half 1 alone is b' to 16 bits (per-logit error <= 2^-15 max|b'| sum_g |S_g|);
// both halves to 24 bits (<= 2^-22 of the same); the tile chooses per token
// tile (see BIAS_COARSE_TOL) and starts at half 1 when half 0 is not needed.
//
// Workgroups [M_pad, M_pad + ceil(V / 64)): the head side, 64 rows each.
// Per-call head preparation (the head is frozen, so this depends on the head
// only):
//
// * The digits of the bias block and, per block of 64 rows, the largest |b'|
//   (fp32 bits; zero for a symmetric head, whose bias block is then skipped).
//   A block whose largest |b'| is 0 writes no digits: the tile reads such a
//   block's bias steps through an empty buffer resource, i.e. as zero bytes,
//   which are its digits (all zero).  A symmetric head's front so writes no
//   bias block at all.
// * Fold ratios of every step, rt[step][v]: 1 for the bias steps, then
//   u_v / s_0, s_0 / s_1, ... with effective scales, and s_last[v] = s_{G-1}.
// One workgroup per 64 rows.  Digits: when a row's group count is a multiple
// of 4 (and the scales and biases are aligned for it), four threads share a
// row, each taking 4 consecutive groups at a time with one vector load per
// operand: the row's max |b'| is a shuffle reduction over the four, and
// each set of 4 digits is one 32-bit store per column part.  Otherwise two flat
// passes: |b'| of every (row, group) with a shared-memory max per row, then
// the digits with lanes over consecutive (row, group) pairs and byte stores.
// Then the ratio table, whose layout is [step][V] (read that way by the
// tile): the scales of 64 groups at a time are staged in LDS with contiguous
// loads, then written with lanes over rows.
constexpr int HP_ROWS = 64, HP_COLS = 64, HP_LD = HP_COLS + 1;

// 4 consecutive scale or bias values from element i (i % 4 == 0, base aligned
// to 4 elements), widened to fp32.
__device__ __forceinline__ void ld_sb4(const void *base, int64_t i, int sbt, float *o) {
  if (sbt == SB_F32) {
    const f32x4_t x = *(const f32x4_t *)(static_cast<const float *>(base) + i);
    o[0] = x[0]; o[1] = x[1]; o[2] = x[2]; o[3] = x[3];
  } else {
    const uint2 w = *(const uint2 *)(static_cast<const uint16_t *>(base) + i);
    o[0] = sb_widen(w.x & 0xFFFFu, sbt); o[1] = sb_widen(w.x >> 16, sbt);
    o[2] = sb_widen(w.y & 0xFFFFu, sbt); o[3] = sb_widen(w.y >> 16, sbt);
  }
}

// Unit of a row whose largest |b'| is m (0 below the range where the digits
// could matter: such a row gets zero digits, an error below 1e-23 |S|).
__device__ __forceinline__ float bias_unit(float m) {
  const float u = m / BIAS_NMAX;
  return u >= 1e-30f ? u : 0.0f;
}

// The three digit bytes (two's complement) of b' in units u (inv = 1/u, or 0).
__device__ __forceinline__ void bias_digits(float bp, float inv, uint32_t &d2b, uint32_t &d1b, uint32_t &d0b) {
  const int n = (int)fminf(fmaxf(rintf(bp * inv), -BIAS_NMAX), BIAS_NMAX);
  const int d0 = ((n + 128) & 255) - 128;  // n - d0 is a multiple of 256
  const int n1 = (n - d0) >> 8;           // |n1| <= 32639
  const int d1 = ((n1 + 128) & 255) - 128;
  const int d2 = (n1 - d1) >> 8;          // |d2| <= 127
  d2b = (uint32_t)d2 & 0xFFu;
  d1b = (uint32_t)d1 & 0xFFu;
  d0b = (uint32_t)d0 & 0xFFu;
}

// The digits of groups 4j .. 4j + 3 of one row, b' taken from bp(k), into
// the row's six columns parts (three per half of the bias block).
template <typename BP>
__device__ __forceinline__ void put_digits4(uint8_t *row, int j, int Gq, int P, float inv, BP bp) {
  uint32_t w2 = 0, w1 = 0, w0 = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t d2b, d1b, d0b;
    bias_digits(bp(k), inv, d2b, d1b, d0b);
    w2 |= d2b << (8 * k);
    w1 |= d1b << (8 * k);
    w0 |= d0b << (8 * k);
  }
  *(uint32_t *)(row + 4 * j) = w2;               // refinement: d2 x 65536 S3
  *(uint32_t *)(row + Gq + 4 * j) = w1;          //             d1 x 256 S2
  *(uint32_t *)(row + 2 * Gq + 4 * j) = w0;      //             d0 x S1
  *(uint32_t *)(row + P + 4 * j) = w2;           // coarse:     d2 x 65536 S1
  *(uint32_t *)(row + P + Gq + 4 * j) = w2;      //             d2 x 65536 S2
  *(uint32_t *)(row + P + 2 * Gq + 4 * j) = w1;  //             d1 x 256 S1
}

// Rows of at most HP_COLS groups, a multiple of 4 (and operands aligned for
// 4-element loads): the block's scales and biases are loaded once, all loads
// issued together (the block's elements are contiguous), into registers.  b'
// is staged in LDS for the row maxima and the digits, then the scales for
// the ratio table: one memory round trip instead of one per pass.
__device__ void head_prep_staged(int64_t blk, const FrontArgs &f, float shift, float *su, float *sT) {
  const int64_t V = f.V;
  const int Gq = f.Gq, Kb = f.Kb, NB = f.NB, P = f.P, sbt = f.sbt;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t v0 = blk * HP_ROWS;
  const int rows = (int)(V - v0 < HP_ROWS ? V - v0 : HP_ROWS);
  unsigned *smax = reinterpret_cast<unsigned *>(su);
  const int64_t e0 = v0 * Gq;
  const int n = rows * Gq;  // a multiple of 4
  constexpr int IT = HP_ROWS * HP_COLS / 1024;  // 4-element slots per thread
  float sc[IT][4], bp[IT][4];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int i = 4 * (tid + 256 * it);
    if (i < n) {
      float bi[4];
      ld_sb4(f.scales, e0 + i, sbt, sc[it]);
      ld_sb4(f.biases, e0 + i, sbt, bi);
#pragma unroll
      for (int k = 0; k < 4; ++k) bp[it][k] = fmaf(shift, sc[it][k], bi[k]);
    }
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int i = 4 * (tid + 256 * it);
    if (i < n) {
      const int r = i / Gq, gi = i - r * Gq;  // the four share a row (Gq % 4 == 0)
#pragma unroll
      for (int k = 0; k < 4; ++k) sT[r * HP_LD + gi + k] = bp[it][k];
    }
  }
  __syncthreads();
  {
    // four threads per row: its max |b'| (a shuffle reduction), then its
    // digits, 4 groups at a time
    const int r = tid >> 2, qd = tid & 3, G4 = Gq >> 2;
    float m = 0.0f;
    if (r < rows)
      for (int gi = qd; gi < Gq; gi += 4) m = fmaxf(m, fabsf(sT[r * HP_LD + gi]));
    m = fmaxf(m, __shfl_xor(m, 1, 64));
    m = fmaxf(m, __shfl_xor(m, 2, 64));
    const bool any = __syncthreads_or(r < rows && m > 0.0f);  // the block carries digits
    if (r < rows) {
      if (qd == 0) smax[r] = __float_as_uint(m);
    }
    if (any && r < rows) {
      const float u = bias_unit(m);
      const float inv = (u > 0.0f) ? 1.0f / u : 0.0f;
      uint8_t *row = f.baug + (v0 + r) * Kb;
      const float *br = sT + r * HP_LD;
      for (int j = qd; j < G4; j += 4) put_digits4(row, j, Gq, P, inv, [&](int k) { return br[4 * j + k]; });
      for (int o = 3 * Gq + 4 * qd; o < P; o += 16) {
        *(uint32_t *)(row + o) = 0u;
        *(uint32_t *)(row + P + o) = 0u;
      }
    }
  }
  __syncthreads();  // b' reads done, smax written
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int i = 4 * (tid + 256 * it);
    if (i < n) {
      const int r = i / Gq, gi = i - r * Gq;
#pragma unroll
      for (int k = 0; k < 4; ++k) sT[r * HP_LD + gi + k] = sc[it][k];
    }
  }
  __syncthreads();
  const int64_t v = v0 + lane;
  if (wave == 0) {  // the block's largest |b'| (0: every digit of its rows is zero)
    unsigned mb = lane < rows ? smax[lane] : 0u;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mb = max(mb, (unsigned)__shfl_xor((int)mb, o, 64));
    if (lane == 0) f.bmxb[blk] = mb;
  }
  if (lane < rows) {
    if (wave == 0)
      for (int s2 = 0; s2 < NB; ++s2) f.rt[s2 * V + v] = 1.0f;
    // group g's entry ratio s_{g-1} / s_g (the bias block's unit before group 0)
    for (int g = wave; g < Gq; g += 4) {
      const float prev = g > 0 ? sT[lane * HP_LD + g - 1] : bias_unit(__uint_as_float(smax[lane]));
      const float e = scale_eff(prev) / scale_eff(sT[lane * HP_LD + g]);
      if (f.gs == 128) {
        f.rt[(int64_t)(NB + 2 * g) * V + v] = e;
        f.rt[(int64_t)(NB + 2 * g + 1) * V + v] = 1.0f;
      } else {
        f.rt[(int64_t)(NB + g) * V + v] = e;
      }
    }
    if (wave == 1) f.slast[v] = scale_eff(sT[lane * HP_LD + Gq - 1]);
  }
}

__device__ void head_prep_block(int64_t blk, const FrontArgs &f, float shift, float *su, float *sT) {
  const int64_t V = f.V;
  const int Gq = f.Gq, Kb = f.Kb, NB = f.NB, P = f.P, sbt = f.sbt;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t v0 = blk * HP_ROWS;
  const int rows = (int)(V - v0 < HP_ROWS ? V - v0 : HP_ROWS);
  unsigned *smax = reinterpret_cast<unsigned *>(su);
  float *sprev = su + HP_ROWS;
  const int64_t e0 = v0 * Gq;  // first (row, group) element of the block
  const uintptr_t al = sbt == SB_F32 ? 15 : 7;
  if ((Gq & 3) == 0 && (((uintptr_t)f.scales | (uintptr_t)f.biases) & al) == 0 && Gq <= HP_COLS) {
    head_prep_staged(blk, f, shift, su, sT);
    return;
  }
  if ((Gq & 3) == 0 && (((uintptr_t)f.scales | (uintptr_t)f.biases) & al) == 0) {
    const int r = tid >> 2, qd = tid & 3, G4 = Gq >> 2;
    const int64_t er = e0 + (int64_t)r * Gq;  // first element of row r
    float m = 0.0f;
    if (r < rows)
      for (int j = qd; j < G4; j += 4) {
        float sc[4], bi[4];
        ld_sb4(f.scales, er + 4 * j, sbt, sc);
        ld_sb4(f.biases, er + 4 * j, sbt, bi);
#pragma unroll
        for (int k = 0; k < 4; ++k) m = fmaxf(m, fabsf(fmaf(shift, sc[k], bi[k])));
      }
    m = fmaxf(m, __shfl_xor(m, 1, 64));
    m = fmaxf(m, __shfl_xor(m, 2, 64));
    if (r < rows) {
      if (qd == 0) smax[r] = __float_as_uint(m);
      const float u = bias_unit(m);
      const float inv = (u > 0.0f) ? 1.0f / u : 0.0f;
      uint8_t *row = f.baug + (v0 + r) * Kb;
      for (int j = qd; j < G4; j += 4) {
        float sc[4], bi[4];
        ld_sb4(f.scales, er + 4 * j, sbt, sc);
        ld_sb4(f.biases, er + 4 * j, sbt, bi);
        put_digits4(row, j, Gq, P, inv, [&](int k) { return fmaf(shift, sc[k], bi[k]); });
      }
      for (int o = 3 * Gq + 4 * qd; o < P; o += 16) {
        *(uint32_t *)(row + o) = 0u;
        *(uint32_t *)(row + P + o) = 0u;
      }
    }
    __syncthreads();
  } else {
    if (tid < HP_ROWS) smax[tid] = 0u;
    __syncthreads();
    const int n = rows * Gq;
    for (int i = tid; i < n; i += 256) {
      const float bp = fmaf(shift, ld_sb(f.scales, e0 + i, sbt), ld_sb(f.biases, e0 + i, sbt));
      atomicMax(&smax[i / Gq], __float_as_uint(fabsf(bp)));  // |b'| >= 0: integer order is float order
    }
    __syncthreads();
    for (int i = tid; i < n; i += 256) {
      const int r = i / Gq, gi = i - r * Gq;
      const float u = bias_unit(__uint_as_float(smax[r]));
      const float inv = (u > 0.0f) ? 1.0f / u : 0.0f;
      uint32_t d2b, d1b, d0b;
      bias_digits(fmaf(shift, ld_sb(f.scales, e0 + i, sbt), ld_sb(f.biases, e0 + i, sbt)), inv, d2b, d1b, d0b);
      uint8_t *row = f.baug + (v0 + r) * Kb;
      row[gi] = (uint8_t)d2b;
      row[Gq + gi] = (uint8_t)d1b;
      row[2 * Gq + gi] = (uint8_t)d0b;
      row[P + gi] = (uint8_t)d2b;
      row[P + Gq + gi] = (uint8_t)d2b;
      row[P + 2 * Gq + gi] = (uint8_t)d1b;
    }
    const int pad = P - 3 * Gq;
    for (int i = tid; i < rows * pad; i += 256) {
      uint8_t *row = f.baug + (v0 + i / pad) * Kb + 3 * Gq + i % pad;
      row[0] = 0;
      row[P] = 0;
    }
  }
  const int64_t v = v0 + lane;
  if (wave == 0) {  // the block's largest |b'| (0: every digit of its rows is zero)
    unsigned mb = lane < rows ? smax[lane] : 0u;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mb = max(mb, (unsigned)__shfl_xor((int)mb, o, 64));
    if (lane == 0) f.bmxb[blk] = mb;
  }
  if (wave == 0 && lane < rows) {
    sprev[lane] = bias_unit(__uint_as_float(smax[lane]));  // the bias block's unit precedes group 0
    for (int s2 = 0; s2 < NB; ++s2) f.rt[s2 * V + v] = 1.0f;
  }
  // group g's entry ratio s_{g-1} / s_g goes to the K step where g starts:
  // groups 32 and 64 -> step g (a step is one group: 32- or 64-wide);
  // 128 -> step 2g (and ratio 1 at step 2g + 1)
  for (int c0 = 0; c0 < Gq; c0 += HP_COLS) {
    const int cw = Gq - c0 < HP_COLS ? Gq - c0 : HP_COLS;
    __syncthreads();  // sprev written, the previous chunk's reads done
    for (int i = tid; i < rows * cw; i += 256) {
      const int r = i / cw, gl = i - r * cw;
      sT[r * HP_LD + gl] = ld_sb(f.scales, e0 + (int64_t)r * Gq + c0 + gl, sbt);
    }
    __syncthreads();
    if (lane < rows) {
      for (int gl = wave; gl < cw; gl += 4) {
        const int g = c0 + gl;
        const float prev = gl > 0 ? sT[lane * HP_LD + gl - 1] : sprev[lane];
        const float e = scale_eff(prev) / scale_eff(sT[lane * HP_LD + gl]);
        if (f.gs == 128) {
          f.rt[(int64_t)(NB + 2 * g) * V + v] = e;
          f.rt[(int64_t)(NB + 2 * g + 1) * V + v] = 1.0f;
        } else {
          f.rt[(int64_t)(NB + g) * V + v] = e;
        }
      }
    }
    __syncthreads();
    if (tid < rows) sprev[tid] = sT[tid * HP_LD + cw - 1];
  }
  if (tid < rows) f.slast[v0 + tid] = scale_eff(sprev[tid]);
}

// Token-side value of bias-block column kk (see the layout above), from the
// row's group sums: S = p1 + p2 + p3, each piece the bf16 rounding of what
// the previous ones leave (the differences are exact in fp32).
__device__ __forceinline__ uint32_t bias_col(const float *sS, int kk, int P, int Gq) {
  const int half = kk >= P ? 1 : 0, kl = kk - half * P;
  const int part = kl / Gq, gi = kl - part * Gq;
  if (part >= 3) return 0u;
  const float S = sS[gi];
  const float p1 = bf16_to_f32(bf16_rne(S));
  const float r1 = S - p1;
  const float p2 = bf16_to_f32(bf16_rne(r1));
  const float p3 = bf16_to_f32(bf16_rne(r1 - p2));
  float x;
  if (half == 1) x = part == 0 ? 65536.0f * p1 : (part == 1 ? 65536.0f * p2 : 256.0f * p1);  // coarse
  else x = part == 0 ? 65536.0f * p3 : (part == 1 ? 256.0f * p2 : p1);                       // refinement
  return bf16_rne(x);  // exact: a bf16 piece times a power of two
}

template <int BITS>
__global__ void __launch_bounds__(256) k_front(FrontArgs f) {
  __shared__ float sS[MAX_GQ];
  __shared__ float sRed[4];
  __shared__ float sT[HP_ROWS * HP_LD];
  const int tid = threadIdx.x;
  constexpr bool DENSE = BITS == 16;  // bf16 head rows: no head side, no group sums
  if (blockIdx.x >= (unsigned)f.M_pad) {
    if constexpr (!DENSE) head_prep_block((int64_t)blockIdx.x - f.M_pad, f, BITS == 8 ? 128.0f : 8.0f, sS, sT);
    return;
  }
  const int r = blockIdx.x;
  int src;
  if (f.compact) {
    // small M: every row block compacts for itself (no separate launch).
    // Thread i scans its slice of the mask; a block scan of the slice counts
    // gives the rank of every slice start.  Row block r takes the r-th
    // supervised token as its source, and fixes inv of token r (r < M).
    __shared__ int sC[4], sSrc;
    const int M = f.M, per = (M + 255) / 256;
    const int t0 = tid * per, t1 = min(M, t0 + per);
    int c = 0;
    for (int t = t0; t < t1; ++t) c += f.mask ? (f.mask[t] != 0) : 1;
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if ((tid & 63) >= o) incl += y;
    }
    if ((tid & 63) == 63) sC[tid >> 6] = incl;
    if (tid == 0) sSrc = -1;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < (tid >> 6); ++w) base += sC[w];
    const int excl = base + incl - c;
    if (r >= excl && r < excl + c) {  // the r-th supervised token is in this slice
      int k = excl;
      for (int t = t0; t < t1; ++t)
        if (!f.mask || f.mask[t] != 0) {
          if (k == r) sSrc = t;
          ++k;
        }
    }
    if (r < M && r >= t0 && r < t1) {  // rank of token r
      int k = excl;
      for (int t = t0; t < r; ++t) k += f.mask ? (f.mask[t] != 0) : 1;
      const bool sup = !f.mask || f.mask[r] != 0;
      f.inv[r] = sup ? k : -1;
      if (!sup && f.out_logp) {
        f.out_logp[r] = 0.0f;
        f.out_lse[r] = 0.0f;
      }
    }
    if (r == 0 && tid == 0) f.cnt[0] = sC[0] + sC[1] + sC[2] + sC[3];
    __syncthreads();
    src = sSrc;
    if (tid == 0) f.idx_out[r] = src;
  } else {
    src = f.idx[r];
  }
  const int H = f.H, Gq = f.Gq, Kb = f.Kb;
  const int64_t ks16 = f.Ka / 16;
  const int nch = H / 8;     // 16-byte chunks of the h part
  const int cpg = f.gs / 8;  // chunks per quantization group (4, 8 or 16)
  float sab = 0.0f;          // sum over groups of |S_g| (this thread's groups)
  for (int c = tid; c < nch; c += 256) {
    const u32x4_t x = (src >= 0) ? *(const u32x4_t *)(f.h + (size_t)src * H + 8 * c) : u32x4_t{0, 0, 0, 0};
    *(u32x4_t *)(f.haug + frag_slot(r, Kb / 8 + c, ks16)) = x;
    if constexpr (DENSE) continue;
    float part = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) part += bf16_to_f32(x[e] & 0xFFFFu) + bf16_to_f32(x[e] >> 16);
    // the chunks of one group sit in cpg consecutive lanes
    for (int o = 1; o < cpg; o <<= 1) part += __shfl_xor(part, o, 16);
    if (c % cpg == 0) {
      sS[c / cpg] = part;
      sab += fabsf(part);
    }
  }
  if constexpr (!DENSE) {
    sab = wave_sum(sab);
    if ((tid & 63) == 0) sRed[tid >> 6] = sab;
  }
  __syncthreads();
  for (int c = tid; c < Kb / 8; c += 256) {
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = bias_col(sS, 8 * c + 2 * e, f.P, Gq) | (bias_col(sS, 8 * c + 2 * e + 1, f.P, Gq) << 16);
    *(u32x4_t *)(f.haug + frag_slot(r, c, ks16)) = u32x4_t{o[0], o[1], o[2], o[3]};
  }
  if (tid == 0) {
    const int tgt = (src >= 0) ? f.targets[src] : -1;
    TokRec rec;
    rec.lse = (src >= 0 && f.lse) ? f.lse[src] : 0.0f;
    rec.g = (src >= 0) ? (f.g ? f.g[src] : 1.0f) : 0.0f;
    rec.tgt = (src >= 0 && tgt >= 0 && (int64_t)tgt < f.V) ? tgt : -1;
    rec.tval = 0.0f;
    f.tok[r] = rec;
    if (!DENSE) f.sabs[r] = sRed[0] + sRed[1] + sRed[2] + sRed[3];
  }
}

// ---------------------------------------------------------------------------
// Cross-split merge (page "mlx-bun 0.0.4 -> 0.0.6", flashCceForward's host
// merge): lse = m* + log sum_s s_s exp(m_s - m*), logp = target logit - lse.
// A group of L lanes per token (L the power of two >= the split count, at
// most 64) reads the token's partials in parallel and reduces with shuffles;
// one token per thread when there are few splits, a wave per token when a
// few supervised tokens carry hundreds of splits.
__global__ void __launch_bounds__(256) k_merge(const float *part, int nblocks, int full_tiles, int tiles,
                                               int max_splits, int M_pad, const int *inv, const int *cnt,
                                               const TokRec *tok, int M, float *logp, float *lse, float *nc) {
  // two partials (vocabulary halves of the tile) per split, over every chunk
  // of the vocabulary the forward's launches covered
  const int nsplit = 2 * vsplit_total(nblocks, active_tiles(cnt), full_tiles, tiles, max_splits);
  int L = 1;
  while (L < nsplit && L < 64) L <<= 1;
  const int per_block = 256 / L;
  if (blockIdx.x * per_block >= M) return;  // the grid is sized for L = 64
  const int t = blockIdx.x * per_block + threadIdx.x / L;
  const int sl = threadIdx.x % L;
  const int r = t < M ? inv[t] : -1;
  float mx = -INFINITY;
  if (r >= 0)
    for (int s = sl; s < nsplit; s += L) mx = fmaxf(mx, part[((size_t)s * M_pad + r) * 2]);
  for (int o = L >> 1; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, L));
  float se = 0.0f;
  if (r >= 0)
    for (int s = sl; s < nsplit; s += L) {
      const float m = part[((size_t)s * M_pad + r) * 2];
      if (m != -INFINITY) se += part[((size_t)s * M_pad + r) * 2 + 1] * __expf(m - mx);
    }
  for (int o = L >> 1; o >= 1; o >>= 1) se += __shfl_xor(se, o, L);
  if (t >= M || sl != 0) return;
  if (r < 0) {
    logp[t] = 0.0f;
    lse[t] = 0.0f;
    return;
  }
  const TokRec rec = tok[r];
  if (nc) {
    // the uncapped single pass: its partials hold the non-target terms; the
    // target's own (its logit is at most the maximum, which spans it) is added
    const float et = rec.tgt >= 0 ? __expf(rec.tval - mx) : 0.0f;
    const float l = mx + logf(se + et);
    lse[t] = l;
    logp[t] = rec.tval - l;
    nc[3 * r] = mx;
    nc[3 * r + 1] = se;
    nc[3 * r + 2] = et;
    return;
  }
  const float l = mx + logf(se);
  lse[t] = l;
  logp[t] = rec.tval - l;
}

// One thread per 16-byte slot of the fragment-major chunks: 1 KiB blocks of 64
// slots, block (T, C) holding tokens 32 T .. + 31 and vocabulary rows 16 C ..
// + 15 (lane l: token 32 T + l % 32, rows 16 C + 8 (l / 32) .. + 8).  Grid:
// x = T, y = C / 4 (four blocks per workgroup, a wave each), z = chunk (the
// chunk count stays small: the whole matrix is kept only up to 32 GiB).
__global__ void __launch_bounds__(256) k_nc_scale(uint16_t *coeff, int64_t ld_coeff, int nchunks, int64_t last_rows,
                                                  int M_pad, const int *cnt, const float *ncR, const float *nc) {
  const int T = blockIdx.x, c = blockIdx.z, l = threadIdx.x & 63;
  const int row = 32 * T + (l & 31);
  const int64_t ksv = ld_coeff / 16;
  const int64_t C = (int64_t)blockIdx.y * 4 + (threadIdx.x >> 6);
  const int64_t col = 16 * C + 8 * (l >> 5);  // chunk-local vocabulary row of the slot's first element
  if (row >= cnt[0] || C >= ksv || col >= (c == nchunks - 1 ? last_rows : ld_coeff)) return;
  const int64_t blk = ((int64_t)c * ld_coeff + col) >> 5;
  const float f = __builtin_amdgcn_exp2f((ncR[blk * M_pad + row] - nc[3 * row]) * 1.4426950408889634f);
  u32x4_t *p = reinterpret_cast<u32x4_t *>(coeff + (size_t)c * M_pad * ld_coeff + (((size_t)T * ksv + C) * 64 + l) * 8);
  u32x4_t x = *p;
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = pack_rne(bf16_to_f32(x[e] & 0xFFFFu) * f, bf16_to_f32(x[e] >> 16) * f);
  *p = x;
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
// zero rows for masked tokens; stored as fp32, or rounded once to bf16.  The
// target's coefficient is tval itself or formed here from the splits'
// non-target mass (ReduceTarget); in the fused pass the slab sum is first
// scaled to the true coefficients.
template <int BITS>
__global__ void __launch_bounds__(256) k_dh_reduce(GemmArgs a, const int *inv, const TokRec *tok, void *dh,
                                                   int out_bf16, ReduceTarget tg) {
  // four consecutive columns per thread (H % 64 == 0): 16-byte slab loads,
  // one code word, scale and bias for the four, one vector store
  const int t = blockIdx.x;
  const int d = (blockIdx.y * 256 + threadIdx.x) * 4;
  const int H = a.H;
  const int r = inv[t];
  const int act = active_tiles(a.cnt);
  // mode 1: the token's non-target mass over the backward's splits; mode 2:
  // S, the sum of e = e^{y - cap} over the non-target columns, from the
  // single pass's split sums.  The token's contiguous run, summed by the
  // workgroup in a fixed order (every thread takes part).
  float S = 0.0f;
  if (tg.mode == 3 && r >= 0) S = tg.nc[3 * r + 1];  // the uncapped single pass: from the merge
  if ((tg.mode == 1 || tg.mode == 2) && r >= 0) {
    __shared__ float sS[4];
    const int ns = 2 * vsplit_total(tg.nblocks, act, tg.full_tiles, tg.tiles, tg.max_splits);
    float x = 0.0f;
    for (int k = threadIdx.x; k < ns; k += 256) x += tg.mass[(size_t)r * tg.mass_ld + k];
    x = wave_sum(x);
    if ((threadIdx.x & 63) == 0) sS[threadIdx.x >> 6] = x;
    __syncthreads();
    S = (sS[0] + sS[1]) + (sS[2] + sS[3]);
    if (tg.mode == 2) S *= 0.25f;  // the single pass's tiles sum 4 e (exact)
  }
  // mode 2 also finishes the forward, in place of a merge launch: with the
  // fixed reference, lse = cap + log(S + e_t) and logp = y_t - lse (the
  // target's e_t from the logit its tile captured); masked tokens get zeros
  if (tg.mode == 2 && blockIdx.y == 0 && threadIdx.x == 0) {
    float l = 0.0f, lp = 0.0f;
    if (r >= 0) {
      const TokRec rec = tok[r];
      const float et = rec.tgt >= 0 ? expf(rec.tval - tg.cap) : 0.0f;
      l = tg.cap + logf(S + et);
      lp = rec.tval - l;
      if (tg.fac) {  // the dense head's dW: the token's factor and its target coefficient in chunk units
        tg.fac[2 * r] = rec.g * (1.0f / (S + et));
        tg.fac[2 * r + 1] = rec.tgt >= 0 ? S * tg.tdc[r] : 0.0f;
      }
    }
    tg.lse[t] = l;
    tg.logp[t] = lp;
  }
  if (tg.mode == 3 && tg.fac && blockIdx.y == 0 && threadIdx.x == 0 && r >= 0) {
    // the dense head's dW without a softcap: as above, against the token's maximum (c' = 1)
    const TokRec rec = tok[r];
    tg.fac[2 * r] = rec.g * (1.0f / (S + tg.nc[3 * r + 2]));
    tg.fac[2 * r + 1] = rec.tgt >= 0 ? S : 0.0f;
  }
  if (d >= H) return;
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  if (r >= 0) {
    int ksd, steps_per;
    dh_split(a, act, ksd, steps_per);
    // the slabs summed in order, eight loads issued before their adds (few
    // tokens have tens of splits, and a load waited for before the next one
    // is issued made the sum a chain of memory latencies)
    const float *sp = a.dh_part + (size_t)r * H + d;
    const size_t sstride = (size_t)act * BM * H;
    int k = 0;
    for (; k + 8 <= ksd; k += 8) {
      f32x4_t x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = *(const f32x4_t *)(sp + (size_t)(k + j) * sstride);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += x[j];
    }
    for (; k < ksd; ++k) acc += *(const f32x4_t *)(sp + (size_t)k * sstride);
    TokRec rec = tok[r];
    const bool ht = rec.tgt >= 0;
    if (tg.mode == 1) {
      rec.tval = ht ? rec.g * S * tg.tdc[r] : 0.0f;
    } else if (tg.mode == 2) {
      // single pass: p_v = e_v / (S + e_t), the slabs sum -e c' w
      const float et = ht ? expf(rec.tval - tg.cap) : 0.0f;
      const float inv_tot = 1.0f / (S + et);
      acc *= rec.g * inv_tot;
      rec.tval = ht ? rec.g * (S * inv_tot) * tg.tdc[r] : 0.0f;
    } else if (tg.mode == 3) {
      // uncapped single pass: the same against the token's largest logit m
      // (the coefficient chunks were brought to it), c' = 1
      const float et = tg.nc[3 * r + 2];
      const float inv_tot = 1.0f / (S + et);
      acc *= rec.g * inv_tot;
      rec.tval = ht ? rec.g * (S * inv_tot) : 0.0f;
    }
    if (rec.tgt >= 0 && (int64_t)rec.tgt < a.V) {
      const uint32_t *row = a.wq + (size_t)rec.tgt * a.wpr;
      float w[4];
      if constexpr (BITS == 16) {  // dense bf16 row
        const uint32_t x0 = row[d / 2], x1 = row[d / 2 + 1];
        w[0] = bf16_to_f32(x0 & 0xFFFFu); w[1] = bf16_to_f32(x0 >> 16);
        w[2] = bf16_to_f32(x1 & 0xFFFFu); w[3] = bf16_to_f32(x1 >> 16);
      } else {
        const int64_t gi = (int64_t)rec.tgt * a.Gq + d / a.gs;  // the four share a group (group >= 32)
        const float sc = ld_sb(a.scales, gi, a.sbt), bi = ld_sb(a.biases, gi, a.sbt);
        const uint32_t word = row[d * BITS / 32] >> ((d * BITS) % 32);
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = sc * (float)((word >> (BITS * e)) & ((1u << BITS) - 1u)) + bi;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += rec.tval * w[e];
    }
  }
  // the ABI asks dh for element alignment only: vector stores when the base allows
  if (out_bf16) {
    uint16_t *o = static_cast<uint16_t *>(dh) + (size_t)t * H + d;
    if (((uintptr_t)dh & 7) == 0) {
      *(uint2 *)o = uint2{bf16_rne(acc[0]) | (bf16_rne(acc[1]) << 16), bf16_rne(acc[2]) | (bf16_rne(acc[3]) << 16)};
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = (uint16_t)bf16_rne(acc[e]);
    }
  } else {
    float *o = static_cast<float *>(dh) + (size_t)t * H + d;
    if (((uintptr_t)dh & 15) == 0) {
      *(f32x4_t *)o = acc;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = acc[e];
    }
  }
}

void launch_compact(hipStream_t st, const uint8_t *mask, int M, int M_pad, int *idx, int *inv, int *cnt,
                    float *out_logp, float *out_lse) {
  hipLaunchKernelGGL(k_compact, dim3(1), dim3(1024), 0, st, mask, M, M_pad, idx, inv, cnt, out_logp, out_lse);
}

void launch_front(hipStream_t st, int bits, const FrontArgs &f) {
  if (bits == 16) {  // dense head: token rows only
    hipLaunchKernelGGL(k_front<16>, dim3((unsigned)f.M_pad), dim3(256), 0, st, f);
    return;
  }
  // token rows [0, M_pad), then the head blocks of HP_ROWS vocabulary rows
  const dim3 grid((unsigned)(f.M_pad + (f.head ? (f.V + HP_ROWS - 1) / HP_ROWS : 0)));
  if (grid.x == 0) return;
  if (bits == 4)
    hipLaunchKernelGGL(k_front<4>, grid, dim3(256), 0, st, f);
  else
    hipLaunchKernelGGL(k_front<8>, grid, dim3(256), 0, st, f);
}

void launch_merge(hipStream_t st, int M, const float *part, int nblocks, int full_tiles, int tiles, int max_splits,
                  int M_pad, const int *inv, const int *cnt, const TokRec *tok, float *logp, float *lse, float *nc) {
  hipLaunchKernelGGL(k_merge, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, st, part, nblocks, full_tiles, tiles,
                     max_splits, M_pad, inv, cnt, tok, M, logp, lse, nc);
}

void launch_nc_scale(hipStream_t st, uint16_t *coeff, int64_t ld_coeff, int nchunks, int64_t last_rows, int M_pad,
                     const int *cnt, const float *ncR, const float *nc) {
  const int64_t ksv = ld_coeff / 16;
  const dim3 grid((unsigned)(M_pad / 32), (unsigned)((ksv + 3) / 4), (unsigned)nchunks);
  hipLaunchKernelGGL(k_nc_scale, grid, dim3(256), 0, st, coeff, ld_coeff, nchunks, last_rows, M_pad, cnt, ncR, nc);
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
                      void *dh, int out_bf16, const ReduceTarget &tg) {
  const dim3 grid((unsigned)M, (unsigned)((ga.H + 1023) / 1024));
  if (bits == 16)
    hipLaunchKernelGGL(k_dh_reduce<16>, grid, dim3(256), 0, st, ga, inv, tok, dh, out_bf16, tg);
  else if (bits == 4)
    hipLaunchKernelGGL(k_dh_reduce<4>, grid, dim3(256), 0, st, ga, inv, tok, dh, out_bf16, tg);
  else
    hipLaunchKernelGGL(k_dh_reduce<8>, grid, dim3(256), 0, st, ga, inv, tok, dh, out_bf16, tg);
}

}  // namespace cce
