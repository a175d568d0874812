// tile.hip -- the logit tile kernel of libcce (forward partials and backward
// coefficients).  Built with the VGPR form of MFMA so the accumulator, which
// the VALU rescales every group, stays in architectural VGPRs.
#include "cce_device.h"

namespace cce {

// ---------------------------------------------------------------------------
// The logit tile: 256 tokens x 256 vocabulary rows per workgroup of 8 waves,
// K = Ka (bias block, then H).  Wave w owns tokens [64(w%4), +64) and vocab
// rows [128(w/4), +128) of the tile as 2 x 4 blocks of
// v_mfma_f32_32x32x16_bf16 (rows = tokens, columns = vocabulary rows).  The
// code tile is unpacked once into LDS (double buffered, one group per step)
// and shared by the eight waves; the token operand is loaded straight from
// the augmented rows into registers (the two waves of a token group load the
// same rows, served once by L2), reloaded for the next step right after its
// last use.
//
// Scale fold without a second accumulator: the accumulator is kept in units of
// the current group's scale, acc <- acc * (s_{g-1} / s_g) + A_g, so the MFMA
// accumulates in place and the VALU does one multiply per element per group.
// After the last group z = acc * s_last.  (The bias block runs first with scale
// 1; a scale of exactly 0 is replaced by 1e-30, whose contribution is nil.)

constexpr int ZROW = 36;  // padded fp32 row stride of the per-wave transpose scratch (32 columns)

template <int BITS>
struct Producer {
  // Thread tid stages row tid/2 (of BNT), K half tid%2 (32 codes) of each
  // step, and (tid even) that row's scale ratio.
  static constexpr int NW = BITS;  // words per thread per step
  uint32_t w[NW];
  float s;
  float s_prev;

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
      s = ok ? a.scales[(size_t)v * a.G + g] : 1.0f;
    }
  }

  __device__ __forceinline__ void store(const TileArgs &a, int64_t v0, int step, int prow, int phalf,
                                        uint16_t *sw, float *sr, float *slast) {
    uint32_t o[16];
    if (step >= a.NB) {
      if (BITS == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) unpack4(w[i], o + 4 * i);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) unpack8(w[i], o + 2 * i);
      }
      if (phalf == 0) {
        const float se = scale_eff(s);
        sr[prow] = __fdividef((step == a.NB) ? 1.0f : s_prev, se);
        s_prev = se;
        if (step == a.NB + a.G - 1) slast[prow] = se;
      }
    } else {
      // bias block chunk: hi/lo splits of the fp32 biases (part 0,1 -> hi; 2 -> lo)
      const int64_t v = v0 + prow;
      const bool ok = v < a.V;
      const float *brow = a.biases + (size_t)(ok ? v : 0) * a.G;
      const int kk0 = step * KSTEP + phalf * 32;
      int part = kk0 / a.G;
      int gi = kk0 - part * a.G;
      uint32_t val[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        uint32_t x = 0;
        if (ok && part < 3) {
          const float b = brow[gi];
          const uint32_t hi = bf16_rne(b);
          x = (part == 2) ? bf16_rne(b - bf16_to_f32(hi)) : hi;
        }
        val[e] = x;
        if (++gi == a.G) { gi = 0; ++part; }
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) o[e] = val[2 * e] | (val[2 * e + 1] << 16);
      if (phalf == 0) sr[prow] = 1.0f;
    }
    uint16_t *dst = sw + prow * WROW + phalf * 32;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(u32x4_t *)(dst + 8 * i) = u32x4_t{o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
  }
};

template <int BITS, bool BWD>
__global__ void __launch_bounds__(TW, 1) k_tile(TileArgs a) {
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  if (bid >= a.nblocks) return;
  const int tt = bid / a.nwr, wr = bid % a.nwr;
  if (tt * BM >= a.cnt[0]) return;
  const int tile_begin = wr * a.tiles_per_wg;
  const int tile_end = min(tile_begin + a.tiles_per_wg, a.range_tiles);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tg = wave & 3, vh = wave >> 2;
  const int l32 = lane & 31, lh = lane >> 5;
  const int prow = tid >> 1, phalf = tid & 1;
  const int steps = a.NB + a.G;

  __shared__ __attribute__((aligned(16))) uint16_t sW[2][BNT * WROW];
  __shared__ __attribute__((aligned(16))) float sR[2][BNT];
  __shared__ __attribute__((aligned(16))) float sLast[BNT];
  __shared__ __attribute__((aligned(16))) float sZ[8][64 * ZROW];

  const int tok0 = tt * BM + tg * 64;
  const int vcol0 = vh * 128;  // this wave's first vocabulary row within the tile
  // fragment-major h rows: one 1 KiB block per (32 tokens, 16 K), 4 per step
  const uint16_t *hp0 = a.haug + ((size_t)(tok0 >> 5) * a.ks16 * 64 + lane) * 8;
  const uint16_t *hp1 = hp0 + (size_t)a.ks16 * 512;
  float *zs = sZ[wave];

  float run_m = -INFINITY, run_s = 0.0f;
  float lse_t = 0.0f, g_t = 0.0f;
  int64_t tgt_t = -1;
  if (BWD) {
    const TokRec rec = a.tok[tok0 + lane];
    lse_t = rec.lse;
    g_t = rec.g;
    tgt_t = rec.tgt;
  }

  const int total = (tile_end - tile_begin) * steps;
  if (total > 0) {
    Producer<BITS> pr;
    pr.s_prev = 1.0f;
    f32x16_t acc[2][4];
    bf16x8_t hA[2][4];
    {
      const int64_t v0 = (int64_t)(a.range_tile0 + tile_begin) * BNT;
      pr.load(a, v0, 0, prow, phalf);
      pr.store(a, v0, 0, prow, phalf, sW[0], sR[0], sLast);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        hA[0][ks] = *(const bf16x8_t *)(hp0 + ks * 512);
        hA[1][ks] = *(const bf16x8_t *)(hp1 + ks * 512);
      }
      __syncthreads();
    }
    int st = 0, tile = tile_begin;
    for (int idx = 0; idx < total; ++idx) {
      const int cb = idx & 1;
      const bool more = idx + 1 < total;
      const int nst = (st + 1 == steps) ? 0 : st + 1;
      const int ntile = (st + 1 == steps) ? tile + 1 : tile;
      const int64_t v0 = (int64_t)(a.range_tile0 + tile) * BNT;
      const int64_t nv0 = (int64_t)(a.range_tile0 + ntile) * BNT;
      if (more) pr.load(a, nv0, nst, prow, phalf);
      if (st == 0) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[rb][c][e] = 0.0f;
      }
      const uint16_t *sw = sW[cb] + (vcol0 + l32) * WROW + lh * 8;
      float r[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) r[c] = sR[cb][vcol0 + c * 32 + l32];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8_t bq[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) bq[c] = *(const bf16x8_t *)(sw + c * 32 * WROW + ks * 16);
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            if (ks == 0) acc[rb][c] *= r[c];
            acc[rb][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hA[rb][ks], bq[c], acc[rb][c], 0, 0, 0);
          }
        if (more) {
          hA[0][ks] = *(const bf16x8_t *)(hp0 + (size_t)(nst * 4 + ks) * 512);
          hA[1][ks] = *(const bf16x8_t *)(hp1 + (size_t)(nst * 4 + ks) * 512);
        }
      }
      if (more) pr.store(a, nv0, nst, prow, phalf, sW[cb ^ 1], sR[cb ^ 1], sLast);

      if (st == steps - 1) {
        // ---- epilogue of this vocabulary tile.  acc[rb][c][4i+j] is the logit
        // (in units of s_last) of token row rb*32 + 8i + 4*lh + j and vocab row
        // v0 + vcol0 + c*32 + l32.  Transpose per wave through LDS so that lane = token,
        // then stream the row in chunks of 16.
        float sl[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) sl[c] = sLast[vcol0 + c * 32 + l32];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          // one 32-column block of the tile: [64 tokens x 32 vocab rows]
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int j = 0; j < 4; ++j)
                zs[(rb * 32 + 8 * i + 4 * lh + j) * ZROW + l32] = acc[rb][c][4 * i + j] * sl[c];
          __syncthreads();
#pragma unroll
          for (int k0 = 0; k0 < 32; k0 += 16) {
            float z[16];
#pragma unroll
            for (int k = 0; k < 16; k += 4) {
              const f32x4_t x = *(const f32x4_t *)(zs + lane * ZROW + k0 + k);
              z[k] = x[0]; z[k + 1] = x[1]; z[k + 2] = x[2]; z[k + 3] = x[3];
            }
            const int64_t vb = v0 + vcol0 + c * 32 + k0;
            if (!BWD) {
              float tmax = -INFINITY;
#pragma unroll
              for (int k = 0; k < 16; ++k) {
                float y = softcap(z[k], a.cap, a.inv_cap);
                y = (vb + k < a.V) ? y : -INFINITY;
                z[k] = y;
                tmax = fmaxf(tmax, y);
              }
              const float mnew = fmaxf(run_m, tmax);
              if (mnew != -INFINITY) {
                float ssum = 0.0f;
#pragma unroll
                for (int k = 0; k < 16; ++k) ssum += __expf(z[k] - mnew);
                run_s = run_s * __expf(run_m - mnew) + ssum;
                run_m = mnew;
              }
            } else {
              // -g * softmax * c'; the target column is left out here and its
              // whole term g * (1 - p) * c' * w is added in fp32 by k_dh_reduce.
              uint32_t pk[8];
#pragma unroll
              for (int k = 0; k < 16; k += 2) {
                float c2[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                  float dc;
                  const float y = softcap_d(z[k + u], a.cap, a.inv_cap, dc);
                  const int64_t v = vb + k + u;
                  const float val = -g_t * __expf(y - lse_t) * dc;
                  c2[u] = (v < a.V && v != tgt_t) ? val : 0.0f;
                }
                pk[k / 2] = pack_rne(c2[0], c2[1]);
              }
              // fragment-major chunk: these 16 vocab rows are K chunks 2m, 2m+1
              const int64_t vloc = (int64_t)tile * BNT + vcol0 + c * 32 + k0;
              const int cm = (int)(vloc >> 3);
              *(u32x4_t *)(a.coeff + frag_slot(tok0 + lane, cm, a.ksv)) = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
              *(u32x4_t *)(a.coeff + frag_slot(tok0 + lane, cm + 1, a.ksv)) = u32x4_t{pk[4], pk[5], pk[6], pk[7]};
            }
          }
          __syncthreads();
        }
      }
      __syncthreads();
      st = nst;
      tile = ntile;
    }
  }

  if (!BWD) {
    float *dst = a.part + ((size_t)(2 * wr + vh) * a.M_pad + tok0 + lane) * 2;
    dst[0] = run_m;
    dst[1] = run_s;
  }
}

void launch_tile(hipStream_t st, int bits, bool bwd, dim3 grid, const TileArgs &a) {
  if (bits == 4) {
    if (bwd) hipLaunchKernelGGL((k_tile<4, true>), grid, dim3(TW), 0, st, a);
    else hipLaunchKernelGGL((k_tile<4, false>), grid, dim3(TW), 0, st, a);
  } else {
    if (bwd) hipLaunchKernelGGL((k_tile<8, true>), grid, dim3(TW), 0, st, a);
    else hipLaunchKernelGGL((k_tile<8, false>), grid, dim3(TW), 0, st, a);
  }
}

}  // namespace cce
