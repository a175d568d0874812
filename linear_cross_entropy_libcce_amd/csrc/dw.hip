// dw.hip -- the head gradient of a trainable dense head: dW = coeff^T . h, the
// contraction of the backward's coefficients with the hidden states over the
// tokens (the weight gradient of the original cut-cross-entropy setting, which
// the quantized head, being frozen, does not need).
//
//   dW[v][d] = sum_t coeff[t][v] * h[t][d],  coeff = g (1[v = target] - p_v) c'(z_v)
//
// Both operands are stored token-minor (fragment-major rows of tokens), so the
// contraction over tokens first transposes them into token-major fragments:
//  * k_hT, once per call: hT[d][r] = h row r (compacted, padded) column d
//    (in the single pass: times the row's factor g / (S + e_t), rounded to
//    bf16; rows past the supervised count are zeros);
//  * k_coeffT, per coefficient chunk: the chunk's [token][vocab] fragments as
//    [vocab][token] fragments, with the target's whole coefficient (kept out
//    of the chunk, where dh adds it in fp32) written in, rounded to bf16 like
//    every other coefficient;
//  * k_dw: 256 vocabulary rows x 256 columns of dW per workgroup over all
//    supervised tokens, MFMA v_mfma_f32_32x32x16_bf16, the coefficient operand
//    from the transposed chunk into registers one step ahead, the hT tile
//    through LDS (double buffered), the same wave layout and swizzle as the
//    dh contraction.  Each workgroup owns its output block: no atomics, no
//    split, repeatable bits.
#include "cce_device.h"

namespace cce {

constexpr int TR = 64;         // tokens x columns (or vocabulary rows) per transpose block
constexpr int TLD = TR + 8;    // LDS row stride of the transpose (keeps 16-byte runs aligned)

// hT[d][r] for r < 256 * active tiles, d < H (haug: [M_pad][Ka] fragment-major,
// the h part starting at K chunk kb8).
__global__ void __launch_bounds__(256) k_hT(const uint16_t *haug, int64_t ks16, int kb8, int M_pad, int H,
                                            const int *cnt, const float *fac, uint16_t *hT, const TokRec *tok,
                                            uint16_t *ctT, int64_t ld_coeff) {
  const int r0 = blockIdx.x * TR, d0 = blockIdx.y * TR;
  if (r0 >= active_tiles(cnt) * BM) return;
  __shared__ __attribute__((aligned(16))) uint16_t sT[TR * TLD];
  const int tid = threadIdx.x;
  const int n = cnt[0];
  if (ctT && blockIdx.y == 0 && tid < TR) {
    // the target entry of row r in the chunk that holds its target, rounded
    // to bf16 like every other coefficient (targets are in [0, V) or -1)
    const int r = r0 + tid;
    const int tgt = tok[r].tgt;
    if (r < n && tgt >= 0) {
      const int64_t c = tgt / ld_coeff, vl = tgt - c * ld_coeff;
      ctT[(size_t)c * ld_coeff * M_pad + frag_slot(vl, r >> 3, M_pad / 16) + (r & 7)] =
          (uint16_t)bf16_rne(fac[2 * r + 1]);
    }
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = tid + 256 * k, r = i >> 3, c = i & 7;
    u32x4_t x = *(const u32x4_t *)(haug + frag_slot(r0 + r, kb8 + (d0 >> 3) + c, ks16));
    if (fac) {
      const float f = (r0 + r < n) ? fac[2 * (r0 + r)] : 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = pack_rne(bf16_to_f32(x[e] & 0xFFFFu) * f, bf16_to_f32(x[e] >> 16) * f);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sT[(8 * c + 2 * e) * TLD + r] = (uint16_t)(x[e] & 0xFFFFu);
      sT[(8 * c + 2 * e + 1) * TLD + r] = (uint16_t)(x[e] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = tid + 256 * k, d = i >> 3, j = i & 7;
    *(u32x4_t *)(hT + (size_t)(d0 + d) * M_pad + r0 + 8 * j) = *(const u32x4_t *)(sT + d * TLD + 8 * j);
  }
}

// coeffT: rows = local vocabulary rows of the chunk, K = tokens (ks16t = M_pad / 16).
__global__ void __launch_bounds__(256) k_coeffT(const uint16_t *coeff, int64_t ksv, const int *cnt,
                                                const TokRec *tok, const float *fac, int64_t V, int64_t chunk_v0,
                                                uint16_t *coeffT, int64_t ks16t) {
  const int r0 = blockIdx.x * TR, c0 = blockIdx.y * TR;
  if (r0 >= active_tiles(cnt) * BM) return;
  __shared__ __attribute__((aligned(16))) uint16_t sT[TR * TLD];
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = tid + 256 * k, r = i >> 3, c = i & 7;
    const u32x4_t x = *(const u32x4_t *)(coeff + frag_slot(r0 + r, (c0 >> 3) + c, ksv));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sT[(8 * c + 2 * e) * TLD + r] = (uint16_t)(x[e] & 0xFFFFu);
      sT[(8 * c + 2 * e + 1) * TLD + r] = (uint16_t)(x[e] >> 16);
    }
  }
  __syncthreads();
  if (tid < TR) {  // the token's target column, if it falls in this block
    const TokRec rec = tok[r0 + tid];
    const int64_t vl = (int64_t)rec.tgt - chunk_v0 - c0;
    const float tv = fac ? fac[2 * (r0 + tid) + 1] : rec.tval;
    if (rec.tgt >= 0 && (int64_t)rec.tgt < V && vl >= 0 && vl < TR) sT[vl * TLD + tid] = (uint16_t)bf16_rne(tv);
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = tid + 256 * k, v = i >> 3, j = i & 7;
    *(u32x4_t *)(coeffT + frag_slot(c0 + v, (r0 >> 3) + j, ks16t)) = *(const u32x4_t *)(sT + v * TLD + 8 * j);
  }
}

constexpr int WKS = 64;  // tokens per K step

// LDS hT tile [256 d][64 tokens] bf16, 16-byte chunk c of row d at c ^ ((d ^ (d >> 2)) & 7).
__device__ __forceinline__ int wswz(int d, int chunk) { return d * WKS + ((chunk ^ ((d ^ (d >> 2)) & 7)) << 3); }

// Producer: thread t copies row d = t >> 1 of the tile, tokens 32 (t & 1) .. +32 of the step.
struct WRegs {
  uint32_t w[16];
};

__global__ void __launch_bounds__(TW, 1) k_dw(DwArgs a) {
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  if (bid >= a.nvt * a.HT) return;
  const int dt = bid % a.HT, vt = bid / a.HT;
  const int d0 = dt * 256;
  const int nsteps = active_tiles(a.cnt) * (BM / WKS);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tg = wave >> 1, dh = wave & 1;
  const int l32 = lane & 31, lh = lane >> 5;

  __shared__ __attribute__((aligned(16))) uint16_t sB[2][256 * WKS];

  const int row0 = tg * 64;  // this wave's first vocabulary row of the tile
  // fragment-major transposed coefficients of the tile's 256 rows: one 1 KiB
  // block per (32 rows, 16 tokens)
  const rsrc_t rc = make_rsrc(a.coeffT + (size_t)(vt * 8) * a.ks16t * 512, (int64_t)8 * a.ks16t * 1024);
  const int cv0 = ((tg * 2) * (int)a.ks16t * 64 + lane) * 16;
  const int cstride = (int)a.ks16t * 1024;
  const int64_t drows = a.H - d0 < 256 ? a.H - d0 : 256;
  const rsrc_t rb_ = make_rsrc(a.hT + (size_t)d0 * a.M_pad, drows * a.M_pad * 2);
  const int pd = tid >> 1, ph = tid & 1;
  const int pv = pd * a.M_pad * 2 + ph * 64;

  f32x16_t acc[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[rb][c][e] = 0.0f;

  if (nsteps > 0) {
    auto load = [&](int st, WRegs &p) {
      const int so = (st < nsteps ? st : nsteps - 1) * WKS * 2;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4_t x = buf_load16(rb_, pv + 16 * i, so);
        p.w[4 * i] = x[0]; p.w[4 * i + 1] = x[1]; p.w[4 * i + 2] = x[2]; p.w[4 * i + 3] = x[3];
      }
    };
    auto store = [&](int i, const WRegs &p, uint16_t *sb) {
      *(u32x4_t *)(sb + wswz(pd, 4 * ph + i)) = u32x4_t{p.w[4 * i], p.w[4 * i + 1], p.w[4 * i + 2], p.w[4 * i + 3]};
    };
    int boff[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) boff[ks] = wswz(dh * 128 + l32, 2 * ks + lh);
    bf16x8_t cA[2][4];
    WRegs P0, P1;
    load(0, P0);
    load(1, P1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      cA[0][ks] = __builtin_bit_cast(bf16x8_t, buf_load16(rc, cv0 + ks * 1024, 0));
      cA[1][ks] = __builtin_bit_cast(bf16x8_t, buf_load16(rc, cv0 + cstride + ks * 1024, 0));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) store(i, P0, sB[0]);
    __syncthreads();

    // step st: MFMAs on buffer st & 1; copy step st + 1 (in `cur`) into the
    // other buffer between them; load step st + 2 into `nxt`.
    auto do_step = [&](int st, WRegs &cur, WRegs &nxt) {
      const int cb = st & 1;
      load(st + 2, nxt);
      const uint16_t *sw = sB[cb];
      const int knext = (st + 1 < nsteps ? st + 1 : st) * 4 * 1024;
      bf16x8_t bq[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) bq[c] = *(const bf16x8_t *)(sw + boff[0] + c * 32 * WKS);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            acc[rb][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cA[rb][ks], bq[c], acc[rb][c], 0, 0, 0);
          if (ks < 3) bq[c] = *(const bf16x8_t *)(sw + boff[ks + 1] + c * 32 * WKS);
        }
        cA[0][ks] = __builtin_bit_cast(bf16x8_t, buf_load16(rc, cv0 + ks * 1024, knext));
        cA[1][ks] = __builtin_bit_cast(bf16x8_t, buf_load16(rc, cv0 + cstride + ks * 1024, knext));
        store(ks, cur, sB[cb ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
      __syncthreads();
    };
    int st = 0;
    for (; st + 1 < nsteps; st += 2) {
      do_step(st, P1, P0);
      do_step(st + 1, P0, P1);
    }
    if (st < nsteps) do_step(st, P1, P0);
  }

  // result lane layout: column d0 + dh*128 + c*32 + l32, rows row0 + rb*32 + 8i + 4*lh + j
  const int64_t v0 = a.chunk_v0 + (int64_t)vt * 256;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int d = d0 + dh * 128 + c * 32 + l32;
    if (d >= a.H) continue;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t v = v0 + row0 + rb * 32 + 8 * i + 4 * lh + j;
          if (v < a.V) a.dw[v * a.H + d] = acc[rb][c][4 * i + j];
        }
  }
}

void launch_hT(hipStream_t st, const uint16_t *haug, int64_t ks16, int kb8, int M_pad, int H, const int *cnt,
               const float *fac, uint16_t *hT, const TokRec *tok, uint16_t *ctT, int64_t ld_coeff) {
  hipLaunchKernelGGL(k_hT, dim3((unsigned)(M_pad / TR), (unsigned)(H / TR)), dim3(256), 0, st, haug, ks16, kb8,
                     M_pad, H, cnt, fac, hT, tok, ctT, ld_coeff);
}

void launch_coeffT(hipStream_t st, const uint16_t *coeff, int64_t ksv, int M_pad, int vrows, const int *cnt,
                   const TokRec *tok, const float *fac, int64_t V, int64_t chunk_v0, uint16_t *coeffT) {
  hipLaunchKernelGGL(k_coeffT, dim3((unsigned)(M_pad / TR), (unsigned)(vrows / TR)), dim3(256), 0, st, coeff, ksv,
                     cnt, tok, fac, V, chunk_v0, coeffT, (int64_t)M_pad / 16);
}

void launch_dw(hipStream_t st, const DwArgs &a) {
  const int n = a.nvt * a.HT;
  hipLaunchKernelGGL(k_dw, dim3((unsigned)((n + 7) / 8 * 8)), dim3(TW), 0, st, a);
}

}  // namespace cce
