// cce_device.h -- shared types and device helpers of libcce's gfx950 kernels (the flash cut-cross-entropy head).
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
//    (S = per-group sum of h) rides along as extra K columns: b' in per-row
//    fixed point as three signed byte digits, S split into three bf16
//    pieces, and the digit x piece products that matter as MFMA columns
//    (a 16-bit block, and a refinement block to 24 bits, see kernels.hip).
//  * The backward contracts bf16 coefficients -g*p*c' with a bf16-dequantized
//    head tile (s*q + b rounded once, in LDS), fp32 accumulation.  The target
//    column's whole term g*(1 - p_t)*c'_t*w_t is kept out of that path and
//    added in fp32, with 1 - p_t = -expm1(y_t - lse): exact for a flat softmax
//    (where that term dominates) and for a peaked one (where it is a small
//    difference of large numbers).  The target logit y_t is taken from the
//    tile that owns the target's column, so it carries the same arithmetic as
//    the lse it is compared with.
//
// MFMA v_mfma_f32_32x32x16_bf16 lane layout (verified on gfx950): operand
// lane l holds row l%32, K elements 8*(l/32)..+8; result lane l holds column
// l%32, rows 8i + 4*(l/32) + j in element 4i + j (i, j in 0..3).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cce {

typedef short bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BM = 256;        // tokens per workgroup tile (4 waves x 64)
constexpr int BNT = 256;       // vocabulary rows per logit tile
constexpr int TW = 512;        // threads per logit-tile workgroup (8 waves)
constexpr int KSTEP = 64;      // K per step = one quantization group
constexpr int MAX_G = 256;     // H <= 16384: K steps of 64
constexpr int MAX_GQ = 512;    // quantization groups per row (group >= 32)

// Per-token side data, one 16-byte record per compacted row.
struct TokRec {
  float lse;   // backward: lse of the token (0 for padding rows)
  float g;     // backward: cotangent (0 for padding rows)
  float tval;  // forward: softcapped target logit; backward: target coefficient.
               // 0 from the front; the tile workgroup whose vocabulary tile
               // holds the target overwrites it (one writer per token)
  int tgt;     // target id in [0, V), or -1 (padding row, out-of-range target)
};

// Bias block precision.  Bound on the error one logit takes from the 16-bit
// (coarse) bias block: 2^-15 * B * T, with B the head's largest |b'| and T the
// token's sum over groups of |S_g|; the refinement block (24 bits) brings it
// to 2^-22 * B * T.  A token tile takes the refinement when the coarse bound
// of any of its tokens exceeds this (absolute logit error).
constexpr float BIAS_COARSE_TOL = 1e-4f;
constexpr float BIAS_COARSE_BOUND = 1.0f / 32768.0f;  // 2^-15
// Fixed-point range of b' in units u_v = max_g |b'| / BIAS_NMAX: three
// balanced signed digits, n = 65536 d2 + 256 d1 + d0, |d| <= 127 at the top.
constexpr float BIAS_NMAX = 8355711.0f;

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats -> one bf16 pair (lo in bits 0..15), round to nearest even
// (one v_cvt_pk_bf16_f32 on gfx950).  Exact for values that fit in bf16.
__device__ __forceinline__ uint32_t pack_rne(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// fp32 -> bf16 bits, round to nearest, ties to even.
__device__ __forceinline__ uint32_t bf16_rne(float f) { return pack_rne(f, 0.0f) & 0xFFFFu; }

// 8 four-bit codes of one word -> 4 dwords of bf16 pairs (exact: codes < 256), in element order.
__device__ __forceinline__ void unpack4(uint32_t w, uint32_t *o) {
  const uint32_t ev = w & 0x0F0F0F0Fu;         // codes 0,2,4,6 in bytes 0..3
  const uint32_t od = (w >> 4) & 0x0F0F0F0Fu;  // codes 1,3,5,7
#pragma unroll
  for (int k = 0; k < 4; ++k)
    o[k] = pack_rne((float)((ev >> (8 * k)) & 0xFFu), (float)((od >> (8 * k)) & 0xFFu));
}

// 4 eight-bit codes of one word -> 2 dwords of exact bf16 pairs.
__device__ __forceinline__ void unpack8(uint32_t w, uint32_t *o) {
  o[0] = pack_rne((float)(w & 0xFFu), (float)((w >> 8) & 0xFFu));
  o[1] = pack_rne((float)((w >> 16) & 0xFFu), (float)(w >> 24));
}

// 4 signed bytes of one word -> 2 dwords of exact bf16 pairs.
__device__ __forceinline__ void unpack8s(uint32_t w, uint32_t *o) {
  o[0] = pack_rne((float)((int)(w << 24) >> 24), (float)((int)(w << 16) >> 24));
  o[1] = pack_rne((float)((int)(w << 8) >> 24), (float)((int)w >> 24));
}

template <int BITS>
__device__ __forceinline__ uint32_t code_at(const uint32_t *row, int d) {
  constexpr int PER = 32 / BITS;
  return (row[d / PER] >> (BITS * (d % PER))) & ((1u << BITS) - 1u);
}

// Fragment-major layout of a bf16 [rows][K] operand (K % 16 == 0): each
// 32-row x 16-K block of v_mfma_f32_32x32x16_bf16 is 1 KiB, stored in the
// order its 64 lanes read it (lane l: row l%32, K 8*(l/32)..+8), so one
// 16-byte-per-lane load covers eight whole cache lines.  ks16 = K / 16.
// Offset (in elements) of the 16-byte slot holding row t, K chunk c (= k/8):
__device__ __forceinline__ size_t frag_slot(int64_t t, int c, int64_t ks16) {
  return ((((size_t)(t >> 5) * ks16 + (c >> 1)) * 64) + (t & 31) + 32 * (c & 1)) * 8;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

struct TileArgs {
  const uint16_t *haug;  // [M_pad][Ka] bf16, fragment-major
  const uint8_t *baug;   // [V][Kb] fixed-point digits (offset by 128): head side of the bias block
  const float *rt;       // [NB + G][V] fold ratio of every step (before its first K column)
  const float *slast;    // [V] effective scale of the last group
  const unsigned *bmxb;  // [nbmx] largest |b'| (fp32 bits) of each 64-row block of the head
  int nbmx;
  const float *sabs;     // [M_pad] sum over groups of |S_g| of each compacted row (0: padding)
  const uint32_t *wq;
  const int *cnt;
  TokRec *tok;           // read: lse, g, tgt; written: tval of the tokens whose target is in the tile
  float *part;           // forward: [nwr][M_pad] x (max, sumexp); uncapped single pass: the same over the
                         // non-target columns
  float *ncR;            // uncapped single pass: [32-row vocabulary block][M_pad] reference of each block's
                         // coefficients (the token's largest logit in the block)
  uint16_t *coeff;       // backward: [M_pad][ld_coeff] bf16 coefficient chunk
  int64_t ld_coeff;
  // dense head's single pass with dW, or NULL: the chunk's coefficients also
  // as dW's operand, [ld_coeff vocabulary rows][M_pad tokens] fragment-major
  // (ks16t = M_pad / 16), the target's entry left 0 for launch_hT to fill
  uint16_t *coeffT;
  int64_t ks16t;
  int64_t V;
  int G, Ka, Kb, NB, wpr, M_pad;  // NB, G: K steps of the bias block and of h (kw columns each)
  int NBr;               // K steps of the bias block's refinement half (its first half)
  int kw;                // K columns per step: 64, or 32 for quantization group 32
  int64_t ks16;          // Ka / 16 (fragment-major h rows)
  int64_t ksv;           // ld_coeff / 16 (fragment-major coefficient chunk)
  int range_tile0, range_tiles;
  int nblocks;           // launched work ids (the split per active token tile is derived on the device)
  int max_splits;        // forward: capacity of the partial buffer in splits per token and chunk
  // The range is chunk `chunk` of a vocabulary cut into chunks of full_tiles
  // tiles (one chunk covering the range: chunk 0, full_tiles = range_tiles);
  // the split size follows the full chunk, so the partials of every chunk
  // are numbered on from the previous chunk's (see vsplit).
  int chunk, full_tiles;
  float *tdc;            // coefficient passes: c'(z) of each compacted row's target, next to its tval
  // backward: 1 = write each split's non-target probability mass to `mass`
  // and the target's logit and c' (tval, tdc), the reduce forming the target's
  // term from them; 0 = tval is the target's whole coefficient, with
  // 1 - p_t = -expm1(y_t - lse) (the skips, and a dense head, whose dW takes
  // the coefficient chunk by chunk)
  int tmass;
  float *mass;           // backward with tmass, single pass: [M_pad][mass_ld] non-target mass (sum) of each split
  int mass_ld;
  // backward of cce_forward_backward without a softcap reference: each lane
  // forms its token's lse from the forward's partials (fpart, the forward
  // launch's split plan f_*) instead of a merge launch, and the workgroup of
  // split 0 of chunk 0 (vocabulary half 0) writes logp and lse of its tokens
  const float *fpart;
  int f_nblocks, f_tiles, f_max_splits;
  float *out_logp, *out_lse;
  float cap, inv_cap;
  // forward, optional: block_max[idx[r]][tile] = largest softcapped logit of
  // vocabulary tile `tile` for compacted row r (nbv = tiles per row)
  float *bmx;
  const int *idx;
  int64_t nbv;
  // backward, optional: fl[tt * fl_ld + tile] = 1 while the (token tile,
  // vocabulary tile) pair is needed; cold pairs (0) are not computed, and the
  // coefficient filter clears the pairs whose non-target |coefficients| all
  // stay below filter_eps (0 = no filter)
  uint8_t *fl;
  int64_t fl_ld;
  float filter_eps;
  int small;             // 1: at most 64 tokens (token group 0 of the tile multiplies); 2: at most 32
};

// Arguments of the front launch (token rows, target logit, head side).
struct FrontArgs {
  const uint16_t *h;       // [M][H] bf16
  const int *idx;          // [M_pad] compacted row -> token (-1: padding)
  const int32_t *targets;
  const float *lse, *g;    // backward only (lse NULL in the forward)
  const uint32_t *wq;
  const void *scales, *biases;  // [V][Gq] of sbt
  TokRec *tok;
  uint16_t *haug;
  uint8_t *baug;           // head side: bias-block digits, fold ratios, last scale
  float *rt, *slast;
  unsigned *bmxb;          // [ceil(V / 64)]: largest |b'| (fp32 bits) of each block of 64 rows
  float *sabs;             // [M_pad]: sum over groups of |S_g| of each compacted row
  int64_t V;
  int H, G, Kb, Ka, NB, wpr, M_pad;  // NB, G: tile K steps of the bias block and of h
  int P;                   // columns of each half of the bias block (Kb = 2 P)
  int gs, Gq, sbt;         // quantization group, groups per row, scale/bias dtype
  float cap;
  int bwd;
  int head;                // 1: the head blocks run (the head side is not prepared)
  // compact != 0: the row blocks compact the mask themselves (small M) and
  // write idx_out, inv and cnt; otherwise idx comes from the compaction launch
  int compact, M;
  const uint8_t *mask;
  int *idx_out, *inv, *cnt;
  // non-NULL: logp and lse of masked tokens are written (0) here
  float *out_logp, *out_lse;
};

struct GemmArgs {
  const uint16_t *coeff;  // fragment-major [M_pad][16 * ksv] bf16 coefficient chunk
  int64_t ksv;            // K blocks of 16 vocabulary rows per 32-token row block of the chunk
  const uint32_t *wq;
  const void *scales;     // [V][Gq] of sbt
  const void *biases;
  const int *cnt;
  float *dh_part;        // [ksplit][M_pad][H]
  int64_t V;
  int64_t chunk_v0;      // first vocabulary row of the chunk
  int H, wpr, M_pad;
  int gs, Gq, sbt;       // quantization group, groups per row, scale/bias dtype
  int chunk_steps;       // 64-row K steps in this chunk
  int max_chunk_steps;   // K steps of a full chunk (fixes the split across chunks)
  int TT, HT, ksplit, nblocks;  // ksplit: slab capacity in units of all TT token tiles
  int accumulate;
  // optional pair flags of the skips (as in TileArgs): a split contracts only
  // the vocabulary tiles whose flag is set for its token tile
  const uint8_t *fl;
  int64_t fl_ld;
  int chunk_tile0;       // first vocabulary tile of the chunk
  int small;             // as in TileArgs
  // uncapped single pass, small-M variant only (or NULL): the coefficients
  // were written against their 32-row block's reference ncR (TileArgs::ncR)
  // and are brought to the token's largest logit nc[3 r] as they are staged:
  // times e^{R - m}, rounded to bf16 (rows from the supervised count on and
  // slots past V as stored)
  const float *ncR;
  const float *nc;
};

// Raw buffer resource over [base, base + bytes): a lane whose byte offset is
// at or past `bytes` reads zeros (and its write is dropped), so ragged tails
// need no per-lane predicate.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7FFFFFFFll ? 0x7FFFFFFFll : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n, 0x00020000);
}
__device__ __forceinline__ u32x4_t buf_load16(rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ float buf_loadf(rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// Work split chosen on the device from the supervised-token count (the host
// does not know it without a synchronization): `nblocks` launched workgroups
// cover act = ceil(cnt / 256) active token tiles, each with as many splits of
// `units` (vocabulary tiles or K steps) as fit; the result is also the number
// of per-token partials to merge.
__device__ __forceinline__ int active_tiles(const int *cnt) { return (cnt[0] + BM - 1) / BM; }
__device__ __forceinline__ int splits_for(int nblocks, int act, int units, int cap) {
  int n = nblocks / (act > 0 ? act : 1);
  n = n < cap ? n : cap;
  n = n < units ? n : units;
  n = n > 1 ? n : 1;
  const int per = (units + n - 1) / n;
  return (units + per - 1) / per;
}

// Vocabulary splits of a tile launch over chunk `chunk` (range_tiles tiles)
// of a vocabulary cut into chunks of full_tiles tiles: nwr_full splits of tpw
// tiles per active token tile for a full chunk, nwr of them for this one,
// whose partials start at split slot0 = chunk * nwr_full.  `nblocks` is the
// work ids of a full chunk's launch (every chunk is launched alike).
struct VSplit {
  int nwr_full, tpw, nwr, slot0;
};
__device__ __forceinline__ VSplit vsplit(int nblocks, int act, int full_tiles, int range_tiles, int chunk, int cap) {
  VSplit v;
  v.nwr_full = splits_for(nblocks, act, full_tiles, cap);
  v.tpw = (full_tiles + v.nwr_full - 1) / v.nwr_full;
  v.nwr = (range_tiles + v.tpw - 1) / v.tpw;
  v.slot0 = chunk * v.nwr_full;
  return v;
}
// Splits (partials per token, in pairs of vocabulary halves) over all `tiles`
// tiles of the vocabulary cut into chunks of full_tiles.
__device__ __forceinline__ int vsplit_total(int nblocks, int act, int full_tiles, int tiles, int cap) {
  const int nch = (tiles + full_tiles - 1) / full_tiles;
  const VSplit v = vsplit(nblocks, act, full_tiles, tiles - (nch - 1) * full_tiles, nch - 1, cap);
  return v.slot0 + v.nwr;
}

// K splits of the dh contraction for act active token tiles: as many as the
// launched workgroups allow, bounded by the slab capacity (ks * act <=
// ksplit * TT, the slabs being laid out over the active rows only).
// Splits hold whole vocabulary tiles (4 K steps each; chunk_steps is a
// multiple of 4), so that a split can leave out the cold tiles of the skips.
__device__ __forceinline__ void dh_split(const GemmArgs &a, int act, int &ks, int &steps_per) {
  const int cap = a.ksplit * a.TT / (act > 0 ? act : 1);
  const int tiles = a.max_chunk_steps >> 2;
  ks = splits_for(a.nblocks / a.HT, act, tiles, cap);
  steps_per = 4 * ((tiles + ks - 1) / ks);
}

// Linear block id -> work id, so that consecutive work ids share an XCD
// (blocks are dispatched to the 8 XCDs round-robin).  nb_grid % 8 == 0.
__device__ __forceinline__ int xcd_remap(int b, int nb_grid) {
  return (b & 7) * (nb_grid >> 3) + (b >> 3);
}

// Scales and biases are stored as fp32, bf16 or fp16 (SB_*); all widen
// exactly to fp32.
enum { SB_F32 = 0, SB_BF16 = 1, SB_F16 = 2 };
// (selects, no branches: this sits in the dh contraction's main loop)
__device__ __forceinline__ float sb_widen(uint32_t bits, int sbt) {
  const float hf = (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
  const float bf = __uint_as_float(bits << 16);
  const float f = __uint_as_float(bits);
  return sbt == SB_F32 ? f : (sbt == SB_BF16 ? bf : hf);
}
__device__ __forceinline__ float ld_sb(const void *base, int64_t i, int sbt) {
  if (sbt == SB_F32) return static_cast<const float *>(base)[i];
  return sb_widen(static_cast<const uint16_t *>(base)[i], sbt);
}

__device__ __forceinline__ float scale_eff(float s) { return (fabsf(s) < 1e-30f) ? 1e-30f : s; }

// tanh from its exponential definition, tanh(x) = sign(x) (1 - e^-2|x|) / (1 + e^-2|x|)
// (relative error a few ulp, no cancellation since e^-2|x| <= 1).
__device__ __forceinline__ float tanh_exp(float x) {
  const float t = __expf(-2.0f * fabsf(x));
  return copysignf(__fdividef(1.0f - t, 1.0f + t), x);
}
// c(z) = cap * tanh(z / cap), identity when cap == 0.
__device__ __forceinline__ float softcap(float z, float cap, float inv_cap) {
  return (cap > 0.0f) ? cap * tanh_exp(z * inv_cap) : z;
}
// c(z) and c'(z) = 1 - tanh^2(z / cap).
__device__ __forceinline__ float softcap_d(float z, float cap, float inv_cap, float &dc) {
  if (cap > 0.0f) {
    const float th = tanh_exp(z * inv_cap);
    dc = 1.0f - th * th;
    return cap * th;
  }
  dc = 1.0f;
  return z;
}


// Launch entry points of the kernel translation units (host side).
// out_logp, out_lse: NULL, or outputs whose masked tokens get 0
void launch_compact(hipStream_t st, const uint8_t *mask, int M, int M_pad, int *idx, int *inv, int *cnt,
                    float *out_logp, float *out_lse);
void launch_front(hipStream_t st, int bits, const FrontArgs &f);
// Passes of the logit tile: forward partials, backward coefficients, or both
// at once (the fused pass, softcap in (0, CAP_FIXED_REF_MAX]; quantized heads).
enum { PASS_FWD = 0, PASS_BWD = 1, PASS_FUSED = 2, PASS_FUSED_NC = 3 };
constexpr float CAP_FIXED_REF_MAX = 40.0f;
void launch_tile(hipStream_t st, int bits, int pass, dim3 grid, const TileArgs &a);
void launch_warm(hipStream_t st, int TT, int64_t tiles, const int *cnt, const int *idx, const TokRec *tok,
                 const float *bmx, int64_t nbv, float log_eps, int block_on, uint8_t *fl);
void launch_bmx_mask(hipStream_t st, int M, int64_t nbv, const int *inv, float *bmx);
// nc (or NULL): the uncapped single pass's partials, which leave the target out;
// the merge then adds the target's own term and writes (m, S, e_t) per row
void launch_merge(hipStream_t st, int M, const float *part, int nblocks, int full_tiles, int tiles, int max_splits,
                  int M_pad, const int *inv, const int *cnt, const TokRec *tok, float *logp, float *lse,
                  float *nc = nullptr);
// The uncapped single pass: every coefficient of the ld_coeff-row chunks
// (nchunks of them, the last holding last_rows valid rows) times
// e^{R - m}, R its 32-row block's reference, m the token's largest logit
// (nc); supervised rows only.
void launch_nc_scale(hipStream_t st, uint16_t *coeff, int64_t ld_coeff, int nchunks, int64_t last_rows, int M_pad,
                     const int *cnt, const float *ncR, const float *nc);
void launch_dh_gemm(hipStream_t st, int bits, dim3 grid, const GemmArgs &a);
// How the split reduce forms the target's term g (1 - p_t) c'_t w_t.
//  mode 0: tval is the whole coefficient (the tile used -expm1(y_t - lse));
//  mode 1: 1 - p_t = S, the backward's non-target probability mass summed
//          over the partial slots in a fixed order; tval = y_t, tdc = c'_t;
//  mode 2: the fused pass: S sums e^{y - cap} over the non-target columns,
//          e_t = e^{y_t - cap}, the slabs (sums of -e c' w) are scaled by
//          g / (S + e_t) and 1 - p_t = S / (S + e_t).
struct ReduceTarget {
  int mode;
  // [M_pad][mass_ld], per split of the tile launches: mode 1 the backward's
  // non-target mass, mode 2 the single pass's sum of 4 e (e = e^{y - cap})
  // over the non-target columns
  const float *mass;
  int mass_ld;
  int nblocks, full_tiles, tiles, max_splits;  // the tile launches' split plan (vsplit_total)
  float cap;
  const float *tdc;    // [M_pad] c' of the target
  float *logp, *lse;   // mode 2: the outputs of the forward (the single pass has no merge launch)
  // mode 2, dense head (or NULL): per compacted row, the token's factor
  // g / (S + e_t) that turns the chunk's coefficients into g (1[v = t] - p_v) c'
  // and the target's coefficient in the chunk's units, S c'_t (read by the
  // dW launches)
  float *fac;
  // mode 3 (the uncapped single pass): per compacted row the token's largest
  // logit m, S (its non-target terms e^{z - m}) and e_t = e^{z_t - m}, from the
  // merge; lse and logp are the merge's
  const float *nc;
};
void launch_dh_reduce(hipStream_t st, int bits, int M, const GemmArgs &ga, const int *inv, const TokRec *tok,
                      void *dh, int out_bf16, const ReduceTarget &rt);

// Head gradient of a dense head (dw.hip): dW rows [chunk_v0, chunk_v0 + 256 nvt)
// of one coefficient chunk, all columns, over the active token tiles.
struct DwArgs {
  const uint16_t *coeffT;  // [local vocab row][token] fragment-major (ks16t = M_pad / 16)
  const uint16_t *hT;      // [H][M_pad] bf16: the compacted, padded hidden states transposed
  const int *cnt;
  float *dw;               // [V][H] fp32
  int64_t V, chunk_v0, ks16t;
  int H, M_pad, HT, nvt;   // HT: 256-column tiles of H; nvt: vocabulary tiles of the chunk
};
// fac (or NULL): the single pass's per-row factors (ReduceTarget::fac); hT then
// holds each row scaled by its factor, and coeffT takes the target's
// coefficient in the chunk's units.  tok (or NULL): the single pass whose
// tiles wrote every chunk's transposed coefficients (ctT, chunks of ld_coeff
// vocabulary rows): each row's target entry is set there to fac[2r + 1].
void launch_hT(hipStream_t st, const uint16_t *haug, int64_t ks16, int kb8, int M_pad, int H, const int *cnt,
               const float *fac, uint16_t *hT, const TokRec *tok = nullptr, uint16_t *ctT = nullptr,
               int64_t ld_coeff = 0);
void launch_coeffT(hipStream_t st, const uint16_t *coeff, int64_t ksv, int M_pad, int vrows, const int *cnt,
                   const TokRec *tok, const float *fac, int64_t V, int64_t chunk_v0, uint16_t *coeffT);
void launch_dw(hipStream_t st, const DwArgs &a);

}  // namespace cce
