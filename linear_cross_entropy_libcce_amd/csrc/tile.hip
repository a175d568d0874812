// tile.hip -- the logit tile kernel of libcce (forward partials and backward
// coefficients).  Built with the VGPR form of MFMA so the accumulator, which
// the VALU rescales every group, stays in architectural VGPRs.
#include "cce_device.h"

namespace cce {

// ---------------------------------------------------------------------------
// The logit tile: 256 tokens x 256 vocabulary rows per workgroup of 8 waves,
// K = Ka (bias block, then H).  Wave w owns tokens [64(w/2), +64) and vocab
// rows [128(w%2), +128) of the tile as 2 x 4 blocks of
// v_mfma_f32_32x32x16_bf16 (rows = tokens, columns = vocabulary rows).
//
// Per K step (one quantization group: 64 columns, 32 for group 32; a group of
// 128 takes two steps, the second with ratio 1):
//  * the code tile of the step is in LDS as bf16 (double buffered) and shared
//    by the eight waves;
//  * the token operand comes straight from the fragment-major augmented rows
//    into registers, one step ahead;
//  * the producer (every thread: 16 K values of two vocabulary rows) unpacks
//    the codes of the NEXT step into the other LDS buffer, in four slices
//    placed between the MFMAs, from words it loaded at the start of the
//    previous step (two register sets, alternating), so global latency is
//    covered by a step of MFMA work and the unpack rides in the MFMA shadow.
// All global reads are raw buffer loads: rows past V read as zeros, so there
// is no per-lane predicate and no branch in the step.
//
// Scale fold without a second accumulator: the accumulator is kept in units of
// the current group's scale, acc <- acc * (s_{g-1} / s_g) + A_g, so the MFMA
// accumulates in place and the VALU does one multiply per element per group.
// After the last group z = acc * s_last.  The ratios come from a table built
// once per call (the head side of the front launch); the bias block runs
// first with ratio 1 in units of the row's fixed-point unit, and a scale of
// exactly 0 is replaced by 1e-30, whose contribution is nil.
//
// Dense bf16 heads (BITS = 16, the trainable-head variant): the 32-wide step
// path with the head rows copied into LDS as they are; no bias block, no
// fold and no final scale.
//
// VAR_SMALL (at most 64 tokens, one token group): every wave multiplies the
// 64 tokens by its own 32 vocabulary rows of the tile (one column block), so
// all eight waves share the MFMA work and the epilogues; the forward
// combines the waves' softmax partials into the two halves' partials at the
// end.  VAR_SMALL32 (at most 32 tokens): the same with one 32-row token block,
// so half the MFMAs, folds, token fragments and coefficient stores; the
// epilogue's lanes 32..63 (padding tokens) compute on zeros and store nothing.
//
// VAR_EXTRA (a second instantiation, so the plain passes carry none of it):
//  * forward: the largest logit of every (token, vocabulary tile), written to
//    block_max after the softcap (monotonic, so the max commutes with it);
//  * backward: the (token tile, vocabulary tile) pairs whose flag is clear
//    are skipped (no MFMA work, no coefficients), and with a filter the flag
//    of a computed pair is cleared when all its non-target |coefficients|
//    are below filter_eps.  The dh contraction reads the same flags.

constexpr int ZROW = 36;  // padded fp32 row stride of the per-wave transpose scratch (32 columns)
constexpr float LOG2E = 1.4426950408889634f;

// MODE_FUSED (softcap <= 40): the forward's fixed reference e^{c(z) - cap}
// also gives every coefficient up to a per-token factor, so one pass writes
// both the partial sums and the unnormalized coefficients -e^{c(z) - cap} c'(z)
// (the split reduce scales them by g e^{cap - lse} once the merge has lse).
// MODE_FUSED_NC (no softcap): no fixed reference exists, so each 32-row
// vocabulary block's coefficients -e^{z - R} are taken against the block's own
// largest logit R (written to ncR), and the forward's (max, sum) partials run
// over the non-target columns; once lse and the token's largest logit are known
// a scaling launch brings every block to one reference.
enum { MODE_FWD = 0, MODE_FWD_CAP = 1, MODE_BWD = 2, MODE_FUSED = 3, MODE_FUSED_NC = 4 };
enum { VAR_PLAIN = 0, VAR_EXTRA = 1, VAR_SMALL = 2, VAR_SMALL32 = 3 };

// One step's worth of head data for one producer thread: 16 K values of each
// of two vocabulary rows (8-bit codes and bias digits: 4 words per row; 4-bit
// codes: the first 2 words per row) -- or, with 32-wide steps, 16 K values of
// one row (dense bf16 heads: all 8 words) -- and the fold ratio of one row.
struct ProdRegs {
  uint32_t w[8];
  float r;
};

// The LDS code tile is [256 rows][KW K] bf16 without padding.  KW = 64: the
// 16-byte chunk c of row n sits at chunk position c ^ ((n >> 1) & 7), which
// spreads both the B-operand reads (consecutive rows, one chunk) and the
// producer writes (4 rows x 4 chunk pairs per 16 lanes) over distinct bank
// groups.  KW = 32 (group 32: one K step per quantization group, one fold per
// step): chunk c of row n at c ^ ((n >> 2) & 3), so that 16 consecutive rows
// of one chunk cover all 64 banks.
template <int KW>
__device__ __forceinline__ int swz(int row, int chunk) {
  if (KW == 64) return row * 64 + ((chunk ^ ((row >> 1) & 7)) << 3);
  return row * 32 + ((chunk ^ ((row >> 2) & 3)) << 3);
}

// Producer mapping, KW = 64: wave w, lane l loads the 16-byte K slice l & 3 of
// rows 32w + (l >> 2) and 32w + 16 + (l >> 2), so one load instruction covers
// 16 rows x 64 contiguous bytes.  KW = 32: thread t loads the K half t & 1 of
// row t >> 1 (16 values: 16 bytes of 8-bit codes or digits, 8 of 4-bit
// codes, 32 of dense bf16 rows), one load instruction covering 32 rows x 32
// K.  Threads 0..255 also carry row t's fold ratio (none for a dense head).
template <int BITS, bool GS32>
struct Producer {
  static constexpr bool DENSE = BITS == 16;  // bf16 head rows: no codes, no scales
  static constexpr int KW = GS32 ? 32 : 64;
  static_assert(!DENSE || GS32, "dense heads use 32-wide steps");
  int row0, q, tid;

  // Issue the loads of step `step` of the vocabulary tile at v0: a bias-block
  // step (step < NB: fixed-point digits) or group step - NB (codes), and the
  // fold ratio of the step from the precomputed table.  The source is chosen
  // with wave-uniform selects, so no branch.
  __device__ __forceinline__ void load(const TileArgs &a, int64_t v0, int step, ProdRegs &p) const {
    const int64_t rows = a.V - v0 < BNT ? a.V - v0 : BNT;
    const bool bias = step < a.NB;
    const int g = step - a.NB;
    // a bias step reads the digits of this wave's 32 rows, which lie in one
    // 64-row block; a block whose largest |b'| is 0 has no digits stored (the
    // front skips it), and an empty resource reads its zero digits as zeros
    int64_t brows = rows;
    if (!DENSE && bias) {  // wave-uniform: only bias steps look the block up
      const int64_t blk = (v0 >> 6) + __builtin_amdgcn_readfirstlane(tid >> 7);
      if (a.bmxb[blk < a.nbmx ? blk : a.nbmx - 1] == 0u) brows = 0;
    }
    const rsrc_t rw = bias ? make_rsrc(a.baug + v0 * a.Kb, brows * a.Kb)
                           : make_rsrc(a.wq + v0 * a.wpr, rows * a.wpr * 4);
    const int rowb = bias ? a.Kb : a.wpr * 4;                // bytes per row
    const int qb = DENSE ? 32 : (bias || BITS == 8) ? 16 : 8;  // bytes per 16 K values
    const int so = bias ? step * KW : g * (KW * BITS / 8);
    if (GS32) {
      // row tid >> 1, K half tid & 1
      const int voff = (tid >> 1) * rowb + (tid & 1) * qb;
      if (DENSE) {
        const u32x4_t x = buf_load16(rw, voff, so), y = buf_load16(rw, voff + 16, so);
        p.w[0] = x[0]; p.w[1] = x[1]; p.w[2] = x[2]; p.w[3] = x[3];
        p.w[4] = y[0]; p.w[5] = y[1]; p.w[6] = y[2]; p.w[7] = y[3];
      } else {
        // 16 bytes for digits and codes alike (a 4-bit code step uses the
        // first 8): one load instruction for both kinds of step
        const u32x4_t x = buf_load16(rw, voff, so);
        p.w[0] = x[0]; p.w[1] = x[1]; p.w[2] = x[2]; p.w[3] = x[3];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const u32x4_t x = buf_load16(rw, (row0 + 16 * i) * rowb + q * qb, so);
        p.w[4 * i] = x[0]; p.w[4 * i + 1] = x[1]; p.w[4 * i + 2] = x[2]; p.w[4 * i + 3] = x[3];
      }
    }
    if (!DENSE) {
      const rsrc_t rr = make_rsrc(a.rt + (int64_t)step * a.V + v0, rows * 4);
      p.r = buf_loadf(rr, (tid & (BNT - 1)) * 4, 0);
    }
  }

  // Slice ks: row row0 + 16 * (ks >> 1), K chunk 2q + (ks & 1) (8 values).
  // 8-bit codes come as unsigned bytes; flipping the top bit gives the signed
  // value q - 128, one sign-extending convert per byte.  Bias digits are
  // stored as signed bytes and pass unflipped.  4-bit codes are used as
  // q - 8.
  // KW = 32: slice ks (0, 1) is K chunk 2 (tid & 1) + ks of row tid >> 1.
  __device__ __forceinline__ void store(bool bias, int ks, const ProdRegs &p, uint16_t *sw) const {
    const int i = GS32 ? 0 : ks >> 1, h = ks & 1;
    uint32_t o[4];
    if (DENSE) {  // bf16 as stored
      o[0] = p.w[4 * h]; o[1] = p.w[4 * h + 1]; o[2] = p.w[4 * h + 2]; o[3] = p.w[4 * h + 3];
    } else if (BITS == 8) {
      const uint32_t flip = bias ? 0u : 0x80808080u;  // wave-uniform
      unpack8s(p.w[4 * i + 2 * h] ^ flip, o);
      unpack8s(p.w[4 * i + 2 * h + 1] ^ flip, o + 2);
    } else {
      // 4-bit head: the eight nibbles of the code word are spread to bytes
      // (codes 0 1 2 3 | 4 5 6 7) as q | 0x80, less 8 per byte (no borrow
      // between bytes): 120 + q, whose flipped top bit is the signed code
      // q - 8.  A uniform select takes those or the two digit words, so both
      // kinds of step share one straight-line unpack.
      const uint32_t w = p.w[4 * i + h];
      const uint32_t ev = (w & 0x0F0F0F0Fu) | 0x80808080u, od = ((w >> 4) & 0x0F0F0F0Fu) | 0x80808080u;
      const uint32_t c0 = __builtin_amdgcn_perm(od, ev, 0x05010400u) - 0x08080808u;  // ev.b0 od.b0 ev.b1 od.b1
      const uint32_t c1 = __builtin_amdgcn_perm(od, ev, 0x07030602u) - 0x08080808u;  // ev.b2 od.b2 ev.b3 od.b3
      unpack8s(bias ? p.w[4 * i + 2 * h] : c0 ^ 0x80808080u, o);
      unpack8s(bias ? p.w[4 * i + 2 * h + 1] : c1 ^ 0x80808080u, o + 2);
    }
    const int off = GS32 ? swz<KW>(tid >> 1, 2 * (tid & 1) + h) : swz<KW>(row0 + 16 * i, 2 * q + h);
    *(u32x4_t *)(sw + off) = u32x4_t{o[0], o[1], o[2], o[3]};
  }

  __device__ __forceinline__ void ratio(const ProdRegs &p, float *sr) const {
    if (!DENSE && tid < BNT) sr[tid] = p.r;
  }
};

// Softcapped logit and its derivative from the exponential form of tanh:
// t = e^{-2|z|/cap}, th = sign(z) (1 - t) / (1 + t), c = cap * th, c' = 1 - th^2.
__device__ __forceinline__ float cap_d(float z, float c1, float cap, float &dc) {
  const float t = __builtin_amdgcn_exp2f(fabsf(z) * c1);
  const float th = copysignf((1.0f - t) * __builtin_amdgcn_rcpf(1.0f + t), z);
  dc = 1.0f - th * th;
  return cap * th;
}

template <int BITS, int MODE, int VAR, bool GS32>
__global__ void __launch_bounds__(TW, 1) k_tile(TileArgs a) {
  constexpr bool BWD = MODE == MODE_BWD;
  constexpr bool FUSED = MODE == MODE_FUSED;
  constexpr bool FNC = MODE == MODE_FUSED_NC;
  constexpr bool COEF = BWD || FUSED || FNC;  // writes coefficients
  constexpr int KW = GS32 ? 32 : 64;  // K columns per step (one quantization group)
  constexpr int NKS = KW / 16;        // MFMA k-steps per step
  constexpr bool DENSE = BITS == 16;  // bf16 head: no fold, no final scale
  constexpr bool EXTRA = VAR == VAR_EXTRA, SMALL = VAR == VAR_SMALL || VAR == VAR_SMALL32;
  constexpr int NRB = VAR == VAR_SMALL32 ? 1 : 2;  // 32-row token blocks per wave
  // epilogue columns per chunk: the fused pass keeps three values per column
  // live (logit, coefficient, probability term) next to the next step's
  // prefetched operands and takes 8 at a time (with 16 its step loop spilled)
  constexpr int EW = (FUSED || FNC) ? 8 : 16;
  // the single pass reads the logit only as 2 z / cap (the capped forward
  // keeps z: its block-maximum variant needs the raw logit, and the two give
  // bit-identical lse)
  constexpr bool ZPRE = FUSED;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  // the launched work ids are spread over the active token tiles only
  const int act = active_tiles(a.cnt);
  const VSplit vs = vsplit(a.nblocks, act, a.full_tiles, a.range_tiles, a.chunk, a.max_splits);
  const int tpw = vs.tpw;
  if (bid >= act * vs.nwr_full || bid % vs.nwr_full >= vs.nwr) return;
  const int tt = bid / vs.nwr_full, wr = bid % vs.nwr_full;
  const int tile_begin = wr * tpw;
  const int tile_end = min(tile_begin + tpw, a.range_tiles);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep it scalar
  // the two waves of a token group sit on two SIMDs; small M: one token group
  // and 32 vocabulary rows per wave
  const int tg = SMALL ? 0 : wave >> 1, vh = SMALL ? wave >> 2 : wave & 1;
  constexpr int NC = SMALL ? 1 : 4;  // 32-row column blocks per wave
  const int l32 = lane & 31, lh = lane >> 5;
  // First K step.  A head whose bias block is all zero digits (every b' = 0:
  // symmetric quantization, b = -128 s or -8 s) starts at the first code
  // step; the bias steps would add exact zeros to an accumulator that starts
  // at zero.  Otherwise the token tile takes the bias block's refinement
  // half only when the coarse half's error bound, 2^-15 B T with B the
  // head's largest |b'| and T the tile's largest sum of |S_g|, exceeds
  // BIAS_COARSE_TOL.  Forward and backward decide alike on the same inputs.
  // (The pipeline looks two steps ahead: at least two steps per tile.)
  __shared__ unsigned sDec[2][8];
  int s0 = 0;
  if (!DENSE) {
    unsigned bm = 0u, tm = 0u;  // fp32 bits of values >= 0: integer order is float order
    for (int i = tid; i < a.nbmx; i += TW) bm = max(bm, a.bmxb[i]);
    if (tid < BM) tm = __float_as_uint(a.sabs[tt * BM + tid]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      bm = max(bm, (unsigned)__shfl_xor((int)bm, o, 64));
      tm = max(tm, (unsigned)__shfl_xor((int)tm, o, 64));
    }
    if (lane == 0) {
      sDec[0][wave] = bm;
      sDec[1][wave] = tm;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      bm = max(bm, sDec[0][w]);
      tm = max(tm, sDec[1][w]);
    }
    const float B = __uint_as_float(bm), T = __uint_as_float(tm);
    s0 = (a.G < 2) ? 0 : (B == 0.0f ? a.NB : (BIAS_COARSE_BOUND * B * T > BIAS_COARSE_TOL ? 0 : a.NBr));
    s0 = __builtin_amdgcn_readfirstlane(s0);
  }
  const int steps = a.NB + a.G - s0;

  __shared__ __attribute__((aligned(16))) uint16_t sW[2][BNT * KW];
  __shared__ __attribute__((aligned(16))) float sR[2][BNT];
  __shared__ __attribute__((aligned(16))) float sZ[8][64 * ZROW];
  __shared__ float sX[2][BM];  // EXTRA: per-wave tile maxima, read after the step's barrier
  // coefficient passes: each lane's running non-target sum (kept in LDS, not
  // in a register the whole step loop would carry)
  __shared__ float sRun[COEF ? 8 : 1][64];
  if (COEF) sRun[wave][lane] = 0.0f;
  // small M: the eight waves multiply the same token rows, so the step's
  // token operand (2 row blocks x 4 k-steps = 8 fragments of 1 KiB) is loaded
  // once per workgroup, one fragment per wave, and shared through LDS (double
  // buffered like the code tile) instead of eight times from L1.
  __shared__ __attribute__((aligned(16))) u32x4_t sH[SMALL ? 2 : 1][SMALL ? 8 * 64 : 1];

  const int tok0 = tt * BM + tg * 64;
  const int vcol0 = SMALL ? wave * 32 : vh * 128;  // this wave's first vocabulary row within the tile
  // fragment-major h rows of the workgroup's 256 tokens: one 1 KiB block per
  // (32 tokens, 16 K); this wave's two token blocks start at hv0, hv0 + hstride.
  const rsrc_t rh = make_rsrc(a.haug + (size_t)(tt * BM >> 5) * a.ks16 * 512, (int64_t)8 * a.ks16 * 1024);
  const int hv0 = ((tg * 2) * (int)a.ks16 * 64 + lane) * 16;
  const int hstride = (int)a.ks16 * 1024;
  float *zs = sZ[wave];
  // small M: wave w stages token fragment (row block w / 4, k-step w % 4) of
  // each step; with one row block only waves 0..3 have one
  const bool hload = NRB == 2 || wave < 4;
  if (NRB == 1)  // padding token rows of the transpose scratch, never written by a tile
    for (int i = lane; i < 32 * ZROW; i += 64) zs[32 * ZROW + i] = 0.0f;

  float run_m = -INFINITY, run_s = 0.0f;
  // Backward: two per-token values carried through the step loop (the tile
  // sits at the register limit): the exponent offset and the coefficient
  // factor of the one epilogue form the softcap selects.
  //   cap > 0: p = exp2(fma(-2 cap log2 e, r, kofs)), kofs = cap log2 e - lse log2 e;
  //            coefficient p (r - r^2) kfac, kfac = -4 g
  //   no cap:  p = exp2(fma(z, log2 e, -kofs)), kofs = lse log2 e; kfac = -g
  float kofs = 0.0f, kfac = 0.0f;
  int tgt_t;
  {
    const TokRec rec = a.tok[tok0 + lane];
    tgt_t = rec.tgt;  // in [0, V), or -1
    if (BWD) {
      float lse_t = rec.lse;
      if (a.fpart) {
        // the forward's partials of this token, merged as the merge launch
        // would: lse = m* + log sum_s s_s e^{m_s - m*}
        // (one pass with a running maximum, eight partials loaded at a time)
        const int r = tok0 + lane;
        const int ns = 2 * vsplit_total(a.f_nblocks, act, a.f_tiles, a.f_tiles, a.f_max_splits);
        const float2 *fp = reinterpret_cast<const float2 *>(a.fpart) + r;
        float mx = -INFINITY, se = 0.0f;
        for (int k0 = 0; k0 < ns; k0 += 8) {
          float2 x[8];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            x[j] = (k0 + j < ns) ? fp[(size_t)(k0 + j) * a.M_pad] : float2{-INFINITY, 0.0f};
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float mn = fmaxf(mx, x[j].x);
            if (mn != -INFINITY) {
              se = se * __expf(mx - mn) + x[j].y * __expf(x[j].x - mn);
              mx = mn;
            }
          }
        }
        lse_t = mx + logf(se);
        if (a.chunk == 0 && wr == 0 && vh == 0 && (!SMALL || wave == 0) && r < a.cnt[0]) {
          const int t = a.idx[r];
          a.out_lse[t] = lse_t;
          a.out_logp[t] = rec.tval - lse_t;  // the forward's capture of the target logit
        }
      }
      const float lse2 = lse_t * LOG2E;
      kofs = a.cap > 0.0f ? LOG2E * a.cap - lse2 : lse2;
      kfac = a.cap > 0.0f ? -4.0f * rec.g : -rec.g;
    }
  }
  const float c1 = -2.0f * LOG2E * a.inv_cap;  // t = exp2(|z| * c1)
  const float c2 = -2.0f * LOG2E * a.cap;      // e^{c(z) - cap} = exp2(c2 / (1 + exp2(c3 z)))
  const float c3 = 2.0f * LOG2E * a.inv_cap;
  const float capl2 = LOG2E * a.cap;           // c(z) * log2(e) = capl2 * tanh(z / cap)
  const float m2capl2 = -2.0f * capl2;         // c(z) log2(e) = fma(m2capl2, r, capl2)

  // EXTRA backward: walk the flagged tiles of the range only
  const uint8_t *fl_row = (BWD && EXTRA) ? a.fl + (int64_t)tt * a.fl_ld + a.range_tile0 : nullptr;
  auto next_tile = [&](int t) {
    ++t;
    if (BWD && EXTRA)
      while (t < tile_end && fl_row[t] == 0) ++t;
    return t;
  };
  int n_tiles = tile_end - tile_begin;
  if (BWD && EXTRA) {
    n_tiles = 0;
    for (int t = tile_begin; t < tile_end; ++t) n_tiles += fl_row[t] != 0;
  }
  const int total = n_tiles * steps;
  if (total > 0) {
    Producer<BITS, GS32> pr;
    pr.row0 = wave * 32 + (lane >> 2);
    pr.q = lane & 3;
    pr.tid = tid;
    // Head words are loaded LA steps ahead into register sets used in turn:
    // two steps (P0, P1), or three for small M (P2 too), whose steps are
    // short enough that one step of cover left the loads waited for; small M
    // stages its token fragments three steps ahead alike (H0..H2).
    constexpr int LA = SMALL ? 3 : 2;
    ProdRegs P0, P1, P2;
    u32x4_t H0, H1, H2;
    // this lane's B-operand chunk offsets (row vcol0 + l32 + 32c, chunk 2ks + lh)
    int boff[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) boff[ks] = swz<KW>(vcol0 + l32, 2 * ks + lh);
    f32x16_t acc[2][NC];
    bf16x8_t hA[2][NKS];
    // small M starts each tile by folding with ratio 0 (see mfma_step): the
    // accumulator must hold finite values before the first tile
    if (SMALL)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[rb][c][e] = 0.0f;

    // step `n` steps after (tile, st)
    auto coords = [&](int tile, int st, int n, int64_t &v0, int &step) {
      int s2 = st + n, t2 = tile;
      while (s2 >= steps) { s2 -= steps; t2 = next_tile(t2); }
      v0 = (int64_t)(a.range_tile0 + t2) * BNT;
      step = s0 + s2;
    };
    const int first_tile = next_tile(tile_begin - 1);
    {
      const int64_t v0 = (int64_t)(a.range_tile0 + first_tile) * BNT;
      int64_t v1; int s1;
      coords(first_tile, 0, 1, v1, s1);
      pr.load(a, v0, s0, P0);
      pr.load(a, v1, s1, P1);
      if (SMALL) {
        int64_t v2; int s2;
        coords(first_tile, 0, 2, v2, s2);
        pr.load(a, v2, s2, P2);
        if (hload) {
          H1 = buf_load16(rh, hv0 + (wave >> 2) * hstride + (wave & 3) * 1024, s1 * NKS * 1024);
          H2 = buf_load16(rh, hv0 + (wave >> 2) * hstride + (wave & 3) * 1024, s2 * NKS * 1024);
        }
      }
#pragma unroll
      for (int part = 0; part < NKS; ++part) pr.store(s0 < a.NB, part, P0, sW[0]);
      pr.ratio(P0, sR[0]);
      if (SMALL) {
        if (hload)
          sH[0][wave * 64 + lane] = buf_load16(rh, hv0 + (wave >> 2) * hstride + (wave & 3) * 1024, s0 * NKS * 1024);
      } else {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          hA[0][ks] = __builtin_bit_cast(bf16x8_t, buf_load16(rh, hv0 + ks * 1024, s0 * NKS * 1024));
          hA[1][ks] = __builtin_bit_cast(bf16x8_t, buf_load16(rh, hv0 + hstride + ks * 1024, s0 * NKS * 1024));
        }
      }
      __syncthreads();
    }

    // The MFMA work of one step on LDS buffer cb, with the producer slices of
    // the next step (words in `cur`) placed between the MFMAs and the loads of
    // the step after next (into `nxt`) issued first.
    auto mfma_step = [&](int cb, bool first, int sn, int64_t vnn, int snn, ProdRegs &cur, ProdRegs &nxt,
                         u32x4_t &hcur, u32x4_t &hnxt) {
      const bool sbias = sn < a.NB;
      const int hnext = sn * NKS * 1024;  // fragment-major: 1 KiB per 16 K of a 32-row block
      // small M: this wave's token fragment of step + LA is loaded before the
      // head words, so that waiting for it does not wait for them too (loads
      // complete in issue order for s_waitcnt)
      if (SMALL && hload) hnxt = buf_load16(rh, hv0 + (wave >> 2) * hstride + (wave & 3) * 1024, snn * NKS * 1024);
      pr.load(a, vnn, snn, nxt);
      const uint16_t *sw = sW[cb];
      float r[NC];
      if (!DENSE)
#pragma unroll
        for (int c = 0; c < NC; ++c) r[c] = sR[cb][vcol0 + c * 32 + l32];
      // small M: a tile's first step clears the accumulator through its fold
      // (ratio 0; the accumulator is finite), one select per column block in
      // place of a select per accumulator element, which the compiler made of
      // the clearing in this three-step loop
      if (SMALL)
#pragma unroll
        for (int c = 0; c < NC; ++c) r[c] = first ? 0.0f : r[c];
      if (SMALL) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          hA[0][ks] = __builtin_bit_cast(bf16x8_t, sH[cb][ks * 64 + lane]);
          if (NRB == 2) hA[1][ks] = __builtin_bit_cast(bf16x8_t, sH[cb][(4 + ks) * 64 + lane]);
        }
      }
      // B operand of column block c for k-step ks + 1 is read as soon as its
      // two MFMAs of k-step ks are issued; a scheduling barrier after each
      // k-step keeps this order (left free, the compiler hoists every LDS read
      // and unpack and runs out of registers).
      bf16x8_t bq[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) bq[c] = *(const bf16x8_t *)(sw + boff[0] + c * 32 * KW);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        {
#pragma unroll
          for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
              if (ks == 0 && !DENSE) acc[rb][c] *= r[c];
              acc[rb][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hA[rb][ks], bq[c], acc[rb][c], 0, 0, 0);
            }
            if (ks < NKS - 1) bq[c] = *(const bf16x8_t *)(sw + boff[ks + 1] + c * 32 * KW);
          }
          // Left free, the compiler hoists the whole fold (128 multiplies)
          // above the first MFMA, and the matrix pipe idles while both waves
          // of a SIMD fold.  Pinned here: column block c's fold, then its two
          // MFMAs (measured 0.5-1.6% faster, except the capped forward).
          if (ks == 0 && !DENSE && MODE != MODE_FWD_CAP) {
#pragma unroll
            for (int c = 0; c < NC; ++c) {
              __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);  // VALU: the fold of acc[0..1][c]
              __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
            }
          }
          if (!SMALL) {
            hA[0][ks] = __builtin_bit_cast(bf16x8_t, buf_load16(rh, hv0 + ks * 1024, hnext));
            hA[1][ks] = __builtin_bit_cast(bf16x8_t, buf_load16(rh, hv0 + hstride + ks * 1024, hnext));
          }
        }
        pr.store(sbias, ks, cur, sW[cb ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
      pr.ratio(cur, sR[cb ^ 1]);
      if (SMALL && hload) sH[cb ^ 1][wave * 64 + lane] = hcur;  // step + 1's: read after the step's barrier
    };

    // ---- epilogue of vocabulary tile `tile`.  acc[rb][c][4i+j] is the logit
    // (in units of s_last) of token row rb*32 + 8i + 4*lh + j and vocab row
    // v0 + vcol0 + c*32 + l32.  Transposed per wave through its own LDS
    // scratch so that lane = token, then streamed in chunks of 16 columns.
    // The scratch is private to the wave: in-order LDS access within a wave
    // needs no workgroup barrier.
    auto epilogue = [&](int tile) {
      const int64_t v0 = (int64_t)(a.range_tile0 + tile) * BNT;
      const bool full = v0 + BNT <= a.V;
      float xm = BWD ? 0.0f : -INFINITY;  // EXTRA: max logit (forward) or max |coefficient| (backward)
      float sl[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) sl[c] = 1.0f;
      if (!DENSE) {
        const rsrc_t rl = make_rsrc(a.slast + v0, (a.V - v0 < BNT ? a.V - v0 : BNT) * 4);
#pragma unroll
        for (int c = 0; c < NC; ++c) sl[c] = buf_loadf(rl, (vcol0 + c * 32 + l32) * 4, 0);
      }
      // ZPRE: the epilogue only ever needs z through 2 z / cap (in log2 units),
      // so the transpose scratch holds acc * (s_last * c3): one multiply per
      // column instead of one per logit
      if (ZPRE)
#pragma unroll
        for (int c = 0; c < NC; ++c) sl[c] *= c3;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              zs[(rb * 32 + 8 * i + 4 * lh + j) * ZROW + l32] = acc[rb][c][4 * i + j] * sl[c];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // FNC: the block's reference, its largest logit over the valid columns
        // (the target's included); a block past V has none and adds nothing
        float Rb = 0.0f, Rb2 = 0.0f, esum = 0.0f;
        bool bvalid = true;
        if (FNC) {
          const int64_t vbk = v0 + vcol0 + c * 32;
          const int nvb = full ? 32 : (int)(a.V - vbk < 0 ? 0 : (a.V - vbk < 32 ? a.V - vbk : 32));
          float mx = -INFINITY;
#pragma unroll
          for (int k = 0; k < 32; k += 4) {
            const f32x4_t x = *(const f32x4_t *)(zs + lane * ZROW + k);
#pragma unroll
            for (int e = 0; e < 4; ++e) mx = fmaxf(mx, (k + e < nvb) ? x[e] : -INFINITY);
          }
          bvalid = nvb > 0;
          Rb = bvalid ? mx : 0.0f;
          a.ncR[(size_t)(vbk >> 5) * a.M_pad + tok0 + lane] = Rb;
          Rb2 = Rb * LOG2E;
        }
#pragma unroll 1
        for (int k0 = 0; k0 < 32; k0 += EW) {
          float z[EW];
#pragma unroll
          for (int k = 0; k < EW; k += 4) {
            const f32x4_t x = *(const f32x4_t *)(zs + lane * ZROW + k0 + k);
            z[k] = x[0]; z[k + 1] = x[1]; z[k + 2] = x[2]; z[k + 3] = x[3];
          }
          const int64_t vb = v0 + vcol0 + c * 32 + k0;
          const int nv = full ? EW : (int)(a.V - vb < 0 ? 0 : (a.V - vb < EW ? a.V - vb : EW));
          // the target's position among these EW columns, or -1 (targets are
          // in [0, V), so a position found is below nv)
          const int64_t dtk = (int64_t)tgt_t - vb;
          const int tk = (tgt_t >= 0 && dtk >= 0 && dtk < EW) ? (int)dtk : -1;
          // The lane whose target falls here writes the target's logit (and,
          // for the coefficient passes, its c') from this tile's own
          // arithmetic -- the rare chunk: a uniform branch; the coefficient
          // passes take it with their masking pass below.
          auto capture = [&]() {
            float zt = 0.0f;
#pragma unroll
            for (int k = 0; k < EW; ++k) zt = (k == tk) ? z[k] : zt;
            if (tk >= 0) {
              float yt = zt, dct = 1.0f;
              if (a.cap > 0.0f) {  // as the epilogues below: r = 1/(1 + e^{2z/cap})
                const float r = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(ZPRE ? zt : zt * c3));
                yt = a.cap * fmaf(-2.0f, r, 1.0f);
                dct = 4.0f * fmaf(-r, r, r);
              }
              if (BWD && !a.tmass) {
                // the target's whole coefficient g (1 - p_t) c'_t with
                // 1 - p_t = -expm1(y_t - lse) (g and lse as given, reloaded
                // here: not worth registers for the whole tile)
                const TokRec rec = a.tok[tok0 + lane];
                a.tok[tok0 + lane].tval = rec.g * -expm1f(yt - rec.lse) * dct;
              } else {
                a.tok[tok0 + lane].tval = yt;
                if (COEF && !FNC) a.tdc[tok0 + lane] = dct;  // the reduce forms the target's term
              }
            }
          };
          if (!COEF && __builtin_amdgcn_ballot_w64(tk >= 0) != 0) capture();
          if (MODE == MODE_FWD_CAP) {
            // |c(z)| <= cap: e^{c(z) - cap} needs no running maximum (cap <= 40,
            // so that even e^{-2 cap} is a normal fp32; see launch_tile).  With
            // c(z) - cap = -2 cap / (1 + e^{2z/cap}): e^{2z/cap} overflowing
            // gives exp(0) = 1 and underflowing e^{-2 cap}, the two limits.
            float ssum = 0.0f;
#pragma unroll
            for (int k = 0; k < EW; ++k) {
              const float tp = __builtin_amdgcn_exp2f(z[k] * c3);
              const float e = __builtin_amdgcn_exp2f(c2 * __builtin_amdgcn_rcpf(1.0f + tp));
              ssum += (k < nv) ? e : 0.0f;
              if (EXTRA) xm = fmaxf(xm, (k < nv) ? z[k] : -INFINITY);
            }
            run_s += ssum;
          } else if (MODE == MODE_FWD) {
            float tmax = -INFINITY;
#pragma unroll
            for (int k = 0; k < EW; ++k) {
              z[k] = (k < nv) ? z[k] : -INFINITY;
              tmax = fmaxf(tmax, z[k]);
            }
            if (EXTRA) xm = fmaxf(xm, tmax);  // raw logits: the softcap is applied to the maximum later
            if (a.cap > 0.0f) {
              // a softcap too large for the fixed reference of MODE_FWD_CAP:
              // c(z) = cap (1 - 2 / (1 + e^{2z/cap})) under a running maximum
              tmax = -INFINITY;
#pragma unroll
              for (int k = 0; k < EW; ++k) {
                const float r = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z[k] * c3));
                z[k] = (k < nv) ? a.cap * fmaf(-2.0f, r, 1.0f) : -INFINITY;
                tmax = fmaxf(tmax, z[k]);
              }
            }
            const float mnew = fmaxf(run_m, tmax);
            if (mnew != -INFINITY) {
              const float mb = mnew * LOG2E;
              float ssum = 0.0f;
#pragma unroll
              for (int k = 0; k < EW; ++k) ssum += __builtin_amdgcn_exp2f(fmaf(z[k], LOG2E, -mb));
              run_s = run_s * __builtin_amdgcn_exp2f((run_m - mnew) * LOG2E) + ssum;
              run_m = mnew;
            }
          } else {
            // Coefficients -g p c' (backward) or -e c' (fused: e = e^{c(z) -
            // cap}, the token's factor g e^{cap - lse} applied by the reduce),
            // and pv = p or e summed over the non-target columns: the mass
            // 1 - p_t of the target's term is that sum (backward), or S / (S +
            // e_t) (fused), formed from the same terms as the coefficients.
            // The target column is left out here; its whole term is added in
            // fp32 by k_dh_reduce.
            float cv[EW], pv[EW];
            if (FNC) {
              // e = e^{z - R} <= 1 against the block's reference
#pragma unroll
              for (int k = 0; k < EW; ++k) {
                pv[k] = __builtin_amdgcn_exp2f(fmaf(z[k], LOG2E, -Rb2));
                cv[k] = -pv[k];
              }
            } else if (FUSED) {
              // c' = 4 r (1 - r); the term is taken as 4 e = exp2(c2 r + 2), so
              // the coefficient -e c' is -(4 e)(r - r^2) and the split sums
              // carry 4 S (the reduce takes the factor 4 back out, exactly)
#pragma unroll
              for (int k = 0; k < EW; ++k) {
                const float r = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z[k]));
                pv[k] = __builtin_amdgcn_exp2f(fmaf(c2, r, 2.0f));
                cv[k] = -pv[k] * fmaf(-r, r, r);
              }
            } else if (a.cap > 0.0f) {
              // with r = 1/(1 + e^{2z/cap}): tanh(z/cap) = 1 - 2r and
              // c'(z) = 1 - tanh^2 = 4 r (1 - r).  e^{2z/cap} overflowing gives
              // r = 0 (tanh = 1, c' = 0); for z far below zero r rounds to 1
              // and c' to 0 where it is below ~1e-7, its absolute error.
#pragma unroll
              for (int k = 0; k < EW; ++k) {
                const float r = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z[k] * c3));
                pv[k] = __builtin_amdgcn_exp2f(fmaf(m2capl2, r, kofs));
                cv[k] = pv[k] * fmaf(-r, r, r) * kfac;
              }
            } else {
#pragma unroll
              for (int k = 0; k < EW; ++k) {
                pv[k] = __builtin_amdgcn_exp2f(fmaf(z[k], LOG2E, -kofs));
                cv[k] = pv[k] * kfac;
              }
            }
            // a ragged chunk, or a lane whose target falls in it: the whole
            // wave takes the masking pass (the common case skips it)
            if (EXTRA || nv < EW || __builtin_amdgcn_ballot_w64(tk >= 0) != 0) {
              capture();
#pragma unroll
              for (int k = 0; k < EW; ++k) {
                cv[k] = (k < nv && k != tk) ? cv[k] : 0.0f;
                pv[k] = (k < nv && k != tk) ? pv[k] : 0.0f;
              }
            }
            if (!EXTRA) {
              float ps = 0.0f;
#pragma unroll
              for (int k = 0; k < EW; ++k) ps += pv[k];
              if (FNC) esum += ps;  // folded into the running partial after the block
              else sRun[wave][lane] += ps;  // the wave's own slot: in order, no barrier
            }
            uint32_t pk[EW / 2];
#pragma unroll
            for (int k = 0; k < EW; k += 2) {
              if (EXTRA) xm = fmaxf(xm, fmaxf(fabsf(cv[k]), fabsf(cv[k + 1])));
              pk[k / 2] = pack_rne(cv[k], cv[k + 1]);
            }
            // fragment-major chunk: these EW vocab rows are K chunk(s) cm (cm + 1)
            const int64_t vloc = (int64_t)tile * BNT + vcol0 + c * 32 + k0;
            const int cm = (int)(vloc >> 3);
            if (NRB == 2 || lane < 32)
#pragma unroll
              for (int q = 0; q < EW / 8; ++q)
                *(u32x4_t *)(a.coeff + frag_slot(tok0 + lane, cm + q, a.ksv)) =
                    u32x4_t{pk[4 * q], pk[4 * q + 1], pk[4 * q + 2], pk[4 * q + 3]};
            if constexpr (DENSE && FUSED) {
              // dW's operand, [vocabulary row][token] 16-byte slots of 8
              // tokens, transposed through this wave's z scratch: columns k0
              // .. k0 + 7 of every lane's row are read (in registers) and free.
              // Lane 8j + i puts its value of row k into the first 16 bytes of
              // lane 8j + k's, at element i; lane 8j + k then holds row vloc +
              // k of tokens tok0 + 8j .. + 7, one whole slot.
              if (a.coeffT) {
                uint16_t *zb = reinterpret_cast<uint16_t *>(zs + k0);
                const int j8 = lane & ~7, i = lane & 7;
#pragma unroll
                for (int k = 0; k < EW; ++k)
                  zb[(j8 + k) * (2 * ZROW) + i] = (uint16_t)((k & 1) ? pk[k / 2] >> 16 : pk[k / 2] & 0xFFFFu);
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                const u32x4_t x = *(const u32x4_t *)(zb + lane * (2 * ZROW));
                *(u32x4_t *)(a.coeffT + frag_slot(vloc + i, (tok0 + j8) >> 3, a.ks16t)) = x;
              }
            }
          }
        }
        if (FNC && bvalid) {
          // the running (max, sum) of the token's non-target terms over this
          // split, the block's terms brought from its reference to the maximum
          const float mn = fmaxf(run_m, Rb);
          const float mn2 = mn * LOG2E;
          sRun[wave][lane] = sRun[wave][lane] * __builtin_amdgcn_exp2f(fmaf(run_m, LOG2E, -mn2)) +
                             esum * __builtin_amdgcn_exp2f(Rb2 - mn2);
          run_m = mn;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
      if (EXTRA) {
        if (BWD) {
#pragma unroll
          for (int o = 32; o >= 1; o >>= 1) xm = fmaxf(xm, __shfl_xor(xm, o, 64));
          if (lane == 0) sX[0][wave] = xm;
        } else {
          sX[vh][tg * 64 + lane] = xm;
        }
      }
    };

    // EXTRA, after the barrier that follows the epilogue of `tile`: combine
    // the waves' maxima of the tile (the next epilogue that rewrites sX is at
    // least one more barrier away).
    auto tile_extra = [&](int tile) {
      if (!BWD) {
        const int r = tok0 + lane;
        if (vh == 0 && r < a.cnt[0]) {
          const float m = fmaxf(sX[0][tg * 64 + lane], sX[1][tg * 64 + lane]);
          float dc;
          const float y = (a.cap > 0.0f) ? cap_d(m, c1, a.cap, dc) : m;
          a.bmx[(int64_t)a.idx[r] * a.nbv + a.range_tile0 + tile] = y;
        }
      } else if (a.filter_eps > 0.0f && tid == 0) {
        float m = 0.0f;
#pragma unroll
        for (int w = 0; w < 8; ++w) m = fmaxf(m, sX[0][w]);
        if (m < a.filter_eps) a.fl[(int64_t)tt * a.fl_ld + a.range_tile0 + tile] = 0;
      }
    };

    // One step: MFMAs on buffer idx & 1, then the tile's epilogue after its
    // last step.
    auto do_step = [&](int idx, int tile, int st, ProdRegs &cur, ProdRegs &nxt, u32x4_t &hcur, u32x4_t &hnxt) {
      int64_t vn, vnn;
      int sn, snn;
      coords(tile, st, 1, vn, sn);     // next step: unpacked now
      coords(tile, st, LA, vnn, snn);  // loaded now
      if (!SMALL && st == 0) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[rb][c][e] = 0.0f;
      }
      mfma_step(idx & 1, st == 0, sn, vnn, snn, cur, nxt, hcur, hnxt);
      if (st == steps - 1) epilogue(tile);
      __syncthreads();
      if (EXTRA && st == steps - 1) tile_extra(tile);
    };

    int st = 0, tile = first_tile;
    auto advance = [&]() {
      if (++st == steps) { st = 0; tile = next_tile(tile); }
    };
    int idx = 0;
    if constexpr (SMALL) {
      // step i unpacks set (i + 1) % 3 and loads step i + 3 into set i % 3
      for (; idx + 2 < total; idx += 3) {
        do_step(idx, tile, st, P1, P0, H1, H0);
        advance();
        do_step(idx + 1, tile, st, P2, P1, H2, H1);
        advance();
        do_step(idx + 2, tile, st, P0, P2, H0, H2);
        advance();
      }
      if (idx < total) do_step(idx, tile, st, P1, P0, H1, H0);
      if (idx + 1 < total) {
        advance();
        do_step(idx + 1, tile, st, P2, P1, H2, H1);
      }
    } else {
      for (; idx + 1 < total; idx += 2) {
        do_step(idx, tile, st, P1, P0, H0, H0);
        advance();
        do_step(idx + 1, tile, st, P0, P1, H0, H0);
        advance();
      }
      if (idx < total) do_step(idx, tile, st, P1, P0, H0, H0);
    }
  }

  // partials: (max, sum-exp) of the forward passes, [slot][M_pad] pairs; the
  // backward's non-target probability mass, or the single pass's sum of 4 e
  // over the non-target columns (its reference is cap), [M_pad][mass_ld]
  // (token-major: the split reduce sums each token's run)
  if (!BWD || (!EXTRA && a.tmass)) {
    if (COEF) run_s = sRun[wave][lane];
    const float m_out = BWD ? 0.0f : (((MODE == MODE_FWD_CAP || FUSED) && total > 0) ? a.cap : run_m);
    auto put = [&](int half, float m, float sum) {
      const int slot = 2 * (vs.slot0 + wr) + half;
      if (COEF && !FNC) {
        a.mass[(size_t)(tok0 + lane) * a.mass_ld + slot] = sum;
      } else {
        float *dst = a.part + ((size_t)slot * a.M_pad + tok0 + lane) * 2;
        dst[0] = m;
        dst[1] = sum;
      }
    };
    if (SMALL) {
      // the four waves of each vocabulary half combine their partials
      float *sp = &sZ[0][0];  // 8 x 64 x (max, sum); the epilogues are done
      __syncthreads();
      sp[(wave * 64 + lane) * 2] = m_out;
      sp[(wave * 64 + lane) * 2 + 1] = run_s;
      __syncthreads();
      if (wave < 2) {
        float m = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) m = fmaxf(m, sp[((4 * wave + w) * 64 + lane) * 2]);
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float mw = sp[((4 * wave + w) * 64 + lane) * 2], sw = sp[((4 * wave + w) * 64 + lane) * 2 + 1];
          sum += (mw == -INFINITY) ? 0.0f : sw * __builtin_amdgcn_exp2f((mw - m) * LOG2E);
        }
        put(wave, m, sum);
      }
    } else {
      put(vh, m_out, run_s);
    }
  }
}

// The forward's fixed reference e^{c(z) - cap} keeps every term <= 1, but the
// largest term of a token can be as small as e^{-2 cap}: it stays a normal
// fp32 for cap <= CAP_FIXED_REF_MAX (40).  Larger softcaps take the
// running-maximum forward (and no fused pass).

void launch_tile(hipStream_t st, int bits, int pass, dim3 grid, const TileArgs &a) {
  const bool bwd = pass == PASS_BWD;
  const int mode = pass == PASS_FUSED ? MODE_FUSED
                   : pass == PASS_FUSED_NC
                       ? MODE_FUSED_NC
                       : (bwd ? MODE_BWD : ((a.cap > 0.0f && a.cap <= CAP_FIXED_REF_MAX) ? MODE_FWD_CAP : MODE_FWD));
  const bool extra = (pass == PASS_FUSED || pass == PASS_FUSED_NC) ? false : (bwd ? a.fl != nullptr : a.bmx != nullptr);
  const bool gs32 = a.kw == 32;
  // group 32 has no small-M instantiation (the plain one is correct there)
  const int var = extra ? VAR_EXTRA : (a.small && !gs32 ? (a.small == 2 ? VAR_SMALL32 : VAR_SMALL) : VAR_PLAIN);
#define CCE_TILE(B, MD)                                                                                          \
  do {                                                                                                           \
    if (gs32) {                                                                                                  \
      if (var == VAR_EXTRA) hipLaunchKernelGGL((k_tile<B, MD, VAR_EXTRA, true>), grid, dim3(TW), 0, st, a);      \
      else hipLaunchKernelGGL((k_tile<B, MD, VAR_PLAIN, true>), grid, dim3(TW), 0, st, a);                       \
    } else {                                                                                                     \
      if (var == VAR_EXTRA) hipLaunchKernelGGL((k_tile<B, MD, VAR_EXTRA, false>), grid, dim3(TW), 0, st, a);     \
      else if (var == VAR_SMALL) hipLaunchKernelGGL((k_tile<B, MD, VAR_SMALL, false>), grid, dim3(TW), 0, st, a); \
      else if (var == VAR_SMALL32)                                                                               \
        hipLaunchKernelGGL((k_tile<B, MD, VAR_SMALL32, false>), grid, dim3(TW), 0, st, a);                       \
      else hipLaunchKernelGGL((k_tile<B, MD, VAR_PLAIN, false>), grid, dim3(TW), 0, st, a);                      \
    }                                                                                                            \
  } while (0)
  // the fused pass: no EXTRA variant (no skips, no block maxima)
#define CCE_TILE_FUSED(B, MD)                                                                                    \
  do {                                                                                                           \
    if (gs32) hipLaunchKernelGGL((k_tile<B, MD, VAR_PLAIN, true>), grid, dim3(TW), 0, st, a);                    \
    else if (var == VAR_SMALL) hipLaunchKernelGGL((k_tile<B, MD, VAR_SMALL, false>), grid, dim3(TW), 0, st, a);  \
    else if (var == VAR_SMALL32)                                                                                 \
      hipLaunchKernelGGL((k_tile<B, MD, VAR_SMALL32, false>), grid, dim3(TW), 0, st, a);                         \
    else hipLaunchKernelGGL((k_tile<B, MD, VAR_PLAIN, false>), grid, dim3(TW), 0, st, a);                        \
  } while (0)
  if (bits == 16) {  // dense bf16 head: 32-wide steps, plain variant only
    if (mode == MODE_FUSED) hipLaunchKernelGGL((k_tile<16, MODE_FUSED, VAR_PLAIN, true>), grid, dim3(TW), 0, st, a);
    else if (mode == MODE_FUSED_NC)
      hipLaunchKernelGGL((k_tile<16, MODE_FUSED_NC, VAR_PLAIN, true>), grid, dim3(TW), 0, st, a);
    else if (mode == MODE_BWD) hipLaunchKernelGGL((k_tile<16, MODE_BWD, VAR_PLAIN, true>), grid, dim3(TW), 0, st, a);
    else if (mode == MODE_FWD_CAP)
      hipLaunchKernelGGL((k_tile<16, MODE_FWD_CAP, VAR_PLAIN, true>), grid, dim3(TW), 0, st, a);
    else hipLaunchKernelGGL((k_tile<16, MODE_FWD, VAR_PLAIN, true>), grid, dim3(TW), 0, st, a);
  } else if (bits == 4) {
    if (mode == MODE_FUSED) CCE_TILE_FUSED(4, MODE_FUSED);
    else if (mode == MODE_FUSED_NC) CCE_TILE_FUSED(4, MODE_FUSED_NC);
    else if (mode == MODE_BWD) CCE_TILE(4, MODE_BWD);
    else if (mode == MODE_FWD_CAP) CCE_TILE(4, MODE_FWD_CAP);
    else CCE_TILE(4, MODE_FWD);
  } else {
    if (mode == MODE_FUSED) CCE_TILE_FUSED(8, MODE_FUSED);
    else if (mode == MODE_FUSED_NC) CCE_TILE_FUSED(8, MODE_FUSED_NC);
    else if (mode == MODE_BWD) CCE_TILE(8, MODE_BWD);
    else if (mode == MODE_FWD_CAP) CCE_TILE(8, MODE_FWD_CAP);
    else CCE_TILE(8, MODE_FWD);
  }
#undef CCE_TILE
#undef CCE_TILE_FUSED
}

}  // namespace cce
