// dh.hip -- the dh contraction of libcce's backward (the second phase of the
// page's backward: the coefficients contracted with the head, summed over
// vocabulary blocks).
#include <type_traits>

#include "cce_device.h"

namespace cce {

// dh_part[k][r][d] (+)= sum_v coeff[r][v] * bf16(s*q + b)[v][d] over the
// vocabulary rows of split k of one coefficient chunk (slabs of the active
// rows r < 256 * ceil(cnt / 256), split count from dh_split).
//
// Workgroup: 256 tokens x 256 dh columns, 8 waves; wave w owns tokens
// [64(w/2), +64) and columns [128(w%2), +128) as 2 x 4 blocks of
// v_mfma_f32_32x32x16_bf16 (rows = tokens, columns = d, K = vocabulary rows).
// Per K step of 64 vocabulary rows:
//  * the head tile of the step is dequantized once (s*q + b, rounded to bf16)
//    into LDS as [d][v] (swizzled, see dswz), double buffered, and shared by
//    the eight waves;
//  * the coefficient operand comes straight from the fragment-major chunk
//    into registers, one step ahead;
//  * the producer (every thread: 8 vocabulary rows x 4 columns) loads the
//    head words two steps ahead into alternating register sets and
//    dequantizes the next step in four slices placed between the MFMAs.
// Reads are raw buffer loads (rows past V read as zeros), so the step has no
// per-lane predicate.  Each split owns its fp32 slab: no atomics, and a
// repeated call gives identical bits.
// SMALL (1: at most 64 tokens, one token group): every wave multiplies the 64
// tokens by its own 32 of the workgroup's 256 dh columns; SMALL = 2 (at most
// 32 tokens) keeps one 32-row token block (half the MFMAs, coefficient
// fragments and slab rows).
// SKIP (second instantiation): the split contracts only the vocabulary tiles
// of its range whose pair flag is set for its token tile; their K steps are
// listed in LDS first, in order.

constexpr int DTW = 256;       // dh columns per workgroup
constexpr int KSTP = 64;       // vocabulary rows per K step

// The LDS head tile is [256 d][64 v] bf16 without padding; the 16-byte chunk c
// (8 vocabulary rows) of row d sits at chunk position c ^ ((d ^ (d >> 2)) & 7).
// The B-operand reads (consecutive d, one chunk) and the producer writes (d
// four apart, one chunk) then spread over distinct 16-byte bank groups; the
// padded alternative puts every fourth producer row on the same banks
// (measured: 17x more LDS bank-conflict cycles).
__device__ __forceinline__ int dswz(int d, int chunk) { return d * KSTP + ((chunk ^ ((d ^ (d >> 2)) & 7)) << 3); }

// Producer mapping: thread (rgp, dc) handles vocabulary rows 8*rgp .. 8*rgp+7
// of the step and columns 4*dc .. 4*dc+3 of the tile; lanes are 16 dc x 4 rgp,
// so one load instruction covers 4 rows and the 16-byte LDS writes of 16
// lanes fall in distinct banks.  The scales and biases of the step's 64 rows
// x 2^LG groups (LG = log2(256 / group)) are loaded once per workgroup (value
// e = tid + 512 k: scales then biases, rows, then groups fastest, so the
// loads are contiguous) into LDS and read back by the dequantizing threads.
// SBW is the stored width of a scale or bias (4: fp32, 2: bf16 or fp16).
constexpr int SB_SLOT = 2 * 8 * KSTP;  // floats of one staged step: 2 x (up to 8 groups) x 64 rows

template <int BITS>
struct DhRegs {
  uint32_t w[BITS == 16 ? 16 : 8];  // 8-bit: 4 codes of row e; 4-bit: 4 codes in the low 16 bits;
                                    // dense: 4 bf16 of row e in words 2e, 2e + 1
  uint32_t sb[2]; // raw bits of the scales or biases this thread stages (widened when staged,
                  // so the load is not waited for before the step's end)
};

// Dense bf16 head (the trainable-head variant): the same thread mapping, the
// 8 rows x 4 columns of a thread are copied (no scales), transposed in
// registers into one 16-byte run of v per column.
struct DhDense {
  int rgp, dc, wcol, tid, gq0;

  __device__ __forceinline__ void load(const GemmArgs &a, int64_t vs, DhRegs<16> &p) const {
    const int64_t rows = a.V - vs < KSTP ? a.V - vs : KSTP;
    const rsrc_t rw = make_rsrc(a.wq + vs * a.wpr, rows * a.wpr * 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b64(rw, (8 * rgp + e) * a.wpr * 4 + wcol, 0, 0);
      p.w[2 * e] = x[0];
      p.w[2 * e + 1] = x[1];
    }
  }
  __device__ __forceinline__ void stage_sb(const DhRegs<16> &, float *, int) const {}
  __device__ __forceinline__ void read_sb(const float *, float (&)[8], float (&)[8]) const {}

  // Column 4*dc + k: the bf16 of rows 8*rgp .. +7, paired into words.
  __device__ __forceinline__ void store(int k, const DhRegs<16> &p, const float (&)[8], const float (&)[8],
                                        uint16_t *sb) const {
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = p.w[2 * (2 * j) + (k >> 1)], hi = p.w[2 * (2 * j + 1) + (k >> 1)];
      o[j] = (k & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
    }
    *(u32x4_t *)(sb + dswz(4 * dc + k, rgp)) = u32x4_t{o[0], o[1], o[2], o[3]};
  }
};

template <int BITS, int LG, int SBW>
struct DhProducer;
template <int BITS, int LG, int SBW>
using DhProd = typename std::conditional<BITS == 16, DhDense, DhProducer<BITS, LG, SBW>>::type;

template <int BITS, int LG, int SBW>
struct DhProducer {
  static constexpr int NVAL = (2 * KSTP) << LG;      // staged values per step
  static constexpr int NK = (NVAL + 511) / 512;      // per thread (1 or 2; half the threads for LG = 1)
  static constexpr int GSH = 6 - LG;                 // column block dc lies in group dc >> GSH
  int rgp, dc;    // rows 8*rgp + e, columns 4*dc + k of the tile
  int wcol;       // byte offset of those columns within a packed row
  int tid;
  int gq0;        // first quantization group of the tile

  // staged value e: (is a bias, row, group within the tile)
  __device__ __forceinline__ void sb_slot(int e, int &isb, int &row, int &g) const {
    // a run of 64 << LG >= 128 consecutive values shares isb, so it is
    // uniform in a wave: keep it scalar (it selects the buffer base)
    isb = __builtin_amdgcn_readfirstlane(e >> (6 + LG));
    row = (e >> LG) & (KSTP - 1);
    g = e & ((1 << LG) - 1);
  }

  __device__ __forceinline__ void load(const GemmArgs &a, int64_t vs, DhRegs<BITS> &p) const {
    const int64_t rows = a.V - vs < KSTP ? a.V - vs : KSTP;
    const rsrc_t rw = make_rsrc(a.wq + vs * a.wpr, rows * a.wpr * 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int voff = (8 * rgp + e) * a.wpr * 4 + wcol;
      if (BITS == 8) p.w[e] = __builtin_amdgcn_raw_buffer_load_b32(rw, voff, 0, 0);
      else p.w[e] = __builtin_amdgcn_raw_buffer_load_b16(rw, voff, 0, 0);
    }
    const int64_t nb = rows * a.Gq * SBW;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int e = tid + 512 * k;
      int isb, row, g;
      sb_slot(e, isb, row, g);
      const rsrc_t rs = make_rsrc(static_cast<const char *>(isb ? a.biases : a.scales) + vs * a.Gq * SBW, nb);
      const int off = (row * a.Gq + gq0 + g) * SBW;
      if (NVAL >= 512 || e < NVAL) {
        if (SBW == 4) p.sb[k] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
        else p.sb[k] = __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0);
      }
    }
  }

  // LDS stage of the step's scales and biases: [group j][row][scale, bias].
  __device__ __forceinline__ void stage_sb(const DhRegs<BITS> &p, float *ssb, int sbt) const {
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int e = tid + 512 * k;
      int isb, row, g;
      sb_slot(e, isb, row, g);
      if (NVAL >= 512 || e < NVAL)
        ssb[(g * KSTP + row) * 2 + isb] = SBW == 4 ? __uint_as_float(p.sb[k]) : sb_widen(p.sb[k], sbt);
    }
  }

  // (scale, bias) of the thread's 8 rows (group j = 4 dc / group).
  __device__ __forceinline__ void read_sb(const float *ssb, float (&s)[8], float (&b)[8]) const {
    const float *src = ssb + ((dc >> GSH) * KSTP + 8 * rgp) * 2;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float2 x = *(const float2 *)(src + 2 * e);
      s[e] = x.x;
      b[e] = x.y;
    }
  }

  // Column 4*dc + k: its 8 rows dequantized and stored as one 16-byte run of v.
  __device__ __forceinline__ void store(int k, const DhRegs<BITS> &p, const float (&s)[8], const float (&b)[8],
                                        uint16_t *sb) const {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t q = (BITS == 8) ? (p.w[e] >> (8 * k)) & 0xFFu : (p.w[e] >> (4 * k)) & 0xFu;
      x[e] = fmaf(s[e], (float)q, b[e]);
    }
    *(u32x4_t *)(sb + dswz(4 * dc + k, rgp)) =
        u32x4_t{pack_rne(x[0], x[1]), pack_rne(x[2], x[3]), pack_rne(x[4], x[5]), pack_rne(x[6], x[7])};
  }
};

constexpr int MAX_LIST = 2048;  // vocabulary tiles per split (a chunk holds at most 2048)

// A staged coefficient fragment (small M) and the inputs of its factor.
struct CFrag {
  u32x4_t x;
  float R, m;
};

template <int BITS, bool SKIP, int SMALL, int LG, int SBW>
__global__ void __launch_bounds__(TW, 1) k_dh(GemmArgs a) {
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  // the launched work ids are spread over the active token tiles only;
  // consecutive work ids share the token tile (and the coefficient rows)
  const int act = active_tiles(a.cnt);
  int ksd, steps_per;
  dh_split(a, act, ksd, steps_per);
  if (bid >= a.HT * act * ksd) return;
  const int dt = bid % a.HT;
  const int tt = (bid / a.HT) % act;
  const int ks_ = bid / (a.HT * act);
  const int d0 = dt * DTW;
  const int step0 = ks_ * steps_per;
  int nsteps = min(steps_per, a.chunk_steps - step0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the two waves of a token group sit on two SIMDs; small M: one token group,
  // 32 columns per wave
  const int tg = SMALL ? 0 : wave >> 1, dh = wave & 1;
  constexpr int NRB = SMALL == 2 ? 1 : 2;  // 32-row token blocks per wave
  // small M: wave w stages coefficient fragment (row block w / 4, k-step w % 4)
  // of each step; with one row block only waves 0..3 have one
  const bool cload = NRB == 2 || wave < 4;
  constexpr int NC = SMALL ? 1 : 4;                 // 32-column blocks per wave
  const int col0 = SMALL ? wave * 32 : dh * 128;   // this wave's first column within the tile
  const int l32 = lane & 31, lh = lane >> 5;

  __shared__ __attribute__((aligned(16))) uint16_t sB[2][DTW * KSTP];
  __shared__ __attribute__((aligned(16))) float sSB[2][SB_SLOT];
  __shared__ uint16_t sList[SKIP ? MAX_LIST : 1];
  __shared__ int sCount[SKIP ? 9 : 1];
  // small M: the eight waves multiply the same coefficient rows, so the
  // step's coefficient operand (2 row blocks x 4 k-steps = 8 fragments of 1
  // KiB) is loaded once per workgroup, one fragment per wave, and shared
  // through LDS (double buffered like the head tile) instead of eight times
  // from L1.
  __shared__ __attribute__((aligned(16))) u32x4_t sCA[SMALL ? 2 : 1][SMALL ? 8 * 64 : 1];

  if (SKIP) {
    // flagged tiles of [step0 / 4, (step0 + nsteps) / 4), compacted in order:
    // thread i owns tiles 4i .. 4i+3 of the range, counts them, and a
    // workgroup scan (waves, then across the 8 wave totals) places them
    const int t0 = step0 >> 2, nt = nsteps > 0 ? nsteps >> 2 : 0;
    const uint8_t *frow = a.fl + (int64_t)tt * a.fl_ld + a.chunk_tile0 + t0;
    int mine = 0;
    for (int j = 0; j < 4; ++j) {
      const int t = 4 * tid + j;
      mine += (t < nt && frow[t] != 0) ? 1 : 0;
    }
    int incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane == 63) sCount[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += sCount[w];
    if (tid == 0) {
      int tot = 0;
      for (int w = 0; w < 8; ++w) tot += sCount[w];
      sCount[8] = tot;
    }
    int pos = base + incl - mine;
    for (int j = 0; j < 4; ++j) {
      const int t = 4 * tid + j;
      if (t < nt && frow[t] != 0) sList[pos++] = (uint16_t)(t0 + t);
    }
    __syncthreads();
    nsteps = 4 * sCount[8];
  }

  const int tok0 = tt * BM + tg * 64;
  // fragment-major coefficients of the workgroup's 256 tokens: one 1 KiB block
  // per (32 tokens, 16 vocabulary rows)
  const rsrc_t rc = make_rsrc(a.coeff + (size_t)(tt * BM >> 5) * a.ksv * 512, (int64_t)8 * a.ksv * 1024);
  const int cv0 = ((tg * 2) * (int)a.ksv * 64 + lane) * 16;
  const int cstride = (int)a.ksv * 1024;

  f32x16_t acc[2][NC];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[rb][c][e] = 0.0f;

  if (nsteps > 0) {
    DhProd<BITS, LG, SBW> pr;
    pr.dc = (lane & 15) + 16 * (wave & 3);
    pr.rgp = (lane >> 4) + 4 * (wave >> 2);
    pr.wcol = (d0 + 4 * pr.dc) * BITS / 8;
    pr.tid = tid;
    pr.gq0 = d0 / a.gs;
    DhRegs<BITS> P0, P1, P2;
    // this lane's B-operand chunk offsets (row col0 + l32 + 32c, chunk 2ks + lh);
    // the swizzle key of row d + 32c equals that of row d
    int boff[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) boff[ks] = dswz(col0 + l32, 2 * ks + lh);
    bf16x8_t cA[2][4];
    float sc[8], bi[8];
    // chunk K step of step i of this split (past the end: the last one)
    auto cstep = [&](int i) {
      if (!SKIP) return step0 + i;
      const int c = i < nsteps ? i : nsteps - 1;
      // the list entry is the same for every lane: keep it scalar (it forms buffer bases)
      return 4 * __builtin_amdgcn_readfirstlane((int)sList[c >> 2]) + (c & 3);
    };
    // vocabulary row of step i of this split
    auto vrow = [&](int i) { return a.chunk_v0 + (int64_t)cstep(i) * KSTP; };
    // K offset (bytes) of step i in the fragment-major chunk
    auto koff = [&](int i) { return cstep(i) * 4 * 1024; };

    // the coefficient fragment this wave stages for step i (small M); with
    // a.ncR also the inputs of its factor e^{R - m} for the lane's token row
    // and the 32-row block of its 8 vocabulary rows (R = m = 0, a factor of
    // exactly 1, outside the supervised rows and V)
    const bool ncs = SMALL && a.ncR != nullptr;
    const int crow = tt * BM + (wave >> 2) * 32 + l32;
    auto cfrag_load = [&](int i) {
      const int ii = i < nsteps ? i : nsteps - 1;
      CFrag f;
      f.x = buf_load16(rc, cv0 + (wave >> 2) * cstride + (wave & 3) * 1024, koff(ii));
      f.R = f.m = 0.0f;
      if (ncs) {
        const int64_t v = a.chunk_v0 + (int64_t)cstep(ii) * KSTP + (wave & 3) * 16 + 8 * lh;
        if (crow < a.cnt[0] && v < a.V) {
          f.R = a.ncR[(size_t)(v >> 5) * a.M_pad + crow];
          f.m = a.nc[3 * crow];
        }
      }
      return f;
    };
    auto cfrag_value = [&](const CFrag &f) {
      if (!ncs) return f.x;
      const float s = __builtin_amdgcn_exp2f((f.R - f.m) * 1.4426950408889634f);
      u32x4_t x = f.x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = pack_rne(bf16_to_f32(x[e] & 0xFFFFu) * s, bf16_to_f32(x[e] >> 16) * s);
      return x;
    };
    CFrag C0, C1, C2;  // small M: staged fragments of three steps, as P0..P2
    pr.load(a, vrow(0), P0);
    pr.load(a, vrow(1), P1);
    if (SMALL) pr.load(a, vrow(2), P2);
    pr.stage_sb(P0, sSB[0], a.sbt);
    pr.stage_sb(P1, sSB[1], a.sbt);
    if (SMALL) {
      if (cload) {
        sCA[0][wave * 64 + lane] = cfrag_value(cfrag_load(0));
        C1 = cfrag_load(1);
        C2 = cfrag_load(2);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        cA[0][ks] = __builtin_bit_cast(bf16x8_t, buf_load16(rc, cv0 + ks * 1024, koff(0)));
        cA[1][ks] = __builtin_bit_cast(bf16x8_t, buf_load16(rc, cv0 + cstride + ks * 1024, koff(0)));
      }
    }
    __syncthreads();
    pr.read_sb(sSB[0], sc, bi);
#pragma unroll
    for (int k = 0; k < 4; ++k) pr.store(k, P0, sc, bi, sB[0]);
    __syncthreads();

    // Step st: MFMAs on buffer st & 1; dequantize step st + 1 (words in `cur`,
    // scales in LDS slot (st + 1) & 1) into the other buffer between them;
    // load step st + LA into `nxt` and stage the scales of step st + 2 (`mid`
    // for small M, else `nxt`) in slot st & 1.  Small M loads its head words
    // three steps ahead (LA = 3, register sets P0..P2 in turn) and its
    // coefficient fragments likewise: a step is short there, and one step of
    // cover left both loads waited for.  The fragment is loaded before the
    // head words (loads complete in issue order for s_waitcnt).
    auto do_step = [&](int st, DhRegs<BITS> &cur, DhRegs<BITS> &mid, DhRegs<BITS> &nxt, CFrag &cfc,
                       CFrag &cfn) {
      const int cb = st & 1;
      const int knext = koff(st + 1 < nsteps ? st + 1 : st);
      if (SMALL && cload) cfn = cfrag_load(st + 3);
      pr.load(a, vrow(st + (SMALL ? 3 : 2)), nxt);  // past the split: valid rows or zeros, never used
      pr.read_sb(sSB[cb ^ 1], sc, bi);
      const uint16_t *sw = sB[cb];
      if (SMALL) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          cA[0][ks] = __builtin_bit_cast(bf16x8_t, sCA[cb][ks * 64 + lane]);
          if (NRB == 2) cA[1][ks] = __builtin_bit_cast(bf16x8_t, sCA[cb][(4 + ks) * 64 + lane]);
        }
      }
      bf16x8_t bq[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) bq[c] = *(const bf16x8_t *)(sw + boff[0] + c * 32 * KSTP);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        {
#pragma unroll
          for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
              acc[rb][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cA[rb][ks], bq[c], acc[rb][c], 0, 0, 0);
            if (ks < 3) bq[c] = *(const bf16x8_t *)(sw + boff[ks + 1] + c * 32 * KSTP);
          }
          if (!SMALL) {
            cA[0][ks] = __builtin_bit_cast(bf16x8_t, buf_load16(rc, cv0 + ks * 1024, knext));
            cA[1][ks] = __builtin_bit_cast(bf16x8_t, buf_load16(rc, cv0 + cstride + ks * 1024, knext));
          }
        }
        pr.store(ks, cur, sc, bi, sB[cb ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
      pr.stage_sb(SMALL ? mid : nxt, sSB[cb], a.sbt);
      if (SMALL && cload) sCA[cb ^ 1][wave * 64 + lane] = cfrag_value(cfc);  // step st + 1's: read after the barrier
      __syncthreads();
    };
    int st = 0;
    if constexpr (SMALL) {
      for (; st + 2 < nsteps; st += 3) {
        do_step(st, P1, P2, P0, C1, C0);
        do_step(st + 1, P2, P0, P1, C2, C1);
        do_step(st + 2, P0, P1, P2, C0, C2);
      }
      if (st < nsteps) do_step(st, P1, P2, P0, C1, C0);
      if (st + 1 < nsteps) do_step(st + 1, P2, P0, P1, C2, C1);
    } else {
      for (; st + 1 < nsteps; st += 2) {
        do_step(st, P1, P0, P0, C0, C0);
        do_step(st + 1, P0, P1, P1, C0, C0);
      }
      if (st < nsteps) do_step(st, P1, P0, P0, C0, C0);
    }
  } else if (a.accumulate) {
    return;
  }

  // result lane layout: column d0 + col0 + c*32 + l32, rows tok0 + rb*32 + 8i + 4*lh + j.
  // Accumulating (later chunks), the 32 old values of a column block are all
  // loaded before any of them is stored: interleaved, every load would wait
  // for the previous store (the compiler cannot prove the rows distinct).
  float *const slab = a.dh_part + ((size_t)ks_ * act * BM + tok0 + 4 * lh) * a.H;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int d = d0 + col0 + c * 32 + l32;
    if (d >= a.H) continue;
    float old[2][16];
    if (a.accumulate) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          old[rb][e] = slab[(size_t)(rb * 32 + 8 * (e >> 2) + (e & 3)) * a.H + d];
    } else {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int e = 0; e < 16; ++e) old[rb][e] = 0.0f;
    }
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        slab[(size_t)(rb * 32 + 8 * (e >> 2) + (e & 3)) * a.H + d] = old[rb][e] + acc[rb][c][e];
  }
}

template <int B, int LG, int SBW>
static void launch_dh_variant(hipStream_t st, dim3 grid, const GemmArgs &a, bool skip, int small) {
  if (skip) {
    hipLaunchKernelGGL((k_dh<B, true, 0, LG, SBW>), grid, dim3(TW), 0, st, a);
    return;
  }
  if constexpr (LG == 2 && SBW == 4) {
    if (small == 2) {
      hipLaunchKernelGGL((k_dh<B, false, 2, LG, SBW>), grid, dim3(TW), 0, st, a);
      return;
    }
    if (small == 1) {
      hipLaunchKernelGGL((k_dh<B, false, 1, LG, SBW>), grid, dim3(TW), 0, st, a);
      return;
    }
  }
  hipLaunchKernelGGL((k_dh<B, false, 0, LG, SBW>), grid, dim3(TW), 0, st, a);
}

template <int B>
static void launch_dh_bits(hipStream_t st, dim3 grid, const GemmArgs &a) {
  const bool skip = a.fl != nullptr;
  const bool wide = a.sbt == SB_F32;
  // the small-M instantiation exists for the default storage only (group 64, fp32)
  const int small = (!skip && a.gs == KSTEP && wide) ? a.small : 0;
  if (a.gs == 64) {
    if (wide) launch_dh_variant<B, 2, 4>(st, grid, a, skip, small);
    else launch_dh_variant<B, 2, 2>(st, grid, a, skip, 0);
  } else if (a.gs == 32) {
    if (wide) launch_dh_variant<B, 3, 4>(st, grid, a, skip, 0);
    else launch_dh_variant<B, 3, 2>(st, grid, a, skip, 0);
  } else {
    if (wide) launch_dh_variant<B, 1, 4>(st, grid, a, skip, 0);
    else launch_dh_variant<B, 1, 2>(st, grid, a, skip, 0);
  }
}

void launch_dh_gemm(hipStream_t st, int bits, dim3 grid, const GemmArgs &a) {
  if (bits == 16) {  // dense bf16 head: exact path only (no skips, no small-M variant)
    hipLaunchKernelGGL((k_dh<16, false, 0, 0, 0>), grid, dim3(TW), 0, st, a);
    return;
  }
  if (bits == 4) launch_dh_bits<4>(st, grid, a);
  else launch_dh_bits<8>(st, grid, a);
}

}  // namespace cce
