// cce.hip -- host side of libcce: argument validation, launch planning,
// workspace carving and the launch sequence on the caller's stream.
// The C ABI is declared in include/cce.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include <mutex>
#include <vector>

#include "cce.h"
#include "cce_device.h"
#include "cce_profile.h"

// The workspace of cce_forward_static: one array per device, which the
// loader allocates with the code object.  Host code never passes its name to
// a kernel (on the host it names a stand-in, not device memory): the device
// address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[CCE_STATIC_SCRATCH_BYTES];

namespace {

using namespace cce;

constexpr int64_t MAX_H = 16384;
constexpr int64_t MAX_M = (int64_t)1 << 24;
constexpr size_t COEFF_BUDGET = (size_t)1 << 30;  // bytes of one coefficient chunk
constexpr int64_t MAX_CHUNK_TILES = 2048;          // vocabulary tiles of one coefficient chunk
constexpr int64_t FUSED_COMPACT_MAX_M = 2048;      // tokens compacted inside the front launch

thread_local char g_err[256];

// ---- opt-in launch timing (cce_profile.h) ----------------------------------
struct ProfRec {
  const char *name;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
std::vector<ProfRec> g_prof;
int g_prof_on = 0;

struct ProfScope {
  ProfRec r{nullptr, nullptr, nullptr};
  hipStream_t st;
  ProfScope(const char *name, hipStream_t s) : st(s) {
    if (!g_prof_on) return;
    r.name = name;
    if (hipEventCreate(&r.a) != hipSuccess || hipEventCreate(&r.b) != hipSuccess) {
      r.name = nullptr;
      return;
    }
    (void)hipEventRecord(r.a, st);
  }
  ~ProfScope() {
    if (!r.name) return;
    (void)hipEventRecord(r.b, st);
    std::lock_guard<std::mutex> g(g_prof_mu);
    g_prof.push_back(r);
  }
};

#define CCE_LAUNCH(NAME, STREAM, CALL)    \
  do {                                    \
    ProfScope prof_scope_(NAME, STREAM);  \
    CALL;                                 \
  } while (0)

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Compute units of the current device (cached per device; 256 on MI355X).
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Plan {
  int64_t M, M_pad, V, H;
  int G, Kb, Ka, NB, bits, wpr, TT, tiles;  // NB, G: tile K steps (kw columns) of the bias block and of h
  int P, NBr;                               // columns of each half of the bias block; steps of its first half
  int kw;                                   // 64, or 32 for quantization group 32 (one group per step)
  int gs, Gq, sbt;                           // quantization group, groups per row, scale/bias dtype
  float cap;
  // forward
  int nsplit, tiles_per_split, fwd_blocks, max_splits;
  // backward
  int chunk_tiles, nchunks, ksplit, k_tiles, HT, bwd_tpw;  // k_tiles: vocabulary tiles per dh split
  int64_t ld_coeff;
  // workspace offsets (bytes)
  size_t o_cnt, o_idx, o_inv, o_tok, o_haug, o_sabs, o_part, o_coeff, o_dhp, o_fl, fwd_bytes, bwd_bytes;
  // the head side (bias-block digits, fold ratios, last scales, digit block
  // maxima): offsets within its region, which is the caller's prepared buffer
  // (head->prep) or lies in the workspace at o_hs
  bool prep;
  size_t o_hs, h_baug, h_rt, h_slast, h_bmx, hs_bytes;
  size_t o_hT, o_coeffT;  // dense heads: transposed h and coefficient chunk of the dW contraction
  // fused pass (softcap in (0, CAP_FIXED_REF_MAX], quantized head): launched
  // work ids per chunk, split capacity per chunk, partials and target c'
  bool fused;
  int fus_blocks, fus_max_splits, mass_ld;
  size_t o_fpart, o_tdc, fus_bytes;
  // cce_forward_backward without the single pass: the forward's partials
  // after the backward's buffers (the backward tile merges them itself)
  size_t o_ppart, twopass_bytes;
  // the dense head's single pass (cce_dense_forward_backward, softcap in (0,
  // CAP_FIXED_REF_MAX]): every coefficient chunk kept until dW, whose
  // launches follow the reduce; dh slabs, split sums, target c', per-row
  // factors, scaled hT and one transposed chunk
  bool dfused;
  size_t df_coeff, df_dhp, df_tdc, df_fpart, df_fac, df_hT, df_coeffT, df_bytes;
  size_t df_part, df_R, df_nc;  // without a softcap: as the quantized head's uncapped single pass
  // the uncapped single pass of a quantized head (cce_forward_backward, no
  // softcap): every coefficient chunk kept until the merge has each token's
  // largest logit; dh slabs, the (max, sum) partials, the 32-row block
  // references and the merge's per-row (m, S, e_t)
  bool ncfused;
  size_t nc_coeff, nc_dhp, nc_part, nc_R, nc_nc, nc_bytes;
};

// A dense bf16 head runs as an internal head of 16 "bits" per element: the
// 32-wide step path of the tile, no bias block, no scales.
constexpr int DENSE_BITS = 16;
constexpr size_t NC_MAX_BYTES = (size_t)32 << 30;  // workspace bound of the uncapped single pass
constexpr int64_t MAX_DW_M_PAD = (int64_t)1 << 21;  // 32-bit buffer offsets of the dW operands

// Layout of the head side (depends on V, H, bits and group only).
struct HeadSide {
  size_t baug, rt, slast, bmx, bytes;
};
HeadSide head_side(const cce_head *hd) {
  const bool dense = hd->bits == DENSE_BITS;
  const int64_t kw = hd->group == 32 ? 32 : KSTEP;
  const int64_t G = hd->H / kw, Gq = hd->H / hd->group;
  const int64_t P = dense ? 0 : cdiv(3 * Gq, KSTEP) * KSTEP;
  const int64_t Kb = 2 * P, NB = Kb / kw;
  HeadSide r{};
  size_t o = 0;
  r.baug = o;  o = align_up(o + (size_t)hd->V * Kb, 256);
  r.rt = o;    o = align_up(o + (dense ? 0 : sizeof(float) * (size_t)(NB + G) * hd->V), 256);
  r.slast = o; o = align_up(o + (dense ? 0 : sizeof(float) * (size_t)hd->V), 256);
  r.bmx = o;   o = align_up(o + (dense ? 0 : sizeof(unsigned) * (size_t)cdiv(hd->V, 64)), 256);
  r.bytes = o;
  return r;
}

// The head's own fields, without a prepared head side.
cce_status check_head_fields(const cce_head *hd) {
  if (!hd || !hd->wq || !hd->scales || !hd->biases) return CCE_ERR_INVALID_ARG;
  if (hd->V < 1 || hd->H < 1) return CCE_ERR_INVALID_ARG;
  if (!(hd->softcap >= 0.0f) || !std::isfinite(hd->softcap)) return CCE_ERR_INVALID_ARG;
  if (hd->bits != 4 && hd->bits != 8) return CCE_ERR_UNSUPPORTED;
  if (hd->group != 32 && hd->group != 64 && hd->group != 128) return CCE_ERR_UNSUPPORTED;
  if (hd->sb_dtype != CCE_SB_F32 && hd->sb_dtype != CCE_SB_BF16 && hd->sb_dtype != CCE_SB_F16)
    return CCE_ERR_UNSUPPORTED;
  if (hd->H % hd->group != 0) return CCE_ERR_INVALID_ARG;
  if (hd->H % KSTEP != 0) return CCE_ERR_UNSUPPORTED;  // group 32 with H an odd multiple of 32
  if (hd->H > MAX_H || hd->V > (int64_t)INT32_MAX - BNT) return CCE_ERR_UNSUPPORTED;
  const uintptr_t sal = hd->sb_dtype == CCE_SB_F32 ? 3 : 1;
  if (((uintptr_t)hd->wq & 15) || ((uintptr_t)hd->scales & sal) || ((uintptr_t)hd->biases & sal))
    return CCE_ERR_INVALID_ARG;
  return CCE_OK;
}

cce_status check_head(const cce_head *hd) {
  const cce_status s = check_head_fields(hd);
  if (s != CCE_OK || !hd->prep) return s;
  if ((uintptr_t)hd->prep & 255) return CCE_ERR_INVALID_ARG;
  return hd->prep_bytes < head_side(hd).bytes ? CCE_ERR_WORKSPACE : CCE_OK;
}

Plan make_plan(const cce_head *hd, int64_t M) {
  Plan p{};
  p.M = M;
  p.M_pad = std::max<int64_t>(BM, cdiv(M, BM) * BM);
  p.V = hd->V;
  p.H = hd->H;
  p.bits = hd->bits;
  p.cap = hd->softcap;
  const bool dense = hd->bits == DENSE_BITS;
  p.gs = hd->group;
  p.kw = p.gs == 32 ? 32 : KSTEP;
  p.G = (int)(p.H / p.kw);
  p.Gq = (int)(p.H / p.gs);
  p.sbt = hd->sb_dtype;
  // bias block: two halves (refinement, coarse) of three columns per
  // quantization group (fixed-point digit x piece of S), each half padded to
  // whole 64-wide steps
  p.P = dense ? 0 : (int)(cdiv(3 * p.Gq, KSTEP) * KSTEP);
  p.Kb = 2 * p.P;
  p.Ka = p.Kb + (int)p.H;
  p.NB = p.Kb / p.kw;
  p.NBr = p.P / p.kw;
  p.wpr = (int)(p.H * p.bits / 32);
  p.TT = (int)(p.M_pad / BM);
  p.tiles = (int)cdiv(p.V, BNT);
  const int64_t cus = device_cus();

  // forward: about one round of tile workgroups (one per CU)
  p.nsplit = (int)std::min<int64_t>(p.tiles, std::max<int64_t>(1, cdiv(cus, p.TT)));
  p.tiles_per_split = (int)cdiv(p.tiles, p.nsplit);
  p.nsplit = (int)cdiv(p.tiles, p.tiles_per_split);
  p.fwd_blocks = p.TT * p.nsplit;
  // Partial slots per token: the kernels give the launched workgroups to the
  // active token tiles only (masked tokens are compacted away), so a few
  // active tiles get more vocabulary splits; bounded to 64 MiB of partials.
  p.max_splits = (int)std::max<int64_t>(
      p.nsplit, std::min<int64_t>(std::min<int64_t>(p.tiles, p.fwd_blocks), ((int64_t)64 << 20) / 16 / p.M_pad));

  // backward: coefficient chunks of at most COEFF_BUDGET bytes
  const int64_t per_tile = p.M_pad * BNT * 2;
  // (at most MAX_CHUNK_TILES: a dh split lists its flagged tiles in LDS)
  p.chunk_tiles = (int)std::max<int64_t>(
      1, std::min<int64_t>(std::min<int64_t>(p.tiles, MAX_CHUNK_TILES), (int64_t)COEFF_BUDGET / per_tile));
  p.nchunks = (int)cdiv(p.tiles, p.chunk_tiles);
  p.ld_coeff = (int64_t)p.chunk_tiles * BNT;
  p.bwd_tpw = (int)std::max<int64_t>(1, std::min<int64_t>(4, (int64_t)p.TT * p.chunk_tiles / (2 * cus)));
  // small M: the tile's small variant is resident once per CU (its LDS), so
  // one round of workgroups, each one unbroken pipeline over its tiles
  if (p.M <= 64) p.bwd_tpw = (int)std::max<int64_t>(1, std::min<int64_t>(8, (int64_t)p.chunk_tiles / cus));
  p.HT = (int)cdiv(p.H, 256);
  // Vocabulary splits of the dh contraction: the fewest that fill whole rounds
  // of resident workgroups (one per CU) to >= 97%, else the best fill of up
  // to 8 -- or, when 8 splits cannot fill one round (few token tiles), of up
  // to a round's worth; each split adds one dh slab, at most 4 GiB of slabs.
  {
    const int64_t slots = cus;
    const int64_t base = (int64_t)p.TT * p.HT;
    const int64_t slab = p.M_pad * p.H * (int64_t)sizeof(float);
    const int64_t reach = base * 8 >= slots ? 8 : std::min<int64_t>(64, cdiv(slots, base));
    const int max_ks = (int)std::max<int64_t>(1, std::min<int64_t>(reach, ((int64_t)4 << 30) / slab));
    int best = 1;
    double best_fill = 0.0;
    for (int ks = 1; ks <= max_ks && ks <= p.chunk_tiles; ++ks) {
      const int64_t n = base * ks;
      const double fill = (double)n / (double)(cdiv(n, slots) * slots);
      if (fill > best_fill + 1e-9) {
        best = ks;
        best_fill = fill;
      }
      if (fill >= 0.97) break;
    }
    p.ksplit = best;
  }
  p.k_tiles = (int)cdiv(p.chunk_tiles, p.ksplit);  // splits hold whole tiles
  p.ksplit = (int)cdiv(p.chunk_tiles, p.k_tiles);

  size_t o = 0;
  p.o_cnt = o;  o = align_up(o + 256, 256);
  p.o_idx = o;  o = align_up(o + sizeof(int) * p.M_pad, 256);
  p.o_inv = o;  o = align_up(o + sizeof(int) * std::max<int64_t>(M, 1), 256);
  p.o_tok = o;  o = align_up(o + sizeof(TokRec) * p.M_pad, 256);
  p.o_haug = o; o = align_up(o + (size_t)2 * p.M_pad * p.Ka, 256);
  {
    const HeadSide hs = head_side(hd);
    p.prep = hd->prep != nullptr;
    p.h_baug = hs.baug;
    p.h_rt = hs.rt;
    p.h_slast = hs.slast;
    p.h_bmx = hs.bmx;
    p.hs_bytes = hs.bytes;
    p.o_hs = o;
    if (!p.prep) o = align_up(o + hs.bytes, 256);
  }
  p.o_sabs = o; o = align_up(o + sizeof(float) * p.M_pad, 256);
  const size_t common = o;
  p.o_part = common;
  p.fwd_bytes = align_up(common + sizeof(float) * 2 * (2 * (size_t)p.max_splits) * p.M_pad, 256);
  p.o_coeff = common;
  o = align_up(common + (size_t)2 * p.M_pad * p.ld_coeff, 256);
  p.o_dhp = o;
  o = align_up(o + sizeof(float) * (size_t)p.ksplit * p.M_pad * p.H, 256);
  p.o_fl = o;  // pair flags of the skips: [TT][tiles] bytes
  o = align_up(o + (size_t)p.TT * p.tiles, 256);
  // The tile launches of the backward and the fused pass: every coefficient
  // chunk with the same grid and split plan (so that the splits of all chunks
  // are numbered in one sequence), at most 64 MiB of per-split partials.
  p.fused = !dense && p.cap > 0.0f && p.cap <= CAP_FIXED_REF_MAX;
  {
    const int64_t nwr = cdiv(p.chunk_tiles, p.bwd_tpw);
    p.fus_blocks = (int)(p.TT * nwr);
    // few token tiles (M <= 1024): one round of workgroups (the tile is
    // resident once per CU, and the device gives fewer active tiles more
    // splits, which would otherwise make a second, shorter-pipelined round)
    if (p.TT <= 4) p.fus_blocks = (int)std::min<int64_t>(p.fus_blocks, cus);
    p.fus_max_splits = (int)std::max<int64_t>(
        nwr, std::min<int64_t>(std::min<int64_t>(p.chunk_tiles, p.fus_blocks),
                               ((int64_t)64 << 20) / 16 / p.M_pad / p.nchunks));
    p.mass_ld = 2 * p.fus_max_splits * p.nchunks;
  }
  // the target's c' per compacted row, then the [M_pad][mass_ld] split sums:
  // the backward's non-target mass or the single pass's non-target sum of 4 e
  p.o_tdc = o;
  o = align_up(o + sizeof(float) * p.M_pad, 256);
  p.o_fpart = o;
  p.bwd_bytes = p.fus_bytes = align_up(o + sizeof(float) * (size_t)p.mass_ld * p.M_pad, 256);
  p.o_ppart = p.bwd_bytes;
  p.twopass_bytes = align_up(p.o_ppart + sizeof(float) * 2 * (2 * (size_t)p.max_splits) * p.M_pad, 256);
  {
    size_t q = common;
    p.nc_coeff = q; q = align_up(q + (size_t)p.nchunks * 2 * p.M_pad * p.ld_coeff, 256);
    p.nc_dhp = q;   q = align_up(q + sizeof(float) * (size_t)p.ksplit * p.M_pad * p.H, 256);
    p.nc_part = q;  q = align_up(q + sizeof(float) * 2 * (size_t)p.mass_ld * p.M_pad, 256);
    p.nc_R = q;     q = align_up(q + sizeof(float) * (size_t)p.tiles * (BNT / 32) * p.M_pad, 256);
    p.nc_nc = q;    q = align_up(q + sizeof(float) * 3 * p.M_pad, 256);
    p.nc_bytes = q;
    // the whole coefficient matrix is kept: beyond NC_MAX_BYTES the two passes run instead
    p.ncfused = !dense && p.cap == 0.0f && p.nc_bytes <= NC_MAX_BYTES;
  }
  if (dense) {
    p.o_hT = p.bwd_bytes;
    o = align_up(p.o_hT + (size_t)2 * p.H * p.M_pad, 256);
    p.o_coeffT = o;
    p.bwd_bytes = align_up(o + (size_t)2 * p.ld_coeff * p.M_pad, 256);
    p.dfused = p.cap >= 0.0f && p.cap <= CAP_FIXED_REF_MAX;
    // with a softcap the tiles write dW's transposed operand of every chunk
    // and dh takes the token-major chunk in turn (one chunk); without, every
    // token-major chunk waits for the scaling and is transposed chunk by chunk
    const size_t chunk_bytes = (size_t)2 * p.M_pad * p.ld_coeff;
    const size_t nkeep = p.cap == 0.0f ? (size_t)p.nchunks : 1, nkeepT = p.cap == 0.0f ? 1 : (size_t)p.nchunks;
    size_t q = common;
    p.df_coeff = q;  q = align_up(q + nkeep * chunk_bytes, 256);
    p.df_dhp = q;    q = align_up(q + sizeof(float) * (size_t)p.ksplit * p.M_pad * p.H, 256);
    p.df_tdc = q;    q = align_up(q + sizeof(float) * p.M_pad, 256);
    p.df_fpart = q;  q = align_up(q + sizeof(float) * (size_t)p.mass_ld * p.M_pad, 256);
    p.df_fac = q;    q = align_up(q + 2 * sizeof(float) * p.M_pad, 256);
    p.df_hT = q;     q = align_up(q + (size_t)2 * p.H * p.M_pad, 256);
    p.df_coeffT = q; q = align_up(q + nkeepT * chunk_bytes, 256);
    if (p.cap == 0.0f) {
      p.df_part = q; q = align_up(q + sizeof(float) * 2 * (size_t)p.mass_ld * p.M_pad, 256);
      p.df_R = q;    q = align_up(q + sizeof(float) * (size_t)p.tiles * (BNT / 32) * p.M_pad, 256);
      p.df_nc = q;   q = align_up(q + sizeof(float) * 3 * p.M_pad, 256);
    }
    p.df_bytes = q;
    if (p.cap == 0.0f && p.df_bytes > NC_MAX_BYTES) p.dfused = false;
  }
  return p;
}

cce_status check_tokens(const void *h, int64_t M, const int32_t *targets, void *workspace) {
  if (M < 0) return CCE_ERR_INVALID_ARG;
  if (M > MAX_M) return CCE_ERR_UNSUPPORTED;
  if (M == 0) return CCE_OK;
  if (!h || !targets) return CCE_ERR_INVALID_ARG;
  if (((uintptr_t)h & 15) || ((uintptr_t)targets & 3)) return CCE_ERR_INVALID_ARG;
  if (workspace && ((uintptr_t)workspace & 255)) return CCE_ERR_INVALID_ARG;
  return CCE_OK;
}

cce_status check_common(const cce_head *hd, const void *h, int64_t M, const int32_t *targets,
                        void *workspace) {
  const cce_status s = check_head(hd);
  return s != CCE_OK ? s : check_tokens(h, M, targets, workspace);
}

// The internal head of a dense bf16 head.
cce_status check_dense(const cce_dense_head *dh, cce_head &q) {
  if (!dh || !dh->w) return CCE_ERR_INVALID_ARG;
  if (dh->V < 1 || dh->H < 1) return CCE_ERR_INVALID_ARG;
  if (!(dh->softcap >= 0.0f) || !std::isfinite(dh->softcap)) return CCE_ERR_INVALID_ARG;
  if (dh->H % KSTEP != 0) return CCE_ERR_UNSUPPORTED;
  if (dh->H > MAX_H || dh->V > (int64_t)INT32_MAX - BNT) return CCE_ERR_UNSUPPORTED;
  if ((uintptr_t)dh->w & 15) return CCE_ERR_INVALID_ARG;
  q = cce_head{static_cast<const uint32_t *>(dh->w), nullptr, nullptr, dh->V, dh->H, DENSE_BITS, 32,
               dh->softcap, CCE_SB_F32};
  return CCE_OK;
}

cce_status hip_status() {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return CCE_OK;
  std::snprintf(g_err, sizeof g_err, "HIP error: %s", hipGetErrorString(e));
  return CCE_ERR_HIP;
}

template <typename T>
T *ws_at(void *ws, size_t off) {
  return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

// an array of the head side: in the prepared buffer, or in the workspace
template <typename T>
T *hs_at(const Plan &p, const cce_head *hd, void *ws, size_t off) {
  char *base = p.prep ? static_cast<char *>(const_cast<void *>(hd->prep)) : static_cast<char *>(ws) + p.o_hs;
  return reinterpret_cast<T *>(base + off);
}

// compaction, augmented rows and token records, target logits
void enqueue_front(const Plan &p, const cce_head *hd, const void *h, const int32_t *targets,
                   const uint8_t *mask, const float *lse, const float *g, void *ws, hipStream_t st,
                   bool bwd, float *out_logp = nullptr, float *out_lse = nullptr) {
  int *cnt = ws_at<int>(ws, p.o_cnt);
  int *idx = ws_at<int>(ws, p.o_idx);
  int *inv = ws_at<int>(ws, p.o_inv);
  TokRec *tok = ws_at<TokRec>(ws, p.o_tok);
  uint16_t *haug = ws_at<uint16_t>(ws, p.o_haug);
  // up to this many tokens the front's row blocks compact the mask themselves
  // (each scans all M mask bytes), one launch fewer
  const bool fuse = p.M <= FUSED_COMPACT_MAX_M;
  if (!fuse)
    CCE_LAUNCH("compact", st, launch_compact(st, mask, (int)p.M, (int)p.M_pad, idx, inv, cnt, out_logp, out_lse));
  FrontArgs f{};
  f.out_logp = out_logp;
  f.out_lse = out_lse;
  f.compact = fuse ? 1 : 0;
  f.M = (int)p.M;
  f.mask = mask;
  f.idx_out = idx;
  f.inv = inv;
  f.cnt = cnt;
  f.h = (const uint16_t *)h;
  f.idx = idx;
  f.targets = targets;
  f.lse = lse;
  f.g = g;
  f.wq = hd->wq;
  f.scales = hd->scales;
  f.biases = hd->biases;
  f.tok = tok;
  f.haug = haug;
  f.baug = hs_at<uint8_t>(p, hd, ws, p.h_baug);
  f.rt = hs_at<float>(p, hd, ws, p.h_rt);
  f.gs = p.gs;
  f.Gq = p.Gq;
  f.sbt = p.sbt;
  f.slast = hs_at<float>(p, hd, ws, p.h_slast);
  f.bmxb = hs_at<unsigned>(p, hd, ws, p.h_bmx);
  f.head = p.prep ? 0 : 1;  // a prepared head: token rows only
  f.sabs = ws_at<float>(ws, p.o_sabs);
  f.P = p.P;
  f.V = p.V;
  f.H = (int)p.H;
  f.G = p.G;
  f.Kb = p.Kb;
  f.Ka = p.Ka;
  f.NB = p.NB;
  f.wpr = p.wpr;
  f.M_pad = (int)p.M_pad;
  f.cap = p.cap;
  f.bwd = bwd ? 1 : 0;
  CCE_LAUNCH("front", st, launch_front(st, p.bits, f));
}

TileArgs tile_args(const Plan &p, const cce_head *hd, void *ws) {
  const bool dense = hd->bits == DENSE_BITS;
  TileArgs a{};
  a.haug = ws_at<const uint16_t>(ws, p.o_haug);
  a.baug = hs_at<const uint8_t>(p, hd, ws, p.h_baug);
  a.rt = hs_at<const float>(p, hd, ws, p.h_rt);
  a.slast = hs_at<const float>(p, hd, ws, p.h_slast);
  a.bmxb = hs_at<const unsigned>(p, hd, ws, p.h_bmx);
  a.nbmx = dense ? 0 : (int)cdiv(p.V, 64);
  a.sabs = ws_at<const float>(ws, p.o_sabs);
  a.wq = hd->wq;
  a.cnt = ws_at<const int>(ws, p.o_cnt);
  a.tok = ws_at<TokRec>(ws, p.o_tok);
  a.V = p.V;
  a.G = p.G;
  a.Ka = p.Ka;
  a.Kb = p.Kb;
  a.NB = p.NB;
  a.NBr = p.NBr;
  a.kw = p.kw;
  a.wpr = p.wpr;
  a.M_pad = (int)p.M_pad;
  a.ks16 = p.Ka / 16;
  a.ksv = p.ld_coeff / 16;
  a.cap = p.cap;
  a.inv_cap = p.cap > 0.0f ? 1.0f / p.cap : 0.0f;
  a.small = p.M <= 32 ? 2 : (p.M <= 64 ? 1 : 0);  // 2: one 32-row token block
  return a;
}

// The launches of a forward on a validated head and token set (M > 0).
cce_status run_forward(const cce_head *head, const void *h, int64_t M, const int32_t *targets, const uint8_t *mask,
                       float *logp, float *lse, float *block_max, void *workspace, size_t workspace_bytes,
                       void *stream) {
  if (!logp || !lse || ((uintptr_t)logp & 3) || ((uintptr_t)lse & 3) || ((uintptr_t)block_max & 3))
    return CCE_ERR_INVALID_ARG;
  const Plan p = make_plan(head, M);
  if (block_max && cdiv(p.tiles, 256) * M > INT32_MAX) return CCE_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < p.fwd_bytes) return CCE_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();

  enqueue_front(p, head, h, targets, mask, nullptr, nullptr, workspace, st, false);
  TileArgs a = tile_args(p, head, workspace);
  a.part = ws_at<float>(workspace, p.o_part);
  a.range_tile0 = 0;
  a.range_tiles = p.tiles;
  a.chunk = 0;
  a.full_tiles = p.tiles;
  a.nblocks = p.fwd_blocks;
  a.max_splits = p.max_splits;
  a.bmx = block_max;
  a.idx = ws_at<const int>(workspace, p.o_idx);
  a.nbv = p.tiles;
  const dim3 grid((unsigned)(cdiv(a.nblocks, 8) * 8));
  CCE_LAUNCH("tile_fwd", st, launch_tile(st, p.bits, PASS_FWD, grid, a));
  CCE_LAUNCH("merge", st, launch_merge(st, (int)M, a.part, a.nblocks, p.tiles, p.tiles, p.max_splits, (int)p.M_pad,
                                       ws_at<const int>(workspace, p.o_inv), a.cnt,
                                       ws_at<const TokRec>(workspace, p.o_tok), logp, lse));
  if (block_max && mask)
    CCE_LAUNCH("bmx_mask", st, launch_bmx_mask(st, (int)M, p.tiles, ws_at<const int>(workspace, p.o_inv), block_max));
  return hip_status();
}

// The launches of a backward on a validated head and token set (M > 0);
// dw (dense heads only) NULL or the [V][H] fp32 head gradient.
cce_status run_backward(const cce_head *head, const void *h, int64_t M, const int32_t *targets,
                        const uint8_t *mask, const float *lse, const float *g, const float *block_max,
                        const cce_skip *skip, void *dh, int32_t dh_dtype, float *dw, void *workspace,
                        size_t workspace_bytes, void *stream) {
  if (dh_dtype != CCE_DH_F32 && dh_dtype != CCE_DH_BF16) return CCE_ERR_INVALID_ARG;
  const uintptr_t dh_align = dh_dtype == CCE_DH_F32 ? 3 : 1;
  if (!lse || !dh || ((uintptr_t)lse & 3) || ((uintptr_t)dh & dh_align) || ((uintptr_t)g & 3))
    return CCE_ERR_INVALID_ARG;
  float block_eps = 0.0f, filter_eps = 0.0f;
  if (skip) {
    block_eps = skip->block_eps;
    filter_eps = skip->filter_eps;
    if (!(block_eps >= 0.0f) || !std::isfinite(block_eps) || !(filter_eps >= 0.0f) || !std::isfinite(filter_eps))
      return CCE_ERR_INVALID_ARG;
    if (block_eps > 0.0f && (!block_max || ((uintptr_t)block_max & 3))) return CCE_ERR_INVALID_ARG;
  }
  const Plan p = make_plan(head, M);
  if (dw && ((uintptr_t)dw & 3)) return CCE_ERR_INVALID_ARG;
  if (dw && p.M_pad > MAX_DW_M_PAD) return CCE_ERR_UNSUPPORTED;
  const bool use_fl = block_eps > 0.0f || filter_eps > 0.0f;
  if (use_fl && cdiv(p.tiles, 64) * p.TT > INT32_MAX) return CCE_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < p.bwd_bytes) return CCE_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();

  enqueue_front(p, head, h, targets, mask, lse, g, workspace, st, true);
  TileArgs a = tile_args(p, head, workspace);
  a.coeff = ws_at<uint16_t>(workspace, p.o_coeff);
  a.ld_coeff = p.ld_coeff;
  a.max_splits = 1 << 30;
  uint8_t *fl = use_fl ? ws_at<uint8_t>(workspace, p.o_fl) : nullptr;
  if (fl)
    CCE_LAUNCH("warm", st, launch_warm(st, p.TT, p.tiles, a.cnt, ws_at<const int>(workspace, p.o_idx), a.tok,
                                       block_max, p.tiles, block_eps > 0.0f ? std::log(block_eps) : 0.0f,
                                       block_eps > 0.0f ? 1 : 0, fl));
  a.fl = fl;
  a.fl_ld = p.tiles;
  a.filter_eps = filter_eps;
  // 1 - p_t from the non-target mass, except under the skips (the target's
  // term is then -expm1(y_t - lse), as the skips' model keeps it) and for a
  // dense head (its dW takes the whole coefficient chunk by chunk; dh is the
  // same with or without dW)
  a.tmass = (fl == nullptr && head->bits != DENSE_BITS) ? 1 : 0;
  a.tdc = ws_at<float>(workspace, p.o_tdc);
  a.mass = ws_at<float>(workspace, p.o_fpart);
  a.mass_ld = p.mass_ld;
  a.full_tiles = p.chunk_tiles;
  a.nblocks = p.fus_blocks;
  a.max_splits = p.fus_max_splits;
  const dim3 g1((unsigned)(cdiv(a.nblocks, 8) * 8));

  GemmArgs ga{};
  ga.coeff = a.coeff;
  ga.ksv = p.ld_coeff / 16;
  ga.wq = head->wq;
  ga.scales = head->scales;
  ga.biases = head->biases;
  ga.cnt = a.cnt;
  ga.dh_part = ws_at<float>(workspace, p.o_dhp);
  ga.V = p.V;
  ga.H = (int)p.H;
  ga.gs = p.gs;
  ga.Gq = p.Gq;
  ga.sbt = p.sbt;
  ga.wpr = p.wpr;
  ga.M_pad = (int)p.M_pad;
  ga.max_chunk_steps = p.chunk_tiles * (BNT / KSTEP);
  ga.TT = p.TT;
  ga.HT = p.HT;
  ga.ksplit = p.ksplit;
  ga.nblocks = p.TT * p.HT * p.ksplit;
  ga.fl = fl;
  ga.fl_ld = p.tiles;
  ga.small = a.small;
  const dim3 g2((unsigned)(cdiv(ga.nblocks, 8) * 8));

  DwArgs wa{};
  if (dw) {
    wa.coeffT = ws_at<const uint16_t>(workspace, p.o_coeffT);
    wa.hT = ws_at<const uint16_t>(workspace, p.o_hT);
    wa.cnt = a.cnt;
    wa.dw = dw;
    wa.V = p.V;
    wa.ks16t = p.M_pad / 16;
    wa.H = (int)p.H;
    wa.M_pad = (int)p.M_pad;
    wa.HT = p.HT;
    CCE_LAUNCH("hT", st, launch_hT(st, a.haug, p.Ka / 16, p.Kb / 8, (int)p.M_pad, (int)p.H, a.cnt, nullptr,
                                   ws_at<uint16_t>(workspace, p.o_hT)));
  }

  for (int c = 0; c < p.nchunks; ++c) {
    const int t0 = c * p.chunk_tiles;
    const int nt = std::min(p.chunk_tiles, p.tiles - t0);
    a.range_tile0 = t0;
    a.range_tiles = nt;
    a.chunk = c;
    CCE_LAUNCH("tile_bwd", st, launch_tile(st, p.bits, PASS_BWD, g1, a));
    ga.chunk_v0 = (int64_t)t0 * BNT;
    ga.chunk_tile0 = t0;
    ga.chunk_steps = nt * (BNT / KSTEP);
    ga.accumulate = c > 0;
    CCE_LAUNCH("dh_gemm", st, launch_dh_gemm(st, p.bits, g2, ga));
    if (dw) {
      CCE_LAUNCH("coeffT", st, launch_coeffT(st, a.coeff, ga.ksv, (int)p.M_pad, nt * BNT, a.cnt, a.tok, nullptr,
                                             p.V, ga.chunk_v0, ws_at<uint16_t>(workspace, p.o_coeffT)));
      wa.chunk_v0 = ga.chunk_v0;
      wa.nvt = nt;
      CCE_LAUNCH("dw_gemm", st, launch_dw(st, wa));
    }
  }
  CCE_LAUNCH("dh_reduce", st, launch_dh_reduce(st, p.bits, (int)M, ga, ws_at<const int>(workspace, p.o_inv),
                                               ws_at<const TokRec>(workspace, p.o_tok), dh,
                                               dh_dtype == CCE_DH_BF16 ? 1 : 0,
                                               ReduceTarget{a.tmass, a.mass, a.mass_ld, a.nblocks, a.full_tiles,
                                                            p.tiles, a.max_splits, 0.0f, a.tdc, nullptr, nullptr}));
  return hip_status();
}

// The single pass of a quantized head without a softcap.  There is no fixed
// reference, so each tile writes its coefficients -e^{z - R} against the
// largest logit R of their 32-row vocabulary block (recorded), and its (max,
// sum) partials over the non-target columns; every chunk is kept.  The merge
// then gives lse, logp and each token's largest logit m, one launch scales
// every coefficient by e^{R - m} (at most 1), and the dh contractions and the
// split reduce proceed as for the capped single pass, against m.  The dh
// contraction's small-M variant applies the factor itself as it stages each
// coefficient fragment (the same arithmetic, so the same bits): no scaling
// launch.
cce_status run_nc_fused(const Plan &p, const cce_head *head, const void *h, int64_t M, const int32_t *targets,
                        const uint8_t *mask, const float *g, float *logp, float *lse, void *dh, int32_t dh_dtype,
                        void *workspace, hipStream_t st) {
  enqueue_front(p, head, h, targets, mask, nullptr, g, workspace, st, false);
  TileArgs a = tile_args(p, head, workspace);
  a.part = ws_at<float>(workspace, p.nc_part);
  a.ncR = ws_at<float>(workspace, p.nc_R);
  a.ld_coeff = p.ld_coeff;
  a.full_tiles = p.chunk_tiles;
  a.nblocks = p.fus_blocks;
  a.max_splits = p.fus_max_splits;
  const dim3 g1((unsigned)(cdiv(a.nblocks, 8) * 8));
  uint16_t *coeff0 = ws_at<uint16_t>(workspace, p.nc_coeff);
  const size_t chunk_elems = (size_t)p.M_pad * p.ld_coeff;
  for (int c = 0; c < p.nchunks; ++c) {
    const int t0 = c * p.chunk_tiles;
    a.coeff = coeff0 + c * chunk_elems;
    a.range_tile0 = t0;
    a.range_tiles = std::min(p.chunk_tiles, p.tiles - t0);
    a.chunk = c;
    CCE_LAUNCH("tile_fused", st, launch_tile(st, p.bits, PASS_FUSED_NC, g1, a));
  }
  const int *inv = ws_at<const int>(workspace, p.o_inv);
  const TokRec *tok = ws_at<const TokRec>(workspace, p.o_tok);
  float *nc = ws_at<float>(workspace, p.nc_nc);
  CCE_LAUNCH("merge", st, launch_merge(st, (int)M, a.part, a.nblocks, p.chunk_tiles, p.tiles, p.fus_max_splits,
                                       (int)p.M_pad, inv, a.cnt, tok, logp, lse, nc));
  // the variant launch_dh_gemm picks for a.small (the default storage only)
  const bool scale_in_dh = a.small != 0 && p.gs == KSTEP && p.sbt == SB_F32;
  if (!scale_in_dh)
    CCE_LAUNCH("nc_scale", st, launch_nc_scale(st, coeff0, p.ld_coeff, p.nchunks,
                                               p.V - (int64_t)(p.nchunks - 1) * p.ld_coeff, (int)p.M_pad, a.cnt,
                                               a.ncR, nc));

  GemmArgs ga{};
  if (scale_in_dh) {
    ga.ncR = a.ncR;
    ga.nc = nc;
  }
  ga.ksv = p.ld_coeff / 16;
  ga.wq = head->wq;
  ga.scales = head->scales;
  ga.biases = head->biases;
  ga.cnt = a.cnt;
  ga.dh_part = ws_at<float>(workspace, p.nc_dhp);
  ga.V = p.V;
  ga.H = (int)p.H;
  ga.gs = p.gs;
  ga.Gq = p.Gq;
  ga.sbt = p.sbt;
  ga.wpr = p.wpr;
  ga.M_pad = (int)p.M_pad;
  ga.max_chunk_steps = p.chunk_tiles * (BNT / KSTEP);
  ga.TT = p.TT;
  ga.HT = p.HT;
  ga.ksplit = p.ksplit;
  ga.nblocks = p.TT * p.HT * p.ksplit;
  ga.small = a.small;
  const dim3 g2((unsigned)(cdiv(ga.nblocks, 8) * 8));
  for (int c = 0; c < p.nchunks; ++c) {
    const int t0 = c * p.chunk_tiles;
    const int nt = std::min(p.chunk_tiles, p.tiles - t0);
    ga.coeff = coeff0 + c * chunk_elems;
    ga.chunk_v0 = (int64_t)t0 * BNT;
    ga.chunk_tile0 = t0;
    ga.chunk_steps = nt * (BNT / KSTEP);
    ga.accumulate = c > 0;
    CCE_LAUNCH("dh_gemm", st, launch_dh_gemm(st, p.bits, g2, ga));
  }
  ReduceTarget rt{};
  rt.mode = 3;
  rt.nc = nc;
  CCE_LAUNCH("dh_reduce", st, launch_dh_reduce(st, p.bits, (int)M, ga, inv, tok, dh, dh_dtype == CCE_DH_BF16 ? 1 : 0,
                                               rt));
  return hip_status();
}

// The single pass of a dense head (softcap in [0, CAP_FIXED_REF_MAX]): the
// fused tile and the dh contraction per chunk as for a quantized head, every
// chunk kept; the split reduce then forms lse, logp, dh and each row's factor
// g / (S + e_t); dW last, chunk by chunk, from the unnormalized coefficients
// and hT scaled by those factors (dW_v = sum_t coefficient_tv (factor_t h_t)).
// Without a softcap the tiles write against their blocks' references and the
// dh contractions wait for the merge and the scaling launch, as in
// run_nc_fused.
cce_status run_dense_fused(const Plan &p, const cce_head *head, const void *h, int64_t M, const int32_t *targets,
                           const uint8_t *mask, const float *g, float *logp, float *lse, float *dh, float *dw,
                           void *workspace, hipStream_t st) {
  enqueue_front(p, head, h, targets, mask, nullptr, g, workspace, st, false);
  const bool nocap = p.cap == 0.0f;  // the uncapped variant: block references, merge, scaling
  TileArgs a = tile_args(p, head, workspace);
  a.mass = ws_at<float>(workspace, p.df_fpart);
  a.mass_ld = p.mass_ld;
  a.ld_coeff = p.ld_coeff;
  a.tdc = ws_at<float>(workspace, p.df_tdc);
  if (nocap) {
    a.part = ws_at<float>(workspace, p.df_part);
    a.ncR = ws_at<float>(workspace, p.df_R);
  }
  a.full_tiles = p.chunk_tiles;
  a.nblocks = p.fus_blocks;
  a.max_splits = p.fus_max_splits;
  const dim3 g1((unsigned)(cdiv(a.nblocks, 8) * 8));
  uint16_t *coeff0 = ws_at<uint16_t>(workspace, p.df_coeff);
  uint16_t *coeffT0 = ws_at<uint16_t>(workspace, p.df_coeffT);
  const size_t chunk_elems = (size_t)p.M_pad * p.ld_coeff;
  a.ks16t = p.M_pad / 16;

  GemmArgs ga{};
  ga.ksv = p.ld_coeff / 16;
  ga.wq = head->wq;
  ga.scales = head->scales;
  ga.biases = head->biases;
  ga.cnt = a.cnt;
  ga.dh_part = ws_at<float>(workspace, p.df_dhp);
  ga.V = p.V;
  ga.H = (int)p.H;
  ga.gs = p.gs;
  ga.Gq = p.Gq;
  ga.sbt = p.sbt;
  ga.wpr = p.wpr;
  ga.M_pad = (int)p.M_pad;
  ga.max_chunk_steps = p.chunk_tiles * (BNT / KSTEP);
  ga.TT = p.TT;
  ga.HT = p.HT;
  ga.ksplit = p.ksplit;
  ga.nblocks = p.TT * p.HT * p.ksplit;
  ga.small = a.small;
  const dim3 g2((unsigned)(cdiv(ga.nblocks, 8) * 8));

  for (int c = 0; c < p.nchunks; ++c) {
    const int t0 = c * p.chunk_tiles;
    const int nt = std::min(p.chunk_tiles, p.tiles - t0);
    a.coeff = nocap ? coeff0 + c * chunk_elems : coeff0;
    a.coeffT = (!nocap && dw) ? coeffT0 + c * chunk_elems : nullptr;
    a.range_tile0 = t0;
    a.range_tiles = nt;
    a.chunk = c;
    CCE_LAUNCH("tile_fused", st, launch_tile(st, p.bits, nocap ? PASS_FUSED_NC : PASS_FUSED, g1, a));
    if (nocap) continue;  // dh once every chunk is at the token's maximum
    ga.coeff = a.coeff;
    ga.chunk_v0 = (int64_t)t0 * BNT;
    ga.chunk_tile0 = t0;
    ga.chunk_steps = nt * (BNT / KSTEP);
    ga.accumulate = c > 0;
    CCE_LAUNCH("dh_gemm", st, launch_dh_gemm(st, p.bits, g2, ga));
  }
  const int *inv = ws_at<const int>(workspace, p.o_inv);
  const TokRec *tok = ws_at<const TokRec>(workspace, p.o_tok);
  float *fac = dw ? ws_at<float>(workspace, p.df_fac) : nullptr;
  ReduceTarget rt{2, a.mass, a.mass_ld, a.nblocks, p.chunk_tiles, p.tiles, p.fus_max_splits, p.cap, a.tdc,
                  logp, lse, fac};
  if (nocap) {
    float *nc = ws_at<float>(workspace, p.df_nc);
    CCE_LAUNCH("merge", st, launch_merge(st, (int)M, a.part, a.nblocks, p.chunk_tiles, p.tiles, p.fus_max_splits,
                                         (int)p.M_pad, inv, a.cnt, tok, logp, lse, nc));
    CCE_LAUNCH("nc_scale", st, launch_nc_scale(st, coeff0, p.ld_coeff, p.nchunks,
                                               p.V - (int64_t)(p.nchunks - 1) * p.ld_coeff, (int)p.M_pad, a.cnt,
                                               a.ncR, nc));
    for (int c = 0; c < p.nchunks; ++c) {
      const int t0 = c * p.chunk_tiles;
      ga.coeff = coeff0 + c * chunk_elems;
      ga.chunk_v0 = (int64_t)t0 * BNT;
      ga.chunk_tile0 = t0;
      ga.chunk_steps = std::min(p.chunk_tiles, p.tiles - t0) * (BNT / KSTEP);
      ga.accumulate = c > 0;
      CCE_LAUNCH("dh_gemm", st, launch_dh_gemm(st, p.bits, g2, ga));
    }
    rt = ReduceTarget{};
    rt.mode = 3;
    rt.nc = nc;
    rt.fac = fac;
  }
  CCE_LAUNCH("dh_reduce", st, launch_dh_reduce(st, p.bits, (int)M, ga, inv, tok, dh, 0, rt));
  if (dw) {
    DwArgs wa{};
    wa.coeffT = ws_at<const uint16_t>(workspace, p.df_coeffT);
    wa.hT = ws_at<const uint16_t>(workspace, p.df_hT);
    wa.cnt = a.cnt;
    wa.dw = dw;
    wa.V = p.V;
    wa.ks16t = p.M_pad / 16;
    wa.H = (int)p.H;
    wa.M_pad = (int)p.M_pad;
    wa.HT = p.HT;
    // with a softcap the tiles wrote every transposed chunk but the target
    // entries, which launch_hT sets
    CCE_LAUNCH("hT", st, launch_hT(st, a.haug, p.Ka / 16, p.Kb / 8, (int)p.M_pad, (int)p.H, a.cnt, fac,
                                   ws_at<uint16_t>(workspace, p.df_hT), nocap ? nullptr : a.tok,
                                   nocap ? nullptr : coeffT0, p.ld_coeff));
    for (int c = 0; c < p.nchunks; ++c) {
      const int t0 = c * p.chunk_tiles;
      const int nt = std::min(p.chunk_tiles, p.tiles - t0);
      const int64_t v0 = (int64_t)t0 * BNT;
      if (nocap) {
        CCE_LAUNCH("coeffT", st, launch_coeffT(st, coeff0 + c * chunk_elems, ga.ksv, (int)p.M_pad, nt * BNT, a.cnt,
                                               a.tok, fac, p.V, v0, coeffT0));
      } else {
        wa.coeffT = coeffT0 + c * chunk_elems;
      }
      wa.chunk_v0 = v0;
      wa.nvt = nt;
      CCE_LAUNCH("dw_gemm", st, launch_dw(st, wa));
    }
  }
  return hip_status();
}

// The single pass (PASS_FUSED) for a quantized head with 0 < softcap <=
// CAP_FIXED_REF_MAX and a known g: per coefficient chunk, the logit tile
// writes its forward partials and the unnormalized coefficients, and the dh
// contraction consumes the chunk; then the split reduce, which also takes
// the place of the merge: it sums each token's split sums into lse and logp,
// scales the slabs by g e^{cap - lse} and adds the target's term.  No logit
// is computed twice.
cce_status run_fused(const Plan &p, const cce_head *head, const void *h, int64_t M, const int32_t *targets,
                     const uint8_t *mask, const float *g, float *logp, float *lse, void *dh, int32_t dh_dtype,
                     void *workspace, hipStream_t st) {
  enqueue_front(p, head, h, targets, mask, nullptr, g, workspace, st, false);
  TileArgs a = tile_args(p, head, workspace);
  a.mass = ws_at<float>(workspace, p.o_fpart);
  a.mass_ld = p.mass_ld;
  a.coeff = ws_at<uint16_t>(workspace, p.o_coeff);
  a.ld_coeff = p.ld_coeff;
  a.tdc = ws_at<float>(workspace, p.o_tdc);
  a.full_tiles = p.chunk_tiles;
  a.nblocks = p.fus_blocks;
  a.max_splits = p.fus_max_splits;
  const dim3 g1((unsigned)(cdiv(a.nblocks, 8) * 8));

  GemmArgs ga{};
  ga.coeff = a.coeff;
  ga.ksv = p.ld_coeff / 16;
  ga.wq = head->wq;
  ga.scales = head->scales;
  ga.biases = head->biases;
  ga.cnt = a.cnt;
  ga.dh_part = ws_at<float>(workspace, p.o_dhp);
  ga.V = p.V;
  ga.H = (int)p.H;
  ga.gs = p.gs;
  ga.Gq = p.Gq;
  ga.sbt = p.sbt;
  ga.wpr = p.wpr;
  ga.M_pad = (int)p.M_pad;
  ga.max_chunk_steps = p.chunk_tiles * (BNT / KSTEP);
  ga.TT = p.TT;
  ga.HT = p.HT;
  ga.ksplit = p.ksplit;
  ga.nblocks = p.TT * p.HT * p.ksplit;
  ga.small = a.small;
  const dim3 g2((unsigned)(cdiv(ga.nblocks, 8) * 8));

  for (int c = 0; c < p.nchunks; ++c) {
    const int t0 = c * p.chunk_tiles;
    const int nt = std::min(p.chunk_tiles, p.tiles - t0);
    a.range_tile0 = t0;
    a.range_tiles = nt;
    a.chunk = c;
    CCE_LAUNCH("tile_fused", st, launch_tile(st, p.bits, PASS_FUSED, g1, a));
    ga.chunk_v0 = (int64_t)t0 * BNT;
    ga.chunk_tile0 = t0;
    ga.chunk_steps = nt * (BNT / KSTEP);
    ga.accumulate = c > 0;
    CCE_LAUNCH("dh_gemm", st, launch_dh_gemm(st, p.bits, g2, ga));
  }
  const int *inv = ws_at<const int>(workspace, p.o_inv);
  const TokRec *tok = ws_at<const TokRec>(workspace, p.o_tok);
  const ReduceTarget rt{2, a.mass, a.mass_ld, a.nblocks, p.chunk_tiles, p.tiles, p.fus_max_splits, p.cap, a.tdc,
                        logp, lse};
  CCE_LAUNCH("dh_reduce", st, launch_dh_reduce(st, p.bits, (int)M, ga, inv, tok, dh, dh_dtype == CCE_DH_BF16 ? 1 : 0,
                                               rt));
  return hip_status();
}

// cce_forward_backward on a head without the single pass (no softcap, or one
// above CAP_FIXED_REF_MAX): one front (with g), the forward tile, then the
// backward chunks, whose tiles form each token's lse from the forward's
// partials themselves (no merge launch; the workgroup of split 0 of chunk 0
// writes logp and lse), the dh contraction and the split reduce.
cce_status run_twopass(const Plan &p, const cce_head *head, const void *h, int64_t M, const int32_t *targets,
                       const uint8_t *mask, const float *g, float *logp, float *lse, void *dh, int32_t dh_dtype,
                       void *workspace, hipStream_t st) {
  enqueue_front(p, head, h, targets, mask, nullptr, g, workspace, st, false, logp, lse);
  TileArgs a = tile_args(p, head, workspace);
  float *ppart = ws_at<float>(workspace, p.o_ppart);
  a.part = ppart;
  a.range_tile0 = 0;
  a.range_tiles = p.tiles;
  a.chunk = 0;
  a.full_tiles = p.tiles;
  a.nblocks = p.fwd_blocks;
  a.max_splits = p.max_splits;
  CCE_LAUNCH("tile_fwd", st, launch_tile(st, p.bits, PASS_FWD, dim3((unsigned)(cdiv(a.nblocks, 8) * 8)), a));

  TileArgs b = tile_args(p, head, workspace);
  b.coeff = ws_at<uint16_t>(workspace, p.o_coeff);
  b.ld_coeff = p.ld_coeff;
  b.tmass = 1;
  b.tdc = ws_at<float>(workspace, p.o_tdc);
  b.mass = ws_at<float>(workspace, p.o_fpart);
  b.mass_ld = p.mass_ld;
  b.full_tiles = p.chunk_tiles;
  b.nblocks = p.fus_blocks;
  b.max_splits = p.fus_max_splits;
  b.fpart = ppart;
  b.f_nblocks = p.fwd_blocks;
  b.f_tiles = p.tiles;
  b.f_max_splits = p.max_splits;
  b.idx = ws_at<const int>(workspace, p.o_idx);
  b.out_logp = logp;
  b.out_lse = lse;
  const dim3 g1((unsigned)(cdiv(b.nblocks, 8) * 8));

  GemmArgs ga{};
  ga.coeff = b.coeff;
  ga.ksv = p.ld_coeff / 16;
  ga.wq = head->wq;
  ga.scales = head->scales;
  ga.biases = head->biases;
  ga.cnt = b.cnt;
  ga.dh_part = ws_at<float>(workspace, p.o_dhp);
  ga.V = p.V;
  ga.H = (int)p.H;
  ga.gs = p.gs;
  ga.Gq = p.Gq;
  ga.sbt = p.sbt;
  ga.wpr = p.wpr;
  ga.M_pad = (int)p.M_pad;
  ga.max_chunk_steps = p.chunk_tiles * (BNT / KSTEP);
  ga.TT = p.TT;
  ga.HT = p.HT;
  ga.ksplit = p.ksplit;
  ga.nblocks = p.TT * p.HT * p.ksplit;
  ga.small = b.small;
  const dim3 g2((unsigned)(cdiv(ga.nblocks, 8) * 8));
  for (int c = 0; c < p.nchunks; ++c) {
    const int t0 = c * p.chunk_tiles;
    const int nt = std::min(p.chunk_tiles, p.tiles - t0);
    b.range_tile0 = t0;
    b.range_tiles = nt;
    b.chunk = c;
    CCE_LAUNCH("tile_bwd", st, launch_tile(st, p.bits, PASS_BWD, g1, b));
    ga.chunk_v0 = (int64_t)t0 * BNT;
    ga.chunk_tile0 = t0;
    ga.chunk_steps = nt * (BNT / KSTEP);
    ga.accumulate = c > 0;
    CCE_LAUNCH("dh_gemm", st, launch_dh_gemm(st, p.bits, g2, ga));
  }
  CCE_LAUNCH("dh_reduce", st, launch_dh_reduce(st, p.bits, (int)M, ga, ws_at<const int>(workspace, p.o_inv),
                                               ws_at<const TokRec>(workspace, p.o_tok), dh,
                                               dh_dtype == CCE_DH_BF16 ? 1 : 0,
                                               ReduceTarget{1, b.mass, b.mass_ld, b.nblocks, b.full_tiles, p.tiles,
                                                            b.max_splits, 0.0f, b.tdc, nullptr, nullptr}));
  return hip_status();
}

// Device address of this device's `scratch`, looked up with the device
// current the first time a call runs on it (nullptr if the lookup fails).
std::mutex g_scratch_mu;
void *g_scratch_ptr[64];

void *scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hip_status();  // keep the HIP error text for cce_status_str
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

size_t fwdbwd_bytes(const Plan &p) { return p.fused ? p.fus_bytes : (p.ncfused ? p.nc_bytes : p.twopass_bytes); }

}  // namespace

extern "C" {

int cce_abi_version(void) { return CCE_ABI_VERSION; }

const char *cce_status_str(cce_status s) {
  switch (s) {
    case CCE_OK: return "ok";
    case CCE_ERR_INVALID_ARG: return "invalid argument";
    case CCE_ERR_UNSUPPORTED: return "unsupported head configuration";
    case CCE_ERR_WORKSPACE: return "workspace missing or too small";
    case CCE_ERR_HIP: return g_err[0] ? g_err : "HIP error";
  }
  return "unknown status";
}

size_t cce_head_prepare_bytes(const cce_head *head) {
  if (check_head_fields(head) != CCE_OK) return 0;
  return head_side(head).bytes;
}

cce_status cce_head_prepare(const cce_head *head, void *prep, size_t prep_bytes, void *stream) {
  const cce_status s = check_head_fields(head);
  if (s != CCE_OK) return s;
  if (!prep || ((uintptr_t)prep & 255)) return CCE_ERR_INVALID_ARG;
  const HeadSide hs = head_side(head);
  if (prep_bytes < hs.bytes) return CCE_ERR_WORKSPACE;
  // the front's head blocks alone (no token rows), into the caller's buffer
  const Plan p = make_plan(head, 0);
  char *b = static_cast<char *>(prep);
  FrontArgs f{};
  f.wq = head->wq;
  f.scales = head->scales;
  f.biases = head->biases;
  f.baug = reinterpret_cast<uint8_t *>(b + hs.baug);
  f.rt = reinterpret_cast<float *>(b + hs.rt);
  f.slast = reinterpret_cast<float *>(b + hs.slast);
  f.bmxb = reinterpret_cast<unsigned *>(b + hs.bmx);
  f.gs = p.gs;
  f.Gq = p.Gq;
  f.sbt = p.sbt;
  f.P = p.P;
  f.V = p.V;
  f.H = (int)p.H;
  f.G = p.G;
  f.Kb = p.Kb;
  f.Ka = p.Ka;
  f.NB = p.NB;
  f.wpr = p.wpr;
  f.M_pad = 0;
  f.cap = p.cap;
  f.head = 1;
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  CCE_LAUNCH("front", st, launch_front(st, p.bits, f));
  return hip_status();
}

size_t cce_forward_workspace_bytes(const cce_head *head, int64_t M) {
  if (check_head(head) != CCE_OK || M < 0 || M > MAX_M) return 0;
  return make_plan(head, M).fwd_bytes;
}

size_t cce_backward_workspace_bytes(const cce_head *head, int64_t M) {
  if (check_head(head) != CCE_OK || M < 0 || M > MAX_M) return 0;
  return make_plan(head, M).bwd_bytes;
}

cce_status cce_forward(const cce_head *head, const void *h, int64_t M, const int32_t *targets,
                       const uint8_t *mask, float *logp, float *lse, void *workspace,
                       size_t workspace_bytes, void *stream) {
  return cce_forward_ex(head, h, M, targets, mask, logp, lse, nullptr, workspace, workspace_bytes, stream);
}

cce_status cce_forward_ex(const cce_head *head, const void *h, int64_t M, const int32_t *targets,
                          const uint8_t *mask, float *logp, float *lse, float *block_max, void *workspace,
                          size_t workspace_bytes, void *stream) {
  cce_status s = check_common(head, h, M, targets, workspace);
  if (s != CCE_OK || M == 0) return s;
  return run_forward(head, h, M, targets, mask, logp, lse, block_max, workspace, workspace_bytes, stream);
}

cce_status cce_backward(const cce_head *head, const void *h, int64_t M, const int32_t *targets,
                        const uint8_t *mask, const float *lse, const float *g, float *dh,
                        void *workspace, size_t workspace_bytes, void *stream) {
  return cce_backward_ex(head, h, M, targets, mask, lse, g, nullptr, nullptr, dh, CCE_DH_F32, workspace,
                         workspace_bytes, stream);
}

cce_status cce_backward_ex(const cce_head *head, const void *h, int64_t M, const int32_t *targets,
                           const uint8_t *mask, const float *lse, const float *g, const float *block_max,
                           const cce_skip *skip, void *dh, int32_t dh_dtype, void *workspace,
                           size_t workspace_bytes, void *stream) {
  cce_status s = check_common(head, h, M, targets, workspace);
  if (s != CCE_OK || M == 0) return s;
  return run_backward(head, h, M, targets, mask, lse, g, block_max, skip, dh, dh_dtype, nullptr, workspace,
                      workspace_bytes, stream);
}

cce_status cce_forward_static(const cce_head *head, const void *h, int64_t M, const int32_t *targets,
                              const uint8_t *mask, float *logp, float *lse, void *stream) {
  cce_status s = check_common(head, h, M, targets, nullptr);
  if (s != CCE_OK || M == 0) return s;
  if (make_plan(head, M).fwd_bytes > CCE_STATIC_SCRATCH_BYTES) return CCE_ERR_WORKSPACE;
  void *ws = scratch_ptr();
  if (!ws) {
    if (!g_err[0]) std::snprintf(g_err, sizeof g_err, "HIP error: no device address for the static scratch");
    return CCE_ERR_HIP;
  }
  return run_forward(head, h, M, targets, mask, logp, lse, nullptr, ws, CCE_STATIC_SCRATCH_BYTES, stream);
}

size_t cce_forward_backward_workspace_bytes(const cce_head *head, int64_t M) {
  if (check_head(head) != CCE_OK || M < 0 || M > MAX_M) return 0;
  return fwdbwd_bytes(make_plan(head, M));
}

cce_status cce_forward_backward(const cce_head *head, const void *h, int64_t M, const int32_t *targets,
                                const uint8_t *mask, const float *g, float *logp, float *lse, void *dh,
                                int32_t dh_dtype, void *workspace, size_t workspace_bytes, void *stream) {
  cce_status s = check_common(head, h, M, targets, workspace);
  if (s != CCE_OK || M == 0) return s;
  if (!logp || !lse || ((uintptr_t)logp & 3) || ((uintptr_t)lse & 3)) return CCE_ERR_INVALID_ARG;
  if (dh_dtype != CCE_DH_F32 && dh_dtype != CCE_DH_BF16) return CCE_ERR_INVALID_ARG;
  if (!dh || ((uintptr_t)dh & (dh_dtype == CCE_DH_F32 ? 3 : 1)) || ((uintptr_t)g & 3)) return CCE_ERR_INVALID_ARG;
  const Plan p = make_plan(head, M);
  if (!workspace || workspace_bytes < fwdbwd_bytes(p)) return CCE_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  if (p.fused) return run_fused(p, head, h, M, targets, mask, g, logp, lse, dh, dh_dtype, workspace, st);
  if (p.ncfused) return run_nc_fused(p, head, h, M, targets, mask, g, logp, lse, dh, dh_dtype, workspace, st);
  return run_twopass(p, head, h, M, targets, mask, g, logp, lse, dh, dh_dtype, workspace, st);
}

size_t cce_dense_forward_workspace_bytes(const cce_dense_head *head, int64_t M) {
  cce_head q;
  if (check_dense(head, q) != CCE_OK || M < 0 || M > MAX_M) return 0;
  return make_plan(&q, M).fwd_bytes;
}

size_t cce_dense_backward_workspace_bytes(const cce_dense_head *head, int64_t M) {
  cce_head q;
  if (check_dense(head, q) != CCE_OK || M < 0 || M > MAX_M) return 0;
  return make_plan(&q, M).bwd_bytes;
}

cce_status cce_dense_forward(const cce_dense_head *head, const void *h, int64_t M, const int32_t *targets,
                             const uint8_t *mask, float *logp, float *lse, void *workspace, size_t workspace_bytes,
                             void *stream) {
  cce_head q;
  cce_status s = check_dense(head, q);
  if (s == CCE_OK) s = check_tokens(h, M, targets, workspace);
  if (s != CCE_OK || M == 0) return s;
  return run_forward(&q, h, M, targets, mask, logp, lse, nullptr, workspace, workspace_bytes, stream);
}

cce_status cce_dense_backward(const cce_dense_head *head, const void *h, int64_t M, const int32_t *targets,
                              const uint8_t *mask, const float *lse, const float *g, float *dh, float *dw,
                              void *workspace, size_t workspace_bytes, void *stream) {
  cce_head q;
  cce_status s = check_dense(head, q);
  if (s == CCE_OK) s = check_tokens(h, M, targets, workspace);
  if (s != CCE_OK || M == 0) return s;
  return run_backward(&q, h, M, targets, mask, lse, g, nullptr, nullptr, dh, CCE_DH_F32, dw, workspace,
                      workspace_bytes, stream);
}

size_t cce_dense_forward_backward_workspace_bytes(const cce_dense_head *head, int64_t M) {
  cce_head q;
  if (check_dense(head, q) != CCE_OK || M < 0 || M > MAX_M) return 0;
  const Plan p = make_plan(&q, M);
  return p.dfused ? p.df_bytes : std::max(p.fwd_bytes, p.bwd_bytes);
}

cce_status cce_dense_forward_backward(const cce_dense_head *head, const void *h, int64_t M, const int32_t *targets,
                                      const uint8_t *mask, const float *g, float *logp, float *lse, float *dh,
                                      float *dw, void *workspace, size_t workspace_bytes, void *stream) {
  cce_head q;
  cce_status s = check_dense(head, q);
  if (s == CCE_OK) s = check_tokens(h, M, targets, workspace);
  if (s != CCE_OK || M == 0) return s;
  if (!logp || !lse || !dh || ((uintptr_t)logp & 3) || ((uintptr_t)lse & 3) || ((uintptr_t)dh & 3) ||
      ((uintptr_t)g & 3) || ((uintptr_t)dw & 3))
    return CCE_ERR_INVALID_ARG;
  const Plan p = make_plan(&q, M);
  if (dw && p.M_pad > MAX_DW_M_PAD) return CCE_ERR_UNSUPPORTED;
  if (!p.dfused) {  // no fixed reference: the forward, then the backward on the same workspace
    s = run_forward(&q, h, M, targets, mask, logp, lse, nullptr, workspace, workspace_bytes, stream);
    if (s != CCE_OK) return s;
    return run_backward(&q, h, M, targets, mask, lse, g, nullptr, nullptr, dh, CCE_DH_F32, dw, workspace,
                        workspace_bytes, stream);
  }
  if (!workspace || workspace_bytes < p.df_bytes) return CCE_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  return run_dense_fused(p, &q, h, M, targets, mask, g, logp, lse, dh, dw, workspace, st);
}

int cce_profile_enable(int on) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  const int prev = g_prof_on;
  g_prof_on = on ? 1 : 0;
  return prev;
}

int cce_profile_read(cce_kernel_time *out, int max) {
  std::vector<ProfRec> recs;
  {
    std::lock_guard<std::mutex> g(g_prof_mu);
    recs.swap(g_prof);
  }
  int n = 0, rc = 0;
  for (const ProfRec &r : recs) {
    float ms = 0.0f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) rc = -1;
    int i = 0;
    while (i < n && std::strncmp(out[i].name, r.name, sizeof out[i].name) != 0) ++i;
    if (i == n && n < max && out) {
      std::memset(&out[n], 0, sizeof out[n]);
      std::strncpy(out[n].name, r.name, sizeof out[n].name - 1);
      ++n;
    }
    if (i < n) {
      out[i].launches += 1;
      out[i].total_ms += ms;
    }
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  return rc < 0 ? -1 : n;
}

}  // extern "C"
