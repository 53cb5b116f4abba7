// hcgr_internal.h -- plan and kernel-launch interface shared by the C ABI
// (hcgr_api.hip) and the kernels (hcgr_kernels.hip). Not installed.
//
// Identity used by every down/inject kernel: rrms is a per-stream scalar and
// k is stream-major, so  xn . W^T = sum_s rrms[s] * P_s  with
// P_s = sum_{c in stream s} R2[s,c]*(1+Wnorm) * W[., s*HS+c]. A workgroup can
// contract a stretch of one stream before that stream's RMS is known and
// scale the partial once the stream's sum of squares is complete.
//
// Four plans, chosen by the token count M (make_plan):
//   SPLIT  (decode sizes). Weight streaming over every CU:
//     K1  hcgr_k1_dec     COMBINE + sums of squares + unscaled partials P for a
//                         (token tile, K chunk inside one stream, row tile)
//     K1r hcgr_k1_reduce  sums the chunk partials per stream, forms rrms,
//                         scales, SiLU(./HC) -> h (workspace), inj_next
//     K2  hcgr_k2_dec     up contraction on MFMA tiles whose 16 rows are
//                         4 channels x 4 streams, Wu rows and h staged in LDS by
//                         direct global->LDS loads; sigmoid + MIX in registers
//   TILE (large sizes). Activation streaming with LDS-staged weights:
//     K1  hcgr_k1_tile    a workgroup owns 64 tokens and every down/inject
//                         row (or a row split); weights, R and y arrive in
//                         LDS by direct global->LDS loads, 2-3 stages deep;
//                         four streams per workgroup (h and inj_next out) or
//                         one (rrms_s * P_s out, summed by hcgr_k1_sum)
//     K2  hcgr_k2_stage   as below
//   STREAM (mid sizes) and FULL. Activation streaming:
//     K1  hcgr_k1_full    a workgroup owns a token tile and every down/inject
//                         row (or a row split) and runs over one stream
//                         (STREAM) or all four (FULL) with two accumulator
//                         sets: the current stream's partial and the
//                         rrms-scaled total. FULL writes h and inj_next
//                         directly; STREAM writes rrms_s * P_s per stream
//     K1s hcgr_k1_sum     (STREAM only) sums the four scaled partials,
//                         SiLU(./HC) -> h, inj_next
//     K2  hcgr_k2_stage   h . Wu^T on MFMA for 128 tokens x 32 channels with
//                         h and Wu staged through LDS by direct global->LDS
//                         loads, R2 and rrms in registers, and the sigmoid +
//                         MIX epilogue in registers
//   Stream counts other than 4 (HC = 1, 2, 8) take the SPLIT plan at decode
//   sizes with the reduction over HC streams and the decode up kernel
//   hcgr_k2_decg (16/HC channels x HC streams per MFMA block), then the TILE
//   plan with one stream per down workgroup, hcgr_k1_sum over the HC stream
//   partials, and K2 hcgr_k2_gen: 64 tokens x 32 channels x HC streams, one
//   16-row MFMA block per stream so that MIX stays lane-local.
//   FUSED and PERSISTENT (decode sizes, any HC; tuned-table choices): see
//   make_fused.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <climits>

namespace hcgr {

enum PlanKind { PLAN_SPLIT = 0, PLAN_STREAM = 1, PLAN_FULL = 2, PLAN_TILE = 3, PLAN_FUSED = 4, PLAN_PERSIST = 5 };

// Arrival counters. The first kCtrBytes of every workspace hold kCtrSlots
// 32-bit counters (one per 128-byte line) that the fused and persistent
// decode plans' workgroups increment; every plan keeps
// its data past them, a counter is reset to zero by the workgroup that sees
// its last arrival, so a workspace zeroed once before its first use stays
// zero there after every completed call.
constexpr int kCtrSlots = 1024, kCtrStride = 32;  // counters; words from one counter to the next
constexpr size_t kCtrBytes = (size_t)kCtrSlots * kCtrStride * 4;  // 128 KiB

// SPLIT-plan down kernel variants: token tile, 16-row blocks per workgroup,
// waves splitting each block's k range, columns per chunk.
enum KDVariant {
  KD_T16_R7_K1_C128 = 0, KD_T16_R1_K4_C512, KD_T16_R3_K1_C256, KD_T16_R3_K2_C512,
  KD_T32_R7_K1_C128, KD_T32_R1_K4_C512, KD_T32_R3_K1_C256, KD_T32_R3_K2_C512,
  KD_T64_R7_K1_C128, KD_T64_R3_K1_C256, KD_T128_R7_K1_C128, KD_T16_R4_K2_C512, KD_T32_R4_K2_C512, KD_NVAR
};
struct KDShape { int tm, rb, kw, kc; };
inline KDShape kd_shape(int v) {
  static const KDShape t[KD_NVAR] = {{16, 7, 1, 128}, {16, 1, 4, 512}, {16, 3, 1, 256}, {16, 3, 2, 512},
                                     {32, 7, 1, 128}, {32, 1, 4, 512}, {32, 3, 1, 256}, {32, 3, 2, 512},
                                     {64, 7, 1, 128}, {64, 3, 1, 256}, {128, 7, 1, 128}, {16, 4, 2, 512},
                                     {32, 4, 2, 512}};
  return t[v];
}
// SPLIT-plan up kernel variants (HC = 4): token tile; the workgroup's
// channels come from the stream width (dec_up_channels), a wave per 4.
enum K2Variant { K2_T16 = 0, K2_T32 = 1, K2_T64S = 2, K2_NVAR };
struct K2Shape { int tm; };
inline K2Shape k2_shape(int v) {
  static const K2Shape t[K2_NVAR] = {{16}, {32}, {64}};
  return t[v];
}
// Dynamic LDS of the SPLIT-plan up kernel for a token tile of tm, rank r and
// cw channels: the workgroup's Wu rows (4 per channel, whole waves of 16) and
// the h tile, the tile's R2 rows of its channels (whole KB), rrms and Wnorm;
// it must fit the 160 KB of one CU.
inline size_t k2_dec_lds(int tm, int r, int cw) {
  return (size_t)((cw + 3) / 4 * 16 + tm) * (size_t)r * 2u + ((size_t)tm * 4 * cw * 2u + 1023) / 1024 * 1024 +
         (size_t)(tm > 64 ? tm : 64) * 16 + 1024;
}
constexpr size_t kLdsPerCu = 160 * 1024;
// Channels per workgroup of the HC = 4 decode up kernel for M tokens in
// tiles of tm (rank r): 10 where HS is a multiple of 2560 (HS / 10
// workgroups per token tile fill whole rounds of the 256 CUs) unless they
// need more rounds than 16 channels, a round being the workgroups that fit
// the CUs' LDS at once; else 16. Measured on MI355X at HS = 2560, r = 320
// (up kernel): 10 channels take 0.12 us off at M = 32 and 0.45 at M = 48
// and 64; with 64-token tiles (two per CU for 10 channels, one for 16) 6.8
// at M = 128 (two tiles), 10.5-10.8 against 11.6-11.9 us at M = 160-192
// (three) and 11.9-12.3 against 16.7-17.1 at M = 224-256 (four); with
// 32-token tiles (two per CU either way) level at four tiles and 1.6-2.7
// us slower at three and from five, where 10 channels need a further round.
inline int dec_up_channels(int hs, int64_t M, int tm, int r) {
  if (hs % 2560 != 0) return 16;
  const int64_t tiles = (M + tm - 1) / tm;
  auto rounds = [&](int cw) {
    const int64_t fit = (int64_t)(kLdsPerCu / k2_dec_lds(tm, r, cw));
    const int64_t slots = 256 * (fit > 1 ? fit : 1);
    return ((int64_t)(hs / cw) * tiles + slots - 1) / slots;
  };
  return rounds(10) <= rounds(16) ? 10 : 16;
}
// Decode up kernel for HC streams: a wave's 16 MFMA rows are 16/HC channels x
// HC streams; NW waves per workgroup (HC waves up to 4 in the split and fused
// plans' up kernel, 4 in the persistent plan). At HC = 8, when HS is a
// multiple of 2560, five waves (10 channels): HS/10 workgroups fill whole
// rounds of the 256 CUs, where eight channels (HS/8 = 320 at HS = 2560) left
// 64 CUs with two workgroups' Wu rows.
inline int decg_waves(int hc, int hs) { return hc < 4 ? hc : (hc == 8 && hs % 2560 == 0) ? 5 : 4; }
inline int decg_channels(int hc, int nw) { return nw * (16 / hc); }
// Its LDS: Wu rows and the h tile, then the tile's R2 rows of its channels,
// rrms and Wnorm (each rounded up to whole 1 KB direct-load instructions) and
// a flag word.
inline size_t k2_decg_lds(int hc, int tm, int r, int nw) {
  const size_t cw = (size_t)decg_channels(hc, nw);
  auto kb = [](size_t b) { return (b + 1023) / 1024 * 1024; };
  return (size_t)(nw * 16 + tm) * (size_t)r * 2u + kb((size_t)tm * hc * cw * 2) + kb((size_t)tm * hc * 4) +
         kb((size_t)hc * cw * 2) + 16;
}
// The reduction kernel gives each of a wave's 4 lane groups up to kRedMaxCpl
// chunks per stream (instantiated: 1, 2, 3, 5, 8).
constexpr int kRedMaxCpl = 8;
inline int red_cpl(int kcps) {
  const int need = (kcps + 3) / 4;
  return need <= 1 ? 1 : need <= 2 ? 2 : need <= 3 ? 3 : need <= 5 ? 5 : 8;
}

// STREAM/FULL down kernel variants: token tile, waves, row blocks per wave,
// k per LDS stage. 8 waves x 3 blocks cover 24 16-row blocks per workgroup.
enum KFVariant { KF_T32 = 0, KF_T64 = 1, KF_NVAR };
struct KFShape { int tm, nw, bpw, ks; };
inline KFShape kf_shape(int v) {
  static const KFShape t[KF_NVAR] = {{32, 8, 3, 128}, {64, 8, 3, 64}};
  return t[v];
}
// Tiled up kernel variants: token tile, channel tile (x 4 streams).
// KT_S128: hcgr_k2_stage (operands staged by direct global->LDS loads);
// KT_SWEEP: hcgr_k2_sweep (h of a 128-token tile held in registers while the
// workgroup sweeps a range of 32-channel groups).
// KT_GEN: hcgr_k2_gen, for stream counts other than 4 (64 tokens x 32
// channels x HC streams per workgroup).
// KT_GEN128: hcgr_k2_gen over 128-token tiles (HC = 2 or 8: each Wu row read
// once per 128 tokens instead of 64).
// KT_SWEEP2: hcgr_k2_sweep2 (hcgr_sweep.hip), the sweep over 256-token tiles:
// each wave owns 32 tokens and every gate row; Wu streams in 16-row blocks
// over the whole of k (fetched once per 256 tokens), and each block's
// sigmoid + MIX runs beside the next block's products.
constexpr int kSweep2Tm = 256;
enum KTVariant { KT_S128 = 0, KT_SWEEP = 1, KT_GEN = 2, KT_GEN128 = 3, KT_SWEEP2 = 4, KT_NVAR };
struct KTShape { int tm, cb; };
inline KTShape kt_shape(int v) {
  static const KTShape t[KT_NVAR] = {{128, 32}, {128, 32}, {64, 32}, {128, 32}, {kSweep2Tm, 32}};
  return t[v];
}
inline bool is_sweep(int kt) { return kt == KT_SWEEP || kt == KT_SWEEP2; }
inline bool is_gen(int kt) { return kt == KT_GEN || kt == KT_GEN128; }
// hcgr_k2_sweep serves 96 <= r <= 320 (2 to 5 k stages of 64) from
// kSweepMinM tokens, with enough channel ranges per token tile to give
// every CU a workgroup.
constexpr int64_t kSweepMinM = 4096;
inline int sweep_nks(int r) { return (r + 63) / 64; }
inline bool sweep_fits(int r) { return r >= 96 && r <= 320; }

struct Shape {
  int hc, hs, r;
  float eps;
  bool wn_full;
  bool merged;
  int n_pad;
  int64_t k() const { return (int64_t)hc * hs; }
  int n_rows() const { return r + hc; }             // down rows + inject rows
  int nblk() const { return (n_rows() + 15) / 16; } // 16-row MFMA blocks
  int np() const { return nblk() * 16; }
};

// hcgr_k2_sweep2 channel ranges hold whole pairs of 32-channel groups (at
// most one range per pair). LDS: a ring of kSweep2Ring Wu stages (4 blocks of
// 16 rows x NC chunks of 64 k, 2 KB per chunk) and 0.25 (1 + Wnorm) of a
// channel range as f32 (four per channel for a full-width Wnorm).
constexpr int kSweep2Ring = 3;
inline int sweep2_pairs(const Shape& s) { return s.hs / 64; }
inline constexpr size_t sweep2_stage_bytes(int nc) { return (size_t)4 * nc * 2048; }
inline size_t sweep2_lds(const Shape& s, int nranges) {
  const int np = sweep2_pairs(s), gmax = 2 * ((np + nranges - 1) / nranges);
  return kSweep2Ring * sweep2_stage_bytes(sweep_nks(s.r)) + (size_t)gmax * 32 * (s.wn_full ? 16 : 4);
}

struct Plan {
  int64_t M = 0, mpad = 0;
  int kind = PLAN_SPLIT;
  // SPLIT
  int tm = 0;
  int k1 = 0, k2 = 0;
  int kc = 0, nkc = 0, kcps = 0;   // k per chunk, chunk count, chunks per stream
  int ntiles_n = 0;                // K1 n tiles
  int cb = 0;                      // K2 channels per workgroup
  // STREAM / FULL
  int kf = 0, kt = 0;              // variants
  int spw = 4;                     // streams per down workgroup (4 or 1)
  int nsplit = 1;                  // row-block splits of the down rows
  int nseg = 1;                    // column segments per stream (TILE, one stream per workgroup)
  int64_t mq = 0;                  // rows of the per-stream partials (STREAM)
  int nranges = 1;                 // channel-group ranges per token tile (hcgr_k2_sweep)
  int xgroup = 0;                  // TILE: the down workgroups of a token tile share an XCD
  // FUSED: chunks per stream (kcps), chunk count (nkc), token tiles, up-kernel waves
  int ntiles = 0, upw = 0;
  size_t off_p = 0, off_ss = 0, off_h = 0, off_q = 0, ws_bytes = 0;
};

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Largest M the heuristic serves with the SPLIT plan, for any shape.
constexpr int64_t kSplitMaxM = 256;
// The split plan's cost grows with M (chunk partials, weights re-read per
// 32-token tile) while the tile plan's stays nearly flat up to a few hundred
// tokens, so the crossover falls as the weights grow: the heuristic takes the
// split plan while M times the down weight's elements (K x padded rows) stays
// under 6.5e8, between 64 and kSplitMaxM tokens (measured on MI355X, HC = 4:
// crossover near 190 tokens at HS, r = 2560, 320, near 145 at 4096, 256,
// beyond 256 at 1536, 192; at 7168, 512 the tile plan was 35% faster
// already at 144 tokens).
inline int64_t split_max(int64_t k, int np) {
  const int64_t m = (int64_t)(6.5e8 / ((double)k * (double)np));
  return m < 64 ? 64 : m > kSplitMaxM ? kSplitMaxM : m;
}
// TILE plan: 64-token down kernel (hcgr_k1_tile) with at most 22 16-row
// blocks per workgroup (4 row quarters of at most 6); taken from kTileMinM
// tokens: one stream per workgroup (split into column segments while that
// leaves the chip short of workgroups), all four once the token tiles alone
// fill it.
constexpr int64_t kTileTm = 64;
constexpr int kTileMaxBlk = 22;
constexpr int64_t kTileMinM = 65;

// SPLIT plan with down-kernel variant kd; false when the stream width does
// not split into chunks of the variant (the caller then takes another plan).
inline bool make_split(const Shape& s, int64_t M, int kd, Plan* out) {
  const KDShape d = kd_shape(kd);
  // the up kernel's token tile: the down kernel's, except 32 under 128-token
  // down tiles (measured on MI355X at M = 128: the 128-token up tile, one
  // workgroup per CU for its LDS, is 1 us slower than four 32-token ones,
  // while the 128-token down tile is 1.2 us faster than four 32-token ones)
  const int k2 = d.tm == 16 ? K2_T16 : d.tm == 64 ? K2_T64S : K2_T32;
  const int tm2 = k2_shape(k2).tm;
  const int cw2 = s.hc == 4 ? dec_up_channels(s.hs, M, tm2, s.r) : decg_channels(s.hc, decg_waves(s.hc, s.hs));
  const size_t lds2 = s.hc == 4 ? k2_dec_lds(tm2, s.r, cw2) : k2_decg_lds(s.hc, tm2, s.r, decg_waves(s.hc, s.hs));
  if (s.hs % d.kc != 0 || s.hs / d.kc > 4 * kRedMaxCpl || lds2 > kLdsPerCu) return false;
  Plan p;
  p.M = M;
  p.kind = PLAN_SPLIT;
  p.k1 = kd;
  p.k2 = k2;
  p.tm = d.tm;
  p.kc = d.kc;
  p.kcps = s.hs / d.kc;
  p.nkc = s.hc * p.kcps;
  p.ntiles_n = (s.nblk() + d.rb - 1) / d.rb;
  p.cb = cw2;  // up-kernel channels per workgroup
  p.mpad = (M + p.tm - 1) / p.tm * p.tm;
  const size_t np = (size_t)s.np();
  p.off_p = kCtrBytes;
  p.off_ss = align256(p.off_p + (size_t)p.nkc * np * (size_t)p.mpad * sizeof(float));
  p.off_h = align256(p.off_ss + (size_t)p.nkc * (size_t)p.mpad * sizeof(float));
  p.ws_bytes = align256(p.off_h + (size_t)p.mpad * (size_t)s.r * sizeof(uint16_t));
  *out = p;
  return true;
}

// FUSED plan (decode sizes, any stream count): two kernels.
//   K1  hcgr_k1_fuse    a workgroup owns one 16-row block of the down/inject
//                       rows and one K chunk inside one stream (HS split into
//                       kcps chunks of whole 128-column units) for a token
//                       tile; weights, R, y and Wnorm arrive in LDS by direct
//                       global->LDS loads; COMBINE, the chunk's sums of squares
//                       and its unscaled partial product go to the workspace,
//                       and the last workgroup to arrive at the block's
//                       counter sums the block's chunks per stream, forms
//                       rrms and writes h, inj_next and rrms
//   K2  hcgr_k2_decg    the decode up kernel for HC streams (below)
// kFuseUmax: widest chunk in 128-column units (the LDS holds R, y and the
// weight rows of one chunk for 32 tokens).
constexpr int kFuseUmax = 7;
constexpr int kFuseTarget = 256;  // workgroups per token tile the chunk count aims at
inline size_t k1_fuse_lds(int tm) {
  const size_t row = (size_t)kFuseUmax * 128 * 2;  // bytes of one chunk row
  return (size_t)(2 * tm + 16) * row + 2048 + (size_t)tm * 12;  // R, y, weights, Wnorm slot, iw and sums
}

// Counter slots of the decode plans (slot i at word i * kCtrStride: every
// counter starts a 128-byte line of its own, since agent-scope atomics on
// one line are serialised; measured on MI355X, 1680 arrivals on 21 counters
// of one line took 13.7 us, on 21 lines of their own 0.5 us): block
// counters [0, 512), then the persistent plan's per-tile "h complete"
// counters [512, 640), its per-tile ready flags [640, 768) that the arrival
// completing a tile's count raises and the up role polls, its per-tile exit
// counters [768, 1023) and the slot kErrSlot that a persistent wait which
// gave up sets to 1.
constexpr int kHdoneSlot = 512, kReadySlot = 640, kExitSlot = 768, kErrSlot = kCtrSlots - 1;

// FUSED plan (persist = false) or PERSISTENT plan (persist = true) with tm
// tokens per tile (16 or 32); false when the shape does not fit their limits
// (counters, LDS, chunk count).
inline bool make_fused(const Shape& s, int64_t M, int tm, Plan* out, bool persist = false) {
  if (M <= 0 || (tm != 16 && tm != 32)) return false;
  const int U = s.hs / 128, nblk = s.nblk();
  // chunks per stream: about kFuseTarget workgroups per token tile, at most
  // 4*kFuseUmax chunks in all (the last arriver stages the block's partials
  // in the y area of its LDS), at least enough that none is wider than
  // kFuseUmax units
  int kcps = kFuseTarget / (nblk * s.hc);
  if (kcps > 4 * kFuseUmax / s.hc) kcps = 4 * kFuseUmax / s.hc;
  const int kmin = (U + kFuseUmax - 1) / kFuseUmax;
  if (kcps < kmin) kcps = kmin;
  if (kcps > U) kcps = U;
  const int nkc = s.hc * kcps;
  const int64_t ntiles = cdiv(M, (int64_t)tm);
  if (nkc > 4 * kFuseUmax || ntiles * nblk > kHdoneSlot) return false;
  if (k1_fuse_lds(tm) > kLdsPerCu) return false;
  if (persist) {
    if (ntiles > kExitSlot - kReadySlot || k2_decg_lds(s.hc, tm, s.r, 4) > kLdsPerCu) return false;
  } else if (k2_decg_lds(s.hc, tm, s.r, decg_waves(s.hc, s.hs)) > kLdsPerCu) {
    return false;
  }
  Plan p;
  p.M = M;
  p.kind = persist ? PLAN_PERSIST : PLAN_FUSED;
  p.tm = tm;
  p.kcps = kcps;
  p.nkc = nkc;
  p.ntiles = (int)ntiles;
  p.upw = persist ? 4 : decg_waves(s.hc, s.hs);
  p.cb = decg_channels(s.hc, p.upw);
  p.mpad = ntiles * tm;
  p.off_p = kCtrBytes;
  p.off_ss = align256(p.off_p + (size_t)ntiles * nblk * nkc * tm * 16 * sizeof(float));
  p.off_h = align256(p.off_ss + (size_t)ntiles * nblk * nkc * tm * sizeof(float));
  p.ws_bytes = align256(p.off_h + (size_t)p.mpad * (size_t)s.r * sizeof(uint16_t));
  *out = p;
  return true;
}
// Largest M the heuristic serves with the FUSED plan.
constexpr int64_t kFusedMaxM = 32;

// TILE plan with explicit parameters: spw streams per down workgroup (1, or 4
// with HC = 4), nseg column segments per stream (spw = 1; divides HS/128),
// up-kernel variant kt (KT_GEN exactly when HC != 4; KT_SWEEP needs
// 96 <= r <= 320) and nranges channel ranges per token tile (KT_SWEEP only,
// 1 .. HS/32) and tm tokens per down tile (64, or 128 with spw = 1). False
// when the parameters cannot run this shape.
inline bool make_tile(const Shape& s, int64_t M, int spw, int nseg, int kt, int nranges, Plan* out,
                      int tm = (int)kTileTm) {
  const bool generic = s.hc != 4;
  if (M <= 0) return false;
  if (tm != 64 && !(tm == 128 && spw == 1)) return false;
  if (spw != 1 && !(spw == 4 && !generic)) return false;
  if (nseg < 1 || (s.hs / 128) % nseg != 0 || (spw == 4 && nseg != 1)) return false;
  if (generic != is_gen(kt) || (kt == KT_GEN128 && s.hc != 2 && s.hc != 8)) return false;
  if (is_sweep(kt)) {
    if (!sweep_fits(s.r) || nranges < 1 || nranges > s.hs / kt_shape(kt).cb) return false;
    if (kt == KT_SWEEP2 && (nranges > sweep2_pairs(s) || sweep2_lds(s, nranges) > kLdsPerCu)) return false;
  } else if (kt != KT_S128 && !is_gen(kt)) {
    return false;
  } else if (nranges != 1) {
    return false;
  }
  const size_t np = (size_t)s.np();
  Plan p;
  p.M = M;
  p.kind = PLAN_TILE;
  p.spw = spw;
  p.nsplit = (int)cdiv(s.nblk(), kTileMaxBlk);  // row splits of the tile down kernel
  p.nseg = nseg;
  p.kt = kt;
  p.nranges = nranges;
  p.tm = tm;
  // 128-token tiles: a tile's down workgroups share an XCD, so y and R come
  // from HBM once per tile (measured 1-2% faster in the down kernel from
  // 4096 tokens on MI355X, bit-identical results)
  p.xgroup = tm == 128 ? 1 : 0;
  const int tm2 = kt_shape(kt).tm;
  p.mpad = cdiv(M, tm2) * tm2;
  p.mq = cdiv(M, (int64_t)tm) * tm;
  p.off_h = kCtrBytes;
  p.off_q = align256(p.off_h + (size_t)p.mpad * (size_t)s.r * sizeof(uint16_t));
  p.ws_bytes = p.off_q;
  if (spw == 1) {
    const size_t parts = (size_t)s.hc * (size_t)nseg;
    p.off_ss = align256(p.off_q + parts * (size_t)p.mq * np * sizeof(float));
    p.ws_bytes = align256(p.off_ss + parts * (size_t)p.mq * sizeof(float));
  }
  *out = p;
  return true;
}

// Pure host planning: tile sizes and split counts by token count M.
inline Plan make_plan(const Shape& s, int64_t M) {
  Plan p;
  p.M = M;
  if (M <= 0) return p;
  const int hs = s.hs;
  const size_t np = (size_t)s.np();
  // stream counts other than 4 (1, 2 or 8) take the split plan with the
  // stream-generic reduction and decode up kernel up to the split limit, then
  // the tile plan: one stream per down workgroup, the stream sum, hcgr_k2_gen
  const bool generic = s.hc != 4;
  if (M <= split_max(s.k(), s.np()) && generic) {
    // down-kernel variant by K, measured on MI355X at HS, r = 2560, 320 (cold
    // buffers): up to 40 128-column chunks (HC = 1, 2) 16-token tiles of
    // 7-row blocks up to 64 tokens (HC = 1: 10.8-12.0 us at M = 1..64, against
    // 11.8-14.6 for the fused plan and 23.6 for the tile plan at 64; HC = 2:
    // 11.8-14.4 us), then 32-token tiles (13.9 and 17.2 us at 128); from 160
    // chunks (HC = 8) 512-column chunks in 4-row blocks with two k waves,
    // 16-token tiles up to 16 tokens: 6 row tiles x 40 chunks = 240
    // workgroups on the 256 CUs, where 3-row blocks (7 x 40 = 280) left 24
    // CUs with two (16.6 against 17.9-18.2 us at M = 8, 16.8 against 18.2 at
    // 16, 19.6 against 21.5 at 32 and 24.9 against 27.4 at 64; one row block
    // with four k waves, 840 workgroups: 18.2 at M = 8)
    const int64_t c128 = s.k() / 128;
    int kd;
    if (c128 <= 40) kd = M <= 64 ? KD_T16_R7_K1_C128 : KD_T32_R7_K1_C128;
    else if (c128 >= 160) kd = M <= 16 ? KD_T16_R4_K2_C512 : KD_T32_R4_K2_C512;
    else kd = M <= 16 ? KD_T16_R7_K1_C128 : KD_T32_R7_K1_C128;
    if (make_split(s, M, kd, &p) || make_split(s, M, M <= 16 ? KD_T16_R3_K2_C512 : KD_T32_R3_K2_C512, &p)) return p;
  }
  if (M <= split_max(s.k(), s.np()) && !generic) {
    // above 16 tokens: 32-token down tiles (they pad M to 32, not 64); at
    // every M, 3-row blocks where those leave fewer padded 16-row blocks than
    // 7-row ones (measured on MI355X at M = 40..128 over HS, r = 1536, 192;
    // 2560, 320; 4096, 256 and 7168, 512: within 4% of the fastest split
    // variant except HS = 7168 from 112 tokens, 5%; 64-token tiles were up
    // to 30% slower at M = 80..96. At M = 1..32 and HS, r = 4096, 256 the
    // 3-row blocks were 13-17% faster than 7-row ones)
    const int nb = s.nblk();
    const bool rb3 = cdiv(nb, 3) * 3 - nb < cdiv(nb, 7) * 7 - nb;
    const int kd = M <= 16 ? (rb3 ? KD_T16_R3_K2_C512 : KD_T16_R7_K1_C128)
                 : M <= 32 ? (rb3 ? KD_T32_R3_K2_C512 : KD_T32_R7_K1_C128)
                 : rb3 ? KD_T32_R3_K1_C256 : KD_T32_R7_K1_C128;
    const int kd_wide = M <= 16 ? KD_T16_R3_K2_C512 : KD_T32_R3_K2_C512;
    if (make_split(s, M, kd, &p) || make_split(s, M, kd_wide, &p)) return p;
  }
  // STREAM / FULL / TILE: aim for at least one down workgroup per CU (256 CUs)
  const int64_t target = 256;
  const int64_t tiles = cdiv(M, kTileTm);
  const int tsplit = (int)cdiv(s.nblk(), kTileMaxBlk);  // row splits of the tile down kernel
  if (M >= kTileMinM || generic) {
    int kt = generic ? KT_GEN : KT_S128, nranges = 1;
    // two streams from 1024 tokens: the 128-token generic up tile (measured on
    // MI355X at HS = 2560, r = 320: 4-6% faster up kernel at M = 1024..32768;
    // with eight streams it was 7-18% slower, one workgroup per CU)
    if (generic && s.hc == 2 && M >= 1024) kt = KT_GEN128;
    // from kSweepMinM tokens the 256-token sweep, with enough channel ranges
    // to give every CU a workgroup (measured on MI355X at HS = 2560, r = 320,
    // against the 128-token sweep: 47 vs 91 us at M = 4096, 87 vs 107 at
    // 8192, 174 vs 339 at 16384, 626 vs 800 at 65536); the 128-token sweep
    // where its LDS does not fit (a full-width Wnorm over few ranges)
    if (M >= kSweepMinM && sweep_fits(s.r) && !generic) {
      const int64_t t2 = cdiv(M, (int64_t)kSweep2Tm);
      const int np = sweep2_pairs(s);
      nranges = (int)(t2 >= target ? 1 : cdiv(target, t2) < np ? cdiv(target, t2) : np);
      kt = KT_SWEEP2;
      if (sweep2_lds(s, nranges) > kLdsPerCu) {
        kt = KT_SWEEP;
        const int64_t t1 = cdiv(M, kt_shape(KT_SWEEP).tm);
        const int ng = hs / kt_shape(KT_SWEEP).cb;
        nranges = (int)(t1 >= target ? 1 : cdiv(target, t1) < ng ? cdiv(target, t1) : ng);
      }
    }
    // once 128-token down tiles alone give every CU a workgroup (one stream
    // each), take them: they stream each weight stage once per 128 tokens
    // instead of 64 (measured on MI355X at HS = 2560, r = 320: the down
    // kernel 16% faster at M = 8192, 20% at M = 65536 than 64-token tiles
    // with four streams per workgroup, the stream sum included)
    if (cdiv(M, (int64_t)128) * s.hc * tsplit >= target) {
      make_tile(s, M, 1, 1, kt, nranges, &p, 128);
      return p;
    }
    const int spw = tiles * tsplit >= target && !generic ? 4 : 1;
    // below one workgroup per CU, split each stream's columns into segments
    // (an even number of 64-column stages each); hcgr_k1_sum then forms rrms.
    // The count minimises a cost fitted to measurements on MI355X (HS = 2560,
    // r = 320), in microseconds: per round of workgroups on the CUs, a fixed
    // 8.5 plus 1.3 per stage (the down kernel runs stages in groups of four),
    // and per segment 0.4 + 0.0004 per token for writing and summing the
    // partials. It depends on M only through the token tile count, so every M
    // with the same tile count gets the same plan (the workspace bound below
    // relies on that).
    int nseg = 1;
    if (spw == 1) {
      const int pairs = s.hs / 128;
      const double mt = (double)(tiles * kTileTm);
      double best = 1e300;
      for (int d = 1; d <= pairs; ++d) {
        if (pairs % d != 0) continue;
        const int64_t rounds = cdiv(tiles * s.hc * tsplit * d, target);
        const int64_t nst = cdiv(2 * pairs / d, 4) * 4;
        const double cost = (double)rounds * (8.5 + 1.3 * (double)nst) + (double)d * (0.4 + 0.0004 * mt);
        if (cost < best) { best = cost; nseg = d; }
      }
    }
    make_tile(s, M, spw, nseg, kt, nranges, &p);
    return p;
  }
  const KFShape f64 = kf_shape(KF_T64);
  const int nmin = (int)cdiv(s.nblk(), (int64_t)f64.nw * f64.bpw);  // row splits the blocks need
  if (cdiv(M, 64) * nmin >= target) {
    p.kind = PLAN_FULL; p.kf = KF_T64; p.spw = 4; p.nsplit = nmin;
  } else if (cdiv(M, 32) * nmin >= target) {
    p.kind = PLAN_FULL; p.kf = KF_T32; p.spw = 4; p.nsplit = nmin;
  } else if (cdiv(M, 32) * 2 * nmin >= target) {
    p.kind = PLAN_FULL; p.kf = KF_T32; p.spw = 4; p.nsplit = 2 * nmin;
  } else if ((hs / kf_shape(KF_T32).ks) % 2 == 0) {
    // one stream per workgroup (the down kernel runs its stages in pairs,
    // so a stream must hold an even number of them)
    p.kind = PLAN_STREAM; p.kf = KF_T32; p.spw = 1;
    p.nsplit = nmin;
    while (cdiv(M, 32) * 4 * p.nsplit < target && p.nsplit * 2 <= s.nblk()) p.nsplit *= 2;
  } else {
    p.kind = PLAN_FULL; p.kf = KF_T32; p.spw = 4;
    p.nsplit = nmin;
    while (cdiv(M, 32) * p.nsplit < target && p.nsplit * 2 <= s.nblk()) p.nsplit *= 2;
  }
  p.kt = KT_S128;
  const int tm1 = kf_shape(p.kf).tm, tm2 = kt_shape(p.kt).tm;
  p.tm = tm1;
  p.mpad = cdiv(M, tm2) * tm2;  // h rows the up kernel may read
  p.mq = cdiv(M, tm1) * tm1;
  p.off_h = kCtrBytes;
  p.off_q = align256(p.off_h + (size_t)p.mpad * (size_t)s.r * sizeof(uint16_t));
  p.ws_bytes = p.off_q;
  if (p.kind == PLAN_STREAM) p.ws_bytes = align256(p.off_q + (size_t)s.hc * (size_t)p.mq * np * sizeof(float));
  return p;
}

// Workspace that serves every token count up to M: the largest plan need
// over M' <= M. Plans are piecewise: the decode plans for M' <= kSplitMaxM,
// then tile plans whose partial-sum storage depends on the 64-token tile count
// only (every M' with the same tile count needs what its largest member
// needs) until the 128-token down tiles take over, whose need grows with M'.
// The maximum is therefore taken over M' = 1 .. kSplitMaxM, the multiples of
// 64 up to the 128-token switch, and M itself.
inline size_t workspace_bound(const Shape& s, int64_t M) {
  if (M <= 0) return 0;
  size_t best = make_plan(s, M).ws_bytes;
  for (int64_t m = 1; m <= M && m <= kSplitMaxM; ++m) {
    const size_t b = make_plan(s, m).ws_bytes;
    best = best > b ? best : b;
  }
  const int64_t tsplit = cdiv(s.nblk(), kTileMaxBlk);
  for (int64_t t = 1; t * kTileTm <= M; ++t) {
    const size_t b = make_plan(s, t * kTileTm).ws_bytes;
    best = best > b ? best : b;
    if (cdiv(t * kTileTm, (int64_t)128) * s.hc * tsplit >= 256) break;  // 128-token tiles from here on
  }
  return best;
}

// ---------------------------------------------------------------------------
// Tuned plans. A Choice names a plan family and its parameters; a table of
// (token count, Choice) entries replaces the heuristic near its keys: a token
// count M resolves to the nearest key in log space (ties to the smaller key);
// below the smallest key, for an entry marked heuristic, and wherever the
// entry's choice cannot run the shape at M, make_plan decides.
constexpr int kChoiceHeuristic = -1;
constexpr int64_t kSplitChoiceMaxM = 256;  // a decode-plan choice serves token counts up to this
struct Choice {
  int kind = kChoiceHeuristic;  // kChoiceHeuristic, PLAN_SPLIT, PLAN_TILE, PLAN_FUSED or PLAN_PERSIST
  int kd = 0;                   // PLAN_SPLIT: down-kernel variant; PLAN_TILE: 0 = 64-token, 1 = 128-token down tiles;
                                // PLAN_FUSED, PLAN_PERSIST: 0 = 16-token, 1 = 32-token tiles
  int spw = 1, nseg = 1, kt = KT_S128, nranges = 1;  // PLAN_TILE: as make_tile
};
struct TableEntry {
  int64_t M;
  Choice c;
};

inline bool plan_from_choice(const Shape& s, int64_t M, const Choice& c, Plan* out) {
  if (c.kind == PLAN_SPLIT)
    return M >= 1 && M <= kSplitChoiceMaxM && c.kd >= 0 && c.kd < KD_NVAR && make_split(s, M, c.kd, out);
  if (c.kind == PLAN_TILE)
    return (c.kd == 0 || c.kd == 1) && make_tile(s, M, c.spw, c.nseg, c.kt, c.nranges, out, c.kd ? 128 : 64);
  if (c.kind == PLAN_FUSED || c.kind == PLAN_PERSIST)
    return M >= 1 && M <= kSplitChoiceMaxM && (c.kd == 0 || c.kd == 1) &&
           make_fused(s, M, c.kd ? 32 : 16, out, c.kind == PLAN_PERSIST);
  return false;
}

// Every choice that can run the shape at M (the candidates a tuner times),
// written to out[0 .. min(count, cap)); returns the count.
inline int plan_choices(const Shape& s, int64_t M, Choice* out, int cap) {
  int n = 0;
  auto add = [&](const Choice& c) {
    Plan p;
    if (!plan_from_choice(s, M, c, &p)) return;
    if (n < cap) out[n] = c;
    ++n;
  };
  for (int kd = 0; kd < KD_NVAR; ++kd) {
    Choice c;
    c.kind = PLAN_SPLIT;
    c.kd = kd;
    add(c);
  }
  for (int kind : {(int)PLAN_FUSED, (int)PLAN_PERSIST})
    for (int kd = 0; kd < 2; ++kd) {
      Choice c;
      c.kind = kind;
      c.kd = kd;
      add(c);
    }
  const int ups[5] = {KT_S128, KT_SWEEP, KT_GEN, KT_GEN128, KT_SWEEP2};
  const int pairs = s.hs / 128;
  for (int big = 0; big < 2; ++big)
    for (int spw : {1, 4})
      for (int d = 1; d <= pairs; ++d) {
        if (pairs % d != 0 || (spw == 4 && d != 1)) continue;
        for (int kt : ups)
          for (int nr = 1; nr <= (kt == KT_SWEEP2 ? 32 : kt == KT_SWEEP ? 8 : 1); nr *= 2) {
            Choice c;
            c.kind = PLAN_TILE;
            c.kd = big;
            c.spw = spw;
            c.nseg = d;
            c.kt = kt;
            c.nranges = nr;
            add(c);
          }
      }
  return n;
}

// Index of the table entry that M resolves to, or -1 (below the smallest key).
inline int table_index(const TableEntry* t, int n, int64_t M) {
  if (n <= 0 || M < t[0].M) return -1;
  int i = 0;
  while (i + 1 < n && t[i + 1].M <= M) ++i;
  if (i + 1 < n && (double)M * (double)M > (double)t[i].M * (double)t[i + 1].M) ++i;  // nearer in log space
  return i;
}

// The plan used for M with a table (n = 0: the heuristic).
inline Plan plan_for(const Shape& s, int64_t M, const TableEntry* t, int n) {
  const int i = table_index(t, n, M);
  Plan p;
  if (i >= 0 && t[i].c.kind != kChoiceHeuristic && plan_from_choice(s, M, t[i].c, &p)) return p;
  return make_plan(s, M);
}

// Workspace that serves every M' <= M with a table. Entry i serves the
// interval of token counts nearer (in log space) to its key than to its
// neighbours', which may start below the key; its choice needs the most at
// the largest M' it serves (a decode-plan choice at the largest M' <= 256),
// and where the choice cannot run, the heuristic serves, which
// workspace_bound covers.
inline size_t workspace_bound_table(const Shape& s, int64_t M, const TableEntry* t, int n) {
  if (M <= 0) return 0;
  if (n <= 0) return workspace_bound(s, M);
  // largest M' that resolves to entry i (entry i + 1 is nearer above it)
  auto last_of = [&](int i) -> int64_t {
    if (i + 1 >= n) return INT64_MAX;
    const double lim = (double)t[i].M * (double)t[i + 1].M;
    int64_t b = (int64_t)__builtin_sqrt(lim);
    while ((double)(b + 1) * (double)(b + 1) <= lim) ++b;
    while ((double)b * (double)b > lim) --b;
    return b;
  };
  size_t best = workspace_bound(s, M < t[0].M ? M : t[0].M);  // heuristic below the first key
  int64_t lo = t[0].M;
  for (int i = 0; i < n && lo <= M; ++i) {
    const int64_t last = last_of(i);
    const int64_t hi = last < M ? last : M;
    const size_t h = workspace_bound(s, hi);  // heuristic wherever entry i falls back
    best = best > h ? best : h;
    Plan p;
    if (t[i].c.kind == PLAN_SPLIT || t[i].c.kind == PLAN_FUSED || t[i].c.kind == PLAN_PERSIST) {
      const int64_t m = hi < kSplitChoiceMaxM ? hi : kSplitChoiceMaxM;
      if (m >= lo && plan_from_choice(s, m, t[i].c, &p)) best = best > p.ws_bytes ? best : p.ws_bytes;
    } else if (t[i].c.kind == PLAN_TILE && plan_from_choice(s, hi, t[i].c, &p)) {
      best = best > p.ws_bytes ? best : p.ws_bytes;
    }
    lo = last == INT64_MAX ? INT64_MAX : last + 1;
  }
  return best;
}

// Arguments of one call. The whole op passes every pointer and res == R2.
// The mix entry point (every step but COMBINE) passes y, inj and R2 as NULL
// and res == R: the down kernels then read y as zeros (R2 = R exactly),
// store no R2, and the up kernel rebuilds xn from the input residual.
// Poll budget of a bounded wait inside one launch (the persistent decode
// plan's up role): the default and the largest a caller may set.
constexpr int kDefaultWaitPolls = 1 << 20, kMaxWaitPolls = 1 << 24;

struct ForwardArgs {
  const uint16_t *R, *y, *inj, *wnorm, *wd, *wi, *wu;
  int64_t ld_inj, ld_inj_next, M;
  uint16_t *R2, *inj_next, *x;
  const uint16_t* res;  // residual the up kernel reads: R2 (whole op) or R (mix)
  float* rrms;
  void* ws;
  int wait_polls = kDefaultWaitPolls;  // polls before a bounded wait gives up (0: at once)
};

struct CombineArgs {
  const uint16_t *R, *y, *inj;
  int64_t ld_inj, M;
  int HS, HC;
  uint16_t* R2;
  int nt = 0;  // set by launch_combine: R read and R2 written with the non-temporal policy
};
// Enqueues the combine-only kernel (R2 = R + y*iw) on `stream`; returns the
// hipError_t of the launch.
int launch_combine(const CombineArgs& a, void* stream);

// Raises the dynamic-LDS limit of the up kernels on the current device.
int configure_kernels();
// The same for the fused decode plan's kernels (hcgr_decode.hip).
int configure_decode_kernels();

// Enqueues the fused or persistent decode plan (hcgr_decode.hip); events as
// launch_forward (the persistent plan's one kernel is stage 0).
int launch_fused(const Shape& s, const Plan& p, const ForwardArgs& a, void* stream, void* const* events);
// The 256-token sweep up kernel (hcgr_sweep.hip): LDS limits, and its launch
// reading h from H; events: null or a (start, end) pair.
int configure_sweep2_kernels();
int launch_sweep2(const Shape& s, const Plan& p, const ForwardArgs& a, const uint16_t* H, void* stream,
                  void* const* events);
// Enqueues the stream-generic decode up kernel over token tiles of tm (16,
// 32 or 64) reading h from H; events: null or a (start, end) pair.
int launch_decg_up(const Shape& s, int tm, const uint16_t* H, const ForwardArgs& a, void* stream, void* const* events);

// Enqueues the plan's kernels on `stream`; returns the hipError_t of the
// launches. With `events` (6 hipEvent_t) events[2i] and events[2i+1] mark the
// start and end of stage i's kernel (a plan without a middle kernel records
// events[2] and events[3] back to back after the first kernel).
int launch_forward(const Shape& s, const Plan& p, const ForwardArgs& a, void* stream, void* const* events);

}  // namespace hcgr
