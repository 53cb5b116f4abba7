// hcgr_internal.h -- plan and kernel-launch interface shared by the C ABI
// (hcgr_api.hip) and the kernels (hcgr_kernels.hip). Not installed.
//
// The op is split into three launches, all on the caller's stream:
//   K1  hcgr_k1_down    COMBINE + the per-stream sums of squares of (N) + the
//                       down/inject contraction (G1, INJ) on bf16 MFMA tiles.
//                       Because rrms is a per-stream scalar and k is
//                       stream-major, xn . W^T = sum_s rrms[s] * P_s with
//                       P_s = sum_{c in stream s} R2*(1+Wnorm)*W: each
//                       workgroup contracts one K chunk that lies inside one
//                       stream and stores the unscaled partial P and the
//                       chunk's sum of squares; no workgroup has to wait for
//                       the whole row's RMS.
//   K1r hcgr_k1_reduce  sums the chunk partials of each stream, forms rrms,
//                       scales and adds the streams, applies SiLU(./HC) for
//                       the down rows (-> h, bf16, workspace) and writes
//                       inj_next for the inject rows.
//   K2  hcgr_k2_up_mix  gate = h . Wu^T on MFMA tiles whose 16 rows are 4
//                       channels x 4 streams, so the sigmoid and the gated
//                       mean over streams (MIX) happen in registers; xn is
//                       rebuilt from the bf16 R2 and rrms; writes x.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace hcgr {

// Kernel variants compiled into the library (template instantiations).
enum K1Variant { K1_T16 = 0, K1_T32 = 1, K1_T64S = 2, K1_T64L = 3, K1_NVAR };
enum K2Variant { K2_T16 = 0, K2_T32 = 1, K2_T64S = 2, K2_T64L = 3, K2_NVAR };

struct K1Shape { int tm, nw, nbw, ks; };
struct K2Shape { int tm, nw, rbw; };

inline K1Shape k1_shape(int v) {
  static const K1Shape t[K1_NVAR] = {{16, 7, 1, 128}, {32, 7, 1, 128}, {64, 7, 1, 128}, {64, 4, 6, 32}};
  return t[v];
}
inline K2Shape k2_shape(int v) {
  static const K2Shape t[K2_NVAR] = {{16, 4, 1}, {32, 4, 1}, {64, 4, 1}, {64, 4, 4}};
  return t[v];
}
// Chunks per stream handled by one lane group of the reduction kernel: the
// split plans keep chunks-per-stream <= 4 * kRedPerLane.
constexpr int kRedPerLane = 8;

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

struct Plan {
  int64_t M = 0, mpad = 0;
  int tm = 0;
  int k1 = 0, k2 = 0;
  int kc = 0, nkc = 0, kcps = 0;   // k per chunk, chunk count, chunks per stream
  int ntiles_n = 0;                // K1 n tiles (split plan)
  int cb = 0;                      // K2 channels per workgroup
  size_t off_p = 0, off_ss = 0, off_h = 0, ws_bytes = 0;
};

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Pure host planning: tile sizes and split counts by token count M.
inline Plan make_plan(const Shape& s, int64_t M) {
  Plan p;
  p.M = M;
  if (M <= 0) return p;
  const int hs = s.hs;
  // split plan: partial sums per K chunk, separate reduction kernel (K1 + K1r + K2)
  int kc;
  if (M <= 16) { p.k1 = K1_T16; p.k2 = K2_T16; kc = 128; }
  else if (M <= 32) { p.k1 = K1_T32; p.k2 = K2_T32; kc = 128; }
  else if (M <= 64) { p.k1 = K1_T64S; p.k2 = K2_T64S; kc = 128; }
  else if (M <= 128) { p.k1 = K1_T64S; p.k2 = K2_T64S; kc = 256; }
  else if (M <= 1024) { p.k1 = K1_T64S; p.k2 = K2_T64L; kc = 640; }
  else {
    p.k1 = K1_T64L; p.k2 = K2_T64L;
    int64_t mt = (M + 63) / 64;
    kc = mt >= 128 ? hs : (mt >= 64 ? hs / 2 : hs / 4);
  }
  const K1Shape a = k1_shape(p.k1);
  const K2Shape b = k2_shape(p.k2);
  // the chunk must divide the stream width and hold whole LDS stages, and a
  // stream may have at most 4 * kRedPerLane chunks (hs itself always fits)
  auto valid = [&](int c) { return c >= a.ks && c % a.ks == 0 && hs % c == 0; };
  while (kc > a.ks && !valid(kc)) kc -= a.ks;
  if (!valid(kc)) kc = a.ks;
  while (hs / kc > 4 * kRedPerLane) {
    int c = kc + a.ks;
    while (!valid(c)) c += a.ks;
    kc = c;
  }
  p.tm = a.tm;  // K1 and K2 share the token tile of a plan
  p.kc = kc;
  p.kcps = hs / kc;
  p.nkc = s.hc * p.kcps;
  int per_tile = a.nw * a.nbw;
  p.ntiles_n = (s.nblk() + per_tile - 1) / per_tile;
  p.cb = b.nw * b.rbw * 4;
  p.mpad = (M + p.tm - 1) / p.tm * p.tm;
  size_t np = (size_t)s.np();
  p.off_p = 0;
  p.off_ss = align256(p.off_p + (size_t)p.nkc * np * (size_t)p.mpad * sizeof(float));
  p.off_h = align256(p.off_ss + (size_t)p.nkc * (size_t)p.mpad * sizeof(float));
  p.ws_bytes = align256(p.off_h + (size_t)p.mpad * (size_t)s.r * sizeof(uint16_t));
  return p;
}

struct ForwardArgs {
  const uint16_t *R, *y, *inj, *wnorm, *wd, *wi, *wu;
  int64_t ld_inj, ld_inj_next, M;
  uint16_t *R2, *inj_next, *x;
  float* rrms;
  void* ws;
};

// Raises the dynamic-LDS limit of the up kernels on the current device (the
// h tile of a 64-token tile takes up to 66.5 KB at r = 512).
int configure_kernels();

// Enqueues K1, K1r and K2 on `stream`; returns the hipError_t of the launches.
// With `events` (4 hipEvent_t) it records events[0] before K1 and events[i]
// after the i-th kernel.
int launch_forward(const Shape& s, const Plan& p, const ForwardArgs& a, void* stream, void* const* events);

}  // namespace hcgr
