// hcgr_sweep.hip -- the up kernel of the Hyper-Connection Gated Residual op
// for large token counts over 256-token tiles (ROCm/aiter pull request #5913,
// "Two-stage Hyper-Connection Gated Residual kernel", section "Technical
// Details": G2 gate = sigmoid(h . Wu^T) and MIX x = mean_s G xn with xn
// rebuilt from R2 * rrms * (1 + Wnorm), so that neither xn nor the gate is
// stored).
//
// hcgr_k2_sweep2: a workgroup owns a tile of 256 tokens and sweeps a range of
// 32-channel groups. Eight waves, two per SIMD; wave w owns tokens 32w ..
// 32w+31 (two blocks of 16) and every gate row.
//  - Gate rows stream through LDS in blocks of 16 (4 channels x 4 streams)
//    over the whole of k: block gb of group g holds, in row 4j + s, stream s
//    of channel 32g + 8j + gb. After one block's products, lane l holds the
//    four stream gates of channel 32g + 8(l/16) + gb for token l % 16 of
//    each token block, so a block's sigmoid + MIX is lane-local and runs
//    while the next block's MFMAs execute (the vector ALU and the matrix
//    cores overlap within and across the two waves of a SIMD).
//  - A Wu stage is four blocks (half a group); a ring of three stages is fed
//    by direct global->LDS loads from all eight waves two stages ahead. LDS
//    layout of a block: k chunks of 64 (2 KB: 16 rows x 128 B), 16-byte
//    piece c of row r in slot c ^ ((r / 2) % 8), so the 16 lanes of one
//    read phase touch all 64 banks once.
//  - h of the wave's tokens: MFMA B fragments in registers, loaded once.
//  - R2 of a group: per lane, token and stream one 16-byte piece (the 8
//    channels 32g + 8(l/16) .. +7 that the lane's 8 blocks need), in
//    registers, prefetched a group ahead into a second set.
//  - (1 + Wnorm) / 4 of the range's channels: f32 in LDS, filled once.
//  - x: the lane's 8 channels of a group, packed as the blocks finish and
//    stored as 16 bytes per token.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include <type_traits>

#include "hcgr_device.h"
#include "hcgr_internal.h"

namespace hcgr {

template <int N>
using icn = std::integral_constant<int, N>;

struct Sweep2Args {
  const uint16_t* h;  // [>= M, r]
  int64_t M;
  int r, HS, K;
  const uint16_t* wu;  // [K, r]
  const uint16_t* R2;  // [M, K]
  const float* rrms;   // [M, 4]
  const uint16_t* wn;
  int wn_len;
  uint16_t* x;   // [M, HS]
  int ngroups;   // HS / 32
  int nranges;   // channel-group ranges per token tile
};

// (MIX) sum_s sigmoid(g_s) rrms_s v_s with the token's rrms folded into the
// gate denominators: d_s = (1 + e^-g_s) / rrms_s, so each term is v_s / d_s,
// and the four terms combine over two pair denominators (v0 d1 + v1 d0) /
// (d0 d1), one reciprocal per pair. e^-g = 2^(-g log2 e) by the hardware
// exponential, its argument clamped at 20 log2 e (g >= -20) so that the pair
// products stay finite; the clamp is a min on the product, which needs no
// NaN canonicalisation, unlike a max on the MFMA result. irr = 1 / rrms.
__device__ __forceinline__ float s2_mix(const float g[4], const float v[4], const float irr[4]) {
  float d[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const float e = __builtin_amdgcn_exp2f(fminf(g[s] * -1.4426950408889634f, 28.853900817779268f));
    d[s] = fmaf(e, irr[s], irr[s]);
  }
  const float n01 = fmaf(v[0], d[1], v[1] * d[0]);
  const float n23 = fmaf(v[2], d[3], v[3] * d[2]);
  return fmaf(n01, __builtin_amdgcn_rcpf(d[0] * d[1]), n23 * __builtin_amdgcn_rcpf(d[2] * d[3]));
}

// Half of one block's A fragments (k steps of 32: step ks sits in chunk
// ks / 2 at offset 2048 (ks / 2), even steps at address a0, odd ones at a1):
// half 0 holds steps 0 .. NC-1, half 1 steps NC .. 2NC-1. Half 0 also reads
// the scale of the block whose epilogue runs beside these products (one
// f32, or four for a full-width Wnorm). Each half is one group of LDS reads
// with its own wait: the compiler cannot tell the ring's in-flight direct
// loads from this data and would otherwise wait for all of them; the second
// half's wait overlaps the first half's MFMAs.
#define S2R(o, a, off) "ds_read_b128 %" #o ", %" #a " offset:" #off "\n\t"
#define S2W32(o, a) "ds_read_b32 %" #o ", %" #a "\n\t"
#define S2W128(o, a) "ds_read_b128 %" #o ", %" #a "\n\t"
#define S2WAIT "s_waitcnt lgkmcnt(0)"
template <int NC, bool FULL>
struct S2Scale { typedef float type; };
template <int NC>
struct S2Scale<NC, true> { typedef f32x4_t type; };

// half 0: outputs af[0..NC-1] (%0 .. %NC-1), w (%NC); inputs a0, a1, wa
template <int NC, bool FULL>
__device__ __forceinline__ void s2_read0(u32x4_t (&af)[NC], typename S2Scale<NC, FULL>::type& w, uint32_t a0,
                                         uint32_t a1, uint32_t wa) {
  if constexpr (NC == 5) {
#define S2H0 S2R(0, 6, 0) S2R(1, 7, 0) S2R(2, 6, 2048) S2R(3, 7, 2048) S2R(4, 6, 4096)
    if constexpr (FULL)
      asm volatile(S2H0 S2W128(5, 8) S2WAIT
                   : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3]), "=&v"(af[4]), "=&v"(w)
                   : "v"(a0), "v"(a1), "v"(wa) : "memory");
    else
      asm volatile(S2H0 S2W32(5, 8) S2WAIT
                   : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3]), "=&v"(af[4]), "=&v"(w)
                   : "v"(a0), "v"(a1), "v"(wa) : "memory");
#undef S2H0
  } else if constexpr (NC == 4) {
#define S2H0 S2R(0, 5, 0) S2R(1, 6, 0) S2R(2, 5, 2048) S2R(3, 6, 2048)
    if constexpr (FULL)
      asm volatile(S2H0 S2W128(4, 7) S2WAIT
                   : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3]), "=&v"(w)
                   : "v"(a0), "v"(a1), "v"(wa) : "memory");
    else
      asm volatile(S2H0 S2W32(4, 7) S2WAIT
                   : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3]), "=&v"(w)
                   : "v"(a0), "v"(a1), "v"(wa) : "memory");
#undef S2H0
  } else if constexpr (NC == 3) {
#define S2H0 S2R(0, 4, 0) S2R(1, 5, 0) S2R(2, 4, 2048)
    if constexpr (FULL)
      asm volatile(S2H0 S2W128(3, 6) S2WAIT
                   : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(w) : "v"(a0), "v"(a1), "v"(wa) : "memory");
    else
      asm volatile(S2H0 S2W32(3, 6) S2WAIT
                   : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(w) : "v"(a0), "v"(a1), "v"(wa) : "memory");
#undef S2H0
  } else {
    static_assert(NC == 2, "two to five k chunks");
    if constexpr (FULL)
      asm volatile(S2R(0, 3, 0) S2R(1, 4, 0) S2W128(2, 5) S2WAIT
                   : "=&v"(af[0]), "=&v"(af[1]), "=&v"(w) : "v"(a0), "v"(a1), "v"(wa) : "memory");
    else
      asm volatile(S2R(0, 3, 0) S2R(1, 4, 0) S2W32(2, 5) S2WAIT
                   : "=&v"(af[0]), "=&v"(af[1]), "=&v"(w) : "v"(a0), "v"(a1), "v"(wa) : "memory");
  }
}
// half 1: outputs af[0..NC-1] = steps NC .. 2NC-1; inputs a0, a1
template <int NC>
__device__ __forceinline__ void s2_read1(u32x4_t (&af)[NC], uint32_t a0, uint32_t a1) {
  if constexpr (NC == 5)
    asm volatile(S2R(0, 6, 4096) S2R(1, 5, 6144) S2R(2, 6, 6144) S2R(3, 5, 8192) S2R(4, 6, 8192) S2WAIT
                 : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3]), "=&v"(af[4]) : "v"(a0), "v"(a1)
                 : "memory");
  else if constexpr (NC == 4)
    asm volatile(S2R(0, 4, 4096) S2R(1, 5, 4096) S2R(2, 4, 6144) S2R(3, 5, 6144) S2WAIT
                 : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3]) : "v"(a0), "v"(a1) : "memory");
  else if constexpr (NC == 3)
    asm volatile(S2R(0, 4, 2048) S2R(1, 3, 4096) S2R(2, 4, 4096) S2WAIT
                 : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]) : "v"(a0), "v"(a1) : "memory");
  else
    asm volatile(S2R(0, 2, 2048) S2R(1, 3, 2048) S2WAIT
                 : "=&v"(af[0]), "=&v"(af[1]) : "v"(a0), "v"(a1) : "memory");
}
// the scale alone (the last block's epilogue, after the last products)
template <bool FULL>
__device__ __forceinline__ void s2_read_w(typename S2Scale<2, FULL>::type& w, uint32_t wa) {
  if constexpr (FULL) asm volatile(S2W128(0, 1) S2WAIT : "=&v"(w) : "v"(wa) : "memory");
  else asm volatile(S2W32(0, 1) S2WAIT : "=&v"(w) : "v"(wa) : "memory");
}
#undef S2R
#undef S2W32
#undef S2W128
#undef S2WAIT

template <int NC, bool FULL>
__global__ __launch_bounds__(512) void hcgr_k2_sweep2(Sweep2Args a) {
  constexpr int TM = kSweep2Tm, NK = 2 * NC, SB = (int)sweep2_stage_bytes(NC);
  constexpr uint32_t kOut = 0x80000000u;
  static_assert(NC >= 2 && NC <= 5, "two to five k chunks of 64");
  typedef typename S2Scale<NC, FULL>::type scale_t;
  extern __shared__ __attribute__((aligned(1024))) uint8_t dl[];
  float* wq = reinterpret_cast<float*>(dl + kSweep2Ring * SB);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = lane >> 4, l16 = lane & 15;
  const int64_t tiles = (a.M + TM - 1) / TM;
  const int64_t tile = (int64_t)blockIdx.x % tiles;
  const int range = (int)((int64_t)blockIdx.x / tiles);
  // ranges hold whole pairs of groups (64 channels: one 128-byte line of a
  // token's stream row)
  const int npairs = (a.ngroups + 1) / 2;
  const int g_begin = 2 * (range * npairs / a.nranges);
  const int g_end = min(2 * ((range + 1) * npairs / a.nranges), a.ngroups);
  const int ng = g_end - g_begin, nch = ng * 32;
  const int64_t m0 = tile * TM;
  const int rows = (int)min((int64_t)TM, a.M - m0);
  const uint32_t rowb = (uint32_t)a.K * 2u, hrow = (uint32_t)a.r * 2u;

  const rsrc_t rH = make_rsrc(a.h + m0 * a.r, (uint32_t)rows * hrow);
  const rsrc_t rWu = make_rsrc(a.wu, (uint32_t)a.K * hrow);
  const rsrc_t rR2 = make_rsrc(a.R2 + m0 * a.K, (uint32_t)rows * rowb);
  const rsrc_t rRr = make_rsrc(a.rrms + m0 * 4, (uint32_t)rows * 16u);
  const rsrc_t rX = make_rsrc(a.x + m0 * a.HS, (uint32_t)rows * (uint32_t)a.HS * 2u);

  // 0.25 (1 + Wnorm) of the range's channels; a full-width Wnorm as
  // [channel][stream], so one 16-byte read gives a channel's four streams
  const size_t c0 = (size_t)g_begin * 32;
  if constexpr (FULL) {
    for (int i = tid; i < 4 * nch; i += 512)
      wq[i] = fmaf(bf1(a.wn[(size_t)(i & 3) * a.HS + c0 + (i >> 2)]), 0.25f, 0.25f);
  } else {
    for (int i = tid; i < nch; i += 512) wq[i] = fmaf(bf1(a.wn[c0 + i]), 0.25f, 0.25f);
  }

  // h of the wave's tokens as B fragments (k past r: zeros) and rrms
  u32x4_t hf[NK][2];
  f32x4_t rr[2];  // rrms of the lane's tokens
  uint32_t r2base[2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const uint32_t t = (uint32_t)(wave * 32 + tb * 16 + l16);
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const int k = ks * 32 + 8 * kg;
      hf[ks][tb] = __builtin_bit_cast(u32x4_t, bld16(rH, k < a.r ? t * hrow + (uint32_t)k * 2u : kOut));
    }
    rr[tb] = __builtin_bit_cast(f32x4_t, bld16(rRr, t * 16u));
    r2base[tb] = t * rowb + (uint32_t)((int)c0 + 8 * kg) * 2u;
  }

  // Wu loads: stage instruction i (0 .. 8 NC - 1, 1 KB each) fills block
  // i / (2 NC), chunk (i % 2NC) / 2, rows 8 (i % 2) .. +7; wave w issues
  // i = w + 8n. Lane -> row 8 (i % 2) + lane / 8, slot lane % 8 holding
  // piece (lane % 8) ^ ((row / 2) % 8).
  // (sized for the largest NC: a lambda capturing an array whose size depends
  // on the template parameters leaves the kernel's host stub undefined)
  uint32_t woff[5];
#pragma unroll
  for (int n = 0; n < NC; ++n) {
    const int i = wave + 8 * n, bb = i / (2 * NC), ii = i % (2 * NC);
    const int row = 8 * (ii & 1) + (lane >> 3);
    const int piece = (lane & 7) ^ ((row >> 1) & 7);
    const int k = (ii >> 1) * 64 + piece * 8;
    woff[n] = k < a.r ? (uint32_t)((row & 3) * a.HS + 8 * (row >> 2) + bb) * hrow + (uint32_t)k * 2u : ~0u;
  }
  auto issue_wu = [&](int q, int slot) {  // stage q of the range; past the sweep: out-of-range loads
    const int gq = q >> 1;
    const bool valid = gq < ng;
    const uint32_t base = (uint32_t)((g_begin + gq) * 32 + 4 * (q & 1)) * hrow;
    uint8_t* buf = dl + slot * SB;
#pragma unroll
    for (int n = 0; n < NC; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rWu, (lds_void_t*)(buf + (wave + 8 * n) * 1024), 16,
                                               valid && woff[n] != ~0u ? woff[n] + base : kOut, 0, 0, 0);
  };
  typedef u32x4_t r2set_t[2][4];
  auto issue_r2 = [&](r2set_t& dst, int gi) {  // R2 pieces of group gi (past the range: zeros)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        dst[tb][s] = __builtin_bit_cast(
            u32x4_t, bld16(rR2, gi < ng ? r2base[tb] + (uint32_t)(s * a.HS + gi * 32) * 2u : kOut));
  };

  const uint32_t ldsb = (uint32_t)(uintptr_t)(lds_u8_t*)dl;
  const uint32_t key = (uint32_t)((l16 >> 1) & 7);
  const uint32_t la0 = ldsb + (uint32_t)(l16 * 128) + (((uint32_t)kg ^ key) * 16u);
  const uint32_t la1 = ldsb + (uint32_t)(l16 * 128) + (((uint32_t)(4 + kg) ^ key) * 16u);
  constexpr uint32_t kWs = FULL ? 16u : 4u;  // scale bytes per channel
  const uint32_t wl = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) float*)wq + (uint32_t)(8 * kg) * kWs;

  f32x4_t acc[2][2];  // [block parity][token block]
  float irr[2][4];    // 1 / rrms of the lane's tokens
  float xo[2];        // the even channel of the pair being packed
  uint32_t out[2][4];
  r2set_t R2a, R2b;

  // (G2) products of half a block (k steps H NC .. H NC + NC - 1) against
  // both token blocks
  auto products = [&](auto H, const u32x4_t (&af)[NC], f32x4_t (&c)[2]) {
    constexpr int h = decltype(H)::value;
#pragma unroll
    for (int i = 0; i < NC; ++i)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
        c[tb] = mfma16(__builtin_bit_cast(uint4, af[i]), __builtin_bit_cast(uint4, hf[h * NC + i][tb]),
                       h == 0 && i == 0 ? f32x4_t{0.0f, 0.0f, 0.0f, 0.0f} : c[tb]);
  };
  // (G2) sigmoid + (MIX) of block gb: x of channel 8 (l/16) + gb of the group
  auto epilogue = [&](auto GB, const f32x4_t (&c)[2], const r2set_t& r2, const scale_t& w) {
    constexpr int gb = decltype(GB)::value;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      float g[4], v[4], ir[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t rw = r2[tb][s][gb >> 1];
        v[s] = (gb & 1) ? bf_hi(rw) : bf_lo(rw);
        if constexpr (FULL) v[s] *= w[s];
        g[s] = c[tb][s];
        ir[s] = irr[tb][s];
      }
      float o = s2_mix(g, v, ir);
      if constexpr (!FULL) o *= w;
      if constexpr (gb & 1) out[tb][gb >> 1] = pack_bf2(xo[tb], o);
      else xo[tb] = o;
    }
  };
  auto store_x = [&](int gi) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const uint32_t t = (uint32_t)(wave * 32 + tb * 16 + l16);
      bst16(rX, (t * (uint32_t)a.HS + (uint32_t)((int)c0 + gi * 32 + 8 * kg)) * 2u,
            make_uint4(out[tb][0], out[tb][1], out[tb][2], out[tb][3]));
    }
  };

  // prologue: stages 0 and 1 of the ring, R2 of the first group, h and rrms
  // above; everything lands before the first barrier
  int rd = 0;  // ring slot of the current stage
  issue_wu(0, 0);
  issue_wu(1, 1);
  issue_r2(R2a, 0);
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  __syncthreads();
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int s = 0; s < 4; ++s) irr[tb][s] = __builtin_amdgcn_rcpf(rr[tb][s]);

  // Group gi (its R2 in cur; prv holds group gi - 1's, whose block 7 the
  // first block here finishes, and then takes group gi + 1's, loaded in
  // block 1). Per wave, the loads in issue order: Wu(q) at the top of stage
  // q - 2, R2(gi + 1) in block 1 of group gi. At the top of stage q the
  // loads issued after Wu(q) are Wu(q + 1) and one group's R2 (8):
  // vmcnt(NC + 8) waits for Wu(q) alone (a store issued in between only
  // lengthens the wait). The barrier then makes every wave's part of stage q
  // visible, and every wave has finished reading stage q - 1, whose slot
  // stage q + 2 takes.
  auto stage_top = [&](int q) {
    if constexpr (NC == 5) asm volatile("s_waitcnt vmcnt(13)" ::: "memory");
    else if constexpr (NC == 4) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    else if constexpr (NC == 3) asm volatile("s_waitcnt vmcnt(11)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
    lds_sync();
    issue_wu(q + 2, rd == 0 ? 2 : rd - 1);
  };
  auto group = [&](auto FIRST, int gi, r2set_t& cur, r2set_t& prv) {
    constexpr bool first = decltype(FIRST)::value;
    const uint32_t wg = wl + (uint32_t)(gi * 32) * kWs;
    auto block = [&](auto GB) {
      constexpr int gb = decltype(GB)::value;
      if constexpr (gb == 4) rd = rd == 2 ? 0 : rd + 1;
      if constexpr (gb % 4 == 0) stage_top(2 * gi + gb / 4);
      if constexpr (gb == 1) issue_r2(prv, gi + 1);
      const uint32_t sb = (uint32_t)(rd * SB + (gb & 3) * NC * 2048);
      u32x4_t af[NC];
      scale_t w;
      // the scale of the previous block: block gb - 1 here, or block 7 of
      // the previous group
      s2_read0<NC, FULL>(af, w, la0 + sb, la1 + sb, gb == 0 ? wg - 25u * kWs : wg + (uint32_t)(gb - 1) * kWs);
      products(icn<0>{}, af, acc[gb & 1]);
      s2_read1<NC>(af, la0 + sb, la1 + sb);
      products(icn<1>{}, af, acc[gb & 1]);
      if constexpr (gb == 0) {
        if constexpr (!first) {
          epilogue(icn<7>{}, acc[1], prv, w);
          store_x(gi - 1);
        }
      } else {
        epilogue(icn<gb - 1>{}, acc[(gb - 1) & 1], cur, w);
      }
      if constexpr (gb == 7) rd = rd == 2 ? 0 : rd + 1;
    };
    block(icn<0>{}); block(icn<1>{}); block(icn<2>{}); block(icn<3>{});
    block(icn<4>{}); block(icn<5>{}); block(icn<6>{}); block(icn<7>{});
  };
  auto finish = [&](const r2set_t& last) {  // block 7 of the last group
    scale_t w;
    s2_read_w<FULL>(w, wl + (uint32_t)((ng - 1) * 32 + 7) * kWs);
    epilogue(icn<7>{}, acc[1], last, w);
    store_x(ng - 1);
  };

  group(std::true_type{}, 0, R2a, R2b);
  int gi = 1;
  for (; gi + 1 < ng; gi += 2) {
    group(std::false_type{}, gi, R2b, R2a);
    group(std::false_type{}, gi + 1, R2a, R2b);
  }
  if (gi < ng) {
    group(std::false_type{}, gi, R2b, R2a);
    finish(R2b);
  } else {
    finish(R2a);
  }
  // the loads issued past the last stage must land before the LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

int configure_sweep2_kernels() {
  const void* fns[8] = {(const void*)hcgr_k2_sweep2<2, false>, (const void*)hcgr_k2_sweep2<3, false>,
                        (const void*)hcgr_k2_sweep2<4, false>, (const void*)hcgr_k2_sweep2<5, false>,
                        (const void*)hcgr_k2_sweep2<2, true>,  (const void*)hcgr_k2_sweep2<3, true>,
                        (const void*)hcgr_k2_sweep2<4, true>,  (const void*)hcgr_k2_sweep2<5, true>};
  for (const void* f : fns) {
    const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsPerCu);
    if (e != hipSuccess) return (int)e;
  }
  return (int)hipSuccess;
}

int launch_sweep2(const Shape& s, const Plan& p, const ForwardArgs& f, const uint16_t* H, void* stream,
                  void* const* events) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const hipEvent_t* ev = reinterpret_cast<const hipEvent_t*>(events);
  Sweep2Args a;
  a.h = H; a.M = f.M; a.r = s.r; a.HS = s.hs; a.K = (int)s.k(); a.wu = f.wu; a.R2 = f.res; a.rrms = f.rrms;
  a.wn = f.wnorm; a.wn_len = s.wn_full ? (int)s.k() : s.hs; a.x = f.x; a.ngroups = s.hs / 32; a.nranges = p.nranges;
  const dim3 g((unsigned)(cdiv(f.M, (int64_t)kSweep2Tm) * p.nranges)), b(512);
  const uint32_t lds = (uint32_t)sweep2_lds(s, p.nranges);
  if (lds > kLdsPerCu) return (int)hipErrorInvalidValue;  // the planner checks this
  hipEvent_t e0 = ev ? ev[0] : nullptr, e1 = ev ? ev[1] : nullptr;
#define S2L(nc, full) hipExtLaunchKernelGGL(hcgr_k2_sweep2<nc, full>, g, b, lds, st, e0, e1, 0u, a)
  switch (sweep_nks(s.r) + (s.wn_full ? 8 : 0)) {
    case 2: S2L(2, false); break;
    case 3: S2L(3, false); break;
    case 4: S2L(4, false); break;
    case 5: S2L(5, false); break;
    case 10: S2L(2, true); break;
    case 11: S2L(3, true); break;
    case 12: S2L(4, true); break;
    case 13: S2L(5, true); break;
    default: return (int)hipErrorInvalidValue;  // the planner takes this kernel for 2..5 k chunks only
  }
#undef S2L
  return (int)hipGetLastError();
}

}  // namespace hcgr
