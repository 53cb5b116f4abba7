// hcgr_sweep.hip -- the up kernel of the Hyper-Connection Gated Residual op
// for large token counts over 256-token tiles (ROCm/aiter pull request #5913,
// "Two-stage Hyper-Connection Gated Residual kernel", section "Technical
// Details": G2 gate = sigmoid(h . Wu^T) and MIX x = mean_s G xn with xn
// rebuilt from R2 * rrms * (1 + Wnorm), so that neither xn nor the gate is
// stored).
//
// hcgr_k2_sweep2: a workgroup owns a tile of 256 tokens and sweeps a range
// of 32-channel groups (x 4 streams = 128 gate rows per group). Eight waves,
// two per SIMD; wave w owns tokens 32w .. 32w+31 and every gate row of the
// group, so each Wu stage (64 k) brought into LDS feeds 32 MFMAs per wave
// between two barriers and is fetched once per 256 tokens.
//  - h of the wave's tokens sits in registers as MFMA B fragments, loaded
//    once per workgroup.
//  - Wu: an LDS ring of NKS stages of 16 KB, loaded by direct global->LDS
//    loads from waves 0-3 NKS-1 stages ahead. LDS row gb*16 + 4j + s holds
//    stream s of channel 8j + gb of the group, its 16-byte piece c in slot
//    c ^ (row & 7); lane l then ends with the four streams of channels
//    8(l/16) .. 8(l/16)+7 for token l % 16, and MIX is lane-local.
//  - R2 of a group (4 streams x 256 tokens x 32 channels, 64 KB) and its
//    Wnorm: one LDS buffer loaded by waves 4-7 after the previous group's
//    epilogue has read it, a whole group ahead of its own use.
//  - Epilogue per group: sigmoid + MIX in registers, x stored as 16 bytes
//    (8 channels) per lane and token.
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

constexpr int kS2Wsb = 128 * 128;              // one Wu stage: 128 rows x 64 k
constexpr int kS2R2b = 4 * kSweep2Tm * 64;     // a group's R2: 4 streams x 256 tokens x 64 B
inline constexpr size_t sweep2_lds(int nks) { return (size_t)nks * kS2Wsb + kS2R2b + 1024 + kSweep2Tm * 16; }

// (MIX) (1/4) sum_s sigmoid(g_s) xn_s with one reciprocal: the four
// denominators d_s = 1 + e^-g_s combine over a common denominator (g clamped
// at -20 so the products stay finite).
__device__ __forceinline__ float mix4s(const float g[4], const float xn[4]) {
  float d[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) d[s] = 1.0f + __expf(-fmaxf(g[s], -20.0f));
  const float d01 = d[0] * d[1], d23 = d[2] * d[3];
  const float n01 = fmaf(xn[0], d[1], xn[1] * d[0]);
  const float n23 = fmaf(xn[2], d[3], xn[3] * d[2]);
  return 0.25f * fmaf(n01, d23, n23 * d01) * __builtin_amdgcn_rcpf(d01 * d23);
}

template <int NKS>
__global__ __launch_bounds__(512) void hcgr_k2_sweep2(Sweep2Args a) {
  constexpr int TM = kSweep2Tm, CG = 32, NTB = 2, NGB = 8, WSB = kS2Wsb;
  constexpr uint32_t kOut = 0x80000000u;
  static_assert(NKS >= 2 && NKS <= 5, "ring of 2..5 k stages");
  static_assert(sweep2_lds(5) <= 160 * 1024, "LDS of one CU");
  extern __shared__ __attribute__((aligned(1024))) uint8_t dl[];
  uint8_t* wring = dl;                  // [NKS][128 rows][128 B]
  uint8_t* r2buf = dl + NKS * WSB;      // [4 streams][256 tokens][4 slots of 16 B]
  uint8_t* wnbuf = r2buf + kS2R2b;      // [4 streams or 1][4 pieces of 16 B]
  uint8_t* rrbuf = wnbuf + 1024;        // [256 tokens][4 streams] rrms

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = lane >> 4, l16 = lane & 15;
  const int64_t tiles = (a.M + TM - 1) / TM;
  const int64_t tile = (int64_t)blockIdx.x % tiles;
  const int range = (int)((int64_t)blockIdx.x / tiles);
  const int g_begin = range * a.ngroups / a.nranges, g_end = (range + 1) * a.ngroups / a.nranges;
  const int64_t m0 = tile * TM;
  const int rows = (int)min((int64_t)TM, a.M - m0);
  const uint32_t rowb = (uint32_t)a.K * 2u, hrow = (uint32_t)a.r * 2u;

  const rsrc_t rH = make_rsrc(a.h + m0 * a.r, (uint32_t)rows * hrow);
  const rsrc_t rWu = make_rsrc(a.wu, (uint32_t)a.K * hrow);
  const rsrc_t rR2 = make_rsrc(a.R2 + m0 * a.K, (uint32_t)rows * rowb);
  const rsrc_t rRr = make_rsrc(a.rrms + m0 * 4, (uint32_t)rows * 16u);
  const rsrc_t rWn = make_rsrc(a.wn, (uint32_t)a.wn_len * 2u);
  const rsrc_t rX = make_rsrc(a.x + m0 * a.HS, (uint32_t)rows * (uint32_t)a.HS * 2u);

  // h of the wave's tokens as B fragments (k past r: zeros); the tile's
  // rrms goes to LDS (one direct load per wave of 4-7), read in the epilogue
  u32x4_t hf[NKS][2][NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    const uint32_t t = (uint32_t)(wave * 32 + tb * 16 + l16);
#pragma unroll
    for (int j = 0; j < NKS; ++j)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int k = j * 64 + ks * 32 + 8 * kg;
        hf[j][ks][tb] = __builtin_bit_cast(u32x4_t, bld16(rH, k < a.r ? t * hrow + (uint32_t)k * 2u : kOut));
      }
  }
  if (wave >= 4)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rRr, (lds_void_t*)(rrbuf + (wave - 4) * 1024), 16,
                                             (uint32_t)(((wave - 4) * 64 + lane) * 16), 0, 0, 0);

  // Wu loads (waves 0-3): instruction i = (wave & 3) + 4n fills stage rows
  // 8i .. 8i+7, lane -> row 8i + lane/8, slot lane % 8 holding piece
  // (lane % 8) ^ (lane / 8)
  const uint32_t swz = (uint32_t)((lane & 7) ^ (lane >> 3));
  uint32_t woff[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int rl = ((wave & 3) + 4 * n) * 8 + (lane >> 3);
    const int gb = rl >> 4, jj = (rl >> 2) & 3, s = rl & 3;
    woff[n] = (uint32_t)(s * a.HS + 8 * jj + gb) * hrow + swz * 16u;
  }
  auto issue_wu = [&](bool valid, int g, int j) {  // !valid: past the sweep, reads zeros
    uint8_t* buf = wring + j * WSB;
    const uint32_t base = (uint32_t)(g * CG) * hrow + (uint32_t)j * 128u;
    const bool inr = valid && j * 64 + (int)swz * 8 < a.r;
#pragma unroll
    for (int n = 0; n < 4; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rWu, (lds_void_t*)(buf + ((wave & 3) + 4 * n) * 1024), 16,
                                               inr ? woff[n] + base : kOut, 0, 0, 0);
  };
  // R2 loads (waves 4-7): instruction i = (wave - 4) + 4n (n < 16) fills
  // stream i / 16, LDS slots p = 64 (i % 16) + lane: token p / 4, piece
  // (p % 4) ^ ((token / 4) % 4) (8 channels); then Wnorm (wave 4)
  auto issue_r2 = [&](int g) {
    const int c0 = g * CG;
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      const int i = (wave - 4) + 4 * n, s = i >> 4;
      const int p = (i & 15) * 64 + lane, t = p >> 2, j = (p & 3) ^ ((t >> 2) & 3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rR2, (lds_void_t*)(r2buf + i * 1024), 16,
                                               (uint32_t)t * rowb + (uint32_t)(s * a.HS + c0 + 8 * j) * 2u, 0, 0, 0);
    }
    if (wave == 4) {
      const bool full = a.wn_len != a.HS;
      const bool live = lane < (full ? 16 : 4);
      const uint32_t wo = (uint32_t)((full ? (lane >> 2) * a.HS : 0) + c0 + (lane & 3) * 8) * 2u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rWn, (lds_void_t*)wnbuf, 16, live ? wo : kOut, 0, 0, 0);
    }
  };

  f32x4_t acc[NGB][NTB];
#pragma unroll
  for (int gb = 0; gb < NGB; ++gb)
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) acc[gb][tb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // (G2) one k stage: A = the group's 128 Wu rows, B = h fragments. The LDS
  // reads are one asm block with its own wait (the compiler cannot tell the
  // ring's later direct loads from this stage's data and would otherwise
  // wait for them); a half last stage past r reads zeros on both sides.
  const uint32_t wbase = (uint32_t)(uintptr_t)(lds_u8_t*)wring + (uint32_t)(l16 * 128);
  const uint32_t slot0 = (uint32_t)((kg ^ (l16 & 7)) * 16);
  const uint32_t slot1 = (uint32_t)(((4 + kg) ^ (l16 & 7)) * 16);
  typedef u32x4_t afrag_t[NGB];
  auto load_a = [&](auto J, afrag_t& af, int ks) {
    constexpr int j = decltype(J)::value;
    const uint32_t ad = wbase + (uint32_t)(j * WSB) + (ks ? slot1 : slot0);
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:2048\n\t"
        "ds_read_b128 %2, %8 offset:4096\n\t"
        "ds_read_b128 %3, %8 offset:6144\n\t"
        "ds_read_b128 %4, %8 offset:8192\n\t"
        "ds_read_b128 %5, %8 offset:10240\n\t"
        "ds_read_b128 %6, %8 offset:12288\n\t"
        "ds_read_b128 %7, %8 offset:14336\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3]), "=&v"(af[4]), "=&v"(af[5]), "=&v"(af[6]),
          "=&v"(af[7])
        : "v"(ad)
        : "memory");
  };
  auto products = [&](auto J, const afrag_t& af, int ks) {
    constexpr int j = decltype(J)::value;
#pragma unroll
    for (int gb = 0; gb < NGB; ++gb)
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb)
        acc[gb][tb] = mfma16(__builtin_bit_cast(uint4, af[gb]), __builtin_bit_cast(uint4, hf[j][ks][tb]), acc[gb][tb]);
  };

  // (G2) sigmoid + (MIX) of a finished group: the lane's R2 pieces (4
  // streams x 2 token blocks) and Wnorm pieces, then x of its 8 channels
  const uint32_t r2lane = (uint32_t)(uintptr_t)(lds_u8_t*)r2buf +
                          (uint32_t)(((wave * 32 + l16) * 4 + (kg ^ ((l16 >> 2) & 3))) * 16);
  const uint32_t wnlane = (uint32_t)(uintptr_t)(lds_u8_t*)wnbuf + (uint32_t)(kg * 16);
  const uint32_t wstep = a.wn_len != a.HS ? 64u : 0u;  // Wnorm indexed by k: one 64-byte row per stream
  auto epilogue = [&](int g) {
    u32x4_t wv[4];
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(wv[0]), "=&v"(wv[1]), "=&v"(wv[2]), "=&v"(wv[3])
        : "v"(wnlane), "v"(wnlane + wstep), "v"(wnlane + 2u * wstep), "v"(wnlane + 3u * wstep)
        : "memory");
    static_assert(4 * TM * 16 == 16384, "stream stride of the R2 buffer");
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      u32x4_t rv[4];  // the token's R2 pieces of streams 0..3 (8 channels each)
      const uint32_t ra = r2lane + (uint32_t)(tb * 1024);
      const f32x4_t rrv = *reinterpret_cast<const f32x4_t*>(rrbuf + (wave * 32 + tb * 16 + l16) * 16);
      asm volatile(
          "ds_read_b128 %0, %4\n\t"
          "ds_read_b128 %1, %4 offset:16384\n\t"
          "ds_read_b128 %2, %4 offset:32768\n\t"
          "ds_read_b128 %3, %4 offset:49152\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(rv[0]), "=&v"(rv[1]), "=&v"(rv[2]), "=&v"(rv[3])
          : "v"(ra)
          : "memory");
      float xo[NGB];
#pragma unroll
      for (int gb = 0; gb < NGB; ++gb) {
        float gs[4], xn[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t rw = rv[s][gb >> 1], ww = wv[s][gb >> 1];
          const float r2 = (gb & 1) ? bf_hi(rw) : bf_lo(rw);
          const float w1 = 1.0f + ((gb & 1) ? bf_hi(ww) : bf_lo(ww));
          gs[s] = acc[gb][tb][s];
          xn[s] = r2 * rrv[s] * w1;
        }
        xo[gb] = mix4s(gs, xn);
      }
      const uint32_t t = (uint32_t)(wave * 32 + tb * 16 + l16);
      bst16(rX, (t * (uint32_t)a.HS + (uint32_t)(g * CG + 8 * kg)) * 2u,
            make_uint4(pack_bf2(xo[0], xo[1]), pack_bf2(xo[2], xo[3]), pack_bf2(xo[4], xo[5]), pack_bf2(xo[6], xo[7])));
    }
  };

  // prologue: Wu of stages 0 .. NKS-2 of the first group (waves 0-3), R2 of
  // the first group (waves 4-7); h and rrms above. vmcnt(0) through the
  // builtin (0x0f70: expcnt and lgkmcnt left open), so the compiler also
  // knows the h and rrms registers have landed.
  if (wave < 4) {
#pragma unroll
    for (int j = 0; j < NKS - 1; ++j) issue_wu(true, g_begin, j);
  } else {
    issue_r2(g_begin);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);
  lds_sync();

  // Stage (g, j). At its top a Wu wave has issued the Wu of every stage up to
  // (g, j) + NKS - 2, four loads per stage (stages past the sweep included,
  // as out-of-range loads, so the count never changes), and possibly x
  // stores after them; vmcnt(4 (NKS - 2)) counts the later loads only (a
  // store may complete ahead of earlier loads, which only makes the wait
  // longer) and leaves the NKS - 2 newer stages in flight. Stage (g, j)
  // loads stage (g, j) + NKS - 1 into ring slot j - 1 (the previous stage's,
  // read before this stage's barrier). After the group's last stage: the R2
  // waves wait for R2(g) (their only loads outstanding besides x stores),
  // every wave runs the epilogue, and once every wave has read R2(g) the R2
  // waves load R2(g + 1) into the same buffer.
  for (int g = g_begin; g < g_end; ++g) {
    auto stage = [&](auto J) {
      constexpr int j = decltype(J)::value;
      if (g != g_begin || j != 0) {
        if (wave < 4) {
          if constexpr (NKS == 2) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          else if constexpr (NKS == 3) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
          else if constexpr (NKS == 4) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
          else asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
        }
        lds_sync();
      }
      if (wave < 4) {
        constexpr int q2 = j + NKS - 1;  // stage (g, q2), or (g + 1, q2 - NKS)
        const int gn = q2 >= NKS ? g + 1 : g;
        issue_wu(gn < g_end, gn, q2 >= NKS ? q2 - NKS : q2);
      }
      afrag_t af;
      load_a(J, af, 0);
      products(J, af, 0);
      load_a(J, af, 1);
      products(J, af, 1);
    };
    stage(icn<0>{});
    stage(icn<1>{});
    if constexpr (NKS > 2) stage(icn<2>{});
    if constexpr (NKS > 3) stage(icn<3>{});
    if constexpr (NKS > 4) stage(icn<4>{});
    if (wave >= 4) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_sync();  // R2(g) landed; every wave is past its last stage
    epilogue(g);
    lds_sync();  // every wave has read R2(g)
    if (wave >= 4 && g + 1 < g_end) issue_r2(g + 1);
#pragma unroll
    for (int gb = 0; gb < NGB; ++gb)
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) acc[gb][tb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
  // the loads issued past the last stage must land before the LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

int configure_sweep2_kernels() {
  hipError_t e;
  if ((e = hipFuncSetAttribute((const void*)hcgr_k2_sweep2<2>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)sweep2_lds(2))) != hipSuccess ||
      (e = hipFuncSetAttribute((const void*)hcgr_k2_sweep2<3>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)sweep2_lds(3))) != hipSuccess ||
      (e = hipFuncSetAttribute((const void*)hcgr_k2_sweep2<4>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)sweep2_lds(4))) != hipSuccess ||
      (e = hipFuncSetAttribute((const void*)hcgr_k2_sweep2<5>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)sweep2_lds(5))) != hipSuccess)
    return (int)e;
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
  hipEvent_t e0 = ev ? ev[0] : nullptr, e1 = ev ? ev[1] : nullptr;
  switch (sweep_nks(s.r)) {
    case 2: hipExtLaunchKernelGGL(hcgr_k2_sweep2<2>, g, b, (uint32_t)sweep2_lds(2), st, e0, e1, 0u, a); break;
    case 3: hipExtLaunchKernelGGL(hcgr_k2_sweep2<3>, g, b, (uint32_t)sweep2_lds(3), st, e0, e1, 0u, a); break;
    case 4: hipExtLaunchKernelGGL(hcgr_k2_sweep2<4>, g, b, (uint32_t)sweep2_lds(4), st, e0, e1, 0u, a); break;
    case 5: hipExtLaunchKernelGGL(hcgr_k2_sweep2<5>, g, b, (uint32_t)sweep2_lds(5), st, e0, e1, 0u, a); break;
    default: return (int)hipErrorInvalidValue;  // the planner takes this kernel for 2..5 k stages only
  }
  return (int)hipGetLastError();
}

}  // namespace hcgr
