// hcgr_decode.hip -- the decode plans of the Hyper-Connection Gated Residual
// op (ROCm/aiter pull request #5913, "Two-stage Hyper-Connection Gated
// Residual kernel", section "Technical Details": COMBINE, N, G1, INJ in the
// down role, G2 and MIX in the up role) for any stream count HC.
//
// The page's "PR Self-Review" section describes a skinny decode path whose
// workgroups publish their partial products with an agent-scope arrival
// counter. Here that becomes a last-arriver reduction: every down workgroup
// writes its fp32 partial for one 16-row block and one K chunk, then bumps the
// block's counter (an agent-scope vector atomic); the workgroup that sees the
// final count sums the block's chunks, forms rrms, writes h and inj_next, and
// resets the counter. Two plans use it:
//   FUSED       two kernels, hcgr_k1_fuse (down role) and hcgr_k2_decg (up
//               role); the kernel boundary hands h to the up kernel.
//   PERSISTENT  one kernel, hcgr_dec_persist, with the down-role workgroups
//               first and the up-role workgroups after them; an up workgroup
//               loads its Wu rows into LDS at once, then waits (bounded) for
//               its token tile's ready flag: every block's last arrival
//               bumps the tile's "h complete" counter after publishing its h
//               rows, and the arrival that completes that count raises the
//               flag.
// Data that crosses workgroups inside a kernel (partials, sums of squares, and
// in the persistent plan R2, rrms and h) moves by agent-coherent stores and
// loads (below), so no L2 write-back or invalidation is needed.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "hcgr_device.h"
#include "hcgr_internal.h"

namespace hcgr {

constexpr uint32_t kOutOfRange = 0x80000000u;  // buffer offset past every range: loads give 0

__device__ __forceinline__ void lds_load16(rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, off, 0, 0, 0);
}
// Agent-coherent accesses (kAgentCoherent, the SC1 policy): the partial
// products that cross workgroups use them, so their publication needs no L2
// write-back or invalidation, only the completion of the stores before the
// counter update.
__device__ __forceinline__ void lds_load16_agent(rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, off, 0, 0, kAgentCoherent);
}
__device__ __forceinline__ void bst16_agent(rsrc_t r, uint32_t off, f32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, (int)off, 0, kAgentCoherent);
}
__device__ __forceinline__ void bst4_agent(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)off, 0, kAgentCoherent);
}
// stores whose cache policy is chosen at compile time (agent-coherent when AG)
template <bool AG>
__device__ __forceinline__ void bst16_p(rsrc_t r, uint32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, (int)off, 0, AG ? kAgentCoherent : 0);
}
template <bool AG>
__device__ __forceinline__ void bst8_p(rsrc_t r, uint32_t off, uint2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, v), r, (int)off, 0, AG ? kAgentCoherent : 0);
}
template <bool AG>
__device__ __forceinline__ void bst2_p(rsrc_t r, uint32_t off, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, (int)off, 0, AG ? kAgentCoherent : 0);
}
template <bool AG>
__device__ __forceinline__ void bst4f_p(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)off, 0, AG ? kAgentCoherent : 0);
}
template <bool AG>
__device__ __forceinline__ void lds_load16_p(rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, off, 0, 0, AG ? kAgentCoherent : 0);
}
// direct global->LDS loads of 4 bytes per lane (256 bytes per instruction)
template <bool AG>
__device__ __forceinline__ void lds_load4_p(rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 4, off, 0, 0, AG ? kAgentCoherent : 0);
}
// Counter slot i of a slot array: each slot starts a 128-byte line of its
// own, since agent-scope atomics on one line are serialised.
__device__ __forceinline__ uint32_t* slot(uint32_t* base, int64_t i) { return base + i * kCtrStride; }

// Bounded wait for the persistent plan's up role: polls the ready flag *flag
// (an agent-coherent load, then a sleep of 8 x 64 cycles) until it is set or
// `polls` polls have found it clear; a wait that gives up raises *err and
// returns false. The flag sits in a line of its own that only the arrival completing
// the count writes: measured on MI355X, 160 workgroups polling the very
// counter that 252 others increment delayed the increments by 2-5 us,
// polling a separate flag by 0.3 us.
__device__ __forceinline__ bool wait_flag(const uint32_t* flag, uint32_t* err, int polls) {
  for (int it = 0; it < polls; ++it) {
    if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) return true;
    __builtin_amdgcn_s_sleep(8);
  }
  __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return false;
}

struct FuseArgs {
  const uint16_t* R;
  const uint16_t* y;
  const uint16_t* inj;
  int64_t ld_inj;
  const uint16_t* wn;
  int wn_full;
  int folded;          // merged/folded weights: the activation omits (1 + Wnorm)
  const uint16_t* w0;  // Wd [r,K] or merged Wm [n_pad,K]
  const uint16_t* w1;  // Wi [HC,K], or nullptr when the inject rows are rows r.. of w0
  int64_t M;
  int K, HS, HC, r, nblk, U, kcps, nkc;
  float eps, inv_hc, inv_hs;
  uint16_t* R2;
  float* rrms;
  uint16_t* h;  // [Mpad, r] SiLU output for the up kernel
  uint16_t* inj_next;
  int64_t ld_inj_next;
  float* P;       // [tiles][nblk][nkc][TM][16] unscaled chunk partials
  float* SS;      // [tiles][nblk][nkc][TM] chunk sums of squares
  uint32_t* ctr;  // [tiles][nblk] arrival counters (zero between calls)
  uint32_t* hdone;  // [tiles] slots, persistent plan: blocks whose h rows are published
  uint32_t* ready;  // [tiles] slots, persistent plan: raised when every block of the tile is published
};

// ---------------------------------------------------------------------------
// hcgr_k1_fuse: workgroup = (16-row block blk of the down/inject rows) x (K
// chunk: 128-column units [u0, u1) of stream s) x (token tile of TM tokens),
// 4 waves. Steps:
//  1. direct global->LDS loads of the block's 16 weight rows over the chunk,
//     the tile's R and y over the chunk, and Wnorm; a tile row holds the
//     chunk's 16-byte pieces with piece c in slot c ^ (row & 7), so the
//     16-row MFMA fragment reads spread over the banks;
//  2. COMBINE (iw in fp64 kept as an fp32 hi + lo pair), the chunk's sum of
//     squares per token, R2 out (block 0 only), and the bf16 activation
//     R2*(1+Wnorm) written over R in LDS;
//  3. partial = W_block . act^T on v_mfma_f32_16x16x32_bf16, the chunk's k
//     steps split over the 4 waves and summed through LDS in a fixed order;
//  4. wave 0 stores the partial and the sums of squares, then arrives at the
//     block's counter; the last arrival stages the block's nkc partials in LDS
//     (one round trip), sums them per stream in chunk order, scales stream s
//     by rrms[s] = 1/sqrt(sum of squares/HS + eps), and writes h =
//     SiLU(v/HC) (down blocks), inj_next (the inject block) and rrms (block
//     0). Every chunk's sums of squares are recomputed by each block, so the
//     blocks form bit-identical rrms.
// ---------------------------------------------------------------------------
template <int TM, bool PERSIST, bool WNT = false>
__device__ __forceinline__ void fuse_down(const FuseArgs& a, int bx, int tile) {
  constexpr int ROWB = kFuseUmax * 128 * 2;  // LDS bytes of one tile row (widest chunk)
  constexpr int NTB = TM / 16;
  constexpr int TPR = 256 / TM;  // combine threads per token row
  extern __shared__ __attribute__((aligned(1024))) uint8_t dl[];
  uint8_t* rl = dl;                 // [TM][cpr] R, then the activation
  uint8_t* yl = rl + TM * ROWB;     // [TM][cpr] y; later the wave sums and the staged partials
  uint8_t* wl = yl + TM * ROWB;     // [16][cpr] weight rows; later the staged sums of squares
  uint8_t* wnl = wl + 16 * ROWB;    // [cpr] Wnorm (2 KB slot)
  float* iwh = reinterpret_cast<float*>(wnl + 2048);
  float* iwl = iwh + TM;
  float* ssl = iwl + TM;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int chunk = bx % a.nkc;
  const int blk = bx / a.nkc;
  const int64_t m0 = (int64_t)tile * TM;
  const int rows = (int)min((int64_t)TM, a.M - m0);
  const int s = chunk / a.kcps, ci = chunk - s * a.kcps;
  const int u0 = ci * a.U / a.kcps, u1 = (ci + 1) * a.U / a.kcps;
  const int cst = u0 * 128;         // first column of the chunk inside stream s
  const int cpr = (u1 - u0) * 16;   // 16-byte pieces per tile row: a multiple of 16
  const int HS = a.HS;
  const uint32_t rowb = (uint32_t)a.K * 2u;
  const uint32_t kcol = (uint32_t)(s * HS + cst) * 2u;  // byte column of the chunk in an R or weight row
  const bool lead = blk == 0;
  const bool inject = blk * 16 >= a.r;  // r is a multiple of 16: the last block holds the HC inject rows

  // 0. injection logit of token tid (issued before the bulk loads)
  const uint16_t injb = (a.inj && tid < TM) ? a.inj[(m0 + min(tid, rows - 1)) * a.ld_inj + s] : (uint16_t)0;

  // 1. global -> LDS. Weights: 16 rows x cpr pieces, exactly cpr/4 instructions.
  const uint16_t* wbase = inject ? (a.w1 ? a.w1 : a.w0 + (size_t)a.r * (size_t)a.K) : a.w0 + (size_t)blk * 16 * (size_t)a.K;
  const rsrc_t rW = make_rsrc(wbase, (uint32_t)(inject ? a.HC : 16) * rowb);  // rows past HC read as zero
  for (int i = wave; i < cpr / 4; i += 4) {
    const int q = i * 64 + lane, row = q / cpr, sl = q - row * cpr;
    const uint32_t woff = (uint32_t)row * rowb + kcol + (uint32_t)(sl ^ (row & 7)) * 16u;
    if constexpr (WNT)  // streamed: one token tile, each weight line read once per call
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rW, (lds_void_t*)(wl + i * 1024), 16, woff, 0, 0, kNonTemporal);
    else
      lds_load16(rW, wl + i * 1024, woff);
  }
  // R and y: the valid rows only (pieces of rows past M read as zero)
  const rsrc_t rR = make_rsrc(a.R + m0 * a.K, (uint32_t)rows * rowb);
  const rsrc_t rY = make_rsrc_opt(a.y, m0 * HS, (uint32_t)rows * (uint32_t)HS * 2u);
  const int na = (rows * cpr + 63) / 64;
  for (int i = wave; i < na; i += 4) {
    const int q = i * 64 + lane, t = q / cpr, sl = q - t * cpr;
    const uint32_t c16 = (uint32_t)(sl ^ (t & 7)) * 16u;
    lds_load16(rR, rl + i * 1024, (uint32_t)t * rowb + kcol + c16);
    lds_load16(rY, yl + i * 1024, (uint32_t)t * (uint32_t)HS * 2u + (uint32_t)cst * 2u + c16);
  }
  const rsrc_t rWn = make_rsrc(a.wn, a.folded ? 0u : (uint32_t)(a.wn_full ? a.K : HS) * 2u);  // folded: reads 0
  if (wave == 0) {
    for (int i = 0; i * 64 < cpr; ++i) {
      const int q = i * 64 + lane;
      const uint32_t off = (uint32_t)((a.wn_full ? s * HS : 0) + cst + q * 8) * 2u;
      lds_load16(rWn, wnl + i * 1024, q < cpr ? off : kOutOfRange);
    }
  }
  // (COMBINE) iw = 2*sigmoid(inj/HC) in fp64 while the loads are in flight
  if (tid < TM) {
    double v = 0.0;
    if (tid < rows) v = 2.0 / (1.0 + exp(-(double)bf1(injb) / (double)a.HC));
    const float hi = (float)v;
    iwh[tid] = hi;
    iwl[tid] = (float)(v - (double)hi);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // 2. (COMBINE, N) thread -> token row t, pieces sub, sub + TPR, ...
  {
    const int t = tid / TPR, sub = tid - t * TPR;
    const rsrc_t rR2 = make_rsrc_opt(a.R2, m0 * a.K, lead ? (uint32_t)rows * rowb : 0u);
    float ss = 0.0f;
    if (t < rows) {
      const float ih = iwh[t], il = iwl[t];
      // batches of PB pieces: every LDS read of a batch is issued before its math
      constexpr int PB = kFuseUmax;
      for (int b0 = sub; b0 < cpr; b0 += PB * TPR) {
        uint4 rv[PB], yv[PB], wv[PB];
#pragma unroll
        for (int p = 0; p < PB; ++p) {
          const int sl = min(b0 + p * TPR, cpr - 1);  // clamped: the read stays inside the row
          rv[p] = ld16(rl + (t * cpr + sl) * 16);
          yv[p] = ld16(yl + (t * cpr + sl) * 16);
          wv[p] = ld16(wnl + (sl ^ (t & 7)) * 16);
        }
#pragma unroll
        for (int p = 0; p < PB; ++p) {
          const int sl = b0 + p * TPR;
          if (sl >= cpr) break;
          const int c = sl ^ (t & 7);
          const uint32_t rw[4] = {rv[p].x, rv[p].y, rv[p].z, rv[p].w};
          const uint32_t yw[4] = {yv[p].x, yv[p].y, yv[p].z, yv[p].w};
          const uint32_t ww[4] = {wv[p].x, wv[p].y, wv[p].z, wv[p].w};
          uint32_t o2[4], ou[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float r0 = fmaf(bf_lo(yw[e]), il, fmaf(bf_lo(yw[e]), ih, bf_lo(rw[e])));
            const float r1 = fmaf(bf_hi(yw[e]), il, fmaf(bf_hi(yw[e]), ih, bf_hi(rw[e])));
            ss = fmaf(r0, r0, ss);
            ss = fmaf(r1, r1, ss);
            o2[e] = pack_bf2(r0, r1);
            ou[e] = pack_bf2(r0 * (1.0f + bf_lo(ww[e])), r1 * (1.0f + bf_hi(ww[e])));
          }
          bst16_p<PERSIST>(rR2, (uint32_t)t * rowb + kcol + (uint32_t)c * 16u, make_uint4(o2[0], o2[1], o2[2], o2[3]));
          st16(rl + (t * cpr + sl) * 16, make_uint4(ou[0], ou[1], ou[2], ou[3]));
        }
      }
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) ss += __shfl_xor(ss, o, 64);
    if (sub == 0) ssl[t] = ss;
  }
  // persistent plan: the up role reads R2 in the same kernel, so every R2
  // store completes before this workgroup can arrive at its block counter
  if (PERSIST) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // 3. (G1, INJ) partial product of the block over the chunk: wave w takes k
  //    steps [w*kq, (w+1)*kq) of 32 columns
  const int kq = cpr / 16;
  const int arow = lane & 15, kg = lane >> 4;
  f32x4_t acc[NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) acc[tb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  {
    // every fragment of the wave's (at most kFuseUmax) k steps is read before the first MFMA
    uint4 af[kFuseUmax], bfr[kFuseUmax][NTB];
#pragma unroll
    for (int jj = 0; jj < kFuseUmax; ++jj) {
      const int c = (wave * kq + min(jj, kq - 1)) * 4 + kg;
      af[jj] = ld16(wl + (arow * cpr + (c ^ (arow & 7))) * 16);
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        const int tt = tb * 16 + arow;
        bfr[jj][tb] = ld16(rl + (tt * cpr + (c ^ (tt & 7))) * 16);
      }
    }
#pragma unroll
    for (int jj = 0; jj < kFuseUmax; ++jj) {
      if (jj >= kq) break;
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) acc[tb] = mfma16(af[jj], bfr[jj][tb], acc[tb]);
    }
  }
  float* red = reinterpret_cast<float*>(yl);  // y is no longer read
  if (wave > 0) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
      *reinterpret_cast<f32x4_t*>(red + (((wave - 1) * NTB + tb) * 64 + lane) * 4) = acc[tb];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 1; w < 4; ++w)
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
      acc[tb] += *reinterpret_cast<const f32x4_t*>(red + (((w - 1) * NTB + tb) * 64 + lane) * 4);

  // 4. publish the chunk's partial and sums of squares (agent-coherent
  //    stores), wait for them to complete, then arrive. The counter update is
  //    an agent-scope vector atomic; the last arrival reads the partials with
  //    agent-coherent loads, so neither side needs cache maintenance.
  const int64_t grp = (int64_t)tile * a.nblk + blk;
  const rsrc_t rP = make_rsrc(a.P + grp * (int64_t)a.nkc * TM * 16, (uint32_t)(a.nkc * TM * 64));
  const rsrc_t rS = make_rsrc(a.SS + grp * (int64_t)a.nkc * TM, (uint32_t)(a.nkc * TM * 4));
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) bst16_agent(rP, (uint32_t)(((chunk * TM + tb * 16 + arow) * 16 + 4 * kg) * 4), acc[tb]);
  if (lane < TM) bst4_agent(rS, (uint32_t)((chunk * TM + lane) * 4), ssl[lane]);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  uint32_t old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(slot(a.ctr, grp), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0, 64);
  if (old != (uint32_t)(a.nkc - 1)) return;

  // last arrival: the block's nkc partials -> y area, sums of squares -> weight area
  for (int i = 0; i < a.nkc * TM / 16; ++i) lds_load16_agent(rP, yl + i * 1024, (uint32_t)(i * 64 + lane) * 16u);
  for (int i = 0; i * 256 < a.nkc * TM; ++i) lds_load16_agent(rS, wl + i * 1024, (uint32_t)(i * 64 + lane) * 16u);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  const float* pl = reinterpret_cast<const float*>(yl);
  const float* sq = reinterpret_cast<const float*>(wl);
  const rsrc_t rRr = make_rsrc(a.rrms + m0 * a.HC, (uint32_t)rows * (uint32_t)a.HC * 4u);
  f32x4_t v[NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) v[tb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  for (int st = 0; st < a.HC; ++st) {
    f32x4_t ps[NTB];
    float sqs[NTB];
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      ps[tb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      sqs[tb] = 0.0f;
    }
    // the stream's chunks in order, four at a time with their reads issued together
    constexpr int KB = 4;
    for (int i0 = 0; i0 < a.kcps; i0 += KB) {
      f32x4_t pv[KB][NTB];
      float sv[KB][NTB];
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int c = st * a.kcps + min(i0 + u, a.kcps - 1);
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
          const int tok = tb * 16 + arow;
          pv[u][tb] = *reinterpret_cast<const f32x4_t*>(pl + (c * TM + tok) * 16 + 4 * kg);
          sv[u][tb] = sq[c * TM + tok];
        }
      }
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        if (i0 + u >= a.kcps) break;
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
          ps[tb] += pv[u][tb];
          sqs[tb] += sv[u][tb];
        }
      }
    }
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      const int tok = tb * 16 + arow;
      const float rr = 1.0f / sqrtf(sqs[tb] * a.inv_hs + a.eps);  // (N) rrms of stream st
      v[tb] += rr * ps[tb];
      if (lead && kg == 0 && tok < rows) bst4f_p<PERSIST>(rRr, (uint32_t)(tok * a.HC + st) * 4u, rr);
    }
  }
  const rsrc_t rH = make_rsrc(a.h + m0 * a.r, (uint32_t)rows * (uint32_t)a.r * 2u);
  const rsrc_t rI = make_rsrc(a.inj_next + m0 * a.ld_inj_next, (uint32_t)((rows - 1) * a.ld_inj_next + a.HC) * 2u);
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    const int tok = tb * 16 + arow;
    if (tok >= rows) continue;
    if (!inject) {
      float hq[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float z = v[tb][q] * a.inv_hc;
        hq[q] = z * sigmoid_f(z);  // (G1) h = SiLU(lora / HC)
      }
      bst8_p<PERSIST>(rH, (uint32_t)(tok * a.r + blk * 16 + 4 * kg) * 2u,
                      make_uint2(pack_bf2(hq[0], hq[1]), pack_bf2(hq[2], hq[3])));
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)  // (INJ), not scaled
        if (4 * kg + q < a.HC) bst2_p<PERSIST>(rI, (uint32_t)(tok * a.ld_inj_next + 4 * kg + q) * 2u, to_bf(v[tb][q]));
    }
  }
  if (PERSIST) {
    // h (and, from block 0, rrms) complete before the tile's "h complete" count
    // moves; the arrival that completes it raises the tile's ready flag
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (lane == 0 &&
        __hip_atomic_fetch_add(slot(a.hdone, tile), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(a.nblk - 1))
      __hip_atomic_store(slot(a.ready, tile), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (lane == 0) __hip_atomic_store(slot(a.ctr, grp), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int TM, bool WNT = false>
__global__ __launch_bounds__(256) void hcgr_k1_fuse(FuseArgs a) {
  fuse_down<TM, false, WNT>(a, (int)blockIdx.x, (int)blockIdx.y);
}

// ---------------------------------------------------------------------------
// hcgr_k2_decg: (G2) gate = h . Wu^T, G = sigmoid(gate), (MIX) x[c] =
// (1/HC) sum_s G[s,c] xn[s,c], for a token tile of TM tokens and CW = NW *
// 16/HC channels x HC streams, NW waves. Wave w's 16 MFMA rows are 16/HC
// channels x HC streams: row i is stream i % HC of channel w*16/HC + i/HC
// (Wu row s*HS + c). Lane l then holds rows 4(l/16) .. 4(l/16)+3 for token
// l % 16: whole channels (HC <= 4: MIX is lane-local) or half of one channel's
// eight streams (HC = 8: the halves meet by one cross-lane add). The
// workgroup's Wu rows, the h tile and the epilogue operands (its R2 rows of
// those channels, rrms, Wnorm) arrive in LDS by direct global->LDS loads; a
// Wu or h row keeps its 16-byte piece c in slot (c & ~3) | ((c ^ row) & 3).
// Channel groups that share a 128-byte line of R2 or x run on one XCD.
// ---------------------------------------------------------------------------
struct DecUpArgs {
  const uint16_t* h;
  int64_t M;
  int r, HS, K;
  const uint16_t* wu;
  const uint16_t* R2;
  const float* rrms;
  const uint16_t* wn;
  int wn_full;
  uint16_t* x;
  // persistent plan only (counter slot arrays)
  uint32_t* hdone;  // [tiles] published blocks of h per token tile
  uint32_t* ready;  // [tiles] raised when the tile's h is complete
  uint32_t* exitc;  // [tiles] up workgroups past their wait
  uint32_t* err;    // raised by a wait that gave up
  int polls;        // poll budget of that wait
};

// LDS of the up role: Wu rows, h tile, R2 rows, rrms, Wnorm, a flag word.
template <int HC, int TM, int NW>
struct DecgLds {
  static constexpr int CW = NW * (16 / HC);
  static constexpr int R2B = (TM * HC * CW * 2 + 1023) / 1024 * 1024, RRB = (TM * HC * 4 + 1023) / 1024 * 1024;
  static constexpr int WNB = (HC * CW * 2 + 1023) / 1024 * 1024;
  static size_t bytes(int r) { return k2_decg_lds(HC, TM, r, NW); }
};

template <int HC, int TM, int NW, bool PERSIST, bool WNT = false>
__device__ __forceinline__ void decg_up(const DecUpArgs& a, int bx, int tile, int ncg) {
  using L = DecgLds<HC, TM, NW>;
  constexpr int CPW = 16 / HC, CW = L::CW, WR = NW * 16;
  constexpr int NTB = TM / 16;
  // the epilogue's R2 rows and Wnorm arrive in pieces of PB bytes: 16 when the
  // workgroup's CW channels of a stream are whole 16-byte pieces, else 4
  constexpr int PB = CW % 8 == 0 ? 16 : 4;
  constexpr int CHP = CW * 2 / PB;  // pieces per (token, stream) row of CW channels
  static_assert(CW % 2 == 0 && HC * CHP <= 64, "whole pieces of R2 and Wnorm per stream, one load for Wnorm");
  extern __shared__ __attribute__((aligned(1024))) uint8_t dl[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = lane >> 4;
  const int64_t m0 = (int64_t)tile * TM;
  const int rows = (int)min((int64_t)TM, a.M - m0);
  // workgroup x runs on XCD x % 8: when the group count allows, XCD k takes a
  // contiguous run of channel groups (neighbours share R2 and x lines)
  const int cg = (ncg & 7) ? bx : (bx & 7) * (ncg >> 3) + (bx >> 3);
  const int cbase = cg * CW;
  const int cpr = a.r / 8;  // 16-byte pieces per Wu or h row (a multiple of 4)
  const uint32_t rowb = (uint32_t)a.r * 2u;
  uint8_t* wl = dl;                   // [WR][r]
  uint8_t* hl = wl + WR * rowb;       // [TM][r]
  uint8_t* r2l = hl + TM * rowb;      // [TM][HC][CW] bf16
  uint8_t* rrl = r2l + L::R2B;        // [TM][HC] float
  uint8_t* wnl = rrl + L::RRB;        // [HC or 1][CW] bf16
  int* flag = reinterpret_cast<int*>(wnl + L::WNB);
  const rsrc_t rWu = make_rsrc(a.wu, (uint32_t)a.K * rowb);
  const rsrc_t rWn = make_rsrc(a.wn, (uint32_t)(a.wn_full ? a.K : a.HS) * 2u);

  // weights first: the persistent plan's wait overlaps them
  for (int i = wave; i * 64 < WR * cpr; i += NW) {
    const int q = i * 64 + lane, row = q / cpr, sl = q - row * cpr;
    const int c = (sl & ~3) | ((sl ^ row) & 3);
    const int i16 = row & 15;
    const int ch = cbase + (row >> 4) * CPW + i16 / HC, st = i16 % HC;
    const uint32_t off = (uint32_t)(st * a.HS + ch) * rowb + (uint32_t)c * 16u;
    if constexpr (WNT)  // streamed: a grid of one or two token tiles (split launch)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rWu, (lds_void_t*)(wl + i * 1024), 16, off, 0, 0, kNonTemporal);
    else
      lds_load16(rWu, wl + i * 1024, off);
  }
  if (wave == 0) {
    const int nwn = a.wn_full ? HC * CHP : CHP;
    const uint32_t wo = (uint32_t)((a.wn_full ? (lane / CHP) * a.HS : 0) + cbase + (lane % CHP) * (PB / 2)) * 2u;
    if constexpr (PB == 16) lds_load16(rWn, wnl, lane < nwn ? wo : kOutOfRange);
    else lds_load4_p<false>(rWn, wnl, lane < nwn ? wo : kOutOfRange);
  }
  if (PERSIST) {
    if (tid == 0) *flag = wait_flag(slot(a.ready, tile), a.err, a.polls) ? 1 : 0;
    __syncthreads();
  }
  const rsrc_t rH = make_rsrc(a.h + m0 * a.r, (uint32_t)rows * rowb);  // rows past M read as zero
  const rsrc_t rR2 = make_rsrc(a.R2 + m0 * a.K, (uint32_t)rows * (uint32_t)a.K * 2u);
  const rsrc_t rRr = make_rsrc(a.rrms + m0 * HC, (uint32_t)rows * HC * 4u);
  for (int i = wave; i * 64 < TM * cpr; i += NW) {
    const int q = i * 64 + lane, row = q / cpr, sl = q - row * cpr;
    const int c = (sl & ~3) | ((sl ^ row) & 3);
    lds_load16_p<PERSIST>(rH, hl + i * 1024, (uint32_t)row * rowb + (uint32_t)c * 16u);
  }
  constexpr int NR2 = TM * HC * CHP;  // pieces of the tile's R2 rows
  for (int i = wave; i * 64 < NR2; i += NW) {
    const int q = i * 64 + lane, t = q / (HC * CHP), st = (q / CHP) % HC, pc = q % CHP;
    const uint32_t off = (uint32_t)t * (uint32_t)a.K * 2u + (uint32_t)(st * a.HS + cbase + pc * (PB / 2)) * 2u;
    if constexpr (PB == 16) lds_load16_p<PERSIST>(rR2, r2l + i * 1024, q < NR2 ? off : kOutOfRange);
    else lds_load4_p<PERSIST>(rR2, r2l + i * 256, q < NR2 ? off : kOutOfRange);
  }
  if (wave == 0)
    for (int i = 0; i * 64 < TM * HC / 4; ++i) lds_load16_p<PERSIST>(rRr, rrl + i * 1024, (uint32_t)(i * 64 + lane) * 16u);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lds_sync();  // every wave's global->LDS loads have landed

  // epilogue operands of the lane's four rows: channel chl (in the
  // workgroup), stream st
  float pr2[NTB][4], prr[NTB][4], pone[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i16 = 4 * kg + q, chl = wave * CPW + i16 / HC, st = i16 % HC;
    pone[q] = 1.0f + bf1(*reinterpret_cast<const uint16_t*>(wnl + ((a.wn_full ? st * CW : 0) + chl) * 2));
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      const int t = tb * 16 + (lane & 15);
      pr2[tb][q] = bf1(*reinterpret_cast<const uint16_t*>(r2l + ((t * HC + st) * CW + chl) * 2));
      prr[tb][q] = *reinterpret_cast<const float*>(rrl + (t * HC + st) * 4);
    }
  }

  f32x4_t acc[NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) acc[tb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int arow = wave * 16 + (lane & 15);
  const int nj = a.r / 32;
  auto kstep = [&](int j, uint4& af, uint4 (&bf)[NTB]) {  // fragments of k step j
    af = ld16(wl + arow * rowb + (uint32_t)(j * 4 + ((kg ^ arow) & 3)) * 16u);
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      const int t = tb * 16 + (lane & 15);
      bf[tb] = ld16(hl + t * rowb + (uint32_t)(j * 4 + ((kg ^ t) & 3)) * 16u);
    }
  };
  int j = 0;
  for (; j + 2 <= nj; j += 2) {  // two k steps' fragments in flight per round trip
    uint4 a0, a1, b0[NTB], b1[NTB];
    kstep(j, a0, b0);
    kstep(j + 1, a1, b1);
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) acc[tb] = mfma16(a1, b1[tb], mfma16(a0, b0[tb], acc[tb]));
  }
  if (j < nj) {
    uint4 a0, b0[NTB];
    kstep(j, a0, b0);
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) acc[tb] = mfma16(a0, b0[tb], acc[tb]);
  }

  constexpr float inv = 1.0f / HC;
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    const int64_t m = m0 + tb * 16 + (lane & 15);
    float g[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) g[q] = sigmoid_f(acc[tb][q]) * (pr2[tb][q] * prr[tb][q] * pone[q]);  // G * xn
    uint16_t* xr = a.x + m * a.HS + cbase + wave * CPW;
    if constexpr (HC == 1) {
      if (m < a.M) *reinterpret_cast<uint2*>(xr + 4 * kg) = make_uint2(pack_bf2(g[0], g[1]), pack_bf2(g[2], g[3]));
    } else if constexpr (HC == 2) {
      if (m < a.M) *reinterpret_cast<uint32_t*>(xr + 2 * kg) = pack_bf2((g[0] + g[1]) * inv, (g[2] + g[3]) * inv);
    } else if constexpr (HC == 4) {
      if (m < a.M) xr[kg] = to_bf(((g[0] + g[1]) + (g[2] + g[3])) * inv);
    } else {
      float part = (g[0] + g[1]) + (g[2] + g[3]);  // streams 4(kg&1) .. +3 of channel kg/2
      part += __shfl_xor(part, 16, 64);
      if (m < a.M && (kg & 1) == 0) xr[kg >> 1] = to_bf(part * inv);
    }
  }
  if (PERSIST && tid == 0) {
    // the tile's last up workgroup returns the tile's counters to zero (its
    // round trip overlaps the x stores: nothing after it waits for it)
    if (__hip_atomic_fetch_add(slot(a.exitc, tile), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(ncg - 1)) {
      __hip_atomic_store(slot(a.hdone, tile), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(slot(a.ready, tile), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(slot(a.exitc, tile), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int HC, int TM, int NW, bool WNT = false>
__global__ __launch_bounds__(64 * NW) void hcgr_k2_decg(DecUpArgs a) {
  decg_up<HC, TM, NW, false, WNT>(a, (int)blockIdx.x, (int)blockIdx.y, (int)gridDim.x);
}

// ---------------------------------------------------------------------------
// hcgr_dec_persist: the persistent decode plan in one launch. Workgroups
// [0, ndown) run the down role (block x chunk x token tile, as hcgr_k1_fuse);
// the ncg channel groups x token tiles after them run the up role with four
// waves. Workgroups are dispatched in increasing index order, so every down
// workgroup is resident or finished before any up workgroup starts to wait,
// and each wait is also bounded.
// ---------------------------------------------------------------------------
template <int HC, int TM, bool WNT = false>
__global__ __launch_bounds__(256) void hcgr_dec_persist(FuseArgs a, DecUpArgs u, int ndown_tile, int ntiles, int ncg) {
  const int b = (int)blockIdx.x;
  if (b < ndown_tile * ntiles) {
    fuse_down<TM, true, WNT>(a, b % ndown_tile, b / ndown_tile);
  } else {
    const int j = b - ndown_tile * ntiles;
    decg_up<HC, TM, 4, true>(u, j % ncg, j / ncg, ncg);
  }
}

// ---------------------------------------------------------------------------
// Host side.
template <typename F, typename... Args>
static void klaunch_d(F k, dim3 grid, dim3 block, size_t lds, hipStream_t st, const hipEvent_t* ev, Args... args) {
  hipExtLaunchKernelGGL(k, grid, block, (uint32_t)lds, st, ev ? ev[0] : nullptr, ev ? ev[1] : nullptr, 0u, args...);
}

// the up kernel's wave counts: HC waves up to 4, and five as well at HC = 8
// (decg_waves picks by HS)
constexpr int decg_nw(int hc) { return hc < 4 ? hc : 4; }

template <int HC, int TM>
static hipError_t set_decg_lds() {
  hipError_t e = hipFuncSetAttribute((const void*)hcgr_k2_decg<HC, TM, decg_nw(HC)>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsPerCu);
  if (e == hipSuccess && HC < 4)
    e = hipFuncSetAttribute((const void*)hcgr_k2_decg<HC, TM, decg_nw(HC), true>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsPerCu);
  if (e == hipSuccess && HC == 8)
    e = hipFuncSetAttribute((const void*)hcgr_k2_decg<HC, TM, 5>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)kLdsPerCu);
  return e;
}

template <int HC, int TM>
static hipError_t set_decode_lds() {
  hipError_t e = set_decg_lds<HC, TM>();
  if (e == hipSuccess)
    e = hipFuncSetAttribute((const void*)hcgr_dec_persist<HC, TM>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)kLdsPerCu);
  if (e == hipSuccess)
    e = hipFuncSetAttribute((const void*)hcgr_dec_persist<HC, TM, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)kLdsPerCu);
  return e;
}

template <int HC>
static hipError_t set_decg64_lds() {
  return set_decg_lds<HC, 64>();
}

int configure_decode_kernels() {
  hipError_t e;
  if ((e = hipFuncSetAttribute((const void*)hcgr_k1_fuse<16>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)k1_fuse_lds(16))) != hipSuccess) return (int)e;
  if ((e = hipFuncSetAttribute((const void*)hcgr_k1_fuse<32>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)k1_fuse_lds(32))) != hipSuccess) return (int)e;
  if ((e = hipFuncSetAttribute((const void*)hcgr_k1_fuse<16, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)k1_fuse_lds(16))) != hipSuccess) return (int)e;
  if ((e = hipFuncSetAttribute((const void*)hcgr_k1_fuse<32, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)k1_fuse_lds(32))) != hipSuccess) return (int)e;
  if ((e = set_decode_lds<1, 16>()) != hipSuccess || (e = set_decode_lds<1, 32>()) != hipSuccess ||
      (e = set_decode_lds<2, 16>()) != hipSuccess || (e = set_decode_lds<2, 32>()) != hipSuccess ||
      (e = set_decode_lds<4, 16>()) != hipSuccess || (e = set_decode_lds<4, 32>()) != hipSuccess ||
      (e = set_decode_lds<8, 16>()) != hipSuccess || (e = set_decode_lds<8, 32>()) != hipSuccess)
    return (int)e;
  // 64-token tiles of the up kernel (the split plan's 64-token down tiles)
  if ((e = set_decg64_lds<1>()) != hipSuccess || (e = set_decg64_lds<2>()) != hipSuccess ||
      (e = set_decg64_lds<4>()) != hipSuccess || (e = set_decg64_lds<8>()) != hipSuccess)
    return (int)e;
  return (int)hipSuccess;
}

template <int TM>
static void launch_decg(int hc, int nw, const DecUpArgs& u, dim3 g, size_t lds, hipStream_t st, const hipEvent_t* ev,
                        bool wnt = false);

int launch_decg_up(const Shape& s, int tm, const uint16_t* H, const ForwardArgs& f, void* stream, void* const* events) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const hipEvent_t* ev = reinterpret_cast<const hipEvent_t*>(events);
  DecUpArgs u;
  u.h = H; u.M = f.M; u.r = s.r; u.HS = s.hs; u.K = (int)s.k(); u.wu = f.wu; u.R2 = f.res; u.rrms = f.rrms;
  u.wn = f.wnorm; u.wn_full = s.wn_full ? 1 : 0; u.x = f.x;
  u.hdone = u.ready = u.exitc = u.err = nullptr; u.polls = 0;
  const int nw = decg_waves(s.hc, s.hs);
  const dim3 g((unsigned)(s.hs / decg_channels(s.hc, nw)), (unsigned)cdiv(f.M, (int64_t)tm));
  const size_t lds = k2_decg_lds(s.hc, tm, s.r, nw);
  // Wu streamed (the non-temporal policy) at HC = 1 and 2 with one or two
  // token tiles: measured per call on MI355X, 0.64 us less at HC = 1, M = 32
  // and 0.23 at HC = 2, M = 32 (two 16-token tiles), level at M = 1; at HC =
  // 8 streaming was 0.4-0.6 us slower even with one tile
  const bool wnt = s.hc < 4 && g.y <= 2;
  if (tm == 16) launch_decg<16>(s.hc, nw, u, g, lds, st, ev, wnt);
  else if (tm == 32) launch_decg<32>(s.hc, nw, u, g, lds, st, ev, wnt);
  else launch_decg<64>(s.hc, nw, u, g, lds, st, ev, wnt);
  return (int)hipGetLastError();
}

// wnt: Wu streamed (HC = 1 and 2 only; the split launch decides)
template <int TM>
static void launch_decg(int hc, int nw, const DecUpArgs& u, dim3 g, size_t lds, hipStream_t st, const hipEvent_t* ev,
                        bool wnt) {
  switch (hc) {
    case 1:
      if (wnt) klaunch_d(hcgr_k2_decg<1, TM, 1, true>, g, dim3(64), lds, st, ev, u);
      else klaunch_d(hcgr_k2_decg<1, TM, 1>, g, dim3(64), lds, st, ev, u);
      break;
    case 2:
      if (wnt) klaunch_d(hcgr_k2_decg<2, TM, 2, true>, g, dim3(128), lds, st, ev, u);
      else klaunch_d(hcgr_k2_decg<2, TM, 2>, g, dim3(128), lds, st, ev, u);
      break;
    case 4: klaunch_d(hcgr_k2_decg<4, TM, 4>, g, dim3(256), lds, st, ev, u); break;
    default:
      if (nw == 5) klaunch_d(hcgr_k2_decg<8, TM, 5>, g, dim3(320), lds, st, ev, u);
      else klaunch_d(hcgr_k2_decg<8, TM, 4>, g, dim3(256), lds, st, ev, u);
      break;
  }
}

template <int TM>
static void launch_persist(int hc, const FuseArgs& a, const DecUpArgs& u, int ndt, int nt, int ncg, size_t lds,
                           hipStream_t st, const hipEvent_t* ev) {
  const dim3 g((unsigned)((ndt + ncg) * nt)), b(256);
  // weights streamed with one token tile (see the fused launch below)
  auto run = [&](auto k, auto k_wnt) {
    if (nt == 1) klaunch_d(k_wnt, g, b, lds, st, ev, a, u, ndt, nt, ncg);
    else klaunch_d(k, g, b, lds, st, ev, a, u, ndt, nt, ncg);
  };
  switch (hc) {
    case 1: run(hcgr_dec_persist<1, TM, false>, hcgr_dec_persist<1, TM, true>); break;
    case 2: run(hcgr_dec_persist<2, TM, false>, hcgr_dec_persist<2, TM, true>); break;
    case 4: run(hcgr_dec_persist<4, TM, false>, hcgr_dec_persist<4, TM, true>); break;
    default: run(hcgr_dec_persist<8, TM, false>, hcgr_dec_persist<8, TM, true>); break;
  }
}

int launch_fused(const Shape& s, const Plan& p, const ForwardArgs& f, void* stream, void* const* events) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const hipEvent_t* ev = reinterpret_cast<const hipEvent_t*>(events);
  char* ws = static_cast<char*>(f.ws);
  uint16_t* H = reinterpret_cast<uint16_t*>(ws + p.off_h);
  uint32_t* ctr = reinterpret_cast<uint32_t*>(ws);
  const int K = (int)s.k();
  FuseArgs a;
  a.R = f.R; a.y = f.y; a.inj = f.inj; a.ld_inj = f.ld_inj;
  a.wn = f.wnorm; a.wn_full = s.wn_full ? 1 : 0; a.folded = s.merged ? 1 : 0;
  a.w0 = f.wd; a.w1 = s.merged ? nullptr : f.wi;
  a.M = f.M; a.K = K; a.HS = s.hs; a.HC = s.hc; a.r = s.r; a.nblk = s.nblk();
  a.U = s.hs / 128; a.kcps = p.kcps; a.nkc = p.nkc;
  a.eps = s.eps; a.inv_hc = 1.0f / (float)s.hc; a.inv_hs = 1.0f / (float)s.hs;
  a.R2 = f.R2; a.rrms = f.rrms; a.h = H; a.inj_next = f.inj_next; a.ld_inj_next = f.ld_inj_next;
  a.P = reinterpret_cast<float*>(ws + p.off_p);
  a.SS = reinterpret_cast<float*>(ws + p.off_ss);
  a.ctr = ctr;
  a.hdone = ctr + kHdoneSlot * kCtrStride;
  a.ready = ctr + kReadySlot * kCtrStride;
  DecUpArgs u;
  u.h = H; u.M = f.M; u.r = s.r; u.HS = s.hs; u.K = K; u.wu = f.wu; u.R2 = f.res; u.rrms = f.rrms;
  u.wn = f.wnorm; u.wn_full = s.wn_full ? 1 : 0; u.x = f.x;
  u.hdone = ctr + kHdoneSlot * kCtrStride; u.ready = ctr + kReadySlot * kCtrStride;
  u.exitc = ctr + kExitSlot * kCtrStride; u.err = ctr + kErrSlot * kCtrStride; u.polls = f.wait_polls;
  hipError_t e;
  if (p.kind == PLAN_PERSIST) {
    const size_t lds = k1_fuse_lds(p.tm) > k2_decg_lds(s.hc, p.tm, s.r, 4) ? k1_fuse_lds(p.tm)
                                                                           : k2_decg_lds(s.hc, p.tm, s.r, 4);
    const int ndt = s.nblk() * p.nkc, ncg = s.hs / p.cb;
    if (p.tm == 16) launch_persist<16>(s.hc, a, u, ndt, p.ntiles, ncg, lds, st, ev);
    else launch_persist<32>(s.hc, a, u, ndt, p.ntiles, ncg, lds, st, ev);
    if ((e = hipGetLastError()) != hipSuccess) return (int)e;
    if (ev) {  // one kernel: empty intervals for the other two stages
      for (int i = 2; i < 6; ++i)
        if ((e = hipEventRecord(ev[i], st)) != hipSuccess) return (int)e;
    }
    return (int)hipSuccess;
  }
  // weight rows streamed (the non-temporal policy) with one token tile, where
  // each weight line is read once per call: measured per call on MI355X
  // against the cached loads (two sessions), fused plan 0.47-0.54 us less at
  // HC = 4, M = 1, 0.38-0.41 at HC = 2, M = 1 and 8, 0.02-0.32 at HC = 1,
  // M = 1..16; persistent plan 0.39-0.43, 0.34-0.46 and 0.02-0.23
  const dim3 g1((unsigned)(s.nblk() * p.nkc), (unsigned)p.ntiles);
  const bool wnt = p.ntiles == 1;
  if (p.tm == 16) {
    if (wnt) klaunch_d(hcgr_k1_fuse<16, true>, g1, dim3(256), k1_fuse_lds(16), st, ev, a);
    else klaunch_d(hcgr_k1_fuse<16>, g1, dim3(256), k1_fuse_lds(16), st, ev, a);
  } else {
    if (wnt) klaunch_d(hcgr_k1_fuse<32, true>, g1, dim3(256), k1_fuse_lds(32), st, ev, a);
    else klaunch_d(hcgr_k1_fuse<32>, g1, dim3(256), k1_fuse_lds(32), st, ev, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  if (ev) {  // no middle kernel: an empty interval right after the down kernel
    if ((e = hipEventRecord(ev[2], st)) != hipSuccess || (e = hipEventRecord(ev[3], st)) != hipSuccess) return (int)e;
  }
  const dim3 g2((unsigned)(s.hs / p.cb), (unsigned)p.ntiles);
  const size_t lds = k2_decg_lds(s.hc, p.tm, s.r, p.upw);
  if (p.tm == 16) launch_decg<16>(s.hc, p.upw, u, g2, lds, st, ev ? ev + 4 : nullptr);
  else launch_decg<32>(s.hc, p.upw, u, g2, lds, st, ev ? ev + 4 : nullptr);
  return (int)hipGetLastError();
}

}  // namespace hcgr
