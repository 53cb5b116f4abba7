// hcgr_kernels.hip -- gfx950 kernels of the Hyper-Connection Gated Residual
// op (ROCm/aiter pull request #5913, "Two-stage Hyper-Connection Gated
// Residual kernel", section "Technical Details": COMBINE, N, G1, G2, MIX, INJ).
//
// Matrix work runs on v_mfma_f32_16x16x32_bf16 (wave64). Operand layout used
// throughout (A is 16 rows x 32 k, B is 32 k x 16 columns, D is 16 x 16):
//   lane l holds A[l % 16][8*(l/16) .. 8*(l/16)+7] and B[same k][l % 16] as
//   8 bf16 (16 bytes), and D[4*(l/16) + q][l % 16] in accumulator q = 0..3.
// A and B use the same k order, so any internal k permutation of the
// instruction cancels; only the row/column assignment matters.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include <functional>
#include <type_traits>

#include "hcgr_device.h"
#include "hcgr_internal.h"

namespace hcgr {

struct DownArgs {
  const uint16_t* R;
  const uint16_t* y;
  const uint16_t* inj;
  int64_t ld_inj;
  const uint16_t* wn;
  int wn_full;
  const uint16_t* w0;  // Wd [r,K] or merged Wm [n_pad,K]
  const uint16_t* w1;  // Wi [HC,K], or nullptr when the inject rows are rows r.. of w0
  int folded;          // merged/folded weights: the activation omits (1 + Wnorm)
  int64_t M;
  int K, HS, HC, r, n_rows;
  int KC, nkc, NP;
  int64_t Mpad;
  float inv_hc;
  uint16_t* R2;
  float* P;   // [nkc][NP][Mpad] partial sums
  float* SS;  // [nkc][Mpad] partial sums of squares
  int wt;     // 1: P, SS and R2 are written through the L2 (decode sizes, below)
  int wnt;    // 1: the variant that reads weight rows with the non-temporal policy (a single token tile, below)
};

// ---------------------------------------------------------------------------
// hcgr_k1_dec (SPLIT plan, decode sizes): COMBINE + per-chunk sums of squares
// + unscaled partial down/inject products.
// Workgroup = (K chunk of KC columns inside one stream) x (row tile of RB
// 16-row blocks) x (token tile of TM rows). NW = RB*KW waves; wave (rb, kw)
// contracts block rb over the kw-th slice (KC/KW columns) of the chunk, and
// the KW slices are summed through LDS. Every global load the workgroup needs
// (weight fragments straight into MFMA A registers, the R/y/Wnorm chunks of
// the activation tile) is issued before any arithmetic, through range-limited
// buffer descriptors (rows past M read as zero), so the workgroup waits for
// one memory round trip; iw is formed while the loads are in flight.
// Partials P[chunk][row][token] and sums of squares SS[chunk][token] are
// stored for valid tokens only. With wt the kernel's outputs (P, SS, R2) go
// out with write-through stores (the SC1 policy), so its end does not wait
// for the write-back of their dirty L2 lines. Measured on MI355X (per call,
// the two forms interleaved): HC = 4, 0.3 us faster at M = 1 (down kernel
// 4.5 -> 4.1 us) and 0.1-0.2 us at M = 32 (5.0 -> 4.9); HC = 2, 0.25 us at
// M = 1; HC = 1 and 8, 0.05-0.2 us slower; from 64 tokens slower for every
// HC (the write-through traffic outweighs it). The launch sets it for HC = 2
// and 4 up to 32 padded tokens.
// WNT (chosen by the launch from wnt) reads the weight rows with the
// non-temporal (streaming) policy: with a single token tile every weight line is read once per call,
// and keeping it out of the caches shortens the call although this kernel's
// own time grows by 0.06-0.2 us. Measured on MI355X (whole calls back to
// back, the two forms interleaved, three sessions): per call 0.43-0.46 us
// less at HC = 4, M = 1, 0.13-0.33 at M = 32, 0.2-0.47 and 0.78-0.80 at HC
// = 8, M = 1 and 32, 0.14-0.18 at HC = 2, M = 1; HC = 4, M = 16 between
// 0.29 less and 0.15 more. With two token tiles (HC = 4, M = 64; HC = 1, M
// = 32 in 16-token tiles) it was 0.2-0.3 us slower, since the second tile
// reads the lines from HBM again. The launch takes it when the plan has one
// token tile; the other variant is the kernel's code as before.
// ---------------------------------------------------------------------------
template <int TM, int RB, int KW, int KC, bool WNT>
__global__ __launch_bounds__(RB * KW * 64) void hcgr_k1_dec(DownArgs a) {
  constexpr int NW = RB * KW;
  constexpr int NT = NW * 64;
  constexpr int KPW = KC / KW;   // columns per wave
  constexpr int NKS = KPW / 32;  // MFMA k steps per wave
  static_assert(NKS >= 1 && KPW % 32 == 0, "whole k steps per wave");
  constexpr int CPR = KC / 8;    // 16-byte chunks per token row of the tile
  constexpr int NCH = TM * CPR;
  constexpr int CPT = (NCH + NT - 1) / NT;
  constexpr int LDA = KC + 8;
  constexpr int NTB = TM / 16;

  __shared__ __attribute__((aligned(16))) uint16_t act[TM * LDA];
  __shared__ float iwh[TM], iwl[TM];
  __shared__ float ssp[NCH];
  __shared__ __attribute__((aligned(16))) float red[KW > 1 ? (KW - 1) * RB * NTB * 256 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rb = wave % RB, kw = wave / RB;
  const int kc = blockIdx.x % a.nkc;
  const int rt = blockIdx.x / a.nkc;
  const int64_t m0 = (int64_t)blockIdx.y * TM;
  const int rows = (int)min((int64_t)TM, a.M - m0);
  const int kbeg = kc * KC;
  const int s = kbeg / a.HS;
  const int cst = kbeg - s * a.HS;
  const bool lead = rt == 0;  // row tile 0 writes R2 and the sums of squares
  const int koff = 8 * (lane >> 4);
  // 0. injection logit of this thread's token (clamped row: no branch)
  const uint16_t injb = a.inj ? a.inj[(m0 + min(tid % TM, rows - 1)) * a.ld_inj + s] : (uint16_t)0;
  const uint32_t rowb = (uint32_t)a.K * 2u;
  const int nblk = (a.n_rows + 15) / 16;

  // 1. weight fragments of this wave's block (rows past the matrix read 0)
  const int nb = rt * RB + rb;
  const bool bval = nb < nblk;  // wave-uniform
  const bool down = nb * 16 < a.r || !a.w1;
  const rsrc_t rW = down ? make_rsrc(a.w0, (uint32_t)(a.w1 ? a.r : a.n_rows) * rowb)
                         : make_rsrc(a.w1, (uint32_t)a.HC * rowb);
  const uint32_t wrow = (uint32_t)((down ? nb * 16 : nb * 16 - a.r) + (lane & 15)) * rowb;
  uint4 wf[NKS];
  if constexpr (WNT) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) wf[ks] = bld16_nt(rW, wrow + (uint32_t)(kbeg + kw * KPW + ks * 32 + koff) * 2u);
  } else {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) wf[ks] = bld16(rW, wrow + (uint32_t)(kbeg + kw * KPW + ks * 32 + koff) * 2u);
  }

  // 2. activation chunks (R, y, Wnorm); a thread's chunks share one column
  const rsrc_t rR = make_rsrc(a.R + m0 * a.K, (uint32_t)rows * rowb);
  const rsrc_t rY = make_rsrc_opt(a.y, m0 * a.HS, (uint32_t)rows * (uint32_t)a.HS * 2u);
  const rsrc_t rWn = make_rsrc(a.wn, a.folded ? 0u : (uint32_t)(a.wn_full ? a.K : a.HS) * 2u);
  uint4 rv[CPT], yv[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int q = min(tid + j * NT, NCH - 1);
    const uint32_t t = q / CPR, col = (q % CPR) * 8;
    rv[j] = bld16(rR, t * rowb + (uint32_t)(kbeg + col) * 2u);
    yv[j] = bld16(rY, (t * (uint32_t)a.HS + cst + col) * 2u);
  }
  uint4 wv[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int q = min(tid + j * NT, NCH - 1);
    wv[j] = bld16(rWn, ((a.wn_full ? (uint32_t)(s * a.HS) : 0u) + cst + (q % CPR) * 8) * 2u);
  }

  // 3. (COMBINE) iw = 2*sigmoid(inj/HC) for this stream, fp64 -> fp32 hi + lo
  //    (R2 = (R + y*hi) + y*lo stays within an ulp of R2 under cancellation)
  if (tid < TM) {
    double v = 0.0;
    if (tid < rows) v = 2.0 / (1.0 + exp(-(double)bf1(injb) / (double)a.HC));
    const float hi = (float)v;
    iwh[tid] = hi;
    iwl[tid] = (float)(v - (double)hi);
  }
  __syncthreads();

  // 4. R2 = R + y*iw (fp32), sum of squares, R2 -> bf16 output, activation
  //    R2*(1+Wnorm) -> LDS (Wnorm reads as 0 for folded weights)
  const rsrc_t rR2 = make_rsrc_opt(a.R2, m0 * a.K, lead ? (uint32_t)rows * rowb : 0u);
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int q = tid + j * NT;
    if (CPT * NT > NCH && q >= NCH) break;
    const int t = q / CPR, col = (q % CPR) * 8;
    const float ih = iwh[t], il = iwl[t];
    const uint32_t rw[4] = {rv[j].x, rv[j].y, rv[j].z, rv[j].w};
    const uint32_t yw[4] = {yv[j].x, yv[j].y, yv[j].z, yv[j].w};
    const uint32_t ww[4] = {wv[j].x, wv[j].y, wv[j].z, wv[j].w};
    uint32_t o2[4], ou[4];
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float r0 = fmaf(bf_lo(yw[e]), il, fmaf(bf_lo(yw[e]), ih, bf_lo(rw[e])));
      const float r1 = fmaf(bf_hi(yw[e]), il, fmaf(bf_hi(yw[e]), ih, bf_hi(rw[e])));
      acc = fmaf(r0, r0, acc);
      acc = fmaf(r1, r1, acc);
      o2[e] = pack_bf2(r0, r1);
      ou[e] = pack_bf2(r0 * (1.0f + bf_lo(ww[e])), r1 * (1.0f + bf_hi(ww[e])));
    }
    ssp[q] = acc;
    const uint32_t o2off = (uint32_t)t * rowb + (uint32_t)(kbeg + col) * 2u;
    if (a.wt) bst16_wt(rR2, o2off, make_uint4(o2[0], o2[1], o2[2], o2[3]));
    else bst16(rR2, o2off, make_uint4(o2[0], o2[1], o2[2], o2[3]));
    st16(&act[t * LDA + col], make_uint4(ou[0], ou[1], ou[2], ou[3]));
  }
  __syncthreads();

  // 5. contraction of this wave's block over its slice of the chunk
  f32x4_t acc[NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) acc[tb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  if (bval) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        const uint4 b =
            *reinterpret_cast<const uint4*>(&act[(tb * 16 + (lane & 15)) * LDA + kw * KPW + ks * 32 + koff]);
        acc[tb] = mfma16(wf[ks], b, acc[tb]);
      }
  }
  // 6. sum the KW slices: waves kw > 0 hand their accumulators to wave kw = 0
  if constexpr (KW > 1) {
    if (kw > 0) {
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb)
        *reinterpret_cast<f32x4_t*>(&red[(((kw - 1) * RB + rb) * NTB + tb) * 256 + lane * 4]) = acc[tb];
    }
    __syncthreads();
    if (kw == 0) {
#pragma unroll
      for (int k2 = 1; k2 < KW; ++k2)
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
          acc[tb] += *reinterpret_cast<const f32x4_t*>(&red[(((k2 - 1) * RB + rb) * NTB + tb) * 256 + lane * 4]);
    }
  }
  if (kw == 0 && bval) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      const int t = tb * 16 + (lane & 15);
      if (t >= rows) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = nb * 16 + 4 * (lane >> 4) + q;
        st_f32(&a.P[((int64_t)kc * a.NP + n) * a.Mpad + m0 + t], acc[tb][q], a.wt);
      }
    }
  }
  // 7. the chunk's sum of squares per token, summed in a fixed order
  if (lead && tid < rows) {
    float t = 0.0f;
    for (int c = 0; c < CPR; ++c) t += ssp[tid * CPR + c];
    st_f32(&a.SS[(int64_t)kc * a.Mpad + m0 + tid], t, a.wt);
  }
}

// ---------------------------------------------------------------------------
// K1r: per token, rrms[s] = 1/sqrt(sum of the stream's chunk sums of squares
// / HS + eps); row n of the contraction = sum_s rrms[s] * (sum of the
// stream's chunk partials); down rows -> h = SiLU(v/HC) (bf16, workspace),
// inject rows -> inj_next (bf16). One wave per (row n, 16 tokens): lane
// l handles token l % 16 and every 4th chunk starting at l / 16; all of a
// lane's loads are issued before the first add (one memory round trip), and
// the four lane groups are then summed with cross-lane adds. HC streams.
// ---------------------------------------------------------------------------
struct ReduceArgs {
  const float* P;
  const float* SS;
  int64_t Mpad, M;
  int NP, kcps, HS, HC, r, n_rows;
  float eps, inv_hc, inv_hs;
  float* rrms;
  uint16_t* h;
  uint16_t* inj_next;
  int64_t ld_inj_next;
};

__device__ __forceinline__ float sum_lane_groups(float v) {
  // lanes l, l^16, l^32, l^48 hold the four chunk groups of one token
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

template <int HC, int CPL>
__global__ __launch_bounds__(256) void hcgr_k1_reduce(ReduceArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t mblocks = a.Mpad / 16;
  const int n = (int)(wid / mblocks);
  if (n >= a.n_rows) return;  // whole wave leaves together
  const int64_t m = (wid % mblocks) * 16 + (lane & 15);
  const int g = lane >> 4;
  const int kcps = a.kcps;  // <= 4 * CPL
  float sv[HC][CPL], pv[HC][CPL];
#pragma unroll
  for (int s = 0; s < HC; ++s)
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = g + 4 * i;
      const int64_t kc = (int64_t)s * kcps + min(c, kcps - 1);  // clamped: no branch around the load
      const float sl = a.SS[kc * a.Mpad + m];
      const float pl = a.P[(kc * a.NP + n) * a.Mpad + m];
      sv[s][i] = c < kcps ? sl : 0.0f;
      pv[s][i] = c < kcps ? pl : 0.0f;
    }
  float ss[HC], ps[HC];
#pragma unroll
  for (int s = 0; s < HC; ++s) {
    float t = 0.0f, u = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      t += sv[s][i];
      u += pv[s][i];
    }
    ss[s] = t;
    ps[s] = u;
  }
  float v = 0.0f;
  float rr[HC];
#pragma unroll
  for (int s = 0; s < HC; ++s) {
    rr[s] = 1.0f / sqrtf(sum_lane_groups(ss[s]) * a.inv_hs + a.eps);
    v = fmaf(rr[s], sum_lane_groups(ps[s]), v);
  }
  if (g != 0) return;
  if (n == 0 && m < a.M) {
#pragma unroll
    for (int s = 0; s < HC; ++s) a.rrms[m * HC + s] = rr[s];
  }
  if (n < a.r) {
    const float z = v * a.inv_hc;
    a.h[m * a.r + n] = (m < a.M) ? to_bf(z * sigmoid_f(z)) : (uint16_t)0;  // (G1) SiLU(lora / HC)
  } else if (m < a.M) {
    a.inj_next[m * a.ld_inj_next + (n - a.r)] = to_bf(v);  // (INJ), not scaled
  }
}

// ---------------------------------------------------------------------------
// hcgr_k2_dec (SPLIT plan, decode sizes): (G2) gate = h . Wu^T, G =
// sigmoid(gate), (MIX) x[c] = 1/4 sum_s G xn, for a token tile of TM tokens
// and CW channels x 4 streams, ceil(CW/4) waves: CW = 16, or 10 where HS is
// a multiple of 2560 (HS/10 workgroups fill whole rounds of the 256 CUs; the
// last wave's rows of channels past CW read as zero and store nothing, and
// the R2 rows and Wnorm of 10 channels arrive in 4-byte pieces). The
// workgroup's Wu rows (r values each) and its h tile arrive in LDS by direct
// global->LDS loads (wide 1 KB
// instructions instead of per-lane fragment loads); inside a row the 16-byte
// chunk c sits in slot (c & ~3) | ((c ^ row) & 3), which spreads the 16-row
// fragment reads over the banks. The epilogue's R2 rows, rrms and Wnorm
// arrive the same way (a few wide loads instead of many 2- and 4-byte ones),
// and the channel groups that share a 128-byte line of R2 or x run on one
// XCD. Wave w owns channels 4w..4w+3: MFMA row
// 4*c + s is stream s of channel c (Wu row s*HS + c), so lane l ends with the
// four streams of channel w*4 + l/16 for token l%16 and the MIX sum is
// lane-local.
// ---------------------------------------------------------------------------
struct UpArgs {
  const uint16_t* h;
  int64_t Mpad, M;
  int r, HS, K;
  const uint16_t* wu;
  const uint16_t* R2;
  const float* rrms;
  const uint16_t* wn;
  int wn_full;
  uint16_t* x;
};

template <int TM, int CW, bool WNT>
__global__ __launch_bounds__((CW + 3) / 4 * 64) void hcgr_k2_dec(UpArgs a) {
  constexpr int NW = (CW + 3) / 4;
  constexpr int NTB = TM / 16;
  constexpr int WR = NW * 16;  // Wu rows of the workgroup (NW * 4 channels x 4 streams, the last CW..4NW-1 zero)
  extern __shared__ __attribute__((aligned(1024))) uint8_t dl[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t m0 = (int64_t)blockIdx.y * TM;
  const int rows = (int)min((int64_t)TM, a.M - m0);
  // channel groups of CW channels; workgroup x goes to XCD x % 8 (the
  // dispatcher's round robin), so XCD k takes a contiguous run of groups and
  // the groups that share a 128-byte line of R2 or x share that XCD's L2
  const int ncg = (int)gridDim.x;  // HS / CW: a multiple of 8 for every accepted HS
  const int cg = (ncg & 7) ? (int)blockIdx.x : (int)((blockIdx.x & 7) * (ncg >> 3) + (blockIdx.x >> 3));
  const int cbase = cg * CW;
  const int cpr = a.r / 8;  // 16-byte chunks per row (a multiple of 4)
  const uint32_t rowb = (uint32_t)a.r * 2u;
  constexpr int RRB = (TM > 64 ? TM : 64) * 16;  // rrms slot: one 16-byte lane per token, 64 lanes at least
  uint8_t* wl = dl;              // [WR][r]: row 4*cl + s = stream s of channel cbase + cl
  uint8_t* hl = dl + WR * rowb;  // [TM][r]
  constexpr int R2B = (TM * 4 * CW * 2 + 1023) / 1024 * 1024;
  uint8_t* r2l = hl + TM * rowb;  // [TM][4 streams][CW channels] bf16, in whole KB
  uint8_t* rrl = r2l + R2B;       // [TM][4] float
  uint8_t* wnl = rrl + RRB;              // [4 streams or 1][CW] bf16 (1 KB slot)
  const rsrc_t rWu = make_rsrc(a.wu, (uint32_t)a.K * rowb);
  const rsrc_t rH = make_rsrc(a.h + m0 * a.r, (uint32_t)rows * rowb);  // rows past M read as zero
  const rsrc_t rR2 = make_rsrc(a.R2 + m0 * a.K, (uint32_t)rows * (uint32_t)a.K * 2u);
  const rsrc_t rRr = make_rsrc(a.rrms + m0 * 4, (uint32_t)rows * 16u);
  const rsrc_t rWn = make_rsrc(a.wn, (uint32_t)(a.wn_full ? a.K : a.HS) * 2u);

  // global -> LDS: instruction i fills LDS chunks [64 i, 64 i + 64) of a
  // block; WR*cpr and TM*cpr are multiples of 64. Wu rows of channels past
  // CW feed only MFMA rows whose results are not stored: the loads stop at
  // the instruction that holds the last real row's chunks.
  for (int i = wave; i * 64 < 4 * CW * cpr; i += NW) {
    const int q = i * 64 + lane, row = q / cpr, sl = q % cpr;
    const int c = (sl & ~3) | ((sl ^ row) & 3);  // the chunk this slot holds
    const bool pad = CW % 4 != 0 && (row >> 2) >= CW;  // rows of channels past CW read zeros
    const uint32_t off = pad ? 0x80000000u : (uint32_t)((row & 3) * a.HS + cbase + (row >> 2)) * rowb + (uint32_t)c * 16u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rWu, (lds_void_t*)(wl + i * 1024), 16, off, 0, 0, WNT ? kNonTemporal : 0);
  }
  for (int i = wave; i * 64 < TM * cpr; i += NW) {
    const int q = i * 64 + lane, row = q / cpr, sl = q % cpr;
    const int c = (sl & ~3) | ((sl ^ row) & 3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rH, (lds_void_t*)(hl + i * 1024), 16, (uint32_t)row * rowb + (uint32_t)c * 16u,
                                             0, 0, 0);
  }
  // epilogue operands, also global -> LDS: the tile's R2 rows of the
  // workgroup's channels, its rrms rows and the channels' Wnorm
  static_assert(TM % 8 == 0 && (CW == 16 || CW == 10), "R2 slots: 8 (16 channels) or 20 (10) per token");
  if constexpr (CW == 16) {  // 16-byte pieces (lane: token q / 8, stream (q / 2) % 4, half q % 2)
    for (int i = wave; i < TM / 8; i += NW) {
      const int q = i * 64 + lane, t = q >> 3, sq = (q >> 1) & 3;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rR2, (lds_void_t*)(r2l + i * 1024), 16,
          (uint32_t)t * (uint32_t)a.K * 2u + (uint32_t)(sq * a.HS + cbase + (q & 1) * 8) * 2u, 0, 0, 0);
    }
  } else {  // 4-byte pieces (lane: token q / 20, stream (q / 5) % 4, channel pair q % 5); TM * 20 = 64 * TM / 16 * 5
    for (int i = wave; i * 64 < TM * 20; i += NW) {
      const int q = i * 64 + lane, t = q / 20, sq = (q / 5) % 4, pc = q % 5;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rR2, (lds_void_t*)(r2l + i * 256), 4,
          (uint32_t)t * (uint32_t)a.K * 2u + (uint32_t)(sq * a.HS + cbase + pc * 2) * 2u, 0, 0, 0);
    }
  }
  if (wave == 0) {
    for (int i = 0; i * 64 < TM; ++i)  // lanes past the tile read zeros into the slot
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rRr, (lds_void_t*)(rrl + i * 1024), 16,
                                               (uint32_t)(i * 64 + lane) * 16u, 0, 0, 0);
    if constexpr (CW == 16) {
      const bool live = lane < (a.wn_full ? 8 : 2);
      const uint32_t wo = (uint32_t)((a.wn_full ? (lane >> 1) * a.HS : 0) + cbase + (lane & 1) * 8) * 2u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rWn, (lds_void_t*)wnl, 16, live ? wo : 0x80000000u, 0, 0, 0);
    } else {
      const bool live = lane < (a.wn_full ? 20 : 5);
      const uint32_t wo = (uint32_t)((a.wn_full ? (lane / 5) * a.HS : 0) + cbase + (lane % 5) * 2) * 2u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rWn, (lds_void_t*)wnl, 4, live ? wo : 0x80000000u, 0, 0, 0);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lds_sync();  // every wave's global->LDS loads have landed

  // lane holds streams q = 0..3 of channel c for token m
  const int cl = wave * 4 + (lane >> 4), c = cbase + cl;
  float pr2[NTB][4], prr[NTB][4], pone[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    pone[q] = 1.0f + bf1(*reinterpret_cast<const uint16_t*>(wnl + ((a.wn_full ? q * CW : 0) + cl) * 2));
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    const int t = tb * 16 + (lane & 15);
    const f32x4_t rr = *reinterpret_cast<const f32x4_t*>(rrl + t * 16);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      pr2[tb][q] = bf1(*reinterpret_cast<const uint16_t*>(r2l + (t * 4 + q) * (CW * 2) + cl * 2));
      prr[tb][q] = rr[q];
    }
  }

  f32x4_t acc[NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) acc[tb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int arow = wave * 16 + (lane & 15);
  const int nj = a.r / 32;
  auto kstep = [&](int j, uint4& af, uint4 (&bf)[NTB]) {  // fragments of k step j
    af = *reinterpret_cast<const uint4*>(wl + arow * rowb + (uint32_t)(j * 4 + (((lane >> 4) ^ arow) & 3)) * 16u);
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      const int t = tb * 16 + (lane & 15);
      bf[tb] = *reinterpret_cast<const uint4*>(hl + t * rowb + (uint32_t)(j * 4 + (((lane >> 4) ^ t) & 3)) * 16u);
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

#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    const int64_t m = m0 + tb * 16 + (lane & 15);
    if (m < a.M && (CW % 4 == 0 || cl < CW)) {
      float sum = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) sum = fmaf(sigmoid_f(acc[tb][q]), pr2[tb][q] * prr[tb][q] * pone[q], sum);
      a.x[m * a.HS + c] = to_bf(sum * 0.25f);
    }
  }
}

// ---------------------------------------------------------------------------
// hcgr_k1_full: COMBINE + N + down/inject contraction for a token tile over
// whole streams (STREAM and FULL plans).
// Workgroup = (token tile of TM rows) x (row split: 16-row blocks [b0, b1) of
// the down/inject rows) x (stream group: streams [s_first, s_first + spw)).
// The loop runs stream-major over LDS stages of KS columns. Per stage every
// thread combines one 16-byte chunk of R/y (two stages of raw loads in
// flight in registers), stores its R2 chunk (row split 0 only) and the bf16
// activation R2*(1+Wnorm) (or R2 for folded weights) into a double-buffered
// LDS tile; each wave then runs its row blocks over the tile with
// v_mfma_f32_16x16x32_bf16 (A = weight rows from global, one stage ahead;
// B = activation from LDS). At each stream end the stream's sum of squares
// gives rrms and the stream accumulator is folded into the total with it.
// Every global access in the loop is an unconditional buffer access through
// a range-limited descriptor (rows past M read as zero, stores past the
// range are dropped), so the loop has no branch around a memory operation
// and the compiler can keep several stages of loads in flight.
// ---------------------------------------------------------------------------
struct FullArgs {
  const uint16_t* R;
  const uint16_t* y;
  const uint16_t* inj;
  int64_t ld_inj;
  const uint16_t* wn;
  int wn_len;
  const uint16_t* w0;  // Wd [r,K] or merged Wm [n_pad,K]
  const uint16_t* w1;  // Wi [HC,K], or nullptr when the inject rows are rows r.. of w0
  int folded;
  int64_t M;
  int K, HS, HC, r, n_rows, nblk;
  int nsplit, spw;
  float eps, inv_hc, inv_hs;
  uint16_t* R2;
  float* rrms;
  uint16_t* h;  // [Mpad, r] (FULL)
  uint16_t* inj_next;
  int64_t ld_inj_next;
  float* Q;  // [HC][Mq][NP] rrms-scaled per-stream partials (STREAM)
  int64_t Mq;
  int NP;
};

template <int B>
using ic = std::integral_constant<int, B>;

template <int TM, int NW, int BPW, int KS>
__global__ __launch_bounds__(NW * 64) void hcgr_k1_full(FullArgs a) {
  constexpr int NT = NW * 64;
  constexpr int CPR = KS / 8;  // 16-byte chunks per token row of a stage
  constexpr int NCH = TM * CPR;
  static_assert(NCH % NT == 0, "whole chunks per thread");
  constexpr int CPT = NCH / NT;
  static_assert(64 % CPR == 0, "a token's chunks lie inside one wave");
  constexpr int LDA = KS + 8;  // padded LDS row, bf16 elements
  constexpr int NTB = TM / 16;
  constexpr int NKS = KS / 32;

  __shared__ __attribute__((aligned(16))) uint16_t act[2][TM * LDA];
  __shared__ float iwh[4][TM], iwl[4][TM], rrs[4][TM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in a scalar register
  const int64_t m0 = (int64_t)blockIdx.x * TM;
  const int rows = (int)min((int64_t)TM, a.M - m0);  // valid token rows of the tile
  const int ngroups = 4 / a.spw;
  const int split = blockIdx.y / ngroups;
  const int s_first = (int)(blockIdx.y % ngroups) * a.spw;
  const int b0 = split * a.nblk / a.nsplit;
  const int b1 = (split + 1) * a.nblk / a.nsplit;
  const bool lead = split == 0;
  const int spp = a.HS / KS;  // stages per stream
  const int nst = a.spw * spp;
  const int koff = 8 * (lane >> 4);
  const uint32_t rowb = (uint32_t)a.K * 2u;  // bytes per R/R2 row

  // range-limited descriptors (scalar)
  const rsrc_t rR = make_rsrc(a.R + m0 * a.K, (uint32_t)rows * rowb);
  const rsrc_t rY = make_rsrc_opt(a.y, m0 * a.HS, (uint32_t)rows * (uint32_t)a.HS * 2u);
  const rsrc_t rWn = make_rsrc(a.wn, a.folded ? 0u : (uint32_t)a.wn_len * 2u);  // folded: reads 0 -> factor 1
  const rsrc_t rR2 = make_rsrc_opt(a.R2, m0 * a.K, lead ? (uint32_t)rows * rowb : 0u);
  const rsrc_t rW0 = make_rsrc(a.w0, (uint32_t)(a.w1 ? a.r : a.n_rows) * rowb);
  const rsrc_t rW1 = make_rsrc(a.w1 ? a.w1 : a.w0, a.w1 ? (uint32_t)a.HC * rowb : 0u);

  // (COMBINE) iw = 2*sigmoid(inj/HC), formed in fp64 and kept as fp32 hi + lo
  // so that R2 = (R + y*hi) + y*lo stays within an ulp of R2 under cancellation
  for (int i = tid; i < 4 * TM; i += NT) {
    const int s = i / TM, t = i % TM;
    const int64_t m = m0 + t;
    double v = 0.0;
    if (t < rows && a.inj) v = 2.0 / (1.0 + exp(-(double)bf1(a.inj[m * a.ld_inj + s]) / (double)a.HC));
    const float hi = (float)v;
    iwh[s][t] = hi;
    iwl[s][t] = (float)(v - (double)hi);
  }

  // weight rows of this wave: block nb covers rows nb*16.., each either all
  // down rows (< r) or all inject/pad rows, so the descriptor is wave-uniform
  rsrc_t wrs[BPW];
  uint32_t wofs[BPW];
  bool bval[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int nb = b0 + wave + NW * i;
    bval[i] = nb < b1;
    const int n = nb * 16 + (lane & 15);
    const bool down = nb * 16 < a.r || !a.w1;
    wrs[i] = down ? rW0 : rW1;
    wofs[i] = (uint32_t)(down ? n : n - a.r) * rowb;
  }
  auto kbase = [&](int st) { return (s_first + st / spp) * a.HS + (st % spp) * KS; };

  uint4 wf[BPW][NKS];
  auto load_w = [&](int st, int ks) {
    const uint32_t k2 = (uint32_t)(kbase(st) + ks * 32 + koff) * 2u;
#pragma unroll
    for (int i = 0; i < BPW; ++i) wf[i][ks] = bld16(wrs[i], wofs[i] + k2);
  };

  uint4 rv[2][CPT], yv[2][CPT], wv[2][CPT];
  auto load_raw = [&](auto BUF, int st) {
    constexpr int b = decltype(BUF)::value;
    const int s = s_first + st / spp;
    const int c0 = (st % spp) * KS;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int q = tid + j * NT;
      const uint32_t t = q / CPR;
      const uint32_t col = (q % CPR) * 8;
      rv[b][j] = bld16(rR, t * rowb + (uint32_t)(s * a.HS + c0 + col) * 2u);
      yv[b][j] = bld16(rY, (t * (uint32_t)a.HS + c0 + col) * 2u);
      wv[b][j] = bld16(rWn, ((a.wn_len == a.HS ? 0u : (uint32_t)(s * a.HS)) + c0 + col) * 2u);
    }
  };

  float ss[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) ss[j] = 0.0f;

  // (COMBINE) R2 = R + y*iw in fp32; sum of squares; R2 -> bf16 output;
  // activation R2*(1+Wnorm) -> LDS (Wnorm reads as 0 for folded weights)
  auto combine = [&](auto BUF, int st) {
    constexpr int b = decltype(BUF)::value;
    const int s = s_first + st / spp;
    const int c0 = (st % spp) * KS;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int q = tid + j * NT;
      const int t = q / CPR;
      const int col = (q % CPR) * 8;
      const float ih = iwh[s][t];
      const float il = iwl[s][t];
      const uint32_t rw[4] = {rv[b][j].x, rv[b][j].y, rv[b][j].z, rv[b][j].w};
      const uint32_t yw[4] = {yv[b][j].x, yv[b][j].y, yv[b][j].z, yv[b][j].w};
      const uint32_t ww[4] = {wv[b][j].x, wv[b][j].y, wv[b][j].z, wv[b][j].w};
      uint32_t o2[4], ou[4];
      float acc = ss[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float r0 = fmaf(bf_lo(yw[e]), il, fmaf(bf_lo(yw[e]), ih, bf_lo(rw[e])));
        const float r1 = fmaf(bf_hi(yw[e]), il, fmaf(bf_hi(yw[e]), ih, bf_hi(rw[e])));
        acc = fmaf(r0, r0, acc);
        acc = fmaf(r1, r1, acc);
        o2[e] = pack_bf2(r0, r1);
        ou[e] = pack_bf2(r0 * (1.0f + bf_lo(ww[e])), r1 * (1.0f + bf_hi(ww[e])));
      }
      ss[j] = acc;
      bst16(rR2, (uint32_t)t * rowb + (uint32_t)(s * a.HS + c0 + col) * 2u, make_uint4(o2[0], o2[1], o2[2], o2[3]));
      st16(&act[b][t * LDA + col], make_uint4(ou[0], ou[1], ou[2], ou[3]));
    }
  };

  f32x4_t acc_t[BPW][NTB], acc_s[BPW][NTB];
#pragma unroll
  for (int i = 0; i < BPW; ++i)
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) acc_t[i][tb] = acc_s[i][tb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  auto contract = [&](auto BUF, int st) {
    constexpr int b = decltype(BUF)::value;
    const uint16_t* buf = act[b];
    const int stn = min(st + 1, nst - 1);  // the last stage reloads itself: no branch around a load
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      uint4 bfr[NTB];
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb)
        bfr[tb] = *reinterpret_cast<const uint4*>(buf + (tb * 16 + (lane & 15)) * LDA + ks * 32 + koff);
#pragma unroll
      for (int i = 0; i < BPW; ++i)
        if (bval[i]) {
#pragma unroll
          for (int tb = 0; tb < NTB; ++tb) acc_s[i][tb] = mfma16(wf[i][ks], bfr[tb], acc_s[i][tb]);
        }
      load_w(stn, ks);
    }
  };

  // (N) stream end: rrms from the stream's sum of squares; fold the stream
  // accumulator into the total
  auto stream_end = [&](int s) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      float v = ss[j];
#pragma unroll
      for (int o = 1; o < CPR; o <<= 1) v += __shfl_xor(v, o, 64);
      ss[j] = 0.0f;
      const int q = tid + j * NT;
      if ((tid % CPR) == 0) rrs[s][q / CPR] = 1.0f / sqrtf(v * a.inv_hs + a.eps);
    }
    __syncthreads();
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      const float rr = rrs[s][tb * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < BPW; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) acc_t[i][tb][q] = fmaf(rr, acc_s[i][tb][q], acc_t[i][tb][q]);
        acc_s[i][tb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }
  };

  auto step = [&](auto BUF, int st) {
    combine(BUF, st);
    load_raw(BUF, min(st + 2, nst - 1));
    __syncthreads();
    contract(BUF, st);
    if ((st + 1) % spp == 0) stream_end(s_first + st / spp);
  };

  // nst is even (the plan guarantees it), so the loop runs whole pairs
  load_raw(ic<0>{}, 0);
  load_raw(ic<1>{}, 1);
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) load_w(0, ks);
  __syncthreads();  // iwh/iwl
  for (int st = 0; st < nst; st += 2) {
    step(ic<0>{}, st);
    step(ic<1>{}, st + 1);
  }

  // outputs: rrms of this workgroup's streams; lane holds rows n0..n0+3 of
  // token m for each of its blocks and token blocks
  if (lead)
    for (int i = tid; i < a.spw * TM; i += NT) {
      const int s = s_first + i / TM, t = i % TM;
      if (t < rows) a.rrms[(m0 + t) * 4 + s] = rrs[s][t];
    }
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    if (!bval[i]) continue;
    const int n0 = (b0 + wave + NW * i) * 16 + 4 * (lane >> 4);
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      const int t = tb * 16 + (lane & 15);
      if (t >= rows) continue;
      const int64_t m = m0 + t;
      const f32x4_t v = acc_t[i][tb];
      if (a.spw == 1) {
        if (n0 < a.n_rows)
          *reinterpret_cast<f32x4_t*>(a.Q + ((int64_t)s_first * a.Mq + m) * a.NP + n0) = v;
      } else if (n0 < a.r) {
        float z[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) z[q] = v[q] * a.inv_hc;
        uint2 o;
        o.x = pack_bf2(z[0] * sigmoid_f(z[0]), z[1] * sigmoid_f(z[1]));  // (G1) SiLU(lora / HC)
        o.y = pack_bf2(z[2] * sigmoid_f(z[2]), z[3] * sigmoid_f(z[3]));
        *reinterpret_cast<uint2*>(a.h + m * a.r + n0) = o;
      } else if (n0 < a.n_rows) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (n0 + q < a.n_rows) a.inj_next[m * a.ld_inj_next + (n0 - a.r + q)] = to_bf(v[q]);  // (INJ)
      }
    }
  }
}

// ---------------------------------------------------------------------------
// hcgr_k1_tile (large token counts): COMBINE + N + down/inject contraction
// for a tile of TM = 64 tokens.
// Workgroup = (token tile) x (row split: 16-row blocks [b0, b1), at most 22)
// x (stream group: SPW = 4 streams, or SPW = 1 stream whose partial goes to
// the workspace) x (column segment of that stream, SPW = 1 only). Eight
// waves, two per SIMD: wave (rq, th) owns row quarter rq of the blocks (at
// most 6) and token half th (two MFMA column blocks of 16 tokens).
// A stage is 64 columns of k. Iteration i contracts stage i (weights and the
// bf16 activation from LDS into v_mfma_f32_16x16x32_bf16) and combines stage
// i+1 (R, y and Wnorm from registers -> R2 to HBM, activation R2*(1+Wnorm)
// to LDS), with one barrier per iteration. Thread t owns one 16-byte chunk
// (token t/8) of every stage and prefetches its R, y and Wnorm chunks D = 4
// stages ahead into a ring of registers, so the workgroup keeps several
// stages of HBM reads in flight without LDS space for them. Weights (read
// from L2) and the activation are double buffered in LDS; the weights arrive
// by direct global->LDS loads, 8 rows x 128 bytes per wave instruction,
// six per wave. Every thread issues the same loads in the same order in
// every iteration (prefetches past the last stage use an offset outside the
// buffer range: they return zeros without touching memory), so the wait at
// the top of an iteration names an exact count of later loads. Inside each
// 128-byte LDS row the 16-byte chunk c of row t sits in slot c ^ (t & 7),
// which spreads MFMA fragment reads (16 rows, one chunk) over the banks. At
// each stream end the stream's sum of squares gives rrms and, with SPW = 4,
// the stream accumulator is folded into the rrms-scaled total (two
// accumulator sets).
// ---------------------------------------------------------------------------
struct Tile1Args {
  const uint16_t* R;
  const uint16_t* y;
  const uint16_t* inj;
  int64_t ld_inj;
  const uint16_t* wn;
  int wn_len;
  int folded;
  const uint16_t* w0;  // down rows: Wd [r,K], or rows 0..r-1 of Wm
  const uint16_t* w1;  // inject rows: Wi [HC,K], or rows r..r+HC-1 of Wm
  int64_t M;
  int K, HS, HC, r, nblk, nsplit;
  float eps, inv_hc, inv_hs;
  uint16_t* R2;
  float* rrms;
  uint16_t* h;  // [>= M, r]        (SPW = 4)
  uint16_t* inj_next;
  int64_t ld_inj_next;
  float* Q;  // [HC*nseg][Mq][NP] per-stream partials (SPW = 1): rrms-scaled, or unscaled when nseg > 1
  int64_t Mq;
  int NP;
  int nseg;    // column segments per stream (SPW = 1 only); > 1: rrms is formed by hcgr_k1_sum
  float* SSp;  // [HC*nseg][Mq] per-segment sums of squares (nseg > 1)
  int tiles;   // token tiles
  int xgroup;  // 1: the workgroups of one token tile share an XCD (grid rounded up to 8 tiles)
  int nt;      // 1: R2 written with the non-temporal policy
  int ntr;     // 1: R read with the non-temporal policy
};

template <int N>
using ic = std::integral_constant<int, N>;

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(ic<I>{});
    static_for<I + 1, N>(f);
  }
}

// TM: tokens per tile (64, or 128 with one stream per workgroup); D: depth of
// the R/y/Wnorm prefetch ring in stages (4 for 64 tokens; 3 for 128, whose
// threads own two tokens' chunks per stage).
template <int SPW, int TM, int D>
__global__ __launch_bounds__(512) void hcgr_k1_tile(Tile1Args a) {
  constexpr int NT = 512, BPW = 6, NTB = TM / 32, TPT = TM / 64;  // TPT: tokens per thread per stage
  constexpr int WGRP = 6;  // 8-row weight groups per wave per stage
  constexpr int WBYTES = 8 * WGRP * 1024, ABYTES = TM * 128;
  constexpr int NSET = SPW == 4 ? 1 : 0;  // rrms-scaled total kept in registers
  constexpr int NL = 2 * TPT + 1;         // prefetch loads per thread per stage: R and y per token, Wnorm
  constexpr int G = D % 2 ? 2 * D : D;    // iterations per unrolled group: ring slot period D, buffer parity 2
  constexpr uint32_t kOut = 0x80000000u;  // offset past every buffer range
  static_assert((TM == 64 || (TM == 128 && SPW == 1)) && D >= 2 && D <= 4, "tile shapes");
  static_assert(8 * WGRP >= 2 * kTileMaxBlk && (kTileMaxBlk * 3) / 4 + BPW <= 8 * WGRP / 2,
                "tile shape: every wave's blocks (read or not) lie inside the weight buffer");
  __shared__ __attribute__((aligned(1024))) uint8_t w_0[WBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t w_1[WBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t act_0[ABYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t act_1[ABYTES];
  __shared__ float iwh[SPW][TM], iwl[SPW][TM], rrs[SPW][TM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rq = wave & 3, th = wave >> 2;
  const int NG = a.HC / SPW;  // stream groups (SPW = 4 only with HC = 4)
  const int nseg = SPW == 1 ? a.nseg : 1;
  // workgroup -> (token tile, row split, stream group, column segment). With
  // xgroup, workgroup b serves tile 8 (q / P) + b % 8, q = b / 8, P = the
  // workgroups of a tile: all of a tile's workgroups share b % 8 and so run
  // on one XCD (workgroups go round-robin over the 8 XCDs), where y and the
  // tile's R rows are fetched from HBM once. Otherwise b = ((tile * nsplit +
  // split) * NG + sg) * nseg + seg.
  int wq, tile_i;
  if (a.xgroup) {
    const int P = a.nsplit * NG * nseg, q = (int)(blockIdx.x >> 3);
    tile_i = (q / P) * 8 + (int)(blockIdx.x & 7);
    wq = q % P;
    if (tile_i >= a.tiles) return;  // grid rounded up to whole octets of tiles
  } else {
    tile_i = (int)(blockIdx.x / (nseg * NG * a.nsplit));
    wq = (int)(blockIdx.x % (nseg * NG * a.nsplit));
  }
  const int seg = wq % nseg;
  const int sg = (wq / nseg) % NG;
  const int split = wq / (nseg * NG);
  const int64_t m0 = (int64_t)tile_i * TM;
  const int rows = (int)min((int64_t)TM, a.M - m0);
  const int s_first = sg * SPW;
  const int b0 = split * a.nblk / a.nsplit, b1 = (split + 1) * a.nblk / a.nsplit;
  const int nbw = b1 - b0;
  const int qb0 = rq * nbw / 4;               // first block of this wave, relative to b0
  const int wcnt = (rq + 1) * nbw / 4 - qb0;  // blocks of this wave (<= BPW)
  const bool lead = split == 0;
  const int HS = a.HS;
  const int c_begin = seg * (HS / nseg), c_end = c_begin + HS / nseg;  // this workgroup's columns of each stream
  const int nst = SPW * (HS / nseg / 64);
  const uint32_t rowb = (uint32_t)a.K * 2u;

  const rsrc_t rR = make_rsrc(a.R + m0 * a.K, (uint32_t)rows * rowb);
  const rsrc_t rY = make_rsrc_opt(a.y, m0 * HS, (uint32_t)rows * (uint32_t)HS * 2u);
  const rsrc_t rWn = make_rsrc(a.wn, a.folded ? 0u : (uint32_t)a.wn_len * 2u);  // folded: reads 0 -> factor 1
  const rsrc_t rR2 = make_rsrc_opt(a.R2, m0 * a.K, lead ? (uint32_t)rows * rowb : 0u);
  const rsrc_t rW0 = make_rsrc(a.w0, (uint32_t)a.r * rowb);
  const rsrc_t rW1 = make_rsrc(a.w1, (uint32_t)a.HC * rowb);  // rows past HC read as zero

  // injection logit of table entry tid (loaded before the prefetches below,
  // which then stay in flight while iw is formed)
  const int it = tid % TM, isl = (tid / TM) % SPW;
  const uint16_t injb = a.inj ? a.inj[(m0 + min(it, rows - 1)) * a.ld_inj + s_first + isl] : (uint16_t)0;

  // chunk this lane moves inside its 128-byte row (rows t with t & 7 == lane >> 3)
  const uint32_t swz = (uint32_t)((lane & 7) ^ (lane >> 3));
  const uint32_t grow = (uint32_t)(lane >> 3);  // row inside an 8-row group
  // weight groups of this wave: 8-row group g = wave + 8 j of the split's rows
  uint32_t woff[WGRP];
  uint32_t winj = 0;  // bit j: group j holds inject rows
#pragma unroll
  for (int j = 0; j < WGRP; ++j) {
    const int g = wave + 8 * j;
    const int n = b0 * 16 + g * 8;  // r is a multiple of 8, so a group never straddles r
    const bool down = n < a.r;
    woff[j] = g < 2 * nbw ? (uint32_t)((down ? n : n - a.r) + (int)grow) * rowb + swz * 16u : kOut;
    if (!down) winj |= 1u << j;
  }
  winj = __builtin_amdgcn_readfirstlane(winj);
  // this thread's chunks of every stage: tokens tok + 64 j (j < TPT), LDS slot
  // tid & 7 (chunk swz) of their rows
  const int tok = tid >> 3;
  const uint32_t offR = (uint32_t)tok * rowb + swz * 16u;
  const uint32_t offY = (uint32_t)tok * (uint32_t)HS * 2u + swz * 16u;
  const uint32_t wnc = a.folded ? 0u : (a.wn_len == HS ? 0u : 1u);  // Wnorm indexed by k
  const uint32_t la_off = (uint32_t)(tok * 128 + (tid & 7) * 16);

  auto issue_w = [&](bool valid, int s, int c0, uint8_t* wbuf) {
    const uint32_t kb = (uint32_t)(s * HS + c0) * 2u;
#pragma unroll
    for (int j = 0; j < WGRP; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds((winj >> j) & 1u ? rW1 : rW0, (lds_void_t*)(wbuf + (wave + 8 * j) * 1024),
                                               16, valid ? woff[j] + kb : kOut, 0, 0, 0);
  };
  u32x4_t rv[D][TPT], yv[D][TPT], wv[D];  // prefetch ring: stage j in slot j % D
  auto load_ry = [&](auto SL, bool valid, int s, int c0) {
    constexpr int k = decltype(SL)::value;
    const uint32_t col = (uint32_t)c0 * 2u;
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      const uint32_t oR = valid ? offR + (uint32_t)(j * 64) * rowb + (uint32_t)(s * HS) * 2u + col : kOut;
      const uint32_t oY = valid ? offY + (uint32_t)(j * 64 * HS) * 2u + col : kOut;
      rv[k][j] = __builtin_bit_cast(u32x4_t, a.ntr ? __builtin_amdgcn_raw_buffer_load_b128(rR, (int)oR, 0, kNonTemporal)
                                                  : __builtin_amdgcn_raw_buffer_load_b128(rR, (int)oR, 0, 0));
      yv[k][j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rY, (int)oY, 0, 0));
    }
    const uint32_t oW = valid ? (wnc ? (uint32_t)(s * HS) * 2u : 0u) + col + swz * 16u : kOut;
    wv[k] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rWn, (int)oW, 0, 0));
  };

  float ss[TPT], ih[TPT], il[TPT];
#pragma unroll
  for (int j = 0; j < TPT; ++j) ss[j] = ih[j] = il[j] = 0.0f;
  // stages past the last one combine the zeros their prefetch returned and
  // store nothing (out-of-range R2 offset); running them keeps every ring
  // slot consumed on every path
  auto combine = [&](auto SL, bool valid, int s, int c0, uint8_t* abuf) {
    constexpr int k = decltype(SL)::value;
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      uint32_t o2[4], ou[4];
      float acc = ss[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t rw = rv[k][j][e], yw = yv[k][j][e], ww = wv[k][e];
        const float r0 = fmaf(bf_lo(yw), il[j], fmaf(bf_lo(yw), ih[j], bf_lo(rw)));
        const float r1 = fmaf(bf_hi(yw), il[j], fmaf(bf_hi(yw), ih[j], bf_hi(rw)));
        acc = fmaf(r0, r0, acc);
        acc = fmaf(r1, r1, acc);
        o2[e] = pack_bf2(r0, r1);
        ou[e] = pack_bf2(r0 * (1.0f + bf_lo(ww)), r1 * (1.0f + bf_hi(ww)));
      }
      ss[j] = acc;
      const uint32_t o2off = valid ? offR + (uint32_t)(j * 64) * rowb + (uint32_t)(s * HS + c0) * 2u : kOut;
      if (a.nt) bst16_nt(rR2, o2off, make_uint4(o2[0], o2[1], o2[2], o2[3]));
      else bst16(rR2, o2off, make_uint4(o2[0], o2[1], o2[2], o2[3]));
      *reinterpret_cast<u32x4_t*>(abuf + la_off + j * 64 * 128) = u32x4_t{ou[0], ou[1], ou[2], ou[3]};
    }
  };
  // (N) the stream's sum of squares -> rrms of this thread's tokens
  auto stream_rrms = [&](int sl) {
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      float v = ss[j];
      v += __shfl_xor(v, 1, 64);
      v += __shfl_xor(v, 2, 64);
      v += __shfl_xor(v, 4, 64);
      ss[j] = 0.0f;
      const int t = tok + 64 * j;
      if ((tid & 7) == 0) {
        if (nseg == 1) {
          rrs[sl][t] = 1.0f / sqrtf(v * a.inv_hs + a.eps);
        } else {  // a segment of the stream: its sum of squares goes out, the partial stays unscaled
          rrs[sl][t] = 1.0f;
          if (lead && t < rows) a.SSp[(int64_t)(s_first * nseg + seg) * a.Mq + m0 + t] = v;
        }
      }
    }
  };
  auto set_iw = [&](int sl) {  // injection weights of stream s_first + sl for this thread's tokens
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      ih[j] = iwh[sl][tok + 64 * j];
      il[j] = iwl[sl][tok + 64 * j];
    }
  };

  f32x4_t acc_s[BPW][NTB];
  f32x4_t acc_t[NSET ? BPW : 1][NSET ? NTB : 1];
#pragma unroll
  for (int i = 0; i < BPW; ++i)
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) acc_s[i][tb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (NSET) {
#pragma unroll
    for (int i = 0; i < BPW; ++i)
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) acc_t[i][tb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // (G1, INJ) contraction of one stage: A = weight rows, B = activation
  const uint32_t bfr_off = (uint32_t)((th * (TM / 2) + (lane & 15)) * 128);
  auto contract = [&](const uint8_t* wbuf, const uint8_t* abuf) {
    u32x4_t bq[2][NTB];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb)
        bq[ks][tb] = *reinterpret_cast<const u32x4_t*>(abuf + bfr_off + tb * 2048 +
                                                       (((ks * 4 + (lane >> 4)) ^ (lane & 7)) * 16));
    // A fragments of k half 0 up front; each is replaced by its k half 1
    // fragment as soon as its two products have issued
    const uint8_t* wrow = wbuf + (qb0 * 16 + (lane & 15)) * 128;
    const int slot0 = (((lane >> 4)) ^ (lane & 7)) * 16, slot1 = ((4 + (lane >> 4)) ^ (lane & 7)) * 16;
    uint4 af[BPW];
#pragma unroll
    for (int i = 0; i < BPW; ++i)  // blocks past wcnt compute unused values (inside the buffer)
      af[i] = *reinterpret_cast<const uint4*>(wrow + i * 2048 + slot0);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < BPW; ++i) {
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
          acc_s[i][tb] = mfma16(af[i], __builtin_bit_cast(uint4, bq[ks][tb]), acc_s[i][tb]);
        if (ks == 0) af[i] = *reinterpret_cast<const uint4*>(wrow + i * 2048 + slot1);
      }
    // schedule: the ten first reads, then each pair of products followed by
    // the read that replaces its A fragment, then the last twelve products
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * NTB + BPW, 0);
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, NTB, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NTB * BPW, 0);
  };
  auto fold = [&](int sl) {  // stream end: total += rrms_s * stream accumulator
    if constexpr (NSET) {
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        const float rr = rrs[sl][th * (TM / 2) + tb * 16 + (lane & 15)];
#pragma unroll
        for (int i = 0; i < BPW; ++i) {
#pragma unroll
          for (int q = 0; q < 4; ++q) acc_t[i][tb][q] = fmaf(rr, acc_s[i][tb][q], acc_t[i][tb][q]);
          acc_s[i][tb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
      }
    }
  };

  // stage pointers (stream, first column): stage i, i+1 and i+D; past the
  // last stage they stay on it (the loads they drive are then out of range)
  const int s_last = s_first + SPW - 1;
  auto advance = [&](int& s, int& c) {
    if (c + 64 < c_end) c += 64;
    else if (s < s_last) { c = c_begin; ++s; }
  };
  int s0 = s_first, c0 = c_begin;
  int s1 = s0, c1 = c0;
  advance(s1, c1);
  int sD = s0, cD = c0;

  // prologue: weights of stage 0, R/y/Wnorm of stages 0 .. D-1
  issue_w(true, s0, c0, w_0);
  static_for<0, D>([&](auto J) {
    load_ry(J, decltype(J)::value < nst, sD, cD);
    advance(sD, cD);
  });
  // (COMBINE) iw = 2*sigmoid(inj/HC) in fp64, kept as fp32 hi + lo
  if (tid < SPW * TM) {
    const double v = it < rows ? 2.0 / (1.0 + exp(-(double)bf1(injb) / (double)a.HC)) : 0.0;
    const float hi = (float)v;
    iwh[isl][it] = hi;
    iwl[isl][it] = (float)(v - (double)hi);
  }
  lds_sync();
  set_iw(0);
  // weights and R/y/Wnorm of stage 0: the NL loads of each of stages 1 .. D-1 stay in flight
  if constexpr (D == 4 && NL == 3) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
  else if constexpr (D == 3 && NL == 5) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
  else static_assert(D == 4 && NL == 3, "prologue wait written for these two shapes");
  combine(ic<0>{}, true, s0, c0, act_0);
  if (c0 + 64 == c_end) stream_rrms(0);

  // Iteration st (position p = st % G in its group: ring slot k = p % D,
  // buffer parity p % 2). On entry the newest memory operations of this
  // thread are, in issue order: the weights of stage st, the R2 stores (and,
  // closing a column segment, sum-of-squares stores), then the NL R/y/Wnorm
  // loads of stage st+D-1. The vector memory counter covers loads and
  // stores; with the stores issued before the prefetch, vmcnt(NL) leaves
  // exactly those prefetch loads in flight whether or not a store may
  // complete ahead of earlier loads. Everything it waits for includes
  // R/y/Wnorm of stage st+1 (issued D-1 iterations back).
  auto iteration = [&](auto P, int st) {
    constexpr int p = decltype(P)::value, k = p % D;
    if constexpr (NL == 3) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
    else if constexpr (NL == 5) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
    else static_assert(NL == 3, "iteration wait written for one or two tokens per thread");
    lds_sync();  // weights of stage st landed for every wave; iteration st-1 fully done
    uint8_t* wcur = (p & 1) ? w_1 : w_0;
    uint8_t* wnxt = (p & 1) ? w_0 : w_1;
    uint8_t* acur = (p & 1) ? act_1 : act_0;
    uint8_t* anxt = (p & 1) ? act_0 : act_1;
    const bool v1 = st + 1 < nst;
    issue_w(v1, s1, c1, wnxt);
    if (v1 && c1 == c_begin) set_iw(s1 - s_first);  // stage st+1 opens stream s1
    combine(ic<(k + 1) % D>{}, v1, s1, c1, anxt);
    if (v1 && c1 + 64 == c_end) stream_rrms(s1 - s_first);  // stage st+1 closes stream s1
    load_ry(ic<k>{}, st + D < nst, sD, cD);  // slot k held stage st, combined in iteration st-1
    if (st < nst) {
      contract(wcur, acur);
      if (c0 + 64 == c_end) fold(s0 - s_first);  // stage st closed stream s0 (its rrms is visible since the barrier)
    }
    s0 = s1; c0 = c1;
    advance(s1, c1);
    advance(sD, cD);
  };
  // groups of G iterations (slots and buffers by position in the group);
  // iterations past the last stage only keep the ring in step
  for (int st = 0; st < nst; st += G) static_for<0, G>([&](auto P) { iteration(P, st + decltype(P)::value); });
  // the loads issued past the last stage must land before the LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  if (lead && nseg == 1)
    for (int i = tid; i < SPW * TM; i += NT) {
      const int sl = i / TM, t = i % TM;
      if (t < rows) a.rrms[(m0 + t) * a.HC + s_first + sl] = rrs[sl][t];
    }
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    if (i >= wcnt) continue;
    const int n0 = (b0 + qb0 + i) * 16 + 4 * (lane >> 4);
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      const int t = th * (TM / 2) + tb * 16 + (lane & 15);
      if (t >= rows) continue;
      const int64_t m = m0 + t;
      if constexpr (NSET) {
        const f32x4_t v = acc_t[i][tb];
        if (n0 < a.r) {
          float z[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) z[q] = v[q] * a.inv_hc;
          uint2 o;
          o.x = pack_bf2(z[0] * sigmoid_f(z[0]), z[1] * sigmoid_f(z[1]));  // (G1) SiLU(lora / HC)
          o.y = pack_bf2(z[2] * sigmoid_f(z[2]), z[3] * sigmoid_f(z[3]));
          *reinterpret_cast<uint2*>(a.h + m * a.r + n0) = o;
        } else if (n0 < a.r + a.HC) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (n0 + q < a.r + a.HC) a.inj_next[m * a.ld_inj_next + (n0 - a.r + q)] = to_bf(v[q]);  // (INJ)
        }
      } else {
        const float rr = rrs[0][t];
        if (n0 < a.r + a.HC) {
          f32x4_t v = acc_s[i][tb];
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] *= rr;
          *reinterpret_cast<f32x4_t*>(a.Q + ((int64_t)(s_first * nseg + seg) * a.Mq + m) * a.NP + n0) = v;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// hcgr_k1_sum (STREAM plan, and TILE with one stream per workgroup):
// v = sum_s rrms_s P_s for each token and row; down rows -> h = SiLU(v/HC)
// (bf16), inject rows -> inj_next. P_s arrives rrms-scaled, or as unscaled
// column-segment partials with their sums of squares, from which rrms is
// formed here (and written). One lane per (token, 8 consecutive rows,
// stream); the four stream lanes are adjacent and combine by shuffles.
// ---------------------------------------------------------------------------
struct SumArgs {
  const float* Q;  // [HC*nseg][Mq][NP]
  int64_t Mq, M;
  int NP, r, n_rows;
  float inv_hc;
  uint16_t* h;
  uint16_t* inj_next;
  int64_t ld_inj_next;
  int nseg;          // > 1: Q holds unscaled segment partials and SSp their sums of squares
  const float* SSp;  // [HC*nseg][Mq]
  float* rrms;       // written when nseg > 1
  float eps, inv_hs;
};

// ONE: a single segment per stream (the large-M plans), straight-line with
// both loads of a lane issued together (measured on MI355X at M = 65536 and
// 8192: 8-13% faster than the segment loop); the segment loop keeps its own
// register budget (eight waves per SIMD).
// SG: lanes sharing one (token, chunk, stream), lane j summing segments
// j, j + SG, ..., for grids smaller than the CU count, where a lane's
// dependent rounds of loads set the time (HC = 2, M = 32, HS = 2560,
// r = 320, 20 segments: 11 workgroups of 256 lanes become 41).
template <int HC, bool ONE, int SG>
__global__ __launch_bounds__(256) void hcgr_k1_sum(SumArgs a) {
  // lane = (token m, chunk c of 8 rows, segment lane j, stream s); s is the
  // fastest index and j the next, so the HC*SG lanes of a (token, chunk)
  // form an aligned group (HC = 1, 2, 4, 8; SG = 1, 4)
  static_assert(HC == 1 || HC == 2 || HC == 4 || HC == 8, "stream lanes form an aligned group");
  static_assert((SG == 1 || SG == 4) && !(ONE && SG != 1), "segment lanes: 1, or 4 in the segment loop");
  constexpr int LG = HC == 1 ? 0 : HC == 2 ? 1 : HC == 4 ? 2 : 3;
  constexpr int LS = SG == 1 ? 0 : 2;
  const int nch = a.r / 8 + (HC + 7) / 8;  // r/8 chunks of h, then the chunk(s) holding the inject rows
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int s = (int)(idx & (HC - 1));
  const int j = (int)((idx >> LG) & (SG - 1));
  const int64_t mc = idx >> (LG + LS);
  const int64_t m = min(mc / nch, a.M - 1);  // lanes past M recompute the last token and store nothing
  const int c = (int)(mc % nch);
  const bool live = mc / nch < a.M;
  const int n = c * 8;
  float rr = 1.0f;  // partials arrive rrms-scaled unless the streams were split into segments
  if (!ONE && a.nseg > 1) {  // (N) rrms of stream s from its segments' sums of squares
    float sq = 0.0f;
    for (int g = j; g < a.nseg; g += SG) sq += a.SSp[(int64_t)(s * a.nseg + g) * a.Mq + m];
#pragma unroll
    for (int d = HC; d < HC * SG; d <<= 1) sq += __shfl_xor(sq, d, 64);
    rr = 1.0f / sqrtf(sq * a.inv_hs + a.eps);
    if (live && c == 0 && j == 0) a.rrms[m * HC + s] = rr;
  }
  float u[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) u[e] = 0.0f;
  const int64_t gstride = a.Mq * a.NP * SG;  // between this lane's segments
  const float* p = a.Q + ((int64_t)(s * a.nseg + j) * a.Mq + m) * a.NP + n;
  const int nmine = ONE ? 1 : (a.nseg - j + SG - 1) / SG;  // segments of this lane
  if constexpr (ONE) {
    const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(p), hi = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      u[e] = lo[e];
      u[e + 4] = hi[e];
    }
  }
  int g = ONE ? nmine : 0;
  for (; g + 4 <= nmine; g += 4) {  // four segments' loads in flight at once
    f32x4_t lo[4], hi[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo[j] = *reinterpret_cast<const f32x4_t*>(p + (g + j) * gstride);
      hi[j] = *reinterpret_cast<const f32x4_t*>(p + (g + j) * gstride + 4);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u[e] += lo[j][e];
        u[e + 4] += hi[j][e];
      }
  }
  for (; g < nmine; ++g) {
    const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(p + g * gstride);
    const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(p + g * gstride + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      u[e] += lo[e];
      u[e + 4] += hi[e];
    }
  }
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {  // sum over the segment lanes, then the HC stream lanes
#pragma unroll
    for (int d = HC; d < HC * SG; d <<= 1) u[e] += __shfl_xor(u[e], d, 64);
    v[e] = rr * u[e];
#pragma unroll
    for (int d = 1; d < HC; d <<= 1) v[e] += __shfl_xor(v[e], d, 64);
  }
  if (!live || s != 0 || j != 0) return;
  if (n < a.r) {
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float z0 = v[2 * e] * a.inv_hc, z1 = v[2 * e + 1] * a.inv_hc;
      o[e] = pack_bf2(z0 * sigmoid_f(z0), z1 * sigmoid_f(z1));  // (G1) SiLU(lora / HC)
    }
    st16(a.h + m * a.r + n, make_uint4(o[0], o[1], o[2], o[3]));
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (n + e < a.n_rows) a.inj_next[m * a.ld_inj_next + (n - a.r + e)] = to_bf(v[e]);  // (INJ)
  }
}

// x = 1/4 sum_s xn_s sigmoid(g_s) with one reciprocal: d_s = 1 + e^(-g_s),
// sum_s xn_s / d_s = N / D, D = d0 d1 d2 d3, N = (xn0 d1 + xn1 d0) d2 d3 +
// (xn2 d3 + xn3 d2) d0 d1. g is clamped below at -20 so that D stays finite
// (d <= 4.9e8, D <= 5.7e34); sigmoid(-20) = 2.1e-9 bounds the change.
__device__ __forceinline__ float mix4(const float g[4], const float xn[4]) {
  float d[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) d[s] = 1.0f + __expf(-fmaxf(g[s], -20.0f));
  const float d01 = d[0] * d[1], d23 = d[2] * d[3];
  const float n01 = fmaf(xn[0], d[1], xn[1] * d[0]);
  const float n23 = fmaf(xn[2], d[3], xn[3] * d[2]);
  return 0.25f * fmaf(n01, d23, n23 * d01) * __builtin_amdgcn_rcpf(d01 * d23);
}

// ---------------------------------------------------------------------------
// hcgr_k2_stage: (G2) + (MIX) for a tile of 128 tokens x 32 channels (x 4
// streams = 128 gate columns), 4 waves; wave (ch, th) owns channels ch*16..
// and tokens th*64.. as 4 x 4 MFMA tiles (A = Wu rows, B = h rows). h and Wu
// pass through LDS in stages of 64 k (one 128-byte line per row) by direct
// global->LDS loads: one 32 KB stage buffer with four workgroups sharing a
// CU, so one's load waits are covered by the others' work, or two buffers
// for small grids (the DB template flag below). Fragment reads are
// batched asm blocks (every LDS read they make is covered by the stage
// wait). Inside a 16-row MFMA block, row 4j+s is stream s of channel 4j+gb
// of the wave's block gb, so lane l ends with the 4 streams of channels
// 4*(l/16)+gb, gb = 0..3, of token l%16: the MIX sum over streams is
// lane-local and each lane moves 8 contiguous bytes of R2 and x per stream
// and token. Workgroups b and b+8 (the same XCD) take the two 32-channel
// halves of a 64-channel group, so the second half of every 128-byte R2
// line is an L2 hit, and each XCD sees a fixed subset of channel groups
// (their Wu slices stay in its L2).
// ---------------------------------------------------------------------------
struct StageArgs {
  const uint16_t* h;  // [>= M, r]
  int64_t M;
  int r, HS, K;
  const uint16_t* wu;
  const uint16_t* R2;
  const float* rrms;
  const uint16_t* wn;
  int wn_len;
  uint16_t* x;
  int npairs;  // 64-channel groups (HS / 64)
};

// DB: two stage buffers (separate arrays, so the compiler sees which one a
// read touches), stage s + 1 loading while stage s contracts, for grids of
// at most two workgroups per CU (the 64 KB of LDS allows two); larger grids
// keep one 32 KB buffer and four workgroups per CU, whose work covers each
// other's load waits. Measured on MI355X (HS = 2560, r = 320): two buffers
// 27% faster at M = 256 (160 workgroups), 12% at 512, 7-9% slower at 1024
// and 2048.
template <bool DB>
__global__ __launch_bounds__(256, DB ? 2 : 4) void hcgr_k2_stage(StageArgs a) {
  constexpr int TM = 128, CG = 32, SB = 16384;  // tokens, channels per workgroup, bytes per h (or Wu) stage
  __shared__ __attribute__((aligned(1024))) uint8_t hb[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t wb[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t hb1[DB ? SB : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t wb1[DB ? SB : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ch = wave & 1, th = wave >> 1;
  // workgroup -> (token tile, 32-channel group): b and b + 8 share a 64-channel pair
  const int b = (int)blockIdx.x;
  const int pair_idx = (b >> 4) * 8 + (b & 7);  // token tile major, 64-channel pair minor
  const int half = (b >> 3) & 1;
  const int64_t tile = pair_idx / a.npairs;
  const int c0 = (pair_idx % a.npairs) * 64 + half * CG;
  const int64_t m0 = tile * TM;
  if (m0 >= a.M) return;  // grid rounded up to 16 workgroups
  const int rows = (int)min((int64_t)TM, a.M - m0);
  const uint32_t rowb = (uint32_t)a.K * 2u, hrow = (uint32_t)a.r * 2u;
  const int nstage = (a.r + 63) / 64;

  const rsrc_t rH = make_rsrc(a.h + m0 * a.r, (uint32_t)rows * hrow);
  const rsrc_t rWu = make_rsrc(a.wu, (uint32_t)a.K * hrow);
  const rsrc_t rR2 = make_rsrc(a.R2 + m0 * a.K, (uint32_t)rows * rowb);
  const rsrc_t rRr = make_rsrc(a.rrms + m0 * 4, (uint32_t)rows * 16u);
  const rsrc_t rX = make_rsrc(a.x + m0 * a.HS, (uint32_t)rows * (uint32_t)a.HS * 2u);

  // DMA: 8-row groups g = wave + 4 i (i < 4) of h and of Wu; lane -> row g*8 + (lane >> 3), 16-byte chunk swz
  const uint32_t swz = (uint32_t)((lane & 7) ^ (lane >> 3));
  uint32_t hoff[4], woff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = wave + 4 * i;
    const int rl = g * 8 + (lane >> 3);  // LDS row
    hoff[i] = (uint32_t)rl * hrow + swz * 16u;
    // Wu LDS row rl: block B = rl / 16 (channel half B / 4, gb = B % 4), row 4j + s
    const int B = rl >> 4, ii = rl & 15, j = ii >> 2, s = ii & 3;
    const int c = c0 + (B >> 2) * 16 + 4 * j + (B & 3);
    woff[i] = (uint32_t)(s * a.HS + c) * hrow + swz * 16u;
  }
  auto issue = [&](int stg, uint8_t* hbuf, uint8_t* wbuf) {
    const uint32_t kb = (uint32_t)stg * 128u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = wave + 4 * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rH, (lds_void_t*)(hbuf + g * 1024), 16, hoff[i] + kb, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rWu, (lds_void_t*)(wbuf + g * 1024), 16, woff[i] + kb, 0, 0, 0);
    }
  };

  f32x4_t acc[4][4];  // [gb][tb]
#pragma unroll
  for (int gb = 0; gb < 4; ++gb)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) acc[gb][tb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // fragment addresses (LDS byte offsets): A block ch*4 + gb at +gb*2048, B token tile th*4 + tb at +tb*2048
  const uint32_t slot0 = (uint32_t)(((lane >> 4) ^ (lane & 7)) * 16);
  const uint32_t slot1 = (uint32_t)(((4 + (lane >> 4)) ^ (lane & 7)) * 16);
  const uint32_t arow = (uint32_t)((ch * 64 + (lane & 15)) * 128), brow = (uint32_t)((th * 64 + (lane & 15)) * 128);
  auto contract = [&](const uint8_t* hbuf, const uint8_t* wbuf, bool both) {
    const uint32_t wa = (uint32_t)(uintptr_t)(lds_u8_t*)wbuf + arow, ha = (uint32_t)(uintptr_t)(lds_u8_t*)hbuf + brow;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (ks == 1 && !both) break;  // half stage (r % 64 == 32)
      const uint32_t sl = ks ? slot1 : slot0;
      u32x4_t af[4], bf[4];
      asm volatile(
          "ds_read_b128 %0, %8\n\t"
          "ds_read_b128 %1, %8 offset:2048\n\t"
          "ds_read_b128 %2, %8 offset:4096\n\t"
          "ds_read_b128 %3, %8 offset:6144\n\t"
          "ds_read_b128 %4, %9\n\t"
          "ds_read_b128 %5, %9 offset:2048\n\t"
          "ds_read_b128 %6, %9 offset:4096\n\t"
          "ds_read_b128 %7, %9 offset:6144\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3]), "=&v"(bf[0]), "=&v"(bf[1]), "=&v"(bf[2]),
            "=&v"(bf[3])
          : "v"(wa + sl), "v"(ha + sl)
          : "memory");
#pragma unroll
      for (int gb = 0; gb < 4; ++gb)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
          acc[gb][tb] = mfma16(__builtin_bit_cast(uint4, af[gb]), __builtin_bit_cast(uint4, bf[tb]), acc[gb][tb]);
    }
  };

  // epilogue operands of this lane: channels cl..cl+3, tokens th*64 + tb*16 + (lane & 15)
  const int cl = c0 + ch * 16 + 4 * (lane >> 4);
  uint2 r2v[4][4];  // [tb][s]
  f32x4_t rrv[4];   // [tb]
  auto load_epilogue = [&]() {
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const uint32_t t = (uint32_t)(th * 64 + tb * 16 + (lane & 15));
      rrv[tb] = __builtin_bit_cast(f32x4_t, bld16(rRr, t * 16u));
#pragma unroll
      for (int s = 0; s < 4; ++s) r2v[tb][s] = bld8(rR2, t * rowb + (uint32_t)(s * a.HS + cl) * 2u);
    }
  };

  // Stage stg in buffer stg % 2. Every thread issues 8 loads per stage (4 of
  // h, 4 of Wu) and no other vector memory operation in the loop, so with
  // the next stage issued, vmcnt(8) leaves exactly its loads in flight.
  auto step = [&](auto P, int stg) {
    constexpr int par = decltype(P)::value;
    if (!DB) {  // one buffer: load, wait, contract
      issue(stg, hb, wb);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_sync();
      contract(hb, wb, 64 * stg + 64 <= a.r);
      lds_sync();
      return;
    }
    if (stg + 1 < nstage) {
      issue(stg + 1, par ? hb : hb1, par ? wb : wb1);
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    lds_sync();                                                          // every wave's part of stage stg has landed
    contract(par ? hb1 : hb, par ? wb1 : wb, 64 * stg + 64 <= a.r);     // a half stage when r % 64 == 32
    lds_sync();                                                          // buffer par is free for stage stg + 2
  };
  if (DB) issue(0, hb, wb);
  for (int stg = 0; stg < nstage; stg += 2) {
    step(ic<0>{}, stg);
    if (stg + 1 < nstage) step(ic<1>{}, stg + 1);
  }
  load_epilogue();

  // (G2) sigmoid and (MIX) over the lane's four stream accumulators
  float onep[4][4];  // [s][gb]
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint2 w = *reinterpret_cast<const uint2*>(a.wn + (a.wn_len == a.HS ? 0 : s * a.HS) + cl);
    onep[s][0] = 1.0f + bf_lo(w.x);
    onep[s][1] = 1.0f + bf_hi(w.x);
    onep[s][2] = 1.0f + bf_lo(w.y);
    onep[s][3] = 1.0f + bf_hi(w.y);
  }
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const uint32_t t = (uint32_t)(th * 64 + tb * 16 + (lane & 15));
    float xo[4];
#pragma unroll
    for (int gb = 0; gb < 4; ++gb) {
      float g[4], xn[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t w = gb < 2 ? r2v[tb][s].x : r2v[tb][s].y;
        const float r2 = (gb & 1) ? bf_hi(w) : bf_lo(w);
        g[s] = acc[gb][tb][s];
        xn[s] = r2 * rrv[tb][s] * onep[s][gb];
      }
      xo[gb] = mix4(g, xn);
    }
    bst8(rX, (t * (uint32_t)a.HS + (uint32_t)cl) * 2u, make_uint2(pack_bf2(xo[0], xo[1]), pack_bf2(xo[2], xo[3])));
  }
}

// ---------------------------------------------------------------------------
// hcgr_k2_sweep (large token counts): (G2) + (MIX) for a tile of 128 tokens
// over a range of 32-channel groups (x 4 streams = 128 gate rows per group).
// The tile's h is loaded once into registers as MFMA B fragments (NKS
// stages of 64 k). A group's Wu rows pass through an LDS ring of NKS stages
// (one per k stage; stage q+NKS-1 loads while stage q contracts) and its R2
// rows and Wnorm through a double-buffered LDS area, all by direct
// global->LDS loads. Waves 0-3 issue only Wu loads and waves 4-7 only R2
// loads, so a wave's loads complete in issue order without one kind waiting
// behind the other. Eight waves, two per SIMD: wave (rq, tq) owns 16
// channels of the group (4 MFMA row blocks; row 4j+s of block gb is stream
// s of channel 4j+gb, so lane l ends with the four streams of channels
// 4*(l/16)+gb, gb = 0..3, and the MIX sum is lane-local) and tokens 32tq..
// (two column blocks). A group's sigmoid + MIX epilogue runs at the next
// group's first stage beside that stage's products.
// ---------------------------------------------------------------------------
struct SweepArgs {
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

constexpr int kSweepTm = 128, kSweepCg = 32;
constexpr int kSweepWsb = 4 * kSweepCg * 128;                    // one Wu stage: 128 rows x 64 k
constexpr int kSweepR2b = 4 * kSweepTm * kSweepCg * 2 + 4 * 1024;  // a group's R2 (4 streams x 128 tokens x 64 B) + 4 Wnorm slots
inline constexpr size_t sweep_lds_bytes(int nks) { return (size_t)nks * kSweepWsb + 2 * (size_t)kSweepR2b; }

template <int NKS>
__global__ __launch_bounds__(512) void hcgr_k2_sweep(SweepArgs a) {
  constexpr int TM = kSweepTm, CG = kSweepCg, NTB = 2, WSB = kSweepWsb, R2B = kSweepR2b;
  constexpr int R2S = TM * CG * 2;  // one stream of a group's R2 (8 KB)
  constexpr uint32_t kOut = 0x80000000u;
  static_assert(NKS >= 2 && NKS <= 5, "ring of 2..5 k stages");
  static_assert(sweep_lds_bytes(5) <= 160 * 1024, "LDS of one CU");
  extern __shared__ __attribute__((aligned(1024))) uint8_t dl[];
  uint8_t* wring = dl;              // [NKS][128 rows][128 B]
  uint8_t* r2buf = dl + NKS * WSB;  // [2]{[4 streams][TM tokens][64 B], [4][1 KB Wnorm slot]}

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rq = wave & 1, tq = wave >> 1;
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

  // h of the lane's tokens as B fragments (past r: zeros), and their rrms
  u32x4_t hf[NKS][2][NTB];
  f32x4_t rrv[NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    const uint32_t t = (uint32_t)(tq * 32 + tb * 16 + (lane & 15));
#pragma unroll
    for (int j = 0; j < NKS; ++j)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int k = j * 64 + ks * 32 + 8 * (lane >> 4);
        hf[j][ks][tb] = __builtin_bit_cast(u32x4_t, bld16(rH, k < a.r ? t * hrow + (uint32_t)k * 2u : kOut));
      }
    rrv[tb] = __builtin_bit_cast(f32x4_t, bld16(rRr, t * 16u));
  }

  // Wu loads (waves 0-3): 8-row groups G = wave + 4 i (i < 4) of the 128
  // stage rows; LDS row rl = 16 blk + 4 jj + s holds stream s of channel
  // 16 (blk / 4) + 4 jj + (blk % 4) of the group, its 16-byte chunk c in slot
  // c ^ (rl & 7); k past r reads zeros
  const uint32_t swz = (uint32_t)((lane & 7) ^ (lane >> 3));
  uint32_t woff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = ((wave & 3) + 4 * i) * 8 + (lane >> 3);
    const int blk = rl >> 4, jj = (rl >> 2) & 3, s = rl & 3;
    woff[i] = (uint32_t)(s * a.HS + 16 * (blk >> 2) + 4 * jj + (blk & 3)) * hrow + swz * 16u;
  }
  auto issue_wu = [&](bool valid, int g, int j) {  // !valid: past the sweep, reads zeros
    uint8_t* buf = wring + j * WSB;
    const uint32_t base = (uint32_t)(g * CG) * hrow + (uint32_t)j * 128u;
    const bool inr = valid && j * 64 + (int)swz * 8 < a.r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rWu, (lds_void_t*)(buf + ((wave & 3) + 4 * i) * 1024), 16,
                                               inr ? woff[i] + base : kOut, 0, 0, 0);
  };
  // R2 loads (waves 4-7): instruction n = wave - 4 + 4 i (i < 8) moves stream
  // n / 8, tokens 16 (n % 8) .. +15, 64 bytes each (lane: token lane / 4,
  // chunk lane % 4); then one Wnorm load per wave into its 1 KB slot (wave 4:
  // the group's values, the others: zeros)
  auto issue_r2 = [&](bool valid, int g, int b) {  // !valid: past the sweep, reads zeros
    uint8_t* buf = r2buf + b * R2B;
    const int c0 = g * CG;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n = (wave - 4) + 4 * i, s = n >> 3;
      const uint32_t t = (uint32_t)((n & 7) * 16 + (lane >> 2));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rR2, (lds_void_t*)(buf + s * R2S + (n & 7) * 1024), 16,
          valid ? t * rowb + (uint32_t)(s * a.HS + c0) * 2u + (uint32_t)(lane & 3) * 16u : kOut, 0, 0, 0);
    }
    const bool full = a.wn_len != a.HS;
    const bool live = valid && wave == 4 && lane < (full ? 16 : 4);
    const uint32_t wo = (uint32_t)((full ? (lane >> 2) * a.HS : 0) + c0 + (full ? (lane & 3) : lane) * 8) * 2u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rWn, (lds_void_t*)(buf + 4 * R2S + (wave - 4) * 1024), 16,
                                             live ? wo : kOut, 0, 0, 0);
  };

  f32x4_t acc[4][NTB];
#pragma unroll
  for (int gb = 0; gb < 4; ++gb)
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) acc[gb][tb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // (G2) one k stage: A = the wave's 64 Wu rows, B = h fragments. Past r (a
  // half last stage) both operands are zeros, so the second k step of that
  // stage adds nothing and runs unconditionally.
  const uint32_t wbase = (uint32_t)(uintptr_t)(lds_u8_t*)wring + (uint32_t)((rq * 64 + (lane & 15)) * 128);
  const uint32_t slot0 = (uint32_t)(((lane >> 4) ^ (lane & 7)) * 16);
  const uint32_t slot1 = (uint32_t)(((4 + (lane >> 4)) ^ (lane & 7)) * 16);
  typedef u32x4_t afrag_t[2][4];
  auto load_a = [&](auto J, afrag_t& af) {
    constexpr int j = decltype(J)::value;
    const uint32_t wa = wbase + (uint32_t)(j * WSB);
    const uint32_t a0 = wa + slot0, a1 = wa + slot1;
    // every LDS read here is covered by the stage wait; one asm block with its
    // wait inside, so the outputs are complete when it ends and the compiler
    // adds no wait for the ring's later loads
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:2048\n\t"
        "ds_read_b128 %2, %8 offset:4096\n\t"
        "ds_read_b128 %3, %8 offset:6144\n\t"
        "ds_read_b128 %4, %9\n\t"
        "ds_read_b128 %5, %9 offset:2048\n\t"
        "ds_read_b128 %6, %9 offset:4096\n\t"
        "ds_read_b128 %7, %9 offset:6144\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(af[0][0]), "=&v"(af[0][1]), "=&v"(af[0][2]), "=&v"(af[0][3]), "=&v"(af[1][0]), "=&v"(af[1][1]),
          "=&v"(af[1][2]), "=&v"(af[1][3])
        : "v"(a0), "v"(a1)
        : "memory");
  };
  auto products = [&](auto J, const afrag_t& af) {
    constexpr int j = decltype(J)::value;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int gb = 0; gb < 4; ++gb)
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
          acc[gb][tb] = mfma16(__builtin_bit_cast(uint4, af[ks][gb]), __builtin_bit_cast(uint4, hf[j][ks][tb]),
                               acc[gb][tb]);
  };

  // (G2) sigmoid + (MIX) of a finished group: x of the lane's 4 channels for
  // each column block. The LDS reads (R2 and Wnorm of the group) come first,
  // apart from the arithmetic, so that the arithmetic can interleave with a
  // stage's products.
  const uint32_t r2lane = (uint32_t)(uintptr_t)(lds_u8_t*)r2buf + (uint32_t)(rq * 32 + 8 * (lane >> 4));
  const uint32_t wstep = a.wn_len != a.HS ? 64u : 0u;  // Wnorm indexed by k: one 64-byte row per stream
  struct EpiIn { u32x2_t wv[4], rv[NTB][4]; };
  auto epi_load = [&](int b, EpiIn& e) {
    const uint32_t rb = r2lane + (uint32_t)(b * R2B);
    const uint32_t wa = rb + (uint32_t)(4 * R2S);
    const uint32_t t0 = rb + (uint32_t)(tq * 32 + (lane & 15)) * 64u;  // column block 0; block 1 is 16 tokens on
    static_assert(NTB == 2 && R2S == 8192, "offsets below");
    asm volatile(
        "ds_read_b64 %0, %12\n\t"
        "ds_read_b64 %1, %13\n\t"
        "ds_read_b64 %2, %14\n\t"
        "ds_read_b64 %3, %15\n\t"
        "ds_read_b64 %4, %16\n\t"
        "ds_read_b64 %5, %16 offset:8192\n\t"
        "ds_read_b64 %6, %16 offset:16384\n\t"
        "ds_read_b64 %7, %16 offset:24576\n\t"
        "ds_read_b64 %8, %16 offset:1024\n\t"
        "ds_read_b64 %9, %16 offset:9216\n\t"
        "ds_read_b64 %10, %16 offset:17408\n\t"
        "ds_read_b64 %11, %16 offset:25600\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(e.wv[0]), "=&v"(e.wv[1]), "=&v"(e.wv[2]), "=&v"(e.wv[3]), "=&v"(e.rv[0][0]), "=&v"(e.rv[0][1]),
          "=&v"(e.rv[0][2]), "=&v"(e.rv[0][3]), "=&v"(e.rv[1][0]), "=&v"(e.rv[1][1]), "=&v"(e.rv[1][2]),
          "=&v"(e.rv[1][3])
        : "v"(wa), "v"(wa + wstep), "v"(wa + 2u * wstep), "v"(wa + 3u * wstep), "v"(t0)
        : "memory");
  };
  // live = false: the x stores go out of range (dropped)
  auto epi_math = [&](const EpiIn& e, bool live, int g, const f32x4_t (&ac)[4][NTB]) {
    float onep[4][4];  // [s][gb]
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      onep[s][0] = 1.0f + bf_lo(e.wv[s][0]);
      onep[s][1] = 1.0f + bf_hi(e.wv[s][0]);
      onep[s][2] = 1.0f + bf_lo(e.wv[s][1]);
      onep[s][3] = 1.0f + bf_hi(e.wv[s][1]);
    }
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      float xq[4];
#pragma unroll
      for (int gb = 0; gb < 4; ++gb) {
        float gs[4], xn[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t w = gb < 2 ? e.rv[tb][s][0] : e.rv[tb][s][1];
          const float r2 = (gb & 1) ? bf_hi(w) : bf_lo(w);
          gs[s] = ac[gb][tb][s];
          xn[s] = r2 * rrv[tb][s] * onep[s][gb];
        }
        xq[gb] = mix4(gs, xn);
      }
      const uint32_t t = (uint32_t)(tq * 32 + tb * 16 + (lane & 15));
      bst8(rX, live ? (t * (uint32_t)a.HS + (uint32_t)(g * CG + rq * 16 + 4 * (lane >> 4))) * 2u : kOut,
           make_uint2(pack_bf2(xq[0], xq[1]), pack_bf2(xq[2], xq[3])));
    }
  };

  // prologue: Wu of stages 0 .. NKS-2 of the first group (waves 0-3), R2 of
  // the first group (waves 4-7); h and rrms above
  if (wave < 4) {
#pragma unroll
    for (int j = 0; j < NKS - 1; ++j) issue_wu(true, g_begin, j);
  } else {
    issue_r2(true, g_begin, 0);
  }
  // vmcnt(0) through the builtin (0x0f70: expcnt and lgkmcnt left open), so the
  // compiler also knows the h and rrms registers have landed
  __builtin_amdgcn_s_waitcnt(0x0f70);
  lds_sync();

  // Stage (g, j). At its top a Wu wave has issued the Wu of every stage up to
  // (g, j) + NKS - 2, 4 loads per stage (stages past the sweep included, as
  // out-of-range loads, so the count never changes); vmcnt(4 (NKS - 2))
  // counts later loads only (a store may complete ahead of earlier loads) and
  // leaves the NKS - 2 newer stages in flight. Stage (g, j) loads the Wu of
  // stage (g, j) + NKS - 1 into ring slot j - 1 (read by the previous stage).
  // The epilogue of group g runs at stage (g + 1, 0), beside that stage's
  // products, from the accumulators set aside at the end of group g; so
  // R2(g) must stay until then, and R2(g + 1) loads at stage (g, 1) into the
  // other buffer (free once the epilogue of g - 1 is done). At stage
  // (g + 1, 0) an R2 wave waits for R2(g) with the 9 loads of R2(g + 1) left
  // in flight.
  f32x4_t accp[4][NTB];  // group g - 1, waiting for its epilogue
#pragma unroll
  for (int gb = 0; gb < 4; ++gb)
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) accp[gb][tb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  for (int g = g_begin; g < g_end; ++g) {
    const int b = (g - g_begin) & 1;
    auto stage = [&](auto J) {
      constexpr int j = decltype(J)::value;
      if (g != g_begin || j != 0) {
        if (wave < 4) {
          if constexpr (NKS == 2) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          else if constexpr (NKS == 3) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
          else if constexpr (NKS == 4) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
          else asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
        } else if (j == 0) {
          asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
        }
        lds_sync();
      }
      if (wave < 4) {
        constexpr int q2 = j + NKS - 1;  // stage (g, q2), or (g + 1, q2 - NKS)
        const int gn = q2 >= NKS ? g + 1 : g;
        issue_wu(gn < g_end, gn, q2 >= NKS ? q2 - NKS : q2);
      } else if (j == 1) {
        issue_r2(g + 1 < g_end, g + 1, b ^ 1);
      }
      afrag_t af;
      load_a(J, af);
      if constexpr (j == 0) {  // the previous group's epilogue beside this stage's products
        EpiIn e;
        epi_load(b ^ 1, e);
        products(J, af);
        epi_math(e, g != g_begin, g - 1, accp);
      } else {
        products(J, af);
      }
      if constexpr (j == NKS - 1) {
#pragma unroll
        for (int gb = 0; gb < 4; ++gb)
#pragma unroll
          for (int tb = 0; tb < NTB; ++tb) {
            accp[gb][tb] = acc[gb][tb];
            acc[gb][tb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
          }
      }
    };
    stage(ic<0>{});
    stage(ic<1>{});
    if constexpr (NKS > 2) stage(ic<2>{});
    if constexpr (NKS > 3) stage(ic<3>{});
    if constexpr (NKS > 4) stage(ic<4>{});
  }
  // the last group's epilogue
  if (wave >= 4) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lds_sync();
  {
    EpiIn e;
    epi_load((g_end - 1 - g_begin) & 1, e);
    epi_math(e, true, g_end - 1, accp);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ---------------------------------------------------------------------------
// hcgr_k2_gen (stream counts other than 4): (G2) gate = h . Wu^T, G =
// sigmoid(gate), (MIX) x[c] = 1/HC sum_s G[s,c] xn[s,c], for a tile of TM =
// 64 or 128 tokens x 32 channels x HC streams, TM / 16 waves (the 128-token
// tile reads each Wu row once per 128 tokens). Wave (ch, th) owns channels
// 16ch.. of the tile and tokens 32th..: for each stream s one 16-row MFMA
// block whose row i is Wu row s*HS + c0 + 16ch + i, so lane l ends with the
// same four channels 4(l/16).. of token l%16 for every stream and the MIX sum
// over streams is lane-local. h (TM rows) and the tile's Wu rows (32 HC rows)
// pass through two LDS stage buffers of 64 k by direct global->LDS loads
// (stage s + 1 loads while stage s contracts), 16-byte chunk c of LDS row t
// in slot c ^ (t & 7); a half last stage (r % 64 == 32) contracts its first
// 32 k only.
// ---------------------------------------------------------------------------
struct GenUpArgs {
  const uint16_t* h;  // [>= M, r]
  int64_t M;
  int r, HS, K;
  const uint16_t* wu;  // [K, r]
  const uint16_t* R2;  // [M, K]
  const float* rrms;   // [M, HC]
  const uint16_t* wn;
  int wn_len;
  uint16_t* x;  // [M, HS]
  int ngroups;  // HS / 32
};

constexpr int kGenCg = 32;

// TM: 64 tokens (4 waves) or 128 (8 waves, HC = 2 or 8); a wave always owns
// 16 channels x 32 tokens of every stream.
template <int HC, int TM>
__global__ __launch_bounds__(TM * 4) void hcgr_k2_gen(GenUpArgs a) {
  constexpr int CG = kGenCg, NTB = 2, NW = TM / 16;
  static_assert((TM == 64 || (TM == 128 && HC % 2 == 0)) && (4 * HC) % NW == 0, "whole Wu loads per wave");
  constexpr int HB = TM * 128, WB = HC * CG * 128;  // LDS bytes of one stage of h and of Wu
  constexpr int NH = TM / 8 / NW, NWU = 4 * HC / NW;  // h and Wu loads per wave per stage
  constexpr int NL = NH + NWU;                        // loads per thread per stage
  // vmcnt(NL): the newest stage's loads stay in flight (expcnt and lgkmcnt left open)
  constexpr int kWaitNewest = (NL & 15) | ((NL >> 4) << 14) | (7 << 4) | (15 << 8);
  // two stage buffers, separate arrays picked at compile time (stage parity
  // P): stage s + 1 loads while stage s contracts, and the compiler can tell
  // that the reads of one buffer do not wait for the loads into the other
  __shared__ __attribute__((aligned(1024))) uint8_t hb0[HB];
  __shared__ __attribute__((aligned(1024))) uint8_t hb1[HB];
  __shared__ __attribute__((aligned(1024))) uint8_t wb0[WB];
  __shared__ __attribute__((aligned(1024))) uint8_t wb1[WB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ch = wave & 1, th = wave >> 1;
  const int64_t tile = (int64_t)blockIdx.x / a.ngroups;
  const int c0 = (int)((int64_t)blockIdx.x % a.ngroups) * CG;
  const int64_t m0 = tile * TM;
  const int rows = (int)min((int64_t)TM, a.M - m0);
  const uint32_t rowb = (uint32_t)a.K * 2u, hrow = (uint32_t)a.r * 2u;
  const int nstage = (a.r + 63) / 64;

  const rsrc_t rH = make_rsrc(a.h + m0 * a.r, (uint32_t)rows * hrow);  // tokens past M read zeros
  const rsrc_t rWu = make_rsrc(a.wu, (uint32_t)a.K * hrow);
  const rsrc_t rR2 = make_rsrc(a.R2 + m0 * a.K, (uint32_t)rows * rowb);
  const rsrc_t rX = make_rsrc(a.x + m0 * a.HS, (uint32_t)rows * (uint32_t)a.HS * 2u);

  // one wave instruction moves 8 rows x 128 bytes: lane -> row lane >> 3, chunk swz
  const uint32_t swz = (uint32_t)((lane & 7) ^ (lane >> 3));
  auto issue = [&](auto P, int stg) {
    const uint32_t kb = (uint32_t)stg * 128u;
    uint8_t* hb = decltype(P)::value ? hb1 : hb0;
    uint8_t* wb = decltype(P)::value ? wb1 : wb0;
#pragma unroll
    for (int i = 0; i < NH; ++i) {  // h: TM / 8 groups of 8 rows over NW waves
      const int g = wave + NW * i;
      const uint32_t row = (uint32_t)(g * 8 + (lane >> 3));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rH, (lds_void_t*)(hb + g * 1024), 16, row * hrow + swz * 16u + kb, 0,
                                               0, 0);
    }
#pragma unroll
    for (int i = 0; i < NWU; ++i) {  // Wu: HC * CG / 8 groups of 8 rows over NW waves
      const int g = wave + NW * i;
      const int rl = g * 8 + (lane >> 3);  // LDS row: stream rl / CG, channel c0 + rl % CG
      const uint32_t grow = (uint32_t)((rl / CG) * a.HS + c0 + rl % CG);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rWu, (lds_void_t*)(wb + g * 1024), 16, grow * hrow + swz * 16u + kb, 0,
                                               0, 0);
    }
  };

  f32x4_t acc[HC][NTB];
#pragma unroll
  for (int s = 0; s < HC; ++s)
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) acc[s][tb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int fr = lane & 15;  // fragment row inside a 16-row block (row & 7 == lane & 7)
  auto step = [&](auto P, int stg) {
    constexpr int par = decltype(P)::value;
    // every thread issues NL loads per stage, so with the next stage issued
    // the wait leaves exactly its loads in flight
    if (stg + 1 < nstage) {
      issue(ic<par ^ 1>{}, stg + 1);
      __builtin_amdgcn_s_waitcnt(kWaitNewest);
    } else {
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    }
    lds_sync();  // every wave's part of stage stg has landed (a barrier that leaves the next stage in flight)
    const uint8_t* hb = par ? hb1 : hb0;
    const uint8_t* wb = par ? wb1 : wb0;
    const int nks = 64 * stg + 64 <= a.r ? 2 : 1;
    for (int ks = 0; ks < nks; ++ks) {
      const int slot = ((ks * 4 + (lane >> 4)) ^ (lane & 7)) * 16;
      // the fragments of this k step, read in one asm block with its own
      // wait: the compiler would otherwise wait for every load in flight
      // (the next stage's included) before reading LDS filled by such loads
      const uint32_t ha = (uint32_t)(uintptr_t)(lds_u8_t*)hb + (uint32_t)((th * 32 + fr) * 128 + slot);
      const uint32_t wa = (uint32_t)(uintptr_t)(lds_u8_t*)wb + (uint32_t)((ch * 16 + fr) * 128 + slot);
      u32x4_t bq[NTB], af[HC];
      static_assert(NTB == 2 && CG * 128 == 4096, "offsets below: column block 1 16 rows on, stream s CG rows on");
      if constexpr (HC == 1) {
        asm volatile(
            "ds_read_b128 %0, %3\n\tds_read_b128 %1, %3 offset:2048\n\tds_read_b128 %2, %4\n\ts_waitcnt lgkmcnt(0)"
            : "=&v"(bq[0]), "=&v"(bq[1]), "=&v"(af[0])
            : "v"(ha), "v"(wa)
            : "memory");
      } else if constexpr (HC == 2) {
        asm volatile(
            "ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:2048\n\tds_read_b128 %2, %5\n\t"
            "ds_read_b128 %3, %5 offset:4096\n\ts_waitcnt lgkmcnt(0)"
            : "=&v"(bq[0]), "=&v"(bq[1]), "=&v"(af[0]), "=&v"(af[1])
            : "v"(ha), "v"(wa)
            : "memory");
      } else {
        static_assert(HC == 8, "stream counts 1, 2 and 8 take this kernel");
        asm volatile(
            "ds_read_b128 %0, %10\n\tds_read_b128 %1, %10 offset:2048\n\t"
            "ds_read_b128 %2, %11\n\tds_read_b128 %3, %11 offset:4096\n\t"
            "ds_read_b128 %4, %11 offset:8192\n\tds_read_b128 %5, %11 offset:12288\n\t"
            "ds_read_b128 %6, %11 offset:16384\n\tds_read_b128 %7, %11 offset:20480\n\t"
            "ds_read_b128 %8, %11 offset:24576\n\tds_read_b128 %9, %11 offset:28672\n\ts_waitcnt lgkmcnt(0)"
            : "=&v"(bq[0]), "=&v"(bq[1]), "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3]), "=&v"(af[4]),
              "=&v"(af[5]), "=&v"(af[6]), "=&v"(af[7])
            : "v"(ha), "v"(wa)
            : "memory");
      }
#pragma unroll
      for (int s = 0; s < HC; ++s)
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
          acc[s][tb] = mfma16(__builtin_bit_cast(uint4, af[s]), __builtin_bit_cast(uint4, bq[tb]), acc[s][tb]);
    }
    lds_sync();  // every wave is done with buffer par before stage stg + 2 refills it
  };
  issue(ic<0>{}, 0);
  for (int stg = 0; stg < nstage; stg += 2) {
    step(ic<0>{}, stg);
    if (stg + 1 < nstage) step(ic<1>{}, stg + 1);
  }

  // (G2) sigmoid and (MIX): lane holds channels cl..cl+3 of token t for every stream
  const int cl = c0 + ch * 16 + 4 * (lane >> 4);
  float onep[HC][4];
#pragma unroll
  for (int s = 0; s < HC; ++s) {
    const uint2 w = *reinterpret_cast<const uint2*>(a.wn + (a.wn_len == a.HS ? 0 : s * a.HS) + cl);
    onep[s][0] = 1.0f + bf_lo(w.x);
    onep[s][1] = 1.0f + bf_hi(w.x);
    onep[s][2] = 1.0f + bf_lo(w.y);
    onep[s][3] = 1.0f + bf_hi(w.y);
  }
  const float inv_hc = 1.0f / (float)HC;
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    const int t = th * 32 + tb * 16 + fr;
    if (t >= rows) continue;
    float xo[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < HC; ++s) {
      const float rr = a.rrms[(m0 + t) * HC + s];
      const uint2 w = bld8(rR2, (uint32_t)t * rowb + (uint32_t)(s * a.HS + cl) * 2u);
      const float r2[4] = {bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y)};
#pragma unroll
      for (int q = 0; q < 4; ++q) xo[q] = fmaf(sigmoid_f(acc[s][tb][q]), r2[q] * rr * onep[s][q], xo[q]);
    }
    bst8(rX, ((uint32_t)t * (uint32_t)a.HS + (uint32_t)cl) * 2u,
         make_uint2(pack_bf2(xo[0] * inv_hc, xo[1] * inv_hc), pack_bf2(xo[2] * inv_hc, xo[3] * inv_hc)));
  }
}

// ---------------------------------------------------------------------------
// hcgr_combine_k: (COMBINE) alone, R2[s,c] = R[s,c] + y[c]*iw[s] with
// iw[s] = 2*sigmoid(inj[s]/HC), for M tokens. Pure streaming: per token it
// reads R (HC*HS values) and y (HS) and writes R2 (HC*HS). Workgroup =
// (token, stream); its 256 threads move 16-byte chunks of that stream's row.
// Workgroup b serves token 8*(b / (8*HC)) + b % 8 and stream (b / 8) % HC, so
// the HC workgroups of one token share b % 8, which places them on one XCD
// (workgroups go round-robin over the 8 XCDs) and lets y come from that XCD's
// L2 after the first read. Every load of a thread is issued before iw is
// formed; iw is formed in fp64 by one wave and kept as an fp32 hi + lo pair,
// so R2 = (R + y*hi) + y*lo stays within an ulp under cancellation.
// ---------------------------------------------------------------------------
constexpr int kCombineThreads = 256;

// CPT: 16-byte chunks per thread per pass (1, 2, 4 or 8; rows longer than
// 8 * 256 * CPT values take several passes)
template <int CPT>
__global__ __launch_bounds__(kCombineThreads) void hcgr_combine_k(CombineArgs a) {
  const int b = (int)blockIdx.x;
  const int s = (b >> 3) % a.HC;
  const int64_t m = (int64_t)(b / (8 * a.HC)) * 8 + (b & 7);
  if (m >= a.M) return;  // whole workgroup
  const int tid = threadIdx.x;
  const int nch = a.HS / 8;  // chunks in a stream row
  const rsrc_t rR = make_rsrc(a.R + m * (int64_t)a.HC * a.HS + (int64_t)s * a.HS, (uint32_t)a.HS * 2u);
  const rsrc_t rY = make_rsrc(a.y + m * a.HS, (uint32_t)a.HS * 2u);
  const rsrc_t rO = make_rsrc(a.R2 + m * (int64_t)a.HC * a.HS + (int64_t)s * a.HS, (uint32_t)a.HS * 2u);
  __shared__ float iw_hl[2];
  for (int c0 = 0; c0 < nch; c0 += kCombineThreads * CPT) {
    uint4 rv[CPT], yv[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {  // chunks past the row read as zero
      const uint32_t off = (uint32_t)(c0 + tid + j * kCombineThreads) * 16u;
      rv[j] = a.nt ? bld16_nt(rR, off) : bld16(rR, off);
      yv[j] = bld16(rY, off);
    }
    if (c0 == 0) {
      if (tid < 64) {
        const double v = 2.0 / (1.0 + exp(-(double)bf1(a.inj[m * a.ld_inj + s]) / (double)a.HC));
        const float hi = (float)v;
        if (tid == 0) {
          iw_hl[0] = hi;
          iw_hl[1] = (float)(v - (double)hi);
        }
      }
      __syncthreads();
    }
    const float ih = iw_hl[0], il = iw_hl[1];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = c0 + tid + j * kCombineThreads;
      if (c >= nch) break;
      const uint32_t rw[4] = {rv[j].x, rv[j].y, rv[j].z, rv[j].w};
      const uint32_t yw[4] = {yv[j].x, yv[j].y, yv[j].z, yv[j].w};
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float r0 = fmaf(bf_lo(yw[e]), il, fmaf(bf_lo(yw[e]), ih, bf_lo(rw[e])));
        const float r1 = fmaf(bf_hi(yw[e]), il, fmaf(bf_hi(yw[e]), ih, bf_hi(rw[e])));
        o[e] = pack_bf2(r0, r1);
      }
      if (a.nt) bst16_nt(rO, (uint32_t)c * 16u, make_uint4(o[0], o[1], o[2], o[3]));
      else bst16(rO, (uint32_t)c * 16u, make_uint4(o[0], o[1], o[2], o[3]));
    }
  }
}

int launch_combine(const CombineArgs& args, void* stream) {
  CombineArgs a = args;
  // streaming policy once R2 outgrows the L2s (8 x 4 MB): 73% -> 81% of HBM
  // peak at M = 8192 (HC = 4, HS = 2560) on MI355X
  a.nt = (double)a.M * a.HC * a.HS * 2.0 > 32.0 * 1024 * 1024 ? 1 : 0;
  const int64_t groups = cdiv(a.M, 8) * 8 * a.HC;  // token octets x streams x 8
  const int passes = (int)cdiv(a.HS / 8, kCombineThreads);  // chunks per thread in one pass
  const dim3 g((unsigned)groups), blk(kCombineThreads);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (passes <= 1) hipLaunchKernelGGL(hcgr_combine_k<1>, g, blk, 0, st, a);
  else if (passes <= 2) hipLaunchKernelGGL(hcgr_combine_k<2>, g, blk, 0, st, a);
  else if (passes <= 4) hipLaunchKernelGGL(hcgr_combine_k<4>, g, blk, 0, st, a);
  else hipLaunchKernelGGL(hcgr_combine_k<8>, g, blk, 0, st, a);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// Every launch goes through hipExtLaunchKernelGGL: with a pair of timing
// events (start, stop) the runtime stamps them at the kernel's own start and
// end, so per-kernel durations exclude the dispatch gaps between kernels.
template <typename F, typename... Args>
static void klaunch(F k, dim3 grid, dim3 block, size_t lds, hipStream_t st, const hipEvent_t* ev, Args... args) {
  hipExtLaunchKernelGGL(k, grid, block, (uint32_t)lds, st, ev ? ev[0] : nullptr, ev ? ev[1] : nullptr, 0u, args...);
}

template <int TM, int RB, int KW, int KC>
static void launch_kd(const DownArgs& d, dim3 grid, hipStream_t st, const hipEvent_t* ev) {
  if (d.wnt)
    klaunch(hcgr_k1_dec<TM, RB, KW, KC, true>, grid, dim3(RB * KW * 64), 0, st, ev, d);
  else
    klaunch(hcgr_k1_dec<TM, RB, KW, KC, false>, grid, dim3(RB * KW * 64), 0, st, ev, d);
}
static void launch_kd_variant(int v, const DownArgs& d, dim3 grid, hipStream_t st, const hipEvent_t* ev = nullptr) {
  switch (v) {
    case KD_T16_R7_K1_C128: launch_kd<16, 7, 1, 128>(d, grid, st, ev); break;
    case KD_T16_R1_K4_C512: launch_kd<16, 1, 4, 512>(d, grid, st, ev); break;
    case KD_T16_R3_K1_C256: launch_kd<16, 3, 1, 256>(d, grid, st, ev); break;
    case KD_T16_R3_K2_C512: launch_kd<16, 3, 2, 512>(d, grid, st, ev); break;
    case KD_T32_R7_K1_C128: launch_kd<32, 7, 1, 128>(d, grid, st, ev); break;
    case KD_T32_R1_K4_C512: launch_kd<32, 1, 4, 512>(d, grid, st, ev); break;
    case KD_T32_R3_K1_C256: launch_kd<32, 3, 1, 256>(d, grid, st, ev); break;
    case KD_T32_R3_K2_C512: launch_kd<32, 3, 2, 512>(d, grid, st, ev); break;
    case KD_T64_R7_K1_C128: launch_kd<64, 7, 1, 128>(d, grid, st, ev); break;
    case KD_T128_R7_K1_C128: launch_kd<128, 7, 1, 128>(d, grid, st, ev); break;
    case KD_T16_R4_K2_C512: launch_kd<16, 4, 2, 512>(d, grid, st, ev); break;
    case KD_T32_R4_K2_C512: launch_kd<32, 4, 2, 512>(d, grid, st, ev); break;
    default: launch_kd<64, 3, 1, 256>(d, grid, st, ev); break;
  }
}
template <int HC>
static void launch_reduce_hc(int cpl, const ReduceArgs& r, dim3 grid, dim3 block, hipStream_t st, const hipEvent_t* ev) {
  switch (cpl) {
    case 1: klaunch(hcgr_k1_reduce<HC, 1>, grid, block, 0, st, ev, r); break;
    case 2: klaunch(hcgr_k1_reduce<HC, 2>, grid, block, 0, st, ev, r); break;
    case 3: klaunch(hcgr_k1_reduce<HC, 3>, grid, block, 0, st, ev, r); break;
    case 5: klaunch(hcgr_k1_reduce<HC, 5>, grid, block, 0, st, ev, r); break;
    default: klaunch(hcgr_k1_reduce<HC, 8>, grid, block, 0, st, ev, r); break;
  }
}
// waves: one per (row, 16 tokens); blocks of 1, 2 or 4 of them, the fewest
// that keep the grid within 704 workgroups. Measured on MI355X (HS = 2560,
// r = 320, whole calls back to back) against four-wave blocks throughout:
// 0.3-0.45 us less per call at M = 32 for HC = 1, 2, 4 and 8 (about 650
// one-wave blocks; HC = 4: 14.29 -> 13.96 us), 0.07-0.27 at M = 1..16,
// 0.16-0.29 with two-wave blocks at 1000-1300 waves except HC = 4, M = 64
// (0.2 more); the reduction kernel's own event time does not change, the
// gain is in the hand-over to the next kernel. One-wave blocks at 2000
// waves and more were 0.6-1.5 us slower.
static void launch_reduce(int hc, int cpl, const ReduceArgs& r, int64_t waves, hipStream_t st, const hipEvent_t* ev = nullptr) {
  const int wpb = waves <= 704 ? 1 : waves <= 2 * 704 ? 2 : 4;
  const dim3 grid((unsigned)cdiv(waves, (int64_t)wpb)), block((unsigned)(64 * wpb));
  switch (hc) {
    case 1: launch_reduce_hc<1>(cpl, r, grid, block, st, ev); break;
    case 2: launch_reduce_hc<2>(cpl, r, grid, block, st, ev); break;
    case 8: launch_reduce_hc<8>(cpl, r, grid, block, st, ev); break;
    default: launch_reduce_hc<4>(cpl, r, grid, block, st, ev); break;
  }
}
template <int TM, int NW, int BPW, int KS>
static void launch_kf(const FullArgs& f, dim3 grid, hipStream_t st, const hipEvent_t* ev) {
  klaunch(hcgr_k1_full<TM, NW, BPW, KS>, grid, dim3(NW * 64), 0, st, ev, f);
}
int configure_kernels() {
  const int lim = (int)kLdsPerCu;  // make_split keeps k2_dec_lds within it
  hipError_t e;
  for (const void* k : {(const void*)hcgr_k2_dec<16, 16, false>, (const void*)hcgr_k2_dec<32, 16, false>,
                        (const void*)hcgr_k2_dec<64, 16, false>, (const void*)hcgr_k2_dec<16, 10, false>,
                        (const void*)hcgr_k2_dec<32, 10, false>, (const void*)hcgr_k2_dec<64, 10, false>,
                        (const void*)hcgr_k2_dec<16, 16, true>, (const void*)hcgr_k2_dec<32, 16, true>,
                        (const void*)hcgr_k2_dec<64, 16, true>, (const void*)hcgr_k2_dec<16, 10, true>,
                        (const void*)hcgr_k2_dec<32, 10, true>, (const void*)hcgr_k2_dec<64, 10, true>})
    if ((e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, lim)) != hipSuccess) return (int)e;
  if ((e = hipFuncSetAttribute((const void*)hcgr_k2_sweep<2>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sweep_lds_bytes(2))) != hipSuccess) return (int)e;
  if ((e = hipFuncSetAttribute((const void*)hcgr_k2_sweep<3>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sweep_lds_bytes(3))) != hipSuccess) return (int)e;
  if ((e = hipFuncSetAttribute((const void*)hcgr_k2_sweep<4>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sweep_lds_bytes(4))) != hipSuccess) return (int)e;
  if ((e = hipFuncSetAttribute((const void*)hcgr_k2_sweep<5>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sweep_lds_bytes(5))) != hipSuccess) return (int)e;
  if ((e = (hipError_t)configure_sweep2_kernels()) != hipSuccess) return (int)e;
  return configure_decode_kernels();
}

// Per-stage timing: events[2i] and events[2i+1] bracket stage i's kernel (null: untimed).
struct Timing {
  const hipEvent_t* ev;
  const hipEvent_t* stage(int i) const { return ev ? ev + 2 * i : nullptr; }
  // a stage the plan does not have: an empty interval right after the previous stage
  hipError_t skip(int i, hipStream_t st) const {
    hipError_t e = hipSuccess;
    if (ev && (e = hipEventRecord(ev[2 * i], st)) == hipSuccess) e = hipEventRecord(ev[2 * i + 1], st);
    return e;
  }
};

static int launch_split(const Shape& s, const Plan& p, const ForwardArgs& f, hipStream_t st, const Timing& tm) {
  hipError_t e;
  char* ws = static_cast<char*>(f.ws);
  float* P = reinterpret_cast<float*>(ws + p.off_p);
  float* SS = reinterpret_cast<float*>(ws + p.off_ss);
  uint16_t* H = reinterpret_cast<uint16_t*>(ws + p.off_h);
  const int K = (int)s.k();

  DownArgs d;
  d.R = f.R; d.y = f.y; d.inj = f.inj; d.ld_inj = f.ld_inj;
  d.wn = f.wnorm; d.wn_full = s.wn_full ? 1 : 0;
  d.w0 = f.wd; d.w1 = s.merged ? nullptr : f.wi; d.folded = s.merged ? 1 : 0;
  d.M = f.M; d.K = K; d.HS = s.hs; d.HC = s.hc; d.r = s.r; d.n_rows = s.n_rows();
  d.KC = p.kc; d.nkc = p.nkc; d.NP = s.np(); d.Mpad = p.mpad;
  d.inv_hc = 1.0f / (float)s.hc;
  d.R2 = f.R2; d.P = P; d.SS = SS;
  d.wt = p.mpad <= 32 && (s.hc == 2 || s.hc == 4) ? 1 : 0;
  d.wnt = p.mpad == p.tm ? 1 : 0;  // one token tile: each weight line is read once
  dim3 g1((unsigned)(p.ntiles_n * p.nkc), (unsigned)(p.mpad / p.tm));
  launch_kd_variant(p.k1, d, g1, st, tm.stage(0));
  if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  ReduceArgs r;
  r.P = P; r.SS = SS; r.Mpad = p.mpad; r.M = f.M;
  r.NP = s.np(); r.kcps = p.kcps; r.HS = s.hs; r.HC = s.hc; r.r = s.r; r.n_rows = s.n_rows();
  r.eps = s.eps; r.inv_hc = 1.0f / (float)s.hc; r.inv_hs = 1.0f / (float)s.hs;
  r.rrms = f.rrms; r.h = H; r.inj_next = f.inj_next; r.ld_inj_next = f.ld_inj_next;
  const int64_t waves = (int64_t)s.n_rows() * (p.mpad / 16);
  launch_reduce(s.hc, red_cpl(p.kcps), r, waves, st, tm.stage(1));
  if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  if (s.hc != 4)  // the stream-generic decode up kernel
    return launch_decg_up(s, k2_shape(p.k2).tm, H, f, st, reinterpret_cast<void* const*>(tm.stage(2)));

  UpArgs u;
  u.h = H; u.Mpad = p.mpad; u.M = f.M; u.r = s.r; u.HS = s.hs; u.K = K;
  u.wu = f.wu; u.R2 = f.res; u.rrms = f.rrms; u.wn = f.wnorm; u.wn_full = s.wn_full ? 1 : 0;
  u.x = f.x;
  // the up kernel's token tiles: every one starts below M (with a smaller
  // tile than the down kernel's, p.mpad / tm2 tiles would not)
  const int tm2 = k2_shape(p.k2).tm;
  const size_t lds = k2_dec_lds(tm2, s.r, p.cb);
  const dim3 g2((unsigned)(s.hs / p.cb), (unsigned)cdiv(f.M, (int64_t)tm2));
  const dim3 b2((unsigned)((p.cb + 3) / 4 * 64));
  // Wu streamed (the non-temporal policy) while the grid has one or two
  // token tiles (measured per call on MI355X, the two forms interleaved in
  // two sessions: 0.24 us less at M = 32, 0.39-0.42 at 16, 0.11 at 48,
  // 0.17-0.40 at 64, level at 1; always streamed, 0.26 more with four tiles
  // at M = 128, where the tiles read each Wu line again)
  const bool wnt = g2.y <= 2;
  auto up = [&](auto k) { klaunch(k, g2, b2, lds, st, tm.stage(2), u); };
  if (p.cb == 10) {
    switch (p.k2) {
      case K2_T16: wnt ? up(hcgr_k2_dec<16, 10, true>) : up(hcgr_k2_dec<16, 10, false>); break;
      case K2_T32: wnt ? up(hcgr_k2_dec<32, 10, true>) : up(hcgr_k2_dec<32, 10, false>); break;
      default: wnt ? up(hcgr_k2_dec<64, 10, true>) : up(hcgr_k2_dec<64, 10, false>); break;
    }
  } else {
    switch (p.k2) {
      case K2_T16: wnt ? up(hcgr_k2_dec<16, 16, true>) : up(hcgr_k2_dec<16, 16, false>); break;
      case K2_T32: wnt ? up(hcgr_k2_dec<32, 16, true>) : up(hcgr_k2_dec<32, 16, false>); break;
      default: wnt ? up(hcgr_k2_dec<64, 16, true>) : up(hcgr_k2_dec<64, 16, false>); break;
    }
  }
  return (int)hipGetLastError();
}

static int launch_tiled(const Shape& s, const Plan& p, const ForwardArgs& f, hipStream_t st, const Timing& tm) {
  hipError_t e;
  char* ws = static_cast<char*>(f.ws);
  uint16_t* H = reinterpret_cast<uint16_t*>(ws + p.off_h);
  float* Q = reinterpret_cast<float*>(ws + p.off_q);
  const int K = (int)s.k();
  const KFShape fs = kf_shape(p.kf);

  if (p.kind == PLAN_TILE) {
    Tile1Args a;
    a.R = f.R; a.y = f.y; a.inj = f.inj; a.ld_inj = f.ld_inj;
    a.wn = f.wnorm; a.wn_len = s.wn_full ? K : s.hs; a.folded = s.merged ? 1 : 0;
    a.w0 = f.wd; a.w1 = s.merged ? f.wd + (size_t)s.r * (size_t)K : f.wi;
    a.M = f.M; a.K = K; a.HS = s.hs; a.HC = s.hc; a.r = s.r; a.nblk = s.nblk(); a.nsplit = p.nsplit;
    a.eps = s.eps; a.inv_hc = 1.0f / (float)s.hc; a.inv_hs = 1.0f / (float)s.hs;
    a.R2 = f.R2; a.rrms = f.rrms; a.h = H; a.inj_next = f.inj_next; a.ld_inj_next = f.ld_inj_next;
    a.Q = Q; a.Mq = p.mq; a.NP = s.np();
    a.nseg = p.nseg; a.SSp = reinterpret_cast<float*>(ws + p.off_ss);
    a.tiles = (int)cdiv(f.M, (int64_t)p.tm);
    a.xgroup = p.xgroup;
    // streaming policy for R2 (and R) under either sweep up kernel (large M:
    // measured on MI355X with the 256-token sweep at M = 8192, R2 168 MB,
    // 218-223 against 229-232 us per call, the down kernel 108.5 against 122
    // us; no change at 4096) or R2 beyond the Infinity Cache; not for the mix
    // entry point, whose up kernel reads R itself again
    a.nt = f.R2 && (is_sweep(p.kt) || (double)f.M * K * 2.0 > kStreamBytes) ? 1 : 0;
    // R itself is read once and is dead after the op (R2 replaces it): the
    // streaming policy at every M, so it does not displace the weights and y
    // that the workgroups re-read through the caches (measured on MI355X,
    // HC = 4: 51.2 against 54.5 us per call at M = 1024, 74-75 against 77-78
    // at 2048; HC = 2: 82 against 86 at 4096; no change at 256 and 4096);
    // not for the mix entry point either
    a.ntr = f.R2 ? 1 : 0;
    const int64_t tiles_g = p.xgroup ? cdiv((int64_t)a.tiles, 8) * 8 : a.tiles;
    const dim3 g1((unsigned)(tiles_g * p.nsplit * (s.hc / p.spw) * p.nseg));
    if (p.spw == 4) klaunch(hcgr_k1_tile<4, 64, 4>, g1, dim3(512), 0, st, tm.stage(0), a);
    else if (p.tm == 128) klaunch(hcgr_k1_tile<1, 128, 3>, g1, dim3(512), 0, st, tm.stage(0), a);
    else klaunch(hcgr_k1_tile<1, 64, 4>, g1, dim3(512), 0, st, tm.stage(0), a);
  } else {
  FullArgs a;
  a.R = f.R; a.y = f.y; a.inj = f.inj; a.ld_inj = f.ld_inj;
  a.wn = f.wnorm; a.wn_len = s.wn_full ? K : s.hs;
  a.w0 = f.wd; a.w1 = s.merged ? nullptr : f.wi; a.folded = s.merged ? 1 : 0;
  a.M = f.M; a.K = K; a.HS = s.hs; a.HC = s.hc; a.r = s.r; a.n_rows = s.n_rows(); a.nblk = s.nblk();
  a.nsplit = p.nsplit; a.spw = p.spw;
  a.eps = s.eps; a.inv_hc = 1.0f / (float)s.hc; a.inv_hs = 1.0f / (float)s.hs;
  a.R2 = f.R2; a.rrms = f.rrms; a.h = H; a.inj_next = f.inj_next; a.ld_inj_next = f.ld_inj_next;
  a.Q = Q; a.Mq = p.mq; a.NP = s.np();
  dim3 g1((unsigned)cdiv(f.M, fs.tm), (unsigned)(p.nsplit * (4 / p.spw)));
  switch (p.kf) {
    case KF_T32: launch_kf<32, 8, 3, 128>(a, g1, st, tm.stage(0)); break;
    default: launch_kf<64, 8, 3, 64>(a, g1, st, tm.stage(0)); break;
  }
  }
  if ((e = hipGetLastError()) != hipSuccess) return (int)e;

  if (p.kind == PLAN_STREAM || (p.kind == PLAN_TILE && p.spw == 1)) {
    SumArgs sa;
    sa.Q = Q; sa.Mq = p.mq; sa.M = f.M; sa.NP = s.np(); sa.r = s.r; sa.n_rows = s.n_rows();
    sa.inv_hc = 1.0f / (float)s.hc; sa.h = H; sa.inj_next = f.inj_next; sa.ld_inj_next = f.ld_inj_next;
    sa.nseg = p.kind == PLAN_TILE ? p.nseg : 1; sa.SSp = reinterpret_cast<const float*>(ws + p.off_ss);
    sa.rrms = f.rrms; sa.eps = s.eps; sa.inv_hs = 1.0f / (float)s.hs;
    const int64_t threads = f.M * (s.r / 8 + 1) * s.hc;
    // four lanes per (token, chunk, stream) while one lane each would leave
    // CUs without a workgroup and each lane has a segment (measured on MI355X
    // at HS = 2560, r = 320: 7.4 -> 4.9 us at HC = 2, M = 32, 9.0 -> 7.6 at
    // HC = 4, M = 256; 1.6-2.2 us slower at 328 workgroups of one lane each)
    const int sg = sa.nseg >= 4 && threads <= 256 * 256 ? 4 : 1;
    const dim3 gs((unsigned)cdiv(threads * sg, 256)), bs(256);
    switch (s.hc) {
      case 1:
        if (sa.nseg == 1) klaunch(hcgr_k1_sum<1, true, 1>, gs, bs, 0, st, tm.stage(1), sa);
        else if (sg == 4) klaunch(hcgr_k1_sum<1, false, 4>, gs, bs, 0, st, tm.stage(1), sa);
        else klaunch(hcgr_k1_sum<1, false, 1>, gs, bs, 0, st, tm.stage(1), sa);
        break;
      case 2:
        if (sa.nseg == 1) klaunch(hcgr_k1_sum<2, true, 1>, gs, bs, 0, st, tm.stage(1), sa);
        else if (sg == 4) klaunch(hcgr_k1_sum<2, false, 4>, gs, bs, 0, st, tm.stage(1), sa);
        else klaunch(hcgr_k1_sum<2, false, 1>, gs, bs, 0, st, tm.stage(1), sa);
        break;
      case 8:
        if (sa.nseg == 1) klaunch(hcgr_k1_sum<8, true, 1>, gs, bs, 0, st, tm.stage(1), sa);
        else if (sg == 4) klaunch(hcgr_k1_sum<8, false, 4>, gs, bs, 0, st, tm.stage(1), sa);
        else klaunch(hcgr_k1_sum<8, false, 1>, gs, bs, 0, st, tm.stage(1), sa);
        break;
      default:
        if (sa.nseg == 1) klaunch(hcgr_k1_sum<4, true, 1>, gs, bs, 0, st, tm.stage(1), sa);
        else if (sg == 4) klaunch(hcgr_k1_sum<4, false, 4>, gs, bs, 0, st, tm.stage(1), sa);
        else klaunch(hcgr_k1_sum<4, false, 1>, gs, bs, 0, st, tm.stage(1), sa);
        break;
    }
    if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  } else if ((e = tm.skip(1, st)) != hipSuccess) {
    return (int)e;
  }

  const KTShape ts = kt_shape(p.kt);
  if (is_gen(p.kt)) {
    GenUpArgs ga;
    ga.h = H; ga.M = f.M; ga.r = s.r; ga.HS = s.hs; ga.K = K; ga.wu = f.wu; ga.R2 = f.res; ga.rrms = f.rrms;
    ga.wn = f.wnorm; ga.wn_len = s.wn_full ? K : s.hs; ga.x = f.x; ga.ngroups = s.hs / kGenCg;
    const dim3 g2((unsigned)(cdiv(f.M, (int64_t)ts.tm) * ga.ngroups)), b2((unsigned)(ts.tm * 4));
    const bool big = p.kt == KT_GEN128;
    switch (s.hc) {
      case 1: klaunch(hcgr_k2_gen<1, 64>, g2, b2, 0, st, tm.stage(2), ga); break;
      case 2:
        if (big) klaunch(hcgr_k2_gen<2, 128>, g2, b2, 0, st, tm.stage(2), ga);
        else klaunch(hcgr_k2_gen<2, 64>, g2, b2, 0, st, tm.stage(2), ga);
        break;
      case 8:
        if (big) klaunch(hcgr_k2_gen<8, 128>, g2, b2, 0, st, tm.stage(2), ga);
        else klaunch(hcgr_k2_gen<8, 64>, g2, b2, 0, st, tm.stage(2), ga);
        break;
      default: return (int)hipErrorInvalidValue;  // make_plan takes this kernel for HC = 1, 2, 8 only
    }
  } else if (p.kt == KT_SWEEP2) {
    return launch_sweep2(s, p, f, H, st, reinterpret_cast<void* const*>(tm.stage(2)));
  } else if (p.kt == KT_SWEEP) {
    SweepArgs wa;
    wa.h = H; wa.M = f.M; wa.r = s.r; wa.HS = s.hs; wa.K = K; wa.wu = f.wu; wa.R2 = f.res; wa.rrms = f.rrms;
    wa.wn = f.wnorm; wa.wn_len = s.wn_full ? K : s.hs; wa.x = f.x; wa.ngroups = s.hs / kSweepCg; wa.nranges = p.nranges;
    const dim3 g2((unsigned)(cdiv(f.M, (int64_t)kSweepTm) * p.nranges));
    const int nks = sweep_nks(s.r);
    switch (nks) {
      case 2: klaunch(hcgr_k2_sweep<2>, g2, dim3(512), sweep_lds_bytes(2), st, tm.stage(2), wa); break;
      case 3: klaunch(hcgr_k2_sweep<3>, g2, dim3(512), sweep_lds_bytes(3), st, tm.stage(2), wa); break;
      case 4: klaunch(hcgr_k2_sweep<4>, g2, dim3(512), sweep_lds_bytes(4), st, tm.stage(2), wa); break;
      case 5: klaunch(hcgr_k2_sweep<5>, g2, dim3(512), sweep_lds_bytes(5), st, tm.stage(2), wa); break;
      default: return (int)hipErrorInvalidValue;  // make_plan takes this kernel for 2..5 k stages only
    }
  } else {
    StageArgs sa;
    sa.h = H; sa.M = f.M; sa.r = s.r; sa.HS = s.hs; sa.K = K; sa.wu = f.wu; sa.R2 = f.res; sa.rrms = f.rrms;
    sa.wn = f.wnorm; sa.wn_len = s.wn_full ? K : s.hs; sa.x = f.x; sa.npairs = s.hs / 64;
    const int64_t pairs = cdiv(f.M, (int64_t)ts.tm) * sa.npairs;
    const dim3 gs2((unsigned)(cdiv(pairs, 8) * 16));
    if (2 * pairs <= 2 * 256) klaunch(hcgr_k2_stage<true>, gs2, dim3(256), 0, st, tm.stage(2), sa);  // <= 2 per CU
    else klaunch(hcgr_k2_stage<false>, gs2, dim3(256), 0, st, tm.stage(2), sa);
  }
  return (int)hipGetLastError();
}

int launch_forward(const Shape& s, const Plan& p, const ForwardArgs& f, void* stream, void* const* events) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const Timing tm{reinterpret_cast<const hipEvent_t*>(events)};
  if (p.kind == PLAN_FUSED || p.kind == PLAN_PERSIST) return launch_fused(s, p, f, stream, events);
  if (p.kind == PLAN_SPLIT) return launch_split(s, p, f, st, tm);
  return launch_tiled(s, p, f, st, tm);
}

}  // namespace hcgr
