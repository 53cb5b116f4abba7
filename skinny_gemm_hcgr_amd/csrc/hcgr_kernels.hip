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
#include <stdint.h>

#include "hcgr_internal.h"

namespace hcgr {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf1(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
// float -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t to_bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ bf16x8_t as_bf8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(a), as_bf8(b), c, 0, 0, 0);
}
// logistic function through the hardware 2^x: 1/(1 + 2^(-v*log2 e))
__device__ __forceinline__ float sigmoid_f(float v) { return 1.0f / (1.0f + __expf(-v)); }

// ---------------------------------------------------------------------------
// K1: COMBINE + sums of squares + down/inject partial contraction.
// Workgroup = (token tile of TM rows) x (K chunk [kbeg, kbeg+KC) inside one
// stream) x (n tile of NW*NBW 16-row blocks of the down/inject rows). The
// activation tile of each LDS stage (TM x KS) is combined once per workgroup
// and shared by all waves through LDS (MFMA B operand); each wave streams its
// own weight rows straight from global memory into registers (A operand),
// one stage ahead of the MFMAs.
// ---------------------------------------------------------------------------
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
};

template <int TM, int NW, int NBW, int KS>
__global__ __launch_bounds__(NW * 64) void hcgr_k1_down(DownArgs a) {
  constexpr int NT = NW * 64;
  constexpr int CPR = KS / 8;               // 16-byte chunks per tile row
  constexpr int NCH = TM * CPR;             // chunks per stage
  constexpr int CPT = (NCH + NT - 1) / NT;  // chunks per thread
  constexpr int LDA = KS + 8;               // padded LDS row, bf16 elements
  constexpr int NTB = TM / 16;
  constexpr int NKS = KS / 32;

  __shared__ __attribute__((aligned(16))) uint16_t act[2][TM * LDA];
  __shared__ float ssp[NCH];
  __shared__ float iwh[TM], iwl[TM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kc = blockIdx.x % a.nkc;
  const int nt = blockIdx.x / a.nkc;
  const int64_t m0 = (int64_t)blockIdx.y * TM;
  const int kbeg = kc * a.KC;
  const int s = kbeg / a.HS;
  const bool lead = (nt == 0);  // the n-tile-0 workgroups write R2 and the sums of squares
  const int nstage = a.KC / KS;
  const int koff = 8 * (lane >> 4);

  // (COMBINE) iw = 2 * sigmoid(inj[s] / HC) for this stream, per token row.
  // Formed in fp64 and kept as an fp32 pair iw = hi + lo (~48 bits): when R
  // and y*iw nearly cancel, R2 is far smaller than y and a single fp32 iw
  // would put an error of |y| * 2^-24 on it, several bf16 ulps of R2.
  if (tid < TM) {
    const int64_t m = m0 + tid;
    double v = 0.0;
    if (m < a.M) v = 2.0 / (1.0 + exp(-(double)bf1(a.inj[m * a.ld_inj + s]) / (double)a.HC));
    const float hi = (float)v;
    iwh[tid] = hi;
    iwl[tid] = (float)(v - (double)hi);
  }

  // weight rows of this wave (A operand rows = down/inject output rows n)
  const uint16_t* wrow[NBW];
  int nblk[NBW];
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int nb = nt * (NW * NBW) + wave + NW * i;
    const int n = nb * 16 + (lane & 15);
    nblk[i] = nb;
    if (n < a.r) wrow[i] = a.w0 + (int64_t)n * a.K;
    else if (n < a.n_rows) wrow[i] = a.w1 ? a.w1 + (int64_t)(n - a.r) * a.K : a.w0 + (int64_t)n * a.K;
    else wrow[i] = nullptr;
  }

  uint4 wnx[NBW][NKS];
  auto load_w = [&](int kst) {
#pragma unroll
    for (int i = 0; i < NBW; ++i)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        wnx[i][ks] = wrow[i] ? ld16(wrow[i] + kst + ks * 32 + koff) : make_uint4(0, 0, 0, 0);
  };

  uint4 rv[CPT], yv[CPT], wv[CPT];
  auto load_a = [&](int kst) {
    const int cst = kst - s * a.HS;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int q = tid + j * NT;
      rv[j] = yv[j] = wv[j] = make_uint4(0, 0, 0, 0);
      if (q < NCH) {
        const int t = q / CPR;
        const int col = (q % CPR) * 8;
        const int64_t m = m0 + t;
        if (m < a.M) {
          rv[j] = ld16(a.R + m * a.K + kst + col);
          yv[j] = ld16(a.y + m * a.HS + cst + col);
        }
        if (!a.folded) wv[j] = ld16(a.wn + (a.wn_full ? kst + col : cst + col));
      }
    }
  };

  float ss[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) ss[j] = 0.0f;

  // (COMBINE) R2 = R + y*iw in fp32; sum of squares; R2 -> bf16 output;
  // activation R2*(1+Wnorm) (or R2 when the weight is folded) -> LDS.
  auto store_a = [&](int kst, int buf) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int q = tid + j * NT;
      if (q < NCH) {
        const int t = q / CPR;
        const int col = (q % CPR) * 8;
        const float ih = iwh[t];
        const float il = iwl[t];
        const uint32_t rw[4] = {rv[j].x, rv[j].y, rv[j].z, rv[j].w};
        const uint32_t yw[4] = {yv[j].x, yv[j].y, yv[j].z, yv[j].w};
        const uint32_t ww[4] = {wv[j].x, wv[j].y, wv[j].z, wv[j].w};
        uint32_t o2[4], ou[4];
        float acc = ss[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // R2 = (R + y*hi) + y*lo: each fma rounds once, relative to R2 itself
          const float r0 = fmaf(bf_lo(yw[e]), il, fmaf(bf_lo(yw[e]), ih, bf_lo(rw[e])));
          const float r1 = fmaf(bf_hi(yw[e]), il, fmaf(bf_hi(yw[e]), ih, bf_hi(rw[e])));
          acc = fmaf(r0, r0, acc);
          acc = fmaf(r1, r1, acc);
          o2[e] = pack_bf2(r0, r1);
          if (a.folded) ou[e] = o2[e];
          else ou[e] = pack_bf2(r0 * (1.0f + bf_lo(ww[e])), r1 * (1.0f + bf_hi(ww[e])));
        }
        ss[j] = acc;
        const int64_t m = m0 + t;
        if (lead && m < a.M) st16(a.R2 + m * a.K + kst + col, make_uint4(o2[0], o2[1], o2[2], o2[3]));
        st16(&act[buf][t * LDA + col], make_uint4(ou[0], ou[1], ou[2], ou[3]));
      }
    }
  };

  f32x4_t acc[NBW][NTB];
#pragma unroll
  for (int i = 0; i < NBW; ++i)
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) acc[i][tb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  load_w(kbeg);
  load_a(kbeg);
  __syncthreads();  // iwh/iwl visible
  store_a(kbeg, 0);
  __syncthreads();

  uint4 wcur[NBW][NKS];
  for (int st = 0; st < nstage; ++st) {
    const int kst = kbeg + st * KS;
#pragma unroll
    for (int i = 0; i < NBW; ++i)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) wcur[i][ks] = wnx[i][ks];
    const bool more = (st + 1 < nstage);
    if (more) {
      load_w(kst + KS);
      load_a(kst + KS);
    }
    const uint16_t* buf = act[st & 1];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        const uint4 b = *reinterpret_cast<const uint4*>(buf + (tb * 16 + (lane & 15)) * LDA + ks * 32 + koff);
#pragma unroll
        for (int i = 0; i < NBW; ++i) acc[i][tb] = mfma16(wcur[i][ks], b, acc[i][tb]);
      }
    }
    if (more) store_a(kst + KS, (st + 1) & 1);
    __syncthreads();
  }

  // partial sums: D[row n][col token]
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    if (nblk[i] * 16 >= a.NP) continue;
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      const int64_t m = m0 + tb * 16 + (lane & 15);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = nblk[i] * 16 + 4 * (lane >> 4) + q;
        a.P[((int64_t)kc * a.NP + n) * a.Mpad + m] = acc[i][tb][q];
      }
    }
  }
  // per-row sum of squares of this chunk, in a fixed order (deterministic)
  if (lead) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int q = tid + j * NT;
      if (q < NCH) ssp[q] = ss[j];
    }
    __syncthreads();
    if (tid < TM) {
      float t = 0.0f;
      for (int c = 0; c < CPR; ++c) t += ssp[tid * CPR + c];
      a.SS[(int64_t)kc * a.Mpad + m0 + tid] = t;
    }
  }
}

// ---------------------------------------------------------------------------
// K1r: per token, rrms[s] = 1/sqrt(sum of the stream's chunk sums of squares
// / HS + eps); row n of the contraction = sum_s rrms[s] * (sum of the
// stream's chunk partials); down rows -> h = SiLU(v/HC) (bf16, workspace),
// inject rows -> inj_next (bf16). One wave per (row n, 16 tokens): lane
// l handles token l % 16 and every 4th chunk starting at l / 16; all of a
// lane's loads are issued before the first add (one memory round trip), and
// the four lane groups are then summed with cross-lane adds. HC = 4.
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

__global__ __launch_bounds__(256) void hcgr_k1_reduce(ReduceArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t mblocks = a.Mpad / 16;
  const int n = (int)(wid / mblocks);
  if (n >= a.n_rows) return;  // whole wave leaves together
  const int64_t m = (wid % mblocks) * 16 + (lane & 15);
  const int g = lane >> 4;
  const int kcps = a.kcps;  // <= 4 * kRedPerLane
  float sv[4][kRedPerLane], pv[4][kRedPerLane];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < kRedPerLane; ++i) {
      const int c = g + 4 * i;
      const int64_t kc = (int64_t)s * kcps + c;
      sv[s][i] = c < kcps ? a.SS[kc * a.Mpad + m] : 0.0f;
      pv[s][i] = c < kcps ? a.P[(kc * a.NP + n) * a.Mpad + m] : 0.0f;
    }
  float ss[4], ps[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    float t = 0.0f, u = 0.0f;
#pragma unroll
    for (int i = 0; i < kRedPerLane; ++i) {
      t += sv[s][i];
      u += pv[s][i];
    }
    ss[s] = t;
    ps[s] = u;
  }
  float v = 0.0f;
  float rr[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    rr[s] = 1.0f / sqrtf(sum_lane_groups(ss[s]) * a.inv_hs + a.eps);
    v = fmaf(rr[s], sum_lane_groups(ps[s]), v);
  }
  if (g != 0) return;
  if (n == 0 && m < a.M) {
#pragma unroll
    for (int s = 0; s < 4; ++s) a.rrms[m * 4 + s] = rr[s];
  }
  if (n < a.r) {
    const float z = v * a.inv_hc;
    a.h[m * a.r + n] = (m < a.M) ? to_bf(z * sigmoid_f(z)) : (uint16_t)0;  // (G1) SiLU(lora / HC)
  } else if (m < a.M) {
    a.inj_next[m * a.ld_inj_next + (n - a.r)] = to_bf(v);  // (INJ), not scaled
  }
}

// ---------------------------------------------------------------------------
// K2: (G2) gate = h . Wu^T, G = sigmoid(gate), (MIX) x[c] = 1/4 sum_s G xn.
// Workgroup = TM tokens x CB = NW*RBW*4 channels. A operand rows: 16 rows =
// 4 channels x 4 streams (row i -> channel i/4, stream i%4, i.e. Wu row
// (i%4)*HS + c), so accumulator q of a lane is stream q of one channel and
// the sum over streams stays in registers. B operand = h tile staged in LDS.
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

template <int TM, int NW, int RBW>
__global__ __launch_bounds__(NW * 64) void hcgr_k2_up_mix(UpArgs a) {
  constexpr int NT = NW * 64;
  constexpr int NTB = TM / 16;
  constexpr int JMAX = 16;  // r <= 512
  extern __shared__ __attribute__((aligned(16))) uint16_t hl[];
  const int ldh = a.r + 8;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t m0 = (int64_t)blockIdx.y * TM;
  const int cbase = blockIdx.x * (NW * RBW * 4);
  const int koff = 8 * (lane >> 4);
  const int nj = a.r / 32;

  const uint16_t* wrow[RBW];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const int c = cbase + (wave * RBW + rb) * 4 + ((lane & 15) >> 2);
    const int s = lane & 3;
    wrow[rb] = a.wu + ((int64_t)s * a.HS + c) * a.r;
  }

  // decode-sized tiles: issue every global load of the wave (weights and the
  // epilogue's R2, rrms and Wnorm) before the first wait
  uint4 wall[RBW == 1 ? JMAX : 1];
  float pr2[RBW == 1 ? NTB : 1][4], prr[RBW == 1 ? NTB : 1][4], pone[4];
  if constexpr (RBW == 1) {
#pragma unroll
    for (int j = 0; j < JMAX; ++j)
      if (j < nj) wall[j] = ld16(wrow[0] + j * 32 + koff);
    const int c = cbase + wave * 4 + (lane >> 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) pone[q] = 1.0f + bf1(a.wn[a.wn_full ? q * a.HS + c : c]);
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      const int64_t m = m0 + tb * 16 + (lane & 15);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        pr2[tb][q] = m < a.M ? bf1(a.R2[m * a.K + q * a.HS + c]) : 0.0f;
        prr[tb][q] = m < a.M ? a.rrms[m * 4 + q] : 0.0f;
      }
    }
  }

  const int cpr = a.r / 8;
  for (int q = tid; q < TM * cpr; q += NT) {
    const int t = q / cpr;
    const int col = (q % cpr) * 8;
    st16(&hl[t * ldh + col], ld16(a.h + (m0 + t) * a.r + col));
  }
  __syncthreads();

  f32x4_t acc[RBW][NTB];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) acc[rb][tb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  if constexpr (RBW == 1) {
#pragma unroll
    for (int j = 0; j < JMAX; ++j) {
      if (j < nj) {
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
          const uint4 b = *reinterpret_cast<const uint4*>(&hl[(tb * 16 + (lane & 15)) * ldh + j * 32 + koff]);
          acc[0][tb] = mfma16(wall[j], b, acc[0][tb]);
        }
      }
    }
  } else {
    uint4 wn_[RBW];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) wn_[rb] = ld16(wrow[rb] + koff);
    for (int j = 0; j < nj; ++j) {
      uint4 wc[RBW];
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) wc[rb] = wn_[rb];
      if (j + 1 < nj) {
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) wn_[rb] = ld16(wrow[rb] + (j + 1) * 32 + koff);
      }
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        const uint4 b = *reinterpret_cast<const uint4*>(&hl[(tb * 16 + (lane & 15)) * ldh + j * 32 + koff]);
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) acc[rb][tb] = mfma16(wc[rb], b, acc[rb][tb]);
      }
    }
  }

  // epilogue: lane holds streams q = 0..3 of channel c for token m
  if constexpr (RBW == 1) {
    const int c = cbase + wave * 4 + (lane >> 4);
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      const int64_t m = m0 + tb * 16 + (lane & 15);
      if (m < a.M) {
        float sum = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) sum = fmaf(sigmoid_f(acc[0][tb][q]), pr2[tb][q] * prr[tb][q] * pone[q], sum);
        a.x[m * a.HS + c] = to_bf(sum * 0.25f);
      }
    }
    return;
  }
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const int c = cbase + (wave * RBW + rb) * 4 + (lane >> 4);
    float onep[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) onep[q] = 1.0f + bf1(a.wn[a.wn_full ? q * a.HS + c : c]);
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      const int64_t m = m0 + tb * 16 + (lane & 15);
      if (m < a.M) {
        float sum = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float g = sigmoid_f(acc[rb][tb][q]);
          const float xn = bf1(a.R2[m * a.K + q * a.HS + c]) * a.rrms[m * 4 + q] * onep[q];
          sum = fmaf(g, xn, sum);
        }
        a.x[m * a.HS + c] = to_bf(sum * 0.25f);
      }
    }
  }
}

// ---------------------------------------------------------------------------
template <int TM, int NW, int NBW, int KS>
static void launch_k1(const DownArgs& d, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((hcgr_k1_down<TM, NW, NBW, KS>), grid, dim3(NW * 64), 0, st, d);
}
template <int TM, int NW, int RBW>
static void launch_k2(const UpArgs& u, dim3 grid, size_t lds, hipStream_t st) {
  hipLaunchKernelGGL((hcgr_k2_up_mix<TM, NW, RBW>), grid, dim3(NW * 64), lds, st, u);
}

int configure_kernels() {
  const int lim = 96 * 1024;
  hipError_t e;
  if ((e = hipFuncSetAttribute((const void*)hcgr_k2_up_mix<16, 4, 1>, hipFuncAttributeMaxDynamicSharedMemorySize, lim)) != hipSuccess) return (int)e;
  if ((e = hipFuncSetAttribute((const void*)hcgr_k2_up_mix<32, 4, 1>, hipFuncAttributeMaxDynamicSharedMemorySize, lim)) != hipSuccess) return (int)e;
  if ((e = hipFuncSetAttribute((const void*)hcgr_k2_up_mix<64, 4, 1>, hipFuncAttributeMaxDynamicSharedMemorySize, lim)) != hipSuccess) return (int)e;
  if ((e = hipFuncSetAttribute((const void*)hcgr_k2_up_mix<64, 4, 4>, hipFuncAttributeMaxDynamicSharedMemorySize, lim)) != hipSuccess) return (int)e;
  return (int)hipSuccess;
}

int launch_forward(const Shape& s, const Plan& p, const ForwardArgs& f, void* stream, void* const* events) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  auto mark = [&](int i) -> hipError_t {
    return events ? hipEventRecord(reinterpret_cast<hipEvent_t>(events[i]), st) : hipSuccess;
  };
  hipError_t e;
  if ((e = mark(0)) != hipSuccess) return (int)e;
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
  dim3 g1((unsigned)(p.ntiles_n * p.nkc), (unsigned)(p.mpad / p.tm));
  switch (p.k1) {
    case K1_T16: launch_k1<16, 7, 1, 128>(d, g1, st); break;
    case K1_T32: launch_k1<32, 7, 1, 128>(d, g1, st); break;
    case K1_T64S: launch_k1<64, 7, 1, 128>(d, g1, st); break;
    default: launch_k1<64, 4, 6, 32>(d, g1, st); break;
  }
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(1)) != hipSuccess) return (int)e;

  ReduceArgs r;
  r.P = P; r.SS = SS; r.Mpad = p.mpad; r.M = f.M;
  r.NP = s.np(); r.kcps = p.kcps; r.HS = s.hs; r.HC = s.hc; r.r = s.r; r.n_rows = s.n_rows();
  r.eps = s.eps; r.inv_hc = 1.0f / (float)s.hc; r.inv_hs = 1.0f / (float)s.hs;
  r.rrms = f.rrms; r.h = H; r.inj_next = f.inj_next; r.ld_inj_next = f.ld_inj_next;
  const int64_t waves = (int64_t)s.n_rows() * (p.mpad / 16);
  hipLaunchKernelGGL(hcgr_k1_reduce, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, r);
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(2)) != hipSuccess) return (int)e;

  UpArgs u;
  u.h = H; u.Mpad = p.mpad; u.M = f.M; u.r = s.r; u.HS = s.hs; u.K = K;
  u.wu = f.wu; u.R2 = f.R2; u.rrms = f.rrms; u.wn = f.wnorm; u.wn_full = s.wn_full ? 1 : 0;
  u.x = f.x;
  const size_t lds = (size_t)p.tm * (s.r + 8) * sizeof(uint16_t);
  dim3 g2((unsigned)(s.hs / p.cb), (unsigned)(p.mpad / p.tm));
  switch (p.k2) {
    case K2_T16: launch_k2<16, 4, 1>(u, g2, lds, st); break;
    case K2_T32: launch_k2<32, 4, 1>(u, g2, lds, st); break;
    case K2_T64S: launch_k2<64, 4, 1>(u, g2, lds, st); break;
    default: launch_k2<64, 4, 4>(u, g2, lds, st); break;
  }
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(3)) != hipSuccess) return (int)e;
  return (int)hipSuccess;
}

}  // namespace hcgr
