// vda_backward: the first stage of the VDA backward pass -- back through the
// epilogue and the readout.
//
// The forward pass ends with o_t = S_q(t) q_t per token ("Video DeltaNet"
// summary, onedev.kr/papers/80, section "어떻게 동작하나": the readout sums
// the forward and reverse states' readouts) and
// y = gamma * o / sqrt(mean o^2 + eps) * sigmoid(g) (section "무엇과 다른가").
// Its derivative with respect to the output adjoint dy is, per token,
//     r = 1 / sqrt(mean o^2 + eps),  n = o r,  s = sigmoid(g),  dn = dy gamma s
//     dg = dn n (1 - s),             do = r (dn - n mean(dn n)),
// and, summed over every token of every frame, head and batch, the gain's
// gradient dgamma = sum dy s n;
// then dq_t = S_q(t)^T do_t per token and dS_q(t) = sum_u do_{t,u} q_{t,u}^T per
// frame (the adjoint of the state the frame's queries read).  The adjoints of
// the records F_j, R_j and of S_T follow from dS_q by the coverage rules and
// are the next stage's input.
//
// Kernels:
//  * pack_states_t: S_q(t)^T of every chunk slot, in the readout kernel's
//    bfloat16 hi + lo operand order (the forward's gather, transposed), so the
//    forward readout kernel run on do computes dq;
//  * readout_bwd_bf16: one (frame, head) per workgroup, the forward readout's
//    recomputation of o (same matrix-core product, same operand) followed by
//    the epilogue's derivative in registers; do (bfloat16) and dgate stream
//    out through the same per-wave LDS tiles that bring q, gate and dy in;
//  * gain_grad_sum: dgamma from the per-workgroup sums readout_bwd_bf16 leaves
//    in the workspace when asked for it;
//  * dS_q: the frame-statistics kernel in its PLAIN mode on (q, do).
#include <algorithm>
#include <type_traits>

#include "vda_internal.h"

namespace vda {
namespace {

__device__ __forceinline__ float sigmoid(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

// Slot c < nc: S_q = wf F_{c-2} Diag(df) + wr R_{c+2} Diag(dr) (S_T/2 for a
// missing side, the bridge products df, dr or ones); slot nc: S_T.  Written
// transposed in the readout's operand order: fragment (mt, ks, lane) holds
// S_q^T[dv_of(mt, lane % 32)][(d/2)(lane / 32) + 8 ks + j] = S_q[...][dv_of(..)]
// for j = 0..7, hi plane then lo plane.
template <int D>
__global__ __launch_bounds__(256) void pack_states_t(const float* __restrict__ s_text,
                                                     const float* __restrict__ fwd,
                                                     const float* __restrict__ rev,
                                                     const float* __restrict__ alpha, uint4* __restrict__ out,
                                                     int nc, int T, int H, int C, int bridge) {
  constexpr int DP = D < 32 ? 32 : D;
  constexpr int HALF = DP / 2;
  constexpr int MT = DP / 32;
  constexpr int KS = D / 16;
  constexpr int NF = MT * KS * 64;
  __shared__ float dfw[D], drv[D];
  const int slot = blockIdx.x % (nc + 1);
  const int bh = blockIdx.x / (nc + 1);
  const int h = bh % H, b = bh / H;
  const size_t head = (size_t)bh;
  for (int k = threadIdx.x; k < D; k += blockDim.x) {
    float df = 1.f, dr = 1.f;
    if (bridge && slot < nc) {
      if (slot >= 1)
        for (int s = C * (slot - 1); s < C * slot; ++s) df *= alpha[(((size_t)b * T + s) * H + h) * D + k];
      if (slot + 1 <= nc - 1)
        for (int s = C * (slot + 1); s < min(C * (slot + 2), T); ++s)
          dr *= alpha[(((size_t)b * T + s) * H + h) * D + k];
    }
    dfw[k] = df;
    drv[k] = dr;
  }
  __syncthreads();
  const float* ST = s_text + head * D * D;
  const float* Fp = nullptr;
  const float* Rp = nullptr;
  if (slot < nc) {
    if (slot >= 2) Fp = fwd + (head * nc + (slot - 2)) * D * D;
    if (slot + 2 <= nc - 1) Rp = rev + (head * nc + (slot + 2)) * D * D;
  }
  const float* Fs = Fp ? Fp : ST;
  const float* Rs = Rp ? Rp : ST;
  const float wf = Fp ? 1.f : 0.5f, wr = Rp ? 1.f : 0.5f;
  auto dv_of = [&](int mt, int m) { return HALF * ((m >> 2) & 1) + 16 * mt + 4 * (m >> 3) + (m & 3); };
  uint4* o = out + (size_t)blockIdx.x * 2 * NF;
  for (int f = threadIdx.x; f < NF; f += blockDim.x) {
    const int lane = f % 64, ks = (f / 64) % KS, mt = f / (64 * KS);
    const int row = dv_of(mt, lane & 31);          // a key channel: an output of dq
    const int v0 = (D / 2) * (lane >> 5) + 8 * ks;  // value channels: the contraction
    const bool live = row < D;
    const int rr = live ? row : 0;
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const size_t i = (size_t)(v0 + j) * D + rr;
      x[j] = live ? wf * Fs[i] * dfw[rr] + wr * Rs[i] * drv[rr] : 0.f;
    }
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      __bf16 h0, l0, h1, l1;
      split_bf16(x[2 * e], h0, l0);
      split_bf16(x[2 * e + 1], h1, l1);
      hi[e] = __builtin_bit_cast(uint32_t, bf16x2{h0, h1});
      lo[e] = __builtin_bit_cast(uint32_t, bf16x2{l0, l1});
    }
    o[f] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    o[NF + f] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  }
}

// Sums over the 32 lanes of one half of the wave (lanes l and l ^ M for M < 32),
// scattered over those lanes: x holds K live values per lane; at the step with
// mask M a lane with bit M set keeps the upper half of them (adding its
// partner's), the other lane the lower half.  Once one value is left the
// remaining steps add it whole.  With K = 2^k values to begin with, lane n
// ends holding in x[0 .. max(K/32, 1) - 1] the sums of values
// (n / max(32/K, 1)) * max(K/32, 1) + 0, 1, ...
template <int N, int K, int M>
__device__ __forceinline__ void fold_lanes(float (&x)[N], int lane) {
  if constexpr (M >= 1) {
    if constexpr (K > 1) {
      const bool up = (lane & M) != 0;
#pragma unroll
      for (int i = 0; i < K / 2; ++i) {
        const float send = up ? x[i] : x[i + K / 2];
        const float keep = up ? x[i + K / 2] : x[i];
        x[i] = keep + __shfl_xor(send, M);
      }
      fold_lanes<N, K / 2, M / 2>(x, lane);
    } else {
      x[0] += __shfl_xor(x[0], M);
      fold_lanes<N, 1, M / 2>(x, lane);
    }
  }
}

// Back through the epilogue: o recomputed as the forward readout computes it,
// then dgate and do per token (see the file comment).  4 waves, each streaming
// 32-token tiles; per wave two LDS tiles (q then dy then do; gate then dgate).
// With DGAIN each lane also sums dy s n over its tiles' tokens (folded over the
// wave's tokens after every tile, two channels kept per lane at d = 128), and
// the workgroup writes its (frame, head)'s sums, channel by channel, to
// GP[blockIdx.x * d ..]; without it GP is not touched.
template <int D, bool GAMMA, bool QN, bool DGAIN>
__global__ __launch_bounds__(256, 1) void readout_bwd_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ G, const uint16_t* __restrict__ DY,
    const float* __restrict__ w, const uint4* __restrict__ rstates, const uint4* __restrict__ rstates_t,
    uint16_t* __restrict__ DO, uint16_t* __restrict__ DG, uint16_t* __restrict__ DQ, int T, int U, int H, int C,
    int nc, float eps, float l2eps, float* __restrict__ GP) {
  constexpr int NW = 4;              // waves per workgroup
  constexpr int DP = D < 32 ? 32 : D;
  constexpr int HALF = DP / 2;       // outputs per lane
  constexpr int MT = DP / 32;
  constexpr int KS = D / 16;
  constexpr int NF = MT * KS * 64;   // 16-byte fragments per part (hi or lo)
  constexpr int NG = HALF / 8;       // 16-byte vectors per lane and token
  constexpr int CH = D / 8;          // 16-byte chunks per token row
  constexpr int RPI = 64 / CH;       // token rows covered by one coalesced wave access
  constexpr int NL = 32 / RPI;       // coalesced accesses per 32-token tile
  constexpr int SWM = (CH < 8 ? CH : 8) - 1;
  constexpr int SWS = CH >= 8 ? 0 : (CH == 4 ? 1 : 2);
  constexpr int STAGE = (3 * NF + 64 * NW - 1) / (64 * NW);
  __shared__ uint4 sfrag[3 * NF];    // S_q hi, S_q lo, S_q^T hi
  __shared__ uint4 xq[NW][32 * CH];  // q rows, then dy rows, then do rows
  __shared__ uint4 xg[NW][32 * CH];  // gate rows, then dgate rows, then dq rows

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int blk = blockIdx.x;
  const int h = blk % H;
  blk /= H;
  const int t = blk % T;
  const int b = blk / T;
  const int slot = (t == 0 || t == T - 1) ? nc : t / C;
  {
    const size_t sl = (size_t)(b * H + h) * (nc + 1) + slot;
    const uint4* src = rstates + sl * 2 * NF;
    const uint4* srt = rstates_t + sl * 2 * NF;  // its hi plane only
    uint4 tmp[STAGE];
#pragma unroll
    for (int i = 0; i < STAGE; ++i) {
      const int f = min(tid + 64 * NW * i, 3 * NF - 1);
      tmp[i] = f < 2 * NF ? src[f] : srt[f - 2 * NF];
    }
#pragma unroll
    for (int i = 0; i < STAGE; ++i)
      if (tid + 64 * NW * i < 3 * NF) sfrag[tid + 64 * NW * i] = tmp[i];
  }
  __syncthreads();

  // buffer descriptors over this frame and head: rows past U read zero and
  // their stores are dropped
  const size_t fbase = (((size_t)b * T + t) * U * H + h) * (size_t)D;
  const uint32_t rowbytes = (uint32_t)H * D * 2;
  const uint32_t nbytes = U > 0 ? (uint32_t)(U - 1) * rowbytes + D * 2 : 0;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(Q + fbase, nbytes);
  const __amdgpu_buffer_rsrc_t gr = make_rsrc(G + fbase, nbytes);
  const __amdgpu_buffer_rsrc_t yr = make_rsrc(DY + fbase, nbytes);
  const __amdgpu_buffer_rsrc_t dor = make_rsrc(DO + fbase, nbytes);
  const __amdgpu_buffer_rsrc_t dgr = make_rsrc(DG + fbase, nbytes);
  const __amdgpu_buffer_rsrc_t dqr = make_rsrc(DQ + fbase, nbytes);

  const int lrow = lane / CH, lch = lane % CH;
  const uint32_t loff = (uint32_t)lrow * rowbytes + 16 * lch;
  auto pos = [](int r, int c) { return r * CH + (c ^ ((r >> SWS) & SWM)); };

  const int n = lane & 31, half = lane >> 5;
  const int dv0 = HALF * half;
  const bool owns = dv0 < D;
  const int ntiles = (U + 31) / 32;
  const int per_wave = (ntiles + NW - 1) / NW;
  uint4* XQ = xq[wave];
  uint4* XG = xg[wave];
  // DGAIN: this lane's share of the gain's gradient, channels
  // dv0 + (n / GR) * GK + k, k < GK (lanes n and n + 1 share them at d <= 32)
  constexpr int GK = HALF >= 32 ? HALF / 32 : 1;
  constexpr int GR = HALF >= 32 ? 1 : 32 / HALF;
  float gsum[GK];
#pragma unroll
  for (int k = 0; k < GK; ++k) gsum[k] = 0.f;

  auto fetch_q = [&](int tile, uint4 (&qv)[NL]) {
    const uint32_t tb = (uint32_t)tile * 32 * rowbytes + loff;
#pragma unroll
    for (int i = 0; i < NL; ++i) qv[i] = buf_load16(qr, tb + (uint32_t)(RPI * i) * rowbytes);
  };
  auto fence = [] {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_wave_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };

  // qv holds this tile's q rows on entry and the next tile's (in flight) on exit
  auto process = [&](int tile, uint4 (&qv)[NL]) {
    const uint32_t tb = (uint32_t)tile * 32 * rowbytes + loff;
#pragma unroll
    for (int i = 0; i < NL; ++i) XQ[pos(RPI * i + lrow, lch)] = qv[i];
    // this tile's gate and dy rows, in flight during the product
    uint4 gv[NL], yv[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) gv[i] = buf_load16(gr, tb + (uint32_t)(RPI * i) * rowbytes);
#pragma unroll
    for (int i = 0; i < NL; ++i) yv[i] = buf_load16(yr, tb + (uint32_t)(RPI * i) * rowbytes);
    fence();
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, XQ[pos(n, (CH / 2) * half + ks)]);
    fence();
    fetch_q(tile + NW, qv);
    // raw query (fused L2 normalisation): 1 / |q| of token n; 1 otherwise
    float qscale = 1.f;
    if constexpr (QN) {
      float qs = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 u = __builtin_bit_cast(uint4, qf[ks]);
        const uint32_t q4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = bf16_lo(q4[e]), c = bf16_hi(q4[e]);
          qs += a * a;
          qs += c * c;
        }
      }
      qs += __shfl_xor(qs, 32);
      qscale = __builtin_amdgcn_rsqf(qs + l2eps);
    }
    f32x16 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 ahi = __builtin_bit_cast(bf16x8, sfrag[(mt * KS + ks) * 64 + lane]);
        const bf16x8 alo = __builtin_bit_cast(bf16x8, sfrag[NF + (mt * KS + ks) * 64 + lane]);
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, qf[ks], acc[mt], 0, 0, 0);
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, qf[ks], acc[mt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // gate rows and dy rows into the tiles (q has been read)
#pragma unroll
    for (int i = 0; i < NL; ++i) XG[pos(RPI * i + lrow, lch)] = gv[i];
#pragma unroll
    for (int i = 0; i < NL; ++i) XQ[pos(RPI * i + lrow, lch)] = yv[i];
    fence();
    // lane holds o[dv0 + 16 mt + r] of token n in acc[mt][r] (o = S_q q / |q| for a raw query)
    if constexpr (QN) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mt][r] *= qscale;
    }
    float ss = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) ss += acc[mt][r] * acc[mt][r];
    ss += __shfl_xor(ss, 32);
    const float rinv = __builtin_amdgcn_rsqf(ss / (float)D + eps);
    auto gains = [&](int i, float (&gm)[8]) {
#pragma unroll
      for (int e = 0; e < 8; ++e) gm[e] = 1.f;
      if constexpr (GAMMA) {  // gains of channels dv0 + 8i .. + 7 (cached reads; LDS is full)
#pragma unroll
        for (int e = 0; e < 8; ++e) gm[e] = dv0 + 8 * i + e < D ? w[dv0 + 8 * i + e] : 1.f;
      }
    };
    // pass 1: mean over the token's channels of dn * n
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const uint4 gq = owns ? XG[pos(n, dv0 / 8 + i)] : make_uint4(0, 0, 0, 0);
      const uint4 yq = owns ? XQ[pos(n, dv0 / 8 + i)] : make_uint4(0, 0, 0, 0);
      const uint32_t g4[4] = {gq.x, gq.y, gq.z, gq.w}, y4[4] = {yq.x, yq.y, yq.z, yq.w};
      float gm[8];
      gains(i, gm);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j0 = 8 * i + 2 * e, j1 = j0 + 1;
        const float n0 = acc[j0 / 16][j0 % 16] * rinv, n1 = acc[j1 / 16][j1 % 16] * rinv;
        dot += bf16_lo(y4[e]) * gm[2 * e] * sigmoid(bf16_lo(g4[e])) * n0;
        dot += bf16_hi(y4[e]) * gm[2 * e + 1] * sigmoid(bf16_hi(g4[e])) * n1;
      }
    }
    dot += __shfl_xor(dot, 32);
    const float m = dot / (float)D;
    // pass 2: do and dgate, written over the chunks just read; do's chunk i is
    // also this lane's operand for k-step i of dq = S_q^T do
    bf16x8 dof[NG];
#pragma unroll
    for (int i = 0; i < NG; ++i) dof[i] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    float gx[DGAIN ? HALF : 1];  // dy s n of this lane's channels dv0 .. dv0 + HALF - 1
#pragma unroll
    for (int j = 0; j < (DGAIN ? HALF : 1); ++j) gx[j] = 0.f;
    if (owns) {
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        const uint4 gq = XG[pos(n, dv0 / 8 + i)];
        const uint4 yq = XQ[pos(n, dv0 / 8 + i)];
        const uint32_t g4[4] = {gq.x, gq.y, gq.z, gq.w}, y4[4] = {yq.x, yq.y, yq.z, yq.w};
        float gm[8];
        gains(i, gm);
        uint32_t dow[4], dgw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j0 = 8 * i + 2 * e, j1 = j0 + 1;
          const float n0 = acc[j0 / 16][j0 % 16] * rinv, n1 = acc[j1 / 16][j1 % 16] * rinv;
          const float s0 = sigmoid(bf16_lo(g4[e])), s1 = sigmoid(bf16_hi(g4[e]));
          const float dn0 = bf16_lo(y4[e]) * gm[2 * e] * s0, dn1 = bf16_hi(y4[e]) * gm[2 * e + 1] * s1;
          dow[e] = pack_bf16x2(rinv * (dn0 - n0 * m), rinv * (dn1 - n1 * m));
          dgw[e] = pack_bf16x2(dn0 * n0 * (1.f - s0), dn1 * n1 * (1.f - s1));
          if constexpr (DGAIN) {
            gx[j0] = bf16_lo(y4[e]) * s0 * n0;
            gx[j1] = bf16_hi(y4[e]) * s1 * n1;
          }
        }
        dof[i] = __builtin_bit_cast(bf16x8, make_uint4(dow[0], dow[1], dow[2], dow[3]));
        if constexpr (QN) {
          // the state's adjoint pass reads do / |q| against the raw query
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j0 = 8 * i + 2 * e, j1 = j0 + 1;
            const float n0 = acc[j0 / 16][j0 % 16] * rinv, n1 = acc[j1 / 16][j1 % 16] * rinv;
            const float s0 = sigmoid(bf16_lo(g4[e])), s1 = sigmoid(bf16_hi(g4[e]));
            const float dn0 = bf16_lo(y4[e]) * gm[2 * e] * s0, dn1 = bf16_hi(y4[e]) * gm[2 * e + 1] * s1;
            dow[e] = pack_bf16x2(qscale * rinv * (dn0 - n0 * m), qscale * rinv * (dn1 - n1 * m));
          }
        }
        XQ[pos(n, dv0 / 8 + i)] = make_uint4(dow[0], dow[1], dow[2], dow[3]);
        XG[pos(n, dv0 / 8 + i)] = make_uint4(dgw[0], dgw[1], dgw[2], dgw[3]);
      }
    }
    if constexpr (DGAIN) {
      // over this tile's 32 tokens (rows past U are zero and add nothing)
      fold_lanes<HALF, HALF, 16>(gx, lane);
#pragma unroll
      for (int k = 0; k < GK; ++k) gsum[k] += gx[k];
    }
    fence();
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      buf_store16(XQ[pos(RPI * i + lrow, lch)], dor, tb + (uint32_t)(RPI * i) * rowbytes);
      buf_store16(XG[pos(RPI * i + lrow, lch)], dgr, tb + (uint32_t)(RPI * i) * rowbytes);
    }
    fence();
    // dq = S_q^T do: the B operand of k-step ks is do's channels
    // (d/2) half + 8 ks .. + 7 of token n, this lane's dof[ks] for d >= 32; at
    // d = 16 half 0 holds all 16 channels and half 1 takes the upper 8 from it
    bf16x8 opf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) opf[ks] = dof[ks];
    if constexpr (D == 16) {
      const uint4 up = __builtin_bit_cast(uint4, dof[1]);
      const uint4 got = make_uint4((uint32_t)__shfl_xor((int)up.x, 32), (uint32_t)__shfl_xor((int)up.y, 32),
                                   (uint32_t)__shfl_xor((int)up.z, 32), (uint32_t)__shfl_xor((int)up.w, 32));
      if (half == 1) opf[0] = __builtin_bit_cast(bf16x8, got);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 at = __builtin_bit_cast(bf16x8, sfrag[2 * NF + (mt * KS + ks) * 64 + lane]);
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(at, opf[ks], acc[mt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (QN) {
      // back through q / |q|: dq = (dq_n - q_n (q_n . dq_n)) / |q| with q_n = q / |q|;
      // the raw query's chunks of this lane's channels come again from L2
      uint4 qc[NG];
      const uint32_t ro = (uint32_t)(tile * 32 + n) * rowbytes + (uint32_t)dv0 * 2;
#pragma unroll
      for (int i = 0; i < NG; ++i) qc[i] = owns ? buf_load16(qr, ro + 16 * i) : make_uint4(0, 0, 0, 0);
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        const uint32_t q4[4] = {qc[i].x, qc[i].y, qc[i].z, qc[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j0 = 8 * i + 2 * e, j1 = j0 + 1;
          dot += bf16_lo(q4[e]) * acc[j0 / 16][j0 % 16] + bf16_hi(q4[e]) * acc[j1 / 16][j1 % 16];
        }
      }
      dot += __shfl_xor(dot, 32);
      const float c3 = qscale * qscale * qscale * dot;
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        const uint32_t q4[4] = {qc[i].x, qc[i].y, qc[i].z, qc[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j0 = 8 * i + 2 * e, j1 = j0 + 1;
          acc[j0 / 16][j0 % 16] = qscale * acc[j0 / 16][j0 % 16] - c3 * bf16_lo(q4[e]);
          acc[j1 / 16][j1 % 16] = qscale * acc[j1 / 16][j1 % 16] - c3 * bf16_hi(q4[e]);
        }
      }
    }
    if (owns) {
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        const int m = (8 * i) / 16, r = (8 * i) % 16;
        XG[pos(n, dv0 / 8 + i)] =
            make_uint4(pack_bf16x2(acc[m][r], acc[m][r + 1]), pack_bf16x2(acc[m][r + 2], acc[m][r + 3]),
                       pack_bf16x2(acc[m][r + 4], acc[m][r + 5]), pack_bf16x2(acc[m][r + 6], acc[m][r + 7]));
      }
    }
    fence();
#pragma unroll
    for (int i = 0; i < NL; ++i) buf_store16(XG[pos(RPI * i + lrow, lch)], dqr, tb + (uint32_t)(RPI * i) * rowbytes);
    fence();
  };

  uint4 qv[NL];
  fetch_q(wave, qv);
  for (int k = 0; k < per_wave; ++k) process(wave + NW * k, qv);

  if constexpr (DGAIN) {
    // the four waves' sums through LDS (the tiles are free once every wave is
    // done), added in wave order: one row of d sums per (frame, head)
    __syncthreads();
    float* red = reinterpret_cast<float*>(&xq[0][0]);  // [NW][DP]
    if (owns && n % GR == 0) {
#pragma unroll
      for (int k = 0; k < GK; ++k) red[wave * DP + dv0 + (n / GR) * GK + k] = gsum[k];
    }
    __syncthreads();
    if (tid < D) {
      float v = red[tid];
#pragma unroll
      for (int w2 = 1; w2 < NW; ++w2) v += red[w2 * DP + tid];
      GP[(size_t)blockIdx.x * D + tid] = v;
    }
  }
}

// dgamma[j] = scale * the sum over the rows of GP [rows][D] (one row per
// (batch, frame, head)) for j < n: 1024 threads, thread (s, j) adding rows
// s, s + S, ... in order, then the S partial sums added in order.
template <int D>
__global__ __launch_bounds__(1024) void gain_grad_sum(const float* __restrict__ GP, float* __restrict__ dgamma,
                                                      int rows, int n, float scale) {
  constexpr int S = 1024 / D;
  __shared__ float part[1024];
  const int tid = threadIdx.x, j = tid % D, sl = tid / D;
  float v = 0.f;
  for (int r = sl; r < rows; r += S) v += GP[(size_t)r * D + j];
  part[tid] = v;
  __syncthreads();
  if (tid < n) {
    float a = part[tid];
    for (int k = 1; k < S; ++k) a += part[k * D + tid];
    dgamma[tid] = a * scale;
  }
}

template <int D>
hipError_t backward_readout_d(const Problem& p, const void* q, const void* gate, const float* rms_weight,
                              const void* dy, const void* rstates, const float* s_text, const float* fwd, const float* rev,
                              const float* alpha, void* rstates_t, void* dout, void* dq, void* dgate,
                              float* dsq, float* gain_part, float* dgamma, int gain_n, float gain_scale,
                              hipStream_t s) {
  hipLaunchKernelGGL(pack_states_t<D>, dim3((unsigned)(p.B * p.H * (p.nc + 1))), dim3(256), 0, s, s_text, fwd,
                     rev, alpha, static_cast<uint4*>(rstates_t), p.nc, p.T, p.H, p.C, p.bridge ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const void* do_ = dy;
  if (p.epilogue) {
    // do, dgate and dq = S_q^T do in one pass
    const unsigned grid = (unsigned)(p.B * p.T * p.H);
    auto u16 = [](const void* x) { return static_cast<const uint16_t*>(x); };
    auto w16 = [](void* x) { return static_cast<uint16_t*>(x); };
    auto launch = [&](auto gamma, auto qn, auto dgain) {
      constexpr bool GM = decltype(gamma)::value, QN = decltype(qn)::value;
      hipLaunchKernelGGL((readout_bwd_bf16<D, GM, QN, decltype(dgain)::value>), dim3(grid), dim3(256), 0, s, u16(q),
                         u16(gate), u16(dy), rms_weight, static_cast<const uint4*>(rstates),
                         static_cast<const uint4*>(rstates_t), w16(dout), w16(dgate), w16(dq), p.T, p.U, p.H, p.C,
                         p.nc, p.rms_eps, p.l2_eps, gain_part);
    };
    using Y = std::true_type;
    using N = std::false_type;
    auto launch_g = [&](auto dgain) {
      if (rms_weight)
        p.qnorm ? launch(Y(), Y(), dgain) : launch(Y(), N(), dgain);
      else
        p.qnorm ? launch(N(), Y(), dgain) : launch(N(), N(), dgain);
    };
    dgamma ? launch_g(Y()) : launch_g(N());
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (dgamma && (e = launch_gain_grad_sum(p, gain_part, dgamma, gain_n, gain_scale, s)) != hipSuccess) return e;
    do_ = dout;
  } else {
    // without the epilogue do is dy: dq = S_q^T dy is the forward readout, raw,
    // on the transposed states
    Problem raw = p;
    raw.qnorm = false;
    e = launch_readout(raw, dy, nullptr, nullptr, rstates_t, dq, s);
    if (e != hipSuccess) return e;
  }
  // dS_q(t) = do_t^T q_t for every frame
  return launch_gram_plain(p, q, do_, dsq, s);
}

// ---------------------------------------------------------------------------
// second stage: from the query-state adjoints to dA_s, dB_s and dalpha_s
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void fill_zero(uint4* __restrict__ p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = make_uint4(0, 0, 0, 0);
}

// The coverage rules backwards: the adjoint of record F_j is the sum of dS_q
// over the non-anchor frames of chunk j + 2, that of R_j over chunk j - 2; S_T
// receives dS_q of the anchors, half of dS_q where a side reads S_T / 2, and
// half of the adjoint of every record the scan never reaches (a record whose
// coverage is empty is S_T / 2 itself).  With the decay bridge a query chunk
// c's side reads its state times Diag(df_c) (forward: alpha over chunk c - 1)
// or Diag(dr_c) (reverse: alpha over chunk c + 1), so that chunk's sum reaches
// the side column-scaled by the same products.  One thread per 4 consecutive
// entries (one row, 4 columns) of the d x d matrices of one (batch, head).
template <int D>
__global__ __launch_bounds__(256) void backward_gather(const float* __restrict__ dsq, float* __restrict__ dF,
                                                       float* __restrict__ dR, float* __restrict__ dST,
                                                       const float* __restrict__ alpha, int T, int C, int nc, int H,
                                                       int bridge) {
  constexpr int N4 = D * D / 4;
  const int per = (N4 + 255) / 256;
  const int head = blockIdx.x / per;
  const int e4 = (blockIdx.x % per) * 256 + threadIdx.x;
  if (e4 >= N4) return;
  const int b = head / H, h = head % H, col = (4 * e4) % D;
  const float4* S = reinterpret_cast<const float4*>(dsq) + (size_t)head * T * N4 + e4;
  float4* F = reinterpret_cast<float4*>(dF) + (size_t)head * nc * N4 + e4;
  float4* R = reinterpret_cast<float4*>(dR) + (size_t)head * nc * N4 + e4;
  auto add = [](float4& a, float4 b, float w) {
    a.x += w * b.x; a.y += w * b.y; a.z += w * b.z; a.w += w * b.w;
  };
  // product of alpha over frames s0 .. s1 - 1 for this thread's 4 columns
  auto decay = [&](int s0, int s1) {
    float4 d = make_float4(1.f, 1.f, 1.f, 1.f);
    for (int s = s0; s < s1; ++s) {
      const float4 a = *reinterpret_cast<const float4*>(alpha + (((size_t)b * T + s) * H + h) * D + col);
      d.x *= a.x; d.y *= a.y; d.z *= a.z; d.w *= a.w;
    }
    return d;
  };
  auto scaled = [](float4 g, float4 d) { return make_float4(g.x * d.x, g.y * d.y, g.z * d.z, g.w * d.w); };
  float4 st = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < nc; ++j) {
    // chunk j's non-anchor frames feed F_{j-2} and R_{j+2}
    float4 g = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int t = C * j; t < min(C * (j + 1), T); ++t)
      if (t != 0 && t != T - 1) add(g, S[(size_t)t * N4], 1.f);
    const float4 one = make_float4(1.f, 1.f, 1.f, 1.f);
    const float4 df = bridge && j >= 1 ? decay(C * (j - 1), C * j) : one;
    const float4 dr = bridge && j + 1 <= nc - 1 ? decay(C * (j + 1), min(C * (j + 2), T)) : one;
    const float4 gf = scaled(g, df), gr = scaled(g, dr);
    if (j >= 2) F[(size_t)(j - 2) * N4] = gf; else add(st, gf, 0.5f);
    if (j + 2 <= nc - 1) R[(size_t)(j + 2) * N4] = gr; else add(st, gr, 0.5f);
  }
  // slots no chunk feeds (F_{nc-2}, F_{nc-1}, R_0, R_1) are not records: zero,
  // since the adjoint scan reads every slot (scaled by zero where it is none)
  for (int j = max(nc - 2, 0); j < nc; ++j) F[(size_t)j * N4] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < min(2, nc); ++j) R[(size_t)j * N4] = make_float4(0.f, 0.f, 0.f, 0.f);
  // records the scan never reaches (empty coverage) are S_T / 2 itself
  for (int j = 0; j <= nc - 3; ++j)
    if (min(C * (j + 1) - 1, T - 2) < 1) add(st, F[(size_t)j * N4], 0.5f);
  for (int j = nc - 1; j >= 2; --j)
    if (max(C * j, 1) > T - 2) add(st, R[(size_t)j * N4], 0.5f);
  if (T >= 1) add(st, S[0], 1.f);
  if (T >= 2) add(st, S[(size_t)(T - 1) * N4], 1.f);
  reinterpret_cast<float4*>(dST)[(size_t)head * N4 + e4] = st;
}

// P = (I + A_s)^{-1} as float32 [d][d] from the solve's two bfloat16 planes
// (hi + lo; fragment f = ((2w + e)(d/32) + ks)*64 + l holds
// P[32 ks + 8 (l/16) + j][32 w + 2 (l%16) + e], j = 0..7).  One workgroup per slot.
template <int D>
__global__ __launch_bounds__(256) void decode_pinv(const uint4* __restrict__ planes, float* __restrict__ P) {
  constexpr int KS = D / 32, NFR = D * D / 8;
  const uint4* src = planes + (size_t)blockIdx.x * 2 * NFR;
  float* dst = P + (size_t)blockIdx.x * D * D;
  for (int f = threadIdx.x; f < NFR; f += 256) {
    const int l = f % 64, ks = (f / 64) % KS, we = (f / 64) / KS;
    const int col = 32 * (we / 2) + 2 * (l % 16) + we % 2, row0 = 32 * ks + 8 * (l / 16);
    const uint4 h = src[f], lo = src[NFR + f];
    const uint32_t hw[4] = {h.x, h.y, h.z, h.w}, lw[4] = {lo.x, lo.y, lo.z, lo.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dst[(row0 + 2 * e) * D + col] = bf16_lo(hw[e]) + bf16_lo(lw[e]);
      dst[(row0 + 2 * e + 1) * D + col] = bf16_hi(hw[e]) + bf16_hi(lw[e]);
    }
  }
}

// One operand of a batched d x d product: matrix (head, slot) at
// base + head * head_stride + (slot + slot_offset) * slot_stride (floats).
struct MatArg {
  const float* base;
  size_t head_stride, slot_stride;
  int slot_offset;
};

// The batched d x d products of the second stage, for every (head, slot) with
// slots 1..T-2 (the absorbed frames) and T (the text frame); workgroup i takes
// head i / n and the (i % n)-th of those n slots:
//   C = alpha sum_p op(A_p) op(B_p) + epilogue,
// with op(X) = X^T where the T flag is set, pair 0's A or B optionally the sum
// of two matrices (ADDA / ADDB: the two scans' adjoints), and the epilogue
//   EPI_PLAIN:  nothing more;
//   EPI_DIAG:   + Diag(a) E, a = alpha_t of the frame (zero for the text slot);
//   EPI_ROWDOT: C is written and, for frames, r[k] = sum_m C[k][m] E[k][m]
//               into the per-frame vector out (dalpha).
// float32 on v_mfma_f32_16x16x4f32.  K runs in panels of KP, both operands'
// panels staged in LDS in their source orientation (rows padded by 4 floats),
// small enough for several workgroups per CU, the next panel loading into
// registers while the current one is multiplied; wave w forms output rows
// (d / NWA) w .. of all columns.
enum { EPI_PLAIN = 0, EPI_DIAG, EPI_ROWDOT };

struct GemmArgs {
  MatArg a[2], b[2];     // product pairs
  MatArg a2, b2;         // pair 0's second summand (ADDA / ADDB)
  MatArg e;              // epilogue operand
  const float* alpha;    // [B, T, H, d] (EPI_DIAG)
  float* out;            // [B, T, H, d] (EPI_ROWDOT)
  float* c;              // C at c + head * c_head + slot * c_slot
  size_t c_head, c_slot;
  float scale;
  int T, H;
};

template <int D, bool TA, bool TB, int NPAIR, bool ADDA, bool ADDB, int EPI>
__global__ __launch_bounds__(256, 2) void gemm_dd(GemmArgs g) {
  constexpr int KP = D < 32 ? D : 32;
  constexpr int NWA = D / 16 >= 4 ? 4 : D / 16;  // waves with rows
  constexpr int MTW = D / 16 / NWA;               // 16-row tiles per such wave
  constexpr int NT = D / 16;
  // panel shapes: op(A) panel is A[k0.., all m] (TA) or A[all m][k0..] (!TA)
  constexpr int LA = TA ? D + 4 : KP + 4, RA = TA ? KP : D, CA = TA ? D : KP;
  constexpr int LB = TB ? KP + 4 : D + 4, RB = TB ? D : KP, CB = TB ? KP : D;
  constexpr int NA4 = RA * CA / 4, NB4 = RB * CB / 4;
  __shared__ float sa[RA * LA], sb[RB * LB];
  const int T = g.T;
  const int nfr = T > 2 ? T - 2 : 0, nslot = nfr + 1;
  const int head = blockIdx.x / nslot, kslot = blockIdx.x % nslot;
  const int slot = kslot < nfr ? 1 + kslot : T;
  auto mat = [&](const MatArg& m) {
    return m.base + head * m.head_stride + (size_t)(slot + m.slot_offset) * m.slot_stride;
  };
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  f32x4 acc[MTW][NT];
#pragma unroll
  for (int mi = 0; mi < MTW; ++mi)
#pragma unroll
    for (int nj = 0; nj < NT; ++nj) acc[mi][nj] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int m0 = 16 * MTW * wave;
  // one panel of both operands in registers: n4 float4 of a block `cols` wide
  // at row r0, column c0 of the source, and of the second source where the
  // pair adds one (added when the panel goes to LDS)
  constexpr int MAXV = ((NA4 > NB4 ? NA4 : NB4) + 255) / 256;
  struct Panel {
    float4 a[MAXV], a2[MAXV], b[MAXV], b2[MAXV];
  };
  auto fetch = [&](float4 (&v)[MAXV], float4 (&v2)[MAXV], int cols, const float* s1, const float* s2, bool add,
                   int r0, int c0, int n4) {
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const int f = tid + 256 * i;
      if (f < n4) {
        const int r = f / (cols / 4), c4 = f % (cols / 4);
        const size_t off = (size_t)(r0 + r) * D + c0 + 4 * c4;
        v[i] = *reinterpret_cast<const float4*>(s1 + off);
        if (add) v2[i] = *reinterpret_cast<const float4*>(s2 + off);
      }
    }
  };
  auto put = [&](float* dst, int ld, int cols, const float4 (&v)[MAXV], const float4 (&v2)[MAXV], bool add, int n4) {
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const int f = tid + 256 * i;
      if (f < n4) {
        const int r = f / (cols / 4), c4 = f % (cols / 4);
        float4 x = v[i];
        if (add) {
          x.x += v2[i].x; x.y += v2[i].y; x.z += v2[i].z; x.w += v2[i].w;
        }
        *reinterpret_cast<float4*>(&dst[r * ld + 4 * c4]) = x;
      }
    }
  };
  // panels in order: pair pr, K-offset k0; panel i + 1 loads into registers
  // while panel i is multiplied
  constexpr int PPP = D / KP;  // panels per pair
  auto fetch_panel = [&](int idx, Panel& P) {
    const int pr = idx / PPP, k0 = (idx % PPP) * KP;
    const bool adda = ADDA && pr == 0, addb = ADDB && pr == 0;
    const float* A1 = mat(g.a[pr]);
    const float* B1 = mat(g.b[pr]);
    fetch(P.a, P.a2, CA, A1, adda ? mat(g.a2) : A1, adda, TA ? k0 : 0, TA ? 0 : k0, NA4);
    fetch(P.b, P.b2, CB, B1, addb ? mat(g.b2) : B1, addb, TB ? 0 : k0, TB ? k0 : 0, NB4);
  };
  Panel P;
  fetch_panel(0, P);
#pragma unroll 1
  for (int idx = 0; idx < NPAIR * PPP; ++idx) {
    const bool adda = ADDA && idx < PPP, addb = ADDB && idx < PPP;
    __syncthreads();  // the previous panel has been read
    put(sa, LA, CA, P.a, P.a2, adda, NA4);
    put(sb, LB, CB, P.b, P.b2, addb, NB4);
    __syncthreads();
    if (idx + 1 < NPAIR * PPP) fetch_panel(idx + 1, P);
    if (wave < NWA) {
      // op(A)[m][k] and op(B)[k][n] of the panel (k local)
      auto opa = [&](int m, int kk) { return TA ? sa[kk * LA + m] : sa[m * LA + kk]; };
      auto opb = [&](int kk, int n) { return TB ? sb[n * LB + kk] : sb[kk * LB + n]; };
#pragma unroll 2
      for (int k4 = 0; k4 < KP / 4; ++k4) {
        const int kk = 4 * k4 + (lane >> 4);
        float av[MTW], bv[NT];
#pragma unroll
        for (int mi = 0; mi < MTW; ++mi) av[mi] = opa(m0 + 16 * mi + (lane & 15), kk);
#pragma unroll
        for (int nj = 0; nj < NT; ++nj) bv[nj] = opb(kk, 16 * nj + (lane & 15));
#pragma unroll
        for (int mi = 0; mi < MTW; ++mi)
#pragma unroll
          for (int nj = 0; nj < NT; ++nj)
            acc[mi][nj] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[mi], bv[nj], acc[mi][nj], 0, 0, 0);
      }
    }
  }
  if (wave >= NWA) return;
  // tile (mi, nj), lane l, reg r: C[m0 + 16 mi + 4 (l/16) + r][16 nj + l%16]
  float* c = g.c + head * g.c_head + (size_t)slot * g.c_slot;
  const float* E = EPI != EPI_PLAIN ? mat(g.e) : nullptr;
  const int b = head / g.H, h = head % g.H;
  const bool frame = slot < T;
#pragma unroll
  for (int mi = 0; mi < MTW; ++mi)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + 16 * mi + 4 * (lane >> 4) + r;
      float arow = 0.f;
      if constexpr (EPI == EPI_DIAG) arow = frame ? g.alpha[(((size_t)b * T + slot) * g.H + h) * D + row] : 0.f;
      float dot = 0.f;
#pragma unroll
      for (int nj = 0; nj < NT; ++nj) {
        const size_t o = (size_t)row * D + 16 * nj + (lane & 15);
        float v = g.scale * acc[mi][nj][r];
        if constexpr (EPI == EPI_DIAG) v += arow * E[o];
        if constexpr (EPI == EPI_ROWDOT) dot += v * E[o];
        c[o] = v;
      }
      if constexpr (EPI == EPI_ROWDOT) {
        dot += __shfl_xor(dot, 1);
        dot += __shfl_xor(dot, 2);
        dot += __shfl_xor(dot, 4);
        dot += __shfl_xor(dot, 8);
        if (frame && (lane & 15) == 0) g.out[(((size_t)b * T + slot) * g.H + h) * D + row] = dot;
      }
    }
}

// The decay bridge's own term of dalpha.  A query chunk c's forward side reads
// wf F_{c-2} Diag(df_c), df_c the product of alpha over chunk c - 1, so frame
// s of chunk c - 1 gets, per key channel k,
//   dalpha_s[k] += sum_i G_c[i][k] wf F_{c-2}[i][k] prod_{s' != s} alpha_{s'}[k]
// with G_c the sum of dS_q over chunk c's non-anchor frames (S_T / 2 for a
// missing record); the reverse side likewise with chunk c + 1 and R_{c+2}.
// Workgroup (head, chunk j) serves the frames of chunk j: the forward term
// from query chunk j + 1 and the reverse term from query chunk j - 1, added
// onto dalpha after the products have written it; thread k owns channel k.
template <int D>
__global__ __launch_bounds__(256) void bridge_dalpha(const float* __restrict__ dsq, const float* __restrict__ s_text,
                                                     const float* __restrict__ fwd, const float* __restrict__ rev,
                                                     const float* __restrict__ alpha, float* __restrict__ dalpha,
                                                     int T, int C, int nc, int H) {
  const int j = blockIdx.x % nc, head = blockIdx.x / nc;
  const int b = head / H, h = head % H;
  const int k = threadIdx.x;
  if (k >= D) return;
  const size_t DD = (size_t)D * D;
  const float* S = dsq + (size_t)head * T * DD;
  const float* ST = s_text + (size_t)head * DD;
  auto al = [&](int s) { return alpha[(((size_t)b * T + s) * H + h) * D + k]; };
  // sum over rows i of G_c[i][k] * w * side[i][k]
  auto coldot = [&](int c, const float* side, float w) {
    float acc = 0.f;
    for (int i = 0; i < D; ++i) {
      float g = 0.f;
      for (int t = C * c; t < min(C * (c + 1), T); ++t)
        if (t != 0 && t != T - 1) g += S[(size_t)t * DD + (size_t)i * D + k];
      acc += g * w * side[(size_t)i * D + k];
    }
    return acc;
  };
  const int s0 = C * j, s1 = min(C * (j + 1), T);
  float cf = 0.f, cr = 0.f;
  bool hf = false, hr = false;
  if (j + 1 <= nc - 1) {  // query chunk c = j + 1 bridges over chunk j forwards
    const int c = j + 1;
    const float* side = c >= 2 ? fwd + ((size_t)head * nc + (c - 2)) * DD : ST;
    cf = coldot(c, side, c >= 2 ? 1.f : 0.5f);
    hf = true;
  }
  if (j >= 1) {  // query chunk c = j - 1 bridges over chunk j backwards
    const int c = j - 1;
    const float* side = c + 2 <= nc - 1 ? rev + ((size_t)head * nc + (c + 2)) * DD : ST;
    cr = coldot(c, side, c + 2 <= nc - 1 ? 1.f : 0.5f);
    hr = true;
  }
  for (int s = s0; s < s1; ++s) {
    float others = 1.f;  // product of alpha over the chunk's other frames
    for (int u = s0; u < s1; ++u)
      if (u != s) others *= al(u);
    float d = 0.f;
    if (hf) d += cf * others;
    if (hr) d += cr * others;
    dalpha[(((size_t)b * T + s) * H + h) * D + k] += d;
  }
}

// The text frame's adjoint: dS_T (from the queries) plus half the final
// adjoint of each scan (both start from S_T / 2), into slot T of lam_f.
__global__ __launch_bounds__(256) void text_adjoint(const float* __restrict__ dST, const float* __restrict__ fin,
                                                    float* __restrict__ lam_f, int T, int DD) {
  const int head = blockIdx.y;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < DD; i += gridDim.x * 256)
    lam_f[((size_t)head * (T + 1) + T) * DD + i] =
        dST[(size_t)head * DD + i] + 0.5f * (fin[((size_t)head * 2) * DD + i] + fin[((size_t)head * 2 + 1) * DD + i]);
}
}  // namespace

hipError_t launch_backward_readout(const Problem& p, const void* q, const void* gate, const float* rms_weight,
                                   const void* dy, const void* rstates, const float* s_text, const float* fwd, const float* rev,
                                   const float* alpha, void* rstates_t, void* dout, void* dq, void* dgate,
                                   float* dsq, float* gain_part, float* dgamma, int gain_n, float gain_scale,
                                   hipStream_t s) {
  if (dgamma && (!p.epilogue || !gain_part || gain_n < 1 || gain_n > p.D)) return hipErrorInvalidValue;
  if (!p.bf16) {
    auto f = [](const void* x) { return static_cast<const float*>(x); };
    auto g = [](void* x) { return static_cast<float*>(x); };
    return launch_backward_readout_f32(p, f(q), f(gate), rms_weight, f(dy), s_text, fwd, rev, alpha, g(rstates_t),
                                       g(dout), g(dq), g(dgate), dsq, gain_part, dgamma, gain_n, gain_scale, s);
  }
  switch (p.D) {
    case 16: return backward_readout_d<16>(p, q, gate, rms_weight, dy, rstates, s_text, fwd, rev, alpha, rstates_t, dout, dq, dgate, dsq, gain_part, dgamma, gain_n, gain_scale, s);
    case 32: return backward_readout_d<32>(p, q, gate, rms_weight, dy, rstates, s_text, fwd, rev, alpha, rstates_t, dout, dq, dgate, dsq, gain_part, dgamma, gain_n, gain_scale, s);
    case 64: return backward_readout_d<64>(p, q, gate, rms_weight, dy, rstates, s_text, fwd, rev, alpha, rstates_t, dout, dq, dgate, dsq, gain_part, dgamma, gain_n, gain_scale, s);
    case 128: return backward_readout_d<128>(p, q, gate, rms_weight, dy, rstates, s_text, fwd, rev, alpha, rstates_t, dout, dq, dgate, dsq, gain_part, dgamma, gain_n, gain_scale, s);
    default: return hipErrorInvalidValue;
  }
}

// second stage orchestration -------------------------------------------------

namespace {

template <int D>
hipError_t backward_scan_d(const Problem& p, const BwdScanBuffers& w, hipStream_t s) {
  const size_t heads = (size_t)p.B * p.H, DD = (size_t)D * D;
  const int T = p.T;
  auto fill = [&](void* ptr, size_t bytes) {
    const size_t n16 = bytes / 16;
    const unsigned grid = (unsigned)std::min<size_t>((n16 + 255) / 256, 4096);
    if (grid) hipLaunchKernelGGL(fill_zero, dim3(grid), dim3(256), 0, s, static_cast<uint4*>(ptr), n16);
    return hipGetLastError();
  };
  hipError_t e;
  if ((e = fill(w.states_f, heads * (T + 2) * DD * 4)) != hipSuccess) return e;
  if ((e = fill(w.states_r, heads * (T + 2) * DD * 4)) != hipSuccess) return e;
  if ((e = fill(w.lam_f, heads * (T + 1) * DD * 4)) != hipSuccess) return e;
  if ((e = fill(w.lam_r, heads * (T + 1) * DD * 4)) != hipSuccess) return e;
  if ((e = fill(w.dA, heads * (T + 1) * DD * 4)) != hipSuccess) return e;
  if ((e = fill(w.dB, heads * (T + 1) * DD * 4)) != hipSuccess) return e;
  if ((e = fill(w.dalpha, (size_t)p.B * T * p.H * D * 4)) != hipSuccess) return e;
  // record adjoints and the queries' part of dS_T
  hipLaunchKernelGGL(backward_gather<D>, dim3((unsigned)(heads * ((DD / 4 + 255) / 256))), dim3(256), 0, s,
                     w.dsq, w.dF, w.dR, w.dST, w.alpha, T, p.C, p.nc, p.H, p.bridge ? 1 : 0);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // every frame's state, then the adjoint scans
  if ((e = launch_scan_states(p, w.stats, w.pinv, w.alpha, w.states_f, w.states_r, s)) != hipSuccess) return e;
  if ((e = launch_scan_adjoint(p, w.stats, w.pinv, w.alpha, w.dF, w.dR, w.lam_f, w.lam_r, w.lam_final, s)) !=
      hipSuccess)
    return e;
  hipLaunchKernelGGL(text_adjoint, dim3(8, (unsigned)heads), dim3(256), 0, s, w.dST, w.lam_final, w.lam_f, T,
                     (int)DD);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // P as float32
  const float* P = w.pinv;
  if (pinv_split(p)) {
    if constexpr (D >= 32) {
      hipLaunchKernelGGL(decode_pinv<D>, dim3((unsigned)(heads * (T + 1))), dim3(256), 0, s,
                         reinterpret_cast<const uint4*>(w.pinv), w.p32);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      P = w.p32;
    }
  }
  // the per-frame products over frames 1..T-2 and the text slot T
  const unsigned grid = (unsigned)(heads * ((T > 2 ? T - 2 : 0) + 1));  // frames 1..T-2 and the text slot
  const size_t hs1 = (T + 1) * DD, hs2 = (T + 2) * DD;
  const MatArg Sf{w.states_f, hs2, DD, -1}, Sr{w.states_r, hs2, DD, 1}, Lf{w.lam_f, hs1, DD, 0},
      Lr{w.lam_r, hs1, DD, 0}, Bs{w.stats + DD, (T + 1) * 2 * DD, 2 * DD, 0}, Pm{P, hs1, DD, 0},
      DP{w.dPinv, hs1, DD, 0}, Tm{w.tmp, hs1, DD, 0};
  const MatArg none{nullptr, 0, 0, 0};
  auto args = [&](float* C, float scale) {
    GemmArgs a;
    a.a[0] = a.a[1] = a.b[0] = a.b[1] = a.a2 = a.b2 = a.e = none;
    a.alpha = w.alpha;
    a.out = w.dalpha;
    a.c = C;
    a.c_head = hs1;
    a.c_slot = DD;
    a.scale = scale;
    a.T = T;
    a.H = p.H;
    return a;
  };
  auto launch = [&](auto kernel, const GemmArgs& a) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
  };
  // M = Sf^T lam_f + Sr^T lam_r; dalpha = rowdot(M, P) (P is symmetric: the diagonal of M P)
  GemmArgs g = args(w.M, 1.f);
  g.a[0] = Sf, g.b[0] = Lf, g.a[1] = Sr, g.b[1] = Lr, g.e = Pm;
  if ((e = launch(gemm_dd<D, true, false, 2, false, false, EPI_ROWDOT>, g)) != hipSuccess) return e;
  // dPinv = B^T (lam_f + lam_r) + Diag(alpha) M
  g = args(w.dPinv, 1.f);
  g.a[0] = Bs, g.b[0] = Lf, g.b2 = Lr, g.e = MatArg{w.M, hs1, DD, 0};
  if ((e = launch(gemm_dd<D, true, false, 1, false, true, EPI_DIAG>, g)) != hipSuccess) return e;
  // dB = (lam_f + lam_r) P
  g = args(w.dB, 1.f);
  g.a[0] = Lf, g.a2 = Lr, g.b[0] = Pm;
  if ((e = launch(gemm_dd<D, false, false, 1, true, false, EPI_PLAIN>, g)) != hipSuccess) return e;
  // dA = -P dPinv P
  g = args(w.tmp, 1.f);
  g.a[0] = DP, g.b[0] = Pm;
  if ((e = launch(gemm_dd<D, false, false, 1, false, false, EPI_PLAIN>, g)) != hipSuccess) return e;
  g = args(w.dA, -1.f);
  g.a[0] = Pm, g.b[0] = Tm;
  if ((e = launch(gemm_dd<D, false, false, 1, false, false, EPI_PLAIN>, g)) != hipSuccess) return e;
  // the decay bridge's own term of dalpha, after the products have written it
  if (p.bridge) {
    hipLaunchKernelGGL(bridge_dalpha<D>, dim3((unsigned)(heads * p.nc)), dim3(D < 64 ? 64 : D), 0, s, w.dsq, w.s_text,
                       w.fwd, w.rev, w.alpha, w.dalpha, T, p.C, p.nc, p.H);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_backward_scan(const Problem& p, const BwdScanBuffers& w, hipStream_t s) {
  if (p.T < 1) return hipErrorInvalidValue;
  switch (p.D) {
    case 16: return backward_scan_d<16>(p, w, s);
    case 32: return backward_scan_d<32>(p, w, s);
    case 64: return backward_scan_d<64>(p, w, s);
    case 128: return backward_scan_d<128>(p, w, s);
    default: return hipErrorInvalidValue;
  }
}

namespace {

// ---------------------------------------------------------------------------
// third stage: dk, dv, dbeta per token from dA_s, dB_s of its frame
// ---------------------------------------------------------------------------
// A_s = sum_u beta_u k_u k_u^T and B_s = sum_u beta_u v_u k_u^T (the frame
// statistics, section "어떻게 쓰나"), so with G = dA + dA^T
//   dk_u = beta_u (G k_u + dB^T v_u),   dv_u = beta_u dB k_u,
//   dbeta_u = k_u^T dA k_u + v_u^T dB k_u = 1/2 k_u . (G k_u) + v_u . (dB k_u).
// dbeta is a sum of d^2 products that largely cancel, so the two products it
// uses, G k and dB k, take their matrices as bfloat16 hi + lo planes (about
// 2^-16 relative operand rounding); dB^T v enters dk only and takes the hi
// plane alone (2^-9, below the bfloat16 output's own rounding).  The five
// planes of a slot are the matrix-core A operands, shared through LDS (160 KB
// at d = 128); the token operands come straight from global memory.

// Planes of a slot, in the readout's operand order (fragment (mt, ks, lane)
// holds M[dv_of(mt, lane % 32)][(d/2)(lane / 32) + 8 ks + j], j = 0..7).
enum { GP_G_HI = 0, GP_G_LO, GP_DB_HI, GP_DB_LO, GP_DBT_HI, GP_PLANES };

template <int D>
__global__ __launch_bounds__(256) void pack_grad_mats(const float* __restrict__ dA, const float* __restrict__ dB,
                                                      uint4* __restrict__ out) {
  constexpr int DP = D < 32 ? 32 : D;
  constexpr int HALF = DP / 2;
  constexpr int MT = DP / 32;
  constexpr int KS = D / 16;
  constexpr int NF = MT * KS * 64;
  const float* a = dA + (size_t)blockIdx.x * D * D;
  const float* bm = dB + (size_t)blockIdx.x * D * D;
  uint4* o = out + (size_t)blockIdx.x * GP_PLANES * NF;
  auto dv_of = [&](int mt, int m) { return HALF * ((m >> 2) & 1) + 16 * mt + 4 * (m >> 3) + (m & 3); };
  // one fragment of each matrix per iteration: G (hi, lo), dB (hi, lo), dB^T (hi)
  for (int f = threadIdx.x; f < 3 * NF; f += 256) {
    const int which = f / NF, g = f % NF;
    const int lane = g % 64, ks = (g / 64) % KS, mt = g / (64 * KS);
    const int row = dv_of(mt, lane & 31);
    const int c0 = (D / 2) * (lane >> 5) + 8 * ks;
    const bool live = row < D;
    const int r = live ? row : 0;
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      __bf16 h2[2], l2[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = c0 + 2 * e + h;
        float v;
        if (which == 0) v = a[(size_t)r * D + c] + a[(size_t)c * D + r];  // G = dA + dA^T
        else if (which == 1) v = bm[(size_t)r * D + c];                   // dB
        else v = bm[(size_t)c * D + r];                                   // dB^T
        split_bf16(live ? v : 0.f, h2[h], l2[h]);
      }
      hi[e] = __builtin_bit_cast(uint32_t, bf16x2{h2[0], h2[1]});
      lo[e] = __builtin_bit_cast(uint32_t, bf16x2{l2[0], l2[1]});
    }
    const uint4 H4 = make_uint4(hi[0], hi[1], hi[2], hi[3]), L4 = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    if (which == 0) {
      o[GP_G_HI * NF + g] = H4;
      o[GP_G_LO * NF + g] = L4;
    } else if (which == 1) {
      o[GP_DB_HI * NF + g] = H4;
      o[GP_DB_LO * NF + g] = L4;
    } else {
      o[GP_DBT_HI * NF + g] = H4;
    }
  }
}

// One part of a launch: frames t_first .. t_first + n_frames - 1 of k, v,
// beta laid out [B, T_in, U, H, d] (beta [B, T_in, U, H]) and their gradients,
// reading the packed planes of slot t + slot_offset.
struct GradPart {
  const uint16_t *k, *v, *beta;
  uint16_t *dk, *dv, *dbeta;
  int T_in, U, t_first, n_frames, slot_offset;
};

// One (frame, head) per workgroup; 4 waves stream 32-token tiles, the next
// tile's operands loading while the current one is multiplied.  Lane
// (n = lane % 32, half = lane / 32) takes token n's channels
// (d/2) half .. (d/2) half + d/2 - 1 as the B operand and, with
// dv0 = HALF * half, holds outputs dv0 + 16 mt + r in acc[mt][r].
template <int D, int NW, bool PREFETCH>
__global__ __launch_bounds__(64 * NW, 1) void gram_bwd_bf16(GradPart part0, GradPart part1, int nblk0,
                                                           const uint4* __restrict__ mats, int H, int T_slots) {
  constexpr int DP = D < 32 ? 32 : D;
  constexpr int HALF = DP / 2;
  constexpr int MT = DP / 32;
  constexpr int KS = D / 16;
  constexpr int NF = MT * KS * 64;
  constexpr int NG = HALF / 8;
  constexpr int NP = GP_PLANES * NF;
  constexpr int STAGE = (NP + 64 * NW - 1) / (64 * NW);
  __shared__ uint4 sm[NP];

  const bool second = (int)blockIdx.x >= nblk0;
  const GradPart g = second ? part1 : part0;
  int blk = (int)blockIdx.x - (second ? nblk0 : 0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blk % H;
  blk /= H;
  const int fi = blk % g.n_frames;
  const int b = blk / g.n_frames;
  const int t = g.t_first + fi;
  {
    const uint4* src = mats + ((size_t)(b * H + h) * T_slots + (t + g.slot_offset)) * NP;
    uint4 tmp[STAGE];
#pragma unroll
    for (int i = 0; i < STAGE; ++i) tmp[i] = src[min(tid + 64 * NW * i, NP - 1)];
#pragma unroll
    for (int i = 0; i < STAGE; ++i)
      if (tid + 64 * NW * i < NP) sm[tid + 64 * NW * i] = tmp[i];
  }
  __syncthreads();

  const int U = g.U;
  const size_t tok0 = ((size_t)b * g.T_in + t) * (size_t)U;
  const size_t fbase = (tok0 * H + h) * (size_t)D;
  const uint32_t rowbytes = (uint32_t)H * D * 2;
  const uint32_t nbytes = U > 0 ? (uint32_t)(U - 1) * rowbytes + D * 2 : 0;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(g.k + fbase, nbytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(g.v + fbase, nbytes);
  const __amdgpu_buffer_rsrc_t dkr = make_rsrc(g.dk + fbase, nbytes);
  const __amdgpu_buffer_rsrc_t dvr = make_rsrc(g.dv + fbase, nbytes);
  const uint32_t bbytes = U > 0 ? (uint32_t)(U - 1) * H * 2 + 2 : 0;
  const __amdgpu_buffer_rsrc_t br = make_rsrc(g.beta + tok0 * H + h, bbytes);
  const __amdgpu_buffer_rsrc_t dbr = make_rsrc(g.dbeta + tok0 * H + h, bbytes);

  const int n = lane & 31, half = lane >> 5;
  const int dv0 = HALF * half;
  const bool owns = dv0 < D;
  const uint32_t coff = (uint32_t)(D / 2) * half * 2;  // first operand byte of this lane in a row
  const int ntiles = (U + 31) / 32;

  struct Frag {
    bf16x8 k[KS], v[KS];
    uint16_t beta;
  };
  auto load = [&](int tile, Frag& f) {
    const uint32_t ro = (uint32_t)(tile * 32 + n) * rowbytes + coff;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) f.k[ks] = __builtin_bit_cast(bf16x8, buf_load16(kr, ro + 16 * ks));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) f.v[ks] = __builtin_bit_cast(bf16x8, buf_load16(vr, ro + 16 * ks));
    f.beta = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(br, (uint32_t)(tile * 32 + n) * H * 2, 0, 0);
  };
  // acc += plane w x operand, over the k-steps
  auto chain = [&](f32x16 (&acc)[MT], int w, const bf16x8 (&op)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, sm[w * NF + (mt * KS + ks) * 64 + lane]);
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, op[ks], acc[mt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // sum over this lane's outputs j of x_j acc[j] (x = the token operand's
  // channel dv0 + j): for d >= 32 those channels are the lane's own operand
  // words; at d = 16 half 0 owns all 16 outputs and takes channels 8..15 from
  // lane n + 32
  auto dotacc = [&](const bf16x8 (&op)[KS], const f32x16 (&acc)[MT]) {
    float s = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 u = __builtin_bit_cast(uint4, op[ks]);
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 8 * ks + 2 * e;
        s += bf16_lo(w4[e]) * acc[j / 16][j % 16] + bf16_hi(w4[e]) * acc[j / 16][(j + 1) % 16];
        if constexpr (D == 16) {
          const uint32_t o = (uint32_t)__shfl_xor((int)w4[e], 32);
          s += bf16_lo(o) * acc[0][8 + 2 * e] + bf16_hi(o) * acc[0][9 + 2 * e];
        }
      }
    }
    return s;
  };

  auto process = [&](int tile, const Frag& f) {
    f32x16 gk[MT], bk[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) gk[mt] = bk[mt] = f32x16{0.f};
    chain(gk, GP_G_HI, f.k);  // G k
    chain(gk, GP_G_LO, f.k);
    chain(bk, GP_DB_HI, f.k);  // dB k
    chain(bk, GP_DB_LO, f.k);
    const float bt = bf16_to_f32(f.beta);
    float dot = 0.5f * dotacc(f.k, gk) + dotacc(f.v, bk);
    if (!owns) dot = 0.f;
    dot += __shfl_xor(dot, 32);
    if (half == 0)
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(pack_bf16x2(dot, 0.f) & 0xffffu), dbr,
                                            (uint32_t)(tile * 32 + n) * H * 2, 0, 0);
    const uint32_t ro = (uint32_t)(tile * 32 + n) * rowbytes + (uint32_t)dv0 * 2;
    // out: beta * acc over the lane's channels dv0 .. dv0 + HALF - 1
    auto emit = [&](const f32x16 (&acc)[MT], const __amdgpu_buffer_rsrc_t& dst) {
      if (!owns) return;
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        const int m = (8 * i) / 16, r = (8 * i) % 16;
        buf_store16(make_uint4(pack_bf16x2(bt * acc[m][r], bt * acc[m][r + 1]),
                               pack_bf16x2(bt * acc[m][r + 2], bt * acc[m][r + 3]),
                               pack_bf16x2(bt * acc[m][r + 4], bt * acc[m][r + 5]),
                               pack_bf16x2(bt * acc[m][r + 6], bt * acc[m][r + 7])),
                    dst, ro + 16 * i);
      }
    };
    emit(bk, dvr);            // dv = beta dB k
    chain(gk, GP_DBT_HI, f.v);  // G k + dB^T v
    emit(gk, dkr);            // dk = beta (G k + dB^T v)
  };

  if constexpr (PREFETCH) {
    // two operand sets: tile i + NW loads while tile i is multiplied
    Frag fa, fb;
    int tile = wave;
    if (tile < ntiles) load(tile, fa);
    for (; tile < ntiles; tile += 2 * NW) {
      if (tile + NW < ntiles) load(tile + NW, fb);
      process(tile, fa);
      if (tile + NW >= ntiles) break;
      if (tile + 2 * NW < ntiles) load(tile + 2 * NW, fa);
      process(tile + NW, fb);
    }
  } else {
    // one operand set; the other wave on the SIMD covers the load latency
    for (int tile = wave; tile < ntiles; tile += NW) {
      Frag f;
      load(tile, f);
      process(tile, f);
    }
  }
}

// The same stage on v_mfma_f32_16x16x32_bf16 for d >= 32: lane (n, q) =
// (lane % 16, lane / 16) takes token n's channels 32 ks + 8 q .. + 7 as the B
// operand of k-step ks, so one load covers 16 tokens x 64 contiguous bytes
// (a quarter of the rows the 32 x 32 layout touches per instruction).  The
// planes' rows are permuted so that the lane's outputs of m-tiles 2p and
// 2p + 1 are channels 32 p + 8 q .. + 7, the same channels as its operand of
// k-step p: the stores are 16 bytes per lane with the loads' pattern, and
// dbeta needs no other lane's operand.  Each A fragment serves two 16-token
// groups (32 tokens per tile).
//   A operand: lane l holds A[l % 16][8 (l / 16) + j]; output: lane l, reg r
//   holds C[4 (l / 16) + r][l % 16]; row i of m-tile mt is channel
//   32 (mt / 2) + 8 (i / 4) + 4 (mt % 2) + i % 4.
template <int D>
__global__ __launch_bounds__(256) void pack_grad_mats16(const float* __restrict__ dA, const float* __restrict__ dB,
                                                        uint4* __restrict__ out) {
  constexpr int MT = D / 16;
  constexpr int KS = D / 32;
  constexpr int NF = MT * KS * 64;
  constexpr int LD = D + 1;  // odd row stride: the transposed reads hit distinct banks
  // the slot's dA and dB through LDS with coalesced loads (the fragments read
  // both orientations)
  __shared__ float sa[D * LD], sb[D * LD];
  {
    const float4* ga = reinterpret_cast<const float4*>(dA + (size_t)blockIdx.x * D * D);
    const float4* gb = reinterpret_cast<const float4*>(dB + (size_t)blockIdx.x * D * D);
    constexpr int N4 = D * D / 4, PER = (N4 + 255) / 256, BATCH = PER < 8 ? PER : 8;
    for (int i0 = 0; i0 < PER; i0 += BATCH) {
      float4 va[BATCH], vb[BATCH];
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
        const int i = threadIdx.x + 256 * (i0 + j);
        va[j] = i < N4 ? ga[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        vb[j] = i < N4 ? gb[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
        const int i = threadIdx.x + 256 * (i0 + j);
        if (i < N4) {
          const int r = (4 * i) / D, c = (4 * i) % D;
          sa[r * LD + c] = va[j].x; sa[r * LD + c + 1] = va[j].y; sa[r * LD + c + 2] = va[j].z; sa[r * LD + c + 3] = va[j].w;
          sb[r * LD + c] = vb[j].x; sb[r * LD + c + 1] = vb[j].y; sb[r * LD + c + 2] = vb[j].z; sb[r * LD + c + 3] = vb[j].w;
        }
      }
    }
  }
  __syncthreads();
  const float* a = sa;
  const float* bm = sb;
  uint4* o = out + (size_t)blockIdx.x * GP_PLANES * NF;
  for (int f = threadIdx.x; f < 3 * NF; f += 256) {
    const int which = f / NF, g = f % NF;
    const int lane = g % 64, ks = (g / 64) % KS, mt = g / (64 * KS);
    const int i = lane & 15;
    const int r = 32 * (mt >> 1) + 8 * (i >> 2) + 4 * (mt & 1) + (i & 3);  // output channel
    const int c0 = 32 * ks + 8 * (lane >> 4);                                // contraction channels
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      __bf16 h2[2], l2[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int c = c0 + 2 * e + hh;
        float v;
        if (which == 0) v = a[r * LD + c] + a[c * LD + r];  // G = dA + dA^T
        else if (which == 1) v = bm[r * LD + c];                // dB
        else v = bm[c * LD + r];                                // dB^T
        split_bf16(v, h2[hh], l2[hh]);
      }
      hi[e] = __builtin_bit_cast(uint32_t, bf16x2{h2[0], h2[1]});
      lo[e] = __builtin_bit_cast(uint32_t, bf16x2{l2[0], l2[1]});
    }
    const uint4 H4 = make_uint4(hi[0], hi[1], hi[2], hi[3]), L4 = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    if (which == 0) {
      o[GP_G_HI * NF + g] = H4;
      o[GP_G_LO * NF + g] = L4;
    } else if (which == 1) {
      o[GP_DB_HI * NF + g] = H4;
      o[GP_DB_LO * NF + g] = L4;
    } else {
      o[GP_DBT_HI * NF + g] = H4;
    }
  }
}

template <int D>
__global__ __launch_bounds__(256, 1) void gram_bwd16(GradPart part0, GradPart part1, int nblk0,
                                                     const uint4* __restrict__ mats, int H, int T_slots) {
  constexpr int NW = 4;
  constexpr int MT = D / 16;
  constexpr int KS = D / 32;
  constexpr int NF = MT * KS * 64;
  constexpr int NP = GP_PLANES * NF;
  constexpr int STAGE = (NP + 64 * NW - 1) / (64 * NW);
  __shared__ uint4 sm[NP];

  const bool second = (int)blockIdx.x >= nblk0;
  const GradPart g = second ? part1 : part0;
  int blk = (int)blockIdx.x - (second ? nblk0 : 0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blk % H;
  blk /= H;
  const int fi = blk % g.n_frames;
  const int b = blk / g.n_frames;
  const int t = g.t_first + fi;
  {
    const uint4* src = mats + ((size_t)(b * H + h) * T_slots + (t + g.slot_offset)) * NP;
    uint4 tmp[STAGE];
#pragma unroll
    for (int i = 0; i < STAGE; ++i) tmp[i] = src[min(tid + 64 * NW * i, NP - 1)];
#pragma unroll
    for (int i = 0; i < STAGE; ++i)
      if (tid + 64 * NW * i < NP) sm[tid + 64 * NW * i] = tmp[i];
  }
  __syncthreads();

  const int U = g.U;
  const size_t tok0 = ((size_t)b * g.T_in + t) * (size_t)U;
  const size_t fbase = (tok0 * H + h) * (size_t)D;
  const uint32_t rowbytes = (uint32_t)H * D * 2;
  const uint32_t nbytes = U > 0 ? (uint32_t)(U - 1) * rowbytes + D * 2 : 0;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(g.k + fbase, nbytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(g.v + fbase, nbytes);
  const __amdgpu_buffer_rsrc_t dkr = make_rsrc(g.dk + fbase, nbytes);
  const __amdgpu_buffer_rsrc_t dvr = make_rsrc(g.dv + fbase, nbytes);
  const uint32_t bbytes = U > 0 ? (uint32_t)(U - 1) * H * 2 + 2 : 0;
  const __amdgpu_buffer_rsrc_t br = make_rsrc(g.beta + tok0 * H + h, bbytes);
  const __amdgpu_buffer_rsrc_t dbr = make_rsrc(g.dbeta + tok0 * H + h, bbytes);

  const int n = lane & 15, q = lane >> 4;
  const uint32_t coff = (uint32_t)q * 16;  // bytes of channel 8 q in a row
  const int ntiles = (U + 31) / 32;

  struct Frag {
    bf16x8 k[2][KS], v[2][KS];
    uint16_t beta[2];
  };
  auto load = [&](int tile, Frag& f) {
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const uint32_t tok = (uint32_t)(tile * 32 + 16 * gi + n);
      const uint32_t ro = tok * rowbytes + coff;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) f.k[gi][ks] = __builtin_bit_cast(bf16x8, buf_load16(kr, ro + 64 * ks));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) f.v[gi][ks] = __builtin_bit_cast(bf16x8, buf_load16(vr, ro + 64 * ks));
      f.beta[gi] = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(br, tok * H * 2, 0, 0);
    }
  };
  // acc[gi] += plane w x operand of token group gi, over the k-steps
  auto chain = [&](f32x4 (&acc)[2][MT], int w, const bf16x8 (&op)[2][KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, sm[w * NF + (mt * KS + ks) * 64 + lane]);
        acc[0][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, op[0][ks], acc[0][mt], 0, 0, 0);
        acc[1][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, op[1][ks], acc[1][mt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // sum over the lane's channels 32 p + 8 q + j of x_j acc (acc[2p + j / 4][j % 4])
  auto dotacc = [&](const bf16x8 (&op)[KS], const f32x4 (&acc)[MT]) {
    float s = 0.f;
#pragma unroll
    for (int p = 0; p < KS; ++p) {
      const uint4 u = __builtin_bit_cast(uint4, op[p]);
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 2 * e;
        s += bf16_lo(w4[e]) * acc[2 * p + j / 4][j % 4] + bf16_hi(w4[e]) * acc[2 * p + (j + 1) / 4][(j + 1) % 4];
      }
    }
    return s;
  };

  auto process = [&](int tile, const Frag& f) {
    f32x4 gk[2][MT], bk[2][MT];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) gk[gi][mt] = bk[gi][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    chain(gk, GP_G_HI, f.k);  // G k
    chain(gk, GP_G_LO, f.k);
    chain(bk, GP_DB_HI, f.k);  // dB k
    chain(bk, GP_DB_LO, f.k);
    float bt[2];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      bt[gi] = bf16_to_f32(f.beta[gi]);
      float dot = 0.5f * dotacc(f.k[gi], gk[gi]) + dotacc(f.v[gi], bk[gi]);
      dot += __shfl_xor(dot, 16);
      dot += __shfl_xor(dot, 32);
      if (q == 0)
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(pack_bf16x2(dot, 0.f) & 0xffffu), dbr,
                                              (uint32_t)(tile * 32 + 16 * gi + n) * H * 2, 0, 0);
    }
    // out: beta * acc over channels 32 p + 8 q .. + 7 (m-tiles 2p, 2p + 1)
    auto emit = [&](const f32x4 (&acc)[2][MT], const __amdgpu_buffer_rsrc_t& dst) {
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const uint32_t ro = (uint32_t)(tile * 32 + 16 * gi + n) * rowbytes + coff;
        const float s = bt[gi];
#pragma unroll
        for (int p = 0; p < KS; ++p) {
          const f32x4 x = acc[gi][2 * p], y = acc[gi][2 * p + 1];
          buf_store16(make_uint4(pack_bf16x2(s * x[0], s * x[1]), pack_bf16x2(s * x[2], s * x[3]),
                                 pack_bf16x2(s * y[0], s * y[1]), pack_bf16x2(s * y[2], s * y[3])),
                      dst, ro + 64 * p);
        }
      }
    };
    emit(bk, dvr);              // dv = beta dB k
    chain(gk, GP_DBT_HI, f.v);  // G k + dB^T v
    emit(gk, dkr);              // dk = beta (G k + dB^T v)
  };

  // two operand sets: tile i + NW loads while tile i is multiplied
  Frag fa, fb;
  int tile = wave;
  if (tile < ntiles) load(tile, fa);
  for (; tile < ntiles; tile += 2 * NW) {
    if (tile + NW < ntiles) load(tile + NW, fb);
    process(tile, fa);
    if (tile + NW >= ntiles) break;
    if (tile + 2 * NW < ntiles) load(tile + 2 * NW, fa);
    process(tile + NW, fb);
  }
}

template <int D>
hipError_t backward_gram_d(const Problem& p, const BwdGramBuffers& w, hipStream_t s) {
  const unsigned nslots = (unsigned)(p.B * p.H * (p.T + 1));
  if constexpr (D >= 32)
    hipLaunchKernelGGL(pack_grad_mats16<D>, dim3(nslots), dim3(256), 0, s, w.dA, w.dB, static_cast<uint4*>(w.mats));
  else
    hipLaunchKernelGGL(pack_grad_mats<D>, dim3(nslots), dim3(256), 0, s, w.dA, w.dB, static_cast<uint4*>(w.mats));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  auto u16 = [](const void* x) { return static_cast<const uint16_t*>(x); };
  auto w16 = [](void* x) { return static_cast<uint16_t*>(x); };
  // every frame (the anchors' slots hold zero matrices, so their gradients are
  // written as zero), then the text frame from slot T
  const GradPart a{u16(w.k), u16(w.v), u16(w.beta), w16(w.dk), w16(w.dv), w16(w.dbeta), p.T, p.U, 0, p.T, 0};
  const GradPart c{u16(w.k_text), u16(w.v_text), u16(w.beta_text), w16(w.dk_text), w16(w.dv_text),
                   w16(w.dbeta_text), 1, p.L, 0, 1, p.T};
  const int nblk0 = p.B * p.T * p.H;
  const unsigned grid = (unsigned)(nblk0 + (p.L > 0 ? p.B * p.H : 0));
  // d >= 32: the 16 x 16 x 32 layout (16 rows per load and store instruction);
  // d = 16: the 32 x 32 x 16 layout.  Four waves, each prefetching its next tile
  // in registers.
  if constexpr (D >= 32)
    hipLaunchKernelGGL(gram_bwd16<D>, dim3(grid), dim3(256), 0, s, a, c, nblk0, static_cast<const uint4*>(w.mats),
                       p.H, p.T + 1);
  else
    hipLaunchKernelGGL((gram_bwd_bf16<D, 4, true>), dim3(grid), dim3(256), 0, s, a, c, nblk0,
                       static_cast<const uint4*>(w.mats), p.H, p.T + 1);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gain_grad_sum(const Problem& p, const float* gain_part, float* dgamma, int n, float scale,
                                hipStream_t s) {
  const int rows = p.B * p.T * p.H;
  switch (p.D) {
    case 16: hipLaunchKernelGGL(gain_grad_sum<16>, dim3(1), dim3(1024), 0, s, gain_part, dgamma, rows, n, scale); break;
    case 32: hipLaunchKernelGGL(gain_grad_sum<32>, dim3(1), dim3(1024), 0, s, gain_part, dgamma, rows, n, scale); break;
    case 64: hipLaunchKernelGGL(gain_grad_sum<64>, dim3(1), dim3(1024), 0, s, gain_part, dgamma, rows, n, scale); break;
    case 128: hipLaunchKernelGGL(gain_grad_sum<128>, dim3(1), dim3(1024), 0, s, gain_part, dgamma, rows, n, scale); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_backward_gram(const Problem& p, const BwdGramBuffers& w, hipStream_t s) {
  if (!p.bf16) return launch_backward_gram_f32(p, w, s);
  switch (p.D) {
    case 16: return backward_gram_d<16>(p, w, s);
    case 32: return backward_gram_d<32>(p, w, s);
    case 64: return backward_gram_d<64>(p, w, s);
    case 128: return backward_gram_d<128>(p, w, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vda
