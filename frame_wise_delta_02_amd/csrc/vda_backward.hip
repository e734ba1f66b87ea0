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
//  * dS_q: the frame-statistics kernel in its PLAIN mode on (q, do).
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

// Back through the epilogue: o recomputed as the forward readout computes it,
// then dgate and do per token (see the file comment).  4 waves, each streaming
// 32-token tiles; per wave two LDS tiles (q then dy then do; gate then dgate).
template <int D, bool GAMMA>
__global__ __launch_bounds__(256, 1) void readout_bwd_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ G, const uint16_t* __restrict__ DY,
    const float* __restrict__ w, const uint4* __restrict__ rstates, uint16_t* __restrict__ DO,
    uint16_t* __restrict__ DG, int T, int U, int H, int C, int nc, float eps) {
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
  constexpr int STAGE = (2 * NF + 64 * NW - 1) / (64 * NW);
  __shared__ uint4 sfrag[2 * NF];
  __shared__ uint4 xq[NW][32 * CH];  // q rows, then dy rows, then do rows
  __shared__ uint4 xg[NW][32 * CH];  // gate rows, then dgate rows
  __shared__ float4 sgam[GAMMA ? DP / 4 : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int blk = blockIdx.x;
  const int h = blk % H;
  blk /= H;
  const int t = blk % T;
  const int b = blk / T;
  const int slot = (t == 0 || t == T - 1) ? nc : t / C;
  {
    const uint4* src = rstates + ((size_t)(b * H + h) * (nc + 1) + slot) * 2 * NF;
    uint4 tmp[STAGE];
#pragma unroll
    for (int i = 0; i < STAGE; ++i) tmp[i] = src[min(tid + 64 * NW * i, 2 * NF - 1)];
#pragma unroll
    for (int i = 0; i < STAGE; ++i)
      if (tid + 64 * NW * i < 2 * NF) sfrag[tid + 64 * NW * i] = tmp[i];
    if constexpr (GAMMA) {
      if (tid < DP) reinterpret_cast<float*>(sgam)[tid] = tid < D ? w[tid] : 1.f;
    }
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
    // lane holds o[dv0 + 16 mt + r] of token n in acc[mt][r]
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
      if constexpr (GAMMA) {
        const float4 a = sgam[(dv0 + 8 * i) / 4], c = sgam[(dv0 + 8 * i) / 4 + 1];
        gm[0] = a.x; gm[1] = a.y; gm[2] = a.z; gm[3] = a.w;
        gm[4] = c.x; gm[5] = c.y; gm[6] = c.z; gm[7] = c.w;
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
    // pass 2: do and dgate, written over the chunks just read
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
        }
        XQ[pos(n, dv0 / 8 + i)] = make_uint4(dow[0], dow[1], dow[2], dow[3]);
        XG[pos(n, dv0 / 8 + i)] = make_uint4(dgw[0], dgw[1], dgw[2], dgw[3]);
      }
    }
    fence();
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      buf_store16(XQ[pos(RPI * i + lrow, lch)], dor, tb + (uint32_t)(RPI * i) * rowbytes);
      buf_store16(XG[pos(RPI * i + lrow, lch)], dgr, tb + (uint32_t)(RPI * i) * rowbytes);
    }
    fence();
  };

  uint4 qv[NL];
  fetch_q(wave, qv);
  for (int k = 0; k < per_wave; ++k) process(wave + NW * k, qv);
}

template <int D>
hipError_t backward_readout_d(const Problem& p, const void* q, const void* gate, const float* rms_weight,
                              const void* dy, const void* rstates, const float* s_text, const float* fwd, const float* rev,
                              const float* alpha, void* rstates_t, void* dout, void* dq, void* dgate,
                              float* dsq, hipStream_t s) {
  hipLaunchKernelGGL(pack_states_t<D>, dim3((unsigned)(p.B * p.H * (p.nc + 1))), dim3(256), 0, s, s_text, fwd,
                     rev, alpha, static_cast<uint4*>(rstates_t), p.nc, p.T, p.H, p.C, p.bridge ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const void* do_ = dy;
  if (p.epilogue) {
    const unsigned grid = (unsigned)(p.B * p.T * p.H);
    if (rms_weight)
      hipLaunchKernelGGL((readout_bwd_bf16<D, true>), dim3(grid), dim3(256), 0, s,
                         static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(gate),
                         static_cast<const uint16_t*>(dy), rms_weight, static_cast<const uint4*>(rstates),
                         static_cast<uint16_t*>(dout), static_cast<uint16_t*>(dgate), p.T, p.U, p.H, p.C, p.nc,
                         p.rms_eps);
    else
      hipLaunchKernelGGL((readout_bwd_bf16<D, false>), dim3(grid), dim3(256), 0, s,
                         static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(gate),
                         static_cast<const uint16_t*>(dy), rms_weight, static_cast<const uint4*>(rstates),
                         static_cast<uint16_t*>(dout), static_cast<uint16_t*>(dgate), p.T, p.U, p.H, p.C, p.nc,
                         p.rms_eps);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    do_ = dout;
  }
  // dq = S_q^T do: the forward readout, raw, on the transposed states
  Problem raw = p;
  raw.epilogue = false;
  raw.qnorm = false;
  e = launch_readout(raw, do_, nullptr, nullptr, rstates_t, dq, s);
  if (e != hipSuccess) return e;
  // dS_q(t) = do_t^T q_t for every frame
  return launch_gram_plain(p, q, do_, dsq, s);
}

}  // namespace

hipError_t launch_backward_readout(const Problem& p, const void* q, const void* gate, const float* rms_weight,
                                   const void* dy, const void* rstates, const float* s_text, const float* fwd, const float* rev,
                                   const float* alpha, void* rstates_t, void* dout, void* dq, void* dgate,
                                   float* dsq, hipStream_t s) {
  if (!p.bf16) return hipErrorInvalidValue;
  switch (p.D) {
    case 16: return backward_readout_d<16>(p, q, gate, rms_weight, dy, rstates, s_text, fwd, rev, alpha, rstates_t, dout, dq, dgate, dsq, s);
    case 32: return backward_readout_d<32>(p, q, gate, rms_weight, dy, rstates, s_text, fwd, rev, alpha, rstates_t, dout, dq, dgate, dsq, s);
    case 64: return backward_readout_d<64>(p, q, gate, rms_weight, dy, rstates, s_text, fwd, rev, alpha, rstates_t, dout, dq, dgate, dsq, s);
    case 128: return backward_readout_d<128>(p, q, gate, rms_weight, dy, rstates, s_text, fwd, rev, alpha, rstates_t, dout, dq, dgate, dsq, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vda
