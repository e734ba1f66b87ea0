// vda_readout: o = (S_fwd + S_rev) q for every token, fused with RMSNorm over d_v
// and the elementwise sigmoid output gate.
//
// Readout o_t = S_t(fwd) q_t + S_t(rev) q_t ("Video DeltaNet" summary,
// onedev.kr/papers/80, section "어떻게 동작하나"); the linear branch's output
// then passes RMS normalisation and its own sigmoid output gate (section
// "무엇과 다른가"; the VDN-H3 write-up, discuss.pytorch.kr, puts the
// elementwise sigmoid gate after RMSNorm).
//
// Every token of a frame reads the same d_v x d_k state (its chunk's
// F_{c-2} + R_{c+2}, or S_T for the two anchor frames), packed beforehand into
// matrix-core operand order by the gather kernel.  A workgroup of 8 waves stages
// that state in LDS once and streams the frame's tokens in 32-token tiles, one
// tile per wave at a time, computing O^T = S Q^T on 32x32 matrix-core tiles:
//   * every global access (Q, gate, output) is a coalesced row access, lanes on
//     consecutive 16-byte chunks of a few token rows; a per-wave LDS tile
//     (XOR-swizzled, conflict-free both ways) turns rows into operand order
//     and the results back into rows;
//   * B operand = Q^T: each lane holds 8 channels of one token;
//   * A operand = S, with its rows permuted so that after the product each lane
//     holds d_v/2 *consecutive* outputs of one token.  RMSNorm is then a sum in
//     registers plus one cross-half lane swap, and the gate and output move
//     between registers and the LDS tile as whole 16-byte chunks.
// bfloat16 path: S = S_hi + S_lo (two bf16 parts, ~16 significant bits) on
// v_mfma_f32_32x32x16_bf16, so the fp32 state is not truncated to 8 bits.
// float32 path: v_mfma_f32_32x32x2f32 with the fp32 state.
// Query L2 normalisation may be fused here (the flag VDN_VDA_QUERY_L2): the
// readout before RMSNorm is linear in q, so the kernel multiplies the raw
// query's products by 1/sqrt(|q|^2 + l2_eps), the squared norm summed in
// float32 from the operand registers (each half-wave holds half the channels
// of a token, the other half one lane swap away).
#include "vda_internal.h"

namespace vda {
namespace {

__device__ __forceinline__ float sigmoid(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

template <int D, bool EPI, bool GAMMA, bool QN>
__global__ __launch_bounds__(512, 1) void readout_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ G, const float* __restrict__ w,
    const uint4* __restrict__ rstates, uint16_t* __restrict__ O, int T, int U, int H, int C,
    int nc, float eps, float l2eps) {
  constexpr int NW = 8;              // waves per workgroup
  constexpr int DP = D < 32 ? 32 : D;
  constexpr int HALF = DP / 2;       // outputs per lane
  constexpr int MT = DP / 32;
  constexpr int KS = D / 16;
  constexpr int NF = MT * KS * 64;   // 16-byte fragments per part (hi or lo)
  constexpr int NG = HALF / 8;       // 16-byte gate / output vectors per lane
  constexpr int CH = D / 8;          // 16-byte chunks per token row
  constexpr int RPI = 64 / CH;       // token rows covered by one coalesced wave access
  constexpr int NL = 32 / RPI;       // coalesced accesses per 32-token tile
  constexpr int SWM = (CH < 8 ? CH : 8) - 1;             // swizzle: XOR mask on the chunk
  constexpr int SWS = CH >= 8 ? 0 : (CH == 4 ? 1 : 2);   // log2 of the rows sharing 128 bytes
  constexpr int STAGE = (2 * NF + 64 * NW - 1) / (64 * NW);
  __shared__ uint4 sfrag[2 * NF];
  __shared__ uint4 xbuf[NW][32 * CH];  // per wave: one 32-token tile, row-major, swizzled
  __shared__ float4 sgam[GAMMA ? DP / 4 : 1];  // RMSNorm gain, padded with ones to DP

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int blk = blockIdx.x;
  const int h = blk % H;
  blk /= H;
  const int t = blk % T;
  const int b = blk / T;
  const int slot = (t == 0 || t == T - 1) ? nc : t / C;
  {
    const uint4* src = rstates + ((size_t)(b * H + h) * (nc + 1) + slot) * 2 * NF;
    uint4 tmp[STAGE];  // all staging loads in flight before the first LDS write
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

  // Buffer descriptors over this frame and head: tokens past U read zero and
  // their stores are dropped, so the tail tile and the prefetch past the last
  // tile need no clamping.
  const size_t fbase = (((size_t)b * T + t) * U * H + h) * (size_t)D;
  const uint32_t rowbytes = (uint32_t)H * D * 2;
  const uint32_t nbytes = U > 0 ? (uint32_t)(U - 1) * rowbytes + D * 2 : 0;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(Q + fbase, nbytes);
  const __amdgpu_buffer_rsrc_t orr = make_rsrc(O + fbase, nbytes);
  const __amdgpu_buffer_rsrc_t gr = make_rsrc(EPI ? G + fbase : Q + fbase, nbytes);

  // Q, the gate and the output are each touched once: non-temporal accesses,
  // so they do not evict the packed states that every frame of a chunk re-reads
  // (and the statistics the next stages read) from L2 and the Infinity Cache.
  // Global traffic is coalesced: access i of a tile covers token rows
  // RPI*i .. RPI*i + RPI-1, consecutive lanes on consecutive 16-byte chunks.
  // The per-wave LDS tile turns rows into matrix-core operand order and back.
  const int lrow = lane / CH, lch = lane % CH;
  const uint32_t loff = (uint32_t)lrow * rowbytes + 16 * lch;
  auto pos = [](int r, int c) { return r * CH + (c ^ ((r >> SWS) & SWM)); };

  const int n = lane & 31, half = lane >> 5;
  const int dv0 = HALF * half;                 // first output channel of this lane
  const bool owns = dv0 < D;                   // false only for the padding half at d = 16
  const int ntiles = (U + 31) / 32;
  const int per_wave = (ntiles + NW - 1) / NW;
  const int steps = (per_wave + 1) & ~1;       // even: the loop has no exit in the middle
  uint4* X = xbuf[wave];

  auto fetch = [&](int tile, uint4 (&qv)[NL], uint4 (&gv)[NL]) {
    const uint32_t tb = (uint32_t)tile * 32 * rowbytes + loff;
#pragma unroll
    for (int i = 0; i < NL; ++i) qv[i] = buf_load16_nt(qr, tb + (uint32_t)(RPI * i) * rowbytes);
    if constexpr (EPI) {
#pragma unroll
      for (int i = 0; i < NL; ++i) gv[i] = buf_load16_nt(gr, tb + (uint32_t)(RPI * i) * rowbytes);
    }
  };
  // LDS accesses of one wave execute in order; these fences only keep the
  // compiler from moving them across one another.
  auto fence = [] {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_wave_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };

  auto process = [&](int tile, const uint4 (&qv)[NL], const uint4 (&gv)[NL]) {
    // Q^T operand: lane (n, half) takes channels 8 * ((CH/2) * half + ks) .. + 7 of token n
#pragma unroll
    for (int i = 0; i < NL; ++i) X[pos(RPI * i + lrow, lch)] = qv[i];
    fence();
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, X[pos(n, (CH / 2) * half + ks)]);
    fence();
    // 1 / |q| of token n (raw query, fused L2 normalisation); 1 otherwise
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
    // the gate rows wait in the same LDS tile until the epilogue
    if constexpr (EPI) {
#pragma unroll
      for (int i = 0; i < NL; ++i) X[pos(RPI * i + lrow, lch)] = gv[i];
    }
    f32x16 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{0.f};
    // k-step outer; the fence keeps the scheduler from hoisting every operand
    // read of the tile at once (which would not fit the register budget)
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
    fence();
    // lane holds o[dv0 + 16*mt + r] of token n in acc[mt][r]; epilogue in place
    if constexpr (EPI) {
      float ss = 0.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) ss += acc[mt][r] * acc[mt][r];
      ss += __shfl_xor(ss, 32);
      // o = qscale * acc, so mean(o^2) = qscale^2 * ss / D
      const float rinv = __builtin_amdgcn_rsqf(ss * (qscale * qscale) / (float)D + eps) * qscale;
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        const uint4 gq = owns ? X[pos(n, dv0 / 8 + i)] : make_uint4(0, 0, 0, 0);
        const uint32_t g4[4] = {gq.x, gq.y, gq.z, gq.w};
        float gm[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
        if constexpr (GAMMA) {  // gains of channels dv0 + 8i .. + 7, read where they are used
          const float4 a = sgam[(dv0 + 8 * i) / 4], c = sgam[(dv0 + 8 * i) / 4 + 1];
          gm[0] = a.x; gm[1] = a.y; gm[2] = a.z; gm[3] = a.w;
          gm[4] = c.x; gm[5] = c.y; gm[6] = c.z; gm[7] = c.w;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j0 = 8 * i + 2 * e, j1 = j0 + 1;
          acc[j0 / 16][j0 % 16] *= rinv * gm[2 * e] * sigmoid(bf16_lo(g4[e]));
          acc[j1 / 16][j1 % 16] *= rinv * gm[2 * e + 1] * sigmoid(bf16_hi(g4[e]));
        }
      }
    } else if constexpr (QN) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mt][r] *= qscale;
    }
    // outputs back to rows in the same LDS tile (each lane overwrites only the
    // gate chunks it has read), then out as coalesced row stores
    if (owns) {
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        const int m = (8 * i) / 16, r = (8 * i) % 16;
        X[pos(n, dv0 / 8 + i)] =
            make_uint4(pack_bf16x2(acc[m][r], acc[m][r + 1]), pack_bf16x2(acc[m][r + 2], acc[m][r + 3]),
                       pack_bf16x2(acc[m][r + 4], acc[m][r + 5]), pack_bf16x2(acc[m][r + 6], acc[m][r + 7]));
      }
    }
    fence();
    const uint32_t tb = (uint32_t)tile * 32 * rowbytes + loff;
#pragma unroll
    for (int i = 0; i < NL; ++i) buf_store16_nt(X[pos(RPI * i + lrow, lch)], orr, tb + (uint32_t)(RPI * i) * rowbytes);
    fence();
  };

  // two register sets: tile i + NW is in flight while tile i is multiplied
  uint4 qa[NL], qb[NL], ga[NL], gb[NL];
  fetch(wave, qa, ga);
  for (int k = 0; k < steps; k += 2) {
    const int tile = wave + NW * k;
    fetch(tile + NW, qb, gb);
    process(tile, qa, ga);
    fetch(tile + 2 * NW, qa, ga);
    process(tile + NW, qb, gb);
  }
}

template <int D>
__global__ __launch_bounds__(256, 2) void readout_f32(
    const float* __restrict__ Q, const float* __restrict__ G, const float* __restrict__ w,
    const float4* __restrict__ rstates, float* __restrict__ O, int T, int U, int H, int C, int nc,
    int epilogue, int qnorm, float eps, float l2eps) {
  constexpr int DP = D < 32 ? 32 : D;
  constexpr int HALF = DP / 2;
  constexpr int MT = DP / 32;
  constexpr int KQ = D / 8;         // float4 groups of k-steps (one channel per half per step)
  constexpr int NF = MT * KQ * 64;
  constexpr int NO = HALF < D ? HALF : D;
  __shared__ float4 sfrag[NF];
  __shared__ float sgam[DP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int blk = blockIdx.x;
  const int h = blk % H;
  blk /= H;
  const int t = blk % T;
  const int b = blk / T;
  const int slot = (t == 0 || t == T - 1) ? nc : t / C;
  {
    constexpr int STAGE = (NF + 255) / 256;
    const float4* src = rstates + ((size_t)(b * H + h) * (nc + 1) + slot) * NF;
    float4 tmp[STAGE];
#pragma unroll
    for (int i = 0; i < STAGE; ++i) tmp[i] = src[min(tid + 256 * i, NF - 1)];
#pragma unroll
    for (int i = 0; i < STAGE; ++i)
      if (tid + 256 * i < NF) sfrag[tid + 256 * i] = tmp[i];
    for (int i = tid; i < DP; i += 256) sgam[i] = (w && i < D) ? w[i] : 1.f;
  }
  __syncthreads();

  const int n = lane & 31, half = lane >> 5;
  const int dv0 = HALF * half;
  const int nout = (dv0 < D) ? NO : 0;
  const size_t row_base = ((size_t)b * T + t) * (size_t)U;
  const int ntiles = (U + 31) / 32;
  for (int tile = wave; tile < ntiles; tile += 4) {
    const int u = tile * 32 + n;
    const bool valid = u < U;
    const size_t row = ((row_base + (valid ? u : 0)) * H + h) * (size_t)D;
    float4 qv[KQ];
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq) qv[kq] = *reinterpret_cast<const float4*>(Q + row + (D / 2) * half + 4 * kq);
    float qscale = 1.f;  // 1 / |q| under the fused query normalisation
    if (qnorm) {
      float qs = 0.f;
#pragma unroll
      for (int kq = 0; kq < KQ; ++kq)
        qs += qv[kq].x * qv[kq].x + qv[kq].y * qv[kq].y + qv[kq].z * qv[kq].z + qv[kq].w * qv[kq].w;
      qs += __shfl_xor(qs, 32);
      qscale = 1.f / __builtin_sqrtf(qs + l2eps);
    }
    f32x16 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{0.f};
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const float4 a = sfrag[(mt * KQ + kq) * 64 + lane];
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, qv[kq].x, acc[mt], 0, 0, 0);
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, qv[kq].y, acc[mt], 0, 0, 0);
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, qv[kq].z, acc[mt], 0, 0, 0);
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, qv[kq].w, acc[mt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (epilogue) {
      float ss = 0.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) ss += acc[mt][r] * acc[mt][r];
      ss += __shfl_xor(ss, 32);
      const float rinv = qscale / __builtin_sqrtf(ss * (qscale * qscale) / (float)D + eps);
      const float* gp = G + row + (nout ? dv0 : 0);
#pragma unroll
      for (int i = 0; i < HALF / 4; ++i) {
        if (4 * i < NO) {
          const float4 g = *reinterpret_cast<const float4*>(gp + 4 * i);
          const float gg[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = 4 * i + e;
            acc[j / 16][j % 16] *= rinv * sgam[dv0 + j] * sigmoid(gg[e]);
          }
        }
      }
    } else if (qnorm) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mt][r] *= qscale;
    }
    if (valid) {
#pragma unroll
      for (int i = 0; i < HALF / 4; ++i)
        if (4 * i < nout) {
          const int m = (4 * i) / 16, r = (4 * i) % 16;
          *reinterpret_cast<float4*>(O + row + dv0 + 4 * i) =
              make_float4(acc[m][r], acc[m][r + 1], acc[m][r + 2], acc[m][r + 3]);
        }
    }
  }
}

template <int D, bool EPI, bool GAMMA, bool QN>
void launch_readout_bf16(const Problem& p, const void* q, const void* gate, const float* w,
                         const void* rstates, void* out, hipStream_t s) {
  hipLaunchKernelGGL((readout_bf16<D, EPI, GAMMA, QN>), dim3((unsigned)(p.B * p.T * p.H)), dim3(512), 0, s,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(gate), w,
                     static_cast<const uint4*>(rstates), static_cast<uint16_t*>(out), p.T, p.U, p.H, p.C,
                     p.nc, p.rms_eps, p.l2_eps);
}

template <int D, bool QN>
void launch_readout_q(const Problem& p, const void* q, const void* gate, const float* w,
                      const void* rstates, void* out, hipStream_t s) {
  if (p.epilogue && w)
    launch_readout_bf16<D, true, true, QN>(p, q, gate, w, rstates, out, s);
  else if (p.epilogue)
    launch_readout_bf16<D, true, false, QN>(p, q, gate, w, rstates, out, s);
  else
    launch_readout_bf16<D, false, false, QN>(p, q, gate, w, rstates, out, s);
}

template <int D>
hipError_t launch_readout_d(const Problem& p, const void* q, const void* gate, const float* w,
                            const void* rstates, void* out, hipStream_t s) {
  if (p.bf16 && p.qnorm)
    launch_readout_q<D, true>(p, q, gate, w, rstates, out, s);
  else if (p.bf16)
    launch_readout_q<D, false>(p, q, gate, w, rstates, out, s);
  else
    hipLaunchKernelGGL(readout_f32<D>, dim3((unsigned)(p.B * p.T * p.H)), dim3(256), 0, s,
                       static_cast<const float*>(q), static_cast<const float*>(gate), w,
                       static_cast<const float4*>(rstates), static_cast<float*>(out), p.T, p.U,
                       p.H, p.C, p.nc, p.epilogue ? 1 : 0, p.qnorm ? 1 : 0, p.rms_eps, p.l2_eps);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_readout(const Problem& p, const void* q, const void* gate, const float* rms_weight,
                          const void* rstates, void* out, hipStream_t s) {
  switch (p.D) {
    case 16: return launch_readout_d<16>(p, q, gate, rms_weight, rstates, out, s);
    case 32: return launch_readout_d<32>(p, q, gate, rms_weight, rstates, out, s);
    case 64: return launch_readout_d<64>(p, q, gate, rms_weight, rstates, out, s);
    case 128: return launch_readout_d<128>(p, q, gate, rms_weight, rstates, out, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vda
