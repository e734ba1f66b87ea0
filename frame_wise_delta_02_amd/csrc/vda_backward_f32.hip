// vda_backward_f32: the first and third stages of the VDA backward pass for
// float32 inputs (the second, on the float32 workspace, is shared with
// bfloat16).  The same derivatives as the bfloat16 stages ("Video DeltaNet"
// summary, onedev.kr/papers/80: the readout of "어떻게 동작하나", the
// epilogue of "무엇과 다른가", the frame statistics of "어떻게 쓰나"), in
// float32 throughout, on the vector ALU: the float32 workloads are small
// (tiny and stress clips) and ask for 1e-3, which bfloat16 operands would not
// give.
//
// Layout: a (frame, head) per workgroup, one d x d matrix (or two) of that
// unit in LDS with rows padded to d + 1 floats, so that a wave reading a row
// per lane and a wave reading a column per lane both hit distinct banks; each
// of the four waves takes one token at a time, lane l holding channels
// l, l + 64 (d = 128), its token's vectors shared through a per-wave LDS row.
#include "vda_internal.h"

namespace vda {
namespace {

__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + __expf(-x)); }

// Values and exchanges between the lanes of one wave, ordered by a wave
// barrier (the lanes of a wave pass vectors through LDS).
__device__ __forceinline__ void wave_sync() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_wave_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Sum over the wave's 64 lanes.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// Slot c < nc: S_q = wf F_{c-2} Diag(df) + wr R_{c+2} Diag(dr) (S_T/2 for a
// missing side; df, dr the decay bridge's products over chunks c - 1 and
// c + 1, or ones); slot nc (the anchors): S_T.  Plain float32 [d_v][d_k].
template <int D>
__global__ __launch_bounds__(256) void slot_states_f32(const float* __restrict__ s_text, const float* __restrict__ fwd,
                                                       const float* __restrict__ rev, const float* __restrict__ alpha,
                                                       float* __restrict__ out, int nc, int T, int H, int C,
                                                       int bridge) {
  __shared__ float dfw[D], drv[D];
  const int slot = blockIdx.x % (nc + 1);
  const int bh = blockIdx.x / (nc + 1);
  const int h = bh % H, b = bh / H;
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
  const float* ST = s_text + (size_t)bh * D * D;
  const float* Fp = nullptr;
  const float* Rp = nullptr;
  if (slot < nc) {
    if (slot >= 2) Fp = fwd + ((size_t)bh * nc + (slot - 2)) * D * D;
    if (slot + 2 <= nc - 1) Rp = rev + ((size_t)bh * nc + (slot + 2)) * D * D;
  }
  const float* Fs = Fp ? Fp : ST;
  const float* Rs = Rp ? Rp : ST;
  const float wf = Fp ? 1.f : 0.5f, wr = Rp ? 1.f : 0.5f;
  float* o = out + (size_t)blockIdx.x * D * D;
  for (int i = threadIdx.x; i < D * D; i += blockDim.x) {
    const int k = i % D;
    o[i] = wf * Fs[i] * dfw[k] + wr * Rs[i] * drv[k];
  }
}

constexpr int NW = 4;  // waves per workgroup

// Back through the epilogue and the readout, per token (file comment of
// vda_backward.hip): o = S_q q (q / |q| with QN), then with EPI
//   r = 1 / sqrt(mean o^2 + eps), n = o r, s = sigmoid(g), dn = dy gamma s,
//   dgate = dn n (1 - s), do = r (dn - n mean(dn n)),
// else do = dy; dq = S_q^T do (with QN back through q / |q|).  Writes dq,
// dgate and DO = do (do / |q| with QN, for dS_q against the raw query); with
// DGAIN the (frame, head)'s sums of dy s n into GP[blockIdx.x * D ..].
template <int D, bool EPI, bool GAMMA, bool QN, bool DGAIN>
__global__ __launch_bounds__(64 * NW) void readout_bwd_f32(
    const float* __restrict__ Q, const float* __restrict__ G, const float* __restrict__ DY,
    const float* __restrict__ w, const float* __restrict__ slots, float* __restrict__ DO, float* __restrict__ DG,
    float* __restrict__ DQ, float* __restrict__ GP, int T, int U, int H, int C, int nc, float eps, float l2eps) {
  constexpr int DS = D + 1;                    // padded row
  constexpr int R = D > 64 ? D / 64 : 1;       // channels per lane
  __shared__ float S[D * DS];
  __shared__ float vec[NW][2][D];              // q (then do) of the wave's token
  __shared__ float red[NW][D];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int blk = blockIdx.x;
  const int h = blk % H;
  blk /= H;
  const int t = blk % T;
  const int b = blk / T;
  const int slot = (t == 0 || t == T - 1) ? nc : t / C;
  const float* src = slots + ((size_t)(b * H + h) * (nc + 1) + slot) * D * D;
  for (int i = tid; i < D * D; i += 64 * NW) S[(i / D) * DS + i % D] = src[i];
  __syncthreads();

  float gsum[R];
#pragma unroll
  for (int r = 0; r < R; ++r) gsum[r] = 0.f;
  const size_t row0 = (((size_t)b * T + t) * U * H + h) * D;  // token u's row: row0 + u H D
  for (int u = wave; u < U; u += NW) {
    const size_t row = row0 + (size_t)u * H * D;
    float q[R], o[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int c = lane + 64 * r;
      q[r] = c < D ? Q[row + c] : 0.f;
      if (c < D) vec[wave][0][c] = q[r];
    }
    wave_sync();
    float qscale = 1.f;
    if constexpr (QN) {
      float ss = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) ss += q[r] * q[r];
      qscale = 1.f / sqrtf(wave_sum(ss) + l2eps);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = lane + 64 * r;
      float a = 0.f;
      if (i < D)
        for (int j = 0; j < D; ++j) a += S[i * DS + j] * vec[wave][0][j];
      o[r] = a * qscale;
    }
    float dov[R];
    if constexpr (EPI) {
      float gv[R], yv[R], gm[R], ss = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int c = lane + 64 * r;
        gv[r] = c < D ? G[row + c] : 0.f;
        yv[r] = c < D ? DY[row + c] : 0.f;
        gm[r] = (GAMMA && c < D) ? w[c] : 1.f;
        ss += o[r] * o[r];
      }
      const float rinv = 1.f / sqrtf(wave_sum(ss) / (float)D + eps);
      float n[R], sg[R], dn[R], dot = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        n[r] = o[r] * rinv;
        sg[r] = sigmoid_f(gv[r]);
        dn[r] = yv[r] * gm[r] * sg[r];
        dot += dn[r] * n[r];
        if constexpr (DGAIN) gsum[r] += yv[r] * sg[r] * n[r];
      }
      const float m = wave_sum(dot) / (float)D;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int c = lane + 64 * r;
        dov[r] = rinv * (dn[r] - n[r] * m);
        if (c < D) {
          DG[row + c] = dn[r] * n[r] * (1.f - sg[r]);
          DO[row + c] = qscale * dov[r];
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int c = lane + 64 * r;
        dov[r] = c < D ? DY[row + c] : 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int c = lane + 64 * r;
      if (c < D) vec[wave][1][c] = dov[r];
    }
    wave_sync();
    // dq_n = S_q^T do: lane j reads column j of S (consecutive across lanes)
    float dq[R], qd = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int j = lane + 64 * r;
      float a = 0.f;
      if (j < D)
        for (int i = 0; i < D; ++i) a += S[i * DS + j] * vec[wave][1][i];
      dq[r] = a;
      qd += q[r] * a;
    }
    if constexpr (QN) {
      // dq = (dq_n - q_n (q_n . dq_n)) / |q| with q_n = q / |q|
      const float c3 = qscale * qscale * qscale * wave_sum(qd);
#pragma unroll
      for (int r = 0; r < R; ++r) dq[r] = qscale * dq[r] - c3 * q[r];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int c = lane + 64 * r;
      if (c < D) DQ[row + c] = dq[r];
    }
    wave_sync();  // vec is rewritten by the next token
  }
  if constexpr (DGAIN) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int c = lane + 64 * r;
      if (c < D) red[wave][c] = gsum[r];
    }
    __syncthreads();
    if (tid < D) {
      float v = red[0][tid];
#pragma unroll
      for (int w2 = 1; w2 < NW; ++w2) v += red[w2][tid];
      GP[(size_t)blockIdx.x * D + tid] = v;
    }
  }
}

// dS_q(t) = sum over frame t's tokens of do q^T, [B, H, T, d_v, d_k]: thread
// (g, j) of D groups of 256 / D sums entries (g + (256 / D) k, j), the tokens
// staged 32 at a time.
template <int D>
__global__ __launch_bounds__(256) void state_adjoint_f32(const float* __restrict__ Q, const float* __restrict__ DO,
                                                         float* __restrict__ dsq, int T, int U, int H) {
  constexpr int NG = 256 / D, RPT = D / NG, TT = 32;
  __shared__ float qs[TT][D], ds[TT][D];
  const int tid = threadIdx.x, j = tid % D, g = tid / D;
  int blk = blockIdx.x;
  const int h = blk % H;
  blk /= H;
  const int t = blk % T;
  const int b = blk / T;
  const size_t row0 = (((size_t)b * T + t) * U * H + h) * D;
  float acc[RPT];
#pragma unroll
  for (int k = 0; k < RPT; ++k) acc[k] = 0.f;
  for (int u0 = 0; u0 < U; u0 += TT) {
    const int n = min(TT, U - u0);
    for (int i = tid; i < TT * D; i += 256) {
      const int uu = i / D, c = i % D;
      const size_t row = row0 + (size_t)(u0 + uu) * H * D + c;
      qs[uu][c] = uu < n ? Q[row] : 0.f;
      ds[uu][c] = uu < n ? DO[row] : 0.f;
    }
    __syncthreads();
    for (int uu = 0; uu < n; ++uu) {
      const float qj = qs[uu][j];
#pragma unroll
      for (int k = 0; k < RPT; ++k) acc[k] += ds[uu][g + NG * k] * qj;
    }
    __syncthreads();
  }
  float* o = dsq + (((size_t)b * H + h) * T + t) * D * D;
#pragma unroll
  for (int k = 0; k < RPT; ++k) o[(size_t)(g + NG * k) * D + j] = acc[k];
}

// One part of the third stage's launch: frames t_first .. t_first + n_frames - 1
// of tensors [B, T_in, U, H, d] (and beta [B, T_in, U, H]), gradients into the
// same layout; statistics-gradient slot t + slot_offset.
struct GradPartF {
  const float *k, *v, *beta;
  float *dk, *dv, *dbeta;
  int T_in, U, t_first, n_frames, slot_offset;
};

// Per token, with G = dA + dA^T and dB of its (frame, head) in LDS:
//   dk = beta (G k + dB^T v),  dv = beta dB k,  dbeta = k.(G k) / 2 + v.(dB k).
template <int D>
__global__ __launch_bounds__(64 * NW) void gram_bwd_f32(GradPartF part0, GradPartF part1, int nblk0,
                                                       const float* __restrict__ dA, const float* __restrict__ dB,
                                                       int H, int T_slots) {
  constexpr int DS = D + 1;
  constexpr int R = D > 64 ? D / 64 : 1;
  __shared__ float Gs[D * DS], Bs[D * DS];
  __shared__ float vec[NW][2][D];
  const bool second = (int)blockIdx.x >= nblk0;
  const GradPartF p = second ? part1 : part0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int blk = (int)blockIdx.x - (second ? nblk0 : 0);
  const int h = blk % H;
  blk /= H;
  const int f = blk % p.n_frames;
  const int b = blk / p.n_frames;
  const int t = p.t_first + f;
  const size_t m0 = (((size_t)b * H + h) * T_slots + t + p.slot_offset) * D * D;
  for (int i = tid; i < D * D; i += 64 * NW) {
    const int r = i / D, c = i % D;
    Gs[r * DS + c] = dA[m0 + i] + dA[m0 + (size_t)c * D + r];
    Bs[r * DS + c] = dB[m0 + i];
  }
  __syncthreads();
  const size_t tok0 = ((size_t)b * p.T_in + t) * p.U;
  for (int u = wave; u < p.U; u += NW) {
    const size_t tk = (tok0 + u) * H + h;  // token-head index
    const size_t row = tk * D;
    float k[R], v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int c = lane + 64 * r;
      k[r] = c < D ? p.k[row + c] : 0.f;
      v[r] = c < D ? p.v[row + c] : 0.f;
      if (c < D) {
        vec[wave][0][c] = k[r];
        vec[wave][1][c] = v[r];
      }
    }
    wave_sync();
    const float beta = p.beta[tk];
    float kgk = 0.f, vbk = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = lane + 64 * r;
      float gk = 0.f, bk = 0.f, btv = 0.f;
      if (i < D)
        for (int j = 0; j < D; ++j) {
          const float kj = vec[wave][0][j];
          gk += Gs[i * DS + j] * kj;           // (G k)_i, row i
          bk += Bs[i * DS + j] * kj;           // (dB k)_i, row i
          btv += Bs[j * DS + i] * vec[wave][1][j];  // (dB^T v)_i, column i
        }
      kgk += k[r] * gk;
      vbk += v[r] * bk;
      if (i < D) {
        p.dk[row + i] = beta * (gk + btv);
        p.dv[row + i] = beta * bk;
      }
    }
    const float db = 0.5f * wave_sum(kgk) + wave_sum(vbk);
    if (lane == 0) p.dbeta[tk] = db;
    wave_sync();
  }
}

}  // namespace

hipError_t launch_backward_readout_f32(const Problem& p, const float* q, const float* gate, const float* rms_weight,
                                       const float* dy, const float* s_text, const float* fwd, const float* rev,
                                       const float* alpha, float* slots, float* dout, float* dq, float* dgate,
                                       float* dsq, float* gain_part, float* dgamma, int gain_n, float gain_scale,
                                       hipStream_t s) {
  const auto go = [&](auto dd) -> hipError_t {
    constexpr int D = decltype(dd)::value;
    hipLaunchKernelGGL(slot_states_f32<D>, dim3((unsigned)(p.B * p.H * (p.nc + 1))), dim3(256), 0, s, s_text, fwd,
                       rev, alpha, slots, p.nc, p.T, p.H, p.C, p.bridge ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned grid = (unsigned)(p.B * p.T * p.H);
    auto launch = [&](auto epi, auto gm, auto qn, auto dg) {
      hipLaunchKernelGGL((readout_bwd_f32<D, decltype(epi)::value, decltype(gm)::value, decltype(qn)::value,
                                          decltype(dg)::value>),
                         dim3(grid), dim3(64 * NW), 0, s, q, gate, dy, rms_weight, slots, dout, dgate, dq, gain_part,
                         p.T, p.U, p.H, p.C, p.nc, p.rms_eps, p.l2_eps);
    };
    using Y = std::true_type;
    using N = std::false_type;
    if (!p.epilogue)
      launch(N(), N(), N(), N());
    else if (dgamma)
      rms_weight ? (p.qnorm ? launch(Y(), Y(), Y(), Y()) : launch(Y(), Y(), N(), Y()))
                 : (p.qnorm ? launch(Y(), N(), Y(), Y()) : launch(Y(), N(), N(), Y()));
    else
      rms_weight ? (p.qnorm ? launch(Y(), Y(), Y(), N()) : launch(Y(), Y(), N(), N()))
                 : (p.qnorm ? launch(Y(), N(), Y(), N()) : launch(Y(), N(), N(), N()));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (dgamma && (e = launch_gain_grad_sum(p, gain_part, dgamma, gain_n, gain_scale, s)) != hipSuccess) return e;
    // dS_q(t) = sum do q^T against the query the readout read (raw with QN)
    hipLaunchKernelGGL(state_adjoint_f32<D>, dim3(grid), dim3(256), 0, s, q, p.epilogue ? dout : dy, dsq, p.T, p.U,
                       p.H);
    return hipGetLastError();
  };
  switch (p.D) {
    case 16: return go(std::integral_constant<int, 16>());
    case 32: return go(std::integral_constant<int, 32>());
    case 64: return go(std::integral_constant<int, 64>());
    case 128: return go(std::integral_constant<int, 128>());
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_backward_gram_f32(const Problem& p, const BwdGramBuffers& w, hipStream_t s) {
  auto f = [](const void* x) { return static_cast<const float*>(x); };
  auto g = [](void* x) { return static_cast<float*>(x); };
  // every frame (the anchors' slots hold zero matrices, so their gradients are
  // written as zero), then the text frame from slot T
  const GradPartF a{f(w.k), f(w.v), f(w.beta), g(w.dk), g(w.dv), g(w.dbeta), p.T, p.U, 0, p.T, 0};
  const GradPartF c{f(w.k_text), f(w.v_text), f(w.beta_text), g(w.dk_text), g(w.dv_text), g(w.dbeta_text),
                    1, p.L, 0, 1, p.T};
  const int nblk0 = p.B * p.T * p.H;
  const unsigned grid = (unsigned)(nblk0 + (p.L > 0 ? p.B * p.H : 0));
  const auto go = [&](auto dd) -> hipError_t {
    constexpr int D = decltype(dd)::value;
    hipLaunchKernelGGL(gram_bwd_f32<D>, dim3(grid), dim3(64 * NW), 0, s, a, c, nblk0, w.dA, w.dB, p.H, p.T + 1);
    return hipGetLastError();
  };
  switch (p.D) {
    case 16: return go(std::integral_constant<int, 16>());
    case 32: return go(std::integral_constant<int, 32>());
    case 64: return go(std::integral_constant<int, 64>());
    case 128: return go(std::integral_constant<int, 128>());
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vda
