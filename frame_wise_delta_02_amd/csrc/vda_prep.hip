// vda_prep: the linear branch's feature preparation.
//
// K and V pass a separable short convolution -- a depthwise 5x5 spatial filter
// on the latent token grid, then a 5-tap temporal filter -- and SiLU; Q and K are
// L2-normalised; the linear branch uses no rotary embedding ("Video DeltaNet"
// summary, onedev.kr/papers/80, section "무엇과 다른가").  Readings taken
// where the page is silent: per-channel weights with no bias, cross-correlation
// orientation, zero padding 2 on every side of rows, columns and frames, and
// centred temporal taps (t-2 .. t+2) because the model attends in both
// directions.
//
// One workgroup produces one grid row of one frame of one head: every thread
// owns 8 consecutive channels (one 16-byte vector) of a run of consecutive
// tokens in that row.  For each of the 5 input frames and 5 kernel rows it
// loads the run plus its 2-token halo once and applies the 5 column taps from
// registers, accumulating the spatial result in fp32, then folds it into the
// temporal sum.  The D/8 threads that share a token sit in adjacent lanes, so
// the L2 norm over d is a 16-lane shuffle reduction fused before the store.
#include "vda_internal.h"

namespace vda {
namespace {

constexpr int XPT = 6;  // tokens per thread along a grid row

template <int D, typename TIO>
__device__ __forceinline__ void load8(const TIO* p, float (&x)[8]) {
  if constexpr (sizeof(TIO) == 2) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_lo(w[i]);
      x[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

template <typename TIO>
__device__ __forceinline__ void store8(TIO* p, const float (&y)[8]) {
  if constexpr (sizeof(TIO) == 2) {
    *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                                              pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7]));
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(y[0], y[1], y[2], y[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(y[4], y[5], y[6], y[7]);
  }
}

// Sum over the D/8 adjacent lanes that hold one token's channels.
template <int D>
__device__ __forceinline__ float token_sum(float v) {
#pragma unroll
  for (int m = 1; m < D / 8; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

template <int D, typename TIO>
__global__ __launch_bounds__(256) void prep_conv(const TIO* __restrict__ X, const float* __restrict__ ws,
                                                 const float* __restrict__ wt, TIO* __restrict__ Y,
                                                 int T, int gh, int gw, int H, int normalise,
                                                 float eps) {
  constexpr int CG = D / 8;     // channel groups (threads per token)
  constexpr int NX = 256 / CG;  // token runs per workgroup
  __shared__ float sw[D][32];   // per channel: 25 spatial taps, then 5 temporal taps

  int blk = blockIdx.x;
  const int y = blk % gh;
  blk /= gh;
  const int h = blk % H;
  blk /= H;
  const int t = blk % T;
  const int b = blk / T;
  const int tid = threadIdx.x;
  for (int i = tid; i < D * 30; i += 256) {
    const int c = i / 30, k = i % 30;
    sw[c][k] = (k < 25) ? ws[((size_t)h * D + c) * 25 + k] : wt[((size_t)h * D + c) * 5 + (k - 25)];
  }
  __syncthreads();

  const int cg = tid % CG, xr = tid / CG;
  const int ch = cg * 8;
  const size_t U = (size_t)gh * gw;
  for (int xb = 0; xb < gw; xb += NX * XPT) {
    const int x0 = xb + xr * XPT;
    float out[XPT][8];
#pragma unroll
    for (int i = 0; i < XPT; ++i)
#pragma unroll
      for (int c = 0; c < 8; ++c) out[i][c] = 0.f;
    for (int tau = 0; tau < 5; ++tau) {
      const int ti = t + tau - 2;
      if (ti < 0 || ti >= T) continue;
      float sp[XPT][8];
#pragma unroll
      for (int i = 0; i < XPT; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c) sp[i][c] = 0.f;
      for (int a = 0; a < 5; ++a) {
        const int yy = y + a - 2;
        if (yy < 0 || yy >= gh) continue;
        float in[XPT + 4][8];
#pragma unroll
        for (int j = 0; j < XPT + 4; ++j) {
          const int xx = x0 + j - 2;
          if (xx >= 0 && xx < gw) {
            const size_t row = (((size_t)b * T + ti) * U + (size_t)yy * gw + xx) * H + h;
            load8<D>(X + row * D + ch, in[j]);
          } else {
#pragma unroll
            for (int c = 0; c < 8; ++c) in[j][c] = 0.f;
          }
        }
#pragma unroll
        for (int cc = 0; cc < 5; ++cc)
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const float wv = sw[ch + c][a * 5 + cc];
#pragma unroll
            for (int i = 0; i < XPT; ++i) sp[i][c] += wv * in[i + cc][c];
          }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float wv = sw[ch + c][25 + tau];
#pragma unroll
        for (int i = 0; i < XPT; ++i) out[i][c] += wv * sp[i][c];
      }
    }
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float v = out[i][c];
        out[i][c] = v / (1.f + __expf(-v));
        ss += out[i][c] * out[i][c];
      }
      if (normalise) {
        ss = token_sum<D>(ss);
        const float r = 1.f / __builtin_sqrtf(ss + eps);
#pragma unroll
        for (int c = 0; c < 8; ++c) out[i][c] *= r;
      }
      const int x = x0 + i;
      if (x < gw) {
        const size_t row = (((size_t)b * T + t) * U + (size_t)y * gw + x) * H + h;
        store8(Y + row * D + ch, out[i]);
      }
    }
  }
}

// q_hat = q / sqrt(|q|^2 + eps) per (token, head); one thread per 8 channels.
template <int D, typename TIO>
__global__ __launch_bounds__(256) void prep_l2(const TIO* __restrict__ X, TIO* __restrict__ Y,
                                               size_t rows, float eps) {
  const size_t g = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t row = g / (D / 8);
  const int ch = (int)(g % (D / 8)) * 8;
  const bool ok = row < rows;
  float x[8];
  if (ok) {
    load8<D>(X + row * D + ch, x);
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = 0.f;
  }
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) ss += x[c] * x[c];
  ss = token_sum<D>(ss);
  const float r = 1.f / __builtin_sqrtf(ss + eps);
#pragma unroll
  for (int c = 0; c < 8; ++c) x[c] *= r;
  if (ok) store8(Y + row * D + ch, x);
}

template <int D, typename TIO>
hipError_t launch_prep_t(const Problem& p, int gh, int gw, const void* q, const void* k,
                         const void* v, const float* wk_s, const float* wk_t, const float* wv_s,
                         const float* wv_t, void* q_hat, void* k_hat, void* v_hat, hipStream_t s) {
  const unsigned grid = (unsigned)(p.B * p.T * p.H * gh);
  hipLaunchKernelGGL((prep_conv<D, TIO>), dim3(grid), dim3(256), 0, s, static_cast<const TIO*>(k),
                     wk_s, wk_t, static_cast<TIO*>(k_hat), p.T, gh, gw, p.H, 1, p.l2_eps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((prep_conv<D, TIO>), dim3(grid), dim3(256), 0, s, static_cast<const TIO*>(v),
                     wv_s, wv_t, static_cast<TIO*>(v_hat), p.T, gh, gw, p.H, 0, p.l2_eps);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t rows = (size_t)p.B * p.T * p.U * p.H;
  const size_t threads = rows * (D / 8);
  hipLaunchKernelGGL((prep_l2<D, TIO>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     static_cast<const TIO*>(q), static_cast<TIO*>(q_hat), rows, p.l2_eps);
  return hipGetLastError();
}

template <int D>
hipError_t launch_prep_d(const Problem& p, int gh, int gw, const void* q, const void* k,
                         const void* v, const float* wk_s, const float* wk_t, const float* wv_s,
                         const float* wv_t, void* q_hat, void* k_hat, void* v_hat, hipStream_t s) {
  if (p.bf16)
    return launch_prep_t<D, uint16_t>(p, gh, gw, q, k, v, wk_s, wk_t, wv_s, wv_t, q_hat, k_hat, v_hat, s);
  return launch_prep_t<D, float>(p, gh, gw, q, k, v, wk_s, wk_t, wv_s, wv_t, q_hat, k_hat, v_hat, s);
}

}  // namespace

hipError_t launch_prep(const Problem& p, int gh, int gw, const void* q, const void* k,
                       const void* v, const float* wk_s, const float* wk_t, const float* wv_s,
                       const float* wv_t, void* q_hat, void* k_hat, void* v_hat, hipStream_t s) {
  switch (p.D) {
    case 16: return launch_prep_d<16>(p, gh, gw, q, k, v, wk_s, wk_t, wv_s, wv_t, q_hat, k_hat, v_hat, s);
    case 32: return launch_prep_d<32>(p, gh, gw, q, k, v, wk_s, wk_t, wv_s, wv_t, q_hat, k_hat, v_hat, s);
    case 64: return launch_prep_d<64>(p, gh, gw, q, k, v, wk_s, wk_t, wv_s, wv_t, q_hat, k_hat, v_hat, s);
    case 128: return launch_prep_d<128>(p, gh, gw, q, k, v, wk_s, wk_t, wv_s, wv_t, q_hat, k_hat, v_hat, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vda
