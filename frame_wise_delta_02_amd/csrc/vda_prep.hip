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
#include <type_traits>

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

// DU: the caller's head width, D >= DU the power of two whose D / 8 lanes hold
// one token's channels (DU < D for the widths between the built ones: the
// lanes of channels DU .. D - 1 load zeros and store nothing).
template <int D, typename TIO, int DU = D>
__global__ __launch_bounds__(256) void prep_conv(const TIO* __restrict__ X, const float* __restrict__ ws,
                                                 const float* __restrict__ wt, TIO* __restrict__ Y,
                                                 int T, int gh, int gw, int H, int normalise,
                                                 float eps) {
  constexpr bool MASK = DU != D;
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
    if (MASK && c >= DU)
      sw[c][k] = 0.f;
    else
      sw[c][k] = (k < 25) ? ws[((size_t)h * DU + c) * 25 + k] : wt[((size_t)h * DU + c) * 5 + (k - 25)];
  }
  __syncthreads();

  const int cg = tid % CG, xr = tid / CG;
  const int ch = cg * 8;
  const bool live = !MASK || ch < DU;  // this lane's channels exist
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
          if (live && xx >= 0 && xx < gw) {
            const size_t row = (((size_t)b * T + ti) * U + (size_t)yy * gw + xx) * H + h;
            load8<D>(X + row * DU + ch, in[j]);
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
      if (live && x < gw) {
        const size_t row = (((size_t)b * T + t) * U + (size_t)y * gw + x) * H + h;
        store8(Y + row * DU + ch, out[i]);
      }
    }
  }
}

// The 768p-class path (bfloat16, d = 128): one workgroup owns a TY x TX tile of
// output positions of one (batch, head) and sweeps every frame in order, so each
// input frame's spatial convolution is computed once and the temporal taps are
// applied from a ring of the last five spatial results held in registers.
//   * Input frame ti's slab -- the tile plus a 2-token halo on every side,
//     (TY+4) x (TX+4) tokens x d channels in bfloat16 -- is staged in LDS,
//     double-buffered: the loads of frame ti+1 are in flight while frame ti is
//     convolved (zero outside the frame: the padding).
//   * Wave w owns a BY x BX block of positions; lane l owns channels 2l, 2l+1,
//     so every LDS read of a token is one conflict-free dword per lane, the 50
//     spatial and 10 temporal weights of the lane's channels sit in registers,
//     and the L2 norm over d is one wave reduction.
//   * After input frame ti, output frame ti-2 is complete: SiLU, the optional
//     L2 normalisation and a coalesced 256-byte store per token.
// Sum over the 64 lanes of a wave, in every lane: DPP within each row of 16
// (swap neighbours, swap pairs, mirror halves of 8, mirror the row), then the
// four row sums through readlane.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  v += dpp_f<0x140>(v);  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

constexpr int PTY = 8, PTX = 12;  // output tile
constexpr int PBY = 2, PBX = 6;   // block of one wave
constexpr int PWY = PTY / PBY, PWX = PTX / PBX;
constexpr int PNW = PWY * PWX;    // 8 waves
constexpr int PSY = PTY + 4, PSX = PTX + 4;  // slab tokens
constexpr int PBLK = PBY * PBX;   // positions per wave

template <int D>
__global__ __launch_bounds__(64 * PNW) void prep_conv_tile(const uint16_t* __restrict__ X,
                                                           const float* __restrict__ ws,
                                                           const float* __restrict__ wt,
                                                           uint16_t* __restrict__ Y, int B, int T, int gh,
                                                           int gw, int H, int normalise, float eps) {
  static_assert(D == 128, "one wave holds one token's channels, two per lane");
  constexpr int CG = D / 8;                 // 16-byte channel groups per token
  constexpr int SLAB = PSY * PSX * CG;      // 16-byte pieces per slab
  constexpr int PER = (SLAB + 64 * PNW - 1) / (64 * PNW);
  __shared__ uint4 slab[2][SLAB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ntx = (gw + PTX - 1) / PTX, nty = (gh + PTY - 1) / PTY;
  const int ntile = ntx * nty;
  // blockIdx -> (b, h, tile); with H divisible by 8 the tiles of one head share
  // an XCD (blockIdx % 8), so the halos re-read by neighbouring tiles meet in L2
  int bid = blockIdx.x, b, h, tile;
  if (H % 8 == 0) {
    const int xcd = bid % 8, j = bid / 8;
    tile = j % ntile;
    const int hq = j / ntile;  // (b, h / 8)
    h = (hq % (H / 8)) * 8 + xcd;
    b = hq / (H / 8);
  } else {
    tile = bid % ntile;
    h = (bid / ntile) % H;
    b = bid / (ntile * H);
  }
  const int y0 = (tile / ntx) * PTY, x0 = (tile % ntx) * PTX;
  const size_t U = (size_t)gh * gw;
  const size_t tokstride = (size_t)H * D;  // elements between consecutive tokens

  // this lane's weights: channels 2l, 2l+1
  float w_s[25][2], w_t[5][2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const size_t c = (size_t)h * D + 2 * lane + e;
#pragma unroll
    for (int k = 0; k < 25; ++k) w_s[k][e] = ws[c * 25 + k];
#pragma unroll
    for (int k = 0; k < 5; ++k) w_t[k][e] = wt[c * 5 + k];
  }

  // staging: piece e of the slab -> (slab row, slab col, channel group)
  uint4 stage[PER];
  auto load_slab = [&](int ti) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = tid + 64 * PNW * q;
      const int tok = e / CG, cg = e % CG;
      const int yy = y0 - 2 + tok / PSX, xx = x0 - 2 + tok % PSX;
      const bool ok = e < SLAB && ti < T && yy >= 0 && yy < gh && xx >= 0 && xx < gw;
      stage[q] = make_uint4(0u, 0u, 0u, 0u);
      if (ok)
        stage[q] = *reinterpret_cast<const uint4*>(
            X + (((size_t)b * T + ti) * U + (size_t)yy * gw + xx) * tokstride + (size_t)h * D + 8 * cg);
    }
  };
  auto put_slab = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = tid + 64 * PNW * q;
      if (e < SLAB) slab[buf][e] = stage[q];
    }
  };

  const int wy = wave / PWX, wx = wave % PWX;
  // spatial result of frame ti for this wave's block, ring slot ti % 5
  float ring[5][PBLK][2];
#pragma unroll
  for (int r = 0; r < 5; ++r)
#pragma unroll
    for (int p = 0; p < PBLK; ++p) ring[r][p][0] = ring[r][p][1] = 0.f;

  // spatial convolution of the staged frame into ring slot R
  auto spatial = [&](int buf, float (&sp)[PBLK][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < PBLK; ++p) sp[p][0] = sp[p][1] = 0.f;
    const uint32_t* sl = reinterpret_cast<const uint32_t*>(slab[buf]);
#pragma unroll
    for (int rr = 0; rr < PBY + 4; ++rr) {
      // input slab row PBY*wy + rr, columns PBX*wx .. PBX*wx + PBX + 3
      float in[PBX + 4][2];
#pragma unroll
      for (int c = 0; c < PBX + 4; ++c) {
        const int tok = (PBY * wy + rr) * PSX + PBX * wx + c;
        const uint32_t wd = sl[tok * (D / 2) + lane];
        in[c][0] = bf16_lo(wd);
        in[c][1] = bf16_hi(wd);
      }
#pragma unroll
      for (int i = 0; i < PBY; ++i) {
        const int a = rr - i;  // kernel row
        if (a < 0 || a > 4) continue;
#pragma unroll
        for (int cx = 0; cx < 5; ++cx)
#pragma unroll
          for (int j = 0; j < PBX; ++j)
#pragma unroll
            for (int e = 0; e < 2; ++e) sp[i * PBX + j][e] += w_s[a * 5 + cx][e] * in[j + cx][e];
      }
    }
  };
  // output frame t from the ring (slot of frame f = f % 5); SiLU, L2, store
  auto emit = [&](int t, auto slot_of) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < PBLK; ++p) {
      float v[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        float o = 0.f;
#pragma unroll
        for (int tau = 0; tau < 5; ++tau) o += w_t[tau][e] * ring[slot_of(tau)][p][e];
        // SiLU with the hardware reciprocal (about 1 ulp)
        v[e] = o * __builtin_amdgcn_rcpf(1.f + __expf(-o));
      }
      if (normalise) {
        const float r = __builtin_amdgcn_rsqf(wave_sum(v[0] * v[0] + v[1] * v[1]) + eps);
        v[0] *= r;
        v[1] *= r;
      }
      const int yy = y0 + PBY * wy + p / PBX, xx = x0 + PBX * wx + p % PBX;
      if (yy < gh && xx < gw)
        *reinterpret_cast<uint32_t*>(Y + (((size_t)b * T + t) * U + (size_t)yy * gw + xx) * tokstride +
                                     (size_t)h * D + 2 * lane) = pack_bf16x2(v[0], v[1]);
    }
  };

  load_slab(0);
  put_slab(0);
  __syncthreads();
  // frame step ti (ring slot R = ti % 5): stage ti+1, convolve ti, emit ti-2
  auto frame = [&](int ti, auto R) __attribute__((always_inline)) {
    constexpr int S = decltype(R)::value;
    load_slab(ti + 1);
    if (ti < T) spatial(ti & 1, ring[S]);
    else {
#pragma unroll
      for (int p = 0; p < PBLK; ++p) ring[S][p][0] = ring[S][p][1] = 0.f;
    }
    // frame f's slot is f % 5; output ti-2 reads frames ti-4 .. ti
    if (ti >= 2) emit(ti - 2, [](int tau) __attribute__((always_inline)) { return (S + 1 + tau) % 5; });
    put_slab((ti + 1) & 1);
    __syncthreads();
  };
  for (int ti = 0; ti < T + 2; ti += 5) {
    frame(ti, std::integral_constant<int, 0>());
    if (ti + 1 < T + 2) frame(ti + 1, std::integral_constant<int, 1>());
    if (ti + 2 < T + 2) frame(ti + 2, std::integral_constant<int, 2>());
    if (ti + 3 < T + 2) frame(ti + 3, std::integral_constant<int, 3>());
    if (ti + 4 < T + 2) frame(ti + 4, std::integral_constant<int, 4>());
  }
}

// q_hat = q / sqrt(|q|^2 + eps) per (token, head); one thread per 8 channels
// (D / 8 threads per row, those past the caller's DU channels idle).
template <int D, typename TIO, int DU = D>
__global__ __launch_bounds__(256) void prep_l2(const TIO* __restrict__ X, TIO* __restrict__ Y,
                                               size_t rows, float eps) {
  constexpr bool MASK = DU != D;
  const size_t g = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t row = g / (D / 8);
  const int ch = (int)(g % (D / 8)) * 8;
  const bool ok = row < rows && (!MASK || ch < DU);
  float x[8];
  if (ok) {
    load8<D>(X + row * DU + ch, x);
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
  if (ok) store8(Y + row * DU + ch, x);
}

template <int D, typename TIO, int DU = D>
hipError_t launch_prep_t(const Problem& p, int gh, int gw, const void* q, const void* k,
                         const void* v, const float* wk_s, const float* wk_t, const float* wv_s,
                         const float* wv_t, void* q_hat, void* k_hat, void* v_hat, hipStream_t s) {
  hipError_t e = hipSuccess;
  if constexpr (D == 128 && DU == D && sizeof(TIO) == 2) {
    const unsigned tiles = (unsigned)(((gh + PTY - 1) / PTY) * ((gw + PTX - 1) / PTX));
    const unsigned grid = (unsigned)(p.B * p.H) * tiles;
    hipLaunchKernelGGL(prep_conv_tile<D>, dim3(grid), dim3(64 * PNW), 0, s, static_cast<const uint16_t*>(k),
                       wk_s, wk_t, static_cast<uint16_t*>(k_hat), p.B, p.T, gh, gw, p.H, 1, p.l2_eps);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prep_conv_tile<D>, dim3(grid), dim3(64 * PNW), 0, s, static_cast<const uint16_t*>(v),
                       wv_s, wv_t, static_cast<uint16_t*>(v_hat), p.B, p.T, gh, gw, p.H, 0, p.l2_eps);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    const unsigned grid = (unsigned)(p.B * p.T * p.H * gh);
    hipLaunchKernelGGL((prep_conv<D, TIO, DU>), dim3(grid), dim3(256), 0, s, static_cast<const TIO*>(k),
                       wk_s, wk_t, static_cast<TIO*>(k_hat), p.T, gh, gw, p.H, 1, p.l2_eps);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prep_conv<D, TIO, DU>), dim3(grid), dim3(256), 0, s, static_cast<const TIO*>(v),
                       wv_s, wv_t, static_cast<TIO*>(v_hat), p.T, gh, gw, p.H, 0, p.l2_eps);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.qnorm) return hipSuccess;  // the readout normalises the query itself
  const size_t rows = (size_t)p.B * p.T * p.U * p.H;
  const size_t threads = rows * (D / 8);
  hipLaunchKernelGGL((prep_l2<D, TIO, DU>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     static_cast<const TIO*>(q), static_cast<TIO*>(q_hat), rows, p.l2_eps);
  return hipGetLastError();
}

template <int D, int DU = D>
hipError_t launch_prep_d(const Problem& p, int gh, int gw, const void* q, const void* k,
                         const void* v, const float* wk_s, const float* wk_t, const float* wv_s,
                         const float* wv_t, void* q_hat, void* k_hat, void* v_hat, hipStream_t s) {
  if (p.bf16)
    return launch_prep_t<D, uint16_t, DU>(p, gh, gw, q, k, v, wk_s, wk_t, wv_s, wv_t, q_hat, k_hat, v_hat, s);
  return launch_prep_t<D, float, DU>(p, gh, gw, q, k, v, wk_s, wk_t, wv_s, wv_t, q_hat, k_hat, v_hat, s);
}

}  // namespace

hipError_t launch_prep(const Problem& p, int gh, int gw, const void* q, const void* k,
                       const void* v, const float* wk_s, const float* wk_t, const float* wv_s,
                       const float* wv_t, void* q_hat, void* k_hat, void* v_hat, hipStream_t s) {
  // the prep works on the caller's tensors at the caller's width: a width
  // between the built ones runs the generic kernels with its last lanes idle
  switch (p.Du) {
    case 16: return launch_prep_d<16>(p, gh, gw, q, k, v, wk_s, wk_t, wv_s, wv_t, q_hat, k_hat, v_hat, s);
    case 32: return launch_prep_d<32>(p, gh, gw, q, k, v, wk_s, wk_t, wv_s, wv_t, q_hat, k_hat, v_hat, s);
    case 48: return launch_prep_d<64, 48>(p, gh, gw, q, k, v, wk_s, wk_t, wv_s, wv_t, q_hat, k_hat, v_hat, s);
    case 64: return launch_prep_d<64>(p, gh, gw, q, k, v, wk_s, wk_t, wv_s, wv_t, q_hat, k_hat, v_hat, s);
    case 80: return launch_prep_d<128, 80>(p, gh, gw, q, k, v, wk_s, wk_t, wv_s, wv_t, q_hat, k_hat, v_hat, s);
    case 96: return launch_prep_d<128, 96>(p, gh, gw, q, k, v, wk_s, wk_t, wv_s, wv_t, q_hat, k_hat, v_hat, s);
    case 112: return launch_prep_d<128, 112>(p, gh, gw, q, k, v, wk_s, wk_t, wv_s, wv_t, q_hat, k_hat, v_hat, s);
    case 128: return launch_prep_d<128>(p, gh, gw, q, k, v, wk_s, wk_t, wv_s, wv_t, q_hat, k_hat, v_hat, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vda
