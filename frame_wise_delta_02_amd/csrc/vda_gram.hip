// vda_gram: per-frame key correlation and value-key write of Video Delta Attention.
//
// For every (batch, frame, head): A_t = K_t^T Diag(beta_t) K_t and
// B_t = V_t^T Diag(beta_t) K_t over the U tokens of the frame ("Video DeltaNet"
// summary, onedev.kr/papers/80, section "어떻게 쓰나").  Both come out of one
// contraction: with Z = sqrt(beta) K and W = sqrt(beta) V (row-scaled per token),
//     [A_t ; B_t] = [Z | W]^T Z,
// a (2d x d) result over U tokens.  Scaling both sides by sqrt(beta) keeps A_t a
// true Gram matrix (symmetric positive semidefinite) after rounding, so I + A_t
// always has a Cholesky factor.
//
// bfloat16 inputs: the contraction runs on v_mfma_f32_16x16x32_f16 with fp32
// accumulation.  The scaled operands sqrt(beta) k and sqrt(beta) v are rounded
// to IEEE half, not bfloat16: the inputs are exact in either, but the products
// keep 11 significant bits instead of 8 at the same matrix-core rate on gfx950
// (keys are unit vectors, so |sqrt(beta) k| <= sqrt(beta); a value entry with
// |sqrt(beta) v| beyond 65504 would overflow the half range).
// The token axis is the contraction axis but is the strided axis in memory
// ([.., U, H, d] layout), so each 64-token tile is staged through LDS
// transposed: every loader thread reads 4 tokens x 8 channels (coalesced 16-byte
// loads along d; K and V come from different waves), scales and rounds them,
// transposes the 4x8 block in registers and writes 8 rows of 8 bytes.  Rows are
// 128 bytes (64 tokens) with an XOR swizzle of the 16-byte chunk index so that
// the MFMA operand reads hit distinct banks.  Eight waves split the (2d x d)
// output 4 x 2, so each holds 64 accumulators; two LDS buffers and two register
// stages keep two tiles of loads in flight behind the current tile's MFMAs.
//
// float32 inputs: v_mfma_f32_16x16x4f32 takes one token per lane, so tiles are
// staged in natural token-major order (rows padded by 16 floats).
#include "vda_internal.h"

namespace vda {
namespace {

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

template <int D>
__global__ __launch_bounds__(512, 1) void gram_bf16(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ beta, float* __restrict__ stats,
    int T_in, int U, int H, int t_first, int n_frames, int slot_offset, int T_slots) {
  constexpr int R = 2 * D;          // rows of [Z | W]^T
  constexpr int CGT = D / 8;        // 16-byte channel groups per token and tensor
  constexpr int PER_T = CGT * 16;   // loader threads per tensor: 16 groups of 4 tokens
  constexpr int MT = R / 16, NT = D / 16;
  constexpr int WM = MT >= 4 ? 4 : MT, WN = NT >= 2 ? 2 : 1;  // wave grid over output tiles
  constexpr int MTW = MT / WM, NTW = NT / WN;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][R * 128];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int blk = blockIdx.x;
  const int h = blk % H;
  blk /= H;
  const int fi = blk % n_frames;
  const int b = blk / n_frames;
  const int t = t_first + fi;
  const size_t tok0 = ((size_t)b * T_in + t) * (size_t)U;

  // loader role: PER_T threads read K and PER_T read V, each 4 consecutive
  // tokens x 8 channels per tile.  Buffer loads
  // over this frame and head return zero past the last token, so the tail tile
  // and the prefetch past the end need no clamping: a zero beta zeroes the token.
  // even waves load K, odd waves V (readfirstlane: the choice, and with it the
  // buffer descriptor, is provably wave-uniform and lives in scalar registers)
  const int which = __builtin_amdgcn_readfirstlane(wave & 1);
  const int local = (wave >> 1) * 64 + lane;
  const bool loader = local < PER_T;
  const int cg = local % CGT, tg = (local / CGT) & 15;
  const uint32_t rowbytes = (uint32_t)H * D * 2;  // bytes between consecutive tokens
  const uint32_t xbytes = U > 0 ? (uint32_t)(U - 1) * rowbytes + D * 2 : 0;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc((which ? V : K) + (tok0 * H + h) * (size_t)D, xbytes);
  const __amdgpu_buffer_rsrc_t br =
      make_rsrc(beta + tok0 * H + h, U > 0 ? (uint32_t)(U - 1) * H * 2 + 2 : 0);
  const uint32_t xoff0 = (loader ? (uint32_t)(tg * 4) * rowbytes : xbytes) + cg * 16;
  const uint32_t boff0 = (loader ? (uint32_t)(tg * 4) : (uint32_t)U) * H * 2;
  const int rowbase = which * D + cg * 8;  // first LDS row this thread writes

  const int wm = wave % WM, wn = (wave / WM) % WN;
  const bool mma = wave < WM * WN;

  f32x4 acc[MTW][NTW];
#pragma unroll
  for (int i = 0; i < MTW; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 reg0[4], reg1[4];
  uint32_t sb0[4], sb1[4];  // raw beta bits (zero past the last token)
  const int ntile = (U + 63) / 64;

  auto load = [&](uint4 (&reg)[4], uint32_t (&sb)[4], int it) {
    const uint32_t xo = xoff0 + (uint32_t)(it * 64) * rowbytes;
    const uint32_t bo = boff0 + (uint32_t)(it * 64) * H * 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      reg[j] = buf_load16(xr, xo + j * rowbytes);
      sb[j] = __builtin_amdgcn_raw_buffer_load_b16(br, bo + j * H * 2, 0, 0);
    }
  };

  // scale by sqrt(beta), round to half, transpose 4 tokens x 8 channels, and
  // write one 8-byte piece (4 tokens) to each of 8 LDS rows
  auto store = [&](const uint4 (&reg)[4], const uint32_t (&sb)[4], int buf) {
    if (!loader) return;
    uint32_t w[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float sc = __builtin_amdgcn_sqrtf(bf16_to_f32((uint16_t)sb[j]));
      const uint32_t x[4] = {reg[j].x, reg[j].y, reg[j].z, reg[j].w};
#pragma unroll
      for (int d = 0; d < 4; ++d) w[j][d] = pack_f16x2(bf16_lo(x[d]) * sc, bf16_hi(x[d]) * sc);
    }
    const int q = tg >> 1, hb = (tg & 1) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t o[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const uint32_t a = w[2 * p][i >> 1], c = w[2 * p + 1][i >> 1];
        o[p] = (i & 1) ? ((a >> 16) | (c & 0xffff0000u)) : ((a & 0xffffu) | (c << 16));
      }
      const int r = rowbase + i;
      *reinterpret_cast<uint2*>(lds[buf] + r * 128 + 16 * (q ^ swz(r)) + hb) = make_uint2(o[0], o[1]);
    }
  };

  auto compute = [&](int buf) {
    if (!mma) return;
    const uint8_t* base = lds[buf];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int q = 4 * s + (lane >> 4);
      f16x8 afr[MTW];
#pragma unroll
      for (int mi = 0; mi < MTW; ++mi) {
        const int r = 16 * (wm * MTW + mi) + (lane & 15);
        afr[mi] = *reinterpret_cast<const f16x8*>(base + r * 128 + 16 * (q ^ swz(r)));
      }
#pragma unroll
      for (int nj = 0; nj < NTW; ++nj) {
        const int r = 16 * (wn * NTW + nj) + (lane & 15);
        const f16x8 bfr = *reinterpret_cast<const f16x8*>(base + r * 128 + 16 * (q ^ swz(r)));
#pragma unroll
        for (int mi = 0; mi < MTW; ++mi)
          acc[mi][nj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(afr[mi], bfr, acc[mi][nj], 0, 0, 0);
      }
    }
  };

  // Software pipeline: tile i sits in LDS buffer i&1 while tiles i+1 and i+2
  // are in flight in the two register stages.
  // The trip count is rounded up to even so the loop has no exit in the middle;
  // a tile wholly past the end loads zeros without touching memory.
  load(reg0, sb0, 0);
  load(reg1, sb1, 1);
  store(reg0, sb0, 0);
  lds_barrier();
  for (int it = 0; it < ntile; it += 2) {
    load(reg0, sb0, it + 2);
    compute(0);
    store(reg1, sb1, 1);
    lds_barrier();
    load(reg1, sb1, it + 3);
    compute(1);
    store(reg0, sb0, 0);
    lds_barrier();
  }

  if (mma) {
    float* out = stats + ((size_t)(b * H + h) * T_slots + (t + slot_offset)) * (size_t)(R * D);
#pragma unroll
    for (int mi = 0; mi < MTW; ++mi)
#pragma unroll
      for (int nj = 0; nj < NTW; ++nj)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          out[(16 * (wm * MTW + mi) + 4 * (lane >> 4) + r) * D + 16 * (wn * NTW + nj) + (lane & 15)] =
              acc[mi][nj][r];
  }
}

template <int D>
__global__ __launch_bounds__(256, 2) void gram_f32(
    const float* __restrict__ K, const float* __restrict__ V, const float* __restrict__ beta,
    float* __restrict__ stats, int T_in, int U, int H, int t_first, int n_frames,
    int slot_offset, int T_slots) {
  constexpr int R = 2 * D;
  constexpr int TT = 16;           // tokens per tile
  constexpr int LD = R + 16;       // padded floats per token row
  constexpr int UNITS = TT * R / 4;  // float4 units per tile
  constexpr int PER = (UNITS + 255) / 256;
  constexpr int MT = R / 16, NT = D / 16;
  constexpr int MTW = (MT + 3) / 4;
  __shared__ __attribute__((aligned(16))) float lds[2][TT * LD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int blk = blockIdx.x;
  const int h = blk % H;
  blk /= H;
  const int fi = blk % n_frames;
  const int b = blk / n_frames;
  const int t = t_first + fi;
  const size_t tok0 = ((size_t)b * T_in + t) * (size_t)U;

  f32x4 acc[MTW][NT];
#pragma unroll
  for (int i = 0; i < MTW; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  float4 reg[PER];
  float sb[PER];
  auto load = [&](int u0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int unit = tid + 256 * i;
      const int tok = (unit % UNITS) / (R / 4), c4 = unit % (R / 4);
      const int u = u0 + tok;
      const bool ok = unit < UNITS && u < U;
      const float* src = (c4 < D / 4) ? K : V;
      const int ch = (c4 % (D / 4)) * 4;
      const size_t row = (tok0 + (ok ? u : 0)) * (size_t)H + h;
      reg[i] = *reinterpret_cast<const float4*>(src + row * D + ch);
      const float bv = beta[row];
      sb[i] = ok ? bv : 0.f;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int unit = tid + 256 * i;
      if (unit < UNITS) {
        const int tok = unit / (R / 4), c4 = unit % (R / 4);
        const float s = __builtin_sqrtf(sb[i]);
        float4 x = reg[i];
        x.x *= s;
        x.y *= s;
        x.z *= s;
        x.w *= s;
        *reinterpret_cast<float4*>(&lds[buf][tok * LD + 4 * c4]) = x;
      }
    }
  };
  auto compute = [&](int buf) {
    const float* base = lds[buf];
#pragma unroll
    for (int ks = 0; ks < TT / 4; ++ks) {
      const float* rowp = base + (4 * ks + (lane >> 4)) * LD + (lane & 15);
      float bfr[NT];
#pragma unroll
      for (int nj = 0; nj < NT; ++nj) bfr[nj] = rowp[16 * nj];
#pragma unroll
      for (int mi = 0; mi < MTW; ++mi) {
        const int m = wave * MTW + mi;
        if (m < MT) {
          const float a = rowp[16 * m];
#pragma unroll
          for (int nj = 0; nj < NT; ++nj)
            acc[mi][nj] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bfr[nj], acc[mi][nj], 0, 0, 0);
        }
      }
    }
  };

  const int ntile = (U + TT - 1) / TT;
  if (ntile > 0) {
    load(0);
    store(0);
  }
  lds_barrier();
  for (int it = 0; it < ntile; ++it) {
    const bool more = it + 1 < ntile;
    if (more) load((it + 1) * TT);
    compute(it & 1);
    if (more) store((it + 1) & 1);
    lds_barrier();
  }

  float* out = stats + ((size_t)(b * H + h) * T_slots + (t + slot_offset)) * (size_t)(R * D);
#pragma unroll
  for (int mi = 0; mi < MTW; ++mi) {
    const int m = wave * MTW + mi;
    if (m < MT) {
#pragma unroll
      for (int nj = 0; nj < NT; ++nj)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          out[(16 * m + 4 * (lane >> 4) + r) * D + 16 * nj + (lane & 15)] = acc[mi][nj][r];
    }
  }
}

template <int D>
hipError_t launch_gram_d(const Problem& p, const void* k, const void* v, const void* beta,
                         int T_in, int U_in, int t_first, int n_frames, int slot_offset,
                         float* stats, hipStream_t s) {
  const unsigned grid = (unsigned)(p.B * n_frames * p.H);
  if (p.bf16) {
    hipLaunchKernelGGL(gram_bf16<D>, dim3(grid), dim3(512), 0, s,
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                       static_cast<const uint16_t*>(beta), stats, T_in, U_in, p.H, t_first,
                       n_frames, slot_offset, p.T + 1);
  } else {
    hipLaunchKernelGGL(gram_f32<D>, dim3(grid), dim3(256), 0, s,
                       static_cast<const float*>(k), static_cast<const float*>(v),
                       static_cast<const float*>(beta), stats, T_in, U_in, p.H, t_first,
                       n_frames, slot_offset, p.T + 1);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gram(const Problem& p, const void* k, const void* v, const void* beta,
                       int T_in, int U_in, int t_first, int n_frames, int slot_offset,
                       float* stats, hipStream_t s) {
  if (n_frames <= 0) return hipSuccess;
  switch (p.D) {
    case 16: return launch_gram_d<16>(p, k, v, beta, T_in, U_in, t_first, n_frames, slot_offset, stats, s);
    case 32: return launch_gram_d<32>(p, k, v, beta, T_in, U_in, t_first, n_frames, slot_offset, stats, s);
    case 64: return launch_gram_d<64>(p, k, v, beta, T_in, U_in, t_first, n_frames, slot_offset, stats, s);
    case 128: return launch_gram_d<128>(p, k, v, beta, T_in, U_in, t_first, n_frames, slot_offset, stats, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vda
