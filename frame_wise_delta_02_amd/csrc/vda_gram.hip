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
// transposed: every loader thread reads 8 tokens x 8 channels (coalesced 16-byte
// loads along d), scales and rounds them, transposes the 8x8 block in registers
// and writes 8 rows of 16 bytes.  Rows are 128 bytes (64 tokens) with an XOR
// swizzle of the 16-byte chunk index so that both the transposed writes and
// the MFMA operand reads hit distinct banks.  Two LDS buffers overlap the next
// tile's global loads with the current tile's MFMAs.
//
// float32 inputs: v_mfma_f32_16x16x4f32 takes one token per lane, so tiles are
// staged in natural token-major order (rows padded by 16 floats).
#include "vda_internal.h"

namespace vda {
namespace {

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

template <int D>
__global__ __launch_bounds__(256, 1) void gram_bf16(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ beta, float* __restrict__ stats,
    int T_in, int U, int H, int t_first, int n_frames, int slot_offset, int T_slots) {
  constexpr int R = 2 * D;          // rows of [Z | W]^T
  constexpr int LG = R / 8;         // 16-byte channel groups per token
  constexpr int LOADERS = LG * 8;   // 8 token groups of 8 tokens
  constexpr int MT = R / 16, NT = D / 16;
  constexpr int MTW = (MT + 3) / 4;  // m-tiles per wave
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][R * 128];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int blk = blockIdx.x;
  const int h = blk % H;
  blk /= H;
  const int fi = blk % n_frames;
  const int b = blk / n_frames;
  const int t = t_first + fi;
  const size_t tok0 = ((size_t)b * T_in + t) * (size_t)U;

  const bool loader = tid < LOADERS;
  const int cg = tid % LG, tg = tid / LG;
  const uint16_t* src = (cg < D / 8) ? K : V;
  const int ch = (cg < D / 8) ? cg * 8 : (cg - D / 8) * 8;
  const int row0 = cg * 8;

  f32x4 acc[MTW][NT];
#pragma unroll
  for (int i = 0; i < MTW; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 reg0[8], reg1[8];
  uint32_t sb0[8], sb1[8];  // raw beta bits; bit 16 set when the token exists

  // Loads are branch-free: a token past the end of the frame (or a thread
  // that does not load) reads a valid row and is zeroed through its beta, so
  // the compiler can keep every load of a tile in flight at once.
  auto load = [&](uint4 (&reg)[8], uint32_t (&sb)[8], int u0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int u = u0 + tg * 8 + j;
      const bool ok = loader && u < U;
      const size_t row = (tok0 + (ok ? u : 0)) * (size_t)H + h;
      reg[j] = *reinterpret_cast<const uint4*>(src + row * D + ch);
      sb[j] = (uint32_t)beta[row] | (ok ? 0x10000u : 0u);
    }
  };

  auto store = [&](const uint4 (&reg)[8], const uint32_t (&sb)[8], int buf) {
    if (!loader) return;
    uint32_t w[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float s = (sb[j] & 0x10000u) ? __builtin_sqrtf(bf16_to_f32((uint16_t)sb[j])) : 0.f;
      const uint32_t x[4] = {reg[j].x, reg[j].y, reg[j].z, reg[j].w};
#pragma unroll
      for (int d = 0; d < 4; ++d) w[j][d] = pack_f16x2(bf16_lo(x[d]) * s, bf16_hi(x[d]) * s);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t o[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t a = w[2 * p][i >> 1], c = w[2 * p + 1][i >> 1];
        o[p] = (i & 1) ? ((a >> 16) | (c & 0xffff0000u)) : ((a & 0xffffu) | (c << 16));
      }
      const int r = row0 + i;
      *reinterpret_cast<uint4*>(lds[buf] + r * 128 + 16 * (tg ^ swz(r))) =
          make_uint4(o[0], o[1], o[2], o[3]);
    }
  };

  auto compute = [&](int buf) {
    const uint8_t* base = lds[buf];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int q = 4 * s + (lane >> 4);
      f16x8 afr[MTW];
#pragma unroll
      for (int mi = 0; mi < MTW; ++mi) {
        const int r = 16 * min(wave * MTW + mi, MT - 1) + (lane & 15);
        afr[mi] = *reinterpret_cast<const f16x8*>(base + r * 128 + 16 * (q ^ swz(r)));
      }
#pragma unroll
      for (int nj = 0; nj < NT; ++nj) {
        const int r = 16 * nj + (lane & 15);
        const f16x8 bfr = *reinterpret_cast<const f16x8*>(base + r * 128 + 16 * (q ^ swz(r)));
#pragma unroll
        for (int mi = 0; mi < MTW; ++mi)
          if (MT % 4 == 0 || wave * MTW + mi < MT)
            acc[mi][nj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(afr[mi], bfr, acc[mi][nj], 0, 0, 0);
      }
    }
  };

  // Software pipeline: tile i sits in LDS buffer i&1 while tiles i+1 and i+2
  // are in flight in the two register stages.
  const int ntile = (U + 63) / 64;
  if (ntile > 0) {
    load(reg0, sb0, 0);
    if (ntile > 1) load(reg1, sb1, 64);
    store(reg0, sb0, 0);
  }
  __syncthreads();
  for (int it = 0; it < ntile; it += 2) {
    if (it + 2 < ntile) load(reg0, sb0, (it + 2) * 64);
    compute(0);
    if (it + 1 < ntile) store(reg1, sb1, 1);
    __syncthreads();
    if (it + 1 >= ntile) break;
    if (it + 3 < ntile) load(reg1, sb1, (it + 3) * 64);
    compute(1);
    if (it + 2 < ntile) store(reg0, sb0, 0);
    __syncthreads();
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
  __syncthreads();
  for (int it = 0; it < ntile; ++it) {
    const bool more = it + 1 < ntile;
    if (more) load((it + 1) * TT);
    compute(it & 1);
    if (more) store((it + 1) & 1);
    __syncthreads();
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
    hipLaunchKernelGGL(gram_bf16<D>, dim3(grid), dim3(256), 0, s,
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
