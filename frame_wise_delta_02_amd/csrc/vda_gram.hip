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
// (keys are unit vectors, so |sqrt(beta) k| <= sqrt(beta)).  A unit whose
// operands leave the half range (|sqrt(beta) v| > 65504, which bfloat16 values
// allow) shows non-finite sums; it is then contracted again on operands scaled
// by powers of two, undone exactly in float32 (the recovery after the main loop).
// The token axis is the contraction axis but is the strided axis in memory
// ([.., U, H, d] layout), so each 64-token tile is staged through LDS
// transposed, one row per channel (128 bytes = 64 tokens, the 16-byte chunk
// index XOR-swizzled so that matrix-core operand reads hit distinct banks).
// The workgroup is split by role, one wave of each role per SIMD, so that the
// conversion work of one overlaps the matrix work of the other:
//   * 4 producer waves (2 on K, 2 on V) read coalesced token rows, each thread
//     d/16 tokens x 8 channels, scale by sqrt(beta) and round to half; pairing
//     two tokens of one channel in each packed conversion gives the transposed
//     row piece directly, written as one 16-byte LDS store at d = 128;
//   * 4 consumer waves run the MFMAs, each holding a (2d/4 x d) output block.
// Two register stages keep two tiles of loads in flight ahead of the tile
// being written, and two LDS buffers let the consumers read one tile while
// the producers write the next; one LDS barrier per tile separates them.
//
// float32 inputs: v_mfma_f32_16x16x4f32 takes one token per lane, so tiles are
// staged in natural token-major order (rows padded by 16 floats).
//
// PLAIN mode (the backward pass): V_t^T K_t only, with no beta, of two
// bfloat16 tensors used as they are (the operands stay bfloat16, the product
// runs on v_mfma_f32_16x16x32_bf16), written as one d_v x d_k slot per frame;
// the waves that would form A_t stay idle.  The backward pass forms the
// adjoint of the state a frame's queries read, dS = dO_t^T Q_t, this way.
#include <type_traits>

#include "vda_internal.h"

namespace vda {
namespace {

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// 2^-e with m 2^-e < 2^14 for m >= 2^14 (so scaled half operands stay far from
// 65504 and their products far from the float32 range), else 1
__device__ __forceinline__ float range_scale(float m) {
  if (!(m >= 16384.f)) return 1.f;
  const int E = ((__float_as_int(m) >> 23) & 0xff) - 127;  // floor(log2 m)
  const int e = min(E - 13, 125);
  return __int_as_float((127 - e) << 23);
}

// One part of a launch: frames t_first .. t_first + n_frames - 1 of inputs laid
// out [B, T_in, U, H, d], written to stats slots t + slot_offset.
template <typename TIO>
struct GramArgs {
  const TIO* K;
  const TIO* V;
  const TIO* beta;
  int T_in, U, t_first, n_frames, slot_offset;
};

template <int D, bool PLAIN = false>
__global__ __launch_bounds__(512, 1) void gram_bf16(GramArgs<uint16_t> part0, GramArgs<uint16_t> part1,
                                                    int nblk0, float* __restrict__ stats, int H,
                                                    int T_slots) {
  // blocks 0 .. nblk0-1 run part 0 (the video frames), the rest part 1 (the
  // text frame, short: it fills the last round of the video blocks)
  const bool second = (int)blockIdx.x >= nblk0;
  const GramArgs<uint16_t> g = second ? part1 : part0;
  const uint16_t* __restrict__ K = g.K;
  const uint16_t* __restrict__ V = g.V;
  const uint16_t* __restrict__ beta = g.beta;
  const int T_in = g.T_in, U = g.U, t_first = g.t_first, n_frames = g.n_frames, slot_offset = g.slot_offset;
  constexpr int R = 2 * D;          // rows of [Z | W]^T
  constexpr int CGT = D / 8;        // 16-byte channel groups per token
  constexpr int TPT = CGT / 2;      // tokens per producer thread and tile (128 threads per tensor)
  constexpr int MT = R / 16, NT = D / 16;
  constexpr int WM = MT >= 4 ? 4 : MT;  // consumer waves, each MT/WM row tiles x all NT column tiles
  constexpr int MTW = MT / WM;
  constexpr int NS = 2;             // producer register stages
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][R * 128];
  // range recovery (see below): set when a consumer's sums are not finite
  __shared__ int s_flag;
  __shared__ float s_max[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (tid == 0) s_flag = 0;  // ordered before any use by the main loop's barriers
  // block decode kept in scalar registers: the buffer descriptors built from it
  // must be provably wave-uniform
  int blk = (int)blockIdx.x - (second ? nblk0 : 0);
  const int h = sgpr(blk % H);
  blk /= H;
  const int fi = sgpr(blk % n_frames);
  const int b = sgpr(blk / n_frames);
  const int t = t_first + fi;
  const size_t tok0 = ((size_t)b * T_in + t) * (size_t)U;
  // tiles processed: a multiple of the stage count, so the loops below have no
  // exit in the middle; tiles wholly past the end are zero and touch no memory
  const int nstep = ((U + 63) / 64 + NS - 1) / NS * NS;

  if (wave < 4) {
    // ---- producers ----------------------------------------------------------
    // K and V are streamed once, with non-temporal loads (measured 0.65 ->
    // 0.58 ms at 768p): the beta lines that all heads of a frame share, and the
    // statistics the solve and scan read next, keep their place in the caches.
    // Buffer loads over this frame and head return zero past the last token, so
    // the tail tile and the loads past the end need no clamping: a zero beta
    // zeroes the token.  The tensor choice, and with it the buffer descriptor,
    // is wave-uniform.
    const int which = wave >> 1;
    const int local = (wave & 1) * 64 + lane;
    const int cg = local % CGT, tq = local / CGT;
    const int tok = TPT * tq;  // first of this thread's TPT consecutive tokens in the tile
    const uint32_t rowbytes = (uint32_t)H * D * 2;  // bytes between consecutive tokens
    const uint32_t xbytes = U > 0 ? (uint32_t)(U - 1) * rowbytes + D * 2 : 0;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc((which ? V : K) + (tok0 * H + h) * (size_t)D, xbytes);
    const __amdgpu_buffer_rsrc_t br =
        make_rsrc(PLAIN ? K : beta + tok0 * H + h, PLAIN || U <= 0 ? 0u : (uint32_t)(U - 1) * H * 2 + 2);
    const uint32_t xoff0 = (uint32_t)tok * rowbytes + cg * 16;
    // Each producer wave covers 32 consecutive tokens of a tile, so one beta load
    // per lane (lanes l and l+32 read the same token) and one square root serve
    // the wave; a thread takes its tokens' sqrt(beta) from lanes tl .. tl+TPT-1.
    const uint32_t boff0 = (uint32_t)(32 * (wave & 1) + (lane & 31)) * H * 2;
    const int tl = TPT * (lane / CGT);  // this thread's first token within the wave's 32
    // this thread writes channels 8cg .. 8cg+7 (rows), tokens tok .. tok+TPT-1
    const int row0 = which * D + 8 * cg;
    const int q = tok / 8, hb = 2 * (tok % 8);

    uint4 x[NS][TPT];
    uint32_t sb[NS];  // raw beta bits of token 32 * (wave & 1) + (lane & 31)
    auto load = [&](int s, int it) {
      const uint32_t xo = xoff0 + (uint32_t)(it * 64) * rowbytes;
#pragma unroll
      for (int j = 0; j < TPT; ++j) x[s][j] = buf_load16_nt(xr, xo + j * rowbytes);
      if constexpr (!PLAIN) sb[s] = __builtin_amdgcn_raw_buffer_load_b16(br, boff0 + (uint32_t)(it * 64) * H * 2, 0, 0);
    };
    // sqrt(beta) of this thread's TPT tokens of stage s, times xs
    auto token_scales = [&](int s, float xs, float (&sc)[TPT]) {
      const int sq = __float_as_int(__builtin_amdgcn_sqrtf(bf16_to_f32((uint16_t)sb[s])));
#pragma unroll
      for (int j = 0; j < TPT; ++j) sc[j] = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (tl + j), sq)) * xs;
    };
    auto store_x = [&](int s, int buf, float xs) {
      if constexpr (PLAIN) {
        // raw bfloat16 halves: channel row i of tokens j, j+1 packed into one word
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          uint32_t t16[TPT];
#pragma unroll
          for (int j = 0; j < TPT; ++j) {
            const uint32_t wd = (i >> 1) == 0 ? x[s][j].x : (i >> 1) == 1 ? x[s][j].y : (i >> 1) == 2 ? x[s][j].z : x[s][j].w;
            t16[j] = (i & 1) ? (wd >> 16) : (wd & 0xffffu);
          }
          const int r = row0 + i;
          uint8_t* dst = lds[buf] + r * 128 + 16 * (q ^ swz(r)) + hb;
          if constexpr (TPT == 8) {
            *reinterpret_cast<uint4*>(dst) = make_uint4(t16[0] | t16[1] << 16, t16[2] | t16[3] << 16,
                                                        t16[4] | t16[5] << 16, t16[6] | t16[7] << 16);
          } else if constexpr (TPT == 4) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(t16[0] | t16[1] << 16, t16[2] | t16[3] << 16);
          } else if constexpr (TPT == 2) {
            *reinterpret_cast<uint32_t*>(dst) = t16[0] | t16[1] << 16;
          } else {
            *reinterpret_cast<uint16_t*>(dst) = (uint16_t)t16[0];
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        return;
      }
      float sc[TPT];
      token_scales(s, xs, sc);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float v[TPT];
#pragma unroll
        for (int j = 0; j < TPT; ++j) {
          const uint32_t wd = (i >> 1) == 0 ? x[s][j].x : (i >> 1) == 1 ? x[s][j].y : (i >> 1) == 2 ? x[s][j].z : x[s][j].w;
          v[j] = ((i & 1) ? bf16_hi(wd) : bf16_lo(wd)) * sc[j];
        }
        const int r = row0 + i;
        uint8_t* dst = lds[buf] + r * 128 + 16 * (q ^ swz(r)) + hb;
        if constexpr (TPT == 8) {
          *reinterpret_cast<uint4*>(dst) = make_uint4(pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]),
                                                      pack_f16x2(v[4], v[5]), pack_f16x2(v[6], v[7]));
        } else if constexpr (TPT == 4) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]));
        } else if constexpr (TPT == 2) {
          *reinterpret_cast<uint32_t*>(dst) = pack_f16x2(v[0], v[1]);
        } else {
          *reinterpret_cast<_Float16*>(dst) = (_Float16)v[0];
        }
        __builtin_amdgcn_sched_barrier(0);  // one row's values live at a time
      }
    };
    auto store = [&](int s, int buf) { store_x(s, buf, 1.f); };

    // tile i+1 is written while the consumers multiply tile i; the stage it
    // came from is refilled at once with tile i+1+NS
#pragma unroll
    for (int s = 0; s < NS; ++s) load(s, s);
    store(0, 0);
    load(0, NS);
    lds_barrier();
    for (int it = 0; it < nstep; it += NS) {
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        const int s = (u + 1) % NS;  // stage holding tile it+u+1
        store(s, (u + 1) & 1);
        load(s, it + u + 1 + NS);
        lds_barrier();
      }
    }
    if constexpr (!PLAIN) {
      lds_barrier();  // the consumers' verdict is in s_flag
      if (s_flag) {
        // the largest |sqrt(beta) x| of this tensor over the unit, every tile
        float m = 0.f;
        for (int it = 0; it < nstep; ++it) {
          load(0, it);
          float sc[TPT];
          token_scales(0, 1.f, sc);
#pragma unroll
          for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < TPT; ++j) {
              const uint32_t wd = (i >> 1) == 0 ? x[0][j].x : (i >> 1) == 1 ? x[0][j].y : (i >> 1) == 2 ? x[0][j].z : x[0][j].w;
              m = fmaxf(m, fabsf(((i & 1) ? bf16_hi(wd) : bf16_lo(wd)) * sc[j]));
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        if (lane == 0) s_max[wave] = m;
        lds_barrier();
        const float xs = range_scale(fmaxf(s_max[2 * which], s_max[2 * which + 1]));
        // the contraction again, one tile at a time, on operands scaled by xs
        for (int it = 0; it < nstep; ++it) {
          load(0, it);
          store_x(0, 0, xs);
          lds_barrier();
          lds_barrier();
        }
      }
    }
  } else {
    // ---- consumers ----------------------------------------------------------
    const int wm = wave - 4;
    // PLAIN: only the waves holding rows of the second tensor (V^T K) multiply
    const bool mma = wm < WM && (!PLAIN || 16 * wm * MTW >= D);
    f32x4 acc[MTW][NT];
#pragma unroll
    for (int i = 0; i < MTW; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int buf) {
      const uint8_t* base = lds[buf];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int qq = 4 * ks + (lane >> 4);
        typedef std::conditional_t<PLAIN, bf16x8, f16x8> op_t;
        op_t afr[MTW];
#pragma unroll
        for (int mi = 0; mi < MTW; ++mi) {
          const int r = 16 * (wm * MTW + mi) + (lane & 15);
          afr[mi] = *reinterpret_cast<const op_t*>(base + r * 128 + 16 * (qq ^ swz(r)));
        }
#pragma unroll
        for (int nj = 0; nj < NT; ++nj) {
          const int r = 16 * nj + (lane & 15);
          const op_t bfr = *reinterpret_cast<const op_t*>(base + r * 128 + 16 * (qq ^ swz(r)));
#pragma unroll
          for (int mi = 0; mi < MTW; ++mi) {
            if constexpr (PLAIN)
              acc[mi][nj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[mi], bfr, acc[mi][nj], 0, 0, 0);
            else
              acc[mi][nj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(afr[mi], bfr, acc[mi][nj], 0, 0, 0);
          }
        }
        // one k-step of operands live at a time (beside 128 accumulators at d = 128)
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    lds_barrier();
    for (int it = 0; it < nstep; it += NS) {
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        if (mma) compute(u & 1);
        lds_barrier();
      }
    }

    // Range recovery.  The half-precision operands hold |sqrt(beta) x| up to
    // 65504; a larger one turns into inf and the sums into inf or NaN.  Then
    // the workgroup finds each tensor's largest |sqrt(beta) x| over the unit,
    // contracts again on operands scaled by powers of two (2^-eK, 2^-eV) that
    // bring it below 2^14, and undoes the scales exactly in float32:
    // A = 2^(2 eK) (Z^T Z), B = 2^(eK + eV) (W^T Z).  Finite inputs in range
    // never take this path; non-finite inputs take it and stay non-finite.
    float unA = 1.f, unB = 1.f;
    if constexpr (!PLAIN) {
      bool bad = false;
      if (mma) {
#pragma unroll
        for (int mi = 0; mi < MTW; ++mi)
#pragma unroll
          for (int nj = 0; nj < NT; ++nj)
#pragma unroll
            for (int r = 0; r < 4; ++r) bad |= !(fabsf(acc[mi][nj][r]) <= 3.0e38f);
      }
      if (bad) s_flag = 1;
      lds_barrier();
      if (s_flag) {
        lds_barrier();  // the producers' maxima are in s_max
        const float sk = range_scale(fmaxf(s_max[0], s_max[1]));
        const float sv = range_scale(fmaxf(s_max[2], s_max[3]));
        unA = 1.f / (sk * sk);
        unB = 1.f / (sv * sk);
#pragma unroll
        for (int i = 0; i < MTW; ++i)
#pragma unroll
          for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int it = 0; it < nstep; ++it) {
          lds_barrier();
          if (mma) compute(0);
          lds_barrier();
        }
      }
    }

    if (mma) {
      // slot of [A_t; B_t] (2d x d), or PLAIN: of V^T K alone (d x d)
      constexpr int OUTR = PLAIN ? D : R, ROW0 = PLAIN ? D : 0;
      float* out = stats + ((size_t)(b * H + h) * T_slots + (t + slot_offset)) * (size_t)(OUTR * D);
#pragma unroll
      for (int mi = 0; mi < MTW; ++mi)
#pragma unroll
        for (int nj = 0; nj < NT; ++nj)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            out[(16 * (wm * MTW + mi) + 4 * (lane >> 4) + r - ROW0) * D + 16 * nj + (lane & 15)] =
                acc[mi][nj][r] * (16 * (wm * MTW + mi) < D ? unA : unB);
    }
  }
}

template <int D>
__global__ __launch_bounds__(256, 2) void gram_f32(GramArgs<float> part0, GramArgs<float> part1, int nblk0,
                                                   float* __restrict__ stats, int H, int T_slots) {
  const bool second = (int)blockIdx.x >= nblk0;
  const GramArgs<float> g = second ? part1 : part0;
  const float* __restrict__ K = g.K;
  const float* __restrict__ V = g.V;
  const float* __restrict__ beta = g.beta;
  const int T_in = g.T_in, U = g.U, t_first = g.t_first, n_frames = g.n_frames, slot_offset = g.slot_offset;
  constexpr int R = 2 * D;
  constexpr int TT = 16;           // tokens per tile
  constexpr int LD = R + 16;       // padded floats per token row
  constexpr int UNITS = TT * R / 4;  // float4 units per tile
  constexpr int PER = (UNITS + 255) / 256;
  constexpr int MT = R / 16, NT = D / 16;
  constexpr int MTW = (MT + 3) / 4;
  __shared__ __attribute__((aligned(16))) float lds[2][TT * LD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int blk = (int)blockIdx.x - (second ? nblk0 : 0);
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
hipError_t launch_gram_d(const Problem& p, const GramPart* parts, int nparts, float* stats, hipStream_t s) {
  const GramPart none = parts[0];
  const GramPart& a = parts[0];
  const GramPart& c = nparts > 1 ? parts[1] : none;
  const int nblk0 = p.B * a.n_frames * p.H;
  const unsigned grid = (unsigned)(nblk0 + (nparts > 1 ? p.B * c.n_frames * p.H : 0));
  if (grid == 0) return hipSuccess;
  if (p.bf16) {
    auto arg = [](const GramPart& q) {
      return GramArgs<uint16_t>{static_cast<const uint16_t*>(q.k), static_cast<const uint16_t*>(q.v),
                                static_cast<const uint16_t*>(q.beta), q.T_in, q.U, q.t_first, q.n_frames,
                                q.slot_offset};
    };
    hipLaunchKernelGGL(gram_bf16<D>, dim3(grid), dim3(512), 0, s, arg(a), arg(c), nblk0, stats, p.H, p.T + 1);
  } else {
    auto arg = [](const GramPart& q) {
      return GramArgs<float>{static_cast<const float*>(q.k), static_cast<const float*>(q.v),
                             static_cast<const float*>(q.beta), q.T_in, q.U, q.t_first, q.n_frames,
                             q.slot_offset};
    };
    hipLaunchKernelGGL(gram_f32<D>, dim3(grid), dim3(256), 0, s, arg(a), arg(c), nblk0, stats, p.H, p.T + 1);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_gram_plain_d(const Problem& p, const void* k, const void* v, int n_frames, float* out,
                               hipStream_t s) {
  const unsigned grid = (unsigned)(p.B * n_frames * p.H);
  if (grid == 0) return hipSuccess;
  const GramArgs<uint16_t> a{static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), nullptr, p.T, p.U, 0,
                             n_frames, 0};
  hipLaunchKernelGGL((gram_bf16<D, true>), dim3(grid), dim3(512), 0, s, a, a, (int)grid, out, p.H, n_frames);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gram_plain(const Problem& p, const void* k, const void* v, float* out, hipStream_t s) {
  if (!p.bf16) return hipErrorInvalidValue;
  switch (p.D) {
    case 16: return launch_gram_plain_d<16>(p, k, v, p.T, out, s);
    case 32: return launch_gram_plain_d<32>(p, k, v, p.T, out, s);
    case 64: return launch_gram_plain_d<64>(p, k, v, p.T, out, s);
    case 128: return launch_gram_plain_d<128>(p, k, v, p.T, out, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gram(const Problem& p, const GramPart* parts, int nparts, float* stats, hipStream_t s) {
  if (nparts < 1 || nparts > 2) return hipErrorInvalidValue;
  switch (p.D) {
    case 16: return launch_gram_d<16>(p, parts, nparts, stats, s);
    case 32: return launch_gram_d<32>(p, parts, nparts, stats, s);
    case 64: return launch_gram_d<64>(p, parts, nparts, stats, s);
    case 128: return launch_gram_d<128>(p, parts, nparts, stats, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vda
