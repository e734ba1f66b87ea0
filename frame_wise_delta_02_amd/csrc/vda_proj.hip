// vda_proj: the linear maps either side of the VDA path.
//
// Before it, the gates read the attention block's input x ("Video DeltaNet"
// summary, onedev.kr/papers/80, section "무엇과 다른가": a sigmoid output gate
// after RMSNorm, separate decay and write gates; section "어떻게 쓰나": alpha
// per key channel per frame, beta per token; section "전제와 한계": the decay
// module in FP32):
//   gate logits  g = W_g x                       per token (H * d_v),
//   write gate   beta = sigmoid(w_beta x)        per token and head,
//   decay gate   alpha_t = sigmoid(W_alpha xbar_t), xbar_t the frame's mean token.
// After it, the branch merge (section "무엇과 다른가": each branch has its own
// output projection and the two are summed into the residual stream):
//   Y = Y_in + O W_O^T.
//
// Kernels:
//  * gemm_nt_bf16: C = A W^T on v_mfma_f32_32x32x16_bf16, A [M, K] and W [N, K]
//    bfloat16 (both K-contiguous), 256 x 256 tiles, K-panels of 64 double-
//    buffered in LDS and prefetched two panels ahead in registers, four waves
//    of 128 x 128 each, tiles ordered in bands of 4 M-tiles so that the tiles
//    an XCD runs at once share both operands' panels in its L2;
//    the epilogue goes through LDS for row-contiguous stores and either splits
//    the columns into gate logits and sigmoid(beta) or adds Y_in;
//  * frame_col_sums / frame_mean: the frames' mean tokens in float32 (split
//    over token ranges, then summed);
//  * alpha_proj: sigmoid(W_alpha xbar) in float32, 16 frames x 32 channels per
//    workgroup with K-panels of 256 in LDS.
#include <algorithm>

#include "vda_internal.h"

namespace vda {
namespace {

constexpr int GBM = 256, GBN = 256, GBK = 64;
constexpr int GROUP_M = 4;                // M-tiles per band of the tile order
constexpr int GLD = GBK + 8;              // LDS row stride of a staged panel (bfloat16 elements)
constexpr int GPANEL = GBM * GLD;         // elements per staged operand panel

enum { PROJ_GATE = 0, PROJ_ADD = 1 };

struct ProjOut {
  uint16_t* c;          // PROJ_GATE: gate logits [M, n_split]; PROJ_ADD: Y [M, N]
  uint16_t* c2;         // PROJ_GATE: beta [M, n2]
  const uint16_t* y_in; // PROJ_ADD: Y_in [M, N] or null
  int n_split, n2;      // PROJ_GATE: columns of the gate logits, of beta
};

__device__ __forceinline__ float sigmoidf_(float z) { return 1.f / (1.f + expf(-z)); }

template <int EPI>
__global__ __launch_bounds__(512, 1) void gemm_nt_bf16(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
                                                       int M, int N, int K, int mtiles, int ntiles, ProjOut out) {
  __shared__ uint4 lds4[2 * 2 * GPANEL / 8];  // two buffers of (A panel, W panel)
  uint16_t* lds = reinterpret_cast<uint16_t*>(lds4);
  // tile order: blocks bid, bid + 8, ... share an XCD, which takes a contiguous
  // run of the tile sequence; the sequence walks bands of GROUP_M M-tiles, M-tile
  // fastest, so the ~32 tiles an XCD runs at once cover a few M-tiles by several
  // N-tiles and share both operands' panels in its L2
  const int bid = blockIdx.x, xcd = bid & 7, slot = bid >> 3;
  const int ntot = mtiles * ntiles, per_xcd = (ntot + 7) / 8;
  const int tau = xcd * per_xcd + slot;
  if (slot >= per_xcd || tau >= ntot) return;
  const int band = tau / (GROUP_M * ntiles), r = tau % (GROUP_M * ntiles);
  const int gm = min(GROUP_M, mtiles - band * GROUP_M);
  const int nt = r / gm, mt = band * GROUP_M + r % gm;
  const int m0 = mt * GBM, n0 = nt * GBN;
  const int mrows = min(GBM, M - m0), nrows = min(GBN, N - n0);
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(A + (size_t)m0 * K, (uint32_t)mrows * K * 2);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(W + (size_t)n0 * K, (uint32_t)nrows * K * 2);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;  // 2 x 4 waves of 128 x 64

  // staging: thread t moves chunks c = t + 512 i (i < 4) of each panel: row c / 8,
  // k-chunk c % 8 (8 bfloat16); chunks at or past K are zero.  Two register
  // sets: while panel k is multiplied, panel k + 2 loads into one set and panel
  // k + 1 (loaded one panel earlier) goes from the other set to LDS, both spread
  // over the panel's k-steps so that the matrix cores keep issuing.
  uint4 ra0[4], rw0[4], ra1[4], rw1[4];
  auto gload = [&](uint4 (&ra)[4], uint4 (&rw)[4], int k0, int i0, int i1) {
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      const int c = tid + 512 * i, row = c >> 3, kc = c & 7;
      const int k = k0 + 8 * kc;
      // past K: an offset beyond either panel's range, which reads zero
      const uint32_t off = k < K ? ((uint32_t)row * K + k) * 2 : 0x80000000u;
      ra[i] = buf_load16(ar, off);
      rw[i] = buf_load16(wr, off);
    }
  };
  auto lstore = [&](const uint4 (&ra)[4], const uint4 (&rw)[4], int buf, int i0, int i1) {
    uint16_t* pa = lds + buf * 2 * GPANEL;
    uint16_t* pw = pa + GPANEL;
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      const int c = tid + 512 * i, row = c >> 3, kc = c & 7;
      *reinterpret_cast<uint4*>(pa + row * GLD + 8 * kc) = ra[i];
      *reinterpret_cast<uint4*>(pw + row * GLD + 8 * kc) = rw[i];
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{0.f};

  const int arow = 128 * wm + (lane & 31), wrow = 64 * wn + (lane & 31), kq = 8 * (lane >> 5);
  // one panel from LDS buffer `buf`: four k-steps of 16, each with one of the
  // four staging parts (loads into set L, LDS stores from set S into the other
  // buffer) after its eight products
  auto stage = [&](int buf, uint4 (&la)[4], uint4 (&lw)[4], int k0_load, const uint4 (&sa)[4],
                   const uint4 (&sw)[4]) {
    const uint16_t* pa = lds + buf * 2 * GPANEL;
    const uint16_t* pw = pa + GPANEL;
#pragma unroll
    for (int s = 0; s < GBK / 16; ++s) {
      bf16x8 af[4], wf[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(pa + (arow + 32 * i) * GLD + 16 * s + kq);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        wf[j] = *reinterpret_cast<const bf16x8*>(pw + (wrow + 32 * j) * GLD + 16 * s + kq);
      gload(la, lw, k0_load, s, s + 1);
      // the SIMD's other wave yields to this one while its products issue
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], wf[j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_s_setprio(0);
      lstore(sa, sw, buf ^ 1, s, s + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int nk = (K + GBK - 1) / GBK;
  gload(ra0, rw0, 0, 0, 4);
  lstore(ra0, rw0, 0, 0, 4);
  gload(ra0, rw0, GBK, 0, 4);
  __syncthreads();
  // panels in pairs: panel kt (even) from buffer 0, loading panel kt + 2 into
  // set 1 and storing panel kt + 1 (set 0) into buffer 1; then the same with the
  // roles swapped.  Loads and stores are unconditional, so the code is
  // straight-line and each wait leaves the newer panel's loads in flight; a
  // panel past K reads zero and lands in a buffer nothing reads.
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    stage(0, ra1, rw1, (kt + 2) * GBK, ra0, rw0);
    __syncthreads();
    stage(1, ra0, rw0, (kt + 3) * GBK, ra1, rw1);
    __syncthreads();
  }
  if (kt < nk) {  // an odd last panel, already in buffer 0
    stage(0, ra1, rw1, nk * GBK + GBK, ra0, rw0);
    __syncthreads();  // before the epilogue reuses the buffers
  }

  // epilogue: the wave's 128 x 64 tile as bfloat16 rows in LDS (acc[i][j][r]
  // is C[32 i + 8 (r / 4) + 4 (lane / 32) + r % 4][32 j + lane % 32]), then
  // row-contiguous 16-byte stores
  constexpr int OLD = 64 + 8;
  uint16_t* po = lds + wave * 128 * OLD;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = 32 * j + (lane & 31);
    bool sig = false;
    if constexpr (EPI == PROJ_GATE) sig = n0 + 64 * wn + col >= out.n_split;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        float v = acc[i][j][r];
        if constexpr (EPI == PROJ_GATE) v = sig ? sigmoidf_(v) : v;
        po[row * OLD + col] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xffffu);
      }
      __builtin_amdgcn_sched_barrier(0);  // one accumulator tile live at a time
    }
  }
  __builtin_amdgcn_wave_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  const int rbase = m0 + 128 * wm, cbase = n0 + 64 * wn;
  if constexpr (EPI == PROJ_GATE) {
    const int ng = out.n_split, nb = out.n2;
    const __amdgpu_buffer_rsrc_t gr = make_rsrc(out.c + (size_t)rbase * ng,
                                                rbase < M ? (uint32_t)min(128, M - rbase) * ng * 2 : 0u);
    const __amdgpu_buffer_rsrc_t br = make_rsrc(out.c2 + (size_t)rbase * nb,
                                                rbase < M ? (uint32_t)min(128, M - rbase) * nb * 2 : 0u);
#pragma unroll 4
    for (int it = 0; it < 16; ++it) {
      const int c = lane + 64 * it, row = c >> 3, ch = c & 7;
      const int n = cbase + 8 * ch;
      const uint4 v = *reinterpret_cast<const uint4*>(po + row * OLD + 8 * ch);
      if (n + 8 <= ng) {
        buf_store16(v, gr, ((uint32_t)row * ng + n) * 2);
      } else if (n < ng + nb) {
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int ne = n + e;
          const uint16_t h = (uint16_t)((e & 1) ? (w4[e >> 1] >> 16) : (w4[e >> 1] & 0xffffu));
          if (ne < ng)
            __builtin_amdgcn_raw_buffer_store_b16(h, gr, ((uint32_t)row * ng + ne) * 2, 0, 0);
          else if (ne < ng + nb)
            __builtin_amdgcn_raw_buffer_store_b16(h, br, ((uint32_t)row * nb + (ne - ng)) * 2, 0, 0);
        }
      }
    }
  } else {
    const uint32_t bytes = rbase < M ? (uint32_t)min(128, M - rbase) * N * 2 : 0u;
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(out.c + (size_t)rbase * N, bytes);
    const __amdgpu_buffer_rsrc_t ir = make_rsrc(out.y_in ? out.y_in + (size_t)rbase * N : out.c, out.y_in ? bytes : 0u);
#pragma unroll 4
    for (int it = 0; it < 16; ++it) {
      const int c = lane + 64 * it, row = c >> 3, ch = c & 7;
      const int n = cbase + 8 * ch;
      if (n + 8 > N) continue;
      const uint32_t off = ((uint32_t)row * N + n) * 2;
      const uint4 v = *reinterpret_cast<const uint4*>(po + row * OLD + 8 * ch);
      const uint4 y0 = buf_load16(ir, off);
      const uint32_t a4[4] = {v.x, v.y, v.z, v.w}, b4[4] = {y0.x, y0.y, y0.z, y0.w};
      uint32_t o4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o4[e] = pack_bf16x2(bf16_lo(a4[e]) + bf16_lo(b4[e]), bf16_hi(a4[e]) + bf16_hi(b4[e]));
      buf_store16(make_uint4(o4[0], o4[1], o4[2], o4[3]), yr, off);
    }
  }
}

// Column sums of x over token range s of every frame: partial [F, S, K] (float32).
// Thread t of workgroup (f, kb, s) owns columns 8 (256 kb + t) .. + 7.
__global__ __launch_bounds__(256) void frame_col_sums(const uint16_t* __restrict__ x, float* __restrict__ partial,
                                                      int U, int K, int S) {
  const int f = blockIdx.x, s = blockIdx.z;
  const int kc = blockIdx.y * 256 + threadIdx.x;
  if (8 * kc >= K) return;
  const int per = (U + S - 1) / S, u0 = s * per, u1 = min(U, u0 + per);
  const uint16_t* base = x + ((size_t)f * U) * K + 8 * kc;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int u = u0;
  for (; u + 4 <= u1; u += 4) {
    uint4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = *reinterpret_cast<const uint4*>(base + (size_t)(u + j) * K);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w4[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += bf16_lo(w4[e]);
        acc[2 * e + 1] += bf16_hi(w4[e]);
      }
    }
  }
  for (; u < u1; ++u) {
    const uint4 v = *reinterpret_cast<const uint4*>(base + (size_t)u * K);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += bf16_lo(w4[e]);
      acc[2 * e + 1] += bf16_hi(w4[e]);
    }
  }
  float* o = partial + ((size_t)f * S + s) * K + 8 * kc;
  *reinterpret_cast<float4*>(o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4*>(o + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

// xbar [F, K] = (sum over the S partial sums) / U.
__global__ __launch_bounds__(256) void frame_mean(const float* __restrict__ partial, float* __restrict__ xbar, int U,
                                                  int K, int S, int F) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)F * K) return;
  const size_t f = i / K, k = i % K;
  float s = 0.f;
  for (int j = 0; j < S; ++j) s += partial[(f * S + j) * K + k];
  xbar[i] = s / (float)U;
}

// alpha [F, NA] = sigmoid(xbar W_alpha^T) in float32.  Workgroup (fb, nb) forms
// frames 16 fb .. + 15 and channels 32 nb .. + 31; K runs in panels of 256
// staged in LDS (xbar panel [16][256], W_alpha panel [32][256 + 1]), every load
// of a panel in flight at once; thread t owns frame t / 16 and channels
// 32 nb + (t % 16) + 16 j, j < 2.
constexpr int AKP = 256, ANT = 32;
__global__ __launch_bounds__(256) void alpha_proj(const float* __restrict__ xbar, const float* __restrict__ wa,
                                                  float* __restrict__ alpha, int F, int K, int NA) {
  __shared__ float sx[16][AKP];
  __shared__ float sw[ANT][AKP + 1];
  const int f0 = blockIdx.x * 16, n0 = blockIdx.y * ANT, tid = threadIdx.x;
  const int fl = tid >> 4, nl = tid & 15;
  float acc[2] = {0.f, 0.f};
  for (int k0 = 0; k0 < K; k0 += AKP) {
    float vx[16 * AKP / 256], vw[ANT * AKP / 256];
#pragma unroll
    for (int j = 0; j < 16 * AKP / 256; ++j) {
      const int i = tid + 256 * j, f = i / AKP, k = i % AKP;
      vx[j] = (f0 + f < F && k0 + k < K) ? xbar[(size_t)(f0 + f) * K + k0 + k] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < ANT * AKP / 256; ++j) {
      const int i = tid + 256 * j, n = i / AKP, k = i % AKP;
      vw[j] = (n0 + n < NA && k0 + k < K) ? wa[(size_t)(n0 + n) * K + k0 + k] : 0.f;
    }
    __syncthreads();  // the previous panel has been read
#pragma unroll
    for (int j = 0; j < 16 * AKP / 256; ++j) {
      const int i = tid + 256 * j;
      sx[i / AKP][i % AKP] = vx[j];
    }
#pragma unroll
    for (int j = 0; j < ANT * AKP / 256; ++j) {
      const int i = tid + 256 * j;
      sw[i / AKP][i % AKP] = vw[j];
    }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < AKP; ++k) {
      const float xv = sx[fl][k];
      acc[0] += xv * sw[nl][k];
      acc[1] += xv * sw[nl + 16][k];
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int f = f0 + fl, n = n0 + nl + 16 * j;
    if (f < F && n < NA) alpha[(size_t)f * NA + n] = sigmoidf_(acc[j]);
  }
}

hipError_t launch_gemm(int epi, int M, int N, int K, const void* a, const void* w, const ProjOut& out, hipStream_t s) {
  const int mtiles = (M + GBM - 1) / GBM, ntiles = (N + GBN - 1) / GBN;
  const long long grid = ((long long)mtiles * ntiles + 7) / 8 * 8;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  auto A = static_cast<const uint16_t*>(a);
  auto Wt = static_cast<const uint16_t*>(w);
  if (epi == PROJ_GATE)
    hipLaunchKernelGGL(gemm_nt_bf16<PROJ_GATE>, dim3((unsigned)grid), dim3(512), 0, s, A, Wt, M, N, K, mtiles, ntiles,
                       out);
  else
    hipLaunchKernelGGL(gemm_nt_bf16<PROJ_ADD>, dim3((unsigned)grid), dim3(512), 0, s, A, Wt, M, N, K, mtiles, ntiles,
                       out);
  return hipGetLastError();
}

}  // namespace

int proj_mean_splits(const Problem& p) { return std::max(1, std::min(8, p.U / 64)); }

hipError_t launch_gates(const Problem& p, int d_model, const void* x, const void* w_gb, const float* w_alpha,
                        void* gate, void* beta, float* alpha, float* partial, float* xbar, hipStream_t s) {
  const int M = p.B * p.T * p.U, F = p.B * p.T, K = d_model;
  const int ng = p.H * p.D, nb = p.H;
  ProjOut o{static_cast<uint16_t*>(gate), static_cast<uint16_t*>(beta), nullptr, ng, nb};
  hipError_t e = launch_gemm(PROJ_GATE, M, ng + nb, K, x, w_gb, o, s);
  if (e != hipSuccess) return e;
  const int S = proj_mean_splits(p);
  hipLaunchKernelGGL(frame_col_sums, dim3((unsigned)F, (unsigned)((K / 8 + 255) / 256), (unsigned)S), dim3(256), 0, s,
                     static_cast<const uint16_t*>(x), partial, p.U, K, S);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t n = (size_t)F * K;
  hipLaunchKernelGGL(frame_mean, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, partial, xbar, p.U, K, S, F);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int NA = p.H * p.D;
  hipLaunchKernelGGL(alpha_proj, dim3((unsigned)((F + 15) / 16), (unsigned)((NA + ANT - 1) / ANT)), dim3(256), 0, s,
                     xbar, w_alpha, alpha, F, K, NA);
  return hipGetLastError();
}

hipError_t launch_out_proj(const Problem& p, int d_model, const void* o, const void* w_o, const void* y_in, void* y,
                           hipStream_t s) {
  const int M = p.B * p.T * p.U, K = p.H * p.D;
  ProjOut out{static_cast<uint16_t*>(y), nullptr, static_cast<const uint16_t*>(y_in), 0, 0};
  return launch_gemm(PROJ_ADD, M, d_model, K, o, w_o, out, s);
}

}  // namespace vda
