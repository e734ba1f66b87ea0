// vda_solve: (I + A_t)^{-1} for every frame of every head, held in LDS: by a
// symmetric block sweep for bfloat16 inputs (solve_sweep, further below), by
// Cholesky for float32 inputs and d = 16 (solve_mfma).
//
// The frame update S_t = (S_{t-1} Diag(alpha_t) + B_t)(I + A_t)^{-1} is solved in
// the d_k x d_k key space ("Video DeltaNet" summary, onedev.kr/papers/80, section
// "어떻게 쓰나"); the VDN-H3 write-up (discuss.pytorch.kr, hybrid attention
// structure) notes that A_t is positive semidefinite, so P = I + A_t is
// symmetric positive definite and has a Cholesky factor.  One workgroup
// (4 waves) inverts one P, held in LDS:
//   1. P = L L^T, right-looking over 16-column panels.  One wave factors the
//      16x16 diagonal block in registers (lane = row, readlane broadcasts) and
//      inverts it; the panel solve L_ik = P_ik L_kk^{-T} and the trailing
//      update P_ij -= L_ik L_jk^T run on v_mfma_f32_16x16x4f32 in all waves.
//   2. W = L^{-1} by blocked substitution down each block column (columns
//      spread over the waves), stored transposed in P's unused upper triangle.
//   3. P^{-1} = W^T W on the same matrix cores.  With float32 inputs (or
//      d = 16) it is written from the accumulators straight to global memory
//      (both triangles).  With bfloat16 inputs and d >= 32 it is split into
//      bfloat16 hi + lo planes, relaid through LDS into the scan's matrix-core
//      operand order (the split layout described with pinv_split) and written
//      coalesced.
// The arithmetic is fp32.  The scan consumes P^{-1} directly:
// S M_t + J_t = (S Diag(alpha_t) + B_t) P^{-1}, so M_t and J_t are never formed.
#include "vda_internal.h"

namespace vda {
namespace {

constexpr int WDS = 17;  // row stride of the 16x16 diagonal-inverse blocks in LDS

__device__ __forceinline__ float rdlane(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

template <int D, bool SPLIT>
__global__ __launch_bounds__(256, 2) void solve_mfma(const float* __restrict__ stats,
                                                    float* __restrict__ pinv, int H, int T,
                                                    int n_video) {
  constexpr int NB = D / 16;     // 16-wide panels
  constexpr int LDP = D + 4;     // padded LDS row (conflict-free operand reads)
  __shared__ __attribute__((aligned(16))) float P[D * LDP];
  __shared__ float Wd[NB][16 * WDS];   // inverses of the diagonal blocks of L

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_slots = n_video + 1;
  int blk = blockIdx.x;
  const int si = blk % n_slots;
  blk /= n_slots;
  const int h = blk % H;
  const int b = blk / H;
  const int slot = (si < n_video) ? 1 + si : T;  // video frames 1..T-2, then the text slot T
  const size_t mat = (size_t)(b * H + h) * (T + 1) + slot;
  const float* A = stats + mat * (size_t)(2 * D * D);
  float* Pout = pinv + mat * (size_t)(D * D);

  // lane roles for 16x16x4 MFMA operands / results
  const int lm = lane & 15, lg = lane >> 4;

  // ---- load P = I + A ------------------------------------------------------
  // every load is issued before the first LDS store: a load-store loop waits a
  // full memory round trip per iteration
  {
    constexpr int NV4 = D * D / 4;               // float4 of A
    constexpr int PER = (NV4 + 255) / 256;
    float4 x[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + 256 * i;
      x[i] = (NV4 % 256 == 0 || e < NV4) ? reinterpret_cast<const float4*>(A)[e] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + 256 * i;
      if (NV4 % 256 == 0 || e < NV4) {
        const int r = e / (D / 4), c = 4 * (e % (D / 4));
        x[i].x += (r == c) ? 1.f : 0.f;
        x[i].y += (r == c + 1) ? 1.f : 0.f;
        x[i].z += (r == c + 2) ? 1.f : 0.f;
        x[i].w += (r == c + 3) ? 1.f : 0.f;
        *reinterpret_cast<float4*>(&P[r * LDP + c]) = x[i];
      }
    }
  }
  __syncthreads();

  // C (+)= sum over 4 k-steps of A(16x16) B(16x16); operand fetchers take (s)
  auto tile_mma = [&](f32x4 acc, auto a_of, auto b_of) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a_of(s), b_of(s), acc, 0, 0, 0);
    return acc;
  };

  // ---- 1. Cholesky ------------------------------------------------------------
  // One wave factors diagonal block k in registers (lane = row, readlane
  // broadcasts; hardware sqrt and reciprocal, about 1 ulp) and writes L_kk and
  // W_kk = L_kk^{-1}.  This serial chain is the critical path of the whole
  // inversion, so it runs ahead: during step k's trailing update, wave 0 first
  // updates block (k+1, k+1) and then factors it, while waves 1-3 update the
  // other trailing blocks.
  auto factor_diag = [&](int k) {
    const int i = lm;  // row of the diagonal block owned by this lane
    float a[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) a[c] = P[(16 * k + i) * LDP + 16 * k + c];
    float rdiag = 0.f;  // 1 / L[i][i] of this lane's row
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float d = __builtin_amdgcn_sqrtf(rdlane(a[j], j));
      const float inv = __builtin_amdgcn_rcpf(d);
      const float l = (i > j) ? a[j] * inv : (i == j ? d : 0.f);
      if (i == j) rdiag = inv;
      a[j] = l;
#pragma unroll
      for (int c = j + 1; c < 16; ++c) a[c] -= l * rdlane(l, c);
    }
    // column c = lane of W_kk = L_kk^{-1} by forward substitution
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float sacc = (r == i) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < r; ++m) sacc -= rdlane(a[m], r) * x[m];
      x[r] = sacc * rdlane(rdiag, r);
    }
    if (lane < 16) {
#pragma unroll
      for (int c = 0; c < 16; ++c) P[(16 * k + i) * LDP + 16 * k + c] = (c <= i) ? a[c] : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) Wd[k][r * WDS + i] = x[r];
    }
  };
  // trailing tile idx of step k (idx -> (i, j) over the lower triangle, row by
  // row; idx 0 is block (k+1, k+1)): P_ij -= L_ik L_jk^T
  auto trailing_tile = [&](int k, int idx) {
    int i = 0, rem = idx;
    while (rem > i) { rem -= i + 1; ++i; }
    const int bi = k + 1 + i, bj = k + 1 + rem;
    f32x4 acc;
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = P[(16 * bi + 4 * lg + r) * LDP + 16 * bj + lm];
    const float* Li = &P[(16 * bi + lm) * LDP + 16 * k + lg];
    const float* Lj = &P[(16 * bj + lm) * LDP + 16 * k + lg];
    acc = tile_mma(acc, [&](int s) { return -Li[4 * s]; }, [&](int s) { return Lj[4 * s]; });
#pragma unroll
    for (int r = 0; r < 4; ++r) P[(16 * bi + 4 * lg + r) * LDP + 16 * bj + lm] = acc[r];
  };

  // two trailing tiles at once (the second may be absent: it then repeats the
  // first and is not stored), so two matrix-core chains run side by side
  auto trailing_pair = [&](int k, int idx0, int idx1) {
    const bool two = idx1 >= 0;
    int bi[2], bj[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int i = 0, rem = (u == 0 || !two) ? idx0 : idx1;
      while (rem > i) { rem -= i + 1; ++i; }
      bi[u] = k + 1 + i;
      bj[u] = k + 1 + rem;
    }
    f32x4 acc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[u][r] = P[(16 * bi[u] + 4 * lg + r) * LDP + 16 * bj[u] + lm];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(-P[(16 * bi[u] + lm) * LDP + 16 * k + 4 * s4 + lg],
                                                      P[(16 * bj[u] + lm) * LDP + 16 * k + 4 * s4 + lg],
                                                      acc[u], 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) P[(16 * bi[0] + 4 * lg + r) * LDP + 16 * bj[0] + lm] = acc[0][r];
    if (two) {
#pragma unroll
      for (int r = 0; r < 4; ++r) P[(16 * bi[1] + 4 * lg + r) * LDP + 16 * bj[1] + lm] = acc[1][r];
    }
  };

  if (wave == 0) factor_diag(0);
  __syncthreads();
  for (int k = 0; k < NB; ++k) {
    // panel: L_ik = P_ik W_kk^T, in place
    for (int i = k + 1 + wave; i < NB; i += 4) {
      const float* Pi = &P[(16 * i + lm) * LDP + 16 * k + lg];
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      acc = tile_mma(acc, [&](int s) { return Pi[4 * s]; },
                     [&](int s) { return Wd[k][lm * WDS + 4 * s + lg]; });
#pragma unroll
      for (int r = 0; r < 4; ++r) P[(16 * i + 4 * lg + r) * LDP + 16 * k + lm] = acc[r];
    }
    __syncthreads();
    // trailing update of the lower blocks, k < j <= i, with diagonal block
    // k+1 updated and factored first by wave 0
    {
      const int m = NB - 1 - k;  // trailing blocks per side
      const int ntr = m * (m + 1) / 2;
      if (m > 0) {
        if (wave == 0) {
          trailing_tile(k, 0);
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          __builtin_amdgcn_wave_barrier();
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          factor_diag(k + 1);
        } else {
          for (int idx = wave; idx < ntr; idx += 6) trailing_pair(k, idx, idx + 3 < ntr ? idx + 3 : -1);
        }
      }
    }
    __syncthreads();
  }

  // ---- 2. W = L^{-1}: block column j, top to bottom ---------------------------
  // W_jj = Wd[j]; W_ij = -W_ii sum_{m=j}^{i-1} L_im W_mj.  W_ij (i > j) is kept
  // transposed in the upper block (j, i).  Columns j and NB-1-j share a wave.
  // The diagonal blocks of P are dead after step 1 (W_jj lives in Wd), so wave
  // w uses diagonal block (w, w) as scratch to relayout a result into an operand.
  auto Wb = [&](int m, int j, int kk, int n) -> float {  // W_mj[kk][n], m >= j
    return (m == j) ? Wd[j][kk * WDS + n] : P[(16 * j + n) * LDP + 16 * m + kk];
  };
  // (with NB < 4 the waves that own no block column take wave 0's address,
  // which they never use, instead of one past P)
  float* Tx = &P[16 * (NB >= 4 || wave < NB ? wave : 0) * (LDP + 1)];
  for (int pass = 0; pass < 2; ++pass) {
    const int j = pass == 0 ? wave : NB - 1 - wave;
    if (j < 0 || j >= NB || (pass == 1 && j < 4)) continue;
    for (int i = j + 1; i < NB; ++i) {
      // two accumulators (even and odd m) halve the dependent matrix-core chain
      f32x4 t0 = f32x4{0.f, 0.f, 0.f, 0.f}, t1 = t0;
      int m = j;
      for (; m + 1 < i; m += 2) {
        const float* L0 = &P[(16 * i + lm) * LDP + 16 * m + lg];
        const float* L1 = L0 + 16;
        t0 = tile_mma(t0, [&](int s) { return L0[4 * s]; }, [&](int s) { return Wb(m, j, 4 * s + lg, lm); });
        t1 = tile_mma(t1, [&](int s) { return L1[4 * s]; }, [&](int s) { return Wb(m + 1, j, 4 * s + lg, lm); });
      }
      if (m < i) {
        const float* L0 = &P[(16 * i + lm) * LDP + 16 * m + lg];
        t0 = tile_mma(t0, [&](int s) { return L0[4 * s]; }, [&](int s) { return Wb(m, j, 4 * s + lg, lm); });
      }
      const f32x4 t = t0 + t1;
      // relayout T through this wave's scratch, then W_ij = -W_ii T
#pragma unroll
      for (int r = 0; r < 4; ++r) Tx[(4 * lg + r) * LDP + lm] = t[r];
      __builtin_amdgcn_wave_barrier();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      f32x4 w = f32x4{0.f, 0.f, 0.f, 0.f};
      w = tile_mma(w, [&](int s) { return -Wd[i][lm * WDS + 4 * s + lg]; },
                   [&](int s) { return Tx[(4 * s + lg) * LDP + lm]; });
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int r = 0; r < 4; ++r) P[(16 * j + lm) * LDP + 16 * i + 4 * lg + r] = w[r];
    }
  }
  __syncthreads();

  // ---- 3. P^{-1} = W^T W: lower blocks (i >= j) --------------------------------
  constexpr int NT = NB * (NB + 1) / 2;
  auto lower_tile = [&](int idx, int& bi, int& bj) {
    int i = 0, rem = idx;
    while (rem > i) { rem -= i + 1; ++i; }
    bi = i;
    bj = rem;
    // A = W_mi^T: A[p][kk] = W_mi[kk][p];  B = W_mj.  Even and odd m go to two
    // accumulators (two independent matrix-core chains).
    f32x4 a0 = f32x4{0.f, 0.f, 0.f, 0.f}, a1 = a0;
    int m = bi;
    for (; m + 1 < NB; m += 2) {
      a0 = tile_mma(a0, [&](int s) { return Wb(m, bi, 4 * s + lg, lm); },
                    [&](int s) { return Wb(m, bj, 4 * s + lg, lm); });
      a1 = tile_mma(a1, [&](int s) { return Wb(m + 1, bi, 4 * s + lg, lm); },
                    [&](int s) { return Wb(m + 1, bj, 4 * s + lg, lm); });
    }
    if (m < NB)
      a0 = tile_mma(a0, [&](int s) { return Wb(m, bi, 4 * s + lg, lm); },
                    [&](int s) { return Wb(m, bj, 4 * s + lg, lm); });
    return a0 + a1;
  };
  if constexpr (!SPLIT) {
    for (int idx = wave; idx < NT; idx += 4) {
      int bi, bj;
      const f32x4 acc = lower_tile(idx, bi, bj);
#pragma unroll
      for (int r = 0; r < 4; ++r) Pout[(16 * bi + 4 * lg + r) * D + 16 * bj + lm] = acc[r];
      if (bi != bj) {
        *reinterpret_cast<float4*>(&Pout[(16 * bj + lm) * D + 16 * bi + 4 * lg]) =
            make_float4(acc[0], acc[1], acc[2], acc[3]);
      }
    }
  } else {
    // every tile of this wave stays in registers until all waves are done
    // reading W from LDS; then P's storage holds Z_hi, Z_lo with
    // Z[c][k] = P^{-1}[k][c] (symmetric), rows of D + 4 bfloat16
    constexpr int NPW = (NT + 3) / 4;
    constexpr int LDZ = D + 4;
    f32x4 res[NPW];
    int tb[NPW];
#pragma unroll
    for (int it = 0; it < NPW; ++it) {
      const int idx = wave + 4 * it;
      res[it] = f32x4{0.f, 0.f, 0.f, 0.f};
      tb[it] = -1;
      if (idx < NT) {
        int bi, bj;
        res[it] = lower_tile(idx, bi, bj);
        tb[it] = bi * NB + bj;
      }
    }
    __syncthreads();
    __bf16* Zh = reinterpret_cast<__bf16*>(P);
    __bf16* Zl = Zh + D * LDZ;
    static_assert(2 * D * LDZ * 2 == D * LDP * 4, "Z planes fill P's storage exactly");
#pragma unroll
    for (int it = 0; it < NPW; ++it) {
      if (tb[it] < 0) continue;
      const int bi = tb[it] / NB, bj = tb[it] % NB;
      __bf16 h[4], l[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) split_bf16(res[it][r], h[r], l[r]);
      // lane value r is P^{-1}[16 bi + 4 lg + r][16 bj + lm]
      const int o = (16 * bj + lm) * LDZ + 16 * bi + 4 * lg;
      *reinterpret_cast<uint2*>(Zh + o) = make_uint2(__builtin_bit_cast(uint32_t, bf16x2{h[0], h[1]}),
                                                     __builtin_bit_cast(uint32_t, bf16x2{h[2], h[3]}));
      *reinterpret_cast<uint2*>(Zl + o) = make_uint2(__builtin_bit_cast(uint32_t, bf16x2{l[0], l[1]}),
                                                     __builtin_bit_cast(uint32_t, bf16x2{l[2], l[3]}));
      if (bi != bj) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          Zh[(16 * bi + 4 * lg + r) * LDZ + 16 * bj + lm] = h[r];
          Zl[(16 * bi + 4 * lg + r) * LDZ + 16 * bj + lm] = l[r];
        }
      }
    }
    __syncthreads();
    // fragment f of a plane: 8 consecutive k of one column
    constexpr int NFR = D * D / 8;
    constexpr int KS2 = D / 32;
    uint4* Fo = reinterpret_cast<uint4*>(Pout);
#pragma unroll 4
    for (int f = tid; f < NFR; f += 256) {
      const int fl = f & 63, ks = (f >> 6) % KS2, we = (f >> 6) / KS2;
      const int c = 32 * (we >> 1) + 2 * (fl & 15) + (we & 1);
      const int o = c * LDZ + 32 * ks + 8 * (fl >> 4);
      const uint2 h0 = *reinterpret_cast<const uint2*>(Zh + o), h1 = *reinterpret_cast<const uint2*>(Zh + o + 4);
      const uint2 l0 = *reinterpret_cast<const uint2*>(Zl + o), l1 = *reinterpret_cast<const uint2*>(Zl + o + 4);
      Fo[f] = make_uint4(h0.x, h0.y, h1.x, h1.y);
      Fo[NFR + f] = make_uint4(l0.x, l0.y, l1.x, l1.y);
    }
  }
}

// ---------------------------------------------------------------------------
// bfloat16 inputs (d >= 32): the inverse by a symmetric block sweep.
//
// Sweeping the 16 x 16 diagonal blocks of P in order (block Gauss-Jordan
// without pivoting, which P = I + A_t, symmetric positive definite with every
// Schur complement >= I, allows) leaves -P^{-1} in place: for pivot block k,
// with X = (P_kk)^{-1},
//     P_ij <- P_ij - (P_ik X) P_kj   (i, j != k),
//     P_ik <- P_ik X,  P_kj <- X P_kj,  P_kk <- -X.
// The sweep keeps P symmetric, so only the lower triangle of 16 x 16 tiles is
// held (in LDS, rows padded to 17 floats: 40 KB at d = 128, four matrices per
// compute unit).  Its only serial part is the chain of d/16 leaf inversions
// (each a scalar sweep of the 16 x 16 block in one wave: lane = row, the pivot
// row broadcast by readlane); everything else is 16 x 16 x 16 tile products on
// v_mfma_f32_16x16x4f32, spread over the four waves by rows.  The products of
// a step contract over a permuted k order (k = 4 (lane / 16) + s), so the
// accumulator of C_i = P_ik X, computed transposed, is already the left
// operand of the updates P_ij -= C_i P_kj and stays in registers.  All
// arithmetic is fp32; the result is written as bfloat16 hi + lo planes in the
// scan's operand order, as solve_mfma does.
template <int D>
__global__ __launch_bounds__(256) void solve_sweep(const float* __restrict__ stats, float* __restrict__ pinv,
                                                   int H, int T, int n_video) {
  constexpr int NB = D / 16;               // 16 x 16 blocks per side
  constexpr int NT = NB * (NB + 1) / 2;    // lower-triangle tiles
  constexpr int LDT = 17;                  // padded tile row (floats)
  constexpr int TS = 16 * LDT;             // floats per tile
  constexpr int RPW = NB == 8 ? 2 : 1;     // block rows per wave
  __shared__ float tl[(NT + 1) * TS];      // tile (R, C), C <= R, at R (R + 1) / 2 + C; then X
  float* XS = tl + NT * TS;
  auto tile = [&](int R, int C) -> float* { return tl + (R * (R + 1) / 2 + C) * TS; };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lm = lane & 15, lg = lane >> 4;
  const int n_slots = n_video + 1;
  int blk = blockIdx.x;
  const int si = blk % n_slots;
  blk /= n_slots;
  const int h = blk % H;
  const int b = blk / H;
  const int slot = (si < n_video) ? 1 + si : T;  // video frames 1..T-2, then the text slot T
  const size_t mat = (size_t)(b * H + h) * (T + 1) + slot;
  const float* A = stats + mat * (size_t)(2 * D * D);
  float* Pout = pinv + mat * (size_t)(D * D);

  // ---- the lower tiles of P = I + A into LDS (every load issued first) ------
  {
    constexpr int NV4 = NT * 64;  // float4 pieces of the lower tiles
    constexpr int PER = (NV4 + 255) / 256;
    float4 x[PER];
    int dst[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = tid + 256 * q;
      x[q] = make_float4(0.f, 0.f, 0.f, 0.f);
      dst[q] = -1;
      if (NV4 % 256 == 0 || e < NV4) {
        const int t = e >> 6, w = e & 63;
        int R = 0;
        while ((R + 1) * (R + 2) / 2 <= t) ++R;
        const int C = t - R * (R + 1) / 2;
        const int row = w >> 2, c4 = w & 3;
        x[q] = *reinterpret_cast<const float4*>(A + (size_t)(16 * R + row) * D + 16 * C + 4 * c4);
        dst[q] = (t * 16 + row) * LDT + 4 * c4;
        if (R == C) {
          x[q].x += (row == 4 * c4) ? 1.f : 0.f;
          x[q].y += (row == 4 * c4 + 1) ? 1.f : 0.f;
          x[q].z += (row == 4 * c4 + 2) ? 1.f : 0.f;
          x[q].w += (row == 4 * c4 + 3) ? 1.f : 0.f;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      if (dst[q] >= 0) {
        tl[dst[q]] = x[q].x;
        tl[dst[q] + 1] = x[q].y;
        tl[dst[q] + 2] = x[q].z;
        tl[dst[q] + 3] = x[q].w;
      }
    }
  }
  __syncthreads();

  // ---- leaf: the 16 x 16 block (k, k) swept in one wave ---------------------
  // Lane i (of 16; the other lanes repeat the rows) holds row i.  For pivot p
  // with d = a_pp and r = 1/d: a_ij -= (a_ip r) a_pj for i, j != p; a_pj *= r;
  // a_ip *= r; a_pp = -r.  Row p's update is written in the same form with
  // a multiplier 1 - r.  The result is -(block)^{-1}: written to the tile (its
  // swept value -X) and, negated, to XS (X itself).
  auto leaf = [&](int k) {
    float* Tk = tile(k, k);
    float a[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) a[j] = Tk[lm * LDT + j];
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      float rowp[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) rowp[j] = rdlane(a[j], p);
      const float d = rowp[p];
      float r = __builtin_amdgcn_rcpf(d);
      r = __builtin_fmaf(r, __builtin_fmaf(-d, r, 1.f), r);  // one Newton step
      const bool me = lm == p;
      const float t = me ? 1.f - r : a[p] * r;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (j != p) a[j] = __builtin_fmaf(-t, rowp[j], a[j]);
      a[p] = me ? -r : t;
    }
    if (lane < 16) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        Tk[lm * LDT + j] = a[j];
        XS[lm * LDT + j] = -a[j];
      }
    }
  };

  // block rows of this wave: w, and with 8 blocks also 7 - w
  auto row_of = [&](int u) { return u == 0 ? wave : NB - 1 - wave; };
  f32x4 creg[RPW];
  // wave 0 sweeps the diagonal blocks (rotating it over the waves measured no
  // faster)
  if (wave == 0) leaf(0);
  __syncthreads();
  for (int k = 0; k < NB; ++k) {
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
      const int i = row_of(u);
      if (i >= NB || i == k) continue;
      // C_i^T = X P_ik^T on the k order 4 s + (lane / 16): lane l, register r
      // then holds C_i[l % 16][4 (l / 16) + r]
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      const float* Pik = i > k ? tile(i, k) : tile(k, i);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float xa = XS[lm * LDT + 4 * s + lg];
        const float pb = i > k ? Pik[lm * LDT + 4 * s + lg] : Pik[(4 * s + lg) * LDT + lm];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa, pb, acc, 0, 0, 0);
      }
      creg[u] = acc;
      // P_ij -= C_i P_kj for every lower tile (i, j), j != k, of this row; the
      // k order here is 4 (lane / 16) + s, so C_i's accumulator is the operand
      for (int j = 0; j <= i; ++j) {
        if (j == k) continue;
        float* Tij = tile(i, j);
        f32x4 c;
#pragma unroll
        for (int r = 0; r < 4; ++r) c[r] = Tij[(4 * lg + r) * LDT + lm];
        const float* Pkj = j < k ? tile(k, j) : tile(j, k);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float pb = j < k ? Pkj[(4 * lg + s) * LDT + lm] : Pkj[lm * LDT + 4 * lg + s];
          c = __builtin_amdgcn_mfma_f32_16x16x4f32(-creg[u][s], pb, c, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) Tij[(4 * lg + r) * LDT + lm] = c[r];
      }
    }
    __syncthreads();  // every read of block column k is done
    // P_ik <- C_i (stored as tile (i, k) for i > k, as tile (k, i) = C_i^T for i < k)
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
      const int i = row_of(u);
      if (i >= NB || i == k) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (i > k)
          tile(i, k)[lm * LDT + 4 * lg + r] = creg[u][r];
        else
          tile(k, i)[(4 * lg + r) * LDT + lm] = creg[u][r];
      }
    }
    if (k + 1 < NB && wave == 0) leaf(k + 1);
    __syncthreads();
  }

  // ---- out: P^{-1} = -(swept P), as bfloat16 hi + lo planes -------------------
  // fragment f = ((2w + e) (d/32) + s) 64 + l holds P^{-1}[32 s + 8 (l/16) + j]
  // [32 w + 2 (l%16) + e], j = 0..7; the symmetric element comes from the
  // lower tile that holds it
  constexpr int NFR = D * D / 8;
  constexpr int KS2 = D / 32;
  uint4* Fo = reinterpret_cast<uint4*>(Pout);
  for (int f = tid; f < NFR; f += 256) {
    const int fl = f & 63, ks = (f >> 6) % KS2, we = (f >> 6) / KS2;
    const int c = 32 * (we >> 1) + 2 * (fl & 15) + (we & 1);
    const int r0 = 32 * ks + 8 * (fl >> 4);
    const int R = r0 >> 4, rr = r0 & 15, Cb = c >> 4, cc = c & 15;
    float v[8];
    if (R >= Cb) {
      const float* Tp = tile(R, Cb);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = -Tp[(rr + j) * LDT + cc];
    } else {
      const float* Tp = tile(Cb, R);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = -Tp[cc * LDT + rr + j];
    }
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      __bf16 h0, l0, h1, l1;
      split_bf16(v[2 * e], h0, l0);
      split_bf16(v[2 * e + 1], h1, l1);
      hw[e] = __builtin_bit_cast(uint32_t, bf16x2{h0, h1});
      lw[e] = __builtin_bit_cast(uint32_t, bf16x2{l0, l1});
    }
    Fo[f] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    Fo[NFR + f] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  }
}

template <int D>
hipError_t launch_solve_d(const Problem& p, const float* stats, float* pinv, hipStream_t s) {
  const int n_video = p.T > 2 ? p.T - 2 : 0;
  const unsigned grid = (unsigned)(p.B * p.H * (n_video + 1));
  if constexpr (D >= 32) {
    if (pinv_split(p)) {
      hipLaunchKernelGGL(solve_sweep<D>, dim3(grid), dim3(256), 0, s, stats, pinv, p.H, p.T, n_video);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((solve_mfma<D, false>), dim3(grid), dim3(256), 0, s, stats, pinv, p.H, p.T, n_video);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_solve(const Problem& p, const float* stats, float* pinv, hipStream_t s) {
  switch (p.D) {
    case 16: return launch_solve_d<16>(p, stats, pinv, s);
    case 32: return launch_solve_d<32>(p, stats, pinv, s);
    case 64: return launch_solve_d<64>(p, stats, pinv, s);
    case 128: return launch_solve_d<128>(p, stats, pinv, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vda
