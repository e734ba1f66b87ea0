// vda_solve: (I + A_t)^{-1} for every frame of every head, by Cholesky.
//
// The frame update S_t = (S_{t-1} Diag(alpha_t) + B_t)(I + A_t)^{-1} is solved in
// the d_k x d_k key space ("Video DeltaNet" summary, onedev.kr/papers/80, section
// "어떻게 쓰나"); the VDN-H3 write-up (discuss.pytorch.kr, hybrid attention
// structure) notes that A_t is positive semidefinite, so P_t = I + A_t is
// symmetric positive definite and has a Cholesky factor.  One workgroup
// inverts one P_t:
//   1. P = L L^T            right-looking blocked Cholesky, 8x8 blocks
//   2. Y = L^{-1}           blocked forward substitution on the identity
//   3. P^{-1} = Y^T Y       accumulated over block rows of Y
// The matrix is distributed as 8x8 register blocks over (d/8)^2 threads; each
// block step broadcasts one block column (or row) through LDS, so every
// trailing update is a register-resident rank-8 update.  Everything is fp32.
// The scan consumes P^{-1} directly: S M_t + J_t = (S Diag(alpha_t) + B_t) P^{-1},
// so neither M_t nor J_t is ever formed in memory.
#include "vda_internal.h"

namespace vda {
namespace {

constexpr int PAD = 68;  // floats per 8x8 block in LDS (64 + 4 avoids bank conflicts)

template <int D>
__global__ __launch_bounds__((D / 8) * (D / 8) > 64 ? (D / 8) * (D / 8) : 64)
void solve_chol(const float* __restrict__ stats, float* __restrict__ pinv, int H, int T,
                int n_video) {
  constexpr int NT = D / 8;
  constexpr int NTH = NT * NT;
  __shared__ __attribute__((aligned(16))) float sdiag[64];
  __shared__ __attribute__((aligned(16))) float scol[2][NT][PAD];  // L blocks, transposed [m][r]
  __shared__ __attribute__((aligned(16))) float srow[2][NT][PAD];  // Y blocks, row-major [m][c]

  const int tid = threadIdx.x;
  const int n_slots = n_video + 1;
  int blk = blockIdx.x;
  const int si = blk % n_slots;
  blk /= n_slots;
  const int h = blk % H;
  const int b = blk / H;
  const int slot = (si < n_video) ? 1 + si : T;  // video frames 1..T-2, then the text slot T
  const size_t mat = (size_t)(b * H + h) * (T + 1) + slot;
  const float* A = stats + mat * (size_t)(2 * D * D);
  float* P = pinv + mat * (size_t)(D * D);

  const bool active = tid < NTH;
  const int ti = active ? tid / NT : 0, tj = active ? tid % NT : 0;

  float a[8][8];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) a[r][c] = 0.f;
  if (active && ti >= tj) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const float4* src = reinterpret_cast<const float4*>(A + (8 * ti + r) * D + 8 * tj);
      const float4 x0 = src[0], x1 = src[1];
      a[r][0] = x0.x; a[r][1] = x0.y; a[r][2] = x0.z; a[r][3] = x0.w;
      a[r][4] = x1.x; a[r][5] = x1.y; a[r][6] = x1.z; a[r][7] = x1.w;
    }
    if (ti == tj) {
#pragma unroll
      for (int r = 0; r < 8; ++r) a[r][r] += 1.f;
    }
  }

  // ---- 1. Cholesky: P = L L^T (lower), block column by block column ----------
  for (int p = 0; p < NT; ++p) {
    if (active && ti == p && tj == p) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float d = __builtin_sqrtf(a[j][j]);
        const float inv = 1.f / d;
        a[j][j] = d;
#pragma unroll
        for (int i = j + 1; i < 8; ++i) a[i][j] *= inv;
#pragma unroll
        for (int i = j + 1; i < 8; ++i)
#pragma unroll
          for (int c = j + 1; c <= i; ++c) a[i][c] -= a[i][j] * a[c][j];
      }
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = r + 1; c < 8; ++c) a[r][c] = 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) sdiag[r * 8 + c] = a[r][c];
    }
    __syncthreads();
    if (active && tj == p && ti > p) {
      // X L_pp^T = A_ip, solved row by row
      float invd[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) invd[c] = 1.f / sdiag[c * 8 + c];
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float x = a[r][c];
#pragma unroll
          for (int m = 0; m < c; ++m) x -= a[r][m] * sdiag[c * 8 + m];
          a[r][c] = x * invd[c];
        }
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int r = 0; r < 8; ++r) scol[0][ti][m * 8 + r] = a[r][m];
    }
    __syncthreads();
    if (active && ti > p && tj > p && ti >= tj) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float4* li = reinterpret_cast<const float4*>(&scol[0][ti][m * 8]);
        const float4* lj = reinterpret_cast<const float4*>(&scol[0][tj][m * 8]);
        const float4 i0 = li[0], i1 = li[1], j0 = lj[0], j1 = lj[1];
        const float vi[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
        const float vj[8] = {j0.x, j0.y, j0.z, j0.w, j1.x, j1.y, j1.z, j1.w};
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
          for (int c = 0; c < 8; ++c) a[r][c] -= vi[r] * vj[c];
      }
    }
  }
  __syncthreads();

  // ---- 2. Y = L^{-1} (lower), block row by block row -------------------------
  float y[8][8];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) y[r][c] = (active && ti == tj && r == c) ? 1.f : 0.f;
  for (int p = 0; p < NT; ++p) {
    const int pb = p & 1;
    if (active && tj == p && ti >= p) {
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int r = 0; r < 8; ++r) scol[pb][ti][m * 8 + r] = a[r][m];
    }
    __syncthreads();
    if (active && ti == p && tj <= p) {
      const float* L = scol[pb][p];  // L[r][m] = L[m * 8 + r]
      float invd[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) invd[r] = 1.f / L[r * 8 + r];
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          float x = y[r][c];
#pragma unroll
          for (int m = 0; m < r; ++m) x -= L[m * 8 + r] * y[m][c];
          y[r][c] = x * invd[r];
        }
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) srow[0][tj][r * 8 + c] = y[r][c];
    }
    __syncthreads();
    if (active && ti > p && tj <= p) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float4* li = reinterpret_cast<const float4*>(&scol[pb][ti][m * 8]);
        const float4* yj = reinterpret_cast<const float4*>(&srow[0][tj][m * 8]);
        const float4 i0 = li[0], i1 = li[1], j0 = yj[0], j1 = yj[1];
        const float vi[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
        const float vj[8] = {j0.x, j0.y, j0.z, j0.w, j1.x, j1.y, j1.z, j1.w};
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
          for (int c = 0; c < 8; ++c) y[r][c] -= vi[r] * vj[c];
      }
    }
  }
  __syncthreads();

  // ---- 3. P^{-1} = Y^T Y, one block row of Y at a time ------------------------
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) a[r][c] = 0.f;
  for (int k = 0; k < NT; ++k) {
    const int kb = k & 1;
    if (active && ti == k && tj <= k) {
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) srow[kb][tj][r * 8 + c] = y[r][c];
    }
    __syncthreads();
    if (active && ti <= k && tj <= k) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float4* yi = reinterpret_cast<const float4*>(&srow[kb][ti][m * 8]);
        const float4* yj = reinterpret_cast<const float4*>(&srow[kb][tj][m * 8]);
        const float4 i0 = yi[0], i1 = yi[1], j0 = yj[0], j1 = yj[1];
        const float vi[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
        const float vj[8] = {j0.x, j0.y, j0.z, j0.w, j1.x, j1.y, j1.z, j1.w};
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
          for (int c = 0; c < 8; ++c) a[r][c] += vi[r] * vj[c];
      }
    }
  }
  if (active) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      float4* dst = reinterpret_cast<float4*>(P + (8 * ti + r) * D + 8 * tj);
      dst[0] = make_float4(a[r][0], a[r][1], a[r][2], a[r][3]);
      dst[1] = make_float4(a[r][4], a[r][5], a[r][6], a[r][7]);
    }
  }
}

template <int D>
hipError_t launch_solve_d(const Problem& p, const float* stats, float* pinv, hipStream_t s) {
  const int n_video = p.T > 2 ? p.T - 2 : 0;
  const unsigned grid = (unsigned)(p.B * p.H * (n_video + 1));
  constexpr int threads = (D / 8) * (D / 8) > 64 ? (D / 8) * (D / 8) : 64;
  hipLaunchKernelGGL(solve_chol<D>, dim3(grid), dim3(threads), 0, s, stats, pinv, p.H, p.T, n_video);
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
