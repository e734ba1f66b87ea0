// vda_pad: head widths between the kernels' tile widths.
//
// The kernels of the path tile the head width in 16- and 32-wide matrix-core
// blocks and are built for d = 16, 32, 64 and 128.  A forward pass at another
// multiple of 16 (48, 80, 96 or 112) runs them at the next built width D on
// copies of the caller's tensors whose channels d .. D-1 are zero.  Zero
// channels leave the method's result unchanged: with k and v zero there, A_t
// and B_t are zero outside their leading d x d blocks, I + A_t is the identity
// outside its block, S_T and every state stay zero outside theirs (a decay on
// zero columns keeps them zero, so those channels of alpha may be zero too),
// and o = S q is zero in channels d .. D-1, which are dropped when the output
// is copied back.  The epilogue's RMSNorm averages over the d true channels:
// sum o^2 / D + eps d / D = (d / D)(sum o^2 / d + eps), so the padded problem
// takes eps d / D and the gain gamma sqrt(d / D) (ones when none is given).
// The query's and the keys' L2 norms are unchanged by zero channels.
#include <algorithm>
#include <cmath>

#include "vda_internal.h"

namespace vda {
namespace {

// dst row r (dst_stride 16-byte chunks) = the first ncopy chunks of src row r
// (src_stride chunks apart), then zeros.  One thread per destination chunk,
// grid-stride; IDX is 32-bit where rows * dst_stride fits.
template <typename IDX>
__global__ __launch_bounds__(256) void copy_rows(const uint4* __restrict__ src, IDX src_stride,
                                                 uint4* __restrict__ dst, IDX dst_stride, IDX ncopy, IDX n) {
  for (IDX i = (IDX)blockIdx.x * 256 + threadIdx.x; i < n; i += (IDX)gridDim.x * 256) {
    const IDX r = i / dst_stride, c = i - r * dst_stride;
    dst[i] = c < ncopy ? src[r * src_stride + c] : make_uint4(0, 0, 0, 0);
  }
}

// The padded problem's gain: (w ? w[j] : 1) * scale for j < d, zero for
// d <= j < D.  One workgroup of 128 threads (D <= 128).
__global__ __launch_bounds__(128) void pad_gain(const float* __restrict__ w, float* __restrict__ dst, int d, int D,
                                                float scale) {
  const int j = threadIdx.x;
  if (j < D) dst[j] = j < d ? (w ? w[j] : 1.f) * scale : 0.f;
}

}  // namespace

hipError_t launch_copy_rows(const void* src, size_t src_row_bytes, void* dst, size_t dst_row_bytes,
                            size_t copy_bytes, size_t rows, hipStream_t s) {
  const size_t ss = src_row_bytes / 16, ds = dst_row_bytes / 16, nc = copy_bytes / 16;
  const size_t n = rows * ds;
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<size_t>((n + 255) / 256, 16384);
  const uint4* sp = static_cast<const uint4*>(src);
  uint4* dp = static_cast<uint4*>(dst);
  if (n + (size_t)grid * 256 < ((size_t)1 << 32))
    hipLaunchKernelGGL(copy_rows<uint32_t>, dim3(grid), dim3(256), 0, s, sp, (uint32_t)ss, dp, (uint32_t)ds,
                       (uint32_t)nc, (uint32_t)n);
  else
    hipLaunchKernelGGL(copy_rows<uint64_t>, dim3(grid), dim3(256), 0, s, sp, (uint64_t)ss, dp, (uint64_t)ds,
                       (uint64_t)nc, (uint64_t)n);
  return hipGetLastError();
}

hipError_t launch_pad_gain(const float* w, float* dst, int d, int D, hipStream_t s) {
  const float scale = std::sqrt((float)d / (float)D);
  hipLaunchKernelGGL(pad_gain, dim3(1), dim3(128), 0, s, w, dst, d, D, scale);
  return hipGetLastError();
}

}  // namespace vda
