// Split-K reduction: C[i][j] = sum_{s=0}^{S-1} W[s][i][j], summed in chunk
// order s = 0, 1, ..., S-1 in FP32 (so the result is the same on every run),
// then written as FP32, or as FP16 or BF16 with one round-to-nearest-even.
//
// W holds the S partial products of a split-K GEMM, each an M x N FP32
// matrix with leading dimension N, planes M*N floats apart.  The kernel is
// a streaming pass bound by HBM: S*M*N*4 bytes read, M*N*(4 or 2) written,
// nothing reused, so it is laid out for coalescing only: each thread owns
// four consecutive columns of one row (one 16-byte load per plane), and
// consecutive threads take consecutive column groups of the row-major
// matrices.  The scalar form handles N or C not aligned to 4 elements.
#include "gemm_internal.h"

namespace gemm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// Output element: FP32, FP16 or BF16.
enum Out { kF32 = 0, kF16 = 1, kBF16 = 2 };

template <int OUT>
__global__ void __launch_bounds__(kThreads)
splitk_reduce_vec(const float* __restrict__ W, int S, int M, int N, void* C, int64_t ldc) {
  const int64_t groups = (int64_t)N / 4;
  const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (g >= (int64_t)M * groups) return;
  const int64_t row = g / groups, c4 = g - row * groups;
  const int64_t plane = (int64_t)M * N;
  const float* w = W + row * N + 4 * c4;
  f32x4 acc = *reinterpret_cast<const f32x4*>(w);
  for (int s = 1; s < S; ++s) acc += *reinterpret_cast<const f32x4*>(w + s * plane);
  if constexpr (OUT != kF32) {
    typedef half_t<OUT == kBF16> H;
    typedef H h16x4 __attribute__((ext_vector_type(4)));
    h16x4 h = {(H)acc[0], (H)acc[1], (H)acc[2], (H)acc[3]};
    *reinterpret_cast<h16x4*>(static_cast<H*>(C) + row * ldc + 4 * c4) = h;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(C) + row * ldc + 4 * c4) = acc;
  }
}

template <int OUT>
__global__ void __launch_bounds__(kThreads)
splitk_reduce_scalar(const float* __restrict__ W, int S, int M, int N, void* C, int64_t ldc) {
  const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (e >= (int64_t)M * N) return;
  const int64_t row = e / N, col = e - row * N;
  const int64_t plane = (int64_t)M * N;
  float acc = W[e];
  for (int s = 1; s < S; ++s) acc += W[e + s * plane];
  if constexpr (OUT != kF32)
    static_cast<unsigned short*>(C)[row * ldc + col] = round16<OUT == kBF16>(acc);
  else
    static_cast<float*>(C)[row * ldc + col] = acc;
}

}  // namespace

hipError_t splitk_reduce(int dtype, const float* W, int S, int M, int N, void* C, int64_t ldc,
                         hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const bool f16 = dtype != GEMM_DTYPE_F32;  // a 16-bit output
  const uintptr_t align = f16 ? 8 : 16;    // bytes of one 4-element store
  const bool vec = N % 4 == 0 && ldc % 4 == 0 && ((uintptr_t)C % align) == 0 &&
                   ((uintptr_t)W % 16) == 0;
  const int64_t work = vec ? (int64_t)M * (N / 4) : (int64_t)M * N;
  const dim3 grid((unsigned)((work + kThreads - 1) / kThreads)), block(kThreads);
  if (vec) {
    if (dtype == GEMM_DTYPE_BF16)
      hipLaunchKernelGGL(splitk_reduce_vec<kBF16>, grid, block, 0, stream, W, S, M, N, C, ldc);
    else if (f16)
      hipLaunchKernelGGL(splitk_reduce_vec<kF16>, grid, block, 0, stream, W, S, M, N, C, ldc);
    else
      hipLaunchKernelGGL(splitk_reduce_vec<kF32>, grid, block, 0, stream, W, S, M, N, C, ldc);
  } else {
    if (dtype == GEMM_DTYPE_BF16)
      hipLaunchKernelGGL(splitk_reduce_scalar<kBF16>, grid, block, 0, stream, W, S, M, N, C, ldc);
    else if (f16)
      hipLaunchKernelGGL(splitk_reduce_scalar<kF16>, grid, block, 0, stream, W, S, M, N, C, ldc);
    else
      hipLaunchKernelGGL(splitk_reduce_scalar<kF32>, grid, block, 0, stream, W, S, M, N, C, ldc);
  }
  return hipGetLastError();
}

}  // namespace gemm
