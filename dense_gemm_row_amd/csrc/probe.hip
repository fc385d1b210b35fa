// Measurement probes (not GEMMs): what the chip sustains with no memory
// traffic, and the shader clock, both read inside the kernel.
//
// * gemm_probe_mfma runs the GEMM kernels' matrix-core stream with its
//   operands in registers: one 256-thread workgroup per CU, each wave a
//   128 x 128 block of 32 x 32 accumulators (256 accumulator registers, the
//   default GEMM tiles' wave tile) fed by eight register fragments of
//   uniform [-1, 1) values in the instruction's element type, rotated so
//   that the multiplier inputs change on every instruction as in a GEMM.
//   Its rate is the ceiling of the matrix-core loop at the clock the power
//   limit allows for that instruction and that data.
// * gemm_probe_mfma16 runs the same stream with the 16 x 16 instructions of
//   the 16- and 8-bit types (8 x 8 blocks of 4 accumulators per wave, the
//   same 256 accumulator registers; the 8 + 8 fragments are all used once
//   per k step, which is twice the 32 x 32 step's k).
// * gemm_probe_clock spins a short dependent vector loop.
// Both record, per workgroup, the shader-cycle counter (s_memtime) and the
// 100 MHz constant clock (s_memrealtime) at start and end, so the clock a
// workgroup ran at is d(memtime) / d(realtime) x 100 MHz.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_probe.h"
#include "gemm_internal.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  // An integer hash (xorshift-multiply finaliser) for operand values.
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// uniform [-1, 1) on a 2^-23 grid
__device__ __forceinline__ float unit(uint32_t h) { return (float)(h >> 8) * (1.0f / 8388608.0f) - 1.0f; }

__device__ __forceinline__ void stamp(uint64_t* stamps, int slot) {
  const uint64_t t = __builtin_amdgcn_s_memtime();
  const uint64_t r = __builtin_amdgcn_s_memrealtime();
  // Lane 0 of wave 0 only, through ordinary (vector) stores.
  if (threadIdx.x == 0) {
    stamps[4 * blockIdx.x + 2 * slot] = t;
    stamps[4 * blockIdx.x + 2 * slot + 1] = r;
  }
}

// Operands per lane for one instruction: FP32 one float, 16-bit eight
// halves, FP8 32 bytes.
template <int TY> struct Op;
template <> struct Op<0> { typedef float T; };
template <> struct Op<1> { typedef gemm::h16x8_t T; };
template <> struct Op<2> { typedef gemm::h16x8_t T; };
template <> struct Op<3> { typedef gemm::i32x8_t T; };
template <> struct Op<4> { typedef gemm::i32x8_t T; };

template <int TY>
__device__ __forceinline__ typename Op<TY>::T make_op(uint32_t seed) {
  if constexpr (TY == 0) {
    return unit(mix32(seed));
  } else if constexpr (TY == 1 || TY == 2) {
    typename Op<TY>::T v;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = unit(mix32(seed * 8u + e));
      v[e] = TY == 1 ? (_Float16)x : __builtin_bit_cast(_Float16, gemm::round16<true>(x));
    }
    return v;
  } else {
    // FP8: bytes of uniform [-1, 1) values rounded to E4M3 (TY 3) or E5M2
    // (TY 4) by the hardware conversion.
    typename Op<TY>::T v;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const float x0 = unit(mix32(seed * 32u + 4 * w)), x1 = unit(mix32(seed * 32u + 4 * w + 1));
      const float x2 = unit(mix32(seed * 32u + 4 * w + 2)), x3 = unit(mix32(seed * 32u + 4 * w + 3));
      int p = 0;
      if constexpr (TY == 3) {
        p = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, p, false);
        p = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, p, true);
      } else {
        p = __builtin_amdgcn_cvt_pk_bf8_f32(x0, x1, p, false);
        p = __builtin_amdgcn_cvt_pk_bf8_f32(x2, x3, p, true);
      }
      v[w] = p;
    }
    return v;
  }
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int TY>
__device__ __forceinline__ f32x16 mma(typename Op<TY>::T a, typename Op<TY>::T b, f32x16 c) {
  if constexpr (TY == 0) return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  else if constexpr (TY == 1) return gemm::mfma16<false>(a, b, c);
  else if constexpr (TY == 2) return gemm::mfma16<true>(a, b, c);
  else return gemm::mfma_f8<TY - 3>(a, b, c);
}

// One k step = 16 instructions (the 4 x 4 blocks of a 128 x 128 wave tile).
constexpr int kFrags = 8;

template <int TY>
__global__ void __launch_bounds__(256) probe_mfma_kernel(int64_t steps, uint64_t* stamps, float* sink) {
  typedef typename Op<TY>::T T;
  const uint32_t base = (blockIdx.x * 256u + threadIdx.x) * 2u * kFrags;
  T fa[kFrags], fb[kFrags];
#pragma unroll
  for (int i = 0; i < kFrags; ++i) {
    fa[i] = make_op<TY>(base + i);
    fb[i] = make_op<TY>(base + kFrags + i);
  }
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  __syncthreads();
  stamp(stamps, 0);
  for (int64_t s = 0; s < steps; s += 2) {
    // Two k steps per trip, so every fragment index is static: step parity
    // q picks fragments 4q..4q+3 for the rows and columns.
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          acc[nb][mb] = mma<TY>(fb[4 * q + nb], fa[(4 * q + mb + nb) % kFrags], acc[nb][mb]);
  }
  stamp(stamps, 1);
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) t += acc[i][j][r];
  sink[blockIdx.x * 256 + threadIdx.x] = t;
}

// The 16 x 16 form: per trip, one k step of 64 instructions, the same
// flops as two 32 x 32 steps (FP32: v_mfma_f32_16x16x4_f32, k 4 against
// the 32 x 32 form's 2; the others twice the 32 x 32 form's k).  (No operand rotation across trips: with
// it the compiler moved accumulators between registers inside the loop.)
template <int TY>
__global__ void __launch_bounds__(256) probe_mfma16_kernel(int64_t steps, uint64_t* stamps, float* sink) {
  typedef typename Op<TY>::T T;
  const uint32_t base = (blockIdx.x * 256u + threadIdx.x) * 2u * kFrags;
  T fa[kFrags], fb[kFrags];
#pragma unroll
  for (int i = 0; i < kFrags; ++i) {
    fa[i] = make_op<TY>(base + i);
    fb[i] = make_op<TY>(base + kFrags + i);
  }
  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;
  __syncthreads();
  stamp(stamps, 0);
  for (int64_t s = 0; s < steps; s += 2) {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        if constexpr (TY == 0) acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x4f32(fb[nb], fa[mb], acc[nb][mb], 0, 0, 0);
        else if constexpr (TY == 1) acc[nb][mb] = gemm::mfma16<false>(fb[nb], fa[mb], acc[nb][mb]);
        else if constexpr (TY == 2) acc[nb][mb] = gemm::mfma16<true>(fb[nb], fa[mb], acc[nb][mb]);
        else acc[nb][mb] = gemm::mfma_f8<TY - 3>(fb[nb], fa[mb], acc[nb][mb]);
      }
  }
  stamp(stamps, 1);
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) t += acc[i][j][r];
  sink[blockIdx.x * 256 + threadIdx.x] = t;
}

__global__ void __launch_bounds__(64) probe_clock_kernel(int64_t iters, uint64_t* stamps, float* sink) {
  stamp(stamps, 0);
  float x = threadIdx.x * 1e-3f, y = 1.0001f;
  for (int64_t i = 0; i < iters; ++i) {
    x = __builtin_fmaf(x, y, 1e-7f);
    y = __builtin_fmaf(y, 0.99999f, 1e-6f);
  }
  stamp(stamps, 1);
  sink[blockIdx.x * 64 + threadIdx.x] = x + y;
}

}  // namespace

extern "C" {

int32_t gemm_probe_workgroups(void) { return 256; }

int32_t gemm_probe_mfma(int32_t dtype, int64_t steps, uint64_t* stamps, float* sink, void* stream) {
  if (steps < 0 || !stamps || !sink) return GEMM_ERR_INVALID_ARG;
  const dim3 grid(256), block(256);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case GEMM_DTYPE_F32: hipLaunchKernelGGL(probe_mfma_kernel<0>, grid, block, 0, s, steps, stamps, sink); break;
    case GEMM_DTYPE_F16: hipLaunchKernelGGL(probe_mfma_kernel<1>, grid, block, 0, s, steps, stamps, sink); break;
    case GEMM_DTYPE_BF16: hipLaunchKernelGGL(probe_mfma_kernel<2>, grid, block, 0, s, steps, stamps, sink); break;
    case GEMM_DTYPE_F8: hipLaunchKernelGGL(probe_mfma_kernel<3>, grid, block, 0, s, steps, stamps, sink); break;
    case GEMM_DTYPE_E5M2: hipLaunchKernelGGL(probe_mfma_kernel<4>, grid, block, 0, s, steps, stamps, sink); break;
    default: return GEMM_ERR_INVALID_ARG;
  }
  return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

int32_t gemm_probe_mfma16(int32_t dtype, int64_t steps, uint64_t* stamps, float* sink, void* stream) {
  if (steps < 0 || !stamps || !sink) return GEMM_ERR_INVALID_ARG;
  const dim3 grid(256), block(256);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case GEMM_DTYPE_F32: hipLaunchKernelGGL(probe_mfma16_kernel<0>, grid, block, 0, s, steps, stamps, sink); break;
    case GEMM_DTYPE_F16: hipLaunchKernelGGL(probe_mfma16_kernel<1>, grid, block, 0, s, steps, stamps, sink); break;
    case GEMM_DTYPE_BF16: hipLaunchKernelGGL(probe_mfma16_kernel<2>, grid, block, 0, s, steps, stamps, sink); break;
    case GEMM_DTYPE_F8: hipLaunchKernelGGL(probe_mfma16_kernel<3>, grid, block, 0, s, steps, stamps, sink); break;
    case GEMM_DTYPE_E5M2: hipLaunchKernelGGL(probe_mfma16_kernel<4>, grid, block, 0, s, steps, stamps, sink); break;
    default: return GEMM_ERR_INVALID_ARG;
  }
  return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

int32_t gemm_probe_clock(int64_t iters, uint64_t* stamps, float* sink, void* stream) {
  if (iters < 0 || !stamps || !sink) return GEMM_ERR_INVALID_ARG;
  hipLaunchKernelGGL(probe_clock_kernel, dim3(256), dim3(64), 0, static_cast<hipStream_t>(stream), iters,
                     stamps, sink);
  return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

}  // extern "C"
