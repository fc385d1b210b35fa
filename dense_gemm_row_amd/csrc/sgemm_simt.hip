// FP32 SGEMM on the vector ALUs (no matrix cores): the ablation that mirrors
// the final kernel of "sgemm - beyond cuBLAS" (section 6: 128x128 block
// tile, BK = 16, 256 threads, 8x8 outputs per thread, transposed and
// swizzled A tile, split 4+4 column ownership for coalesced stores, two
// shared-memory buffers with one barrier per K step), re-derived for
// 64-lane waves and the 64-bank LDS of gfx950.
//
// * Threads: tx = tid % 16, ty = tid / 16.  Thread (ty, tx) owns rows
//   {4ty..4ty+3} and {64+4ty..64+4ty+3} and columns {4tx..4tx+3} and
//   {64+4tx..64+4tx+3} of the tile.  A wave holds 4 values of ty and all 16
//   of tx, so its A reads are 4 broadcast addresses and its B reads one
//   contiguous 256-byte run per half.
// * A tile stored transposed, As[k][m]: each thread loads 4 consecutive k of
//   one row with a 16-byte load and stores them as 4 scalars down a column.
//   Writing column m of row k at position m ^ (16 * (k / 4)) spreads the 64
//   lanes of one scalar store (16 rows m, 4 chunks k/4) over all 64 banks;
//   the XOR only touches bits 4-5 of the column, so the 16-byte reads of 4
//   consecutive m stay contiguous and inside their half of the row.  (The
//   page's version, col ^ ((row >> 2) << 3), is the same idea for 32 banks
//   and 32-lane warps.)
// * Accumulation with scalar v_fma_f32: the build disables packed FP32
//   instructions, so the vector-ALU ceiling of this kernel is half of the
//   packed FP32 rate.
#include "gemm_internal.h"

namespace gemm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 16, NT = 256;
constexpr int A_STAGE = BK * BM, B_STAGE = BK * BN, STAGE = A_STAGE + B_STAGE;  // floats
constexpr int LDS_BYTES = 2 * STAGE * 4;

__host__ __device__ constexpr int a_pos(int k, int m) { return k * BM + (m ^ (16 * (k >> 2))); }
__host__ __device__ constexpr int b_pos(int k, int n) { return A_STAGE + k * BN + n; }

template <bool VEC>
__global__ void __launch_bounds__(NT) sgemm_simt_kernel(Params p, TileMap map) {
  __shared__ __attribute__((aligned(16))) float smem[2 * STAGE];

  int tm, tn;
  tile_of_block(blockIdx.x, map, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int M = p.M, N = p.N, K = p.K;
  const float* __restrict__ A = static_cast<const float*>(p.A);
  const float* __restrict__ B = static_cast<const float*>(p.B);
  float* __restrict__ C = static_cast<float*>(p.C);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;

  // Staging: two A chunks (row m, 4 k) and two B chunks (row k, 4 n).
  int a_m[2], a_q[2], b_k[2], b_n[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int id = tid + i * NT;
    a_m[i] = id >> 2;
    a_q[i] = id & 3;
    b_k[i] = id >> 5;
    b_n[i] = 4 * (id & 31);
  }
  f32x4 ra[2], rb[2];

  auto load_slice = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int gm = m0 + a_m[i], gk = k0 + 4 * a_q[i];
      const float* src = A + (int64_t)(gm < M ? gm : 0) * p.lda + gk;
      if (VEC) {
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (gm < M && gk < K) v = *reinterpret_cast<const f32x4*>(src);
        ra[i] = v;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) ra[i][e] = (gm < M && gk + e < K) ? src[e] : 0.f;
      }
      const int gk2 = k0 + b_k[i], gn = n0 + b_n[i];
      const float* bsrc = B + (int64_t)(gk2 < K ? gk2 : 0) * p.ldb + gn;
      if (VEC) {
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (gk2 < K && gn < N) v = *reinterpret_cast<const f32x4*>(bsrc);
        rb[i] = v;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) rb[i][e] = (gk2 < K && gn + e < N) ? bsrc[e] : 0.f;
      }
    }
  };
  auto store_slice = [&](int stage) {
    float* s = smem + stage * STAGE;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) s[a_pos(4 * a_q[i] + e, a_m[i])] = ra[i][e];
      *reinterpret_cast<f32x4*>(s + b_pos(b_k[i], b_n[i])) = rb[i];
    }
  };

  float acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;

  const int T = (K + BK - 1) / BK;
  if (T > 0) {
    load_slice(0);
    store_slice(0);
    __syncthreads();
    for (int t = 0; t < T; ++t) {
      const int cur = t & 1;
      if (t + 1 < T) load_slice((t + 1) * BK);
      const float* s = smem + cur * STAGE;
#pragma unroll
      for (int k = 0; k < BK; ++k) {
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(s + a_pos(k, 4 * ty));
        const f32x4 a1 = *reinterpret_cast<const f32x4*>(s + a_pos(k, 64 + 4 * ty));
        const f32x4 b0 = *reinterpret_cast<const f32x4*>(s + b_pos(k, 4 * tx));
        const f32x4 b1 = *reinterpret_cast<const f32x4*>(s + b_pos(k, 64 + 4 * tx));
        const float av[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        const float bv[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
      }
      if (t + 1 < T) store_slice(cur ^ 1);
      __syncthreads();
    }
  }

#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = m0 + (i < 4 ? 4 * ty + i : 64 + 4 * ty + (i - 4));
    if (row >= M) continue;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int col = n0 + 64 * half + 4 * tx;
      float* dst = C + (int64_t)row * p.ldc + col;
      if (VEC) {
        if (col < N) {
          f32x4 v = {acc[i][4 * half], acc[i][4 * half + 1], acc[i][4 * half + 2], acc[i][4 * half + 3]};
          *reinterpret_cast<f32x4*>(dst) = v;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (col + e < N) dst[e] = acc[i][4 * half + e];
      }
    }
  }
}

hipError_t launch(const Params& p, const TileMap& map, bool vec, hipStream_t stream) {
  const dim3 grid(map.tiles_m * map.tiles_n), block(NT);
  if (vec)
    hipLaunchKernelGGL(sgemm_simt_kernel<true>, grid, block, 0, stream, p, map);
  else
    hipLaunchKernelGGL(sgemm_simt_kernel<false>, grid, block, 0, stream, p, map);
  return hipGetLastError();
}

int layout_check(int banks, int64_t out[2]) {
  int64_t wconf = 0, rconf = 0;
  static unsigned char cover[STAGE * 4];
  for (int i = 0; i < STAGE * 4; ++i) cover[i] = 0;
  int addr[64];
  for (int i = 0; i < 2; ++i)
    for (int w = 0; w < NT / 64; ++w) {
      for (int e = 0; e < 4; ++e) {
        for (int l = 0; l < 64; ++l) {
          const int id = w * 64 + l + i * NT;
          const int off = 4 * a_pos(4 * (id & 3) + e, id >> 2);
          if (off < 0 || off + 4 > A_STAGE * 4) return 1;
          for (int b = 0; b < 4; ++b) cover[off + b]++;
          addr[l] = off;
        }
        wconf += lds_conflicts(addr, 4, banks);
      }
      for (int l = 0; l < 64; ++l) {
        const int id = w * 64 + l + i * NT;
        const int off = 4 * b_pos(id >> 5, 4 * (id & 31));
        if (off < A_STAGE * 4 || off + 16 > STAGE * 4) return 2;
        for (int b = 0; b < 16; ++b) cover[off + b]++;
        addr[l] = off;
      }
      wconf += lds_conflicts(addr, 16, banks);
    }
  for (int i = 0; i < STAGE * 4; ++i)
    if (cover[i] != 1) return 3;
  for (int w = 0; w < NT / 64; ++w)
    for (int k = 0; k < BK; ++k)
      for (int part = 0; part < 4; ++part) {
        for (int l = 0; l < 64; ++l) {
          const int tid = w * 64 + l, tx = tid & 15, ty = tid >> 4;
          int off;
          if (part == 0) off = 4 * a_pos(k, 4 * ty);
          else if (part == 1) off = 4 * a_pos(k, 64 + 4 * ty);
          else if (part == 2) off = 4 * b_pos(k, 4 * tx);
          else off = 4 * b_pos(k, 64 + 4 * tx);
          if (off < 0 || off + 16 > STAGE * 4) return 4;
          addr[l] = off;
        }
        rconf += lds_conflicts(addr, 16, banks);
      }
  // The swizzle must keep each thread's 4 rows contiguous in one row half.
  for (int k = 0; k < BK; ++k)
    for (int m = 0; m < BM; m += 4)
      for (int e = 1; e < 4; ++e)
        if (a_pos(k, m + e) != a_pos(k, m) + e) return 5;
  out[0] = wconf;
  out[1] = rconf;
  return 0;
}

const Variant kVariants[] = {
    Variant{gemm_config_t{0, GEMM_DTYPE_F32, GEMM_FAMILY_SIMT, BM, BN, BK, 8, 8, NT, 2, LDS_BYTES,
                          GEMM_ORDER_XCD, 8, 1, "simt_f32_128x128x16_t8x8"},
            &launch, &layout_check, nullptr, 0.32f},
};

}  // namespace

const Variant* sgemm_simt_variants(int* count) {
  *count = sizeof(kVariants) / sizeof(kVariants[0]);
  return kVariants;
}

}  // namespace gemm
