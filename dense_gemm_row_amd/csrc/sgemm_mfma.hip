// FP32 SGEMM on the gfx950 matrix cores: C = A x B, row-major, FP32 in/out.
//
// Design (the ideas of the SIMT ladder in "sgemm - beyond cuBLAS", sections
// 2-6, and the register blocking of "GEMM: from naive to shared memory
// tiling and register blocking", section 3, re-done for CDNA4 matrix cores):
//
// * Workgroup tile BM x BN, K consumed in slices of BK.  The grid is 1-D;
//   tile_of_block maps workgroup ids to tiles (row order, banded, or banded
//   after gathering each XCD's workgroups).
// * Waves: (BM/WM) x (BN/WN) waves of 64 lanes, each owning a WM x WN wave
//   tile made of (WM/32) x (WN/32) blocks of v_mfma_f32_32x32x2_f32.
// * Operand lane maps of v_mfma_f32_32x32x2_f32 (checked on the device):
//   lane l supplies A[l%32][l/32] and B[l/32][l%32]; accumulator register r
//   of lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.
// * K permutation: the sum over k is order-free, so within each group of 8
//   consecutive k the MFMA step s (0..3) feeds lane half h the physical
//   k = 4h + s.  Then one 16-byte LDS read gives a lane its A values for 4
//   steps (A tile row-major, K contiguous), with no transposed store.
// * Column interleave: block nb of a wave tile covers the columns
//   wn0 + NB*j + nb (j = 0..31, NB = WN/32), so one lane reads NB adjacent
//   B values per step (one 4*NB-byte LDS read) and, in the epilogue, owns
//   NB adjacent output columns of each row it holds: direct 4*NB-byte
//   stores, 32 lanes covering 128*NB contiguous bytes of a row (the
//   coalesced write-back of section 5, without an LDS round trip).
// * LDS: A tile BM x BK row-major with the chunk XOR swizzle swz_row (rows of
//   BK*4 bytes), B tile BK x BN row-major (reads and writes are contiguous
//   runs, conflict-free without a swizzle).  Two stages: the next slice is
//   loaded from global memory into registers while the current stage feeds
//   the MFMAs, then stored to the other stage; one barrier per slice (the
//   double buffer of section 6).
// * Edges: rows/columns beyond M/N and k beyond K load as zero; stores are
//   masked.  VEC=true assumes 16-byte aligned A, B, C, and K, N, lda, ldb,
//   ldc multiples of 4 (128-bit global loads, whole-chunk masks); VEC=false
//   loads and stores element by element.
#include "gemm_internal.h"

namespace gemm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int NB> struct VecF;
template <> struct VecF<1> { typedef float T; };
template <> struct VecF<2> { typedef f32x2 T; };
template <> struct VecF<4> { typedef f32x4 T; };

template <int BM, int BN, int BK, int WM, int WN>
struct Shape {
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int NT = WAVES_M * WAVES_N * 64;
  static constexpr int MB = WM / 32, NB = WN / 32;
  static constexpr int A_ROW_BYTES = BK * 4;
  static constexpr int A_CHUNKS = BM * BK / 4;  // 16-byte chunks per stage
  static constexpr int B_CHUNKS = BK * BN / 4;
  static constexpr int CA = A_CHUNKS / NT, CB = B_CHUNKS / NT;
  static constexpr int A_STAGE = BM * BK, B_STAGE = BK * BN;  // floats
  static constexpr int STAGE = A_STAGE + B_STAGE;
  static constexpr int LDS_BYTES = 2 * STAGE * 4;
  static_assert(BM % WM == 0 && BN % WN == 0, "wave grid");
  static_assert(WM % 32 == 0 && (NB == 1 || NB == 2 || NB == 4), "wave tile");
  static_assert(BK % 8 == 0 && BK >= 8, "K slice");
  static_assert(A_CHUNKS % NT == 0 && B_CHUNKS % NT == 0, "staging split");
  static_assert((BN / 4) % 16 == 0, "B rows are written by whole 16-lane groups");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");

  // LDS float offset of A chunk (row r, chunk q) and of B chunk (row k, nq).
  __host__ __device__ static constexpr int a_chunk(int r, int q) {
    return swz_off(r, q, A_ROW_BYTES) / 4;
  }
  __host__ __device__ static constexpr int b_chunk(int k, int nq) { return k * BN + 4 * nq; }
  // A fragment read of wave row block: lane reads chunk (kk/4 + h) of row r.
  __host__ __device__ static constexpr int a_frag(int r, int kk, int h) {
    return swz_off(r, kk / 4 + h, A_ROW_BYTES) / 4;
  }
  __host__ __device__ static constexpr int b_frag(int kk, int h, int s, int col) {
    return (kk + 4 * h + s) * BN + col;
  }
};

__device__ inline f32x16 mfma(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// BT: B given transposed (p.bt: Bt, N x K row-major).  A thread loads four
// consecutive k of one column (one 16-byte load in VEC form) and stores them
// down that column of the row-major B tile; consecutive lanes take
// consecutive columns, so each 4-byte store of a wave covers 64 banks.
template <int BM, int BN, int BK, int WM, int WN, bool VEC, bool EPI, bool BT>
__global__ void __launch_bounds__((Shape<BM, BN, BK, WM, WN>::NT))
sgemm_mfma_kernel(Params p, TileMap map) {
  using S = Shape<BM, BN, BK, WM, WN>;
  constexpr int NT = S::NT, MB = S::MB, NB = S::NB, CA = S::CA, CB = S::CB;
  typedef typename VecF<NB>::T vecNB;

  __shared__ __attribute__((aligned(16))) float smem[2 * S::STAGE];

  int tm, tn;
  tile_of_block(blockIdx.x, map, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int M = p.M, N = p.N, K = p.K;
  const float* __restrict__ A = static_cast<const float*>(p.A);
  const float* __restrict__ B = static_cast<const float*>(p.B);
  float* __restrict__ C = static_cast<float*>(p.C);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 31, h = lane >> 5;
  const int wm0 = (wave / S::WAVES_N) * WM, wn0 = (wave % S::WAVES_N) * WN;

  // Per-thread staging assignment (fixed over the K loop).
  const float* a_src[CA];
  bool a_row_ok[CA];
  int a_kq[CA], a_dst[CA];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int id = tid + i * NT;
    const int r = id / (BK / 4), q = id % (BK / 4);
    a_row_ok[i] = (m0 + r) < M;
    a_src[i] = A + (int64_t)(a_row_ok[i] ? m0 + r : 0) * p.lda + 4 * q;
    a_kq[i] = 4 * q;
    a_dst[i] = S::a_chunk(r, q);
  }
  const float* b_src[CB];
  int b_k[CB], b_col[CB], b_dst[CB];
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int id = tid + i * NT;
    const int k = id / (BN / 4), nq = id % (BN / 4);
    b_k[i] = k;
    b_col[i] = n0 + 4 * nq;
    b_src[i] = B + (int64_t)k * p.ldb + (b_col[i] < N ? b_col[i] : 0);
    b_dst[i] = S::b_chunk(k, nq);
  }

  // BT staging: (column n, k chunk q) per slot.
  const float* bt_src[CB];
  bool bt_ok[CB];
  int bt_k[CB], bt_dst[CB];
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int id = tid + i * NT;
    const int n = id % BN, q = id / BN;
    bt_ok[i] = (n0 + n) < N;
    bt_src[i] = B + (int64_t)(bt_ok[i] ? n0 + n : 0) * p.ldb + 4 * q;
    bt_k[i] = 4 * q;
    bt_dst[i] = (4 * q) * BN + n;
  }

  f32x4 ra[CA], rb[CB];

  auto load_slice = [&](int k0) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int kg = k0 + a_kq[i];
      if (VEC) {
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (a_row_ok[i] && kg < K) v = *reinterpret_cast<const f32x4*>(a_src[i] + k0);
        ra[i] = v;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          ra[i][e] = (a_row_ok[i] && kg + e < K) ? a_src[i][k0 + e] : 0.f;
      }
    }
    if constexpr (BT) {
#pragma unroll
      for (int i = 0; i < CB; ++i) {
        const int kg = k0 + bt_k[i];
        if (VEC) {
          f32x4 v = {0.f, 0.f, 0.f, 0.f};
          if (bt_ok[i] && kg < K) v = *reinterpret_cast<const f32x4*>(bt_src[i] + k0);
          rb[i] = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) rb[i][e] = (bt_ok[i] && kg + e < K) ? bt_src[i][k0 + e] : 0.f;
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int kg = k0 + b_k[i];
      const float* src = b_src[i] + (int64_t)k0 * p.ldb;
      if (VEC) {
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (kg < K && b_col[i] < N) v = *reinterpret_cast<const f32x4*>(src);
        rb[i] = v;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          rb[i][e] = (kg < K && b_col[i] + e < N) ? src[e] : 0.f;
      }
    }
  };

  auto store_slice = [&](int stage) {
    float* As = smem + stage * S::STAGE;
    float* Bs = As + S::A_STAGE;
#pragma unroll
    for (int i = 0; i < CA; ++i) *reinterpret_cast<f32x4*>(As + a_dst[i]) = ra[i];
    if constexpr (BT) {
#pragma unroll
      for (int i = 0; i < CB; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) Bs[bt_dst[i] + e * BN] = rb[i][e];
      return;
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) *reinterpret_cast<f32x4*>(Bs + b_dst[i]) = rb[i];
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.f;

  const int T = (K + BK - 1) / BK;
  if (T > 0) {
    load_slice(0);
    store_slice(0);
    __syncthreads();
    for (int t = 0; t < T; ++t) {
      const int cur = t & 1;
      if (t + 1 < T) load_slice((t + 1) * BK);
      const float* As = smem + cur * S::STAGE;
      const float* Bs = As + S::A_STAGE;
#pragma unroll
      for (int kk = 0; kk < BK; kk += 8) {
        f32x4 a[MB];
        vecNB b[4];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          a[mb] = *reinterpret_cast<const f32x4*>(As + S::a_frag(wm0 + 32 * mb + lrow, kk, h));
#pragma unroll
        for (int s = 0; s < 4; ++s)
          b[s] = *reinterpret_cast<const vecNB*>(Bs + S::b_frag(kk, h, s, wn0 + NB * lrow));
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              float bv;
              if constexpr (NB == 1) bv = b[s]; else bv = b[s][nb];
              acc[mb][nb] = mfma(a[mb][s], bv, acc[mb][nb]);
            }
      }
      if (t + 1 < T) store_slice(cur ^ 1);
      __syncthreads();
    }
  }

  // Epilogue: lane owns NB adjacent columns of each of its rows.  EPI:
  // the fused epilogue (alpha, beta with the old C, bias, activation) on
  // the FP32 accumulators before the store.
  const int col = n0 + wn0 + NB * lrow;
  auto out = [&](int mb, int nb, int r, const float* dst) -> float {
    if constexpr (!EPI) {
      return acc[mb][nb][r];
    } else {
      const float c_old = p.epi.beta != 0.f ? dst[nb] : 0.f;
      const float bias = p.epi.bias ? p.epi.bias[col + nb] : 0.f;
      return epi_value(p.epi, acc[mb][nb][r], c_old, bias);
    }
  };
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm0 + 32 * mb + 8 * (r / 4) + 4 * h + (r % 4);
      if (row >= M) continue;
      float* dst = C + (int64_t)row * p.ldc + col;
      if (VEC) {
        if (col < N) {
          vecNB v;
          if constexpr (NB == 1) {
            v = out(mb, 0, r, dst);
          } else {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) v[nb] = out(mb, nb, r, dst);
          }
          *reinterpret_cast<vecNB*>(dst) = v;
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          if (col + nb < N) dst[nb] = out(mb, nb, r, dst);
      }
    }
  }
}

template <int BM, int BN, int BK, int WM, int WN>
hipError_t launch(const Params& p, const TileMap& map, bool vec, hipStream_t stream) {
  using S = Shape<BM, BN, BK, WM, WN>;
  const dim3 grid(map.tiles_m * map.tiles_n), block(S::NT);
#define SGEMM_MFMA_LAUNCH(V, E, T) \
  hipLaunchKernelGGL((sgemm_mfma_kernel<BM, BN, BK, WM, WN, V, E, T>), grid, block, 0, stream, p, map)
  if (p.bt) {  // transposed B (the fused epilogue is not combined with it)
    if (p.epi.on) return hipErrorNotSupported;
    if (vec) SGEMM_MFMA_LAUNCH(true, false, true);
    else SGEMM_MFMA_LAUNCH(false, false, true);
  } else if (p.epi.on) {
    if (vec) SGEMM_MFMA_LAUNCH(true, true, false);
    else SGEMM_MFMA_LAUNCH(false, true, false);
  } else {
    if (vec) SGEMM_MFMA_LAUNCH(true, false, false);
    else SGEMM_MFMA_LAUNCH(false, false, false);
  }
#undef SGEMM_MFMA_LAUNCH
  return hipGetLastError();
}

// Host replay of every LDS access of one K slice (staging writes, fragment
// reads), wave by wave: checks that writes cover the stage exactly once and
// reads stay in bounds, and counts bank conflicts.  Returns 0 when valid.
template <int BM, int BN, int BK, int WM, int WN>
int layout_check(int banks, int64_t out[2]) {
  using S = Shape<BM, BN, BK, WM, WN>;
  int64_t wconf = 0, rconf = 0;
  static unsigned char cover[S::STAGE * 4];
  for (int i = 0; i < S::STAGE * 4; ++i) cover[i] = 0;
  int addr[64];
  // Staging writes: A chunks then B chunks, per wave and per chunk index.
  for (int i = 0; i < S::CA; ++i)
    for (int w = 0; w < S::NT / 64; ++w) {
      for (int l = 0; l < 64; ++l) {
        const int id = w * 64 + l + i * S::NT;
        const int off = 4 * S::a_chunk(id / (BK / 4), id % (BK / 4));
        if (off < 0 || off + 16 > S::A_STAGE * 4) return 1;
        for (int b = 0; b < 16; ++b) cover[off + b]++;
        addr[l] = off;
      }
      wconf += lds_conflicts(addr, 16, banks);
    }
  for (int i = 0; i < S::CB; ++i)
    for (int w = 0; w < S::NT / 64; ++w) {
      for (int l = 0; l < 64; ++l) {
        const int id = w * 64 + l + i * S::NT;
        const int off = 4 * (S::A_STAGE + S::b_chunk(id / (BN / 4), id % (BN / 4)));
        if (off < 4 * S::A_STAGE || off + 16 > S::STAGE * 4) return 2;
        for (int b = 0; b < 16; ++b) cover[off + b]++;
        addr[l] = off;
      }
      wconf += lds_conflicts(addr, 16, banks);
    }
  for (int i = 0; i < S::STAGE * 4; ++i)
    if (cover[i] != 1) return 3;
  // Fragment reads of every wave for every k group.
  for (int w = 0; w < S::NT / 64; ++w) {
    const int wm0 = (w / S::WAVES_N) * WM, wn0 = (w % S::WAVES_N) * WN;
    for (int kk = 0; kk < BK; kk += 8) {
      for (int mb = 0; mb < S::MB; ++mb) {
        for (int l = 0; l < 64; ++l) {
          const int off = 4 * S::a_frag(wm0 + 32 * mb + (l & 31), kk, l >> 5);
          if (off < 0 || off + 16 > S::A_STAGE * 4) return 4;
          addr[l] = off;
        }
        rconf += lds_conflicts(addr, 16, banks);
      }
      for (int s = 0; s < 4; ++s) {
        for (int l = 0; l < 64; ++l) {
          const int off = 4 * (S::A_STAGE + S::b_frag(kk, l >> 5, s, wn0 + S::NB * (l & 31)));
          if (off < 4 * S::A_STAGE || off + 4 * S::NB > S::STAGE * 4) return 5;
          addr[l] = off;
        }
        rconf += lds_conflicts(addr, 4 * S::NB, banks);
      }
    }
  }
  out[0] = wconf;
  out[1] = rconf;
  return 0;
}

#define SGEMM_MFMA_VARIANT(BM, BN, BK, WM, WN, EFF)                                               \
  Variant {                                                                                  \
    gemm_config_t{0, GEMM_DTYPE_F32, GEMM_FAMILY_MFMA, BM, BN, BK, WM, WN,                   \
                  Shape<BM, BN, BK, WM, WN>::NT, 2, Shape<BM, BN, BK, WM, WN>::LDS_BYTES,    \
                  GEMM_ORDER_XCD, 8, 1, "mfma_f32_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN},      \
        &launch<BM, BN, BK, WM, WN>, &layout_check<BM, BN, BK, WM, WN>, nullptr, EFF,        \
        &launch<BM, BN, BK, WM, WN>, &launch<BM, BN, BK, WM, WN>                             \
  }

const Variant kVariants[] = {
    SGEMM_MFMA_VARIANT(128, 128, 32, 64, 64, 0.75f),
    SGEMM_MFMA_VARIANT(128, 128, 16, 64, 64, 0.72f),
    SGEMM_MFMA_VARIANT(256, 128, 32, 128, 64, 0.80f),
    SGEMM_MFMA_VARIANT(256, 256, 32, 128, 128, 0.83f),
    SGEMM_MFMA_VARIANT(128, 256, 32, 64, 128, 0.80f),
    SGEMM_MFMA_VARIANT(64, 64, 32, 32, 32, 0.55f),
    SGEMM_MFMA_VARIANT(128, 64, 32, 64, 32, 0.65f),
};

}  // namespace

hipError_t sgemm_launch_shape(int bm, int bn, int wm, int wn, const Params& p, const TileMap& map,
                              bool vec, hipStream_t stream) {
  // The tile map depends on the workgroup tile only: any wave split of the
  // same bm x bn tile computes the same tiles.  Prefer the same wave tile.
  const Variant* pick = nullptr;
  for (const Variant& v : kVariants)
    if (v.desc.bm == bm && v.desc.bn == bn && (!pick || (v.desc.wm == wm && v.desc.wn == wn)))
      pick = &v;
  return pick ? pick->launch(p, map, vec, stream) : hipErrorInvalidValue;
}

const Variant* sgemm_mfma_variants(int* count) {
  *count = sizeof(kVariants) / sizeof(kVariants[0]);
  return kVariants;
}

}  // namespace gemm
