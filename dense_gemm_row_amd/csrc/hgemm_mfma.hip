// FP16 HGEMM on the gfx950 matrix cores: C = A x B with binary16 inputs,
// FP32 accumulation and one round-to-nearest-even conversion per output.
// (The HGEMM of "hgemm_naive_kernel explained", whose kernels accumulate in
// FP16; here the accumulator is FP32.)
//
// * v_mfma_f32_32x32x16_f16 lane maps (checked on the device): lane l
//   supplies A[l%32][8*(l/32) .. +7] and B[8*(l/32) .. +7][l%32], eight
//   consecutive k per lane; accumulator register r of lane l holds row
//   8*(r/4) + 4*(l/32) + r%4, column l%32.
// * Both operands must therefore be K-contiguous per lane.  A is (row-major
//   A has k contiguous): its LDS tile is BM rows of BK = 64 halves (128
//   bytes) and a lane's fragment is one 16-byte read.  B is row-major with n
//   contiguous, so the staging step transposes it: each thread loads an
//   8 (k) x 8 (n) block with eight 16-byte loads, transposes it in
//   registers with byte permutes, and writes eight 16-byte rows of the
//   transposed LDS tile (one LDS row per output column).  This is the
//   transposed-operand idea of "sgemm - beyond cuBLAS" (section 3) and of
//   the s_a[BK][BM] tile in "hgemm_naive_kernel explained" (section 7.1),
//   applied to the operand that the matrix core needs transposed.
// * LDS rows use the chunk XOR swizzle swz_row (128-byte rows), and the B
//   rows are permuted by bt_row (column interleave + parity flip), which
//   keeps the staging writes and fragment reads conflict-free in 16-lane
//   groups over 64 banks.
// * Column interleave as in the FP32 kernel: block nb of a wave tile covers
//   columns wn0 + NB*j + nb, so each lane stores NB adjacent FP16 outputs
//   (2*NB bytes) per row, 32 lanes writing 64*NB contiguous bytes.
// * Two LDS stages, global loads of slice t+1 in flight while slice t feeds
//   the MFMAs, one barrier per slice (the double buffer of section 8 of the
//   HGEMM article, with the buffer index computed, not fixed).
// * VEC=true: A, B, C 16-byte aligned and K, N, lda, ldb, ldc multiples of
//   8 (whole 16-byte chunks in or out of range).  VEC=false: element loads
//   and stores with per-element masks.
// * FP8 operands off the LDS-direct kernels' layout (IN = 1 E4M3, 2 E5M2)
//   run here too: the masked element loads read bytes and widen each to its
//   bfloat16 value, which is exact (at most 4 significant bits, exponents in
//   range), and the bf16 form computes the same FP32-accumulated product
//   into a bfloat16 C.
#include <type_traits>

#include "gemm_internal.h"

namespace gemm {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int BK = 64;         // halves per K slice
constexpr int ROW_BYTES = 128; // one LDS row = BK halves

template <int BM, int BN, int WM, int WN>
struct Shape {
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int NT = WAVES_M * WAVES_N * 64;
  static constexpr int MB = WM / 32, NB = WN / 32;
  static constexpr int A_CHUNKS = BM * (BK / 8);      // 16-byte chunks
  static constexpr int B_BLOCKS = (BK / 8) * (BN / 8); // 8x8 blocks
  static constexpr int CA = A_CHUNKS / NT;
  static constexpr int CB = (B_BLOCKS + NT - 1) / NT;
  static constexpr int CBT = BN * (BK / 8) / NT;  // B given transposed: Bt chunks per thread
  static constexpr int A_STAGE = BM * ROW_BYTES, B_STAGE = BN * ROW_BYTES;  // bytes
  static constexpr int STAGE = A_STAGE + B_STAGE;
  static constexpr int LDS_BYTES = 2 * STAGE;
  static_assert(BM % WM == 0 && BN % WN == 0, "wave grid");
  static_assert(WM % 32 == 0 && (NB == 1 || NB == 2 || NB == 4), "wave tile");
  static_assert(A_CHUNKS % NT == 0 && (BN * (BK / 8)) % NT == 0, "A / Bt staging split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");

  // A chunk q (8 halves) of tile row r.
  __host__ __device__ static constexpr int a_chunk(int r, int q) { return swz_off(r, q, ROW_BYTES); }
  // Transposed B: k-chunk q of tile column n.
  __host__ __device__ static constexpr int b_chunk(int n, int q) {
    return A_STAGE + swz_off(bt_row(n, WN), q, ROW_BYTES);
  }
  // Fragment reads: A row r, B LDS row for (wave column origin wn0, block nb,
  // lane row j), both at k-chunk q.
  __host__ __device__ static constexpr int b_frag(int wn0, int nb, int j, int q) {
    return A_STAGE + swz_off(wn0 + 32 * nb + bt_sigma(j, NB), q, ROW_BYTES);
  }
};

// The 16-bit pattern of input element x: itself, or an FP8 byte widened to
// bfloat16.
template <int IN, class T>
__device__ __forceinline__ unsigned short in16(T x) {
  if constexpr (IN == 1) return e4m3_to_bf16(x);
  else if constexpr (IN == 2) return e5m2_to_bf16(x);
  else return x;
}

// BT: B given transposed (p.bt: Bt, N x K row-major).  Its rows are already
// k-contiguous per output column, so they are staged like A's chunks into
// the transposed B tile (no register transpose).  BF: the elements are
// bfloat16 (v_mfma_f32_32x32x16_bf16 and bfloat16 conversions; the staging
// moves 16-bit patterns either way).  IN: 0 for 16-bit inputs, 1 / 2 for
// FP8 E4M3 / E5M2 bytes (element loads only, widened to bfloat16).
template <int BM, int BN, int WM, int WN, bool VEC, bool EPI, bool BT, bool BF, int IN = 0>
__global__ void __launch_bounds__((Shape<BM, BN, WM, WN>::NT))
hgemm_mfma_kernel(Params p, TileMap map) {
  using S = Shape<BM, BN, WM, WN>;
  constexpr int NT = S::NT, MB = S::MB, NB = S::NB, CA = S::CA, CB = S::CB;
  static_assert(IN == 0 || (BF && !VEC), "FP8 inputs: bfloat16 compute, element loads");
  using In = std::conditional_t<IN == 0, unsigned short, unsigned char>;

  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * S::STAGE];

  int tm, tn;
  tile_of_block(blockIdx.x, map, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int M = p.M, N = p.N, K = p.K;
  const In* __restrict__ A = static_cast<const In*>(p.A);
  const In* __restrict__ B = static_cast<const In*>(p.B);
  unsigned short* __restrict__ C = static_cast<unsigned short*>(p.C);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 31, h = lane >> 5;
  const int wm0 = (wave / S::WAVES_N) * WM, wn0 = (wave % S::WAVES_N) * WN;

  // A staging: chunk (row r, k-chunk q) per slot.
  const In* a_src[CA];
  bool a_row_ok[CA];
  int a_k[CA], a_dst[CA];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int id = tid + i * NT;
    const int r = id / (BK / 8), q = id % (BK / 8);
    a_row_ok[i] = (m0 + r) < M;
    a_src[i] = A + (int64_t)(a_row_ok[i] ? m0 + r : 0) * p.lda + 8 * q;
    a_k[i] = 8 * q;
    a_dst[i] = S::a_chunk(r, q);
  }
  // B staging: 8x8 block (k-group r, column chunk c) per slot.
  const In* b_src[CB];
  bool b_on[CB];
  int b_k[CB], b_col[CB], b_c[CB], b_r[CB];
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int id = tid + i * NT;
    b_on[i] = id < S::B_BLOCKS;
    const int r = id % (BK / 8), c = id / (BK / 8);
    b_r[i] = r;
    b_c[i] = c;
    b_k[i] = 8 * r;
    b_col[i] = n0 + 8 * c;
    b_src[i] = B + (int64_t)(8 * r) * p.ldb + (b_col[i] < N ? b_col[i] : 0);
  }

  // BT staging: Bt chunk (tile column n, k chunk q) per slot.
  const In* bt_src[S::CBT];
  bool bt_ok[S::CBT];
  int bt_k[S::CBT], bt_dst[S::CBT];
#pragma unroll
  for (int i = 0; i < S::CBT; ++i) {
    const int id = tid + i * NT;
    const int n = id / (BK / 8), q = id % (BK / 8);
    bt_ok[i] = (n0 + n) < N;
    bt_src[i] = B + (int64_t)(bt_ok[i] ? n0 + n : 0) * p.ldb + 8 * q;
    bt_k[i] = 8 * q;
    bt_dst[i] = S::b_chunk(n, q);
  }

  u32x4 ra[CA];
  u32x4 rb[CB][8];
  u32x4 rbt[S::CBT];

  auto load_slice = [&](int k0) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int kg = k0 + a_k[i];
      if constexpr (VEC) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (a_row_ok[i] && kg < K) v = *reinterpret_cast<const u32x4*>(a_src[i] + k0);
        ra[i] = v;
      } else {
        unsigned short e[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) e[t] = (a_row_ok[i] && kg + t < K) ? in16<IN>(a_src[i][k0 + t]) : 0;
#pragma unroll
        for (int d = 0; d < 4; ++d) ra[i][d] = e[2 * d] | ((unsigned)e[2 * d + 1] << 16);
      }
    }
    if constexpr (BT) {
#pragma unroll
      for (int i = 0; i < S::CBT; ++i) {
        const int kg = k0 + bt_k[i];
        if constexpr (VEC) {
          u32x4 v = {0u, 0u, 0u, 0u};
          if (bt_ok[i] && kg < K) v = *reinterpret_cast<const u32x4*>(bt_src[i] + k0);
          rbt[i] = v;
        } else {
          unsigned short e[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) e[t] = (bt_ok[i] && kg + t < K) ? in16<IN>(bt_src[i][k0 + t]) : 0;
#pragma unroll
          for (int d = 0; d < 4; ++d) rbt[i][d] = e[2 * d] | ((unsigned)e[2 * d + 1] << 16);
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kg = k0 + b_k[i] + e;
        const In* src = b_src[i] + (int64_t)(k0 + e) * p.ldb;
        if constexpr (VEC) {
          u32x4 v = {0u, 0u, 0u, 0u};
          if (b_on[i] && kg < K && b_col[i] < N) v = *reinterpret_cast<const u32x4*>(src);
          rb[i][e] = v;
        } else {
          unsigned short x[8];
#pragma unroll
          for (int t = 0; t < 8; ++t)
            x[t] = (b_on[i] && kg < K && b_col[i] + t < N) ? in16<IN>(src[t]) : 0;
#pragma unroll
          for (int d = 0; d < 4; ++d) rb[i][e][d] = x[2 * d] | ((unsigned)x[2 * d + 1] << 16);
        }
      }
    }
  };

  auto store_slice = [&](int stage) {
    unsigned char* base = smem + stage * S::STAGE;
#pragma unroll
    for (int i = 0; i < CA; ++i) *reinterpret_cast<u32x4*>(base + a_dst[i]) = ra[i];
    if constexpr (BT) {
#pragma unroll
      for (int i = 0; i < S::CBT; ++i) *reinterpret_cast<u32x4*>(base + bt_dst[i]) = rbt[i];
      return;
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      if (!b_on[i]) continue;
      // rb[i][e] holds row k = 8r+e, columns 8c..8c+7 as 4 dwords of 2
      // halves.  Column j of the transposed block: dword d gathers rows
      // 2d (low half) and 2d+1 (high half) of column j.
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;
        u32x4 t;
#pragma unroll
        for (int d = 0; d < 4; ++d)
          t[d] = __builtin_amdgcn_perm(rb[i][2 * d + 1][j >> 1], rb[i][2 * d][j >> 1], sel);
        *reinterpret_cast<u32x4*>(base + S::b_chunk(8 * b_c[i] + j, b_r[i])) = t;
      }
    }
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
      const unsigned char* base = smem + cur * S::STAGE;
#pragma unroll
      for (int kk = 0; kk < BK; kk += 16) {
        const int q = kk / 8 + h;
        f16x8 a[MB], b[NB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          a[mb] = *reinterpret_cast<const f16x8*>(base + S::a_chunk(wm0 + 32 * mb + lrow, q));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          b[nb] = *reinterpret_cast<const f16x8*>(base + S::b_frag(wn0, nb, lrow, q));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma16<BF>(a[mb], b[nb], acc[mb][nb]);
      }
      if (t + 1 < T) store_slice(cur ^ 1);
      __syncthreads();
    }
  }

  // Epilogue: FP32 -> FP16 or BF16 (RNE), NB adjacent columns per lane and
  // row.  EPI: the fused epilogue (alpha, beta with the old 16-bit C, bias,
  // activation) in FP32 before the one rounding.
  const int col = n0 + wn0 + NB * lrow;
  auto out = [&](int mb, int nb, int r, const unsigned short* dst) -> unsigned short {
    if constexpr (!EPI) {
      return round16<BF>(acc[mb][nb][r]);
    } else {
      const float c_old = p.epi.beta != 0.f ? widen16<BF>(dst[nb]) : 0.f;
      const float bias = p.epi.bias ? p.epi.bias[col + nb] : 0.f;
      return round16<BF>(epi_value(p.epi, acc[mb][nb][r], c_old, bias));
    }
  };
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm0 + 32 * mb + 8 * (r / 4) + 4 * h + (r % 4);
      if (row >= M) continue;
      unsigned short* dst = C + (int64_t)row * p.ldc + col;
      if constexpr (VEC) {
        if (col < N) {
          if constexpr (NB == 4) {
            uint2 v;
            v.x = out(mb, 0, r, dst) | ((unsigned)out(mb, 1, r, dst) << 16);
            v.y = out(mb, 2, r, dst) | ((unsigned)out(mb, 3, r, dst) << 16);
            *reinterpret_cast<uint2*>(dst) = v;
          } else if constexpr (NB == 2) {
            *reinterpret_cast<unsigned*>(dst) = out(mb, 0, r, dst) | ((unsigned)out(mb, 1, r, dst) << 16);
          } else {
            *dst = out(mb, 0, r, dst);
          }
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          if (col + nb < N) dst[nb] = out(mb, nb, r, dst);
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, bool BF>
hipError_t launch_typed(const Params& p, const TileMap& map, bool vec, hipStream_t stream) {
  using S = Shape<BM, BN, WM, WN>;
  const dim3 grid(map.tiles_m * map.tiles_n), block(S::NT);
  if (p.bt) {  // transposed B (the fused epilogue is not combined with it)
    if (p.epi.on) return hipErrorNotSupported;
    if (vec)
      hipLaunchKernelGGL((hgemm_mfma_kernel<BM, BN, WM, WN, true, false, true, BF>), grid, block, 0, stream, p, map);
    else
      hipLaunchKernelGGL((hgemm_mfma_kernel<BM, BN, WM, WN, false, false, true, BF>), grid, block, 0, stream, p, map);
  } else if (p.epi.on) {
    if (vec)
      hipLaunchKernelGGL((hgemm_mfma_kernel<BM, BN, WM, WN, true, true, false, BF>), grid, block, 0, stream, p, map);
    else
      hipLaunchKernelGGL((hgemm_mfma_kernel<BM, BN, WM, WN, false, true, false, BF>), grid, block, 0, stream, p, map);
  } else {
    if (vec)
      hipLaunchKernelGGL((hgemm_mfma_kernel<BM, BN, WM, WN, true, false, false, BF>), grid, block, 0, stream, p, map);
    else
      hipLaunchKernelGGL((hgemm_mfma_kernel<BM, BN, WM, WN, false, false, false, BF>), grid, block, 0, stream, p, map);
  }
  return hipGetLastError();
}

// One launch function for both element types: p.bf16 picks the instance.
// FP8 operands (p.f8): element loads widened to bfloat16, bf16 compute.
template <int BM, int BN, int WM, int WN, int IN>
hipError_t launch_f8(const Params& p, const TileMap& map, hipStream_t stream) {
  using S = Shape<BM, BN, WM, WN>;
  const dim3 grid(map.tiles_m * map.tiles_n), block(S::NT);
  if (p.bt) {
    if (p.epi.on) return hipErrorNotSupported;
    hipLaunchKernelGGL((hgemm_mfma_kernel<BM, BN, WM, WN, false, false, true, true, IN>), grid, block, 0, stream, p, map);
  } else if (p.epi.on) {
    hipLaunchKernelGGL((hgemm_mfma_kernel<BM, BN, WM, WN, false, true, false, true, IN>), grid, block, 0, stream, p, map);
  } else {
    hipLaunchKernelGGL((hgemm_mfma_kernel<BM, BN, WM, WN, false, false, false, true, IN>), grid, block, 0, stream, p, map);
  }
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
hipError_t launch(const Params& p, const TileMap& map, bool vec, hipStream_t stream) {
  if (p.f8) return p.f8 == 1 ? launch_f8<BM, BN, WM, WN, 1>(p, map, stream)
                             : launch_f8<BM, BN, WM, WN, 2>(p, map, stream);
  return p.bf16 ? launch_typed<BM, BN, WM, WN, true>(p, map, vec, stream)
                : launch_typed<BM, BN, WM, WN, false>(p, map, vec, stream);
}

// Host replay of one K slice's LDS accesses (see the FP32 kernel).
template <int BM, int BN, int WM, int WN>
int layout_check(int banks, int64_t out[2]) {
  using S = Shape<BM, BN, WM, WN>;
  int64_t wconf = 0, rconf = 0;
  static unsigned char cover[S::STAGE];
  for (int i = 0; i < S::STAGE; ++i) cover[i] = 0;
  int addr[64];
  for (int i = 0; i < S::CA; ++i)
    for (int w = 0; w < S::NT / 64; ++w) {
      for (int l = 0; l < 64; ++l) {
        const int id = w * 64 + l + i * S::NT;
        const int off = S::a_chunk(id / (BK / 8), id % (BK / 8));
        if (off < 0 || off + 16 > S::A_STAGE) return 1;
        for (int b = 0; b < 16; ++b) cover[off + b]++;
        addr[l] = off;
      }
      wconf += lds_conflicts(addr, 16, banks);
    }
  for (int i = 0; i < S::CB; ++i)
    for (int w = 0; w < S::NT / 64; ++w) {
      for (int j = 0; j < 8; ++j) {
        int active = 0;
        for (int l = 0; l < 64; ++l) {
          const int id = w * 64 + l + i * S::NT;
          if (id >= S::B_BLOCKS) { addr[l] = -1; continue; }
          ++active;
          const int r = id % (BK / 8), c = id / (BK / 8);
          const int off = S::b_chunk(8 * c + j, r);
          if (off < S::A_STAGE || off + 16 > S::STAGE) return 2;
          for (int b = 0; b < 16; ++b) cover[off + b]++;
          addr[l] = off;
        }
        if (active) wconf += lds_conflicts(addr, 16, banks);
      }
    }
  for (int i = 0; i < S::STAGE; ++i)
    if (cover[i] != 1) return 3;
  for (int w = 0; w < S::NT / 64; ++w) {
    const int wm0 = (w / S::WAVES_N) * WM, wn0 = (w % S::WAVES_N) * WN;
    for (int kk = 0; kk < BK; kk += 16) {
      for (int mb = 0; mb < S::MB; ++mb) {
        for (int l = 0; l < 64; ++l) {
          const int off = S::a_chunk(wm0 + 32 * mb + (l & 31), kk / 8 + (l >> 5));
          if (off < 0 || off + 16 > S::A_STAGE) return 4;
          addr[l] = off;
        }
        rconf += lds_conflicts(addr, 16, banks);
      }
      for (int nb = 0; nb < S::NB; ++nb) {
        for (int l = 0; l < 64; ++l) {
          const int off = S::b_frag(wn0, nb, l & 31, kk / 8 + (l >> 5));
          if (off < S::A_STAGE || off + 16 > S::STAGE) return 5;
          addr[l] = off;
        }
        rconf += lds_conflicts(addr, 16, banks);
      }
    }
  }
  // The fragment read of (wn0, nb, j) must be the row the staging wrote for
  // the column the epilogue assigns to that lane: wn0 + NB*j + nb.
  for (int n = 0; n < BN; ++n) {
    const int wn0 = (n / WN) * WN, np = n % WN;
    if (S::b_frag(wn0, np % S::NB, np / S::NB, 0) != S::b_chunk(n, 0)) return 6;
  }
  out[0] = wconf;
  out[1] = rconf;
  return 0;
}

#define HGEMM_MFMA_VARIANT(DT, TAG, BM, BN, WM, WN, EFF)                                        \
  Variant {                                                                                  \
    gemm_config_t{0, DT, GEMM_FAMILY_MFMA, BM, BN, BK, WM, WN,                               \
                  Shape<BM, BN, WM, WN>::NT, 2, Shape<BM, BN, WM, WN>::LDS_BYTES,            \
                  GEMM_ORDER_XCD, 4, 1, "mfma_" TAG "_" #BM "x" #BN "x64_w" #WM "x" #WN},     \
        &launch<BM, BN, WM, WN>, &layout_check<BM, BN, WM, WN>, nullptr, EFF,                \
        &launch<BM, BN, WM, WN>, &launch<BM, BN, WM, WN>                                     \
  }

#define HGEMM_MFMA_TABLE(DT, TAG)                                \
  {HGEMM_MFMA_VARIANT(DT, TAG, 256, 256, 128, 128, 0.80f),       \
   HGEMM_MFMA_VARIANT(DT, TAG, 256, 128, 128, 64, 0.72f),        \
   HGEMM_MFMA_VARIANT(DT, TAG, 128, 256, 64, 128, 0.72f),        \
   HGEMM_MFMA_VARIANT(DT, TAG, 128, 128, 64, 64, 0.60f),         \
   HGEMM_MFMA_VARIANT(DT, TAG, 64, 64, 32, 32, 0.20f)}

const Variant kVariants[] = HGEMM_MFMA_TABLE(GEMM_DTYPE_F16, "f16");
const Variant kVariantsBf[] = HGEMM_MFMA_TABLE(GEMM_DTYPE_BF16, "bf16");

}  // namespace

hipError_t hgemm_launch_shape(int bm, int bn, int wm, int wn, const Params& p, const TileMap& map,
                              bool vec, hipStream_t stream) {
  // The tile map depends on the workgroup tile only: any wave split of the
  // same bm x bn tile computes the same tiles.  Prefer the same wave tile.
  // (The launch reads p.bf16, so the binary16 table serves both types.)
  const Variant* pick = nullptr;
  for (const Variant& v : kVariants)
    if (v.desc.bm == bm && v.desc.bn == bn && (!pick || (v.desc.wm == wm && v.desc.wn == wn)))
      pick = &v;
  return pick ? pick->launch(p, map, vec, stream) : hipErrorInvalidValue;
}

const Variant* hgemm_mfma_variants(int* count, bool bf16) {
  *count = bf16 ? sizeof(kVariantsBf) / sizeof(kVariantsBf[0])
                : sizeof(kVariants) / sizeof(kVariants[0]);
  return bf16 ? kVariantsBf : kVariants;
}

}  // namespace gemm
