// FP16 HGEMM, software-pipelined variant for aligned operands (the vector
// path): binary16 A and B, FP32 accumulation on v_mfma_f32_32x32x16_f16, one
// round-to-nearest-even conversion per output.
//
// Same data layout as hgemm_mfma.hip (A tile row-major, B tile transposed in
// registers at staging and stored one LDS row per output column, chunk XOR
// swizzle, column interleave for the epilogue), with a deeper pipeline built
// from gfx950 memory instructions:
//
// * A goes straight from global memory into LDS (buffer_load_dwordx4 ... lds):
//   one instruction moves 1 KB per wave, lane l landing at byte 16*l of the
//   wave's block, so each lane fetches the global chunk whose swizzled LDS
//   position is 16*l.  No VGPR staging and no ds_write for A.
// * All global loads are buffer loads with 32-bit offsets.  A chunk outside
//   the matrix (row >= M, column >= N, k >= K) gets an offset past the
//   buffer's range, and the hardware returns zeros: no branches, and the
//   whole K loop (including slices past K, which load nothing) is one
//   straight-line body.
// * Prefetch distances: A one K slice ahead (into the other LDS stage), B two
//   slices ahead (in registers), MFMA fragments one 16-deep k step ahead.
//   Per slice t: MFMAs of k steps 0-2 on stage t, with B(t+1) written
//   (transposed) to stage t+1 and B(t+2) loaded into registers; wait for
//   A(t+1); one barrier; issue A(t+2) into the stage just freed; first
//   fragments of stage t+1 under the MFMAs of k step 3.  This is the double
//   buffer of "sgemm - beyond cuBLAS" (section 6) and of the HGEMM
//   article's section 8, plus the asynchronous
//   copy stage that the lqnn.cn SGEMM article adds in its last version
//   (section 3.5), done with LDS-direct buffer loads.
// * Operands must be 16-byte aligned with K, N, lda, ldb, ldc multiples of 8
//   and byte offsets within 2^31 (the launcher checks; other cases run the
//   general kernel of hgemm_mfma.hip with the same tile).
#include "gemm_internal.h"

namespace gemm {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BK = 64;
constexpr int ROW_BYTES = 128;
constexpr unsigned OOB = 0x80000000u;  // past every buffer's num_records

template <int BM, int BN, int WM, int WN>
struct Shape {
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN, NW = WAVES_M * WAVES_N;
  static constexpr int NT = NW * 64;
  static constexpr int MB = WM / 32, NB = WN / 32;
  static constexpr int A_STAGE = BM * ROW_BYTES, B_STAGE = BN * ROW_BYTES;
  static constexpr int STAGE = A_STAGE + B_STAGE;
  static constexpr int LDS_BYTES = 2 * STAGE;
  static constexpr int A_BLOCKS = A_STAGE / 1024;  // 1 KB direct-load blocks
  static constexpr int IA = A_BLOCKS / NW;         // per wave
  static constexpr int B_BLOCKS = (BK / 8) * (BN / 8);
  // Waves [0, B_WAVES) stage B (CB blocks per thread); the rest only A.
  static constexpr int CB = B_BLOCKS >= NT ? B_BLOCKS / NT : 1;
  static constexpr int B_WAVES = B_BLOCKS >= NT ? NW : B_BLOCKS / 64;
  static_assert(BM % WM == 0 && BN % WN == 0, "wave grid");
  static_assert(WM % 32 == 0 && (NB == 1 || NB == 2 || NB == 4), "wave tile");
  static_assert(A_BLOCKS % NW == 0 && IA >= 1, "A direct-load split");
  static_assert(B_BLOCKS % 64 == 0 && (B_BLOCKS < NT || B_BLOCKS % NT == 0), "B staging split");
  static_assert(8 * CB <= 15, "vmcnt field");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");

  __host__ __device__ static constexpr int a_chunk(int r, int q) { return swz_off(r, q, ROW_BYTES); }
  __host__ __device__ static constexpr int b_chunk(int n, int q) {
    return A_STAGE + swz_off(bt_row(n, WN), q, ROW_BYTES);
  }
  __host__ __device__ static constexpr int b_frag(int wn0, int nb, int j, int q) {
    return A_STAGE + swz_off(wn0 + 32 * nb + bt_sigma(j, NB), q, ROW_BYTES);
  }
  // Direct load: lane l of wave w, instruction i lands at byte
  // 1024*(i*NW + w) + 16*l of the A stage: its tile row and logical chunk.
  __host__ __device__ static constexpr int a_dl_row(int i, int w, int l) { return 8 * (i * NW + w) + l / 8; }
  __host__ __device__ static constexpr int a_dl_chunk(int i, int w, int l) {
    return (l % 8) ^ swz_row(a_dl_row(i, w, l), ROW_BYTES);
  }
};

__device__ inline f32x16 mfma(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int SG_VALU = 0x002, SG_MFMA = 0x008, SG_VMEM_RD = 0x020, SG_DS_RD = 0x100,
              SG_DS_WR = 0x200;

// Interleave requests for one phase of 16 MFMAs: after each MFMA, issue a
// few of the phase's other instructions, so that they execute while the
// matrix pipe is busy instead of in a burst between MFMA groups (which
// drains the pipe).  `slot(i)` lists what follows MFMA number i.
#define SGB(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

__device__ inline unsigned short f16_bits(float x) {
  return __builtin_bit_cast(unsigned short, static_cast<_Float16>(x));
}

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  // Raw buffer (stride 0); num_records in bytes; loads past it return 0.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__((Shape<BM, BN, WM, WN>::NT))
hgemm_pipe_kernel(Params p, TileMap map, int64_t a_bytes, int64_t b_bytes) {
  using S = Shape<BM, BN, WM, WN>;
  constexpr int NW = S::NW, MB = S::MB, NB = S::NB, IA = S::IA, CB = S::CB;

  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * S::STAGE];

  int tm, tn;
  tile_of_block(blockIdx.x, map, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int M = p.M, N = p.N, K = p.K;
  const int lda = (int)p.lda, ldb = (int)p.ldb;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, a_bytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B, b_bytes);
  unsigned short* __restrict__ C = static_cast<unsigned short*>(p.C);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 31, h = lane >> 5;
  const int wm0 = (wave / S::WAVES_N) * WM, wn0 = (wave % S::WAVES_N) * WN;

  // A direct loads: byte offset of (row, k = 8*chunk) at k0 = 0, and the
  // logical k of the chunk (for the K edge).
  unsigned a_off[IA];
  int a_k[IA];
  bool a_ok[IA];
#pragma unroll
  for (int i = 0; i < IA; ++i) {
    const int r = S::a_dl_row(i, wave, lane), q = S::a_dl_chunk(i, wave, lane);
    a_ok[i] = (m0 + r) < M;
    a_off[i] = 2u * ((unsigned)(m0 + r) * (unsigned)lda + 8u * q);
    a_k[i] = 8 * q;
  }
  const bool stages_b = (S::B_WAVES == NW) || wave < S::B_WAVES;
  // B staging: 8x8 block (k-group r, column chunk c) per slot.
  int b_col[CB], b_c[CB], b_r[CB];
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int id = tid + i * S::NT;
    b_r[i] = id % (BK / 8);
    b_c[i] = id / (BK / 8);
    b_col[i] = n0 + 8 * b_c[i];
  }

  u32x4 rbuf[CB][8];

  auto issue_a = [&](int k0, int stage) {
#pragma unroll
    for (int i = 0; i < IA; ++i) {
      // Bitwise predicate and select: no exec-mask region, which would split
      // the scheduling region of the interleaved phase.
      const bool ok = a_ok[i] & (k0 + a_k[i] < K);
      const unsigned off = ok ? a_off[i] + (unsigned)(2 * k0) : OOB;
      lds_void* dst = (lds_void*)(smem + stage * S::STAGE + 1024 * (i * NW + wave));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, off, 0, 0, 0);
    }
  };
  auto issue_b = [&](int k0) {
    if (!stages_b) return;
#pragma unroll
    for (int i = 0; i < CB; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kg = k0 + 8 * b_r[i] + e;
        const bool ok = (kg < K) & (b_col[i] < N);
        const unsigned off = ok ? 2u * ((unsigned)kg * (unsigned)ldb + (unsigned)b_col[i]) : OOB;
        rbuf[i][e] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0));
      }
  };
  // Wait until this wave's LDS-direct A copies have landed (its B loads,
  // issued after them, may still be in flight).
  auto wait_a = [&]() {
    if (stages_b)
      __builtin_amdgcn_s_waitcnt(0x0F70 | (8 * CB));
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);
  };
  auto write_b = [&](int stage) {
    if (!stages_b) return;
    unsigned char* base = smem + stage * S::STAGE;
#pragma unroll
    for (int i = 0; i < CB; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // rbuf[i][e] holds row k = 8r+e, columns 8c..8c+7 as 4 dwords of 2
        // halves; dword d of transposed column j gathers rows 2d and 2d+1.
        const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;
        u32x4 t;
#pragma unroll
        for (int d = 0; d < 4; ++d)
          t[d] = __builtin_amdgcn_perm(rbuf[i][2 * d + 1][j >> 1], rbuf[i][2 * d][j >> 1], sel);
        *reinterpret_cast<u32x4*>(base + S::b_chunk(8 * b_c[i] + j, b_r[i])) = t;
      }
  };

  f16x8 fa[2][MB], fb[2][NB];
  auto load_frags = [&](int buf, int stage, int kk) {
    const unsigned char* base = smem + stage * S::STAGE;
    const int q = kk / 8 + h;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      fa[buf][mb] = *reinterpret_cast<const f16x8*>(base + S::a_chunk(wm0 + 32 * mb + lrow, q));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      fb[buf][nb] = *reinterpret_cast<const f16x8*>(base + S::b_frag(wn0, nb, lrow, q));
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.f;

  auto mma = [&](int buf) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma(fa[buf][mb], fb[buf][nb], acc[mb][nb]);
  };

  const int T = (K + BK - 1) / BK;
  if (T > 0) {
    // Prologue: slice 0 into stage 0, slice 1 of B into registers, slice 1
    // of A on its way into stage 1.
    issue_b(0);
    issue_a(0, 0);
    write_b(0);
    issue_b(BK);
    wait_a();
    __syncthreads();
    issue_a(BK, 1);
    load_frags(0, 0, 0);

    // Phases fenced with sched_barrier so the scheduler keeps the prefetch
    // distances (it otherwise sinks loads towards their first use).  Both
    // A(t+2) (issued right after the barrier that frees its stage) and
    // B(t+2) (issued right after B(t+1) leaves the registers) get four
    // k steps of MFMAs before they are needed.  The last k step's MFMAs
    // run after the barrier: they only read registers, and they cover the
    // latency of the next stage's first fragment reads.
    for (int t = 0; t < T; ++t) {
      const int cur = t & 1, nxt = cur ^ 1;
      const int k2 = (t + 2) * BK;
      // k step 0: fragments of step 1 between the MFMAs.
      load_frags(1, cur, 16);
      mma(0);
#pragma unroll
      for (int i = 0; i < 8; ++i) { SGB(SG_MFMA, 1); SGB(SG_DS_RD, 1); }
      SGB(SG_MFMA, 8);
      __builtin_amdgcn_sched_barrier(0);
      // k step 1: B(t+1) transposed into stage t+1, B(t+2) loads, fragments
      // of step 2.
      write_b(nxt);
      issue_b(k2);
      load_frags(0, cur, 32);
      mma(1);
#pragma unroll
      for (int i = 0; i < 8; ++i) { SGB(SG_MFMA, 1); SGB(SG_VALU, 5); SGB(SG_DS_WR, 1); }
#pragma unroll
      for (int i = 0; i < 8; ++i) { SGB(SG_MFMA, 1); SGB(SG_VALU, 3); SGB(SG_VMEM_RD, 1); SGB(SG_DS_RD, 1); }
      __builtin_amdgcn_sched_barrier(0);
      // k step 2: fragments of step 3.
      load_frags(1, cur, 48);
      mma(0);
#pragma unroll
      for (int i = 0; i < 8; ++i) { SGB(SG_MFMA, 1); SGB(SG_DS_RD, 1); }
      SGB(SG_MFMA, 8);
      __builtin_amdgcn_sched_barrier(0);
      // A(t+1) was issued before B(t+2): waiting until at most the B loads
      // are outstanding means the LDS-direct copies are done.
      wait_a();
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      // k step 3 (registers only): A(t+2) into the freed stage, first
      // fragments of stage t+1.
      issue_a(k2, cur);
      load_frags(0, nxt, 0);
      mma(1);
#pragma unroll
      for (int i = 0; i < 8; ++i) { SGB(SG_MFMA, 1); SGB(SG_VALU, 2); SGB(SG_VMEM_RD, 1); SGB(SG_DS_RD, 1); }
      SGB(SG_MFMA, 8);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }

  // Epilogue: FP32 -> FP16 (RNE), NB adjacent columns per lane and row.
  const int col = n0 + wn0 + NB * lrow;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm0 + 32 * mb + 8 * (r / 4) + 4 * h + (r % 4);
      if (row >= M || col >= N) continue;
      unsigned short* dst = C + (int64_t)row * p.ldc + col;
      if constexpr (NB == 4) {
        uint2 v;
        v.x = f16_bits(acc[mb][0][r]) | ((unsigned)f16_bits(acc[mb][1][r]) << 16);
        v.y = f16_bits(acc[mb][2][r]) | ((unsigned)f16_bits(acc[mb][3][r]) << 16);
        *reinterpret_cast<uint2*>(dst) = v;
      } else if constexpr (NB == 2) {
        *reinterpret_cast<unsigned*>(dst) = f16_bits(acc[mb][0][r]) | ((unsigned)f16_bits(acc[mb][1][r]) << 16);
      } else {
        *dst = f16_bits(acc[mb][0][r]);
      }
    }
  }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch(const Params& p, const TileMap& map, bool vec, hipStream_t stream) {
  using S = Shape<BM, BN, WM, WN>;
  const int64_t lim = 0x7fffffff;
  // Byte offsets of every row the tile grid touches (rows past M and K are
  // sent out of range, but their offsets are still formed) must fit 31 bits.
  if (!vec || (int64_t)(p.M + BM) * p.lda * 2 > lim || (int64_t)(p.K + 2 * BK) * p.ldb * 2 > lim)
    return hgemm_launch_shape(BM, BN, WM, WN, p, map, vec, stream);
  const int64_t a_bytes = p.K > 0 ? ((int64_t)(p.M - 1) * p.lda + p.K) * 2 : 0;
  const int64_t b_bytes = p.K > 0 ? ((int64_t)(p.K - 1) * p.ldb + p.N) * 2 : 0;
  const dim3 grid(map.tiles_m * map.tiles_n), block(S::NT);
  hipLaunchKernelGGL((hgemm_pipe_kernel<BM, BN, WM, WN>), grid, block, 0, stream, p, map, a_bytes,
                     b_bytes);
  return hipGetLastError();
}

// Host replay of one slice's LDS accesses (direct A loads, B staging writes,
// fragment reads).
template <int BM, int BN, int WM, int WN>
int layout_check(int banks, int64_t out[2]) {
  using S = Shape<BM, BN, WM, WN>;
  int64_t wconf = 0, rconf = 0;
  static unsigned char cover[S::STAGE];
  for (int i = 0; i < S::STAGE; ++i) cover[i] = 0;
  int addr[64];
  // Direct loads: the chunk each lane fetches must be the chunk its LDS
  // position holds under the swizzle, and all positions are covered.
  for (int i = 0; i < S::IA; ++i)
    for (int w = 0; w < S::NW; ++w)
      for (int l = 0; l < 64; ++l) {
        const int off = 1024 * (i * S::NW + w) + 16 * l;
        const int r = S::a_dl_row(i, w, l), q = S::a_dl_chunk(i, w, l);
        if (r >= BM || S::a_chunk(r, q) != off) return 1;
        for (int b = 0; b < 16; ++b) cover[off + b]++;
      }
  for (int i = 0; i < S::CB; ++i)
    for (int w = 0; w < S::B_WAVES; ++w)
      for (int j = 0; j < 8; ++j) {
        for (int l = 0; l < 64; ++l) {
          const int id = w * 64 + l + i * S::NT;
          const int r = id % (BK / 8), c = id / (BK / 8);
          const int off = S::b_chunk(8 * c + j, r);
          if (off < S::A_STAGE || off + 16 > S::STAGE) return 2;
          for (int b = 0; b < 16; ++b) cover[off + b]++;
          addr[l] = off;
        }
        wconf += lds_conflicts(addr, 16, banks);
      }
  for (int i = 0; i < S::STAGE; ++i)
    if (cover[i] != 1) return 3;
  for (int w = 0; w < S::NW; ++w) {
    const int wm0 = (w / S::WAVES_N) * WM, wn0 = (w % S::WAVES_N) * WN;
    for (int kk = 0; kk < BK; kk += 16) {
      for (int mb = 0; mb < S::MB; ++mb) {
        for (int l = 0; l < 64; ++l) addr[l] = S::a_chunk(wm0 + 32 * mb + (l & 31), kk / 8 + (l >> 5));
        rconf += lds_conflicts(addr, 16, banks);
      }
      for (int nb = 0; nb < S::NB; ++nb) {
        for (int l = 0; l < 64; ++l) addr[l] = S::b_frag(wn0, nb, l & 31, kk / 8 + (l >> 5));
        rconf += lds_conflicts(addr, 16, banks);
      }
    }
  }
  for (int n = 0; n < BN; ++n) {
    const int wn0 = (n / WN) * WN, np = n % WN;
    if (S::b_frag(wn0, np % S::NB, np / S::NB, 0) != S::b_chunk(n, 0)) return 6;
  }
  out[0] = wconf;
  out[1] = rconf;
  return 0;
}

#define HGEMM_PIPE_VARIANT(BM, BN, WM, WN, EFF)                                                 \
  Variant {                                                                                  \
    gemm_config_t{0, GEMM_DTYPE_F16, GEMM_FAMILY_MFMA, BM, BN, BK, WM, WN,                   \
                  Shape<BM, BN, WM, WN>::NT, 2, Shape<BM, BN, WM, WN>::LDS_BYTES,            \
                  GEMM_ORDER_XCD, 4, 1, "pipe_f16_" #BM "x" #BN "x64_w" #WM "x" #WN},           \
        &launch<BM, BN, WM, WN>, &layout_check<BM, BN, WM, WN>, nullptr, EFF                 \
  }

const Variant kVariants[] = {
    HGEMM_PIPE_VARIANT(256, 256, 128, 128, 0.85f),
    HGEMM_PIPE_VARIANT(256, 128, 128, 64, 0.78f),
    HGEMM_PIPE_VARIANT(128, 256, 64, 128, 0.78f),
    HGEMM_PIPE_VARIANT(128, 128, 64, 64, 0.65f),
    HGEMM_PIPE_VARIANT(256, 256, 128, 64, 0.80f),
    HGEMM_PIPE_VARIANT(256, 256, 64, 128, 0.80f),
};

}  // namespace

const Variant* hgemm_pipe_variants(int* count) {
  *count = sizeof(kVariants) / sizeof(kVariants[0]);
  return kVariants;
}

}  // namespace gemm
