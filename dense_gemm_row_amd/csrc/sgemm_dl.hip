// FP32 SGEMM for aligned operands on the gfx950 matrix cores, fed by
// LDS-direct copies: C = A x B, row-major, FP32 in and out, accumulated by
// v_mfma_f32_32x32x2_f32.
//
// Same arithmetic and register layout as sgemm_mfma.hip (the K permutation
// inside groups of 8, the column interleave of the B fragment, direct
// epilogue stores); what changes is how the operands reach LDS and how the
// loop is scheduled:
//
// * A and B go from global memory straight into LDS with
//   buffer_load_dwordx4 ... lds: one instruction fills 1 KB of LDS per wave,
//   lane l writing bytes [16l, 16l+16) of the wave's block, so each lane
//   fetches the 16-byte global chunk whose LDS position is 16l.  The A tile
//   is row-major (k contiguous, 4*BK-byte rows, chunk XOR swz_row), the B
//   tile row-major as in memory.  No VGPR staging, no ds_write, no wait for
//   the copy before a store: the copy of slice t+NS flies while slices
//   t+1 .. t+NS-1 are computed.
// * K advances by moving the buffer descriptors' base address and shrinking
//   their range; loads outside the matrix (rows past M or K, columns past N)
//   are range-checked by the hardware and return zeros; the last, partial K
//   slice of A is masked per lane.
// * Fragments are double-buffered in registers: the LDS reads of k group
//   g+1 are interleaved with the MFMAs of group g.  One barrier per slice;
//   the MFMAs of the slice's last group (registers only) run after it,
//   covering the first fragment reads of the next stage.
// * NS stages, each its own __shared__ array, the loop unrolled NS times so
//   that every LDS access names its array statically (the compiler can then
//   see that a copy into one stage does not alias reads of another).
//
// This is the double buffer of "sgemm - beyond cuBLAS" (section 6) with the
// asynchronous global-to-shared copies of the lqnn.cn SGEMM article
// (section 3.5), done with gfx950's LDS-direct buffer loads.
#include <type_traits>
#include <utility>

#include "gemm_internal.h"

namespace gemm {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

template <int NB> struct VecF;
template <> struct VecF<1> { typedef float T; };
template <> struct VecF<2> { typedef f32x2 T; };
template <> struct VecF<4> { typedef f32x4 T; };

constexpr unsigned OOB = 0x80000000u;  // offset past every buffer's range
constexpr int MAX_STAGES = 4;

template <int I>
using IC = std::integral_constant<int, I>;

template <class F, int... I>
__device__ __forceinline__ void static_for(F&& f, std::integer_sequence<int, I...>) {
  (f(IC<I>{}), ...);
}

// EPI_: the form with the fused epilogue (alpha, beta, bias, activation).
// BT_: B given transposed (Bt, N x K row-major, i.e. column-major B): its
// tile is staged like A's, one LDS row per output column with k contiguous,
// the columns of each wave block de-interleaved (LDS row wn0 + 32nb + j
// holds column wn0 + NB*j + nb) so that a lane's 16-byte read gives four k
// steps of its column and 16 lanes read 16 consecutive rows.
// Q8_: the fused epilogue writes INT8 codes (C is int8, beta is 0).
// AT_: A given transposed (At, K x M row-major, i.e. column-major A): its
// tile is staged like B's, one LDS row per k with BM m values, and a lane
// reads, per MFMA step, the MB adjacent values m = wm0 + MB*(l%32) + mb of
// its k row (the row interleave that B's columns use), so output rows of
// block mb are m = wm0 + MB*i + mb.
template <int BM_, int BN_, int WM_, int WN_, int BK_, int NS_, bool EPI_ = false, bool BT_ = false,
          bool Q8_ = false, bool AT_ = false>
struct Shape {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, NS = NS_;
  static constexpr bool EPI = EPI_ || Q8_, BT = BT_, Q8 = Q8_, AT = AT_;
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN, NW = WAVES_M * WAVES_N;
  static constexpr int NT = NW * 64;
  static constexpr int MB = WM / 32, NB = WN / 32, KG = BK / 8;  // k groups of 8 per slice
  static constexpr int A_ROW = AT ? BM * 4 : BK * 4, A_CPR = A_ROW / 16;  // bytes / chunks per A row
  static constexpr int B_ROW = BT ? BK * 4 : BN * 4;                      // bytes per B row
  static constexpr int A_STAGE = AT ? BK * A_ROW : BM * A_ROW, B_STAGE = BT ? BN * B_ROW : BK * B_ROW;
  static constexpr int LDS_BYTES = NS * (A_STAGE + B_STAGE);
  static constexpr int IA = A_STAGE / 1024 / NW, IB = B_STAGE / 1024 / NW, LPS = IA + IB;
  static_assert(BK == 16 || BK == 32 || BK == 64, "K slice");
  static_assert(KG % 2 == 0, "fragment double buffer alternates within a slice");
  static_assert(NS >= 2 && NS <= MAX_STAGES, "stages");
  static_assert(BM % WM == 0 && BN % WN == 0, "wave grid");
  static_assert(WM % 32 == 0 && (NB == 1 || NB == 2 || NB == 4), "wave tile");
  static_assert(A_STAGE % (1024 * NW) == 0 && B_STAGE % (1024 * NW) == 0, "direct-load split");
  static_assert(B_ROW % 1024 == 0 || 1024 % B_ROW == 0, "B rows tile the 1 KB blocks");
  static_assert(!BT || (NB - 1) * 32 * B_ROW < 65536, "immediate offsets (BT)");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert((NS - 1) * LPS <= 63, "vmcnt field");
  static_assert((AT ? BK * A_ROW : (MB - 1) * 32 * A_ROW) < 65536 && BK * B_ROW < 65536,
                "immediate offsets");
  static_assert(!AT || A_ROW % 1024 == 0 || 1024 % A_ROW == 0, "A^T rows tile the 1 KB blocks");

  // Byte offsets within one stage array.
  __host__ __device__ static constexpr int a_byte(int r, int q) { return swz_off(r, q, A_ROW); }
  __host__ __device__ static constexpr int b_byte(int k, int n) { return k * B_ROW + 4 * n; }
  // Direct loads: lane l of wave w, instruction i.
  __host__ __device__ static constexpr int a_dl_row(int i, int w, int l) {
    return (1024 / A_ROW) * (i * NW + w) + l / A_CPR;
  }
  __host__ __device__ static constexpr int a_dl_q(int i, int w, int l) {
    return (l % A_CPR) ^ swz_row(a_dl_row(i, w, l), A_ROW);
  }
  __host__ __device__ static constexpr int b_dl_k(int i, int w, int l) {
    return (1024 * (i * NW + w) + 16 * l) / B_ROW;
  }
  __host__ __device__ static constexpr int b_dl_c(int i, int w, int l) {
    return (1024 * (i * NW + w) + 16 * l) % B_ROW / 16;
  }
  // Fragment reads for k group g of a slice.  Within the group, MFMA step s
  // (0..3) takes physical k = 8g + 4h + s in lane half h = l/32.
  //  A: lane reads row wm0 + 32mb + l%32, chunk 2g + h (k = 8g + 4h .. +3).
  __host__ __device__ static constexpr int a_frag(int wm0, int mb, int g, int l) {
    return a_byte(wm0 + 32 * mb + l % 32, 2 * g + l / 32);
  }
  //  B: lane reads row 8g + 4h + s, the NB columns wn0 + NB*(l%32) + nb.
  __host__ __device__ static constexpr int b_frag(int wn0, int g, int s, int l) {
    return b_byte(8 * g + 4 * (l / 32) + s, wn0 + NB * (l % 32));
  }
  // AT: A^T tile row k, m value m; direct loads; the fragment read of k
  // group g, step s: row 8g + 4h + s, the MB rows wm0 + MB*(l%32) + mb.
  __host__ __device__ static constexpr int at_byte(int k, int m) { return k * A_ROW + 4 * m; }
  __host__ __device__ static constexpr int at_dl_k(int i, int w, int l) {
    return (1024 * (i * NW + w) + 16 * l) / A_ROW;
  }
  __host__ __device__ static constexpr int at_dl_c(int i, int w, int l) {
    return (1024 * (i * NW + w) + 16 * l) % A_ROW / 16;
  }
  __host__ __device__ static constexpr int at_frag(int wm0, int g, int s, int l) {
    return at_byte(8 * g + 4 * (l / 32) + s, wm0 + MB * (l % 32));
  }
  // BT direct loads: Bt rows (B_ROW bytes) placed like row-major A's rows,
  // by B's own row length (with A transposed the two differ).
  __host__ __device__ static constexpr int bt_dl_row(int i, int w, int l) {
    return (1024 / B_ROW) * (i * NW + w) + l / (B_ROW / 16);
  }
  __host__ __device__ static constexpr int bt_dl_q(int i, int w, int l) {
    return (l % (B_ROW / 16)) ^ swz_row(bt_dl_row(i, w, l), B_ROW);
  }
  // BT: tile column held by LDS row R, the LDS placement of (row R, k
  // chunk q), and the fragment read of block nb in k group g: LDS row
  // wn0 + 32nb + l%32 (column wn0 + NB*(l%32) + nb), chunk 2g + l/32.
  __host__ __device__ static constexpr int bt_col(int R) {
    return (R / WN) * WN + NB * (R % 32) + (R % WN) / 32;
  }
  __host__ __device__ static constexpr int bt_byte(int R, int q) { return swz_off(R, q, B_ROW); }
  __host__ __device__ static constexpr int bt_frag(int wn0, int nb, int g, int l) {
    return bt_byte(wn0 + 32 * nb + l % 32, 2 * g + l / 32);
  }
};

__device__ inline f32x16 mfma(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const unsigned char* base, int64_t bytes) {
  // Raw buffer (stride 0); num_records in bytes; loads past it return 0.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(base), 0,
                                           (int)(bytes > 0 ? bytes : 0), 0x00020000);
}

constexpr int SG_MFMA = 0x008, SG_VMEM_RD = 0x020, SG_DS_RD = 0x100;

// s_waitcnt immediate: vmcnt(n) (6 bits, split 4 + 2) with expcnt and
// lgkmcnt left at their maximum (no wait).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
// The same with lgkmcnt(0): this wave's LDS reads have returned.
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0070; }

// Workgroup barrier for the K loop, after this wave's fragment reads have
// returned and all but its N most recent copies have landed.  No memory
// fence: the loop's only LDS traffic is the fragment reads and the
// LDS-direct copies, both covered by the explicit wait, while the release
// fence of __syncthreads() would also wait for every copy still in flight
// (vmcnt(0)) and collapse the stage pipeline to one slice.
// (The empty asm statements keep the compiler from moving memory accesses
// across the barrier, which the fence would otherwise have prevented.)
template <int N>
__device__ __forceinline__ void loop_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(N));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
#define SGB(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

// Issue the LDS-direct copies of K slice s into one stage.  A device
// function, not a kernel lambda: lambdas of a kernel are also compiled for
// the host, and a descriptor value there makes the host pass drop the
// kernel's launch stub.  Slices past the last one (issued only to keep the
// wait counts uniform) get empty descriptors and touch no memory.
template <class S>
__device__ __forceinline__ void issue_slice(const unsigned char* Ab, const unsigned char* Bb,
                                            int64_t a_bytes, int64_t b_bytes, int s, bool live,
                                            const unsigned* a_vo, const unsigned* b_vo,
                                            unsigned char* lds_a, unsigned char* lds_b, int wave,
                                            int lda, int ldb) {
  const int64_t ka = S::AT ? (int64_t)s * S::BK * lda * 4 : 4 * (int64_t)s * S::BK;
  const int64_t kb = S::BT ? 4 * (int64_t)s * S::BK : (int64_t)s * S::BK * ldb * 4;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ab + ka, live ? a_bytes - ka : 0);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bb + kb, live ? b_bytes - kb : 0);
#pragma unroll
  for (int i = 0; i < S::IA; ++i) {
    lds_void* dst = (lds_void*)(lds_a + 1024 * (i * S::NW + wave));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, a_vo[i], 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < S::IB; ++i) {
    lds_void* dst = (lds_void*)(lds_b + 1024 * (i * S::NW + wave));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, dst, 16, b_vo[i], 0, 0, 0);
  }
}

template <class S>
__global__ void __launch_bounds__(S::NT)
sgemm_dl_kernel(Params p, TileMap map, int64_t a_bytes, int64_t b_bytes) {
  trace_stamp(p, 0);
  constexpr int NS = S::NS, KG = S::KG, MB = S::MB, NB = S::NB, IA = S::IA, IB = S::IB;
  constexpr int BM = S::BM, BN = S::BN, WM = S::WM, WN = S::WN, BK = S::BK;
  typedef typename VecF<NB>::T vecNB;
  typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
  typedef __attribute__((address_space(3))) vecNB lds_vecNB;

  // Stage arrays (unused ones are dropped by the compiler).
  __shared__ __attribute__((aligned(1024))) unsigned char la0[S::A_STAGE], lb0[S::B_STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char la1[S::A_STAGE], lb1[S::B_STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char la2[S::A_STAGE], lb2[S::B_STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char la3[S::A_STAGE], lb3[S::B_STAGE];
  auto A_of = [&](auto I) -> unsigned char* {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) return la0;
    else if constexpr (i == 1) return la1;
    else if constexpr (i == 2) return la2;
    else return la3;
  };
  auto B_of = [&](auto I) -> unsigned char* {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) return lb0;
    else if constexpr (i == 1) return lb1;
    else if constexpr (i == 2) return lb2;
    else return lb3;
  };

  int tm, tn;
  tile_of_block(blockIdx.x, map, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lda = (int)p.lda, ldb = (int)p.ldb;
  // Split-K: workgroup row sk takes K chunk [sk*kc, min(K, (sk+1)*kc)); the
  // operand bases and buffer ranges move to the chunk, C to its partial.
  const int sk = blockIdx.y;
  const int kc = p.splits > 1 ? p.kc : p.K;
  const int M = p.M, N = p.N, K = min(kc, p.K - sk * kc);
  const int64_t ashift = S::AT ? 4 * (int64_t)sk * kc * lda : 4 * (int64_t)sk * kc;
  const unsigned char* Ab = static_cast<const unsigned char*>(p.A) + ashift;
  const int64_t bshift = S::BT ? 4 * (int64_t)sk * kc : 4 * (int64_t)sk * kc * ldb;
  const unsigned char* Bb = static_cast<const unsigned char*>(p.B) + bshift;
  a_bytes -= ashift;
  b_bytes -= bshift;

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave / S::WAVES_N) * WM, wn0 = (wave % S::WAVES_N) * WN;
  const int T = (K + BK - 1) / BK;

  // Direct-load offsets (relative to the slice's descriptor base).
  unsigned a_vo[IA], a_vo_tail[IA], b_vo[IB], b_vo_tail[IB];
#pragma unroll
  for (int i = 0; i < IA; ++i) {
    if constexpr (S::AT) {
      const int k = S::at_dl_k(i, wave, l), c = S::at_dl_c(i, wave, l);
      const bool ok = (m0 + 4 * c) < M;
      a_vo[i] = ok ? 4u * ((unsigned)k * (unsigned)lda + (unsigned)(m0 + 4 * c)) : OOB;
      a_vo_tail[i] = a_vo[i];  // rows past K are past the buffer's range
    } else {
      const int r = S::a_dl_row(i, wave, l), q = S::a_dl_q(i, wave, l);
      const bool ok = (m0 + r) < M;
      a_vo[i] = ok ? 4u * ((unsigned)(m0 + r) * (unsigned)lda + 4u * q) : OOB;
      a_vo_tail[i] = ((T - 1) * BK + 4 * q < K) ? a_vo[i] : OOB;
    }
  }
#pragma unroll
  for (int i = 0; i < IB; ++i) {
    if constexpr (S::BT) {
      // LDS row R holds Bt row n0 + bt_col(R); k chunk q as for A.
      const int R = S::bt_dl_row(i, wave, l), q = S::bt_dl_q(i, wave, l);
      const int n = n0 + S::bt_col(R);
      b_vo[i] = n < N ? 4u * ((unsigned)n * (unsigned)ldb + 4u * q) : OOB;
      b_vo_tail[i] = ((T - 1) * BK + 4 * q < K) ? b_vo[i] : OOB;
    } else {
      const int k = S::b_dl_k(i, wave, l), c = S::b_dl_c(i, wave, l);
      const bool ok = (n0 + 4 * c) < N;
      b_vo[i] = ok ? 4u * ((unsigned)k * (unsigned)ldb + (unsigned)(n0 + 4 * c)) : OOB;
      b_vo_tail[i] = b_vo[i];  // rows past K are past the buffer's range
    }
  }
  // Fragment byte offsets: group g of A (other row blocks are immediate
  // offsets), and group 0 step 0 of B (other steps and groups likewise).
  int a_fb[KG];
#pragma unroll
  for (int g = 0; g < KG; ++g) a_fb[g] = S::AT ? 0 : S::a_frag(wm0, 0, g, l);
  const int at_fb = S::AT ? S::at_frag(wm0, 0, 0, l) : 0;
  const int b_fb = S::BT ? 0 : S::b_frag(wn0, 0, 0, l);
  int bt_fb[KG];
#pragma unroll
  for (int g = 0; g < KG; ++g) bt_fb[g] = S::BT ? S::bt_frag(wn0, 0, g, l) : 0;

  auto issue = [&](int s, unsigned char* la, unsigned char* lb) __attribute__((always_inline)) {
    issue_slice<S>(Ab, Bb, a_bytes, b_bytes, s, s < T, s == T - 1 ? a_vo_tail : a_vo,
                   s == T - 1 ? b_vo_tail : b_vo, la, lb, wave, lda, ldb);
  };

  typedef typename VecF<MB>::T vecMB;
  typedef __attribute__((address_space(3))) vecMB lds_vecMB;
  f32x4 fa[2][MB];   // A: four k steps of each row block
  vecMB fat[2][4];   // A^T: each k step's MB rows
  vecNB fb[2][4];
  auto load_frags = [&](int buf, const unsigned char* la, const unsigned char* lb, int g)
      __attribute__((always_inline)) {
    if constexpr (S::AT) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
        fat[buf][s] = *(const lds_vecMB*)(la + at_fb + (8 * g + s) * S::A_ROW);
    } else {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        fa[buf][mb] = *(const lds_f32x4*)(la + a_fb[g] + mb * 32 * S::A_ROW);
    }
    if constexpr (S::BT) {
      // One 16-byte read per block nb: its column's values for steps 0..3.
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const f32x4 t = *(const lds_f32x4*)(lb + bt_fb[g] + nb * 32 * S::B_ROW);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if constexpr (NB == 1) fb[buf][s] = t[s];
          else fb[buf][s][nb] = t[s];
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s)
        fb[buf][s] = *(const lds_vecNB*)(lb + b_fb + (8 * g + s) * S::B_ROW);
    }
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.f;
  auto mma = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          float av, bv;
          if constexpr (!S::AT) av = fa[buf][mb][s];
          else if constexpr (MB == 1) av = fat[buf][s];
          else av = fat[buf][s][mb];
          if constexpr (NB == 1) bv = fb[buf][s]; else bv = fb[buf][s][nb];
          acc[mb][nb] = mfma(av, bv, acc[mb][nb]);
        }
  };

  constexpr int NMMA = 4 * MB * NB;  // MFMAs per k group
  constexpr int NRD = (S::AT ? 4 : MB) + (S::BT ? NB : 4);  // LDS reads per k group
  // (The lambdas are forced inline: a slice of the larger tiles is several
  // hundred MFMAs, past the inliner's budget, and an out-of-line call would
  // move the accumulators to scratch memory.)
  // Slice t from stage c: groups 0..KG-2 with the next group's fragments
  // in flight; wait for slice t+1; barrier; issue slice t+NS into stage c;
  // last group's MFMAs under the first fragment reads of stage c+1.
  auto slice = [&](int t, auto C_) __attribute__((always_inline)) {
    constexpr int c = decltype(C_)::value, n = (c + 1) % NS;
    unsigned char* ca = A_of(IC<c>{});
    unsigned char* cb = B_of(IC<c>{});
#pragma unroll
    for (int g = 0; g + 1 < KG; ++g) {
      load_frags((g + 1) & 1, ca, cb, g + 1);
      mma(g & 1);
#pragma unroll
      for (int i = 0; i < NMMA; ++i) {
        SGB(SG_MFMA, 1);
        if (i < NRD) SGB(SG_DS_RD, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    loop_barrier<(NS - 2) * S::LPS>();
    __builtin_amdgcn_sched_barrier(0);
    issue(t + NS, ca, cb);
    load_frags(0, A_of(IC<n>{}), B_of(IC<n>{}), 0);
    mma((KG - 1) & 1);
#pragma unroll
    for (int i = 0; i < NMMA; ++i) {
      SGB(SG_MFMA, 1);
      if (i < NRD) SGB(SG_DS_RD, 1);
      if (i < S::LPS) SGB(SG_VMEM_RD, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  if (T > 0) {
    static_for([&](auto I) { issue(decltype(I)::value, A_of(I), B_of(I)); },
               std::make_integer_sequence<int, NS>{});
    loop_barrier<(NS - 1) * S::LPS>();  // slice 0 landed
    trace_stamp(p, 1);
    load_frags(0, la0, lb0, 0);
    int t = 0;
    for (; t + NS <= T; t += NS)
      static_for([&](auto I) { slice(t + decltype(I)::value, I); }, std::make_integer_sequence<int, NS>{});
    static_for([&](auto I) { if (t + decltype(I)::value < T) slice(t + decltype(I)::value, I); },
               std::make_integer_sequence<int, NS>{});
    // The copies issued past the last slice still write LDS: they must land
    // before the workgroup ends and its LDS is handed to another.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  }
  trace_stamp(p, 2);

  // Epilogue: acc[mb][nb] register r of lane l holds C[m][n] with
  // m = wm0 + 32mb + 8(r/4) + 4(l/32) + r%4 and n = wn0 + NB*(l%32) + nb:
  // the lane's NB columns of a row are adjacent (one 4*NB-byte store; 32
  // lanes cover 128*NB contiguous bytes of the row).
  float* __restrict__ C = static_cast<float*>(p.C) + sk * p.c_stride;
  const int col = n0 + wn0 + NB * (l % 32);
  // (A^T: block mb's row i is m = wm0 + MB*i + mb.)
  auto row_of = [&](int mb, int r) {
    const int i = 8 * (r / 4) + 4 * (l / 32) + (r % 4);
    return S::AT ? m0 + wm0 + MB * i + mb : m0 + wm0 + 32 * mb + i;
  };
  auto acc_vec = [&](int mb, int r) {
    vecNB v;
    if constexpr (NB == 1) {
      v = acc[mb][0][r];
    } else {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) v[nb] = acc[mb][nb][r];
    }
    return v;
  };
  if constexpr (!S::EPI) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row_of(mb, r);
        if (row < M && col < N)  // streaming store (C is written once)
          __builtin_nontemporal_store(acc_vec(mb, r), reinterpret_cast<vecNB*>(C + (int64_t)row * p.ldc + col));
      }
  } else if constexpr (S::Q8) {
    // INT8-quantising epilogue: the lane's NB adjacent columns of a row
    // become NB bytes, stored branch-free through a byte-addressed buffer
    // descriptor over C (out-of-range elements: an offset past its range).
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(reinterpret_cast<const unsigned char*>(p.C), (int64_t)(M - 1) * p.ldc + N);
    vecNB bias = {};
    if (p.epi.bias && col < N) bias = *reinterpret_cast<const vecNB*>(p.epi.bias + col);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row_of(mb, r);
        const unsigned off = ((row < M) & (col < N)) ? (unsigned)row * (unsigned)p.ldc + (unsigned)col : OOB;
        const vecNB v = acc_vec(mb, r);
        if constexpr (NB == 4) {
          const int w = pack_i8x4(quantize_i8(epi_value(p.epi, v[0], 0.f, bias[0])),
                                  quantize_i8(epi_value(p.epi, v[1], 0.f, bias[1])),
                                  quantize_i8(epi_value(p.epi, v[2], 0.f, bias[2])),
                                  quantize_i8(epi_value(p.epi, v[3], 0.f, bias[3])));
          __builtin_amdgcn_raw_buffer_store_b32(w, rq, off, 0, 0);
        } else if constexpr (NB == 2) {
          const int w = (quantize_i8(epi_value(p.epi, v[0], 0.f, bias[0])) & 0xff) |
                        (quantize_i8(epi_value(p.epi, v[1], 0.f, bias[1])) << 8);
          __builtin_amdgcn_raw_buffer_store_b16((short)w, rq, off, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b8((char)quantize_i8(epi_value(p.epi, v, 0.f, bias)), rq, off, 0, 0);
        }
      }
  } else {
    // Fused epilogue on the FP32 accumulators.  The bias of the lane's
    // columns is loaded once; the old C (read only when beta != 0) is
    // loaded BATCH rows at a time ahead of their stores; the old C and the
    // result go through a buffer descriptor over C, out-of-range elements
    // getting an offset past its range (loads return 0, stores are
    // dropped), so there are no per-element branches, across which the
    // compiler would wait for every memory operation, stores included.
    typedef int vi4 __attribute__((ext_vector_type(4)));
    typedef int vi2 __attribute__((ext_vector_type(2)));
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(reinterpret_cast<const unsigned char*>(C), ((int64_t)(M - 1) * p.ldc + N) * 4);
    auto load = [&](unsigned off) -> vecNB {
      if constexpr (NB == 4) return __builtin_bit_cast(vecNB, __builtin_amdgcn_raw_buffer_load_b128(rc, off, 0, 0));
      else if constexpr (NB == 2) return __builtin_bit_cast(vecNB, __builtin_amdgcn_raw_buffer_load_b64(rc, off, 0, 0));
      else return __builtin_bit_cast(vecNB, __builtin_amdgcn_raw_buffer_load_b32(rc, off, 0, 0));
    };
    auto store = [&](vecNB v, unsigned off) {
      if constexpr (NB == 4) __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(vi4, v), rc, off, 0, 0);
      else if constexpr (NB == 2) __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(vi2, v), rc, off, 0, 0);
      else __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), rc, off, 0, 0);
    };
    vecNB bias = {};
    if (p.epi.bias && col < N) bias = *reinterpret_cast<const vecNB*>(p.epi.bias + col);
    constexpr int BATCH = NB == 4 ? 4 : 8;  // registers: BATCH * NB floats in flight
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r0 = 0; r0 < 16; r0 += BATCH) {
        unsigned off[BATCH];
        vecNB c_old[BATCH];
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
          const int row = row_of(mb, r0 + i);
          off[i] = ((row < M) & (col < N)) ? 4u * ((unsigned)row * (unsigned)p.ldc + (unsigned)col) : OOB;
          c_old[i] = vecNB{};
        }
        if (p.epi.beta != 0.f) {
#pragma unroll
          for (int i = 0; i < BATCH; ++i) c_old[i] = load(off[i]);
        }
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
          vecNB v = acc_vec(mb, r0 + i);
          if constexpr (NB == 1) {
            v = epi_value(p.epi, v, c_old[i], bias);
          } else {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) v[nb] = epi_value(p.epi, v[nb], c_old[i][nb], bias[nb]);
          }
          store(v, off[i]);
        }
      }
  }
  trace_stamp(p, 3);
}

template <class S>
hipError_t launch(const Params& p, const TileMap& map, bool vec, hipStream_t stream) {
  const int64_t lim = 0x7fffffff;
  // Every offset (rows past M and K included) must fit the 31-bit range.
  const bool a_far = S::AT ? (int64_t)(S::BK + 2) * p.lda * 4 > lim ||
                                 ((int64_t)(p.K > 0 ? p.K - 1 : 0) * p.lda + p.M) * 4 > lim
                           : (int64_t)(p.M + S::BM) * p.lda * 4 > lim;
  if (!vec || a_far || (int64_t)(S::BK + 2) * p.ldb * 4 > lim ||
      (S::BT ? (int64_t)(p.N + S::BN) * p.ldb * 4 > lim
             : ((int64_t)(p.K > 0 ? p.K - 1 : 0) * p.ldb + p.N) * 4 > lim) ||
      (S::EPI && (int64_t)p.M * p.ldc * 4 > lim)) {
    // The general kernel has no split-K form (the caller runs unsplit) and
    // no INT8 or transposed-A form (the caller reports the operands
    // unsupported).
    if (p.splits > 1 || S::Q8 || S::AT) return hipErrorNotSupported;
    return sgemm_launch_shape(S::BM, S::BN, S::WM, S::WN, p, map, vec, stream);
  }
  const int64_t a_bytes = p.K <= 0 ? 0
                          : S::AT ? ((int64_t)(p.K - 1) * p.lda + p.M) * 4
                                  : ((int64_t)(p.M - 1) * p.lda + p.K) * 4;
  const int64_t b_bytes = p.K <= 0 ? 0
                          : S::BT ? ((int64_t)(p.N - 1) * p.ldb + p.K) * 4
                                  : ((int64_t)(p.K - 1) * p.ldb + p.N) * 4;
  const dim3 grid(map.tiles_m * map.tiles_n, p.splits), block(S::NT);
  hipLaunchKernelGGL(sgemm_dl_kernel<S>, grid, block, 0, stream, p, map, a_bytes, b_bytes);
  return hipGetLastError();
}

// Host replay of the transposed-B form's B side: Bt rows placed by the
// direct loads (each LDS byte once, row R holding column bt_col(R)), and the
// fragment reads giving each lane the element its MFMA step needs; bank
// conflicts are added to *rconf.  Returns 0 when valid, else a code from 20.
template <class S>
int layout_check_bt(int banks, int64_t* rconf) {
  static_assert(S::BT, "transposed-B shape");
  static int n_of[S::B_STAGE], k_of[S::B_STAGE];
  for (int i = 0; i < S::B_STAGE; ++i) n_of[i] = -1;
  for (int i = 0; i < S::IB; ++i)
    for (int w = 0; w < S::NW; ++w)
      for (int l = 0; l < 64; ++l) {
        const int off = 1024 * (i * S::NW + w) + 16 * l;
        const int R = S::bt_dl_row(i, w, l), q = S::bt_dl_q(i, w, l);
        if (R >= S::BN || q >= S::BK / 4 || S::bt_byte(R, q) != off) return 20;
        for (int e = 0; e < 4; ++e) {
          if (n_of[off + 4 * e] != -1) return 21;
          n_of[off + 4 * e] = S::bt_col(R);
          k_of[off + 4 * e] = 4 * q + e;
        }
      }
  for (int i = 0; i < S::B_STAGE; i += 4)
    if (n_of[i] < 0) return 22;
  int addr[64];
  for (int w = 0; w < S::NW; ++w) {
    const int wn0 = (w % S::WAVES_N) * S::WN;
    for (int g = 0; g < S::KG; ++g)
      for (int nb = 0; nb < S::NB; ++nb) {
        for (int l = 0; l < 64; ++l) {
          addr[l] = S::bt_frag(wn0, nb, g, l);
          if (addr[l] < 0 || addr[l] + 16 > S::B_STAGE) return 23;
          if (addr[l] != S::bt_frag(wn0, 0, g, l) + nb * 32 * S::B_ROW) return 24;
          // Step s: B[k = 8g + 4(l/32) + s][n = wn0 + NB*(l%32) + nb].
          for (int st = 0; st < 4; ++st)
            if (n_of[addr[l] + 4 * st] != wn0 + S::NB * (l % 32) + nb ||
                k_of[addr[l] + 4 * st] != 8 * g + 4 * (l / 32) + st)
              return 25;
        }
        *rconf += lds_conflicts(addr, 16, banks);
      }
  }
  return 0;
}

// Host replay of the transposed-A form's A side: A^T rows placed as loaded,
// and the fragment reads checked for coverage, bounds, the element each
// lane must see in each MFMA step, and bank conflicts (added to *rconf).
// Returns 0 when valid, else a code from 30.
template <class S>
int layout_check_at(int banks, int64_t* rconf) {
  static_assert(S::AT, "transposed-A shape");
  static int m_of[S::A_STAGE], k_of[S::A_STAGE];
  for (int i = 0; i < S::A_STAGE; ++i) m_of[i] = -1;
  for (int i = 0; i < S::IA; ++i)
    for (int w = 0; w < S::NW; ++w)
      for (int l = 0; l < 64; ++l) {
        const int off = 1024 * (i * S::NW + w) + 16 * l;
        const int k = S::at_dl_k(i, w, l), c = S::at_dl_c(i, w, l);
        if (k >= S::BK || S::at_byte(k, 4 * c) != off) return 30;
        for (int e = 0; e < 4; ++e) {
          if (m_of[off + 4 * e] != -1) return 31;
          m_of[off + 4 * e] = 4 * c + e;
          k_of[off + 4 * e] = k;
        }
      }
  for (int i = 0; i < S::A_STAGE; i += 4)
    if (m_of[i] < 0) return 32;
  int addr[64];
  for (int w = 0; w < S::NW; ++w) {
    const int wm0 = (w / S::WAVES_N) * S::WM;
    for (int g = 0; g < S::KG; ++g)
      for (int st = 0; st < 4; ++st) {
        for (int l = 0; l < 64; ++l) {
          addr[l] = S::at_frag(wm0, 0, 0, l) + (8 * g + st) * S::A_ROW;
          if (addr[l] != S::at_frag(wm0, g, st, l)) return 33;
          if (addr[l] < 0 || addr[l] + 4 * S::MB > S::A_STAGE) return 34;
          // Step st, block mb: A[m = wm0 + MB*(l%32) + mb][k = 8g + 4(l/32) + st].
          for (int mb = 0; mb < S::MB; ++mb)
            if (m_of[addr[l] + 4 * mb] != wm0 + S::MB * (l % 32) + mb ||
                k_of[addr[l] + 4 * mb] != 8 * g + 4 * (l / 32) + st)
              return 35;
        }
        *rconf += lds_conflicts(addr, 4 * S::MB, banks);
      }
  }
  return 0;
}

// Host replay: direct-load placement and fragment reads (bounds, the element
// each lane must see in each MFMA step, bank conflicts).  Returns 0 when
// valid.
template <class S>
int layout_check(int banks, int64_t out[2]) {
  constexpr int BM = S::BM, BK = S::BK, NB = S::NB;
  int64_t rconf = 0;
  static int a_row_of[S::A_STAGE], a_k_of[S::A_STAGE], b_k_of[S::B_STAGE], b_n_of[S::B_STAGE];
  for (int i = 0; i < S::A_STAGE; ++i) a_row_of[i] = -1;
  for (int i = 0; i < S::B_STAGE; ++i) b_k_of[i] = -1;
  for (int i = 0; i < S::IA; ++i)
    for (int w = 0; w < S::NW; ++w)
      for (int l = 0; l < 64; ++l) {
        const int off = 1024 * (i * S::NW + w) + 16 * l;
        const int r = S::a_dl_row(i, w, l), q = S::a_dl_q(i, w, l);
        if (r >= BM || q >= S::A_CPR || S::a_byte(r, q) != off) return 1;
        for (int e = 0; e < 4; ++e) {
          if (a_row_of[off + 4 * e] != -1) return 2;
          a_row_of[off + 4 * e] = r;
          a_k_of[off + 4 * e] = 4 * q + e;
        }
      }
  for (int i = 0; i < S::IB; ++i)
    for (int w = 0; w < S::NW; ++w)
      for (int l = 0; l < 64; ++l) {
        const int off = 1024 * (i * S::NW + w) + 16 * l;
        const int k = S::b_dl_k(i, w, l), c = S::b_dl_c(i, w, l);
        if (k >= BK || S::b_byte(k, 4 * c) != off) return 3;
        for (int e = 0; e < 4; ++e) {
          if (b_k_of[off + 4 * e] != -1) return 4;
          b_k_of[off + 4 * e] = k;
          b_n_of[off + 4 * e] = 4 * c + e;
        }
      }
  for (int i = 0; i < S::A_STAGE; i += 4)
    if (a_row_of[i] < 0) return 5;
  for (int i = 0; i < S::B_STAGE; i += 4)
    if (b_k_of[i] < 0) return 6;
  int addr[64];
  for (int w = 0; w < S::NW; ++w) {
    const int wm0 = (w / S::WAVES_N) * S::WM, wn0 = (w % S::WAVES_N) * S::WN;
    for (int g = 0; g < S::KG; ++g) {
      for (int mb = 0; mb < S::MB; ++mb) {
        for (int l = 0; l < 64; ++l) {
          addr[l] = S::a_frag(wm0, mb, g, l);
          if (addr[l] < 0 || addr[l] + 16 > S::A_STAGE) return 7;
          if (addr[l] != S::a_frag(wm0, 0, g, l) + mb * 32 * S::A_ROW) return 8;
          // Step s: A[m = wm0 + 32mb + l%32][k = 8g + 4(l/32) + s].
          for (int s = 0; s < 4; ++s) {
            const int b = addr[l] + 4 * s;
            if (a_row_of[b] != wm0 + 32 * mb + l % 32 || a_k_of[b] != 8 * g + 4 * (l / 32) + s) return 9;
          }
        }
        rconf += lds_conflicts(addr, 16, banks);
      }
      for (int s = 0; s < 4; ++s) {
        for (int l = 0; l < 64; ++l) {
          addr[l] = S::b_frag(wn0, g, s, l);
          if (addr[l] < 0 || addr[l] + 4 * NB > S::B_STAGE) return 10;
          if (addr[l] != S::b_frag(wn0, 0, 0, l) + (8 * g + s) * S::B_ROW) return 11;
          // Block nb, step s: B[k = 8g + 4(l/32) + s][n = wn0 + NB*(l%32) + nb].
          for (int nb = 0; nb < NB; ++nb) {
            const int b = addr[l] + 4 * nb;
            if (b_k_of[b] != 8 * g + 4 * (l / 32) + s || b_n_of[b] != wn0 + NB * (l % 32) + nb) return 12;
          }
        }
        rconf += lds_conflicts(addr, 4 * NB, banks);
      }
    }
  }
  int rc = layout_check_bt<Shape<S::BM, S::BN, S::WM, S::WN, S::BK, S::NS, false, true>>(banks, &rconf);
  if (rc != 0) return rc;
  rc = layout_check_at<Shape<S::BM, S::BN, S::WM, S::WN, S::BK, S::NS, false, false, false, true>>(banks, &rconf);
  if (rc != 0) return rc;
  // Both transposed: B's side must not depend on A's row length.
  rc = layout_check_bt<Shape<S::BM, S::BN, S::WM, S::WN, S::BK, S::NS, false, true, false, true>>(banks, &rconf);
  if (rc != 0) return rc;
  out[0] = 0;  // no LDS writes by the waves (copies are LDS-direct)
  out[1] = rconf;
  return 0;
}

#define SGEMM_DL_VARIANT(BM, BN, WM, WN, BK, NS, GM, EFF)                                         \
  Variant {                                                                                  \
    gemm_config_t{0, GEMM_DTYPE_F32, GEMM_FAMILY_MFMA, BM, BN, BK, WM, WN,                   \
                  Shape<BM, BN, WM, WN, BK, NS>::NT, NS, Shape<BM, BN, WM, WN, BK, NS>::LDS_BYTES, \
                  GEMM_ORDER_XCD, GM, 1,                                                     \
                  "dl_f32_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_s" #NS},                  \
        &launch<Shape<BM, BN, WM, WN, BK, NS>>, &layout_check<Shape<BM, BN, WM, WN, BK, NS>>, \
        &launch<Shape<BM, BN, WM, WN, BK, NS>>, EFF,                                        \
        &launch<Shape<BM, BN, WM, WN, BK, NS, true>>,                                       \
        &launch<Shape<BM, BN, WM, WN, BK, NS, false, true>>,                                \
        &launch<Shape<BM, BN, WM, WN, BK, NS, false, false, true>>,                         \
        &launch<Shape<BM, BN, WM, WN, BK, NS, false, false, false, true>>,                  \
        &launch<Shape<BM, BN, WM, WN, BK, NS, false, true, false, true>>                    \
  }

const Variant kVariants[] = {
    SGEMM_DL_VARIANT(256, 256, 128, 128, 32, 2, 4, 1.00f),
    SGEMM_DL_VARIANT(256, 256, 128, 128, 16, 4, 4, 0.99f),
    SGEMM_DL_VARIANT(256, 128, 128, 64, 32, 3, 8, 0.97f),
    SGEMM_DL_VARIANT(128, 256, 64, 128, 32, 3, 8, 0.97f),
    SGEMM_DL_VARIANT(128, 128, 64, 64, 32, 3, 8, 0.95f),
    SGEMM_DL_VARIANT(64, 64, 32, 32, 64, 2, 8, 0.92f),
};

}  // namespace

const Variant* sgemm_dl_variants(int* count) {
  *count = sizeof(kVariants) / sizeof(kVariants[0]);
  return kVariants;
}

}  // namespace gemm
