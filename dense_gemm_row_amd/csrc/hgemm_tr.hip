// FP16 HGEMM for aligned operands, built around gfx950's LDS-direct loads and
// LDS transpose reads: binary16 A and B, FP32 accumulation on
// v_mfma_f32_32x32x16_f16, one round-to-nearest-even conversion per output.
// The same kernel, with v_mfma_f32_32x32x16_bf16 and bfloat16 conversions,
// is the BF16 GEMM, and with 8-bit elements, v_mfma_f32_32x32x64_f8f6f4
// (k 64 per MFMA) and bfloat16 output it is the FP8 GEMM, E4M3 or E5M2 by
// the instruction's operand format (Shape's TY_): the data path moves bit
// patterns and never looks inside them.  For
// FP8, a lane's operand is 32 bytes (two 16-byte A chunks; four
// ds_read_b64_tr_b8 reads of B, the byte form of the transpose read below:
// output lane j of a 16-lane group gets byte j%8 of the 8-byte pieces of
// lanes j/8 + 2t, t = 0..7, measured on the device), and B's 16-byte chunk
// index is XORed by 2*(k%8) instead of 4*(k%4).
//
// Data path per K slice (no VGPR staging, no VALU in the main loop):
// * A and B move from global memory straight into LDS with
//   buffer_load_dwordx4 ... lds: one instruction fills 1 KB of LDS per wave,
//   lane l writing bytes [16l, 16l+16) of the wave's block, so each lane
//   fetches the 16-byte global chunk whose (swizzled) LDS position is 16l.
//   The A tile is row-major (k contiguous, 2*BK-byte rows, chunk XOR
//   swz_row); the B tile is row-major as in memory (n contiguous, BN*2-byte
//   rows) with the 16-byte chunk index XORed by 4*(k%4).
// * The matrix core needs B down columns (8 consecutive k per lane).  The
//   transpose read ds_read_b64_tr_b16 provides that: within each group of
//   16 lanes, output lane j receives element j%4 of the 8-byte pieces
//   addressed by lanes j/4, 4+j/4, 8+j/4 and 12+j/4 (lane-map checked on the
//   device), so pointing lane 4t+q at row k+t, columns c+4q..c+4q+3 hands
//   lane j the four values B[k..k+3][c+j].  Two such reads give the eight k
//   values of one MFMA operand.
// * Operands are swapped in the MFMA: it computes blocks of C^T = B^T A^T,
//   so an accumulator register group holds four consecutive output columns
//   of one output row.  This is the transposed-operand idea of "sgemm -
//   beyond cuBLAS" (section 3) and of "hgemm_naive_kernel explained"
//   (section 7.1), done by the hardware transpose read instead of a
//   transposed store.
// * K advances by moving the buffer descriptors' base address and shrinking
//   their range (scalar adds); loads outside the matrix (rows past M or K,
//   columns past N) are range-checked by the hardware and return zeros.  The
//   last, partial K slice of A is masked per lane.  Fragment addresses are
//   per-lane constants plus immediate offsets.
// * NS LDS stages (K slices of BK = 32 or 64), one barrier per slice; the
//   last k step's MFMAs (registers only) run after the barrier, covering
//   the first fragment reads of the next stage.  With two stages the copy
//   of slice t+2 is issued in one burst right after the barrier that frees
//   its stage.  With three or more, the copies of slice t+NS-1 are spread
//   evenly over all k steps of slice t (a few per k step between MFMAs):
//   a wave that issues an LDS-direct copy can stall at issue when the
//   vector memory path is busy, and a burst of copies stalls the MFMA
//   stream behind it.  The barrier itself carries no memory fence (see
//   loop_barrier), so copies of later slices stay in flight across it.  This generalises the double buffer of
//   "sgemm - beyond cuBLAS" (section 6) with the asynchronous copies that
//   the lqnn.cn SGEMM article adds in section 3.5.  Each stage is its own
//   __shared__ array and the loop is unrolled NS times, so every access
//   names its array statically and the compiler can see that copies into
//   one stage do not alias reads of another (otherwise it waits for all
//   copies before every read).
// * Epilogue through LDS: each wave stores its FP16 tile row-major into its
//   share of the stage arrays (8-byte slots XOR-swizzled by row:
//   conflict-free writes), then reads whole 16-byte row chunks back and
//   writes C with WN/8 lanes per row segment (the coalesced write-back of
//   section 5).
#include <type_traits>
#include <utility>

#include "gemm_internal.h"

namespace gemm {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) f16x8 lds_f16x8;

constexpr unsigned OOB = 0x80000000u;  // offset past every buffer's range
constexpr int MAX_STAGES = 5;

template <int I>
using IC = std::integral_constant<int, I>;

template <class F, int... I>
__device__ __forceinline__ void static_for(F&& f, std::integer_sequence<int, I...>) {
  (f(IC<I>{}), ...);
}

// Template parameters beyond the tile (BM x BN, wave tiles WM x WN, K slice
// BK, NS stages):
// * MODE_: 0 the plain kernel; 1 the split-K form, whose epilogue writes
//   FP32 partials; 2 the form with the fused epilogue (alpha, beta, bias,
//   activation); 3 the fused epilogue writing INT8 codes (C is int8, beta 0).
// * BT_: B is given transposed (Bt, N x K row-major, i.e. column-major B);
//   its tile is then staged and read exactly like A's (one LDS row per
//   output column, k contiguous), with no transpose read.
// * TY_: the element types, 0 binary16 in and out, 1 bfloat16 in and out,
//   2 FP8 E4M3 in and bfloat16 out, 3 FP8 E5M2 in and bfloat16 out.
// * AT_: A given transposed (At, K x M row-major, i.e. column-major A): its
//   tile is staged and read exactly like B's (k rows of BM values, chunk XOR
//   by k, transpose reads), which hands each lane the same k run of its row
//   as the direct read of row-major A.
// * PW_: producer waves (0: none).  With PW_ > 0 the workgroup is split by
//   role: the NW compute waves only read LDS and run MFMAs, and PW_ further
//   waves only issue the LDS-direct copies and wait for them to land; both
//   meet at the one barrier per K slice.  This is the load/compute
//   separation that "hgemm_naive_kernel explained" lists among its further
//   directions (section 10.3), with LDS-direct copies in the role that
//   "nxbn.cn GB300 GEMM" (section 3.2) gives to a copy engine driven by a
//   few threads.
// * MI_: the matrix instruction's output block, 32 (32 x 32, k 16 or 64)
//   or 16 (16 x 16, twice the k: v_mfma_f32_16x16x32_f16 / _bf16,
//   v_mfma_f32_16x16x128_f8f6f4).  Both take the same operand registers
//   (8 16-bit or 32 8-bit k values per lane) and do the same work per
//   cycle, but under MI355X's power limit the 16 x 16 stream runs at a
//   higher clock (register-only rate on the device: FP16 about 1960 against
//   1735 TFLOP/s, FP8 4640 against 4255).  A 16 x 16 block's operand lane l
//   holds row (column) l%16 and k run l/16 of four; its accumulator
//   register r holds output row 4(l/16) + r, column l%16.
template <int BM_, int BN_, int WM_, int WN_, int BK_, int NS_, int MODE_ = 0, bool BT_ = false,
          int TY_ = 0, bool AT_ = false, int PW_ = 0, int MI_ = 32>
struct Shape {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, NS = NS_, TY = TY_;
  static constexpr int PW = PW_, MI = MI_;
  static constexpr bool AT = AT_;
  static constexpr bool PARTIAL = MODE_ == 1, EPI = MODE_ == 2 || MODE_ == 3, Q8 = MODE_ == 3, BT = BT_;
  static constexpr bool BF = TY != 0;   // C (and the epilogue's old C) is bfloat16
  static constexpr bool F8 = TY >= 2;   // A and B are FP8 (E4M3, or E5M2 when TY == 3)
  static constexpr int ES = F8 ? 1 : 2;    // input element bytes
  static constexpr int CE = 16 / ES;       // input elements per 16-byte chunk
  static_assert(MI == 32 || MI == 16, "matrix instruction");
  static constexpr int KW = (F8 ? 64 : 16) * (32 / MI);  // k per MFMA
  static constexpr int LG = 64 / MI, KL = KW / LG;  // lane groups along k; k per lane
  static constexpr int AR = MI * MI / 64, RQ = AR / 4;  // accumulators per block; 4-column groups
  static constexpr int FR = F8 ? 2 : 1;    // 16-byte chunks per lane in an A / Bt operand
  static constexpr int TRN = F8 ? 4 : 2;   // transpose reads per B operand
  static constexpr int RR = F8 ? 8 : 4;    // k rows (elements per lane) of one transpose read
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN, NW = WAVES_M * WAVES_N;
  // NL waves issue the copies: the producers, or every wave.
  static constexpr int NL = PW > 0 ? PW : NW, NT = (NW + PW) * 64;
  static constexpr int MB = WM / MI, NB = WN / MI, KS = BK / KW;
  static constexpr int NMMA_ = MB * NB;  // MFMAs per k step
  // A rows: BM rows of BK k values, or (AT) BK rows of BM values.
  static constexpr int A_ROW = AT ? BM * ES : BK * ES, A_CPR = A_ROW / 16;  // bytes / chunks
  // B rows: BK rows of BN columns, or (BT) BN rows of BK k values.
  static constexpr int B_ROW = BT ? BK * ES : BN * ES, B_CPR = B_ROW / 16;  // bytes / chunks
  static constexpr int A_STAGE = AT ? BK * A_ROW : BM * A_ROW, B_STAGE = BT ? BN * B_ROW : BK * B_ROW;
  static constexpr int LDS_BYTES = NS * (A_STAGE + B_STAGE);
  static constexpr int IA = A_STAGE / 1024 / NL, IB = B_STAGE / 1024 / NL, LPS = IA + IB;
  // With three or more stages a slice's copies are spread over the k steps
  // of the slice before (PP per step); with two they go out in one burst
  // after the barrier that frees their stage.
  // (Producer waves have nothing else to do: they issue in bursts.)
  static constexpr bool SPREAD = NS >= 3 && PW == 0;
  static constexpr int PP = LPS / KS;
  // Epilogue: wave w stages its tile in P of the 2*NS stage arrays
  // (A arrays first), RPA rows per array.
  static constexpr int EPI_ROW = WN * 2, EPI_SPR = WN / 4;
  static constexpr int P = (2 * NS) / NW, RPA = WM / P;
  static constexpr int EPI_CPR = WN / 8, EPI_RPI = 64 / EPI_CPR;  // store pass shape
  // The persistent form's wave-private epilogue staging: 32 rows.
  static constexpr int PS_EPI_BYTES = 32 * EPI_ROW;
  static_assert(F8 ? (BK == 64 || BK == 128) : (BK == 32 || BK == 64), "K slice");
  static_assert(BK % KW == 0, "whole matrix instructions per K slice");
  // Fragments alternate between two register sets by global k step
  // (slice * KS + step); the slice loop is unrolled NS times, so the set of
  // each step is static when NS * KS is even.
  static_assert((NS * KS) % 2 == 0, "k steps per unrolled slice group");
  __host__ __device__ static constexpr int frag_set(int stage, int j) { return (stage * KS + j) & 1; }
  static_assert(NS >= 2 && NS <= MAX_STAGES, "stages");
  static_assert(BM % WM == 0 && BN % WN == 0, "wave grid");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile");
  // The 16 x 16 epilogue staging XORs 16-byte chunks by the row's low 4 bits.
  static_assert(MI == 32 || WN * 2 >= 256, "16 x 16 blocks: wave tiles at least 128 wide");
  static_assert(A_STAGE % (1024 * NL) == 0 && B_STAGE % (1024 * NL) == 0, "direct-load split");
  // A compute wave and a producer wave share a SIMD, so the compute waves
  // must fit half of its 512 registers: wave tiles of at most 128 x 64.
  static_assert(PW == 0 || (WM * WN <= 128 * 64 && NW == 4 && PW <= 4), "producer waves");
  static_assert(BT || B_CPR >= 16, "B rows of at least 256 bytes (the k%4 chunk XOR)");
  static_assert(!AT || A_CPR >= 16, "A^T rows of at least 256 bytes (the chunk XOR)");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert((NS - 1) * LPS <= 63, "vmcnt field");
  static_assert(!SPREAD || (LPS % KS == 0 && PP <= NMMA_), "copies split evenly over k steps");
  // Spread: MFMA slot i of a k step carries a copy when i*PP/NMMA steps up.
  __host__ __device__ static constexpr bool copy_slot(int i) {
    return (i + 1) * PP / NMMA_ > i * PP / NMMA_;
  }
  static_assert(P >= 1 && WM % P == 0 && RPA % 32 == 0 && RPA % EPI_RPI == 0 &&
                RPA * EPI_ROW <= A_STAGE && RPA * EPI_ROW <= B_STAGE, "epilogue staging");
  // Fragment reads use a per-lane base plus immediate offsets (< 64 KB).
  static_assert((AT ? (BK - KW + RR * (TRN - 1)) * A_ROW : (MB - 1) * MI * A_ROW) < 65536 &&
                (BK - KW + RR * (TRN - 1)) * B_ROW < 65536 && (NB - 1) * MI * B_ROW < 65536,
                "immediate offsets");

  // Byte offsets within one stage array.
  __host__ __device__ static constexpr int a_byte(int r, int q) { return swz_off(r, q, A_ROW); }
  // B chunk XOR: the rows one transpose read touches (4 for 16-bit, 8 for
  // 8-bit) land on distinct 16-byte (32-byte) bank slots.  With 16 x 16
  // blocks the second 16 lanes of a read take the next k run (KL rows on)
  // of the same columns instead of the next 16 columns, so the run's
  // parity also flips one chunk-index bit.
  __host__ __device__ static constexpr int b_swz(int k) {
    return (F8 ? 2 * (k % 8) : 4 * (k % 4)) ^ (MI == 16 ? (F8 ? 1 : 2) * ((k / KL) % 2) : 0);
  }
  __host__ __device__ static constexpr int b_phys(int k, int c) { return c ^ b_swz(k); }
  __host__ __device__ static constexpr int b_byte(int k, int n) {
    return k * B_ROW + 16 * b_phys(k, n / CE) + ES * (n % CE);
  }
  // Direct loads: lane l of loading wave w, instruction i.
  __host__ __device__ static constexpr int a_dl_row(int i, int w, int l) {
    return (1024 / A_ROW) * (i * NL + w) + l / A_CPR;
  }
  __host__ __device__ static constexpr int a_dl_q(int i, int w, int l) {
    return (l % A_CPR) ^ swz_row(a_dl_row(i, w, l), A_ROW);
  }
  __host__ __device__ static constexpr int b_dl_k(int i, int w, int l) {
    return (1024 * (i * NL + w) + 16 * l) / B_ROW;
  }
  __host__ __device__ static constexpr int b_dl_c(int i, int w, int l) {
    return ((1024 * (i * NL + w) + 16 * l) % B_ROW / 16) ^ b_swz(b_dl_k(i, w, l));
  }
  // Fragment reads for k step j of a slice.  Lane l's operand holds k
  // KW*j + KL*(l/MI) + 0 .. KL-1 (any k order common to both operands
  // gives the same product; this one keeps each lane's k run contiguous).
  //  B_op (A values): lane reads row wm0 + MI*mb + l%MI, chunks
  //  FR*(LG*j + l/MI) + part.
  __host__ __device__ static constexpr int a_frag(int wm0, int mb, int j, int l, int part = 0) {
    return a_byte(wm0 + MI * mb + l % MI, FR * (LG * j + l / MI) + part);
  }
  //  A_op (B values, transpose read jr of TRN): lane LPR*t + q of 16-lane
  //  group g (LPR = 16/RR lanes per row) points at row KW*j + KL*(l/MI) +
  //  RR*jr + t, columns wn0 + MI*nb + 16((l%MI)/16) + (8/ES)q.
  __host__ __device__ static constexpr int b_frag(int wn0, int nb, int j, int jr, int l) {
    return b_byte(KW * j + KL * (l / MI) + RR * jr + (l % 16) / (16 / RR),
                  wn0 + MI * nb + 16 * ((l % MI) / 16) + (8 / ES) * (l % (16 / RR)));
  }
  // AT: A^T tile row k, value m (B's layout with BM values per row); the
  // direct loads; the transpose read jr of k step j for row block mb
  // (b_frag's lane map with wm0 + 32mb for wn0 + 32nb).
  __host__ __device__ static constexpr int at_byte(int k, int m) {
    return k * A_ROW + 16 * b_phys(k, m / CE) + ES * (m % CE);
  }
  __host__ __device__ static constexpr int at_dl_k(int i, int w, int l) {
    return (1024 * (i * NL + w) + 16 * l) / A_ROW;
  }
  __host__ __device__ static constexpr int at_dl_c(int i, int w, int l) {
    return ((1024 * (i * NL + w) + 16 * l) % A_ROW / 16) ^ b_swz(at_dl_k(i, w, l));
  }
  __host__ __device__ static constexpr int at_frag(int wm0, int mb, int j, int jr, int l) {
    return at_byte(KW * j + KL * (l / MI) + RR * jr + (l % 16) / (16 / RR),
                   wm0 + MI * mb + 16 * ((l % MI) / 16) + (8 / ES) * (l % (16 / RR)));
  }
  // BT direct loads: Bt rows (B_ROW bytes) placed like row-major A's rows,
  // by B's own row length (with A transposed the two differ).
  __host__ __device__ static constexpr int bt_dl_row(int i, int w, int l) {
    return (1024 / B_ROW) * (i * NL + w) + l / (B_ROW / 16);
  }
  __host__ __device__ static constexpr int bt_dl_q(int i, int w, int l) {
    return (l % (B_ROW / 16)) ^ swz_row(bt_dl_row(i, w, l), B_ROW);
  }
  // BT: B tile row n (one output column), 16-byte k chunk q, placed and read
  // with A's maps (B_ROW == A_ROW): lane reads column wn0 + MI*nb + l%MI,
  // chunks FR*(LG*j + l/MI) + part of k step j (the MFMA A operand of C^T
  // directly).
  __host__ __device__ static constexpr int bt_byte(int n, int q) { return swz_off(n, q, B_ROW); }
  __host__ __device__ static constexpr int bt_frag(int wn0, int nb, int j, int l, int part = 0) {
    return bt_byte(wn0 + MI * nb + l % MI, FR * (LG * j + l / MI) + part);
  }
  // 16 x 16 K loop: each k step is a fixed sequence of the MB x NB MFMAs;
  // the next step's operand read f (A's MB operands, then B's NB) is
  // placed after MFMA rd_after(f), the slice's copy q after MFMA
  // cp_after(q) (at most one of each after any MFMA).  The copies go one
  // per four MFMAs (one per 64 cycles of the matrix core): packed one per
  // MFMA they stalled the MFMA stream (2.9 K against 2.3 K cycles per
  // slice at 4096^3; every second MFMA, 2.6 K), LDS-direct copies stalling
  // at issue while the vector memory path is busy.
  // With 8-bit operands (32 bytes per lane) the B operands have one
  // register set (FBS): B's block nb is re-read right after the last MFMA
  // that uses it (MB*nb + MB-1), 56 MFMAs before the next step needs it,
  // and only A's operands alternate between two sets; the A reads go early
  // (after MFMA 2f), since the next step's first MFMAs need all of them.
  static constexpr int FBS = (MI == 16 && F8) ? 1 : 2;
  __host__ __device__ static constexpr int fb_set(int buf, int nb) { return FBS == 1 ? 0 * nb : buf; }
  // With one k step per slice (FP8's 128-k slices), the slice's barrier
  // sits inside the step, after MFMA BAR_AFTER, so that the previous step's
  // last operand reads (issued after its last MFMA) land meanwhile; the
  // reads from the next stage and the copies come after it.
  static constexpr int BAR_AFTER = (MI == 16 && KS == 1) ? 15 : -1;
  __host__ __device__ static constexpr int rd_after(int f) {
    return FBS == 1 ? (f < MB ? BAR_AFTER + 1 + 2 * f
                              : (MB * (f - MB) + MB - 1 > BAR_AFTER + 1 + 2 * MB + 4 * (f - MB)
                                     ? MB * (f - MB) + MB - 1
                                     : BAR_AFTER + 1 + 2 * MB + 4 * (f - MB)))
                    : BAR_AFTER + 1 + 4 * f;
  }
  // (One copy per 64 matrix-core cycles: every fourth 16-cycle 16-bit MFMA,
  // every second 32-cycle FP8 one; FP8's copies land before the next
  // slice's barrier, 32 MFMAs after the last one.)
  __host__ __device__ static constexpr int cp_after(int q) {
    return BAR_AFTER >= 0 ? BAR_AFTER + 2 + (F8 ? 2 : 4) * q : 4 * q + 2;
  }
  // Every operand read and copy has its own slot among the step's MFMAs,
  // a single-set B operand is re-read only after its last MFMA, and with
  // the barrier inside the step everything reads or writes after it.
  __host__ __device__ static constexpr bool schedule_ok() {
    for (int a = 0; a < MB + NB; ++a) {
      const int x = rd_after(a);
      if (x < 0 || x >= MB * NB || x <= BAR_AFTER) return false;
      if (a >= MB && fb_set(1, a - MB) == 0 && x < MB * (a - MB) + MB - 1) return false;
      for (int b = a + 1; b < MB + NB; ++b)
        if (rd_after(b) == x) return false;
    }
    for (int a = 0; a < LPS; ++a) {
      const int x = cp_after(a);
      if (x < 0 || x >= MB * NB || x <= BAR_AFTER) return false;
      for (int b = a + 1; b < LPS; ++b)
        if (cp_after(b) == x) return false;
    }
    return true;
  }
  __host__ __device__ static constexpr int rd_at(int i) {
    for (int f = 0; f < MB + NB; ++f)
      if (rd_after(f) == i) return f;
    return -1;
  }
  __host__ __device__ static constexpr int cp_at(int i) {
    for (int q = 0; q < LPS; ++q)
      if (cp_after(q) == i) return q;
    return -1;
  }
  // Accumulator block (nb, mb), register 4rq + e of lane l: C[m][n] with
  // m = MI*mb + l%MI and n = MI*nb + 8rq + 4(l/MI) + e (wave-tile
  // coordinates): four consecutive columns of one row per register group.
  __host__ __device__ static constexpr int acc_row(int mb, int l) { return MI * mb + l % MI; }
  __host__ __device__ static constexpr int acc_col(int nb, int rq, int l) { return MI * nb + 8 * rq + 4 * (l / MI); }
  // Epilogue staging: 8-byte slot s (columns 4s..4s+3) of local row m of an
  // array, XOR-swizzled by the row so that the rows written by one
  // instruction hit different bank pairs (32 rows of one slot for 32 x 32
  // blocks; 16 rows of two adjacent slots for 16 x 16 blocks, so there the
  // 16-byte chunk is XORed by the row's low 4 bits); read back 8 bytes at a
  // time.
  __host__ __device__ static constexpr int epi_byte(int m, int s) {
    return MI == 32 ? m * EPI_ROW + 8 * (s ^ (m % EPI_SPR))
                    : m * EPI_ROW + 16 * ((s / 2) ^ (m % 16)) + 8 * (s % 2);
  }
  // Read back 16-byte chunk c (columns 8c..8c+7) of local row m: two
  // 8-byte slots, or with 16 x 16 blocks one 16-byte read (the slots are
  // adjacent there).
  __device__ static u32x4 epi_chunk(const unsigned char* base, int m, int c) {
    if constexpr (MI == 16) {
      return *reinterpret_cast<const u32x4*>(base + epi_byte(m, 2 * c));
    } else {
      const uint2 lo = *reinterpret_cast<const uint2*>(base + epi_byte(m, 2 * c));
      const uint2 hi = *reinterpret_cast<const uint2*>(base + epi_byte(m, 2 * c + 1));
      return u32x4{lo.x, lo.y, hi.x, hi.y};
    }
  }
  // Fused-epilogue staging (FP32, two passes of WM/2 rows in the same
  // region): R32 rows per array, 16-byte chunk q of local row m at chunk
  // position q ^ (m % CPR32); RPI32 rows per read instruction.
  static constexpr int CPR32 = WN / 4, ROW32 = WN * 4, R32 = RPA / 2, RPI32 = 64 / CPR32;
  static_assert(MB % 2 == 0 && CPR32 >= 16 && R32 % RPI32 == 0 && R32 % 32 == 0 &&
                R32 * ROW32 == RPA * EPI_ROW, "fused-epilogue staging");
  __host__ __device__ static constexpr int epi32_byte(int m, int q) {
    return m * ROW32 + 16 * (q ^ (m % CPR32));
  }
};

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

// The 16 x 16 matrix instruction as inline assembly (16-bit operands: k 32;
// FP8: k 128), its accumulator tied in place ("+a").  With the builtin, the register
// allocator kept reassigning the 64 four-register accumulators of a
// 128 x 128 wave tile and moved most of them between registers on every
// pass of the K loop (hundreds of extra instructions per slice); tied
// operands keep each in its registers.  The compiler's hazard checks do
// not see into the assembly, so the kernels (a) write the accumulators
// only before a guard (mfma_guard) that precedes the first MFMA, read them
// only after one that follows the last, and (b) feed srcA / srcB only from
// LDS reads, whose arrival the compiler's own waits cover.
template <int TY, class Frag>
__device__ __forceinline__ void mfma16_asm(f32x4& c, const Frag& a, const Frag& b) {
  // (Device pass only: the host pass checks asm operand constraints against
  // the host target, which has no 256-bit "v" registers.)
#if defined(__HIP_DEVICE_COMPILE__)
  if constexpr (TY == 0)
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  else if constexpr (TY == 1)
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  else if constexpr (TY == 2)  // E4M3 operands (format fields 0)
    asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  else  // E5M2 operands (format fields 1)
    asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0 cbsz:1 blgp:1" : "+a"(c) : "v"(a), "v"(b));
#endif
}

// 24 wait states, with nothing scheduled across: more than any matrix-core
// hazard of gfx950 needs (an XDL result read by a vector instruction, the
// longest, needs under 20).
__device__ __forceinline__ void mfma_guard() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Issue the LDS-direct copies of K slice s into one stage.  The buffer
// descriptors start at the slice (base moved by s*BK along k) and end at the
// matrix end, so rows past K (and anything past the last element) load as
// zeros.  A device function rather than a kernel lambda: lambdas of a kernel
// are also compiled for the host, and a descriptor value there makes the
// host pass drop the kernel's launch stub.
template <class S, int Q0 = 0, int Q1 = S::LPS>
__device__ __forceinline__ void issue_slice(const unsigned char* Ab, const unsigned char* Bb,
                                            int64_t a_bytes, int64_t b_bytes, int s, bool live,
                                            const unsigned* a_vo, const unsigned* b_vo,  // this slice's
                                            unsigned char* lds_a, unsigned char* lds_b, int wave,
                                            int lda, int ldb) {
  // Slices past the last one (issued only to keep the wait counts uniform)
  // get empty descriptors: they load zeros without touching memory.
  const int64_t ka = S::AT ? (int64_t)s * S::BK * lda * S::ES : S::ES * (int64_t)s * S::BK;
  const int64_t kb = S::BT ? S::ES * (int64_t)s * S::BK : (int64_t)s * S::BK * ldb * S::ES;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ab + ka, live ? a_bytes - ka : 0);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bb + kb, live ? b_bytes - kb : 0);
  // Copy instructions Q0 .. Q1-1 of the slice: A's IA blocks, then B's IB.
#pragma unroll
  for (int q = Q0; q < Q1; ++q) {
    if (q < S::IA) {
      lds_void* dst = (lds_void*)(lds_a + 1024 * (q * S::NL + wave));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, a_vo[q], 0, 0, 0);
    } else {
      lds_void* dst = (lds_void*)(lds_b + 1024 * ((q - S::IA) * S::NL + wave));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, dst, 16, b_vo[q - S::IA], 0, 0, 0);
    }
  }
}

// Copy q alone of the persistent kernel's slice s (issue_slice_ps's copy q).
template <class S>
__device__ __forceinline__ void issue_copy_ps(const unsigned char* Ab, const unsigned char* Bb,
                                              int64_t a_bytes, int64_t b_bytes, int s, bool live,
                                              bool last, const unsigned* a_vo, unsigned a_tail,
                                              const unsigned* b_vo, unsigned char* lds_a,
                                              unsigned char* lds_b, int wave, int lda, int ldb, int q) {
  if (q < S::IA) {
    const int64_t ka = S::ES * (int64_t)s * S::BK;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ab + ka, live ? a_bytes - ka : 0);
    lds_void* dst = (lds_void*)(lds_a + 1024 * (q * S::NL + wave));
    const unsigned off = (last && !((a_tail >> q) & 1u)) ? OOB : a_vo[q];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, off, 0, 0, 0);
  } else {
    const int64_t kb = (int64_t)s * S::BK * ldb * S::ES;
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bb + kb, live ? b_bytes - kb : 0);
    lds_void* dst = (lds_void*)(lds_b + 1024 * ((q - S::IA) * S::NL + wave));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, dst, 16, b_vo[q - S::IA], 0, 0, 0);
  }
}

// Copy q alone of slice s (issue_slice's copy q), for the 16 x 16 K loop,
// which places each copy between two MFMAs.  (Its own function: see
// issue_slice_ps.)
template <class S>
__device__ __forceinline__ void issue_copy(const unsigned char* Ab, const unsigned char* Bb,
                                           int64_t a_bytes, int64_t b_bytes, int s, bool live,
                                           const unsigned* a_vo, const unsigned* b_vo,
                                           unsigned char* lds_a, unsigned char* lds_b, int wave,
                                           int lda, int ldb, int q) {
  const int64_t ka = S::AT ? (int64_t)s * S::BK * lda * S::ES : S::ES * (int64_t)s * S::BK;
  const int64_t kb = S::BT ? S::ES * (int64_t)s * S::BK : (int64_t)s * S::BK * ldb * S::ES;
  if (q < S::IA) {
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ab + ka, live ? a_bytes - ka : 0);
    lds_void* dst = (lds_void*)(lds_a + 1024 * (q * S::NL + wave));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, a_vo[q], 0, 0, 0);
  } else {
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bb + kb, live ? b_bytes - kb : 0);
    lds_void* dst = (lds_void*)(lds_b + 1024 * ((q - S::IA) * S::NL + wave));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, dst, 16, b_vo[q - S::IA], 0, 0, 0);
  }
}

// The persistent kernel's copies of slice s (row-major A and B): the same
// copies as issue_slice, with the last slice's A tail mask given as one
// bit per copy (bit i clear: copy i of A reads past K and is dropped), so
// that each offset is a select, not a choice between two offset arrays.
// (Its own function: the host pass leaves a device function template's
// specialisation unusable for a second kernel once one kernel has
// instantiated it.)
template <class S>
__device__ __forceinline__ void issue_slice_ps(const unsigned char* Ab, const unsigned char* Bb,
                                               int64_t a_bytes, int64_t b_bytes, int s, bool live,
                                               bool last, const unsigned* a_vo, unsigned a_tail,
                                               const unsigned* b_vo, unsigned char* lds_a,
                                               unsigned char* lds_b, int wave, int lda, int ldb) {
  const int64_t ka = S::ES * (int64_t)s * S::BK;
  const int64_t kb = (int64_t)s * S::BK * ldb * S::ES;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ab + ka, live ? a_bytes - ka : 0);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bb + kb, live ? b_bytes - kb : 0);
#pragma unroll
  for (int q = 0; q < S::IA; ++q) {
    lds_void* dst = (lds_void*)(lds_a + 1024 * (q * S::NL + wave));
    const unsigned off = (last && !((a_tail >> q) & 1u)) ? OOB : a_vo[q];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, off, 0, 0, 0);
  }
#pragma unroll
  for (int q = 0; q < S::IB; ++q) {
    lds_void* dst = (lds_void*)(lds_b + 1024 * (q * S::NL + wave));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, dst, 16, b_vo[q], 0, 0, 0);
  }
}

template <class S>
__global__ void __launch_bounds__(S::NT)
hgemm_tr_kernel(Params p, TileMap map, int64_t a_bytes, int64_t b_bytes) {
  constexpr int NS = S::NS, KS = S::KS, MB = S::MB, NB = S::NB, IA = S::IA, IB = S::IB;
  constexpr int BM = S::BM, BN = S::BN, WM = S::WM, WN = S::WN, BK = S::BK;

  // Stage arrays: A stages la0..la{NS-1}, B stages lb0..lb{NS-1} (unused
  // ones are dropped by the compiler).
  __shared__ __attribute__((aligned(1024))) unsigned char la0[S::A_STAGE], lb0[S::B_STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char la1[S::A_STAGE], lb1[S::B_STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char la2[S::A_STAGE], lb2[S::B_STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char la3[S::A_STAGE], lb3[S::B_STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char la4[S::A_STAGE], lb4[S::B_STAGE];
  auto A_of = [&](auto I) -> unsigned char* {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) return la0;
    else if constexpr (i == 1) return la1;
    else if constexpr (i == 2) return la2;
    else if constexpr (i == 3) return la3;
    else return la4;
  };
  auto B_of = [&](auto I) -> unsigned char* {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) return lb0;
    else if constexpr (i == 1) return lb1;
    else if constexpr (i == 2) return lb2;
    else if constexpr (i == 3) return lb3;
    else return lb4;
  };
  // Array k of the epilogue list [A stages..., B stages...].
  auto E_of = [&](auto I) -> unsigned char* {
    constexpr int i = decltype(I)::value;
    if constexpr (i < NS) return A_of(IC<i>{});
    else return B_of(IC<(i - NS) % NS>{});
  };

  trace_stamp(p, 0);
  int tm, tn;
  tile_of_block(blockIdx.x, map, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lda = (int)p.lda, ldb = (int)p.ldb;
  // Split-K: workgroup row sk takes K chunk [sk*kc, min(K, (sk+1)*kc)); the
  // operand bases and buffer ranges move to the chunk, C to its partial.
  const int sk = blockIdx.y;
  const int kc = p.splits > 1 ? p.kc : p.K;
  const int M = p.M, N = p.N, K = min(kc, p.K - sk * kc);
  const int64_t ashift = S::AT ? S::ES * (int64_t)sk * kc * lda : S::ES * (int64_t)sk * kc;
  const unsigned char* Ab = static_cast<const unsigned char*>(p.A) + ashift;
  const int64_t bshift = S::BT ? S::ES * (int64_t)sk * kc : S::ES * (int64_t)sk * kc * ldb;
  const unsigned char* Bb = static_cast<const unsigned char*>(p.B) + bshift;
  a_bytes -= ashift;
  b_bytes -= bshift;

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave / S::WAVES_N) * WM, wn0 = (wave % S::WAVES_N) * WN;
  // This wave's index among the waves that issue copies (producer waves
  // follow the NW compute waves).
  const int lw = S::PW > 0 ? wave - S::NW : wave;
  const int T = (K + BK - 1) / BK;

  // Direct-load offsets (relative to the slice's descriptor base).
  unsigned a_vo[IA], a_vo_tail[IA], b_vo[IB], b_vo_tail[IB];
#pragma unroll
  for (int i = 0; i < IA; ++i) {
    if constexpr (S::AT) {
      const int k = S::at_dl_k(i, lw, l), c = S::at_dl_c(i, lw, l);
      const bool ok = (m0 + S::CE * c) < M;
      a_vo[i] = ok ? (unsigned)S::ES * ((unsigned)k * (unsigned)lda + (unsigned)(m0 + S::CE * c)) : OOB;
      a_vo_tail[i] = a_vo[i];  // rows past K are past the buffer's range
    } else {
      const int r = S::a_dl_row(i, lw, l), q = S::a_dl_q(i, lw, l);
      const bool ok = (m0 + r) < M;
      a_vo[i] = ok ? (unsigned)S::ES * ((unsigned)(m0 + r) * (unsigned)lda + (unsigned)S::CE * q) : OOB;
      a_vo_tail[i] = ((T - 1) * BK + S::CE * q < K) ? a_vo[i] : OOB;
    }
  }
#pragma unroll
  for (int i = 0; i < IB; ++i) {
    if constexpr (S::BT) {
      // Bt row n0 + r (output column), k chunk q: row-major A's placement.
      const int r = S::bt_dl_row(i, lw, l), q = S::bt_dl_q(i, lw, l);
      const bool ok = (n0 + r) < N;
      b_vo[i] = ok ? (unsigned)S::ES * ((unsigned)(n0 + r) * (unsigned)ldb + (unsigned)S::CE * q) : OOB;
      b_vo_tail[i] = ((T - 1) * BK + S::CE * q < K) ? b_vo[i] : OOB;
    } else {
      const int k = S::b_dl_k(i, lw, l), c = S::b_dl_c(i, lw, l);
      const bool ok = (n0 + S::CE * c) < N;
      b_vo[i] = ok ? (unsigned)S::ES * ((unsigned)k * (unsigned)ldb + (unsigned)(n0 + S::CE * c)) : OOB;
      b_vo_tail[i] = b_vo[i];  // rows past K are past the buffer's range
    }
  }
  // Fragment byte offsets: k step j of A and block nb of B; other blocks
  // and k steps are immediate offsets.
  constexpr int FR = S::FR;
  int a_fb[S::AT ? MB : KS * FR], b_fb[S::BT ? KS * FR : NB];
  if constexpr (S::AT) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) a_fb[mb] = S::at_frag(wm0, mb, 0, 0, l);
  } else {
#pragma unroll
    for (int j = 0; j < KS; ++j)
#pragma unroll
      for (int q = 0; q < FR; ++q) a_fb[j * FR + q] = S::a_frag(wm0, 0, j, l, q);
  }
  if constexpr (S::BT) {
#pragma unroll
    for (int j = 0; j < KS; ++j)
#pragma unroll
      for (int q = 0; q < FR; ++q) b_fb[j * FR + q] = S::bt_frag(wn0, 0, j, l, q);
  } else {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) b_fb[nb] = S::b_frag(wn0, nb, 0, 0, l);
  }

  // Slice s's copies into one stage (all of them; with producer waves, the
  // producer's share).
  auto produce = [&](int s, unsigned char* la, unsigned char* lb) __attribute__((always_inline)) {
    issue_slice<S>(Ab, Bb, a_bytes, b_bytes, s, s < T, s == T - 1 ? a_vo_tail : a_vo,
                   s == T - 1 ? b_vo_tail : b_vo, la, lb, lw, lda, ldb);
  };
  if constexpr (S::PW > 0) {
    if (wave >= S::NW) {
      // Producer wave: the compute waves' schedule of copies and barriers
      // (one barrier before the loop, one per slice, then the epilogue's),
      // without their LDS reads and MFMAs.  All NS stages are filled first;
      // the barrier that ends slice t's reads (once slice t+1 has landed)
      // frees stage t % NS for slice t + NS.
      if (T > 0) {
        static_for([&](auto I) { produce(decltype(I)::value, A_of(I), B_of(I)); },
                   std::make_integer_sequence<int, NS>{});
        loop_barrier<(NS - 1) * S::LPS>();  // slice 0 landed
        int t = 0;
        for (; t + NS <= T; t += NS)
          static_for([&](auto I) {
            loop_barrier<(NS - 2) * S::LPS>();  // slice t+I+1 landed, stage I read
            produce(t + decltype(I)::value + NS, A_of(I), B_of(I));
          }, std::make_integer_sequence<int, NS>{});
        static_for([&](auto I) {
          if (t + decltype(I)::value < T) {
            loop_barrier<(NS - 2) * S::LPS>();
            produce(t + decltype(I)::value + NS, A_of(I), B_of(I));
          }
        }, std::make_integer_sequence<int, NS>{});
        // Every copy (the zero-filled ones past T included) lands before
        // the epilogue reuses the stages.
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      }
      if constexpr (!S::PARTIAL) __syncthreads();
      if constexpr (!S::PARTIAL && !S::EPI) __syncthreads();
      return;
    }
  }
  // The compute waves' own copies (none when producer waves issue them).
  auto issue = [&](int s, unsigned char* la, unsigned char* lb) __attribute__((always_inline)) {
    if constexpr (S::PW == 0) produce(s, la, lb);
  };
  // Part j (of KS) of slice s's copies.
  auto issue_part = [&](int s, auto J, unsigned char* la, unsigned char* lb) __attribute__((always_inline)) {
    constexpr int j = decltype(J)::value;
    if constexpr (S::PW == 0)
      issue_slice<S, j * S::PP, (j + 1) * S::PP>(Ab, Bb, a_bytes, b_bytes, s, s < T,
                                                 s == T - 1 ? a_vo_tail : a_vo,
                                                 s == T - 1 ? b_vo_tail : b_vo, la, lb, wave, lda, ldb);
  };

  // An operand: 8 16-bit or 32 8-bit values per lane.
  typedef std::conditional_t<S::F8, i32x8_t, f16x8> Frag;
  Frag fa[2][MB], fb[S::FBS][NB];
  // Two 16-byte chunks of one lane's FP8 operand (positions differ by the
  // row's XOR).
  auto two_chunks = [](const unsigned char* p0, const unsigned char* p1) __attribute__((always_inline)) {
    const u32x4 x0 = *(const lds_u32x4*)p0, x1 = *(const lds_u32x4*)p1;
    return __builtin_bit_cast(i32x8_t, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // The transpose reads of one operand from a row-major (k rows) tile at
  // byte b, rows `row` bytes apart.
  auto tr_operand = [](const unsigned char* b, int row) __attribute__((always_inline)) {
    if constexpr (S::F8) {
      const i32x2 r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)b);
      const i32x2 r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(b + 8 * row));
      const i32x2 r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(b + 16 * row));
      const i32x2 r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(b + 24 * row));
      const i32x4 lo = __builtin_shufflevector(r0, r1, 0, 1, 2, 3);
      const i32x4 hi = __builtin_shufflevector(r2, r3, 0, 1, 2, 3);
      return Frag(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)b);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b + 4 * row));
      return Frag(__builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)));
    }
  };
  // The operands of k step j: A's row block mb, B's column block nb.
  auto load_a = [&](int buf, const unsigned char* la, int j, int mb) __attribute__((always_inline)) {
    if constexpr (S::AT)
      fa[buf][mb] = tr_operand(la + a_fb[mb] + S::KW * j * S::A_ROW, S::A_ROW);
    else if constexpr (S::F8)
      fa[buf][mb] = two_chunks(la + a_fb[2 * j] + mb * S::MI * S::A_ROW, la + a_fb[2 * j + 1] + mb * S::MI * S::A_ROW);
    else
      fa[buf][mb] = *(const lds_f16x8*)(la + a_fb[j] + mb * S::MI * S::A_ROW);
  };
  auto load_b = [&](int buf, const unsigned char* lb, int j, int nb) __attribute__((always_inline)) {
    if constexpr (!S::BT)
      fb[S::fb_set(buf, nb)][nb] = tr_operand(lb + b_fb[nb] + S::KW * j * S::B_ROW, S::B_ROW);
    else if constexpr (S::F8)
      fb[S::fb_set(buf, nb)][nb] = two_chunks(lb + b_fb[2 * j] + nb * S::MI * S::B_ROW, lb + b_fb[2 * j + 1] + nb * S::MI * S::B_ROW);
    else
      fb[S::fb_set(buf, nb)][nb] = *(const lds_f16x8*)(lb + b_fb[j] + nb * S::MI * S::B_ROW);
  };
  auto load_frags = [&](int buf, const unsigned char* la, const unsigned char* lb, int j)
      __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) load_a(buf, la, j, mb);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) load_b(buf, lb, j, nb);
  };

  // acc[nb][mb]: block of C^T (rows n, columns m).
  typedef std::conditional_t<S::MI == 32, f32x16, f32x4> Acc;
  Acc acc[NB][MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < S::AR; ++r) acc[nb][mb][r] = 0.f;
  // 16 x 16 blocks: the zeros are in the accumulator registers before the
  // hazard guard, and the first MFMA comes after it (see mfma16_asm).
  if constexpr (S::MI == 16) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) asm volatile("" : "+a"(acc[nb][mb]));
    mfma_guard();
  }
  auto mma = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        if constexpr (S::F8)
          acc[nb][mb] = mfma_f8<S::TY - 2>(fb[buf][nb], fa[buf][mb], acc[nb][mb]);
        else
          acc[nb][mb] = mfma16<S::BF>(fb[buf][nb], fa[buf][mb], acc[nb][mb]);
      }
  };

  // 16 x 16 blocks: k step `cur` as a fixed sequence, MFMA i on block
  // (i / MB, i % MB), with scheduling barriers between them that place the
  // next step's operand reads (rd(f) after MFMA rd_after(f): A's MB
  // operands first, which the next step's first MFMAs need, then B's) and
  // the copies (cp(q) after MFMA cp_after(q)).  The builtin's scheduling
  // groups cannot place inline assembly.
  auto mma16 = [&](int cur, auto&& rd, auto&& cp, auto&& bar) __attribute__((always_inline)) {
    if constexpr (S::MI == 16) {
      static_assert(S::schedule_ok(), "16 x 16 step schedule");
      static_for([&](auto I) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        mfma16_asm<S::TY>(acc[i / MB][i % MB], fb[S::fb_set(cur, i / MB)][i / MB], fa[cur][i % MB]);
        if constexpr (i == S::BAR_AFTER) {
          __builtin_amdgcn_sched_barrier(0);
          bar();
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (S::rd_at(i) >= 0) rd(IC<S::rd_at(i)>{});
        if constexpr (S::cp_at(i) >= 0) cp(IC<S::cp_at(i)>{});
        __builtin_amdgcn_sched_barrier(0);
      }, std::make_integer_sequence<int, MB * NB>{});
    }
  };
  // Operand f of k step j (f < MB: A's block f; else B's block f - MB).
  auto rd_op = [&](int buf, const unsigned char* la, const unsigned char* lb, int j, auto F)
      __attribute__((always_inline)) {
    constexpr int f = decltype(F)::value;
    if constexpr (f < MB) load_a(buf, la, j, f);
    else load_b(buf, lb, j, f - MB);
  };

  // (The lambdas are forced inline: an out-of-line call would move the
  // accumulators to scratch memory.)
  constexpr int NMMA = MB * NB;     // MFMAs per k step
  constexpr int NRD = MB * (S::AT ? S::TRN : FR) + (S::BT ? FR : S::TRN) * NB;  // LDS reads per k step
  // Slice t from stage c: k steps 0..KS-2 with the next step's fragments
  // in flight; wait for slice t+1; barrier; issue slice t+NS into the freed
  // stage c; last k step (registers only) under the first fragment reads of
  // stage c+1.
  auto slice = [&](int t, auto C_) __attribute__((always_inline)) {
    constexpr int c = decltype(C_)::value, n = (c + 1) % NS, f = (c + NS - 1) % NS;
    unsigned char* ca = A_of(IC<c>{});
    unsigned char* cb = B_of(IC<c>{});
    if constexpr (S::MI == 16) {
      static_assert(!S::SPREAD && S::PW == 0, "16 x 16 blocks: two stages, no producer waves");
      // Steps 0..KS-2 with the next step's operands read from stage c.
      static_for([&](auto J) __attribute__((always_inline)) {
        constexpr int j = decltype(J)::value;
        mma16(S::frag_set(c, j),
              [&](auto F) __attribute__((always_inline)) { rd_op(S::frag_set(c, j + 1), ca, cb, j + 1, F); },
              [](auto) {}, [] {});
      }, std::make_integer_sequence<int, KS - 1>{});
      // Slice t+1 landed and stage c read by every wave: before the last
      // step, or inside it (BAR_AFTER).
      auto bar = [&]() __attribute__((always_inline)) { loop_barrier<(NS - 2) * S::LPS>(); };
      if constexpr (S::BAR_AFTER < 0) {
        bar();
        __builtin_amdgcn_sched_barrier(0);
      }
      // Last step: slice t+NS's copies into stage c and the next stage's
      // first operands (after cp_after / rd_after).
      mma16(S::frag_set(c, KS - 1),
            [&](auto F) __attribute__((always_inline)) {
              rd_op(S::frag_set(c + 1, 0), A_of(IC<n>{}), B_of(IC<n>{}), 0, F);
            },
            [&](auto Q) __attribute__((always_inline)) {
              constexpr int q = decltype(Q)::value;
              if constexpr (q < S::LPS)
                issue_copy<S>(Ab, Bb, a_bytes, b_bytes, t + NS, t + NS < T,
                              t + NS == T - 1 ? a_vo_tail : a_vo, t + NS == T - 1 ? b_vo_tail : b_vo,
                              ca, cb, lw, lda, ldb, q);
            },
            [&]() __attribute__((always_inline)) {
              if constexpr (S::BAR_AFTER >= 0) bar();
            });
      return;
    }
    static_for([&](auto J) __attribute__((always_inline)) {
      constexpr int j = decltype(J)::value;
      load_frags(S::frag_set(c, j + 1), ca, cb, j + 1);
      // Spread: parts 1..KS-1 of slice t+NS-1 into stage f (free since the
      // last barrier), the PP copies evenly among the k step's MFMAs.
      if constexpr (S::SPREAD) issue_part(t + NS - 1, IC<j + 1>{}, A_of(IC<f>{}), B_of(IC<f>{}));
      mma(S::frag_set(c, j));
#pragma unroll
      for (int i = 0; i < NMMA; ++i) {
        SGB(SG_MFMA, 1);
        if (i < NRD) SGB(SG_DS_RD, 1);
        if constexpr (S::SPREAD)
          if (S::copy_slot(i)) SGB(SG_VMEM_RD, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }, std::make_integer_sequence<int, KS - 1>{});
    // Slice t+1 has landed; the copies of the later slices may still fly.
    loop_barrier<(NS - 2) * S::LPS>();
    __builtin_amdgcn_sched_barrier(0);
    // Stage c is free now: slice t+NS goes there (burst: all of it; spread:
    // part 0, the rest during the next slice's k steps).
    if constexpr (S::SPREAD) issue_part(t + NS, IC<0>{}, ca, cb);
    else issue(t + NS, ca, cb);
    load_frags(S::frag_set(c + 1, 0), A_of(IC<n>{}), B_of(IC<n>{}), 0);
    mma(S::frag_set(c, KS - 1));
#pragma unroll
    for (int i = 0; i < NMMA; ++i) {
      SGB(SG_MFMA, 1);
      if (i < NRD) SGB(SG_DS_RD, 1);
      if constexpr (S::SPREAD) {
        if (S::copy_slot(i)) SGB(SG_VMEM_RD, 1);
      } else {
        if (S::PW == 0 && i < S::LPS) SGB(SG_VMEM_RD, 1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  if (T > 0) {
    if constexpr (S::SPREAD) {
      // Slices 0..NS-2 whole, part 0 of slice NS-1 (the first slice's k
      // steps issue the rest); then wait for slice 0.
      static_for([&](auto I) { issue(decltype(I)::value, A_of(I), B_of(I)); },
                 std::make_integer_sequence<int, NS - 1>{});
      issue_part(NS - 1, IC<0>{}, A_of(IC<NS - 1>{}), B_of(IC<NS - 1>{}));
      loop_barrier<(NS - 2) * S::LPS + S::PP>();  // slice 0 landed
    } else {
      static_for([&](auto I) { issue(decltype(I)::value, A_of(I), B_of(I)); },
                 std::make_integer_sequence<int, NS>{});
      loop_barrier<(NS - 1) * S::LPS>();  // slice 0 landed
    }
    trace_stamp(p, 1);
    load_frags(0, la0, lb0, 0);
    int t = 0;
    for (; t + NS <= T; t += NS)
      static_for([&](auto I) { slice(t + decltype(I)::value, I); }, std::make_integer_sequence<int, NS>{});
    // (16 x 16 blocks: guards wherever control flow joins after MFMAs.)
    if constexpr (S::MI == 16) mfma_guard();
    static_for([&](auto I) {
      if (t + decltype(I)::value < T) {
        slice(t + decltype(I)::value, I);
        if constexpr (S::MI == 16) mfma_guard();
      }
    }, std::make_integer_sequence<int, NS>{});
    // The copies of the slices past T (out of range: they write zeros)
    // must land before the epilogue reuses the LDS.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    if constexpr (S::MI == 16) mfma_guard();
  }
  if constexpr (S::MI == 16) mfma_guard();  // the last MFMA's results
  trace_stamp(p, 2);
  if constexpr (S::PARTIAL) {
    // Split-K partial: FP32 C (the workspace) written straight from the
    // accumulators, no FP16 rounding, no LDS round trip.
    // acc[nb][mb] register 4rq+e of lane l is C[m][n], m = wm0 +
    // acc_row(mb, l), n = wn0 + acc_col(nb, rq, l) + e: one 16-byte store
    // each.
    float* __restrict__ Cf = static_cast<float*>(p.C) + sk * p.c_stride;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int rq = 0; rq < S::RQ; ++rq) {
          const int row = m0 + wm0 + S::acc_row(mb, l);
          const int col = n0 + wn0 + S::acc_col(nb, rq, l);
          if (row < M && col < N) {
            f32x4 v = {acc[nb][mb][4 * rq], acc[nb][mb][4 * rq + 1], acc[nb][mb][4 * rq + 2],
                       acc[nb][mb][4 * rq + 3]};
            *reinterpret_cast<f32x4*>(Cf + (int64_t)row * p.ldc + col) = v;
          }
        }
    trace_stamp(p, 3);
    return;
  }
  __syncthreads();

  // Epilogue.  acc[nb][mb] register 4rq + e of lane l holds C[m][n] with
  // m = wm0 + acc_row(mb, l) and n = wn0 + acc_col(nb, rq, l) + e: four
  // consecutive columns per register group.  Stage the wave's FP16 tile in
  // its P arrays (row-major, 8-byte slots swizzled by row), then write it
  // out in 16-byte row chunks.
  unsigned char* ep[S::P];
  static_for([&](auto I) {
    constexpr int i = decltype(I)::value;
    unsigned char* sel = E_of(IC<i>{});
    static_for([&](auto W) {
      if (wave == decltype(W)::value) sel = E_of(IC<decltype(W)::value * S::P + i>{});
    }, std::make_integer_sequence<int, S::NW>{});
    ep[i] = sel;
  }, std::make_integer_sequence<int, S::P>{});
  if constexpr (S::EPI) {
    // Fused epilogue: the FP32 accumulators go through the same LDS region
    // in two passes of WM/2 rows (FP32 takes twice the FP16 bytes), 16-byte
    // chunks XOR-swizzled by row (conflict-free writes and reads); each
    // lane then reads four adjacent FP32 values of one row, applies alpha,
    // beta with the old FP16 C (read only when beta != 0), bias and the
    // activation, rounds once and stores 8 bytes: 32 lanes per 256-byte row
    // segment, coalesced like the plain epilogue.
    typedef half_t<S::BF> H;
    typedef H h16x4 __attribute__((ext_vector_type(4)));
    typedef int v2i __attribute__((ext_vector_type(2)));
    // C's element: 2 bytes (FP16 / BF16), or 1 (INT8 codes).
    constexpr unsigned CB = S::Q8 ? 1u : 2u;
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(static_cast<const unsigned char*>(p.C), ((int64_t)(M - 1) * p.ldc + N) * CB);
    constexpr int R32 = S::R32, CPR32 = S::CPR32, RPI32 = S::RPI32;
    const int q = l % CPR32, col = n0 + wn0 + 4 * q;  // this lane's four columns
    f32x4 bias = {};
    if (p.epi.bias && col < N) bias = *reinterpret_cast<const f32x4*>(p.epi.bias + col);
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mbl = 0; mbl < MB / 2; ++mbl)
#pragma unroll
          for (int rq = 0; rq < S::RQ; ++rq) {
            const int mb = pass * (MB / 2) + mbl;
            const int m = S::acc_row(mbl, l), q = S::acc_col(nb, rq, l) / 4;
            f32x4 v = {acc[nb][mb][4 * rq], acc[nb][mb][4 * rq + 1], acc[nb][mb][4 * rq + 2],
                       acc[nb][mb][4 * rq + 3]};
            *reinterpret_cast<f32x4*>(ep[m / R32] + S::epi32_byte(m % R32, q)) = v;
          }
      // Old-C loads batched (eight rows, then one wait), bias loaded once,
      // and no branches: the old C is read and the result written through
      // a buffer descriptor over C, out-of-range elements getting an offset
      // past its range (loads return 0, stores are dropped).  Per-element
      // branches would split the code into blocks across which the
      // compiler waits for every memory operation, stores included.
      constexpr int ITS = (WM / 2) / RPI32, BATCH = 8;
      static_assert(ITS % BATCH == 0, "epilogue batches");
#pragma unroll
      for (int b0 = 0; b0 < ITS; b0 += BATCH) {
        unsigned off[BATCH];
        v2i c_old[BATCH];
        f32x4 v[BATCH];
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
          const int row = m0 + wm0 + pass * (WM / 2) + (b0 + i) * RPI32 + l / CPR32;
          off[i] = ((row < M) & (col < N)) ? CB * ((unsigned)row * (unsigned)p.ldc + (unsigned)col) : OOB;
          c_old[i] = v2i{0, 0};
        }
        if (!S::Q8 && p.epi.beta != 0.f) {
#pragma unroll
          for (int i = 0; i < BATCH; ++i) c_old[i] = __builtin_amdgcn_raw_buffer_load_b64(rc, off[i], 0, 0);
        }
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
          const int r = (b0 + i) * RPI32 + l / CPR32;
          v[i] = *reinterpret_cast<const f32x4*>(ep[((b0 + i) * RPI32) / R32] + S::epi32_byte(r % R32, q));
        }
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
          if constexpr (S::Q8) {
            const int w = pack_i8x4(quantize_i8(epi_value(p.epi, v[i][0], 0.f, bias[0])),
                                    quantize_i8(epi_value(p.epi, v[i][1], 0.f, bias[1])),
                                    quantize_i8(epi_value(p.epi, v[i][2], 0.f, bias[2])),
                                    quantize_i8(epi_value(p.epi, v[i][3], 0.f, bias[3])));
            __builtin_amdgcn_raw_buffer_store_b32(w, rc, off[i], 0, 0);
          } else {
            const h16x4 c = __builtin_bit_cast(h16x4, c_old[i]);
            h16x4 h;
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = (H)epi_value(p.epi, v[i][e], (float)c[e], bias[e]);
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2i, h), rc, off[i], 0, 0);
          }
        }
      }
    }
    trace_stamp(p, 3);
    return;
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int rq = 0; rq < S::RQ; ++rq) {
        uint2 v;
        v.x = round16<S::BF>(acc[nb][mb][4 * rq + 0]) |
              ((unsigned)round16<S::BF>(acc[nb][mb][4 * rq + 1]) << 16);
        v.y = round16<S::BF>(acc[nb][mb][4 * rq + 2]) |
              ((unsigned)round16<S::BF>(acc[nb][mb][4 * rq + 3]) << 16);
        const int row = S::acc_row(mb, l), slot = S::acc_col(nb, rq, l) / 4;
        *reinterpret_cast<uint2*>(ep[row / S::RPA] + S::epi_byte(row % S::RPA, slot)) = v;
      }
  __syncthreads();
  constexpr int CPR = S::EPI_CPR, RPI = S::EPI_RPI;
  unsigned short* __restrict__ C = static_cast<unsigned short*>(p.C);
  const int rl = l / CPR, c = l % CPR;
  const int col = n0 + wn0 + 8 * c;
#pragma unroll
  for (int pass = 0; pass < WM / RPI; ++pass) {
    const int row = pass * RPI + rl;
    const unsigned char* e = ep[(pass * RPI) / S::RPA];
    const int lr = row % S::RPA;
    const u32x4 v = S::epi_chunk(e, lr, c);
    const int grow = m0 + wm0 + row;
    if (grow < M && col < N) {
      // Streaming store: C is written once and not read back here (about
      // 1 % faster than a plain store for the end-of-kernel write burst).
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(C + (int64_t)grow * p.ldc + col));
    }
  }
  trace_stamp(p, 3);
}

// Persistent form of the plain kernel (two stages, row-major A and B, no
// producer waves).  gridDim.x workgroups (at most one per CU) walk the
// tiles v = blockIdx.x, blockIdx.x + gridDim.x, ... in the tile map's order
// (gridDim.x is a multiple of the XCD count, so every tile a workgroup
// takes belongs to its own XCD's run of the map), and the slice pipeline
// runs on across tiles: the two stages that a tile's last two slices free
// receive the next tile's first two slices, so those copies are in flight
// while this tile's C is written.  The C tile therefore leaves the
// accumulators through a wave-private LDS region, not the stages: 32 rows
// of the wave tile per round, written as 8-byte slots XOR-swizzled by row
// (conflict-free), read back as 16-byte row chunks and stored with
// WN/8 lanes per row segment (the coalesced write-back of "sgemm - beyond
// cuBLAS", section 5), branch-free through a buffer descriptor over C.
// The number of K slices must be even, so that every tile starts on stage
// 0 (the launch runs the one-tile-per-workgroup kernel otherwise).
//
// The first wait of each later tile lets the copies of its second slice
// and the previous tile's C stores (issued after the first slice's copies)
// stay in flight: vector memory operations of a wave complete in issue
// order, loads and stores alike (gfx9 has one counter for both, and the
// compiler's own waits for this target assume the same order).
template <class S>
__global__ void __launch_bounds__(S::NT)
hgemm_tr_persistent_kernel(Params p, TileMap map, int64_t a_bytes, int64_t b_bytes) {
  static_assert(S::NS == 2 && S::PW == 0 && !S::BT && !S::AT && !S::PARTIAL && !S::EPI,
                "persistent form: plain two-stage kernel");
  constexpr int KS = S::KS, MB = S::MB, NB = S::NB, IA = S::IA, IB = S::IB;
  constexpr int BM = S::BM, BN = S::BN, WM = S::WM, WN = S::WN, BK = S::BK;
  __shared__ __attribute__((aligned(1024))) unsigned char la0[S::A_STAGE], lb0[S::B_STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char la1[S::A_STAGE], lb1[S::B_STAGE];
  // Epilogue staging, one region per wave: 32 rows of EPI_ROW bytes.
  __shared__ __attribute__((aligned(1024))) unsigned char lep[S::NW * S::PS_EPI_BYTES];

  trace_stamp(p, 0);
  const int ntiles = map.tiles_m * map.tiles_n;
  const int M = p.M, N = p.N, K = p.K;
  const int lda = (int)p.lda, ldb = (int)p.ldb;
  const unsigned char* Ab = static_cast<const unsigned char*>(p.A);
  const unsigned char* Bb = static_cast<const unsigned char*>(p.B);
  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave / S::WAVES_N) * WM, wn0 = (wave % S::WAVES_N) * WN;
  const int lw = S::PW > 0 ? wave - S::NW : wave;  // index among the copying waves
  const int T = (K + BK - 1) / BK;
  unsigned char* ep = lep + wave * S::PS_EPI_BYTES;

  // Direct-load offsets of one tile (relative to the slice's descriptor
  // base), as in the one-tile kernel.
  unsigned a_vo[IA], b_vo[IB];
  // Bit i: copy i of A stays within K in the last (partial) slice.
  unsigned a_tail = 0;
  // The lane index as a value the compiler cannot see through: the per-lane
  // terms of the offsets below are then recomputed where they are used
  // instead of being hoisted out of the tile loop and kept live across it,
  // which spills registers to scratch memory (whose loads share the wait
  // counter with the stage copies).
  auto opaque_lane = [&]() __attribute__((always_inline)) {
    int v = l;
    asm volatile("" : "+v"(v));
    return v;
  };
  // Everything per lane that the K loop needs is (re)computed at the top of
  // each tile (and the copy offsets again for the next tile two slices
  // before the end), so that none of it is live across the epilogue, which
  // needs the registers.
  auto set_tile = [&](int m0, int n0) __attribute__((always_inline)) {
    const int l = opaque_lane();
    a_tail = 0;
#pragma unroll
    for (int i = 0; i < IA; ++i)
      a_tail |= ((T - 1) * BK + S::CE * S::a_dl_q(i, lw, l) < K) ? 1u << i : 0u;
#pragma unroll
    for (int i = 0; i < IA; ++i) {
      const int r = S::a_dl_row(i, lw, l), q = S::a_dl_q(i, lw, l);
      a_vo[i] = (m0 + r) < M ? (unsigned)S::ES * ((unsigned)(m0 + r) * (unsigned)lda + (unsigned)S::CE * q) : OOB;
    }
    // (B rows past K are past the buffer's range.)
#pragma unroll
    for (int i = 0; i < IB; ++i) {
      const int k = S::b_dl_k(i, lw, l), c = S::b_dl_c(i, lw, l);
      b_vo[i] = (n0 + S::CE * c) < N ? (unsigned)S::ES * ((unsigned)k * (unsigned)ldb + (unsigned)(n0 + S::CE * c))
                                     : OOB;
    }
  };
  // Fragment byte offsets (tile-independent; recomputed per tile).
  constexpr int FR = S::FR;
  int a_fb[KS * FR], b_fb[NB];
  auto set_frags = [&]() __attribute__((always_inline)) {
    const int l = opaque_lane();
#pragma unroll
    for (int j = 0; j < KS; ++j)
#pragma unroll
      for (int q = 0; q < FR; ++q) a_fb[j * FR + q] = S::a_frag(wm0, 0, j, l, q);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) b_fb[nb] = S::b_frag(wn0, nb, 0, 0, l);
  };

  // Slice s of the current tile's offsets (s >= T: zeros, no memory read).
#define PS_PRODUCE(s_, la_, lb_)                                                              \
  issue_slice_ps<S>(Ab, Bb, a_bytes, b_bytes, (s_), (s_) < T, (s_) == T - 1, a_vo, a_tail, b_vo, \
                    (la_), (lb_), lw, lda, ldb)

  typedef std::conditional_t<S::F8, i32x8_t, f16x8> Frag;
  Frag fa[2][MB], fb[S::FBS][NB];
  auto two_chunks = [](const unsigned char* p0, const unsigned char* p1) __attribute__((always_inline)) {
    const u32x4 x0 = *(const lds_u32x4*)p0, x1 = *(const lds_u32x4*)p1;
    return __builtin_bit_cast(i32x8_t, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto tr_operand = [](const unsigned char* b, int row) __attribute__((always_inline)) {
    if constexpr (S::F8) {
      const i32x2 r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)b);
      const i32x2 r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(b + 8 * row));
      const i32x2 r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(b + 16 * row));
      const i32x2 r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(b + 24 * row));
      const i32x4 lo = __builtin_shufflevector(r0, r1, 0, 1, 2, 3);
      const i32x4 hi = __builtin_shufflevector(r2, r3, 0, 1, 2, 3);
      return Frag(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)b);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b + 4 * row));
      return Frag(__builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)));
    }
  };
  auto load_a = [&](int buf, const unsigned char* la, int j, int mb) __attribute__((always_inline)) {
    if constexpr (S::F8)
      fa[buf][mb] = two_chunks(la + a_fb[2 * j] + mb * S::MI * S::A_ROW, la + a_fb[2 * j + 1] + mb * S::MI * S::A_ROW);
    else
      fa[buf][mb] = *(const lds_f16x8*)(la + a_fb[j] + mb * S::MI * S::A_ROW);
  };
  auto load_b = [&](int buf, const unsigned char* lb, int j, int nb) __attribute__((always_inline)) {
    fb[S::fb_set(buf, nb)][nb] = tr_operand(lb + b_fb[nb] + S::KW * j * S::B_ROW, S::B_ROW);
  };
  auto load_frags = [&](int buf, const unsigned char* la, const unsigned char* lb, int j)
      __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) load_a(buf, la, j, mb);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) load_b(buf, lb, j, nb);
  };
  typedef std::conditional_t<S::MI == 32, f32x16, f32x4> Acc;
  Acc acc[NB][MB];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < S::AR; ++r) acc[nb][mb][r] = 0.f;
  };
  auto mma = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        if constexpr (S::F8)
          acc[nb][mb] = mfma_f8<S::TY - 2>(fb[buf][nb], fa[buf][mb], acc[nb][mb]);
        else
          acc[nb][mb] = mfma16<S::BF>(fb[buf][nb], fa[buf][mb], acc[nb][mb]);
      }
  };
  constexpr int NMMA = MB * NB;
  constexpr int NRD = MB * FR + S::TRN * NB;
  // 16 x 16 blocks: the one-tile kernel's fixed MFMA sequence (mma16 there).
  auto mma16 = [&](int cur, auto&& rd, auto&& cp, auto&& bar) __attribute__((always_inline)) {
    if constexpr (S::MI == 16) {
      static_assert(S::schedule_ok(), "16 x 16 step schedule");
      static_for([&](auto I) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        mfma16_asm<S::TY>(acc[i / MB][i % MB], fb[S::fb_set(cur, i / MB)][i / MB], fa[cur][i % MB]);
        if constexpr (i == S::BAR_AFTER) {
          __builtin_amdgcn_sched_barrier(0);
          bar();
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (S::rd_at(i) >= 0) rd(IC<S::rd_at(i)>{});
        if constexpr (S::cp_at(i) >= 0) cp(IC<S::cp_at(i)>{});
        __builtin_amdgcn_sched_barrier(0);
      }, std::make_integer_sequence<int, MB * NB>{});
    }
  };
  auto rd_op = [&](int buf, const unsigned char* la, const unsigned char* lb, int j, auto F)
      __attribute__((always_inline)) {
    constexpr int f = decltype(F)::value;
    if constexpr (f < MB) load_a(buf, la, j, f);
    else load_b(buf, lb, j, f - MB);
  };
  // The accumulators' zeros in place before the guard that precedes the
  // next MFMA (16 x 16 blocks; see mfma16_asm).
  auto pin_zero = [&]() __attribute__((always_inline)) {
    if constexpr (S::MI == 16) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) asm volatile("" : "+a"(acc[nb][mb]));
      mfma_guard();
    }
  };

  int v = blockIdx.x;
  int tm, tn;
  tile_of_block(v, map, tm, tn);
  int m0 = tm * BM, n0 = tn * BN;
  int vn = v + gridDim.x;
  bool has_next = vn < ntiles;
  int m0n = 0, n0n = 0;
  if (has_next) {
    tile_of_block(vn, map, tm, tn);
    m0n = tm * BM;
    n0n = tn * BN;
  }
  set_tile(m0, n0);

  // Slice t of the current tile from stage c (as the one-tile kernel's
  // two-stage slice), except that the copy issued into the freed stage is
  // slice t+2 of this tile, or, past its last slice, slice t+2-T of the
  // next tile (the offsets switch to the next tile at its first copy).
  auto slice = [&](int t, auto C_) __attribute__((always_inline)) {
    constexpr int c = decltype(C_)::value, n = (c + 1) % 2;
    unsigned char* ca = c == 0 ? la0 : la1;
    unsigned char* cb = c == 0 ? lb0 : lb1;
    // Every copy of this tile is issued by now (slice T-1 went out in
    // slice T-3): the offsets can move to the next tile.
    if (has_next && t == T - 2) set_tile(m0n, n0n);
    if constexpr (S::MI == 16) {
      static_for([&](auto J) __attribute__((always_inline)) {
        constexpr int j = decltype(J)::value;
        mma16(S::frag_set(c, j),
              [&](auto F) __attribute__((always_inline)) { rd_op(S::frag_set(c, j + 1), ca, cb, j + 1, F); },
              [](auto) {}, [] {});
      }, std::make_integer_sequence<int, KS - 1>{});
      // Slice t+1 landed (and any earlier stores done): before the last
      // step, or inside it (BAR_AFTER).
      auto bar = [&]() __attribute__((always_inline)) { loop_barrier<0>(); };
      if constexpr (S::BAR_AFTER < 0) {
        bar();
        __builtin_amdgcn_sched_barrier(0);
      }
      const int s = has_next && t + 2 >= T ? t + 2 - T : t + 2;
      mma16(S::frag_set(c, KS - 1),
            [&](auto F) __attribute__((always_inline)) {
              rd_op(S::frag_set(c + 1, 0), n == 0 ? la0 : la1, n == 0 ? lb0 : lb1, 0, F);
            },
            [&](auto Q) __attribute__((always_inline)) {
              constexpr int q = decltype(Q)::value;
              if constexpr (q < S::LPS)
                issue_copy_ps<S>(Ab, Bb, a_bytes, b_bytes, s, s < T, s == T - 1, a_vo, a_tail, b_vo, ca, cb,
                                 lw, lda, ldb, q);
            },
            [&]() __attribute__((always_inline)) {
              if constexpr (S::BAR_AFTER >= 0) bar();
            });
      return;
    }
    static_for([&](auto J) __attribute__((always_inline)) {
      constexpr int j = decltype(J)::value;
      load_frags(S::frag_set(c, j + 1), ca, cb, j + 1);
      mma(S::frag_set(c, j));
#pragma unroll
      for (int i = 0; i < NMMA; ++i) {
        SGB(SG_MFMA, 1);
        if (i < NRD) SGB(SG_DS_RD, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }, std::make_integer_sequence<int, KS - 1>{});
    loop_barrier<0>();  // slice t+1 landed (and any earlier stores done)
    __builtin_amdgcn_sched_barrier(0);
    {
      const int s = has_next && t + 2 >= T ? t + 2 - T : t + 2;
      PS_PRODUCE(s, ca, cb);
    }
    load_frags(S::frag_set(c + 1, 0), n == 0 ? la0 : la1, n == 0 ? lb0 : lb1, 0);
    mma(S::frag_set(c, KS - 1));
#pragma unroll
    for (int i = 0; i < NMMA; ++i) {
      SGB(SG_MFMA, 1);
      if (i < NRD) SGB(SG_DS_RD, 1);
      if (i < S::LPS) SGB(SG_VMEM_RD, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  typedef int v4i __attribute__((ext_vector_type(4)));
  const __amdgpu_buffer_rsrc_t rc =
      make_rsrc(static_cast<const unsigned char*>(p.C), ((int64_t)(M - 1) * p.ldc + N) * 2);
  constexpr int CPR = S::EPI_CPR, RPI = S::EPI_RPI;
  // Rounds of 32 rows (row blocks per round); store instructions of one
  // tile's epilogue per wave.
  constexpr int BPR = 32 / S::MI, ROUNDS = MB / BPR;
  constexpr int PS_STORES = ROUNDS * (32 / RPI);
  static_assert(S::LPS + PS_STORES <= 63, "vmcnt field");

  zero_acc();
  pin_zero();
  if (T > 0) {
    PS_PRODUCE(0, la0, lb0);
    PS_PRODUCE(1, la1, lb1);
  }
  bool first = true;
  for (;;) {
    set_tile(m0, n0);
    set_frags();
    if (T > 0) {
      // Slice 0 of this tile landed: with slice 1's copies still in flight,
      // and for later tiles also the previous tile's C stores (see above).
      if (first) {
        loop_barrier<S::LPS>();
        trace_stamp(p, 1);
      } else {
        loop_barrier<S::LPS + PS_STORES>();
      }
      load_frags(0, la0, lb0, 0);
      for (int t = 0; t < T; t += 2) {
        slice(t, IC<0>{});
        slice(t + 1, IC<1>{});
      }
      if constexpr (S::MI == 16) mfma_guard();  // the tile's last MFMA results
    }
    if constexpr (S::MI == 16) mfma_guard();
    first = false;
    // Epilogue: round rd stages rows wm0 + 32rd .. +31 of the wave tile
    // (BPR row blocks).
    const int l = opaque_lane();
#pragma unroll
    for (int rd = 0; rd < ROUNDS; ++rd) {
      // One round at a time (the scheduler would otherwise hoist every
      // round's accumulator reads and run out of registers).
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mbl = 0; mbl < BPR; ++mbl)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int rq = 0; rq < S::RQ; ++rq) {
            const int mb = rd * BPR + mbl;
            uint2 w;
            w.x = round16<S::BF>(acc[nb][mb][4 * rq + 0]) | ((unsigned)round16<S::BF>(acc[nb][mb][4 * rq + 1]) << 16);
            w.y = round16<S::BF>(acc[nb][mb][4 * rq + 2]) | ((unsigned)round16<S::BF>(acc[nb][mb][4 * rq + 3]) << 16);
            *reinterpret_cast<uint2*>(ep + S::epi_byte(S::acc_row(mbl, l), S::acc_col(nb, rq, l) / 4)) = w;
          }
      // All the round's row chunks are read back first, then stored: one
      // wait for the LDS reads instead of one per store.
      const int col = n0 + wn0 + 8 * (l % CPR);
      constexpr int PASSES = 32 / RPI;
      v4i val[PASSES];
#pragma unroll
      for (int pass = 0; pass < PASSES; ++pass) {
        const int r = pass * RPI + l / CPR;
        val[pass] = __builtin_bit_cast(v4i, S::epi_chunk(ep, r, l % CPR));
      }
#pragma unroll
      for (int pass = 0; pass < PASSES; ++pass) {
        const int row = m0 + wm0 + 32 * rd + pass * RPI + l / CPR;
        const unsigned off = ((row < M) & (col < N)) ? 2u * ((unsigned)row * (unsigned)p.ldc + (unsigned)col) : OOB;
        __builtin_amdgcn_raw_buffer_store_b128(val[pass], rc, off, 0, 0);
      }
    }
    if (!has_next) break;
    v = vn;
    m0 = m0n;
    n0 = n0n;
    vn = v + gridDim.x;
    has_next = vn < ntiles;
    if (has_next) {
      tile_of_block(vn, map, tm, tn);
      m0n = tm * BM;
      n0n = tn * BN;
    }
    zero_acc();
    pin_zero();
  }
  trace_stamp(p, 2);
  // The zero-filling copies past the last tile's last slice must land
  // before the workgroup ends and its LDS is handed to another.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  trace_stamp(p, 3);
#undef PS_PRODUCE
}

// With S::PARTIAL this is the split-K partial launch (FP32 partials).
template <class S>
hipError_t launch(const Params& p, const TileMap& map, bool vec, hipStream_t stream) {
  const int64_t lim = 0x7fffffff;
  // Every offset (rows past M, N and K included) must fit the 31-bit range.
  constexpr int ES = S::ES;
  const bool b_far = S::BT ? (int64_t)(p.N + S::BN) * p.ldb * ES > lim
                           : (int64_t)(S::BK + 2) * p.ldb * ES > lim ||
                                 ((int64_t)(p.K > 0 ? p.K - 1 : 0) * p.ldb + p.N) * ES > lim;
  const bool a_far = S::AT ? (int64_t)(S::BK + 2) * p.lda * ES > lim ||
                                 ((int64_t)(p.K > 0 ? p.K - 1 : 0) * p.lda + p.M) * ES > lim
                           : (int64_t)(p.M + S::BM) * p.lda * ES > lim || (int64_t)p.M * p.lda * ES > lim;
  if (!vec || a_far || b_far || (S::EPI && (int64_t)p.M * p.ldc * 2 > lim)) {
    // The general kernel has no split-K form (the caller runs unsplit) and
    // no INT8-output or transposed-A form (the caller reports the operands
    // unsupported); it takes FP8 operands through p.f8.
    if (p.splits > 1 || S::Q8 || S::AT) return hipErrorNotSupported;
    return hgemm_launch_shape(S::BM, S::BN, S::WM, S::WN, p, map, vec, stream);
  }
  const int64_t a_bytes = p.K <= 0 ? 0
                          : S::AT ? ((int64_t)(p.K - 1) * p.lda + p.M) * ES
                                  : ((int64_t)(p.M - 1) * p.lda + p.K) * ES;
  const int64_t b_bytes = p.K <= 0 ? 0
                          : S::BT ? ((int64_t)(p.N - 1) * p.ldb + p.K) * ES
                                  : ((int64_t)(p.K - 1) * p.ldb + p.N) * ES;
  const dim3 grid(map.tiles_m * map.tiles_n, p.splits), block(S::NT);
  hipLaunchKernelGGL(hgemm_tr_kernel<S>, grid, block, 0, stream, p, map, a_bytes, b_bytes);
  return hipGetLastError();
}

// The persistent form's launch: min(tiles, 256) workgroups (one per CU of
// MI355X) when the K slices are even in number and C's offsets fit the
// buffer store's 32 bits; the one-tile kernel otherwise (which also takes
// the operands off the vector layout to the general kernel).
template <class S>
hipError_t launch_persistent(const Params& p, const TileMap& map, bool vec, hipStream_t stream) {
  static_assert(S::LDS_BYTES + S::NW * S::PS_EPI_BYTES <= 160 * 1024, "LDS");
  const int T = (p.K + S::BK - 1) / S::BK;
  const int64_t lim = 0x7fffffff;
  constexpr int ES = S::ES;
  const bool far = (int64_t)(S::BK + 2) * p.ldb * ES > lim ||
                   ((int64_t)(p.K > 0 ? p.K - 1 : 0) * p.ldb + p.N) * ES > lim ||
                   (int64_t)(p.M + S::BM) * p.lda * ES > lim || (int64_t)p.M * p.lda * ES > lim ||
                   ((int64_t)p.M * p.ldc + S::BN) * 2 > lim;
  if (!vec || far || T == 0 || T % 2 != 0 || p.splits > 1) return launch<S>(p, map, vec, stream);
  const int64_t a_bytes = ((int64_t)(p.M - 1) * p.lda + p.K) * ES;
  const int64_t b_bytes = ((int64_t)(p.K - 1) * p.ldb + p.N) * ES;
  const int tiles = map.tiles_m * map.tiles_n;
  const dim3 grid(tiles < 256 ? tiles : 256), block(S::NT);
  hipLaunchKernelGGL(hgemm_tr_persistent_kernel<S>, grid, block, 0, stream, p, map, a_bytes, b_bytes);
  return hipGetLastError();
}

// Host replay of the transposed-B form's B side: direct-load placement of
// Bt rows (A's maps) and the fragment reads, checked for coverage, bounds,
// the element each lane must see and bank conflicts (added to *rconf).
// Returns 0 when valid, else a code from 20.
template <class S>
int layout_check_bt(int banks, int64_t* rconf) {
  static_assert(S::BT, "transposed-B shape");
  static int n_of[S::B_STAGE], k_of[S::B_STAGE];
  for (int i = 0; i < S::B_STAGE; ++i) n_of[i] = -1;
  for (int i = 0; i < S::IB; ++i)
    for (int w = 0; w < S::NL; ++w)
      for (int l = 0; l < 64; ++l) {
        const int off = 1024 * (i * S::NL + w) + 16 * l;
        const int r = S::bt_dl_row(i, w, l), q = S::bt_dl_q(i, w, l);
        if (r >= S::BN || q >= S::B_CPR || S::bt_byte(r, q) != off) return 20;
        for (int e = 0; e < S::CE; ++e) {
          if (n_of[off + S::ES * e] != -1) return 21;
          n_of[off + S::ES * e] = r;
          k_of[off + S::ES * e] = S::CE * q + e;
        }
      }
  for (int i = 0; i < S::B_STAGE; i += S::ES)
    if (n_of[i] < 0) return 22;
  int addr[64];
  for (int w = 0; w < S::NW; ++w) {
    const int wn0 = (w % S::WAVES_N) * S::WN;
    for (int j = 0; j < S::KS; ++j)
      for (int nb = 0; nb < S::NB; ++nb)
        for (int part = 0; part < S::FR; ++part) {
          for (int l = 0; l < 64; ++l) {
            addr[l] = S::bt_frag(wn0, nb, j, l, part);
            if (addr[l] < 0 || addr[l] + 16 > S::B_STAGE) return 23;
            if (addr[l] != S::bt_frag(wn0, 0, j, l, part) + nb * S::MI * S::B_ROW) return 24;
            // A_op lane l, element e of this chunk:
            // B[k = KW j + KL(l/MI) + CE part + e][n = wn0 + MI nb + l%MI].
            for (int e = 0; e < S::CE; ++e)
              if (n_of[addr[l] + S::ES * e] != wn0 + S::MI * nb + l % S::MI ||
                  k_of[addr[l] + S::ES * e] != S::KW * j + S::KL * (l / S::MI) + S::CE * part + e)
                return 25;
          }
          *rconf += lds_conflicts(addr, 16, banks);
        }
  }
  return 0;
}

// Host replay of the transposed-A form's A side: A^T rows placed by the
// direct loads (B's maps with BM values per row) and the transpose reads of
// each row block, checked for coverage, bounds, the element each lane must
// see and bank conflicts (added to *rconf).  Returns 0 when valid, else a
// code from 40.
template <class S>
int layout_check_at(int banks, int64_t* rconf) {
  static_assert(S::AT, "transposed-A shape");
  static int m_of[S::A_STAGE], k_of[S::A_STAGE];
  for (int i = 0; i < S::A_STAGE; ++i) m_of[i] = -1;
  for (int i = 0; i < S::IA; ++i)
    for (int w = 0; w < S::NL; ++w)
      for (int l = 0; l < 64; ++l) {
        const int off = 1024 * (i * S::NL + w) + 16 * l;
        const int k = S::at_dl_k(i, w, l), c = S::at_dl_c(i, w, l);
        if (k >= S::BK || c >= S::A_CPR || S::at_byte(k, S::CE * c) != off) return 40;
        for (int e = 0; e < S::CE; ++e) {
          if (m_of[off + S::ES * e] != -1) return 41;
          m_of[off + S::ES * e] = S::CE * c + e;
          k_of[off + S::ES * e] = k;
        }
      }
  for (int i = 0; i < S::A_STAGE; i += S::ES)
    if (m_of[i] < 0) return 42;
  int addr[64];
  constexpr int LPR = 16 / S::RR;
  for (int w = 0; w < S::NW; ++w) {
    const int wm0 = (w / S::WAVES_N) * S::WM;
    for (int j = 0; j < S::KS; ++j)
      for (int mb = 0; mb < S::MB; ++mb)
        for (int jr = 0; jr < S::TRN; ++jr) {
          for (int l = 0; l < 64; ++l) {
            addr[l] = S::at_frag(wm0, mb, j, jr, l);
            if (addr[l] != S::at_frag(wm0, mb, 0, 0, l) + (S::KW * j + S::RR * jr) * S::A_ROW) return 43;
          }
          for (int l = 0; l < 64; ++l)
            for (int t = 0; t < S::RR; ++t) {
              const int g = l / 16, jj = l % 16;
              const int src = addr[16 * g + LPR * t + jj / S::RR] + S::ES * (jj % S::RR);
              if (src < 0 || src >= S::A_STAGE) return 44;
              // B_op lane l, element RR*jr + t:
              // A[m = wm0 + MI mb + l%MI][k = KW j + KL(l/MI) + RR jr + t].
              if (k_of[src] != S::KW * j + S::KL * (l / S::MI) + S::RR * jr + t ||
                  m_of[src] != wm0 + S::MI * mb + l % S::MI)
                return 45;
            }
          *rconf += lds_conflicts(addr, 8, banks);
        }
  }
  return 0;
}

// Host replay: direct-load placement, fragment reads (including the lane
// exchange of the transpose read), and epilogue staging, all checked for
// bounds, for matching the element each lane must see, and for bank
// conflicts; then the transposed-B form's B side.  Returns 0 when valid.
template <class S>
int layout_check(int banks, int64_t out[2]) {
  constexpr int BM = S::BM, WM = S::WM, WN = S::WN, BK = S::BK;
  int64_t wconf = 0, rconf = 0;
  // Inverse maps of the two tile layouts: LDS byte -> (row, k) / (k, n).
  static int a_row_of[S::A_STAGE], a_k_of[S::A_STAGE], b_k_of[S::B_STAGE], b_n_of[S::B_STAGE];
  for (int i = 0; i < S::A_STAGE; ++i) a_row_of[i] = -1;
  for (int i = 0; i < S::B_STAGE; ++i) b_k_of[i] = -1;
  for (int i = 0; i < S::IA; ++i)
    for (int w = 0; w < S::NL; ++w)
      for (int l = 0; l < 64; ++l) {
        const int off = 1024 * (i * S::NL + w) + 16 * l;
        const int r = S::a_dl_row(i, w, l), q = S::a_dl_q(i, w, l);
        if (r >= BM || q >= S::A_CPR || S::a_byte(r, q) != off) return 1;
        for (int e = 0; e < S::CE; ++e) {
          if (a_row_of[off + S::ES * e] != -1) return 2;
          a_row_of[off + S::ES * e] = r;
          a_k_of[off + S::ES * e] = S::CE * q + e;
        }
      }
  for (int i = 0; i < S::IB; ++i)
    for (int w = 0; w < S::NL; ++w)
      for (int l = 0; l < 64; ++l) {
        const int off = 1024 * (i * S::NL + w) + 16 * l;
        const int k = S::b_dl_k(i, w, l), c = S::b_dl_c(i, w, l);
        if (k >= BK || c >= S::B_CPR || S::b_byte(k, S::CE * c) != off) return 3;
        for (int e = 0; e < S::CE; ++e) {
          if (b_k_of[off + S::ES * e] != -1) return 4;
          b_k_of[off + S::ES * e] = k;
          b_n_of[off + S::ES * e] = S::CE * c + e;
        }
      }
  for (int i = 0; i < S::A_STAGE; i += S::ES)
    if (a_row_of[i] < 0) return 5;
  for (int i = 0; i < S::B_STAGE; i += S::ES)
    if (b_k_of[i] < 0) return 6;
  int addr[64];
  for (int w = 0; w < S::NW; ++w) {
    const int wm0 = (w / S::WAVES_N) * WM, wn0 = (w % S::WAVES_N) * WN;
    for (int j = 0; j < S::KS; ++j) {
      for (int mb = 0; mb < S::MB; ++mb)
        for (int part = 0; part < S::FR; ++part) {
          for (int l = 0; l < 64; ++l) {
            addr[l] = S::a_frag(wm0, mb, j, l, part);
            if (addr[l] < 0 || addr[l] + 16 > S::A_STAGE) return 15;
            // B_op lane l, element e of this chunk:
            // A[m = wm0 + MI mb + l%MI][k = KW j + KL(l/MI) + CE part + e].
            for (int e = 0; e < S::CE; ++e) {
              const int b = addr[l] + S::ES * e;
              if (a_row_of[b] != wm0 + S::MI * mb + l % S::MI ||
                  a_k_of[b] != S::KW * j + S::KL * (l / S::MI) + S::CE * part + e)
                return 7;
            }
            if (addr[l] != S::a_frag(wm0, 0, j, l, part) + mb * S::MI * S::A_ROW) return 8;
          }
          rconf += lds_conflicts(addr, 16, banks);
        }
      for (int nb = 0; nb < S::NB; ++nb)
        for (int jr = 0; jr < S::TRN; ++jr) {
          for (int l = 0; l < 64; ++l) {
            addr[l] = S::b_frag(wn0, nb, j, jr, l);
            if (addr[l] != S::b_frag(wn0, nb, 0, 0, l) + (S::KW * j + S::RR * jr) * S::B_ROW) return 9;
          }
          // Transpose read of RR elements per lane: output lane jj of a
          // 16-lane group receives element jj%RR of the piece addressed by
          // lane LPR*t + jj/RR of the group (LPR = 16/RR lanes per row).
          constexpr int LPR = 16 / S::RR;
          for (int l = 0; l < 64; ++l)
            for (int t = 0; t < S::RR; ++t) {
              const int g = l / 16, jj = l % 16;
              const int src = addr[16 * g + LPR * t + jj / S::RR] + S::ES * (jj % S::RR);
              if (src < 0 || src >= S::B_STAGE) return 14;
              // A_op lane l, element RR*jr + t:
              // B[k = KW j + KL(l/MI) + RR jr + t][n = wn0 + MI nb + l%MI].
              if (b_k_of[src] != S::KW * j + S::KL * (l / S::MI) + S::RR * jr + t ||
                  b_n_of[src] != wn0 + S::MI * nb + l % S::MI)
                return 10;
            }
          rconf += lds_conflicts(addr, 8, banks);
        }
    }
  }
  // Epilogue staging: writes and reads cover the wave's rows exactly once
  // per array and agree on the element.
  constexpr int EW = S::RPA * S::EPI_ROW;
  static int ep_row[S::P][EW], ep_col[S::P][EW];
  for (int a = 0; a < S::P; ++a)
    for (int i = 0; i < EW; ++i) ep_row[a][i] = -1;
  // Accumulator register 4rq + e of lane l in block (nb, mb) holds row
  // MI mb + l%MI, column MI nb + 8rq + 4(l/MI) + e of the wave tile (the
  // matrix instruction's output layout, operands swapped).
  constexpr int MI = S::MI;
  for (int nb = 0; nb < S::NB; ++nb)
    for (int mb = 0; mb < S::MB; ++mb)
      for (int rq = 0; rq < S::RQ; ++rq) {
        for (int l = 0; l < 64; ++l) {
          const int row = MI * mb + l % MI, slot = (MI / 4) * nb + 2 * rq + l / MI;
          const int a = row / S::RPA;
          addr[l] = S::epi_byte(row % S::RPA, slot);
          if (a >= S::P || addr[l] < 0 || addr[l] + 8 > EW) return 13;
          for (int e = 0; e < 4; ++e) {
            if (ep_row[a][addr[l] + 2 * e] != -1) return 11;
            ep_row[a][addr[l] + 2 * e] = row;
            ep_col[a][addr[l] + 2 * e] = MI * nb + 8 * rq + 4 * (l / MI) + e;
          }
        }
        wconf += lds_conflicts(addr, 8, banks);
      }
  constexpr int CPR = S::EPI_CPR, RPI = S::EPI_RPI;
  for (int pass = 0; pass < WM / RPI; ++pass)
    for (int half = 0; half < (MI == 16 ? 1 : 2); ++half) {
      // 16 x 16 blocks: one 16-byte read of both slots.
      const int width = MI == 16 ? 16 : 8;
      for (int l = 0; l < 64; ++l) {
        const int row = pass * RPI + l / CPR, c = l % CPR;
        const int a = (pass * RPI) / S::RPA;
        addr[l] = S::epi_byte(row % S::RPA, 2 * c + half);
        for (int e = 0; e < width / 2; ++e)
          if (ep_row[a][addr[l] + 2 * e] != row || ep_col[a][addr[l] + 2 * e] != 8 * c + 4 * half + e)
            return 12;
      }
      rconf += lds_conflicts(addr, width, banks);
    }
  // Fused-epilogue staging (one pass; both passes use the same map): FP32
  // writes cover the wave's region once, reads return the element written.
  {
    constexpr int R32 = S::R32, CPR32 = S::CPR32, RPI32 = S::RPI32, E32 = R32 * S::ROW32;
    static int e_row[S::P][E32 / 4], e_col[S::P][E32 / 4];
    for (int a = 0; a < S::P; ++a)
      for (int i = 0; i < E32 / 4; ++i) e_row[a][i] = -1;
    for (int nb = 0; nb < S::NB; ++nb)
      for (int mbl = 0; mbl < S::MB / 2; ++mbl)
        for (int rq = 0; rq < S::RQ; ++rq) {
          for (int l = 0; l < 64; ++l) {
            const int m = MI * mbl + l % MI, q = (MI / 4) * nb + 2 * rq + l / MI;
            const int a = m / R32;
            addr[l] = S::epi32_byte(m % R32, q);
            if (a >= S::P || addr[l] < 0 || addr[l] + 16 > E32) return 16;
            for (int e = 0; e < 4; ++e) {
              if (e_row[a][addr[l] / 4 + e] != -1) return 17;
              e_row[a][addr[l] / 4 + e] = m;
              e_col[a][addr[l] / 4 + e] = MI * nb + 8 * rq + 4 * (l / MI) + e;
            }
          }
          wconf += lds_conflicts(addr, 16, banks);
        }
    for (int it = 0; it < (WM / 2) / RPI32; ++it) {
      for (int l = 0; l < 64; ++l) {
        const int r = it * RPI32 + l / CPR32, q = l % CPR32;
        const int a = (it * RPI32) / R32;
        if (r / R32 != a) return 18;
        addr[l] = S::epi32_byte(r % R32, q);
        for (int e = 0; e < 4; ++e)
          if (e_row[a][addr[l] / 4 + e] != r || e_col[a][addr[l] / 4 + e] != 4 * q + e) return 19;
      }
      rconf += lds_conflicts(addr, 16, banks);
    }
  }
  int rc = layout_check_bt<Shape<S::BM, S::BN, S::WM, S::WN, S::BK, S::NS, 0, true, S::TY, false, S::PW, S::MI>>(
      banks, &rconf);
  if (rc != 0) return rc;
  if constexpr (S::BM * S::ES >= 256) {
    rc = layout_check_at<Shape<S::BM, S::BN, S::WM, S::WN, S::BK, S::NS, 0, false, S::TY, true, S::PW, S::MI>>(
        banks, &rconf);
    if (rc != 0) return rc;
    // Both transposed: B's side must not depend on A's row length.
    rc = layout_check_bt<Shape<S::BM, S::BN, S::WM, S::WN, S::BK, S::NS, 0, true, S::TY, true, S::PW, S::MI>>(
        banks, &rconf);
    if (rc != 0) return rc;
  }
  out[0] = wconf;
  out[1] = rconf;
  return 0;
}

// The transposed-A launches, for tiles whose A^T rows (BM values) span the
// 256 bytes the chunk XOR needs; none otherwise.
template <int BM, int BN, int WM, int WN, int BK, int NS, int TY, bool BT, int PW, int MI>
constexpr LaunchFn at_launch() {
  if constexpr (BM * (TY >= 2 ? 1 : 2) >= 256)
    return &launch<Shape<BM, BN, WM, WN, BK, NS, 0, BT, TY, true, PW, MI>>;
  else
    return nullptr;
}

// PW producer waves (0: none); their count is the name's _p suffix.  MI:
// the matrix instruction's block (16: the name's _mi16 suffix).
#define HGEMM_TR_VARIANT_MI(TY, DT, TAG, BM, BN, WM, WN, BK, NS, PW, MI, SFX, EFF)               \
  Variant {                                                                                  \
    gemm_config_t{0, DT, GEMM_FAMILY_MFMA, BM, BN, BK, WM, WN,                               \
                  Shape<BM, BN, WM, WN, BK, NS, 0, false, TY, false, PW, MI>::NT, NS,        \
                  Shape<BM, BN, WM, WN, BK, NS, 0, false, TY, false, PW, MI>::LDS_BYTES,     \
                  GEMM_ORDER_XCD, 4, 1,                                                      \
                  "tr_" TAG "_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_s" #NS SFX},          \
        &launch<Shape<BM, BN, WM, WN, BK, NS, 0, false, TY, false, PW, MI>>,                 \
        &layout_check<Shape<BM, BN, WM, WN, BK, NS, 0, false, TY, false, PW, MI>>,           \
        &launch<Shape<BM, BN, WM, WN, BK, NS, 1, false, TY, false, PW, MI>>, EFF,            \
        &launch<Shape<BM, BN, WM, WN, BK, NS, 2, false, TY, false, PW, MI>>,                 \
        &launch<Shape<BM, BN, WM, WN, BK, NS, 0, true, TY, false, PW, MI>>,                  \
        &launch<Shape<BM, BN, WM, WN, BK, NS, 3, false, TY, false, PW, MI>>,                 \
        at_launch<BM, BN, WM, WN, BK, NS, TY, false, PW, MI>(),                              \
        at_launch<BM, BN, WM, WN, BK, NS, TY, true, PW, MI>()                                \
  }
#define HGEMM_TR_VARIANT_PW(TY, DT, TAG, BM, BN, WM, WN, BK, NS, PW, SFX, EFF) \
  HGEMM_TR_VARIANT_MI(TY, DT, TAG, BM, BN, WM, WN, BK, NS, PW, 32, SFX, EFF)
// The persistent form of a two-stage tile: the plain call only.
#define HGEMM_TR_VARIANT_PS_MI(TY, DT, TAG, BM, BN, WM, WN, BK, MI, SFX, EFF)                        \
  Variant {                                                                                      \
    gemm_config_t{0, DT, GEMM_FAMILY_MFMA, BM, BN, BK, WM, WN,                                   \
                  Shape<BM, BN, WM, WN, BK, 2, 0, false, TY, false, 0, MI>::NT, 2,               \
                  Shape<BM, BN, WM, WN, BK, 2, 0, false, TY, false, 0, MI>::LDS_BYTES +          \
                      Shape<BM, BN, WM, WN, BK, 2, 0, false, TY, false, 0, MI>::NW *             \
                          Shape<BM, BN, WM, WN, BK, 2, 0, false, TY, false, 0, MI>::PS_EPI_BYTES, \
                  GEMM_ORDER_XCD, 4, 1,                                                          \
                  "tr_" TAG "_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_s2" SFX "_ps"},           \
        &launch_persistent<Shape<BM, BN, WM, WN, BK, 2, 0, false, TY, false, 0, MI>>,            \
        &layout_check<Shape<BM, BN, WM, WN, BK, 2, 0, false, TY, false, 0, MI>>, nullptr, EFF,  \
        nullptr, nullptr, nullptr, nullptr, nullptr, true                                        \
  }
#define HGEMM_TR_VARIANT_PS(TY, DT, TAG, BM, BN, WM, WN, BK, EFF) \
  HGEMM_TR_VARIANT_PS_MI(TY, DT, TAG, BM, BN, WM, WN, BK, 32, "", EFF)
#define HGEMM_TR_VARIANT(TY, DT, TAG, BM, BN, WM, WN, BK, NS, EFF) \
  HGEMM_TR_VARIANT_PW(TY, DT, TAG, BM, BN, WM, WN, BK, NS, 0, "", EFF)

// The 16-bit LDS layouts and data path do not depend on the element type,
// so FP16 and BF16 share the tiles and the measured tile efficiencies.  The
// 16 x 16 instruction's form of the default tile (_mi16) runs 13-16 % above
// it with all CUs busy (FP16 4096^3 +15 %, BF16 +13 %).  FP8
// moves 128 k per slice in the same bytes; its B rows must span 256 bytes
// (the 2*(k%8) chunk XOR), so its tiles are 256 columns wide.
#define HGEMM_TR_TABLE(TY, DT, TAG)                                   \
  {HGEMM_TR_VARIANT(TY, DT, TAG, 256, 256, 128, 128, 64, 2, 1.00f), \
   HGEMM_TR_VARIANT(TY, DT, TAG, 256, 256, 128, 128, 32, 4, 0.99f), \
   HGEMM_TR_VARIANT(TY, DT, TAG, 256, 256, 128, 128, 32, 5, 0.99f), \
   HGEMM_TR_VARIANT(TY, DT, TAG, 256, 128, 128, 64, 64, 3, 0.90f),  \
   HGEMM_TR_VARIANT(TY, DT, TAG, 128, 256, 64, 128, 64, 3, 0.89f),  \
   HGEMM_TR_VARIANT(TY, DT, TAG, 128, 128, 64, 64, 64, 2, 0.71f),                 \
   HGEMM_TR_VARIANT_PW(TY, DT, TAG, 256, 128, 128, 64, 64, 3, 4, "_p4", 0.895f),   \
   HGEMM_TR_VARIANT_PW(TY, DT, TAG, 256, 128, 128, 64, 64, 3, 2, "_p2", 0.89f),    \
   HGEMM_TR_VARIANT_PS(TY, DT, TAG, 256, 256, 128, 128, 64, 1.00f),               \
   HGEMM_TR_VARIANT_MI(TY, DT, TAG, 256, 256, 128, 128, 64, 2, 0, 16, "_mi16", 1.14f), \
   HGEMM_TR_VARIANT_PS_MI(TY, DT, TAG, 256, 256, 128, 128, 64, 16, "_mi16", 1.14f)}

const Variant kVariants[] = HGEMM_TR_TABLE(0, GEMM_DTYPE_F16, "f16");
const Variant kVariantsBf[] = HGEMM_TR_TABLE(1, GEMM_DTYPE_BF16, "bf16");
// The two FP8 encodings share the tiles (the data path moves bytes; only
// the matrix instruction's operand format differs).
#define HGEMM_TR_F8_TABLE(TY, DT, TAG)                                              \
  {HGEMM_TR_VARIANT(TY, DT, TAG, 256, 256, 128, 128, 128, 2, 1.00f),              \
   HGEMM_TR_VARIANT(TY, DT, TAG, 256, 256, 128, 128, 64, 4, 0.85f),               \
   HGEMM_TR_VARIANT(TY, DT, TAG, 128, 256, 64, 128, 128, 3, 0.89f),               \
   HGEMM_TR_VARIANT_PW(TY, DT, TAG, 128, 256, 64, 128, 128, 3, 4, "_p4", 0.88f),  \
   HGEMM_TR_VARIANT_PS(TY, DT, TAG, 256, 256, 128, 128, 128, 1.00f),              \
   HGEMM_TR_VARIANT_MI(TY, DT, TAG, 256, 256, 128, 128, 128, 2, 0, 16, "_mi16", 1.00f), \
   HGEMM_TR_VARIANT_PS_MI(TY, DT, TAG, 256, 256, 128, 128, 128, 16, "_mi16", 1.00f)}
const Variant kVariantsF8[] = HGEMM_TR_F8_TABLE(2, GEMM_DTYPE_F8, "f8");
const Variant kVariantsE5[] = HGEMM_TR_F8_TABLE(3, GEMM_DTYPE_E5M2, "e5m2");

}  // namespace

const Variant* hgemm_tr_variants(int* count, int ty) {
  if (ty == 3) {
    *count = sizeof(kVariantsE5) / sizeof(kVariantsE5[0]);
    return kVariantsE5;
  }
  const Variant* v = ty == 2 ? kVariantsF8 : ty == 1 ? kVariantsBf : kVariants;
  *count = ty == 2 ? sizeof(kVariantsF8) / sizeof(kVariantsF8[0])
                   : ty == 1 ? sizeof(kVariantsBf) / sizeof(kVariantsBf[0])
                             : sizeof(kVariants) / sizeof(kVariants[0]);
  return v;
}

}  // namespace gemm
