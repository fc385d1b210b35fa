// Internal declarations shared by the libgemm kernels and the C-ABI layer.
//
// Everything in this header is either plain data passed to kernels or an
// integer index map marked __host__ __device__, so that the host-side checks
// (tile map bijection, LDS layout bijection and bank-conflict counts) run the
// very functions the kernels run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm.h"

namespace gemm {

// ---------------------------------------------------------------------------
// Kernel arguments.
// ---------------------------------------------------------------------------
// Fused epilogue of gemm_*_epi (on = false: plain C = A x B).
struct Epi {
  bool on = false;
  float alpha = 1.f, beta = 0.f;
  const float* bias = nullptr;
  int act = GEMM_ACT_NONE;
};

// INT8 code of a fused-epilogue value (the quantising epilogue: alpha
// carries the scale): round to nearest with ties to even (v_rndne_f32) after
// saturating to [-128, 127]; NaN gives 0.
__device__ __forceinline__ int quantize_i8(float v) {
  v = v == v ? v : 0.f;
  return (int)__builtin_rintf(__builtin_fminf(__builtin_fmaxf(v, -128.f), 127.f));
}

// Four INT8 codes packed little-endian into one 32-bit word.
__device__ __forceinline__ int pack_i8x4(int a, int b, int c, int d) {
  return (a & 0xff) | ((b & 0xff) << 8) | ((c & 0xff) << 16) | (d << 24);
}

// One output of the fused epilogue: alpha*acc (+ beta*c_old when beta != 0)
// (+ bias when there is one), then the activation; FP32 throughout.  The
// caller reads c_old and bias only when they take part (C must not be read
// when beta == 0).
__device__ __forceinline__ float epi_value(const Epi& e, float acc, float c_old, float bias) {
  float v = e.alpha * acc;
  if (e.beta != 0.f) v = __builtin_fmaf(e.beta, c_old, v);
  if (e.bias) v += bias;
  if (e.act == GEMM_ACT_RELU) v = v < 0.f ? 0.f : v;
  return v;
}

struct Params {
  const void* A;
  const void* B;
  void* C;
  int64_t lda, ldb, ldc;
  int M, N, K;
  // Split-K (kernels with a partial form only): workgroup row blockIdx.y =
  // s < splits computes K range [s*kc, min(K, (s+1)*kc)) into the FP32
  // partial C + s*c_stride.  splits = 1: the whole K into C.
  int splits = 1, kc = 0;
  int64_t c_stride = 0;
  Epi epi;
  // B given transposed: B points at Bt (N x K row-major, leading dimension
  // ldb), i.e. column-major B.  Kernels without such a form ignore it and
  // must not be launched with it.
  bool bt = false;
  // 16-bit kernels: A, B and C (and the old C read by the fused epilogue)
  // hold bfloat16 instead of binary16.  The general FP16 kernel reads it at
  // launch; the LDS-direct kernels have it (and FP8) in their template.
  bool bf16 = false;
  // FP8 A and B (0: none, 1: E4M3, 2: E5M2; C is bfloat16).  The
  // LDS-direct kernels have the format in their template; the general
  // 16-bit kernel reads this at launch and widens each FP8 element to
  // bfloat16 (exactly) while staging, so FP8 operands off the vector layout
  // run there on the bf16 matrix instruction.
  int f8 = 0;
  // Per-workgroup timestamps (gemm_trace_set): when non-null, the kernels
  // that record them write, for workgroup w = blockIdx.y * gridDim.x +
  // blockIdx.x below trace_cap, the shader-cycle counter and the 100 MHz
  // constant clock at four points (entry, first K slice landed, K loop
  // done, C issued) into trace[8w + 2 * point] and trace[8w + 2 * point + 1].
  unsigned long long* trace = nullptr;
  int trace_cap = 0;
};

// One timestamp of gemm_trace_set's record (see Params::trace): a uniform
// branch when tracing is off; when on, lane 0 of the workgroup's first wave
// stores the two counters with ordinary vector stores.
__device__ __forceinline__ void trace_stamp(const Params& p, int point) {
  if (p.trace) {
    const unsigned w = blockIdx.y * gridDim.x + blockIdx.x;
    if (w < (unsigned)p.trace_cap) {
      const unsigned long long t = __builtin_amdgcn_s_memtime();
      const unsigned long long r = __builtin_amdgcn_s_memrealtime();
      if (threadIdx.x == 0) {
        p.trace[8 * w + 2 * point] = t;
        p.trace[8 * w + 2 * point + 1] = r;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// FP8 byte -> bfloat16 bit pattern, exact (every E4M3 and E5M2 value is a
// bfloat16 value: at most 4 significant bits, exponents within bfloat16's
// range).  From the OCP 8-bit definitions: E4M3 has exponent bias 7,
// subnormals fraction * 2^-9, NaN at exponent 15 with fraction 7 and no
// infinities; E5M2 has bias 15, subnormals fraction * 2^-16, infinities and
// NaN at exponent 31.  A subnormal fraction m with leading bit p becomes
// the normal 2^(p - scale) * (1 + (m - 2^p) / 2^p).
// ---------------------------------------------------------------------------
__host__ __device__ constexpr unsigned short e4m3_to_bf16(unsigned char b) {
  const unsigned s = (b & 0x80u) << 8, e = (b >> 3) & 0xfu, m = b & 0x7u;
  if (e == 0xf && m == 0x7) return (unsigned short)(s | 0x7fc0u);
  if (e == 0) {
    if (m == 0) return (unsigned short)s;
    const unsigned p = m >= 4 ? 2 : m >= 2 ? 1 : 0;  // m * 2^-9 = 2^(p-9) * ...
    return (unsigned short)(s | ((p + 118u) << 7) | ((m << (7 - p)) & 0x7fu));
  }
  return (unsigned short)(s | ((e + 120u) << 7) | (m << 4));
}
__host__ __device__ constexpr unsigned short e5m2_to_bf16(unsigned char b) {
  const unsigned s = (b & 0x80u) << 8, e = (b >> 2) & 0x1fu, m = b & 0x3u;
  if (e == 0x1f) return (unsigned short)(s | (m ? 0x7fc0u : 0x7f80u));
  if (e == 0) {
    if (m == 0) return (unsigned short)s;
    const unsigned p = m >= 2 ? 1 : 0;  // m * 2^-16 = 2^(p-16) * ...
    return (unsigned short)(s | ((p + 111u) << 7) | ((m << (7 - p)) & 0x7fu));
  }
  return (unsigned short)(s | ((e + 112u) << 7) | (m << 5));
}

// ---------------------------------------------------------------------------
// The two 16-bit element types of the half-precision kernels: binary16
// (_Float16) and bfloat16 (__bf16, the upper half of a binary32).  Both
// enter the matrix cores as 8-element operands of v_mfma_f32_32x32x16_*
// (FP32 accumulation) and leave through one round-to-nearest-even
// conversion per output.  Operands travel as _Float16 vectors either way
// (the bits are what matter) and are reinterpreted for the bf16 form.
// ---------------------------------------------------------------------------
template <bool BF>
using half_t = std::conditional_t<BF, __bf16, _Float16>;
typedef _Float16 h16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <bool BF>
__device__ __forceinline__ f32x16_t mfma16(h16x8_t a, h16x8_t b, f32x16_t c) {
  if constexpr (BF)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(b16x8_t, a),
                                                    __builtin_bit_cast(b16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// The 16 x 16 instruction on the same operand registers (twice the k per
// instruction, a quarter of the accumulators): v_mfma_f32_16x16x32_f16 /
// _bf16, picked by the accumulator type.
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <bool BF>
__device__ __forceinline__ f32x4_t mfma16(h16x8_t a, h16x8_t b, f32x4_t c) {
  if constexpr (BF)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b16x8_t, a),
                                                    __builtin_bit_cast(b16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// FP8 operands, 32 per lane (k 64 per instruction):
// v_mfma_f32_32x32x64_f8f6f4 with both operand-format fields FMT (0: OCP
// E4M3, 1: OCP E5M2) and no block scales (the scaled builtin with zero
// scale operands selects the unscaled instruction; checked on the device:
// scale 0 and 127 both give x1).
typedef int i32x8_t __attribute__((ext_vector_type(8)));

template <int FMT>
__device__ __forceinline__ f32x16_t mfma_f8(i32x8_t a, i32x8_t b, f32x16_t c) {
  static_assert(FMT == 0 || FMT == 1, "E4M3 or E5M2");
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT, FMT, 0, 0, 0, 0);
}

// The 16 x 16 form, k 128 per instruction: v_mfma_f32_16x16x128_f8f6f4.
template <int FMT>
__device__ __forceinline__ f32x4_t mfma_f8(i32x8_t a, i32x8_t b, f32x4_t c) {
  static_assert(FMT == 0 || FMT == 1, "E4M3 or E5M2");
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FMT, FMT, 0, 0, 0, 0);
}

// float -> 16-bit pattern, rounded to nearest even (v_cvt_f16_f32 or
// v_cvt_pk_bf16_f32), and the exact widening back.
template <bool BF>
__device__ __forceinline__ unsigned short round16(float x) {
  return __builtin_bit_cast(unsigned short, static_cast<half_t<BF>>(x));
}
template <bool BF>
__device__ __forceinline__ float widen16(unsigned short h) {
  return static_cast<float>(__builtin_bit_cast(half_t<BF>, h));
}

// Workgroup -> output tile order.  See gemm_order_t in gemm.h.
struct TileMap {
  int tiles_m, tiles_n;
  int order;    // gemm_order_t
  int group_m;  // band height for GROUPED / XCD
  int xcds;     // number of XCDs the dispatcher deals workgroups over
};

// Number of XCDs on MI355X; the command processor hands consecutive
// workgroup ids of a dispatch to the XCDs in round-robin order.
constexpr int kXcds = 8;

// Tile computed by workgroup `b`.  A bijection from [0, tiles_m*tiles_n)
// onto the tile grid for every order (checked on the host for every
// variant and shape in the tests).
__host__ __device__ inline void tile_of_block(int b, const TileMap& t, int& tm, int& tn) {
  const int G = t.tiles_m * t.tiles_n;
  if (t.order == GEMM_ORDER_ROW) {
    tm = b / t.tiles_n;
    tn = b - tm * t.tiles_n;
    return;
  }
  int bb = b;
  if (t.order == GEMM_ORDER_XCD && t.xcds > 1) {
    // Workgroup b runs on XCD x = b % xcds as that XCD's (b / xcds)-th
    // workgroup.  XCD x owns q + (x < r) workgroups (q = G / xcds,
    // r = G % xcds); give it the contiguous run of linear tile ids starting
    // at x*q + min(x, r) so that its workgroups share operand panels in
    // that XCD's L2.
    const int x = b % t.xcds;
    const int q = G / t.xcds, r = G % t.xcds;
    bb = x * q + (x < r ? x : r) + b / t.xcds;
  }
  // A band never exceeds the grid, so width <= G fits an int for any group_m.
  const int gm = t.group_m < 1 ? 1 : (t.group_m > t.tiles_m ? t.tiles_m : t.group_m);
  const int width = gm * t.tiles_n;  // tiles in one band
  const int band = bb / width;
  const int first_m = band * gm;
  const int rows = (t.tiles_m - first_m) < gm ? (t.tiles_m - first_m) : gm;
  const int in = bb - band * width;
  tm = first_m + in % rows;
  tn = in / rows;
}

// ---------------------------------------------------------------------------
// LDS model used by the layout derivations (measured on gfx950): 64 banks of
// 4 bytes.  A wave's ds_read/ds_write of W bytes per lane is serviced in
// groups of 256/W consecutive lanes (16 lanes for 16-byte accesses); an
// access group is conflict-free when its lanes touch distinct banks (equal
// addresses broadcast).
// ---------------------------------------------------------------------------
constexpr int kLdsBanks = 64;

// XOR swizzle for a row-major LDS tile whose rows are `row_bytes` long and
// are read or written in 16-byte chunks.  Chunk q of row r is stored at
// chunk position q ^ swz_row(r).  With R = 256 / row_bytes rows per 256-byte
// bank line and CPR = row_bytes / 16 chunks per row, swz_row(r) =
// (r / R) % CPR makes
//   * 16 consecutive rows read at one chunk index land on 16 distinct
//     16-byte bank slots (fragment reads), and
//   * one row written chunk by chunk by consecutive lanes stays a
//     permutation of its own slots (staging writes),
// which is the wave64 / 64-bank re-derivation of the column XOR used for
// the transposed A tile in "sgemm - beyond cuBLAS" (section 4).
__host__ __device__ constexpr int swz_row(int r, int row_bytes) {
  return row_bytes >= 256 ? (r % (row_bytes / 16))
                          : ((r / (256 / row_bytes)) % (row_bytes / 16));
}

// Byte offset of 16-byte chunk q of row r in a swizzled tile.
__host__ __device__ constexpr int swz_off(int r, int q, int row_bytes) {
  return r * row_bytes + 16 * (q ^ swz_row(r, row_bytes));
}

// FP16 B tile (stored transposed, one LDS row per output column): the LDS
// row that holds tile column n.  Columns are interleaved so that, for a
// wave tile of WN columns split into NB = WN/32 MFMA blocks, block nb's lane
// i owns column NB*i + nb (the epilogue then writes NB adjacent columns per
// lane); sigma flips the row parity between neighbouring 8-column staging
// blocks so that two such blocks written by one 16-lane group use different
// halves of the 256-byte bank line.
__host__ __device__ constexpr int log2i(int v) { return v <= 1 ? 0 : 1 + log2i(v / 2); }

__host__ __device__ constexpr int bt_sigma(int i, int NB) {
  return i ^ ((i >> (3 - log2i(NB))) & 1);
}

__host__ __device__ constexpr int bt_row(int n, int WN) {
  const int NB = WN / 32;
  const int wn = n / WN, np = n % WN;
  return wn * WN + 32 * (np % NB) + bt_sigma(np / NB, NB);
}

// ---------------------------------------------------------------------------
// Variant table.
// ---------------------------------------------------------------------------
using LaunchFn = hipError_t (*)(const Params&, const TileMap&, bool vec, hipStream_t);
using LayoutFn = int (*)(int banks, int64_t out[2]);

struct Variant {
  gemm_config_t desc;  // id / order / group_m are defaults, filled at init
  LaunchFn launch;
  LayoutFn layout_check;
  // Launch of the split-K partial products (FP32 output into the
  // workspace, grid rows = p.splits), or nullptr when the kernel has none.
  LaunchFn launch_partial;
  // Throughput of one workgroup of this variant relative to the best tile
  // of its dtype, both with the GPU full (measured at 4096^3 on MI355X);
  // the shape heuristic's cost model divides tile work by it.
  float eff;
  // Launch with the fused epilogue (p.epi.on), or nullptr when the kernel
  // has no such form.
  LaunchFn launch_epi;
  // Launch with B given transposed (p.bt), or nullptr when the kernel has
  // no such form.
  LaunchFn launch_bt;
  // Launch of the INT8-quantising fused epilogue (C holds int8 codes,
  // p.epi.beta == 0), or nullptr when the kernel has no such form.
  LaunchFn launch_q8;
  // Launches with A given transposed (p.A is At, K x M row-major), B as
  // usual (launch_at) or also transposed (launch_atbt); nullptr when the
  // kernel has no such form.
  LaunchFn launch_at;
  LaunchFn launch_atbt;
  // The persistent form of a tile (workgroups walk several output tiles):
  // the cost model prices it per round against its one-tile twin.
  bool persistent = false;
};

// Per-family registration (each kernel file defines its table).
const Variant* sgemm_dl_variants(int* count);
const Variant* sgemm_mfma_variants(int* count);
const Variant* sgemm_simt_variants(int* count);
// The 16-bit families register a binary16 table and, where they have a
// bfloat16 form, a bfloat16 one (bf16 = true); the LDS-direct family also
// an FP8 E4M3 one (ty: 0 FP16, 1 BF16, 2 FP8 with BF16 output).
const Variant* hgemm_mfma_variants(int* count, bool bf16 = false);
// ty: 0 FP16, 1 BF16, 2 FP8 E4M3, 3 FP8 E5M2.
const Variant* hgemm_tr_variants(int* count, int ty = 0);

// Launch the general 16-bit kernel (any alignment, 64-bit addressing; FP16
// or, with p.bf16, BF16) with the given workgroup tile (and the given wave
// tile when it has one); used by the pipelined variants for operands they
// do not take.
hipError_t hgemm_launch_shape(int bm, int bn, int wm, int wn, const Params& p, const TileMap& map,
                              bool vec, hipStream_t stream);
// The same for FP32: the general SGEMM kernel (sgemm_mfma.hip) with the given
// workgroup tile, for operands the LDS-direct variants do not take.
hipError_t sgemm_launch_shape(int bm, int bn, int wm, int wn, const Params& p, const TileMap& map,
                              bool vec, hipStream_t stream);

// Split-K reduction: C[i][j] = sum over s < S (in order) of
// W[s*M*N + i*N + j], written as FP32 (dtype F32), or as FP16 (dtype F16)
// or BF16 (dtype BF16) rounded to nearest even.  Enqueued on `stream`.
hipError_t splitk_reduce(int dtype, const float* W, int S, int M, int N, void* C, int64_t ldc,
                         hipStream_t stream);

// Host bank-conflict accounting for one wave-wide LDS access: `addr[64]`
// byte addresses of `width` bytes each.  Returns the extra passes over the
// conflict-free minimum.
int lds_conflicts(const int* addr, int width, int banks);

}  // namespace gemm
