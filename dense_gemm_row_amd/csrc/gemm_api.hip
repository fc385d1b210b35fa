// C-ABI entry points of libgemm (declared in include/gemm.h): argument
// validation, variant selection (tuning table, then shape heuristic),
// launch on the caller's stream, and the host-only checks.
//
// The user-facing call mirrors the bindings of the GEMM articles
// ("sgemm - beyond cuBLAS", section 1 and 2 bindings: infer M, K, N from the
// operands, compute the grid, launch on the current stream) with explicit
// sizes and leading dimensions instead of tensors.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "gemm_internal.h"

namespace gemm {

int lds_conflicts(const int* addr, int width, int banks) {
  const int group = (banks * 4) / width < 64 ? (banks * 4) / width : 64;
  int extra = 0;
  for (int g0 = 0; g0 < 64; g0 += group) {
    // For each bank, the distinct word addresses touched by this group.
    int worst = 0;
    for (int bank = 0; bank < banks; ++bank) {
      int words[64 * 4];
      int n = 0;
      for (int l = g0; l < g0 + group && l < 64; ++l) {
        if (addr[l] < 0) continue;
        for (int w = 0; w < width / 4; ++w) {
          const int word = addr[l] / 4 + w;
          if (word % banks != bank) continue;
          bool seen = false;
          for (int t = 0; t < n; ++t) seen = seen || words[t] == word;
          if (!seen) words[n++] = word;
        }
      }
      if (n > worst) worst = n;
    }
    if (worst > 1) extra += worst - 1;
  }
  return extra;
}

namespace {

thread_local char g_err[512] = "";

gemm_status_t fail(gemm_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
gemm_status_t fail(gemm_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

// F32, F16, BF16, F8 (E4M3 in, BF16 out), E5M2 (E5M2 in, BF16 out)
constexpr int kDtypes = 5;

bool valid_dtype(int d) { return d >= GEMM_DTYPE_F32 && d <= GEMM_DTYPE_E5M2; }
// Either 8-bit input type.
bool is_f8(int d) { return d == GEMM_DTYPE_F8 || d == GEMM_DTYPE_E5M2; }

const char* dtype_name(int d) {
  return d == GEMM_DTYPE_F32    ? "f32"
         : d == GEMM_DTYPE_F16  ? "f16"
         : d == GEMM_DTYPE_BF16 ? "bf16"
         : d == GEMM_DTYPE_F8   ? "f8"
                                : "e5m2";
}

// Bytes of one A / B element and of one C element.
size_t in_bytes(int d) { return d == GEMM_DTYPE_F32 ? 4 : is_f8(d) ? 1 : 2; }
size_t out_bytes(int d) { return d == GEMM_DTYPE_F32 ? 4 : 2; }
// The type of C (the split-K reduction writes it).
int out_dtype(int d) { return is_f8(d) ? GEMM_DTYPE_BF16 : d; }

// One workgroup with its CU to itself, measured on MI355X with 64
// workgroups of each variant while the other CUs idle, at two K (1024 and
// 8192; FP32 512 and 4096): eff1 = the loop's rate from the slope, relative
// to the cost model's per-CU rate R; fixed_us = the intercept (launch,
// pipeline fill, epilogue).  With few CUs busy the 16- and 8-bit matrix
// instructions keep a higher clock, so eff1 exceeds the full-GPU eff of the
// large tiles; small tiles cannot hide their latency alone and fall below
// it.  E5M2 takes E4M3's figures (same tiles); variants not listed use eff
// and no fixed cost.
struct AloneRate {
  const char* name;
  float eff1, fixed_us;
};
const AloneRate kAlone[] = {
    {"dl_f32_256x256x32_w128x128_s2", 1.017f, 10.52f},
    {"dl_f32_256x256x16_w128x128_s4", 1.005f, 7.65f},
    {"dl_f32_256x128x32_w128x64_s3", 0.996f, 7.40f},
    {"dl_f32_128x256x32_w64x128_s3", 1.005f, 5.82f}, {"dl_f32_128x128x32_w64x64_s3", 0.997f, 5.18f},
    {"dl_f32_64x64x64_w32x32_s2", 0.906f, 3.74f},
    {"mfma_f32_128x128x32_w64x64", 0.759f, 4.35f}, {"mfma_f32_128x128x16_w64x64", 0.735f, 4.51f},
    {"mfma_f32_256x128x32_w128x64", 0.837f, 7.04f}, {"mfma_f32_256x256x32_w128x128", 0.893f, 8.31f},
    {"mfma_f32_128x256x32_w64x128", 0.825f, 4.98f}, {"mfma_f32_64x64x32_w32x32", 0.585f, 3.17f},
    {"mfma_f32_128x64x32_w64x32", 0.669f, 3.94f}, {"tr_f16_256x256x64_w128x128_s2", 1.556f, 8.31f},
    {"tr_f16_256x256x32_w128x128_s4", 1.716f, 8.42f},
    {"tr_f16_256x256x32_w128x128_s5", 1.771f, 8.69f},
    {"tr_f16_256x128x64_w128x64_s3", 1.721f, 5.93f},
    {"tr_f16_128x256x64_w64x128_s3", 1.691f, 6.18f}, {"tr_f16_128x128x64_w64x64_s2", 0.767f, 1.36f},
    {"tr_f16_256x128x64_w128x64_s3_p4", 1.835f, 5.86f},
    {"tr_f16_256x128x64_w128x64_s3_p2", 1.854f, 6.37f},
    {"tr_f16_256x256x64_w128x128_s2_ps", 1.556f, 8.31f},
    {"tr_f16_256x256x64_w128x128_s2_mi16", 1.859f, 8.60f},
    {"tr_f16_256x256x64_w128x128_s2_mi16_ps", 1.625f, 9.82f},
    {"mfma_f16_256x256x64_w128x128", 0.840f, 8.11f}, {"mfma_f16_256x128x64_w128x64", 0.545f, 6.93f},
    {"mfma_f16_128x256x64_w64x128", 0.547f, 2.75f}, {"mfma_f16_128x128x64_w64x64", 0.381f, 2.74f},
    {"mfma_f16_64x64x64_w32x32", 0.126f, 1.30f}, {"tr_bf16_256x256x64_w128x128_s2", 1.554f, 8.22f},
    {"tr_bf16_256x256x32_w128x128_s4", 1.746f, 8.66f},
    {"tr_bf16_256x256x32_w128x128_s5", 1.784f, 9.04f},
    {"tr_bf16_256x128x64_w128x64_s3", 1.721f, 6.07f},
    {"tr_bf16_128x256x64_w64x128_s3", 1.677f, 6.24f},
    {"tr_bf16_128x128x64_w64x64_s2", 0.770f, 1.69f},
    {"tr_bf16_256x128x64_w128x64_s3_p4", 1.841f, 5.98f},
    {"tr_bf16_256x128x64_w128x64_s3_p2", 1.870f, 6.54f},
    {"tr_bf16_256x256x64_w128x128_s2_ps", 1.554f, 8.22f},
    {"tr_bf16_256x256x64_w128x128_s2_mi16", 1.862f, 8.94f},
    {"tr_bf16_256x256x64_w128x128_s2_mi16_ps", 1.629f, 9.97f},
    {"mfma_bf16_256x256x64_w128x128", 0.849f, 7.43f},
    {"mfma_bf16_256x128x64_w128x64", 0.547f, 5.94f},
    {"mfma_bf16_128x256x64_w64x128", 0.546f, 2.76f}, {"mfma_bf16_128x128x64_w64x64", 0.381f, 2.79f},
    {"mfma_bf16_64x64x64_w32x32", 0.126f, 1.39f}, {"tr_f8_256x256x128_w128x128_s2", 1.774f, 8.60f},
    {"tr_f8_256x256x64_w128x128_s4", 1.597f, 8.70f},
    {"tr_f8_256x256x128_w128x128_s2_ps", 1.774f, 8.60f},
    {"tr_f8_256x256x128_w128x128_s2_mi16", 1.778f, 9.00f},
    {"tr_f8_256x256x128_w128x128_s2_mi16_ps", 1.663f, 9.72f},
    {"tr_f8_128x256x128_w64x128_s3", 1.687f, 6.30f},
    {"tr_f8_128x256x128_w64x128_s3_p4", 1.788f, 6.16f},
};

double model_rate(int dtype);

// Persistent tiles against their one-tile twin, per round of tiles (one
// 256 x 256 tile per CU), from same-box timings at 8192 x 8192 x 1024 and
// 4096 x 11008 x 4096 with in-kernel timestamps: saved_us, the per-tile
// fixed cost saved (launch, pipeline fill and the epilogue's exposed part
// overlap the neighbouring tiles' work), and slice_us, the extra loop time
// per K slice (the previous tile's C stores share the memory path).  Per
// round, time = twin's - saved_us + slices * slice_us: the persistent form
// wins at short K (below about 53 slices for 16-bit, 33 for 8-bit; for the
// 16 x 16 tiles, whose one-tile form already overlaps more of a tile's
// fixed cost, 17).  E5M2 takes E4M3's figures.
struct PsRate {
  const char* name;
  float saved_us, slice_us;
};
const PsRate kPs[] = {
    {"tr_f16_256x256x64_w128x128_s2_ps", 3.7f, 0.07f},
    {"tr_bf16_256x256x64_w128x128_s2_ps", 3.7f, 0.07f},
    {"tr_f16_256x256x64_w128x128_s2_mi16_ps", 1.2f, 0.07f},
    {"tr_bf16_256x256x64_w128x128_s2_mi16_ps", 1.2f, 0.07f},
    {"tr_f8_256x256x128_w128x128_s2_ps", 3.7f, 0.11f},
};

// The loop rate (relative to R) of one workgroup per CU with all 256 CUs
// busy, for a tile that fills its CU's LDS: eff with the fixed cost taken
// out of the time eff gives for one round at K = 4096.
double full_loop_rate(int dtype, const Variant& v, const AloneRate& a) {
  const double eff = v.eff > 0.f ? v.eff : 0.1;
  const double work = 2.0 * v.desc.bm * v.desc.bn * 4096.0;
  const double inv = 1.0 / eff - a.fixed_us * 1e-6 * model_rate(dtype) / work;
  return inv > 0.0 ? 1.0 / inv : eff;
}

struct Table {
  std::vector<Variant> v[kDtypes];  // per dtype
  std::vector<AloneRate> alone[kDtypes];  // per variant: kAlone's figures, else {eff, 0}
  std::vector<PsRate> ps[kDtypes];        // per variant: kPs's figures, else {0, 0}
  // Loop rate with all 256 CUs busy over eff1, per dtype, from the default
  // tile (at most 1): the matrix units' clock falls as more CUs run them.
  double derate[kDtypes];
  Table() {
    int n = 0;
    const Variant* p = sgemm_dl_variants(&n);
    v[0].insert(v[0].end(), p, p + n);
    p = sgemm_mfma_variants(&n);
    v[0].insert(v[0].end(), p, p + n);
    p = sgemm_simt_variants(&n);
    v[0].insert(v[0].end(), p, p + n);
    p = hgemm_tr_variants(&n);
    v[1].insert(v[1].end(), p, p + n);
    p = hgemm_mfma_variants(&n);
    v[1].insert(v[1].end(), p, p + n);
    p = hgemm_tr_variants(&n, 1);
    v[2].insert(v[2].end(), p, p + n);
    p = hgemm_mfma_variants(&n, true);
    v[2].insert(v[2].end(), p, p + n);
    p = hgemm_tr_variants(&n, 2);
    v[3].insert(v[3].end(), p, p + n);
    p = hgemm_tr_variants(&n, 3);
    v[4].insert(v[4].end(), p, p + n);
    for (int d = 0; d < kDtypes; ++d) {
      derate[d] = 1.0;
      for (size_t i = 0; i < v[d].size(); ++i) {
        v[d][i].desc.id = (int32_t)i;
        std::string name = v[d][i].desc.name;
        if (name.rfind("tr_e5m2_", 0) == 0) name = "tr_f8_" + name.substr(8);
        AloneRate r{v[d][i].desc.name, v[d][i].eff, 0.f};
        for (const AloneRate& a : kAlone)
          if (name == a.name) r = AloneRate{v[d][i].desc.name, a.eff1, a.fixed_us};
        alone[d].push_back(r);
        PsRate q{v[d][i].desc.name, 0.f, 0.f};
        for (const PsRate& a : kPs)
          if (name == a.name) q = PsRate{v[d][i].desc.name, a.saved_us, a.slice_us};
        ps[d].push_back(q);
      }
      if (!v[d].empty() && alone[d][0].eff1 > 0.f)
        derate[d] = std::min(1.0, full_loop_rate(d, v[d][0], alone[d][0]) / alone[d][0].eff1);
    }
  }
};

const Table& table() {
  static Table t;
  return t;
}

// The cost model's per-CU rate R for a dtype (FP32 matrix, 16-bit, 8-bit).
double model_rate(int dtype) {
  return dtype == GEMM_DTYPE_F32 ? 0.59e12 : is_f8(dtype) ? 9.4e12 : 4.7e12;
}

struct TuneEntry {
  int dtype;
  int64_t M, N, K;
  int id, order, group_m, splits;
};
std::vector<TuneEntry> g_tuning;
std::mutex g_tuning_mu;

int find_by_name(int dtype, const char* name) {
  const auto& v = table().v[dtype];
  for (size_t i = 0; i < v.size(); ++i)
    if (strcmp(v[i].desc.name, name) == 0) return (int)i;
  return -1;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Split-K chunking: Kc = roundup(ceil(K / splits), align), S = ceil(K / Kc).
// align is a multiple of every K slice of the dtype's variants (BK <= 64
// for 32- and 16-bit elements, <= 128 for 8-bit ones), so every chunk but
// the last is a whole number of slices: a slice never reaches into the next
// chunk's rows of B, whose values could otherwise meet A's zero padding
// (0 * Inf = NaN).  Chunk bases stay 16-byte aligned.
int64_t chunk_align(int dtype) { return is_f8(dtype) ? 128 : 64; }
void split_shape(int dtype, int64_t K, int64_t splits, int64_t& S, int64_t& Kc) {
  if (splits < 1) splits = 1;
  const int64_t align = chunk_align(dtype);
  Kc = cdiv(cdiv(K, splits), align) * align;
  if (Kc < 1) Kc = align;
  S = K > 0 ? cdiv(K, Kc) : 1;
}

// Workspace bytes of S FP32 partial planes of M x N, or -1 when the product
// does not fit an int64.
int64_t partial_bytes(int64_t S, int64_t M, int64_t N) {
  const __int128 b = (__int128)S * M * N * 4;
  return b > (__int128)INT64_MAX ? -1 : (int64_t)b;
}

// Shape heuristic: a cost model over the matrix-core variants (a tuning
// table entry overrides it for its exact shape).  Times in seconds:
//   a launch of at most one workgroup per CU (WGs <= 256, unsplit or a
//   split's partials):
//           fixed + 2*bm*bn*Kc / (r * R), fixed and r = the workgroup's
//           measured intercept and loop rate alone (kAlone), r lowered
//           linearly from 64 to 256 busy CUs to its loop rate with all
//           CUs busy;
//   GEMM otherwise:
//           ceil(WGs / 256) * 2*bm*bn*Kc / (eff * R): the busiest CU's
//           tiles at the CU's rate, which its w concurrent workgroups
//           share (w as LDS allows, at most 2),
//           R = per-CU rate of the best tile with the GPU full (measured
//           on MI355X at 4096^3), eff = the variant's relative whole-GPU
//           rate when full;
//   split:  the partials' launch as above (several rounds: each with the
//           variant's fixed cost) + (2*S*M*N*4 + M*N*es) bytes / 4 TB/s +
//           a launch, for the partials written, read back and the result
//           written.
// Ties go to the earlier table entry.
struct Choice {
  int id = -1;
  int64_t splits = 1;
  double t = 1e30;
};

double gemm_seconds(int dtype, const Variant& v, int64_t M, int64_t N, int64_t Kc, int64_t S) {
  const gemm_config_t& d = v.desc;
  const double rate = model_rate(dtype);
  int64_t per_cu = (160 * 1024) / (d.lds_bytes > 0 ? d.lds_bytes : 1);
  per_cu = per_cu < 1 ? 1 : per_cu > 2 ? 2 : per_cu;
  const int64_t wgs = cdiv(M, d.bm) * cdiv(N, d.bn) * S;
  if (v.persistent) {
    // Only several rounds of tiles give it anything to overlap; with one
    // round (or split partials, which it has no form for) its twin runs.
    if (S != 1 || wgs <= 256) return 1e30;
    const PsRate& q = table().ps[dtype][d.id];
    const int64_t rounds = cdiv(wgs, 256);
    const double twin = (double)rounds * 2.0 * d.bm * d.bn * (double)(Kc > 0 ? Kc : 1) /
                        ((v.eff > 0.f ? v.eff : 0.1) * rate);
    return twin - (double)rounds * (q.saved_us - (double)cdiv(Kc, d.bk) * q.slice_us) * 1e-6;
  }
  if (wgs <= 256) {
    // One workgroup per CU at most (unsplit, or a split's partials): the
    // fixed cost plus the loop at its rate alone, eff1 with up to 64 CUs
    // busy, linearly down to its rate with all 256 busy.  That is
    // full_loop_rate for a tile that fills its CU's LDS (eff was measured
    // with one workgroup per CU); for a smaller one, which eff measured two
    // to a CU, eff for a split's partials and, unsplit, the dtype's derate
    // of eff1, at most eff.
    const Table& t = table();
    const AloneRate& a = t.alone[dtype][d.id];
    const double e1 = a.eff1 > 0.f ? a.eff1 : 0.1;
    const double eff = v.eff > 0.f ? v.eff : 0.1;
    const double full = per_cu == 1 ? full_loop_rate(dtype, v, a)
                                    : S > 1 ? eff : std::min(eff, e1 * t.derate[dtype]);
    const double f = wgs <= 64 ? 0.0 : (double)(wgs - 64) / 192.0;
    const double r = e1 + (full - e1) * f;
    return a.fixed_us * 1e-6 + 2.0 * d.bm * d.bn * (double)(Kc > 0 ? Kc : 1) / (r * rate);
  }
  const int64_t rounds = cdiv(wgs, 256 * per_cu);
  const double eff = v.eff > 0.f ? v.eff : 0.1;
  // A CU running w workgroups at once gives each 1/w of its rate, so the
  // busiest CU, with ceil(WGs / 256) workgroups, takes that many tiles'
  // work at the CU's rate (a CU whose last workgroup runs alone runs it at
  // least that fast).  Split partials, short K chunks, pay each round's
  // fixed cost on top (eff, measured at K = 4096, holds it for the unsplit
  // rounds).
  const double fixed = S > 1 ? (double)rounds * table().alone[dtype][d.id].fixed_us * 1e-6 : 0.0;
  return fixed + (double)cdiv(wgs, 256) * 2.0 * d.bm * d.bn * (double)(Kc > 0 ? Kc : 1) / (eff * rate);
}

Choice heuristic(int dtype, int64_t M, int64_t N, int64_t K, bool allow_split, bool need_epi = false,
                 bool need_bt = false, bool need_q8 = false, bool need_at = false) {
  const auto& v = table().v[dtype];
  const double es = (double)out_bytes(dtype);
  Choice best;
  for (size_t i = 0; i < v.size(); ++i) {
    if (v[i].desc.family != GEMM_FAMILY_MFMA) continue;
    if (need_epi && !v[i].launch_epi) continue;
    if (need_bt && !v[i].launch_bt) continue;
    if (need_q8 && !v[i].launch_q8) continue;
    if (need_at && !(need_bt ? v[i].launch_atbt : v[i].launch_at)) continue;
    const double t1 = gemm_seconds(dtype, v[i], M, N, K, 1);
    if (t1 < best.t) best = Choice{(int)i, 1, t1};
    if (!allow_split || !v[i].launch_partial || M == 0 || N == 0) continue;
    for (int64_t want = 2; want <= 32; ++want) {
      int64_t S, Kc;
      split_shape(dtype, K, want, S, Kc);
      if (S != want) continue;
      if (Kc < 256) break;
      const double t = gemm_seconds(dtype, v[i], M, N, Kc, S) +
                       (2.0 * S * M * N * 4.0 + M * N * es) / 4.0e12 + 4e-6;
      if (t < best.t) best = Choice{(int)i, S, t};
    }
  }
  if (best.id < 0) best.id = 0;
  return best;
}

// Plain calls (split = false) never split; split-K calls may.
gemm_config_t select(int dtype, int64_t M, int64_t N, int64_t K, bool split = false,
                     bool need_epi = false, bool need_bt = false, bool need_q8 = false,
                     bool need_at = false) {
  {
    std::lock_guard<std::mutex> lk(g_tuning_mu);
    for (const auto& e : g_tuning)
      if (e.dtype == dtype && e.M == M && e.N == N && e.K == K && (split || e.splits <= 1) &&
          (!need_epi || table().v[dtype][e.id].launch_epi) && !need_bt && !need_q8 && !need_at) {
        gemm_config_t d = table().v[dtype][e.id].desc;
        d.order = e.order;
        d.group_m = e.group_m;
        d.splits = split ? e.splits : 1;
        return d;
      }
  }
  const Choice c = heuristic(dtype, M, N, K, split, need_epi, need_bt, need_q8, need_at);
  gemm_config_t d = table().v[dtype][c.id].desc;
  d.splits = (int32_t)c.splits;
  return d;
}

TileMap make_map(const gemm_config_t& c, int64_t M, int64_t N) {
  TileMap t;
  t.tiles_m = (int)cdiv(M, c.bm);
  t.tiles_n = (int)cdiv(N, c.bn);
  t.order = c.order;
  // Bands taller than the grid are the whole grid (and keep the band
  // width, group_m * tiles_n, within an int for any requested group_m).
  t.group_m = c.group_m < 1 ? 1 : (int)std::min<int64_t>(c.group_m, t.tiles_m);
  t.xcds = kXcds;
  return t;
}

bool overlap(const void* a, size_t abytes, const void* b, size_t bbytes) {
  if (!a || !b || abytes == 0 || bbytes == 0) return false;
  const unsigned __int128 a0 = (uintptr_t)a, b0 = (uintptr_t)b;  // no wrap at the top
  return a0 < b0 + bbytes && b0 < a0 + abytes;
}

// Byte range of a rows x cols operand with leading dimension ld (>= 1),
// saturated at 2^63: validate() rejects operands that reach it.
constexpr size_t kSpanLimit = (size_t)1 << 63;
size_t span_bytes(int64_t rows, int64_t cols, int64_t ld, size_t es) {
  if (rows <= 0 || cols <= 0) return 0;
  const unsigned __int128 s =
      ((unsigned __int128)(uint64_t)(rows - 1) * (uint64_t)ld + (uint64_t)cols) * es;
  return s >= kSpanLimit ? kSpanLimit : (size_t)s;
}

// bt: B is given transposed (Bt, N x K row-major, leading dimension ldb).
// c_es: bytes of one C element when not the dtype's (INT8 codes: 1).
// at: A is given transposed (At, K x M row-major, leading dimension lda).
gemm_status_t validate(int dtype, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                       const void* B, int64_t ldb, const void* C, int64_t ldc, bool bt = false,
                       size_t c_es = 0, bool at = false) {
  if (M < 0 || N < 0 || K < 0) return fail(GEMM_ERR_INVALID_ARG, "negative dimension");
  const int64_t lim = 0x7fffffff;
  if (M > lim || N > lim || K > lim) return fail(GEMM_ERR_INVALID_ARG, "dimension above 2^31-1");
  if (!at && lda < (K > 1 ? K : 1)) return fail(GEMM_ERR_INVALID_ARG, "lda < max(1, K)");
  if (at && lda < (M > 1 ? M : 1)) return fail(GEMM_ERR_INVALID_ARG, "lda < max(1, M) (A transposed)");
  if (!bt && ldb < (N > 1 ? N : 1)) return fail(GEMM_ERR_INVALID_ARG, "ldb < max(1, N)");
  if (bt && ldb < (K > 1 ? K : 1)) return fail(GEMM_ERR_INVALID_ARG, "ldbt < max(1, K)");
  if (ldc < (N > 1 ? N : 1)) return fail(GEMM_ERR_INVALID_ARG, "ldc < max(1, N)");
  if (M > 0 && K > 0 && !A) return fail(GEMM_ERR_INVALID_ARG, "A is NULL");
  if (K > 0 && N > 0 && !B) return fail(GEMM_ERR_INVALID_ARG, "B is NULL");
  if (M > 0 && N > 0 && !C) return fail(GEMM_ERR_INVALID_ARG, "C is NULL");
  const int64_t tiles_lim = 0x7fffffff;
  if (cdiv(M, 64) * cdiv(N, 64) > tiles_lim) return fail(GEMM_ERR_INVALID_ARG, "output too large");
  const size_t es = in_bytes(dtype);
  const size_t cb = span_bytes(M, N, ldc, c_es ? c_es : out_bytes(dtype));
  const size_t ab = at ? span_bytes(K, M, lda, es) : span_bytes(M, K, lda, es);
  const size_t bb = bt ? span_bytes(N, K, ldb, es) : span_bytes(K, N, ldb, es);
  if (ab >= kSpanLimit || bb >= kSpanLimit || cb >= kSpanLimit)
    return fail(GEMM_ERR_INVALID_ARG, "an operand's byte range reaches 2^63 (leading dimension too large)");
  if (overlap(C, cb, A, ab) || overlap(C, cb, B, bb)) return fail(GEMM_ERR_ALIAS, "C overlaps A or B");
  return GEMM_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Environment, read once: GEMM_FORCE_CONFIG names a variant that replaces
// the library's own choice in calls of that variant's element type that do
// not force one themselves (ignored where the variant lacks the call's
// form); GEMM_LOG (any value but "0") prints each call's shape, form and
// configuration to stderr.
struct Env {
  std::string force;
  bool log = false;
};
const Env& env() {
  static const Env e = [] {
    Env x;
    if (const char* f = getenv("GEMM_FORCE_CONFIG")) x.force = f;
    const char* l = getenv("GEMM_LOG");
    x.log = l && *l && strcmp(l, "0") != 0;
    return x;
  }();
  return e;
}

gemm_status_t resolve_forced(int dtype, int64_t M, int64_t N, int64_t K, const gemm_config_t* forced,
                             bool split, gemm_config_t& cfg, bool need_epi, bool need_bt,
                             bool need_q8, bool need_at);

// Resolves the configuration of a call: the forced one (checked), the
// GEMM_FORCE_CONFIG variant, or the selection for the shape.
gemm_status_t resolve(int dtype, int64_t M, int64_t N, int64_t K, const gemm_config_t* forced,
                      bool split, gemm_config_t& cfg, bool need_epi = false, bool need_bt = false,
                      bool need_q8 = false, bool need_at = false) {
  gemm_status_t st = GEMM_OK;
  if (forced) {
    st = resolve_forced(dtype, M, N, K, forced, split, cfg, need_epi, need_bt, need_q8, need_at);
  } else {
    cfg = select(dtype, M, N, K, split, need_epi, need_bt, need_q8, need_at);
    const int id = env().force.empty() ? -1 : find_by_name(dtype, env().force.c_str());
    if (id >= 0) {
      gemm_config_t f = table().v[dtype][id].desc;
      f.splits = 0;  // split calls: the model's best count for this variant
      gemm_config_t g;
      if (resolve_forced(dtype, M, N, K, &f, split, g, need_epi, need_bt, need_q8, need_at) == GEMM_OK)
        cfg = g;
      g_err[0] = 0;
    }
  }
  if (st == GEMM_OK && env().log)
    fprintf(stderr, "libgemm: %s %lldx%lldx%lld%s%s%s%s%s -> %s order=%d group_m=%d splits=%d\n",
            dtype_name(dtype), (long long)M, (long long)N, (long long)K, split ? " splitk" : "",
            need_epi ? " epi" : "", need_q8 ? " q8" : "", need_at ? " at" : "", need_bt ? " bt" : "",
            cfg.name, cfg.order, cfg.group_m, cfg.splits);
  return st;
}

gemm_status_t resolve_forced(int dtype, int64_t M, int64_t N, int64_t K, const gemm_config_t* forced,
                             bool split, gemm_config_t& cfg, bool need_epi, bool need_bt,
                             bool need_q8, bool need_at) {
  const auto& v = table().v[dtype];
  if (forced->id < 0 || forced->id >= (int32_t)v.size())
    return fail(GEMM_ERR_UNSUPPORTED, "config id %d not in the %s table", forced->id,
                dtype_name(dtype));
  if (forced->order < GEMM_ORDER_ROW || forced->order > GEMM_ORDER_XCD || forced->group_m < 1)
    return fail(GEMM_ERR_UNSUPPORTED, "bad tile order %d / group_m %d", forced->order,
                forced->group_m);
  if (split && forced->splits < 0) return fail(GEMM_ERR_UNSUPPORTED, "negative splits");
  if (need_epi && !v[forced->id].launch_epi)
    return fail(GEMM_ERR_UNSUPPORTED, "variant %s has no fused-epilogue form", v[forced->id].desc.name);
  if (need_bt && !v[forced->id].launch_bt)
    return fail(GEMM_ERR_UNSUPPORTED, "variant %s has no transposed-B form", v[forced->id].desc.name);
  if (need_q8 && !v[forced->id].launch_q8)
    return fail(GEMM_ERR_UNSUPPORTED, "variant %s has no INT8-epilogue form", v[forced->id].desc.name);
  if (need_at && !(need_bt ? v[forced->id].launch_atbt : v[forced->id].launch_at))
    return fail(GEMM_ERR_UNSUPPORTED, "variant %s has no transposed-A form", v[forced->id].desc.name);
  cfg = v[forced->id].desc;
  cfg.order = forced->order;
  cfg.group_m = forced->group_m;
  cfg.splits = split ? forced->splits : 1;
  if (split && cfg.splits == 0) {
    // The model's best split count for this variant.
    double best = 1e30;
    cfg.splits = 1;
    for (int64_t want = 1; want <= 32; ++want) {
      int64_t S, Kc;
      split_shape(dtype, K, want, S, Kc);
      if (S != want) continue;
      if (want > 1 && (Kc < 256 || !v[forced->id].launch_partial)) break;
      const double es = (double)out_bytes(dtype);
      const double t = gemm_seconds(dtype, v[forced->id], M, N, Kc, S) +
                       (S > 1 ? (2.0 * S * M * N * 4.0 + M * N * es) / 4.0e12 + 4e-6 : 0.0);
      if (t < best) {
        best = t;
        cfg.splits = (int32_t)S;
      }
    }
  }
  return GEMM_OK;
}

bool vector_path(int dtype, const void* A, int64_t lda, const void* B, int64_t ldb, const void* C,
                 int64_t ldc, int64_t K, int64_t N, size_t c_es = 0) {
  const int64_t w = 16 / (int64_t)in_bytes(dtype);  // elements per 16 bytes
  const int64_t wc = 16 / (int64_t)(c_es ? c_es : out_bytes(dtype));
  // FP8 with K = 0 reads neither A nor B (C = 0): only C's layout matters.
  if (is_f8(dtype) && K == 0) return aligned16(C) && ldc % wc == 0 && N % wc == 0;
  return aligned16(A) && aligned16(B) && aligned16(C) && lda % w == 0 && ldb % w == 0 &&
         ldc % wc == 0 && K % w == 0 && N % w == 0;
}

// FP8 operands off the vector layout run on the general 16-bit kernel
// (widened to bfloat16 while staging); a form that it lacks is refused.
gemm_status_t f8_unsupported() {
  return fail(GEMM_ERR_UNSUPPORTED,
              "this FP8 form needs 16-byte aligned A, B, C, K, N, lda and ldb multiples of 16, "
              "ldc a multiple of 8, and byte offsets below 2^31");
}

// gemm_trace_set's buffer and capacity, per host thread.
thread_local unsigned long long* g_trace = nullptr;
thread_local int g_trace_cap = 0;

Params make_params(int dtype, const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                   int64_t ldc, int64_t M, int64_t N, int64_t K) {
  Params p;
  p.trace = g_trace;
  p.trace_cap = g_trace_cap;
  p.bf16 = dtype == GEMM_DTYPE_BF16;
  p.f8 = dtype == GEMM_DTYPE_F8 ? 1 : dtype == GEMM_DTYPE_E5M2 ? 2 : 0;
  p.A = A;
  p.B = B;
  p.C = C;
  p.lda = lda;
  p.ldb = ldb;
  p.ldc = ldc;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  return p;
}

gemm_status_t launch_plain(int dtype, const gemm_config_t& cfg, int64_t M, int64_t N, int64_t K,
                           const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                           int64_t ldc, void* stream) {
  const Params p = make_params(dtype, A, lda, B, ldb, C, ldc, M, N, K);
  const bool vec = vector_path(dtype, A, lda, B, ldb, C, ldc, K, N);
  const TileMap map = make_map(cfg, M, N);
  const hipError_t e = table().v[dtype][cfg.id].launch(p, map, vec, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported && is_f8(dtype)) return f8_unsupported();
  if (e != hipSuccess) return fail(GEMM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return GEMM_OK;
}

gemm_status_t run(int dtype, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                  const void* B, int64_t ldb, void* C, int64_t ldc, void* stream,
                  const gemm_config_t* forced) {
  g_err[0] = 0;
  gemm_status_t st = validate(dtype, M, N, K, A, lda, B, ldb, C, ldc);
  if (st != GEMM_OK) return st;
  gemm_config_t cfg;
  st = resolve(dtype, M, N, K, forced, false, cfg);
  if (st != GEMM_OK) return st;
  if (M == 0 || N == 0) return GEMM_OK;
  return launch_plain(dtype, cfg, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

gemm_status_t run_bt(int dtype, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                     const void* Bt, int64_t ldbt, void* C, int64_t ldc, void* stream,
                     const gemm_config_t* forced) {
  g_err[0] = 0;
  gemm_status_t st = validate(dtype, M, N, K, A, lda, Bt, ldbt, C, ldc, true);
  if (st != GEMM_OK) return st;
  gemm_config_t cfg;
  st = resolve(dtype, M, N, K, forced, false, cfg, false, true);
  if (st != GEMM_OK) return st;
  if (M == 0 || N == 0) return GEMM_OK;
  Params p = make_params(dtype, A, lda, Bt, ldbt, C, ldc, M, N, K);
  p.bt = true;
  const bool vec = vector_path(dtype, A, lda, Bt, ldbt, C, ldc, K, N);
  const TileMap map = make_map(cfg, M, N);
  const hipError_t e =
      table().v[dtype][cfg.id].launch_bt(p, map, vec, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported && is_f8(dtype)) return f8_unsupported();
  if (e != hipSuccess) return fail(GEMM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return GEMM_OK;
}

gemm_status_t run_epi(int dtype, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                      const void* B, int64_t ldb, void* C, int64_t ldc, void* stream,
                      const gemm_config_t* forced, const gemm_epilogue_t* epi) {
  g_err[0] = 0;
  gemm_status_t st = validate(dtype, M, N, K, A, lda, B, ldb, C, ldc);
  if (st != GEMM_OK) return st;
  if (!epi) return fail(GEMM_ERR_INVALID_ARG, "epi is NULL");
  if (epi->act != GEMM_ACT_NONE && epi->act != GEMM_ACT_RELU)
    return fail(GEMM_ERR_INVALID_ARG, "unknown activation %d", epi->act);
  if (epi->bias && overlap(epi->bias, (size_t)N * 4, C, span_bytes(M, N, ldc, out_bytes(dtype))))
    return fail(GEMM_ERR_ALIAS, "bias overlaps C");
  gemm_config_t cfg;
  st = resolve(dtype, M, N, K, forced, false, cfg, true);
  if (st != GEMM_OK) return st;
  if (M == 0 || N == 0) return GEMM_OK;
  Params p = make_params(dtype, A, lda, B, ldb, C, ldc, M, N, K);
  p.epi.on = true;
  p.epi.alpha = epi->alpha;
  p.epi.beta = epi->beta;
  p.epi.bias = epi->bias;
  p.epi.act = epi->act;
  // The vector forms read the bias four floats at a time.
  const bool vec = vector_path(dtype, A, lda, B, ldb, C, ldc, K, N) &&
                   (!epi->bias || aligned16(epi->bias));
  const TileMap map = make_map(cfg, M, N);
  const hipError_t e =
      table().v[dtype][cfg.id].launch_epi(p, map, vec, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported && is_f8(dtype)) return f8_unsupported();
  if (e != hipSuccess) return fail(GEMM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return GEMM_OK;
}

// INT8-quantising epilogue: Q = sat8(rne(act(alpha * A x B + bias))).
gemm_status_t run_q8(int dtype, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                     const void* B, int64_t ldb, int8_t* Q, int64_t ldq, void* stream,
                     const gemm_config_t* forced, const gemm_epilogue_t* epi) {
  g_err[0] = 0;
  gemm_status_t st = validate(dtype, M, N, K, A, lda, B, ldb, Q, ldq, false, 1);
  if (st != GEMM_OK) return st;
  if (!epi) return fail(GEMM_ERR_INVALID_ARG, "epi is NULL");
  if (epi->act != GEMM_ACT_NONE && epi->act != GEMM_ACT_RELU)
    return fail(GEMM_ERR_INVALID_ARG, "unknown activation %d", epi->act);
  if (epi->beta != 0.f)
    return fail(GEMM_ERR_INVALID_ARG, "the INT8 epilogue has no beta term (epi->beta must be 0)");
  if (epi->bias && overlap(epi->bias, (size_t)N * 4, Q, span_bytes(M, N, ldq, 1)))
    return fail(GEMM_ERR_ALIAS, "bias overlaps Q");
  gemm_config_t cfg;
  st = resolve(dtype, M, N, K, forced, false, cfg, false, false, true);
  if (st != GEMM_OK) return st;
  if (M == 0 || N == 0) return GEMM_OK;
  Params p = make_params(dtype, A, lda, B, ldb, Q, ldq, M, N, K);
  p.epi.on = true;
  p.epi.alpha = epi->alpha;
  p.epi.beta = 0.f;
  p.epi.bias = epi->bias;
  p.epi.act = epi->act;
  const bool vec = vector_path(dtype, A, lda, B, ldb, Q, ldq, K, N, 1) &&
                   (!epi->bias || aligned16(epi->bias));
  auto unsupported = [] {
    return fail(GEMM_ERR_UNSUPPORTED,
                "the INT8 epilogue needs 16-byte aligned operands, Q and bias, K and N multiples "
                "of 16 bytes of A and B elements, ldq a multiple of 16, and byte offsets below 2^31");
  };
  if (!vec) return unsupported();
  const TileMap map = make_map(cfg, M, N);
  const hipError_t e = table().v[dtype][cfg.id].launch_q8(p, map, vec, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return unsupported();
  if (e != hipSuccess) return fail(GEMM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return GEMM_OK;
}

// C = op(A) op(B) for the four layouts; the two with A transposed run on
// the LDS-direct kernels' transposed-A forms (vector layout only).
gemm_status_t run_trans(int dtype, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                        const void* B, int64_t ldb, void* C, int64_t ldc, void* stream,
                        const gemm_config_t* forced, int32_t trans_a, int32_t trans_b) {
  g_err[0] = 0;
  if ((trans_a != 0 && trans_a != 1) || (trans_b != 0 && trans_b != 1))
    return fail(GEMM_ERR_INVALID_ARG, "trans_a and trans_b must be 0 or 1");
  if (!trans_a) return trans_b ? run_bt(dtype, M, N, K, A, lda, B, ldb, C, ldc, stream, forced)
                               : run(dtype, M, N, K, A, lda, B, ldb, C, ldc, stream, forced);
  const bool bt = trans_b != 0;
  gemm_status_t st = validate(dtype, M, N, K, A, lda, B, ldb, C, ldc, bt, 0, true);
  if (st != GEMM_OK) return st;
  gemm_config_t cfg;
  st = resolve(dtype, M, N, K, forced, false, cfg, false, bt, false, true);
  if (st != GEMM_OK) return st;
  if (M == 0 || N == 0) return GEMM_OK;
  Params p = make_params(dtype, A, lda, B, ldb, C, ldc, M, N, K);
  p.bt = bt;
  // 16-byte chunks: A^T rows of M values, B rows of N (or Bt rows of K).
  const int64_t w = 16 / (int64_t)in_bytes(dtype), wc = 16 / (int64_t)out_bytes(dtype);
  const bool vec = aligned16(A) && aligned16(B) && aligned16(C) && lda % w == 0 && ldb % w == 0 &&
                   ldc % wc == 0 && M % w == 0 && (bt ? K % w == 0 : N % w == 0) && N % wc == 0;
  auto unsupported = [] {
    return fail(GEMM_ERR_UNSUPPORTED,
                "A transposed needs 16-byte aligned A, B and C, M, lda, ldb and N (K when B is "
                "transposed too) multiples of 16 bytes of elements, ldc likewise for C, and byte "
                "offsets below 2^31");
  };
  if (!vec) return unsupported();
  const Variant& var = table().v[dtype][cfg.id];
  const TileMap map = make_map(cfg, M, N);
  const hipError_t e =
      (bt ? var.launch_atbt : var.launch_at)(p, map, vec, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return unsupported();
  if (e != hipSuccess) return fail(GEMM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return GEMM_OK;
}

gemm_status_t run_splitk(int dtype, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                         const void* B, int64_t ldb, void* C, int64_t ldc, void* ws,
                         int64_t ws_bytes, void* stream, const gemm_config_t* forced) {
  g_err[0] = 0;
  gemm_status_t st = validate(dtype, M, N, K, A, lda, B, ldb, C, ldc);
  if (st != GEMM_OK) return st;
  if (ws_bytes < 0) return fail(GEMM_ERR_INVALID_ARG, "negative workspace size");
  gemm_config_t cfg;
  st = resolve(dtype, M, N, K, forced, true, cfg);
  if (st != GEMM_OK) return st;
  if (M == 0 || N == 0) return GEMM_OK;
  int64_t S, Kc;
  split_shape(dtype, K, cfg.splits, S, Kc);
  const Variant& var = table().v[dtype][cfg.id];
  const bool vec = vector_path(dtype, A, lda, B, ldb, C, ldc, K, N);
  if (S <= 1 || K == 0 || !vec || !var.launch_partial)
    return launch_plain(dtype, cfg, M, N, K, A, lda, B, ldb, C, ldc, stream);
  const int64_t need = partial_bytes(S, M, N);
  if (need < 0) return fail(GEMM_ERR_INVALID_ARG, "workspace size overflows int64");
  if (!ws) return fail(GEMM_ERR_INVALID_ARG, "workspace is NULL (%lld bytes needed)", (long long)need);
  if (ws_bytes < need)
    return fail(GEMM_ERR_INVALID_ARG, "workspace of %lld bytes, %lld needed", (long long)ws_bytes,
                (long long)need);
  if (!aligned16(ws)) return fail(GEMM_ERR_INVALID_ARG, "workspace not 16-byte aligned");
  const size_t es = in_bytes(dtype);
  if (overlap(ws, (size_t)need, A, span_bytes(M, K, lda, es)) ||
      overlap(ws, (size_t)need, B, span_bytes(K, N, ldb, es)) ||
      overlap(ws, (size_t)need, C, span_bytes(M, N, ldc, out_bytes(dtype))))
    return fail(GEMM_ERR_ALIAS, "workspace overlaps A, B or C");
  Params p = make_params(dtype, A, lda, B, ldb, ws, N, M, N, K);
  p.splits = (int)S;
  p.kc = (int)Kc;
  p.c_stride = M * N;
  const TileMap map = make_map(cfg, M, N);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = var.launch_partial(p, map, vec, hs);
  if (e == hipErrorNotSupported)  // offsets beyond the fast kernel's range
    return launch_plain(dtype, cfg, M, N, K, A, lda, B, ldb, C, ldc, stream);
  if (e == hipSuccess)
    e = splitk_reduce(out_dtype(dtype), static_cast<const float*>(ws), (int)S, (int)M, (int)N, C, ldc, hs);
  if (e != hipSuccess) return fail(GEMM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return GEMM_OK;
}

// ---------------------------------------------------------------------------
// Split-K without a caller workspace: the partial planes live in a static
// device array.  Each GPU the library runs on holds its own copy of it
// (kScratchBytes) until the process ends; its device address is looked up
// once per device, with that device current, and kept.  Host code never
// passes the array's own name to a kernel or a copy (on the host that name
// is a stand-in, not a device address).
constexpr int64_t kScratchBytes = GEMM_SPLITK_STATIC_MAX_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's address on the device that runs `stream`.
gemm_status_t scratch_for(void* stream, void** out) {
  int dev = -1;
  const hipError_t e0 = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev)
                               : hipGetDevice(&dev);
  if (e0 != hipSuccess) return fail(GEMM_ERR_HIP, "no device for the stream: %s", hipGetErrorString(e0));
  if (dev < 0 || dev >= kMaxDevices) return fail(GEMM_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess || !p)
      return fail(GEMM_ERR_HIP, "scratch address on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GEMM_OK;
}

gemm_status_t run_splitk_static(int dtype, int64_t M, int64_t N, int64_t K, const void* A,
                                int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                                void* stream, const gemm_config_t* forced) {
  g_err[0] = 0;
  if (!valid_dtype(dtype)) return fail(GEMM_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  gemm_status_t st = validate(dtype, M, N, K, A, lda, B, ldb, C, ldc);
  if (st != GEMM_OK) return st;
  gemm_config_t cfg;
  st = resolve(dtype, M, N, K, forced, true, cfg);
  if (st != GEMM_OK) return st;
  if (M == 0 || N == 0) return GEMM_OK;
  int64_t S, Kc;
  split_shape(dtype, K, cfg.splits, S, Kc);
  const bool vec = vector_path(dtype, A, lda, B, ldb, C, ldc, K, N);
  // The same cases as the workspace form run unsplit and touch no scratch.
  if (S <= 1 || K == 0 || !vec || !table().v[dtype][cfg.id].launch_partial)
    return launch_plain(dtype, cfg, M, N, K, A, lda, B, ldb, C, ldc, stream);
  const int64_t need = partial_bytes(S, M, N);
  if (need < 0 || need > kScratchBytes)
    return fail(GEMM_ERR_INVALID_ARG,
                "split-K needs %lld bytes of partials (%lld chunks of %lld x %lld FP32); the static "
                "scratch holds %lld: use the workspace form or fewer splits",
                (long long)need, (long long)S, (long long)M, (long long)N, (long long)kScratchBytes);
  void* ws = nullptr;
  st = scratch_for(stream, &ws);
  if (st != GEMM_OK) return st;
  return run_splitk(dtype, M, N, K, A, lda, B, ldb, C, ldc, ws, kScratchBytes, stream, forced);
}

}  // namespace
}  // namespace gemm

using namespace gemm;

extern "C" {

gemm_status_t gemm_f32(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                       const float* B, int64_t ldb, float* C, int64_t ldc, void* stream) {
  return run(GEMM_DTYPE_F32, M, N, K, A, lda, B, ldb, C, ldc, stream, nullptr);
}

gemm_status_t gemm_f16(int64_t M, int64_t N, int64_t K, const gemm_f16_t* A, int64_t lda,
                       const gemm_f16_t* B, int64_t ldb, gemm_f16_t* C, int64_t ldc,
                       void* stream) {
  return run(GEMM_DTYPE_F16, M, N, K, A, lda, B, ldb, C, ldc, stream, nullptr);
}

gemm_status_t gemm_bf16(int64_t M, int64_t N, int64_t K, const gemm_bf16_t* A, int64_t lda,
                        const gemm_bf16_t* B, int64_t ldb, gemm_bf16_t* C, int64_t ldc,
                        void* stream) {
  return run(GEMM_DTYPE_BF16, M, N, K, A, lda, B, ldb, C, ldc, stream, nullptr);
}

gemm_status_t gemm_f32_ex(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                          const float* B, int64_t ldb, float* C, int64_t ldc, void* stream,
                          const gemm_config_t* cfg) {
  if (!cfg) return fail(GEMM_ERR_INVALID_ARG, "cfg is NULL");
  return run(GEMM_DTYPE_F32, M, N, K, A, lda, B, ldb, C, ldc, stream, cfg);
}

gemm_status_t gemm_f16_ex(int64_t M, int64_t N, int64_t K, const gemm_f16_t* A, int64_t lda,
                          const gemm_f16_t* B, int64_t ldb, gemm_f16_t* C, int64_t ldc,
                          void* stream, const gemm_config_t* cfg) {
  if (!cfg) return fail(GEMM_ERR_INVALID_ARG, "cfg is NULL");
  return run(GEMM_DTYPE_F16, M, N, K, A, lda, B, ldb, C, ldc, stream, cfg);
}

gemm_status_t gemm_bf16_ex(int64_t M, int64_t N, int64_t K, const gemm_bf16_t* A, int64_t lda,
                           const gemm_bf16_t* B, int64_t ldb, gemm_bf16_t* C, int64_t ldc,
                           void* stream, const gemm_config_t* cfg) {
  if (!cfg) return fail(GEMM_ERR_INVALID_ARG, "cfg is NULL");
  return run(GEMM_DTYPE_BF16, M, N, K, A, lda, B, ldb, C, ldc, stream, cfg);
}

gemm_status_t gemm_f32_bt(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                          const float* Bt, int64_t ldbt, float* C, int64_t ldc, void* stream,
                          const gemm_config_t* cfg) {
  return run_bt(GEMM_DTYPE_F32, M, N, K, A, lda, Bt, ldbt, C, ldc, stream, cfg);
}

gemm_status_t gemm_f16_bt(int64_t M, int64_t N, int64_t K, const gemm_f16_t* A, int64_t lda,
                          const gemm_f16_t* Bt, int64_t ldbt, gemm_f16_t* C, int64_t ldc,
                          void* stream, const gemm_config_t* cfg) {
  return run_bt(GEMM_DTYPE_F16, M, N, K, A, lda, Bt, ldbt, C, ldc, stream, cfg);
}

gemm_status_t gemm_bf16_bt(int64_t M, int64_t N, int64_t K, const gemm_bf16_t* A, int64_t lda,
                           const gemm_bf16_t* Bt, int64_t ldbt, gemm_bf16_t* C, int64_t ldc,
                           void* stream, const gemm_config_t* cfg) {
  return run_bt(GEMM_DTYPE_BF16, M, N, K, A, lda, Bt, ldbt, C, ldc, stream, cfg);
}

gemm_status_t gemm_f32_epi(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                           const float* B, int64_t ldb, float* C, int64_t ldc, void* stream,
                           const gemm_config_t* cfg, const gemm_epilogue_t* epi) {
  return run_epi(GEMM_DTYPE_F32, M, N, K, A, lda, B, ldb, C, ldc, stream, cfg, epi);
}

gemm_status_t gemm_f16_epi(int64_t M, int64_t N, int64_t K, const gemm_f16_t* A, int64_t lda,
                           const gemm_f16_t* B, int64_t ldb, gemm_f16_t* C, int64_t ldc,
                           void* stream, const gemm_config_t* cfg, const gemm_epilogue_t* epi) {
  return run_epi(GEMM_DTYPE_F16, M, N, K, A, lda, B, ldb, C, ldc, stream, cfg, epi);
}

gemm_status_t gemm_bf16_epi(int64_t M, int64_t N, int64_t K, const gemm_bf16_t* A, int64_t lda,
                            const gemm_bf16_t* B, int64_t ldb, gemm_bf16_t* C, int64_t ldc,
                            void* stream, const gemm_config_t* cfg, const gemm_epilogue_t* epi) {
  return run_epi(GEMM_DTYPE_BF16, M, N, K, A, lda, B, ldb, C, ldc, stream, cfg, epi);
}

gemm_status_t gemm_f32_splitk(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                              const float* B, int64_t ldb, float* C, int64_t ldc, void* workspace,
                              int64_t workspace_bytes, void* stream, const gemm_config_t* cfg) {
  return run_splitk(GEMM_DTYPE_F32, M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes,
                    stream, cfg);
}

gemm_status_t gemm_f16_splitk(int64_t M, int64_t N, int64_t K, const gemm_f16_t* A, int64_t lda,
                              const gemm_f16_t* B, int64_t ldb, gemm_f16_t* C, int64_t ldc,
                              void* workspace, int64_t workspace_bytes, void* stream,
                              const gemm_config_t* cfg) {
  return run_splitk(GEMM_DTYPE_F16, M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes,
                    stream, cfg);
}

gemm_status_t gemm_bf16_splitk(int64_t M, int64_t N, int64_t K, const gemm_bf16_t* A,
                               int64_t lda, const gemm_bf16_t* B, int64_t ldb, gemm_bf16_t* C,
                               int64_t ldc, void* workspace, int64_t workspace_bytes, void* stream,
                               const gemm_config_t* cfg) {
  return run_splitk(GEMM_DTYPE_BF16, M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes,
                    stream, cfg);
}

gemm_status_t gemm_f8(int64_t M, int64_t N, int64_t K, const gemm_f8_t* A, int64_t lda,
                      const gemm_f8_t* B, int64_t ldb, gemm_bf16_t* C, int64_t ldc, void* stream) {
  return run(GEMM_DTYPE_F8, M, N, K, A, lda, B, ldb, C, ldc, stream, nullptr);
}

gemm_status_t gemm_f8_ex(int64_t M, int64_t N, int64_t K, const gemm_f8_t* A, int64_t lda,
                         const gemm_f8_t* B, int64_t ldb, gemm_bf16_t* C, int64_t ldc, void* stream,
                         const gemm_config_t* cfg) {
  if (!cfg) return fail(GEMM_ERR_INVALID_ARG, "cfg is NULL");
  return run(GEMM_DTYPE_F8, M, N, K, A, lda, B, ldb, C, ldc, stream, cfg);
}

gemm_status_t gemm_f8_bt(int64_t M, int64_t N, int64_t K, const gemm_f8_t* A, int64_t lda,
                         const gemm_f8_t* Bt, int64_t ldbt, gemm_bf16_t* C, int64_t ldc,
                         void* stream, const gemm_config_t* cfg) {
  return run_bt(GEMM_DTYPE_F8, M, N, K, A, lda, Bt, ldbt, C, ldc, stream, cfg);
}

gemm_status_t gemm_f8_epi(int64_t M, int64_t N, int64_t K, const gemm_f8_t* A, int64_t lda,
                          const gemm_f8_t* B, int64_t ldb, gemm_bf16_t* C, int64_t ldc,
                          void* stream, const gemm_config_t* cfg, const gemm_epilogue_t* epi) {
  return run_epi(GEMM_DTYPE_F8, M, N, K, A, lda, B, ldb, C, ldc, stream, cfg, epi);
}

gemm_status_t gemm_f8_splitk(int64_t M, int64_t N, int64_t K, const gemm_f8_t* A, int64_t lda,
                             const gemm_f8_t* B, int64_t ldb, gemm_bf16_t* C, int64_t ldc,
                             void* workspace, int64_t workspace_bytes, void* stream,
                             const gemm_config_t* cfg) {
  return run_splitk(GEMM_DTYPE_F8, M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes,
                    stream, cfg);
}

gemm_status_t gemm_f32_epi_q8(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                              const float* B, int64_t ldb, int8_t* Q, int64_t ldq, void* stream,
                              const gemm_config_t* cfg, const gemm_epilogue_t* epi) {
  return run_q8(GEMM_DTYPE_F32, M, N, K, A, lda, B, ldb, Q, ldq, stream, cfg, epi);
}

gemm_status_t gemm_f16_epi_q8(int64_t M, int64_t N, int64_t K, const gemm_f16_t* A, int64_t lda,
                              const gemm_f16_t* B, int64_t ldb, int8_t* Q, int64_t ldq,
                              void* stream, const gemm_config_t* cfg, const gemm_epilogue_t* epi) {
  return run_q8(GEMM_DTYPE_F16, M, N, K, A, lda, B, ldb, Q, ldq, stream, cfg, epi);
}

gemm_status_t gemm_bf16_epi_q8(int64_t M, int64_t N, int64_t K, const gemm_bf16_t* A, int64_t lda,
                               const gemm_bf16_t* B, int64_t ldb, int8_t* Q, int64_t ldq,
                               void* stream, const gemm_config_t* cfg, const gemm_epilogue_t* epi) {
  return run_q8(GEMM_DTYPE_BF16, M, N, K, A, lda, B, ldb, Q, ldq, stream, cfg, epi);
}

gemm_status_t gemm_f8_epi_q8(int64_t M, int64_t N, int64_t K, const gemm_f8_t* A, int64_t lda,
                             const gemm_f8_t* B, int64_t ldb, int8_t* Q, int64_t ldq, void* stream,
                             const gemm_config_t* cfg, const gemm_epilogue_t* epi) {
  return run_q8(GEMM_DTYPE_F8, M, N, K, A, lda, B, ldb, Q, ldq, stream, cfg, epi);
}

gemm_status_t gemm_f32_trans(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                             const float* B, int64_t ldb, float* C, int64_t ldc, void* stream,
                             const gemm_config_t* cfg, int32_t trans_a, int32_t trans_b) {
  return run_trans(GEMM_DTYPE_F32, M, N, K, A, lda, B, ldb, C, ldc, stream, cfg, trans_a, trans_b);
}

gemm_status_t gemm_f16_trans(int64_t M, int64_t N, int64_t K, const gemm_f16_t* A, int64_t lda,
                             const gemm_f16_t* B, int64_t ldb, gemm_f16_t* C, int64_t ldc,
                             void* stream, const gemm_config_t* cfg, int32_t trans_a,
                             int32_t trans_b) {
  return run_trans(GEMM_DTYPE_F16, M, N, K, A, lda, B, ldb, C, ldc, stream, cfg, trans_a, trans_b);
}

gemm_status_t gemm_bf16_trans(int64_t M, int64_t N, int64_t K, const gemm_bf16_t* A, int64_t lda,
                              const gemm_bf16_t* B, int64_t ldb, gemm_bf16_t* C, int64_t ldc,
                              void* stream, const gemm_config_t* cfg, int32_t trans_a,
                              int32_t trans_b) {
  return run_trans(GEMM_DTYPE_BF16, M, N, K, A, lda, B, ldb, C, ldc, stream, cfg, trans_a, trans_b);
}

gemm_status_t gemm_f8_trans(int64_t M, int64_t N, int64_t K, const gemm_f8_t* A, int64_t lda,
                            const gemm_f8_t* B, int64_t ldb, gemm_bf16_t* C, int64_t ldc,
                            void* stream, const gemm_config_t* cfg, int32_t trans_a,
                            int32_t trans_b) {
  return run_trans(GEMM_DTYPE_F8, M, N, K, A, lda, B, ldb, C, ldc, stream, cfg, trans_a, trans_b);
}

int64_t gemm_splitk_workspace_bytes(int32_t dtype, int64_t M, int64_t N, int64_t K, int32_t splits) {
  if (!valid_dtype(dtype) || M < 0 || N < 0 || K < 0) return -1;
  const int64_t lim = 0x7fffffff;
  if (M > lim || N > lim || K > lim || cdiv(M, 64) * cdiv(N, 64) > lim) return -1;
  if (splits <= 0) splits = select(dtype, M, N, K, true).splits;
  int64_t S, Kc;
  split_shape(dtype, K, splits, S, Kc);
  return (S > 1 && M > 0 && N > 0) ? partial_bytes(S, M, N) : 0;
}

gemm_status_t gemm_select_splitk_config(int32_t dtype, int64_t M, int64_t N, int64_t K,
                                        gemm_config_t* out) {
  if (!valid_dtype(dtype))
    return fail(GEMM_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (!out || M < 0 || N < 0 || K < 0) return fail(GEMM_ERR_INVALID_ARG, "bad arguments");
  *out = select(dtype, M, N, K, true);
  return GEMM_OK;
}

int32_t gemm_num_configs(int32_t dtype) {
  if (!valid_dtype(dtype)) return 0;
  return (int32_t)table().v[dtype].size();
}

gemm_status_t gemm_get_config(int32_t dtype, int32_t idx, gemm_config_t* out) {
  if (!valid_dtype(dtype))
    return fail(GEMM_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (!out) return fail(GEMM_ERR_INVALID_ARG, "out is NULL");
  const auto& v = table().v[dtype];
  if (idx < 0 || idx >= (int32_t)v.size()) return fail(GEMM_ERR_INVALID_ARG, "index out of range");
  *out = v[idx].desc;
  return GEMM_OK;
}

gemm_status_t gemm_select_config(int32_t dtype, int64_t M, int64_t N, int64_t K,
                                 gemm_config_t* out) {
  if (!valid_dtype(dtype))
    return fail(GEMM_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (!out || M < 0 || N < 0 || K < 0) return fail(GEMM_ERR_INVALID_ARG, "bad arguments");
  *out = select(dtype, M, N, K);
  return GEMM_OK;
}

gemm_status_t gemm_tile_of_block(const gemm_config_t* cfg, int64_t M, int64_t N, int64_t block,
                                 int64_t* tile_m, int64_t* tile_n) {
  if (!cfg || !tile_m || !tile_n || M <= 0 || N <= 0 || cfg->bm <= 0 || cfg->bn <= 0)
    return fail(GEMM_ERR_INVALID_ARG, "bad arguments");
  const TileMap map = make_map(*cfg, M, N);
  if (block < 0 || block >= (int64_t)map.tiles_m * map.tiles_n)
    return fail(GEMM_ERR_INVALID_ARG, "block out of range");
  int tm, tn;
  tile_of_block((int)block, map, tm, tn);
  *tile_m = tm;
  *tile_n = tn;
  return GEMM_OK;
}

gemm_status_t gemm_layout_check(int32_t dtype, int32_t idx, int32_t banks, int64_t out[2]) {
  if (!valid_dtype(dtype))
    return fail(GEMM_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  const auto& v = table().v[dtype];
  if (idx < 0 || idx >= (int32_t)v.size() || !out || banks <= 0 || banks > 64 || (banks & (banks - 1)))
    return fail(GEMM_ERR_INVALID_ARG, "bad arguments");
  const int rc = v[idx].layout_check(banks, out);
  if (rc != 0) return fail(GEMM_ERR_UNSUPPORTED, "layout check %s failed with code %d", v[idx].desc.name, rc);
  return GEMM_OK;
}

gemm_status_t gemm_load_tuning(const char* path) {
  std::vector<TuneEntry> entries;
  if (path) {
    FILE* f = fopen(path, "r");
    if (!f) return fail(GEMM_ERR_INVALID_ARG, "cannot open %s", path);
    char line[512];
    int lineno = 0;
    while (fgets(line, sizeof line, f)) {
      ++lineno;
      if (line[0] == '#' || line[0] == '\n') continue;
      char dt[16], name[64];
      long long M, N, K;
      int order, gm, splits = 1;
      const int got = sscanf(line, "%15s %lld %lld %lld %63s %d %d %d", dt, &M, &N, &K, name, &order,
                             &gm, &splits);
      if (got != 7 && got != 8) {
        fclose(f);
        return fail(GEMM_ERR_INVALID_ARG, "%s:%d: expected 'dtype M N K name order group_m [splits]'", path, lineno);
      }
      int dtype = -1;
      for (int d = 0; d < kDtypes; ++d)
        if (strcmp(dt, dtype_name(d)) == 0) dtype = d;
      const int id = dtype < 0 ? -1 : find_by_name(dtype, name);
      if (id < 0 || order < GEMM_ORDER_ROW || order > GEMM_ORDER_XCD || gm < 1 || splits < 1) {
        fclose(f);
        return fail(GEMM_ERR_INVALID_ARG, "%s:%d: unknown dtype/variant or bad order", path, lineno);
      }
      entries.push_back(TuneEntry{dtype, M, N, K, id, order, gm, splits});
    }
    fclose(f);
  }
  std::lock_guard<std::mutex> lk(g_tuning_mu);
  g_tuning.swap(entries);
  return GEMM_OK;
}

const char* gemm_status_string(gemm_status_t s) {
  switch (s) {
    case GEMM_OK: return "GEMM_OK";
    case GEMM_ERR_INVALID_ARG: return "GEMM_ERR_INVALID_ARG";
    case GEMM_ERR_UNSUPPORTED: return "GEMM_ERR_UNSUPPORTED";
    case GEMM_ERR_HIP: return "GEMM_ERR_HIP";
    case GEMM_ERR_ALIAS: return "GEMM_ERR_ALIAS";
  }
  return "unknown gemm_status_t";
}

const char* gemm_last_error(void) { return g_err; }
const char* gemm_last_hip_error(void) { return g_err; }

gemm_status_t gemm_trace_set(uint64_t* stamps, int64_t workgroups) {
  g_err[0] = 0;
  if (workgroups < 0 || workgroups > 0x7fffffff || (stamps && workgroups == 0))
    return fail(GEMM_ERR_INVALID_ARG, "trace capacity %lld", (long long)workgroups);
  g_trace = stamps ? reinterpret_cast<unsigned long long*>(stamps) : nullptr;
  g_trace_cap = stamps ? (int)workgroups : 0;
  return GEMM_OK;
}

gemm_status_t gemm_splitk_static(int32_t dtype, int64_t M, int64_t N, int64_t K, const void* A,
                                 int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                                 void* stream, const gemm_config_t* cfg) {
  return run_splitk_static(dtype, M, N, K, A, lda, B, ldb, C, ldc, stream, cfg);
}

const char* gemm_version(void) { return "libgemm 0.1.0 (gfx950)"; }

// FP8 E5M2: the FP8 entry points with the other operand format.
gemm_status_t gemm_e5m2(int64_t M, int64_t N, int64_t K, const gemm_e5m2_t* A, int64_t lda,
                        const gemm_e5m2_t* B, int64_t ldb, gemm_bf16_t* C, int64_t ldc, void* stream) {
  return run(GEMM_DTYPE_E5M2, M, N, K, A, lda, B, ldb, C, ldc, stream, nullptr);
}

gemm_status_t gemm_e5m2_ex(int64_t M, int64_t N, int64_t K, const gemm_e5m2_t* A, int64_t lda,
                           const gemm_e5m2_t* B, int64_t ldb, gemm_bf16_t* C, int64_t ldc, void* stream,
                           const gemm_config_t* cfg) {
  if (!cfg) return fail(GEMM_ERR_INVALID_ARG, "cfg is NULL");
  return run(GEMM_DTYPE_E5M2, M, N, K, A, lda, B, ldb, C, ldc, stream, cfg);
}

gemm_status_t gemm_e5m2_bt(int64_t M, int64_t N, int64_t K, const gemm_e5m2_t* A, int64_t lda,
                           const gemm_e5m2_t* Bt, int64_t ldbt, gemm_bf16_t* C, int64_t ldc,
                           void* stream, const gemm_config_t* cfg) {
  return run_bt(GEMM_DTYPE_E5M2, M, N, K, A, lda, Bt, ldbt, C, ldc, stream, cfg);
}

gemm_status_t gemm_e5m2_epi(int64_t M, int64_t N, int64_t K, const gemm_e5m2_t* A, int64_t lda,
                            const gemm_e5m2_t* B, int64_t ldb, gemm_bf16_t* C, int64_t ldc,
                            void* stream, const gemm_config_t* cfg, const gemm_epilogue_t* epi) {
  return run_epi(GEMM_DTYPE_E5M2, M, N, K, A, lda, B, ldb, C, ldc, stream, cfg, epi);
}

gemm_status_t gemm_e5m2_splitk(int64_t M, int64_t N, int64_t K, const gemm_e5m2_t* A, int64_t lda,
                               const gemm_e5m2_t* B, int64_t ldb, gemm_bf16_t* C, int64_t ldc,
                               void* workspace, int64_t workspace_bytes, void* stream,
                               const gemm_config_t* cfg) {
  return run_splitk(GEMM_DTYPE_E5M2, M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes,
                    stream, cfg);
}

gemm_status_t gemm_e5m2_epi_q8(int64_t M, int64_t N, int64_t K, const gemm_e5m2_t* A, int64_t lda,
                               const gemm_e5m2_t* B, int64_t ldb, int8_t* Q, int64_t ldq, void* stream,
                               const gemm_config_t* cfg, const gemm_epilogue_t* epi) {
  return run_q8(GEMM_DTYPE_E5M2, M, N, K, A, lda, B, ldb, Q, ldq, stream, cfg, epi);
}

gemm_status_t gemm_e5m2_trans(int64_t M, int64_t N, int64_t K, const gemm_e5m2_t* A, int64_t lda,
                              const gemm_e5m2_t* B, int64_t ldb, gemm_bf16_t* C, int64_t ldc,
                              void* stream, const gemm_config_t* cfg, int32_t trans_a,
                              int32_t trans_b) {
  return run_trans(GEMM_DTYPE_E5M2, M, N, K, A, lda, B, ldb, C, ldc, stream, cfg, trans_a, trans_b);
}

}  // extern "C"
