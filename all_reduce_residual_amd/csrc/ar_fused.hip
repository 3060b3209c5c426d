// ar_fused.hip -- host side of the C ABI declared in include/ar_fused.h: argument validation,
// the launch-shape heuristic, and dispatch to the gfx950 kernels in ar_kernels.hpp (instantiated
// per element type in inst_*.hip; the all-gather kernel is instantiated here).
//
// Nothing here allocates device memory or synchronises: each entry point validates, picks a
// launch shape and enqueues its kernel on the caller's stream (two for the two-kernel path).
// Validation runs before any HIP call, so a rejected call touches neither the device nor the
// outputs.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "ar_dispatch.hpp"
#include "ar_fused.h"
#include "ar_kernels.hpp"

namespace {

using arf::u32x4;

constexpr int kVecBytes = 16;

int elem_size(int dtype) { return dtype == AR_DTYPE_FP32 ? 4 : 2; }
bool valid_dtype(int dtype) {
  return dtype == AR_DTYPE_FP32 || dtype == AR_DTYPE_FP16 || dtype == AR_DTYPE_BF16;
}
bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
int64_t pow2_ceil(int64_t x) {
  int64_t p = 1;
  while (p < x) p <<= 1;
  return p;
}

// ---- shape-level checks ---------------------------------------------------------------------

// Status for (pattern, W, M, H, dtype) alone.  Supported world sizes follow the pages' set
// {2, 4, 8, 16, 32, 64} (vLLM pull request "[Perf] Tune FlashInfer all-reduce selection on
// SM103", Scope) plus W = 1.
int check_shape(int pattern, int W, int64_t M, int64_t H, int dtype) {
  if (pattern != AR_PATTERN_ALLREDUCE && pattern != AR_PATTERN_AR_RESIDUAL_RMSNORM)
    return AR_ERR_INVALID_ARG;
  if (W < 1 || M < 0 || H < 1 || !valid_dtype(dtype)) return AR_ERR_INVALID_ARG;
  if (W > AR_MAX_W || !is_pow2(W)) return AR_ERR_UNSUPPORTED;
  const int64_t es = elem_size(dtype);
  // Keep every byte offset far from int64 overflow (M * H * es <= 2^60, computed by division).
  if (M > 0 && H > ((int64_t(1) << 60) / es) / M) return AR_ERR_UNSUPPORTED;
  if (pattern == AR_PATTERN_AR_RESIDUAL_RMSNORM) {
    const int64_t vec = kVecBytes / es;
    if (H % vec != 0) return AR_ERR_UNSUPPORTED;
    if (H > (dtype == AR_DTYPE_FP32 ? AR_MAX_H_FP32 : AR_MAX_H_16BIT)) return AR_ERR_UNSUPPORTED;
  }
  return AR_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range range_of(const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }
// An output may coincide exactly with a same-sized input (in place); any other overlap is
// rejected.  Each element is read and written by the same thread, reads first.
bool bad_alias_with_input(Range out, Range in) {
  return overlap(out, in) && !(out.lo == in.lo && out.hi == in.hi);
}

// ---- device facts -----------------------------------------------------------------------------

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int query_cu_count(int* cu) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return AR_ERR_DEVICE;
  if (dev < kMaxDevices) {
    const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) {
      *cu = cached;
      return AR_OK;
    }
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    return AR_ERR_DEVICE;
  if (dev < kMaxDevices) g_cu_count[dev].store(n, std::memory_order_relaxed);
  *cu = n;
  return AR_OK;
}

// ---- launch-shape heuristic ---------------------------------------------------------------------
//
// The MI355X counterpart of the pages' thread-block / cluster sizing against the SM count
// (flashinfer pull request "update allreduce to match trtllm", Description and Summary).  The
// pages give no formula; this one is derived from the gfx950 machine: 256 CUs in 8 XCDs,
// 64-lane waves, at most 1024 threads per block, and a bandwidth-bound kernel that needs many
// 16-byte loads in flight on every CU.

int cap_grid(int64_t blocks) {
  if (blocks < 1) return 1;
  return blocks > INT_MAX ? INT_MAX : static_cast<int>(blocks);
}

// max_resident_u: the largest vectors per thread the one-round shapes below may use -- 4 for the
// plain sum; 2 for the two-kernel path's residual sum (its kernel is built for one or two
// vectors per thread); 0 for none (the Lamport consumer keeps the single-wave shape it was
// tuned with).
void plan_sum(int W, int64_t n, int dtype, int cu, ar_launch_cfg_t* c, int max_resident_u = 4) {
  const int64_t vec = kVecBytes / elem_size(dtype);
  const int64_t nvec = n / vec;
  // Single-wave blocks, one 16-byte vector per thread, one block per 64 vectors: the most
  // independent waves for the dispatcher to spread over the 256 CUs.  Small payloads (fewer
  // than 8 such blocks per CU) do better with two vectors per thread and half the blocks; from
  // 8 to 16 blocks per CU one vector stayed ahead (W = 2 / 4 / 8, H = 7168: bf16 3-7.5 %,
  // binary32 1.5-10 % faster in 17 of 18 cases).
  int threads = 64;
  // (Two vectors per thread only for W <= 8: beyond that the doubled loads and rank pointers no
  // longer fit the registers and spill.)
  int u = (W <= 8 && ceil_div(nvec, threads) < int64_t(cu) * 8) ? 2 : 1;
  // Mid-size payloads that one resident round of 3/4 to 2 blocks of 256 threads per CU covers
  // exactly: one launch round with no block scheduling behind it beats many single-wave blocks
  // (W = 8, H = 7168 bf16: M = 64 / 128 11 % and 8 % faster at one vector per thread, M = 512
  // 2-5 % at four; W = 32 / 64 at M = 512 8-14 %).  One vector per thread only for W <= 8
  // (with more ranks it measured from 8 % slower to 9 % faster), four only for W >= 8 (2-5 %
  // slower at W = 2 and 4).
  if (max_resident_u >= 1) {
    const int64_t b1 = ceil_div(nvec, int64_t(256));
    const int64_t b4 = ceil_div(nvec, int64_t(1024));
    if (W <= 8 && b1 >= int64_t(cu) * 3 / 4 && b1 <= int64_t(cu) * 2) {
      threads = 256;
      u = 1;
    } else if (max_resident_u >= 4 && W >= 8 && b4 >= int64_t(cu) * 3 / 2 &&
               b4 <= int64_t(cu) * (W >= 16 ? 8 : 2)) {
      // With 16 or more ranks the 4-vector blocks stay ahead up to 8 blocks per CU (W = 16 / 32
      // / 64, M = 1024 / 2048, H = 7168 bf16 and 8192 fp16: 1-9 % faster; beyond, -3 ... +2 %).
      threads = 256;
      u = 4;
    }
  }
  c->threads_per_block = threads;
  c->vecs_per_thread = u;
  c->lanes_per_row = 0;
  c->rows_per_block = 0;
  c->grid = cap_grid(ceil_div(nvec, int64_t(threads) * u));
  c->flat = 1;
  c->ranks_per_batch = 0;
  // Non-temporal stores measured faster except for outputs that are large next to the reads
  // (W <= 4 at 64 MiB and beyond, W = 8 at 160 MiB): there ordinary stores win by 3-8 %.
  const int64_t out_bytes = n * elem_size(dtype);
  c->nt_store = out_bytes < int64_t(W) * (12 << 20) ? 1 : 0;
}

void plan_norm(int W, int64_t M, int64_t H, int dtype, int cu, ar_launch_cfg_t* c) {
  const int64_t vec = kVecBytes / elem_size(dtype);
  const int64_t V = H / vec;
  int vpt, lanes, threads;
  if (V <= 32) {
    // Narrow rows: a power-of-two lane segment per row, several rows per wave.
    vpt = 1;
    lanes = static_cast<int>(pow2_ceil(V));
    const int64_t rows_per_wave = 64 / lanes;
    threads = (M >= int64_t(cu) * rows_per_wave * 4 * 4) ? 256 : 64;
  } else {
    // Wide rows: one row per block of up to 512 threads (two 16-byte vectors per thread at
    // H = 7168 bf16: 7 waves), the shape that measured fastest from decode to prefill sizes
    // for W >= 4.  With one or two partials a row is few bytes, and once there are more rows
    // than CUs the block per row shrinks in proportion (512 lanes / rows per CU, at least one
    // wave) with more vectors per thread: more rows in flight per CU (W = 2, M = 2048,
    // H = 4096: one wave of 8 vectors per thread per row, 13 % faster than 512 lanes; at
    // W = 4 the 512-lane shape stays ahead, measured).
    int64_t target = 512;
    const int64_t rows_per_cu = M / cu;
    // Two partials with 16-bit rows at 12 or more rows per CU: the shape of W >= 4 again (up
    // to 512 lanes); the narrower rows below lost there by 1-14 % (W = 2, M = 3072 ... 8192;
    // H = 8192 fp16 M = 4096: 61.7 -> 55.4 us, H = 4096 M = 8192: 62.1 -> 54.4 us).
    const bool wide_again = W == 2 && elem_size(dtype) == 2 && rows_per_cu >= 12;
    if (W <= 2 && !wide_again)
      target = std::max<int64_t>(64, 512 / std::max<int64_t>(1, rows_per_cu));
    // Many ranks at eight or more rows per CU (16-bit types): one vector per thread over the
    // whole row (up to 1024 lanes).  A thread's rank batches then hold one chain instead of two,
    // half the round trips per row, and the other rows on the CU keep it busy (W = 32 / 64,
    // M = 2048, H = 7168 bf16: 184 -> 170 / 350 -> 326 us; H = 8192 fp16 W = 32: 3 % faster).
    // At M <= 512, at W = 16 and for binary32 the two-vector rows stayed ahead (2-26 %).
    if (W >= 32 && elem_size(dtype) == 2 && M >= int64_t(cu) * 8) target = 1024;
    // Binary32 rows of 1025 to 2048 vectors while a quarter of the CUs or fewer hold a row, or
    // at eight or more rows per CU: two vectors per thread over up to 1024 lanes instead of four
    // over up to 512 -- twice the waves per row, and a thread's rank batch (16 loads) spans 8
    // ranks instead of 4.  H = 7168, W = 2 ... 64: M <= 64 2-14 % faster (W = 32, M = 16:
    // 24.4 -> 21.0 us), M = 2048 / 4096 1-6.5 %; H = 5120 and 8192 alike.  Between the two
    // (M = 128 ... 1024) it ranged from 9 % slower to 6 % faster.
    if (elem_size(dtype) == 4 && V > 1024 && V <= 2048 &&
        (M * 4 <= int64_t(cu) || M >= int64_t(cu) * 8))
      target = 1024;
    vpt = 1;
    while (vpt < 8 && ceil_div(V, vpt) > target) vpt *= 2;
    while (vpt < 8 && round_up(ceil_div(V, vpt), 64) > 1024) vpt *= 2;
    // Eight or more partials on rows of over 2048 vectors: four vectors per thread while the
    // row fits 768 lanes (1024 for W = 16) rather than eight over up to 512 (16-bit rows
    // H = 20480 / 24576 / 32768: W = 16 5-30 % faster than its staged 8-vector form, W = 32 / 64
    // 6-20 % at M = 1 and 9-12 % at M = 1024, mixed beyond 3072 vectors; W = 8 2-13 % at 2560
    // vectors).  Binary32 rows only while a quarter of the CUs or fewer hold a row: 5-39 %
    // faster at M = 1, but 1.5-7 % slower at M = 256 and mixed at 1024.
    if (vpt == 8 && W >= 8 && (elem_size(dtype) == 2 || M * 4 <= int64_t(cu)) &&
        round_up(ceil_div(V, 4), 64) <= (W == 16 ? 1024 : 768))
      vpt = 4;
    // Rounding the lane count up to whole waves can leave a vector slot that no lane uses
    // (e.g. 1792 vectors at 8 per thread on 256 lanes); halve the vectors per thread instead --
    // except for a single tensor (W = 1, the RMSNorm step alone) once rows outnumber CUs
    // eightfold, where 8 vectors per thread stay faster despite the idle slots (H = 7168,
    // M = 2048: 13.5 -> 10.6 us; at M <= 4 rows per CU halving measured 4-11 % faster).
    // Two partials with 16-bit rows from 4 rows per CU on keep them too (W = 2, H = 7168 bf16,
    // M = 1024 / 2048: 14.7 -> 12.7 / 28.2 -> 26.3 us; binary32 rows lost 7-10 % that way).
    const bool keep_wide = (W == 1 && M >= int64_t(cu) * 8) ||
                           (W == 2 && elem_size(dtype) == 2 && rows_per_cu >= 4);
    while (!keep_wide && vpt > 1 &&
           round_up(ceil_div(V, vpt), 64) * vpt - V >= round_up(ceil_div(V, vpt), 64) &&
           round_up(ceil_div(V, vpt / 2), 64) <= 1024)
      vpt /= 2;
    lanes = static_cast<int>(round_up(ceil_div(V, vpt), 64));
    threads = lanes;
  }
  c->threads_per_block = threads;
  c->vecs_per_thread = vpt;
  c->lanes_per_row = lanes;
  c->rows_per_block = threads / lanes;
  c->grid = cap_grid(ceil_div(M, c->rows_per_block));
  c->flat = 0;
  c->nt_store = 1;  // measured faster from decode to prefill sizes
  // Fixed rank batches for whole rows (one row per block).  One rank per batch while every row
  // is resident at once with one to three rows per CU (cu < M <= 3 cu; 2 vectors per thread for
  // 4 to 16 partials, or 4 for 2 or 4): the CUs then run in the same phase, and reading the
  // tensors one after another instead of all together is what HBM serves faster.  Interleaved
  // A/B of the planned shapes: W = 8 H = 7168 bf16 M = 384 / 512 / 768 2.7 / 6.1 / 4.1 % faster;
  // W = 4 2.7 / 8.5 / 0.5 % (binary32 M = 512 / 768: 2.9 / 8.7 %); fp16 W = 16 H = 8192
  // 11.3 / 4.0 / 3.8 %; W = 2 with 4 vectors (H = 7168, M = 512 / 768) 8.1 / 5.4 %.  W = 2 with
  // 2 vectors, whose chains are staged already, lost up to 6 % (H = 4096, M = 512).  With fewer
  // rows each row's chain of W + 1 round trips is the latency (W = 8 M = 128: 30 % slower).
  // From more than 3 rows per CU the blocks drift apart and one rank per batch lost 5-7 %, but
  // batches of two ranks (four at W = 8 with 16-bit rows) still beat the default 16 loads over
  // 8 ranks.  Two vectors per thread, M = 800 ... 4096, interleaved A/B of three rounds: W = 8
  // H = 7168 bf16 1-2 % faster with 4 ranks (2 ranks were 1-3 % slower from M = 1536), fp16
  // H = 8192 4-7 %, binary32 H = 4096 1-7 % (2 ranks); W = 4 H = 7168 bf16 1-4 %; W = 16 1-5 %
  // (fp16 H = 8192 M = 3072: 1 % slower); W = 32 / 64 4-7 %.  One vector per thread at W >= 32 (the 1024-lane rows, and rows of up to
  // 512 vectors), 2 ranks: 16-bit rows 2.5-10 % faster (W = 32 M = 2048 H = 8192 fp16:
  // 203.5 -> 183.5 us), binary32 H = 2048 W = 32 M = 2048 10 % faster but W = 64 M = 1024 4 %
  // slower, so binary32 takes it from 8 rows per CU.  One vector at W = 8 / 16 was mixed.
  int rpb = 0;
  if (c->rows_per_block == 1 && M > cu) {
    if (M <= int64_t(cu) * 3) {
      if ((vpt == 2 && W >= 4 && W <= 16) || (vpt == 4 && W >= 2 && W <= 4)) rpb = 1;
    } else if (vpt == 2 && W >= 4) {
      rpb = (W == 8 && elem_size(dtype) == 2) ? 4 : 2;
    } else if (vpt == 1 && W >= 32 && (elem_size(dtype) == 2 || M >= int64_t(cu) * 8)) {
      rpb = 2;
    }
  }
  c->ranks_per_batch = rpb;
}

// A caller-supplied shape must be well formed and cover the row; then every kernel access is
// in bounds for any grid.
int check_cfg(int pattern, int W, int64_t H, int dtype, const ar_launch_cfg_t* c) {
  if (!c) return AR_ERR_INVALID_ARG;
  const int rpb = c->ranks_per_batch;
  if (rpb != 0 && rpb != 1 && rpb != 2 && rpb != 4) return AR_ERR_INVALID_ARG;
  const int t = c->threads_per_block;
  if (t < 64 || t > arf::kMaxThreads || t % 64 != 0) return AR_ERR_INVALID_ARG;
  const int u = c->vecs_per_thread;
  if (u != 1 && u != 2 && u != 4 && u != 8) return AR_ERR_INVALID_ARG;
  if (c->grid < 1) return AR_ERR_INVALID_ARG;
  if (c->nt_store != 0 && c->nt_store != 1) return AR_ERR_INVALID_ARG;
  if (pattern == AR_PATTERN_ALLREDUCE) {
    if (c->flat != 1 || u == 8 || rpb) return AR_ERR_INVALID_ARG;
    return AR_OK;
  }
  // Fixed rank batches exist for the shapes the planner uses them on.
  if (rpb && (!c->nt_store || !arf::rank_batch_instantiated(W, u, rpb))) return AR_ERR_INVALID_ARG;
  if (c->flat != 0) return AR_ERR_INVALID_ARG;
  const int L = c->lanes_per_row;
  const bool seg_ok = (L >= 1 && L <= 64 && is_pow2(L)) || (L > 64 && L % 64 == 0);
  if (!seg_ok || L > t || t % L != 0) return AR_ERR_INVALID_ARG;
  if (c->rows_per_block != t / L) return AR_ERR_INVALID_ARG;
  const int64_t V = H / (kVecBytes / elem_size(dtype));
  if (int64_t(L) * u < V) return AR_ERR_INVALID_ARG;
  return AR_OK;
}

// ---- dispatch -----------------------------------------------------------------------------------

// ---- argument validation shared by the entry points ----------------------------------------------

int validate_sum(const void* const* inputs, int W, int64_t M, int64_t H, int dtype,
                 const void* out) {
  const int st = check_shape(AR_PATTERN_ALLREDUCE, W, M, H, dtype);
  if (st != AR_OK) return st;
  if (M == 0) return AR_OK;
  if (!inputs || !out) return AR_ERR_INVALID_ARG;
  for (int r = 0; r < W; ++r)
    if (!inputs[r]) return AR_ERR_INVALID_ARG;
  for (int r = 0; r < W; ++r)
    if (!aligned16(inputs[r])) return AR_ERR_MISALIGNED;
  if (!aligned16(out)) return AR_ERR_MISALIGNED;
  const int64_t bytes = M * H * elem_size(dtype);
  const Range o = range_of(out, bytes);
  for (int r = 0; r < W; ++r)
    if (bad_alias_with_input(o, range_of(inputs[r], bytes))) return AR_ERR_ALIAS;
  return AR_OK;
}

// shape_pattern: AR_PATTERN_AR_RESIDUAL_RMSNORM for the fused kernel (whole vectors per row,
// register-resident rows); AR_PATTERN_ALLREDUCE for the two-kernel path (any row width).
int validate_norm(const void* const* inputs, int W, int64_t M, int64_t H, int dtype,
                  const void* residual, const float* gamma, float eps, const void* residual_out,
                  const void* norm_out, int shape_pattern = AR_PATTERN_AR_RESIDUAL_RMSNORM) {
  const int st = check_shape(shape_pattern, W, M, H, dtype);
  if (st != AR_OK) return st;
  if (!std::isfinite(eps) || eps < 0.0f) return AR_ERR_INVALID_ARG;
  if (M == 0) return AR_OK;
  if (!inputs || !residual || !gamma || !residual_out || !norm_out) return AR_ERR_INVALID_ARG;
  for (int r = 0; r < W; ++r)
    if (!inputs[r]) return AR_ERR_INVALID_ARG;
  for (int r = 0; r < W; ++r)
    if (!aligned16(inputs[r])) return AR_ERR_MISALIGNED;
  if (!aligned16(residual) || !aligned16(gamma) || !aligned16(residual_out) ||
      !aligned16(norm_out))
    return AR_ERR_MISALIGNED;
  const int64_t bytes = M * H * elem_size(dtype);
  const Range ro = range_of(residual_out, bytes);
  const Range no = range_of(norm_out, bytes);
  const Range g = range_of(gamma, H * int64_t(sizeof(float)));
  if (overlap(ro, no) || overlap(ro, g) || overlap(no, g)) return AR_ERR_ALIAS;
  const Range res = range_of(residual, bytes);
  if (bad_alias_with_input(ro, res) || bad_alias_with_input(no, res)) return AR_ERR_ALIAS;
  for (int r = 0; r < W; ++r) {
    const Range in = range_of(inputs[r], bytes);
    if (bad_alias_with_input(ro, in) || bad_alias_with_input(no, in)) return AR_ERR_ALIAS;
  }
  return AR_OK;
}

int run_sum(const void* const* inputs, int W, int64_t M, int64_t H, int dtype, void* out,
            void* stream, const ar_launch_cfg_t* user_cfg) {
  int st = validate_sum(inputs, W, M, H, dtype, out);
  if (st != AR_OK) return st;
  if (user_cfg) {
    st = check_cfg(AR_PATTERN_ALLREDUCE, W, H, dtype, user_cfg);
    if (st != AR_OK) return st;
  }
  if (M == 0) return AR_OK;
  ar_launch_cfg_t cfg;
  if (user_cfg) {
    cfg = *user_cfg;
  } else {
    int cu = 0;
    st = query_cu_count(&cu);
    if (st != AR_OK) return st;
    plan_sum(W, M * H, dtype, cu, &cfg);
  }
  const int64_t vec = kVecBytes / elem_size(dtype);
  const int64_t n = M * H;
  const int64_t nvec = n / vec;
  const int tail = static_cast<int>(n - nvec * vec);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (dtype) {
    case AR_DTYPE_FP32: e = arfh::launch_sum_f32(inputs, W, out, nvec, tail, cfg, s); break;
    case AR_DTYPE_FP16: e = arfh::launch_sum_f16(inputs, W, out, nvec, tail, cfg, s); break;
    default: e = arfh::launch_sum_bf16(inputs, W, out, nvec, tail, cfg, s); break;
  }
  return e == hipSuccess ? AR_OK : AR_ERR_LAUNCH;
}

int run_norm(const void* const* inputs, int W, int64_t M, int64_t H, int dtype,
             const void* residual, const float* gamma, float eps, void* residual_out,
             void* norm_out, void* stream, const ar_launch_cfg_t* user_cfg) {
  int st = validate_norm(inputs, W, M, H, dtype, residual, gamma, eps, residual_out, norm_out);
  if (st != AR_OK) return st;
  if (user_cfg) {
    st = check_cfg(AR_PATTERN_AR_RESIDUAL_RMSNORM, W, H, dtype, user_cfg);
    if (st != AR_OK) return st;
  }
  if (M == 0) return AR_OK;
  ar_launch_cfg_t cfg;
  if (user_cfg) {
    cfg = *user_cfg;
  } else {
    int cu = 0;
    st = query_cu_count(&cu);
    if (st != AR_OK) return st;
    plan_norm(W, M, H, dtype, cu, &cfg);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (dtype) {
    case AR_DTYPE_FP32:
      e = arfh::launch_norm_f32(inputs, W, residual, gamma, eps, residual_out, norm_out, M, H,
                                cfg, s);
      break;
    case AR_DTYPE_FP16:
      e = arfh::launch_norm_f16(inputs, W, residual, gamma, eps, residual_out, norm_out, M, H,
                                cfg, s);
      break;
    default:
      e = arfh::launch_norm_bf16(inputs, W, residual, gamma, eps, residual_out, norm_out, M, H,
                                 cfg, s);
      break;
  }
  return e == hipSuccess ? AR_OK : AR_ERR_LAUNCH;
}

// ---- kARResidualRMSNorm with a row split over several blocks ---------------------------------------
//
// For few rows: S blocks per row exchange their partial sums of squares through a caller
// workspace of AR_SPLIT_SLOTS 8-byte slots per row (see the kernel).  The exchange is what lets a
// row's W + 1 input streams spread over S CUs instead of one.

constexpr int64_t kSplitSlotBytes = 8;
constexpr uint32_t kDefaultMaxPolls = 1u << 14;

int64_t split_workspace_bytes(int64_t M) { return M * arf::kSplitSlots * kSplitSlotBytes; }

int split_segments(int64_t V, int threads, int vpt) {
  return static_cast<int>(ceil_div(V, int64_t(threads) * vpt));
}

int check_split_cfg(int64_t M, int64_t H, int dtype, const ar_split_cfg_t* c) {
  if (!c) return AR_ERR_INVALID_ARG;
  const int t = c->threads_per_block;
  if (t < 64 || t > arf::kMaxThreads || t % 64 != 0) return AR_ERR_INVALID_ARG;
  if (c->vecs_per_thread != 1 && c->vecs_per_thread != 2) return AR_ERR_INVALID_ARG;
  const int64_t V = H / (kVecBytes / elem_size(dtype));
  const int64_t S = ceil_div(V, int64_t(t) * c->vecs_per_thread);
  if (S > arf::kSplitSlots || c->segments != S) return AR_ERR_INVALID_ARG;
  if (M > arf::split_max_rows) return AR_ERR_UNSUPPORTED;  // grid: S x M blocks (y <= 65535)
  return AR_OK;
}

// The planned split for (W, M, H): false when one block per row is the better kernel.  From
// launch sweeps on the MI355X (W = 2 ... 64, H = 4096 ... 8192, M = 1 ... 256):
//  * the split pays once a row's inputs are large: (W + 1) H sizeof(T) >= 64 KiB (W = 2,
//    H = 4096, 24 KiB rows: the exchange costs more than it saves at every M);
//  * one vector per thread, and the narrowest segments (64 lanes, one wave) that keep the grid
//    within one block per CU: M S <= CUs (M <= 16 at H = 7168: 14 segments, 4.7 -> 3.5 us);
//  * at least 4 segments, or 2 for rows of >= 192 KiB: with 2 the gain ranged from -4 % (W = 8,
//    H = 7168, M = 128) to +11 % (W = 64, H = 4096); or 2 for rows of >= 112 KiB while the
//    grid of two segments per row leaves an eighth of the CUs free (M <= 112 on 256 CUs):
//    W = 8, H = 7168 / 8192, M = 80 ... 112: 0-13 % faster (interleaved A/B), W = 4 rows
//    (70-80 KiB) never gained.
bool plan_split(int W, int64_t M, int64_t H, int dtype, int cu, ar_split_cfg_t* c) {
  const int64_t V = H / (kVecBytes / elem_size(dtype));
  const int64_t row_bytes = int64_t(W + 1) * H * elem_size(dtype);
  if (M < 1 || row_bytes < (int64_t(64) << 10)) return false;
  const int64_t s_cap = std::min<int64_t>(arf::kSplitSlots, int64_t(cu) / M);
  const bool two_ok = row_bytes >= (int64_t(192) << 10) ||
                      (row_bytes >= (int64_t(112) << 10) && M * 16 <= int64_t(cu) * 7);
  const int64_t s_min = two_ok ? 2 : 4;
  if (s_cap < s_min) return false;
  int threads = 64;
  while (ceil_div(V, threads) > s_cap && threads < arf::kMaxThreads) threads *= 2;
  const int S = split_segments(V, threads, 1);
  if (S < s_min || S > s_cap) return false;
  c->threads_per_block = threads;
  c->vecs_per_thread = 1;
  c->segments = S;
  c->max_polls = kDefaultMaxPolls;
  return true;
}

// Workspace checks beside validate_norm's.  alias_free: the outputs must not overlap the residual
// or any input at all (a block that stops waiting re-reads other segments' inputs).
int validate_split(const void* const* inputs, int W, int64_t M, int64_t H, int dtype,
                   const void* residual, const float* gamma, const void* residual_out,
                   const void* norm_out, const void* workspace, int64_t workspace_bytes,
                   bool* alias_free) {
  if (!workspace) return AR_ERR_INVALID_ARG;
  if (!aligned16(workspace)) return AR_ERR_MISALIGNED;
  if (workspace_bytes < split_workspace_bytes(M)) return AR_ERR_INVALID_ARG;
  const int64_t bytes = M * H * elem_size(dtype);
  const Range ws = range_of(workspace, split_workspace_bytes(M));
  const Range ro = range_of(residual_out, bytes), no = range_of(norm_out, bytes);
  const Range res = range_of(residual, bytes);
  if (overlap(ws, ro) || overlap(ws, no) || overlap(ws, res) ||
      overlap(ws, range_of(gamma, H * int64_t(sizeof(float)))))
    return AR_ERR_ALIAS;
  bool free_ = !overlap(ro, res) && !overlap(no, res);
  for (int r = 0; r < W; ++r) {
    const Range in = range_of(inputs[r], bytes);
    if (overlap(ws, in)) return AR_ERR_ALIAS;
    if (overlap(ro, in) || overlap(no, in)) free_ = false;
  }
  *alias_free = free_;
  return AR_OK;
}

// planned (user_cfg null): the split kernel when the plan splits and no output aliases an input,
// else the one-block-per-row kernel.  With user_cfg: the split kernel with that shape, or
// AR_ERR_ALIAS when an output aliases an input.
int run_norm_ws(const void* const* inputs, int W, int64_t M, int64_t H, int dtype,
                const void* residual, const float* gamma, float eps, void* residual_out,
                void* norm_out, void* workspace, int64_t workspace_bytes, void* stream,
                const ar_split_cfg_t* user_cfg) {
  int st = validate_norm(inputs, W, M, H, dtype, residual, gamma, eps, residual_out, norm_out);
  if (st != AR_OK) return st;
  if (user_cfg) {
    st = check_split_cfg(M, H, dtype, user_cfg);
    if (st != AR_OK) return st;
  }
  if (M == 0) return AR_OK;
  bool alias_free = false;
  st = validate_split(inputs, W, M, H, dtype, residual, gamma, residual_out, norm_out, workspace,
                      workspace_bytes, &alias_free);
  if (st != AR_OK) return st;
  ar_split_cfg_t cfg;
  if (user_cfg) {
    if (!alias_free) return AR_ERR_ALIAS;
    cfg = *user_cfg;
  } else {
    int cu = 0;
    st = query_cu_count(&cu);
    if (st != AR_OK) return st;
    if (!alias_free || !plan_split(W, M, H, dtype, cu, &cfg))
      return run_norm(inputs, W, M, H, dtype, residual, gamma, eps, residual_out, norm_out,
                      stream, nullptr);
  }
  const arfh::SplitLaunch c{cfg.threads_per_block, cfg.vecs_per_thread, cfg.segments,
                            cfg.max_polls};
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (dtype) {
    case AR_DTYPE_FP32:
      e = arfh::launch_norm_split_f32(inputs, W, residual, gamma, eps, residual_out, norm_out, M,
                                      H, workspace, c, s);
      break;
    case AR_DTYPE_FP16:
      e = arfh::launch_norm_split_f16(inputs, W, residual, gamma, eps, residual_out, norm_out, M,
                                      H, workspace, c, s);
      break;
    default:
      e = arfh::launch_norm_split_bf16(inputs, W, residual, gamma, eps, residual_out, norm_out,
                                       M, H, workspace, c, s);
      break;
  }
  return e == hipSuccess ? AR_OK : AR_ERR_LAUNCH;
}

int run_workspace_clear(void* workspace, int64_t bytes, void* stream) {
  if (!workspace || bytes < 0) return AR_ERR_INVALID_ARG;
  if (!aligned16(workspace)) return AR_ERR_MISALIGNED;
  if (bytes % kSplitSlotBytes != 0) return AR_ERR_INVALID_ARG;
  if (bytes == 0) return AR_OK;
  int cu = 0;
  const int st = query_cu_count(&cu);
  if (st != AR_OK) return st;
  uint64_t* p = static_cast<uint64_t*>(workspace);
  int64_t n = bytes / kSplitSlotBytes;
  void* args[] = {&p, &n};
  const int grid = static_cast<int>(std::max<int64_t>(1, std::min(ceil_div(n, 256), int64_t(cu) * 4)));
  const hipError_t e =
      hipLaunchKernel(reinterpret_cast<const void*>(&arf::ar_fill_zero_kernel<uint64_t>),
                      dim3(grid), dim3(256), args, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? AR_OK : AR_ERR_LAUNCH;
}

// ---- the split form without a caller workspace -----------------------------------------------------
//
// For callers that cannot allocate: the split kernel's exchange slots live in this file-scope
// device array, one copy per GPU (zero-filled when the code object is loaded, and cleared again
// by the first call on each device).  In host code `scratch` names a host-side stand-in, never
// the device memory: the device address comes from hipGetSymbolAddress, once per device with that
// device current, and only that address is passed to kernels.
constexpr int64_t kScratchWords = int64_t(AR_NOALLOC_MAX_ROWS) * arf::kSplitSlots;
static __device__ __align__(256) uint64_t scratch[kScratchWords];

std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// This device's copy of `scratch` (set up on the first call on the device: the symbol's device
// address, then a zero fill on `stream`).  AR_ERR_DEVICE if the device or symbol query fails.
int device_scratch(hipStream_t stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return AR_ERR_DEVICE;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
      void* q = nullptr;
      if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return AR_ERR_DEVICE;
      const int st = run_workspace_clear(q, kScratchWords * kSplitSlotBytes, stream);
      if (st != AR_OK) return st;
      g_scratch_ptr[dev].store(q, std::memory_order_release);
      p = q;
    }
  }
  *out = p;
  return AR_OK;
}

int run_norm_noalloc(const void* const* inputs, int W, int64_t M, int64_t H, int dtype,
                     const void* residual, const float* gamma, float eps, void* residual_out,
                     void* norm_out, void* stream) {
  int st = check_shape(AR_PATTERN_AR_RESIDUAL_RMSNORM, W, M, H, dtype);
  if (st != AR_OK) return st;
  if (M > AR_NOALLOC_MAX_ROWS) return AR_ERR_UNSUPPORTED;  // more rows than `scratch` holds
  st = validate_norm(inputs, W, M, H, dtype, residual, gamma, eps, residual_out, norm_out);
  if (st != AR_OK) return st;
  if (M == 0) return AR_OK;
  void* ws = nullptr;
  st = device_scratch(static_cast<hipStream_t>(stream), &ws);
  if (st != AR_OK) return st;
  return run_norm_ws(inputs, W, M, H, dtype, residual, gamma, eps, residual_out, norm_out, ws,
                     kScratchWords * kSplitSlotBytes, stream, nullptr);
}

// ---- two-kernel (unfused) path and the stand-alone RMSNorm ----------------------------------------
//
// The route for kARResidualRMSNorm shapes the fused kernel does not take (rows that are not whole
// 16-byte vectors, or wider than a block keeps in registers): the pages' policy layer sends such
// calls to an unfused fallback (tokenspeed pull request, Body / Routing; vLLM pull request,
// Scope).  Kernel 1 is the flat sum kernel with the residual as one more addend, so residual_out
// is bit-identical to the fused kernel's; kernel 2 is RMSNorm of residual_out.

bool norm_fits_fused(int64_t H, int dtype) {
  return check_shape(AR_PATTERN_AR_RESIDUAL_RMSNORM, 1, 0, H, dtype) == AR_OK;
}

int validate_rmsnorm(const void* x, int64_t M, int64_t H, int dtype, const float* gamma,
                     float eps, const void* y) {
  int st = check_shape(AR_PATTERN_ALLREDUCE, 1, M, H, dtype);
  if (st != AR_OK) return st;
  if (!std::isfinite(eps) || eps < 0.0f) return AR_ERR_INVALID_ARG;
  if (M == 0) return AR_OK;
  if (!x || !gamma || !y) return AR_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(gamma) || !aligned16(y)) return AR_ERR_MISALIGNED;
  const int64_t bytes = M * H * elem_size(dtype);
  const Range yr = range_of(y, bytes);
  if (bad_alias_with_input(yr, range_of(x, bytes))) return AR_ERR_ALIAS;
  if (overlap(yr, range_of(gamma, H * int64_t(sizeof(float))))) return AR_ERR_ALIAS;
  return AR_OK;
}

// Launches RMSNorm of x into y (validated arguments, M > 0): the fused kernel in norm-only mode
// when rows fit it, else the row kernel for rows of any width.
int launch_rmsnorm(const void* x, int64_t M, int64_t H, int dtype, const float* gamma, float eps,
                   void* y, hipStream_t s) {
  int cu = 0;
  const int st = query_cu_count(&cu);
  if (st != AR_OK) return st;
  hipError_t e;
  if (norm_fits_fused(H, dtype)) {
    ar_launch_cfg_t cfg;
    plan_norm(1, M, H, dtype, cu, &cfg);
    switch (dtype) {
      case AR_DTYPE_FP32: e = arfh::launch_rmsnorm_f32(x, gamma, eps, y, M, H, cfg, s); break;
      case AR_DTYPE_FP16: e = arfh::launch_rmsnorm_f16(x, gamma, eps, y, M, H, cfg, s); break;
      default: e = arfh::launch_rmsnorm_bf16(x, gamma, eps, y, M, H, cfg, s); break;
    }
  } else {
    // One block per row, grid stride over rows (at most 8 blocks per CU).  A row spans at most
    // H / vec + 2 aligned vectors, and the kernel's slots start at the 128-byte line that holds
    // the row's first element, up to 7 vectors earlier: H / vec + 9 slots.  The fewest vectors
    // per thread (1, 2, 4 or 8) that keep the block at <= 512 threads (640 for 4, 1024 for 8)
    // hold the row in registers, else two passes.  (Rows of 2049-2560 vectors: 4 vectors over
    // up to 640 threads ran 8-39 % faster than 8 over 320 at M = 768 ... 4096, bf16
    // H = 16386 / 20002, fp16 18434, binary32 9002; bf16 H = 16386, M = 2048: 41.1 -> 30.0 us.)
    const int vec = kVecBytes / elem_size(dtype);
    const int64_t nv = H / vec + 9;
    int vpt = 0;
    int64_t threads = 1024;
    for (int k = 1; k <= 8; k *= 2) {
      if (ceil_div(nv, k) <= (k == 8 ? 1024 : k == 4 ? 640 : 512)) {
        vpt = k;
        threads = round_up(ceil_div(nv, k), 64);
        break;
      }
    }
    // At most one row per CU: the fewest vectors per thread that one block of up to 1024
    // threads allows (more waves for the one row each CU holds); two rows per CU: the same
    // up to 704 threads.  Eight or more rows per CU: small blocks, at most 192 threads (128
    // with 8 vectors per thread), so more rows are in flight on each CU.  Interleaved A/B over
    // 17 odd widths, 16-bit and binary32: M <= 256 up to 23 % faster, never slower by more than
    // 0.5 % (bf16 H = 16386, M = 8: 7.43 -> 5.69 us); M = 384 / 512 5-18 % (the 1024 bound
    // there ranged from -17 to +5 %); M = 2048 / 4096 5-29 % (bf16 H = 7170, M = 2048:
    // 16.0 -> 13.5 us; fp16 H = 5122: 13.9 -> 9.8 us).  From 3 to 7 rows per CU the 704 bound
    // lost up to 39 %, so those keep the shape above.
    int64_t cap = 0;  // 0: keep the shape above; -1: the small-block bound
    if (M <= int64_t(cu)) {
      cap = 1024;
    } else if (M <= int64_t(cu) * 2) {
      cap = 704;
    } else if (M >= int64_t(cu) * 8) {
      cap = -1;
    }
    if (cap != 0) {
      for (int k = 1; k <= 8; k *= 2) {
        const int64_t tk = round_up(ceil_div(nv, k), 64);
        if (tk <= (cap > 0 ? cap : (k == 8 ? 128 : 192))) {
          vpt = k;
          threads = tk;
          break;
        }
      }
    }
    const int t = static_cast<int>(threads);
    const int grid = cap_grid(std::min<int64_t>(M, int64_t(cu) * 8));
    switch (dtype) {
      case AR_DTYPE_FP32:
        e = arfh::launch_rmsnorm_rows_f32(x, gamma, eps, y, M, H, grid, t, vpt, s);
        break;
      case AR_DTYPE_FP16:
        e = arfh::launch_rmsnorm_rows_f16(x, gamma, eps, y, M, H, grid, t, vpt, s);
        break;
      default: e = arfh::launch_rmsnorm_rows_bf16(x, gamma, eps, y, M, H, grid, t, vpt, s); break;
    }
  }
  return e == hipSuccess ? AR_OK : AR_ERR_LAUNCH;
}

int run_rmsnorm(const void* x, int64_t M, int64_t H, int dtype, const float* gamma, float eps,
                void* y, void* stream) {
  const int st = validate_rmsnorm(x, M, H, dtype, gamma, eps, y);
  if (st != AR_OK || M == 0) return st;
  return launch_rmsnorm(x, M, H, dtype, gamma, eps, y, static_cast<hipStream_t>(stream));
}

int run_unfused(const void* const* inputs, int W, int64_t M, int64_t H, int dtype,
                const void* residual, const float* gamma, float eps, void* residual_out,
                void* norm_out, void* stream) {
  int st = validate_norm(inputs, W, M, H, dtype, residual, gamma, eps, residual_out, norm_out,
                         AR_PATTERN_ALLREDUCE);
  if (st != AR_OK || M == 0) return st;
  int cu = 0;
  st = query_cu_count(&cu);
  if (st != AR_OK) return st;
  ar_launch_cfg_t cfg;
  plan_sum(W + 1, M * H, dtype, cu, &cfg, 2);
  const int64_t vec = kVecBytes / elem_size(dtype);
  const int64_t nvec = M * H / vec;
  const int tail = static_cast<int>(M * H - nvec * vec);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (dtype) {
    case AR_DTYPE_FP32:
      e = arfh::launch_sum_residual_f32(inputs, W, residual, residual_out, nvec, tail, cfg, s);
      break;
    case AR_DTYPE_FP16:
      e = arfh::launch_sum_residual_f16(inputs, W, residual, residual_out, nvec, tail, cfg, s);
      break;
    default:
      e = arfh::launch_sum_residual_bf16(inputs, W, residual, residual_out, nvec, tail, cfg, s);
      break;
  }
  if (e != hipSuccess) return AR_ERR_LAUNCH;
  return launch_rmsnorm(residual_out, M, H, dtype, gamma, eps, norm_out, s);
}

// ---- two-shot share ------------------------------------------------------------------------------

void row_slice(int W, int64_t M, int rank, int64_t* begin, int64_t* count) {
  // floor(rank * M / W) without overflow for any M < 2^62 / 64.
  const int64_t b = (M / W) * rank + ((M % W) * rank) / W;
  const int64_t e = (M / W) * (rank + 1) + ((M % W) * (rank + 1)) / W;
  *begin = b;
  *count = e - b;
}

int run_gather(const void* const* slices, int W, int64_t M, int64_t H, int dtype, void* out,
               void* stream) {
  // The sum pattern's shape rules plus whole 16-byte vectors per row (every slice then starts
  // on a vector boundary of `out`).
  int st = check_shape(AR_PATTERN_ALLREDUCE, W, M, H, dtype);
  if (st != AR_OK) return st;
  if (H % (kVecBytes / elem_size(dtype)) != 0) return AR_ERR_UNSUPPORTED;
  if (M == 0) return AR_OK;
  if (!slices || !out) return AR_ERR_INVALID_ARG;
  if (!aligned16(out)) return AR_ERR_MISALIGNED;
  const int64_t es = elem_size(dtype);
  const int64_t V = H / (kVecBytes / es);
  arf::GatherArgs a;
  uint64_t skip = 0;
  const Range o = range_of(out, M * H * es);
  for (int j = 0; j < W; ++j) {
    int64_t b, c;
    row_slice(W, M, j, &b, &c);
    a.vec_begin[j] = b * V;
    a.src[j] = static_cast<const u32x4*>(slices[j]);
    if (c == 0) {
      skip |= uint64_t(1) << j;  // empty slice: pointer may be null
      continue;
    }
    if (!slices[j]) return AR_ERR_INVALID_ARG;
    if (!aligned16(slices[j])) return AR_ERR_MISALIGNED;
    const Range in = range_of(slices[j], c * H * es);
    const Range place = range_of(static_cast<const char*>(out) + b * H * es, c * H * es);
    if (in.lo == place.lo) {
      skip |= uint64_t(1) << j;  // already in place
    } else if (overlap(in, o)) {
      return AR_ERR_ALIAS;
    }
  }
  a.vec_begin[W] = M * V;
  int64_t max_vecs = 0;
  for (int j = 0; j < W; ++j) max_vecs = std::max(max_vecs, a.vec_begin[j + 1] - a.vec_begin[j]);
  int cu = 0;
  st = query_cu_count(&cu);
  if (st != AR_OK) return st;
  // Measured on MI355X: large gathers (>= 4096 vectors per CU) run best as single-wave blocks
  // covering every vector once; smaller ones as 256-thread blocks, at most 16 per CU over all
  // slices.  Non-temporal stores won at every size.
  const bool large = M * V >= int64_t(cu) * 4096;
  // (Two or four vectors per thread measured 3-7 % slower at every size.)
  const int threads = large ? 64 : 256;
  const int64_t cap = large ? int64_t(INT_MAX) : std::max<int64_t>(1, int64_t(cu) * 16 / W);
  const int gx = static_cast<int>(std::min(ceil_div(max_vecs, threads), cap));
  hipStream_t s = static_cast<hipStream_t>(stream);
  u32x4* dst = static_cast<u32x4*>(out);
  void* args[] = {&a, &dst, &skip};
  const void* fn = reinterpret_cast<const void*>(&arf::ar_gather_kernel<true, 1>);
  const hipError_t e = hipLaunchKernel(fn, dim3(std::max(gx, 1), W), dim3(threads), args, 0, s);
  return e == hipSuccess ? AR_OK : AR_ERR_LAUNCH;
}

// ---- Lamport-style exchange ----------------------------------------------------------------------

constexpr uint32_t kDefaultSpinLimit = 1u << 16;
// Vectors per thread of the Lamport fused consumer: 8 for W <= 4, 4 beyond (its polled batch
// spills at 8), so rows of up to 1024 lanes x that many 16-byte vectors.
int lamport_max_vpt(int W) { return W <= 4 ? 8 : 4; }

constexpr int kLamportBuffers = AR_LAMPORT_BUFFERS;

int check_lamport_shape(int pattern, int W, int64_t M, int64_t H, int dtype) {
  int st = check_shape(AR_PATTERN_ALLREDUCE, W, M, H, dtype);
  if (st != AR_OK) return st;
  // The receive buffer is 3 x W slots: keep 3 W M H es <= 2^60 as well.
  if (M > 0 && H > ((int64_t(1) << 60) / (int64_t(kLamportBuffers) * W * elem_size(dtype))) / M)
    return AR_ERR_UNSUPPORTED;
  const int64_t vec = kVecBytes / elem_size(dtype);
  if (H % vec != 0) return AR_ERR_UNSUPPORTED;
  if (pattern == AR_PATTERN_AR_RESIDUAL_RMSNORM && H / vec > 1024 * lamport_max_vpt(W))
    return AR_ERR_UNSUPPORTED;
  return AR_OK;
}

int lamport_grid(int64_t items, int cu) {
  return static_cast<int>(std::max<int64_t>(1, std::min(ceil_div(items, 256), int64_t(cu) * 16)));
}

int run_lamport_arm(void* rbuf, int W, int64_t M, int64_t H, int dtype, void* stream) {
  int st = check_lamport_shape(AR_PATTERN_ALLREDUCE, W, M, H, dtype);
  if (st != AR_OK) return st;
  if (M == 0) return AR_OK;
  if (!rbuf) return AR_ERR_INVALID_ARG;
  if (!aligned16(rbuf)) return AR_ERR_MISALIGNED;
  int cu = 0;
  st = query_cu_count(&cu);
  if (st != AR_OK) return st;
  u32x4* buf = static_cast<u32x4*>(rbuf);
  int64_t nvec = int64_t(kLamportBuffers) * W * M * H * elem_size(dtype) / kVecBytes;
  void* args[] = {&buf, &nvec};
  const hipError_t e =
      hipLaunchKernel(reinterpret_cast<const void*>(&arf::ar_lamport_arm_kernel<u32x4>),
                      dim3(lamport_grid(nvec, cu)), dim3(256), args, 0,
                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? AR_OK : AR_ERR_LAUNCH;
}

// Byte offset of slot `rank` of buffer `buffer` (0, 1 or 2).
int64_t lamport_slot(int buffer, int W, int rank, int64_t slot_bytes) {
  return (int64_t(buffer) * W + rank) * slot_bytes;
}
// The buffer round `round` (>= 0) uses, and the next one (computed without round + 1, which
// overflows at the largest round).
int lamport_buffer(int64_t round) { return static_cast<int>(round % kLamportBuffers); }
int lamport_next_buffer(int64_t round) { return (lamport_buffer(round) + 1) % kLamportBuffers; }

int run_lamport_push(const void* partial, int rank, void* rbuf, int W, int64_t M, int64_t H,
                     int dtype, int64_t round, void* stream) {
  int st = check_lamport_shape(AR_PATTERN_ALLREDUCE, W, M, H, dtype);
  if (st != AR_OK) return st;
  if (rank < 0 || rank >= W || round < 0) return AR_ERR_INVALID_ARG;
  if (M == 0) return AR_OK;
  if (!partial || !rbuf) return AR_ERR_INVALID_ARG;
  if (!aligned16(partial) || !aligned16(rbuf)) return AR_ERR_MISALIGNED;
  const int64_t slot_bytes = M * H * elem_size(dtype);
  if (overlap(range_of(partial, slot_bytes), range_of(rbuf, slot_bytes * W * kLamportBuffers)))
    return AR_ERR_ALIAS;
  int cu = 0;
  st = query_cu_count(&cu);
  if (st != AR_OK) return st;
  // This round's slot, and the same rank's slot of the next buffer (used two rounds ago), which
  // this push empties.
  char* base = static_cast<char*>(rbuf);
  void* slot = base + lamport_slot(lamport_buffer(round), W, rank, slot_bytes);
  void* next = base + lamport_slot(lamport_next_buffer(round), W, rank, slot_bytes);
  const int64_t nvec = slot_bytes / kVecBytes;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // One vector per thread and a grid that covers the slot: the kernel runs no loop.
  (void)cu;
  const int grid = cap_grid(ceil_div(nvec, 256));
  hipError_t e;
  switch (dtype) {
    case AR_DTYPE_FP32: e = arfh::launch_lamport_push_f32(partial, slot, next, nvec, grid, s); break;
    case AR_DTYPE_FP16: e = arfh::launch_lamport_push_f16(partial, slot, next, nvec, grid, s); break;
    default: e = arfh::launch_lamport_push_bf16(partial, slot, next, nvec, grid, s); break;
  }
  return e == hipSuccess ? AR_OK : AR_ERR_LAUNCH;
}

// Pointer checks shared by the two Lamport consumers: nothing the kernel writes may overlap the
// receive buffer or the status word except as allowed for the plain entry points.
int check_lamport_buffers(void* rbuf, int W, int64_t M, int64_t H, int dtype, const int* status) {
  if (!rbuf || !status) return AR_ERR_INVALID_ARG;
  if (!aligned16(rbuf)) return AR_ERR_MISALIGNED;
  if ((reinterpret_cast<uintptr_t>(status) & 3u) != 0) return AR_ERR_MISALIGNED;
  const int64_t slot_bytes = M * H * elem_size(dtype);
  if (overlap(range_of(status, 4), range_of(rbuf, slot_bytes * W * kLamportBuffers)))
    return AR_ERR_ALIAS;
  return AR_OK;
}

int run_lamport_sum(void* rbuf, int W, int64_t M, int64_t H, int dtype, int64_t round, void* out,
                    int* status, uint32_t spin_limit, void* stream) {
  int st = check_lamport_shape(AR_PATTERN_ALLREDUCE, W, M, H, dtype);
  if (st != AR_OK) return st;
  if (round < 0) return AR_ERR_INVALID_ARG;
  if (M == 0) return AR_OK;
  if (!out) return AR_ERR_INVALID_ARG;
  st = check_lamport_buffers(rbuf, W, M, H, dtype, status);
  if (st != AR_OK) return st;
  if (!aligned16(out)) return AR_ERR_MISALIGNED;
  const int64_t bytes = M * H * elem_size(dtype);
  const Range o = range_of(out, bytes);
  if (overlap(o, range_of(rbuf, bytes * W * kLamportBuffers)) || overlap(o, range_of(status, 4)))
    return AR_ERR_ALIAS;
  void* buf = static_cast<char*>(rbuf) + lamport_slot(lamport_buffer(round), W, 0, bytes);
  int cu = 0;
  st = query_cu_count(&cu);
  if (st != AR_OK) return st;
  ar_launch_cfg_t cfg;
  plan_sum(W, M * H, dtype, cu, &cfg, 0);
  cfg.vecs_per_thread = 1;  // the Lamport consumer is instantiated for one vector per thread
  const int64_t nvec = M * H / (kVecBytes / elem_size(dtype));
  cfg.grid = cap_grid(ceil_div(nvec, cfg.threads_per_block));
  cfg.nt_store = 1;
  // Polled batches of two ranks instead of eight from 1024 vectors per CU on (W = 4 ... 16).
  // Consumer alone over rotated receive buffers, H = 7168, three interleaved rounds: W = 8 bf16
  // M = 512 / 1024 / 2048 8.8 / 4.9 / 1.5 % faster (M = 4096 even); W = 4 2-3.5 %, W = 16
  // 1.2-10 % (bf16 and binary32, M = 512 and 2048).  With fewer vectors per CU it ranged from
  // 9 % faster to 18 % slower (W = 16 bf16 M = 128).
  cfg.ranks_per_batch = (W >= 4 && W <= 16 && nvec >= int64_t(cu) * 1024) ? 2 : 0;
  arf::LamportSource src{status, spin_limit ? spin_limit : kDefaultSpinLimit};
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (dtype) {
    case AR_DTYPE_FP32: e = arfh::launch_lamport_sum_f32(buf, W, M, H, out, cfg, src, s); break;
    case AR_DTYPE_FP16: e = arfh::launch_lamport_sum_f16(buf, W, M, H, out, cfg, src, s); break;
    default: e = arfh::launch_lamport_sum_bf16(buf, W, M, H, out, cfg, src, s); break;
  }
  return e == hipSuccess ? AR_OK : AR_ERR_LAUNCH;
}

int run_lamport_norm(void* rbuf, int W, int64_t M, int64_t H, int dtype, int64_t round,
                     const void* residual, const float* gamma, float eps, void* residual_out,
                     void* norm_out, int* status, uint32_t spin_limit, void* stream) {
  int st = check_lamport_shape(AR_PATTERN_AR_RESIDUAL_RMSNORM, W, M, H, dtype);
  if (st != AR_OK) return st;
  if (!std::isfinite(eps) || eps < 0.0f || round < 0) return AR_ERR_INVALID_ARG;
  if (M == 0) return AR_OK;
  if (!residual || !gamma || !residual_out || !norm_out) return AR_ERR_INVALID_ARG;
  st = check_lamport_buffers(rbuf, W, M, H, dtype, status);
  if (st != AR_OK) return st;
  if (!aligned16(residual) || !aligned16(gamma) || !aligned16(residual_out) ||
      !aligned16(norm_out))
    return AR_ERR_MISALIGNED;
  const int64_t bytes = M * H * elem_size(dtype);
  const Range rb = range_of(rbuf, bytes * W * kLamportBuffers);
  const Range ro = range_of(residual_out, bytes);
  const Range no = range_of(norm_out, bytes);
  const Range res = range_of(residual, bytes);
  const Range g = range_of(gamma, H * int64_t(sizeof(float)));
  const Range stw = range_of(status, 4);
  if (overlap(ro, no) || overlap(ro, g) || overlap(no, g)) return AR_ERR_ALIAS;
  if (overlap(ro, rb) || overlap(no, rb) || overlap(res, rb) || overlap(g, rb)) return AR_ERR_ALIAS;
  if (overlap(ro, stw) || overlap(no, stw)) return AR_ERR_ALIAS;
  if (bad_alias_with_input(ro, res) || bad_alias_with_input(no, res)) return AR_ERR_ALIAS;
  int cu = 0;
  st = query_cu_count(&cu);
  if (st != AR_OK) return st;
  ar_launch_cfg_t cfg;
  plan_norm(W, M, H, dtype, cu, &cfg);
  const int vmax = lamport_max_vpt(W);
  if (cfg.vecs_per_thread > vmax) {
    const int64_t V = H / (kVecBytes / elem_size(dtype));
    cfg.vecs_per_thread = vmax;
    cfg.lanes_per_row = static_cast<int>(round_up(ceil_div(V, vmax), 64));
    cfg.threads_per_block = cfg.lanes_per_row;
    cfg.rows_per_block = 1;
    cfg.grid = cap_grid(M);
  }
  // Few rows (a quarter of the CUs or fewer hold one): each row's block is latency-bound, and a
  // polled batch holds half the stream source's loads, so two vectors per thread cost W = 8 two
  // round trips where one vector costs one.  Take the fewest vectors per thread (1 or 2) that
  // one block of up to 1024 threads allows: H = 7168 bf16, M = 1 ... 48: 5-28 % faster at
  // W = 2 ... 64 (W = 8: 7.8 -> 6.2 us at M = 1); two instead of four at H = 16384: 13-35 %
  // (W = 64, M = 2: 119 -> 78 us); binary32 W = 8 M = 32: 16.5 -> 12.4 us.  From 128 rows on
  // the planned shape stays ahead (W = 8: 12.8 against 15.6 us).
  if (M * 4 <= cu && cfg.rows_per_block == 1) {
    const int64_t V = H / (kVecBytes / elem_size(dtype));
    const int v = round_up(V, 64) <= 1024 ? 1 : 2;
    const int64_t lanes = round_up(ceil_div(V, v), 64);
    if (v < cfg.vecs_per_thread && lanes <= 1024) {
      cfg.vecs_per_thread = v;
      cfg.lanes_per_row = static_cast<int>(lanes);
      cfg.threads_per_block = static_cast<int>(lanes);
      cfg.grid = cap_grid(M);
    }
  }
  cfg.nt_store = 1;
  // Polled batches of a quarter of the stream source's loads instead of half beyond one row per
  // CU (W = 4 ... 16; two ranks at 2 vectors per thread, one at 4).  Consumer alone over rotated
  // receive buffers, H = 7168, three interleaved rounds: W = 8 bf16 M = 512 / 1024 / 2048 / 4096
  // 3.7 / 2.5 / 3.7 / 1.8 % faster; W = 4 and 16, bf16 and binary32, M = 512 and 2048: 1-5.5 %.
  // At M = 128 it was even to 10 % slower.
  cfg.ranks_per_batch = 0;
  if (M > cu && cfg.rows_per_block == 1 && W >= 4 && W <= 16) {
    if (cfg.vecs_per_thread == 2) cfg.ranks_per_batch = 2;
    if (cfg.vecs_per_thread == 4) cfg.ranks_per_batch = 1;
  }
  arf::LamportSource src{status, spin_limit ? spin_limit : kDefaultSpinLimit};
  void* buf = static_cast<char*>(rbuf) + lamport_slot(lamport_buffer(round), W, 0, bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (dtype) {
    case AR_DTYPE_FP32:
      e = arfh::launch_lamport_norm_f32(buf, W, residual, gamma, eps, residual_out, norm_out, M,
                                        H, cfg, src, s);
      break;
    case AR_DTYPE_FP16:
      e = arfh::launch_lamport_norm_f16(buf, W, residual, gamma, eps, residual_out, norm_out, M,
                                        H, cfg, src, s);
      break;
    default:
      e = arfh::launch_lamport_norm_bf16(buf, W, residual, gamma, eps, residual_out, norm_out,
                                         M, H, cfg, src, s);
      break;
  }
  return e == hipSuccess ? AR_OK : AR_ERR_LAUNCH;
}

}  // namespace

// ---- C ABI ----------------------------------------------------------------------------------------

extern "C" {

int ar_sum(const void* const* inputs, int W, int64_t M, int64_t H, int dtype, void* out,
           void* stream) {
  return run_sum(inputs, W, M, H, dtype, out, stream, nullptr);
}

int ar_sum_with_config(const void* const* inputs, int W, int64_t M, int64_t H, int dtype,
                       void* out, void* stream, const ar_launch_cfg_t* cfg) {
  if (!cfg) return AR_ERR_INVALID_ARG;
  return run_sum(inputs, W, M, H, dtype, out, stream, cfg);
}

int ar_residual_rmsnorm(const void* const* inputs, int W, int64_t M, int64_t H, int dtype,
                        const void* residual, const float* gamma, float eps, void* residual_out,
                        void* norm_out, void* stream) {
  return run_norm(inputs, W, M, H, dtype, residual, gamma, eps, residual_out, norm_out, stream,
                  nullptr);
}

int ar_residual_rmsnorm_with_config(const void* const* inputs, int W, int64_t M, int64_t H,
                                    int dtype, const void* residual, const float* gamma,
                                    float eps, void* residual_out, void* norm_out, void* stream,
                                    const ar_launch_cfg_t* cfg) {
  if (!cfg) return AR_ERR_INVALID_ARG;
  return run_norm(inputs, W, M, H, dtype, residual, gamma, eps, residual_out, norm_out, stream,
                  cfg);
}

int64_t ar_split_workspace_bytes(int64_t M) {
  if (M < 0 || M > (int64_t(1) << 40)) return -1;
  return split_workspace_bytes(M);
}

int ar_workspace_clear(void* workspace, int64_t workspace_bytes, void* stream) {
  return run_workspace_clear(workspace, workspace_bytes, stream);
}

int ar_split_config(int W, int64_t M, int64_t H, int dtype, int cu_count, ar_split_cfg_t* cfg) {
  if (!cfg) return AR_ERR_INVALID_ARG;
  const int st = check_shape(AR_PATTERN_AR_RESIDUAL_RMSNORM, W, M, H, dtype);
  if (st != AR_OK) return st;
  int cu = cu_count;
  if (cu <= 0) {
    const int q = query_cu_count(&cu);
    if (q != AR_OK) return q;
  }
  if (!plan_split(W, M, H, dtype, cu, cfg) || check_split_cfg(M, H, dtype, cfg) != AR_OK) {
    *cfg = ar_split_cfg_t{0, 0, 0, 0};
  }
  return AR_OK;
}

int ar_residual_rmsnorm_ws(const void* const* inputs, int W, int64_t M, int64_t H, int dtype,
                           const void* residual, const float* gamma, float eps,
                           void* residual_out, void* norm_out, void* workspace,
                           int64_t workspace_bytes, void* stream) {
  return run_norm_ws(inputs, W, M, H, dtype, residual, gamma, eps, residual_out, norm_out,
                     workspace, workspace_bytes, stream, nullptr);
}

int ar_residual_rmsnorm_noalloc(const void* const* inputs, int W, int64_t M, int64_t H,
                                int dtype, const void* residual, const float* gamma, float eps,
                                void* residual_out, void* norm_out, void* stream) {
  return run_norm_noalloc(inputs, W, M, H, dtype, residual, gamma, eps, residual_out, norm_out,
                          stream);
}

int ar_residual_rmsnorm_split_with_config(const void* const* inputs, int W, int64_t M, int64_t H,
                                          int dtype, const void* residual, const float* gamma,
                                          float eps, void* residual_out, void* norm_out,
                                          void* workspace, int64_t workspace_bytes, void* stream,
                                          const ar_split_cfg_t* cfg) {
  if (!cfg) return AR_ERR_INVALID_ARG;
  return run_norm_ws(inputs, W, M, H, dtype, residual, gamma, eps, residual_out, norm_out,
                     workspace, workspace_bytes, stream, cfg);
}

int ar_rmsnorm(const void* x, int64_t M, int64_t H, int dtype, const float* gamma, float eps,
               void* y, void* stream) {
  return run_rmsnorm(x, M, H, dtype, gamma, eps, y, stream);
}

int ar_residual_rmsnorm_unfused(const void* const* inputs, int W, int64_t M, int64_t H,
                                int dtype, const void* residual, const float* gamma, float eps,
                                void* residual_out, void* norm_out, void* stream) {
  return run_unfused(inputs, W, M, H, dtype, residual, gamma, eps, residual_out, norm_out, stream);
}

int ar_supports(int pattern, int W, int64_t M, int64_t H, int dtype) {
  return check_shape(pattern, W, M, H, dtype);
}

int ar_launch_config(int pattern, int W, int64_t M, int64_t H, int dtype, int cu_count,
                     ar_launch_cfg_t* cfg) {
  if (!cfg) return AR_ERR_INVALID_ARG;
  const int st = check_shape(pattern, W, M, H, dtype);
  if (st != AR_OK) return st;
  int cu = cu_count;
  if (cu <= 0) {
    const int q = query_cu_count(&cu);
    if (q != AR_OK) return q;
  }
  if (pattern == AR_PATTERN_ALLREDUCE) {
    plan_sum(W, M * H, dtype, cu, cfg);
  } else {
    plan_norm(W, M, H, dtype, cu, cfg);
  }
  return AR_OK;
}

int ar_row_partition(int W, int64_t M, int rank, int64_t* row_begin, int64_t* row_count) {
  if (!row_begin || !row_count || W < 1 || W > AR_MAX_W || M < 0 || rank < 0 || rank >= W)
    return AR_ERR_INVALID_ARG;
  row_slice(W, M, rank, row_begin, row_count);
  return AR_OK;
}

int ar_all_gather(const void* const* slices, int W, int64_t M, int64_t H, int dtype, void* out,
                  void* stream) {
  return run_gather(slices, W, M, H, dtype, out, stream);
}

int ar_lamport_arm(void* rbuf, int W, int64_t M, int64_t H, int dtype, void* stream) {
  return run_lamport_arm(rbuf, W, M, H, dtype, stream);
}

int ar_lamport_push(const void* partial, int rank, void* rbuf, int W, int64_t M, int64_t H,
                    int dtype, int64_t round, void* stream) {
  return run_lamport_push(partial, rank, rbuf, W, M, H, dtype, round, stream);
}

int ar_lamport_sum(void* rbuf, int W, int64_t M, int64_t H, int dtype, int64_t round, void* out,
                   int* status, uint32_t spin_limit, void* stream) {
  return run_lamport_sum(rbuf, W, M, H, dtype, round, out, status, spin_limit, stream);
}

int ar_lamport_residual_rmsnorm(void* rbuf, int W, int64_t M, int64_t H, int dtype, int64_t round,
                                const void* residual, const float* gamma, float eps,
                                void* residual_out, void* norm_out, int* status,
                                uint32_t spin_limit, void* stream) {
  return run_lamport_norm(rbuf, W, M, H, dtype, round, residual, gamma, eps, residual_out,
                          norm_out, status, spin_limit, stream);
}

int ar_policy_default(int W, ar_policy_t* policy) {
  if (!policy || W < 1) return AR_ERR_INVALID_ARG;
  // Two-shot beats one-shot once S (1 - 2/W) / link_bw > t_exchange (see the header).
  constexpr double kLinkBytesPerSec = 153e9;
  constexpr double kExchangeSec = 5e-6;
  policy->min_tokens = 32;
  policy->two_shot_min_bytes =
      W <= 2 ? INT64_MAX
             : static_cast<int64_t>(kExchangeSec * kLinkBytesPerSec / (1.0 - 2.0 / W));
  policy->max_payload_bytes = 0;
  return AR_OK;
}

int ar_route(int pattern, int W, int64_t M, int64_t H, int dtype, const ar_policy_t* policy,
             int* route) {
  if (!policy || !route) return AR_ERR_INVALID_ARG;
  if (pattern != AR_PATTERN_ALLREDUCE && pattern != AR_PATTERN_AR_RESIDUAL_RMSNORM)
    return AR_ERR_INVALID_ARG;
  if (policy->min_tokens < 0 || policy->two_shot_min_bytes < 0 || policy->max_payload_bytes < 0)
    return AR_ERR_INVALID_ARG;
  const bool fused_ok = check_shape(pattern, W, M, H, dtype) == AR_OK;
  // A norm row the fused kernel does not take still has the two-kernel path.
  const bool unfused_ok = !fused_ok && pattern == AR_PATTERN_AR_RESIDUAL_RMSNORM &&
                          check_shape(AR_PATTERN_ALLREDUCE, W, M, H, dtype) == AR_OK;
  if (!fused_ok && !unfused_ok) {
    *route = AR_ROUTE_FALLBACK;
    return AR_OK;
  }
  const int64_t payload = M * H * elem_size(dtype);
  if (policy->max_payload_bytes > 0 && payload > policy->max_payload_bytes) {
    *route = AR_ROUTE_FALLBACK;
  } else if (unfused_ok) {
    *route = AR_ROUTE_UNFUSED;
  } else if (M < policy->min_tokens || payload < policy->two_shot_min_bytes) {
    *route = AR_ROUTE_ONE_SHOT;
  } else {
    // Two-shot needs whole vectors per row for the gather; otherwise stay on one-shot.
    const bool gatherable = H % (kVecBytes / elem_size(dtype)) == 0;
    *route = gatherable ? AR_ROUTE_TWO_SHOT : AR_ROUTE_ONE_SHOT;
  }
  return AR_OK;
}

int ar_allreduce_routed(int pattern, const void* const* inputs, int W, int64_t M, int64_t H,
                        int dtype, const void* residual, const float* gamma, float eps, void* out,
                        void* norm_out, int rank, const ar_policy_t* policy, int* route,
                        void* stream) {
  if (!route) return AR_ERR_INVALID_ARG;
  int r = AR_ROUTE_FALLBACK;
  const int st = ar_route(pattern, W, M, H, dtype, policy, &r);
  if (st != AR_OK) return st;
  if (rank < 0 || rank >= W) return AR_ERR_INVALID_ARG;
  *route = r;
  const bool norm = pattern == AR_PATTERN_AR_RESIDUAL_RMSNORM;
  switch (r) {
    case AR_ROUTE_ONE_SHOT:
      return norm ? run_norm(inputs, W, M, H, dtype, residual, gamma, eps, out, norm_out, stream,
                             nullptr)
                  : run_sum(inputs, W, M, H, dtype, out, stream, nullptr);
    case AR_ROUTE_UNFUSED:
      return run_unfused(inputs, W, M, H, dtype, residual, gamma, eps, out, norm_out, stream);
    case AR_ROUTE_TWO_SHOT: {
      // This rank's reduce-scatter share: the same reduction on its row slice, in place in the
      // outputs.  The route guarantees whole 16-byte vectors per row, so every slice stays
      // aligned.
      if (!inputs) return AR_ERR_INVALID_ARG;
      int64_t b = 0, c = 0;
      row_slice(W, M, rank, &b, &c);
      const int64_t off = b * H * elem_size(dtype);
      auto shift = [off](const void* p) -> const void* {
        return p ? static_cast<const char*>(p) + off : nullptr;
      };
      auto shift_out = [off](void* p) -> void* { return p ? static_cast<char*>(p) + off : nullptr; };
      const void* rows[AR_MAX_W];
      for (int j = 0; j < W; ++j) {
        if (!inputs[j]) return AR_ERR_INVALID_ARG;
        rows[j] = shift(inputs[j]);
      }
      if (!out || (norm && (!residual || !norm_out))) return AR_ERR_INVALID_ARG;
      return norm ? run_norm(rows, W, c, H, dtype, shift(residual), gamma, eps, shift_out(out),
                             shift_out(norm_out), stream, nullptr)
                  : run_sum(rows, W, c, H, dtype, shift_out(out), stream, nullptr);
    }
    default:
      return AR_ERR_UNSUPPORTED;  // the caller's own collective takes this call
  }
}

const char* ar_status_string(int status) {
  switch (status) {
    case AR_OK: return "ok";
    case AR_ERR_INVALID_ARG: return "invalid argument";
    case AR_ERR_UNSUPPORTED: return "unsupported shape or world size";
    case AR_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case AR_ERR_ALIAS: return "output buffers overlap";
    case AR_ERR_LAUNCH: return "kernel launch failed";
    case AR_ERR_DEVICE: return "no usable HIP device";
    default: return "unknown status";
  }
}

int ar_device_cu_count(int* cu_count) {
  if (!cu_count) return AR_ERR_INVALID_ARG;
  return query_cu_count(cu_count);
}

}  // extern "C"
