// ar_dispatch.hpp -- launch helpers shared by the per-element-type translation units.
//
// Each inst_<type>.hip instantiates the kernels of one element type and exports the
// launch_<pattern>_<type> functions declared at the bottom; ar_fused.hip (validation, the
// launch-shape heuristic and the C ABI) calls them.  Splitting the ~300 kernel instantiations
// over several translation units lets the build compile them in parallel.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "ar_fused.h"
#include "ar_kernels.hpp"

namespace arfh {

using arf::F16;
using arf::F32;
using arf::Bf16;
using arf::RankPtrs;
using arf::u32x4;
using arf::f32x4;

template <int W>
RankPtrs<W> pack_ptrs(const void* const* inputs) {
  RankPtrs<W> p;
  for (int r = 0; r < W; ++r) p.p[r] = static_cast<const u32x4*>(inputs[r]);
  return p;
}

template <class T, int W, int U>
hipError_t launch_sum_u(const void* const* inputs, void* out, int64_t nvec, int tail,
                        const ar_launch_cfg_t& c, hipStream_t s) {
  RankPtrs<W> p = pack_ptrs<W>(inputs);
  u32x4* o = static_cast<u32x4*>(out);
  arf::StreamSource src;
  void* args[] = {&p, &o, &nvec, &tail, &src};
  const void* fn = c.nt_store ? reinterpret_cast<const void*>(&arf::ar_sum_kernel<T, W, U, true>)
                              : reinterpret_cast<const void*>(&arf::ar_sum_kernel<T, W, U, false>);
  return hipLaunchKernel(fn, dim3(c.grid), dim3(c.threads_per_block), args, 0, s);
}

template <class T, int W>
hipError_t launch_sum_w(const void* const* inputs, void* out, int64_t nvec, int tail,
                        const ar_launch_cfg_t& c, hipStream_t s) {
  switch (c.vecs_per_thread) {
    case 1: return launch_sum_u<T, W, 1>(inputs, out, nvec, tail, c, s);
    case 2: return launch_sum_u<T, W, 2>(inputs, out, nvec, tail, c, s);
    default: return launch_sum_u<T, W, 4>(inputs, out, nvec, tail, c, s);
  }
}

template <class T>
inline hipError_t launch_sum_t(const void* const* inputs, int W, void* out, int64_t nvec, int tail,
                        const ar_launch_cfg_t& c, hipStream_t s) {
  switch (W) {
    case 1: return launch_sum_w<T, 1>(inputs, out, nvec, tail, c, s);
    case 2: return launch_sum_w<T, 2>(inputs, out, nvec, tail, c, s);
    case 4: return launch_sum_w<T, 4>(inputs, out, nvec, tail, c, s);
    case 8: return launch_sum_w<T, 8>(inputs, out, nvec, tail, c, s);
    case 16: return launch_sum_w<T, 16>(inputs, out, nvec, tail, c, s);
    case 32: return launch_sum_w<T, 32>(inputs, out, nvec, tail, c, s);
    default: return launch_sum_w<T, 64>(inputs, out, nvec, tail, c, s);
  }
}

template <class T, int W, int VPT>
hipError_t launch_norm_v(const void* const* inputs, const void* residual, const float* gamma,
                         float eps, void* residual_out, void* norm_out, int64_t M, int64_t H,
                         const ar_launch_cfg_t& c, hipStream_t s) {
  RankPtrs<W> p = pack_ptrs<W>(inputs);
  const u32x4* res = static_cast<const u32x4*>(residual);
  const f32x4* gam = reinterpret_cast<const f32x4*>(gamma);
  u32x4* ro = static_cast<u32x4*>(residual_out);
  u32x4* no = static_cast<u32x4*>(norm_out);
  int V = static_cast<int>(H / T::kVec);
  int L = c.lanes_per_row;
  int R = c.rows_per_block;
  float count_h = static_cast<float>(H);  // exact: H <= 2^16
  arf::StreamSource src;
  void* args[] = {&p, &res, &gam, &ro, &no, &M, &V, &L, &R, &eps, &count_h, &src};
  const void* fn =
      c.nt_store ? reinterpret_cast<const void*>(&arf::ar_norm_kernel<T, W, VPT, true>)
                 : reinterpret_cast<const void*>(&arf::ar_norm_kernel<T, W, VPT, false>);
  // Fixed rank batches: instantiated for the shapes the launch checks allow.
  if constexpr (arf::rank_batch_instantiated(W, VPT, 1)) {
    if (c.ranks_per_batch == 1)
      fn = reinterpret_cast<const void*>(
          &arf::ar_norm_kernel<T, W, VPT, true, arf::StreamSource, false, 1>);
  }
  if constexpr (arf::rank_batch_instantiated(W, VPT, 2)) {
    if (c.ranks_per_batch == 2)
      fn = reinterpret_cast<const void*>(
          &arf::ar_norm_kernel<T, W, VPT, true, arf::StreamSource, false, 2>);
  }
  if constexpr (arf::rank_batch_instantiated(W, VPT, 4)) {
    if (c.ranks_per_batch == 4)
      fn = reinterpret_cast<const void*>(
          &arf::ar_norm_kernel<T, W, VPT, true, arf::StreamSource, false, 4>);
  }
  return hipLaunchKernel(fn, dim3(c.grid), dim3(c.threads_per_block), args, 0, s);
}

template <class T, int W>
hipError_t launch_norm_w(const void* const* inputs, const void* residual, const float* gamma,
                         float eps, void* residual_out, void* norm_out, int64_t M, int64_t H,
                         const ar_launch_cfg_t& c, hipStream_t s) {
  switch (c.vecs_per_thread) {
    case 1:
      return launch_norm_v<T, W, 1>(inputs, residual, gamma, eps, residual_out, norm_out, M, H,
                                    c, s);
    case 2:
      return launch_norm_v<T, W, 2>(inputs, residual, gamma, eps, residual_out, norm_out, M, H,
                                    c, s);
    case 4:
      return launch_norm_v<T, W, 4>(inputs, residual, gamma, eps, residual_out, norm_out, M, H,
                                    c, s);
    default:
      return launch_norm_v<T, W, 8>(inputs, residual, gamma, eps, residual_out, norm_out, M, H,
                                    c, s);
  }
}

template <class T>
inline hipError_t launch_norm_t(const void* const* inputs, int W, const void* residual,
                         const float* gamma, float eps, void* residual_out, void* norm_out,
                         int64_t M, int64_t H, const ar_launch_cfg_t& c, hipStream_t s) {
#define AR_NORM_W(w)                                                                        \
  case w:                                                                                   \
    return launch_norm_w<T, w>(inputs, residual, gamma, eps, residual_out, norm_out, M, H, \
                               c, s);
  switch (W) {
    AR_NORM_W(1)
    AR_NORM_W(2)
    AR_NORM_W(4)
    AR_NORM_W(8)
    AR_NORM_W(16)
    AR_NORM_W(32)
    default:
      return launch_norm_w<T, 64>(inputs, residual, gamma, eps, residual_out, norm_out, M, H, c,
                                  s);
  }
#undef AR_NORM_W
}


// ---- Lamport-style exchange (one receive buffer of W slots, slot r at rbuf + r * slot_vecs) -------

template <int W>
RankPtrs<W> slot_ptrs(const void* rbuf, int64_t slot_vecs) {
  RankPtrs<W> p;
  for (int r = 0; r < W; ++r) p.p[r] = static_cast<const u32x4*>(rbuf) + r * slot_vecs;
  return p;
}

template <class T, int W>
hipError_t launch_lamport_sum_w(void* rbuf, int64_t slot_vecs, void* out, int64_t nvec,
                                const ar_launch_cfg_t& c, arf::LamportSource src, hipStream_t s) {
  RankPtrs<W> p = slot_ptrs<W>(rbuf, slot_vecs);
  u32x4* o = static_cast<u32x4*>(out);
  int tail = 0;
  // Polled batches of two ranks (ranks_per_batch = 2): built for W = 4 ... 16.
  arf::LamportSourceT<2> src2{src.status, src.spin_limit};
  void* args[] = {&p, &o, &nvec, &tail, &src};
  void* args2[] = {&p, &o, &nvec, &tail, &src2};
  if constexpr (W >= 4 && W <= 16) {
    if (c.ranks_per_batch == 2)
      return hipLaunchKernel(
          reinterpret_cast<const void*>(&arf::ar_sum_kernel<T, W, 1, true, arf::LamportSourceT<2>>),
          dim3(c.grid), dim3(c.threads_per_block), args2, 0, s);
  }
  const void* fn =
      reinterpret_cast<const void*>(&arf::ar_sum_kernel<T, W, 1, true, arf::LamportSource>);
  return hipLaunchKernel(fn, dim3(c.grid), dim3(c.threads_per_block), args, 0, s);
}

template <class T, int W, int VPT>
hipError_t launch_lamport_norm_v(void* rbuf, int64_t slot_vecs, const void* residual,
                                 const float* gamma, float eps, void* residual_out,
                                 void* norm_out, int64_t M, int64_t H, const ar_launch_cfg_t& c,
                                 arf::LamportSource src, hipStream_t s) {
  RankPtrs<W> p = slot_ptrs<W>(rbuf, slot_vecs);
  const u32x4* res = static_cast<const u32x4*>(residual);
  const f32x4* gam = reinterpret_cast<const f32x4*>(gamma);
  u32x4* ro = static_cast<u32x4*>(residual_out);
  u32x4* no = static_cast<u32x4*>(norm_out);
  int V = static_cast<int>(H / T::kVec);
  int L = c.lanes_per_row;
  int R = c.rows_per_block;
  float count_h = static_cast<float>(H);
  // Polled batches of two ranks at 2 vectors per thread, one at 4 (ranks_per_batch): built for
  // W = 4 ... 16.
  arf::LamportSourceT<1> src1{src.status, src.spin_limit};
  arf::LamportSourceT<2> src2{src.status, src.spin_limit};
  void* args[] = {&p, &res, &gam, &ro, &no, &M, &V, &L, &R, &eps, &count_h, &src};
  void* args1[] = {&p, &res, &gam, &ro, &no, &M, &V, &L, &R, &eps, &count_h, &src1};
  void* args2[] = {&p, &res, &gam, &ro, &no, &M, &V, &L, &R, &eps, &count_h, &src2};
  if constexpr (W >= 4 && W <= 16 && VPT == 2) {
    if (c.ranks_per_batch == 2)
      return hipLaunchKernel(reinterpret_cast<const void*>(
                                 &arf::ar_norm_kernel<T, W, VPT, true, arf::LamportSourceT<2>>),
                             dim3(c.grid), dim3(c.threads_per_block), args2, 0, s);
  }
  if constexpr (W >= 4 && W <= 16 && VPT == 4) {
    if (c.ranks_per_batch == 1)
      return hipLaunchKernel(reinterpret_cast<const void*>(
                                 &arf::ar_norm_kernel<T, W, VPT, true, arf::LamportSourceT<1>>),
                             dim3(c.grid), dim3(c.threads_per_block), args1, 0, s);
  }
  const void* fn = reinterpret_cast<const void*>(
      &arf::ar_norm_kernel<T, W, VPT, true, arf::LamportSource>);
  return hipLaunchKernel(fn, dim3(c.grid), dim3(c.threads_per_block), args, 0, s);
}

#define AR_W_SWITCH(W, CALL)        \
  switch (W) {                      \
    case 1: return CALL(1);         \
    case 2: return CALL(2);         \
    case 4: return CALL(4);         \
    case 8: return CALL(8);         \
    case 16: return CALL(16);       \
    case 32: return CALL(32);       \
    default: return CALL(64);       \
  }

template <class T>
inline hipError_t launch_lamport_sum_t(void* rbuf, int W, int64_t M, int64_t H, void* out,
                                       const ar_launch_cfg_t& c, arf::LamportSource src,
                                       hipStream_t s) {
  const int64_t nvec = M * H / T::kVec;
#define AR_CALL(w) launch_lamport_sum_w<T, w>(rbuf, nvec, out, nvec, c, src, s)
  AR_W_SWITCH(W, AR_CALL)
#undef AR_CALL
}

template <class T>
inline hipError_t launch_lamport_norm_t(void* rbuf, int W, const void* residual,
                                        const float* gamma, float eps, void* residual_out,
                                        void* norm_out, int64_t M, int64_t H,
                                        const ar_launch_cfg_t& c, arf::LamportSource src,
                                        hipStream_t s) {
  const int64_t nvec = M * H / T::kVec;
#define AR_CALL_V(v)                                                                       \
  if (c.vecs_per_thread == v) {                                                            \
    switch (W) {                                                                           \
      case 1: return launch_lamport_norm_v<T, 1, v>(rbuf, nvec, residual, gamma, eps,      \
                                                    residual_out, norm_out, M, H, c, src, s); \
      case 2: return launch_lamport_norm_v<T, 2, v>(rbuf, nvec, residual, gamma, eps,      \
                                                    residual_out, norm_out, M, H, c, src, s); \
      case 4: return launch_lamport_norm_v<T, 4, v>(rbuf, nvec, residual, gamma, eps,      \
                                                    residual_out, norm_out, M, H, c, src, s); \
      case 8: return launch_lamport_norm_v<T, 8, v>(rbuf, nvec, residual, gamma, eps,      \
                                                    residual_out, norm_out, M, H, c, src, s); \
      case 16: return launch_lamport_norm_v<T, 16, v>(rbuf, nvec, residual, gamma, eps,    \
                                                      residual_out, norm_out, M, H, c, src, s); \
      case 32: return launch_lamport_norm_v<T, 32, v>(rbuf, nvec, residual, gamma, eps,    \
                                                      residual_out, norm_out, M, H, c, src, s); \
      default: return launch_lamport_norm_v<T, 64, v>(rbuf, nvec, residual, gamma, eps,    \
                                                      residual_out, norm_out, M, H, c, src, s); \
    }                                                                                      \
  }
  AR_CALL_V(1)
  AR_CALL_V(2)
  AR_CALL_V(4)
#undef AR_CALL_V
  // 8 vectors per thread only for W <= 4 (beyond, the polled batch spills); the host rejects
  // rows that would need them.
  switch (W) {
    case 1: return launch_lamport_norm_v<T, 1, 8>(rbuf, nvec, residual, gamma, eps, residual_out,
                                                  norm_out, M, H, c, src, s);
    case 2: return launch_lamport_norm_v<T, 2, 8>(rbuf, nvec, residual, gamma, eps, residual_out,
                                                  norm_out, M, H, c, src, s);
    case 4: return launch_lamport_norm_v<T, 4, 8>(rbuf, nvec, residual, gamma, eps, residual_out,
                                                  norm_out, M, H, c, src, s);
    default: return hipErrorInvalidConfiguration;
  }
}

template <class T>
inline hipError_t launch_lamport_push_t(const void* partial, void* slot, void* next, int64_t nvec,
                                        int grid, hipStream_t s) {
  const u32x4* src = static_cast<const u32x4*>(partial);
  u32x4* dst = static_cast<u32x4*>(slot);
  u32x4* nxt = static_cast<u32x4*>(next);
  void* args[] = {&src, &dst, &nxt, &nvec};
  return hipLaunchKernel(reinterpret_cast<const void*>(&arf::ar_lamport_push_kernel<T>),
                         dim3(grid), dim3(256), args, 0, s);
}

// ---- two-kernel (unfused) path -------------------------------------------------------------------

template <class T, int W, int U>
hipError_t launch_sum_residual_u(const void* const* inputs, const void* residual, void* out,
                                 int64_t nvec, int tail, const ar_launch_cfg_t& c, hipStream_t s) {
  RankPtrs<W> p = pack_ptrs<W>(inputs);
  u32x4* o = static_cast<u32x4*>(out);
  arf::ResidualSource src{static_cast<const u32x4*>(residual)};
  void* args[] = {&p, &o, &nvec, &tail, &src};
  const void* fn =
      c.nt_store
          ? reinterpret_cast<const void*>(&arf::ar_sum_kernel<T, W, U, true, arf::ResidualSource>)
          : reinterpret_cast<const void*>(&arf::ar_sum_kernel<T, W, U, false, arf::ResidualSource>);
  return hipLaunchKernel(fn, dim3(c.grid), dim3(c.threads_per_block), args, 0, s);
}

// vecs_per_thread 1 or 2 (the values plan_sum picks).
template <class T>
inline hipError_t launch_sum_residual_t(const void* const* inputs, int W, const void* residual,
                                        void* out, int64_t nvec, int tail,
                                        const ar_launch_cfg_t& c, hipStream_t s) {
  if (c.vecs_per_thread == 1) {
#define AR_CALL(w) launch_sum_residual_u<T, w, 1>(inputs, residual, out, nvec, tail, c, s)
    AR_W_SWITCH(W, AR_CALL)
#undef AR_CALL
  }
#define AR_CALL(w) launch_sum_residual_u<T, w, 2>(inputs, residual, out, nvec, tail, c, s)
  AR_W_SWITCH(W, AR_CALL)
#undef AR_CALL
}

template <class T, int VPT>
hipError_t launch_rmsnorm_v(const void* x, const float* gamma, float eps, void* y, int64_t M,
                            int64_t H, const ar_launch_cfg_t& c, hipStream_t s) {
  RankPtrs<1> p;
  p.p[0] = static_cast<const u32x4*>(x);
  const u32x4* res = nullptr;
  const f32x4* gam = reinterpret_cast<const f32x4*>(gamma);
  u32x4* ro = nullptr;
  u32x4* no = static_cast<u32x4*>(y);
  int V = static_cast<int>(H / T::kVec);
  int L = c.lanes_per_row;
  int R = c.rows_per_block;
  float count_h = static_cast<float>(H);  // exact: H <= 2^16
  arf::StreamSource src;
  void* args[] = {&p, &res, &gam, &ro, &no, &M, &V, &L, &R, &eps, &count_h, &src};
  const void* fn =
      c.nt_store
          ? reinterpret_cast<const void*>(
                &arf::ar_norm_kernel<T, 1, VPT, true, arf::StreamSource, true>)
          : reinterpret_cast<const void*>(
                &arf::ar_norm_kernel<T, 1, VPT, false, arf::StreamSource, true>);
  return hipLaunchKernel(fn, dim3(c.grid), dim3(c.threads_per_block), args, 0, s);
}

template <class T>
inline hipError_t launch_rmsnorm_t(const void* x, const float* gamma, float eps, void* y,
                                   int64_t M, int64_t H, const ar_launch_cfg_t& c, hipStream_t s) {
  switch (c.vecs_per_thread) {
    case 1: return launch_rmsnorm_v<T, 1>(x, gamma, eps, y, M, H, c, s);
    case 2: return launch_rmsnorm_v<T, 2>(x, gamma, eps, y, M, H, c, s);
    case 4: return launch_rmsnorm_v<T, 4>(x, gamma, eps, y, M, H, c, s);
    default: return launch_rmsnorm_v<T, 8>(x, gamma, eps, y, M, H, c, s);
  }
}

// vecs_per_thread: 1, 2, 4 or 8 (row values kept in registers) or 0 (two passes over memory).
// The register forms need H / vec + 9 slots per block (a row's vectors from the start of its
// first 128-byte line); a smaller shape is refused rather than run.
template <class T>
inline hipError_t launch_rmsnorm_rows_t(const void* x, const float* gamma, float eps, void* y,
                                        int64_t M, int64_t H, int grid, int threads,
                                        int vecs_per_thread, hipStream_t s) {
  if (vecs_per_thread > 0 && int64_t(vecs_per_thread) * threads < H / T::kVec + 9)
    return hipErrorInvalidValue;
  float count_h = static_cast<float>(H);
  void* args[] = {&x, &gamma, &y, &M, &H, &eps, &count_h};
  const void* fn;
  switch (vecs_per_thread) {
    case 1: fn = reinterpret_cast<const void*>(&arf::ar_rmsnorm_rows_kernel<T, 1>); break;
    case 2: fn = reinterpret_cast<const void*>(&arf::ar_rmsnorm_rows_kernel<T, 2>); break;
    case 4: fn = reinterpret_cast<const void*>(&arf::ar_rmsnorm_rows_kernel<T, 4>); break;
    case 8: fn = reinterpret_cast<const void*>(&arf::ar_rmsnorm_rows_kernel<T, 8>); break;
    default: fn = reinterpret_cast<const void*>(&arf::ar_rmsnorm_rows_kernel<T, 0>); break;
  }
  return hipLaunchKernel(fn, dim3(grid), dim3(threads), args, 0, s);
}

// ---- kARResidualRMSNorm with a row split over several blocks ------------------------------------

struct SplitLaunch {
  int threads, vpt, segments;
  uint32_t max_polls;
};

template <class T, int W, int VPT>
hipError_t launch_norm_split_v(const void* const* inputs, const void* residual,
                               const float* gamma, float eps, void* residual_out, void* norm_out,
                               int64_t M, int64_t H, void* workspace, const SplitLaunch& c,
                               hipStream_t s) {
  RankPtrs<W> p = pack_ptrs<W>(inputs);
  const u32x4* res = static_cast<const u32x4*>(residual);
  const f32x4* gam = reinterpret_cast<const f32x4*>(gamma);
  u32x4* ro = static_cast<u32x4*>(residual_out);
  u32x4* no = static_cast<u32x4*>(norm_out);
  int V = static_cast<int>(H / T::kVec);
  int S = c.segments;
  float count_h = static_cast<float>(H);  // exact: H <= 2^16
  uint64_t* slots = static_cast<uint64_t*>(workspace);
  uint32_t polls = c.max_polls;
  int rows = static_cast<int>(M);
  void* args[] = {&p, &res, &gam, &ro, &no, &V, &S, &eps, &count_h, &slots, &polls, &rows};
  const void* fn = reinterpret_cast<const void*>(&arf::ar_norm_split_kernel<T, W, VPT, true>);
  const arf::SplitDims g = arf::split_dims(M, S);
  return hipLaunchKernel(fn, dim3(static_cast<unsigned>(g.x), static_cast<unsigned>(g.y)),
                         dim3(c.threads), args, 0, s);
}

// vecs_per_thread 1 or 2.
template <class T>
inline hipError_t launch_norm_split_t(const void* const* inputs, int W, const void* residual,
                                      const float* gamma, float eps, void* residual_out,
                                      void* norm_out, int64_t M, int64_t H, void* workspace,
                                      const SplitLaunch& c, hipStream_t s) {
  if (c.vpt == 1) {
#define AR_CALL(w)                                                                            \
  launch_norm_split_v<T, w, 1>(inputs, residual, gamma, eps, residual_out, norm_out, M, H, \
                               workspace, c, s)
    AR_W_SWITCH(W, AR_CALL)
#undef AR_CALL
  }
#define AR_CALL(w)                                                                            \
  launch_norm_split_v<T, w, 2>(inputs, residual, gamma, eps, residual_out, norm_out, M, H, \
                               workspace, c, s)
  AR_W_SWITCH(W, AR_CALL)
#undef AR_CALL
}

// ---- per-element-type entry points (defined in inst_bf16.hip, inst_f16.hip, inst_f32.hip) ----

#define AR_DECLARE_LAUNCHERS(suffix)                                                         \
  hipError_t launch_sum_##suffix(const void* const* inputs, int W, void* out, int64_t nvec,  \
                                 int tail, const ar_launch_cfg_t& c, hipStream_t s);         \
  hipError_t launch_norm_##suffix(const void* const* inputs, int W, const void* residual,    \
                                  const float* gamma, float eps, void* residual_out,         \
                                  void* norm_out, int64_t M, int64_t H,                      \
                                  const ar_launch_cfg_t& c, hipStream_t s);                  \
  hipError_t launch_lamport_sum_##suffix(void* rbuf, int W, int64_t M, int64_t H, void* out,  \
                                         const ar_launch_cfg_t& c, arf::LamportSource src,    \
                                         hipStream_t s);                                      \
  hipError_t launch_lamport_norm_##suffix(void* rbuf, int W, const void* residual,            \
                                          const float* gamma, float eps, void* residual_out,  \
                                          void* norm_out, int64_t M, int64_t H,               \
                                          const ar_launch_cfg_t& c, arf::LamportSource src,   \
                                          hipStream_t s);                                     \
  hipError_t launch_lamport_push_##suffix(const void* partial, void* slot, void* next,        \
                                          int64_t nvec, int grid, hipStream_t s);             \
  hipError_t launch_sum_residual_##suffix(const void* const* inputs, int W,                   \
                                          const void* residual, void* out, int64_t nvec,      \
                                          int tail, const ar_launch_cfg_t& c, hipStream_t s); \
  hipError_t launch_rmsnorm_##suffix(const void* x, const float* gamma, float eps, void* y,   \
                                     int64_t M, int64_t H, const ar_launch_cfg_t& c,          \
                                     hipStream_t s);                                          \
  hipError_t launch_rmsnorm_rows_##suffix(const void* x, const float* gamma, float eps,       \
                                          void* y, int64_t M, int64_t H, int grid,            \
                                          int threads, int vecs_per_thread, hipStream_t s);\
  hipError_t launch_norm_split_##suffix(const void* const* inputs, int W, const void* residual, \
                                        const float* gamma, float eps, void* residual_out,    \
                                        void* norm_out, int64_t M, int64_t H,                 \
                                        void* workspace, const SplitLaunch& c, hipStream_t s);
AR_DECLARE_LAUNCHERS(bf16)
AR_DECLARE_LAUNCHERS(f16)
AR_DECLARE_LAUNCHERS(f32)
#undef AR_DECLARE_LAUNCHERS

}  // namespace arfh
