// ar_kernels.hpp -- gfx950 device code of the fused all-reduce-sum (+ residual + RMSNorm) core.
//
// The two core kernels, templated on the element type T, the number of partials W, the number
// of 16-byte vectors per thread and the store policy:
//
//   ar_sum_kernel   kAllReduce.  A flat walk over the [M, H] tensors viewed as 16-byte vectors.
//                   Each thread issues the W loads of its vectors before it starts the binary32
//                   chain, so a wave keeps W x U x 1 KiB of reads in flight.
//   ar_norm_kernel  kARResidualRMSNorm.  `lanes_per_row` consecutive threads own one row; each
//                   holds its vectors' rounded residual_out values in registers between the sum
//                   and the norm, so every byte is read once and written once.  The per-row sum
//                   of squares is reduced with DPP lane moves and a swizzle inside a wave, then
//                   across waves through LDS with one barrier per row (LDS slots alternate
//                   between two banks so consecutive rows need no second barrier).
//
// Around them: ar_norm_split_kernel (few rows: a row split over several blocks that exchange
// partial sums of squares through a caller workspace), ar_rmsnorm_rows_kernel (RMSNorm of rows
// of any width, the two-kernel path's second step), the Lamport-style exchange (a polling input
// source plus producer and arming kernels) and ar_gather_kernel (the two-shot all-gather share).
//
// The fusion patterns are the ones named in the tokenspeed pull request "perf(comm): route
// generic MNNVL AR patterns to upstream flashinfer" (Summary).  The peers' buffers are passed as
// a by-value pointer array in the kernel arguments (they land in scalar registers), the AMD
// counterpart of the GPU-side pointer array in the flashinfer pull request "Optimizations for
// TRTLLM MNNVL Allreduce" (Description).
//
// Arithmetic contract (identical for every launch shape):
//  * rank sum: binary32, rank order 0..W-1, one round-to-nearest-even per add, started from
//    -0.0f (-0 + x == x for every x, so this equals seeding with x_0 and keeps -0 sums);
//  * residual: added after the W partials; one rounding to T (v_cvt_pk_bf16_f32 /
//    v_cvt_pk_f16_f32 round to nearest even in the default mode);
//  * norm: computed from the rounded residual_out; no flush of subnormals.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

// Phase hooks: the benchmark's timing probe defines AR_PHASE(phase, value, tensor) before it
// includes this header, to record when a block reaches each phase of a kernel (after `value` is
// computed; `tensor` identifies the call); in the library they expand to nothing.
#ifndef AR_PHASE
#define AR_PHASE(phase, value, tensor) ((void)0)
#endif

namespace arf {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// Four floats at a 4-byte-aligned address (a 16-byte load the hardware splits as needed).
typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxThreads = 1024;
constexpr int kMaxWavesPerBlock = kMaxThreads / 64;

template <int W>
struct RankPtrs {
  const u32x4* p[W];
};

// ---- element types: a 16-byte vector <-> binary32 lanes ------------------------------------

struct Bf16 {
  static constexpr int kVec = 8;
  __device__ static inline void widen(u32x4 v, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
  }
  __device__ static inline u32x4 narrow(const float (&f)[8]) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2 h = __builtin_convertvector(f32x2{f[2 * i], f[2 * i + 1]}, bf16x2);
      r[i] = __builtin_bit_cast(uint32_t, h);
    }
    return r;
  }
  __device__ static inline float widen1(const void* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
  }
  __device__ static inline void store1(void* p, int64_t i, float x) {
    static_cast<__bf16*>(p)[i] = static_cast<__bf16>(x);
  }
};

struct F16 {
  static constexpr int kVec = 8;
  __device__ static inline void widen(u32x4 v, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // The word goes through a scalar first: this compiler folds __builtin_bit_cast of a
      // vector subscript (v[i]) to element 0 for every i.
      const uint32_t word = v[i];
      const f32x2 w = __builtin_convertvector(__builtin_bit_cast(f16x2, word), f32x2);
      f[2 * i] = w.x;
      f[2 * i + 1] = w.y;
    }
  }
  __device__ static inline u32x4 narrow(const float (&f)[8]) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x2 h = __builtin_convertvector(f32x2{f[2 * i], f[2 * i + 1]}, f16x2);
      r[i] = __builtin_bit_cast(uint32_t, h);
    }
    return r;
  }
  __device__ static inline float widen1(const void* p, int64_t i) {
    return static_cast<float>(static_cast<const _Float16*>(p)[i]);
  }
  __device__ static inline void store1(void* p, int64_t i, float x) {
    static_cast<_Float16*>(p)[i] = static_cast<_Float16>(x);
  }
};

struct F32 {
  static constexpr int kVec = 4;
  __device__ static inline void widen(u32x4 v, float (&f)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
  __device__ static inline u32x4 narrow(const float (&f)[4]) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(f[i]);
    return r;
  }
  __device__ static inline float widen1(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  __device__ static inline void store1(void* p, int64_t i, float x) {
    static_cast<float*>(p)[i] = x;
  }
};

// ---- memory access ----------------------------------------------------------------------------
//
// Every input byte is read exactly once, so loads are non-temporal (global_load_dwordx4 ... nt):
// they do not displace useful lines from L2 and the Infinity Cache.  Stores are non-temporal
// when the launch shape asks for it (large outputs that no cache would keep anyway).

__device__ inline u32x4 load_stream(const u32x4* p) { return __builtin_nontemporal_load(p); }

// The policy is a template parameter: with a run-time flag the compiler merges the two stores
// and drops the non-temporal hint.
template <bool kNt>
__device__ inline void store_vec(u32x4* p, u32x4 v) {
  if constexpr (kNt) {
    __builtin_nontemporal_store(v, p);
  } else {
    *p = v;
  }
}

// ---- wave-level reduction -------------------------------------------------------------------

// x + (x of the lane selected by a DPP control).  All four controls used here stay inside a
// 16-lane DPP row, so every source lane exists.
template <int kCtrl>
__device__ inline float dpp_add(float x) {
  const int y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false);
  return x + __int_as_float(y);
}

// Sum of x over aligned groups of min(seg, 64) lanes; seg is a power of two <= 64 or a multiple
// of 64, uniform across the wave, and every lane of the wave is active.  Each step adds a lane
// to its partner under an involution, so every lane of a group ends with the same value.
__device__ inline float segment_sum(float x, int seg) {
  if (seg >= 2) x = dpp_add<0xB1>(x);    // quad_perm [1,0,3,2]: lane ^ 1
  if (seg >= 4) x = dpp_add<0x4E>(x);    // quad_perm [2,3,0,1]: lane ^ 2
  if (seg >= 8) x = dpp_add<0x141>(x);   // row_half_mirror: lane i <-> 7 - i within 8
  if (seg >= 16) x = dpp_add<0x140>(x);  // row_mirror: lane i <-> 15 - i within 16
  if (seg >= 32) {                       // ds_swizzle bit mode, xor 0x10: lane ^ 16 within 32
    x = x + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
  }
  if (seg >= 64) {                       // halves of the wave, lane 0 + lane 32, uniform
    x = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0)) +
        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  }
  return x;
}

// ---- rows outside the binary32 range of the sum of squares ----------------------------------------
//
// The norm kernels reduce a row's sum of squares ss in binary32.  That meets the norm bar while
// x = ss / H + eps is a normal number of at least 2^-100: a square that lost bits to the subnormal
// range is off by at most 2^-150, so all of them together move x by at most 2^-134 (H <= 2^16),
// a relative 2^-34.  Two kinds of finite rows fall outside: rows whose squares overflow (ss = inf
// from an RMS of about 1.8e19 / sqrt(H), or one element above 1.8e19, on: rstd would be 0 and
// norm_out 0), and rows with eps below 2^-100 whose squares underflow (eps = 0 and elements below
// about 2^-63: rstd would be inf or far off).  Such a row is normalised again from the same
// rounded values scaled by an exact power of two 2^k: the sum of squares S' of v 2^k is S 4^k,
// so rstd' = 1 / sqrt(S' / H + eps 4^k) = rstd 2^-k, and y = (v 2^k * rstd') * gamma.
//   * overflow (x = inf): k = -73.  Every |v| <= 2^128 becomes <= 2^55, so even 2^16 squares
//     sum to at most 2^126; S >= 2^128, so S' >= 2^-18 and the squares that now underflow
//     (|v| < 2^-1.5) change S' by at most 2^-133 in all, a relative 2^-115.
//   * underflow (x < 2^-100, so eps < 2^-100 and every |v| < 2^-42): k = 90.  Every square
//     of v 2^90 lies in [2^-118, 2^96] (from the smallest subnormal up), normal and exact to
//     binary32 rounding, and eps 4^90 < 2^80.
// The scaling is exact (ldexp) except where v 2^k underflows, and then y is tiny anyway.  The
// test costs one compare per row and a branch the row's threads take together; rows inside the
// range compute exactly what they computed without it.  A row holding an infinity also lands
// here (x = inf) and gets the binary32 path's results (rstd' = 0); NaN compares false.
__device__ inline bool outside_binary32_range(float x) {
  return x < 0x1p-100f || x > 3.40282347e38f;
}

// The scale exponent k for a row outside the range (see above).
__device__ inline int wide_scale(float x) { return x > 1.0f ? -73 : 90; }

// v 2^k, exact unless the result is subnormal.
__device__ inline float scaled(float v, int k) { return __builtin_amdgcn_ldexpf(v, k); }

// One element normalised with rstd = m 2^E: (v 2^E * m) * gamma.  For E = 0 (every row inside
// the range) this is (v * rstd) * gamma, bit for bit.
__device__ inline float norm_elem_scaled(float v, float m, int E, float g) {
  return (scaled(v, E) * m) * g;
}

// rstd' of a row whose values were scaled by 2^k, from their sum of squares S'.
__device__ inline float rstd_of_scaled(float S, int k, float count_h, float eps) {
  return rsqrtf(S / count_h + scaled(eps, 2 * k));
}

// ---- addressing ---------------------------------------------------------------------------------
//
// Every address is a wave-uniform base (a tensor pointer plus a uniform element offset, computed
// in scalar registers) plus a 32-bit per-lane byte offset.  That maps onto the scalar-base +
// vector-offset form of the global memory instructions: one VGPR per vector slot, shared by all
// W + 1 input tensors and both outputs, instead of a 64-bit VGPR pair per load.

template <class P>
__device__ inline P* at(P* base, uint32_t byte_off) {
  using C = typename std::conditional<std::is_const<P>::value, const char, char>::type;
  return reinterpret_cast<P*>(reinterpret_cast<C*>(base) + byte_off);
}

// ---- rank batching ----------------------------------------------------------------------------
//
// A thread sums W ranks for each of its N vectors.  Left alone, the compiler hoists every load
// of the unrolled rank loop to the top, which for large W x N needs more than the 128 VGPRs a
// 1024-thread block allows and spills to scratch.  The rank loop is therefore cut into batches
// of kBatch ranks (at most 8 or 16 16-byte loads in flight per thread) with a compiler fence
// after each batch: an empty asm statement that reads and writes every accumulator and clobbers
// memory, so the batch's adds stay before it and the next batch's loads stay after it.  It
// emits no instruction.  Latency is hidden by the other waves on the SIMD.

// Reads a kernel's arguments in one round: up to 16 rank pointers and the given scalars are made
// operands of one empty asm at the kernel's start.  Left alone, the compiler read the arguments
// in two or three dependent rounds (each a scalar-cache miss) before the first load, which a
// decode-size call pays in full.  With more than 16 ranks the pointers are left to the walk over
// groups of 16 (forced reads there put full waits inside the sum kernel's fp16 rank batches), and
// only the scalars are read at once.
#define AR_RANK_PTR(i) "s"(in.p[(i) < W ? (i) : W - 1])
#define AR_READ_ARGS(...)                                                                      \
  do {                                                                                         \
    if constexpr (W <= 16) {                                                                   \
      asm volatile("" ::AR_RANK_PTR(0), AR_RANK_PTR(1), AR_RANK_PTR(2), AR_RANK_PTR(3),        \
                   AR_RANK_PTR(4), AR_RANK_PTR(5), AR_RANK_PTR(6), AR_RANK_PTR(7),             \
                   AR_RANK_PTR(8), AR_RANK_PTR(9), AR_RANK_PTR(10), AR_RANK_PTR(11),           \
                   AR_RANK_PTR(12), AR_RANK_PTR(13), AR_RANK_PTR(14), AR_RANK_PTR(15),         \
                   __VA_ARGS__);                                                               \
    } else {                                                                                   \
      asm volatile("" ::__VA_ARGS__);                                                          \
    }                                                                                          \
  } while (0)

template <int W, int N, int kMaxLoads>
constexpr int rank_batch() {
  int b = kMaxLoads / N;
  if (b < 1) b = 1;
  return b > W ? W : b;
}

template <int N, int K>
__device__ inline void batch_fence(float (&acc)[N][K]) {
#pragma unroll
  for (int k = 0; k < N; ++k) {
#pragma unroll
    for (int e = 0; e < K; ++e) asm volatile("" : "+v"(acc[k][e]) : : "memory");
  }
}

// acc[k] += x_R0[k] + x_{R0+1}[k] + ... + x_{W-1}[k] (in that order) for the N vectors at
// element offset `base` (uniform) + byte offset boff[k] (per lane) of every partial.
//
// kStage: every batch's loads are issued, then made visible to the arithmetic all at once
// through an empty asm per loaded vector (memory clobber: no load moves past them), then added.
// Without it the scheduler may, to reach its occupancy target, issue one load and wait for it
// before the next (seen at W = 8 with 4-8 vectors per thread: 2x slower); with it the batch
// costs more registers, which the fused kernel's 2-vector rows measured slower for.
template <class T, int N>
constexpr int default_max_loads() {
  return N * T::kVec >= 32 ? 8 : 16;
}

template <class T, int W, int N, int R0 = 0, int kMaxLoads = default_max_loads<T, N>(),
          bool kStage = false>
__device__ inline void rank_sum_range(const RankPtrs<W>& in, int64_t base,
                                      const uint32_t (&boff)[N], float (&acc)[N][T::kVec]) {
  constexpr int kBatch = rank_batch<W - R0 < 1 ? 1 : W - R0, N, kMaxLoads>();
  // At W = 32 the grouped walk below pays only with small batches (the norm kernel's
  // one-vector-at-a-time chains for very wide rows: 2x faster); with 16-load batches the
  // unrolled form is faster (measured).
  constexpr bool kGrouped = W > 32 || (W == 32 && kBatch <= 8);
  if constexpr (kGrouped && R0 == 0 && 16 % kBatch == 0) {
    // About as many rank pointers as scalar registers (2 per pointer): left to itself the compiler
    // spills them to VGPR lanes and, reloading them one at a time, issues one load per DRAM
    // round trip.  Instead walk groups of 16 ranks in a loop that is not unrolled, so each
    // group's pointers are read from the kernel arguments when the group is reached, and stage
    // every batch in registers (all loads first, then the adds in rank order).
#pragma unroll 1
    for (int g = 0; g < W; g += 16) {
#pragma unroll
      for (int r0 = 0; r0 < 16; r0 += kBatch) {
        u32x4 raw[kBatch][N];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const u32x4* src = in.p[g + r0 + j] + base;
#pragma unroll
          for (int k = 0; k < N; ++k) raw[j][k] = load_stream(at(src, boff[k]));
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
#pragma unroll
          for (int k = 0; k < N; ++k) {
            float x[T::kVec];
            T::widen(raw[j][k], x);
#pragma unroll
            for (int e = 0; e < T::kVec; ++e) acc[k][e] = acc[k][e] + x[e];
          }
        }
        batch_fence(acc);
      }
    }
    return;
  }
#pragma unroll
  for (int r0 = R0; r0 < W; r0 += kBatch) {
    if constexpr (kStage) {
      u32x4 raw[kBatch][N];
#pragma unroll
      for (int r = r0; r < r0 + kBatch && r < W; ++r) {
        const u32x4* src = in.p[r] + base;
#pragma unroll
        for (int k = 0; k < N; ++k) raw[r - r0][k] = load_stream(at(src, boff[k]));
      }
#pragma unroll
      for (int r = r0; r < r0 + kBatch && r < W; ++r) {
#pragma unroll
        for (int k = 0; k < N; ++k) asm volatile("" : "+v"(raw[r - r0][k]) : : "memory");
      }
#pragma unroll
      for (int r = r0; r < r0 + kBatch && r < W; ++r) {
#pragma unroll
        for (int k = 0; k < N; ++k) {
          float x[T::kVec];
          T::widen(raw[r - r0][k], x);
#pragma unroll
          for (int e = 0; e < T::kVec; ++e) acc[k][e] = acc[k][e] + x[e];
        }
      }
    } else {
#pragma unroll
      for (int r = r0; r < r0 + kBatch && r < W; ++r) {
        const u32x4* src = in.p[r] + base;
#pragma unroll
        for (int k = 0; k < N; ++k) {
          float x[T::kVec];
          T::widen(load_stream(at(src, boff[k])), x);
#pragma unroll
          for (int e = 0; e < T::kVec; ++e) acc[k][e] = acc[k][e] + x[e];
        }
      }
    }
    if (r0 + kBatch < W) batch_fence(acc);
  }
}

// acc[k] = -0 + x_0[k] + x_1[k] + ... + x_{W-1}[k].
template <class T, int W, int N, int kMaxLoads = default_max_loads<T, N>(), bool kStage = false>
__device__ inline void rank_sum(const RankPtrs<W>& in, int64_t base, const uint32_t (&boff)[N],
                                float (&acc)[N][T::kVec]) {
#pragma unroll
  for (int k = 0; k < N; ++k) {
#pragma unroll
    for (int e = 0; e < T::kVec; ++e) acc[k][e] = -0.0f;
  }
  rank_sum_range<T, W, N, 0, kMaxLoads, kStage>(in, base, boff, acc);
}

// ---- input sources ------------------------------------------------------------------------------
//
// The kernels read the W partials through a source policy.  StreamSource reads ordinary device
// buffers (the one-shot path).  LamportSource reads the slots of a receive buffer that producers
// fill concurrently (see the Lamport section below).

// `ok[k]` says whether vector slot k is a real one; slots that are not re-read a valid vector
// (their offsets are clamped) and their result is discarded.
struct StreamSource {
  template <class T, int W, int N, int kMaxLoads = default_max_loads<T, N>(), bool kStage = false>
  __device__ inline void sum(const RankPtrs<W>& in, int64_t base, const uint32_t (&boff)[N],
                             const bool (&ok)[N], float (&acc)[N][T::kVec]) const {
    (void)ok;
    rank_sum<T, W, N, kMaxLoads, kStage>(in, base, boff, acc);
  }
  // Terms after the W partials for the element-wise tail of the flat sum: none.
  template <class T>
  __device__ inline float tail_extra(float a, int64_t) const { return a; }
};

// ---- kAllReduce -----------------------------------------------------------------------------

// out = RN_T(x_0 + ... + x_{W-1}) for one chunk of blockDim.x * U vectors starting at vector
// `cbase` (uniform); lane t owns vectors cbase + t + u * blockDim.x.
template <class T, int W, int U, bool kNtStore, class Src>
__device__ inline void sum_chunk(const RankPtrs<W>& in, u32x4* out, int64_t nvec, int64_t cbase,
                                 int64_t chunk, const Src& src) {
  uint32_t boff[U];
  float acc[U][T::kVec];
  if (cbase + chunk <= nvec) {
    // Whole chunk in range (uniform branch): no predicate anywhere near the loads.
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      boff[u] = (threadIdx.x + u * blockDim.x) * 16u;
      ok[u] = true;
    }
    src.template sum<T, W, U, default_max_loads<T, U>(), (U >= 2)>(in, cbase, boff, ok, acc);
#pragma unroll
    for (int u = 0; u < U; ++u) store_vec<kNtStore>(at(out + cbase, boff[u]), T::narrow(acc[u]));
  } else {
    // Last, partial chunk: slots past the end re-read the last vector (a clamp, not a branch,
    // so the loads stay unconditional) and are not stored.
    const uint32_t last = static_cast<uint32_t>(nvec - cbase - 1);
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t i = threadIdx.x + u * blockDim.x;
      boff[u] = (i < last ? i : last) * 16u;
      ok[u] = i <= last;
    }
    src.template sum<T, W, U, default_max_loads<T, U>(), (U >= 2)>(in, cbase, boff, ok, acc);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ok[u]) store_vec<kNtStore>(at(out + cbase, boff[u]), T::narrow(acc[u]));
    }
  }
}

// out = RN_T(x_0 + ... + x_{W-1}) over n elements: nvec full 16-byte vectors, then a tail of
// fewer than one vector handled element by element by block 0.  When the grid covers every
// chunk (the launch heuristic always sizes it so) each block sums its one chunk with no loop;
// a smaller grid walks the chunks with a grid stride.  The loop-free form matters: inside a
// loop the compiler hoists each tensor's per-lane address out as a 64-bit pointer stepped per
// iteration (instead of the scalar base + 32-bit offset form) and, for some (W, U), then issues
// the loads a round trip apart.
template <class T, int W, int U, bool kNtStore, class Src = StreamSource>
__global__ __launch_bounds__(kMaxThreads) void ar_sum_kernel(RankPtrs<W> in, u32x4* out,
                                                             int64_t nvec, int tail, Src src) {
  constexpr int kVec = T::kVec;
  // Every argument the first loads need is read at once (left alone: two dependent rounds).
  AR_READ_ARGS("s"(out), "s"(nvec), "s"(tail), "s"(blockDim.x), "s"(gridDim.x));
  AR_PHASE(0, 0, in.p[0]);
  const int64_t chunk = static_cast<int64_t>(blockDim.x) * U;
  if (static_cast<int64_t>(gridDim.x) * chunk >= nvec) {
    const int64_t cbase = blockIdx.x * chunk;
    if (cbase < nvec) sum_chunk<T, W, U, kNtStore>(in, out, nvec, cbase, chunk, src);
    AR_PHASE(7, 0, in.p[0]);
  } else {
    for (int64_t cbase = blockIdx.x * chunk; cbase < nvec; cbase += gridDim.x * chunk)
      sum_chunk<T, W, U, kNtStore>(in, out, nvec, cbase, chunk, src);
  }
  if (tail > 0 && blockIdx.x == 0 && static_cast<int>(threadIdx.x) < tail) {
    const int64_t i = nvec * kVec + threadIdx.x;
    float a = -0.0f;
#pragma unroll
    for (int r = 0; r < W; ++r) a = a + T::widen1(in.p[r], i);
    T::store1(out, i, src.template tail_extra<T>(a, i));
  }
}

// ---- kARResidualRMSNorm ---------------------------------------------------------------------

// acc += widen(v), element by element (one binary32 add each).
template <class T>
__device__ inline void accumulate(float (&acc)[T::kVec], u32x4 v) {
  float x[T::kVec];
  T::widen(v, x);
#pragma unroll
  for (int e = 0; e < T::kVec; ++e) acc[e] = acc[e] + x[e];
}

// The W partials and then the residual as one more addend, so the flat sum kernel computes
// residual_out = RN_T(x_0 + ... + x_{W-1} + residual) with the same binary32 chain as the fused
// kernel: the first kernel of the two-kernel (unfused) path, which accepts rows of any width.
struct ResidualSource {
  const u32x4* residual;
  template <class T, int W, int N, int kMaxLoads = default_max_loads<T, N>(), bool kStage = false>
  __device__ inline void sum(const RankPtrs<W>& in, int64_t base, const uint32_t (&boff)[N],
                             const bool (&ok)[N], float (&acc)[N][T::kVec]) const {
    (void)ok;
    rank_sum<T, W, N, kMaxLoads, kStage>(in, base, boff, acc);
#pragma unroll
    for (int k = 0; k < N; ++k) accumulate<T>(acc[k], load_stream(at(residual + base, boff[k])));
  }
  template <class T>
  __device__ inline float tail_extra(float a, int64_t i) const {
    return a + T::widen1(residual, i);
  }
};

// The kVec gamma values of element vector `vec` (gamma is binary32 [H], 16-byte aligned).
template <int kVec>
__device__ inline void load_gamma(const f32x4* gamma, uint32_t vec, float (&g)[kVec]) {
#pragma unroll
  for (int j = 0; j < kVec / 4; ++j) {
    const f32x4 q = *at(gamma, (vec * (kVec / 4) + j) * 16u);
    g[4 * j + 0] = q.x;
    g[4 * j + 1] = q.y;
    g[4 * j + 2] = q.z;
    g[4 * j + 3] = q.w;
  }
}

// The fixed rank batches the norm kernel is instantiated with (stream source, non-temporal
// stores): one rank for two vectors per thread at W = 4 ... 16 and for four at W = 2 and 4; two
// ranks for two vectors at W >= 4 and for one at W >= 32; four ranks for two vectors at W = 8.
constexpr bool rank_batch_instantiated(int W, int vpt, int n) {
  return (n == 1 && ((vpt == 2 && W >= 4 && W <= 16) || (vpt == 4 && (W == 2 || W == 4)))) ||
         (n == 2 && ((vpt == 2 && W >= 4) || (vpt == 1 && W >= 32))) ||
         (n == 4 && vpt == 2 && W == 8);
}

// One row = V vectors of 16 bytes.  Thread t of a block serves row slot t / L (R slots per
// block) and, within the row, vectors lane + k * L for k < VPT.  L * VPT >= V.  Blocks walk
// groups of R rows with a grid stride.
//
// kNormOnly: the RMSNorm step alone on a stored tensor x = in.p[0] (W = 1; residual and
// residual_out are unused): norm_out = RMSNorm(x) * gamma.  The second kernel of the two-kernel
// path, and a stand-alone RMSNorm.
//
// kRankBatch (whole-row chains of one or two vectors per thread, or one rank's four vectors; 0
// = the default batches of up to 16 loads across ranks): each thread loads kRankBatch ranks'
// vectors per batch, so a block reads that many tensors' rows at a time.  The launch planner
// takes one rank per batch while every row of a call is resident at once (one to three rows per
// CU): all CUs then run the same phase, and reading the W + 1 tensors one after another, rather
// than all of them together, is what HBM serves faster there.  With more rows per CU the blocks
// drift apart; there batches of two ranks (four at W = 8 with 16-bit rows) are the fastest
// middle ground.  The arithmetic is the same.
template <class T, int W, int VPT, bool kNtStore, class Src = StreamSource, bool kNormOnly = false,
          int kRankBatch = 0>
__global__ __launch_bounds__(kMaxThreads) void ar_norm_kernel(
    RankPtrs<W> in, const u32x4* residual, const f32x4* gamma, u32x4* residual_out,
    u32x4* norm_out, int64_t M, int V, int L, int R, float eps, float count_h, Src src) {
  constexpr int kVec = T::kVec;
  __shared__ float red[2][kMaxWavesPerBlock];
  // The exchanges of rows outside the binary32 range.  A wave writes each of them again only
  // after a later barrier that every wave passes only after reading them.
  __shared__ float red_wide[2][kMaxWavesPerBlock];
  __shared__ bool wide_sh[kMaxWavesPerBlock];

  // Every argument the first loads need is read at once: left alone, the compiler read the
  // arguments in three dependent rounds (and divided by L and R) before the first load, which
  // a decode-size call pays in full.
  AR_READ_ARGS("s"(residual), "s"(gamma), "s"(residual_out), "s"(norm_out), "s"(M), "s"(V),
               "s"(L), "s"(R), "s"(blockDim.x), "s"(gridDim.x));
  const int tid = threadIdx.x;
  int slot = 0, lane = tid;  // one row per block (R = 1): no division
  if (R > 1) {
    slot = tid / L;
    lane = tid - slot * L;
  }
  const int wave = tid >> 6;

  int idx[VPT];
  bool col_ok[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int i = lane + k * L;
    col_ok[k] = i < V;
    idx[k] = col_ok[k] ? i : 0;
  }

  // Byte offsets of this thread's vectors inside its row group (uniform base: the group's
  // first row).  A slot past the last row re-reads the group's first row (never stored).
  auto group_offsets = [&](int64_t grp, uint32_t (&boff)[VPT]) {
    const bool ok = grp * R + slot < M;
#pragma unroll
    for (int k = 0; k < VPT; ++k) boff[k] = ((ok ? slot * V : 0) + idx[k]) * 16u;
  };

  // gamma does not depend on the row.  With few vectors per thread this thread's slice is
  // loaded once and kept in registers; with many it is re-read (from L2) in the epilogue.
  // (Kept for 4 vectors with one or two partials: 7 % faster at 2 rows per CU, 20-30 % slower
  // from 3 on -- the extra registers cost waves; measured.)
  constexpr bool kKeepGamma = VPT <= 2;
  float gam[kKeepGamma ? VPT : 1][kVec];
  if constexpr (kKeepGamma) {
#pragma unroll
    for (int k = 0; k < VPT; ++k) load_gamma(gamma, idx[k], gam[k]);
  }

  // gamma of this thread's vector k (kept in registers, or re-read from L2).
  auto gamma_of = [&](int k, float (&g)[kVec]) {
    if constexpr (kKeepGamma) {
#pragma unroll
      for (int e = 0; e < kVec; ++e) g[e] = gam[k][e];
    } else {
      // Opaque index: keeps the compiler from hoisting these loop-invariant loads out of
      // the row loop, where all VPT x kVec values would stay live in registers.
      int gi = idx[k];
      asm volatile("" : "+v"(gi));
      load_gamma(gamma, gi, g);
    }
  };

  // The row's sum of squares of this thread's values scaled by 2^k, reduced over the row in the
  // same tree as the loop's (inside the wave, then the row's waves in order through LDS bank
  // `b`: two banks, so that two reductions in a row need no barrier between them).
  auto scaled_row_sum = [&](const u32x4 (&vals)[VPT], const bool (&okv)[VPT], int k2,
                            int b) -> float {
    float s2 = 0.0f;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      if (okv[k]) {
        float v[kVec];
        T::widen(vals[k], v);
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
          const float u = scaled(v[e], k2);
          s2 += u * u;
        }
      }
    }
    s2 = segment_sum(s2, L);
    if (L > 64) {
      if ((tid & 63) == 0) red_wide[b][wave] = s2;
      __syncthreads();
      const int waves_per_row = L >> 6;
      const int w0 = slot * waves_per_row;
      float t = red_wide[b][w0];
      for (int j = 1; j < waves_per_row; ++j) t += red_wide[b][w0 + j];
      s2 = t;
    }
    return s2;
  };
  // norm_out of this thread's vectors with rstd = m 2^k2.
  auto store_scaled = [&](const u32x4 (&vals)[VPT], const bool (&okv)[VPT], int64_t base,
                          const uint32_t (&boff)[VPT], float m, int k2) {
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      if (okv[k]) {
        float v[kVec];
        T::widen(vals[k], v);
        float g[kVec];
        gamma_of(k, g);
        float y[kVec];
#pragma unroll
        for (int e = 0; e < kVec; ++e) y[e] = norm_elem_scaled(v[e], m, k2, g[e]);
        store_vec<kNtStore>(at(norm_out + base, boff[k]), T::narrow(y));
      }
    }
  };

  AR_PHASE(0, 0, in.p[0]);
  int bank = 0;
  // Whether a row of this wave (of this block, for rows of several waves) was outside the
  // binary32 range of the sum of squares: with the partials' sum those rows are normalised
  // again after the loop (see below).
  bool any_wide = false;
  for (int64_t grp = blockIdx.x; grp * R < M; grp += gridDim.x) {
    const bool row_ok = grp * R + slot < M;
    const int64_t base = grp * R * static_cast<int64_t>(V);
    uint32_t boff[VPT];
    group_offsets(grp, boff);

    bool ok[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) ok[k] = row_ok && col_ok[k];

    // Sum of the W partials and the residual, binary32 in rank order, rounded once to T.
    u32x4 rounded[VPT];
    if constexpr (kNormOnly) {
      static_assert(W == 1, "the norm-only mode reads one tensor");
#pragma unroll
      for (int k = 0; k < VPT; ++k) rounded[k] = load_stream(at(in.p[0] + base, boff[k]));
    } else if constexpr (VPT <= 2 || (W + 1) * VPT <= 20) {
      // All vectors' chains together: the most independent loads per batch (with few
      // partials even 4-8 vectors' accumulators fit beside a batch of loads, no spill).
      // Staged with two or four partials and two vectors: left alone, the scheduler issued
      // those loads one rank at a time, each a round trip after the previous one.  The staged
      // form issues the residual's loads first (its fences would otherwise hold them back a
      // round trip); it is still added after the W partials.
      // One rank's 4 vectors per batch are staged too, with the residual first: left alone,
      // the fp16 W = 4 form issued them a round trip apart.
      constexpr bool kStageChains =
          ((W == 2 || W == 4) && VPT == 2) || (kRankBatch == 1 && VPT >= 4);
      u32x4 res_v[VPT];
      if constexpr (kStageChains) {
#pragma unroll
        for (int k = 0; k < VPT; ++k) res_v[k] = load_stream(at(residual + base, boff[k]));
      }
      float acc[VPT][kVec];
      constexpr int kLoads = kRankBatch > 0 ? kRankBatch * VPT : default_max_loads<T, VPT>();
      src.template sum<T, W, VPT, kLoads, kStageChains>(in, base, boff, ok, acc);
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        if constexpr (!kStageChains) res_v[k] = load_stream(at(residual + base, boff[k]));
        accumulate<T>(acc[k], res_v[k]);
        rounded[k] = T::narrow(acc[k]);
      }
    } else {
      // G vectors' chains at a time (G the largest power of two with (W + 1) G <= 20, at least
      // one) keep the live accumulators and loads in registers; a fence after each group stops
      // the next group's loads from being hoisted over it.  (One vector at a time cost a round
      // trip per vector: W = 8 with 8 vectors per thread ran 6x slower at small M.)
      constexpr int G = (W + 1) * 4 <= 20 ? 4 : (W + 1) * 2 <= 20 ? 2 : 1;
      // Loads per staged batch: 16 x G (all W ranks at once up to W = 16); 8 with 8 vectors
      // per thread (the 32 registers of rounded values leave no room for more: it spilled);
      // 8 for the grouped walk of W >= 32 (its groups of 16 ranks need a batch dividing 16).
      constexpr int kLoads = (W >= 32 || VPT >= 8) ? 8 : 16 * G;
#pragma unroll
      for (int k0 = 0; k0 < VPT; k0 += G) {
        uint32_t boff_g[G];
        bool ok_g[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          boff_g[g] = boff[k0 + g];
          ok_g[g] = ok[k0 + g];
        }
        float acc[G][kVec];
        // Staged for groups of several vectors: that is where the scheduler otherwise issues
        // the loads one round trip apart (W = 8: 2x); single-vector chains (W >= 16) measured
        // faster unstaged -- except W = 16 with 8 vectors per thread, whose unstaged 8-load
        // batches compiled to a full wait after every load (136 loads, 135 waits).
        constexpr bool kStageGroup = G >= 2 || (W == 16 && VPT >= 8);
        src.template sum<T, W, G, kLoads, kStageGroup>(in, base, boff_g, ok_g, acc);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          accumulate<T>(acc[g], load_stream(at(residual + base, boff_g[g])));
          rounded[k0 + g] = T::narrow(acc[g]);
        }
        batch_fence(acc);
      }
    }
    AR_PHASE(1, rounded[0].x, in.p[0]);
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      if (ok[k]) {
        if constexpr (!kNormOnly) store_vec<kNtStore>(at(residual_out + base, boff[k]), rounded[k]);
        float v[kVec];
        T::widen(rounded[k], v);
#pragma unroll
        for (int e = 0; e < kVec; ++e) ss += v[e] * v[e];
      }
    }

    // Row sum of squares: inside the wave, then across the row's waves through LDS.
    ss = segment_sum(ss, L);
    if (L > 64) {
      if ((tid & 63) == 0) red[bank][wave] = ss;
      __syncthreads();
      const int waves_per_row = L >> 6;
      const int w0 = slot * waves_per_row;
      float t = red[bank][w0];
      for (int j = 1; j < waves_per_row; ++j) t += red[bank][w0 + j];
      ss = t;
      bank ^= 1;
    }
    const float rstd = rsqrtf(ss / count_h + eps);
    AR_PHASE(2, rstd, in.p[0]);
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      if (ok[k]) {
        float v[kVec];
        T::widen(rounded[k], v);
        float g[kVec];
        gamma_of(k, g);
        float y[kVec];
#pragma unroll
        for (int e = 0; e < kVec; ++e) y[e] = (v[e] * rstd) * g[e];
        store_vec<kNtStore>(at(norm_out + base, boff[k]), T::narrow(y));
      }
    }

    AR_PHASE(7, 0, in.p[0]);
    // Rows outside the binary32 range of the sum of squares get norm_out again, from the same
    // rounded values scaled by 2^kw, stored over the values above.  The fused patterns do that
    // after the chunk (re-reading residual_out), so that the row loop holds exactly the code it
    // holds without it; the norm-only mode, whose output may overwrite its input, does it here.
    const bool wide = row_ok && outside_binary32_range(ss / count_h + eps);
    if constexpr (!kNormOnly) {
      any_wide = any_wide || __builtin_amdgcn_ballot_w64(wide) != 0;
    } else {
      // wide_any: a row outside the range shares this wave (L <= 64) or, for rows of several
      // waves, this block, whose barrier the second reduction below uses.  Several such rows
      // per block (a shape the launch planner does not pick) need one more exchange for that.
      bool wide_any;
      if (L <= 64) {
        wide_any = __builtin_amdgcn_ballot_w64(wide) != 0;
      } else if (R == 1) {
        wide_any = wide;
      } else {
        if ((tid & 63) == 0) wide_sh[wave] = wide;
        __syncthreads();
        wide_any = false;
        for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w)
          wide_any = wide_any || wide_sh[w];
      }
      if (wide_any) {
        const int kw = wide ? wide_scale(ss / count_h + eps) : 0;
        const float s2 = scaled_row_sum(rounded, ok, kw, 1);
        if (wide) {
          const float m = rstd_of_scaled(s2, kw, count_h, eps);
          store_scaled(rounded, ok, base, boff, m, kw);
        }
      }
    }
  }
  if constexpr (!kNormOnly) {
    // The rows outside the range, again.  Every wave that shares a barrier must take the same
    // path, so rows of several waves agree on the block's flag first.
    if (L > 64 && R > 1) {
      if ((tid & 63) == 0) wide_sh[wave] = any_wide;
      __syncthreads();
      any_wide = false;
      for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) any_wide = any_wide || wide_sh[w];
    }
    if (any_wide) {
      // This thread's residual_out stores visible, then every row group of this block read
      // back (the rounded values) and checked again: the same values in the same order give
      // the same sums of squares, so exactly the rows found outside the range above.
      __threadfence();
      for (int64_t grp = blockIdx.x; grp * R < M; grp += gridDim.x) {
        const bool row_ok = grp * R + slot < M;
        const int64_t base = grp * R * static_cast<int64_t>(V);
        uint32_t boff[VPT];
        group_offsets(grp, boff);
        bool ok[VPT];
        u32x4 rounded[VPT];
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
          ok[k] = row_ok && col_ok[k];
          rounded[k] = *at(residual_out + base, boff[k]);
        }
        const float ss = scaled_row_sum(rounded, ok, 0, 0);
        const bool wide = row_ok && outside_binary32_range(ss / count_h + eps);
        const int kw = wide ? wide_scale(ss / count_h + eps) : 0;
        const float s2 = scaled_row_sum(rounded, ok, kw, 1);
        if (wide) {
          const float m = rstd_of_scaled(s2, kw, count_h, eps);
          store_scaled(rounded, ok, base, boff, m, kw);
        }
      }
    }
  }
}

// ---- RMSNorm of rows of any width ----------------------------------------------------------------
//
// The second kernel of the two-kernel path when a row is not a whole number of 16-byte vectors
// (or too wide for the row kernel).  Row m spans elements [e0, e1) = [m H, m H + H) of a
// 16-byte-aligned tensor; the row is walked as the aligned 16-byte vectors v0 .. v0 + nv - 1 that
// cover it.  Vectors wholly inside the row are loaded and stored whole; the (at most two)
// vectors the row shares with its neighbours are read and written element by element, only the
// row's own elements, so no access leaves the tensor and no block writes another row's data.

// The kVec values of vector v restricted to [e0, e1) (zeros elsewhere).
template <class T, bool kStream>
__device__ inline void load_row_vec(const void* x, int64_t e0, int64_t e1, int64_t v,
                                    float (&f)[T::kVec]) {
  const int64_t a = v * T::kVec;
  if (a >= e0 && a + T::kVec <= e1) {
    const u32x4* p = static_cast<const u32x4*>(x) + v;
    T::widen(kStream ? load_stream(p) : *p, f);
  } else {
#pragma unroll
    for (int e = 0; e < T::kVec; ++e) {
      const int64_t idx = a + e;
      f[e] = (idx >= e0 && idx < e1) ? T::widen1(x, idx) : 0.0f;
    }
  }
}

// y = RN_T(norm(f, gamma)) for the row's elements of vector v.
template <class T, class Norm>
__device__ inline void store_row_vec(void* y, const float* gamma, int64_t e0, int64_t e1,
                                     int64_t v, const float (&f)[T::kVec], Norm norm) {
  const int64_t a = v * T::kVec;
  if (a >= e0 && a + T::kVec <= e1) {
    const float* g = gamma + (a - e0);
    float o[T::kVec];
#pragma unroll
    for (int e = 0; e < T::kVec; ++e) o[e] = norm(f[e], g[e]);
    store_vec<true>(static_cast<u32x4*>(y) + v, T::narrow(o));
  } else {
    // A vector the row shares with a neighbour: element stores.  gamma is read for every
    // element first, at indices clamped into the row, so its loads go out together: read
    // under each element's branch they went out a round trip apart (H = 7170 bf16 M = 2048:
    // the row ends cost 0.96 of 12.6 us).
    float g[T::kVec];
#pragma unroll
    for (int e = 0; e < T::kVec; ++e) {
      const int64_t idx = a + e;
      const int64_t gi = idx < e0 ? 0 : (idx < e1 ? idx - e0 : e1 - 1 - e0);
      g[e] = gamma[gi];
    }
#pragma unroll
    for (int e = 0; e < T::kVec; ++e) {
      const int64_t idx = a + e;
      if (idx >= e0 && idx < e1) T::store1(y, idx, norm(f[e], g[e]));
    }
  }
}

// Block-wide sum of one value per thread (every thread gets the total); `red` holds one float
// per wave and is free again when this returns.
__device__ inline float block_sum(float v, float* red) {
  v = segment_sum(v, 64);
  if (blockDim.x == 64) return v;  // one wave: its sum is the block's
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = red[0];
  for (int j = 1; j < static_cast<int>(blockDim.x >> 6); ++j) t += red[j];
  __syncthreads();  // every wave has read red before it is written again
  return t;
}

// One block per row (grid stride over rows).  K > 0: thread t owns slots t + k * blockDim.x
// (k < K), slot j being the j-th 16-byte vector from the 128-byte line that holds the row's
// first element, and keeps their values in registers between the sum of squares and the scaling,
// so x is read once.  Every one of those K vectors is loaded whole and unconditionally first (a
// slot outside the row re-reads the row's first vector), so the K loads are in flight together;
// elements of a vector that belong to a neighbouring row are then masked to zero.  Only a vector that runs
// past the end of the tensor (the last row's last vector when M * H is not a multiple of the
// vector width) is read element by element.  K = 0 (rows longer than 8 vectors per thread of a
// 1024-thread block): the row is read twice, the second time normally from cache.  y may be x
// itself: every element is read (pass 1) before the barrier and written afterwards by the thread
// that read it (a whole-vector load may also read a neighbouring row's elements while that row's
// block rewrites them; those values are discarded).
template <class T, int K>
// K < 8: held to 64 VGPRs (8 waves per SIMD); left alone, the row-end code below took K = 4 to 68
// and the blocks of 640 threads from three per CU to two (H = 16386 bf16 M = 768: 13 % slower).
__global__ __launch_bounds__(kMaxThreads) __attribute__((amdgpu_waves_per_eu(K == 8 ? 1 : 8)))
void ar_rmsnorm_rows_kernel(const void* x,
                                                                      const float* gamma,
                                                                      void* y, int64_t M,
                                                                      int64_t H, float eps,
                                                                      float count_h) {
  constexpr int kVec = T::kVec;
  __shared__ float red[kMaxWavesPerBlock];
  // gamma's first and last 8 values (indices clamped into the row): a row's partial first
  // vector needs gamma[0, 8), its partial last one gamma[H - 8, H).
  __shared__ float gends[16];
  // The arguments in one round (left alone: two dependent rounds before the first load).
  asm volatile("" ::"s"(x), "s"(gamma), "s"(y), "s"(M), "s"(H), "s"(blockDim.x),
               "s"(gridDim.x));
  // Written to LDS in the first row, after its loads are out (a barrier at the start would put a
  // round trip before every block's first load).  With 8 vectors per thread the value is read at
  // the start (0.3 us of a 12 us call at H = 7170); with fewer, where registers bound the waves
  // per SIMD, where it is stored.
  auto gamma_end = [&]() {
    const int64_t i = threadIdx.x < 8 ? int64_t(threadIdx.x) : H - 16 + int64_t(threadIdx.x);
    return gamma[i < 0 ? 0 : (i < H ? i : H - 1)];
  };
  float gend = 0.0f;
  bool gends_set = false;
  if constexpr (K == 8) {
    if (threadIdx.x < 16) gend = gamma_end();
  }
  const int64_t nthreads = blockDim.x;
  // Whole vectors in the tensor; a vector index at or past this one is not wholly inside it.
  const int64_t nfull = (M * H) / kVec;
  const u32x4* xv = static_cast<const u32x4*>(x);
  for (int64_t m = blockIdx.x; m < M; m += gridDim.x) {
    const int64_t e0 = m * H;
    const int64_t e1 = e0 + H;
    const int64_t v0 = e0 / kVec;
    const int64_t nv = (e1 + kVec - 1) / kVec - v0;
    float ss = 0.0f;
    if constexpr (K > 0) {
      // Slot j of the block holds vector vb + j, vb the first vector of the 128-byte line that
      // holds the row's first element, so every wave-wide access covers whole lines (a row of
      // an odd width starts anywhere in a line).  The row's vectors are slots [off, off + nv);
      // only its first and last can be partial: elements [lo, hi) belong to the row, lo = s
      // in the first, hi = t in the last, whole vectors otherwise.  (The launch gives the block
      // K * blockDim.x >= nv + 7 slots.)
      // Slot arithmetic in 32 bits (a row spans at most H / kVec + 2 vectors, H <= 65536; slots
      // < K blockDim.x): the 64-bit compares and selects it replaced were a measurable part of
      // each row's latency.
      const int64_t vb = v0 & ~int64_t(7);
      const int off = static_cast<int>(v0 - vb);
      const int nvi = static_cast<int>(nv);
      const int nt32 = static_cast<int>(nthreads);
      const int s = static_cast<int>(e0 - v0 * kVec);
      const int t = static_cast<int>(e1 - (v0 + nv - 1) * kVec);
      auto live = [&](int j) { return j >= off && j < off + nvi; };
      auto lo_of = [&](int j) { return j == off ? s : 0; };
      auto hi_of = [&](int j) { return j == off + nvi - 1 ? t : kVec; };
      // Slots from this one on hold vectors past the last whole one of the tensor.
      const int64_t jf64 = nfull - vb;
      const int jfull = jf64 > INT32_MAX ? INT32_MAX : static_cast<int>(jf64);
      float f[K][kVec];
      if (nfull > 0) {
        // Uniform base and 32-bit lane offsets.  A slot outside the row re-reads the row's first
        // vector (a line the wave loads anyway) rather than a neighbouring row's data.
        const int64_t bidx = vb < nfull ? vb : nfull - 1;
        const u32x4* xb = xv + bidx;
        const int shift = static_cast<int>(vb - bidx);  // > 0 only past the last whole vector
        const int64_t lim64 = nfull - 1 - bidx;
        const int lim = lim64 > INT32_MAX ? INT32_MAX : static_cast<int>(lim64);
        u32x4 raw[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const int j = static_cast<int>(threadIdx.x) + k * nt32;
          int r = (live(j) ? j : off) + shift;
          r = r < lim ? r : lim;
          raw[k] = load_stream(at(xb, static_cast<uint32_t>(r) * 16u));
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const int j = static_cast<int>(threadIdx.x) + k * nt32;
          if (!live(j)) raw[k] = u32x4{0, 0, 0, 0};
          T::widen(raw[k], f[k]);
          const int lo = lo_of(j), hi = hi_of(j);
          if (lo > 0 || hi < kVec) {
#pragma unroll
            for (int e = 0; e < kVec; ++e) f[k][e] = (e >= lo && e < hi) ? f[k][e] : 0.0f;
          }
        }
      } else {
#pragma unroll
        for (int k = 0; k < K; ++k) {
#pragma unroll
          for (int e = 0; e < kVec; ++e) f[k][e] = 0.0f;
        }
      }
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int j = static_cast<int>(threadIdx.x) + k * nt32;
        if (live(j) && j >= jfull) load_row_vec<T, false>(x, e0, e1, vb + j, f[k]);
#pragma unroll
        for (int e = 0; e < kVec; ++e) ss += f[k][e] * f[k][e];
      }
      // gamma is read in the epilogue, per vector (L2): moving all of it before the barrier
      // measured slower (H = 7170: 15.9 -> 18.3 us), the other blocks on the CU hide its latency.
      // gamma's ends go to LDS before the block's first barrier (a one-wave block has none, and
      // its LDS accesses stay in program order).
      if (!gends_set) {
        if (threadIdx.x < 16) gends[threadIdx.x] = K == 8 ? gend : gamma_end();
        gends_set = true;
        if (nthreads == 64) __builtin_amdgcn_wave_barrier();
      }
      const float x32 = block_sum(ss, red) / count_h + eps;
      float m = rsqrtf(x32);
      int E = 0;
      if (outside_binary32_range(x32)) {
        // The sum of squares again, of the values in registers (zeros outside the row) scaled.
        E = wide_scale(x32);
        float s2 = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
#pragma unroll
          for (int e = 0; e < kVec; ++e) {
            const float u = scaled(f[k][e], E);
            s2 += u * u;
          }
        }
        m = rstd_of_scaled(block_sum(s2, red), E, count_h, eps);
      }
      auto norm = [&](float a, float g) { return norm_elem_scaled(a, m, E, g); };
      u32x4* yb = static_cast<u32x4*>(y) + vb;
      const int Hi = static_cast<int>(H);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int j = static_cast<int>(threadIdx.x) + k * nt32;
        if (!live(j)) continue;
        if (lo_of(j) == 0 && hi_of(j) == kVec) {
          // A whole vector of the row (so wholly inside the tensor): gamma[(j - off) kVec - s ...]
          // as dword-aligned 16-byte loads, the vector as one 16-byte store.
          const float* g = gamma + ((j - off) * kVec - s);
          float gv[kVec];
#pragma unroll
          for (int q = 0; q < kVec; q += 4) {
            const f32x4u g4 = *reinterpret_cast<const f32x4u*>(g + q);
            gv[q] = g4.x;
            gv[q + 1] = g4.y;
            gv[q + 2] = g4.z;
            gv[q + 3] = g4.w;
          }
          float o[kVec];
#pragma unroll
          for (int e = 0; e < kVec; ++e) o[e] = norm(f[k][e], gv[e]);
          store_vec<true>(at(yb, static_cast<uint32_t>(j) * 16u), T::narrow(o));
        } else {
          // A vector the row shares with a neighbour (its first or last): element stores,
          // gamma from the block's copy of its first and last 8 values in LDS (a read of
          // global gamma here cost the row a round trip at its end).
          const int lo = lo_of(j), hi = hi_of(j);
          const int gb = (j - off) * kVec - s;  // gamma index of the vector's element 0
          void* yv = yb + j;
#pragma unroll
          for (int e = 0; e < kVec; ++e) {
            const int gi = gb + e;
            if (e >= lo && e < hi) T::store1(yv, e, norm(f[k][e], gends[gi < 8 ? gi : gi - Hi + 16]));
          }
        }
      }
    } else {
      for (int64_t j = threadIdx.x; j < nv; j += nthreads) {
        float f[kVec];
        load_row_vec<T, false>(x, e0, e1, v0 + j, f);
#pragma unroll
        for (int e = 0; e < kVec; ++e) ss += f[e] * f[e];
      }
      const float x32 = block_sum(ss, red) / count_h + eps;
      float m = rsqrtf(x32);
      int E = 0;
      if (outside_binary32_range(x32)) {
        // The sum of squares again, scaled: one more pass over the row before any element is
        // written.
        E = wide_scale(x32);
        float s2 = 0.0f;
        for (int64_t j = threadIdx.x; j < nv; j += nthreads) {
          float f[kVec];
          load_row_vec<T, false>(x, e0, e1, v0 + j, f);
#pragma unroll
          for (int e = 0; e < kVec; ++e) {
            const float u = scaled(f[e], E);
            s2 += u * u;
          }
        }
        m = rstd_of_scaled(block_sum(s2, red), E, count_h, eps);
      }
      auto norm = [&](float a, float g) { return norm_elem_scaled(a, m, E, g); };
      for (int64_t j = threadIdx.x; j < nv; j += nthreads) {
        float f[kVec];
        load_row_vec<T, false>(x, e0, e1, v0 + j, f);
        store_row_vec<T>(y, gamma, e0, e1, v0 + j, f, norm);
      }
    }
  }
}

// ---- kARResidualRMSNorm with a row split over several blocks -------------------------------------
//
// With few rows, one block per row leaves most CUs idle and one CU has to stream the whole row of
// W + 1 inputs (W = 8, H = 7168 bf16: 126 KiB through one CU, the bound at M = 1).  Here a row
// gets S blocks ("segments") of L threads x VPT vectors.  Each block sums its segment, stores
// residual_out, reduces the segment's sum of squares and publishes it; the row's blocks then read
// each other's partial sums, add them in segment order and finish the norm from registers.
//
// Exchange: a caller workspace of kSplitSlots 8-byte slots per row; slot j of row m holds
// (tag << 32) | bits(partial sum of segment j).  Between calls every slot of a row carries the
// same tag t (a zero-filled workspace: t = 0).  A block reads t from its own slot (no other block
// writes that slot), and the call leaves tag t + 1 in all kSplitSlots slots of each of its rows
// (segment sums in the first S, zeros after, written by the last segment), so a slot showing
// t + 1 holds this call's value.  Tag and value travel in one naturally aligned 8-byte store,
// which is single-copy atomic, so no fence has to order them; the accesses are relaxed
// agent-scope atomics, coherent across the XCDs.
//
// Waits are bounded: after `max_polls` polls a block stops waiting and computes every segment's
// partial sum itself with the same code and the same reduction order, so the result is
// bit-identical either way.  That recomputation re-reads other segments' inputs, so the outputs
// may not alias any input; and calls that share a workspace must not overlap in time.
constexpr int kSplitSlots = 64;

// The VPT vectors of segment `seg` owned by this thread: seg * L * VPT + threadIdx.x + k * L
// (L = blockDim.x); vectors past the row's V are !ok and re-read vector 0.
template <int VPT>
__device__ inline void split_offsets(int V, int seg, uint32_t (&boff)[VPT], bool (&ok)[VPT]) {
  const int L = blockDim.x;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int i = seg * L * VPT + static_cast<int>(threadIdx.x) + k * L;
    ok[k] = i < V;
    boff[k] = static_cast<uint32_t>(ok[k] ? i : 0) * 16u;
  }
}

// This thread's sum of squares of its rounded values scaled by 2^k (vectors in order, then
// elements in order; k = 0 gives the sum of the unscaled squares).
template <class T, int VPT>
__device__ inline float sum_squares(const u32x4 (&rounded)[VPT], const bool (&ok)[VPT], int k) {
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    if (ok[j]) {
      float v[T::kVec];
      T::widen(rounded[j], v);
#pragma unroll
      for (int e = 0; e < T::kVec; ++e) {
        const float u = scaled(v[e], k);
        ss += u * u;
      }
    }
  }
  return ss;
}

// Sums this thread's vectors of a segment in rank order with the residual last, rounds them to
// T, and returns this thread's sum of squares of the rounded values.
template <class T, int W, int VPT>
__device__ inline float split_segment(const RankPtrs<W>& in, const u32x4* residual, int64_t base,
                                    const uint32_t (&boff)[VPT], const bool (&ok)[VPT],
                                    u32x4 (&rounded)[VPT]) {
  constexpr int kVec = T::kVec;
  // A segment block is often the only wave on its CU, so its loads in flight are all the memory
  // parallelism there is: the residual loads go first and every rank batch is staged.  Left
  // alone, the scheduler issued the second vector's loads and the residual's a round trip late
  // (two vectors per thread) or recycled registers after ~10 loads (W >= 16).
  u32x4 rv[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) rv[k] = load_stream(at(residual + base, boff[k]));
  float acc[VPT][kVec];
  rank_sum<T, W, VPT, default_max_loads<T, VPT>(), true>(in, base, boff, acc);
  float ss = 0.0f;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    accumulate<T>(acc[k], rv[k]);
    rounded[k] = T::narrow(acc[k]);
    if (ok[k]) {
      float v[kVec];
      T::widen(rounded[k], v);
#pragma unroll
      for (int e = 0; e < kVec; ++e) ss += v[e] * v[e];
    }
  }
  return ss;
}

// Launch grid of the split kernel (blocks in x and y).  The dispatcher places workgroups on the
// 8 XCDs round-robin in linear order (x fastest).  With fewer rows than XCDs an 8 x S grid puts
// the S segments of row m on XCD m (block (m, s)), so a row's blocks share one L2: 4-8 % faster
// at M = 1 and 2 (W = 4, 8, 16) than segments spread over the XCDs.  Otherwise an S x M grid
// (block (s, m)) for up to 65535 rows.  Results do not depend on the placement.
constexpr int split_xcds = 8;
constexpr int64_t split_max_rows = 65535;
struct SplitDims {
  int64_t x, y;
};
inline SplitDims split_dims(int64_t M, int64_t S) {
  return M < split_xcds ? SplitDims{split_xcds, S} : SplitDims{S, M};
}

// Grid: split_dims(M, S) blocks of L threads (blocks that map to no row return at once).
// Requires 1 <= S <= kSplitSlots, L a multiple of 64, and S * L * VPT >= V.
template <class T, int W, int VPT, bool kNtStore>
__global__ __launch_bounds__(kMaxThreads) void ar_norm_split_kernel(
    RankPtrs<W> in, const u32x4* residual, const f32x4* gamma, u32x4* residual_out,
    u32x4* norm_out, int V, int S, float eps, float count_h, uint64_t* slots,
    uint32_t max_polls, int M) {
  constexpr int kVec = T::kVec;
  __shared__ float red[kMaxWavesPerBlock];
  __shared__ float part[kSplitSlots];
  __shared__ float total_sh;
  __shared__ int missing_sh;

  const int tid = threadIdx.x;
  AR_PHASE(0, 0, in.p[0]);
  const bool few = M < split_xcds;
  const int m = static_cast<int>(few ? blockIdx.x : blockIdx.y);
  const int s = static_cast<int>(few ? blockIdx.y : blockIdx.x);
  // The arguments the block needs first are read with M, before the branch below: left alone,
  // the compiler read M, branched, then read the rest, a round trip more before the first load.
  AR_READ_ARGS("s"(residual), "s"(gamma), "s"(residual_out), "s"(norm_out), "s"(slots), "s"(V),
               "s"(S), "s"(blockDim.x), "s"(M));
  if (m >= M) return;  // the whole block, before any barrier
  const int64_t base = static_cast<int64_t>(m) * V;
  uint64_t* row = slots + static_cast<int64_t>(m) * kSplitSlots;

  // Wave 0 reads the row's slots (lane j: slot j) while the data loads are in flight; only this
  // block's own slot s is used (its tag is the row's current tag, and nobody else writes it).
  uint64_t slot = 0;
  if (tid < 64) slot = __hip_atomic_load(row + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  uint32_t boff[VPT];
  bool ok[VPT];
  split_offsets<VPT>(V, s, boff, ok);
  // gamma first: issued with the data loads, not a round trip after them.
  float gam[VPT][kVec];
#pragma unroll
  for (int k = 0; k < VPT; ++k) load_gamma(gamma, boff[k] / 16u, gam[k]);
  u32x4 rounded[VPT];
  const float ss = split_segment<T, W, VPT>(in, residual, base, boff, ok, rounded);
  AR_PHASE(1, ss, in.p[0]);
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    if (ok[k]) store_vec<kNtStore>(at(residual_out + base, boff[k]), rounded[k]);
  }
  const float mine = block_sum(ss, red);
  AR_PHASE(2, mine, in.p[0]);

  float total = 0.0f;  // the row's sum of squares (every thread, once known)
  bool all = false;    // every segment's sum arrived
  if (tid < 64) {
    const int lane = tid;
    const uint32_t want =
        static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(slot >> 32), s)) + 1u;
    const uint64_t tag = static_cast<uint64_t>(want) << 32;
    if (lane == s) {
      slot = tag | __float_as_uint(mine);
      __hip_atomic_store(row + s, slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (s == S - 1 && lane >= S)
      __hip_atomic_store(row + lane, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // Polls with two loads in flight: each check waits for the older load only, so a value
    // that lands between two polls is seen about half a round trip sooner than with one poll
    // at a time.
    AR_PHASE(3, slot, in.p[0]);
    bool have = lane >= S || lane == s;
    if (__builtin_amdgcn_ballot_w64(!have) != 0 && max_polls > 0) {
      uint64_t a = have ? slot : __hip_atomic_load(row + lane, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      for (uint32_t n = 1;; ++n) {
        const bool more = n < max_polls;
        uint64_t b = a;
        if (!have && more)
          b = __hip_atomic_load(row + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (!have && static_cast<uint32_t>(a >> 32) == want) {
          slot = a;
          have = true;
        }
        if (__builtin_amdgcn_ballot_w64(!have) == 0 || !more) break;
        a = b;
      }
    }
    all = __builtin_amdgcn_ballot_w64(!have) == 0;
    AR_PHASE(4, static_cast<int>(all), in.p[0]);
    if (all) total = segment_sum(lane < S ? __uint_as_float(static_cast<uint32_t>(slot)) : 0.0f, 64);
    if (blockDim.x > 64) {
      if (lane == 0) {
        total_sh = total;
        missing_sh = all ? 0 : 1;
      }
    }
  }
  // One wave: wave 0 is the block and holds the total already.
  if (blockDim.x > 64) {
    __syncthreads();
    total = total_sh;
    all = missing_sh == 0;
  }
  if (!all) {
    // Some segment did not arrive in time: compute every segment's partial sum here.
    for (int j = 0; j < S; ++j) {
      float pj = mine;
      if (j != s) {
        uint32_t bj[VPT];
        bool okj[VPT];
        u32x4 rj[VPT];
        split_offsets<VPT>(V, j, bj, okj);
        pj = block_sum(split_segment<T, W, VPT>(in, residual, base, bj, okj, rj), red);
      }
      if (tid == 0) part[j] = pj;
    }
    __syncthreads();
    if (tid < 64) {
      const float p = segment_sum(tid < S ? part[tid] : 0.0f, 64);
      if (tid == 0) total_sh = p;
    }
    __syncthreads();
    total = total_sh;
  }
  const float rstd = rsqrtf(total / count_h + eps);
  AR_PHASE(5, rstd, in.p[0]);
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    if (ok[k]) {
      float v[kVec];
      T::widen(rounded[k], v);
      float y[kVec];
#pragma unroll
      for (int e = 0; e < kVec; ++e) y[e] = (v[e] * rstd) * gam[k][e];
      store_vec<kNtStore>(at(norm_out + base, boff[k]), T::narrow(y));
    }
  }
  AR_PHASE(7, 0, in.p[0]);
  // A row outside the binary32 range of the sum of squares (total_sh is the same in every thread
  // of the block: the branch is uniform): norm_out again from the values scaled by 2^E, stored
  // over the values above.  The exchange carries unscaled segment sums, so every block of the
  // row recomputes the other segments (re-reading their inputs) and adds them in segment order
  // the same way: all blocks reach the same sum.
  const float x32 = total / count_h + eps;
  if (outside_binary32_range(x32)) {
    const int E = wide_scale(x32);
    float sq = 0.0f;
    for (int j = 0; j < S; ++j) {
      if (j != s) {
        uint32_t bj[VPT];
        bool okj[VPT];
        u32x4 rj[VPT];
        split_offsets<VPT>(V, j, bj, okj);
        (void)split_segment<T, W, VPT>(in, residual, base, bj, okj, rj);
        sq += sum_squares<T, VPT>(rj, okj, E);
      } else {
        sq += sum_squares<T, VPT>(rounded, ok, E);
      }
    }
    const float m = rstd_of_scaled(block_sum(sq, red), E, count_h, eps);
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      if (ok[k]) {
        float v[kVec];
        T::widen(rounded[k], v);
        float y[kVec];
#pragma unroll
        for (int e = 0; e < kVec; ++e) y[e] = norm_elem_scaled(v[e], m, E, gam[k][e]);
        store_vec<kNtStore>(at(norm_out + base, boff[k]), T::narrow(y));
      }
    }
  }
}

// Zero-fills n 8-byte words (the split kernel's workspace), without a memset node in graphs.
template <class V>
__global__ __launch_bounds__(kMaxThreads) void ar_fill_zero_kernel(V* p, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0;
}

// ---- Lamport-style one-shot exchange (receive side) ---------------------------------------------
//
// The one-shot exchange of the MNNVL all-reduce (flashinfer pull request "Optimizations for
// TRTLLM MNNVL Allreduce", Description and Summary: Lamport polling with vectorized loads, buffer
// state kept in the data) needs no separate flag: a receive slot per rank, every element of an
// empty slot holding a sentinel bit pattern (all ones: a NaN in every element type), and a
// producer's data can never equal it because the producer replaces an all-ones element by the same
// value with its lowest bit cleared (still a NaN).  The consumer polls each element until it is not
// the sentinel and reduces.  Three receive buffers rotate by round (round k uses buffer k mod 3):
// the producer of round k writes its slot of buffer k mod 3 and empties its slot of buffer
// (k + 1) mod 3, the one round k - 2 used, so the consumer only reads and the emptying is off its
// path.  That buffer is free once every consumer of round k - 2 is done, which a rank's round-k
// push implies when each rank pushes round k only after consuming round k - 1 (that consumer needed
// every rank's round k - 1 push, made after its own consumer of round k - 2).
//
// Slots are moved as 16-byte buffer loads and stores carrying the device-coherence cache bit
// (sc1, the form of a relaxed agent-scope atomic on this architecture) and the streaming hint:
// a producer kernel and a consumer kernel running at the same time on different XCDs see each
// other's data.  A 16-byte access is not atomic as a whole, but each naturally aligned dword of
// it is, and an element (2 or 4 bytes) never straddles a dword, so every element the consumer
// reads is either the sentinel or the producer's complete value; the consumer checks elements,
// not vectors.  Every wait is bounded: after `spin_limit` polls of one vector the consumer gives
// up, sets bit 0 of `*status` and continues with what it read (the affected outputs are then
// meaningless; the caller checks the status).

template <class T>
struct LaneMask;
template <>
struct LaneMask<Bf16> {
  static constexpr uint64_t kLow = 0x0001000100010001ull, kHigh = 0x8000800080008000ull;
};
template <>
struct LaneMask<F16> : LaneMask<Bf16> {};
template <>
struct LaneMask<F32> {
  static constexpr uint64_t kLow = 0x0000000100000001ull, kHigh = 0x8000000080000000ull;
};

// Per element lane of w: the lane's high bit set iff the element is the all-ones sentinel
// (classic "lane is zero" test applied to ~w).
template <class T>
__device__ inline uint64_t sentinel_lanes(uint64_t w) {
  const uint64_t x = ~w;
  return (x - LaneMask<T>::kLow) & ~x & LaneMask<T>::kHigh;
}

template <class T>
__device__ inline uint64_t canonicalize(uint64_t w) {
  // An all-ones element becomes all ones with the lowest bit cleared.
  const uint64_t high = sentinel_lanes<T>(w);
  const int shift = (LaneMask<T>::kHigh == 0x8000800080008000ull) ? 15 : 31;
  return w & ~(high >> shift);
}

__device__ inline uint64_t lo64(u32x4 v) { return v.x | (static_cast<uint64_t>(v.y) << 32); }
__device__ inline uint64_t hi64(u32x4 v) { return v.z | (static_cast<uint64_t>(v.w) << 32); }

template <class T>
__device__ inline bool has_sentinel(u32x4 v) {
  return (sentinel_lanes<T>(lo64(v)) | sentinel_lanes<T>(hi64(v))) != 0;
}

// Cache-policy bits of a buffer access: sc1 (device coherence) | nt (streaming).
constexpr int kCoherentNt = 16 | 2;
// Raw buffer over [base, base + 4 GiB): word 3 selects 32-bit data format, no swizzle.
__device__ inline __amdgpu_buffer_rsrc_t coherent_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, -1, 0x00020000);
}
// The 16 bytes at byte offset boff of a uniform base, device-coherent.
__device__ inline u32x4 load_coherent(const u32x4* base, uint32_t boff) {
  return __builtin_bit_cast(
      u32x4, __builtin_amdgcn_raw_buffer_load_b128(coherent_rsrc(base), boff, 0, kCoherentNt));
}
__device__ inline void store_coherent(u32x4* base, uint32_t boff, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, coherent_rsrc(base), boff, 0, kCoherentNt);
}

// kRanks: ranks per polled batch (0: half the stream source's batch of loads).  Beyond one row
// (or 1024 vectors) per CU smaller polled batches run faster; the launch planner picks them.
template <int kRanks = 0>
struct LamportSourceT {
  int* status;          // bit 0 set on a poll timeout
  uint32_t spin_limit;  // polls per vector before giving up

  // Polls the vector at base + boff until no element is empty.  After its first timeout a
  // thread stops waiting (`gave_up`), so a missing producer costs each thread at most one spin
  // limit.  The empty asm with a memory clobber keeps the reload inside the loop.
  template <class T>
  __device__ inline u32x4 wait_vec(const u32x4* base, uint32_t boff, u32x4 v,
                                   bool& gave_up) const {
    uint32_t n = 0;
    while (!gave_up && has_sentinel<T>(v)) {
      if (n++ >= spin_limit) {
        __hip_atomic_fetch_or(status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        gave_up = true;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
      asm volatile("" : : : "memory");
      v = load_coherent(base, boff);
    }
    return v;
  }

  // acc[k] = -0 + slot_0[k] + ... + slot_{W-1}[k]: all vectors of a batch are loaded first, then
  // only vectors still holding an empty element are polled again, then the batch is accumulated
  // in rank order.  Slots that are not real (ok[k] false) read nothing.
  // (kStage is accepted for the common interface; the polled batch is staged already.)
  template <class T, int W, int N, int kMaxLoads = default_max_loads<T, N>(), bool kStage = false>
  __device__ inline void sum(const RankPtrs<W>& in, int64_t base, const uint32_t (&boff)[N],
                             const bool (&ok)[N], float (&acc)[N][T::kVec]) const {
    // Polled vectors stay live until accumulated: half the stream source's batch by default.
    constexpr int kBatch = kRanks > 0 ? (kRanks < W ? kRanks : W)
                                      : rank_batch<W, N, (kMaxLoads / 2 > 0 ? kMaxLoads / 2 : 1)>();
    bool gave_up = false;
#pragma unroll
    for (int k = 0; k < N; ++k) {
#pragma unroll
      for (int e = 0; e < T::kVec; ++e) acc[k][e] = -0.0f;
    }
#pragma unroll
    for (int r0 = 0; r0 < W; r0 += kBatch) {
      u32x4 w[kBatch][N];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (r0 + j >= W) break;
#pragma unroll
        for (int k = 0; k < N; ++k) {
          w[j][k] = ok[k] ? load_coherent(in.p[r0 + j] + base, boff[k]) : u32x4{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (r0 + j >= W) break;
        const u32x4* slot = in.p[r0 + j] + base;
#pragma unroll
        for (int k = 0; k < N; ++k) {
          const u32x4 v = wait_vec<T>(slot, boff[k], w[j][k], gave_up);
          float x[T::kVec];
          T::widen(v, x);
#pragma unroll
          for (int e = 0; e < T::kVec; ++e) acc[k][e] = acc[k][e] + x[e];
        }
      }
      if (r0 + kBatch < W) batch_fence(acc);
    }
  }

  // The exchange moves whole vectors only: no element-wise tail.
  template <class T>
  __device__ inline float tail_extra(float a, int64_t) const { return a; }
};
using LamportSource = LamportSourceT<0>;

// Producer: next[i] = empty, then slot[i] = canonicalize(src[i]), for nvec 16-byte vectors,
// device-coherent stores.  The thread waits for its emptying store to complete before it stores
// the data, so the emptied vector is visible no later than the data: a consumer that has seen
// this round's data, and every later kernel on its stream, sees next[i] empty, never the older
// round's value.  One 16-byte
// vector per thread; a grid that covers every vector runs no loop.
template <class T>
__global__ __launch_bounds__(kMaxThreads) void ar_lamport_push_kernel(const u32x4* src,
                                                                      u32x4* slot, u32x4* next,
                                                                      int64_t nvec) {
  const int64_t chunk = blockDim.x;
  const uint32_t boff = threadIdx.x * 16u;
  const u32x4 empty = {~0u, ~0u, ~0u, ~0u};
  auto one = [&](int64_t cbase) {
    if (cbase + threadIdx.x < nvec) {
      const u32x4 v = load_stream(at(src + cbase, boff));
      store_coherent(next + cbase, boff, empty);
      const uint64_t lo = canonicalize<T>(lo64(v)), hi = canonicalize<T>(hi64(v));
      const u32x4 c = {static_cast<uint32_t>(lo), static_cast<uint32_t>(lo >> 32),
                       static_cast<uint32_t>(hi), static_cast<uint32_t>(hi >> 32)};
      // The emptying store must be visible before the data is.  A device-coherent store is
      // acknowledged once it is visible device-wide, so waiting for the memory counter orders the
      // two; an agent-scope release fence would do the same but also write back the whole L2.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      store_coherent(slot + cbase, boff, c);
    }
  };
  if (static_cast<int64_t>(gridDim.x) * chunk >= nvec) {
    one(blockIdx.x * chunk);
  } else {
    for (int64_t cbase = blockIdx.x * chunk; cbase < nvec; cbase += gridDim.x * chunk) one(cbase);
  }
}

// Arms (empties) nvec 16-byte vectors of a receive buffer.  (A template so that the header
// defines no kernel by itself: it is instantiated in one translation unit only.)
template <class V>
__global__ __launch_bounds__(kMaxThreads) void ar_lamport_arm_kernel(V* buf, int64_t nvec) {
  const int64_t chunk = blockDim.x;
  const uint32_t boff = threadIdx.x * 16u;
  const V empty = {~0u, ~0u, ~0u, ~0u};
  for (int64_t cbase = blockIdx.x * chunk; cbase < nvec; cbase += gridDim.x * chunk) {
    if (cbase + threadIdx.x < nvec) store_coherent(buf + cbase, boff, empty);
  }
}

// ---- all-gather share (two-shot) ----------------------------------------------------------------

struct GatherArgs {
  const u32x4* src[64];     // slice j, [row_count(j) * V] vectors
  int64_t vec_begin[65];    // first vector of slice j in `out`; vec_begin[W] = M * V
};

// out[vec_begin[j] + i] = src[j][i].  blockIdx.y = slice; the blocks of a slice take chunks of
// blockDim.x * U vectors (lane t owns t + u * blockDim.x, all U loads issued before the stores),
// loop-free when the grid covers the largest slice, else with a grid stride.  Slices whose bit
// is set in `skip` are already in place.
template <bool kNtStore, int U>
__global__ __launch_bounds__(kMaxThreads) void ar_gather_kernel(GatherArgs a, u32x4* out,
                                                                uint64_t skip) {
  const int j = blockIdx.y;
  if ((skip >> j) & 1u) return;
  const int64_t begin = a.vec_begin[j];
  const int64_t n = a.vec_begin[j + 1] - begin;
  const u32x4* src = a.src[j];
  u32x4* dst = out + begin;
  const int64_t chunk = static_cast<int64_t>(blockDim.x) * U;
  auto one = [&](int64_t cbase) {
    if (cbase + chunk <= n) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        v[u] = load_stream(at(src + cbase, (threadIdx.x + u * blockDim.x) * 16u));
#pragma unroll
      for (int u = 0; u < U; ++u)
        store_vec<kNtStore>(at(dst + cbase, (threadIdx.x + u * blockDim.x) * 16u), v[u]);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t i = threadIdx.x + u * blockDim.x;
        if (cbase + i < n) store_vec<kNtStore>(at(dst + cbase, i * 16u), load_stream(at(src + cbase, i * 16u)));
      }
    }
  };
  if (static_cast<int64_t>(gridDim.x) * chunk >= n) {
    const int64_t cbase = blockIdx.x * chunk;
    if (cbase < n) one(cbase);
  } else {
    for (int64_t cbase = blockIdx.x * chunk; cbase < n; cbase += gridDim.x * chunk) one(cbase);
  }
}

}  // namespace arf
