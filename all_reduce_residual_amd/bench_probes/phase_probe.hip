// phase_probe.hip -- ar_probe_phases (ar_probe.h): the library's kernels compiled again with
// their phase hooks storing a clock per block and phase (benchmark only; not linked into the
// all-reduce library, whose build leaves the hooks empty).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

namespace arfp {
__device__ uint64_t* g_stamps;  // [sets][grid][8] clock values
__device__ uintptr_t g_base;    // partial 0's allocation: the call's set is its offset in it
__device__ uint32_t g_set_shift;  // log2 of the (power-of-two) set stride

// Thread 0 of the block stores the real-time clock for `phase` once `value` is computed (the
// empty asm makes the stamp wait for it).
template <class V>
__device__ inline void stamp(int phase, V value, const void* tensor) {
  asm volatile("" ::"v"(value));
  if (threadIdx.x == 0) {
    const uint64_t set = (reinterpret_cast<uintptr_t>(tensor) - g_base) >> g_set_shift;
    const uint64_t blocks = uint64_t(gridDim.x) * gridDim.y;
    const uint64_t b = uint64_t(blockIdx.y) * gridDim.x + blockIdx.x;
    g_stamps[(set * blocks + b) * 8 + phase] = __builtin_amdgcn_s_memrealtime();
  }
}
}  // namespace arfp

#define AR_PHASE(phase, value, tensor) ::arfp::stamp(phase, value, tensor)
#include "../csrc/ar_kernels.hpp"
#include "ar_probe.h"

namespace {

using namespace arf;

__global__ void empty_kernel(const void* tensor) { AR_PHASE(0, 0, tensor); AR_PHASE(7, 0, tensor); }

struct Shape {
  int kind, M, H, threads, vpt, grid, segments;
};

#define PK(x)                                \
  do {                                       \
    if ((x) != hipSuccess) return 2;         \
  } while (0)

double median(std::vector<double> v) {
  if (v.empty()) return -1.0;
  std::sort(v.begin(), v.end());
  return v[v.size() / 2];
}

template <int W>
int run(const Shape& c, double* out) {
  const int V = c.H / 8;
  const size_t used = size_t(c.M) * c.H * 2;  // bytes of one [M, H] tensor
  uint32_t shift = 4;
  while ((size_t(1) << shift) < used) ++shift;
  const size_t tb = size_t(1) << shift;  // set stride: a power of two (the stamp's set index
                                         // is then a shift)
  const size_t foot = used * (W + 3);
  int sets = static_cast<int>(std::min<size_t>(4096, ((size_t(512) << 20) + foot - 1) / foot));
  const int calls = sets * std::max(1, (200 + sets - 1) / sets);
  std::vector<char*> role(W + 3, nullptr);
  float* gamma = nullptr;
  uint64_t* stamps = nullptr;
  uint64_t* ws = nullptr;
  hipStream_t s = nullptr;
  hipGraph_t gr = nullptr;
  hipGraphExec_t ge = nullptr;
  const size_t sbytes = size_t(sets) * c.grid * 8 * 8;
  int rc = 0;
  auto body = [&]() -> int {
    for (auto& r : role) {
      PK(hipMalloc(&r, tb * sets));
      PK(hipMemset(r, 0x3c, tb * sets));  // bf16 ~1.0
    }
    PK(hipMalloc(&gamma, c.H * 4));
    std::vector<float> g(c.H, 1.0f);
    PK(hipMemcpy(gamma, g.data(), c.H * 4, hipMemcpyHostToDevice));
    PK(hipMalloc(&stamps, sbytes));
    PK(hipMemcpyToSymbol(HIP_SYMBOL(arfp::g_stamps), &stamps, sizeof(stamps)));
    uintptr_t base = reinterpret_cast<uintptr_t>(role[0]);
    PK(hipMemcpyToSymbol(HIP_SYMBOL(arfp::g_base), &base, sizeof(base)));
    PK(hipMemcpyToSymbol(HIP_SYMBOL(arfp::g_set_shift), &shift, sizeof(shift)));
    PK(hipMalloc(&ws, size_t(c.M) * kSplitSlots * 8));
    PK(hipMemset(ws, 0, size_t(c.M) * kSplitSlots * 8));
    PK(hipStreamCreate(&s));
    float eps = 1e-6f, ch = float(c.H);
    PK(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
    for (int i = 0; i < calls; ++i) {
      const int set = i % sets;
      RankPtrs<W> in;
      for (int r = 0; r < W; ++r) in.p[r] = reinterpret_cast<const u32x4*>(role[r] + tb * set);
      const u32x4* res = reinterpret_cast<const u32x4*>(role[W] + tb * set);
      u32x4* ro = reinterpret_cast<u32x4*>(role[W + 1] + tb * set);
      u32x4* no = reinterpret_cast<u32x4*>(role[W + 2] + tb * set);
      int64_t M64 = c.M;
      int Vv = V, L = c.threads, R = 1;
      StreamSource src;
      const f32x4* gm = reinterpret_cast<const f32x4*>(gamma);
      hipError_t e;
      if (c.kind == 3) {
        const void* t = in.p[0];
        void* a[] = {&t};
        e = hipLaunchKernel((const void*)&empty_kernel, dim3(1), dim3(64), a, 0, s);
      } else if (c.kind == 0) {
        int64_t nvec = int64_t(c.M) * V;
        int tail = 0;
        void* a[] = {&in, &ro, &nvec, &tail, &src};
        const void* fn = c.vpt == 1 ? (const void*)&ar_sum_kernel<Bf16, W, 1, true>
                                    : (const void*)&ar_sum_kernel<Bf16, W, 2, true>;
        e = hipLaunchKernel(fn, dim3(c.grid), dim3(c.threads), a, 0, s);
      } else if (c.kind == 1) {
        void* a[] = {&in, &res, &gm, &ro, &no, &M64, &Vv, &L, &R, &eps, &ch, &src};
        const void* fn = c.vpt == 1 ? (const void*)&ar_norm_kernel<Bf16, W, 1, true>
                                    : (const void*)&ar_norm_kernel<Bf16, W, 2, true>;
        e = hipLaunchKernel(fn, dim3(c.grid), dim3(c.threads), a, 0, s);
      } else {
        int S = c.segments;
        uint32_t polls = 1u << 14;
        int rows = c.M;
        void* a[] = {&in, &res, &gm, &ro, &no, &Vv, &S, &eps, &ch, &ws, &polls, &rows};
        const SplitDims g = split_dims(c.M, S);
        e = hipLaunchKernel((const void*)&ar_norm_split_kernel<Bf16, W, 1, true>,
                            dim3(unsigned(g.x), unsigned(g.y)), dim3(c.threads), a, 0, s);
      }
      if (e != hipSuccess) {
        hipGraph_t dead = nullptr;
        (void)hipStreamEndCapture(s, &dead);
        if (dead) (void)hipGraphDestroy(dead);
        return 2;
      }
    }
    PK(hipStreamEndCapture(s, &gr));
    PK(hipGraphInstantiate(&ge, gr, nullptr, nullptr, 0));
    std::vector<double> percall, span, gap, phase[8];
    std::vector<uint64_t> h(sbytes / 8);
    for (int rep = 0; rep < 6; ++rep) {
      PK(hipMemsetAsync(stamps, 0, sbytes, s));
      hipEvent_t e0, e1;
      PK(hipEventCreate(&e0));
      PK(hipEventCreate(&e1));
      PK(hipEventRecord(e0, s));
      PK(hipGraphLaunch(ge, s));
      PK(hipEventRecord(e1, s));
      PK(hipStreamSynchronize(s));
      float ms = 0.0f;
      PK(hipEventElapsedTime(&ms, e0, e1));
      PK(hipEventDestroy(e0));
      PK(hipEventDestroy(e1));
      if (rep == 0) continue;
      percall.push_back(ms * 1000.0 / calls);
      PK(hipMemcpy(h.data(), stamps, sbytes, hipMemcpyDeviceToHost));
      struct K {
        double st, en, ph[8];
      };
      std::vector<K> ks;
      for (int set = 0; set < sets; ++set) {
        uint64_t first = ~0ull, last[8] = {0};
        for (int b = 0; b < c.grid; ++b) {
          const uint64_t* q = &h[(size_t(set) * c.grid + b) * 8];
          if (!q[0]) continue;
          first = std::min(first, q[0]);
          for (int p = 1; p < 8; ++p) last[p] = std::max(last[p], q[p]);
        }
        if (first == ~0ull || !last[7]) continue;
        K k;
        k.st = first * 0.01;  // 100 MHz clock: 0.01 us per tick
        k.en = last[7] * 0.01;
        for (int p = 1; p < 8; ++p) k.ph[p] = last[p] ? (last[p] - first) * 0.01 : -1.0;
        ks.push_back(k);
      }
      std::sort(ks.begin(), ks.end(), [](const K& a, const K& b) { return a.st < b.st; });
      for (size_t i = 0; i < ks.size(); ++i) {
        span.push_back(ks[i].en - ks[i].st);
        if (i + 1 < ks.size()) gap.push_back(ks[i + 1].st - ks[i].en);
        for (int p = 1; p < 7; ++p)
          if (ks[i].ph[p] >= 0) phase[p].push_back(ks[i].ph[p]);
      }
    }
    out[0] = median(percall);
    out[1] = median(span);
    out[2] = median(gap);
    for (int p = 1; p < 7; ++p) out[2 + p] = median(phase[p]);
    out[9] = sets;
    out[10] = calls;
    return 0;
  };
  rc = body();
  if (ge) (void)hipGraphExecDestroy(ge);
  if (gr) (void)hipGraphDestroy(gr);
  if (s) (void)hipStreamDestroy(s);
  for (auto& r : role)
    if (r) (void)hipFree(r);
  if (gamma) (void)hipFree(gamma);
  if (stamps) (void)hipFree(stamps);
  if (ws) (void)hipFree(ws);
  return rc;
}

}  // namespace

extern "C" int ar_probe_phases(int kind, int W, int M, int H, int threads, int vpt, int grid,
                               int segments, double* out) {
  if (!out || kind < 0 || kind > 3 || M < 1 || M > 4096 || H < 8 || H % 8 != 0 || H > 65536)
    return 1;
  if (threads < 64 || threads > 1024 || threads % 64 != 0 || (vpt != 1 && vpt != 2) || grid < 1)
    return 1;
  const int64_t V = H / 8;
  // Every launch must cover exactly its set's vectors (no access outside the buffers).
  if (kind == 0 && int64_t(grid) * threads * vpt != int64_t(M) * V) return 1;
  if (kind == 1 && (grid != M || int64_t(threads) * vpt < V)) return 1;
  if (kind == 2 && (segments < 1 || segments > kSplitSlots ||
                    grid != split_dims(M, segments).x * split_dims(M, segments).y || vpt != 1 ||
                    int64_t(segments) * threads < V))
    return 1;
  if (kind == 3 && grid != 1) return 1;
  const Shape c{kind, M, H, threads, vpt, grid, segments};
  switch (W) {
    case 2: return run<2>(c, out);
    case 4: return run<4>(c, out);
    case 8: return run<8>(c, out);
    case 16: return run<16>(c, out);
    default: return 1;
  }
}
