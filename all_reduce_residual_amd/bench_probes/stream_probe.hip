// stream_probe.hip -- the streaming-bandwidth probe declared in ar_probe.h (benchmark
// calibration only; not linked into the all-reduce library).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ar_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Streams {
  const u32x4* p[16];
};

template <int NR, int NW>
__global__ __launch_bounds__(1024) void probe_kernel(Streams in, int64_t nvec, u32x4* o0,
                                                     u32x4* o1) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= nvec) return;
  u32x4 v[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) v[r] = __builtin_nontemporal_load(in.p[r] + i);
  u32x4 a = v[0];
#pragma unroll
  for (int r = 1; r < NR; ++r) a ^= v[r];
  __builtin_nontemporal_store(a, o0 + i);
  if constexpr (NW == 2) __builtin_nontemporal_store(a + 1u, o1 + i);
}

bool aligned16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <int NR>
void launch(unsigned blocks, int threads, hipStream_t st, const Streams& s, int64_t nvec, int nw,
            u32x4* o0, u32x4* o1) {
  if (nw == 2) {
    probe_kernel<NR, 2><<<dim3(blocks), dim3(threads), 0, st>>>(s, nvec, o0, o1);
  } else {
    probe_kernel<NR, 1><<<dim3(blocks), dim3(threads), 0, st>>>(s, nvec, o0, o1);
  }
}

}  // namespace

extern "C" int ar_probe_stream(const void* const* inputs, int nr, int nw, int64_t nvec, void* out0,
                               void* out1, int threads, void* stream) {
  const bool nr_ok = nr == 1 || nr == 2 || nr == 4 || nr == 8 || nr == 9 || nr == 16;
  if (!inputs || !nr_ok || (nw != 1 && nw != 2) || nvec < 0) return 1;
  if (threads < 64 || threads > 1024 || threads % 64 != 0) return 1;
  if (nvec == 0) return 0;
  Streams s{};
  for (int r = 0; r < nr; ++r) {
    if (!aligned16(inputs[r])) return 1;
    s.p[r] = static_cast<const u32x4*>(inputs[r]);
  }
  if (!aligned16(out0) || (nw == 2 && !aligned16(out1))) return 1;
  const int64_t blocks = (nvec + threads - 1) / threads;
  if (blocks > INT32_MAX) return 1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  u32x4* o0 = static_cast<u32x4*>(out0);
  u32x4* o1 = static_cast<u32x4*>(nw == 2 ? out1 : out0);
  const unsigned b = static_cast<unsigned>(blocks);
  switch (nr) {
    case 1: launch<1>(b, threads, st, s, nvec, nw, o0, o1); break;
    case 2: launch<2>(b, threads, st, s, nvec, nw, o0, o1); break;
    case 4: launch<4>(b, threads, st, s, nvec, nw, o0, o1); break;
    case 8: launch<8>(b, threads, st, s, nvec, nw, o0, o1); break;
    case 9: launch<9>(b, threads, st, s, nvec, nw, o0, o1); break;
    default: launch<16>(b, threads, st, s, nvec, nw, o0, o1); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
