// inst_f16.hip -- kernel instantiations and launchers for one element type (F16).
#include "ar_dispatch.hpp"

namespace arfh {

hipError_t launch_sum_f16(const void* const* inputs, int W, void* out, int64_t nvec, int tail,
                          const ar_launch_cfg_t& c, hipStream_t s) {
  return launch_sum_t<F16>(inputs, W, out, nvec, tail, c, s);
}

hipError_t launch_norm_f16(const void* const* inputs, int W, const void* residual,
                           const float* gamma, float eps, void* residual_out, void* norm_out,
                           int64_t M, int64_t H, const ar_launch_cfg_t& c, hipStream_t s) {
  return launch_norm_t<F16>(inputs, W, residual, gamma, eps, residual_out, norm_out, M, H, c,
                              s);
}

hipError_t launch_lamport_sum_f16(void* rbuf, int W, int64_t M, int64_t H, void* out,
                                  const ar_launch_cfg_t& c, arf::LamportSource src,
                                  hipStream_t s) {
  return launch_lamport_sum_t<F16>(rbuf, W, M, H, out, c, src, s);
}

hipError_t launch_lamport_norm_f16(void* rbuf, int W, const void* residual, const float* gamma,
                                   float eps, void* residual_out, void* norm_out, int64_t M,
                                   int64_t H, const ar_launch_cfg_t& c, arf::LamportSource src,
                                   hipStream_t s) {
  return launch_lamport_norm_t<F16>(rbuf, W, residual, gamma, eps, residual_out, norm_out, M,
                                      H, c, src, s);
}

hipError_t launch_lamport_push_f16(const void* partial, void* slot, void* next, int64_t nvec,
                                   int grid, hipStream_t s) {
  return launch_lamport_push_t<F16>(partial, slot, next, nvec, grid, s);
}

hipError_t launch_sum_residual_f16(const void* const* inputs, int W, const void* residual,
                                  void* out, int64_t nvec, int tail, const ar_launch_cfg_t& c,
                                  hipStream_t s) {
  return launch_sum_residual_t<F16>(inputs, W, residual, out, nvec, tail, c, s);
}

hipError_t launch_rmsnorm_f16(const void* x, const float* gamma, float eps, void* y,
                             int64_t M, int64_t H, const ar_launch_cfg_t& c, hipStream_t s) {
  return launch_rmsnorm_t<F16>(x, gamma, eps, y, M, H, c, s);
}

hipError_t launch_rmsnorm_rows_f16(const void* x, const float* gamma, float eps, void* y,
                                  int64_t M, int64_t H, int grid, int threads, int vecs_per_thread,
                                  hipStream_t s) {
  return launch_rmsnorm_rows_t<F16>(x, gamma, eps, y, M, H, grid, threads, vecs_per_thread, s);
}

hipError_t launch_norm_split_f16(const void* const* inputs, int W, const void* residual,
                              const float* gamma, float eps, void* residual_out, void* norm_out,
                              int64_t M, int64_t H, void* workspace, const SplitLaunch& c,
                              hipStream_t s) {
  return launch_norm_split_t<F16>(inputs, W, residual, gamma, eps, residual_out, norm_out, M, H,
                                  workspace, c, s);
}

}  // namespace arfh
