// ar_oracle.cpp -- the plain CPU oracle for the fused all-reduce-sum (+ residual + RMSNorm) path.
//
// TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct definition that the HIP
// kernels are checked against.  Only the test suite, the smoke check and the benchmark's CPU
// baseline leg may load it.  The product library never links, loads or calls it, and it shares
// no code, header, table or helper with the HIP path.
//
// What is computed (sources):
//  * The two fusion patterns are named "kAllReduce" and "kARResidualRMSNorm" in the tokenspeed
//    pull request "perf(comm): route generic MNNVL AR patterns to upstream flashinfer"
//    (Summary / Routing).  The pages give the names only; the arithmetic below is the plainest
//    reading of those names:
//      kAllReduce          out          = sum over ranks r = 0..W-1 of x_r
//      kARResidualRMSNorm  residual_out = sum over ranks + residual
//                          norm_out     = RMSNorm(residual_out) * gamma
//  * The rank sum is an element-wise binary32 sum in the fixed rank order 0..W-1, one rounding
//    per add (round-to-nearest-even), seeded with the first rank's value (so -0 survives a sum
//    of negative zeros).  The residual enters after all W partials, and the result is rounded
//    once to the storage type T.
//  * RMSNorm is the textbook form (Zhang & Sennrich 2019, "Root Mean Square Layer
//    Normalization"): mean of squares over the whole hidden row, eps added to that mean inside
//    the square root, gamma applied after normalising, no bias.  It reads the stored, rounded
//    residual_out, so norm_out equals RMSNorm of the tensor an unfused caller would see.  The
//    pages give no formula; this is a stated reading.
//  * The norm is evaluated in binary64 (sum of squares, mean, reciprocal square root, scale),
//    then rounded to binary32 and then to T.
//  * World sizes: the vLLM pull request "[Perf] Tune FlashInfer all-reduce selection on SM103"
//    (Scope) gives {2, 4, 8, 16, 32, 64} as the supported set.  The oracle accepts any W >= 1;
//    range checks belong to the library boundary.
//
// Storage types: 0 = binary32, 1 = binary16, 2 = bfloat16.  16-bit values are carried as raw
// uint16 bit patterns.  The conversions below are this file's own, written from the IEEE 754
// definition of round-to-nearest-even (nearest representable value, ties to an even
// significand), with overflow to infinity and subnormal results kept (no flush to zero).
//
// Build: g++ -O2 -fPIC -shared -ffp-contract=off (no -ffast-math): x86-64 SSE arithmetic, no
// excess precision, no FTZ/DAZ.
//
// Parity status: every function here is pinned by the host tests: the conversions against
// numpy's and torch's casts (all 2^16 patterns for widening; every sign/exponent crossed with
// every rounding-critical low-bit pattern, plus a random sample, for narrowing), the sum by
// exact integer sums, closed forms, an exact-rational replay and the recursive-summation error
// bound, the norm by torch's float64 rms_norm, closed forms and exact invariances, and all of
// it by hand-derived golden rows.  No function here is "parity unpinned".

#include <cfenv>
#include <cmath>
#include <cstdint>
#include <cstring>

namespace {

enum StorageType { kF32 = 0, kF16 = 1, kBF16 = 2 };

uint32_t float_bits(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  return u;
}

float bits_float(uint32_t u) {
  float x;
  std::memcpy(&x, &u, 4);
  return x;
}

// Round a non-negative, finite double `a` to the nearest multiple of 2^q with ties to even.
// Returns the integer multiple.  `a / 2^q` is exact (a power-of-two scaling of a value that is
// far from the double range limits here), and nearbyint rounds ties to even in the default
// FE_TONEAREST mode.
double round_to_quantum(double a, int q) { return std::nearbyint(std::ldexp(a, -q)); }

// Generic binary32 -> narrow binary format, round-to-nearest-even.
//   mant_bits : stored significand bits of the target (10 for binary16, 7 for bfloat16)
//   exp_bits  : exponent field width of the target (5 for binary16, 8 for bfloat16)
// Result is the 16-bit pattern sign | exponent | significand.
uint16_t round_binary32_to_narrow(float x, int mant_bits, int exp_bits) {
  const uint32_t u = float_bits(x);
  const uint16_t sign = static_cast<uint16_t>((u >> 31) << 15);
  const uint16_t exp_all_ones = static_cast<uint16_t>(((1u << exp_bits) - 1u) << mant_bits);
  if (std::isnan(x)) {
    // Quiet NaN of the same sign; the top payload bits are kept and the quiet bit is set.
    const uint16_t payload = static_cast<uint16_t>((u & 0x007FFFFFu) >> (23 - mant_bits));
    return static_cast<uint16_t>(sign | exp_all_ones | (1u << (mant_bits - 1)) | payload);
  }
  if (std::isinf(x)) return static_cast<uint16_t>(sign | exp_all_ones);

  const double a = std::fabs(static_cast<double>(x));
  if (a == 0.0) return sign;

  const int bias = (1 << (exp_bits - 1)) - 1;
  const int emin = 1 - bias;                   // exponent of the smallest normal
  const int emax = bias;                       // exponent of the largest finite value
  int e2;
  std::frexp(a, &e2);                          // a = f * 2^e2, f in [0.5, 1)
  int e = e2 - 1;                              // a in [2^e, 2^(e+1))
  if (e < emin) {
    // Subnormal range of the target: fixed quantum 2^(emin - mant_bits).
    const double n = round_to_quantum(a, emin - mant_bits);
    // n in [0, 2^mant_bits]; n == 2^mant_bits is the smallest normal, whose bit pattern is
    // exactly n (exponent field 1, significand 0).
    return static_cast<uint16_t>(sign | static_cast<uint16_t>(n));
  }
  double n = round_to_quantum(a, e - mant_bits);  // n in [2^mant_bits, 2^(mant_bits+1)]
  if (n == std::ldexp(1.0, mant_bits + 1)) {     // rounded up into the next binade
    n = std::ldexp(1.0, mant_bits);
    e += 1;
  }
  if (e > emax) return static_cast<uint16_t>(sign | exp_all_ones);  // overflow -> infinity
  const uint32_t field = static_cast<uint32_t>(e + bias) << mant_bits;
  const uint32_t frac = static_cast<uint32_t>(n) - (1u << mant_bits);
  return static_cast<uint16_t>(sign | field | frac);
}

// bfloat16 is the top half of a binary32 pattern, so widening is a 16-bit shift.
float widen_bf16(uint16_t b) { return bits_float(static_cast<uint32_t>(b) << 16); }

// binary16 -> binary32, from the definition of the binary16 encoding.
float widen_f16(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int field = (h >> 10) & 0x1F;
  const int frac = h & 0x3FF;
  if (field == 0x1F) {
    // Infinity or NaN: same sign, all-ones exponent, payload moved to the top of the field.
    return bits_float((static_cast<uint32_t>(sign) << 31) | 0x7F800000u |
                      (static_cast<uint32_t>(frac) << 13));
  }
  double mag;
  if (field == 0) {
    mag = std::ldexp(static_cast<double>(frac), -24);            // subnormal: frac * 2^-24
  } else {
    mag = std::ldexp(static_cast<double>(1024 + frac), field - 25);  // (1.frac) * 2^(field-15)
  }
  const float v = static_cast<float>(mag);  // exact: binary16 values are binary32 values
  return sign ? -v : v;
}

// Read element i of a buffer of storage type `dtype`, widened exactly to binary32.
float load_widened(const void* p, int64_t i, int dtype) {
  if (dtype == kF32) return static_cast<const float*>(p)[i];
  const uint16_t b = static_cast<const uint16_t*>(p)[i];
  return dtype == kBF16 ? widen_bf16(b) : widen_f16(b);
}

// Round a binary32 value to the storage type and write it as element i.
void store_rounded(void* p, int64_t i, int dtype, float v) {
  if (dtype == kF32) {
    static_cast<float*>(p)[i] = v;
  } else if (dtype == kBF16) {
    static_cast<uint16_t*>(p)[i] = round_binary32_to_narrow(v, 7, 8);
  } else {
    static_cast<uint16_t*>(p)[i] = round_binary32_to_narrow(v, 10, 5);
  }
}

bool valid_dtype(int dtype) { return dtype == kF32 || dtype == kF16 || dtype == kBF16; }

// The binary32 rank chain for one element: a = x_0; a = a + x_1; ...; a = a + x_{W-1}.
float rank_sum(const void* const* inputs, int W, int64_t idx, int dtype) {
  float a = load_widened(inputs[0], idx, dtype);
  for (int r = 1; r < W; ++r) {
    const float x = load_widened(inputs[r], idx, dtype);
    a = a + x;  // one binary32 add, round-to-nearest-even
  }
  return a;
}

}  // namespace

extern "C" {

// ---- conversions (exposed so the tests can pin them exhaustively) --------------------------

uint16_t oracle_round_f32_to_bf16(float x) { return round_binary32_to_narrow(x, 7, 8); }
uint16_t oracle_round_f32_to_f16(float x) { return round_binary32_to_narrow(x, 10, 5); }
float oracle_widen_bf16(uint16_t b) { return widen_bf16(b); }
float oracle_widen_f16(uint16_t h) { return widen_f16(h); }

// Element-wise array forms of the above (dtype 1 = binary16, 2 = bfloat16).  Return 0, or -1
// for a bad dtype.
int oracle_round_f32_array(int dtype, const float* x, uint16_t* y, int64_t n) {
  if (dtype != kF16 && dtype != kBF16) return -1;
  for (int64_t i = 0; i < n; ++i) {
    y[i] = dtype == kBF16 ? round_binary32_to_narrow(x[i], 7, 8)
                          : round_binary32_to_narrow(x[i], 10, 5);
  }
  return 0;
}

int oracle_widen_array(int dtype, const uint16_t* x, float* y, int64_t n) {
  if (dtype != kF16 && dtype != kBF16) return -1;
  for (int64_t i = 0; i < n; ++i) y[i] = dtype == kBF16 ? widen_bf16(x[i]) : widen_f16(x[i]);
  return 0;
}

// ---- kAllReduce ------------------------------------------------------------------------------
//
// out[m, i] = RN_T( x_0[m, i] + x_1[m, i] + ... + x_{W-1}[m, i] ), binary32 chain in rank order.
// All buffers are row-major [M, H] of storage type `dtype`; rows [row0, row1) are computed.
// Returns 0, or -1 on a bad argument.
int oracle_ar_sum_rows(const void* const* inputs, int W, int64_t M, int64_t H, int dtype,
                       void* out, int64_t row0, int64_t row1) {
  if (!inputs || W < 1 || M < 0 || H < 0 || !valid_dtype(dtype) || !out) return -1;
  if (row0 < 0 || row1 > M || row0 > row1) return -1;
  if (std::fegetround() != FE_TONEAREST) return -1;
  for (int64_t m = row0; m < row1; ++m) {
    for (int64_t i = 0; i < H; ++i) {
      const int64_t idx = m * H + i;
      store_rounded(out, idx, dtype, rank_sum(inputs, W, idx, dtype));
    }
  }
  return 0;
}

int oracle_ar_sum(const void* const* inputs, int W, int64_t M, int64_t H, int dtype, void* out) {
  return oracle_ar_sum_rows(inputs, W, M, H, dtype, out, 0, M);
}

// ---- RMSNorm of one stored row ---------------------------------------------------------------------
//
// Row m of x ([M, H], storage type T):
//   v_i   = x_i widened exactly, then to binary64
//   rstd  = 1 / sqrt( (sum_i v_i^2) / H + eps )       (binary64, sequential sum over i = 0..H-1)
//   y_i   = v_i * rstd * gamma_i                       (binary64)
//   out_i = RN_T( RN_binary32(y_i) )
static void rmsnorm_row(const void* x, int64_t m, int64_t H, int dtype, const float* gamma,
                        float eps, void* out, double* y_dbg, double* rstd_dbg) {
  double sum_sq = 0.0;
  for (int64_t i = 0; i < H; ++i) {
    const double v = static_cast<double>(load_widened(x, m * H + i, dtype));
    sum_sq += v * v;
  }
  const double mean_sq = sum_sq / static_cast<double>(H);
  const double rstd = 1.0 / std::sqrt(mean_sq + static_cast<double>(eps));
  if (rstd_dbg) rstd_dbg[m] = rstd;
  for (int64_t i = 0; i < H; ++i) {
    const int64_t idx = m * H + i;
    const double v = static_cast<double>(load_widened(x, idx, dtype));
    const double y = v * rstd * static_cast<double>(gamma[i]);
    if (y_dbg) y_dbg[idx] = y;
    store_rounded(out, idx, dtype, static_cast<float>(y));
  }
}

// ---- kARResidualRMSNorm ------------------------------------------------------------------------
//
// For every row m in [row0, row1):
//   a_i            = x_0 + x_1 + ... + x_{W-1} + residual          (binary32 chain, in that order)
//   residual_out_i = RN_T(a_i)
//   v_i            = residual_out_i widened exactly, then to binary64
//   rstd           = 1 / sqrt( (sum_i v_i^2) / H + eps )           (binary64, sequential sum)
//   y_i            = v_i * rstd * gamma_i                          (binary64)
//   norm_out_i     = RN_T( RN_binary32(y_i) )
// gamma is binary32 [H] for every storage type.  y_dbg ([M, H] binary64) and rstd_dbg ([M]
// binary64) receive the unrounded intermediates when non-null.
// Returns 0, or -1 on a bad argument.
int oracle_ar_residual_rmsnorm_rows(const void* const* inputs, int W, int64_t M, int64_t H,
                                    int dtype, const void* residual, const float* gamma,
                                    float eps, void* residual_out, void* norm_out, double* y_dbg,
                                    double* rstd_dbg, int64_t row0, int64_t row1) {
  if (!inputs || W < 1 || M < 0 || H < 1 || !valid_dtype(dtype)) return -1;
  if (!residual || !gamma || !residual_out || !norm_out) return -1;
  if (row0 < 0 || row1 > M || row0 > row1) return -1;
  if (std::fegetround() != FE_TONEAREST) return -1;
  for (int64_t m = row0; m < row1; ++m) {
    // Residual add: the residual is one more term after the W partials.
    for (int64_t i = 0; i < H; ++i) {
      const int64_t idx = m * H + i;
      float a = rank_sum(inputs, W, idx, dtype);
      a = a + load_widened(residual, idx, dtype);
      store_rounded(residual_out, idx, dtype, a);
    }
    // RMSNorm of the stored residual_out row.
    rmsnorm_row(residual_out, m, H, dtype, gamma, eps, norm_out, y_dbg, rstd_dbg);
  }
  return 0;
}

int oracle_ar_residual_rmsnorm(const void* const* inputs, int W, int64_t M, int64_t H, int dtype,
                               const void* residual, const float* gamma, float eps,
                               void* residual_out, void* norm_out, double* y_dbg,
                               double* rstd_dbg) {
  return oracle_ar_residual_rmsnorm_rows(inputs, W, M, H, dtype, residual, gamma, eps,
                                         residual_out, norm_out, y_dbg, rstd_dbg, 0, M);
}

// ---- RMSNorm of a stored tensor -----------------------------------------------------------------
//
// The normalisation step of kARResidualRMSNorm applied to a tensor x that is already stored in T:
// out = RMSNorm(x) * gamma row by row, exactly as rmsnorm_row defines it (this is what an unfused
// caller runs after a separate sum-and-residual step).  Rows [row0, row1) only; y_dbg / rstd_dbg
// as above.  Returns 0, or -1 on a bad argument.
int oracle_rmsnorm_rows(const void* x, int64_t M, int64_t H, int dtype, const float* gamma,
                        float eps, void* out, double* y_dbg, double* rstd_dbg, int64_t row0,
                        int64_t row1) {
  if (!x || M < 0 || H < 1 || !valid_dtype(dtype) || !gamma || !out) return -1;
  if (row0 < 0 || row1 > M || row0 > row1) return -1;
  if (std::fegetround() != FE_TONEAREST) return -1;
  for (int64_t m = row0; m < row1; ++m) rmsnorm_row(x, m, H, dtype, gamma, eps, out, y_dbg, rstd_dbg);
  return 0;
}

}  // extern "C"
