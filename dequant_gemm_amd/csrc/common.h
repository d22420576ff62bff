// common.h -- device helpers shared by the HIP kernels of libcubic (gfx950).
//
// Format and decode follow the CubicQuant article on ModelScope
// ("CubicQuant：用三次曲线重塑低比特量化，Kimi K3 2.5Bit 模型首发实践"), section
// "CubicQuant 核心：把直线网格掰弯": code k, Kmax = 2^(B-1) - 1, t = |k| / Kmax,
// q(t) = a t + b t^2 + (1 - a - b) t^3, w = s * sign(k) * q(t).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cubic {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kChunk = 32;      // codes per lane chunk: `bits` dwords of stream
constexpr int kStep = 128;      // codes per row per K-step (4 chunks)

__host__ __device__ constexpr int kmax_of(int bits) { return (1 << (bits - 1)) - 1; }

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

__device__ __forceinline__ double f16_bits_to_f64(uint16_t h) {
  _Float16 v = __builtin_bit_cast(_Float16, h);
  return static_cast<double>(v);
}

__device__ __forceinline__ uint16_t f16_bits(float v) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}

// Kmax^3 * q(j / Kmax) = a j Kmax^2 + b j^2 Kmax + (1 - a - b) j^3. For fp16 a, b
// with |a|, |b| <= 16 every term is an exact multiple of 2^-24 below 2^28, so the
// fp64 result is exact (core section of the CubicQuant article gives q and c).
__device__ __forceinline__ double level_numerator(double a, double b, int j, int km) {
  const double J = static_cast<double>(j), K = static_cast<double>(km);
  const double c = 1.0 - a - b;
  return a * (J * K * K) + b * (J * J * K) + c * (J * J * J);
}

// q(j / Kmax) in fp64 with a single rounding (IEEE division).
__device__ __forceinline__ double level_q(double a, double b, int j, int km) {
  const double K = static_cast<double>(km);
  return level_numerator(a, b, j, km) / (K * K * K);
}

// Two's complement value of a `bits`-wide field.
__device__ __forceinline__ int sign_extend(uint32_t field, int bits) {
  return static_cast<int>(field << (32 - bits)) >> (32 - bits);
}

// Field i (0..31) of a 32-code chunk held in `bits` consecutive dwords w[].
template <int BITS>
__device__ __forceinline__ uint32_t chunk_field(const uint32_t* w, int i) {
  const int bit = i * BITS;
  const int d = bit >> 5, off = bit & 31;
  uint32_t v;
  if (off + BITS <= 32) {
    v = w[d] >> off;
  } else {
    v = __builtin_amdgcn_alignbit(w[d + 1], w[d], off);
  }
  return v & ((1u << BITS) - 1u);
}

// The A8 carrier: clamp(RNE(127 * Q / Kmax^3), -127, 127), decided exactly with
// integers. a and b are fp16 so A = a * 2^24 and Bi = b * 2^24 are integers and
// Q * 2^24 = A j Kmax^2 + Bi j^2 Kmax + (2^24 - A - Bi) j^3 (int64, |.| < 2^52 for
// |a|,|b| <= 16). The quotient is estimated in fp64 and corrected by comparing
// twice the numerator against odd multiples of the denominator.
__device__ __forceinline__ int carrier_level(double a, double b, int j, int km) {
  const long long A = static_cast<long long>(a * 16777216.0);
  const long long Bi = static_cast<long long>(b * 16777216.0);
  const long long C = 16777216LL - A - Bi;
  const long long J = j, K = km;
  const long long Q = A * (J * K * K) + Bi * (J * J * K) + C * (J * J * J);
  const long long num = 127LL * Q;
  const long long den = (K * K * K) << 24;
  // Clamp early: beyond +-128 the exact rounding no longer matters.
  if (num >= 128LL * den) return 127;
  if (num <= -128LL * den) return -127;
  long long n = static_cast<long long>(rint(static_cast<double>(num) / static_cast<double>(den)));
  // Exact correction: r = 2*num - 2*n*den lies in (-den, den] after adjustment.
  long long r = 2 * num - 2 * n * den;
  while (r > den) { n += 1; r -= 2 * den; }
  while (r < -den) { n -= 1; r += 2 * den; }
  if (r == den && (n & 1)) n += 1;          // tie above n: go to even
  if (r == -den && (n & 1)) n -= 1;         // tie below n: go to even
  if (n > 127) n = 127;
  if (n < -127) n = -127;
  return static_cast<int>(n);
}

// Power-of-two prescale of a row before its fp16 conversion: returns the shift
// n such that ldexpf(amax, n) lies in [2^14, 2^15), and writes 2^-n to *back.
// Zero, NaN and Inf rows are left unscaled (n = 0).
__device__ __forceinline__ int row_prescale(float amax, float* back) {
  if (!(amax > 0.0f) || !(amax <= 3.4e38f)) {
    *back = 1.0f;
    return 0;
  }
  const int e = ilogbf(amax);                   // floor(log2(amax)), exact
  *back = ldexpf(1.0f, e - 14);                 // >= 2^-147: representable
  return 14 - e;
}

// Orders this wave's earlier LDS writes before its later LDS reads. The LDS
// executes one wave's instructions in order, so only the compiler must not
// move memory accesses across this point; unlike a release fence it does not
// wait for outstanding global loads.
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// Wave-wide max via xor shuffles.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace cubic
