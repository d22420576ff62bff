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


// The format's fp32 value of a level: RN32(s * q(j / Kmax)), the exact product
// s * Q_j / Kmax^3 rounded once to the nearest fp32 value (ties to even), an
// exact zero as +0.0 (core section of the CubicQuant article gives q; the storage
// section stores s in fp32 and a, b in fp16). Exact for every finite fp32 s and
// every finite fp16 a, b; a non-finite s gives the fp64 product's rounding.
//
// Fast path: R = Q_j * 2^24 is an integer (a, b are multiples of 2^-24). When
// |R| < 2^53, y = fl(s * fl(R * fl(2^-24 / Kmax^3))) carries three roundings and
// lies within 2^-51 |V| of V = s * Q_j / Kmax^3; if no fp32 rounding boundary
// (the midpoint between two neighbouring fp32 values) lies within 2^-51 |y| of
// y, RN32(V) = RN32(y). Otherwise the exact path decides with 128-bit integers:
// |V| = P * 2^(es - 24) / D with P = |S * R|, s = S * 2^es and D = Kmax^3, its
// binade E found exactly, and the significand n = |V| / 2^(E - 23) rounded
// half to even from the integer remainder.
namespace level_detail {
typedef __int128 i128;
typedef unsigned __int128 u128;

__host__ __device__ inline double u128_to_f64(u128 v) {
  return static_cast<double>(static_cast<uint64_t>(v >> 64)) * 0x1p64 +
         static_cast<double>(static_cast<uint64_t>(v));
}

// P >= D * 2^t, exactly (P < 2^90, D < 2^21).
__host__ __device__ inline bool ge_pow2(u128 P, u128 D, int t) {
  if (t >= 0) return t < 100 && P >= (D << t);
  const int u = -t;
  if (u >= 64) return true;                       // P >= 1 > D * 2^-64
  return P >= ((D + ((static_cast<u128>(1) << u) - 1)) >> u);
}

__host__ __device__ __attribute__((noinline)) inline float exact(float s, i128 R, int64_t km) {
  const uint32_t sb = __builtin_bit_cast(uint32_t, s);
  const int ex = static_cast<int>((sb >> 23) & 0xffu);
  uint64_t S = sb & 0x7fffffu;
  int es;
  if (ex == 0) {
    es = -149;
  } else {
    S |= 0x800000u;
    es = ex - 150;
  }
  const bool neg = ((sb >> 31) != 0) != (R < 0);
  const u128 P = static_cast<u128>(R < 0 ? -R : R) * S;
  if (P == 0) return 0.0f;
  const u128 D = static_cast<u128>(km * km * km);
  int xe = 0;
  frexp(ldexp(u128_to_f64(P) / u128_to_f64(D), es - 24), &xe);
  int E = xe - 1;                                 // estimate of floor(log2 |V|)
  for (int it = 0; it < 4 && !ge_pow2(P, D, E + 24 - es); ++it) --E;
  for (int it = 0; it < 4 && ge_pow2(P, D, E + 25 - es); ++it) ++E;
  if (E >= 128) return neg ? -__builtin_inff() : __builtin_inff();
  const int u = (E < -126 ? -126 : E) - 23;       // exponent of the fp32 ulp at |V|
  const int sh = es - 24 - u;                     // n = P * 2^sh / D
  const u128 num = sh >= 0 ? (P << sh) : P;
  const u128 den = sh >= 0 ? D : (D << (-sh));
  uint64_t n = static_cast<uint64_t>(u128_to_f64(num) / u128_to_f64(den));
  i128 r = static_cast<i128>(num) - static_cast<i128>(n) * static_cast<i128>(den);
  for (int it = 0; it < 4 && r < 0; ++it) { --n; r += static_cast<i128>(den); }
  for (int it = 0; it < 4 && r >= static_cast<i128>(den); ++it) { ++n; r -= static_cast<i128>(den); }
  const i128 r2 = 2 * r;
  if (r2 > static_cast<i128>(den) || (r2 == static_cast<i128>(den) && (n & 1u))) ++n;
  const float v = ldexpf(static_cast<float>(n), u);   // n <= 2^24: exact
  return neg ? -v : v;
}
}  // namespace level_detail

// RN32(y) when y (within 2^-51 |V| of V) decides RN32(V); false otherwise.
// In the normal fp32 range, rounding y to fp32 drops the low 29 bits of its
// fp64 significand, and the fp32 rounding boundaries (midpoints) are where
// those bits equal 2^28. |V - y| < 2^-51 |y| < 4 fp64 ulps of y, so when the
// dropped bits lie more than 8 ulps from 2^28, V rounds like y (near the
// representable points at 0 and 2^29 both round to the same fp32 number, also
// across a power of two). Outside the normal range the caller decides exactly.
__host__ __device__ inline bool level_fast(double y, float* out) {
  const uint64_t u = __builtin_bit_cast(uint64_t, y);
  const uint32_t ex = static_cast<uint32_t>(u >> 52) & 0x7ffu;
  if (ex < 1023u - 126u || ex > 1023u + 127u) return false;
  const uint32_t low = static_cast<uint32_t>(u) & ((1u << 29) - 1u);
  const uint32_t dist = low > (1u << 28) ? low - (1u << 28) : (1u << 28) - low;
  if (dist <= 8u) return false;
  *out = static_cast<float>(y);
  return true;
}

// Kmax^3 * q(j / Kmax) * 2^24 as an exact integer, for fp16 values a, b.
__host__ __device__ inline level_detail::i128 level_numerator_i(float a, float b, int j, int km) {
  using level_detail::i128;
  const int64_t A = static_cast<int64_t>(static_cast<double>(a) * 16777216.0);
  const int64_t Bq = static_cast<int64_t>(static_cast<double>(b) * 16777216.0);
  const int64_t C = 16777216 - A - Bq;
  const int64_t J = j, K = km;
  return static_cast<i128>(A) * (J * K * K) + static_cast<i128>(Bq) * (J * J * K) +
         static_cast<i128>(C) * (J * J * J);
}

// level_rn32 for a numerator R = Kmax^3 q_j 2^24 given as an integer-valued
// double with |R| < 2^53 (exact), and a finite s.
__host__ __device__ inline float level_rn32_r(float s, double R, int km) {
  if (R == 0.0 || s == 0.0f) return 0.0f;
  const double inv = 0x1p-24 / static_cast<double>(static_cast<int64_t>(km) * km * km);
  float v;
  if (level_fast(static_cast<double>(s) * (R * inv), &v)) return v;
  return level_detail::exact(s, static_cast<level_detail::i128>(static_cast<int64_t>(R)), km);
}

__host__ __device__ inline float level_rn32(float s, float a, float b, int j, int km) {
  using level_detail::i128;
  const i128 R = level_numerator_i(a, b, j, km);
  if (R == 0 || s == 0.0f) return 0.0f;
  const double inv = 0x1p-24 / static_cast<double>(static_cast<int64_t>(km) * km * km);
  if (!(fabsf(s) <= 3.4028234663852886e38f))
    return static_cast<float>(static_cast<double>(s) * (level_detail::u128_to_f64(R < 0 ? -R : R) * inv) *
                              (R < 0 ? -1.0 : 1.0));
  const i128 lim = static_cast<i128>(1) << 53;
  if (R < lim && R > -lim) {
    float v;
    if (level_fast(static_cast<double>(s) * (static_cast<double>(static_cast<int64_t>(R)) * inv), &v)) return v;
  }
  return level_detail::exact(s, R, km);
}

// bf16 bit pattern of an fp32 value, rounded to nearest even (finite values).
__device__ __forceinline__ uint32_t bf16_rne_bits(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Output element idx of a row-major array of fp32, or of bf16 when bf16 is set
// (the fp32 value rounded to nearest even; NaN stays a quiet NaN).
__device__ __forceinline__ void store_out(float* y, bool bf16, int64_t idx, float v) {
  if (bf16) {
    const uint32_t h = (v != v) ? ((__float_as_uint(v) >> 16) | 0x40u) : bf16_rne_bits(v);
    reinterpret_cast<uint16_t*>(y)[idx] = static_cast<uint16_t>(h);
  } else {
    y[idx] = v;
  }
}

// Four consecutive outputs starting at idx (idx a multiple of 4, the array
// 16-byte aligned): one 16-byte fp32 or 8-byte bf16 store.
__device__ __forceinline__ void store_out4(float* y, bool bf16, int64_t idx, const float* v) {
  if (bf16) {
    uint32_t h[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) h[r] = (v[r] != v[r]) ? ((__float_as_uint(v[r]) >> 16) | 0x40u) : bf16_rne_bits(v[r]);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + idx) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
  } else {
    *reinterpret_cast<f32x4*>(y + idx) = f32x4{v[0], v[1], v[2], v[3]};
  }
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

// carrier_level for fp16 a and b with |a|, |b| <= 16, in fp64 with no integer
// products and no division. S = Kmax^3 q(j / Kmax) = a X + b Y + j^3 (X = j Kmax^2
// - j^3, Y = j^2 Kmax - j^3, integers below 2^21 for j <= 128) is a multiple of
// 2^-24 below 2^27 in magnitude, so the two fmas that form it are exact. Then
// Xq = S * fl(127 / Kmax^3) lies within 2^-44 of 127 S / Kmax^3, so n0 = rint(Xq)
// is the correctly rounded carrier or one off it next to a tie; the residual D =
// 127 S - Kmax^3 n0 (a multiple of 2^-24 below 2^21) comes out of one fma
// exactly, and comparing it with Kmax^3 / 2 settles the off-by-one case and ties
// (to even).
__device__ __forceinline__ int carrier_exact(double a, double b, int j, int km) {
  const double j3 = static_cast<double>(j * j * j);
  const double X = static_cast<double>(j * km * km) - j3;
  const double Y = static_cast<double>(j * j * km) - j3;
  const double K3 = static_cast<double>(km * km * km);
  const double S = fma(a, X, fma(b, Y, j3));
  const double Xq = S * (127.0 / K3);
  if (Xq >= 127.75) return 127;                 // rounds to 128 or more: clamped
  if (Xq <= -127.75) return -127;
  const double n0 = rint(Xq);
  const double D = fma(127.0, S, -K3 * n0);
  const double h = 0.5 * K3;
  int n = static_cast<int>(n0);
  const bool odd = (n & 1) != 0;
  n += (D > h || (D == h && odd)) ? 1 : 0;
  n -= (D < -h || (D == -h && odd)) ? 1 : 0;
  return n > 127 ? 127 : (n < -127 ? -127 : n);
}

// carrier_level for fp16 a and b, decided in fp32 where that is safe: with
// X = j K^2 - j^3 and Y = j^2 K - j^3 (integers below 2^21), y = 127 (j^3 + a X +
// b Y) / K^3 takes two fmas and one multiply. For |a|, |b| <= 16 and K <= 127 the
// terms stay below 2^26, so y is within 3e-4 of 127 q_j; when y lies within 1e-3
// of a half-integer (a possible tie or a rounding the estimate could get wrong)
// carrier_exact decides, and for a or b outside that range the integer rule.
__device__ __forceinline__ int carrier_fast(float a, float b, int j, int km) {
  const float j3 = static_cast<float>(j * j * j);
  const float X = static_cast<float>(j * km * km) - j3;
  const float Y = static_cast<float>(j * j * km) - j3;
  const float y = fmaf(a, X, fmaf(b, Y, j3)) * (127.0f / static_cast<float>(km * km * km));
  const float r = rintf(y);
  const bool near_tie = fabsf(fabsf(y - r) - 0.5f) < 1e-3f;
  const bool small = fabsf(a) <= 16.0f && fabsf(b) <= 16.0f;
  if (near_tie || !small) {
    return small ? carrier_exact(static_cast<double>(a), static_cast<double>(b), j, km)
                 : carrier_level(static_cast<double>(a), static_cast<double>(b), j, km);
  }
  const int n = static_cast<int>(r);
  return n > 127 ? 127 : (n < -127 ? -127 : n);
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

// 64-bit left shift of a register pair by a constant, as one v_lshlrev_b64
// (the compiler otherwise splits a constant 64-bit shift into 32-bit ones).
template <int S>
__device__ __forceinline__ uint64_t shl64(uint64_t v) {
  uint64_t r;
  asm("v_lshlrev_b64 %0, %1, %2" : "=v"(r) : "n"(S), "v"(v));
  return r;
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
