// decode.h -- tile-local decode of a lane's 32-code chunk into MFMA operand
// registers (8 fp16 per fragment, 4 fragments per chunk).
//
// The fused path of the CubicQuant article (section "压缩权重必须边解码、边计算",
// flow figure): codes and group parameters are unpacked inside the tile, turned
// into levels in a temporary dtype and fed straight into the dot product; the
// group scale is applied in fp32 afterwards. Here the temporary dtype is fp16
// holding the normalised level q (|q| <= 1 for the symmetric codes), and the
// fp32 group scale multiplies each group's MFMA partial sums.
//
// The order in which a chunk's 32 codes land in the 32 k-slots of the four
// fragments is free (the reduction does not care) as long as the activation
// fragments use the same order; slot_to_code() gives that order and the
// activation staging code writes x in it.
#pragma once
#include "common.h"

namespace cubic {

// ---------------------------------------------------------------------------
// 2-bit codes. The symmetric codes {-1, 0, +1} are 11, 00, 01. Shifting the
// chunk word so that code i sits at bits [15:14] and code i+8 at [31:30] and
// masking with 0xC000C000 yields the 16-bit pair (2k_i, 2k_{i+8}) with 0x4000 =
// +2, 0xC000 = -2, 0 = 0: the same bit patterns in bf16 and fp16. These levels
// (in units of s/2) are exact in bf16, so 2-bit weights multiply the bf16
// activations directly on the bf16 MFMA (every product exact, no conversion or
// prescale of x). The fourth field value 10 (code -2, which a symmetric
// quantiser never writes) reads as -0.0 and contributes nothing; when a wave
// sees it, two more MFMAs add x * hi and x * lo at those positions, with
// hi = bf16(-2 q(2)) and lo = bf16(-2 q(2) - hi) (~16 significant bits).
// ---------------------------------------------------------------------------
struct DecodeW2 {
  static constexpr int kBits = 2;
  static constexpr bool kBf16 = true;
  static constexpr float kLevelUnit = 0.5f;   // decoded value * s * 0.5 = weight

  __host__ __device__ static int slot_to_code(int slot) {
    const int r = slot >> 1, h = slot & 1;
    return 16 * (r >> 3) + (r & 7) + 8 * h;
  }
  __host__ __device__ static int code_to_slot(int c) {
    const int d = c >> 4, rem = c & 15, h = rem >> 3, i = rem & 7;
    return 2 * (8 * d + i) + h;
  }
  // bit 2j+1 set iff field j of the word is 10 (code -2)
  __device__ static uint32_t extra_bits(uint32_t w) { return w & ~(w << 1) & 0xAAAAAAAAu; }
  __device__ static void fast(const uint32_t* w, uint32_t* r) {
#pragma unroll
    for (int d = 0; d < 2; ++d) {
#pragma unroll
      for (int i = 0; i < 8; ++i) r[8 * d + i] = (w[d] << (14 - 2 * i)) & 0xC000C000u;
    }
  }
  // Fragments holding hi (rhi) and lo (rlo) at the halves whose field is 10
  // (code -2) and zero elsewhere; fast() contributes exactly 0 (-0.0) there.
  __device__ static void extra(const uint32_t* w, uint32_t hi, uint32_t lo, uint32_t* rhi,
                               uint32_t* rlo) {
    const uint32_t hi2 = (hi & 0xffffu) | (hi << 16);
    const uint32_t lo2 = (lo & 0xffffu) | (lo << 16);
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const uint32_t e = extra_bits(w[d]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t m = (e << (14 - 2 * i)) & 0x80008000u;    // flags at bits 15 and 31
        const uint32_t mm = (m >> 15) * 0xffffu;
        rhi[8 * d + i] = mm & hi2;
        rlo[8 * d + i] = mm & lo2;
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Any width: natural order (register r holds codes 2r, 2r+1); each field indexes
// a per-row fp16 table of 2^B normalised levels kept in LDS. Level unit 1.
// ---------------------------------------------------------------------------
template <int BITS>
struct DecodeTable {
  static constexpr int kBits = BITS;
  static constexpr bool kBf16 = false;
  static constexpr float kLevelUnit = 1.0f;
  __host__ __device__ static int slot_to_code(int slot) { return slot; }
  __host__ __device__ static int code_to_slot(int c) { return c; }
  // tab: this lane's row table (2^B fp16 entries)
  __device__ static void decode(const uint32_t* w, const uint16_t* tab, uint32_t* r) {
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const uint32_t lo = tab[chunk_field<BITS>(w, 2 * p)];
      const uint32_t hi = tab[chunk_field<BITS>(w, 2 * p + 1)];
      r[p] = lo | (hi << 16);
    }
  }
};

// Normalised fp16 level of field value v (two's complement, `bits` wide).
// bf16 bit pattern of v, round to nearest even (finite v).
__device__ __forceinline__ uint32_t bf16_rne_bits(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint16_t table_entry(double a, double b, uint32_t v, int bits) {
  const int k = sign_extend(v, bits);
  const int j = k < 0 ? -k : k;
  const int km = kmax_of(bits);
  const double K = static_cast<double>(km);
  const float q = static_cast<float>(level_numerator(a, b, j, km) * (1.0 / (K * K * K)));
  return f16_bits(k < 0 ? -q : q);
}

}  // namespace cubic
