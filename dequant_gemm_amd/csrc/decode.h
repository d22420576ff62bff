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
// masking with 0xC000C000 yields the fp16 pair (2k_i, 2k_{i+8}): 0x4000 = +2,
// 0xC000 = -2, 0 = 0. The fourth field value 10 (code -2, never produced by a
// symmetric quantiser) would read as -0.0; it is detected per chunk and, when
// present anywhere in the wave, the chunk is decoded again through the full
// four-entry table {0, 2, -2 q(2), -2}. Levels are in units of s/2.
// ---------------------------------------------------------------------------
struct DecodeW2 {
  static constexpr int kBits = 2;
  static constexpr float kLevelUnit = 0.5f;   // decoded value * s * 0.5 = weight

  __device__ static int slot_to_code(int slot) {
    const int r = slot >> 1, h = slot & 1;
    return 16 * (r >> 3) + (r & 7) + 8 * h;
  }
  __device__ static int code_to_slot(int c) {
    const int d = c >> 4, rem = c & 15, h = rem >> 3, i = rem & 7;
    return 2 * (8 * d + i) + h;
  }
  // true if a field value 10 (code -2) is present in the chunk
  __device__ static bool has_extra(const uint32_t* w) {
    const uint32_t t = ((w[0] & ~(w[0] << 1)) | (w[1] & ~(w[1] << 1))) & 0xAAAAAAAAu;
    return t != 0u;
  }
  __device__ static void fast(const uint32_t* w, uint32_t* r) {
#pragma unroll
    for (int d = 0; d < 2; ++d) {
#pragma unroll
      for (int i = 0; i < 8; ++i) r[8 * d + i] = (w[d] << (14 - 2 * i)) & 0xC000C000u;
    }
  }
  // Full table decode; q2 = q(2) of the current group (t = 2 for Kmax = 1).
  __device__ static void full(const uint32_t* w, float q2, uint32_t* r) {
    const uint32_t t2 = f16_bits(-2.0f * q2);
    const uint32_t tab_lo = 0x40000000u | 0x00000000u;   // fields 0, 1 -> 0x0000, 0x4000
    const uint32_t tab_hi = 0xC0000000u | t2;            // fields 2, 3 -> -2 q(2), 0xC000
#pragma unroll
    for (int d = 0; d < 2; ++d) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t f0 = (w[d] >> (2 * i)) & 3u, f1 = (w[d] >> (2 * i + 16)) & 3u;
        const uint32_t v0 = (f0 < 2 ? (tab_lo >> (16 * f0)) : (tab_hi >> (16 * (f0 - 2)))) & 0xffffu;
        const uint32_t v1 = (f1 < 2 ? (tab_lo >> (16 * f1)) : (tab_hi >> (16 * (f1 - 2)))) & 0xffffu;
        r[8 * d + i] = v0 | (v1 << 16);
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
  static constexpr float kLevelUnit = 1.0f;
  __device__ static int slot_to_code(int slot) { return slot; }
  __device__ static int code_to_slot(int c) { return c; }
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
__device__ __forceinline__ uint16_t table_entry(double a, double b, uint32_t v, int bits) {
  const int k = sign_extend(v, bits);
  const int j = k < 0 ? -k : k;
  const int km = kmax_of(bits);
  const double K = static_cast<double>(km);
  const float q = static_cast<float>(level_numerator(a, b, j, km) * (1.0 / (K * K * K)));
  return f16_bits(k < 0 ? -q : q);
}

}  // namespace cubic
