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
#include <utility>

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
// F16: the same decode against fp16 activations (the values 0, +-2.0 have the
// same bit patterns in fp16), multiplied on the fp16 MFMA.
template <bool F16>
struct DecodeW2T {
  static constexpr int kBits = 2;
  static constexpr bool kBf16 = !F16;
  static constexpr bool kSplit = false;
  static constexpr bool kDirect = false;
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
  // The OR of extra_bits over NW words (NW even): each pair w[d + 1]:w[d] is
  // shifted as one 64-bit word; the bit w[d] carries into w[d + 1] lands at bit
  // 0, which the mask clears.
  template <int NW>
  __device__ static uint32_t extra_bits_or(const uint32_t* w) {
    uint32_t acc = 0;
#pragma unroll
    for (int d = 0; d < NW; d += 2) {
      const uint64_t t = shl64<1>((static_cast<uint64_t>(w[d + 1]) << 32) | w[d]);
      acc |= w[d] & ~static_cast<uint32_t>(t);
      acc |= w[d + 1] & ~static_cast<uint32_t>(t >> 32);
    }
    return acc & 0xAAAAAAAAu;
  }
  // r[i] and r[8 + i] come from one 64-bit shift of the pair w[1]:w[0]: the
  // bits w[0] carries into w[1] land below bit 14 and are masked off.
  __device__ static void fast(const uint32_t* w, uint32_t* r) {
    const uint64_t v = (static_cast<uint64_t>(w[1]) << 32) | w[0];
    auto one = [&](auto i_c) {
      constexpr int i = decltype(i_c)::value;
      uint64_t t = v;                        // i = 7: the fields are in place
      if constexpr (i < 7) t = shl64<14 - 2 * i>(v);
      r[i] = static_cast<uint32_t>(t) & 0xC000C000u;
      r[8 + i] = static_cast<uint32_t>(t >> 32) & 0xC000C000u;
    };
    [&]<int... I>(std::integer_sequence<int, I...>) {
      (one(std::integral_constant<int, I>{}), ...);
    }(std::make_integer_sequence<int, 8>{});
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
using DecodeW2 = DecodeW2T<false>;
using DecodeW2H = DecodeW2T<true>;

// ---------------------------------------------------------------------------
// Any width: natural order (register r holds codes 2r, 2r+1); each field indexes
// a per-row fp16 table of 2^B normalised levels kept in LDS. Level unit 1.
// ---------------------------------------------------------------------------
template <int BITS>
struct DecodeTable {
  static constexpr int kBits = BITS;
  static constexpr bool kBf16 = false;
  static constexpr bool kSplit = false;
  static constexpr bool kDirect = false;
  static constexpr float kLevelUnit = 1.0f;
  __host__ __device__ static int slot_to_code(int slot) { return slot; }
  __host__ __device__ static int code_to_slot(int c) { return c; }
  // Rows of a wave's tables are 2^B / 2 LDS words apart, so rows n and
  // n + 64 / 2^B share banks, and skewed code distributions (most fields near
  // zero) make their lanes collide. Entry f of row n is therefore stored at
  // f ^ swizzle(n), which spreads those rows over different words.
  __host__ __device__ static constexpr int swizzle(int n) {
    return (1 << BITS) > 64 ? 0 : 2 * ((n / (64 >> BITS)) % ((1 << BITS) / 2));
  }
  // tab: this lane's row table (2^B fp16 entries), aligned to its own size, so
  // the byte address of entry f is tab | ((f ^ swz) << 1): two ALU ops per code
  // (shift, and-xor). The two entries of a pair load straight into the low and
  // high halves of r[p] (ds_read_u16_d16 / _d16_hi).
  __device__ static void decode(const uint32_t* w, const uint16_t* tab, int swz, uint32_t* r) {
    typedef __attribute__((address_space(3))) const uint16_t lds_u16;
    typedef unsigned short u16x2v __attribute__((ext_vector_type(2)));
    const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(tab)) |
                          (static_cast<uint32_t>(swz) << 1);
    constexpr uint32_t kMask2 = ((1u << BITS) - 1u) << 1;
    auto addr = [&](int i) {
      const int bit = i * BITS;
      const int d = bit >> 5, off = bit & 31;
      uint32_t v;
      if (off == 0) {
        v = w[d] << 1;
      } else if (off + BITS <= 32) {
        v = w[d] >> (off - 1);
      } else {
        v = __builtin_amdgcn_alignbit(w[d + 1], w[d], off - 1);
      }
      return (v & kMask2) ^ base;
    };
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      u16x2v h;
      h.x = *reinterpret_cast<const lds_u16*>(static_cast<uintptr_t>(addr(2 * p)));
      h.y = *reinterpret_cast<const lds_u16*>(static_cast<uintptr_t>(addr(2 * p + 1)));
      r[p] = __builtin_bit_cast(uint32_t, h);
    }
  }
};

// Normalised fp16 level of field value v (two's complement, `bits` wide).
// bf16 bit pattern of v, round to nearest even (finite v).
// The same level in fp32, for the per-group tables of the products: with
// X = j K^2 - j^3 and Y = j^2 K - j^3 (integers, exact in fp32), a X and b Y
// are exact fp32 products of fp16 values while X, Y stay below 2^13 (B <= 5)
// and round once otherwise, so Q = j^3 + a X + b Y carries a few roundings in
// fp32, then one more by 1/K^3, before the 16-bit rounding of the entry: a few
// fp32 ulps, far inside the products' tolerance.
__device__ __forceinline__ float table_level_f32(float a, float b, uint32_t v, int bits) {
  const int k = sign_extend(v, bits);
  const int j = k < 0 ? -k : k;
  const int km = kmax_of(bits);
  const float X = static_cast<float>(j * km * km - j * j * j);
  const float Y = static_cast<float>(j * j * km - j * j * j);
  const float q = fmaf(a, X, fmaf(b, Y, static_cast<float>(j * j * j))) *
                  (1.0f / static_cast<float>(km * km * km));
  return k < 0 ? -q : q;
}

__device__ __forceinline__ uint16_t table_entry_f32(float a, float b, uint32_t v, int bits) {
  return f16_bits(table_level_f32(a, b, v, bits));
}

// A level as two bf16 halves of one dword: hi = rne(q) in the low half,
// lo = rne(q - hi) in the high half (hi + lo carries about 16 significant bits).
__device__ __forceinline__ uint32_t split_bf16_pair(float q) {
  const uint32_t hi = bf16_rne_bits(q);
  const uint32_t lo = bf16_rne_bits(q - __uint_as_float(hi << 16));
  return hi | (lo << 16);
}

// ---------------------------------------------------------------------------
// Any width, against raw bf16 activations: the per-row table holds every level
// as a bf16 (hi, lo) pair in one dword (split_bf16_pair), so the activations
// need neither a prescale nor a conversion. Natural order, level unit 1. A pair
// of codes gives one hi fragment dword and one lo fragment dword (two v_perm),
// and the chunk takes two bf16 MFMAs per fragment: sum x * hi + sum x * lo.
// ---------------------------------------------------------------------------
template <int BITS>
struct DecodeTableSplit {
  static constexpr int kBits = BITS;
  static constexpr bool kBf16 = true;
  static constexpr bool kSplit = true;
  static constexpr bool kDirect = false;
  static constexpr float kLevelUnit = 1.0f;
  __host__ __device__ static int slot_to_code(int slot) { return slot; }
  __host__ __device__ static int code_to_slot(int c) { return c; }
  // Rows are 2^B LDS words apart; entry f of row n sits at f ^ swizzle(n) so
  // that rows n and n + 32 / 2^B, which share banks, use different words.
  __host__ __device__ static constexpr int swizzle(int n) {
    return (1 << BITS) >= 32 ? 0 : (n / (32 >> BITS)) % (1 << BITS);
  }
  // tab: this lane's row table (2^B dwords), aligned to its own size: entry f
  // is at byte tab | ((f ^ swz) << 2).
  __device__ static void decode(const uint32_t* w, const uint32_t* tab, int swz, uint32_t* rhi,
                                uint32_t* rlo) {
    typedef __attribute__((address_space(3))) const uint32_t lds_u32;
    const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(tab)) |
                          (static_cast<uint32_t>(swz) << 2);
    constexpr uint32_t kMask4 = ((1u << BITS) - 1u) << 2;
    auto addr = [&](int i) {
      const int bit = i * BITS;
      const int d = bit >> 5, off = bit & 31;
      uint32_t v;
      if (off < 2) {
        v = w[d] << (2 - off);
      } else if (off + BITS <= 32) {
        v = w[d] >> (off - 2);
      } else {
        v = __builtin_amdgcn_alignbit(w[d + 1], w[d], off - 2);
      }
      return (v & kMask4) ^ base;
    };
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const uint32_t d0 = *reinterpret_cast<const lds_u32*>(static_cast<uintptr_t>(addr(2 * p)));
      const uint32_t d1 = *reinterpret_cast<const lds_u32*>(static_cast<uintptr_t>(addr(2 * p + 1)));
      rhi[p] = __builtin_amdgcn_perm(d1, d0, 0x05040100u);
      rlo[p] = __builtin_amdgcn_perm(d1, d0, 0x07060302u);
    }
  }
};

// ---------------------------------------------------------------------------
// Wide codes (7 and 8 bits), levels computed per code: a row's 2^B-entry table
// would be rebuilt for every group (128 codes per row at G = 128) and cost more
// than the codes it serves. With t = |k| / Kmax the level is
// q = t (a + t (b + t c)), c = 1 - a - b, in fp32 (a few ulps), signed like k,
// then rounded to the operand type. SPLIT: bf16 hi = rne(q) and lo = rne(q - hi)
// against raw bf16 activations (two MFMAs per fragment); otherwise fp16 against
// prescaled fp16 activations. Natural order, level unit 1.
// ---------------------------------------------------------------------------
template <int BITS, bool SPLIT>
struct DecodeDirect {
  static constexpr int kBits = BITS;
  static constexpr bool kBf16 = SPLIT;
  static constexpr bool kSplit = SPLIT;
  static constexpr bool kDirect = true;
  static constexpr float kLevelUnit = 1.0f;
  __host__ __device__ static int slot_to_code(int slot) { return slot; }
  __host__ __device__ static int code_to_slot(int c) { return c; }
  __host__ __device__ static constexpr int swizzle(int) { return 0; }

  // Per-group constants of the Horner form, from the (a, b) word.
  struct Coef {
    float a, b, c;
  };
  __device__ static Coef coef(uint32_t ab) {
    const float a = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(ab & 0xffffu)));
    const float b = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(ab >> 16)));
    return Coef{a, b, (1.0f - a) - b};
  }

  // q of the chunk's 32 codes (w: BITS dwords), as 16 fp16 pairs (r) or 16 bf16
  // hi pairs (r) and 16 bf16 lo pairs (rl).
  __device__ static void decode(const uint32_t* w, const Coef& k, uint32_t* r, uint32_t* rl) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    constexpr float kInv = 1.0f / static_cast<float>((1 << (BITS - 1)) - 1);
    auto level = [&](int i) {
      const int bit = i * BITS;
      const int d = bit >> 5, off = bit & 31;
      int v;
      if (off + BITS <= 32) {
        v = __builtin_amdgcn_sbfe(w[d], off, BITS);
      } else {
        v = __builtin_amdgcn_sbfe(__builtin_amdgcn_alignbit(w[d + 1], w[d], off), 0, BITS);
      }
      const float kf = static_cast<float>(v);
      const float t = fabsf(kf) * kInv;
      const float q = t * fmaf(t, fmaf(t, k.c, k.b), k.a);
      return copysignf(q, kf);
    };
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const f2 q = {level(2 * p), level(2 * p + 1)};
      if constexpr (SPLIT) {
        const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(q, b2));
        const f2 h = {__uint_as_float(hi << 16), __uint_as_float(hi & 0xffff0000u)};
        r[p] = hi;
        rl[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(q - h, b2));
      } else {
        r[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(q, h2));
      }
    }
  }
};

}  // namespace cubic
