// gemv_core.h -- the streaming decode + MFMA loop shared by the small-M A16
// product (gemv.hip) and the routed-expert grouped product (moe.hip).
#pragma once
#include <utility>

#include "decode.h"

namespace cubic {

template <int BITS>
__device__ __forceinline__ void load_chunk(const uint32_t* src, uint32_t* w) {
  if constexpr (BITS == 2) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(src);
    w[0] = v.x; w[1] = v.y;
  } else if constexpr (BITS == 4) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(src);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (BITS == 8) {
    const u32x4 v0 = reinterpret_cast<const u32x4*>(src)[0];
    const u32x4 v1 = reinterpret_cast<const u32x4*>(src)[1];
    w[0] = v0.x; w[1] = v0.y; w[2] = v0.z; w[3] = v0.w;
    w[4] = v1.x; w[5] = v1.y; w[6] = v1.z; w[7] = v1.w;
  } else {
#pragma unroll
    for (int d = 0; d < BITS; ++d) w[d] = src[d];
  }
}

template <class Dec> struct IsW2 { static constexpr bool value = false; };
template <> struct IsW2<DecodeW2> { static constexpr bool value = true; };

// Decode this lane's chunk into 16 packed fp16 pairs.
template <class Dec>
__device__ __forceinline__ void decode_chunk(const uint32_t* w, uint32_t gab,
                                             const uint16_t* tab, uint32_t* r) {
  if constexpr (IsW2<Dec>::value) {
    if (__any(DecodeW2::has_extra(w))) {          // wave-uniform slow path
      const double a = f16_bits_to_f64(static_cast<uint16_t>(gab & 0xffffu));
      const double b = f16_bits_to_f64(static_cast<uint16_t>(gab >> 16));
      const float q2 = static_cast<float>(level_numerator(a, b, 2, 1));
      DecodeW2::full(w, q2, r);
    } else {
      DecodeW2::fast(w, r);
    }
  } else {
    Dec::decode(w, tab, r);
  }
}

template <class Dec>
__device__ __forceinline__ void build_table(uint16_t* tab_wave, int nl, int kb, uint32_t gab) {
  if constexpr (!IsW2<Dec>::value) {
    constexpr int B = Dec::kBits;
    const double a = f16_bits_to_f64(static_cast<uint16_t>(gab & 0xffffu));
    const double b = f16_bits_to_f64(static_cast<uint16_t>(gab >> 16));
    uint16_t* t = tab_wave + nl * (1 << B);
#pragma unroll
    for (int v = kb; v < (1 << B); v += 4) t[v] = table_entry(a, b, static_cast<uint32_t>(v), B);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// LDS bytes of the per-wave level tables.
template <class Dec>
__host__ __device__ constexpr int tab_bytes_per_wave() {
  return IsW2<Dec>::value ? 0 : 16 * (1 << Dec::kBits) * 2;
}

// Per-wave state of the streaming loop.
struct CoreArgs {
  const uint32_t* crow;     // this lane's weight row (code stream)
  const float* srow;        // its scales
  const uint32_t* abrow;    // its (a, b) pairs
  int group;
  int sb, se;               // K steps of this wave
  int nl, kb;               // lane coordinates (row in tile, chunk in step)
  int M;                    // valid activation rows in the MFMA tile (<= 16)
  int64_t K;
  const uint16_t* xrow;     // prepared activation row of A-lane nl (global variant)
  const uint16_t* xs_wave;  // LDS activations of this wave (in-kernel variant)
  int spw;
  uint16_t* tab_wave;       // LDS level tables of this wave (table decoders)
};

// Streams this lane's chunks for steps [sb, se), P steps in flight, and returns
// the group-scaled 16x16 partial of this wave (rows: activations, cols: weights).
template <class Dec, bool INK, int P>
__device__ __forceinline__ f32x4 gemv_core(const CoreArgs& c) {
  constexpr int B = Dec::kBits;
  const int kb = c.kb, nl = c.nl, sb = c.sb, se = c.se;
  uint32_t cb[P][B];
  float sbuf[P];
  uint32_t abuf[P];
  u32x4 xa[INK ? 1 : P][4];

  auto load_step = [&](auto u_c, int s) {
    constexpr int u = decltype(u_c)::value;
    load_chunk<B>(c.crow + static_cast<int64_t>(s * 4 + kb) * B, cb[u]);
    const int g = static_cast<int>((static_cast<int64_t>(s) * kStep) / c.group);
    sbuf[u] = c.srow[g];
    abuf[u] = c.abrow[g];
    if constexpr (!INK) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xa[u][j] = u32x4{0u, 0u, 0u, 0u};
        if (nl < c.M)
          xa[u][j] = *reinterpret_cast<const u32x4*>(c.xrow + (s * 4 + kb) * 32 + 8 * j);
      }
    }
  };

  [&]<int... U>(std::integer_sequence<int, U...>) {
    ((sb + U < se ? load_step(std::integral_constant<int, U>{}, sb + U) : void()), ...);
  }(std::make_integer_sequence<int, P>{});

  f32x4 acc = {0.f, 0.f, 0.f, 0.f}, part = {0.f, 0.f, 0.f, 0.f};
  int gcur = -1;
  float gscale = 0.0f;
  for (int s0 = sb; s0 < se; s0 += P) {
    [&]<int... U>(std::integer_sequence<int, U...>) {
      (([&] {
         constexpr int u = U;
         const int s = s0 + u;
         if (s < se) {
           const int g = static_cast<int>((static_cast<int64_t>(s) * kStep) / c.group);
           if (g != gcur) {
             acc += gscale * part;
             part = f32x4{0.f, 0.f, 0.f, 0.f};
             gcur = g;
             gscale = sbuf[u] * Dec::kLevelUnit;
             build_table<Dec>(c.tab_wave, nl, kb, abuf[u]);
           }
           uint32_t r[16];
           decode_chunk<Dec>(cb[u], abuf[u], c.tab_wave + nl * (1 << B), r);
#pragma unroll
           for (int j = 0; j < 4; ++j) {
             u32x4 av;
             if constexpr (INK) {
               av = u32x4{0u, 0u, 0u, 0u};
               if (nl < c.M)
                 av = *reinterpret_cast<const u32x4*>(
                     c.xs_wave + ((nl * c.spw + (s - sb)) * 4 + kb) * 32 + 8 * j);
             } else {
               av = xa[u][j];
             }
             const u32x4 bv = {r[4 * j], r[4 * j + 1], r[4 * j + 2], r[4 * j + 3]};
             part = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av),
                                                           __builtin_bit_cast(f16x8, bv), part,
                                                           0, 0, 0);
           }
           if (s + P < se) load_step(std::integral_constant<int, u>{}, s + P);
         }
       }()),
       ...);
    }(std::make_integer_sequence<int, P>{});
  }
  acc += gscale * part;
  return acc;
}

}  // namespace cubic
