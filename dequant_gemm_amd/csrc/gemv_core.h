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
template <bool F16> struct IsW2<DecodeW2T<F16>> { static constexpr bool value = true; };

template <class Dec>
__device__ __forceinline__ void build_table(uint16_t* tab_wave, int nl, int kb, uint32_t gab) {
  // Levels in fp32 (table_level_f32: a few fp32 ulps for every width, far
  // below the 16-bit entries), each of the four lanes of a row taking every
  // fourth entry.
  constexpr int B = Dec::kBits;
  constexpr int kUnroll = B <= 4 ? 4 : 8;
  if constexpr (Dec::kDirect) {
    // no table: the levels are computed per code
  } else if constexpr (Dec::kSplit) {
    // bf16 (hi, lo) pairs, one dword per entry
    uint32_t* t = reinterpret_cast<uint32_t*>(tab_wave) + nl * (1 << B);
    const int swz = Dec::swizzle(nl);
    const float a = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(gab & 0xffffu)));
    const float b = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(gab >> 16)));
#pragma unroll kUnroll
    for (int v = kb; v < (1 << B); v += 4)
      t[v ^ swz] = split_bf16_pair(table_level_f32(a, b, static_cast<uint32_t>(v), B));
    wave_lds_order();
  } else if constexpr (!IsW2<Dec>::value) {
    uint16_t* t = tab_wave + nl * (1 << B);
    const int swz = Dec::swizzle(nl);           // entry v of row nl sits at v ^ swz
    const float a = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(gab & 0xffffu)));
    const float b = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(gab >> 16)));
#pragma unroll kUnroll
    for (int v = kb; v < (1 << B); v += 4) t[v ^ swz] = table_entry_f32(a, b, static_cast<uint32_t>(v), B);
    wave_lds_order();
  }
}

// LDS bytes of the per-wave level tables.
template <class Dec>
__host__ __device__ constexpr int tab_bytes_per_wave() {
  return (IsW2<Dec>::value || Dec::kDirect) ? 0 : 16 * (1 << Dec::kBits) * (Dec::kSplit ? 4 : 2);
}

// Per-wave state of the streaming loop.
//
// Work unit: a "macro step" of SPL x 128 codes per row. Lane (n, kb) owns the
// SPL consecutive 32-code chunks kb*SPL .. kb*SPL+SPL-1 of each macro step of
// row n, fetched with one load of SPL*bits dwords; sub-step h feeds MFMAs with
// chunk kb*SPL + h from every kb lane, so a sub-step spans 4 chunks spread over
// the macro step, which must lie in one group (group % (128*SPL) == 0).
// 16x16x32 MFMA with bf16 or fp16 operands (8 per lane), fp32 accumulation.
template <bool BF16>
__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

constexpr int kGpRegs = 8;     // group-parameter registers per lane: <= 32 groups per wave

struct CoreArgs {
  const uint32_t* crow;     // this lane's weight row (code stream)
  const float* srow;        // its scales [groups]
  const uint32_t* abrow;    // its (a, b) pairs [groups]
  int mpg;                  // macro steps per group
  int tb, te;               // macro steps of this wave
  int nl, kb;               // lane coordinates (row in tile, chunk slot)
  int M;                    // valid activation rows in the MFMA tile (<= 16)
  const uint16_t* xrow;     // activation row of A-lane nl (global variant): prepared fp16, or
                            // the caller's bf16 for split-level decoders
  const uint16_t* xs_wave;  // LDS activations of this wave (in-kernel variant), chunk-major
  int nch_w;                // chunks per row reserved in xs_wave
  uint16_t* tab_wave;       // LDS level tables of this wave (table decoders)
  uint32_t* gp_wave;        // LDS group parameters of this wave: [16 rows][gmax][2]
  int gmax;
};

template <int N>
__device__ __forceinline__ void load_dwords(const uint32_t* src, uint32_t* w) {
  if constexpr (N == 2) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(src);
    w[0] = v.x; w[1] = v.y;
  } else if constexpr (N % 4 == 0) {
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
      const u32x4 v = reinterpret_cast<const u32x4*>(src)[q];
      w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int d = 0; d < N; ++d) w[d] = src[d];
  }
}

// Accumulators of the streaming loop: the open group's MFMA partial (part, one
// chain of MFMAs; several waves per SIMD hide their latency), the group-scaled
// total (acc) and the current group's parameters. When a group opens, the
// previous group's partial is scaled into acc and part is cleared; the macro
// step that opens the next group is kept as a counter (no division per step).
struct StreamState {
  f32x4 acc;
  f32x4 part;
  float gscale;
  uint32_t gab;
  int gcur;
  int tnext;                 // the macro step at which the next group opens
  float ca, cb, cc;          // Horner coefficients of the group (direct-level decoders)
  // tb: the first macro step streamed (in order from there), g0 its group
  __device__ __forceinline__ void reset(int tb, int g0) {
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
    part = f32x4{0.f, 0.f, 0.f, 0.f};
    gscale = 0.0f;
    gab = 0u;
    gcur = g0 - 1;
    tnext = tb;
  }
  template <bool BF16>
  __device__ __forceinline__ void mac(const u32x4& a, const u32x4& b) {
    part = mfma16<BF16>(a, b, part);
  }
  // fold the open group's partial into acc
  __device__ __forceinline__ f32x4 total() const {
    return acc + gscale * part;
  }
};

// One macro step t of this lane: w holds its SPL*bits code dwords. At a group
// boundary the previous group's partials are scaled into acc and the new
// group's parameters are read from gp_wave (entry g - g0). Activations come
// from LDS (INK) or from xa[SPL][4] (registers).
template <class Dec, bool INK, int SPL>
__device__ __forceinline__ void step_macro(const CoreArgs& c, StreamState& st, const uint32_t* w,
                                           const u32x4 (*xa)[4], int t, int g0, int ml) {
  constexpr int B = Dec::kBits;
  const int kb = c.kb, nl = c.nl;
  if (t == st.tnext) {                   // wave-uniform: a group opens
    const int g = st.gcur + 1;
    st.tnext = (g + 1) * c.mpg;
    st.acc += st.gscale * st.part;       // the previous group (zero before the first)
    st.part = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint32_t* gp = c.gp_wave + (nl * c.gmax + (g - g0)) * 2;
    st.gscale = __uint_as_float(gp[0]) * Dec::kLevelUnit;
    st.gab = gp[1];
    st.gcur = g;
    if constexpr (Dec::kDirect) {
      const auto k = Dec::coef(st.gab);
      st.ca = k.a;
      st.cb = k.b;
      st.cc = k.c;
    }
    build_table<Dec>(c.tab_wave, nl, kb, st.gab);
  }
  // 2-bit codes: one test per macro step for the field value 10 (code -2)
  bool extra = false;
  if constexpr (IsW2<Dec>::value) {
    uint32_t ex = 0;
#pragma unroll
    for (int d = 0; d < B * SPL; d += 2) {
      // w[d + 1]:w[d] shifted left by one as a pair; the bit carried into
      // w[d + 1] lands on an even (masked) position
      const uint64_t sv = shl64<1>((static_cast<uint64_t>(w[d + 1]) << 32) | w[d]);
      ex |= (w[d] & ~static_cast<uint32_t>(sv)) | (w[d + 1] & ~static_cast<uint32_t>(sv >> 32));
    }
    extra = __any((ex & 0xAAAAAAAAu) != 0u);
  }
#pragma unroll
  for (int h = 0; h < SPL; ++h) {
    u32x4 av[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (INK) {
        av[j] = *reinterpret_cast<const u32x4*>(
            c.xs_wave + (ml * c.nch_w + (t - c.tb) * 4 * SPL + kb * SPL + h) * 32 + 8 * j);
      } else {
        av[j] = xa[h][j];
      }
    }
    uint32_t r[16];
    if constexpr (Dec::kDirect) {
      uint32_t rl[16];
      Dec::decode(&w[h * B], typename Dec::Coef{st.ca, st.cb, st.cc}, r, rl);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        st.template mac<Dec::kBf16>(av[j], u32x4{r[4 * j], r[4 * j + 1], r[4 * j + 2], r[4 * j + 3]});
        if constexpr (Dec::kSplit)
          st.template mac<true>(av[j], u32x4{rl[4 * j], rl[4 * j + 1], rl[4 * j + 2], rl[4 * j + 3]});
      }
    } else if constexpr (Dec::kSplit) {
      uint32_t rl[16];
      Dec::decode(&w[h * B], reinterpret_cast<const uint32_t*>(c.tab_wave) + nl * (1 << B),
                  Dec::swizzle(nl), r, rl);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        st.template mac<true>(av[j], u32x4{r[4 * j], r[4 * j + 1], r[4 * j + 2], r[4 * j + 3]});
        st.template mac<true>(av[j], u32x4{rl[4 * j], rl[4 * j + 1], rl[4 * j + 2], rl[4 * j + 3]});
      }
    } else {
      if constexpr (IsW2<Dec>::value) {
        Dec::fast(&w[h * B], r);
      } else {
        Dec::decode(&w[h * B], c.tab_wave + nl * (1 << B), Dec::swizzle(nl), r);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        st.template mac<Dec::kBf16>(av[j], u32x4{r[4 * j], r[4 * j + 1], r[4 * j + 2], r[4 * j + 3]});
    }
    if constexpr (IsW2<Dec>::value) {
      const uint32_t* wv = &w[h * B];
      if (extra && __any(Dec::template extra_bits_or<2>(wv) != 0u)) {
        // rare (wave-uniform): code -2 present; correct r and add the lo part
        const double a = f16_bits_to_f64(static_cast<uint16_t>(st.gab & 0xffffu));
        const double b = f16_bits_to_f64(static_cast<uint16_t>(st.gab >> 16));
        const float v = static_cast<float>(-2.0 * level_numerator(a, b, 2, 1));
        // hi + lo in the MFMA's 16-bit type
        uint32_t hi, lo;
        if constexpr (Dec::kBf16) {
          hi = bf16_rne_bits(v);
          lo = bf16_rne_bits(v - __uint_as_float(hi << 16));
        } else {
          hi = f16_bits(v);
          lo = f16_bits(v - static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(hi))));
        }
        // The operand barrier keeps this rare path's arithmetic inside
        // the branch (otherwise it is speculated into the hot path).
        uint32_t wl[2] = {wv[0], wv[1]};
        asm volatile("" : "+v"(wl[0]), "+v"(wl[1]));
        uint32_t rhi[16], rlo[16];
        Dec::extra(wl, hi, lo, rhi, rlo);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          st.template mac<Dec::kBf16>(av[j], u32x4{rhi[4 * j], rhi[4 * j + 1], rhi[4 * j + 2], rhi[4 * j + 3]});
          st.template mac<Dec::kBf16>(av[j], u32x4{rlo[4 * j], rlo[4 * j + 1], rlo[4 * j + 2], rlo[4 * j + 3]});
        }
      }
    }
  }
}

// Streams this lane's chunks for macro steps [tb, te), P macro steps in flight,
// and returns the group-scaled 16x16 partial of this wave (rows: activations,
// cols: weights). issue_x() runs before the weight loads are issued and
// finish_x() after them, so that waiting for the activations never waits for
// the weight stream; each macro step then waits only for its own load. ALLIN:
// the caller guarantees te - tb <= P, so every load is issued up front and
// nothing is refilled.
template <class Dec, bool INK, int SPL, int P, bool ALLIN, class IssueX, class FinishX>
__device__ __forceinline__ f32x4 gemv_core(const CoreArgs& c, IssueX&& issue_x, FinishX&& finish_x) {
  constexpr int B = Dec::kBits;
  constexpr int DW = B * SPL;                  // dwords per lane per macro step
  const int kb = c.kb, nl = c.nl, tb = c.tb, te = c.te, mpg = c.mpg;
  uint32_t cb[P][DW];
  u32x4 xa[INK ? 1 : P][SPL][4];

  // Group parameters of the wave's range: entry (row, g - g0) of gp_wave holds
  // (scale bits, a|b); 16 rows x gn groups, four lanes per row, loaded into
  // registers now (with the code loads) and written to LDS after the prologue.
  const int g0 = tb / mpg;
  const int gn = te > tb ? (te - 1) / mpg - g0 + 1 : 0;
  uint32_t gsc[kGpRegs], gabr[kGpRegs];
  // Only the groups the wave spans (uniform bound; all of these loads are waited
  // for before the main loop, so a variable count costs no pipelining).
#pragma unroll
  for (int q = 0; q < kGpRegs; ++q) {
    if (4 * q < gn) {
      const int gi = kb + 4 * q;
      const int g = g0 + (gi < gn ? gi : 0);
      gsc[q] = __float_as_uint(c.srow[g]);
      gabr[q] = c.abrow[g];
    }
  }

  // Every global load below is unconditional (macro steps past the wave's range
  // are clamped to its last one; lanes past the activation rows read row 0 and
  // their MFMA output rows are never stored), so the compiler can count the
  // outstanding loads and wait only for the oldest.
  auto load_step = [&](auto u_c, int t_req) {
    constexpr int u = decltype(u_c)::value;
    int t = t_req < te ? t_req : te - 1;
    t = t < 0 ? 0 : t;
    load_dwords<DW>(c.crow + (t * 4 * SPL + kb * SPL) * B, cb[u]);
    if constexpr (!INK) {
#pragma unroll
      for (int h = 0; h < SPL; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          xa[u][h][j] = *reinterpret_cast<const u32x4*>(
              c.xrow + (t * 4 * SPL + kb * SPL + h) * 32 + 8 * j);
    }
  };

  issue_x();
  __builtin_amdgcn_sched_barrier(0);             // activation loads stay ahead of the weights
  [&]<int... U>(std::integer_sequence<int, U...>) {
    (load_step(std::integral_constant<int, U>{}, tb + U), ...);
  }(std::make_integer_sequence<int, P>{});
  __builtin_amdgcn_sched_barrier(0);

  finish_x();
#pragma unroll
  for (int q = 0; q < kGpRegs; ++q) {
    const int gi = kb + 4 * q;
    if (4 * q < gn && gi < gn) {
      c.gp_wave[(nl * c.gmax + gi) * 2] = gsc[q];
      c.gp_wave[(nl * c.gmax + gi) * 2 + 1] = gabr[q];
    }
  }
  wave_lds_order();

  StreamState st;
  st.reset(tb, g0);
  const int ml = nl < c.M ? nl : 0;
  for (int t0 = tb; t0 < te; t0 += P) {
    [&]<int... U>(std::integer_sequence<int, U...>) {
      (([&] {
         constexpr int u = U;
         const int t = t0 + u;
         if (t < te) {
           // operand barrier: decode this slot here, not hoisted ahead of the loop
#pragma unroll
           for (int d = 0; d < DW; ++d) asm volatile("" : "+v"(cb[u][d]));
           step_macro<Dec, INK, SPL>(c, st, cb[u], xa[INK ? 0 : u], t, g0, ml);
         }
         if constexpr (!ALLIN)
           load_step(std::integral_constant<int, u>{}, t + P);   // unconditional (clamped)
         __builtin_amdgcn_sched_barrier(0);       // keep each slot's decode next to its MFMAs
       }()),
       ...);
    }(std::make_integer_sequence<int, P>{});
  }
  return st.total();
}

// Per-wave staging of bf16 activation rows into LDS for the streaming loop's
// in-kernel mode: each wave copies its own K slice of up to MT rows, chunk-major
// and in the decoder's slot order.
//  - bf16 decoders (2-bit codes): raw bf16, only permuted (v_perm), back = 1.
//  - fp16 decoders: a power-of-two prescale per (row, slice), then fp16; back
//    is the factor that undoes it on the wave's partial sums.
// issue() loads the first XB 16-element blocks per lane and row into registers
// (indices clamped, so the loads are unconditional) and should run before the
// weight loads; finish() writes them and copies any longer tail.
template <class Dec, int MT, int XB, bool XF16 = false>
struct XStage {
  u32x4 reg[MT][XB][2];

  __device__ __forceinline__ void issue(const u32x4* const* xv, int nblk, int lane) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int q = 0; q < XB; ++q) {
        int i = lane + 64 * q;
        i = i < nblk ? i : 0;
        reg[m][q][0] = xv[m][2 * i];
        reg[m][q][1] = xv[m][2 * i + 1];
      }
  }

  // xs_wave: the wave's LDS rows (nch_w chunks of 32 each); back[m] receives the
  // back multiplier of row m (rows >= M are left alone).
  __device__ __forceinline__ void finish(const u32x4* const* xv, uint16_t* xs_wave, int nch_w,
                                         int nblk, int lane, int M, float* back) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= M) break;
      uint16_t* xo = xs_wave + m * nch_w * 32;
      if constexpr (IsW2<Dec>::value) {
        // x is already in the MFMA's type (bf16, or fp16 for DecodeW2H): only permuted.
        // 16 consecutive codes 16d..16d+15 fill slots 16d..16d+15 as pairs
        // (code i, code i+8): out[2k] / out[2k+1] take the low / high halves
        // of input registers k and 4+k.
        auto put = [&](int i, const u32x4& lo, const u32x4& hi) {
          const uint32_t in[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
          uint32_t o[8];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            o[2 * k] = __builtin_amdgcn_perm(in[4 + k], in[k], 0x05040100u);
            o[2 * k + 1] = __builtin_amdgcn_perm(in[4 + k], in[k], 0x07060302u);
          }
          u32x4* dst = reinterpret_cast<u32x4*>(xo + 16 * i);
          dst[0] = u32x4{o[0], o[1], o[2], o[3]};
          dst[1] = u32x4{o[4], o[5], o[6], o[7]};
        };
        // unconditional: lanes past the slice rewrite block 0 with block 0's data
        // (a conditional use would let the compiler sink the loads behind the
        // weight stream)
#pragma unroll
        for (int q = 0; q < XB; ++q) {
          const int i = lane + 64 * q;
          put(i < nblk ? i : 0, reg[m][q][0], reg[m][q][1]);
        }
        for (int i = lane + 64 * XB; i < nblk; i += 64) put(i, xv[m][2 * i], xv[m][2 * i + 1]);
        back[m] = 1.0f;
      } else if constexpr (XF16) {
        // fp16 activations against fp16 levels: copied as they are, back = 1
        auto put = [&](int i, const u32x4& lo, const u32x4& hi) {
          u32x4* dst = reinterpret_cast<u32x4*>(xo + 16 * i);
          dst[0] = lo;
          dst[1] = hi;
        };
#pragma unroll
        for (int q = 0; q < XB; ++q) {
          const int i = lane + 64 * q;
          put(i < nblk ? i : 0, reg[m][q][0], reg[m][q][1]);
        }
        for (int i = lane + 64 * XB; i < nblk; i += 64) put(i, xv[m][2 * i], xv[m][2 * i + 1]);
        back[m] = 1.0f;
      } else {
        auto absmax8 = [](const u32x4& v, float a) {
          const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            a = fmaxf(a, fabsf(__uint_as_float(u[h] << 16)));
            a = fmaxf(a, fabsf(__uint_as_float(u[h] & 0xffff0000u)));
          }
          return a;
        };
        float amax = 0.0f;
#pragma unroll
        for (int q = 0; q < XB; ++q)
          if (lane + 64 * q < nblk) amax = absmax8(reg[m][q][1], absmax8(reg[m][q][0], amax));
        for (int i = lane + 64 * XB; i < nblk; i += 64)
          amax = absmax8(xv[m][2 * i + 1], absmax8(xv[m][2 * i], amax));
        amax = wave_max(amax);
        const int sh = row_prescale(amax, &back[m]);
        auto put8 = [&](int v8, const u32x4& v) {        // natural order: 8 elements -> 16 B
          const uint32_t u[4] = {v.x, v.y, v.z, v.w};
          uint32_t o[4];
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const uint32_t e0 = f16_bits(ldexpf(__uint_as_float(u[h] << 16), sh));
            const uint32_t e1 = f16_bits(ldexpf(__uint_as_float(u[h] & 0xffff0000u), sh));
            o[h] = e0 | (e1 << 16);
          }
          *reinterpret_cast<u32x4*>(xo + 8 * v8) = u32x4{o[0], o[1], o[2], o[3]};
        };
#pragma unroll
        for (int q = 0; q < XB; ++q) {
          const int i = lane + 64 * q;
          if (i < nblk) {
            put8(2 * i, reg[m][q][0]);
            put8(2 * i + 1, reg[m][q][1]);
          }
        }
        for (int i = lane + 64 * XB; i < nblk; i += 64) {
          put8(2 * i, xv[m][2 * i]);
          put8(2 * i + 1, xv[m][2 * i + 1]);
        }
      }
    }
  }
};

// Launch geometry shared by the host launcher and the kernel.
struct GemvGeom {
  int nmacro;     // macro steps per row
  int mpw;        // macro steps reserved per wave (LDS sizing)
  int nch_w;      // activation chunks reserved per wave and row
  int mpg;        // macro steps per group
  int gmax;       // groups a wave can span
};

__host__ __device__ inline GemvGeom gemv_geom(int64_t K, int group, int spl, int waves = 4) {
  GemvGeom g;
  g.nmacro = static_cast<int>(K) / (kStep * spl);     // K <= 2^28 (gemv_supported)
  g.mpw = (g.nmacro + waves - 1) / waves;
  g.nch_w = g.mpw * 4 * spl;
  g.mpg = group / (kStep * spl);
  g.gmax = (g.mpw + g.mpg - 1) / g.mpg + 1;
  return g;
}

template <class Dec>
__host__ __device__ constexpr size_t gemv_lds_fixed(int gmax, int waves = 4) {
  return static_cast<size_t>(waves) * (16 * 16 * 4 + tab_bytes_per_wave<Dec>() + 16 * gmax * 8);
}

}  // namespace cubic
