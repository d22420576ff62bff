// skinny.hip -- A16 product for small batches (17 <= M <= 64; smaller M runs on
// the GEMV) with 2- to 8-bit codes.
//
// The CubicQuant article (section "压缩权重必须边解码、边计算") decodes each
// weight tile inside the kernel that consumes it and scales group partial sums
// in fp32. With up to 64 activation rows one decoded weight fragment feeds one
// or two MFMAs, so the layout is built around the weight stream:
//  - a 512-thread workgroup owns 32 weight rows; wave w walks an eighth of K
//    (steps of 64) against all activation rows (one or two 32-row blocks of
//    v_mfma_f32_32x32x16_f16), and the eight partial tiles are summed in LDS
//    in a fixed order at the end (deterministic, no atomics). Two waves per
//    SIMD hide each other's memory and LDS latencies;
//  - every load of the step loop goes from global memory straight into the
//    wave's own LDS ring (buffer_load ... lds): the fp16 activation chunk of the
//    step (prepared by k_xprep, XOR-swizzled), the 32 rows' code words and
//    their group parameters. A wave only reads what it loaded itself, so the
//    loop needs no workgroup barrier, only its own memory counter;
//  - lane (c, h) decodes row c, codes 32 h .. 32 h + 31 of the step, by lookups
//    in the row's fp16 table of levels s q 2^-e (2^B entries in LDS, rebuilt at
//    each group's first step from parameters that came with the stage of the
//    step before). 2^e is a power of two at or
//    above the row's largest |s| in the wave's K range, so every level fits
//    fp16 whatever s is, and the MFMA sums need no per-group scaling: the
//    wave's partial tile is multiplied by 2^e once, at the end;
//  - a step issues all of its LDS reads (code words, activation fragments,
//    table lookups) before its MFMAs, so their latencies overlap.
// Within a step, MFMA sub-step kb takes codes 8 kb .. 8 kb + 7 of each 32-code
// half, and the activation fragments follow the same K order.
#include "common.h"
#include "decode.h"
#include "launch.h"

namespace cubic {
namespace {

constexpr int SK_ROWS = 32;            // weight rows per workgroup
constexpr int SK_K = 64;               // K per step
constexpr uint32_t kSkRsrcWord3 = 0x00020000u;   // raw buffer, 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t sk_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0),
                                           static_cast<int>(bytes), static_cast<int>(kSkRsrcWord3));
}

// s_waitcnt immediate: vmcnt(n) (n < 64), expcnt not waited for, lgkmcnt(0).
constexpr int sk_wait_vm(int n) { return (n & 15) | (7 << 4) | (((n >> 4) & 3) << 14); }

// Per-wave LDS ring stage: activations [32 MB rows][64 k] fp16 (16-byte chunk
// q of row r at chunk q ^ (r & 7) ^ ((r >> 3) & 1)), then the code words, then the group
// parameters of the step after it (64 scales, 64 (a, b) words; lanes 32..63
// repeat rows 0..31). Code words of lane l (row l / 2, half l % 2): 2-bit codes,
// dword d at 256 d + 4 l; 3- and 4-bit codes, 16 l; wider codes, dwords 0..3 at
// 16 l and the rest at 1024 + 4 l (5-bit), 1024 + 4 l and 1280 + 4 l (6-bit) or
// 1024 + 16 l (7- and 8-bit).
template <int B> constexpr size_t sk_code_bytes() {
  return B <= 4 ? 1024 : (B == 5 ? 1280 : (B == 6 ? 1536 : 2048));
}
template <int MB> constexpr size_t sk_x_bytes() { return static_cast<size_t>(32 * MB) * SK_K * 2; }
template <int B, int MB> constexpr size_t sk_stage_bytes() { return sk_x_bytes<MB>() + sk_code_bytes<B>() + 512; }
// 7- and 8-bit codes compute each level (no table); narrower codes look levels
// up in a per-row table of 2^B fp16 entries.
template <int B> constexpr bool sk_direct() { return B >= 7; }
template <int B> constexpr size_t sk_tab_bytes() {
  return sk_direct<B>() ? 0 : static_cast<size_t>(SK_ROWS) * (1 << B) * 2;
}
// Ring depth: the most stages (up to 6) that W waves fit in one compute unit's LDS.
template <int B, int W, int MB> constexpr int sk_stages() {
  int n = 6;
  while (n > 2 && W * (n * sk_stage_bytes<B, MB>() + sk_tab_bytes<B>()) > 160 * 1024) --n;
  return n;
}
template <int B, int MB, int W>
constexpr size_t sk_lds_bytes() {
  return W * (sk_stages<B, W, MB>() * sk_stage_bytes<B, MB>() + sk_tab_bytes<B>());
}
// Waves per workgroup: two per SIMD where the LDS allows a ring of two stages,
// else one.
template <int B, int MB> constexpr int sk_waves() {
  return 8 * (2 * sk_stage_bytes<B, MB>() + sk_tab_bytes<B>()) <= 160 * 1024 ? 8 : 4;
}

// Normalised level q of field value v (two's complement, B bits) in fp32: with
// X = j K^2 - j^3 and Y = j^2 K - j^3 (integers), Q = j^3 + a X + b Y is
// evaluated with two fmas and scaled by 1/K^3: a few fp32 ulps (for up to 4-bit
// codes a X and b Y are exact, X and Y being below 2^10), far below the fp16
// rounding of the table entry that follows.
template <int B>
__device__ __forceinline__ float sk_level(float a, float b, int v) {
  constexpr int km = kmax_of(B);
  const int k = v >= (1 << (B - 1)) ? v - (1 << B) : v;
  const int j = k < 0 ? -k : k;
  const float X = static_cast<float>(j * km * km - j * j * j);
  const float Y = static_cast<float>(j * j * km - j * j * j);
  const float q = fmaf(a, X, fmaf(b, Y, static_cast<float>(j * j * j))) *
                  (1.0f / static_cast<float>(km * km * km));
  return k < 0 ? -q : q;
}

template <int B, int MB, int SK_WAVES>
__global__ __launch_bounds__(64 * SK_WAVES, 1) void k_skinny(TiledParams p) {
  extern __shared__ __align__(1024) unsigned char smem[];   // row tables rely on this alignment
  static_assert(B >= 2 && B <= 8, "2- to 8-bit codes");
  constexpr int NST = sk_stages<B, SK_WAVES, MB>();
  constexpr size_t kStage = sk_stage_bytes<B, MB>();
  constexpr size_t kCodeOff = sk_x_bytes<MB>();
  constexpr size_t kParamOff = kCodeOff + sk_code_bytes<B>();
  constexpr int NX = 4 * MB;                     // activation loads per step (1 KB each)
  constexpr int NC = B == 2 ? 2 : (B <= 4 ? 1 : (B == 6 ? 3 : 2));   // code loads per step
  constexpr int NV = NX + NC + 2;                // + codes + scales + (a, b)
  static_assert(NST * NV < 64, "vmcnt holds at most 63");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 31, h = lane >> 5;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * SK_ROWS;
  const int nsteps = static_cast<int>(p.K / SK_K);
  const int sb = wave * nsteps / SK_WAVES, se = (wave + 1) * nsteps / SK_WAVES;
  const int gpr = static_cast<int>(p.K / p.group);
  const uint32_t row_bytes = static_cast<uint32_t>(p.K * B / 8);

  unsigned char* ring = smem + static_cast<size_t>(wave) * NST * kStage;
  uint16_t* tab_wave =
      reinterpret_cast<uint16_t*>(smem + SK_WAVES * NST * kStage + wave * sk_tab_bytes<B>());

  // ---- loads of one step into a stage (this wave's own) ----
  // activations: load i covers rows 8 i .. 8 i + 7; lane l -> row r = 8 i + l / 8,
  // physical chunk l % 8 = logical chunk (l % 8) ^ sw(r), sw(r) = (r & 7) ^
  // ((r >> 3) & 1) (rows are 128 bytes: without the second term rows r and r + 8
  // of a 16-lane group share banks). Rows past M read 0.
  const __amdgpu_buffer_rsrc_t xrs = sk_rsrc(p.xa, static_cast<uint32_t>(p.M * p.K * 2));
  const uint32_t xoff0 = static_cast<uint32_t>(((lane >> 3) * p.K + 8 * ((lane & 7) ^ ((lane >> 3) & 7))) * 2);
  const uint32_t xoff1 = static_cast<uint32_t>(((lane >> 3) * p.K + 8 * ((lane & 7) ^ ((lane >> 3) & 7) ^ 1)) * 2);
  // code words: lane l -> row n0 + l / 2, codes 32 (l % 2) .. + 31 of the step.
  // Rows past N read 0.
  const __amdgpu_buffer_rsrc_t crs = sk_rsrc(p.codes, static_cast<uint32_t>(p.N) * row_bytes);
  const uint32_t coff = static_cast<uint32_t>(n0 + (lane >> 1)) * row_bytes +
                        static_cast<uint32_t>((lane & 1) * 4 * B);
  // group parameters of row n0 + l % 32 (clamped to a valid row)
  const int64_t prow = n0 + c < p.N ? n0 + c : p.N - 1;
  const __amdgpu_buffer_rsrc_t srs = sk_rsrc(p.scales, static_cast<uint32_t>(p.N * gpr * 4));
  const __amdgpu_buffer_rsrc_t brs = sk_rsrc(p.shapes, static_cast<uint32_t>(p.N * gpr * 4));
  const uint32_t poff = static_cast<uint32_t>(prow * gpr * 4);
  auto issue = [&](int s, int stage) {
    const int sv = s < se ? s : sb;            // past the wave's range: reload its first step
    unsigned char* st = ring + stage * kStage;
#pragma unroll
    for (int i = 0; i < NX; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xrs, st + 1024 * i, 16,
          (i & 1 ? xoff1 : xoff0) + static_cast<uint32_t>(8 * i) * static_cast<uint32_t>(p.K) * 2 +
              static_cast<uint32_t>(sv) * (SK_K * 2),
          0, 0, 0);
    if constexpr (B == 4) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(crs, st + kCodeOff, 16,
                                               coff + static_cast<uint32_t>(sv) * (8 * B), 0, 0, 0);
    } else if constexpr (B == 2) {
      // the lane's two dwords as two 4-byte loads (4-byte lane stride): dword d
      // of every lane lands in its own 256-byte area
#pragma unroll
      for (int d = 0; d < 2; ++d)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(crs, st + kCodeOff + 256 * d, 4,
                                                 coff + static_cast<uint32_t>(sv) * (8 * B) + 4 * d, 0, 0,
                                                 0);
    } else if constexpr (B == 3) {
      // 12-byte loads land at a 16-byte lane stride
      __builtin_amdgcn_raw_ptr_buffer_load_lds(crs, st + kCodeOff, 12,
                                               coff + static_cast<uint32_t>(sv) * (8 * B), 0, 0, 0);
    } else {
      // dwords 0..3, then the rest (4-byte loads at a 4-byte lane stride, or one
      // 12- or 16-byte load at a 16-byte stride)
      const uint32_t o = coff + static_cast<uint32_t>(sv) * (8 * B);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(crs, st + kCodeOff, 16, o, 0, 0, 0);
      if constexpr (B == 5 || B == 6) {
#pragma unroll
        for (int d = 4; d < B; ++d)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(crs, st + kCodeOff + 1024 + 256 * (d - 4), 4, o + 4 * d, 0,
                                                   0, 0);
      } else if constexpr (B == 7) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(crs, st + kCodeOff + 1024, 12, o + 16, 0, 0, 0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(crs, st + kCodeOff + 1024, 16, o + 16, 0, 0, 0);
      }
    }
    int g = (sv + 1) * SK_K / p.group;         // the group of the step after sv
    g = g < gpr ? g : gpr - 1;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, st + kParamOff, 4, poff + 4u * static_cast<uint32_t>(g),
                                             0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(brs, st + kParamOff + 256, 4,
                                             poff + 4u * static_cast<uint32_t>(g), 0, 0, 0);
  };

  f32x16 acc[MB];
#pragma unroll
  for (int j = 0; j < MB; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;

  // Level table of each row (entries fp16(s q 2^-e) for field values 0 ..
  // 2^B - 1), rebuilt at a group's first step from the parameters that came
  // with the stage of the step before it.
  constexpr int TE = 1 << B;                    // entries per row table
  // Entry v of row c sits at v ^ tswz. Row tables are TE / 2 words apart, so
  // rows c and c + 64 / TE share LDS banks; XOR-ing 2 (c / (64 / TE)) into the
  // entry index moves them apart, and the 32 rows of a half wave reading the
  // same field value hit 32 different banks.
  const int tswz = sk_direct<B>() ? 0 : 2 * (c / (TE >= 64 ? 1 : 64 / TE));
  float inv_rs = 1.0f, rs = 1.0f;               // 2^-e and 2^e of the row (set below)
  // 7- and 8-bit codes: the level of |k| = t Kmax is t (a' + t (b' + t c')) with
  // the group's s 2^-e folded into a', b', c' (Horner form in fp32)
  float ha = 0.0f, hb = 0.0f, hc = 0.0f;
  auto build = [&](int buf, uint32_t sbits, uint32_t ab) {
    const float a = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(ab & 0xffffu)));
    const float b = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(ab >> 16)));
    const float sk = __uint_as_float(sbits) * inv_rs;    // exact (power of two)
    if constexpr (sk_direct<B>()) {
      ha = sk * a;
      hb = sk * b;
      hc = sk * ((1.0f - a) - b);
    } else {
      uint16_t* t = tab_wave + (buf * SK_ROWS + c) * TE;   // buf is 0 (one table per row)
#pragma unroll
      for (int v = h; v < TE; v += 2) t[v ^ tswz] = f16_bits(sk * sk_level<B>(a, b, v));
    }
  };

  // ---- prologue: steps sb .. sb + NST - 2 in flight first, then the row
  // scale and the first group's table (their loads overlap the ring's) ----
#pragma unroll
  for (int t = 0; t < NST - 1; ++t) issue(sb + t, t);
  // ---- the row's level scale over this wave's K range: a power of two
  // 2^e >= max |s| of its groups there, so that fp16(s q 2^-e) fits whatever s
  // is. The row's two lanes take alternate groups; loads past the range read
  // an offset outside the buffer (0).
  {
    const int g_lo = sb * SK_K / p.group;
    const int g_hi = se > sb ? ((se * SK_K - 1) / p.group) : g_lo;   // last group touched
    float smax = 0.0f;
    for (int g0 = g_lo; g0 <= g_hi; g0 += 32) {
      float v[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int g = g0 + 2 * t + h;
        const uint32_t off = g <= g_hi ? poff + 4u * static_cast<uint32_t>(g) : 0xFFFFFFF0u;
        v[t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, off, 0, 0));
      }
#pragma unroll
      for (int t = 0; t < 16; ++t) smax = fmaxf(smax, fabsf(v[t]));
    }
    smax = fmaxf(smax, __shfl_xor(smax, 32, 64));
    int e = 0;
    if (smax > 0.0f && smax <= 3.4e38f) e = ilogbf(smax) + 1;
    inv_rs = ldexpf(1.0f, -e);
    rs = ldexpf(1.0f, e);
  }

  uint32_t psb = 0u, pab = 0u;                   // parameters of the next group
  {
    const uint32_t g0 = static_cast<uint32_t>(sb * SK_K / p.group);
    build(0, __builtin_amdgcn_raw_buffer_load_b32(srs, poff + 4u * g0, 0, 0),
          __builtin_amdgcn_raw_buffer_load_b32(brs, poff + 4u * g0, 0, 0));
  }

  for (int s = sb; s < se; ++s) {
    const int stage = (s - sb) % NST;
    const unsigned char* st = ring + stage * kStage;
    // Stage s has landed once only the loads of the next NST - 2 steps remain;
    // lgkmcnt(0) also ends this wave's reads of the stage refilled next.
    __builtin_amdgcn_s_waitcnt(sk_wait_vm((NST - 2) * NV));
    asm volatile("" ::: "memory");
    issue(s + NST - 1, (stage + NST - 1) % NST);
    if (s > sb && (s * SK_K) % p.group == 0) build(0, psb, pab);   // a new group's table
    // all of the step's LDS reads first: code words, activation fragments
    uint32_t w[B];
    if constexpr (B == 2) {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(st + kCodeOff) + (2 * c + h);
      w[0] = src[0];
      w[1] = src[64];
    } else if constexpr (B <= 4) {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(st + kCodeOff) + 4 * (2 * c + h);
#pragma unroll
      for (int d = 0; d < B; ++d) w[d] = src[d];
    } else {
      const u32x4 lo = *reinterpret_cast<const u32x4*>(st + kCodeOff + 16 * (2 * c + h));
      w[0] = lo.x; w[1] = lo.y; w[2] = lo.z; w[3] = lo.w;
      if constexpr (B == 5 || B == 6) {
#pragma unroll
        for (int d = 4; d < B; ++d)
          w[d] = reinterpret_cast<const uint32_t*>(st + kCodeOff + 1024 + 256 * (d - 4))[2 * c + h];
      } else {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(st + kCodeOff + 1024) + 4 * (2 * c + h);
#pragma unroll
        for (int d = 4; d < B; ++d) w[d] = src[d - 4];
      }
    }
    f16x8 fa[4][MB];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        // activation rows 32 j + c, logical chunk 4 h + kb
        const int r = 32 * j + c;
        fa[kb][j] = *reinterpret_cast<const f16x8*>(st + r * 128 + 16 * ((4 * h + kb) ^ (r & 7) ^ ((r >> 3) & 1)));
      }
    // the next step starts a group: its table and scale (parameters of the
    // group of step s + 1 come with stage s)
    const bool gnext = s + 1 < se && ((s + 1) * SK_K) % p.group == 0;
    if (gnext) {
      // parameters of the group of step s + 1 (its table is built there)
      const uint32_t* par = reinterpret_cast<const uint32_t*>(st + kParamOff);
      psb = par[c];
      pab = par[64 + c];
    }
    // weight fragments: codes 8 kb .. 8 kb + 7 of the lane's 32, via the row
    // table (up to 6-bit codes) or computed per code (7- and 8-bit)
    u32x4 fb[4];
    if constexpr (sk_direct<B>()) {
      typedef float f2 __attribute__((ext_vector_type(2)));
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
      constexpr float kInv = 1.0f / static_cast<float>(kmax_of(B));
      auto level = [&](int i) {
        const int bit = i * B;
        const int d = bit >> 5, off = bit & 31;
        int v;
        if (off + B <= 32) {
          v = __builtin_amdgcn_sbfe(w[d], off, B);
        } else {
          v = __builtin_amdgcn_sbfe(__builtin_amdgcn_alignbit(w[d + 1], w[d], off), 0, B);
        }
        const float kf = static_cast<float>(v);
        const float t = fabsf(kf) * kInv;
        return copysignf(t * fmaf(t, fmaf(t, hc, hb), ha), kf);
      };
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        uint32_t r[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f2 lv = {level(8 * kb + 2 * q), level(8 * kb + 2 * q + 1)};
          r[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lv, h2));
        }
        fb[kb] = u32x4{r[0], r[1], r[2], r[3]};
      }
    } else {
    const uint32_t tkey = static_cast<uint32_t>(tswz << 1) | static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>(tab_wave + c * TE));
    {
      typedef __attribute__((address_space(3))) const uint16_t lds_u16;
      typedef unsigned short u16x2v __attribute__((ext_vector_type(2)));
      constexpr uint32_t kMask2 = ((1u << B) - 1u) << 1;
      auto addr = [&](int i) {
        const int bit = i * B;
        const int d = bit >> 5, off = bit & 31;
        uint32_t v;
        if (off == 0) {
          v = w[d] << 1;
        } else if (off + B <= 32) {
          v = w[d] >> (off - 1);
        } else {
          v = __builtin_amdgcn_alignbit(w[d + 1], w[d], off - 1);
        }
        return (v & kMask2) ^ tkey;            // ((field ^ tswz) << 1) | row base
      };
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        uint32_t r[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          u16x2v hv;
          hv.x = *reinterpret_cast<const lds_u16*>(static_cast<uintptr_t>(addr(8 * kb + 2 * q)));
          hv.y = *reinterpret_cast<const lds_u16*>(static_cast<uintptr_t>(addr(8 * kb + 2 * q + 1)));
          r[q] = __builtin_bit_cast(uint32_t, hv);
        }
        fb[kb] = u32x4{r[0], r[1], r[2], r[3]};
      }
    }
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int j = 0; j < MB; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[kb][j], __builtin_bit_cast(f16x8, fb[kb]),
                                                        acc[j], 0, 0, 0);
  }
  // the row's level scale back (this lane's output column)
#pragma unroll
  for (int j = 0; j < MB; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] *= rs;
  __builtin_amdgcn_s_waitcnt(0);                // loads past the range target stages nobody reads
  __syncthreads();

  // ---- sum of the eight waves' partial tiles, in wave order ----
  // D element (row m of activation block j, column n): lane n + 32 ((m / 4) % 2),
  // register 4 (m / 8) + m % 4.
  float* red = reinterpret_cast<float*>(smem);  // [wave][j][e][lane]
#pragma unroll
  for (int j = 0; j < MB; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) red[((wave * MB + j) * 16 + e) * 64 + lane] = acc[j][e];
  __syncthreads();
  const int t = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 16 * MB / SK_WAVES; ++k) {
    const int o = t + 64 * SK_WAVES * k;        // o = 32 m + n over 32 MB activation rows
    const int n = o & 31, m = o >> 5;
    const int j = m >> 5, mm = m & 31;
    const int l = n + 32 * ((mm >> 2) & 1), e = 4 * (mm >> 3) + (mm & 3);
    float v = 0.0f;
#pragma unroll
    for (int wv = 0; wv < SK_WAVES; ++wv) v += red[((wv * MB + j) * 16 + e) * 64 + l];
    if (m < p.M && n0 + n < p.N) store_out(p.y, p.ybf16 != 0, static_cast<int64_t>(m) * p.N + n0 + n, v * (p.xs ? p.xs[m] : 1.0f));
  }
}

}  // namespace

bool skinny_supported(int64_t M, int64_t N, int64_t K, int bits, int group) {
  if (bits < 2 || bits > 8) return false;
  if (M < 1 || M > 64 || K % SK_K != 0 || K / SK_K < 8) return false;   // a step per wave
  if (group % SK_K != 0) return false;
  if (64 * K * 2 >= (int64_t{1} << 32)) return false;   // activation offsets of 64 rows
  if ((N + SK_ROWS) * K * bits / 8 >= (int64_t{1} << 32)) return false;
  if (N * (K / group) * 4 >= (int64_t{1} << 32)) return false;
  return (N + SK_ROWS - 1) / SK_ROWS <= INT32_MAX;
}

template <int B, int MB>
static hipError_t launch_skinny_k(const TiledParams& p, hipStream_t st) {
  constexpr int W = sk_waves<B, MB>();
  auto kern = k_skinny<B, MB, W>;
  constexpr size_t lds = sk_lds_bytes<B, MB, W>();
  static_assert(lds <= 160 * 1024, "one compute unit's LDS");
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(lds));
  if (e != hipSuccess) return e;
  const unsigned grid = static_cast<unsigned>((p.N + SK_ROWS - 1) / SK_ROWS);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * W), lds, st, p);
  return hipGetLastError();
}

template <int B>
static hipError_t launch_skinny_b(const TiledParams& p, hipStream_t st) {
  return p.M <= 32 ? launch_skinny_k<B, 1>(p, st) : launch_skinny_k<B, 2>(p, st);
}

hipError_t launch_skinny_a16(const TiledParams& p, int bits, hipStream_t st) {
  switch (bits) {
    case 2: return launch_skinny_b<2>(p, st);
    case 3: return launch_skinny_b<3>(p, st);
    case 4: return launch_skinny_b<4>(p, st);
    case 5: return launch_skinny_b<5>(p, st);
    case 6: return launch_skinny_b<6>(p, st);
    case 7: return launch_skinny_b<7>(p, st);
    default: return launch_skinny_b<8>(p, st);
  }
}

}  // namespace cubic
