// tiled.hip -- A16 and Dynamic A8 products for prefill-sized M (MFMA bound).
//
// The CubicQuant article (section "压缩权重必须边解码、边计算") describes a 2-D
// dense kernel that decodes a weight tile inside the tile and consumes it at
// once. Here a 256-thread workgroup computes a 128 x 128 output tile; per K step
// of 64 codes every thread decodes one 32-code chunk of one weight row (through
// a per-(row, group) table in LDS for up to 6-bit codes, computed per code for 7
// and 8 bits) into an fp16 (A16) or INT8-carrier (A8) tile in LDS, next to the
// activation tile, and four waves run 32x32 MFMAs on it.
//  - A16: levels are fp16(s * q) (group scale folded in), activations fp16 after
//    the per-row power-of-two prescale of k_xprep; fp32 accumulation.
//  - A8: INT8 carrier clamp(rne(127 q)) (CubicQuant article, A16/A8 section),
//    int32 MFMA per group, then fp32 accumulation of fp32(s / 127) * I, and the
//    per-row activation scale in the epilogue.
#include "decode.h"
#include "launch.h"

namespace cubic {

constexpr int TBM = 128, TBN = 128, TBK = 64;
constexpr int A16_LDS_STRIDE = TBK + 8;     // fp16 elements per LDS row (pad 16 B)
constexpr int A8_LDS_STRIDE = TBK + 16;     // int8 elements per LDS row (pad 16 B)

template <int BITS>
__device__ __forceinline__ void load_codes(const uint32_t* src, uint32_t* w) {
#pragma unroll
  for (int d = 0; d < BITS; ++d) w[d] = src[d];
}

template <int BITS>
__global__ __launch_bounds__(256) void k_tiled_a16(TiledParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* As = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Bs = As + TBM * A16_LDS_STRIDE;
  uint16_t* tab = Bs + TBN * A16_LDS_STRIDE;               // [TBN][2^B] (table widths)
  constexpr int NT = 1 << BITS;
  constexpr int km = kmax_of(BITS);
  // 7- and 8-bit codes compute each level s q(|k| / Kmax) in fp32 (Horner form,
  // the scale folded into the coefficients); narrower codes build a per-(row,
  // group) table of fp16(s q) in fp32.
  constexpr bool kDirect = BITS >= 7;
  float ha = 0.0f, hb = 0.0f, hc = 0.0f;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * TBM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * TBN;
  const uint16_t* X = static_cast<const uint16_t*>(p.xa);

  // loader roles: row r (0..127) and half h (0..1) of the 64-wide K step
  const int r = tid >> 1, h = tid & 1;
  const int64_t am = m0 + r;
  const bool a_ok = am < p.M;
  const int64_t bn = (n0 + r < p.N) ? (n0 + r) : (p.N - 1);
  const int64_t rowwords = p.K * BITS / 32;
  const uint32_t* crow = reinterpret_cast<const uint32_t*>(p.codes) + bn * rowwords;
  const int64_t gpr = p.K / p.group;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int nsteps = static_cast<int>(p.K / TBK);
  int gcur = -1;
  for (int ks = 0; ks < nsteps; ++ks) {
    const int64_t k0 = static_cast<int64_t>(ks) * TBK;
    // global -> registers
    u32x4 av[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      av[q] = u32x4{0u, 0u, 0u, 0u};
      if (a_ok) av[q] = *reinterpret_cast<const u32x4*>(X + am * p.K + k0 + h * 32 + q * 8);
    }
    uint32_t w[BITS];
    load_codes<BITS>(crow + (k0 + h * 32) * BITS / 32, w);
    const int g = static_cast<int>(k0 / p.group);
    const bool newg = g != gcur;
    float s = 0.0f;
    uint32_t ab = 0u;
    if (newg) {
      s = p.scales[bn * gpr + g];
      ab = reinterpret_cast<const uint32_t*>(p.shapes)[bn * gpr + g];
    }
    __syncthreads();                                   // previous MFMAs done with LDS
    if (newg) {
      const float a = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(ab & 0xffffu)));
      const float b = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(ab >> 16)));
      if constexpr (kDirect) {
        ha = s * a;
        hb = s * b;
        hc = s * ((1.0f - a) - b);
      } else {
#pragma unroll 4
        for (int v = h * (NT / 2); v < (h + 1) * (NT / 2); ++v)
          tab[r * NT + v] = f16_bits(s * table_level_f32(a, b, static_cast<uint32_t>(v), BITS));
      }
      gcur = g;
      if constexpr (!kDirect) __syncthreads();
    }
    // A tile
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<u32x4*>(As + r * A16_LDS_STRIDE + h * 32 + q * 8) = av[q];
    // B tile: decode 32 codes
    {
      uint32_t o[16];
      if constexpr (kDirect) {
        typedef float f2 __attribute__((ext_vector_type(2)));
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        constexpr float kInv = 1.0f / static_cast<float>(km);
        auto level = [&](int i) {
          const int kf = sign_extend(chunk_field<BITS>(w, i), BITS);
          const float t = static_cast<float>(kf < 0 ? -kf : kf) * kInv;
          return copysignf(t * fmaf(t, fmaf(t, hc, hb), ha), static_cast<float>(kf));
        };
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const f2 lv = {level(2 * i), level(2 * i + 1)};
          o[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lv, h2));
        }
      } else {
        const uint16_t* t = tab + r * NT;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          o[i] = static_cast<uint32_t>(t[chunk_field<BITS>(w, 2 * i)]) |
                 (static_cast<uint32_t>(t[chunk_field<BITS>(w, 2 * i + 1)]) << 16);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<u32x4*>(Bs + r * A16_LDS_STRIDE + h * 32 + q * 8) =
            u32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
    }
    __syncthreads();
    // MFMA: 4 sub-steps of 16 in K
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      f16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const f16x8*>(
            As + (wm * 64 + i * 32 + (lane & 31)) * A16_LDS_STRIDE + kk * 16 + 8 * (lane >> 5));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const f16x8*>(
            Bs + (wn * 64 + j * 32 + (lane & 31)) * A16_LDS_STRIDE + kk * 16 + 8 * (lane >> 5));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
  // epilogue. 32x32 D layout: lane l, register e -> column l%32,
  // row 8*(e/4) + 4*(l/32) + e%4.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t m = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      if (m >= p.M) continue;
      const float back = p.xs ? p.xs[m] : 1.0f;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t n = n0 + wn * 64 + j * 32 + (lane & 31);
        if (n < p.N) store_out(p.y, p.ybf16 != 0, m * p.N + n, acc[i][j][e] * back);
      }
    }
  }
}

template <int BITS>
__global__ __launch_bounds__(256) void k_tiled_a8(TiledParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  // 7- and 8-bit codes compute each carrier (carrier_fast); narrower codes build
  // a per-(row, group) table of the 2^B carriers.
  constexpr bool kDirect = BITS >= 7;
  constexpr int NT = 1 << BITS;
  constexpr int km = kmax_of(BITS);
  int8_t* As = reinterpret_cast<int8_t*>(smem);
  int8_t* Bs = As + TBM * A8_LDS_STRIDE;
  int8_t* tab = Bs + TBN * A8_LDS_STRIDE;                   // [TBN][2^B] (table widths)
  float* scs = reinterpret_cast<float*>(tab + (kDirect ? 0 : TBN * NT));   // [TBN]
  float ga = 0.0f, gb = 0.0f;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * TBM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * TBN;
  const int8_t* X = static_cast<const int8_t*>(p.xa);

  const int r = tid >> 1, h = tid & 1;
  const int64_t am = m0 + r;
  const bool a_ok = am < p.M;
  const int64_t bn = (n0 + r < p.N) ? (n0 + r) : (p.N - 1);
  const int64_t rowwords = p.K * BITS / 32;
  const uint32_t* crow = reinterpret_cast<const uint32_t*>(p.codes) + bn * rowwords;
  const int64_t gpr = p.K / p.group;

  i32x16 acci[2][2];
  f32x16 accf[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        acci[i][j][e] = 0;
        accf[i][j][e] = 0.0f;
      }

  const int nsteps = static_cast<int>(p.K / TBK);
  const int steps_per_group = p.group / TBK;
  float gsc[2] = {0.0f, 0.0f};
  for (int ks = 0; ks < nsteps; ++ks) {
    const int64_t k0 = static_cast<int64_t>(ks) * TBK;
    u32x4 av[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      av[q] = u32x4{0u, 0u, 0u, 0u};
      if (a_ok) av[q] = *reinterpret_cast<const u32x4*>(X + am * p.K + k0 + h * 32 + q * 16);
    }
    uint32_t w[BITS];
    load_codes<BITS>(crow + (k0 + h * 32) * BITS / 32, w);
    const int g = static_cast<int>(k0 / p.group);
    const bool newg = (ks % steps_per_group) == 0;
    float s = 0.0f;
    uint32_t ab = 0u;
    if (newg) {
      s = p.scales[bn * gpr + g];
      ab = reinterpret_cast<const uint32_t*>(p.shapes)[bn * gpr + g];
    }
    __syncthreads();
    if (newg) {
      const float a = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(ab & 0xffffu)));
      const float b = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(ab >> 16)));
      if constexpr (kDirect) {
        ga = a;
        gb = b;
      } else {
        for (int v = h * (NT / 2); v < (h + 1) * (NT / 2); ++v) {
          const int k = sign_extend(static_cast<uint32_t>(v), BITS);
          const int j = k < 0 ? -k : k;
          const int cv = j == 0 ? 0 : (j == km ? 127 : carrier_fast(a, b, j, km));
          tab[r * NT + v] = static_cast<int8_t>(k < 0 ? -cv : cv);
        }
      }
      if (h == 0) scs[r] = __fdiv_rn(s, 127.0f);
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 2; ++j) gsc[j] = scs[wn * 64 + j * 32 + (lane & 31)];
    }
#pragma unroll
    for (int q = 0; q < 2; ++q)
      *reinterpret_cast<u32x4*>(As + r * A8_LDS_STRIDE + h * 32 + q * 16) = av[q];
    {
      const int8_t* t = tab + r * NT;
      uint32_t o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t v = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          int cv;
          if constexpr (kDirect) {
            const int k = sign_extend(chunk_field<BITS>(w, 4 * i + e), BITS);
            const int j = k < 0 ? -k : k;
            const int c = j == 0 ? 0 : (j == km ? 127 : carrier_fast(ga, gb, j, km));
            cv = k < 0 ? -c : c;
          } else {
            cv = t[chunk_field<BITS>(w, 4 * i + e)];
          }
          v |= (static_cast<uint32_t>(cv) & 0xffu) << (8 * e);
        }
        o[i] = v;
      }
#pragma unroll
      for (int q = 0; q < 2; ++q)
        *reinterpret_cast<u32x4*>(Bs + r * A8_LDS_STRIDE + h * 32 + q * 16) =
            u32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      i32x4 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const i32x4*>(
            As + (wm * 64 + i * 32 + (lane & 31)) * A8_LDS_STRIDE + kk * 32 + 16 * (lane >> 5));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const i32x4*>(
            Bs + (wn * 64 + j * 32 + (lane & 31)) * A8_LDS_STRIDE + kk * 32 + 16 * (lane >> 5));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acci[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acci[i][j], 0, 0, 0);
    }
    if ((ks % steps_per_group) == steps_per_group - 1) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            accf[i][j][e] = fmaf(static_cast<float>(acci[i][j][e]), gsc[j], accf[i][j][e]);
            acci[i][j][e] = 0;
          }
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t m = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      if (m >= p.M) continue;
      const float sx = p.xs[m];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t n = n0 + wn * 64 + j * 32 + (lane & 31);
        if (n < p.N) store_out(p.y, p.ybf16 != 0, m * p.N + n, accf[i][j][e] * sx);
      }
    }
  }
}

template <int B>
static hipError_t launch_a16_b(const TiledParams& p, hipStream_t st) {
  const size_t lds = (TBM + TBN) * A16_LDS_STRIDE * 2 + (B >= 7 ? 0 : TBN * (1 << B) * 2);
  auto kern = k_tiled_a16<B>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  dim3 grid(static_cast<unsigned>((p.N + TBN - 1) / TBN), static_cast<unsigned>((p.M + TBM - 1) / TBM));
  hipLaunchKernelGGL(kern, grid, dim3(256), lds, st, p);
  return hipGetLastError();
}

template <int B>
static hipError_t launch_a8_b(const TiledParams& p, hipStream_t st) {
  const size_t lds = (TBM + TBN) * A8_LDS_STRIDE + (B >= 7 ? 0 : TBN * (1 << B)) + TBN * 4;
  dim3 grid(static_cast<unsigned>((p.N + TBN - 1) / TBN), static_cast<unsigned>((p.M + TBM - 1) / TBM));
  hipLaunchKernelGGL(k_tiled_a8<B>, grid, dim3(256), lds, st, p);
  return hipGetLastError();
}

hipError_t launch_tiled_a16(const TiledParams& p, int bits, hipStream_t st) {
  switch (bits) {
    case 2: return launch_a16_b<2>(p, st);
    case 3: return launch_a16_b<3>(p, st);
    case 4: return launch_a16_b<4>(p, st);
    case 5: return launch_a16_b<5>(p, st);
    case 6: return launch_a16_b<6>(p, st);
    case 7: return launch_a16_b<7>(p, st);
    default: return launch_a16_b<8>(p, st);
  }
}

hipError_t launch_tiled_a8(const TiledParams& p, int bits, hipStream_t st) {
  switch (bits) {
    case 2: return launch_a8_b<2>(p, st);
    case 3: return launch_a8_b<3>(p, st);
    case 4: return launch_a8_b<4>(p, st);
    case 5: return launch_a8_b<5>(p, st);
    case 6: return launch_a8_b<6>(p, st);
    case 7: return launch_a8_b<7>(p, st);
    default: return launch_a8_b<8>(p, st);
  }
}

}  // namespace cubic
