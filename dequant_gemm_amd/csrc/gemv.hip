// gemv.hip -- A16 product for small M (decode-sized batches), memory bound.
//
// Layout of the work: a 256-thread workgroup owns 16 weight rows (one MFMA
// column tile) and its four waves split the K steps (128 codes per row per
// step). A lane (n, kb) = (lane % 16, lane / 16) streams chunk kb (32 codes,
// `bits` dwords) of row n per step, decodes it in registers (decode.h) and
// feeds four v_mfma_f32_16x16x32_f16 whose other operand holds up to 16
// activation rows. Group partial sums are scaled by the fp32 group scale
// (CubicQuant article, fused-decode flow figure: FP32 group scaling and
// accumulation after the tile-local dot product). The waves' partial outputs
// are summed in LDS in a fixed order, so results are deterministic.
//
// Activations: fp16 after a per-row power-of-two prescale (exact for bf16 in
// range). With M <= 4 each wave prescales and converts its own K slice into
// LDS (the prescale is per (row, wave) and is undone on the wave's partial
// before the sum), so the whole product is one kernel. Larger M use x
// prepared once by k_xprep (per-row prescale) and read from global memory.
#include "gemv_core.h"
#include "launch.h"

namespace cubic {

// P = steps kept in flight per lane; INK = activations converted in-kernel.
template <class Dec, bool INK, int P>
__global__ __launch_bounds__(256) void k_gemv(GemvParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int B = Dec::kBits;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, kb = lane >> 4;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int64_t nrow = (n0 + nl < p.N) ? (n0 + nl) : (p.N - 1);
  const int nsteps = static_cast<int>(p.K / kStep);
  const int sb = wave * nsteps / 4, se = (wave + 1) * nsteps / 4;
  const int spw = (nsteps + 3) / 4;               // LDS steps reserved per wave
  const int M = p.M;

  // LDS carve-up: [red 4x16x16 f32][tables][xs (INK only)]
  float* red = reinterpret_cast<float*>(smem);
  uint16_t* tab_wave = reinterpret_cast<uint16_t*>(smem + 4 * 16 * 16 * 4) +
                       wave * (tab_bytes_per_wave<Dec>() / 2);
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem + 4 * 16 * 16 * 4 + 4 * tab_bytes_per_wave<Dec>());
  uint16_t* xs_wave = xs + static_cast<int64_t>(wave) * M * spw * kStep;

  float xb[4] = {1.0f, 1.0f, 1.0f, 1.0f};        // per-row back multipliers (INK)
  if constexpr (INK) {
    const int64_t k0 = static_cast<int64_t>(sb) * kStep;
    const int nvec = (se - sb) * (kStep / 8);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (m >= M) break;
      const u32x4* xv = reinterpret_cast<const u32x4*>(p.x + m * p.K + k0);
      float amax = 0.0f;
      for (int i = lane; i < nvec; i += 64) {
        const u32x4 v = xv[i];
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          amax = fmaxf(amax, fabsf(__uint_as_float(u[q] << 16)));
          amax = fmaxf(amax, fabsf(__uint_as_float(u[q] & 0xffff0000u)));
        }
      }
      amax = wave_max(amax);
      float back;
      const int sh = row_prescale(amax, &back);
      xb[m] = back;
      for (int i = lane; i < nvec; i += 64) {
        const u32x4 v = xv[i];
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t bits = (e & 1) ? (u[e >> 1] & 0xffff0000u) : (u[e >> 1] << 16);
          const int kl = 8 * i + e;                         // index within the slice
          const int ls = kl >> 7, kc = (kl >> 5) & 3, cc = kl & 31;
          xs_wave[((m * spw + ls) * 4 + kc) * 32 + Dec::code_to_slot(cc)] =
              f16_bits(ldexpf(__uint_as_float(bits), sh));
        }
      }
    }
    __syncthreads();
  }

  CoreArgs c;
  const int64_t gpr = p.K / p.group;
  c.crow = reinterpret_cast<const uint32_t*>(p.codes + nrow * (p.K * B / 8));
  c.srow = p.scales + nrow * gpr;
  c.abrow = reinterpret_cast<const uint32_t*>(p.shapes + nrow * gpr * 2);
  c.group = p.group;
  c.sb = sb; c.se = se; c.nl = nl; c.kb = kb; c.M = M; c.K = p.K;
  c.xrow = INK ? nullptr : p.xp + static_cast<int64_t>(nl < M ? nl : 0) * p.K;
  c.xs_wave = xs_wave; c.spw = spw; c.tab_wave = tab_wave;
  f32x4 acc = gemv_core<Dec, INK, P>(c);

  // D layout of the 16x16 MFMA: lane holds rows 4*(lane/16) + r of column lane%16.
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * kb + r;
    float v = acc[r];
    if constexpr (INK) v *= (kb == 0) ? xb[r] : 1.0f;
    red[(wave * 16 + m) * 16 + nl] = v;
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < M * 16) {
    const int m = t >> 4, cc = t & 15;
    if (n0 + cc < p.N) {
      float v = red[(0 * 16 + m) * 16 + cc];
      v += red[(1 * 16 + m) * 16 + cc];
      v += red[(2 * 16 + m) * 16 + cc];
      v += red[(3 * 16 + m) * 16 + cc];
      if constexpr (!INK) v *= p.xback[m];
      p.y[static_cast<int64_t>(m) * p.N + n0 + cc] = v;
    }
  }
}

// One 256-thread block per row: per-row prescale, fp16 conversion and the
// decoder's chunk permutation; writes xp[m][K] and xback[m].
template <class Dec>
__global__ __launch_bounds__(256) void k_xprep(const uint16_t* __restrict__ x, int64_t K,
                                               uint16_t* __restrict__ xp,
                                               float* __restrict__ xback) {
  const int64_t m = blockIdx.x;
  const uint16_t* row = x + m * K;
  const int tid = threadIdx.x;
  const int64_t nvec = K / 8;
  const u32x4* rv = reinterpret_cast<const u32x4*>(row);
  float amax = 0.0f;
  for (int64_t i = tid; i < nvec; i += 256) {
    const u32x4 v = rv[i];
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      amax = fmaxf(amax, fabsf(__uint_as_float(u[q] << 16)));
      amax = fmaxf(amax, fabsf(__uint_as_float(u[q] & 0xffff0000u)));
    }
  }
  __shared__ float red[4];
  amax = wave_max(amax);
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float back;
  const int sh = row_prescale(amax, &back);
  if (tid == 0) xback[m] = back;
  uint16_t* out = xp + m * K;
  const int64_t nchunk = K / 32;
  for (int64_t c = tid; c < nchunk; c += 256) {
    uint32_t o[16];
#pragma unroll
    for (int sl = 0; sl < 32; sl += 2) {
      const uint32_t b0 = row[c * 32 + Dec::slot_to_code(sl)];
      const uint32_t b1 = row[c * 32 + Dec::slot_to_code(sl + 1)];
      const uint32_t h0 = f16_bits(ldexpf(__uint_as_float(b0 << 16), sh));
      const uint32_t h1 = f16_bits(ldexpf(__uint_as_float(b1 << 16), sh));
      o[sl >> 1] = h0 | (h1 << 16);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(out + c * 32);
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = u32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
template <class Dec, bool INK, int P>
static hipError_t launch_gemv_t(const GemvParams& p, hipStream_t st) {
  const int nsteps = static_cast<int>(p.K / kStep);
  const int spw = (nsteps + 3) / 4;
  size_t lds = 4 * 16 * 16 * 4 + 4 * tab_bytes_per_wave<Dec>();
  if (INK) lds += static_cast<size_t>(4) * p.M * spw * kStep * 2;
  auto kern = k_gemv<Dec, INK, P>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  const unsigned grid = static_cast<unsigned>((p.N + 15) / 16);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, st, p);
  return hipGetLastError();
}

// LDS bytes the in-kernel path needs (the dispatcher falls back to the prepared
// path when this exceeds the 160 KiB of a gfx950 CU).
size_t gemv_ink_lds_bytes(int64_t M, int64_t K, int bits) {
  const int64_t nsteps = K / kStep;
  const int64_t spw = (nsteps + 3) / 4;
  const size_t tab = bits == 2 ? 0 : static_cast<size_t>(16) * (1 << bits) * 2;
  return 4 * 16 * 16 * 4 + 4 * tab + static_cast<size_t>(4) * M * spw * kStep * 2;
}

hipError_t launch_gemv(const GemvParams& p, int bits, bool ink, hipStream_t st) {
  switch (bits) {
    case 2: return ink ? launch_gemv_t<DecodeW2, true, 8>(p, st)
                       : launch_gemv_t<DecodeW2, false, 4>(p, st);
    case 3: return ink ? launch_gemv_t<DecodeTable<3>, true, 8>(p, st)
                       : launch_gemv_t<DecodeTable<3>, false, 4>(p, st);
    case 4: return ink ? launch_gemv_t<DecodeTable<4>, true, 6>(p, st)
                       : launch_gemv_t<DecodeTable<4>, false, 4>(p, st);
    case 5: return ink ? launch_gemv_t<DecodeTable<5>, true, 4>(p, st)
                       : launch_gemv_t<DecodeTable<5>, false, 2>(p, st);
    case 6: return ink ? launch_gemv_t<DecodeTable<6>, true, 4>(p, st)
                       : launch_gemv_t<DecodeTable<6>, false, 2>(p, st);
    case 7: return ink ? launch_gemv_t<DecodeTable<7>, true, 4>(p, st)
                       : launch_gemv_t<DecodeTable<7>, false, 2>(p, st);
    default: return ink ? launch_gemv_t<DecodeTable<8>, true, 4>(p, st)
                        : launch_gemv_t<DecodeTable<8>, false, 2>(p, st);
  }
}

hipError_t launch_xprep(const uint16_t* x, int64_t M, int64_t K, bool w2_order, uint16_t* xp,
                        float* xback, hipStream_t st) {
  if (w2_order)
    hipLaunchKernelGGL(k_xprep<DecodeW2>, dim3(static_cast<unsigned>(M)), dim3(256), 0, st, x, K,
                       xp, xback);
  else
    hipLaunchKernelGGL(k_xprep<DecodeTable<3>>, dim3(static_cast<unsigned>(M)), dim3(256), 0, st,
                       x, K, xp, xback);
  return hipGetLastError();
}

}  // namespace cubic
