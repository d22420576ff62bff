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
// Activations, M <= 4: each wave copies its own K slice into LDS (2-bit codes:
// raw bf16; wider codes: fp16 after a power-of-two prescale per (row, wave),
// exact for bf16 in range and undone on the wave's partial before the sum), so
// the whole product is one kernel. 5 <= M <= 16, wider codes: the caller's bf16
// rows are read from global memory as they are, against per-row tables of
// split bf16 levels (hi + lo, two MFMAs per fragment; DecodeTableSplit), again
// one kernel. 5 <= M <= 16, 2-bit codes: k_xprep reorders x once into the
// decoder's slot order.
#include "gemv_core.h"
#include "launch.h"

namespace cubic {

constexpr int kInkWaves = 4;   // waves per workgroup of the single-kernel (in-kernel x) path

// SPL = steps per load, P = macro steps in flight per lane, INK = activations
// converted in-kernel (M <= 4).
// MT: compile-time bound on M for the in-kernel activation path (1 or 4).
// W: waves per workgroup, each streaming 1/W of the K range of the 16 rows.
// XF16: the activations are fp16 (staged as they are; with table decoders the
// in-kernel staging copies them without a prescale).
template <class Dec, bool INK, int SPL, int P, bool ALLIN, int MT, int W, bool XF16>
__global__ __launch_bounds__(64 * W, 3) void k_gemv(GemvParams p) {
  extern __shared__ __align__(1024) unsigned char smem[];   // table rows rely on this alignment
  constexpr int B = Dec::kBits;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nl = lane & 15, kb = lane >> 4;
  // The workgroup owns p.rows (<= 16) weight rows; MFMA columns past them
  // repeat rows of the same workgroup (cache hits) and are not stored.
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * p.rows;
  const int64_t nsrc = n0 + (nl < p.rows ? nl : nl - p.rows);
  const int64_t nrow = nsrc < p.N ? nsrc : p.N - 1;
  const GemvGeom geo = gemv_geom(p.K, p.group, SPL, W);
  const int tb = wave * geo.nmacro / W, te = (wave + 1) * geo.nmacro / W;
  const int M = p.M;

  // LDS: [red 4x16x16 f32][tables per wave][group params per wave][xs per wave]
  float* red = reinterpret_cast<float*>(smem);
  unsigned char* q = smem + W * 16 * 16 * 4;
  uint16_t* tab_wave = reinterpret_cast<uint16_t*>(q + wave * tab_bytes_per_wave<Dec>());
  q += W * tab_bytes_per_wave<Dec>();
  uint32_t* gp_wave = reinterpret_cast<uint32_t*>(q) + wave * 16 * geo.gmax * 2;
  q += static_cast<size_t>(W) * 16 * geo.gmax * 8;
  uint16_t* xs_wave = reinterpret_cast<uint16_t*>(q) + static_cast<int64_t>(wave) * M * geo.nch_w * 32;

  float xb[4] = {1.0f, 1.0f, 1.0f, 1.0f};        // per-row back multipliers (INK)
  // In-kernel activation staging (XStage): each wave copies its own K slice of x
  // into its own LDS region, loads issued before the weight stream.
  constexpr int XB = 2;
  const int64_t k0 = static_cast<int64_t>(tb) * kStep * SPL;
  const int nblk = (te - tb) * kStep * SPL / 16;       // 16-element blocks in the slice
  XStage<Dec, INK ? MT : 1, XB, XF16> xst;
  const u32x4* xv[INK ? MT : 1] = {};
  if constexpr (INK) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
      xv[m] = reinterpret_cast<const u32x4*>(p.x + (m < M ? m : 0) * p.K + k0);
  }
  auto issue_x = [&]() {
    if constexpr (INK) xst.issue(xv, nblk, lane);
  };
  auto finish_x = [&]() {
    if constexpr (INK) xst.finish(xv, xs_wave, geo.nch_w, nblk, lane, M, xb);
  };

  CoreArgs c;
  const int gpr = static_cast<int>(p.K) / p.group;
  c.crow = reinterpret_cast<const uint32_t*>(p.codes + nrow * (p.K * B / 8));
  c.srow = p.scales + nrow * gpr;
  c.abrow = reinterpret_cast<const uint32_t*>(p.shapes + nrow * gpr * 2);
  c.mpg = geo.mpg;
  c.tb = tb; c.te = te; c.nl = nl; c.kb = kb; c.M = M;
  c.xrow = INK ? nullptr : (Dec::kSplit ? p.x : p.xp) + static_cast<int64_t>(nl < M ? nl : 0) * p.K;
  c.xs_wave = xs_wave; c.nch_w = geo.nch_w; c.tab_wave = tab_wave;
  c.gp_wave = gp_wave; c.gmax = geo.gmax;
  f32x4 acc = gemv_core<Dec, INK, SPL, P, ALLIN>(c, issue_x, finish_x);

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
    if (cc < p.rows && n0 + cc < p.N) {
      float v = red[m * 16 + cc];
#pragma unroll
      for (int w = 1; w < W; ++w) v += red[(w * 16 + m) * 16 + cc];
      if constexpr (!INK && !Dec::kSplit) v *= p.xback ? p.xback[m] : 1.0f;
      store_out(p.y, p.ybf16 != 0, static_cast<int64_t>(m) * p.N + n0 + cc, v);
    }
  }
}

// Activations for the prepared (multi-kernel) paths, one 256-thread block per
// row. W2 order: raw bf16 in the 2-bit decoder's slot order, xback = 1.
// Otherwise: per-row power-of-two prescale and fp16 in natural order; with
// V > 0 the row (at most 256 * V vectors of 8) is read once into registers,
// with V == 0 (longer rows) twice, the second pass hitting L2.
template <bool W2ORDER, int V>
__global__ __launch_bounds__(256) void k_xprep(const uint16_t* __restrict__ x, int64_t K,
                                               uint16_t* __restrict__ xp,
                                               float* __restrict__ xback) {
  const int64_t m = blockIdx.x;
  const uint16_t* row = x + m * K;
  uint16_t* out = xp + m * K;
  const int tid = threadIdx.x;
  if constexpr (W2ORDER) {
    for (int64_t i = tid; i < K / 16; i += 256) {
      const u32x4 lo = reinterpret_cast<const u32x4*>(row)[2 * i];
      const u32x4 hi = reinterpret_cast<const u32x4*>(row)[2 * i + 1];
      const uint32_t in[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      uint32_t o[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        o[2 * k] = __builtin_amdgcn_perm(in[4 + k], in[k], 0x05040100u);
        o[2 * k + 1] = __builtin_amdgcn_perm(in[4 + k], in[k], 0x07060302u);
      }
      u32x4* dst = reinterpret_cast<u32x4*>(out + 16 * i);
      dst[0] = u32x4{o[0], o[1], o[2], o[3]};
      dst[1] = u32x4{o[4], o[5], o[6], o[7]};
    }
    if (tid == 0) xback[m] = 1.0f;
    return;
  } else {
    const int64_t nvec = K / 8;
    const u32x4* rv = reinterpret_cast<const u32x4*>(row);
    u32x4* ov = reinterpret_cast<u32x4*>(out);
    auto absmax8 = [](const u32x4& v, float a) {
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a = fmaxf(a, fabsf(__uint_as_float(u[q] << 16)));
        a = fmaxf(a, fabsf(__uint_as_float(u[q] & 0xffff0000u)));
      }
      return a;
    };
    auto to_f16 = [](const u32x4& v, int sh) {
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
      uint32_t o[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint32_t e0 = f16_bits(ldexpf(__uint_as_float(u[h] << 16), sh));
        const uint32_t e1 = f16_bits(ldexpf(__uint_as_float(u[h] & 0xffff0000u), sh));
        o[h] = e0 | (e1 << 16);
      }
      return u32x4{o[0], o[1], o[2], o[3]};
    };
    __shared__ float red[4];
    auto prescale = [&](float amax) {
      amax = wave_max(amax);
      if ((tid & 63) == 0) red[tid >> 6] = amax;
      __syncthreads();
      amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
      float back;
      const int sh = row_prescale(amax, &back);
      if (tid == 0) xback[m] = back;
      return sh;
    };
    float amax = 0.0f;
    if constexpr (V > 0) {
      u32x4 v[V];
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const int64_t i = tid + 256 * j;
        v[j] = i < nvec ? rv[i] : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int j = 0; j < V; ++j) amax = absmax8(v[j], amax);
      const int sh = prescale(amax);
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const int64_t i = tid + 256 * j;
        if (i < nvec) ov[i] = to_f16(v[j], sh);
      }
    } else {
      for (int64_t i = tid; i < nvec; i += 256) amax = absmax8(rv[i], amax);
      const int sh = prescale(amax);
      for (int64_t i = tid; i < nvec; i += 256) ov[i] = to_f16(rv[i], sh);
    }
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
template <class Dec, bool INK, int SPL, int P, bool XF16 = false>
static hipError_t launch_gemv_t(const GemvParams& p, hipStream_t st) {
  constexpr int W = INK ? kInkWaves : 4;
  constexpr int MTB = INK ? 4 : 1;                  // MT only matters in-kernel
  const GemvGeom geo = gemv_geom(p.K, p.group, SPL, W);
  size_t lds = gemv_lds_fixed<Dec>(geo.gmax, W);
  if (INK) lds += static_cast<size_t>(W) * p.M * geo.nch_w * 32 * 2;
  auto kern = geo.mpw <= P
                  ? (p.M == 1 ? k_gemv<Dec, INK, SPL, P, true, 1, W, XF16> : k_gemv<Dec, INK, SPL, P, true, MTB, W, XF16>)
                  : (p.M == 1 ? k_gemv<Dec, INK, SPL, P, false, 1, W, XF16>
                              : k_gemv<Dec, INK, SPL, P, false, MTB, W, XF16>);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  // Rows per workgroup: when 16-row workgroups would leave the last round of
  // compute units partly idle (e.g. 384 on 256 CUs), spread the rows over a
  // whole number of rounds instead (512 workgroups of 12 rows).
  GemvParams q = p;
  const int64_t tiles16 = (p.N + 15) / 16;
  const int64_t cus = device_cu_count();
  q.rows = 16;
  if (cus > 0 && tiles16 > cus) {
    const int64_t rounds = (tiles16 + cus - 1) / cus;
    q.rows = static_cast<int>((p.N + rounds * cus - 1) / (rounds * cus));
  }
  const unsigned grid = static_cast<unsigned>((p.N + q.rows - 1) / q.rows);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * W), lds, st, q);
  return hipGetLastError();
}

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = cus;
  }
  return cached[dev];
}

static int gemv_spl(int bits, int group) { return (bits == 2 && group % 256 == 0) ? 2 : 1; }

// LDS bytes and group span of the GEMV paths (the dispatcher uses the tiled
// kernel when a wave would span more groups than it stages, or LDS overflows).
size_t gemv_ink_lds_bytes(int64_t M, int64_t K, int bits, int group) {
  const GemvGeom geo = gemv_geom(K, group, gemv_spl(bits, group), kInkWaves);
  const size_t tab = bits == 2 ? 0 : static_cast<size_t>(16) * (1 << bits) * 2;
  return static_cast<size_t>(kInkWaves) * (16 * 16 * 4 + tab + 16 * geo.gmax * 8) +
         static_cast<size_t>(kInkWaves) * M * geo.nch_w * 32 * 2;
}

bool gemv_supported(int64_t K, int bits, int group) {
  if (K > (int64_t{1} << 28)) return false;
  const GemvGeom geo = gemv_geom(K, group, gemv_spl(bits, group));
  return geo.gmax <= 4 * kGpRegs;
}

hipError_t launch_gemv(const GemvParams& p, int bits, bool ink, bool xf16, hipStream_t st) {
  // one activation row of 2-bit codes: whole rows per wave load (gemv_rows.hip)
  if (ink && gemv_rows_supported(p.M, p.N, p.K, bits, p.group)) return launch_gemv_rows(p, xf16, st);
  const bool spl2 = gemv_spl(bits, p.group) == 2;
  if (xf16) {
    // fp16 activations: 2-bit codes on the fp16 MFMA (x only permuted, by k_xprep for
    // the multi-row path); wider codes against fp16 levels, x staged in-kernel
    // (M <= 4) or read as the prepared rows (p.xp = the caller's x, p.xback = NULL)
    switch (bits) {
      case 2:
        if (spl2) return ink ? launch_gemv_t<DecodeW2H, true, 2, 8, true>(p, st)
                             : launch_gemv_t<DecodeW2H, false, 2, 2, true>(p, st);
        return ink ? launch_gemv_t<DecodeW2H, true, 1, 8, true>(p, st)
                   : launch_gemv_t<DecodeW2H, false, 1, 4, true>(p, st);
      case 3: return ink ? launch_gemv_t<DecodeTable<3>, true, 1, 8, true>(p, st)
                         : launch_gemv_t<DecodeTable<3>, false, 1, 4, true>(p, st);
      case 4: return ink ? launch_gemv_t<DecodeTable<4>, true, 1, 6, true>(p, st)
                         : launch_gemv_t<DecodeTable<4>, false, 1, 4, true>(p, st);
      case 5: return ink ? launch_gemv_t<DecodeTable<5>, true, 1, 4, true>(p, st)
                         : launch_gemv_t<DecodeTable<5>, false, 1, 2, true>(p, st);
      case 6: return ink ? launch_gemv_t<DecodeTable<6>, true, 1, 4, true>(p, st)
                         : launch_gemv_t<DecodeTable<6>, false, 1, 2, true>(p, st);
      case 7: return ink ? launch_gemv_t<DecodeDirect<7, false>, true, 1, 4, true>(p, st)
                         : launch_gemv_t<DecodeDirect<7, false>, false, 1, 4, true>(p, st);
      default: return ink ? launch_gemv_t<DecodeDirect<8, false>, true, 1, 4, true>(p, st)
                          : launch_gemv_t<DecodeDirect<8, false>, false, 1, 4, true>(p, st);
    }
  }
  switch (bits) {
    case 2:
      if (spl2) return ink ? launch_gemv_t<DecodeW2, true, 2, 8>(p, st)
                           : launch_gemv_t<DecodeW2, false, 2, 2>(p, st);
      return ink ? launch_gemv_t<DecodeW2, true, 1, 8>(p, st)
                 : launch_gemv_t<DecodeW2, false, 1, 4>(p, st);
    // wider codes without in-kernel staging read the caller's bf16 rows
    // directly against split bf16 levels (no preparation kernel)
    case 3: return ink ? launch_gemv_t<DecodeTable<3>, true, 1, 8>(p, st)
                       : launch_gemv_t<DecodeTableSplit<3>, false, 1, 4>(p, st);
    case 4: return ink ? launch_gemv_t<DecodeTable<4>, true, 1, 6>(p, st)
                       : launch_gemv_t<DecodeTableSplit<4>, false, 1, 4>(p, st);
    case 5: return ink ? launch_gemv_t<DecodeTable<5>, true, 1, 4>(p, st)
                       : launch_gemv_t<DecodeTableSplit<5>, false, 1, 2>(p, st);
    case 6: return ink ? launch_gemv_t<DecodeTable<6>, true, 1, 4>(p, st)
                       : launch_gemv_t<DecodeTableSplit<6>, false, 1, 2>(p, st);
    // 7- and 8-bit codes: levels computed per code (a table per 128-code group
    // would cost more than the codes; measured for 5-bit codes, tables win)
    case 7: return ink ? launch_gemv_t<DecodeDirect<7, false>, true, 1, 4>(p, st)
                       : launch_gemv_t<DecodeDirect<7, true>, false, 1, 4>(p, st);
    default: return ink ? launch_gemv_t<DecodeDirect<8, false>, true, 1, 4>(p, st)
                        : launch_gemv_t<DecodeDirect<8, true>, false, 1, 4>(p, st);
  }
}

hipError_t launch_xprep(const uint16_t* x, int64_t M, int64_t K, bool w2_order, uint16_t* xp,
                        float* xback, hipStream_t st) {
  // fp16 prescale: registers per thread, the row's vectors over 256 threads in
  // steps of powers of two
  const int64_t per = (K / 8 + 255) / 256;
  auto kern = w2_order ? k_xprep<true, 0>
              : per <= 1 ? k_xprep<false, 1> : per <= 2 ? k_xprep<false, 2>
              : per <= 4 ? k_xprep<false, 4> : per <= 8 ? k_xprep<false, 8> : k_xprep<false, 0>;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(M)), dim3(256), 0, st, x, K, xp, xback);
  return hipGetLastError();
}

}  // namespace cubic
