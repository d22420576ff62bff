// rows.h -- the whole-row streaming layout of the one-row decode GEMV
// (gemv_rows.hip).
//
// A wave load covers R = 16 / S whole rows of S = K / G groups: lane (i, kq) =
// (lane % 16, lane / 16) takes quarter kq of group g of row r, slot i = r S + g.
// The lane's activations (the same K range for every row) stay in registers;
// one 16 x 16 x 32 MFMA with A = the lane's eight decoded codes and B = its eight
// activations puts the 32-product partial of slot i on the diagonal D[i][i]
// (the off-diagonal elements mix slots and are not used). The fused path of the
// CubicQuant article (section "压缩权重必须边解码、边计算", flow figure): codes
// decoded in registers into the dot product, fp32 group scaling after it.
#pragma once
#include "gemv_core.h"

namespace cubic {
namespace rows {

constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer, 32-bit data format

// Sum over the 64 lanes in a fixed order: within each 16-lane row by DPP
// (quad swaps, then the half-row and row mirrors), then the four row sums.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add<0xB1>(v);      // quad_perm [1, 0, 3, 2]
  v = dpp_add<0x4E>(v);      // quad_perm [2, 3, 0, 1]
  v = dpp_add<0x141>(v);     // row_half_mirror
  v = dpp_add<0x140>(v);     // row_mirror
  const int b = __builtin_bit_cast(int, v);
  return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
         (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48)));
}

// LDS bytes of the staged activation row: K values and 16 bytes of padding
// after each group (the lanes of one 16-lane pass of a fragment read take the
// same offset in different groups, which the padding puts in different banks).
__host__ __device__ inline size_t lds_bytes(int64_t K, int G) {
  return static_cast<size_t>(K) * 2 + 16 * static_cast<size_t>(K / G);
}

// Activation row staging, issued before the code loads so that waiting for it
// never waits for the code stream: thread t takes 32-value sub-chunk t (K <= 8192).
struct XStageRow {
  u32x4 v[4];
  __device__ __forceinline__ void issue(const uint16_t* x, int64_t K, int tid) {
    const int nsub = static_cast<int>(K / 32);
    const u32x4* xg = reinterpret_cast<const u32x4*>(x) + 4 * (tid < nsub ? tid : 0);
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = xg[k];
  }
  // into LDS in the decoder's slot order: dword r of a sub-chunk holds the pair
  // (x[n], x[n + 8]), n = 16 (r >> 3) + (r & 7) (DecodeW2T::slot_to_code)
  template <int G>
  __device__ __forceinline__ void store(uint32_t* xl, int64_t K, int tid) const {
    if (tid >= static_cast<int>(K / 32)) return;
    uint32_t nat[16], o[16];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      nat[4 * k] = v[k].x; nat[4 * k + 1] = v[k].y; nat[4 * k + 2] = v[k].z; nat[4 * k + 3] = v[k].w;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int n = 16 * (r >> 3) + (r & 7);
      const uint32_t lo = nat[n >> 1], hi = nat[(n >> 1) + 4];
      o[r] = (n & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
    uint32_t* dst = xl + 16 * tid + 4 * (32 * tid / G);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      *reinterpret_cast<u32x4*>(dst + 4 * k) = u32x4{o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]};
  }
};

// The lane's activations (group gi, quarter kq): sub-chunk c, four fragments.
template <int G>
__device__ __forceinline__ void load_lane_x(const uint32_t* xl, int gi, int kq, u32x4 (*xa)[4]) {
  constexpr int CL = G / 4, NSC = CL / 32;
  const uint32_t* xrow = xl + (gi * G + kq * CL) / 2 + 4 * gi;   // (the group's padding)
#pragma unroll
  for (int c = 0; c < NSC; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) xa[c][j] = *reinterpret_cast<const u32x4*>(xrow + 16 * c + 4 * j);
}

// The MFMA output of one wave load: its diagonal holds each slot's partial.
// cw: the lane's G / 64 code dwords; gab: its group's (a, b) (for the code -2).
template <class Dec, int G>
__device__ __forceinline__ f32x4 wave_load_dot(const uint32_t* cw, const u32x4 (*xa)[4], uint32_t gab,
                                               bool active) {
  constexpr int NSC = G / 128, DWL = G / 64;
  // two MFMA chains (even and odd sub-chunks), added at the end
  f32x4 dc[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
  for (int c = 0; c < NSC; ++c) {
    uint32_t r[16];
    Dec::fast(&cw[2 * c], r);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dc[c & 1] = mfma16<Dec::kBf16>(u32x4{r[4 * j], r[4 * j + 1], r[4 * j + 2], r[4 * j + 3]}, xa[c][j], dc[c & 1]);
  }
  f32x4 d = dc[0] + dc[1];
  // field value 10 (code -2, never written by a symmetric quantiser): its level
  // -2 q(2) in units of s / 2 as hi + lo in the MFMA's 16-bit type
  const uint32_t ex = Dec::template extra_bits_or<DWL>(cw);
  if (__any(active && ex != 0u)) {
    const double a = f16_bits_to_f64(static_cast<uint16_t>(gab & 0xffffu));
    const double b = f16_bits_to_f64(static_cast<uint16_t>(gab >> 16));
    const float v = static_cast<float>(-2.0 * level_numerator(a, b, 2, 1));
    uint32_t hi, lo;
    if constexpr (Dec::kBf16) {
      hi = bf16_rne_bits(v);
      lo = bf16_rne_bits(v - __uint_as_float(hi << 16));
    } else {
      hi = f16_bits(v);
      lo = f16_bits(v - static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(hi))));
    }
#pragma unroll
    for (int c = 0; c < NSC; ++c) {
      uint32_t rhi[16], rlo[16];
      Dec::extra(&cw[2 * c], hi, lo, rhi, rlo);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        d = mfma16<Dec::kBf16>(u32x4{rhi[4 * j], rhi[4 * j + 1], rhi[4 * j + 2], rhi[4 * j + 3]}, xa[c][j], d);
        d = mfma16<Dec::kBf16>(u32x4{rlo[4 * j], rlo[4 * j + 1], rlo[4 * j + 2], rlo[4 * j + 3]}, xa[c][j], d);
      }
    }
  }
  return d;
}

// Slot i's scaled partial on the lane that holds diagonal element i (lane
// i + 16 (i / 4), register i % 4), zero elsewhere.
template <class Dec>
__device__ __forceinline__ float slot_partial(const f32x4& d, int lane, bool active, float s) {
  const int i = lane & 15;
  const bool diag = (lane >> 4) == (i >> 2);
  const float dv = (i & 3) == 0 ? d[0] : (i & 3) == 1 ? d[1] : (i & 3) == 2 ? d[2] : d[3];
  return (diag && active) ? dv * (s * Dec::kLevelUnit) : 0.0f;
}

}  // namespace rows
}  // namespace cubic
