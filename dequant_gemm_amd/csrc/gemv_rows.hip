// gemv_rows.hip -- the one-row A16 product for 2-bit codes (decode GEMV),
// streamed whole rows at a time.
//
// The fused path of the CubicQuant article (section "压缩权重必须边解码、边计算",
// flow figure): codes are decoded in registers straight into the operands of the
// dot product and each group's partial sum is scaled by its fp32 scale.
//
// Work layout. One wave-load is one 16-byte-aligned read of R whole weight rows
// (R = 16 / S rows of S = K / G groups each): lane (i, kq) = (lane % 16,
// lane / 16) takes quarter kq of group g of row r, where slot i = r * S + g, so
// each load instruction covers whole rows of the code stream (few DRAM pages)
// rather than a short piece of 16 rows. Measured with load-only probes on the
// 6144 x 7168 W2 matrix (libcubic_floors.so), a wave's first data then arrives
// 0.5 to 0.9 us earlier and the arrivals spread out, so the decode can overlap
// the stream.
//
// Product. The lane's activation slice (the same K range for every row it
// reads) stays in registers for the whole launch; the workgroup stages the row
// once in LDS, already in the decoder's slot order. One 16 x 16 x 32 MFMA takes
// A = the decoded codes and B = the matching activations of each lane, so its
// diagonal element D[i][i] sums the 32 products of slot i (four lanes x eight
// codes); the off-diagonal elements mix slots and are not used. Each diagonal
// element is one (row, group) partial: it is scaled by its group's fp32 scale
// and the slots of a row are summed across the wave in a fixed order (DPP
// within 16-lane rows, then the four row sums), so results are deterministic.
#include "gemv_core.h"
#include "launch.h"

namespace cubic {
namespace {

constexpr uint32_t kRowsRsrcWord3 = 0x00020000u;   // raw buffer, 32-bit data format

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

// XF16: fp16 activations (fp16 MFMA) instead of bf16. G: group size (256 or
// 512). WL: wave-loads per wave, all issued up front.
template <bool XF16, int G, int WL>
__global__ __launch_bounds__(256) void k_gemv_rows(GemvParams p, int S, int R, int L) {
  using Dec = DecodeW2T<XF16>;
  constexpr int CL = G / 4;                // codes per lane and wave-load
  constexpr int DWL = CL / 16;             // code dwords per lane and wave-load
  constexpr int NSC = CL / 32;             // 32-code sub-chunks per lane
  extern __shared__ __align__(16) unsigned char smem[];
  // The activation row, with 16 bytes of padding after each group: the lanes of
  // one 16-lane pass of a fragment read take the same offset in different
  // groups, which the padding puts in different LDS banks.
  uint32_t* xl = reinterpret_cast<uint32_t*>(smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, kq = lane >> 4;
  const bool active = i < R * S;
  const int ri = active ? i / S : 0;
  const int gi = active ? i % S : 0;
  const int gpr = static_cast<int>(p.K / G);
  const uint32_t row_bytes = static_cast<uint32_t>(p.K / 4);

  // the activation row into LDS (issued first, so that waiting for it never
  // waits for the code stream): thread t takes 32-value sub-chunk t (K <= 8192)
  const int nsub = static_cast<int>(p.K / 32);
  const u32x4* xg = reinterpret_cast<const u32x4*>(p.x) + 4 * (tid < nsub ? tid : 0);
  u32x4 xv[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) xv[v] = xg[v];

  // codes and group parameters of this wave's WL wave-loads
  const __amdgpu_buffer_rsrc_t crs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.codes), static_cast<short>(0),
                                        static_cast<int>(static_cast<uint32_t>(p.N) * row_bytes),
                                        static_cast<int>(kRowsRsrcWord3));
  const int gw = static_cast<int>(blockIdx.x) * 4 + wave;
  uint32_t cw[WL][DWL];
  float gs[WL];
  uint32_t gab[WL];
#pragma unroll
  for (int u = 0; u < WL; ++u) {
    const int q0 = gw * WL + u;
    const int q = q0 < L ? q0 : L - 1;     // past the last wave-load: reload it, store nothing
    const int64_t n = static_cast<int64_t>(q) * R + ri;
    const int64_t nc = n < p.N ? n : p.N - 1;
    const uint32_t off = static_cast<uint32_t>(nc) * row_bytes + static_cast<uint32_t>(gi * (G / 4) + kq * (G / 16));
#pragma unroll
    for (int d = 0; d < DWL; d += 4) {
      const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(crs, off + 4 * d, 0, 0);
      cw[u][d] = w.x; cw[u][d + 1] = w.y; cw[u][d + 2] = w.z; cw[u][d + 3] = w.w;
    }
    gs[u] = p.scales[nc * gpr + gi];
    gab[u] = reinterpret_cast<const uint32_t*>(p.shapes)[nc * gpr + gi];
  }

  // stored in the decoder's slot order: dword r of a sub-chunk holds the pair
  // (x[n], x[n + 8]), n = 16 (r >> 3) + (r & 7) (DecodeW2T::slot_to_code)
  if (tid < nsub) {
    uint32_t nat[16], o[16];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      nat[4 * v] = xv[v].x; nat[4 * v + 1] = xv[v].y; nat[4 * v + 2] = xv[v].z; nat[4 * v + 3] = xv[v].w;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int n = 16 * (r >> 3) + (r & 7);
      const uint32_t lo = nat[n >> 1], hi = nat[(n >> 1) + 4];
      o[r] = (n & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
    uint32_t* dst = xl + 16 * tid + 4 * (32 * tid / G);
#pragma unroll
    for (int v = 0; v < 4; ++v)
      *reinterpret_cast<u32x4*>(dst + 4 * v) = u32x4{o[4 * v], o[4 * v + 1], o[4 * v + 2], o[4 * v + 3]};
  }
  __syncthreads();

  // this lane's activations: sub-chunk c of its quarter, four fragments
  u32x4 xa[NSC][4];
  {
    const int k0 = gi * G + kq * CL;       // the lane's first code along K
    const uint32_t* xrow = xl + k0 / 2 + 4 * gi;   // (its group's padding)
#pragma unroll
    for (int c = 0; c < NSC; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) xa[c][j] = *reinterpret_cast<const u32x4*>(xrow + 16 * c + 4 * j);
  }

  // the lane that holds diagonal element i of the MFMA output (register i % 4)
  const bool diag = (lane >> 4) == (i >> 2);
#pragma unroll
  for (int u = 0; u < WL; ++u) {
    // two MFMA chains (even and odd sub-chunks), added at the end
    f32x4 dc[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int c = 0; c < NSC; ++c) {
      uint32_t r[16];
      Dec::fast(&cw[u][2 * c], r);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dc[c & 1] = mfma16<Dec::kBf16>(u32x4{r[4 * j], r[4 * j + 1], r[4 * j + 2], r[4 * j + 3]}, xa[c][j], dc[c & 1]);
    }
    f32x4 d = dc[0] + dc[1];
    // field value 10 (code -2, never written by a symmetric quantiser): its
    // level -2 q(2) in units of s / 2 as hi + lo in the MFMA's 16-bit type
    uint32_t ex = 0;
#pragma unroll
    for (int dd = 0; dd < DWL; ++dd) ex |= Dec::extra_bits(cw[u][dd]);
    if (__any(active && ex != 0u)) {
      const double a = f16_bits_to_f64(static_cast<uint16_t>(gab[u] & 0xffffu));
      const double b = f16_bits_to_f64(static_cast<uint16_t>(gab[u] >> 16));
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
        Dec::extra(&cw[u][2 * c], hi, lo, rhi, rlo);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          d = mfma16<Dec::kBf16>(u32x4{rhi[4 * j], rhi[4 * j + 1], rhi[4 * j + 2], rhi[4 * j + 3]}, xa[c][j], d);
          d = mfma16<Dec::kBf16>(u32x4{rlo[4 * j], rlo[4 * j + 1], rlo[4 * j + 2], rlo[4 * j + 3]}, xa[c][j], d);
        }
      }
    }
    // scale each (row, group) partial; the slots of each row are summed over the wave
    const float dv = (i & 3) == 0 ? d[0] : (i & 3) == 1 ? d[1] : (i & 3) == 2 ? d[2] : d[3];
    const float part = (diag && active) ? dv * (gs[u] * Dec::kLevelUnit) : 0.0f;
    const int q0 = gw * WL + u;
    for (int rr = 0; rr < R; ++rr) {
      const float tot = wave_sum(ri == rr ? part : 0.0f);
      const int64_t n = static_cast<int64_t>(q0) * R + rr;
      if (lane == 0 && q0 < L && n < p.N) store_out(p.y, p.ybf16 != 0, n, tot);
    }
  }
}

template <bool XF16, int G>
hipError_t launch_rows_g(const GemvParams& p, int S, int R, int L, int wl, hipStream_t st) {
  const int waves = (L + wl - 1) / wl;
  const unsigned grid = static_cast<unsigned>((waves + 3) / 4);
  const size_t lds = static_cast<size_t>(p.K) * 2 + 16 * static_cast<size_t>(p.K / G);   // K <= 8192
  switch (wl) {
    case 1: hipLaunchKernelGGL((k_gemv_rows<XF16, G, 1>), dim3(grid), dim3(256), lds, st, p, S, R, L); break;
    case 2: hipLaunchKernelGGL((k_gemv_rows<XF16, G, 2>), dim3(grid), dim3(256), lds, st, p, S, R, L); break;
    case 3: hipLaunchKernelGGL((k_gemv_rows<XF16, G, 3>), dim3(grid), dim3(256), lds, st, p, S, R, L); break;
    default: hipLaunchKernelGGL((k_gemv_rows<XF16, G, 4>), dim3(grid), dim3(256), lds, st, p, S, R, L); break;
  }
  return hipGetLastError();
}

}  // namespace

bool gemv_rows_supported(int64_t M, int64_t N, int64_t K, int bits, int group) {
  if (M != 1 || bits != 2 || (group != 256 && group != 512)) return false;
  if (K <= 0 || K % group != 0 || K > 8192 || K / group > 16) return false;
  return N > 0 && N * (K / 4) < (int64_t{1} << 32);
}

hipError_t launch_gemv_rows(const GemvParams& p, bool xf16, hipStream_t st) {
  const int S = static_cast<int>(p.K / p.group);
  const int R = 16 / S;
  const int64_t L64 = (p.N + R - 1) / R;
  if (L64 > 0x3fffffff) return hipErrorInvalidValue;
  const int L = static_cast<int>(L64);
  // Wave-loads per wave: one while that keeps at most 16 waves per CU, else as
  // few as keep it there. Measured on the K3 shapes (graph replays, 50 rotating
  // copies): down (3584 wave-loads) 5.16 us with one against 5.74 us with two;
  // gate_up (6144) 7.25 us with two against 8.05 with one and 7.88 with three.
  const int64_t cus = device_cu_count() > 0 ? device_cu_count() : 256;
  int64_t wl = (L + cus * 16 - 1) / (cus * 16);
  wl = wl < 1 ? 1 : (wl > 4 ? 4 : wl);
  if (p.group == 512)
    return xf16 ? launch_rows_g<true, 512>(p, S, R, L, static_cast<int>(wl), st)
                : launch_rows_g<false, 512>(p, S, R, L, static_cast<int>(wl), st);
  return xf16 ? launch_rows_g<true, 256>(p, S, R, L, static_cast<int>(wl), st)
              : launch_rows_g<false, 256>(p, S, R, L, static_cast<int>(wl), st);
}

}  // namespace cubic
