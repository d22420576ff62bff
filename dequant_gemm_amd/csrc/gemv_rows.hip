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
#include "launch.h"
#include "rows.h"

namespace cubic {
namespace {

// Zero, computed from v: an address that adds it is only formed once the load
// that produced v has returned (the compiler waits for v before the asm).
__device__ __forceinline__ uint32_t zero_after(uint32_t v) {
  uint32_t z;
  asm volatile("v_and_b32 %0, 0, %1" : "=v"(z) : "v"(v));
  return z;
}

// XF16: fp16 activations (fp16 MFMA) instead of bf16. G: group size (256 or
// 512). WL: wave-loads per wave, all issued up front. NW: waves per workgroup.
template <bool XF16, int G, int WL, int NW>
__global__ __launch_bounds__(64 * NW) void k_gemv_rows(GemvParams p, int S, int R, int L) {
  using Dec = DecodeW2T<XF16>;
  constexpr int DWL = G / 64;              // code dwords per lane and wave-load
  constexpr int NSC = G / 128;             // 32-code sub-chunks per lane
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* xl = reinterpret_cast<uint32_t*>(smem);   // the staged activation row

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, kq = lane >> 4;
  const bool active = i < R * S;
  const int ri = active ? i / S : 0;
  const int gi = active ? i % S : 0;
  const int gpr = static_cast<int>(p.K / G);
  const uint32_t row_bytes = static_cast<uint32_t>(p.K / 4);

  // Staging x. Every workgroup reads the same row, so its loads hit the L2; but
  // sent behind the code loads of the waves started before them, they were
  // measured to come in behind those, and the barrier below then held every
  // wave's decode until most of the compute unit's codes were in. So the
  // staging waves (the first of the workgroup) wait for x, one round trip,
  // before they issue their codes, and all of x goes out before any code load.
  if (wave * 64 < static_cast<int>(p.K / 32)) {
    rows::XStageRow xs;
    xs.issue(p.x, p.K, tid);
    xs.store<G>(xl, p.K, tid);
  }

  // codes and group parameters of this wave's WL wave-loads
  const __amdgpu_buffer_rsrc_t crs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.codes), static_cast<short>(0),
                                        static_cast<int>(static_cast<uint32_t>(p.N) * row_bytes),
                                        static_cast<int>(rows::kRsrcWord3));
  const int gw = static_cast<int>(blockIdx.x) * NW + wave;
  // Order of a wave. Wave-load 0 goes out before the barrier; the barrier
  // then waits only for x and for every wave to have issued it (an earlier
  // order, which also waited for each wave's first data before the barrier,
  // measured gate_up 6.27-6.33 us against 5.71-5.76 us). After it, wave-load
  // u > 0 goes out once the first data of wave-load u - 1 is in (its addresses
  // take a zero computed from that data): the first wave-loads come back from
  // a less crowded memory system and their decode overlaps the later ones
  // (gate_up 6.32-6.43 us against 7.03-7.07 us with every load issued at once,
  // both with the earlier barrier). Scheduling barriers keep the compiler from
  // moving the decode of wave-load 0 ahead of the barrier.
  uint32_t cw[WL][DWL];
  float gs[WL];
  uint32_t gab[WL];
  // With one wave-load a wave (small N) there is nothing to stagger within a
  // wave, so the upper half of the workgroup issues its codes after the
  // barrier (down 7168 x 3072 run that way: 4.83-4.91 us against 4.94-4.97 us
  // with every wave issuing at once).
  const bool late = WL == 1 && wave >= NW / 2;
  auto issue = [&](auto u0c, auto u1c) {
    constexpr int U0 = decltype(u0c)::value, U1 = decltype(u1c)::value;
    uint32_t after = 0;
#pragma unroll
    for (int u = U0; u < U1; ++u) {
      if (u > 0) after = zero_after(cw[u - 1][0]);
      const int q0 = gw * WL + u;
      const int q = q0 < L ? q0 : L - 1;     // past the last wave-load: reload it, store nothing
      const int64_t n = static_cast<int64_t>(q) * R + ri;
      const int64_t nc = n < p.N ? n : p.N - 1;
      const uint32_t off = static_cast<uint32_t>(nc) * row_bytes + static_cast<uint32_t>(gi * (G / 4) + kq * (G / 16)) + after;
#pragma unroll
      for (int d = 0; d < DWL; d += 4) {
        const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(crs, off + 4 * d, 0, 0);
        cw[u][d] = w.x; cw[u][d + 1] = w.y; cw[u][d + 2] = w.z; cw[u][d + 3] = w.w;
      }
      gs[u] = p.scales[nc * gpr + gi + after];
      gab[u] = reinterpret_cast<const uint32_t*>(p.shapes)[nc * gpr + gi + after];
    }
  };
  if (!late) issue(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{});

  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
  if (late) issue(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{});
  u32x4 xa[NSC][4];
  rows::load_lane_x<G>(xl, gi, kq, xa);
  issue(std::integral_constant<int, 1>{}, std::integral_constant<int, WL>{});
  __builtin_amdgcn_sched_barrier(0);

#pragma unroll
  for (int u = 0; u < WL; ++u) {
    const f32x4 d = rows::wave_load_dot<Dec, G>(cw[u], xa, gab[u], active);
    // each (row, group) partial scaled; the slots of each row summed over the wave
    const float part = rows::slot_partial<Dec>(d, lane, active, gs[u]);
    const int q0 = gw * WL + u;
    for (int rr = 0; rr < R; ++rr) {
      const float tot = rows::wave_sum(ri == rr ? part : 0.0f);
      const int64_t n = static_cast<int64_t>(q0) * R + rr;
      if (lane == 0 && q0 < L && n < p.N) store_out(p.y, p.ybf16 != 0, n, tot);
    }
  }
}

template <bool XF16, int G>
hipError_t launch_rows_g(const GemvParams& p, int S, int R, int L, int wl, int64_t cus, hipStream_t st) {
  const int waves = (L + wl - 1) / wl;
  const size_t lds = rows::lds_bytes(p.K, G);   // K <= 8192
  // Workgroups of 12 waves when that still fills every compute unit (one each,
  // which the dispatcher starts sooner than three of 4: gate_up 7.04-7.06 us
  // against 7.15-7.33 us with 4 and 7.32 us with 8, before the staggering);
  // otherwise of 8 (down 7168 x 3072 with two wave-loads a wave: 4.66-4.70 us
  // against 4.70-4.72 us with 7 and 5.07-5.08 us with 4). A workgroup of 12
  // code waves and 4 waves that only stage x measured 7.3 us for gate_up.
  if (wl == 1) {
    hipLaunchKernelGGL((k_gemv_rows<XF16, G, 1, 8>), dim3(static_cast<unsigned>((waves + 7) / 8)), dim3(512),
                       lds, st, p, S, R, L);
    return hipGetLastError();
  }
  if (wl == 2 && waves < 12 * cus) {
    hipLaunchKernelGGL((k_gemv_rows<XF16, G, 2, 8>), dim3(static_cast<unsigned>((waves + 7) / 8)), dim3(512),
                       lds, st, p, S, R, L);
    return hipGetLastError();
  }
  const unsigned grid = static_cast<unsigned>((waves + 11) / 12);
  switch (wl) {
    case 2: hipLaunchKernelGGL((k_gemv_rows<XF16, G, 2, 12>), dim3(grid), dim3(768), lds, st, p, S, R, L); break;
    case 3: hipLaunchKernelGGL((k_gemv_rows<XF16, G, 3, 12>), dim3(grid), dim3(768), lds, st, p, S, R, L); break;
    default: hipLaunchKernelGGL((k_gemv_rows<XF16, G, 4, 12>), dim3(grid), dim3(768), lds, st, p, S, R, L); break;
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
  // Wave-loads per wave: as few as keep at most 16 waves per CU, but two
  // (staggered) once there are at least two per CU. Measured on the K3 shapes
  // (graph replays, 50 rotating copies): gate_up (6144 wave-loads) 5.71-5.76 us
  // with two against 6.4-6.6 us with three in 8-wave workgroups; down (3584)
  // 4.66-4.70 us with two against 4.76-4.85 us with one.
  const int64_t cus = device_cu_count() > 0 ? device_cu_count() : 256;
  int64_t wl = (L + cus * 16 - 1) / (cus * 16);
  wl = wl < 1 ? 1 : (wl > 4 ? 4 : wl);
  if (wl == 1 && L >= 2 * cus) wl = 2;
  if (p.group == 512)
    return xf16 ? launch_rows_g<true, 512>(p, S, R, L, static_cast<int>(wl), cus, st)
                : launch_rows_g<false, 512>(p, S, R, L, static_cast<int>(wl), cus, st);
  return xf16 ? launch_rows_g<true, 256>(p, S, R, L, static_cast<int>(wl), cus, st)
              : launch_rows_g<false, 256>(p, S, R, L, static_cast<int>(wl), cus, st);
}

}  // namespace cubic
