// moe.hip -- routed-expert A16 products grouped by expert on the device.
//
// The K3 expert layer (Kimi K3 guide, model-card table: 896 experts, 16 active
// per token) runs every (token, slot) pair against its expert's Cubic weights.
// The CubicQuant article (section on the A16/A8 crossover) notes that routing
// density changes which kernel wins; here the pairs are grouped per expert so
// that every touched expert's weights stream from HBM once per launch, whatever
// the number of tokens that picked it.
//
// k_moe_route (one block): per-expert counts, exclusive scan into offsets,
// the compacted list of touched experts, and the pair ids sorted by expert.
// Invalid ids are counted in hdr[0] and their output rows zeroed. No host sync.
// k_moe_gemv: one workgroup per (touched expert, 16-row tile); the expert's
// pairs form the activation rows of the MFMA tile (up to two per pass).
#include "gemv_core.h"
#include "launch.h"

namespace cubic {

__global__ __launch_bounds__(1024) void k_moe_route(const int32_t* __restrict__ ids, int P, int E,
                                                    int64_t N, float* __restrict__ y,
                                                    int32_t* __restrict__ hdr,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ active,
                                                    int32_t* __restrict__ sorted) {
  __shared__ int32_t s_sum[1024];
  __shared__ int32_t s_act[1024];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 1024) counts[e] = 0;
  if (tid == 0) hdr[0] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += 1024) {
    const int e = ids[p];
    if (e >= 0 && e < E) {
      atomicAdd(&counts[e], 1);
    } else {
      atomicAdd(&hdr[0], 1);
    }
  }
  // zero the output rows of invalid pairs (rare)
  for (int p = 0; p < P; ++p) {
    const int e = ids[p];
    if (e < 0 || e >= E) {
      for (int64_t n = tid; n < N; n += 1024) y[static_cast<int64_t>(p) * N + n] = 0.0f;
    }
  }
  __syncthreads();
  // each thread scans a contiguous segment of experts
  const int seg = (E + 1023) / 1024;
  const int e0 = tid * seg, e1 = min(E, e0 + seg);
  int sum = 0, act = 0;
  for (int e = e0; e < e1; ++e) {
    sum += counts[e];
    act += counts[e] > 0;
  }
  s_sum[tid] = sum;
  s_act[tid] = act;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 1024 per-thread totals
  for (int o = 1; o < 1024; o <<= 1) {
    const int a = tid >= o ? s_sum[tid - o] : 0;
    const int b = tid >= o ? s_act[tid - o] : 0;
    __syncthreads();
    s_sum[tid] += a;
    s_act[tid] += b;
    __syncthreads();
  }
  int run = s_sum[tid] - sum, arun = s_act[tid] - act;
  for (int e = e0; e < e1; ++e) {
    offsets[e] = run;
    const int c = counts[e];
    if (c > 0) active[arun++] = e;
    run += c;
  }
  if (tid == 1023) {
    offsets[E] = s_sum[1023];
    hdr[1] = s_act[1023];
  }
  __syncthreads();
  // counts become write cursors
  for (int e = e0; e < e1; ++e) counts[e] = offsets[e];
  __syncthreads();
  for (int p = tid; p < P; p += 1024) {
    const int e = ids[p];
    if (e >= 0 && e < E) sorted[atomicAdd(&counts[e], 1)] = p;
  }
}

// One workgroup per work item (touched expert a, 16-row tile): the grid covers
// the largest possible number of touched experts and items past the device-side
// count exit at once. The expert's pairs are taken MT at a time; each wave
// copies its K slice of those tokens' prepared rows into its own LDS region (the
// layout the streaming loop reads in its in-kernel mode), so activations are
// read from LDS by the MFMA lanes instead of from global memory, and the four
// waves' partial sums meet in LDS in a fixed order.
template <class Dec, int SPL, int P, bool ALLIN, int MT>
__global__ __launch_bounds__(256, 3) void k_moe_gemv(MoeGemvParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int B = Dec::kBits;
  constexpr int XB = 4;                         // 16-byte vectors per lane and row issued ahead
  const int64_t tiles = (p.N + 15) / 16;
  const int a = static_cast<int>(blockIdx.x / tiles);
  if (a >= p.hdr[1]) return;                    // fewer experts touched than the grid allows
  const int64_t n0 = (blockIdx.x - static_cast<int64_t>(a) * tiles) * 16;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nl = lane & 15, kb = lane >> 4;
  const GemvGeom geo = gemv_geom(p.K, p.group, SPL);
  float* red = reinterpret_cast<float*>(smem);
  unsigned char* q = smem + 4 * 16 * 16 * 4;
  uint16_t* tab_wave = reinterpret_cast<uint16_t*>(q + wave * tab_bytes_per_wave<Dec>());
  q += 4 * tab_bytes_per_wave<Dec>();
  uint32_t* gp_wave = reinterpret_cast<uint32_t*>(q) + wave * 16 * geo.gmax * 2;
  q += static_cast<size_t>(4) * 16 * geo.gmax * 8;
  uint16_t* xs_wave = reinterpret_cast<uint16_t*>(q) + static_cast<int64_t>(wave) * MT * geo.nch_w * 32;
  const int tb = wave * geo.nmacro / 4, te = (wave + 1) * geo.nmacro / 4;
  const int64_t k0 = static_cast<int64_t>(tb) * kStep * SPL;
  const int nvec = (te - tb) * kStep * SPL / 8;  // 16-byte vectors in the wave's slice of a row
  const int64_t gpr = p.K / p.group;

  const int e = p.active[a];
  const int beg = p.offsets[e], cnt = p.offsets[e + 1] - beg;
  const int64_t nrow = (n0 + nl < p.N) ? (n0 + nl) : (p.N - 1);
  CoreArgs c;
  c.crow = reinterpret_cast<const uint32_t*>(p.codes + e * p.code_bytes + nrow * (p.K * B / 8));
  c.srow = p.scales + (static_cast<int64_t>(e) * p.N + nrow) * gpr;
  c.abrow = reinterpret_cast<const uint32_t*>(p.shapes + ((static_cast<int64_t>(e) * p.N + nrow) * gpr) * 2);
  c.mpg = geo.mpg;
  c.tb = tb; c.te = te; c.nl = nl; c.kb = kb;
  c.xrow = nullptr; c.xs_wave = xs_wave; c.nch_w = geo.nch_w; c.tab_wave = tab_wave;
  c.gp_wave = gp_wave; c.gmax = geo.gmax;

  for (int mt = 0; mt < cnt; mt += MT) {
    const int Mt = min(MT, cnt - mt);
    c.M = Mt;
    const u32x4* xv[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int tok = p.sorted[beg + mt + (m < Mt ? m : 0)] / p.topk;
      xv[m] = reinterpret_cast<const u32x4*>(p.xp + static_cast<int64_t>(tok) * p.K + k0);
    }
    // The first XB vectors per lane and row are loaded before the weight stream
    // (indices clamped, so the loads are unconditional) and written to LDS after
    // it has been issued; longer slices copy the rest there.
    u32x4 xreg[MT][XB];
    auto issue_x = [&]() {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int v = 0; v < XB; ++v) {
          const int i = lane + 64 * v;
          xreg[m][v] = xv[m][i < nvec ? i : 0];
        }
    };
    auto finish_x = [&]() {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m >= Mt) break;
        u32x4* dst = reinterpret_cast<u32x4*>(xs_wave + m * geo.nch_w * 32);
#pragma unroll
        for (int v = 0; v < XB; ++v) {
          const int i = lane + 64 * v;
          if (i < nvec) dst[i] = xreg[m][v];
        }
        for (int i = lane + 64 * XB; i < nvec; i += 64) dst[i] = xv[m][i];
      }
    };
    const f32x4 acc = gemv_core<Dec, true, SPL, P, ALLIN>(c, issue_x, finish_x);
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wave * 16 + 4 * kb + r) * 16 + nl] = acc[r];
    __syncthreads();
    const int t = threadIdx.x;
    if (t < Mt * 16) {
      const int m = t >> 4, cc = t & 15;
      if (n0 + cc < p.N) {
        const int pr = p.sorted[beg + mt + m];
        float v = red[(0 * 16 + m) * 16 + cc];
        v += red[(1 * 16 + m) * 16 + cc];
        v += red[(2 * 16 + m) * 16 + cc];
        v += red[(3 * 16 + m) * 16 + cc];
        p.y[static_cast<int64_t>(pr) * p.N + n0 + cc] = v * p.xback[pr / p.topk];
      }
    }
    if (mt + MT < cnt) __syncthreads();   // red and the LDS slices are reused by the next pass
  }
}

// LDS of the grouped kernel for MT activation rows per pass.
template <class Dec>
static size_t moe_lds_bytes(const GemvGeom& geo, int mt) {
  return gemv_lds_fixed<Dec>(geo.gmax) + static_cast<size_t>(4) * mt * geo.nch_w * 32 * 2;
}

template <class Dec, int SPL, int P>
static hipError_t launch_moe_gemv_t(const MoeGemvParams& p, int64_t blocks, int tokens,
                                    hipStream_t st) {
  const GemvGeom geo = gemv_geom(p.K, p.group, SPL);
  // Rows per pass: a single token needs one; otherwise two while two
  // workgroups still fit in one compute unit's LDS (experts picked by more
  // tokens take several passes over their codes, which then come from L2).
  int mt = tokens <= 1 ? 1 : 2;
  if (mt == 2 && moe_lds_bytes<Dec>(geo, 2) > 80 * 1024) mt = 1;
  const size_t lds = moe_lds_bytes<Dec>(geo, mt);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  const bool allin = geo.mpw <= P;
  auto pick = [&]() {
    if (allin) return mt == 1 ? k_moe_gemv<Dec, SPL, P, true, 1> : k_moe_gemv<Dec, SPL, P, true, 2>;
    return mt == 1 ? k_moe_gemv<Dec, SPL, P, false, 1> : k_moe_gemv<Dec, SPL, P, false, 2>;
  };
  auto kern = pick();
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(256), lds, st, p);
  return hipGetLastError();
}

size_t moe_lds_min_bytes(int64_t K, int bits, int group) {
  const int spl = (bits == 2 && group % 256 == 0) ? 2 : 1;
  const GemvGeom geo = gemv_geom(K, group, spl);
  return bits == 2 ? moe_lds_bytes<DecodeW2>(geo, 1) : moe_lds_bytes<DecodeTable<8>>(geo, 1);
}

hipError_t launch_moe(const int32_t* ids, int T, int E, int topk, const MoeGemvParams& base,
                      int32_t* hdr, int32_t* counts, int32_t* offsets, int32_t* active,
                      int32_t* sorted, int bits, hipStream_t st) {
  const int P = T * topk;
  hipLaunchKernelGGL(k_moe_route, dim3(1), dim3(1024), 0, st, ids, P, E, base.N, base.y, hdr,
                     counts, offsets, active, sorted);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  MoeGemvParams p = base;
  p.topk = topk;
  p.hdr = hdr; p.offsets = offsets; p.active = active; p.sorted = sorted;
  const int64_t tiles = (p.N + 15) / 16;
  const int64_t blocks = static_cast<int64_t>(min(E, P)) * tiles;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  switch (bits) {
    case 2:
      if (p.group % 256 == 0) return launch_moe_gemv_t<DecodeW2, 2, 8>(p, blocks, T, st);
      return launch_moe_gemv_t<DecodeW2, 1, 8>(p, blocks, T, st);
    case 3: return launch_moe_gemv_t<DecodeTable<3>, 1, 8>(p, blocks, T, st);
    case 4: return launch_moe_gemv_t<DecodeTable<4>, 1, 6>(p, blocks, T, st);
    case 5: return launch_moe_gemv_t<DecodeTable<5>, 1, 2>(p, blocks, T, st);
    case 6: return launch_moe_gemv_t<DecodeTable<6>, 1, 2>(p, blocks, T, st);
    case 7: return launch_moe_gemv_t<DecodeTable<7>, 1, 2>(p, blocks, T, st);
    default: return launch_moe_gemv_t<DecodeTable<8>, 1, 2>(p, blocks, T, st);
  }
}

}  // namespace cubic
