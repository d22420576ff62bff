// Data-free group fitting (CubicQuant article, the section on data-free in-group
// fitting): per group, search monotone (a, b) shape candidates, choose the scale
// together with its soft-clip threshold, give every weight its nearest level, and
// store a, b in fp16 and s in fp32. The article fixes neither the grid nor the
// loss; this library searches
//   a = i/8 (i = 0 .. 24), b = j/8 (j = -24 .. 24), monotone pairs only,
//   s = fl32(rho * max|w|), rho = 1 - r/32 (r = 0 .. 15): the clip threshold is s,
//       weights beyond it take the top level,
// and minimises the group's sum of squared errors to the candidate's fp32 levels
// (the format's values RN32(s q_j), level_rn32). Candidate c = pair * 16 + r; the
// first candidate of smallest loss wins. The codes of the chosen (s, a, b) are
// written by cubic_encode's kernel right after (exact nearest level, ties to the
// smaller |k|).
// Multiples of 1/8 in [-3, 3] are exact in fp16, so storing a, b changes nothing.
#include "common.h"
#include "decode.h"
#include "launch.h"

namespace cubic {
namespace {

constexpr int kFitClipSteps = 16;
constexpr int kFitMaxGroup = 2048;

struct FitPairs {
  int n;
  signed char p[25 * 49][2];   // (8a, 8b)
};

// q(t) = a t + b t^2 + c t^3, c = 1 - a - b, is non-decreasing on [0, 1] iff
// q'(t) = a + 2bt + 3ct^2 >= 0 there. With A = 8a, Bq = 8b, C = 8c integers:
// q'(0) = a >= 0; q'(1) = 3 - 2a - b >= 0, i.e. 24 - 2A - Bq >= 0; and when q' is
// convex (c > 0) with its minimum t* = -b/(3c) inside (0, 1) (Bq < 0, -Bq < 3C),
// q'(t*) = a - b^2/(3c) >= 0, i.e. 3AC >= Bq^2. For c <= 0 the ends decide.
constexpr bool fit_monotone(int A, int Bq) {
  const int C = 8 - A - Bq;
  if (A < 0 || 24 - 2 * A - Bq < 0) return false;
  if (C > 0 && Bq < 0 && -Bq < 3 * C && 3 * A * C < Bq * Bq) return false;
  return true;
}

constexpr FitPairs make_fit_pairs() {
  FitPairs t{};
  for (int i = 0; i <= 24; ++i)
    for (int j = -24; j <= 24; ++j)
      if (fit_monotone(i, j)) {
        t.p[t.n][0] = static_cast<signed char>(i);
        t.p[t.n][1] = static_cast<signed char>(j);
        ++t.n;
      }
  return t;
}

constexpr FitPairs kFitPairs = make_fit_pairs();
constexpr int kFitCandidates = kFitPairs.n * kFitClipSteps;
static_assert(kFitPairs.n == 532, "monotone shape pairs on the 1/8 grid");

__constant__ FitPairs g_fit_pairs = kFitPairs;

__device__ __forceinline__ uint16_t f16_of(float v) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}

// One workgroup per group (row-major [N][K/group]). Each thread walks candidates
// threadIdx.x, +256, ...; for each it forms the fp32 levels v_j = s q_j and sums,
// over the group's weights in order, the square of the distance to the nearest
// level. The group's |w| sit in LDS and every lane reads the same word (broadcast).
template <int B>
__global__ __launch_bounds__(256) void k_fit(const float* __restrict__ w, int64_t K, int group,
                                             float* __restrict__ scales,
                                             uint32_t* __restrict__ shapes, float* __restrict__ loss) {
#pragma clang fp contract(off)
  constexpr int KM = (1 << (B - 1)) - 1;
  __shared__ __attribute__((aligned(16))) float aw[kFitMaxGroup];
  __shared__ float red_f[4];
  __shared__ int red_i[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t gpr = K / group;
  const int64_t gi = blockIdx.x;
  const int64_t n = gi / gpr, k0 = (gi - n * gpr) * group;
  const float* wg = w + n * K + k0;

  float m = 0.0f;
  for (int i = tid; i < group; i += 256) {
    const float x = fabsf(wg[i]);
    aw[i] = x;
    m = fmaxf(m, x);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if (lane == 0) red_f[wave] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(red_f[0], red_f[1]), fmaxf(red_f[2], red_f[3]));

  float best = INFINITY;
  int bidx = 0;
  for (int c = tid; c < kFitCandidates; c += 256) {
    const int p = c / kFitClipSteps, r = c - p * kFitClipSteps;
    const float a = 0.125f * static_cast<float>(g_fit_pairs.p[p][0]);
    const float b = 0.125f * static_cast<float>(g_fit_pairs.p[p][1]);
    const float s = (1.0f - static_cast<float>(r) * (1.0f / 32.0f)) * amax;
    // R_j = Kmax^3 q_j 2^24 = (A j K^2 + Bq j^2 K + C j^3) 2^21 with A = 8a,
    // Bq = 8b, C = 8 - A - Bq: small integers, exact in fp64
    const double A = static_cast<double>(g_fit_pairs.p[p][0]), Bq = static_cast<double>(g_fit_pairs.p[p][1]);
    const double C = 8.0 - A - Bq;
    float v[KM + 1];
    v[0] = 0.0f;
#pragma unroll
    for (int j = 1; j <= KM; ++j) {
      const double J = j, Kd = KM;
      v[j] = level_rn32_r(s, (A * (J * Kd * Kd) + Bq * (J * J * Kd) + C * (J * J * J)) * 0x1p21, KM);
    }
    float sse = 0.0f;
    for (int i = 0; i < group; i += 4) {
      const f32x4 x4 = *reinterpret_cast<const f32x4*>(aw + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float d = x4[e];                      // level 0
#pragma unroll
        for (int j = 1; j <= KM; ++j) d = fminf(d, fabsf(x4[e] - v[j]));
        sse = fmaf(d, d, sse);
      }
    }
    if (sse < best) {                         // candidates rise: the first minimum stays
      best = sse;
      bidx = c;
    }
  }
  // lexicographic (loss, index) minimum over the workgroup
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ob = __shfl_xor(best, off, 64);
    const int oi = __shfl_xor(bidx, off, 64);
    if (ob < best || (ob == best && oi < bidx)) {
      best = ob;
      bidx = oi;
    }
  }
  __syncthreads();                            // red_f's maximum has been read by every wave
  if (lane == 0) {
    red_f[wave] = best;
    red_i[wave] = bidx;
  }
  __syncthreads();
  best = red_f[0];
  bidx = red_i[0];
#pragma unroll
  for (int q = 1; q < 4; ++q)
    if (red_f[q] < best || (red_f[q] == best && red_i[q] < bidx)) {
      best = red_f[q];
      bidx = red_i[q];
    }

  const int p = bidx / kFitClipSteps, r = bidx - p * kFitClipSteps;
  const float a = 0.125f * static_cast<float>(g_fit_pairs.p[p][0]);
  const float b = 0.125f * static_cast<float>(g_fit_pairs.p[p][1]);
  const float s = (1.0f - static_cast<float>(r) * (1.0f / 32.0f)) * amax;
  if (tid == 0) {
    scales[gi] = s;
    shapes[gi] = static_cast<uint32_t>(f16_of(a)) | (static_cast<uint32_t>(f16_of(b)) << 16);
    if (loss) loss[gi] = best;
  }
}

}  // namespace

int fit_max_group() { return kFitMaxGroup; }

hipError_t launch_fit(const float* w, int64_t N, int64_t K, int bits, int group, int8_t* codes,
                      float* scales, uint16_t* shapes, float* loss, hipStream_t st) {
  const int64_t groups = N * (K / group);
  if (groups == 0) return hipSuccess;
  uint32_t* ab = reinterpret_cast<uint32_t*>(shapes);
#define CUBIC_FIT(BB)                                                                              \
  hipLaunchKernelGGL(k_fit<BB>, dim3(static_cast<unsigned>(groups)), dim3(256), 0, st, w, K, group, \
                     scales, ab, loss)
  switch (bits) {
    case 2: CUBIC_FIT(2); break;
    case 3: CUBIC_FIT(3); break;
    case 4: CUBIC_FIT(4); break;
    case 5: CUBIC_FIT(5); break;
    case 6: CUBIC_FIT(6); break;
    case 7: CUBIC_FIT(7); break;
    default: CUBIC_FIT(8); break;
  }
#undef CUBIC_FIT
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the codes of the chosen (s, a, b) by the nearest-level rule of cubic_encode
  return launch_encode(w, N, K, bits, group, scales, shapes, codes, st);
}

}  // namespace cubic
