// basic.hip -- code-stream pack/unpack, fp32 dequant and per-row INT8
// activation quantisation (HBM-bound elementwise kernels).
//
// Stream layout: one LSB-first bit stream over the row-major [N][K] code matrix,
// each code a `bits`-wide two's complement field (the CubicQuant article on
// ModelScope only says the codes are plain 1-8 bit integers packed densely; the
// bit order is this library's reading). With K a multiple of 32 each block of 32
// consecutive codes of a row occupies exactly `bits` dwords, so one thread owns
// one block and no two threads touch the same dword.
#include "common.h"
#include "decode.h"
#include "launch.h"

namespace cubic {

__device__ unsigned int g_pack_range_error;   // set by k_pack, read by the host

__global__ void k_clear_pack_flag() {
  if (threadIdx.x == 0 && blockIdx.x == 0) g_pack_range_error = 0u;
}

template <int BITS>
__global__ __launch_bounds__(256) void k_pack(const int8_t* __restrict__ codes,
                                              uint32_t* __restrict__ out, int64_t nblocks) {
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (blk >= nblocks) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(codes + blk * 32);
  const u32x4 lo = src[0], hi = src[1];
  const uint32_t words[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  constexpr int km = kmax_of(BITS);
  uint32_t w[BITS];
#pragma unroll
  for (int d = 0; d < BITS; ++d) w[d] = 0u;
  bool bad = false;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int k = static_cast<int8_t>((words[i >> 2] >> (8 * (i & 3))) & 0xffu);
    bad |= (k > km) | (k < -km);
    const uint32_t f = static_cast<uint32_t>(k) & ((1u << BITS) - 1u);
    const int bit = i * BITS, d = bit >> 5, off = bit & 31;
    w[d] |= f << off;
    if (off + BITS > 32) w[d + 1] |= f >> (32 - off);
  }
  uint32_t* dst = out + blk * BITS;
#pragma unroll
  for (int d = 0; d < BITS; ++d) dst[d] = w[d];
  if (bad) atomicOr(&g_pack_range_error, 1u);
}

template <int BITS>
__global__ __launch_bounds__(256) void k_unpack(const uint32_t* __restrict__ in,
                                                int8_t* __restrict__ codes, int64_t nblocks) {
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (blk >= nblocks) return;
  uint32_t w[BITS];
  const uint32_t* src = in + blk * BITS;
#pragma unroll
  for (int d = 0; d < BITS; ++d) w[d] = src[d];
  uint32_t words[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) words[q] = 0u;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int k = sign_extend(chunk_field<BITS>(w, i), BITS);
    words[i >> 2] |= (static_cast<uint32_t>(k) & 0xffu) << (8 * (i & 3));
  }
  u32x4* dst = reinterpret_cast<u32x4*>(codes + blk * 32);
  dst[0] = u32x4{words[0], words[1], words[2], words[3]};
  dst[1] = u32x4{words[4], words[5], words[6], words[7]};
}

// One thread per 32-code block: each weight is the format's fp32 value
// RN32(s * sign(k) * q(|k| / Kmax)) (level_rn32); a zero weight is +0.0.
template <int BITS>
__global__ __launch_bounds__(256) void k_dequant(const uint32_t* __restrict__ stream,
                                                 const float* __restrict__ scales,
                                                 const uint16_t* __restrict__ shapes,
                                                 float* __restrict__ out, int64_t nblocks,
                                                 int64_t K, int group) {
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (blk >= nblocks) return;
  const int64_t k0 = blk * 32;                  // flat index of the first code
  const int64_t n = k0 / K, kk = k0 - n * K;
  const int64_t g = n * (K / group) + kk / group;
  const float s = scales[g];
  const float a = static_cast<float>(f16_bits_to_f64(shapes[2 * g]));
  const float b = static_cast<float>(f16_bits_to_f64(shapes[2 * g + 1]));
  constexpr int km = kmax_of(BITS);
  uint32_t w[BITS];
  const uint32_t* src = stream + blk * BITS;
#pragma unroll
  for (int d = 0; d < BITS; ++d) w[d] = src[d];
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int k = sign_extend(chunk_field<BITS>(w, i), BITS);
    const int j = k < 0 ? -k : k;
    const float mag = level_rn32(s, a, b, j, km);
    v[i] = (mag == 0.0f) ? 0.0f : (k < 0 ? -mag : mag);
  }
  f32x4* dst = reinterpret_cast<f32x4*>(out + k0);
#pragma unroll
  for (int q = 0; q < 8; ++q) dst[q] = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
}

// Per-row INT8 quantisation (the msModelSlim article's per-token dynamic scheme,
// with this library's reading of the A8 scale): sx = fp32(amax / 127) and
// q = clamp(rne(fp32(x / sx)), -127, 127), bit for bit.
//
// The quotient is not formed per element. With r = v_rcp_f32(sx) (1 ulp),
// x * r is within 2^-16 of x / sx for |x| <= amax, and the IEEE quotient within
// 2^-18, so whenever x * r lies more than 2^-14 from every half-integer both
// round to the same integer. One fma against 1.5 * 2^23 rounds x * r to the
// nearest integer n (ties to even) and leaves n in the low byte of its bits;
// a second fma gives the residual x * r - n. Lanes with a residual within 2^-14
// of one half, and rows whose scale lies outside [2^-100, 2^100] (tiny or huge
// rows, where the bound or the reciprocal fails), take the IEEE division.
constexpr float kRneMagic = 12582912.0f;        // 1.5 * 2^23

// Eight bf16 values (one 16-byte vector) to eight int8 codes.
// Eight bf16 (or, with XF16, fp16) values of one 16-byte vector as fp32 (exact).
template <bool XF16>
__device__ __forceinline__ void unpack8(const u32x4& v, float* xv) {
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if constexpr (XF16) {
      xv[2 * q] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(u[q] & 0xffffu)));
      xv[2 * q + 1] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(u[q] >> 16)));
    } else {
      xv[2 * q] = __uint_as_float(u[q] << 16);
      xv[2 * q + 1] = __uint_as_float(u[q] & 0xffff0000u);
    }
  }
}

template <bool XF16>
__device__ __forceinline__ uint2 quant8(const u32x4& v, float sx, float rcp, bool fast) {
  float xv[8];
  unpack8<XF16>(v, xv);
  uint32_t f[8];
  bool exact = !fast;
  if (fast) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float y = fmaf(xv[e], rcp, kRneMagic);
      const float n = y - kRneMagic;                 // exact: the rounded integer
      const float t = fmaf(xv[e], rcp, -n);          // x * r - n, one rounding
      exact = exact || fabsf(t) > 0.5f - 0x1p-14f;
      f[e] = __float_as_uint(y);                     // low byte: n (two's complement)
    }
  }
  if (exact) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int qi = 0;
      if (sx != 0.0f) {
        float r = rintf(__fdiv_rn(xv[e], sx));
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        qi = static_cast<int>(r);
      }
      f[e] = static_cast<uint32_t>(qi);
    }
  }
  const uint32_t lo = __builtin_amdgcn_perm(f[1], f[0], 0x0c0c0400u) | __builtin_amdgcn_perm(f[3], f[2], 0x04000c0cu);
  const uint32_t hi = __builtin_amdgcn_perm(f[5], f[4], 0x0c0c0400u) | __builtin_amdgcn_perm(f[7], f[6], 0x04000c0cu);
  return make_uint2(lo, hi);
}

template <bool XF16>
__device__ __forceinline__ float absmax8(const u32x4& v, float a) {
  float xv[8];
  unpack8<XF16>(v, xv);
#pragma unroll
  for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(xv[e]));
  return a;
}

// Row maximum over the block's 256 threads; returns sx, written by thread 0.
__device__ __forceinline__ float row_scale(float amax, float* red, float* xs_m) {
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sx = __fdiv_rn(amax, 127.0f);
  if (threadIdx.x == 0) *xs_m = sx;
  return sx;
}

// One 256-thread block per row. V > 0: the row (at most 256 * V vectors of 8)
// is read once into registers, all of its loads in flight together. V == 0:
// rows of any length, two passes (the second hits L2).
template <int V, bool XF16>
__global__ __launch_bounds__(256) void k_act_quant(const uint16_t* __restrict__ x, int64_t K,
                                                   int8_t* __restrict__ xq,
                                                   float* __restrict__ xs) {
  __shared__ float red[4];
  const int64_t m = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t nvec = K / 8;                   // K is a multiple of 8 (checked on the host)
  const u32x4* rv = reinterpret_cast<const u32x4*>(x + m * K);
  uint2* qv = reinterpret_cast<uint2*>(xq + m * K);
  float amax = 0.0f;
  if constexpr (V > 0) {
    u32x4 v[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int64_t i = tid + 256 * j;
      v[j] = i < nvec ? rv[i] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < V; ++j) amax = absmax8<XF16>(v[j], amax);
    const float sx = row_scale(amax, red, xs + m);
    const bool fast = sx >= 0x1p-100f && sx <= 0x1p100f;
    const float rcp = __builtin_amdgcn_rcpf(sx);
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int64_t i = tid + 256 * j;
      if (i < nvec) qv[i] = quant8<XF16>(v[j], sx, rcp, fast);
    }
  } else {
    for (int64_t i = tid; i < nvec; i += 256) amax = absmax8<XF16>(rv[i], amax);
    const float sx = row_scale(amax, red, xs + m);
    const bool fast = sx >= 0x1p-100f && sx <= 0x1p100f;
    const float rcp = __builtin_amdgcn_rcpf(sx);
    for (int64_t i = tid; i < nvec; i += 256) qv[i] = quant8<XF16>(rv[i], sx, rcp, fast);
  }
}

// Nearest-level encoding (CubicQuant article, Core: each weight takes the code
// of its group's nearest reconstruction level). The levels are the format's
// fp32 values L_{+-j} = +-v_j, v_j = level_rn32(s, a, b, j) for j = 0 .. Kmax;
// the code is the first j (smallest |k|) of smallest exact distance
// | |w| - |v_j| |, with k = j * sign(w) * sign(v_j).
//
// A workgroup covers 2048 consecutive weights (whole groups, since K is a
// multiple of the group): its threads first build the |v_j| and signs of every
// group it touches in LDS, then each thread encodes 8 weights. Distances are
// compared in fp32 first: rounding is monotone, so a smaller rounded distance
// means a smaller exact one and a larger means larger. Only equal rounded
// distances are decided exactly, in fp64, where x = |w| and y = |v_j| are exact
// and Fast2Sum gives hi = fl(max - min), lo = (max - hi) - min with hi + lo =
// |x - y|, compared lexicographically. NaN distances never win (a NaN weight
// takes code 0).
constexpr int kEncodeWeights = 2048;            // per workgroup: 256 threads x 8

__device__ __forceinline__ bool exact_closer(float x, float y, float yb) {
  const double xd = x, a = y, b = yb;
  const bool ga = xd >= a, gb = xd >= b;
  const double pa = ga ? xd : a, ma = ga ? a : xd, pb = gb ? xd : b, mb = gb ? b : xd;
  const double ha = pa - ma, la = (pa - ha) - ma;
  const double hb = pb - mb, lb = (pb - hb) - mb;
  return ha < hb || (ha == hb && la < lb);
}

template <int B>
__global__ __launch_bounds__(256) void k_encode(const float* __restrict__ w, int64_t nvec, int64_t K,
                                                int group, const float* __restrict__ scales,
                                                const uint32_t* __restrict__ shapes,
                                                int8_t* __restrict__ codes) {
#pragma clang fp contract(off)
  constexpr int KM = (1 << (B - 1)) - 1;
  constexpr int L = KM + 1;
  constexpr int kMaxGroups = kEncodeWeights / 128 + 1;
  __shared__ float s_lv[kMaxGroups * L];        // |v_j| of each group the workgroup touches
  __shared__ uint32_t s_neg[kMaxGroups * L];    // 1 where v_j is negative
  const int tid = threadIdx.x;
  const int64_t w0 = static_cast<int64_t>(blockIdx.x) * kEncodeWeights;
  const int64_t total = nvec * 8;
  const int64_t g0 = w0 / group;
  const int64_t wlast = min(w0 + kEncodeWeights, total) - 1;
  const int ng = static_cast<int>(wlast / group - g0) + 1;
  for (int t = tid; t < ng * L; t += 256) {
    const int gl = t / L, j = t - gl * L;
    const int64_t gi = g0 + gl;
    const uint32_t ab = shapes[gi];
    const float a = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(ab & 0xffffu)));
    const float b = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(ab >> 16)));
    const float lv = level_rn32(scales[gi], a, b, j, KM);
    s_lv[t] = fabsf(lv);
    s_neg[t] = __builtin_signbit(lv) ? 1u : 0u;
  }
  __syncthreads();
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + tid;
  if (i >= nvec) return;
  const int64_t e0 = i * 8;                     // first weight (row-major [N][K])
  const int gl = static_cast<int>(e0 / group - g0);
  const float* lv = s_lv + gl * L;
  const f32x4 lo4 = reinterpret_cast<const f32x4*>(w + e0)[0];
  const f32x4 hi4 = reinterpret_cast<const f32x4*>(w + e0)[1];
  const float wv[8] = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
  float x[8], bd[8], by[8];
  int bj[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x[e] = fabsf(wv[e]);
    bd[e] = x[e];                               // j = 0: v_0 = +0, distance |w| exactly
    by[e] = 0.0f;
    bj[e] = 0;
  }
  for (int j = 1; j <= KM; ++j) {
    const float y = lv[j];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = fabsf(x[e] - y);
      bool better = d < bd[e];
      if (d == bd[e]) better = exact_closer(x[e], y, by[e]);
      bd[e] = better ? d : bd[e];
      by[e] = better ? y : by[e];
      bj[e] = better ? j : bj[e];
    }
  }
  uint32_t o[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const bool neg = s_neg[gl * L + bj[e]] != 0u;
    const int k = (__builtin_signbit(wv[e]) != neg) ? -bj[e] : bj[e];
    o[e >> 2] |= (static_cast<uint32_t>(k) & 0xffu) << (8 * (e & 3));
  }
  reinterpret_cast<uint2*>(codes + e0)[0] = make_uint2(o[0], o[1]);
}

__global__ __launch_bounds__(256) void k_fill_zero(float* __restrict__ y, int64_t n, int bf16) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    store_out(y, bf16 != 0, i, 0.0f);
}

}  // namespace cubic

// ---------------------------------------------------------------------------
// Host-side launchers (called from api.cpp after validation).
// ---------------------------------------------------------------------------
namespace cubic {

#define CUBIC_DISPATCH_BITS(bits, FN, ...)              \
  switch (bits) {                                       \
    case 2: FN<2>(__VA_ARGS__); break;                  \
    case 3: FN<3>(__VA_ARGS__); break;                  \
    case 4: FN<4>(__VA_ARGS__); break;                  \
    case 5: FN<5>(__VA_ARGS__); break;                  \
    case 6: FN<6>(__VA_ARGS__); break;                  \
    case 7: FN<7>(__VA_ARGS__); break;                  \
    default: FN<8>(__VA_ARGS__); break;                 \
  }

template <int B>
static void launch_pack_b(const int8_t* codes, uint8_t* packed, int64_t nblocks, hipStream_t st) {
  const unsigned grid = static_cast<unsigned>((nblocks + 255) / 256);
  hipLaunchKernelGGL(k_pack<B>, dim3(grid), dim3(256), 0, st, codes,
                     reinterpret_cast<uint32_t*>(packed), nblocks);
}

template <int B>
static void launch_unpack_b(const uint8_t* packed, int8_t* codes, int64_t nblocks, hipStream_t st) {
  const unsigned grid = static_cast<unsigned>((nblocks + 255) / 256);
  hipLaunchKernelGGL(k_unpack<B>, dim3(grid), dim3(256), 0, st,
                     reinterpret_cast<const uint32_t*>(packed), codes, nblocks);
}

template <int B>
static void launch_dequant_b(const uint8_t* stream, const float* scales, const uint16_t* shapes,
                             float* out, int64_t nblocks, int64_t K, int group, hipStream_t st) {
  const unsigned grid = static_cast<unsigned>((nblocks + 255) / 256);
  hipLaunchKernelGGL(k_dequant<B>, dim3(grid), dim3(256), 0, st,
                     reinterpret_cast<const uint32_t*>(stream), scales, shapes, out, nblocks, K,
                     group);
}

hipError_t launch_pack(const int8_t* codes, uint8_t* packed, int64_t N, int64_t K, int bits,
                       hipStream_t st, unsigned int* range_error) {
  hipLaunchKernelGGL(k_clear_pack_flag, dim3(1), dim3(64), 0, st);
  const int64_t nblocks = N * K / 32;
  CUBIC_DISPATCH_BITS(bits, launch_pack_b, codes, packed, nblocks, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  unsigned int flag = 0;
  e = hipMemcpyFromSymbolAsync(&flag, HIP_SYMBOL(g_pack_range_error), sizeof(flag), 0,
                               hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(st);
  *range_error = flag;
  return e;
}

hipError_t launch_unpack(const uint8_t* packed, int8_t* codes, int64_t N, int64_t K, int bits,
                         hipStream_t st) {
  const int64_t nblocks = N * K / 32;
  CUBIC_DISPATCH_BITS(bits, launch_unpack_b, packed, codes, nblocks, st);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* stream, const float* scales, const uint16_t* shapes,
                          float* out, int64_t N, int64_t K, int bits, int group, hipStream_t st) {
  const int64_t nblocks = N * K / 32;
  CUBIC_DISPATCH_BITS(bits, launch_dequant_b, stream, scales, shapes, out, nblocks, K, group, st);
  return hipGetLastError();
}

template <bool XF16>
static auto act_quant_kernel(int64_t K) {
  // registers per thread: the row's vectors over 256 threads, in steps of powers of two
  const int64_t per = (K / 8 + 255) / 256;
  return per <= 1 ? k_act_quant<1, XF16> : per <= 2 ? k_act_quant<2, XF16> : per <= 4 ? k_act_quant<4, XF16>
                  : per <= 8 ? k_act_quant<8, XF16> : k_act_quant<0, XF16>;
}

hipError_t launch_act_quant(const uint16_t* x, bool xf16, int64_t M, int64_t K, int8_t* xq, float* xs,
                            hipStream_t st) {
  auto kern = xf16 ? act_quant_kernel<true>(K) : act_quant_kernel<false>(K);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(M)), dim3(256), 0, st, x, K, xq, xs);
  return hipGetLastError();
}

hipError_t launch_encode(const float* w, int64_t N, int64_t K, int bits, int group, const float* scales,
                         const uint16_t* shapes, int8_t* codes, hipStream_t st) {
  const int64_t nvec = N * K / 8;
  if (nvec == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>((nvec * 8 + kEncodeWeights - 1) / kEncodeWeights);
  const uint32_t* ab = reinterpret_cast<const uint32_t*>(shapes);
#define CUBIC_ENCODE(BB)                                                                            \
  hipLaunchKernelGGL(k_encode<BB>, dim3(grid), dim3(256), 0, st, w, nvec, K, group, scales, ab, codes)
  switch (bits) {
    case 2: CUBIC_ENCODE(2); break;
    case 3: CUBIC_ENCODE(3); break;
    case 4: CUBIC_ENCODE(4); break;
    case 5: CUBIC_ENCODE(5); break;
    case 6: CUBIC_ENCODE(6); break;
    case 7: CUBIC_ENCODE(7); break;
    default: CUBIC_ENCODE(8); break;
  }
#undef CUBIC_ENCODE
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* y, int64_t n, bool bf16, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_fill_zero, dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)), dim3(256),
                     0, st, y, n, bf16 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace cubic
