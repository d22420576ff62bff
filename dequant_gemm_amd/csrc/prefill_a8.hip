// prefill_a8.hip -- Dynamic A8 product for prefill-sized M with 2- and 3-bit
// codes (int8 MFMA bound).
//
// The CubicQuant article (section "一份 checkpoint，同时服务 A16 与 Dynamic A8")
// runs the A8 path as: per-token INT8 activations, an INT8 carrier of each
// weight level, an integer dot product per group and an fp32 group scale.
// Here one 256-thread workgroup owns a 256 (weight rows n) x 128 (activation
// rows m) output tile and walks K in steps of 128:
//  - wave w owns weight rows 64 w .. 64 w + 63 against all 128 activation rows
//    (2 x 4 blocks of 32 x 32): int32 accumulators for the open group and fp32
//    accumulators that take acc_i32 * fp32(s / 127) at every group end;
//  - each lane decodes its own weight fragments in registers: the int8 carriers
//    of a row's 2^B field values sit in two registers, and one v_perm turns four
//    codes (their fields spread into a byte selector) into four carriers;
//  - the int8 activation tile goes from global memory straight into a 4-stage
//    LDS ring (buffer_load ... lds), three steps ahead, in an XOR-swizzled
//    layout that keeps the 16-byte fragment reads free of bank conflicts;
//  - within a step, lane half h takes codes 64 h .. 64 h + 63: codes
//    64 h + 16 ks .. + 15 feed MFMA sub-step ks (0..3), and the activation
//    fragments follow the same K order.
// Carriers are exact: clamp(rne(127 q), +-127) decided with integer arithmetic
// (carrier_level); each lane computes one of its two rows' tables and the pair
// is exchanged across the wave halves (permlane32_swap).
#include "common.h"
#include "launch.h"

namespace cubic {
namespace {

constexpr int A8N = 256;             // weight rows per tile
constexpr int A8M = 128;             // activation rows per tile
constexpr int A8K = 128;             // K per step
constexpr int kA8Threads = 256;
constexpr int kA8Stages = 4;
constexpr size_t kA8StageBytes = static_cast<size_t>(A8M) * A8K;     // int8
constexpr size_t kA8Lds = kA8Stages * kA8StageBytes;
constexpr uint32_t kA8RsrcWord3 = 0x00020000u;   // raw buffer, 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t a8_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0),
                                           static_cast<int>(bytes), static_cast<int>(kA8RsrcWord3));
}

// Byte selector for four consecutive B-bit fields in the low 4B bits of v
// (field i -> byte i), by two multiplies whose terms never overlap.
template <int B>
__device__ __forceinline__ uint32_t a8_selector(uint32_t v) {
  constexpr uint32_t fm = (1u << B) - 1u;
  constexpr uint32_t me = fm | (fm << (2 * B));
  constexpr uint32_t mo = (fm << B) | (fm << (3 * B));
  const uint32_t e = (v & me) * (1u + (1u << (16 - 2 * B)));
  const uint32_t o = (v & mo) * ((1u << (8 - B)) + (1u << (24 - 3 * B)));
  return ((e & 0x00FF00FFu) | (o & 0xFF00FF00u)) & (fm * 0x01010101u);
}

// Fields 4q .. 4q + 3 of a lane's 64 codes w[2B].
template <int B>
__device__ __forceinline__ uint32_t a8_quad(const uint32_t* w, int q) {
  const int bit = 4 * B * q;
  const int d = bit >> 5, off = bit & 31;
  uint32_t v;
  if (off + 4 * B <= 32) {
    v = w[d] >> off;
  } else {
    v = __builtin_amdgcn_alignbit(w[d + 1], w[d], off);
  }
  return v & ((1u << (4 * B)) - 1u);
}

// int8 carriers of field values 0..2^B-1 (two's complement codes) of one row
// and group, bytes of t0 (fields 0..3) and t1 (fields 4..7).
template <int B>
__device__ __forceinline__ void carrier_table(uint32_t ab, uint32_t& t0, uint32_t& t1) {
  static_assert(B == 2 || B == 3, "at most 8 carriers per table");
  constexpr int K = kmax_of(B);
  const double a = f16_bits_to_f64(static_cast<uint16_t>(ab & 0xffffu));
  const double b = f16_bits_to_f64(static_cast<uint16_t>(ab >> 16));
  auto byte = [](int v) { return static_cast<uint32_t>(v) & 0xffu; };
  if constexpr (B == 3) {
    // fields 0..7 -> codes 0, 1, 2, 3, -4, -3, -2, -1 (code 3 = Kmax: q = 1 -> 127)
    const int c1 = carrier_level(a, b, 1, K), c2 = carrier_level(a, b, 2, K);
    const int c4 = carrier_level(a, b, 4, K);
    t0 = byte(0) | (byte(c1) << 8) | (byte(c2) << 16) | (byte(127) << 24);
    t1 = byte(-c4) | (byte(-127) << 8) | (byte(-c2) << 16) | (byte(-c1) << 24);
  } else {
    // fields 0..3 -> codes 0, 1, -2, -1 (code 1 = Kmax: 127)
    const int c2 = carrier_level(a, b, 2, K);
    t0 = byte(0) | (byte(127) << 8) | (byte(-c2) << 16) | (byte(-127) << 24);
    t1 = 0u;
  }
}

// s_waitcnt immediate: vmcnt(n) (n < 64: low 4 bits in [3:0], high 2 bits in
// [15:14]), expcnt not waited for, lgkmcnt(0).
constexpr int a8_wait_vm(int n) { return (n & 15) | (7 << 4) | (((n >> 4) & 3) << 14); }

// A lane's 64 codes of one row and step: 2B dwords, loaded as 16-byte (2-bit)
// or two 12-byte (3-bit) pieces.
constexpr int a8_code_loads(int B) { return B == 2 ? 1 : 2; }

template <int B>
__device__ __forceinline__ void load_codes64(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t* w) {
  if constexpr (B == 2) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else {
    typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
    const u32x3 v0 = __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0);
    const u32x3 v1 = __builtin_amdgcn_raw_buffer_load_b96(r, off + 12, 0, 0);
    w[0] = v0.x; w[1] = v0.y; w[2] = v0.z;
    w[3] = v1.x; w[4] = v1.y; w[5] = v1.z;
  }
}

// Swizzled position of 16-byte chunk q (0..7) of activation row r (128 bytes)
// in a stage: any 16 consecutive rows read at one chunk hit 16 distinct
// 16-byte bank groups (row parity and the XOR of the low three row bits and
// row bit 3 into the chunk index determine the address modulo 256).
__device__ __forceinline__ int a8_slot(int r, int q) {
  return r * 8 + (q ^ (r & 7) ^ ((r >> 3) & 1));
}

template <int B>
__global__ __launch_bounds__(kA8Threads, 1) void k_prefill_a8(TiledParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  int8_t* As = reinterpret_cast<int8_t*>(smem);              // [4][A8M * A8K] swizzled

  const int tiles_n = static_cast<int>((p.N + A8N - 1) / A8N);
  const int ntiles = tiles_n * static_cast<int>((p.M + A8M - 1) / A8M);
  int t = static_cast<int>(blockIdx.x);
  // consecutive workgroup ids go to different XCDs: give each XCD a contiguous
  // run of tiles (which share activation rows) when the count divides
  if (ntiles % 8 == 0) t = (t % 8) * (ntiles / 8) + t / 8;
  const int64_t m0 = static_cast<int64_t>(t / tiles_n) * A8M;
  const int64_t n0 = static_cast<int64_t>(t % tiles_n) * A8N;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, h = lane >> 5;
  const int gpr = static_cast<int>(p.K / p.group);
  const int nsteps = static_cast<int>(p.K / A8K);
  const int spg = p.group / A8K;

  // ---- this lane's weight rows n0 + 64 wave + 32 i + c (i = 0, 1) ----
  const uint32_t row_bytes = static_cast<uint32_t>(p.K * B / 8);
  const __amdgpu_buffer_rsrc_t crs = a8_rsrc(p.codes, static_cast<uint32_t>(p.N) * row_bytes);
  uint32_t coff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t n = n0 + 64 * wave + 32 * i + c;
    coff[i] = static_cast<uint32_t>(n) * row_bytes + static_cast<uint32_t>(h * 8 * B);
  }
  // group parameters: this lane fetches those of its row i = h (the other half
  // of the wave fetches row 1 - h) and the two are exchanged after the decode
  const int64_t nown = n0 + 64 * wave + 32 * h + c;
  const int64_t nc = nown < p.N ? nown : p.N - 1;
  const float* srow = p.scales + nc * gpr;
  const uint32_t* abrow = reinterpret_cast<const uint32_t*>(p.shapes) + nc * gpr;

  // ---- activation stages: global -> LDS ----
  // Wave w fills slots 256 w + 64 i + lane (i = 0..3) of a stage.
  const __amdgpu_buffer_rsrc_t xrs = a8_rsrc(p.xa, static_cast<uint32_t>(p.M * p.K));
  uint32_t aoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int slot = 256 * wave + 64 * i + lane;
    const int r = slot >> 3;
    const int q = (slot & 7) ^ (r & 7) ^ ((r >> 3) & 1);     // inverse of a8_slot
    aoff[i] = static_cast<uint32_t>((m0 + r) * p.K + 16 * q);  // rows past M read 0
  }
  auto issue_a = [&](int s, int stage) {
    int8_t* dst = As + stage * kA8StageBytes + wave * 4096;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, dst + i * 1024, 16,
                                               aoff[i] + static_cast<uint32_t>(s) * A8K, 0, 0, 0);
  };

  // ---- NV vector loads per step, in this order: 4 activation loads (to LDS)
  // for step s + 3, then the code words of both rows and the 2 group
  // parameters for step s + 2 (codes run one step behind the activations, so
  // three code slots are live instead of four) ----
  constexpr int CW = 2 * B;                     // code dwords per row and step
  constexpr int NV = 4 + 2 * a8_code_loads(B) + 2;
  uint32_t cw[4][2][CW];
  float gs[4];
  uint32_t gab[4];
  auto issue_codes = [&](int sc, int par) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      load_codes64<B>(crs, coff[i] + static_cast<uint32_t>(sc) * (A8K * B / 8), cw[par][i]);
    int g = sc / spg;
    g = g < gpr ? g : gpr - 1;
    gs[par] = srow[g];
    gab[par] = abrow[g];
  };
  auto issue_step = [&](int sa, int pa, int sc, int pc) {
    issue_a(sa, pa);
    __builtin_amdgcn_sched_barrier(0);          // the activation loads go first
    issue_codes(sc, pc);
    __builtin_amdgcn_sched_barrier(0);
  };

  i32x16 acci[2][4];                           // the open group's sums (set by its first step)
  f32x16 accf[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        acci[i][j][e] = 0;
        accf[i][j][e] = 0.0f;
      }

  // prologue: activations of steps 0..2 and codes of steps 0..1; after stage
  // 2 a filler (codes of step 0 into the slot of step 3, overwritten later)
  // keeps NV - 4 code-side loads behind every stage, so the count below holds
  // from the first step on
  issue_step(0, 0, 0, 0);
  issue_step(1, 1, 1, 1);
  issue_step(2, 2, 0, 3);

  uint32_t t0[2] = {0u, 0u}, t1[2] = {0u, 0u};
  float sc[2] = {0.0f, 0.0f};
  int mg = 0;                                   // s % spg

  auto step = [&](int s, auto ph_c) {
    constexpr int ph = decltype(ph_c)::value;  // s % 4
    constexpr int ph3 = (ph + 3) % 4;
    // Stage s is complete once only the loads issued after it remain: the code
    // and parameter loads that follow it and the NV loads of each of the next
    // two stages. The bare barrier then publishes every wave's part of it, and
    // every wave has finished reading stage s - 1, which the loads of step s + 3
    // overwrite.
    static_assert(3 * NV - 4 < 64, "vmcnt holds at most 63");
    __builtin_amdgcn_s_waitcnt(a8_wait_vm(3 * NV - 4));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    {
      // past K: step 0 again into the free stage / slot (never read), so the
      // counts still hold
      const int sa = s + 3 < nsteps ? s + 3 : 0;
      const int sc = s + 2 < nsteps ? s + 2 : 0;
      issue_step(sa, ph3, sc, (ph + 2) % 4);
    }
    if (mg == 0) {
      // new group: carriers and scale of this lane's own row, then the pair
      uint32_t a0, a1;
      carrier_table<B>(gab[ph], a0, a1);
      const float so = __fdiv_rn(gs[ph], 127.0f);
      const auto x0 = __builtin_amdgcn_permlane32_swap(a0, a0, false, false);
      const auto x1 = __builtin_amdgcn_permlane32_swap(a1, a1, false, false);
      const auto xs = __builtin_amdgcn_permlane32_swap(__float_as_uint(so), __float_as_uint(so),
                                                       false, false);
      t0[0] = x0[0]; t0[1] = x0[1];
      t1[0] = x1[0]; t1[1] = x1[1];
      sc[0] = __uint_as_float(xs[0]);
      sc[1] = __uint_as_float(xs[1]);
    }
    const int8_t* Ab = As + ph * kA8StageBytes;
    const bool fresh = mg == 0;                // the group's first step: int32 sums start at 0
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      i32x4 fa[4], fb[2];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 32 * j + c;
        fa[j] = *reinterpret_cast<const i32x4*>(Ab + 16 * a8_slot(r, 4 * h + ks));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        uint32_t o[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          o[u] = __builtin_amdgcn_perm(t1[i], t0[i], a8_selector<B>(a8_quad<B>(cw[ph][i], 4 * ks + u)));
        fb[i] = i32x4{static_cast<int>(o[0]), static_cast<int>(o[1]), static_cast<int>(o[2]),
                      static_cast<int>(o[3])};
      }
      if (ks == 0 && fresh) {
        const i32x16 zero = {};
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acci[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[j], fb[i], zero, 0, 0, 0);
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acci[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[j], fb[i], acci[i][j], 0, 0, 0);
      }
    }
    mg = mg + 1 == spg ? 0 : mg + 1;
    if (mg == 0 || s + 1 == nsteps) {
      // group end: fp32 group scale (exact int32 dot, |I| < 2^24)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            accf[i][j][e] = fmaf(static_cast<float>(acci[i][j][e]), sc[i], accf[i][j][e]);
    }
  };
  int s = 0;
  for (; s + 3 < nsteps; s += 4) {
    step(s, std::integral_constant<int, 0>{});
    step(s + 1, std::integral_constant<int, 1>{});
    step(s + 2, std::integral_constant<int, 2>{});
    step(s + 3, std::integral_constant<int, 3>{});
  }
  if (s < nsteps) step(s, std::integral_constant<int, 0>{});
  if (s + 1 < nsteps) step(s + 1, std::integral_constant<int, 1>{});
  if (s + 2 < nsteps) step(s + 2, std::integral_constant<int, 2>{});
  __builtin_amdgcn_s_waitcnt(0);               // loads past K target stages nobody reads

  // ---- epilogue: D row m = 8 (e / 4) + 4 h + e % 4 of block j, column n = c of block i ----
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t m = m0 + 32 * j + 8 * (e >> 2) + 4 * h + (e & 3);
      if (m >= p.M) continue;
      const float sx = p.xs[m];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int64_t n = n0 + 64 * wave + 32 * i + c;
        if (n < p.N) p.y[m * p.N + n] = accf[i][j][e] * sx;
      }
    }
  }
}

}  // namespace

// 2- and 3-bit codes, groups a multiple of 128 up to 1024 (exact int32 group
// dots), and byte sizes of the activation and code buffers below 2^32.
bool prefill_a8_supported(int64_t M, int64_t N, int64_t K, int bits, int group) {
  if (bits != 2 && bits != 3) return false;
  if (group % A8K != 0 || group > 1024 || K % A8K != 0) return false;
  if (M * K >= (int64_t{1} << 32)) return false;
  if (N * K * bits / 8 >= (int64_t{1} << 32)) return false;
  const int64_t tiles = ((M + A8M - 1) / A8M) * ((N + A8N - 1) / A8N);
  return tiles <= INT32_MAX;
}

template <int B>
static hipError_t launch_prefill_a8_b(const TiledParams& p, hipStream_t st) {
  auto kern = k_prefill_a8<B>;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(kA8Lds));
  if (e != hipSuccess) return e;
  const int64_t tiles = ((p.M + A8M - 1) / A8M) * ((p.N + A8N - 1) / A8N);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(tiles)), dim3(kA8Threads), kA8Lds, st, p);
  return hipGetLastError();
}

hipError_t launch_prefill_a8(const TiledParams& p, int bits, hipStream_t st) {
  return bits == 2 ? launch_prefill_a8_b<2>(p, st) : launch_prefill_a8_b<3>(p, st);
}

}  // namespace cubic
