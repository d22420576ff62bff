// prefill_a8.hip -- Dynamic A8 product for prefill-sized M with 2- and 3-bit
// codes (int8 MFMA bound).
//
// The CubicQuant article (section "一份 checkpoint，同时服务 A16 与 Dynamic A8")
// runs the A8 path as: per-token INT8 activations, an INT8 carrier of each
// weight level, an integer dot product per group and an fp32 group scale.
// Here one 256-thread workgroup owns a 128 (weight rows n) x 256 (activation
// rows m) output tile and walks K in steps of 128:
//  - wave w owns weight rows 32 w .. 32 w + 31 against all 256 activation rows
//    (8 blocks of 32 x 32): int32 accumulators for the open group and fp32
//    accumulators that take acc_i32 * fp32(s / 127) at every group end. Each
//    decoded weight fragment feeds 8 MFMAs;
//  - each lane decodes its row's codes in registers: the int8 carriers of the
//    row's 2^B field values sit in two registers, and one v_perm turns four
//    codes (their fields spread into a byte selector) into four carriers;
//  - every load of the step loop goes from global memory straight into a
//    4-stage LDS ring (buffer_load ... lds), three steps ahead: the int8
//    activation tile (XOR-swizzled so that the 16-byte fragment reads are free
//    of bank conflicts), the tile's code words and its group parameters. With
//    no vector load writing a register, the loop's only memory wait is the one
//    before each step's barrier;
//  - within a step, lane half h takes codes 64 h .. 64 h + 63 of its row: codes
//    64 h + 16 ks .. + 15 feed MFMA sub-step ks (0..3), and the activation
//    fragments follow the same K order.
// Carriers are exact: clamp(rne(127 q), +-127) decided with integer arithmetic
// (carrier_level), once per row and group in each lane of the row.
#include "common.h"
#include "launch.h"

namespace cubic {
namespace {

constexpr int A8N = 128;             // weight rows per tile
constexpr int A8M = 256;             // activation rows per tile
constexpr int A8K = 128;             // K per step
constexpr int kA8Threads = 256;
constexpr int kA8Stages = 4;
constexpr uint32_t kA8RsrcWord3 = 0x00020000u;   // raw buffer, 32-bit data format

// Stage layout: activations [A8M][A8K] int8, then the code words of the tile's
// A8N rows (A8K B / 8 bytes each, row-major), then the group parameters (per
// wave 512 bytes: 64 scales, 64 (a, b) words; lanes 32..63 repeat rows 0..31).
constexpr size_t kA8XBytes = static_cast<size_t>(A8M) * A8K;
constexpr size_t a8_code_bytes(int B) { return static_cast<size_t>(A8N) * A8K * B / 8; }
constexpr size_t kA8ParamBytes = 4 * 512;
constexpr size_t a8_stage_bytes(int B) { return kA8XBytes + a8_code_bytes(B) + kA8ParamBytes; }
constexpr size_t a8_lds_bytes(int B) { return kA8Stages * a8_stage_bytes(B); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t a8_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0),
                                           static_cast<int>(bytes), static_cast<int>(kA8RsrcWord3));
}

// s_waitcnt immediate: vmcnt(n) (n < 64: low 4 bits in [3:0], high 2 bits in
// [15:14]), expcnt not waited for, lgkmcnt(0).
constexpr int a8_wait_vm(int n) { return (n & 15) | (7 << 4) | (((n >> 4) & 3) << 14); }

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

// Swizzled position of 16-byte chunk q (0..7) of activation row r (128 bytes)
// in a stage: any 16 consecutive rows read at one chunk hit 16 distinct
// 16-byte bank groups (row parity and the XOR of the low three row bits and
// row bit 3 into the chunk index determine the address modulo 256).
__device__ __forceinline__ int a8_slot(int r, int q) {
  return r * 8 + (q ^ (r & 7) ^ ((r >> 3) & 1));
}

template <int B>
__global__ __launch_bounds__(kA8Threads, 1) void k_prefill_a8(TiledParams p) {
  extern __shared__ __align__(16) unsigned char smem[];       // kA8Stages stages
  constexpr int DPR = A8K * B / 32;             // code dwords per row and step
  constexpr size_t kStage = a8_stage_bytes(B);
  constexpr size_t kCodeOff = kA8XBytes;
  constexpr size_t kParamOff = kA8XBytes + a8_code_bytes(B);

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
  const uint32_t row_bytes = static_cast<uint32_t>(p.K * B / 8);
  const int64_t nrow = n0 + 32 * wave + c;      // this lane's weight row

  // ---- the step's loads: global -> LDS stage ----
  // activations: wave w fills slots 512 w + 64 i + lane (i = 0..7), 16 bytes each
  const __amdgpu_buffer_rsrc_t xrs = a8_rsrc(p.xa, static_cast<uint32_t>(p.M * p.K));
  uint32_t aoff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int slot = 512 * wave + 64 * i + lane;
    const int r = slot >> 3;
    const int q = (slot & 7) ^ (r & 7) ^ ((r >> 3) & 1);     // inverse of a8_slot
    aoff[i] = static_cast<uint32_t>((m0 + r) * p.K + 16 * q);  // rows past M read 0
  }
  // code words: dword slots of the tile's rows (row-major); wave w fills slots
  // 64 (NC w + i) + lane (i < NC); rows past N read 0
  constexpr int NC = A8N * DPR / 256;           // code loads per wave and step
  const __amdgpu_buffer_rsrc_t crs = a8_rsrc(p.codes, static_cast<uint32_t>(p.N) * row_bytes);
  uint32_t coff[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int slot = 64 * (NC * wave + i) + lane;
    const int r = slot / DPR, d = slot % DPR;
    coff[i] = static_cast<uint32_t>(n0 + r) * row_bytes + 4u * static_cast<uint32_t>(d);
  }
  // group parameters of the wave's 32 rows (lanes 32..63 repeat them)
  const int64_t pc = nrow < p.N ? nrow : p.N - 1;
  const __amdgpu_buffer_rsrc_t srs = a8_rsrc(p.scales, static_cast<uint32_t>(p.N * gpr * 4));
  const __amdgpu_buffer_rsrc_t brs = a8_rsrc(p.shapes, static_cast<uint32_t>(p.N * gpr * 4));
  const uint32_t poff = static_cast<uint32_t>(pc * gpr * 4);
  constexpr int NV = 8 + NC + 2;                // loads per wave and step
  auto issue_step = [&](int s, int stage) {
    unsigned char* st = smem + stage * kStage;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, st + wave * 8192 + i * 1024, 16,
                                               aoff[i] + static_cast<uint32_t>(s) * A8K, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < NC; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(crs, st + kCodeOff + 256 * (NC * wave + i), 4,
                                               coff[i] + static_cast<uint32_t>(s) * (4 * DPR), 0, 0, 0);
    int g = s / spg;
    g = g < gpr ? g : gpr - 1;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, st + kParamOff + 512 * wave, 4,
                                             poff + 4u * static_cast<uint32_t>(g), 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(brs, st + kParamOff + 512 * wave + 256, 4,
                                             poff + 4u * static_cast<uint32_t>(g), 0, 0, 0);
  };

  i32x16 acci[8];                              // the open group's sums (set by its first step)
  f32x16 accf[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      acci[j][e] = 0;
      accf[j][e] = 0.0f;
    }

  issue_step(0, 0);
  issue_step(1, 1);
  issue_step(2, 2);

  uint32_t t0 = 0u, t1 = 0u;
  float sc = 0.0f;
  int mg = 0;                                   // s % spg

  auto step = [&](int s, auto ph_c) {
    constexpr int ph = decltype(ph_c)::value;  // s % 4
    constexpr int ph3 = (ph + 3) % 4;
    // Stage s is complete once only the loads of the next two stages remain.
    // The bare barrier then publishes every wave's part of it, and every wave
    // has finished reading stage s - 1, which the loads of step s + 3 overwrite.
    static_assert(2 * NV < 64, "vmcnt holds at most 63");
    __builtin_amdgcn_s_waitcnt(a8_wait_vm(2 * NV));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // past K: step 0 again into the free stage (never read), so the count holds
    issue_step(s + 3 < nsteps ? s + 3 : 0, ph3);
    const unsigned char* st = smem + ph * kStage;
    uint32_t cw[2 * B];                         // this lane's 64 codes of the step
    {
      const uint32_t* src =
          reinterpret_cast<const uint32_t*>(st + kCodeOff) + DPR * (32 * wave + c) + 2 * B * h;
#pragma unroll
      for (int d = 0; d < 2 * B; ++d) cw[d] = src[d];
    }
    const bool fresh = mg == 0;                // the group's first step: int32 sums start at 0
    if (fresh) {
      // new group: the row's carriers and scale
      const uint32_t* par = reinterpret_cast<const uint32_t*>(st + kParamOff + 512 * wave);
      carrier_table<B>(par[64 + c], t0, t1);
      sc = __fdiv_rn(__uint_as_float(par[c]), 127.0f);
    }
    const int8_t* Ab = reinterpret_cast<const int8_t*>(st);
    // Activation fragments roll through one set of registers: right after MFMA
    // j of sub-step ks consumes fragment j, fragment j of sub-step ks + 1 is
    // read into it. The weight fragment of sub-step ks + 1 is decoded under
    // sub-step ks's MFMAs.
    i32x4 fa[8];
    auto read_a = [&](int ks, int j) {
      return *reinterpret_cast<const i32x4*>(Ab + 16 * a8_slot(32 * j + c, 4 * h + ks));
    };
    auto decode = [&](int ks) {
      uint32_t o[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        o[u] = __builtin_amdgcn_perm(t1, t0, a8_selector<B>(a8_quad<B>(cw, 4 * ks + u)));
      return i32x4{static_cast<int>(o[0]), static_cast<int>(o[1]), static_cast<int>(o[2]),
                   static_cast<int>(o[3])};
    };
#pragma unroll
    for (int j = 0; j < 8; ++j) fa[j] = read_a(0, j);
    i32x4 fb = decode(0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const i32x4 fbn = ks < 3 ? decode(ks + 1) : fb;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (ks == 0 && fresh) {
          acci[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[j], fb, i32x16{}, 0, 0, 0);
        } else {
          acci[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[j], fb, acci[j], 0, 0, 0);
        }
        if (ks < 3) fa[j] = read_a(ks + 1, j);
      }
      fb = fbn;
      __builtin_amdgcn_sched_barrier(0);
    }
    mg = mg + 1 == spg ? 0 : mg + 1;
    if (mg == 0) {
      // group end: fp32 group scale (exact int32 dot, |I| < 2^24)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          accf[j][e] = fmaf(static_cast<float>(acci[j][e]), sc, accf[j][e]);
        __builtin_amdgcn_sched_barrier(0);     // one block at a time (few temporaries)
      }
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
  __syncthreads();

  // ---- epilogue: the tile's activation scales through LDS (one load per
  // thread), then D row m = 8 (e / 4) + 4 h + e % 4 of block j, column n = c ----
  float* sxs = reinterpret_cast<float*>(smem);
  {
    const int64_t m = m0 + tid;
    sxs[tid] = m < p.M ? p.xs[m] : 0.0f;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int ml = 32 * j + 8 * (e >> 2) + 4 * h + (e & 3);
      const int64_t m = m0 + ml;
      if (m < p.M && nrow < p.N) p.y[m * p.N + nrow] = accf[j][e] * sxs[ml];
    }
  }
}

}  // namespace

// 2- and 3-bit codes, groups a multiple of 128 up to 1024 (exact int32 group
// dots), and byte sizes of the activation, code and parameter buffers (with a
// tile's overhang) below 2^32.
bool prefill_a8_supported(int64_t M, int64_t N, int64_t K, int bits, int group) {
  if (bits != 2 && bits != 3) return false;
  if (group % A8K != 0 || group > 1024 || K % A8K != 0) return false;
  if ((M + A8M) * K >= (int64_t{1} << 32)) return false;
  if ((N + A8N) * K * bits / 8 >= (int64_t{1} << 32)) return false;
  if (N * (K / group) * 4 >= (int64_t{1} << 32)) return false;
  const int64_t tiles = ((M + A8M - 1) / A8M) * ((N + A8N - 1) / A8N);
  return tiles <= INT32_MAX;
}

template <int B>
static hipError_t launch_prefill_a8_b(const TiledParams& p, hipStream_t st) {
  auto kern = k_prefill_a8<B>;
  constexpr size_t lds = a8_lds_bytes(B);
  static_assert(lds <= 160 * 1024, "one compute unit's LDS");
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(lds));
  if (e != hipSuccess) return e;
  const int64_t tiles = ((p.M + A8M - 1) / A8M) * ((p.N + A8N - 1) / A8N);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(tiles)), dim3(kA8Threads), lds, st, p);
  return hipGetLastError();
}

hipError_t launch_prefill_a8(const TiledParams& p, int bits, hipStream_t st) {
  return bits == 2 ? launch_prefill_a8_b<2>(p, st) : launch_prefill_a8_b<3>(p, st);
}

}  // namespace cubic
