// prefill.hip -- A16 product for prefill-sized M with 2- and 3-bit codes
// (MFMA bound).
//
// The CubicQuant article (section "压缩权重必须边解码、边计算") decodes each
// weight tile inside the kernel that consumes it. Here one 256-thread workgroup
// owns a 256 (weight rows n) x 256 (activation rows m) output tile and walks K in
// steps of 64:
//  - wave w owns weight rows 64w .. 64w + 63 of the tile against all 256
//    activation rows (2 x 8 blocks of 32 x 32, 256 fp32 accumulators);
//  - each lane decodes its own weight fragments straight into MFMA operand
//    registers: lane (c, h) holds row 32 i + c and codes 32 h .. 32 h + 31 of the
//    step; each code is looked up in the row's level table held in four
//    registers (byte-wise v_perm: lo and hi bytes of 2^B fp16 levels). No weight
//    value passes through LDS and no row is decoded twice;
//  - the fp16 activation tile (prepared by k_xprep) goes from global memory
//    straight into LDS (buffer_load ... lds), double buffered, in an XOR-swizzled
//    layout that keeps the MFMA fragment reads free of bank conflicts;
//  - within a step the K order is permuted identically on both operands: MFMA
//    block kb takes codes 8 kb .. 8 kb + 7 of each 32-code half.
// Levels are fp16(s * q * 2^-e_n), with 2^e_n a per-row power of two at or above
// the row's largest group scale, so every level fits fp16 whatever s is; the
// epilogue multiplies by 2^e_n and by the activation row's prescale factor.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace cubic {
namespace {

constexpr int PT = 256;              // tile edge (rows of W and of x)
constexpr int PK = 64;               // K per step
constexpr int kPrefillThreads = 256;
constexpr size_t kABufBytes = static_cast<size_t>(PT) * PK * 2;     // one activation buffer
constexpr int kABufs = 3;                                           // activation stages
constexpr size_t kPrefillLds = kABufs * kABufBytes + 2 * PT * sizeof(float);

constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer, 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0),
                                           static_cast<int>(bytes), static_cast<int>(kRsrcWord3));
}

// v_perm selector for four consecutive B-bit codes held in the low 4B bits of v:
// code i goes to byte i. Codes 0 and 2 (mask me) are moved with one multiply,
// codes 1 and 3 (mask mo) with another; the multiplier terms never overlap, so
// no carries spill between fields.
template <int B>
__device__ __forceinline__ uint32_t perm_selector(uint32_t v) {
  constexpr uint32_t fm = (1u << B) - 1u;
  constexpr uint32_t me = fm | (fm << (2 * B));
  constexpr uint32_t mo = (fm << B) | (fm << (3 * B));
  const uint32_t e = (v & me) * (1u + (1u << (16 - 2 * B)));
  const uint32_t o = (v & mo) * ((1u << (8 - B)) + (1u << (24 - 3 * B)));
  return ((e & 0x00FF00FFu) | (o & 0xFF00FF00u)) & (fm * 0x01010101u);
}

// Field of 4B bits starting at bit 4B*j of the step's code words.
template <int B>
__device__ __forceinline__ uint32_t quad_field(const uint32_t* w, int j) {
  const int bit = 4 * B * j;
  const int d = bit >> 5, off = bit & 31;
  uint32_t v;
  if (off + 4 * B <= 32) {
    v = w[d] >> off;
  } else {
    v = __builtin_amdgcn_alignbit(w[d + 1], w[d], off);
  }
  return v & ((1u << (4 * B)) - 1u);
}

// Level table of one row and group as lo and hi bytes of the fp16 levels of
// field values 0..7 (entries past 2^B are unused).
struct PermTable {
  uint32_t lo0, lo1, hi0, hi1;
};

// Level of magnitude j, times Kmax^3: Q_j = a (j K^2 - j^3) + b (j^2 K - j^3) + j^3
// (K = Kmax; the cubic with c = 1 - a - b collected by a and b). The products
// with fp16 a, b are exact in fp32; the two additions round at most twice,
// far below the fp16 resolution of the table entries.
template <int B>
__device__ __forceinline__ uint32_t table_level(float a, float b, float sk, int j) {
  constexpr int K = kmax_of(B);
  const float al = static_cast<float>(j * K * K - j * j * j);
  const float be = static_cast<float>(j * j * K - j * j * j);
  const float q = fmaf(a, al, fmaf(b, be, static_cast<float>(j * j * j)));
  return f16_bits(sk * q);
}

// fp16 levels of field values 0..2^B-1 (two's complement codes) of one row and
// group, scaled by s * 2^-e_n, as lo and hi bytes: code +-j share the lo byte,
// the negative one flips the sign bit of the hi byte.
template <int B>
__device__ __forceinline__ PermTable make_perm_table(float s, uint32_t ab, float inv_rowscale) {
  static_assert(B == 2 || B == 3, "perm tables hold at most 8 levels");
  constexpr int K = kmax_of(B);
  const float a = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(ab & 0xffffu)));
  const float b = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(ab >> 16)));
  const float sc = s * inv_rowscale;                     // exact (power of two)
  const float sk = sc * (1.0f / static_cast<float>(K * K * K));
  PermTable t;
  if constexpr (B == 3) {
    // field values 0..7 -> codes 0, 1, 2, 3, -4, -3, -2, -1
    const uint32_t L1 = table_level<3>(a, b, sk, 1), L2 = table_level<3>(a, b, sk, 2);
    const uint32_t L3 = f16_bits(sc), L4 = table_level<3>(a, b, sk, 4);
    const uint32_t P = L1 | (L2 << 16), Q = L3 | (L4 << 16);
    t.lo0 = __builtin_amdgcn_perm(Q, P, 0x0402000Cu);    // 0, L1, L2, L3
    t.lo1 = __builtin_amdgcn_perm(Q, P, 0x00020406u);    // L4, L3, L2, L1
    t.hi0 = __builtin_amdgcn_perm(Q, P, 0x0503010Cu);
    t.hi1 = __builtin_amdgcn_perm(Q, P, 0x01030507u) ^ 0x80808080u;
  } else {
    // field values 0..3 -> codes 0, 1, -2, -1
    const uint32_t L1 = f16_bits(sc), L2 = table_level<2>(a, b, sk, 2);
    const uint32_t P = L1 | (L2 << 16);
    t.lo0 = __builtin_amdgcn_perm(0u, P, 0x0002000Cu);   // 0, L1, L2, L1
    t.hi0 = __builtin_amdgcn_perm(0u, P, 0x0103010Cu) ^ 0x80800000u;
    t.lo1 = 0u;
    t.hi1 = 0u;
  }
  return t;
}

template <int B>
__device__ __forceinline__ void load_half_codes(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t* w) {
  if constexpr (B == 2) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    w[0] = v.x; w[1] = v.y;
  } else {
    typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
    const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0);
    w[0] = v.x; w[1] = v.y; w[2] = v.z;
  }
}

// Codes 8 kb .. 8 kb + 7 of a lane's 32-code half chunk -> one f16x8 fragment.
template <int B>
__device__ __forceinline__ f16x8 decode8(const uint32_t* w, const PermTable& t, int kb) {
  uint32_t o[4];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint32_t sel = perm_selector<B>(quad_field<B>(w, 2 * kb + u));
    const uint32_t lo = __builtin_amdgcn_perm(t.lo1, t.lo0, sel);
    const uint32_t hi = __builtin_amdgcn_perm(t.hi1, t.hi0, sel);
    o[2 * u] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    o[2 * u + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
  }
  return __builtin_bit_cast(f16x8, u32x4{o[0], o[1], o[2], o[3]});
}

template <int B>
__global__ __launch_bounds__(kPrefillThreads, 1) void k_prefill_a16(TiledParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* As = reinterpret_cast<uint16_t*>(smem);                 // [3][PT * PK] swizzled
  float* colmul = reinterpret_cast<float*>(smem + kABufs * kABufBytes);   // [PT] 2^e_n
  float* rowmul = colmul + PT;                                      // [PT] xback

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, h = lane >> 5;

  // Tile order: consecutive workgroup ids go to different XCDs; give each XCD a
  // contiguous run of tiles (same activation rows) when the count divides.
  const int tiles_n = static_cast<int>((p.N + PT - 1) / PT);
  const int tiles = static_cast<int>(gridDim.x);
  int t = static_cast<int>(blockIdx.x);
  if (tiles % 8 == 0) t = (t % 8) * (tiles / 8) + t / 8;
  const int64_t m0 = static_cast<int64_t>(t / tiles_n) * PT;
  const int64_t n0 = static_cast<int64_t>(t % tiles_n) * PT;

  const int gpr = static_cast<int>(p.K / p.group);
  const int nsteps = static_cast<int>(p.K / PK);
  const int spg = p.group / PK;

  // ---- weight rows of this lane: n0 + 64 wave + 32 i + c (i = 0, 1) ----
  const uint32_t row_bytes = static_cast<uint32_t>(p.K * B / 8);
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(p.codes, static_cast<uint32_t>(p.N) * row_bytes);
  const float* srow[2];
  const uint32_t* abrow[2];
  uint32_t coff[2];
  float inv_rowscale[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int nl = 64 * wave + 32 * i + c;
    const int64_t n = n0 + nl;
    const int64_t nc = n < p.N ? n : p.N - 1;          // parameters of a valid row
    srow[i] = p.scales + nc * gpr;
    abrow[i] = reinterpret_cast<const uint32_t*>(p.shapes) + nc * gpr;
    coff[i] = static_cast<uint32_t>(n) * row_bytes + static_cast<uint32_t>(h * 4 * B);
    float smax = 0.0f;
    for (int g = 0; g < gpr; ++g) smax = fmaxf(smax, fabsf(srow[i][g]));
    int e = 0;                                          // 2^e >= smax
    if (smax > 0.0f && smax <= 3.4e38f) e = ilogbf(smax) + 1;
    inv_rowscale[i] = ldexpf(1.0f, -e);
    if (h == 0) colmul[nl] = ldexpf(1.0f, e);
  }
  {
    const int64_t m = m0 + tid;
    rowmul[tid] = m < p.M ? p.xs[m] : 0.0f;
  }

  // ---- activation tile: global -> LDS, 16-byte slots, XOR swizzle ----
  // Slot (row r, chunk q) of a buffer holds the 8 fp16 x[m0 + r][k0 + 8 (q ^ (r & 7))].
  // Wave w fills slots 512 w + 64 i + lane (i = 0..7): row 64 w + 8 i + lane / 8.
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(p.xa, static_cast<uint32_t>(p.M * p.K * 2));
  uint32_t aoff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 64 * wave + 8 * i + (lane >> 3);
    const int q = (lane & 7) ^ (r & 7);
    aoff[i] = static_cast<uint32_t>(((m0 + r) * p.K + 8 * q) * 2);
  }
  auto issue_a = [&](int s, int buf, int i0, int i1) {
    uint16_t* dst = As + buf * (kABufBytes / 2) + wave * 4096;
#pragma unroll
    for (int i = i0; i < i1; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, dst + i * 512, 16, aoff[i] + s * (PK * 2), 0,
                                               0, 0);
  };

  // ---- codes and group parameters, two steps ahead ----
  uint32_t cw[3][2][B];     // [step % 3][row i][dword]
  float gs[3][2];
  uint32_t gab[3][2];
  // Code words every step; group parameters only for a step that starts a
  // group (the level table changes only there).
  auto load_codes = [&](int s, int par) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      load_half_codes<B>(crs, coff[i] + static_cast<uint32_t>(s) * (PK * B / 8), cw[par][i]);
    if (s % spg == 0) {
      const int g = (s < nsteps ? s : nsteps - 1) / spg;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        gs[par][i] = srow[i][g];
        gab[par][i] = abrow[i][g];
      }
    }
  };

  f32x16 acc[2][8];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Three activation stages in LDS; step s multiplies stage s % 3. Loads are
  // spread over the step so that the four waves never flood the address FIFO
  // of the texture unit (a wave stalls in order behind a VMEM it cannot
  // issue): the 8 activation loads of a stage go out two per MFMA block.
  // Stage (s + 2) % 3 is filled during blocks 0..2 of step s and block 3 of
  // step s - 1 (it was last read before the barrier of step s - 1), after the
  // code words and group parameters of step s + 2 (block 3 of step s - 1).
  // The one barrier of a step sits after MFMA block 2; it waits until only
  // the 8 activation loads of stage s + 2 may still be in flight, so stage
  // s + 1 is complete, and every wave has finished reading stage s. After it,
  // under the MFMAs of block 3, the wave reads the block-0 fragments of step
  // s + 1 and decodes that step's first weight fragments with its level table.
  // Weight fragments are always decoded one MFMA block ahead, so the decode
  // VALU work runs in the shadow of the MFMAs.
  load_codes(0, 0);
  load_codes(1, 1);
  load_codes(2, 2);
  issue_a(0, 0, 0, 8);
  issue_a(1, 1, 0, 8);
  issue_a(2, 2, 0, 2);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // fragment of activation block j for MFMA block kb: row 32 j + c, chunk 4 h + kb
  auto read_fa = [&](const uint16_t* Ab, int kb, f16x8* fa) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 32 * j + c;
      const int q = (4 * h + kb) ^ (r & 7);
      fa[j] = *reinterpret_cast<const f16x8*>(Ab + (r * 8 + q) * 8);
    }
  };

  PermTable tab[2];
  f16x8 fb[2];
  f16x8 fa[2][8];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    tab[i] = make_perm_table<B>(gs[0][i], gab[0][i], inv_rowscale[i]);
    fb[i] = decode8<B>(cw[0][i], tab[i], 0);
  }
  read_fa(As, 0, fa[0]);

  auto step = [&](int s, auto ph_c) {
    constexpr int ph = decltype(ph_c)::value;          // s % 3
    constexpr int ph1 = (ph + 1) % 3, ph2 = (ph + 2) % 3;
    const uint16_t* Ab = As + ph * (kABufBytes / 2);
    const uint16_t* An = As + ph1 * (kABufBytes / 2);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int cb = kb & 1;
      f16x8 fn[2];
      if (kb < 3) {
        issue_a(s + 2, ph2, 2 * kb + 2, 2 * kb + 4);
        read_fa(Ab, kb + 1, fa[cb ^ 1]);
#pragma unroll
        for (int i = 0; i < 2; ++i) fn[i] = decode8<B>(cw[ph][i], tab[i], kb + 1);
      } else {
        load_codes(s + 3, ph);
        __builtin_amdgcn_sched_barrier(0);
        issue_a(s + 3, ph, 0, 2);
        read_fa(An, 0, fa[0]);
        // The candidate table is built every step (it stays interleaved with
        // the MFMAs) and taken only when step s + 1 starts a group; otherwise
        // its parameters are stale and it is discarded.
        const bool newg = (s + 1) % spg == 0;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const PermTable nt = make_perm_table<B>(gs[ph1][i], gab[ph1][i], inv_rowscale[i]);
          tab[i].lo0 = newg ? nt.lo0 : tab[i].lo0;
          tab[i].lo1 = newg ? nt.lo1 : tab[i].lo1;
          tab[i].hi0 = newg ? nt.hi0 : tab[i].hi0;
          tab[i].hi1 = newg ? nt.hi1 : tab[i].hi1;
          fn[i] = decode8<B>(cw[ph1][i], tab[i], 0);
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[i], fa[cb][j], acc[i][j], 0, 0, 0);
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (kb < 3) {
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        } else {
          __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
        }
        if (u < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (u == 4 || u == 12) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (kb == 2) {
        // vmcnt(8), lgkmcnt(0): only the 8 activation loads of stage s + 2
        // may still be in flight, so this wave's part of stage s + 1 is in
        // LDS and its reads of stage s are done. A bare s_barrier (a release
        // fence would also drain the loads still in flight) publishes that to
        // the other waves.
        __builtin_amdgcn_s_waitcnt(0x0078);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
      fb[0] = fn[0];
      fb[1] = fn[1];
    }
  };
  int s = 0;
  for (; s + 2 < nsteps; s += 3) {
    step(s, std::integral_constant<int, 0>{});
    step(s + 1, std::integral_constant<int, 1>{});
    step(s + 2, std::integral_constant<int, 2>{});
  }
  if (s < nsteps) step(s, std::integral_constant<int, 0>{});
  if (s + 1 < nsteps) step(s + 1, std::integral_constant<int, 1>{});
  // Drain the loads that ran past K before the workgroup ends (they target
  // LDS stages nobody reads).
  __builtin_amdgcn_s_waitcnt(0);

  // ---- epilogue: D row = weight row n (8 (r / 4) + 4 h + r % 4), column = m ----
  const bool vec = (p.N & 3) == 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int ml = 32 * j + c;
    const int64_t m = m0 + ml;
    if (m >= p.M) continue;
    const float xm = rowmul[ml];
    float* yrow = p.y + m * p.N;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = 64 * wave + 32 * i + 8 * q + 4 * h;
        const int64_t n = n0 + nl;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * q + r] * xm * colmul[nl + r];
        if (vec && n + 3 < p.N) {
          *reinterpret_cast<f32x4*>(yrow + n) = f32x4{v[0], v[1], v[2], v[3]};
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < p.N) yrow[n + r] = v[r];
        }
      }
    }
  }
}

}  // namespace

// 2- and 3-bit codes, fp16 activations of k_xprep; the byte sizes of the
// activation and code buffers must stay below 2^32 (buffer addressing).
bool prefill_supported(int64_t M, int64_t N, int64_t K, int bits, int group) {
  if (bits != 2 && bits != 3) return false;
  if (group % PK != 0 || K % PK != 0) return false;
  if (M * K * 2 >= (int64_t{1} << 32)) return false;
  if (N * K * bits / 8 >= (int64_t{1} << 32)) return false;
  const int64_t tiles = ((M + PT - 1) / PT) * ((N + PT - 1) / PT);
  return tiles <= INT32_MAX;
}

template <int B>
static hipError_t launch_prefill_b(const TiledParams& p, hipStream_t st) {
  auto kern = k_prefill_a16<B>;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(kPrefillLds));
  if (e != hipSuccess) return e;
  const int64_t tiles = ((p.M + PT - 1) / PT) * ((p.N + PT - 1) / PT);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(tiles)), dim3(kPrefillThreads), kPrefillLds,
                     st, p);
  return hipGetLastError();
}

hipError_t launch_prefill_a16(const TiledParams& p, int bits, hipStream_t st) {
  return bits == 2 ? launch_prefill_b<2>(p, st) : launch_prefill_b<3>(p, st);
}

}  // namespace cubic
