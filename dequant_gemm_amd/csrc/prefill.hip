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
//    straight into LDS (buffer_load ... lds), in three stages, in an XOR-swizzled
//    layout that keeps the MFMA fragment reads free of bank conflicts (any 16
//    consecutive rows read at one chunk hit 16 distinct 16-byte bank groups);
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
// the negative one flips the sign bit of the hi byte. Built in four stages so
// that the work can be spread between MFMAs.
// Empty asm that takes and returns a register: pure arithmetic cannot be moved
// past it, so work written between two MFMAs is also emitted there.
__device__ __forceinline__ void pin(uint32_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }

struct TableBuild {
  float a, b, sc, sk;
  uint32_t L1, L2, P, Q;
};

template <int B>
__device__ __forceinline__ void table_stage(TableBuild& tb, PermTable& t, int stage, float s,
                                            uint32_t ab, float inv_rowscale) {
  static_assert(B == 2 || B == 3, "perm tables hold at most 8 levels");
  constexpr int K = kmax_of(B);
  if (stage == 0) {
    tb.a = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(ab & 0xffffu)));
    tb.b = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(ab >> 16)));
    tb.sc = s * inv_rowscale;                              // exact (power of two)
    tb.sk = tb.sc * (1.0f / static_cast<float>(K * K * K));
    pin(tb.a);
    pin(tb.b);
    pin(tb.sc);
    pin(tb.sk);
  } else if (stage == 1) {
    if constexpr (B == 3) {
      tb.L1 = table_level<3>(tb.a, tb.b, tb.sk, 1);
      tb.L2 = table_level<3>(tb.a, tb.b, tb.sk, 2);
    } else {
      tb.L1 = f16_bits(tb.sc);
      tb.L2 = table_level<2>(tb.a, tb.b, tb.sk, 2);
    }
    pin(tb.L1);
    pin(tb.L2);
  } else if (stage == 2) {
    tb.P = tb.L1 | (tb.L2 << 16);
    pin(tb.P);
    if constexpr (B == 3) {
      tb.Q = f16_bits(tb.sc) | (table_level<3>(tb.a, tb.b, tb.sk, 4) << 16);
      pin(tb.Q);
    }
  } else {
    if constexpr (B == 3) {
      // field values 0..7 -> codes 0, 1, 2, 3, -4, -3, -2, -1
      t.lo0 = __builtin_amdgcn_perm(tb.Q, tb.P, 0x0402000Cu);   // 0, L1, L2, L3
      t.lo1 = __builtin_amdgcn_perm(tb.Q, tb.P, 0x00020406u);   // L4, L3, L2, L1
      t.hi0 = __builtin_amdgcn_perm(tb.Q, tb.P, 0x0503010Cu);
      t.hi1 = __builtin_amdgcn_perm(tb.Q, tb.P, 0x01030507u) ^ 0x80808080u;
    } else {
      // field values 0..3 -> codes 0, 1, -2, -1
      t.lo0 = __builtin_amdgcn_perm(0u, tb.P, 0x0002000Cu);     // 0, L1, L2, L1
      t.hi0 = __builtin_amdgcn_perm(0u, tb.P, 0x0103010Cu) ^ 0x80800000u;
      t.lo1 = 0u;
      t.hi1 = 0u;
    }
    pin(t.lo0);
    pin(t.lo1);
    pin(t.hi0);
    pin(t.hi1);
  }
}

template <int B>
__device__ __forceinline__ PermTable make_perm_table(float s, uint32_t ab, float inv_rowscale) {
  TableBuild tb;
  PermTable t;
#pragma unroll
  for (int st = 0; st < 4; ++st) table_stage<B>(tb, t, st, s, ab, inv_rowscale);
  return t;
}

// One code quad (4 codes -> 2 dwords of fp16 pairs) in four pieces.
struct QuadState {
  uint32_t e, o, sel, lo, hi;
};

template <int B>
__device__ __forceinline__ void quad_piece(QuadState& st, int piece, const uint32_t* w, int qf,
                                           const PermTable& t, uint32_t* out) {
  constexpr uint32_t fm = (1u << B) - 1u;
  constexpr uint32_t me = fm | (fm << (2 * B));
  constexpr uint32_t mo = (fm << B) | (fm << (3 * B));
  if (piece == 0) {
    const uint32_t v = quad_field<B>(w, qf);
    st.e = v & me;
    st.o = v & mo;
    pin(st.e);
    pin(st.o);
  } else if (piece == 1) {
    const uint32_t e = st.e * (1u + (1u << (16 - 2 * B)));
    const uint32_t o = st.o * ((1u << (8 - B)) + (1u << (24 - 3 * B)));
    st.sel = ((e & 0x00FF00FFu) | (o & 0xFF00FF00u)) & (fm * 0x01010101u);
    pin(st.sel);
  } else if (piece == 2) {
    st.lo = __builtin_amdgcn_perm(t.lo1, t.lo0, st.sel);
    st.hi = __builtin_amdgcn_perm(t.hi1, t.hi0, st.sel);
    pin(st.lo);
    pin(st.hi);
  } else {
    out[0] = __builtin_amdgcn_perm(st.hi, st.lo, 0x05010400u);
    out[1] = __builtin_amdgcn_perm(st.hi, st.lo, 0x07030602u);
    pin(out[0]);
    pin(out[1]);
  }
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

// One output tile: 64 NB weight rows n0.. x 256 activation rows m0.. (NB = 2:
// the full 256 x 256 tile; NB = 1: half a tile, used to even out the last round
// of workgroups).
template <int B, int NB>
__device__ __forceinline__ void prefill_tile(const TiledParams& p, int64_t m0, int64_t n0,
                                             unsigned char* smem) {
  static_assert(NB == 2 || NB == 1, "2 or 1 weight blocks per wave");
  constexpr int MB = 8;                       // activation blocks per wave (256 rows)
  constexpr int Q = MB / 4;                   // activation loads per wave and MFMA block
  constexpr int NS = NB * MB;                 // MFMA slots per K block
  uint16_t* As = reinterpret_cast<uint16_t*>(smem);                 // [3][PT * PK] swizzled
  float* colmul = reinterpret_cast<float*>(smem + kABufs * kABufBytes);   // [PT] 2^e_n
  float* rowmul = colmul + PT;                                      // [PT] xback

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, h = lane >> 5;

  const int gpr = static_cast<int>(p.K / p.group);
  const int nsteps = static_cast<int>(p.K / PK);
  const int spg = p.group / PK;

  // ---- weight rows of this lane: n0 + 64 wave + 32 i + c (i = 0, 1) ----
  const uint32_t row_bytes = static_cast<uint32_t>(p.K * B / 8);
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(p.codes, static_cast<uint32_t>(p.N) * row_bytes);
  const float* srow[NB];
  const uint32_t* abrow[NB];
  uint32_t coff[NB];
  float inv_rowscale[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int nl = 32 * NB * wave + 32 * i + c;
    const int64_t n = n0 + nl;
    const int64_t nc = n < p.N ? n : p.N - 1;          // parameters of a valid row
    srow[i] = p.scales + nc * gpr;
    abrow[i] = reinterpret_cast<const uint32_t*>(p.shapes) + nc * gpr;
    coff[i] = static_cast<uint32_t>(n) * row_bytes + static_cast<uint32_t>(h * 4 * B);
  }
  // ---- activation tile: global -> LDS, 16-byte slots, XOR swizzle ----
  // Slot (row r, chunk q) of a buffer holds the 8 fp16 x[m0 + r][k0 + 8 (q ^ sw(r))],
  // sw(r) = (r & 7) ^ ((r >> 3) & 1): rows are 128 bytes, so rows r and r + 8 of
  // a 16-lane group would share banks under r & 7 alone.
  // Wave w fills slots 64 MB w + 64 i + lane (i < MB): row 8 MB w + 8 i + lane / 8.
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(p.xa, static_cast<uint32_t>(p.M * p.K * 2));
  uint32_t aoff[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int r = 8 * MB * wave + 8 * i + (lane >> 3);
    const int q = (lane & 7) ^ (r & 7) ^ ((r >> 3) & 1);
    aoff[i] = static_cast<uint32_t>(((m0 + r) * p.K + 8 * q) * 2);
  }
  auto issue_a = [&](int s, int buf, int i0, int i1) {
    uint16_t* dst = As + buf * (kABufBytes / 2) + wave * (512 * MB);
#pragma unroll
    for (int i = i0; i < i1; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, dst + i * 512, 16, aoff[i] + s * (PK * 2), 0,
                                               0, 0);
  };

  // ---- codes and group parameters, two steps ahead ----
  uint32_t cw[3][NB][B];    // [step % 3][row i][dword]
  float gs[3][NB];
  uint32_t gab[3][NB];
  // Code words every step; group parameters only for a step that starts a
  // group (the level table changes only there).
  auto load_codes = [&](int s, int par, bool group_start, int g) {
#pragma unroll
    for (int i = 0; i < NB; ++i)
      load_half_codes<B>(crs, coff[i] + static_cast<uint32_t>(s) * (PK * B / 8), cw[par][i]);
    if (group_start) {
      const int gc = g < gpr ? g : gpr - 1;
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        gs[par][i] = srow[i][gc];
        gab[par][i] = abrow[i][gc];
      }
    }
  };
#pragma unroll
  for (int t = 0; t < 3; ++t)
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      gs[t][i] = 0.0f;
      gab[t][i] = 0u;
    }

  f32x16 acc[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Three activation stages in LDS; step s multiplies stage s % 3. Loads are
  // spread over the step so that the four waves never flood the address FIFO
  // of the texture unit (a wave stalls in order behind a VMEM it cannot
  // issue): the MB activation loads of a stage go out MB / 4 per MFMA block.
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
  load_codes(0, 0, true, 0);
  load_codes(1, 1, 1 % spg == 0, 1 / spg);
  load_codes(2, 2, 2 % spg == 0, 2 / spg);
  issue_a(0, 0, 0, MB);
  issue_a(1, 1, 0, MB);
  issue_a(2, 2, 0, Q);
  // The row scale scan below is issued after the pipeline fill above, so the two
  // memory round trips of a tile's start overlap (the scan's values are used only
  // by the level tables, after the wait below).
  // Largest |s| of each row: the row's two lanes (h = 0, 1) take alternate
  // groups, and all loads of a batch of 32 groups are issued before any is
  // used (a dependent chain of loads here would cost one memory latency per
  // group). Loads past the row go to an offset outside the buffer and read 0.
  {
    const __amdgpu_buffer_rsrc_t srs =
        make_rsrc(p.scales, static_cast<uint32_t>(p.N * gpr * 4));
    float smax[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) smax[i] = 0.0f;
    for (int g0 = 0; g0 < gpr; g0 += 32) {
      float v[NB][16];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int64_t n = n0 + 32 * NB * wave + 32 * i + c;
        const int64_t nc = n < p.N ? n : p.N - 1;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int g = g0 + 2 * t + h;
          const uint32_t off = g < gpr ? static_cast<uint32_t>((nc * gpr + g) * 4) : 0xFFFFFFF0u;
          v[i][t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, off, 0, 0));
        }
      }
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int t = 0; t < 16; ++t) smax[i] = fmaxf(smax[i], fabsf(v[i][t]));
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const float m = fmaxf(smax[i], __shfl_xor(smax[i], 32, 64));
      int e = 0;                                        // 2^e >= m
      if (m > 0.0f && m <= 3.4e38f) e = ilogbf(m) + 1;
      inv_rowscale[i] = ldexpf(1.0f, -e);
      if (h == 0) colmul[32 * NB * wave + 32 * i + c] = ldexpf(1.0f, e);
    }
  }
  {
    const int64_t m = m0 + tid;
    rowmul[tid] = m < p.M ? (p.xs ? p.xs[m] : 1.0f) : 0.0f;
  }

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // one fragment: activation block j for MFMA block kb, row 32 j + c, chunk 4 h + kb
  auto read_frag = [&](const uint16_t* Ab, int kb, int j) {
    const int r = 32 * j + c;
    const int q = (4 * h + kb) ^ (r & 7) ^ ((r >> 3) & 1);
    return *reinterpret_cast<const f16x8*>(Ab + (r * 8 + q) * 8);
  };

  PermTable tab[NB];
  f16x8 fb[NB];
  f16x8 fa[2][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    tab[i] = make_perm_table<B>(gs[0][i], gab[0][i], inv_rowscale[i]);
    fb[i] = decode8<B>(cw[0][i], tab[i], 0);
  }
#pragma unroll
  for (int j = 0; j < MB; ++j) fa[0][j] = read_frag(As, 0, j);

  // Step s multiplies activation stage s % 3; every MFMA block kb is a fixed
  // schedule of NB * MB slots, each one MFMA followed by its share of the other
  // work (sched_barrier keeps the compiler from regrouping it):
  //  - one fragment read for the next MFMA block (slots 0 .. MB - 1);
  //  - one of the 8 NB pieces that decode the weight fragments of the next
  //    block (2 NB code quads of 4 pieces);
  //  - in block 0 the 4 NB stages of the candidate level table of step s + 1;
  //    it is taken in block 3 when step s + 1 starts a group;
  //  - the activation loads for the stage two steps ahead (two slots).
  // Block 3 also issues the code words (and group parameters) of step s + 3
  // first, then reads and decodes for step s + 1 from the next stage.
  int m1 = 1 % spg, m3 = 3 % spg, g3 = 3 / spg;   // (s + 1) % spg, (s + 3) % spg, (s + 3) / spg
  auto step = [&](int s, auto ph_c) {
    constexpr int ph = decltype(ph_c)::value;          // s % 3
    constexpr int ph1 = (ph + 1) % 3, ph2 = (ph + 2) % 3;
    const uint16_t* Ab = As + ph * (kABufBytes / 2);
    const uint16_t* An = As + ph1 * (kABufBytes / 2);
    const bool newg1 = m1 == 0;
    TableBuild tbs[NB];
    PermTable tn[NB];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int cb = kb & 1;
      const int kbn = kb < 3 ? kb + 1 : 0;
      const uint16_t* Ard = kb < 3 ? Ab : An;
      const int wp = kb < 3 ? ph : ph1;
      if (kb == 3) {
        load_codes(s + 3, ph, m3 == 0, g3);
        __builtin_amdgcn_sched_barrier(0);
      }
      QuadState qs[2 * NB];
      uint32_t out[NB][4];
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        const int i = u / MB, j = u % MB;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[i], fa[cb][j], acc[i][j], 0, 0, 0);
        if (u < MB) fa[cb ^ 1][u] = read_frag(Ard, kbn, u);
        if (kb == 3 && u == 0) {
#pragma unroll
          for (int r = 0; r < NB; ++r) {
            tab[r].lo0 = newg1 ? tn[r].lo0 : tab[r].lo0;
            tab[r].lo1 = newg1 ? tn[r].lo1 : tab[r].lo1;
            tab[r].hi0 = newg1 ? tn[r].hi0 : tab[r].hi0;
            tab[r].hi1 = newg1 ? tn[r].hi1 : tab[r].hi1;
            pin(tab[r].lo0);
            pin(tab[r].lo1);
            pin(tab[r].hi0);
            pin(tab[r].hi1);
          }
        }
        {
          const int q = u >> 2, iq = q >> 1, t = q & 1;
          quad_piece<B>(qs[q], u & 3, cw[wp][iq], 2 * kbn + t, tab[iq], &out[iq][2 * t]);
        }
        if (kb == 0 && (u & 1)) {
          // candidate table stages: 4 NB pieces (NB rows x 4 stages)
          const int tp = u >> 1;
          table_stage<B>(tbs[tp >> 2], tn[tp >> 2], tp & 3, gs[ph1][tp >> 2], gab[ph1][tp >> 2],
                         inv_rowscale[tp >> 2]);
        }
        if (u % (NS / 2) == NS / 4) {
          const int k = u / (NS / 2);
          if (k < Q) {
            if (kb < 3) {
              issue_a(s + 2, ph2, Q * (kb + 1) + k, Q * (kb + 1) + k + 1);
            } else {
              issue_a(s + 3, ph, k, k + 1);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (kb == 2) {
        // vmcnt(MB), lgkmcnt(0): only the MB activation loads of stage s + 2
        // may still be in flight, so this wave's part of stage s + 1 is in
        // LDS and its reads of stage s are done. A bare s_barrier (a release
        // fence would also drain the loads still in flight) publishes that to
        // the other waves.
        __builtin_amdgcn_s_waitcnt(0x0070 | MB);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
#pragma unroll
      for (int r = 0; r < NB; ++r)
        fb[r] = __builtin_bit_cast(f16x8, u32x4{out[r][0], out[r][1], out[r][2], out[r][3]});
    }
    m1 = m1 + 1 == spg ? 0 : m1 + 1;
    m3 = m3 + 1 == spg ? 0 : m3 + 1;
    g3 += m3 == 0 ? 1 : 0;
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
  for (int j = 0; j < MB; ++j) {
    const int ml = 32 * j + c;
    const int64_t m = m0 + ml;
    if (m >= p.M) continue;
    const float xm = rowmul[ml];
    const int64_t yrow = m * p.N;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = 32 * NB * wave + 32 * i + 8 * q + 4 * h;
        const int64_t n = n0 + nl;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * q + r] * xm * colmul[nl + r];
        if (vec && n + 3 < p.N) {
          store_out4(p.y, p.ybf16 != 0, yrow + n, v);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < p.N) store_out(p.y, p.ybf16 != 0, yrow + n + r, v[r]);
        }
      }
    }
  }
}

// Workgroups below full_tiles each take one 256 x 256 tile (consecutive ids go
// to different XCDs, so each XCD gets a contiguous run of tiles that share
// activation rows, when the count divides); the ones above take half tiles
// (128 weight rows) of the remaining tiles, two per tile, so that the last
// round of workgroups keeps every compute unit busy.
template <int B>
__global__ __launch_bounds__(kPrefillThreads, 1) void k_prefill_a16(TiledParams p, int full_tiles) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tiles_n = static_cast<int>((p.N + PT - 1) / PT);
  const int b = static_cast<int>(blockIdx.x);
  if (b < full_tiles) {
    int t = b;
    if (full_tiles % 8 == 0) t = (b % 8) * (full_tiles / 8) + b / 8;
    prefill_tile<B, 2>(p, static_cast<int64_t>(t / tiles_n) * PT,
                       static_cast<int64_t>(t % tiles_n) * PT, smem);
  } else {
    const int j = b - full_tiles;
    const int t = full_tiles + j / 2;
    prefill_tile<B, 1>(p, static_cast<int64_t>(t / tiles_n) * PT,
                       static_cast<int64_t>(t % tiles_n) * PT + (PT / 2) * (j & 1), smem);
  }
}

}  // namespace

// 2- and 3-bit codes, fp16 activations of k_xprep; the byte sizes of the
// activation and code buffers (with a tile's overhang past N) must stay below
// 2^32 (buffer addressing).
bool prefill_supported(int64_t M, int64_t N, int64_t K, int bits, int group) {
  if (bits != 2 && bits != 3) return false;
  if (group % PK != 0 || K % PK != 0) return false;
  if (M * K * 2 >= (int64_t{1} << 32)) return false;
  if ((N + PT) * K * bits / 8 >= (int64_t{1} << 32)) return false;   // rows past N read 0
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
  // One workgroup per compute unit (LDS). When the tiles overflow the last
  // round by at most half the compute units, the overflow tiles are run as two
  // half tiles each.
  const int64_t cus = device_cu_count();
  int64_t full = tiles, grid = tiles;
  if (cus > 0 && tiles > cus) {
    const int64_t rem = tiles % cus;
    if (rem > 0 && 2 * rem <= cus) {
      full = tiles - rem;
      grid = full + 2 * rem;
    }
  }
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kPrefillThreads), kPrefillLds,
                     st, p, static_cast<int>(full));
  return hipGetLastError();
}

hipError_t launch_prefill_a16(const TiledParams& p, int bits, hipStream_t st) {
  return bits == 2 ? launch_prefill_b<2>(p, st) : launch_prefill_b<3>(p, st);
}

}  // namespace cubic
