// prefill_a8.hip -- Dynamic A8 product for prefill-sized M with 2- and 3-bit
// codes (int8 MFMA bound).
//
// The CubicQuant article (section "一份 checkpoint，同时服务 A16 与 Dynamic A8")
// runs the A8 path as: per-token INT8 activations, an INT8 carrier of each
// weight level, an integer dot product per group and an fp32 group scale.
// Here one 256-thread workgroup owns a 128 (weight rows n) x 256 (activation
// rows m) output tile and walks K in steps of 128:
//  - wave w owns weight rows 32 w .. 32 w + 31 against all 256 activation rows
//    (8 blocks of 32 x 32): int32 sums for the open group and fp32 sums that
//    take int32 sum * fp32(s / 127) once the group is complete. Each decoded
//    weight fragment feeds 8 MFMAs;
//  - each lane decodes its row's codes in registers: the int8 carriers of the
//    row's 2^B field values sit in two registers, and one v_perm turns four
//    codes (their fields spread into a byte selector) into four carriers;
//  - a group's int32 sums are scaled into the fp32 sums in the first sub-step
//    of the next group, block by block: block j is read out right before the
//    MFMA that restarts it from zero, and its fp32 update runs beside the
//    following MFMAs;
//  - every load of the step loop goes from global memory straight into a
//    4-stage LDS ring (buffer_load ... lds): the int8 activation tile
//    (XOR-swizzled so that the 16-byte fragment reads are free of bank
//    conflicts), the tile's code words and the group parameters of the next
//    group. The one barrier of step s sits after three quarters of its MFMAs:
//    it waits until stage s + 1 has landed, so the rest of step s reads and
//    decodes the first fragments of step s + 1. The stage it frees is refilled
//    for step s + 4, one load per MFMA slot: the activations in the last
//    sub-step of step s, the code words and parameters in the first sub-step
//    of step s + 1;
//  - within a step, lane half h takes codes 64 h .. 64 h + 63 of its row: codes
//    64 h + 16 ks .. + 15 feed MFMA sub-step ks (0..3), and the activation
//    fragments follow the same K order.
// Every MFMA slot of a sub-step is followed by a fixed share of the other work
// (sched_barrier keeps the compiler from regrouping it), so the VALU work runs
// in the shadow of the MFMAs.
#include "common.h"
#include "launch.h"

namespace cubic {
namespace {

constexpr int A8N = 128;             // weight rows per tile
constexpr int A8M = 256;             // activation rows per tile (NB = 8 blocks of 32)
constexpr int A8K = 128;             // K per step
constexpr int kA8Threads = 256;
constexpr int kA8Stages = 4;
constexpr uint32_t kA8RsrcWord3 = 0x00020000u;   // raw buffer, 32-bit data format

// Stage layout: activations [A8M][A8K] int8, then the code words of the tile's
// A8N rows (A8K B / 8 bytes each, row-major), then group parameters (per wave
// 512 bytes: 64 scales, 64 (a, b) words; lanes 32..63 repeat rows 0..31).
// NB: 32-row activation blocks per tile (8: 256 rows; 2: 64 rows for small M).
constexpr size_t a8_x_bytes(int NB) { return static_cast<size_t>(32 * NB) * A8K; }
constexpr size_t a8_code_bytes(int B) { return static_cast<size_t>(A8N) * A8K * B / 8; }
constexpr size_t kA8ParamBytes = 4 * 512;
constexpr size_t a8_stage_bytes(int B, int NB) { return a8_x_bytes(NB) + a8_code_bytes(B) + kA8ParamBytes; }
constexpr size_t a8_lds_bytes(int B, int NB) { return kA8Stages * a8_stage_bytes(B, NB); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t a8_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0),
                                           static_cast<int>(bytes), static_cast<int>(kA8RsrcWord3));
}

// s_waitcnt immediate: vmcnt(n) (n < 64: low 4 bits in [3:0], high 2 bits in
// [15:14]), expcnt not waited for, lgkmcnt(0).
constexpr int a8_wait_vm(int n) { return (n & 15) | (7 << 4) | (((n >> 4) & 3) << 14); }

// Empty asm that takes and returns a register: arithmetic written in one MFMA
// slot cannot be moved past it into another.
__device__ __forceinline__ void pin(uint32_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(int& x) { asm volatile("" : "+v"(x)); }
// Orders 16 values before a use of `a`: the MFMA that takes `a` can only issue
// once the 16 values exist (the read-out of a block's sums before the MFMA
// that restarts them).
__device__ __forceinline__ void hold16(float* f, i32x4& a) {
  asm volatile(""
               : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3]), "+v"(f[4]), "+v"(f[5]),
                 "+v"(f[6]), "+v"(f[7]), "+v"(f[8]), "+v"(f[9]), "+v"(f[10]), "+v"(f[11]),
                 "+v"(f[12]), "+v"(f[13]), "+v"(f[14]), "+v"(f[15]), "+v"(a));
}

// Carrier of level j (|code| = j): clamp(rne(127 q(j / K)), -127, 127), K = Kmax.
// With S = K^3 q(j / K) = a j K^2 + b j^2 K + (1 - a - b) j^3, exact rounding
// of 127 S / K^3 is decided in fp64:
//  - S is exact: a and b are fp16 (multiples of 2^-24 below 2^16), j <= 4 and
//    K <= 3, so every partial sum is a multiple of 2^-24 below 2^24;
//  - X = S * fl(127 / K^3) is within 2^-44 of the true quotient when |X| < 128;
//  - n0 = rint(X) is then the rounded quotient or one off it, and the residual
//    D = 127 S - K^3 n0 (a multiple of 2^-24 below 2^6) comes out of one fma
//    exactly, so comparing D with K^3 / 2 settles ties (to even) and the
//    off-by-one case.
template <int B>
__device__ __forceinline__ int a8_carrier(double a, double b, double c, int j) {
  constexpr int K = kmax_of(B);
  constexpr double K3 = static_cast<double>(K * K * K);
  const double S = fma(a, static_cast<double>(j * K * K),
                       fma(b, static_cast<double>(j * j * K), c * static_cast<double>(j * j * j)));
  const double X = S * (127.0 / K3);
  if (X >= 127.75) return 127;                 // rounds to 128 or more: clamped
  if (X <= -127.75) return -127;
  const double n0 = rint(X);
  const double D = fma(127.0, S, -K3 * n0);
  const bool odd = (static_cast<int>(n0) & 1) != 0;
  int n = static_cast<int>(n0);
  n += (D > 0.5 * K3 || (D == 0.5 * K3 && odd)) ? 1 : 0;
  n -= (D < -0.5 * K3 || (D == -0.5 * K3 && odd)) ? 1 : 0;
  return n > 127 ? 127 : (n < -127 ? -127 : n);
}

// int8 carriers of field values 0..2^B-1 (two's complement codes) of one row
// and group, as bytes of t0 (fields 0..3) and t1 (fields 4..7), built in four
// pieces so that the work can be spread between MFMAs.
struct CarrierBuild {
  int c1, c2, c4;
};

template <int B>
__device__ __forceinline__ void carrier_piece(CarrierBuild& cb, int piece, uint32_t ab, uint32_t sbits,
                                              uint32_t& t0, uint32_t& t1, float& sc) {
  static_assert(B == 2 || B == 3, "at most 8 carriers per table");
  auto byte = [](int v) { return static_cast<uint32_t>(v) & 0xffu; };
  const double a = f16_bits_to_f64(static_cast<uint16_t>(ab & 0xffffu));
  const double b = f16_bits_to_f64(static_cast<uint16_t>(ab >> 16));
  const double c = (1.0 - a) - b;               // exact: both are fp16 values
  if (piece == 0) {
    cb.c2 = a8_carrier<B>(a, b, c, 2);
    pin(cb.c2);
  } else if (piece == 1) {
    if constexpr (B == 3) {
      cb.c1 = a8_carrier<B>(a, b, c, 1);
      pin(cb.c1);
    }
  } else if (piece == 2) {
    if constexpr (B == 3) {
      cb.c4 = a8_carrier<B>(a, b, c, 4);
      pin(cb.c4);
    }
  } else {
    sc = __fdiv_rn(__uint_as_float(sbits), 127.0f);
    if constexpr (B == 3) {
      // fields 0..7 -> codes 0, 1, 2, 3, -4, -3, -2, -1 (code 3 = Kmax: q = 1 -> 127)
      t0 = byte(0) | (byte(cb.c1) << 8) | (byte(cb.c2) << 16) | (byte(127) << 24);
      t1 = byte(-cb.c4) | (byte(-127) << 8) | (byte(-cb.c2) << 16) | (byte(-cb.c1) << 24);
    } else {
      // fields 0..3 -> codes 0, 1, -2, -1 (code 1 = Kmax: 127)
      t0 = byte(0) | (byte(127) << 8) | (byte(-cb.c2) << 16) | (byte(-127) << 24);
      t1 = 0u;
    }
    pin(t0);
    pin(t1);
    pin(sc);
  }
}

// Fields 4q .. 4q + 3 of a lane's 64 codes w[2B] at bits 0 .. 4B - 1 (higher
// bits are garbage; the selector masks ignore them).
template <int B>
__device__ __forceinline__ uint32_t a8_quad(const uint32_t* w, int q) {
  const int bit = 4 * B * q;
  const int d = bit >> 5, off = bit & 31;
  if (off == 0) return w[d];
  if (off + 4 * B <= 32) return w[d] >> off;
  return __builtin_amdgcn_alignbit(w[d + 1], w[d], off);
}

// One code quad (four codes -> one dword of int8 carriers) in two pieces: the
// fields of codes 0 and 2 (mask me) and of codes 1 and 3 (mask mo) are moved
// into bytes 0..3 by two multiplies whose terms never overlap, then v_perm
// looks the four field values up in the carrier table.
struct A8Quad {
  uint32_t e, o;
};

template <int B>
__device__ __forceinline__ void a8_quad_piece(A8Quad& qs, int piece, const uint32_t* w, int q,
                                              uint32_t t0, uint32_t t1, uint32_t& out) {
  constexpr uint32_t fm = (1u << B) - 1u;
  constexpr uint32_t me = fm | (fm << (2 * B));
  constexpr uint32_t mo = (fm << B) | (fm << (3 * B));
  if (piece == 0) {
    const uint32_t v = a8_quad<B>(w, q);
    qs.e = v & me;
    qs.o = v & mo;
    pin(qs.e);
    pin(qs.o);
  } else {
    const uint32_t e = __umul24(qs.e, 1u + (1u << (16 - 2 * B)));     // fields < 2^12
    const uint32_t o = __umul24(qs.o, (1u << (8 - B)) + (1u << (24 - 3 * B)));
    const uint32_t sel = (e & (fm * 0x00010001u)) | (o & (fm * 0x01000100u));
    out = __builtin_amdgcn_perm(t1, t0, sel);
    pin(out);
  }
}

// Swizzled position of 16-byte chunk q (0..7) of activation row r (128 bytes)
// in a stage: any 16 consecutive rows read at one chunk hit 16 distinct
// 16-byte bank groups (row parity and the XOR of the low three row bits and
// row bit 3 into the chunk index determine the address modulo 256).
__device__ __forceinline__ int a8_slot(int r, int q) {
  return r * 8 + (q ^ (r & 7) ^ ((r >> 3) & 1));
}

// SPG: steps per group when it is 1 or 2 (then known for each of the four
// unrolled steps), or 0 for any group length (decided at run time). NB: 32-row
// activation blocks per tile (8, or 2 for small M). With gridDim.y = 2 the two
// workgroups of a tile take the first and the second half of the groups and
// add their results into y, which holds zeros before (fp32 only): the two
// additions onto zero give the same sum in either order.
template <int B, int SPG, int NB>
__global__ __launch_bounds__(kA8Threads, 1) void k_prefill_a8(TiledParams p) {
  extern __shared__ __align__(16) unsigned char smem[];       // kA8Stages stages
  constexpr int DPR = A8K * B / 32;             // code dwords per row and step
  constexpr int AM = 32 * NB;                   // activation rows per tile
  constexpr size_t kStage = a8_stage_bytes(B, NB);
  constexpr size_t kCodeOff = a8_x_bytes(NB);
  constexpr size_t kParamOff = a8_x_bytes(NB) + a8_code_bytes(B);
  static_assert(NB == 2 || NB == 4 || NB == 8, "even block counts keep the row-parity swizzle");

  const int tiles_n = static_cast<int>((p.N + A8N - 1) / A8N);
  const int ntiles = tiles_n * static_cast<int>((p.M + AM - 1) / AM);
  int t = static_cast<int>(blockIdx.x);
  // consecutive workgroup ids go to different XCDs: give each XCD a contiguous
  // run of tiles (which share activation rows) when the count divides
  if (ntiles % 8 == 0) t = (t % 8) * (ntiles / 8) + t / 8;
  const int64_t m0 = static_cast<int64_t>(t / tiles_n) * AM;
  const int64_t n0 = static_cast<int64_t>(t % tiles_n) * A8N;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, h = lane >> 5;
  const int gpr = static_cast<int>(p.K / p.group);
  const int spg = SPG != 0 ? SPG : p.group / A8K;
  // this workgroup's steps [sb, se): whole groups, split gridDim.y ways
  const int split = NB == 8 ? 1 : static_cast<int>(gridDim.y);   // 256-row tiles: never split
  const int z = NB == 8 ? 0 : static_cast<int>(blockIdx.y);
  const int sb = (z * gpr / split) * spg, se = ((z + 1) * gpr / split) * spg;
  const uint32_t row_bytes = static_cast<uint32_t>(p.K * B / 8);
  const int64_t nrow = n0 + 32 * wave + c;      // this lane's weight row

  // ---- the step's loads: global -> LDS stage ----
  // activations: wave w fills slots 64 NB w + 64 i + lane (i < NB), 16 bytes
  // each: row r = 8 NB w + 8 i + lane / 8, chunk (lane % 8) ^ (r % 8) ^ (i % 2)
  // (the inverse of a8_slot; NB is even), so the offset is one of two per-lane
  // bases (by the parity of i) plus 8 i K. Rows past M read 0.
  const __amdgpu_buffer_rsrc_t xrs = a8_rsrc(p.xa, static_cast<uint32_t>(p.M * p.K));
  uint32_t abase[2];
  {
    const int64_t r = m0 + 8 * NB * wave + (lane >> 3);
    const int q = (lane & 7) ^ ((lane >> 3) & 7);
    abase[0] = static_cast<uint32_t>(r * p.K + 16 * q);
    abase[1] = static_cast<uint32_t>(r * p.K + 16 * (q ^ 1));
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
  constexpr int NV = NB + NC + 2;               // loads per wave and step
  static_assert(NC + 2 <= 8, "one code or parameter load per slot of a sub-step");
  static_assert(3 * NV < 64, "vmcnt holds at most 63");
  // Load i (0 .. NV - 1) of step s into a stage. The parameter slots of step
  // s hold the group after the one step s belongs to (read in that group's
  // last step to prepare the next carriers). Past the workgroup's steps, its
  // first step is loaded again into a stage nobody reads, so that the load
  // count per step stays fixed.
  auto issue_load = [&](int s, int stage, int i) {
    unsigned char* st = smem + stage * kStage;
    const int sv = s < se ? s : sb;
    if (i < NB) {
      const uint32_t ko = static_cast<uint32_t>(8 * i) * static_cast<uint32_t>(p.K) +
                          static_cast<uint32_t>(sv) * A8K;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, st + wave * (NB * 1024) + i * 1024, 16,
                                               abase[i & 1] + ko, 0, 0, 0);
    } else if (i < NB + NC) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(crs, st + kCodeOff + 256 * (NC * wave + i - NB), 4,
                                               coff[i - NB] + static_cast<uint32_t>(sv) * (4 * DPR),
                                               0, 0, 0);
    } else {
      int g = sv / spg + 1;
      g = g < gpr ? g : gpr - 1;
      const bool ab = i == NB + NC + 1;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ab ? brs : srs, st + kParamOff + 512 * wave + (ab ? 256 : 0),
                                               4, poff + 4u * static_cast<uint32_t>(g), 0, 0, 0);
    }
  };
  auto issue_step = [&](int s, int stage) {
#pragma unroll
    for (int i = 0; i < NV; ++i) issue_load(s, stage, i);
  };

  i32x16 acc[NB];                               // int32 sums of the open group
  f32x16 accf[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      acc[j][e] = 0;
      accf[j][e] = 0.0f;
    }

  // ---- prologue: group 0's carriers, stages 0..2, then stage 3 ----
  uint32_t t0 = 0u, t1 = 0u;                    // carriers of the group being decoded
  float sc = 0.0f;                              // s / 127 of the group in the int32 sums
  {
    const uint32_t go = poff + 4u * static_cast<uint32_t>(sb / spg);   // the first group
    const uint32_t sbits = __builtin_amdgcn_raw_buffer_load_b32(srs, go, 0, 0);
    const uint32_t ab = __builtin_amdgcn_raw_buffer_load_b32(brs, go, 0, 0);
    CarrierBuild cb;
#pragma unroll
    for (int piece = 0; piece < 4; ++piece) carrier_piece<B>(cb, piece, ab, sbits, t0, t1, sc);
  }
  issue_step(sb, 0);
  issue_step(sb + 1, 1);
  issue_step(sb + 2, 2);
  __builtin_amdgcn_s_waitcnt(a8_wait_vm(2 * NV));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  // step 3: its activation loads here (they belong to the last sub-step of
  // step -1), its code and parameter loads in the first sub-step of step 0
#pragma unroll
  for (int i = 0; i < NB; ++i) issue_load(sb + 3, 3, i);

  uint32_t cw[2 * B];                           // this lane's 64 codes of the current step
  auto read_codes = [&](const unsigned char* st, uint32_t* w) {
    const uint32_t* src =
        reinterpret_cast<const uint32_t*>(st + kCodeOff) + DPR * (32 * wave + c) + 2 * B * h;
#pragma unroll
    for (int d = 0; d < 2 * B; ++d) w[d] = src[d];
  };
  // Activation fragment j (rows 32 j .. 32 j + 31) of sub-step ks sits at byte
  // 4096 j + 128 c + 16 ((4 h) ^ sw ^ ks) of a stage, sw = (c % 8) ^ (c / 8 % 2)
  // (a8_slot with row 32 j + c and chunk 4 h + ks).
  const uint32_t xlane = static_cast<uint32_t>(128 * c + 16 * ((4 * h) ^ (c & 7) ^ ((c >> 3) & 1)));
  auto read_a = [&](const unsigned char* st, uint32_t xl, int ks, int j) {
    return *reinterpret_cast<const i32x4*>(st + (xl ^ (16u * ks)) + 4096 * j);
  };
  i32x4 fa[NB];
  i32x4 fb;
  read_codes(smem, cw);
#pragma unroll
  for (int j = 0; j < NB; ++j) fa[j] = read_a(smem, xlane, 0, j);
  {
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      A8Quad qs;
      a8_quad_piece<B>(qs, 0, cw, q, t0, t1, o[q]);
      a8_quad_piece<B>(qs, 1, cw, q, t0, t1, o[q]);
    }
    fb = i32x4{static_cast<int>(o[0]), static_cast<int>(o[1]), static_cast<int>(o[2]),
               static_cast<int>(o[3])};
  }

  float sc_prev = 0.0f;                         // s / 127 of the group before (zero sums at first)
  int mg = 0;                                   // s % spg
  // One sub-step: 8 MFMA slots, then the barrier after sub-step 2. FIRST: the
  // group's first sub-step (the sums restart from zero after their update).
  auto step = [&](int s, auto ph_c) {
    constexpr int ph = decltype(ph_c)::value;  // s % 4
    constexpr int ph1 = (ph + 1) % 4;
    const bool first = SPG == 1 ? true : (SPG == 2 ? ph % 2 == 0 : mg == 0);
    const bool last = SPG == 1 ? true : (SPG == 2 ? ph % 2 == 1 : mg == spg - 1);
    const unsigned char* st = smem + ph * kStage;
    const unsigned char* stn = smem + ph1 * kStage;
    uint32_t xl = xlane;                        // re-derived per step: not kept per stage
    pin(xl);

    uint32_t cwn[2 * B];
    uint32_t t0n = t0, t1n = t1;
    float scn = sc;
    uint32_t pab = 0u, psb = 0u;
    CarrierBuild cb;
    if (last) {
      const uint32_t* par = reinterpret_cast<const uint32_t*>(st + kParamOff + 512 * wave);
      psb = par[c];
      pab = par[64 + c];
    }
    auto sub_step = [&](int ks, auto first_c) {
      constexpr bool restart = decltype(first_c)::value;
      A8Quad qs[4];
      uint32_t o[4];
      if (ks == 3) {
        // past the barrier: stage s + 1 is complete; the next step's codes and
        // the carriers it decodes with
        read_codes(stn, cwn);
      }
      const uint32_t* wsrc = ks < 3 ? cw : cwn;
      const uint32_t d0 = ks < 3 ? t0 : (last ? t0n : t0);
      const uint32_t d1 = ks < 3 ? t1 : (last ? t1n : t1);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        // slot u: block u's MFMA (u < NB), then a share of the other work
        if constexpr (restart) {
          if (u < NB) {
            // the finished group's sums of block u: out before the MFMA restarts
            // them, into fp32 beside it (exact: |sum| < 2^24)
            float f[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) f[e] = static_cast<float>(acc[u][e]);
            hold16(f, fa[u]);
            acc[u] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[u], fb, i32x16{}, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              float v = fmaf(f[e], sc_prev, accf[u][e]);
              pin(v);
              accf[u][e] = v;
            }
          }
        } else {
          if (u < NB) acc[u] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[u], fb, acc[u], 0, 0, 0);
        }
        if (u < NB) fa[u] = ks < 3 ? read_a(st, xl, ks + 1, u) : read_a(stn, xl, 0, u);
        // decode of the next sub-step's fragment: quad piece u (sub-steps 0..2),
        // or from slot 1 on once the next step's codes are read (sub-step 3)
        if (ks < 3) {
          a8_quad_piece<B>(qs[u >> 1], u & 1, wsrc, 4 * (ks + 1) + (u >> 1), d0, d1, o[u >> 1]);
        } else if (u >= 1) {
          if (u == 1) a8_quad_piece<B>(qs[0], 0, wsrc, 0, d0, d1, o[0]);
          a8_quad_piece<B>(qs[u >> 1], u & 1, wsrc, u >> 1, d0, d1, o[u >> 1]);
        }
        if (last && ks == 1 && (u & 1)) carrier_piece<B>(cb, u >> 1, pab, psb, t0n, t1n, scn);
        // refill of the stage freed by the barrier of step s - 1 or s: the
        // activation loads of step s + 4 in the last sub-step, the code and
        // parameter loads of step s + 3 in the first (one load per slot)
        if (ks == 3 && u < NB) issue_load(s + 4, ph, u);
        if (ks == 0 && NB + u < NV) issue_load(s + 3, (ph + 3) % 4, NB + u);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (ks == 2) {
        // Stage s + 1 is complete once only the loads of stages s + 2 and s + 3
        // remain; lgkmcnt(0) ends this wave's reads of stage s. The bare barrier
        // publishes both, so stage s can be refilled for step s + 4.
        __builtin_amdgcn_s_waitcnt(a8_wait_vm(2 * NV));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
      fb = i32x4{static_cast<int>(o[0]), static_cast<int>(o[1]), static_cast<int>(o[2]),
                 static_cast<int>(o[3])};
    };
    if (first) {
      sub_step(0, std::true_type{});
    } else {
      sub_step(0, std::false_type{});
    }
    sub_step(1, std::false_type{});
    sub_step(2, std::false_type{});
    sub_step(3, std::false_type{});
#pragma unroll
    for (int d = 0; d < 2 * B; ++d) cw[d] = cwn[d];
    if (last) {
      t0 = t0n;
      t1 = t1n;
      sc_prev = sc;
      sc = scn;
    }
    mg = last ? 0 : mg + 1;
  };
  int s = sb;
  for (; s + 3 < se; s += 4) {
    step(s, std::integral_constant<int, 0>{});
    step(s + 1, std::integral_constant<int, 1>{});
    step(s + 2, std::integral_constant<int, 2>{});
    step(s + 3, std::integral_constant<int, 3>{});
  }
  if (s < se) step(s, std::integral_constant<int, 0>{});
  if (s + 1 < se) step(s + 1, std::integral_constant<int, 1>{});
  if (s + 2 < se) step(s + 2, std::integral_constant<int, 2>{});
  // the last group's sums (its scale moved to sc_prev at its last step)
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) accf[j][e] = fmaf(static_cast<float>(acc[j][e]), sc_prev, accf[j][e]);
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
  for (int j = 0; j < NB; ++j) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int ml = 32 * j + 8 * (e >> 2) + 4 * h + (e & 3);
      const int64_t m = m0 + ml;
      if (m < p.M && nrow < p.N) {
        const float v = accf[j][e] * sxs[ml];
        if (split > 1) {
          atomicAdd(p.y + m * p.N + nrow, v);
        } else {
          store_out(p.y, p.ybf16 != 0, m * p.N + nrow, v);
        }
      }
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

template <int B, int SPG, int NB>
static hipError_t launch_prefill_a8_k(const TiledParams& p, int split, hipStream_t st) {
  auto kern = k_prefill_a8<B, SPG, NB>;
  constexpr size_t lds = a8_lds_bytes(B, NB);
  static_assert(lds <= 160 * 1024, "one compute unit's LDS");
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(lds));
  if (e != hipSuccess) return e;
  const int64_t tiles = ((p.M + 32 * NB - 1) / (32 * NB)) * ((p.N + A8N - 1) / A8N);
  if (split > 1) {
    const hipError_t z = launch_fill_zero(p.y, p.M * p.N, false, st);   // the two halves add into y
    if (z != hipSuccess) return z;
  }
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(tiles), static_cast<unsigned>(split)), dim3(kA8Threads),
                     lds, st, p);
  return hipGetLastError();
}

// Tiles of 256 activation rows while they fill the compute units; below that,
// tiles of 64 rows, and the groups split between two workgroups per tile while
// the 64-row tiles fill at most three quarters of the compute units (fp32
// output only; measured on the expert shapes).
template <int B, int SPG>
static hipError_t launch_prefill_a8_s(const TiledParams& p, hipStream_t st) {
  const int64_t cus = device_cu_count();
  const int64_t tn = (p.N + A8N - 1) / A8N;
  if (((p.M + 255) / 256) * tn >= cus) return launch_prefill_a8_k<B, SPG, 8>(p, 1, st);
  const int64_t t2 = ((p.M + 63) / 64) * tn;
  const int split = (4 * t2 <= 3 * cus && p.ybf16 == 0 && p.K / p.group >= 2) ? 2 : 1;
  return launch_prefill_a8_k<B, SPG, 2>(p, split, st);
}

template <int B>
static hipError_t launch_prefill_a8_b(const TiledParams& p, hipStream_t st) {
  const int spg = p.group / A8K;
  if (spg == 1) return launch_prefill_a8_s<B, 1>(p, st);
  if (spg == 2) return launch_prefill_a8_s<B, 2>(p, st);
  return launch_prefill_a8_s<B, 0>(p, st);
}

hipError_t launch_prefill_a8(const TiledParams& p, int bits, hipStream_t st) {
  return bits == 2 ? launch_prefill_a8_b<2>(p, st) : launch_prefill_a8_b<3>(p, st);
}

}  // namespace cubic
