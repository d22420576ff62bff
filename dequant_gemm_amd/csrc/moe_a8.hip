// moe_a8.hip -- routed-expert products in the Dynamic A8 mode.
//
// The CubicQuant article (section on serving A16 and Dynamic A8 from one
// checkpoint) runs A8 as per-token INT8 activations, an INT8 carrier of each
// weight level, an exact integer dot product per group and one fp32 scale per
// group. Here that product runs on the routed experts: the pairs are grouped by
// expert with the A16 path's routing kernel, and one workgroup per (touched
// expert, 16-row tile) streams the tile's codes once per pass of up to MT pairs.
//
// Work split: the four waves take a quarter of K each, in steps of 128 codes.
// Lane (row nl of the tile, slot kb) takes chunk kb (32 codes, B dwords) of
// each step of its row, decodes it in registers into 32 int8 carriers and feeds
// two v_mfma_i32_16x16x64_i8 whose other operand holds the pass's activation
// rows (staged in LDS per wave). Int32 sums per group are exact (|sum| <= G *
// 127^2 < 2^24 for G <= 1024, so also exact in fp32); at the end of a group they
// are scaled by fp32(s / 127) into fp32, and the token's scale multiplies the
// sum of the four waves' partials.
//
// Carriers (sign(k) * clamp(rne(127 q(|k| / Kmax)), -127, 127), decided exactly
// by carrier_exact, or carrier_level for shapes beyond 16 in magnitude):
//  - 2-bit codes: the row's four carriers sit in one register. For 16 codes
//    in a dword w, (w >> 2j) & 0x03030303 holds the fields of codes j, 4 + j,
//    8 + j, 12 + j as byte selectors, and one v_perm per j turns them into
//    carriers: 7 bit operations and 4 permutes per 16 codes. The carriers come
//    out transposed within each 16 codes (byte b of dword j is code 4b + j);
//    the activations are staged in LDS in the same order.
//  - 3- and 4-bit codes: the row's 8 (16) carriers in two (four) registers;
//    four fields are moved into byte selectors by two multiplies whose terms
//    never overlap, then v_perm (4-bit: two of them and a bit select) looks
//    them up. Natural order.
//  - 5- to 8-bit codes: a table of the row's 2^B carriers in LDS, rebuilt at
//    each group (carrier_fast), one byte read per code. Natural order.
// The per-row carrier registers and the group scale are computed once per
// workgroup, each lane of a row taking every fourth group of the wave's range,
// and read from LDS at each group boundary.
#include <utility>

#include "common.h"
#include "launch.h"

namespace cubic {
namespace {

template <int B>
struct A8Cfg {
  static constexpr int kSlots = B == 2 ? 16 : (B == 3 ? 10 : (B == 4 ? 8 : 4));   // steps in flight
  static constexpr bool kRegTable = B <= 4;
  static constexpr bool kDirect = B >= 7;            // carriers computed per code, no table
  // LDS entry per (row, group): scale, then the carriers (up to 4 bits) or (a, b)
  static constexpr int kGpDwords = B == 2 ? 2 : (B == 3 ? 3 : (B == 4 ? 5 : 2));
};

constexpr int kA8GpRegs = 8;        // group-parameter registers per lane: <= 32 groups per wave

__device__ __forceinline__ uint32_t carrier_byte(int v) { return static_cast<uint32_t>(v) & 0xffu; }

// Carriers of the field values 0 .. 2^B - 1 (two's complement codes) of one
// row and group, four per dword, field f in byte f % 4 of T[f / 4]. C_Kmax is
// 127 exactly (q(1) = 1), C_0 is 0.
template <int B>
__device__ __forceinline__ void carrier_regs(uint32_t ab, uint32_t* T) {
  constexpr int km = kmax_of(B);
  constexpr int NF = 1 << B;
  const double a = f16_bits_to_f64(static_cast<uint16_t>(ab & 0xffffu));
  const double b = f16_bits_to_f64(static_cast<uint16_t>(ab >> 16));
  int C[NF / 2 + 1];
  C[0] = 0;
#pragma unroll
  for (int j = 1; j <= NF / 2; ++j) {
    C[j] = j == km ? 127 : (fabs(a) <= 16.0 && fabs(b) <= 16.0 ? carrier_exact(a, b, j, km)
                                                               : carrier_level(a, b, j, km));
  }
#pragma unroll
  for (int d = 0; d < NF / 4; ++d) {
    uint32_t v = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = 4 * d + i;
      const int k = f < NF / 2 ? f : f - NF;
      v |= carrier_byte(k < 0 ? -C[-k] : C[k]) << (8 * i);
    }
    T[d] = v;
  }
}

// 2-bit codes: chunk w[2] (codes 0..31) -> out[8]; out[4h + j] byte b is the
// carrier of code 16h + 4b + j.
__device__ __forceinline__ void decode_w2(const uint32_t* w, uint32_t t0, uint32_t* out) {
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      out[4 * h + j] = __builtin_amdgcn_perm(0u, t0, (w[h] >> (2 * j)) & 0x03030303u);
}

// Fields 4q .. 4q + 3 of a 32-code chunk w[B] (B <= 4) as the four byte
// selectors of v_perm. The even fields (codes 0, 2) and the odd ones (1, 3) are
// each moved into place by one 24-bit multiply; the partial products land in
// disjoint bit ranges (or sum below the next kept range), so nothing carries
// into a kept byte.
template <int B>
__device__ __forceinline__ uint32_t quad_selectors(const uint32_t* w, int q) {
  const int bit = 4 * B * q;
  const int d = bit >> 5, off = bit & 31;
  uint32_t v;
  if (off == 0) {
    v = w[d];
  } else if (off + 4 * B <= 32) {
    v = w[d] >> off;
  } else {
    v = __builtin_amdgcn_alignbit(w[d + 1], w[d], off);
  }
  constexpr uint32_t fm = (1u << B) - 1u;
  const uint32_t e = __umul24(v & (fm | (fm << (2 * B))), 1u + (1u << (16 - 2 * B)));
  const uint32_t o = __umul24(v & ((fm << B) | (fm << (3 * B))), (1u << (8 - B)) + (1u << (24 - 3 * B)));
  return (e & (fm * 0x00010001u)) | (o & (fm * 0x01000100u));
}

// 3- and 4-bit codes: chunk w[B] -> out[8], natural order (byte i of out[q] is
// code 4q + i).
template <int B>
__device__ __forceinline__ void decode_regs(const uint32_t* w, const uint32_t* T, uint32_t* out) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint32_t sel = quad_selectors<B>(w, q);
    if constexpr (B == 3) {
      out[q] = __builtin_amdgcn_perm(T[1], T[0], sel);
    } else {
      const uint32_t s7 = sel & 0x07070707u;
      const uint32_t lo = __builtin_amdgcn_perm(T[1], T[0], s7);
      const uint32_t hi = __builtin_amdgcn_perm(T[3], T[2], s7);
      const uint32_t m = ((sel >> 3) & 0x01010101u) * 0xffu;
      out[q] = (hi & m) | (lo & ~m);
    }
  }
}

// 5- to 8-bit codes: chunk w[B] -> out[8] through the row's LDS table.
template <int B>
__device__ __forceinline__ void decode_lds(const uint32_t* w, const int8_t* tab_row, uint32_t* out) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint32_t v = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v |= static_cast<uint32_t>(static_cast<uint8_t>(tab_row[chunk_field<B>(w, 4 * q + i)])) << (8 * i);
    out[q] = v;
  }
}

// 7- and 8-bit codes: chunk w[B] -> out[8], each carrier computed from the
// group's (a, b). With a table of 2^B entries per row and group against the 32
// codes a lane decodes per step, this is the cheaper side at these widths.
template <int B>
__device__ __forceinline__ void decode_direct(const uint32_t* w, float a, float b, uint32_t* out) {
  constexpr int km = kmax_of(B);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint32_t v = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = sign_extend(chunk_field<B>(w, 4 * q + i), B);
      const int c = carrier_fast(a, b, k < 0 ? -k : k, km);
      v |= carrier_byte(k < 0 ? -c : c) << (8 * i);
    }
    out[q] = v;
  }
}

// The LDS table of one row and group: the four lanes of the row take every
// fourth field value.
template <int B>
__device__ __forceinline__ void build_lds_table(int8_t* tab_row, int kb, uint32_t ab) {
  constexpr int km = kmax_of(B);
  const float a = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(ab & 0xffffu)));
  const float b = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(ab >> 16)));
  for (int f = kb; f < (1 << B); f += 4) {
    const int k = sign_extend(static_cast<uint32_t>(f), B);
    const int j = k < 0 ? -k : k;
    const int c = j == 0 ? 0 : (j == km ? 127 : carrier_fast(a, b, j, km));
    tab_row[f] = static_cast<int8_t>(k < 0 ? -c : c);
  }
}

template <int B>
__device__ __forceinline__ void load_chunk_dwords(const uint32_t* src, uint32_t* w) {
  if constexpr (B == 2) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(src);
    w[0] = v.x; w[1] = v.y;
  } else if constexpr (B == 4 || B == 8) {
#pragma unroll
    for (int q = 0; q < B / 4; ++q) {
      const u32x4 v = reinterpret_cast<const u32x4*>(src)[q];
      w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int d = 0; d < B; ++d) w[d] = src[d];
  }
}

// 16 activation bytes in the 2-bit decoder's order: out dword j byte b = in
// byte 4b + j (a 4 x 4 byte transpose).
__device__ __forceinline__ u32x4 transpose16(const u32x4& v) {
  const uint32_t p0 = __builtin_amdgcn_perm(v.y, v.x, 0x05010400u);   // x0 y0 x1 y1
  const uint32_t q0 = __builtin_amdgcn_perm(v.w, v.z, 0x05010400u);   // z0 w0 z1 w1
  const uint32_t p1 = __builtin_amdgcn_perm(v.y, v.x, 0x07030602u);   // x2 y2 x3 y3
  const uint32_t q1 = __builtin_amdgcn_perm(v.w, v.z, 0x07030602u);   // z2 w2 z3 w3
  return u32x4{__builtin_amdgcn_perm(q0, p0, 0x05040100u), __builtin_amdgcn_perm(q0, p0, 0x07060302u),
               __builtin_amdgcn_perm(q1, p1, 0x05040100u), __builtin_amdgcn_perm(q1, p1, 0x07060302u)};
}

__device__ __forceinline__ i32x4 mfma_i8(const u32x4& a, const u32x4& b, const i32x4& c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c,
                                               0, 0, 0);
}

// Geometry shared by the kernel and its launcher.
// A step is 128 sub codes of a row: each lane takes sub 32-code chunks of it
// (sub = 2 for 2-bit codes when K and the group are multiples of 256, so that a
// lane's code load is 16 bytes).
struct A8Geom {
  int nstep;   // steps per row
  int mpw;     // steps reserved per wave
  int spg;     // steps per group
  int gmax;    // groups a wave can span
};

__host__ __device__ inline A8Geom a8_geom(int64_t K, int group, int sub = 1) {
  A8Geom g;
  g.nstep = static_cast<int>(K / (128 * sub));
  g.mpw = (g.nstep + 3) / 4;
  g.spg = group / (128 * sub);
  g.gmax = (g.mpw + g.spg - 1) / g.spg + 1;
  return g;
}

// nrg: 16-row groups per workgroup (four waves each); the groups share the
// activation slices.
template <int B>
__host__ __device__ inline size_t a8_lds_bytes(const A8Geom& g, int mt, int nrg = 1, int sub = 1) {
  const size_t w = static_cast<size_t>(4) * nrg;
  const size_t tab = (A8Cfg<B>::kRegTable || A8Cfg<B>::kDirect) ? 0 : w * 16 * (1 << B);
  return w * 16 * 16 * 4 +                                                      // partials
         w * 16 * g.gmax * A8Cfg<B>::kGpDwords * 4 +                            // group entries
         tab + static_cast<size_t>(4) * mt * (g.mpw * 128 * sub + 16);          // activations
}

// One workgroup per (touched expert slot, 16-row tile); slots past the touched
// count exit at once. ALLIN: every step of a wave fits the load slots. DENSE:
// the plain A8 product of p.dense_m activation rows with one weight (expert 0,
// row m of x and of y for pair m; no routing): one workgroup per tile of 16
// NRG rows. With NRG = 2, waves 4..7 take the second 16 rows against the same
// activation slices as waves 0..3 (the two groups stage half of the rows each).
template <int B, int MT, bool ALLIN, bool DENSE = false, int NRG = 1, int SUB = 1>
__global__ __launch_bounds__(256 * NRG) void k_moe_a8(MoeA8Params p) {
  using Cfg = A8Cfg<B>;
  static_assert(SUB == 1 || B == 2, "16-byte code loads for 2-bit codes");
  constexpr int PS = Cfg::kSlots / SUB;
  constexpr int DW = B * SUB;                    // code dwords per lane and step
  constexpr int GPD = Cfg::kGpDwords;
  constexpr int TR = 16 * NRG;                   // weight rows per tile
  static_assert(NRG == 1 || (NRG == 2 && MT == 16), "two row groups share 16-row passes");
  extern __shared__ __align__(16) unsigned char smem[];
  const unsigned tiles = static_cast<unsigned>((p.N + TR - 1) / TR);
  const unsigned a = blockIdx.x / tiles;
  i32x8 rec;
  if constexpr (DENSE) {
    rec = i32x8{0, 0, p.dense_m, 0, p.dense_m > 1 ? 1 : 0, 0, 0, 0};
  } else {
    if (p.direct) {
      if (blockIdx.x == 0 && threadIdx.x < 64) {
        // the invalid-id count (npairs <= 64 in direct mode)
        const int l = threadIdx.x;
        const int e = l < p.npairs ? p.ids[l] : 0;
        const unsigned long long bad = __ballot(static_cast<unsigned>(e) >= static_cast<unsigned>(p.E));
        if (l == 0) *p.bad_count = __popcll(bad);
      }
      // pair a alone: expert 0's codes stand in for an invalid id, whose rows
      // are stored as zeros
      const int e = p.ids[a];
      const int ok = static_cast<unsigned>(e) < static_cast<unsigned>(p.E);
      rec = i32x8{ok ? e : 0, static_cast<int>(a), 1, static_cast<int>(a), static_cast<int>(a), 1 - ok, 0, 0};
    } else {
      rec = *reinterpret_cast<const i32x8*>(p.erec + 8 * a);
    }
  }
  if (rec[2] == 0) return;
  const bool bad_pair = !DENSE && p.direct && rec[5] != 0;
  const int64_t t0n = static_cast<int64_t>(blockIdx.x - a * tiles) * TR;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kq = wave & 3, rg = wave >> 2;       // K quarter, row group
  const int64_t n0 = t0n + 16 * rg;
  const int nl = lane & 15, kb = lane >> 4;
  const A8Geom geo = a8_geom(p.K, p.group, SUB);
  const int tb = kq * geo.nstep / 4, te = (kq + 1) * geo.nstep / 4;
  const int g0 = tb / geo.spg;
  const int gn = te > tb ? (te - 1) / geo.spg - g0 + 1 : 0;
  const int gpr = static_cast<int>(p.K / p.group);
  // activation rows of a wave's slice, 16 bytes apart in bank position: the
  // fragment reads of 16 different rows then hit different banks
  const int xrow_bytes = geo.mpw * 128 * SUB + 16;

  float* red = reinterpret_cast<float*>(smem);
  unsigned char* q = smem + 4 * NRG * 16 * 16 * 4;
  uint32_t* gp_row = reinterpret_cast<uint32_t*>(q) + static_cast<int64_t>(wave * 16 + nl) * geo.gmax * GPD;
  q += static_cast<size_t>(4) * NRG * 16 * geo.gmax * GPD * 4;
  int8_t* tab_row = reinterpret_cast<int8_t*>(q) + (wave * 16 + nl) * (1 << B);
  if constexpr (!Cfg::kRegTable && !Cfg::kDirect) q += static_cast<size_t>(4) * NRG * 16 * (1 << B);
  int8_t* xw = reinterpret_cast<int8_t*>(q) + static_cast<int64_t>(kq) * MT * xrow_bytes;

  const int e = rec[0], beg = rec[1], cnt = rec[2];
  const int64_t nrow = n0 + nl < p.N ? n0 + nl : p.N - 1;
  const int64_t erow = static_cast<int64_t>(e) * p.N + nrow;
  // code loads: a wave-uniform base (the expert) plus a 32-bit per-lane offset
  const unsigned char* ebase = p.codes + e * p.code_bytes;
  const uint32_t voff = static_cast<uint32_t>(nrow * (p.K * B / 8)) + static_cast<uint32_t>(kb * DW * 4);

  // Group parameters of the wave's range (entry gi = g - g0 of each row): the
  // raw (s, a|b) into LDS first, then each lane of a row turns every fourth
  // entry into (fp32(s / 127), carriers).
#pragma unroll
  for (int r = 0; r < kA8GpRegs; ++r) {
    if (4 * r < gn) {
      const int gi = kb + 4 * r;
      const int g = g0 + (gi < gn ? gi : 0);
      const uint32_t sv = __float_as_uint(p.scales[erow * gpr + g]);
      const uint32_t abv = reinterpret_cast<const uint32_t*>(p.shapes)[erow * gpr + g];
      if (gi < gn) {
        gp_row[gi * GPD] = sv;
        gp_row[gi * GPD + 1] = abv;
      }
    }
  }

  const int nv = (te - tb) * 8 * SUB;           // 16-byte activation vectors of the wave's slice
  for (int mt = 0; mt < cnt; mt += MT) {
    const int Mt = min(MT, cnt - mt);
    int pr[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int mm = m < Mt ? m : 0;            // rows past the pass repeat its first pair
      if constexpr (DENSE) {
        pr[m] = mt + mm;
      } else {
        pr[m] = (mt == 0 && mm < 2) ? rec[3 + mm] : p.sorted[__builtin_amdgcn_readfirstlane(beg + mt + mm)];
      }
    }
    const u32x4* xv[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
      xv[m] = reinterpret_cast<const u32x4*>(p.xq + static_cast<int64_t>(pr[m] / p.topk) * p.K +
                                             static_cast<int64_t>(tb) * 128 * SUB);
    // Up to four rows a pass: the first activation vectors of each row first
    // (unconditional, indices clamped), then the code stream. More rows copy
    // their activations after the code loads are issued.
    constexpr int XR = MT <= 4 ? 2 : 0;
    static_assert(XR > 0 || MT % 4 == 0, "wide passes stage four rows at a time");
    u32x4 xr[MT][XR > 0 ? XR : 1];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < XR; ++r) {
        const int i = lane + 64 * r;
        xr[m][r] = xv[m][i < nv ? i : 0];
      }
    __builtin_amdgcn_sched_barrier(0);
    uint32_t cb[PS][DW];
    auto load_step = [&](auto u_c, int treq) {
      constexpr int u = decltype(u_c)::value;
      int t = treq < te ? treq : te - 1;
      t = t < 0 ? 0 : t;
      const unsigned char* sb = ebase + static_cast<int64_t>(t) * (16 * DW);  // uniform
      load_chunk_dwords<DW>(reinterpret_cast<const uint32_t*>(sb + voff), cb[u]);
    };
    [&]<int... U>(std::integer_sequence<int, U...>) {
      (load_step(std::integral_constant<int, U>{}, tb + U), ...);
    }(std::make_integer_sequence<int, PS>{});
    __builtin_amdgcn_sched_barrier(0);

    if (mt == 0) {
      wave_lds_order();
#pragma unroll 1
      for (int gi = kb; gi < gn; gi += 4) {
        uint32_t* ent = gp_row + gi * GPD;
        const float s = __uint_as_float(ent[0]);
        const uint32_t ab = ent[1];
        ent[0] = __float_as_uint(__fdiv_rn(s, 127.0f));
        if constexpr (Cfg::kRegTable) {
          uint32_t T[(1 << B) / 4];
          carrier_regs<B>(ab, T);
#pragma unroll
          for (int d = 0; d < (1 << B) / 4; ++d) ent[1 + d] = T[d];
        }
      }
    }
    // this pass's activation rows into the wave's LDS slice
    auto put = [&](int m, int i, const u32x4& v) {
      u32x4* xo = reinterpret_cast<u32x4*>(xw + m * xrow_bytes);
      if constexpr (B == 2) {
        xo[i] = transpose16(v);
      } else {
        xo[i] = v;
      }
    };
    if constexpr (XR > 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m >= Mt) break;
#pragma unroll
        for (int r = 0; r < XR; ++r) {
          const int i = lane + 64 * r;
          if (i < nv) put(m, i, xr[m][r]);
        }
        for (int i = lane + 64 * XR; i < nv; i += 64) put(m, i, xv[m][i]);
      }
    } else {
      // four rows by two vectors a batch: eight loads in flight per lane; with
      // two row groups each stages half of the rows
#pragma unroll
      for (int m0 = (MT / NRG) * rg; m0 < (MT / NRG) * (rg + 1); m0 += 4) {
        if (m0 >= Mt) break;
        for (int i0 = lane; i0 < nv; i0 += 128) {
          u32x4 v[4][2];
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int r = 0; r < 2; ++r) {
              const int i = i0 + 64 * r;
              v[m][r] = xv[m0 + m][i < nv ? i : 0];
            }
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int r = 0; r < 2; ++r) {
              const int i = i0 + 64 * r;
              if (m0 + m < Mt && i < nv) put(m0 + m, i, v[m][r]);
            }
        }
      }
    }
    if constexpr (NRG > 1) {
      __syncthreads();                           // the other row group's half of the rows
    } else {
      wave_lds_order();
    }

    // the stream: int32 sums per group, fp32 across groups
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    i32x4 isum = {0, 0, 0, 0};
    bool fresh = true;
    float sc = 0.0f;
    int gi_next = 0, t_next = tb;                // next group entry and the step that opens it
    uint32_t T[Cfg::kRegTable ? (1 << B) / 4 : 1];
    float ga = 0.0f, gb = 0.0f;                 // the open group's (a, b) (per-code carriers)
    const int ml = nl < Mt ? nl : 0;
    const int8_t* xa = xw + ml * xrow_bytes;
    for (int t0 = tb; t0 < te; t0 += PS) {
      [&]<int... U>(std::integer_sequence<int, U...>) {
        (([&] {
           constexpr int u = U;
           const int t = t0 + u;
           if (t < te) {
#pragma unroll
             for (int d = 0; d < DW; ++d) asm volatile("" : "+v"(cb[u][d]));
             if (t == t_next) {                   // wave-uniform: a group opens
               if (!fresh) {
#pragma unroll
                 for (int r = 0; r < 4; ++r) acc[r] = fmaf(static_cast<float>(isum[r]), sc, acc[r]);
               }
               fresh = true;
               const uint32_t* ent = gp_row + gi_next * GPD;
               ++gi_next;
               t_next = (g0 + gi_next) * geo.spg;
               sc = __uint_as_float(ent[0]);
               if constexpr (Cfg::kRegTable) {
#pragma unroll
                 for (int d = 0; d < (1 << B) / 4; ++d) T[d] = ent[1 + d];
               } else if constexpr (Cfg::kDirect) {
                 ga = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(ent[1] & 0xffffu)));
                 gb = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(ent[1] >> 16)));
               } else {
                 wave_lds_order();                // earlier reads of the old table stay ahead
                 build_lds_table<B>(tab_row, kb, ent[1]);
                 wave_lds_order();
               }
             }
#pragma unroll
             for (int h = 0; h < SUB; ++h) {
               // chunk h of the lane's SUB chunks: codes 32 (SUB kb + h) .. + 31 of the step
               uint32_t car[8];
               if constexpr (B == 2) {
                 decode_w2(cb[u] + B * h, T[0], car);
               } else if constexpr (Cfg::kRegTable) {
                 decode_regs<B>(cb[u], T, car);
               } else if constexpr (Cfg::kDirect) {
                 decode_direct<B>(cb[u], ga, gb, car);
               } else {
                 decode_lds<B>(cb[u], tab_row, car);
               }
               const u32x4* xf = reinterpret_cast<const u32x4*>(xa + (((t - tb) * 4 + kb) * SUB + h) * 32);
               isum = mfma_i8(xf[0], u32x4{car[0], car[1], car[2], car[3]}, fresh ? i32x4{0, 0, 0, 0} : isum);
               isum = mfma_i8(xf[1], u32x4{car[4], car[5], car[6], car[7]}, isum);
               fresh = false;
             }
           }
           if constexpr (!ALLIN) load_step(std::integral_constant<int, u>{}, t + PS);
           __builtin_amdgcn_sched_barrier(0);
         }()),
         ...);
      }(std::make_integer_sequence<int, PS>{});
    }
    if (!fresh) {
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = fmaf(static_cast<float>(isum[r]), sc, acc[r]);
    }

    // acc row 4 kb + r is activation row m of this pass, column nl the weight row
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wave * 16 + 4 * kb + r) * 16 + nl] = acc[r];
    __syncthreads();
    // thread tt of row group rg (tt / 256 = rg) sums that group's four partials
    const int tt = threadIdx.x & 255;
    if (tt < Mt * 16) {
      const int m = tt >> 4, cc = tt & 15;
      if (n0 + cc < p.N) {
        int qp = pr[0];
#pragma unroll
        for (int k = 1; k < MT; ++k) qp = m == k ? pr[k] : qp;
        const float* rr = red + rg * 4 * 16 * 16;
        float v = rr[(0 * 16 + m) * 16 + cc];
        v += rr[(1 * 16 + m) * 16 + cc];
        v += rr[(2 * 16 + m) * 16 + cc];
        v += rr[(3 * 16 + m) * 16 + cc];
        v *= p.xs[qp / p.topk];
        store_out(p.y, p.ybf16 != 0, static_cast<int64_t>(qp) * p.N + n0 + cc, bad_pair ? 0.0f : v);
      }
    }
    if (mt + MT < cnt) __syncthreads();   // red and the activation slices are reused by the next pass
  }
}

// 2-bit codes take 16-byte code loads per lane (two 32-code chunks a step) when
// K and the group are multiples of 256.
inline bool a8_sub2(int bits, int64_t K, int group) { return bits == 2 && K % 256 == 0 && group % 256 == 0; }

template <int B, int SUB>
hipError_t launch_moe_a8_bs(const MoeA8Params& p, int64_t blocks, int T, hipStream_t st) {
  const A8Geom geo = a8_geom(p.K, p.group, SUB);
  const bool allin = geo.mpw <= A8Cfg<B>::kSlots / SUB;
  // One row per pass for one token (decode), four when several tokens are
  // routed and the slices fit; more pairs of an expert take more passes.
  int mt = T <= 1 ? 1 : 4;
  if (mt == 4 && a8_lds_bytes<B>(geo, 4, 1, SUB) > 80 * 1024) mt = 1;
  const size_t lds = a8_lds_bytes<B>(geo, mt, 1, SUB);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  auto kern = mt == 1 ? (allin ? k_moe_a8<B, 1, true, false, 1, SUB> : k_moe_a8<B, 1, false, false, 1, SUB>)
                      : (allin ? k_moe_a8<B, 4, true, false, 1, SUB> : k_moe_a8<B, 4, false, false, 1, SUB>);
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(256), lds, st, p);
  return hipGetLastError();
}

template <int B>
hipError_t launch_moe_a8_b(const MoeA8Params& p, int64_t blocks, int T, hipStream_t st) {
  if constexpr (B == 2) {
    if (a8_sub2(B, p.K, p.group)) return launch_moe_a8_bs<B, 2>(p, blocks, T, st);
  }
  return launch_moe_a8_bs<B, 1>(p, blocks, T, st);
}

}  // namespace

bool moe_a8_supported(int64_t K, int bits, int group) {
  if (bits < 2 || bits > 8 || K < 0 || K > (int64_t{1} << 28)) return false;
  if (K % 128 != 0 || group % 128 != 0 || group > 1024 || (K > 0 && K % group != 0)) return false;
  const int sub = a8_sub2(bits, K, group) ? 2 : 1;
  const A8Geom geo = a8_geom(K, group, sub);
  if (geo.gmax > 4 * kA8GpRegs) return false;
  size_t lds = 0;
  switch (bits) {
    case 2: lds = a8_lds_bytes<2>(geo, 1, 1, sub); break;
    case 3: lds = a8_lds_bytes<3>(geo, 1); break;
    case 4: lds = a8_lds_bytes<4>(geo, 1); break;
    case 5: lds = a8_lds_bytes<5>(geo, 1); break;
    case 6: lds = a8_lds_bytes<6>(geo, 1); break;
    case 7: lds = a8_lds_bytes<7>(geo, 1); break;
    default: lds = a8_lds_bytes<8>(geo, 1); break;
  }
  return lds <= 160 * 1024;
}

template <int B, int SUB>
hipError_t launch_gemv_a8_bs(const MoeA8Params& p, hipStream_t st) {
  const A8Geom geo = a8_geom(p.K, p.group, SUB);
  const bool allin = geo.mpw <= A8Cfg<B>::kSlots / SUB;
  // Rows per pass: all 16 rows of the MFMA's activation side for more than
  // four rows when their slices fit the LDS, else four, else one.
  // 16-row passes take two 16-row groups per workgroup (eight waves) where both
  // groups' tables fit: the 16 activation rows of a slice take most of the LDS,
  // so one workgroup a compute unit, and 32 rows keep every tile in one round.
  int mt = p.dense_m <= 1 ? 1 : (p.dense_m <= 4 ? 4 : 16);
  int nrg = 1;
  if (mt == 16 && a8_lds_bytes<B>(geo, 16, 2, SUB) <= 160 * 1024) nrg = 2;
  if (mt == 16 && nrg == 1 && a8_lds_bytes<B>(geo, 16, 1, SUB) > 160 * 1024) mt = 4;
  if (mt == 4 && a8_lds_bytes<B>(geo, 4, 1, SUB) > 160 * 1024) mt = 1;
  const size_t lds = a8_lds_bytes<B>(geo, mt, nrg, SUB);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  auto kern = mt == 1 ? (allin ? k_moe_a8<B, 1, true, true, 1, SUB> : k_moe_a8<B, 1, false, true, 1, SUB>)
              : mt == 4 ? (allin ? k_moe_a8<B, 4, true, true, 1, SUB> : k_moe_a8<B, 4, false, true, 1, SUB>)
              : nrg == 1 ? (allin ? k_moe_a8<B, 16, true, true, 1, SUB> : k_moe_a8<B, 16, false, true, 1, SUB>)
                         : (allin ? k_moe_a8<B, 16, true, true, 2, SUB> : k_moe_a8<B, 16, false, true, 2, SUB>);
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  const int64_t tiles = (p.N + 16 * nrg - 1) / (16 * nrg);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(tiles)), dim3(256 * nrg), lds, st, p);
  return hipGetLastError();
}

template <int B>
hipError_t launch_gemv_a8_b(const MoeA8Params& p, hipStream_t st) {
  if constexpr (B == 2) {
    if (a8_sub2(B, p.K, p.group)) return launch_gemv_a8_bs<B, 2>(p, st);
  }
  return launch_gemv_a8_bs<B, 1>(p, st);
}

hipError_t launch_gemv_a8(const MoeA8Params& p, int bits, hipStream_t st) {
  if (p.dense_m <= 0 || p.N <= 0) return hipSuccess;
  if ((p.N + 15) / 16 > 0x7fffffff) return hipErrorInvalidValue;
  switch (bits) {
    case 2: return launch_gemv_a8_b<2>(p, st);
    case 3: return launch_gemv_a8_b<3>(p, st);
    case 4: return launch_gemv_a8_b<4>(p, st);
    case 5: return launch_gemv_a8_b<5>(p, st);
    case 6: return launch_gemv_a8_b<6>(p, st);
    case 7: return launch_gemv_a8_b<7>(p, st);
    default: return launch_gemv_a8_b<8>(p, st);
  }
}

hipError_t launch_moe_a8_product(const MoeA8Params& p, int P, int E, int T, int bits, hipStream_t st) {
  const int64_t tiles = (p.N + 15) / 16;
  const int64_t blocks = static_cast<int64_t>(min(E, P)) * tiles;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  switch (bits) {
    case 2: return launch_moe_a8_b<2>(p, blocks, T, st);
    case 3: return launch_moe_a8_b<3>(p, blocks, T, st);
    case 4: return launch_moe_a8_b<4>(p, blocks, T, st);
    case 5: return launch_moe_a8_b<5>(p, blocks, T, st);
    case 6: return launch_moe_a8_b<6>(p, blocks, T, st);
    case 7: return launch_moe_a8_b<7>(p, blocks, T, st);
    default: return launch_moe_a8_b<8>(p, blocks, T, st);
  }
}

// One token (at most 64 pairs): the product reads the ids itself and no
// routing kernel runs. Sets p's direct fields and returns true when this applies.
static bool moe_a8_set_direct(MoeA8Params& p, const int32_t* ids, int T, int P, int E, int32_t* hdr) {
  if (T != 1 || P < 1 || P > 64) return false;
  p.direct = 1;
  p.npairs = P;
  p.E = E;
  p.ids = ids;
  p.bad_count = hdr;
  p.hdr = hdr; p.erec = ids; p.sorted = ids;
  return true;
}

hipError_t launch_moe_a8(const int32_t* ids, int T, int E, int topk, const MoeA8Params& base, int32_t* hdr,
                         int32_t* erec, int32_t* sorted, int bits, hipStream_t st) {
  const int P = T * topk;
  MoeA8Params p = base;
  p.topk = topk;
  p.direct = 0;
  if (moe_a8_set_direct(p, ids, T, P, E, hdr)) return launch_moe_a8_product(p, P, P, T, bits, st);
  hipError_t err = launch_moe_route(ids, P, E, base.N, base.y, base.ybf16, hdr, erec, sorted, st);
  if (err != hipSuccess) return err;
  p.hdr = hdr; p.erec = erec; p.sorted = sorted;
  return launch_moe_a8_product(p, P, E, T, bits, st);
}

hipError_t launch_moe_mlp_a8(const uint16_t* x, const int32_t* ids, const float* topk_w, int T, int E, int topk,
                             const MoeA8Params& up, int up_bits, const MoeA8Params& dn, int dn_bits,
                             int32_t* hdr, int32_t* erec, int32_t* sorted, const MoeMlpA8Buffers& b, float* out,
                             hipStream_t st) {
  const int P = T * topk;
  const int64_t H = up.K, I = dn.K;
  hipError_t err = launch_act_quant(x, false, T, H, b.xq, b.xs, st);
  if (err != hipSuccess) return err;
  MoeA8Params pu = up;
  pu.xq = b.xq; pu.xs = b.xs; pu.y = b.y1; pu.ybf16 = 0;
  err = launch_moe_a8(ids, T, E, topk, pu, hdr, erec, sorted, up_bits, st);
  if (err != hipSuccess) return err;
  err = launch_moe_act(b.y1, P, I, b.h, st);
  if (err != hipSuccess) return err;
  err = launch_act_quant(b.h, false, P, I, b.hq, b.hs, st);
  if (err != hipSuccess) return err;
  MoeA8Params pd = dn;
  pd.topk = 1;                                 // one activation row per pair
  pd.xq = b.hq; pd.xs = b.hs; pd.y = b.y2; pd.ybf16 = 0;
  pd.direct = 0;
  // one token: both products read the ids themselves (launch_moe_a8 took the
  // same decision for gate_up); otherwise the gate_up product's routing
  if (moe_a8_set_direct(pd, ids, T, P, E, hdr)) {
    err = launch_moe_a8_product(pd, P, P, T, dn_bits, st);
  } else {
    pd.hdr = hdr; pd.erec = erec; pd.sorted = sorted;
    err = launch_moe_a8_product(pd, P, E, T, dn_bits, st);
  }
  if (err != hipSuccess) return err;
  return launch_moe_combine(b.y2, ids, topk_w, T, topk, E, dn.N, out, st);
}

}  // namespace cubic
