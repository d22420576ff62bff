// moe.hip -- routed-expert A16 products grouped by expert on the device.
//
// The K3 expert layer (Kimi K3 guide, model-card table: 896 experts, 16 active
// per token) runs every (token, slot) pair against its expert's Cubic weights.
// The CubicQuant article (section on the A16/A8 crossover) notes that routing
// density changes which kernel wins; here the pairs are grouped per expert so
// that every touched expert's weights stream from HBM once per launch, whatever
// the number of tokens that picked it.
//
// k_moe_route (one block): per-expert counts and prefix sums in LDS, the pair
// ids grouped by expert, and a compact record per touched expert.
// Invalid ids are counted in hdr[0] and their output rows zeroed. No host sync.
// k_moe_gemv: one workgroup per (touched expert, 16-row tile); the expert's
// pairs form the activation rows of the MFMA tile (up to two per pass).
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "gemv_core.h"
#include "launch.h"

namespace cubic {

constexpr int kRouteExperts = 2048;   // experts per LDS chunk of the routing kernel
constexpr int kRouteIdRegs = 4;       // pair ids held in registers per thread (4096 pairs)

// Exclusive prefix sums over the 1024 threads of two per-thread values
// (wave shuffles, then the 16 wave totals); returns the block totals.
__device__ __forceinline__ void block_scan2(int a, int b, int* s_w, int& ea, int& eb, int& ta,
                                            int& tb) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = a, y = b;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(x, o), v = __shfl_up(y, o);
    if (lane >= o) { x += u; y += v; }
  }
  if (lane == 63) { s_w[w] = x; s_w[16 + w] = y; }
  __syncthreads();
  int pa = 0, pb = 0;
  ta = 0; tb = 0;
  for (int k = 0; k < 16; ++k) {
    const int wa = s_w[k], wb = s_w[16 + k];
    if (k < w) { pa += wa; pb += wb; }
    ta += wa; tb += wb;
  }
  ea = pa + x - a;
  eb = pb + y - b;
  __syncthreads();                             // s_w is reused by the next call
}

// One block of 1024 threads. Counts, prefix sums and write cursors live in LDS,
// over experts in chunks of kRouteExperts; pair ids are read once into
// registers (up to 4096 pairs, beyond that re-read per pass).
__global__ __launch_bounds__(1024) void k_moe_route(const int32_t* __restrict__ ids, int P, int E,
                                                    int64_t N, float* __restrict__ y, int ybf16,
                                                    int32_t* __restrict__ hdr,
                                                    int32_t* __restrict__ erec,
                                                    int32_t* __restrict__ sorted) {
  constexpr int kBadList = 256;                 // invalid pairs whose rows are cleared cooperatively
  constexpr int EPT = kRouteExperts / 1024;     // experts per thread in a chunk
  __shared__ int32_t s_cnt[kRouteExperts];      // counts, then write cursors
  __shared__ int32_t s_beg[kRouteExperts];      // first position of each expert in sorted
  __shared__ int32_t s_first[kRouteExperts][2]; // first two pair ids of each expert
  __shared__ int32_t s_w[32];
  __shared__ int32_t s_bad[kBadList];
  __shared__ int32_t s_nbad;
  const int tid = threadIdx.x;
  int idr[kRouteIdRegs];
#pragma unroll
  for (int r = 0; r < kRouteIdRegs; ++r) {
    const int p = tid + 1024 * r;
    idr[r] = p < P ? ids[p] : -1;
  }
  // f(e, p) for every pair p of this thread: the first kRouteIdRegs from registers
  auto each_pair = [&](auto&& f) {
#pragma unroll
    for (int r = 0; r < kRouteIdRegs; ++r) {
      const int p = tid + 1024 * r;
      if (p < P) f(idr[r], p);
    }
    for (int p = tid + 1024 * kRouteIdRegs; p < P; p += 1024) f(ids[p], p);
  };
  if (tid == 0) s_nbad = 0;
  __syncthreads();
  each_pair([&](int e, int p) {
    if (e < 0 || e >= E) {
      const int k = atomicAdd(&s_nbad, 1);
      if (k < kBadList) {
        s_bad[k] = p;
      } else {                                  // beyond the list: this thread clears the row
        for (int64_t n = 0; n < N; ++n) store_out(y, ybf16 != 0, static_cast<int64_t>(p) * N + n, 0.0f);
      }
    }
  });
  __syncthreads();
  // output rows of invalid pairs are zero
  const int nbad = min(s_nbad, kBadList);
  for (int b = 0; b < nbad; ++b) {
    const int64_t row = s_bad[b];
    for (int64_t n = tid; n < N; n += 1024) store_out(y, ybf16 != 0, row * N + n, 0.0f);
  }
  if (tid == 0) hdr[0] = s_nbad;

  int base_pairs = 0, base_act = 0;             // totals of the chunks before (block-uniform)
  for (int c0 = 0; c0 < E; c0 += kRouteExperts) {
    const int c1 = min(E, c0 + kRouteExperts);
    for (int k = tid; k < kRouteExperts; k += 1024) s_cnt[k] = 0;
    __syncthreads();
    each_pair([&](int e, int) {
      if (e >= c0 && e < c1) atomicAdd(&s_cnt[e - c0], 1);
    });
    __syncthreads();
    // this thread's experts c0 + EPT*tid + i: first pair offsets and record slots
    int cnt[EPT], sum = 0, act = 0;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      cnt[i] = s_cnt[EPT * tid + i];
      sum += cnt[i];
      act += cnt[i] > 0;
    }
    int off, slot, tot, tact;
    block_scan2(sum, act, s_w, off, slot, tot, tact);
    off += base_pairs;
    slot += base_act;
    int beg[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      beg[i] = off;
      s_beg[EPT * tid + i] = off;
      s_cnt[EPT * tid + i] = off;              // becomes the write cursor
      off += cnt[i];
    }
    __syncthreads();
    each_pair([&](int e, int p) {
      if (e >= c0 && e < c1) {
        const int pos = atomicAdd(&s_cnt[e - c0], 1);
        sorted[pos] = p;
        const int rank = pos - s_beg[e - c0];
        if (rank < 2) s_first[e - c0][rank] = p;
      }
    });
    __syncthreads();
    // One record per touched expert, in expert order: what a workgroup of the
    // product needs before it can issue its loads (expert, first pair, pair
    // count, the first two pair ids), in one 32-byte read.
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int k = EPT * tid + i;
      if (cnt[i] > 0) {
        const int f0 = s_first[k][0];
        erec[8 * slot] = c0 + k;
        erec[8 * slot + 1] = beg[i];
        erec[8 * slot + 2] = cnt[i];
        erec[8 * slot + 3] = f0;
        erec[8 * slot + 4] = cnt[i] > 1 ? s_first[k][1] : f0;
        ++slot;
      }
    }
    base_pairs += tot;
    base_act += tact;
    __syncthreads();                           // LDS arrays are reset by the next chunk
  }
  // Record slots up to the grid's bound get a zero pair count: a workgroup of the
  // product decides from its record alone whether it has work.
  if (tid == 0) hdr[1] = base_act;
  for (int a = base_act + tid; a < min(E, P); a += 1024) erec[8 * a + 2] = 0;
}

// One workgroup per work item (touched expert a, 16-row tile): the grid covers
// the largest possible number of touched experts and items past the device-side
// count exit at once. The expert's pairs are taken MT at a time; each wave
// copies its K slice of those tokens' prepared rows into its own LDS region (the
// layout the streaming loop reads in its in-kernel mode), so activations are
// read from LDS by the MFMA lanes instead of from global memory, and the four
// waves' partial sums meet in LDS in a fixed order.
template <class Dec, int SPL, int P, bool ALLIN, int MT, bool XF16>
__global__ __launch_bounds__(256, 3) void k_moe_gemv(MoeGemvParams p) {
  static_assert(MT == 1 || MT == 2, "one or two activation rows per pass");
  extern __shared__ __align__(1024) unsigned char smem[];   // table rows rely on this alignment
  constexpr int B = Dec::kBits;
  constexpr int XB = 2;                         // 16-element blocks per lane and row issued ahead
  const unsigned tiles = static_cast<unsigned>((p.N + 15) / 16);
  const unsigned a = blockIdx.x / tiles;
  const i32x8 rec = *reinterpret_cast<const i32x8*>(p.erec + 8 * a);
  if (rec[2] == 0) return;                      // fewer experts touched than the grid allows
  const int64_t n0 = static_cast<int64_t>(blockIdx.x - a * tiles) * 16;
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
  const int nblk = (te - tb) * kStep * SPL / 16;  // 16-element blocks in the wave's slice of a row
  const int gpr = static_cast<int>(p.K) / p.group;

  const int e = rec[0], beg = rec[1], cnt = rec[2];
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
    int pr[MT];                                 // pair ids of this pass (the first from the record)
#pragma unroll
    for (int m = 0; m < MT; ++m)
      pr[m] = mt == 0 ? (m == 0 ? rec[3] : rec[4]) : p.sorted[beg + mt + (m < Mt ? m : 0)];
    const u32x4* xv[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
      xv[m] = reinterpret_cast<const u32x4*>(p.x + static_cast<int64_t>(pr[m] / p.topk) * p.K + k0);
    XStage<Dec, MT, XB, XF16> xst;
    float xb[MT];
    auto issue_x = [&]() { xst.issue(xv, nblk, lane); };
    auto finish_x = [&]() { xst.finish(xv, xs_wave, geo.nch_w, nblk, lane, Mt, xb); };
    const f32x4 acc = gemv_core<Dec, true, SPL, P, ALLIN>(c, issue_x, finish_x);
    // acc row 4 kb + r is activation row m of this pass; undo the wave's prescale
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = acc[r];
      if (kb == 0 && r < Mt) v *= xb[r < MT ? r : 0];
      red[(wave * 16 + 4 * kb + r) * 16 + nl] = v;
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < Mt * 16) {
      const int m = t >> 4, cc = t & 15;
      if (n0 + cc < p.N) {
        const int q = MT == 1 || m == 0 ? pr[0] : pr[MT - 1];
        float v = red[(0 * 16 + m) * 16 + cc];
        v += red[(1 * 16 + m) * 16 + cc];
        v += red[(2 * 16 + m) * 16 + cc];
        v += red[(3 * 16 + m) * 16 + cc];
        store_out(p.y, p.ybf16 != 0, static_cast<int64_t>(q) * p.N + n0 + cc, v);
      }
    }
    if (mt + MT < cnt) __syncthreads();   // red and the LDS slices are reused by the next pass
  }
}

// Persistent variant: the items (touched expert, 16-row tile) are dealt to the
// workgroups in runs of `run` consecutive items, round robin, and each item
// is taken in passes of MT pairs. Within a run the units mostly share an expert
// and its token set, so the staged activation rows are reused (their loads are
// issued only when the token set changes); across the grid the workgroups stay
// within a window of gridDim.x runs, which keeps the pages and DRAM rows in use
// at any time few. While it computes
// one unit its lanes already have the next unit's loads in flight: every lane
// refills the code slot of macro step t with the next unit's macro step t right
// after consuming it, and the next unit's group parameters (and activation rows,
// when they change) are fetched one unit ahead into registers. So the memory
// pipe never drains at a unit boundary. Needs te - tb <= PM for every wave (one slot per macro step)
// and at most 4 * GPR groups per wave. OCC workgroups per compute unit.
template <class Dec, int SPL, int PM, int MT, int GPR, int OCC, bool XF16>
__global__ __launch_bounds__(256, OCC) void k_moe_stream(MoeGemvParams p,
                                                         const int32_t* __restrict__ erec,
                                                         const int32_t* __restrict__ sorted,
                                                         float* __restrict__ y, unsigned run) {
  static_assert(MT == 1 || MT == 2 || MT == 4, "one, two or four activation rows per pass");
  extern __shared__ __align__(1024) unsigned char smem[];   // table rows rely on this alignment
  constexpr int B = Dec::kBits;
  constexpr int DW = B * SPL;
  constexpr int XB = 2;
  const unsigned tiles = static_cast<unsigned>((p.N + 15) / 16);
  // Direct mode (one token, no routing kernel): item it is pair it / tiles,
  // whose expert erec[pair] holds (erec is the caller's id array then).
  const unsigned items = static_cast<unsigned>(p.direct ? p.npairs : p.hdr[1]) * tiles;
  const int lane = threadIdx.x & 63;
  if (p.direct && blockIdx.x == 0 && threadIdx.x < 64) {
    // the invalid-id count (npairs <= 64 in direct mode)
    const int e = lane < p.npairs ? erec[lane] : 0;
    const unsigned long long bad = __ballot(static_cast<unsigned>(e) >= static_cast<unsigned>(p.E));
    if (lane == 0) *p.bad_count = __popcll(bad);
  }
  // this workgroup's runs start at run * (blockIdx.x + j * gridDim.x)
  unsigned run_beg = run * blockIdx.x;
  if (run_beg >= items) return;
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
  const int nblk = (te - tb) * kStep * SPL / 16;
  const int gpr = static_cast<int>(p.K) / p.group;
  const int g0 = tb / geo.mpg;
  const int gn = te > tb ? (te - 1) / geo.mpg - g0 + 1 : 0;
  const int64_t row_bytes = p.K * B / 8;

  // A unit: item it (expert slot it / tiles, tile it % tiles) and pass mt.
  struct Unit {
    unsigned it;
    int mt, e, beg, cnt, M;
    int bad;                 // direct mode: invalid id, the unit stores zeros
    int pr[MT];
    int64_t n0;
  };
  auto make_unit = [&](unsigned it, int mt, const i32x8& rec) {
    Unit u;
    u.it = it;
    u.mt = mt;
    u.e = rec[0]; u.beg = rec[1]; u.cnt = rec[2];
    u.bad = p.direct ? rec[5] : 0;
    u.M = min(MT, u.cnt - mt);
    u.n0 = static_cast<int64_t>(it % tiles) * 16;
    // wave-uniform indices (readfirstlane) make these scalar loads, which do
    // not wait behind the vector loads in flight
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      // rows past the pass's M repeat its first pair (their loads are cache hits)
      const int mm = m < u.M ? m : 0;
      u.pr[m] = mt == 0 && mm < 2 ? (mm == 0 ? rec[3] : rec[4])
                                  : sorted[__builtin_amdgcn_readfirstlane(u.beg + mt + mm)];
    }
    return u;
  };
  auto load_rec = [&](unsigned it) {
    const int a = __builtin_amdgcn_readfirstlane(static_cast<int>(it / tiles));
    if (p.direct) {
      // a record of one pair: expert (expert 0's codes stand in for an invalid
      // id, whose rows are then stored as zeros), first position, one pair
      const int e = erec[a];
      const int ok = static_cast<unsigned>(e) < static_cast<unsigned>(p.E);
      return i32x8{ok ? e : 0, a, 1, a, a, 1 - ok, 0, 0};
    }
    return *reinterpret_cast<const i32x8*>(erec + 8 * a);
  };
  auto row_of = [&](const Unit& u) {
    const int64_t n = u.n0 + nl;
    return static_cast<int64_t>(u.e) * p.N + (n < p.N ? n : p.N - 1);
  };

  uint32_t cb[PM][DW];
  uint32_t gsc[GPR], gabr[GPR];
  XStage<Dec, MT, XB, XF16> xst;
  const u32x4* xv[MT];
  float xb[MT];
  auto issue_gp = [&](const Unit& u) {
    const int64_t r = row_of(u);
    const float* srow = p.scales + r * gpr;
    const uint32_t* abrow = reinterpret_cast<const uint32_t*>(p.shapes + r * gpr * 2);
#pragma unroll
    for (int k = 0; k < GPR; ++k) {
      const int gi = kb + 4 * k;
      const int g = g0 + (gi < gn ? gi : 0);
      gsc[k] = __float_as_uint(srow[g]);
      gabr[k] = abrow[g];
    }
  };
  auto set_x = [&](const Unit& u) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
      xv[m] = reinterpret_cast<const u32x4*>(p.x + static_cast<int64_t>(u.pr[m] / p.topk) * p.K + k0);
  };
  // A unit's code stream: a buffer resource on the tile's first row (wave-
  // uniform), a per-lane offset (row in the tile, chunk) and a per-slot
  // wave-uniform offset, so no per-slot address occupies vector registers.
  static_assert(DW == 4, "one 16-byte code load per lane and macro step");
  struct CodeSrc {
    __amdgpu_buffer_rsrc_t rs;
    uint32_t voff;
  };
  auto code_src = [&](const Unit& u) {
    const unsigned char* base = p.codes + u.e * p.code_bytes + u.n0 * row_bytes;
    const int64_t n = u.n0 + nl;
    const int64_t r = (n < p.N ? n : p.N - 1) - u.n0;   // rows past N repeat the last one
    CodeSrc c;
    c.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(base), static_cast<short>(0),
                                             static_cast<int>(16 * row_bytes), static_cast<int>(0x00020000u));
    c.voff = static_cast<uint32_t>(r * row_bytes) + static_cast<uint32_t>(kb * SPL * B * 4);
    return c;
  };
  auto issue_slot = [&](auto u_c, const CodeSrc& src) {
    constexpr int u = decltype(u_c)::value;
    int t = tb + u < te ? tb + u : te - 1;     // slots past the wave's range repeat its last step
    t = t < 0 ? 0 : t;                         // (a wave without steps reads step 0, unused)
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(src.rs, src.voff, t * (4 * SPL * B * 4), 0);
    cb[u][0] = v.x; cb[u][1] = v.y; cb[u][2] = v.z; cb[u][3] = v.w;
  };

  // first unit: everything issued now
  i32x8 rec = load_rec(run_beg);
  Unit cur = make_unit(run_beg, 0, rec);
  issue_gp(cur);
  set_x(cur);
  xst.issue(xv, nblk, lane);
  const u32x4* xv_cur[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) xv_cur[m] = xv[m];
  // parameters and activations stay ahead of the code loads (in the loop too), so
  // waiting for them never waits for the code stream
  __builtin_amdgcn_sched_barrier(0);
  {
    const CodeSrc src = code_src(cur);
    [&]<int... U>(std::integer_sequence<int, U...>) {
      (issue_slot(std::integral_constant<int, U>{}, src), ...);
    }(std::make_integer_sequence<int, PM>{});
  }
  bool xfresh = true;

  CoreArgs c;
  c.mpg = geo.mpg;
  c.tb = tb; c.te = te; c.nl = nl; c.kb = kb;
  c.xrow = nullptr; c.xs_wave = xs_wave; c.nch_w = geo.nch_w; c.tab_wave = tab_wave;
  c.gp_wave = gp_wave; c.gmax = geo.gmax;

  for (;;) {
    // the current unit's activations and group parameters into LDS
    if (xfresh) xst.finish(xv_cur, xs_wave, geo.nch_w, nblk, lane, cur.M, xb);
#pragma unroll
    for (int k = 0; k < GPR; ++k) {
      const int gi = kb + 4 * k;
      if (gi < gn) {
        gp_wave[(nl * geo.gmax + gi) * 2] = gsc[k];
        gp_wave[(nl * geo.gmax + gi) * 2 + 1] = gabr[k];
      }
    }
    wave_lds_order();

    // the next unit (the current one again when there is none: its loads are
    // then redundant cache hits and never used)
    bool has_next = true;
    Unit nxt;
    if (cur.mt + MT < cur.cnt) {
      nxt = make_unit(cur.it, cur.mt + MT, rec);
    } else {
      unsigned it_n = cur.it + 1;
      if (it_n == run_beg + run) {             // wave-uniform: on to the next run
        run_beg += run * gridDim.x;
        it_n = run_beg;
      }
      has_next = it_n < items;
      if (has_next) {
        rec = load_rec(it_n);
        nxt = make_unit(it_n, 0, rec);
      } else {
        nxt = cur;
      }
    }
    issue_gp(nxt);
    set_x(nxt);
    bool same_x = nxt.M == cur.M;
#pragma unroll
    for (int m = 0; m < MT; ++m)
      same_x = same_x && (m >= cur.M || nxt.pr[m] / p.topk == cur.pr[m] / p.topk);
    if (!same_x) xst.issue(xv, nblk, lane);  // wave-uniform
    __builtin_amdgcn_sched_barrier(0);

    // stream the current unit; each slot is refilled with the next unit's step
    StreamState st;
    st.reset(tb, g0);
    const int ml = nl < cur.M ? nl : 0;
    const CodeSrc src_n = code_src(nxt);
    [&]<int... U>(std::integer_sequence<int, U...>) {
      (([&] {
         constexpr int u = U;
         const int t = tb + u;
         if (t < te) {
#pragma unroll
           for (int d = 0; d < DW; ++d) asm volatile("" : "+v"(cb[u][d]));
           step_macro<Dec, true, SPL>(c, st, cb[u], nullptr, t, g0, ml);
         }
         issue_slot(std::integral_constant<int, u>{}, src_n);
         __builtin_amdgcn_sched_barrier(0);
       }()),
       ...);
    }(std::make_integer_sequence<int, PM>{});
    const f32x4 acc = st.total();

    // partial sums of the four waves meet in LDS in a fixed order
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = acc[r];
      if (kb == 0 && r < cur.M) v *= xb[r < MT ? r : 0];
      red[(wave * 16 + 4 * kb + r) * 16 + nl] = v;
    }
    __syncthreads();
    const int tt = threadIdx.x;
    if (tt < cur.M * 16) {
      const int m = tt >> 4, cc = tt & 15;
      if (cur.n0 + cc < p.N) {
        int qp = cur.pr[0];
#pragma unroll
        for (int k = 1; k < MT; ++k) qp = m == k ? cur.pr[k] : qp;
        float v = red[(0 * 16 + m) * 16 + cc];
        v += red[(1 * 16 + m) * 16 + cc];
        v += red[(2 * 16 + m) * 16 + cc];
        v += red[(3 * 16 + m) * 16 + cc];
        store_out(y, p.ybf16 != 0, static_cast<int64_t>(qp) * p.N + cur.n0 + cc, cur.bad ? 0.0f : v);
      }
    }
    __syncthreads();                          // red is rewritten by the next unit
    if (!has_next) break;
    cur = nxt;
#pragma unroll
    for (int m = 0; m < MT; ++m) xv_cur[m] = xv[m];
    xfresh = !same_x;
  }
}

// LDS of the grouped kernel for MT activation rows per pass.
template <class Dec>
static size_t moe_lds_bytes(const GemvGeom& geo, int mt) {
  return gemv_lds_fixed<Dec>(geo.gmax) + static_cast<size_t>(4) * mt * geo.nch_w * 32 * 2;
}

template <class Dec, int SPL, int P, bool XF16>
static hipError_t launch_moe_gemv_t(const MoeGemvParams& p, int64_t blocks, int tokens,
                                    hipStream_t st) {
  const GemvGeom geo = gemv_geom(p.K, p.group, SPL);
  // Rows per pass: two for the 2-bit (bf16) path when several tokens are routed
  // and two workgroups still fit in one compute unit's LDS, else one (the fp16
  // staging of two rows does not fit the register budget). Experts picked by
  // more tokens take several passes over their codes, which then come from L2.
  int mt = (tokens <= 1 || !IsW2<Dec>::value) ? 1 : 2;
  if (mt == 2 && moe_lds_bytes<Dec>(geo, 2) > 80 * 1024) mt = 1;
  const size_t lds = moe_lds_bytes<Dec>(geo, mt);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  const bool allin = geo.mpw <= P;
  constexpr int MT2 = IsW2<Dec>::value ? 2 : 1;
  auto pick = [&]() {
    if (allin) return mt == 1 ? k_moe_gemv<Dec, SPL, P, true, 1, XF16> : k_moe_gemv<Dec, SPL, P, true, MT2, XF16>;
    return mt == 1 ? k_moe_gemv<Dec, SPL, P, false, 1, XF16> : k_moe_gemv<Dec, SPL, P, false, MT2, XF16>;
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

// Workgroups per compute unit of the one-row (decode) instance of k_moe_stream
// (133 VGPRs a wave; four, at 128 VGPRs, measured slower: 54.5 against 51-52 us
// for the 16-expert decode step).
constexpr int kStreamOcc1 = 3;

// The persistent kernel for 2-bit codes with groups of 256 or more: PM slots
// cover a wave's macro steps, GPR registers its groups.
template <int PM, int GPR, bool XF16>
static hipError_t launch_moe_stream_t(const MoeGemvParams& p, int64_t blocks, int tokens,
                                      hipStream_t st) {
  using Dec = typename std::conditional<XF16, DecodeW2H, DecodeW2>::type;
  const GemvGeom geo = gemv_geom(p.K, p.group, 2);
  // Rows per pass: one token routes one row; with several, four rows per pass
  // (fewer passes, so fewer decodes and code re-reads, for experts picked by
  // more tokens), or two when four do not fit two workgroups' LDS.
  int mt = tokens <= 1 ? 1 : 4;
  if (mt == 4 && moe_lds_bytes<DecodeW2>(geo, 4) > 80 * 1024) mt = 2;
  if (mt == 2 && moe_lds_bytes<DecodeW2>(geo, 2) > 80 * 1024) mt = 1;
  const size_t lds = moe_lds_bytes<DecodeW2>(geo, mt);
  // several rows per pass need more registers: two workgroups per compute unit
  // (two rows a pass at three workgroups, 151 VGPRs, measured slower on 64
  // tokens routed to 16 of 896 experts: 2.37 against 2.26 ms with four rows at two)
  auto kern = mt == 1 ? k_moe_stream<Dec, 2, PM, 1, GPR, kStreamOcc1, XF16>
                      : (mt == 2 ? k_moe_stream<Dec, 2, PM, 2, GPR, 2, XF16>
                                 : k_moe_stream<Dec, 2, PM, 4, GPR, 2, XF16>);
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  // The resident workgroups walk the units in runs of up to 8 items: the
  // longest run that keeps the busiest workgroup's item count (for the largest
  // possible item count) lowest.
  const int64_t cus = device_cu_count();
  const int64_t occ = mt == 1 ? kStreamOcc1 : 2;
  const int64_t cap = (cus > 0 ? cus : 256) * occ;
  int64_t run = 1, best = INT64_MAX;
  for (int64_t r = 8; r >= 1; --r) {
    const int64_t runs = (blocks + r - 1) / r;
    const int64_t g = std::min(runs, cap);
    const int64_t span = (runs + g - 1) / g * r;
    if (span < best) { best = span; run = r; }
  }
  const int64_t want = (blocks + run - 1) / run;
  const unsigned grid = static_cast<unsigned>(want < cap ? want : cap);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, st, p, p.erec, p.sorted, p.y,
                     static_cast<unsigned>(run));
  return hipGetLastError();
}

size_t moe_lds_min_bytes(int64_t K, int bits, int group) {
  const int spl = (bits == 2 && group % 256 == 0) ? 2 : 1;
  const GemvGeom geo = gemv_geom(K, group, spl);
  return bits == 2 ? moe_lds_bytes<DecodeW2>(geo, 1) : moe_lds_bytes<DecodeTable<8>>(geo, 1);
}

// The grouped product over a routing already in hdr / erec / sorted (p holds
// them): P pairs, activation row of pair q = q / p.topk, output row q.
template <bool XF16>
static hipError_t launch_moe_product_t(const MoeGemvParams& p, int64_t blocks, int T, int bits,
                                       hipStream_t st) {
  using W2 = typename std::conditional<XF16, DecodeW2H, DecodeW2>::type;
  switch (bits) {
    case 2:
      if (p.group % 256 == 0) {
        const GemvGeom geo = gemv_geom(p.K, p.group, 2);
        if (geo.mpw <= 4 && geo.gmax <= 4) return launch_moe_stream_t<4, 1, XF16>(p, blocks, T, st);
        if (geo.mpw <= 7 && geo.gmax <= 8) return launch_moe_stream_t<7, 2, XF16>(p, blocks, T, st);
        if (geo.mpw <= 8 && geo.gmax <= 8) return launch_moe_stream_t<8, 2, XF16>(p, blocks, T, st);
        return launch_moe_gemv_t<W2, 2, 8, XF16>(p, blocks, T, st);
      }
      return launch_moe_gemv_t<W2, 1, 8, XF16>(p, blocks, T, st);
    case 3: return launch_moe_gemv_t<DecodeTable<3>, 1, 6, XF16>(p, blocks, T, st);
    case 4: return launch_moe_gemv_t<DecodeTable<4>, 1, 4, XF16>(p, blocks, T, st);
    case 5: return launch_moe_gemv_t<DecodeTable<5>, 1, 2, XF16>(p, blocks, T, st);
    case 6: return launch_moe_gemv_t<DecodeTable<6>, 1, 2, XF16>(p, blocks, T, st);
    case 7: return launch_moe_gemv_t<DecodeDirect<7, false>, 1, 2, XF16>(p, blocks, T, st);
    default: return launch_moe_gemv_t<DecodeDirect<8, false>, 1, 2, XF16>(p, blocks, T, st);
  }
}

// The grouped product over a routing already in hdr / erec / sorted (p holds
// them): P pairs, activation row of pair q = q / p.topk, output row q.
static hipError_t launch_moe_product(const MoeGemvParams& p, int P, int E, int T, int bits,
                                     bool xf16, hipStream_t st) {
  const int64_t tiles = (p.N + 15) / 16;
  const int64_t blocks = static_cast<int64_t>(min(E, P)) * tiles;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  return xf16 ? launch_moe_product_t<true>(p, blocks, T, bits, st)
              : launch_moe_product_t<false>(p, blocks, T, bits, st);
}

hipError_t launch_moe_route(const int32_t* ids, int P, int E, int64_t N, float* y, int ybf16, int32_t* hdr,
                            int32_t* erec, int32_t* sorted, hipStream_t st) {
  hipLaunchKernelGGL(k_moe_route, dim3(1), dim3(1024), 0, st, ids, P, E, N, y, ybf16, hdr, erec, sorted);
  return hipGetLastError();
}

// One token (its pairs all distinct rows of one activation row, at most 64)
// on the streaming kernel: the product reads the ids itself, and no routing
// kernel runs. Sets p's direct fields and returns true when this applies.
static bool moe_set_direct(MoeGemvParams& p, const int32_t* ids, int T, int P, int E, int bits,
                           int32_t* hdr) {
  if (T != 1 || P < 1 || P > 64 || bits != 2 || p.group % 256 != 0) return false;
  const GemvGeom geo = gemv_geom(p.K, p.group, 2);
  if (!(geo.mpw <= 8 && geo.gmax <= 8)) return false;   // launch_moe_product_t's k_moe_stream cases
  p.direct = 1;
  p.npairs = P;
  p.E = E;
  p.ids = ids;
  p.bad_count = hdr;
  p.hdr = hdr;
  p.erec = ids;
  p.sorted = ids;
  return true;
}

hipError_t launch_moe(const int32_t* ids, int T, int E, int topk, const MoeGemvParams& base,
                      int32_t* hdr, int32_t* erec, int32_t* sorted, int bits, bool xf16, hipStream_t st) {
  const int P = T * topk;
  MoeGemvParams p = base;
  p.topk = topk;
  p.direct = 0;
  if (moe_set_direct(p, ids, T, P, E, bits, hdr))
    return launch_moe_product(p, P, P, T, bits, xf16, st);
  const hipError_t err = launch_moe_route(ids, P, E, base.N, base.y, base.ybf16, hdr, erec, sorted, st);
  if (err != hipSuccess) return err;
  p.hdr = hdr; p.erec = erec; p.sorted = sorted;
  return launch_moe_product(p, P, E, T, bits, xf16, st);
}

// ---------------------------------------------------------------------------
// The routed-expert MLP step around the two grouped products: h = SiLU(gate) *
// up in fp32, rounded to bf16 (the down product's activation rows, one per
// pair), and the router-weighted sum of each token's pair outputs.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_moe_act(const float* __restrict__ y1, int64_t P, int64_t I,
                                                 uint16_t* __restrict__ h) {
  const int64_t nvec = P * I / 4;
  for (int64_t v = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; v < nvec;
       v += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t q = v / (I / 4), i = (v - q * (I / 4)) * 4;
    const f32x4 g = *reinterpret_cast<const f32x4*>(y1 + q * 2 * I + i);
    const f32x4 u = *reinterpret_cast<const f32x4*>(y1 + q * 2 * I + I + i);
    uint32_t o[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float h0 = g[2 * e] / (1.0f + expf(-g[2 * e])) * u[2 * e];
      const float h1 = g[2 * e + 1] / (1.0f + expf(-g[2 * e + 1])) * u[2 * e + 1];
      o[e] = bf16_rne_bits(h0) | (bf16_rne_bits(h1) << 16);
    }
    *reinterpret_cast<uint2*>(h + q * I + i) = make_uint2(o[0], o[1]);
  }
}

__global__ __launch_bounds__(256) void k_moe_combine(const float* __restrict__ y2,
                                                     const int32_t* __restrict__ ids,
                                                     const float* __restrict__ w, int64_t T, int topk,
                                                     int E, int64_t H, float* __restrict__ out) {
  const int64_t nvec = T * H / 4;
  for (int64_t v = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; v < nvec;
       v += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t t = v / (H / 4), n = (v - t * (H / 4)) * 4;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    // Eight slots at a time: every load of a chunk is issued before the first
    // sum (rows q < T * topk all lie inside y2, so a slot past topk or with an
    // invalid id loads a row in bounds and is then left out); the sums still
    // run in slot order, so the result does not depend on the chunking.
    for (int j0 = 0; j0 < topk; j0 += 8) {
      bool ok[8];
      float wj[8];
      f32x4 r[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u < topk ? j0 + u : topk - 1;
        const int64_t q = t * topk + j;
        const int id = ids[q];
        ok[u] = j0 + u < topk && id >= 0 && id < E;    // invalid ids add nothing
        wj[u] = w[q];
        r[u] = *reinterpret_cast<const f32x4*>(y2 + q * H + n);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (!ok[u]) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = fmaf(wj[u], r[u][e], acc[e]);
      }
    }
    *reinterpret_cast<f32x4*>(out + t * H + n) = acc;
  }
}

static unsigned elementwise_grid(int64_t nvec) {
  const int64_t b = (nvec + 255) / 256;
  return static_cast<unsigned>(b < 8192 ? (b > 0 ? b : 1) : 8192);
}

hipError_t launch_moe_act(const float* y1, int64_t P, int64_t I, uint16_t* h, hipStream_t st) {
  hipLaunchKernelGGL(k_moe_act, dim3(elementwise_grid(P * I / 4)), dim3(256), 0, st, y1, P, I, h);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const float* y2, const int32_t* ids, const float* topk_w, int64_t T, int topk,
                              int E, int64_t H, float* out, hipStream_t st) {
  hipLaunchKernelGGL(k_moe_combine, dim3(elementwise_grid(T * H / 4)), dim3(256), 0, st, y2, ids, topk_w, T,
                     topk, E, H, out);
  return hipGetLastError();
}

hipError_t launch_moe_mlp(const int32_t* ids, const float* topk_w, int T, int E, int topk,
                          const MoeGemvParams& up, int up_bits, const MoeGemvParams& dn, int dn_bits,
                          int32_t* hdr, int32_t* erec, int32_t* sorted, uint16_t* h, float* out,
                          hipStream_t st) {
  const int P = T * topk;
  const int64_t I = dn.K, H = dn.N;
  MoeGemvParams p = dn;
  p.topk = 1;                                  // one activation row per pair
  p.x = h;
  p.direct = 0;
  // The down product reuses the gate_up product's routing, unless it reads the
  // ids itself; the routing kernel then runs only for a routed gate_up.
  const bool dn_direct = moe_set_direct(p, ids, T, P, E, dn_bits, hdr);
  hipError_t err;
  if (dn_direct) {
    err = launch_moe(ids, T, E, topk, up, hdr, erec, sorted, up_bits, false, st);
  } else {
    // the gate_up product must be routed too, so that the routing exists for down
    err = launch_moe_route(ids, P, E, up.N, up.y, up.ybf16, hdr, erec, sorted, st);
    if (err == hipSuccess) {
      MoeGemvParams u = up;
      u.topk = topk;
      u.direct = 0;
      u.hdr = hdr; u.erec = erec; u.sorted = sorted;
      err = launch_moe_product(u, P, E, T, up_bits, false, st);
    }
  }
  if (err != hipSuccess) return err;
  err = launch_moe_act(up.y, P, I, h, st);
  if (err != hipSuccess) return err;
  if (!dn_direct) { p.hdr = hdr; p.erec = erec; p.sorted = sorted; }
  err = launch_moe_product(p, P, E, T, dn_bits, false, st);
  if (err != hipSuccess) return err;
  return launch_moe_combine(dn.y, ids, topk_w, T, topk, E, H, out, st);
}

// ---------------------------------------------------------------------------
// Library-owned routing scratch for callers that cannot allocate device memory.
// The routing header, the per-expert records and the pair lists of one grouped
// product live here instead of in a caller's workspace. Each device holds its
// own copy for the life of the process; host code never passes `scratch` itself
// to a kernel, only the device address looked up once per device below.
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kMoeScratchBytes = size_t{2} << 20;
constexpr int kMoeScratchDevices = 64;
static __device__ __align__(256) unsigned char scratch[kMoeScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMoeScratchDevices] = {};
}  // namespace

size_t moe_scratch_bytes() { return kMoeScratchBytes; }

hipError_t moe_scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMoeScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // this device is current
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace cubic
