// api.cpp -- the C ABI of libcubic.so (declared in include/cubic.h): argument
// validation on the host, shape dispatch, kernel launches on the caller's
// stream. No device memory is allocated here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "../../include/cubic.h"
#include "launch.h"

#define CUBIC_API extern "C" __attribute__((visibility("default")))


using namespace cubic;

namespace {

constexpr size_t kLdsLimit = 160 * 1024;   // LDS of one gfx950 compute unit
// A8 rows taken by the routed kernel's organisation (passes of 16 rows): up to
// 32 for 2- and 3-bit codes (the A8 tile kernel is faster beyond), 256 for
// 4-bit codes, 128 for wider ones (measured on the expert shapes)
constexpr int64_t gemv_a8_max_m(int bits) { return bits <= 3 ? 32 : (bits == 4 ? 256 : 128); }
constexpr int64_t kSkinnyRows = 64;          // rows of one small-batch A16 pass
constexpr int64_t kSkinnyPassMaxM = 256;     // A16 rows taken as passes of the small-batch kernel
constexpr int64_t kGemvMaxM = 16;          // one MFMA activation tile
constexpr int64_t kGemvMaxMW2 = 8;         // 2-bit codes: the small-batch kernel is faster above
constexpr int64_t kInkMaxM = 4;            // single-kernel A16 path
constexpr int64_t kPrefillMinM = 256;      // 256 x 256 tile kernel (2-/3-bit codes)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

int check_weight(const cubic_weight* w) {
  if (!w) return CUBIC_ERR_NULL;
  if (w->N < 0 || w->K < 0) return CUBIC_ERR_SHAPE;
  if (w->bits < 2 || w->bits > 8) return CUBIC_ERR_BITS;
  if (w->group <= 0 || w->group % 128 != 0 || w->K % w->group != 0) return CUBIC_ERR_GROUP;
  if (w->N > 0 && w->K > 0) {
    if (!w->codes || !w->scales || !w->shapes) return CUBIC_ERR_NULL;
    if (!aligned16(w->codes) || !aligned16(w->scales) || !aligned16(w->shapes)) return CUBIC_ERR_ALIGN;
  }
  return CUBIC_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? CUBIC_OK : CUBIC_ERR_HIP; }

// Single-kernel A16 path: M <= 4, and for every width and group size (the worst
// case is 8 bits, group 128) the per-wave activation slices, level tables and
// group parameters fit in LDS and a wave spans few enough groups. Depends on
// (M, K) only, so the workspace size needs no weight description.
bool a16_inkernel(int64_t M, int64_t K) {
  return M <= kInkMaxM && K >= 128 && gemv_supported(K, 8, 128) && gemv_supported(K, 3, 128) &&
         gemv_ink_lds_bytes(M, K, 8, 128) <= kLdsLimit;
}

std::mutex g_pack_mutex[64];

}  // namespace

CUBIC_API size_t cubic_code_bytes(int64_t N, int64_t K, int bits) {
  if (N < 0 || K < 0 || bits < 2 || bits > 8) return 0;
  const int64_t b = N * K * bits;
  if (b % 8) return 0;
  return static_cast<size_t>(b / 8);
}

CUBIC_API size_t cubic_storage_bytes(int64_t N, int64_t K, int bits, int group) {
  if (group <= 0 || K % group != 0) return 0;
  const size_t c = cubic_code_bytes(N, K, bits);
  if (c == 0 && N * K != 0) return 0;
  return c + static_cast<size_t>(8) * N * (K / group);
}

CUBIC_API const char* cubic_status_string(int status) {
  switch (status) {
    case CUBIC_OK: return "ok";
    case CUBIC_ERR_NULL: return "null pointer";
    case CUBIC_ERR_SHAPE: return "invalid shape";
    case CUBIC_ERR_BITS: return "bits outside [2, 8]";
    case CUBIC_ERR_GROUP: return "group must be a multiple of 128 dividing K";
    case CUBIC_ERR_ALIGN: return "pointer not 16-byte aligned";
    case CUBIC_ERR_CODE_RANGE: return "code outside [-Kmax, Kmax]";
    case CUBIC_ERR_WORKSPACE: return "workspace missing or too small";
    case CUBIC_ERR_HIP: return "HIP runtime error";
    case CUBIC_ERR_DTYPE: return "unsupported activation or output dtype";
    default: return "unknown status";
  }
}

CUBIC_API const char* cubic_version(void) { return "cubic 0.1 gfx950"; }

CUBIC_API int cubic_pack(const int8_t* codes, int64_t N, int64_t K, int bits, uint8_t* packed,
                         cubic_stream_t stream) {
  if (N < 0 || K < 0 || K % 32 != 0) return CUBIC_ERR_SHAPE;
  if (bits < 2 || bits > 8) return CUBIC_ERR_BITS;
  if (N == 0 || K == 0) return CUBIC_OK;
  if (!codes || !packed) return CUBIC_ERR_NULL;
  if (!aligned16(codes) || !aligned16(packed)) return CUBIC_ERR_ALIGN;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return CUBIC_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_pack_mutex[dev & 63]);
  unsigned int bad = 0;
  const hipError_t e = launch_pack(codes, packed, N, K, bits, static_cast<hipStream_t>(stream), &bad);
  if (e != hipSuccess) return CUBIC_ERR_HIP;
  return bad ? CUBIC_ERR_CODE_RANGE : CUBIC_OK;
}

CUBIC_API int cubic_unpack(const uint8_t* packed, int64_t N, int64_t K, int bits, int8_t* codes,
                           cubic_stream_t stream) {
  if (N < 0 || K < 0 || K % 32 != 0) return CUBIC_ERR_SHAPE;
  if (bits < 2 || bits > 8) return CUBIC_ERR_BITS;
  if (N == 0 || K == 0) return CUBIC_OK;
  if (!codes || !packed) return CUBIC_ERR_NULL;
  if (!aligned16(codes) || !aligned16(packed)) return CUBIC_ERR_ALIGN;
  return hip_status(launch_unpack(packed, codes, N, K, bits, static_cast<hipStream_t>(stream)));
}

CUBIC_API int cubic_dequant(const cubic_weight* w, float* out, cubic_stream_t stream) {
  const int st = check_weight(w);
  if (st != CUBIC_OK) return st;
  if (w->N == 0 || w->K == 0) return CUBIC_OK;
  if (!out) return CUBIC_ERR_NULL;
  if (!aligned16(out)) return CUBIC_ERR_ALIGN;
  return hip_status(launch_dequant(w->codes, w->scales, w->shapes, out, w->N, w->K, w->bits,
                                   w->group, static_cast<hipStream_t>(stream)));
}

CUBIC_API int cubic_encode(const float* w, int64_t N, int64_t K, int bits, int group,
                           const float* scales, const uint16_t* shapes, int8_t* codes,
                           cubic_stream_t stream) {
  if (N < 0 || K < 0) return CUBIC_ERR_SHAPE;
  if (bits < 2 || bits > 8) return CUBIC_ERR_BITS;
  if (group <= 0 || group % 128 != 0 || K % group != 0) return CUBIC_ERR_GROUP;
  if (N == 0 || K == 0) return CUBIC_OK;
  if (!w || !scales || !shapes || !codes) return CUBIC_ERR_NULL;
  if (!aligned16(w) || !aligned16(scales) || !aligned16(shapes) || !aligned16(codes)) return CUBIC_ERR_ALIGN;
  if ((N * K / 8 + 255) / 256 > INT32_MAX) return CUBIC_ERR_SHAPE;
  return hip_status(launch_encode(w, N, K, bits, group, scales, shapes, codes,
                                  static_cast<hipStream_t>(stream)));
}

CUBIC_API int cubic_fit(const float* w, int64_t N, int64_t K, int bits, int group, int8_t* codes,
                        float* scales, uint16_t* shapes, float* loss, cubic_stream_t stream) {
  if (N < 0 || K < 0) return CUBIC_ERR_SHAPE;
  if (bits < 2 || bits > 8) return CUBIC_ERR_BITS;
  if (group <= 0 || group % 128 != 0 || group > fit_max_group() || K % group != 0) return CUBIC_ERR_GROUP;
  if (N == 0 || K == 0) return CUBIC_OK;
  if (!w || !codes || !scales || !shapes) return CUBIC_ERR_NULL;
  if (!aligned16(w) || !aligned16(codes) || !aligned16(scales) || !aligned16(shapes)) return CUBIC_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(loss) & 3u) != 0) return CUBIC_ERR_ALIGN;
  if (N * (K / group) > INT32_MAX) return CUBIC_ERR_SHAPE;
  return hip_status(launch_fit(w, N, K, bits, group, codes, scales, shapes, loss,
                               static_cast<hipStream_t>(stream)));
}

CUBIC_API size_t cubic_gemm_a16_workspace_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K < 0) return 0;
  if (a16_inkernel(M, K)) return 0;
  return align256(static_cast<size_t>(M) * K * 2) + align256(static_cast<size_t>(M) * 4);
}

namespace {
bool dtype_in_ok(int d) { return d == CUBIC_DTYPE_BF16 || d == CUBIC_DTYPE_F16; }
bool dtype_out_ok(int d) { return d == CUBIC_DTYPE_F32 || d == CUBIC_DTYPE_BF16; }

int gemm_a16_impl(const uint16_t* x, bool xf16, int64_t M, const cubic_weight* w, float* y, bool ybf16,
                  void* workspace, size_t ws_bytes, cubic_stream_t stream) {
  const int st = check_weight(w);
  if (st != CUBIC_OK) return st;
  if (M < 0) return CUBIC_ERR_SHAPE;
  if (M == 0 || w->N == 0) return CUBIC_OK;
  if (!x || !y) return CUBIC_ERR_NULL;
  if (!aligned16(x) || !aligned16(y)) return CUBIC_ERR_ALIGN;
  if (M > INT32_MAX / 2) return CUBIC_ERR_SHAPE;
  const size_t need = cubic_gemm_a16_workspace_bytes(M, w->K);
  if (need > 0) {
    if (!workspace || ws_bytes < need) return CUBIC_ERR_WORKSPACE;
    if (!aligned16(workspace)) return CUBIC_ERR_ALIGN;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int yb = ybf16 ? 1 : 0;
  if (w->K == 0) return hip_status(launch_fill_zero(y, M * w->N, ybf16, s));
  if (need == 0) {
    GemvParams p{w->codes, w->scales, w->shapes, w->N, w->K, w->group, static_cast<int>(M),
                 x, nullptr, nullptr, y, 0, yb};
    return hip_status(launch_gemv(p, w->bits, true, xf16, s));
  }
  uint16_t* xp = static_cast<uint16_t*>(workspace);
  float* xback = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                          align256(static_cast<size_t>(M) * w->K * 2));
  // up to 16 activation rows (2-bit codes: 8): the GEMV; 2- to 4-bit codes
  // with up to 64 rows: the small-batch MFMA kernel
  const bool use_gemv = M <= (w->bits == 2 ? kGemvMaxMW2 : kGemvMaxM) &&
                        gemv_supported(w->K, w->bits, w->group);
  const bool use_skinny = !use_gemv && skinny_supported(M, w->N, w->K, w->bits, w->group);
  // up to kSkinnyPassMaxM rows: the small-batch kernel in passes of 64 rows
  // (each pass streams the weight again; the tile kernels get too few tiles here)
  const bool use_passes = !use_gemv && !use_skinny && M <= kSkinnyPassMaxM &&
                          skinny_supported(kSkinnyRows, w->N, w->K, w->bits, w->group);
  if (use_gemv && w->bits > 2) {
    // 3- to 8-bit codes: the GEMV reads the caller's rows as they are (bf16:
    // against split bf16 levels; fp16: against fp16 levels)
    GemvParams p{w->codes, w->scales, w->shapes, w->N, w->K, w->group, static_cast<int>(M),
                 xf16 ? nullptr : x, xf16 ? x : nullptr, nullptr, y, 0, yb};
    return hip_status(launch_gemv(p, w->bits, false, xf16, s));
  }
  // fp16 rows are already what the multi-row kernels read (fp16, back factor 1);
  // bf16 rows are converted (or, for the 2-bit GEMV, reordered) first
  const uint16_t* xa = x;
  const float* xs = nullptr;
  if (!xf16 || use_gemv) {
    hipError_t e = launch_xprep(x, M, w->K, use_gemv, xp, xback, s);
    if (e != hipSuccess) return CUBIC_ERR_HIP;
    xa = xp;
    xs = xback;
  }
  if (use_gemv) {
    GemvParams p{w->codes, w->scales, w->shapes, w->N, w->K, w->group, static_cast<int>(M),
                 nullptr, xa, xs, y, 0, yb};
    return hip_status(launch_gemv(p, w->bits, false, xf16, s));
  }
  TiledParams p{w->codes, w->scales, w->shapes, M, w->N, w->K, w->group, xa, xs, y, yb};
  if (use_skinny) return hip_status(launch_skinny_a16(p, w->bits, s));
  if (use_passes) {
    for (int64_t r0 = 0; r0 < M; r0 += kSkinnyRows) {
      TiledParams q = p;
      q.M = std::min(kSkinnyRows, M - r0);
      q.xa = xa + r0 * w->K;
      q.xs = xs ? xs + r0 : nullptr;
      q.y = ybf16 ? reinterpret_cast<float*>(reinterpret_cast<uint16_t*>(y) + r0 * w->N) : y + r0 * w->N;
      const hipError_t e = launch_skinny_a16(q, w->bits, s);
      if (e != hipSuccess) return hip_status(e);
    }
    return CUBIC_OK;
  }
  if (M >= kPrefillMinM && prefill_supported(M, w->N, w->K, w->bits, w->group))
    return hip_status(launch_prefill_a16(p, w->bits, s));
  return hip_status(launch_tiled_a16(p, w->bits, s));
}

int act_quant_impl(const uint16_t* x, bool xf16, int64_t M, int64_t K, int8_t* xq, float* x_scale,
                   cubic_stream_t stream) {
  if (M < 0 || K < 0 || K % 8 != 0) return CUBIC_ERR_SHAPE;
  if (M == 0) return CUBIC_OK;
  if (!x || !xq || !x_scale) return CUBIC_ERR_NULL;
  if (!aligned16(x) || !aligned16(xq) || !aligned16(x_scale)) return CUBIC_ERR_ALIGN;
  if (M > INT32_MAX) return CUBIC_ERR_SHAPE;
  return hip_status(launch_act_quant(x, xf16, M, K, xq, x_scale, static_cast<hipStream_t>(stream)));
}

int gemm_a8_impl(const int8_t* xq, const float* x_scale, int64_t M, const cubic_weight* w, float* y,
                 bool ybf16, cubic_stream_t stream) {
  const int st = check_weight(w);
  if (st != CUBIC_OK) return st;
  if (w->group > 1024) return CUBIC_ERR_GROUP;
  if (M < 0) return CUBIC_ERR_SHAPE;
  if (M == 0 || w->N == 0) return CUBIC_OK;
  if (!xq || !x_scale || !y) return CUBIC_ERR_NULL;
  if (!aligned16(xq) || !aligned16(x_scale) || !aligned16(y)) return CUBIC_ERR_ALIGN;
  if ((M + 127) / 128 > 65535) return CUBIC_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (w->K == 0) return hip_status(launch_fill_zero(y, M * w->N, ybf16, s));
  if (M <= gemv_a8_max_m(w->bits) && moe_a8_supported(w->K, w->bits, w->group) &&
      cubic_code_bytes(w->N, w->K, w->bits) <= UINT32_MAX) {
    // small M: the routed A8 kernel's organisation on one weight, no routing,
    // in passes of 16 rows
    MoeA8Params q{};
    q.codes = w->codes;
    q.scales = w->scales;
    q.shapes = w->shapes;
    q.N = w->N;
    q.K = w->K;
    q.group = w->group;
    q.topk = 1;
    q.code_bytes = static_cast<int64_t>(cubic_code_bytes(w->N, w->K, w->bits));
    q.xq = xq;
    q.xs = x_scale;
    q.y = y;
    q.ybf16 = ybf16 ? 1 : 0;
    q.dense_m = static_cast<int>(M);
    return hip_status(launch_gemv_a8(q, w->bits, s));
  }
  TiledParams p{w->codes, w->scales, w->shapes, M, w->N, w->K, w->group, xq, x_scale, y, ybf16 ? 1 : 0};
  if (prefill_a8_supported(M, w->N, w->K, w->bits, w->group)) return hip_status(launch_prefill_a8(p, w->bits, s));
  return hip_status(launch_tiled_a8(p, w->bits, s));
}
}  // namespace

CUBIC_API int cubic_gemm_a16(const uint16_t* x_bf16, int64_t M, const cubic_weight* w, float* y,
                             void* workspace, size_t ws_bytes, cubic_stream_t stream) {
  return gemm_a16_impl(x_bf16, false, M, w, y, false, workspace, ws_bytes, stream);
}

CUBIC_API int cubic_gemm_a16_ex(const void* x, int x_dtype, int64_t M, const cubic_weight* w, void* y,
                                int y_dtype, void* workspace, size_t ws_bytes, cubic_stream_t stream) {
  if (!dtype_in_ok(x_dtype) || !dtype_out_ok(y_dtype)) return CUBIC_ERR_DTYPE;
  return gemm_a16_impl(static_cast<const uint16_t*>(x), x_dtype == CUBIC_DTYPE_F16, M, w, static_cast<float*>(y),
                       y_dtype == CUBIC_DTYPE_BF16, workspace, ws_bytes, stream);
}

CUBIC_API int act_quant_int8_per_token(const uint16_t* x_bf16, int64_t M, int64_t K, int8_t* xq,
                                       float* x_scale, cubic_stream_t stream) {
  return act_quant_impl(x_bf16, false, M, K, xq, x_scale, stream);
}

CUBIC_API int act_quant_int8_per_token_ex(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* xq,
                                          float* x_scale, cubic_stream_t stream) {
  if (!dtype_in_ok(x_dtype)) return CUBIC_ERR_DTYPE;
  return act_quant_impl(static_cast<const uint16_t*>(x), x_dtype == CUBIC_DTYPE_F16, M, K, xq, x_scale, stream);
}

CUBIC_API int cubic_gemm_a8(const int8_t* xq, const float* x_scale, int64_t M,
                            const cubic_weight* w, float* y, cubic_stream_t stream) {
  return gemm_a8_impl(xq, x_scale, M, w, y, false, stream);
}

CUBIC_API int cubic_gemm_a8_ex(const int8_t* xq, const float* x_scale, int64_t M, const cubic_weight* w,
                               void* y, int y_dtype, cubic_stream_t stream) {
  if (!dtype_out_ok(y_dtype)) return CUBIC_ERR_DTYPE;
  return gemm_a8_impl(xq, x_scale, M, w, static_cast<float*>(y), y_dtype == CUBIC_DTYPE_BF16, stream);
}

// The measured A16/A8 crossover of 2- and 3-bit codes on the expert shapes: A8
// from 128 rows (its tile kernel), and in the 8..16-row window for long rows
// (K >= 4096), where one 16-row A8 pass streams the weight once against the
// A16 GEMV's one MFMA tile.
constexpr int64_t kLinearA8MinM = 128;
constexpr int64_t kLinearA8WindowLo = 8, kLinearA8WindowHi = 16, kLinearA8WindowMinK = 4096;

CUBIC_API int cubic_linear_mode(int64_t M, int64_t N, int64_t K, int bits, int group) {
  if (!(bits == 2 || bits == 3) || N <= 0 || K <= 0 || group <= 0) return CUBIC_MODE_A16;
  if (M >= kLinearA8MinM && prefill_a8_supported(M, N, K, bits, group)) return CUBIC_MODE_A8;
  if (M >= kLinearA8WindowLo && M <= kLinearA8WindowHi && K >= kLinearA8WindowMinK &&
      moe_a8_supported(K, bits, group) && cubic_code_bytes(N, K, bits) <= UINT32_MAX)
    return CUBIC_MODE_A8;
  return CUBIC_MODE_A16;
}

CUBIC_API size_t cubic_linear_workspace_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K < 0) return 0;
  const size_t a8 = align256(static_cast<size_t>(M) * K) + align256(static_cast<size_t>(M) * 4);
  const size_t a16 = cubic_gemm_a16_workspace_bytes(M, K);
  return a8 > a16 ? a8 : a16;
}

CUBIC_API int cubic_linear(const uint16_t* x_bf16, int64_t M, const cubic_weight* w, float* y,
                           void* workspace, size_t ws_bytes, cubic_stream_t stream) {
  const int st = check_weight(w);
  if (st != CUBIC_OK) return st;
  if (M < 0) return CUBIC_ERR_SHAPE;
  if (cubic_linear_mode(M, w->N, w->K, w->bits, w->group) == CUBIC_MODE_A16)
    return cubic_gemm_a16(x_bf16, M, w, y, workspace, ws_bytes, stream);
  if (!x_bf16 || !y) return CUBIC_ERR_NULL;
  if (!aligned16(x_bf16) || !aligned16(y)) return CUBIC_ERR_ALIGN;
  const size_t xq_bytes = align256(static_cast<size_t>(M) * w->K);
  if (!workspace || ws_bytes < xq_bytes + align256(static_cast<size_t>(M) * 4)) return CUBIC_ERR_WORKSPACE;
  if (!aligned16(workspace)) return CUBIC_ERR_ALIGN;
  int8_t* xq = static_cast<int8_t*>(workspace);
  float* xs = reinterpret_cast<float*>(static_cast<char*>(workspace) + xq_bytes);
  const int q = act_quant_int8_per_token(x_bf16, M, w->K, xq, xs, stream);
  if (q != CUBIC_OK) return q;
  return cubic_gemm_a8(xq, xs, M, w, y, stream);
}

namespace {
struct MoeLayout {
  size_t hdr, erec, sorted, total;
};
MoeLayout moe_layout(int64_t T, int topk, int E) {
  MoeLayout L;
  const size_t P = static_cast<size_t>(T) * topk;
  size_t o = 0;
  L.hdr = o;     o += align256(16);
  L.erec = o;    o += align256(32 * static_cast<size_t>(E));
  L.sorted = o;  o += align256(4 * P);
  L.total = o;
  return L;
}
}  // namespace

namespace {
struct MlpLayout {
  MoeLayout route;
  size_t y1, h, y2, total;
};
MlpLayout mlp_layout(int64_t T, int topk, int E, int64_t H, int64_t I) {
  MlpLayout L;
  L.route = moe_layout(T, topk, E);
  const size_t P = static_cast<size_t>(T) * topk;
  size_t o = L.route.total;
  L.y1 = o;  o += align256(P * static_cast<size_t>(2 * I) * 4);
  L.h = o;   o += align256(P * static_cast<size_t>(I) * 2);
  L.y2 = o;  o += align256(P * static_cast<size_t>(H) * 4);
  L.total = o;
  return L;
}

int moe_weight_fits(const cubic_weight* w) {
  if (w->K > 0 && (!gemv_supported(w->K, w->bits, w->group) ||
                   moe_lds_min_bytes(w->K, w->bits, w->group) > kLdsLimit))
    return CUBIC_ERR_SHAPE;
  return CUBIC_OK;
}
}  // namespace

CUBIC_API size_t cubic_moe_mlp_workspace_bytes(int64_t T, int topk, int E, int64_t H, int64_t I) {
  if (T < 0 || topk <= 0 || E <= 0 || H < 0 || I < 0) return 0;
  return mlp_layout(T, topk, E, H, I).total;
}

CUBIC_API int cubic_moe_mlp(const uint16_t* x_bf16, int64_t T, const int32_t* topk_ids,
                            const float* topk_weights, int topk, const cubic_weight* gate_up0,
                            const cubic_weight* down0, int E, float* y, void* workspace, size_t ws_bytes,
                            cubic_stream_t stream) {
  int st = check_weight(gate_up0);
  if (st != CUBIC_OK) return st;
  st = check_weight(down0);
  if (st != CUBIC_OK) return st;
  if (T < 0 || topk <= 0 || E <= 0) return CUBIC_ERR_SHAPE;
  const int64_t H = gate_up0->K, I = down0->K;
  if (gate_up0->N != 2 * I || down0->N != H || H == 0 || I == 0) return CUBIC_ERR_SHAPE;
  if (T == 0) return CUBIC_OK;
  if (T * topk > INT32_MAX / 2) return CUBIC_ERR_SHAPE;
  if ((st = moe_weight_fits(gate_up0)) != CUBIC_OK || (st = moe_weight_fits(down0)) != CUBIC_OK) return st;
  if (!x_bf16 || !topk_ids || !topk_weights || !y || !workspace) return CUBIC_ERR_NULL;
  if (!aligned16(x_bf16) || !aligned16(topk_ids) || !aligned16(topk_weights) || !aligned16(y) ||
      !aligned16(workspace))
    return CUBIC_ERR_ALIGN;
  const MlpLayout L = mlp_layout(T, topk, E, H, I);
  if (ws_bytes < L.total) return CUBIC_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  auto params = [&](const cubic_weight* w, const uint16_t* x, float* out) {
    MoeGemvParams p{};
    p.codes = w->codes;
    p.scales = w->scales;
    p.shapes = w->shapes;
    p.N = w->N;
    p.K = w->K;
    p.group = w->group;
    p.topk = topk;
    p.code_bytes = static_cast<int64_t>(cubic_code_bytes(w->N, w->K, w->bits));
    p.x = x;
    p.y = out;
    return p;
  };
  float* y1 = reinterpret_cast<float*>(ws + L.y1);
  float* y2 = reinterpret_cast<float*>(ws + L.y2);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + L.h);
  const hipError_t e = launch_moe_mlp(
      topk_ids, topk_weights, static_cast<int>(T), E, topk, params(gate_up0, x_bf16, y1), gate_up0->bits,
      params(down0, h, y2), down0->bits, reinterpret_cast<int32_t*>(ws + L.route.hdr),
      reinterpret_cast<int32_t*>(ws + L.route.erec), reinterpret_cast<int32_t*>(ws + L.route.sorted), h, y,
      static_cast<hipStream_t>(stream));
  return hip_status(e);
}

namespace {
struct MlpA8Layout {
  MoeLayout route;
  size_t xq, xs, y1, h, hq, hs, y2, total;
};
MlpA8Layout mlp_a8_layout(int64_t T, int topk, int E, int64_t H, int64_t I) {
  MlpA8Layout L;
  L.route = moe_layout(T, topk, E);
  const size_t P = static_cast<size_t>(T) * topk;
  size_t o = L.route.total;
  L.xq = o;  o += align256(static_cast<size_t>(T) * H);
  L.xs = o;  o += align256(static_cast<size_t>(T) * 4);
  L.y1 = o;  o += align256(P * static_cast<size_t>(2 * I) * 4);
  L.h = o;   o += align256(P * static_cast<size_t>(I) * 2);
  L.hq = o;  o += align256(P * static_cast<size_t>(I));
  L.hs = o;  o += align256(P * 4);
  L.y2 = o;  o += align256(P * static_cast<size_t>(H) * 4);
  L.total = o;
  return L;
}
}  // namespace

CUBIC_API size_t cubic_moe_mlp_a8_workspace_bytes(int64_t T, int topk, int E, int64_t H, int64_t I) {
  if (T < 0 || topk <= 0 || E <= 0 || H < 0 || I < 0) return 0;
  return mlp_a8_layout(T, topk, E, H, I).total;
}

CUBIC_API int cubic_moe_mlp_a8(const uint16_t* x_bf16, int64_t T, const int32_t* topk_ids,
                               const float* topk_weights, int topk, const cubic_weight* gate_up0,
                               const cubic_weight* down0, int E, float* y, void* workspace, size_t ws_bytes,
                               cubic_stream_t stream) {
  int st = check_weight(gate_up0);
  if (st != CUBIC_OK) return st;
  st = check_weight(down0);
  if (st != CUBIC_OK) return st;
  if (gate_up0->group > 1024 || down0->group > 1024) return CUBIC_ERR_GROUP;
  if (T < 0 || topk <= 0 || E <= 0) return CUBIC_ERR_SHAPE;
  const int64_t H = gate_up0->K, I = down0->K;
  if (gate_up0->N != 2 * I || down0->N != H || H == 0 || I == 0) return CUBIC_ERR_SHAPE;
  if (T == 0) return CUBIC_OK;
  if (T * topk > INT32_MAX / 2) return CUBIC_ERR_SHAPE;
  for (const cubic_weight* w : {gate_up0, down0})
    if (!moe_a8_supported(w->K, w->bits, w->group) || cubic_code_bytes(w->N, w->K, w->bits) > UINT32_MAX)
      return CUBIC_ERR_SHAPE;
  if (!x_bf16 || !topk_ids || !topk_weights || !y || !workspace) return CUBIC_ERR_NULL;
  if (!aligned16(x_bf16) || !aligned16(topk_ids) || !aligned16(topk_weights) || !aligned16(y) ||
      !aligned16(workspace))
    return CUBIC_ERR_ALIGN;
  const MlpA8Layout L = mlp_a8_layout(T, topk, E, H, I);
  if (ws_bytes < L.total) return CUBIC_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  auto params = [&](const cubic_weight* w) {
    MoeA8Params p{};
    p.codes = w->codes;
    p.scales = w->scales;
    p.shapes = w->shapes;
    p.N = w->N;
    p.K = w->K;
    p.group = w->group;
    p.topk = topk;
    p.code_bytes = static_cast<int64_t>(cubic_code_bytes(w->N, w->K, w->bits));
    return p;
  };
  MoeMlpA8Buffers b;
  b.xq = reinterpret_cast<int8_t*>(ws + L.xq);
  b.xs = reinterpret_cast<float*>(ws + L.xs);
  b.y1 = reinterpret_cast<float*>(ws + L.y1);
  b.h = reinterpret_cast<uint16_t*>(ws + L.h);
  b.hq = reinterpret_cast<int8_t*>(ws + L.hq);
  b.hs = reinterpret_cast<float*>(ws + L.hs);
  b.y2 = reinterpret_cast<float*>(ws + L.y2);
  const hipError_t e = launch_moe_mlp_a8(
      x_bf16, topk_ids, topk_weights, static_cast<int>(T), E, topk, params(gate_up0), gate_up0->bits,
      params(down0), down0->bits, reinterpret_cast<int32_t*>(ws + L.route.hdr),
      reinterpret_cast<int32_t*>(ws + L.route.erec), reinterpret_cast<int32_t*>(ws + L.route.sorted), b, y,
      static_cast<hipStream_t>(stream));
  return hip_status(e);
}

CUBIC_API size_t cubic_moe_workspace_bytes(int64_t T, int topk, int E) {
  if (T < 0 || topk <= 0 || E <= 0) return 0;
  return moe_layout(T, topk, E).total;
}

namespace {
// The grouped product behind both routed-expert entry points; `workspace` is
// the caller's buffer or the library's routing scratch (nullptr: look it up
// after validation, so a rejected call touches no device state).
int moe_grouped(const uint16_t* x_bf16, bool xf16, int64_t T, const int32_t* topk_ids, int topk,
                const cubic_weight* expert0, int E, float* y, bool ybf16, void* workspace, size_t ws_bytes,
                bool library_scratch, cubic_stream_t stream) {
  const int st = check_weight(expert0);
  if (st != CUBIC_OK) return st;
  if (T < 0 || topk <= 0 || E <= 0) return CUBIC_ERR_SHAPE;
  if (T == 0 || expert0->N == 0) return CUBIC_OK;
  if (T * topk > INT32_MAX / 2) return CUBIC_ERR_SHAPE;
  if (expert0->K > 0 && (!gemv_supported(expert0->K, expert0->bits, expert0->group) ||
                         moe_lds_min_bytes(expert0->K, expert0->bits, expert0->group) > kLdsLimit))
    return CUBIC_ERR_SHAPE;
  if (!x_bf16 || !topk_ids || !y || (!workspace && !library_scratch)) return CUBIC_ERR_NULL;
  if (!aligned16(x_bf16) || !aligned16(topk_ids) || !aligned16(y) || !aligned16(workspace))
    return CUBIC_ERR_ALIGN;
  const MoeLayout L = moe_layout(T, topk, E);
  if (ws_bytes < L.total) return CUBIC_ERR_WORKSPACE;
  if (library_scratch) {
    const hipError_t a = moe_scratch_address(&workspace);
    if (a != hipSuccess) return CUBIC_ERR_HIP;
  }
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (expert0->K == 0) return hip_status(launch_fill_zero(y, T * topk * expert0->N, ybf16, s));
  MoeGemvParams p{};
  p.codes = expert0->codes;
  p.scales = expert0->scales;
  p.shapes = expert0->shapes;
  p.N = expert0->N;
  p.K = expert0->K;
  p.group = expert0->group;
  p.topk = topk;
  p.code_bytes = static_cast<int64_t>(cubic_code_bytes(expert0->N, expert0->K, expert0->bits));
  p.x = x_bf16;
  p.y = y;
  p.ybf16 = ybf16 ? 1 : 0;
  const hipError_t e = launch_moe(topk_ids, static_cast<int>(T), E, topk, p,
                                  reinterpret_cast<int32_t*>(ws + L.hdr),
                                  reinterpret_cast<int32_t*>(ws + L.erec),
                                  reinterpret_cast<int32_t*>(ws + L.sorted), expert0->bits, xf16, s);
  return hip_status(e);
}
}  // namespace

CUBIC_API int cubic_moe_grouped_gemm(const uint16_t* x_bf16, int64_t T, const int32_t* topk_ids,
                                     int topk, const cubic_weight* expert0, int E, float* y,
                                     void* workspace, size_t ws_bytes, cubic_stream_t stream) {
  return moe_grouped(x_bf16, false, T, topk_ids, topk, expert0, E, y, false, workspace, ws_bytes, false, stream);
}

CUBIC_API int cubic_moe_grouped_gemm_ex(const void* x, int x_dtype, int64_t T, const int32_t* topk_ids,
                                        int topk, const cubic_weight* expert0, int E, void* y, int y_dtype,
                                        void* workspace, size_t ws_bytes, cubic_stream_t stream) {
  if (!dtype_in_ok(x_dtype) || !dtype_out_ok(y_dtype)) return CUBIC_ERR_DTYPE;
  return moe_grouped(static_cast<const uint16_t*>(x), x_dtype == CUBIC_DTYPE_F16, T, topk_ids, topk, expert0, E,
                     static_cast<float*>(y), y_dtype == CUBIC_DTYPE_BF16, workspace, ws_bytes, false, stream);
}

CUBIC_API int cubic_moe_grouped_gemm_a8(const int8_t* xq, const float* x_scale, int64_t T,
                                        const int32_t* topk_ids, int topk, const cubic_weight* expert0, int E,
                                        void* y, int y_dtype, void* workspace, size_t ws_bytes,
                                        cubic_stream_t stream) {
  if (!dtype_out_ok(y_dtype)) return CUBIC_ERR_DTYPE;
  const int st = check_weight(expert0);
  if (st != CUBIC_OK) return st;
  if (expert0->group > 1024) return CUBIC_ERR_GROUP;
  if (T < 0 || topk <= 0 || E <= 0) return CUBIC_ERR_SHAPE;
  if (T == 0 || expert0->N == 0) return CUBIC_OK;
  if (T * topk > INT32_MAX / 2) return CUBIC_ERR_SHAPE;
  if (!moe_a8_supported(expert0->K, expert0->bits, expert0->group)) return CUBIC_ERR_SHAPE;
  if (cubic_code_bytes(expert0->N, expert0->K, expert0->bits) > UINT32_MAX) return CUBIC_ERR_SHAPE;
  if (!xq || !x_scale || !topk_ids || !y || !workspace) return CUBIC_ERR_NULL;
  if (!aligned16(xq) || !aligned16(x_scale) || !aligned16(topk_ids) || !aligned16(y) || !aligned16(workspace))
    return CUBIC_ERR_ALIGN;
  const MoeLayout L = moe_layout(T, topk, E);
  if (ws_bytes < L.total) return CUBIC_ERR_WORKSPACE;
  const bool ybf16 = y_dtype == CUBIC_DTYPE_BF16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (expert0->K == 0) return hip_status(launch_fill_zero(static_cast<float*>(y), T * topk * expert0->N, ybf16, s));
  char* ws = static_cast<char*>(workspace);
  MoeA8Params p{};
  p.codes = expert0->codes;
  p.scales = expert0->scales;
  p.shapes = expert0->shapes;
  p.N = expert0->N;
  p.K = expert0->K;
  p.group = expert0->group;
  p.topk = topk;
  p.code_bytes = static_cast<int64_t>(cubic_code_bytes(expert0->N, expert0->K, expert0->bits));
  p.xq = xq;
  p.xs = x_scale;
  p.y = static_cast<float*>(y);
  p.ybf16 = ybf16 ? 1 : 0;
  return hip_status(launch_moe_a8(topk_ids, static_cast<int>(T), E, topk, p,
                                  reinterpret_cast<int32_t*>(ws + L.hdr), reinterpret_cast<int32_t*>(ws + L.erec),
                                  reinterpret_cast<int32_t*>(ws + L.sorted), expert0->bits, s));
}

CUBIC_API size_t cubic_moe_grouped_gemm_static_max_bytes(void) { return moe_scratch_bytes(); }

CUBIC_API int cubic_moe_grouped_gemm_static(const uint16_t* x_bf16, int64_t T, const int32_t* topk_ids,
                                            int topk, const cubic_weight* expert0, int E, float* y,
                                            cubic_stream_t stream) {
  return moe_grouped(x_bf16, false, T, topk_ids, topk, expert0, E, y, false, nullptr, moe_scratch_bytes(), true,
                     stream);
}
