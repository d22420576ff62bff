/* cubic.h -- C ABI of libcubic.so: CubicQuant weight-only dequant-GEMM for AMD
 * Instinct MI355X (gfx950).
 *
 * Method: the CubicQuant article on ModelScope ("CubicQuant：用三次曲线重塑低比特量化，
 * Kimi K3 2.5Bit 模型首发实践"). Each weight is a B-bit signed integer code k; per
 * group of G weights the format stores one fp32 scale s and two fp16 shape
 * parameters a, b (section "存储开销是透明的：B+64/G bit", so B + 64/G bits per
 * weight). With Kmax = 2^(B-1) - 1 and t = |k| / Kmax the weight is
 *     w = s * sign(k) * q(t),   q(t) = a t + b t^2 + (1 - a - b) t^3
 * (section "CubicQuant 核心：把直线网格掰弯"; its equations did not survive text
 * extraction and this is the reading the library implements). A16 multiplies
 * bf16 activations with these continuous levels; Dynamic A8 quantises each
 * activation row to INT8 at run time and multiplies it with an INT8 carrier of
 * the levels, scaling each group in fp32 (section "一份 checkpoint，同时服务 A16 与
 * Dynamic A8"). Decoding happens tile-locally inside the product kernels and no
 * full-precision weight matrix is ever written (section "压缩权重必须边解码、边计算").
 *
 * General contract
 *  - Every array argument is a DEVICE pointer owned by the caller. The library
 *    never allocates or frees device memory; scratch space is passed in as
 *    `workspace` where a call needs it. The one exception is the routing
 *    scratch of cubic_moe_grouped_gemm_static: a fixed 2 MiB buffer that the
 *    library holds on each device it runs on, for callers that cannot allocate.
 *  - Calls validate all arguments on the host first. On a validation error
 *    nothing is enqueued and nothing is written; the error code is returned.
 *  - Valid calls enqueue kernels on `stream` (a hipStream_t; NULL = the null
 *    stream) and return without waiting, except cubic_pack (see there).
 *  - Launch failures are reported as CUBIC_ERR_HIP.
 *  - Outputs must not alias inputs. Non-finite inputs propagate unchecked.
 *  - Every pointer must be 16-byte aligned.
 *
 * Weight layout (struct cubic_weight)
 *  - codes : uint8 [N][K*bits/8]. One LSB-first bit stream over the row-major
 *            [N][K] code matrix; each code is a `bits`-wide two's complement
 *            field. Rows are byte-aligned (K*bits is a multiple of 8).
 *  - scales: fp32 [N][K/group]: s of group g = k / group of row n.
 *  - shapes: fp16 bit patterns [N][K/group][2]: a, then b.
 *  - bits in [2, 8]; group a multiple of 128; K a multiple of group.
 *    Codes are expected in [-Kmax, Kmax]; the extra field value -2^(B-1)
 *    decodes by the same formula (t > 1).
 */
#ifndef CUBIC_H
#define CUBIC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* cubic_stream_t;

enum {
  CUBIC_OK = 0,
  CUBIC_ERR_NULL = -1,        /* a required pointer is NULL                    */
  CUBIC_ERR_SHAPE = -2,       /* negative size, or K/N/M not as required       */
  CUBIC_ERR_BITS = -3,        /* bits outside [2, 8]                           */
  CUBIC_ERR_GROUP = -4,       /* group not a multiple of 128, or K % group     */
  CUBIC_ERR_ALIGN = -5,       /* a pointer is not 16-byte aligned              */
  CUBIC_ERR_CODE_RANGE = -6,  /* cubic_pack found a code with |k| > Kmax       */
  CUBIC_ERR_WORKSPACE = -7,   /* workspace missing or smaller than required    */
  CUBIC_ERR_HIP = -8,         /* a HIP runtime call or a launch failed         */
  CUBIC_ERR_DTYPE = -9        /* an activation or output dtype not supported   */
};

/* Element types of the _ex entry points' activations and outputs (CubicQuant
 * article, section "一份 checkpoint，同时服务 A16 与 Dynamic A8": activations in
 * FP16 or BF16; flow figure of section "压缩权重必须边解码、边计算": results
 * leave the kernel in the model's dtype). */
enum {
  CUBIC_DTYPE_F32 = 0,        /* fp32 (outputs)                                */
  CUBIC_DTYPE_BF16 = 1,       /* bf16 bit patterns (activations, outputs)      */
  CUBIC_DTYPE_F16 = 2         /* fp16 bit patterns (activations)               */
};

typedef struct cubic_weight {
  const uint8_t* codes;
  const float* scales;
  const uint16_t* shapes;
  int64_t N, K;
  int32_t bits, group;
} cubic_weight;

/* Size helpers (host only, no GPU needed). Storage section of the CubicQuant
 * article: B bits per weight plus 64 bits per group. Return 0 for invalid args. */
size_t cubic_code_bytes(int64_t N, int64_t K, int bits);
size_t cubic_storage_bytes(int64_t N, int64_t K, int bits, int group);
const char* cubic_status_string(int status);
/* Library version string, e.g. "cubic 0.1 gfx950". */
const char* cubic_version(void);

/* Pack int8 codes [N][K] into the bit stream packed[N][K*bits/8] (CubicQuant
 * article, Storage section: the codes are plain B-bit integers stored densely,
 * B bits per weight; the LSB-first two's complement layout is this library's
 * reading). K must be a multiple of 32. Codes with |k| > Kmax are written as their
 * low `bits` bits AND make the call return CUBIC_ERR_CODE_RANGE: to report
 * that, this call waits for its own kernel (one stream synchronisation).
 * Calls on one device are serialised by a host lock around that check. */
int cubic_pack(const int8_t* codes, int64_t N, int64_t K, int bits,
               uint8_t* packed, cubic_stream_t stream);

/* Unpack the bit stream into int8 codes [N][K] (sign-extended fields, including
 * -2^(B-1)); the inverse of cubic_pack (CubicQuant article, Storage section).
 * K must be a multiple of 32. Bit-exact. */
int cubic_unpack(const uint8_t* packed, int64_t N, int64_t K, int bits,
                 int8_t* codes, cubic_stream_t stream);

/* Materialise the decoded weights out[N][K] in fp32 (a test and inspection
 * utility; the GEMMs never call it). CubicQuant article, Core section (the
 * reconstructed weight) and Storage section (s kept in fp32): each value is
 * RN32(s * sign(k) * q(|k| / Kmax)), the exact real value rounded once to the
 * nearest fp32 number, ties to even, for every finite s and fp16 a, b. A zero
 * weight is +0.0 (code 0 always); codes +-Kmax give +-s exactly. */
int cubic_dequant(const cubic_weight* w, float* out, cubic_stream_t stream);

/* Nearest-level encoding (CubicQuant article, Core section: each weight takes
 * the code of its group's nearest reconstruction level), for given scales and
 * shapes. w: fp32 [N][K]; scales, shapes as in cubic_weight; codes: int8 [N][K]
 * out, in [-Kmax, Kmax] (pack them with cubic_pack). The levels are the
 * format's fp32 values L_k = RN32(s * sign(k) * q(|k| / Kmax)), exactly those
 * cubic_dequant returns, and distances |w - L_k| are compared exactly: the code
 * is the k of smallest distance, the smaller |k| on ties (so 0 for a zero
 * weight of either sign); the code -2^(B-1) is never chosen. NaN weights take
 * code 0. Codes are bit-exact whatever the arithmetic order. Errors as for the
 * other calls (bits, group, alignment, NULL); N == 0 or K == 0 is a no-op. */
int cubic_encode(const float* w, int64_t N, int64_t K, int bits, int group,
                 const float* scales, const uint16_t* shapes, int8_t* codes,
                 cubic_stream_t stream);

/* Data-free group fitting (CubicQuant article, data-free in-group fitting: per
 * group a search over monotone (a, b), the scale chosen with its soft-clip
 * threshold, nearest-level codes, a and b kept in fp16 and s in fp32). The
 * article leaves the grid and the loss open; this call searches
 *   a = i/8 (i = 0..24) x b = j/8 (j = -24..24), pairs for which
 *       q(t) = a t + b t^2 + (1-a-b) t^3 is non-decreasing on [0, 1] (532 pairs),
 *   s = fl32(rho * max|w|) with rho = 1 - r/32, r = 0..15 (weights beyond s take
 *       the top level),
 * minimising the group's sum of squared distances from |w| to its nearest fp32
 * level RN32(s * q_j) (the levels of cubic_dequant; fp32 sums in weight order). Candidate index = pair * 16 + r, pairs
 * in the order above; the first smallest loss wins. codes follow cubic_encode's
 * rule for the chosen s, a, b, so cubic_pack of them with scales/shapes is the
 * fitted weight. w fp32 [N][K] (finite), codes int8 [N][K], scales fp32 [N][K/group],
 * shapes fp16 pairs [N][K/group][2], loss fp32 [N][K/group] or NULL. group a
 * multiple of 128 up to 2048. A group of zeros gets s = 0, (a, b) = (0, 0), codes 0.
 * Asynchronous on `stream`. */
int cubic_fit(const float* w, int64_t N, int64_t K, int bits, int group, int8_t* codes,
              float* scales, uint16_t* shapes, float* loss, cubic_stream_t stream);

/* A16 product y[M][N] = x[M][K] * W^T, x in bf16 (bit patterns), y in fp32
 * (CubicQuant article, section "一份 checkpoint，同时服务 A16 与 Dynamic A8": A16
 * multiplies FP16/BF16 activations with the continuous levels; section
 * "压缩权重必须边解码、边计算": the codes are decoded inside the product's tiles,
 * scaled per group in FP32, and no dequantised matrix is written).
 * For 2-bit weights x is used in bf16 as is (the valid levels are -s, 0, s, so
 * every product is exact before the fp32 group scaling). For wider codes and
 * 5 <= M <= 16, x is also used as is, against levels held as two bf16 halves
 * (hi + lo, about 16 significant bits). Otherwise, for wider codes, x is
 * converted to fp16 after scaling each row by a power of two so that its
 * largest magnitude sits just below 2^15 (exact unless elements drop below
 * fp16's normal range), and levels are fp16. Accumulation is fp32 throughout.
 * Rows with M <= 4 take a single-kernel path that needs no workspace; larger M
 * may first write reordered or converted activations into `workspace` (the
 * 5..16-row paths of wider codes do not touch it).
 * cubic_gemm_a16_workspace_bytes(M, K) gives the required size (0 when none is
 * needed); `workspace` may be NULL when that size is 0. M == 0 is a no-op. */
size_t cubic_gemm_a16_workspace_bytes(int64_t M, int64_t K);
int cubic_gemm_a16(const uint16_t* x_bf16, int64_t M, const cubic_weight* w,
                   float* y, void* workspace, size_t ws_bytes, cubic_stream_t stream);

/* cubic_gemm_a16 with the activation and output types chosen: x_dtype
 * CUBIC_DTYPE_BF16 or CUBIC_DTYPE_F16 (bit patterns [M][K]); y_dtype
 * CUBIC_DTYPE_F32 or CUBIC_DTYPE_BF16 ([M][N]). fp16 activations are used as
 * they are: 2-bit codes multiply them on the fp16 MFMA (every product exact),
 * wider codes against fp16 levels, with no prescale (an fp16 row already fits).
 * A bf16 output is the fp32 result rounded to nearest even in the kernel's
 * epilogue (NaN stays NaN). Other arguments, workspace sizes and errors as for
 * cubic_gemm_a16; CUBIC_ERR_DTYPE for other dtypes. */
int cubic_gemm_a16_ex(const void* x, int x_dtype, int64_t M, const cubic_weight* w,
                      void* y, int y_dtype, void* workspace, size_t ws_bytes,
                      cubic_stream_t stream);

/* Dynamic per-token INT8 quantisation (msModelSlim article on Kimi K3 INT
 * quantisation, routed-expert W4A8 scheme; CubicQuant article, A16/A8 section):
 * for each row m, amax = max |x[m][:]|, x_scale[m] = fp32(amax / 127) (IEEE
 * division), xq[m][k] = clamp(rint(fp32(x[m][k] / x_scale[m])), -127, 127) with
 * ties to even. An all-zero row gives x_scale = 0 and xq = 0. Bit-exact. */
int act_quant_int8_per_token(const uint16_t* x_bf16, int64_t M, int64_t K,
                             int8_t* xq, float* x_scale, cubic_stream_t stream);
/* The same for x_dtype CUBIC_DTYPE_BF16 or CUBIC_DTYPE_F16 (every fp16 value is
 * exact in fp32, so the rule above applies unchanged). */
int act_quant_int8_per_token_ex(const void* x, int x_dtype, int64_t M, int64_t K,
                                int8_t* xq, float* x_scale, cubic_stream_t stream);

/* Dynamic A8 product y[M][N] (fp32) from xq/x_scale of act_quant_int8_per_token
 * (CubicQuant article, section "一份 checkpoint，同时服务 A16 与 Dynamic A8": the
 * levels map to a deterministic INT8 carrier, the product is an integer dot per
 * group, scaled per group in FP32; the carrier's formula did not survive text
 * extraction and the one below is this library's reading). Each code maps to the INT8 carrier C = sign(k) * clamp(rne(127 * q(|k|/Kmax)),
 * -127, 127) (computed exactly with integer arithmetic); per group the exact
 * int32 dot I = sum xq * C is scaled by fp32(s / 127) and accumulated in fp32;
 * the row result is multiplied by x_scale[m]. group must be <= 1024 so that I
 * stays below 2^24. M == 0 is a no-op. */
int cubic_gemm_a8(const int8_t* xq, const float* x_scale, int64_t M,
                  const cubic_weight* w, float* y, cubic_stream_t stream);
/* cubic_gemm_a8 with y_dtype CUBIC_DTYPE_F32 or CUBIC_DTYPE_BF16 (the fp32
 * result rounded to nearest even in the epilogue). */
int cubic_gemm_a8_ex(const int8_t* xq, const float* x_scale, int64_t M,
                     const cubic_weight* w, void* y, int y_dtype, cubic_stream_t stream);

/* Shape dispatcher between the two activation modes (CubicQuant article, A16/A8
 * section and its kernel comparison: A16 serves decode-sized batches best, the
 * integer path once each decoded weight serves enough rows). The rule is
 * static and comes from the A16-vs-A8 sweep of this library on MI355X:
 * Dynamic A8 for 2- and 3-bit codes with M >= 128 (where its tile kernel
 * runs) or with 8 <= M <= 16 and K >= 4096 (one 16-row pass of its small-batch
 * kernel), A16 otherwise. The modes differ in numerics (A8 quantises the
 * activations); cubic_linear_mode tells which one a shape takes. It is a host
 * function and needs no device. */
enum { CUBIC_MODE_A16 = 0, CUBIC_MODE_A8 = 1 };
int cubic_linear_mode(int64_t M, int64_t N, int64_t K, int bits, int group);
/* Workspace that cubic_linear needs for any weight with this K: the larger of
 * the A16 workspace and the A8 staging (xq: M*K bytes, then x_scale: 4*M bytes,
 * each rounded up to 256). */
size_t cubic_linear_workspace_bytes(int64_t M, int64_t K);
/* y[M][N] (fp32) by the mode of cubic_linear_mode: cubic_gemm_a16, or
 * act_quant_int8_per_token into the workspace followed by cubic_gemm_a8. The
 * results equal those calls' results bit for bit. Arguments and errors as for
 * cubic_gemm_a16. A workspace of cubic_linear_workspace_bytes(M, K) always
 * suffices; each route checks only what it uses (the A16 route the A16
 * workspace, the A8 route its staging) and returns CUBIC_ERR_WORKSPACE below. */
int cubic_linear(const uint16_t* x_bf16, int64_t M, const cubic_weight* w, float* y,
                 void* workspace, size_t ws_bytes, cubic_stream_t stream);

/* Routed-expert A16 products (Kimi K3 guide, model-card table: a layer routes
 * each token to 16 of its experts; CubicQuant article, section "Kimi-K3-Cubic-
 * 2.5Bit 是怎样得到 2.4986 bit 的？": the routed experts carry the Cubic weights,
 * and the A16/A8 section notes that routing density decides which kernel wins).
 * E experts with identical (N, K, bits, group) lie back to back: expert e's codes start at expert0->codes + e*code_bytes, its
 * scales at expert0->scales + e*N*(K/group), its shapes at expert0->shapes +
 * 2*e*N*(K/group). For every pair (t, j): y[t][j][:] = x[t][:] * W_{topk_ids[t][j]}^T
 * (fp32 out, layout [T][topk][N]). Ids outside [0, E) produce zero rows and are
 * counted; the count is left in the first 4 bytes of the workspace (int32).
 * Grouping by expert happens on the device (no host synchronisation); each
 * touched expert's codes are read from HBM once per launch (an expert picked by
 * more than four tokens takes one pass per up to four of them, the later passes
 * reading its codes from cache). Requires K <= 2^28 and the per-wave activation
 * slice to fit in LDS (CUBIC_ERR_SHAPE otherwise). x_bf16 [T][K] is read directly.
 * The workspace holds a 16-byte header, one 32-byte record per expert and the
 * pair ids grouped by expert (each part 256-byte aligned); its size depends on
 * T, topk and E only. Returns 0 for invalid arguments. */
size_t cubic_moe_workspace_bytes(int64_t T, int topk, int E);
int cubic_moe_grouped_gemm(const uint16_t* x_bf16, int64_t T,
                           const int32_t* topk_ids, int topk,
                           const cubic_weight* expert0, int E,
                           float* y, void* workspace, size_t ws_bytes,
                           cubic_stream_t stream);
/* cubic_moe_grouped_gemm with x_dtype CUBIC_DTYPE_BF16 or CUBIC_DTYPE_F16 and
 * y_dtype CUBIC_DTYPE_F32 or CUBIC_DTYPE_BF16 (as in cubic_gemm_a16_ex; rows of
 * invalid ids are zero in either output type). */
int cubic_moe_grouped_gemm_ex(const void* x, int x_dtype, int64_t T,
                              const int32_t* topk_ids, int topk,
                              const cubic_weight* expert0, int E,
                              void* y, int y_dtype, void* workspace, size_t ws_bytes,
                              cubic_stream_t stream);

/* Routed-expert products in the Dynamic A8 mode (CubicQuant article, section
 * "一份 checkpoint，同时服务 A16 与 Dynamic A8": the same checkpoint serves the
 * integer path; its deployment section switches the routed experts to it). For
 * every pair (t, j) with e = topk_ids[t][j] in [0, E): y[t][j][:] is the
 * cubic_gemm_a8 product of row t of xq [T][K] (int8) and x_scale [T] (fp32),
 * the output of act_quant_int8_per_token, with expert e (same carriers, exact
 * int32 group dots, fp32(s / 127) per group, x_scale[t] last). Experts lie back
 * to back as in cubic_moe_grouped_gemm; invalid ids give zero rows and are
 * counted in the workspace's first int32; the workspace is the one
 * cubic_moe_workspace_bytes(T, topk, E) sizes. y_dtype CUBIC_DTYPE_F32 or
 * CUBIC_DTYPE_BF16, layout [T][topk][N]. group must be <= 1024
 * (CUBIC_ERR_GROUP); K a multiple of 128 whose per-wave activation slice fits
 * in LDS (CUBIC_ERR_SHAPE otherwise). */
int cubic_moe_grouped_gemm_a8(const int8_t* xq, const float* x_scale, int64_t T,
                              const int32_t* topk_ids, int topk,
                              const cubic_weight* expert0, int E,
                              void* y, int y_dtype, void* workspace, size_t ws_bytes,
                              cubic_stream_t stream);

/* cubic_moe_grouped_gemm for callers that cannot allocate device memory: code
 * under HIP graph capture, serving loops and harnesses that forbid hipMalloc.
 * Same arguments, kernels and results (bit for bit) as cubic_moe_grouped_gemm,
 * but the routing scratch (header, per-expert records, pair ids) is a buffer of
 * cubic_moe_grouped_gemm_static_max_bytes() = 2 MiB that the library holds on
 * each device for the life of the process, instead of a workspace argument.
 * The call allocates and frees nothing. Returns CUBIC_ERR_WORKSPACE when
 * cubic_moe_workspace_bytes(T, topk, E) exceeds that maximum (nothing is
 * enqueued then). The routing kernel rewrites everything the product reads, so
 * the buffer needs no clearing between calls. All calls on one device share the
 * buffer: calls that overlap on that device (other streams, or other host
 * threads) race and must be serialised by the caller. The invalid-id count is
 * kept in the library's buffer and is not reported. */
size_t cubic_moe_grouped_gemm_static_max_bytes(void);
int cubic_moe_grouped_gemm_static(const uint16_t* x_bf16, int64_t T,
                                  const int32_t* topk_ids, int topk,
                                  const cubic_weight* expert0, int E,
                                  float* y, cubic_stream_t stream);

/* The routed-expert MLP step of a Kimi-K3-style layer (Kimi K3 guide, model
 * card: routed experts with a fused gate_up and a down projection; CubicQuant
 * article, A16/A8 section: the expert weights are Cubic-coded):
 *   [g | u] = x_t * GU_e^T    (gate_up expert e: N = 2I rows, K = H; gate rows
 *                              0 .. I-1, up rows I .. 2I-1), for every pair (t, j)
 *   h       = bf16(SiLU(g) * u)          (fp32, rounded to bf16, nearest even)
 *   o_tj    = h * D_e^T       (down expert e: N = H rows, K = I)
 *   y[t]    = sum_j topk_weights[t][j] * o_tj   (fp32, slots in order)
 * e = topk_ids[t][j]; pairs with ids outside [0, E) add nothing. Experts of each
 * kind lie back to back as in cubic_moe_grouped_gemm (gate_up0, down0: expert 0).
 * x_bf16 [T][H], topk_ids int32 [T][topk], topk_weights fp32 [T][topk], y fp32
 * [T][H]. One routing feeds both grouped products; the intermediates live in
 * the workspace, whose size cubic_moe_mlp_workspace_bytes gives: first the
 * routing part (cubic_moe_workspace_bytes(T, topk, E) bytes), then the gate_up
 * outputs [T*topk][2I] fp32, h [T*topk][I] bf16 and the down outputs
 * [T*topk][H] fp32, each starting at the next multiple of 256 bytes; they stay
 * there after the call (a pair with an invalid id leaves its rows unspecified). Errors as
 * for cubic_moe_grouped_gemm; CUBIC_ERR_SHAPE when the two weights disagree
 * (gate_up N != 2 * down K or down N != gate_up K). */
size_t cubic_moe_mlp_workspace_bytes(int64_t T, int topk, int E, int64_t H, int64_t I);
int cubic_moe_mlp(const uint16_t* x_bf16, int64_t T, const int32_t* topk_ids,
                  const float* topk_weights, int topk, const cubic_weight* gate_up0,
                  const cubic_weight* down0, int E, float* y, void* workspace, size_t ws_bytes,
                  cubic_stream_t stream);

/* The routed-expert MLP step in the Dynamic A8 mode (CubicQuant article,
 * section "一份 checkpoint，同时服务 A16 与 Dynamic A8": one checkpoint serves
 * both modes; its deployment section switches the routed experts to A8). As
 * cubic_moe_mlp, with both grouped products on int8 activations:
 *   (xq, sx) = act_quant_int8_per_token(x)     per token, [T][H]
 *   [g | u]  = cubic_moe_grouped_gemm_a8 of (xq, sx) with gate_up (fp32)
 *   h        = bf16(SiLU(g) * u)
 *   (hq, hs) = act_quant_int8_per_token(h)     per pair, [T*topk][I]
 *   o_tj     = cubic_moe_grouped_gemm_a8 of (hq, hs) with down (fp32)
 *   y[t]     = sum_j topk_weights[t][j] * o_tj  (fp32, slots in order)
 * Same argument layout and validation as cubic_moe_mlp, plus the grouped A8
 * product's limits (group <= 1024: CUBIC_ERR_GROUP). The workspace
 * (cubic_moe_mlp_a8_workspace_bytes) holds, each part starting at the next
 * multiple of 256 bytes: the routing part (cubic_moe_workspace_bytes(T, topk,
 * E) bytes), xq [T][H] int8, sx [T] fp32, the gate_up outputs [T*topk][2I]
 * fp32, h [T*topk][I] bf16, hq [T*topk][I] int8, hs [T*topk] fp32 and the down
 * outputs [T*topk][H] fp32; they stay there after the call. */
size_t cubic_moe_mlp_a8_workspace_bytes(int64_t T, int topk, int E, int64_t H, int64_t I);
int cubic_moe_mlp_a8(const uint16_t* x_bf16, int64_t T, const int32_t* topk_ids,
                     const float* topk_weights, int topk, const cubic_weight* gate_up0,
                     const cubic_weight* down0, int E, float* y, void* workspace, size_t ws_bytes,
                     cubic_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* CUBIC_H */
