// launch.h -- parameter blocks and host launchers shared by the kernel files
// and the C ABI layer (api.cpp). Host-visible only; no device code here.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace cubic {

struct GemvParams {
  const uint8_t* codes;
  const float* scales;
  const uint16_t* shapes;
  int64_t N, K;
  int group;
  int M;
  const uint16_t* x;      // bf16 [M][K] (in-kernel conversion)
  const uint16_t* xp;     // fp16 [M][K] prepared, chunk-permuted (prepared variant)
  const float* xback;     // per-row back multiplier of xp
  float* y;               // [M][N] fp32, or bf16 when ybf16
  int rows;               // weight rows per workgroup (<= 16; the launcher sets it)
  int ybf16;              // outputs rounded to bf16 (nearest even) and stored as 16-bit
};

struct TiledParams {
  const uint8_t* codes;
  const float* scales;
  const uint16_t* shapes;
  int64_t M, N, K;
  int group;
  const void* xa;         // A16: fp16 [M][K] prepared; A8: int8 [M][K]
  const float* xs;        // A16: per-row back multiplier; A8: per-row scale
  float* y;               // [M][N] fp32, or bf16 when ybf16
  int ybf16;
};

struct MoeGemvParams {
  const uint8_t* codes;   // expert 0
  const float* scales;
  const uint16_t* shapes;
  int64_t N, K;
  int group, topk;
  int64_t code_bytes;     // per expert
  const int32_t* hdr;     // [1]: touched experts
  const int32_t* erec;    // per touched expert: expert, first pair, pairs, pair ids 0 and 1
  const int32_t* sorted;  // pair ids grouped by expert
  const uint16_t* x;      // bf16 activations [T][K]
  float* y;               // [T*topk][N] fp32, or bf16 when ybf16
  int ybf16;
  // Direct mode (one token): no routing kernel; pair q's expert is read from
  // ids[q] by the product itself, invalid ids give zero rows, and the first
  // workgroup writes their count to bad_count.
  int direct;
  int npairs;             // pairs (direct mode)
  int E;                  // experts (direct mode)
  const int32_t* ids;     // [npairs] (direct mode)
  int32_t* bad_count;     // (direct mode)
};

// Routed experts in the Dynamic A8 mode: int8 activations with per-token scales.
struct MoeA8Params {
  const uint8_t* codes;   // expert 0
  const float* scales;
  const uint16_t* shapes;
  int64_t N, K;
  int group, topk;
  int64_t code_bytes;     // per expert
  const int32_t* hdr;
  const int32_t* erec;
  const int32_t* sorted;
  const int8_t* xq;       // [T][K] int8 activations
  const float* xs;        // [T] per-token scales
  float* y;               // [T*topk][N] fp32, or bf16 when ybf16
  int ybf16;
  int dense_m;            // launch_gemv_a8: activation rows of a plain product (no routing)
  // Direct mode (one token): no routing kernel; the workgroups of pair q read
  // its expert from ids[q], invalid ids give zero rows, and block 0 writes
  // their count to bad_count.
  int direct;
  int npairs;             // pairs (direct mode, at most 64)
  int E;                  // experts (direct mode)
  const int32_t* ids;     // [npairs] (direct mode)
  int32_t* bad_count;     // (direct mode)
};

int device_cu_count();   // compute units of the current device (0 if unknown)
hipError_t launch_pack(const int8_t* codes, uint8_t* packed, int64_t N, int64_t K, int bits,
                       hipStream_t st, unsigned int* range_error);
hipError_t launch_unpack(const uint8_t* packed, int8_t* codes, int64_t N, int64_t K, int bits,
                         hipStream_t st);
hipError_t launch_dequant(const uint8_t* stream, const float* scales, const uint16_t* shapes,
                          float* out, int64_t N, int64_t K, int bits, int group, hipStream_t st);
hipError_t launch_fill_zero(float* y, int64_t n, bool bf16, hipStream_t st);
hipError_t launch_encode(const float* w, int64_t N, int64_t K, int bits, int group, const float* scales,
                         const uint16_t* shapes, int8_t* codes, hipStream_t st);
int fit_max_group();
hipError_t launch_fit(const float* w, int64_t N, int64_t K, int bits, int group, int8_t* codes,
                      float* scales, uint16_t* shapes, float* loss, hipStream_t st);
hipError_t launch_act_quant(const uint16_t* x, bool xf16, int64_t M, int64_t K, int8_t* xq, float* xs,
                            hipStream_t st);
// xf16: the activations are fp16 (x, or xp with xback NULL on the multi-row path)
hipError_t launch_gemv(const GemvParams& p, int bits, bool ink, bool xf16, hipStream_t st);
// One activation row of 2-bit codes with groups of 256 or 512 and at most 16
// groups per row: the whole-row streaming GEMV (gemv_rows.hip).
bool gemv_rows_supported(int64_t M, int64_t N, int64_t K, int bits, int group);
hipError_t launch_gemv_rows(const GemvParams& p, bool xf16, hipStream_t st);
size_t gemv_ink_lds_bytes(int64_t M, int64_t K, int bits, int group);
bool gemv_supported(int64_t K, int bits, int group);
hipError_t launch_xprep(const uint16_t* x, int64_t M, int64_t K, bool w2_order, uint16_t* xp,
                        float* xback, hipStream_t st);
hipError_t launch_tiled_a16(const TiledParams& p, int bits, hipStream_t st);
hipError_t launch_tiled_a8(const TiledParams& p, int bits, hipStream_t st);
bool prefill_supported(int64_t M, int64_t N, int64_t K, int bits, int group);
hipError_t launch_prefill_a16(const TiledParams& p, int bits, hipStream_t st);
bool prefill_a8_supported(int64_t M, int64_t N, int64_t K, int bits, int group);
bool skinny_supported(int64_t M, int64_t N, int64_t K, int bits, int group);
hipError_t launch_skinny_a16(const TiledParams& p, int bits, hipStream_t st);
hipError_t launch_prefill_a8(const TiledParams& p, int bits, hipStream_t st);
// LDS the grouped kernel needs with one activation row per pass.
size_t moe_lds_min_bytes(int64_t K, int bits, int group);
hipError_t launch_moe(const int32_t* ids, int T, int E, int topk, const MoeGemvParams& base,
                      int32_t* hdr, int32_t* erec, int32_t* sorted, int bits, bool xf16, hipStream_t st);
// The routing kernel alone: pair ids grouped by expert into hdr / erec / sorted,
// output rows of invalid pairs cleared.
hipError_t launch_moe_route(const int32_t* ids, int P, int E, int64_t N, float* y, int ybf16, int32_t* hdr,
                            int32_t* erec, int32_t* sorted, hipStream_t st);
bool moe_a8_supported(int64_t K, int bits, int group);
hipError_t launch_moe_a8(const int32_t* ids, int T, int E, int topk, const MoeA8Params& base, int32_t* hdr,
                         int32_t* erec, int32_t* sorted, int bits, hipStream_t st);
// The plain A8 product of p.dense_m rows (small M) on the routed kernel's
// organisation: one workgroup per 16-row tile, passes of up to four rows.
hipError_t launch_gemv_a8(const MoeA8Params& p, int bits, hipStream_t st);
// The A8 grouped product over a routing already in p.hdr / p.erec / p.sorted.
hipError_t launch_moe_a8_product(const MoeA8Params& p, int P, int E, int T, int bits, hipStream_t st);
// The MLP step's elementwise kernels: h = bf16(SiLU(gate) * up) from the gate_up
// outputs y1 [P][2I], and the router-weighted sum of the pair outputs y2 [P][H].
hipError_t launch_moe_act(const float* y1, int64_t P, int64_t I, uint16_t* h, hipStream_t st);
hipError_t launch_moe_combine(const float* y2, const int32_t* ids, const float* topk_w, int64_t T, int topk,
                              int E, int64_t H, float* out, hipStream_t st);
// The MLP step in the Dynamic A8 mode: the token rows (x bf16 [T][H]) and the
// intermediate rows h are each quantised per row before their grouped product.
struct MoeMlpA8Buffers {
  int8_t* xq; float* xs;       // [T][H], [T]
  float* y1;                   // [P][2I]
  uint16_t* h;                 // [P][I] bf16
  int8_t* hq; float* hs;       // [P][I], [P]
  float* y2;                   // [P][H]
};
hipError_t launch_moe_mlp_a8(const uint16_t* x, const int32_t* ids, const float* topk_w, int T, int E, int topk,
                             const MoeA8Params& up, int up_bits, const MoeA8Params& dn, int dn_bits,
                             int32_t* hdr, int32_t* erec, int32_t* sorted, const MoeMlpA8Buffers& b, float* out,
                             hipStream_t st);
// Library-owned routing scratch (one per device): its size, and its device
// address on the current device (looked up on first use per device).
size_t moe_scratch_bytes();
hipError_t moe_scratch_address(void** out);
// up.y: [T*topk][2I] fp32 scratch; dn.y: [T*topk][H] fp32 scratch; h: [T*topk][I] bf16 scratch.
hipError_t launch_moe_mlp(const int32_t* ids, const float* topk_w, int T, int E, int topk,
                          const MoeGemvParams& up, int up_bits, const MoeGemvParams& dn, int dn_bits,
                          int32_t* hdr, int32_t* erec, int32_t* sorted, uint16_t* h, float* out,
                          hipStream_t st);

}  // namespace cubic
