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
  float* y;               // [M][N]
  int rows;               // weight rows per workgroup (<= 16; the launcher sets it)
};

struct TiledParams {
  const uint8_t* codes;
  const float* scales;
  const uint16_t* shapes;
  int64_t M, N, K;
  int group;
  const void* xa;         // A16: fp16 [M][K] prepared; A8: int8 [M][K]
  const float* xs;        // A16: per-row back multiplier; A8: per-row scale
  float* y;
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
  float* y;               // [T*topk][N]
};

int device_cu_count();   // compute units of the current device (0 if unknown)
hipError_t launch_pack(const int8_t* codes, uint8_t* packed, int64_t N, int64_t K, int bits,
                       hipStream_t st, unsigned int* range_error);
hipError_t launch_unpack(const uint8_t* packed, int8_t* codes, int64_t N, int64_t K, int bits,
                         hipStream_t st);
hipError_t launch_dequant(const uint8_t* stream, const float* scales, const uint16_t* shapes,
                          float* out, int64_t N, int64_t K, int bits, int group, hipStream_t st);
hipError_t launch_fill_zero(float* y, int64_t n, hipStream_t st);
hipError_t launch_encode(const float* w, int64_t N, int64_t K, int bits, int group, const float* scales,
                         const uint16_t* shapes, int8_t* codes, hipStream_t st);
int fit_max_group();
hipError_t launch_fit(const float* w, int64_t N, int64_t K, int bits, int group, int8_t* codes,
                      float* scales, uint16_t* shapes, float* loss, hipStream_t st);
hipError_t launch_act_quant(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, float* xs,
                            hipStream_t st);
hipError_t launch_gemv(const GemvParams& p, int bits, bool ink, hipStream_t st);
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
                      int32_t* hdr, int32_t* erec, int32_t* sorted, int bits, hipStream_t st);
// up.y: [T*topk][2I] fp32 scratch; dn.y: [T*topk][H] fp32 scratch; h: [T*topk][I] bf16 scratch.
hipError_t launch_moe_mlp(const int32_t* ids, const float* topk_w, int T, int E, int topk,
                          const MoeGemvParams& up, int up_bits, const MoeGemvParams& dn, int dn_bits,
                          int32_t* hdr, int32_t* erec, int32_t* sorted, uint16_t* h, float* out,
                          hipStream_t st);

}  // namespace cubic
