// floors.hip -- measurement kernels for the floors a single launch of the
// decode product cannot beat on this part (built into libcubic_floors.so, which
// only the benchmark loads; the product library does not contain them):
//  - an empty kernel with a given grid (launch and dispatch cost);
//  - a load-only stream over a weight-sized buffer, with the decode GEMV's
//    access pattern (16 rows x 64 bytes per wave load, 12-row workgroups, a
//    quarter of each row per wave) or with contiguous 1 KB wave loads (one, or
//    eight, in flight per lane);
//  - a dependent-load chase through a cyclic permutation (latency of one
//    access that misses every cache).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4f __attribute__((ext_vector_type(4)));

namespace {

__global__ void k_floor_empty(uint32_t* out) {
  if (threadIdx.x == 0x7fffffff) out[0] = 0;   // never taken: nothing is written
}

// The GEMV pattern over rows of `row_bytes` (a multiple of 256): workgroup b owns
// rows 12 b .. 12 b + 11 (lanes past 12 repeat rows), wave w the bytes
// [w row_bytes / 4, (w + 1) row_bytes / 4) of each, lane (nl, kb) 16 bytes at
// 64 t + 16 kb for t < row_bytes / 256.
__global__ __launch_bounds__(256) void k_floor_rows(const unsigned char* __restrict__ w, int64_t rows,
                                                    int64_t row_bytes, uint32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nl = lane & 15, kb = lane >> 4;
  int64_t row = static_cast<int64_t>(blockIdx.x) * 12 + (nl < 12 ? nl : nl - 12);
  row = row < rows ? row : rows - 1;
  const unsigned char* p = w + row * row_bytes + wave * (row_bytes / 4) + kb * 16;
  const int steps = static_cast<int>(row_bytes / 256);
  uint32_t z = 0;
  for (int t0 = 0; t0 < steps; t0 += 8) {
    u32x4f v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = t0 + u < steps ? t0 + u : steps - 1;
      v[u] = *reinterpret_cast<const u32x4f*>(p + 64 * t);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) z ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  out[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = z;
}

// Contiguous: workgroup b reads bytes [b chunk, (b + 1) chunk) in 1 KB wave loads.
__global__ __launch_bounds__(256) void k_floor_contig(const unsigned char* __restrict__ w, int64_t chunk,
                                                      uint32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned char* base = w + static_cast<int64_t>(blockIdx.x) * chunk;
  uint32_t z = 0;
  for (int64_t off = (static_cast<int64_t>(wave) * 64 + lane) * 16; off < chunk; off += 4096) {
    const u32x4f v = *reinterpret_cast<const u32x4f*>(base + off);
    z ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = z;
}

// Contiguous with 8 loads in flight per lane: workgroup b reads bytes
// [b chunk, (b + 1) chunk) (chunk a multiple of 32 KB), each wave 1 KB per load.
__global__ __launch_bounds__(256) void k_floor_contig8(const unsigned char* __restrict__ w, int64_t chunk,
                                                       uint32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned char* base = w + static_cast<int64_t>(blockIdx.x) * chunk;
  uint32_t z = 0;
  for (int64_t o = 0; o < chunk; o += 32768) {
    u32x4f v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = *reinterpret_cast<const u32x4f*>(base + o + (static_cast<int64_t>(u * 4 + wave) * 64 + lane) * 16);
#pragma unroll
    for (int u = 0; u < 8; ++u) z ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  out[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = z;
}

// One lane follows next[] for `steps` dependent loads (next is a cyclic
// permutation of [0, n), so every index stays in range).
__global__ void k_floor_chase(const uint32_t* __restrict__ next, int64_t steps, uint32_t* __restrict__ out) {
  uint32_t i = 0;
  for (int64_t s = 0; s < steps; ++s) i = next[i];
  out[0] = i;
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) int floors_empty(unsigned grid, unsigned block, void* out,
                                                        void* stream) {
  hipLaunchKernelGGL(k_floor_empty, dim3(grid), dim3(block), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint32_t*>(out));
  return static_cast<int>(hipGetLastError());
}

// out: grid * 256 uint32 (grid = ceil(rows / 12)).
__attribute__((visibility("default"))) int floors_rows(const void* w, int64_t rows, int64_t row_bytes, void* out,
                                                       void* stream) {
  if (rows <= 0 || row_bytes <= 0 || row_bytes % 256 != 0) return -1;
  const unsigned grid = static_cast<unsigned>((rows + 11) / 12);
  hipLaunchKernelGGL(k_floor_rows, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const unsigned char*>(w), rows, row_bytes, static_cast<uint32_t*>(out));
  return static_cast<int>(hipGetLastError());
}

// out: grid * 256 uint32; bytes = grid * chunk, chunk a multiple of 16.
__attribute__((visibility("default"))) int floors_contig(const void* w, unsigned grid, int64_t chunk, void* out,
                                                         void* stream) {
  if (grid == 0 || chunk <= 0 || chunk % 16 != 0) return -1;
  hipLaunchKernelGGL(k_floor_contig, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const unsigned char*>(w), chunk, static_cast<uint32_t*>(out));
  return static_cast<int>(hipGetLastError());
}

// out: grid * 256 uint32; bytes = grid * chunk, chunk a multiple of 32768.
__attribute__((visibility("default"))) int floors_contig8(const void* w, unsigned grid, int64_t chunk, void* out,
                                                          void* stream) {
  if (grid == 0 || chunk <= 0 || chunk % 32768 != 0) return -1;
  hipLaunchKernelGGL(k_floor_contig8, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const unsigned char*>(w), chunk, static_cast<uint32_t*>(out));
  return static_cast<int>(hipGetLastError());
}

__attribute__((visibility("default"))) int floors_chase(const void* next, int64_t steps, void* out, void* stream) {
  hipLaunchKernelGGL(k_floor_chase, dim3(1), dim3(1), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint32_t*>(next), steps, static_cast<uint32_t*>(out));
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
