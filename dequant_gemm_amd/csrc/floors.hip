// floors.hip -- measurement kernels for the floors a single launch of the
// decode product cannot beat on this part (built into libcubic_floors.so, which
// only the benchmark loads; the product library does not contain them):
//  - an empty kernel with a given grid (launch and dispatch cost);
//  - a load-only stream over a weight-sized buffer, with the decode GEMV's
//    access pattern (16 rows x 64 bytes per wave load, 12-row workgroups, a
//    quarter of each row per wave) or with contiguous 1 KB wave loads (one, or
//    eight, in flight per lane);
//  - a dependent-load chase through a cyclic permutation (latency of one
//    access that misses every cache);
//  - arrival probes: load-only kernels whose waves timestamp their start, the
//    arrival of their first load and of their last (gate_up rows of 1792 bytes),
//    for the old GEMV's pattern and for whole rows per wave load.
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

// 100 MHz wall clock; the wait in the same asm block keeps the read ordered.
__device__ __forceinline__ unsigned long long wall_clock() {
  unsigned long long t;
  asm volatile("s_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t));
  return t;
}
__device__ __forceinline__ void consumed(uint32_t s) { asm volatile("" ::"v"(s)); }

// Arrival probe, the old GEMV's pattern on rows of 1792 bytes: workgroup b owns
// rows 12 b .. 12 b + 11 (lanes past 12 repeat rows), wave w the 7 steps of 64
// bytes at 448 w, lane (nl, kb) 16 bytes at 64 t + 16 kb. out[3 wave + 0..2]:
// start, first load consumed, last load consumed.
__global__ __launch_bounds__(256) void k_floor_arrival16(const unsigned char* __restrict__ w, int64_t rows,
                                                         unsigned long long* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nl = lane & 15, kb = lane >> 4;
  int64_t row = static_cast<int64_t>(blockIdx.x) * 12 + (nl < 12 ? nl : nl - 12);
  row = row < rows ? row : rows - 1;
  const unsigned char* p = w + row * 1792 + wave * 448 + kb * 16;
  const unsigned long long t0 = wall_clock();
  u32x4f v[7];
#pragma unroll
  for (int t = 0; t < 7; ++t) v[t] = *reinterpret_cast<const u32x4f*>(p + 64 * t);
  asm volatile("" : "+v"(v[0]));
  uint32_t z = v[0].x ^ v[0].y ^ v[0].z ^ v[0].w;
  consumed(z);
  const unsigned long long t1 = wall_clock();
#pragma unroll
  for (int t = 1; t < 7; ++t) asm volatile("" : "+v"(v[t]));
#pragma unroll
  for (int t = 1; t < 7; ++t) z ^= v[t].x ^ v[t].y ^ v[t].z ^ v[t].w;
  consumed(z);
  const unsigned long long t2 = wall_clock();
  if (lane == 0) {
    const int64_t g = static_cast<int64_t>(blockIdx.x) * 4 + wave;
    out[3 * g] = t0; out[3 * g + 1] = t1; out[3 * g + 2] = t2 + (z == 0x5a5a5a5au ? 1 : 0);
  }
}

// Arrival probe, whole rows: wave g reads rows 3 g .. 3 g + 2, each with one
// wave load (lane l, l % 16 < 14, takes 32 bytes at 128 (l % 16) + 32 (l / 16)).
__global__ __launch_bounds__(256) void k_floor_arrival_rows(const unsigned char* __restrict__ w, int64_t rows,
                                                            unsigned long long* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t g = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  const int i = lane & 15, kq = lane >> 4;
  const int off = (i < 14 ? i : 13) * 128 + kq * 32;
  const unsigned long long t0 = wall_clock();
  u32x4f v[3][2];
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    int64_t row = 3 * g + r;
    row = row < rows ? row : rows - 1;
    const unsigned char* p = w + row * 1792 + off;
    v[r][0] = *reinterpret_cast<const u32x4f*>(p);
    v[r][1] = *reinterpret_cast<const u32x4f*>(p + 16);
  }
  asm volatile("" : "+v"(v[0][0]), "+v"(v[0][1]));
  uint32_t z = v[0][0].x ^ v[0][0].y ^ v[0][1].z ^ v[0][1].w;
  consumed(z);
  const unsigned long long t1 = wall_clock();
#pragma unroll
  for (int r = 1; r < 3; ++r) asm volatile("" : "+v"(v[r][0]), "+v"(v[r][1]));
#pragma unroll
  for (int r = 1; r < 3; ++r) z ^= v[r][0].x ^ v[r][0].y ^ v[r][1].z ^ v[r][1].w;
  consumed(z);
  const unsigned long long t2 = wall_clock();
  if (lane == 0) { out[3 * g] = t0; out[3 * g + 1] = t1; out[3 * g + 2] = t2 + (z == 0x5a5a5a5au ? 1 : 0); }
}

}  // namespace

extern "C" {

// Arrival probes over `rows` rows of 1792 bytes. kind 0: the old GEMV's pattern
// (grid ceil(rows / 12), 4 waves each); kind 1: whole rows (grid ceil(rows / 12),
// 4 waves of 3 rows). out: 3 uint64 per wave, 4 * grid waves.
__attribute__((visibility("default"))) int floors_arrival(int kind, const void* w, int64_t rows, void* out,
                                                          void* stream) {
  if (rows <= 0 || (kind != 0 && kind != 1)) return -1;
  const unsigned grid = static_cast<unsigned>((rows + 11) / 12);
  if (kind == 0)
    hipLaunchKernelGGL(k_floor_arrival16, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const unsigned char*>(w), rows, static_cast<unsigned long long*>(out));
  else
    hipLaunchKernelGGL(k_floor_arrival_rows, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const unsigned char*>(w), rows, static_cast<unsigned long long*>(out));
  return static_cast<int>(hipGetLastError());
}

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
