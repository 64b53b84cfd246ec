// pa_read_probe.hip -- HBM read-rate probes for the benchmark's context line.
//
// Not part of the decode path: libpaprobe.so is loaded by the benchmark only,
// to state what rate a plain read reaches on the same GPU next to the decode
// kernel's. Two access patterns:
//
//   pa_probe_stream_read  one contiguous buffer read front to back, 16-byte
//                         non-temporal loads, grid-stride (the sequential
//                         ceiling);
//   pa_probe_tile_gather  whole tiles of tile_bytes (a multiple of 1 KB) read
//                         in the order a table gives, one wave per workgroup
//                         with three tiles in flight, 16-byte non-temporal
//                         loads (the shape of the decode kernel's paged K/V
//                         reads: one (block, KV head) tile per 16-token
//                         chunk, a short ring of chunks per wave).
//
// Both fold what they read into one word per thread and store it only if it
// equals a constant the data practically never produces, so the loads stay
// and nothing is written. Arguments are device pointers; the caller checks
// that the table's entries lie in [0, bytes / tile_bytes). Returns 0, or -1
// on a bad size or count (nothing is launched then), or the launch's HIP
// error code.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint32_t kNever = 0x9e3779b9u;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4* __restrict__ src, int64_t n,
                                                          uint32_t* sink) {
  const int64_t step = (int64_t)gridDim.x * 1024;
  uint32_t acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * 1024 + threadIdx.x; i < n; i += step) {
    u32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      v[k] = i + 256 * k < n ? __builtin_nontemporal_load(src + i + 256 * k) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < 4; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  if (acc == kNever) sink[blockIdx.x] = acc;
}

// One wave per workgroup; wave w reads tiles w, w + n, w + 2n, ... (n waves),
// three tiles in flight (all loads of three tiles issued before any is used).
__global__ void __launch_bounds__(64) tile_gather_kernel(const char* __restrict__ pool,
                                                         const int32_t* __restrict__ tiles,
                                                         int ntiles, int tile_kb, uint32_t* sink) {
  const int lane = threadIdx.x;
  const int wave = blockIdx.x;
  const int nwaves = gridDim.x;
  uint32_t acc = 0;
  for (int t0 = wave; t0 < ntiles; t0 += 3 * nwaves) {
    u32x4 v[3][16];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int t = t0 + k * nwaves;
      const u32x4* base = (const u32x4*)(pool + (int64_t)tiles[t < ntiles ? t : t0] * tile_kb * 1024) + lane;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        v[k][j] = (t < ntiles && j < tile_kb) ? __builtin_nontemporal_load(base + 64 * j) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc ^= v[k][j].x ^ v[k][j].y ^ v[k][j].z ^ v[k][j].w;
  }
  if (acc == kNever) sink[wave] = acc;
}

}  // namespace

extern "C" int pa_probe_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int blocks,
                                    hipStream_t s) {
  if (!buf || !sink || bytes <= 0 || bytes % 16 || blocks <= 0) return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, s, (const u32x4*)buf, bytes / 16,
                     sink);
  return (int)hipGetLastError();
}

// blocks: waves (one per workgroup); sink holds at least blocks words; tile_bytes is
// 1..16 KB in whole KB
extern "C" int pa_probe_tile_gather(const void* pool, const int32_t* tiles, int ntiles,
                                    int tile_bytes, uint32_t* sink, int blocks, hipStream_t s) {
  if (!pool || !tiles || !sink || ntiles <= 0 || tile_bytes <= 0 || tile_bytes % 1024 ||
      tile_bytes > 16384 || blocks <= 0)
    return -1;
  hipLaunchKernelGGL(tile_gather_kernel, dim3(blocks), dim3(64), 0, s, (const char*)pool, tiles, ntiles,
                     tile_bytes / 1024, sink);
  return (int)hipGetLastError();
}
