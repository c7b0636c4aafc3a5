// Read-bandwidth probes for the benchmark: the measured ceiling that the
// decode path's effective bandwidth is compared with, on the same device.
// Not part of the decode library or its ABI; bench.py loads libpkv_probe.so.
//
//  * linear: every lane streams 16-byte non-temporal loads over the buffer.
//  * chunks: each 256-thread workgroup reads batches of 32 KB made of 2 KB
//    chunks at the offsets listed in `idx` (page-like random placement).
// Both fold what they read into one word written only if it matches an
// impossible value, so no load is optimised away and nothing else is written.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) probe_linear(const u4* __restrict__ p, uint64_t n16, uint32_t* sink) {
  uint32_t acc = 0;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const u4 x = __builtin_nontemporal_load(p + i);
    acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

// idx: chunk numbers (2 KB units) into p, 16 per 32 KB batch; batches
// [blockIdx.x * per_wg, (blockIdx.x + 1) * per_wg).
__global__ void __launch_bounds__(256) probe_chunks(const u4* __restrict__ p, const uint32_t* __restrict__ idx,
                                                    int per_wg, uint32_t* sink) {
  uint32_t acc = 0;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int b = 0; b < per_wg; ++b) {
    const uint64_t batch = (uint64_t)blockIdx.x * per_wg + b;
    u4 x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t boff = (uint32_t)(4 * j + w) << 10;  // 1 KB slice of the batch
      const uint64_t chunk = idx[batch * 16 + (boff >> 11)];
      x[j] = __builtin_nontemporal_load(p + ((chunk << 11) + (boff & 2047u)) / 16 + lane);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= x[j][j & 3];
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

extern "C" {

// Streams `bytes` (a multiple of 16, buffer 16-byte aligned) with `grid`
// workgroups of 256 threads. Returns 0, or -1 on bad arguments, -4 if the
// launch failed.
int pkv_probe_read_linear(const void* buf, uint64_t bytes, uint32_t* sink, int grid, void* stream) {
  if (!buf || !sink || bytes % 16 || grid < 1 || (reinterpret_cast<uintptr_t>(buf) & 15)) return -1;
  hipLaunchKernelGGL(probe_linear, dim3(grid), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<const u4*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Reads grid * per_wg batches of 32 KB, each 16 chunks of 2 KB numbered by
// `idx` (grid * per_wg * 16 entries, every chunk number < buf_bytes / 2048).
// The caller guarantees the index bounds; the buffer must be 16-byte aligned.
int pkv_probe_read_chunks(const void* buf, const uint32_t* idx, int grid, int per_wg, uint32_t* sink,
                          void* stream) {
  if (!buf || !idx || !sink || grid < 1 || per_wg < 1 || (reinterpret_cast<uintptr_t>(buf) & 15)) return -1;
  hipLaunchKernelGGL(probe_chunks, dim3(grid), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<const u4*>(buf), idx, per_wg, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
