// Read-bandwidth probe: the HBM read rate this device reaches with the decode
// kernel's kind of load (16-byte non-temporal vector loads), reported next to
// the nominal 8 TB/s peak of the part so that a kernel's fraction can also be
// read against what a plain stream of reads achieves.  Two access orders:
// sequential, and tiles of a given size visited in a caller-given order (the
// gather through a block table reads 4 KiB (block, head) tiles in a shuffled
// order).  Every byte read enters an XOR that goes to `sink`, so nothing is
// skipped.
#include <hip/hip_ext.h>

#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;  // 16-byte loads in flight per lane (tiles)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 load_nt16(const u32x4* p) { return __builtin_nontemporal_load(p); }

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Sequential: grid-strided passes over n16 16-byte words, one load in
// flight per lane (measured faster here than 4 or 8: more requests in
// flight than the memory serves well).
__global__ __launch_bounds__(kProbeThreads) void probe_seq_kernel(const u32x4* __restrict__ buf,
                                                                  int64_t n16,
                                                                  uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  for (int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n16; i += stride)
    acc ^= fold(load_nt16(buf + i));
  // one XOR per lane into the sink (a wave reduction would hide nothing)
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) atomicXor(sink, acc);
}

// Tiles: tile t of the visiting order is bytes [order[t] * tile_bytes, +
// tile_bytes); one workgroup instruction covers 4 KiB, so a workgroup reads a
// 4 KiB tile per pass and tiles of 8 KiB and more in several.  An order
// entry outside the buffer's tiles reads tile 0.
__global__ __launch_bounds__(kProbeThreads) void probe_tiles_kernel(
    const u32x4* __restrict__ buf, const int32_t* __restrict__ order, int64_t num_tiles,
    int32_t tile16, int64_t buf_tiles, uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t per_wg = (int64_t)kProbeThreads;  // 16-byte words per pass of a workgroup
  const int64_t words = num_tiles * tile16;
  const int64_t stride = (int64_t)gridDim.x * per_wg;
  for (int64_t base = (int64_t)blockIdx.x * per_wg; base < words; base += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
    bool ok[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const int64_t w = base + u * stride + threadIdx.x;  // word of the visiting order
      ok[u] = w < words;
      const int64_t t = ok[u] ? w / tile16 : 0;
      const int64_t in_tile = ok[u] ? w - t * tile16 : 0;
      const int64_t ot = order[t];
      v[u] = load_nt16(buf + (ot >= 0 && ot < buf_tiles ? ot : 0) * tile16 + in_tile);
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= ok[u] ? fold(v[u]) : 0u;
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) atomicXor(sink, acc);
}

}  // namespace

hipError_t launch_read_probe(const void* buf, int64_t bytes, const int32_t* order,
                             int64_t num_tiles, int32_t tile_bytes, uint32_t* sink, int grid,
                             hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  const u32x4* b = static_cast<const u32x4*>(buf);
  if (!order && !start && !stop) {
    hipLaunchKernelGGL(probe_seq_kernel, dim3(grid), dim3(kProbeThreads), 0, stream, b, bytes / 16,
                       sink);
  } else if (!order) {
    hipExtLaunchKernelGGL(probe_seq_kernel, dim3(grid), dim3(kProbeThreads), 0, stream, start,
                          stop, 0, b, bytes / 16, sink);
  } else {
    hipExtLaunchKernelGGL(probe_tiles_kernel, dim3(grid), dim3(kProbeThreads), 0, stream, start,
                          stop, 0, b, order, num_tiles, tile_bytes / 16, bytes / tile_bytes, sink);
  }
  return hipGetLastError();
}

}  // namespace pa
