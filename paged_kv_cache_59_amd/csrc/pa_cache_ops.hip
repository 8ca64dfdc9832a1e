// Cache-side kernels: the append of new tokens into their slots and the
// block copy of copy-on-write.
//
// Append: the cache grows by one K and one V entry per token ("PagedAttention
// and Continuous Batching Explained (2026)", "TL;DR" and "Why the KV cache is
// the problem"); the entry's slot is physical block * 16 + offset, the block
// coming from the sequence's block table (same page, "PagedAttention: a block
// table for the KV cache").
// Copy: a shared block is duplicated whole before a holder appends to it
// ("KV Cache in Serving Engines ...", section 2 "Sharing Blocks").
//
// Both are pure data movement (bit copies), bound by HBM bandwidth and far
// smaller than the attention read; each lane moves 16 bytes per access.
#include "pa_internal.h"

namespace pa {

// One lane per (token, KV head, 16-byte chunk of the head dimension).
// K: the chunk lands whole at k[b][h][chunk][o][0..7] (16 contiguous bytes).
// V: its 8 elements land at v[b][h][o/8][d][o%8], one element per 16 bytes.
template <int D>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const half_t* __restrict__ k, const half_t* __restrict__ v, half_t* __restrict__ k_cache,
    half_t* __restrict__ v_cache, const int64_t* __restrict__ slot_mapping, int64_t num_tokens,
    int num_kv_heads, int64_t num_blocks) {
  constexpr int kChunks = D / kChunk;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_token = (int64_t)num_kv_heads * kChunks;
  if (idx >= num_tokens * per_token) return;
  const int64_t t = idx / per_token;
  const int rem = (int)(idx - t * per_token);
  const int h = rem / kChunks;
  const int c = rem - h * kChunks;
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_blocks * kBlockSize) return;
  const int64_t b = slot / kBlockSize;
  const int o = (int)(slot - b * kBlockSize);
  const int64_t src = (t * num_kv_heads + h) * D + c * kChunk;
  const int64_t tile = (b * num_kv_heads + h) * (int64_t)(kBlockSize * D);

  const half8_t kv = *reinterpret_cast<const half8_t*>(k + src);
  *reinterpret_cast<half8_t*>(k_cache + tile + ((int64_t)c * kBlockSize + o) * kChunk) = kv;

  const half8_t vv = *reinterpret_cast<const half8_t*>(v + src);
  half_t* vdst = v_cache + tile + ((int64_t)(o / kChunk) * D + c * kChunk) * kChunk + (o % kChunk);
#pragma unroll
  for (int e = 0; e < kChunk; ++e) vdst[e * kChunk] = vv[e];
}

// One workgroup per (pair, KV head, K|V): the (block, head) tile is 16*D
// contiguous elements in both pools, copied 16 bytes per lane.
template <int D>
__global__ __launch_bounds__(256) void copy_blocks_kernel(half_t* __restrict__ k_cache,
                                                          half_t* __restrict__ v_cache,
                                                          const int64_t* __restrict__ block_mapping,
                                                          int num_kv_heads, int64_t num_blocks) {
  constexpr int kTile = kBlockSize * D;
  const int64_t pair = blockIdx.x;
  const int h = blockIdx.y;
  half_t* pool = blockIdx.z == 0 ? k_cache : v_cache;
  const int64_t src = block_mapping[2 * pair];
  const int64_t dst = block_mapping[2 * pair + 1];
  if (src == dst || src < 0 || dst < 0 || src >= num_blocks || dst >= num_blocks) return;
  const half_t* s = pool + (src * num_kv_heads + h) * (int64_t)kTile;
  half_t* d = pool + (dst * num_kv_heads + h) * (int64_t)kTile;
  for (int i = threadIdx.x; i < kTile / kChunk; i += blockDim.x)
    reinterpret_cast<half8_t*>(d)[i] = reinterpret_cast<const half8_t*>(s)[i];
}

hipError_t launch_reshape_and_cache(const half_t* k, const half_t* v, half_t* k_cache,
                                    half_t* v_cache, const int64_t* slot_mapping,
                                    int64_t num_tokens, int num_kv_heads, int head_dim,
                                    int64_t num_blocks, hipStream_t stream) {
  const int64_t lanes = num_tokens * num_kv_heads * (head_dim / kChunk);
  const unsigned grid = (unsigned)((lanes + 255) / 256);
  if (head_dim == 128)
    hipLaunchKernelGGL(reshape_and_cache_kernel<128>, dim3(grid), dim3(256), 0, stream, k, v,
                       k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads, num_blocks);
  else
    hipLaunchKernelGGL(reshape_and_cache_kernel<64>, dim3(grid), dim3(256), 0, stream, k, v,
                       k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads, num_blocks);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(half_t* k_cache, half_t* v_cache, const int64_t* block_mapping,
                              int64_t num_pairs, int num_kv_heads, int head_dim,
                              int64_t num_blocks, hipStream_t stream) {
  const dim3 grid((unsigned)num_pairs, (unsigned)num_kv_heads, 2);
  if (head_dim == 128)
    hipLaunchKernelGGL(copy_blocks_kernel<128>, grid, dim3(256), 0, stream, k_cache, v_cache,
                       block_mapping, num_kv_heads, num_blocks);
  else
    hipLaunchKernelGGL(copy_blocks_kernel<64>, grid, dim3(128), 0, stream, k_cache, v_cache,
                       block_mapping, num_kv_heads, num_blocks);
  return hipGetLastError();
}

}  // namespace pa
