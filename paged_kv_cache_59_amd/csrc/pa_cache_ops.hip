// Cache-side kernels: the append of new tokens into their slots and the
// block copy of copy-on-write.
//
// Append: the cache grows by one K and one V entry per token ("PagedAttention
// and Continuous Batching Explained (2026)", "TL;DR" and "Why the KV cache is
// the problem"); the entry's slot is physical block * 16 + offset, the block
// coming from the sequence's block table (same page, "PagedAttention: a block
// table for the KV cache").
// Copy: a shared block is duplicated whole before a holder appends to it
// ("KV Cache in Serving Engines ...", section 2 "Sharing Blocks"); the same
// kernel moves blocks between the device pool and a host pool for
// preemption by swap ("Continuous batching and paged attention", "Why they
// depend on each other").
//
// Both are pure data movement (bit copies), bound by HBM bandwidth and far
// smaller than the attention read; each lane moves 16 bytes per access.
#include "pa_internal.h"

namespace pa {

// One lane per (token, KV head, 16-byte chunk of the head dimension), for a
// block size BS of 8, 16 or 32 token slots.
// K: a token's chunk lands at k[b][h][chunk][o][0..7] (16 contiguous bytes;
// the 8 slots of an aligned group make 128 contiguous bytes).
// V: its 8 elements land at v[b][h][o/8][d][o%8], 8 consecutive slots of one
// dimension per 16 bytes.
// When the 8 tokens t..t+7 fill one aligned 8-slot group (slot of t a
// multiple of 8, slots consecutive: the usual case for a prefill chunk), the
// lane of token t gathers their 8 K and 8 V rows and writes 128 contiguous
// bytes of each pool; the lanes of t+1..t+7 leave the group to it.  Any other
// token (a decode step's single tokens, a group only partly in the batch)
// writes its own K chunk and its 8 V elements one by one.  Lead and members
// test the same 8 slot entries, so every element is written exactly once.
// Round trips: the slot with the lane's own rows, then the group's 8 slots
// (all in flight together), then, for a group's lead, the other 7 rows.
template <int D, int BS>
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
  const int64_t row = (int64_t)num_kv_heads * D;  // elements per token of k and v
  const int64_t src = t * row + h * D + c * kChunk;

  const int64_t slot = slot_mapping[t];
  const half8_t kv = *reinterpret_cast<const half8_t*>(k + src);
  const half8_t vv = *reinterpret_cast<const half8_t*>(v + src);
  // Empty asm uses keep each load at the top, all in flight together; the
  // compiler would otherwise sink a load into the branch that first needs it.
  asm volatile("" ::"v"(slot), "v"(kv), "v"(vv));
  if (slot < 0 || slot >= num_blocks * BS) return;
  const int64_t b = slot / BS;
  const int o = (int)(slot - b * BS);
  const int64_t tile = (b * num_kv_heads + h) * (int64_t)(BS * D);

  // the aligned 8-slot group of this token is tokens lead .. lead+7; it is
  // whole when they hold slots slot-o8 .. slot-o8+7 in order (a token outside
  // the batch reads -1, which never matches since slot - o8 >= 0)
  const int o8 = (int)(slot % kChunk);
  const int64_t lead = t - o8;
  int64_t grp[kChunk];
#pragma unroll
  for (int i = 0; i < kChunk; ++i) {
    const int64_t u = lead + i;
    const int64_t uc = u < 0 ? 0 : (u >= num_tokens ? num_tokens - 1 : u);
    grp[i] = slot_mapping[uc];
    if (u != uc) grp[i] = -1;
  }
#pragma unroll
  for (int i = 0; i < kChunk; ++i) asm volatile("" ::"v"(grp[i]));
  int mismatch = 0;
#pragma unroll
  for (int i = 0; i < kChunk; ++i) mismatch |= (int)(grp[i] != slot - o8 + i);

  half_t* kdst = k_cache + tile + ((int64_t)c * BS + o) * kChunk;
  // dims c*8 .. c*8+7 of the 8-slot group start here
  half_t* vgrp = v_cache + tile + ((int64_t)(o / kChunk) * D + c * kChunk) * kChunk;
  if (mismatch == 0) {
    if (o8 != 0) return;  // the group's first token writes it
    half8_t krows[kChunk], vrows[kChunk];
    krows[0] = kv;
    vrows[0] = vv;
#pragma unroll
    for (int i = 1; i < kChunk; ++i) {
      krows[i] = *reinterpret_cast<const half8_t*>(k + src + i * row);
      vrows[i] = *reinterpret_cast<const half8_t*>(v + src + i * row);
    }
#pragma unroll
    for (int i = 1; i < kChunk; ++i) asm volatile("" ::"v"(krows[i]), "v"(vrows[i]));
#pragma unroll
    for (int i = 0; i < kChunk; ++i) reinterpret_cast<half8_t*>(kdst)[i] = krows[i];
#pragma unroll
    for (int e = 0; e < kChunk; ++e) {
      half8_t col;
#pragma unroll
      for (int i = 0; i < kChunk; ++i) col[i] = vrows[i][e];
      *reinterpret_cast<half8_t*>(vgrp + e * kChunk) = col;
    }
    return;
  }
  *reinterpret_cast<half8_t*>(kdst) = kv;
#pragma unroll
  for (int e = 0; e < kChunk; ++e) vgrp[e * kChunk + o8] = vv[e];
}

// One workgroup per (pair, KV head, K|V): the (block, head) tile is BS*D
// contiguous elements in both pools, copied 16 bytes per lane, from block
// src of the source pools to block dst of the destination pools.  Within one
// pool (copy-on-write) src == dst is a no-op; between two pools (swap) it is
// an ordinary copy.
template <int D, int BS>
__global__ __launch_bounds__(256) void copy_blocks_kernel(
    const half_t* __restrict__ src_k, const half_t* __restrict__ src_v, half_t* __restrict__ dst_k,
    half_t* __restrict__ dst_v, const int64_t* __restrict__ block_mapping, int num_kv_heads,
    int64_t src_blocks, int64_t dst_blocks, int same_pool) {
  constexpr int kTile = BS * D;
  const int64_t pair = blockIdx.x;
  const int h = blockIdx.y;
  const half_t* from = blockIdx.z == 0 ? src_k : src_v;
  half_t* to = blockIdx.z == 0 ? dst_k : dst_v;
  const int64_t src = block_mapping[2 * pair];
  const int64_t dst = block_mapping[2 * pair + 1];
  if ((same_pool && src == dst) || src < 0 || dst < 0 || src >= src_blocks || dst >= dst_blocks)
    return;
  const half_t* s = from + (src * num_kv_heads + h) * (int64_t)kTile;
  half_t* d = to + (dst * num_kv_heads + h) * (int64_t)kTile;
  for (int i = threadIdx.x; i < kTile / kChunk; i += blockDim.x)
    reinterpret_cast<half8_t*>(d)[i] = reinterpret_cast<const half8_t*>(s)[i];
}

template <int D, int BS>
void launch_append_t(const half_t* k, const half_t* v, half_t* k_cache, half_t* v_cache,
                     const int64_t* slot_mapping, int64_t num_tokens, int num_kv_heads,
                     int64_t num_blocks, hipStream_t stream) {
  const int64_t lanes = num_tokens * num_kv_heads * (D / kChunk);
  const unsigned grid = (unsigned)((lanes + 255) / 256);
  hipLaunchKernelGGL((reshape_and_cache_kernel<D, BS>), dim3(grid), dim3(256), 0, stream, k, v,
                     k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads, num_blocks);
}

hipError_t launch_reshape_and_cache(const half_t* k, const half_t* v, half_t* k_cache,
                                    half_t* v_cache, const int64_t* slot_mapping,
                                    int64_t num_tokens, int num_kv_heads, int head_dim,
                                    int block_size, int64_t num_blocks, hipStream_t stream) {
#define PA_APPEND(D, BS)                                                                     \
  if (head_dim == D && block_size == BS)                                                     \
    launch_append_t<D, BS>(k, v, k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads,   \
                           num_blocks, stream);
  PA_APPEND(128, 16) PA_APPEND(64, 16) PA_APPEND(128, 8) PA_APPEND(64, 8) PA_APPEND(128, 32)
  PA_APPEND(64, 32)
#undef PA_APPEND
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const half_t* src_k, const half_t* src_v, half_t* dst_k,
                              half_t* dst_v, const int64_t* block_mapping, int64_t num_pairs,
                              int num_kv_heads, int head_dim, int block_size, int64_t src_blocks,
                              int64_t dst_blocks, bool same_pool, hipStream_t stream) {
  const dim3 grid((unsigned)num_pairs, (unsigned)num_kv_heads, 2);
  const int threads = block_size * head_dim / kChunk >= 256 ? 256 : block_size * head_dim / kChunk;
#define PA_COPY(D, BS)                                                                        \
  if (head_dim == D && block_size == BS)                                                      \
    hipLaunchKernelGGL((copy_blocks_kernel<D, BS>), grid, dim3(threads), 0, stream, src_k,    \
                       src_v, dst_k, dst_v, block_mapping, num_kv_heads, src_blocks,          \
                       dst_blocks, same_pool ? 1 : 0);
  PA_COPY(128, 16) PA_COPY(64, 16) PA_COPY(128, 8) PA_COPY(64, 8) PA_COPY(128, 32)
  PA_COPY(64, 32)
#undef PA_COPY
  return hipGetLastError();
}

}  // namespace pa
