// C ABI of the library: argument checks on the host, then kernel launches on
// the caller's stream.  Nothing here allocates, synchronises or reads device
// memory.  The operations and their sources are described in include/pa.h.
#include "pa.h"

#include <cmath>

#include "pa_internal.h"

namespace {

constexpr int kVersion = 100;  // 0.1.0
constexpr int kMaxGroup = 4;   // query heads per KV head the decode kernel holds
constexpr int kMaxGridYZ = 65535;

bool head_dim_supported(int32_t d) { return d == 64 || d == 128; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int32_t auto_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len) {
  // Start at 512 tokens and halve while the batch offers fewer than 4096
  // (sequence, KV head, partition) items: 256 CUs want many more than one
  // wave each to hide HBM latency and ragged lengths.
  const int64_t ctx = max_context_len > 0 ? max_context_len : 1;
  int32_t p = 512;
  while (p > 64 && (int64_t)num_seqs * num_kv_heads * ceil_div(ctx, p) < 4096) p /= 2;
  while (ceil_div(ctx, p) > pa::kMaxPartitions) p *= 2;
  return p;
}

// Partition size to use, or a negative PA code.
int32_t resolve_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                          int32_t partition_size) {
  if (partition_size < 0 || partition_size % pa::kGroupTokens != 0) return PA_ERR_INVALID_ARG;
  if (partition_size == 0) return auto_partition(num_seqs, num_kv_heads, max_context_len);
  const int64_t ctx = max_context_len > 0 ? max_context_len : 1;
  if (ceil_div(ctx, partition_size) > pa::kMaxPartitions) return PA_ERR_INVALID_ARG;
  return partition_size;
}

}  // namespace

extern "C" {

const char* pa_strerror(int code) {
  switch (code) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case PA_ERR_HIP: return "HIP kernel launch failed";
    default: return "unknown error code";
  }
}

int pa_version(void) { return kVersion; }

int pa_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int64_t num_blocks,
                         hipStream_t stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0)
    return PA_ERR_INVALID_ARG;
  if (block_size != PA_BLOCK_SIZE || !head_dim_supported(head_dim)) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PA_ERR_INVALID_ARG;
  const int64_t lanes = num_tokens * num_kv_heads * (head_dim / 8);
  if (num_tokens > ((int64_t)1 << 40) / num_kv_heads || ceil_div(lanes, 256) > 0x7fffffff)
    return PA_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  const hipError_t e = pa::launch_reshape_and_cache(
      static_cast<const pa::half_t*>(k), static_cast<const pa::half_t*>(v),
      static_cast<pa::half_t*>(k_cache), static_cast<pa::half_t*>(v_cache), slot_mapping,
      num_tokens, num_kv_heads, head_dim, num_blocks, stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping, int64_t num_pairs,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                   hipStream_t stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0)
    return PA_ERR_INVALID_ARG;
  if (block_size != PA_BLOCK_SIZE || !head_dim_supported(head_dim)) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_mapping) return PA_ERR_INVALID_ARG;
  if (num_pairs > 0x7fffffff || num_kv_heads > kMaxGridYZ) return PA_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  const hipError_t e = pa::launch_copy_blocks(static_cast<pa::half_t*>(k_cache),
                                              static_cast<pa::half_t*>(v_cache), block_mapping,
                                              num_pairs, num_kv_heads, head_dim, num_blocks, stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_kv_heads,
                                 int32_t max_context_len) {
  if (num_seqs < 0 || num_kv_heads <= 0 || max_context_len < 0) return PA_ERR_INVALID_ARG;
  return auto_partition(num_seqs, num_kv_heads, max_context_len);
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_context_len,
                                int32_t partition_size) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_context_len < 0)
    return 0;
  const int32_t p = resolve_partition(num_seqs, num_kv_heads, max_context_len, partition_size);
  if (p <= 0) return 0;
  const int64_t np = ceil_div(max_context_len > 0 ? max_context_len : 1, p);
  if (np <= 1) return 0;
  return pa::decode_workspace_bytes(num_seqs, num_q_heads, head_dim, np);
}

int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens, float scale,
              int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
              int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
              int32_t max_context_len, int32_t partition_size, void* workspace,
              size_t workspace_bytes, hipStream_t stream) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_blocks_per_seq <= 0 || num_blocks <= 0 || max_context_len < 0 || !std::isfinite(scale))
    return PA_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (block_size != PA_BLOCK_SIZE || !head_dim_supported(head_dim)) return PA_ERR_UNSUPPORTED;
  if (num_q_heads / num_kv_heads > kMaxGroup) return PA_ERR_UNSUPPORTED;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * PA_BLOCK_SIZE)
    return PA_ERR_INVALID_ARG;
  const int32_t p = resolve_partition(num_seqs, num_kv_heads, max_context_len, partition_size);
  if (p < 0) return p;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return PA_ERR_INVALID_ARG;
  if (num_seqs > kMaxGridYZ || num_kv_heads > kMaxGridYZ) return PA_ERR_UNSUPPORTED;

  const int64_t np = ceil_div(max_context_len > 0 ? max_context_len : 1, p);
  pa::DecodeArgs a{};
  if (np > 1) {
    const size_t need = pa::decode_workspace_bytes(num_seqs, num_q_heads, head_dim, np);
    if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255))
      return PA_ERR_WORKSPACE;
    a.ws = pa::decode_workspace_carve(workspace, num_seqs, num_q_heads, np);
  }
  a.out = static_cast<pa::half_t*>(out);
  a.q = static_cast<const pa::half_t*>(q);
  a.k_cache = static_cast<const pa::half_t*>(k_cache);
  a.v_cache = static_cast<const pa::half_t*>(v_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e) = 1 / ln 2
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.max_context_len = max_context_len;
  a.partition_size = p;
  a.num_partitions = (int)np;
  (void)hipGetLastError();
  return pa::launch_decode(a, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"
