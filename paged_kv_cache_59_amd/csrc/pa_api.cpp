// C ABI of the library: argument checks on the host, then kernel launches on
// the caller's stream.  Nothing here allocates, synchronises or reads device
// memory.  The operations and their sources are described in include/pa.h.
#include "pa.h"

#include <atomic>
#include <cmath>
#include <cstdlib>

#include "pa_internal.h"

namespace {

constexpr int kVersion = 500;  // 0.5.0
using pa::kMaxGroup;

// Bound on the waits between a decode worker's waves: pa::kSpinLimit, or
// PA_DECODE_SPIN_LIMIT (0 .. kSpinLimit) from the environment, read at each
// call, with which tests force a wait to give up and check that the status
// word reports it.
int spin_limit() {
  const char* e = std::getenv("PA_DECODE_SPIN_LIMIT");
  if (!e || !*e) return pa::kSpinLimit;
  char* end = nullptr;
  const long v = std::strtol(e, &end, 10);
  if (end == e || v < 0) return pa::kSpinLimit;
  return v < pa::kSpinLimit ? (int)v : pa::kSpinLimit;
}
constexpr int kMaxGridYZ = 65535;

bool head_dim_supported(int32_t d) { return d == 64 || d == 128; }
// block sizes the cache operations take (the attention kernels: see each)
bool block_size_supported(int32_t bs) { return bs == 8 || bs == 16 || bs == 32; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// A KV head of G > kMaxGroup query heads is attended in ceil(G / kMaxGroup)
// sub-groups of up to kMaxGroup query heads (num_q_heads a multiple of
// num_kv_heads): the prefix pass's heads; the decode takes up to 4 of them
// per pass (decode_split).
int32_t kv_split(int32_t num_q_heads, int32_t num_kv_heads) {
  return (int32_t)ceil_div(num_q_heads / num_kv_heads, kMaxGroup);
}
// Sequences of one decode launch: its copies of the batch (split of them)
// fill at most kMaxSeqsPerLaunch virtual sequences.
int64_t seqs_per_launch(int64_t num_seqs, int32_t split) {
  const int64_t cap = pa::kMaxSeqsPerLaunch / split;
  return num_seqs < cap ? num_seqs : cap;
}

// Decode workers for the current device: kWorkersPerCU per compute unit,
// rounded up to a multiple of 8 (the XCD count).  Cached per device; calls
// from several threads may each fill an entry, with the same value.
int32_t auto_workers() {
  static std::atomic<int32_t> cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
  if (dev >= 0 && dev < 64) {
    const int32_t c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return PA_ERR_HIP;
  const int32_t w = ((cus * pa::kWorkersPerCU + 7) / 8) * 8;
  if (dev >= 0 && dev < 64) cache[dev].store(w, std::memory_order_relaxed);
  return w;
}

// Workers to use, or a negative PA code.
int32_t resolve_workers(int32_t num_workers) {
  if (num_workers < 0 || num_workers > pa::kMaxWorkers) return PA_ERR_INVALID_ARG;
  return num_workers == 0 ? auto_workers() : num_workers;
}

}  // namespace

extern "C" {

const char* pa_strerror(int code) {
  switch (code) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case PA_ERR_HIP: return "HIP runtime call or kernel launch failed";
    case PA_ERR_SCRATCH_LIMIT:
      return "batch needs more decode scratch than the library's static array holds "
             "(32 MiB); pass a workspace to pa_decode_append instead";
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
  if (!block_size_supported(block_size) || !head_dim_supported(head_dim))
    return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PA_ERR_INVALID_ARG;
  const int64_t lanes = num_tokens * num_kv_heads * (head_dim / 8);
  if (num_tokens > ((int64_t)1 << 40) / num_kv_heads || ceil_div(lanes, 256) > 0x7fffffff)
    return PA_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  const hipError_t e = pa::launch_reshape_and_cache(
      static_cast<const pa::half_t*>(k), static_cast<const pa::half_t*>(v),
      static_cast<pa::half_t*>(k_cache), static_cast<pa::half_t*>(v_cache), slot_mapping,
      num_tokens, num_kv_heads, head_dim, block_size, num_blocks, stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping, int64_t num_pairs,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                   hipStream_t stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0)
    return PA_ERR_INVALID_ARG;
  if (!block_size_supported(block_size) || !head_dim_supported(head_dim))
    return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_mapping) return PA_ERR_INVALID_ARG;
  if (num_pairs > 0x7fffffff || num_kv_heads > kMaxGridYZ) return PA_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  pa::half_t* k = static_cast<pa::half_t*>(k_cache);
  pa::half_t* v = static_cast<pa::half_t*>(v_cache);
  const hipError_t e = pa::launch_copy_blocks(k, v, k, v, block_mapping, num_pairs, num_kv_heads,
                                              head_dim, block_size, num_blocks, num_blocks, true,
                                              stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                   const int64_t* block_mapping, int64_t num_pairs, int32_t num_kv_heads,
                   int32_t head_dim, int32_t block_size, int64_t src_num_blocks,
                   int64_t dst_num_blocks, hipStream_t stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || src_num_blocks <= 0 ||
      dst_num_blocks <= 0)
    return PA_ERR_INVALID_ARG;
  if (!block_size_supported(block_size) || !head_dim_supported(head_dim))
    return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !block_mapping) return PA_ERR_INVALID_ARG;
  if (src_k == dst_k || src_v == dst_v) return PA_ERR_INVALID_ARG;  // one pool: pa_copy_blocks
  if (num_pairs > 0x7fffffff || num_kv_heads > kMaxGridYZ) return PA_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  const hipError_t e = pa::launch_copy_blocks(
      static_cast<const pa::half_t*>(src_k), static_cast<const pa::half_t*>(src_v),
      static_cast<pa::half_t*>(dst_k), static_cast<pa::half_t*>(dst_v), block_mapping, num_pairs,
      num_kv_heads, head_dim, block_size, src_num_blocks, dst_num_blocks, false, stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int32_t pa_decode_num_workers(void) { return auto_workers(); }

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_context_len, int32_t num_workers) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_context_len < 0 || num_q_heads % num_kv_heads != 0)
    return 0;
  const int32_t w = resolve_workers(num_workers);
  if (w <= 0) return 0;
  const int32_t split = pa::decode_split(kv_split(num_q_heads, num_kv_heads));
  return pa::decode_workspace_bytes(seqs_per_launch(num_seqs, split) * split, num_kv_heads,
                                    head_dim, pa::decode_slot_factor(split) * w);
}

}  // extern "C"

namespace {

// Decode, and with k_new non-null the fused append (see pa_decode_append).
int decode_impl(void* out, const void* q, const void* k_new, const void* v_new,
                const int64_t* slot_mapping, const void* k_cache, const void* v_cache,
                const int32_t* block_tables, const int32_t* context_lens, float scale,
                int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                int32_t max_context_len, int32_t num_workers, void* workspace,
                size_t workspace_bytes, hipStream_t stream, hipEvent_t kernel_start,
                hipEvent_t kernel_stop, uint32_t flags = 0, bool static_scratch = false) {
  const bool fused = k_new || v_new || slot_mapping;
  if (flags & ~(uint32_t)PA_DECODE_SHARED_BLOCKS) return PA_ERR_INVALID_ARG;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_blocks_per_seq <= 0 || num_blocks <= 0 || max_context_len < 0 || !std::isfinite(scale))
    return PA_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (!block_size_supported(block_size) || !head_dim_supported(head_dim))
    return PA_ERR_UNSUPPORTED;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return PA_ERR_INVALID_ARG;
  if (num_workers < 0 || num_workers > pa::kMaxWorkers) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return PA_ERR_INVALID_ARG;
  // the fused append moves the new rows in 16-byte pieces
  if (fused && (!k_new || !v_new || !slot_mapping || (reinterpret_cast<uintptr_t>(k_new) & 15) ||
                (reinterpret_cast<uintptr_t>(v_new) & 15)))
    return PA_ERR_INVALID_ARG;
  // A KV head of more than kMaxGroup query heads is attended in split
  // sub-groups: the launch's merger sees split x n virtual sequences (one
  // per sub-group and sequence), at most kMaxSeqsPerLaunch; its 64-token
  // units (all heads) must fit a 32-bit index
  // (split: the decode's sub-groups, a count above 4 rounded up to a
  // multiple of 4 with empty ones; the prefix pass takes the sub-groups that
  // hold query heads)
  const int32_t groups = kv_split(num_q_heads, num_kv_heads);
  const int32_t split = pa::decode_split(groups);
  const int64_t per_launch = seqs_per_launch(num_seqs, split);
  const int64_t vseqs = per_launch * split;
  if (vseqs * num_kv_heads * ceil_div(max_context_len, pa::kGroupTokens) > 0x7fffffff)
    return PA_ERR_UNSUPPORTED;
  const int32_t w = resolve_workers(num_workers);
  if (w < 0) return w;
  // (sub-groups attended together: a share slot per worker for each)
  const int32_t slot_workers = pa::decode_slot_factor(split) * w;
  const size_t need =
      pa::decode_workspace_bytes(vseqs, num_kv_heads, head_dim, slot_workers);
  if (static_scratch) {
    // the library's own device array stands in for the workspace
    if (need > pa::kStaticScratchBytes ||
        pa::decode_control_bytes(vseqs, num_kv_heads) > pa::kStaticControlBytes)
      return PA_ERR_SCRATCH_LIMIT;
    if (pa::decode_static_scratch(stream, &workspace) != hipSuccess) return PA_ERR_HIP;
    workspace_bytes = pa::kStaticScratchBytes;
  }
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return PA_ERR_WORKSPACE;

  pa::DecodeArgs a{};
  a.ws = pa::decode_workspace_carve(workspace, workspace_bytes, vseqs, num_kv_heads, head_dim,
                                    slot_workers);
  a.k_cache = static_cast<const pa::half_t*>(k_cache);
  a.v_cache = static_cast<const pa::half_t*>(v_cache);
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e) = 1 / ln 2
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.kv_split = split;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.max_context_len = max_context_len;
  a.num_workers = w;
  a.spin_limit = spin_limit();
  // Batches whose sequences share prefix blocks: per launch, the prefix pass
  // (pa_prefix.hip) finds the groups of sequences with a common prefix and
  // attends every group's query rows to its prefix once; the decode kernel
  // covers the rest of each sequence and folds both together.
  const bool shared = fused && (flags & PA_DECODE_SHARED_BLOCKS);
  // chunks of the longest prefix a group can have (one short of the
  // longest context, in whole 64-token units)
  const int max_chunks = pa::prefix_chunks(
      (max_context_len > 0 ? max_context_len - 1 : 0) / pa::kGroupTokens * pa::kGroupTokens);
  (void)hipGetLastError();
  // launches on one stream run in order, so they share the workspace
  for (int64_t s0 = 0; s0 < num_seqs; s0 += per_launch) {
    const int64_t n = num_seqs - s0 < per_launch ? num_seqs - s0 : per_launch;
    const int64_t row = s0 * num_q_heads * head_dim;
    a.out = static_cast<pa::half_t*>(out) + row;
    a.q = static_cast<const pa::half_t*>(q) + row;
    a.block_tables = block_tables + s0 * max_blocks_per_seq;
    a.context_lens = context_lens + s0;
    a.num_seqs = (int)(n * split);
    if (fused) {
      const int64_t rows = s0 * num_kv_heads * head_dim;
      a.k_new = static_cast<const pa::half_t*>(k_new) + rows;
      a.v_new = static_cast<const pa::half_t*>(v_new) + rows;
      a.slot_mapping = slot_mapping + s0;
      a.k_cache_w = const_cast<pa::half_t*>(a.k_cache);
      a.v_cache_w = const_cast<pa::half_t*>(a.v_cache);
    }
    hipEvent_t start = s0 == 0 ? kernel_start : nullptr;
    hipEvent_t stop = s0 + n >= num_seqs ? kernel_stop : nullptr;
    if (shared) {
      pa::PrefixArgs p{};
      p.q = a.q;
      p.k_cache = a.k_cache;
      p.v_cache = a.v_cache;
      p.block_tables = a.block_tables;
      p.context_lens = a.context_lens;
      p.scale_log2 = a.scale_log2;
      p.num_seqs = (int)n;
      p.num_q_heads = num_q_heads;
      p.num_kv_heads = num_kv_heads * groups;  // (the pass takes sub-groups as heads)
      p.kv_split = groups;
      p.head_dim = head_dim;
      p.block_size = block_size;
      p.max_blocks_per_seq = max_blocks_per_seq;
      p.num_blocks = num_blocks;
      p.max_context_len = max_context_len;
      p.max_chunks = max_chunks > 0 ? max_chunks : 1;  // (the workgroups of chunk 0 write pre_len)
      p.pre_len = a.ws.pre_len;
      p.pre_o = a.ws.pre_o;
      p.pre_lse = a.ws.pre_lse;
      if (pa::launch_prefix(p, stream, start) != hipSuccess) return PA_ERR_HIP;
      start = nullptr;
      a.pre_len = a.ws.pre_len;
      a.pre_o = a.ws.pre_o;
      a.pre_lse = a.ws.pre_lse;
    }
    if (pa::launch_decode(a, stream, start, stop) != hipSuccess) return PA_ERR_HIP;
  }
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_decode_timed(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens, float scale,
                    int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads,
                    int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                    int64_t num_blocks, int32_t max_context_len, int32_t num_workers,
                    void* workspace, size_t workspace_bytes, hipStream_t stream,
                    hipEvent_t kernel_start, hipEvent_t kernel_stop) {
  return decode_impl(out, q, nullptr, nullptr, nullptr, k_cache, v_cache, block_tables,
                     context_lens, scale, num_kv_heads, num_seqs, num_q_heads, head_dim,
                     block_size, max_blocks_per_seq, num_blocks, max_context_len, num_workers,
                     workspace, workspace_bytes, stream, kernel_start, kernel_stop);
}

int pa_decode_append_timed(void* out, const void* q, const void* k_new, const void* v_new,
                           const int64_t* slot_mapping, void* k_cache, void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens, float scale,
                           int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads,
                           int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                           int64_t num_blocks, int32_t max_context_len, int32_t num_workers,
                           uint32_t flags, void* workspace, size_t workspace_bytes,
                           hipStream_t stream, hipEvent_t kernel_start, hipEvent_t kernel_stop) {
  if (num_seqs > 0 && (!k_new || !v_new || !slot_mapping)) return PA_ERR_INVALID_ARG;
  return decode_impl(out, q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables,
                     context_lens, scale, num_kv_heads, num_seqs, num_q_heads, head_dim,
                     block_size, max_blocks_per_seq, num_blocks, max_context_len, num_workers,
                     workspace, workspace_bytes, stream, kernel_start, kernel_stop, flags);
}

int pa_decode_append(void* out, const void* q, const void* k_new, const void* v_new,
                     const int64_t* slot_mapping, void* k_cache, void* v_cache,
                     const int32_t* block_tables, const int32_t* context_lens, float scale,
                     int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads,
                     int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                     int64_t num_blocks, int32_t max_context_len, int32_t num_workers,
                     uint32_t flags, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  return pa_decode_append_timed(out, q, k_new, v_new, slot_mapping, k_cache, v_cache,
                                block_tables, context_lens, scale, num_kv_heads, num_seqs,
                                num_q_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                                max_context_len, num_workers, flags, workspace, workspace_bytes,
                                stream, nullptr, nullptr);
}

int pa_decode_append_noalloc(void* out, const void* q, const void* k_new, const void* v_new,
                             const int64_t* slot_mapping, void* k_cache, void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens,
                             float scale, int32_t num_kv_heads, int32_t num_seqs,
                             int32_t num_q_heads, int32_t head_dim, int32_t block_size,
                             int32_t max_blocks_per_seq, int64_t num_blocks,
                             int32_t max_context_len, int32_t num_workers, uint32_t flags,
                             hipStream_t stream) {
  if (num_seqs > 0 && (!k_new || !v_new || !slot_mapping)) return PA_ERR_INVALID_ARG;
  return decode_impl(out, q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables,
                     context_lens, scale, num_kv_heads, num_seqs, num_q_heads, head_dim,
                     block_size, max_blocks_per_seq, num_blocks, max_context_len, num_workers,
                     nullptr, 0, stream, nullptr, nullptr, flags, /*static_scratch=*/true);
}

int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens, float scale,
              int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
              int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
              int32_t max_context_len, int32_t num_workers, void* workspace,
              size_t workspace_bytes, hipStream_t stream) {
  return pa_decode_timed(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                         num_kv_heads, num_seqs, num_q_heads, head_dim, block_size,
                         max_blocks_per_seq, num_blocks, max_context_len, num_workers, workspace,
                         workspace_bytes, stream, nullptr, nullptr);
}

int pa_read_probe(const void* buf, int64_t bytes, const int32_t* tile_order, int64_t num_tiles,
                  int32_t tile_bytes, uint32_t* sink, hipStream_t stream, hipEvent_t kernel_start,
                  hipEvent_t kernel_stop) {
  if (!buf || !sink || bytes <= 0 || (bytes & 15) || (reinterpret_cast<uintptr_t>(buf) & 15))
    return PA_ERR_INVALID_ARG;
  if (tile_order && (num_tiles <= 0 || tile_bytes < 16 || (tile_bytes & 15) || bytes < tile_bytes ||
                     num_tiles > ((int64_t)1 << 40) / tile_bytes))
    return PA_ERR_INVALID_ARG;
  const int32_t w = auto_workers();  // 2 per compute unit
  if (w < 0) return w;
  (void)hipGetLastError();
  const hipError_t e = pa::launch_read_probe(buf, bytes, tile_order, num_tiles, tile_bytes, sink,
                                             4 * w, stream, kernel_start, kernel_stop);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, const int32_t* context_lens,
               const int32_t* query_start, int32_t num_tokens, float scale,
               int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
               int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
               int32_t max_context_len, int32_t max_query_len, hipStream_t stream) {
  if (num_seqs < 0 || num_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_blocks_per_seq <= 0 || num_blocks <= 0 || max_context_len < 0 || max_query_len < 0 ||
      !std::isfinite(scale))
    return PA_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (!block_size_supported(block_size) || !head_dim_supported(head_dim))
    return PA_ERR_UNSUPPORTED;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size ||
      max_query_len > max_context_len)
    return PA_ERR_INVALID_ARG;
  if (num_seqs == 0 || max_query_len == 0 || num_tokens == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
    return PA_ERR_INVALID_ARG;
  const int64_t G = num_q_heads / num_kv_heads;
  const int64_t tile_groups =
      ceil_div((int64_t)max_query_len * G, pa::kPrefillWaves * pa::kPrefillWaveRows);
  if (((int64_t)num_seqs * num_kv_heads + 7) / 8 * 8 * tile_groups > 0x7fffffff)
    return PA_ERR_UNSUPPORTED;
  pa::PrefillArgs a{};
  a.out = static_cast<pa::half_t*>(out);
  a.q = static_cast<const pa::half_t*>(q);
  a.k_cache = static_cast<const pa::half_t*>(k_cache);
  a.v_cache = static_cast<const pa::half_t*>(v_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.num_tokens = num_tokens;
  // the kernel takes a positive factor: a negative scale becomes a sign flip
  // of q (exact), and a zero one a factor far below any logit's resolution
  const double sl2 = std::fabs((double)scale) * 1.4426950408889634;  // log2(e) = 1 / ln 2
  a.scale_log2 = (float)(sl2 > 1e-30 ? sl2 : 1e-30);
  a.negate_q = scale < 0.0f ? 1 : 0;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.max_context_len = max_context_len;
  a.max_query_len = max_query_len;
  a.tile_groups = (int)tile_groups;
  (void)hipGetLastError();
  return pa::launch_prefill(a, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"
