// Internal declarations shared by the library's translation units (not ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

typedef _Float16 half_t;
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef unsigned int uint4_t __attribute__((ext_vector_type(4)));

constexpr int kBlockSize = 16;    // token slots per block (the default; 8 and 32 also built)
constexpr int kChunk = 8;         // fp16 elements per 16-byte chunk
constexpr int kGroupTokens = 64;  // tokens one wave handles per step of its loop (a "unit")
constexpr int kWorkersPerCU = 2;  // decode waves per compute unit
constexpr int kMaxWorkers = 1 << 16;
constexpr int kMaxGroup = 4;      // query heads per KV head the decode kernel holds
// Sequences one decode launch takes (their unit offsets and lengths sit in
// LDS, 8 bytes each); the host splits larger batches into several launches.
constexpr int kMaxSeqsPerLaunch = 4096;

// LDS exchange between a decode workgroup's two waves: cut pieces the
// streamer hands to the merger (a ring of kRing) and the control words.
constexpr int kRing = 4;
enum { kCtlRingMade = 0, kCtlRingTaken, kCtlDone };
// Bound on every wait between the waves (about 0.5 s of s_sleep): a wait
// that long means a broken invariant, and the kernel then ends with wrong
// results rather than never, and sets the workspace's status word.
constexpr int kSpinLimit = 1 << 23;

// Decode workspace.  Partial slots first: one per (sequence, KV head) run
// (the piece that starts it) and one per share (the piece that starts the
// share inside a run), each holding for 4 query-head rows a (max, sum) pair
// and a D-vector of unnormalised fp32 output.  Then, against the workspace's
// end, one arrival counter per run, zero between calls.
struct DecodeWorkspace {
  float* ml;      // [slots][4][2]
  float* o;       // [slots][4][D]
  int* counters;  // [S][Hkv] units arrived
  uint64_t* trace;  // measurement builds only: [workers][kTraceSlots] at the workspace's start
  // Batches that share prefix blocks: per sequence the prefix length its
  // group's pass attended ([S]), and per (chunk, sequence, query head) that
  // pass's normalised row ([kPrefixMaxChunks][S][4 Hkv][D], fp16) and its
  // log2-domain log-sum-exp ([kPrefixMaxChunks][S][4 Hkv]); rows are indexed
  // (chunk * S + s) * num_q_heads + head.
  int* pre_len;
  half_t* pre_o;
  float* pre_lse;
  // the workspace's last int32: 0, or 1 once a bounded wait of a call gave up
  // (that call's results are undefined); the caller clears it
  int* status;
};

// Measurement builds (compiled with PA_DECODE_TRACE) put per-worker
// timestamps and counts at the start of the decode workspace.
#ifdef PA_DECODE_TRACE
constexpr bool kTrace = true;
#else
constexpr bool kTrace = false;
#endif
constexpr int kTraceSlots = 32;
// Measurement builds compiled with PA_DECODE_VALU form the decode's q.K and
// P.V with v_dot2_f32_f16 on the vector ALUs instead of the 4x4x4 MFMA.
#ifdef PA_DECODE_VALU
constexpr bool kValu = true;
#else
constexpr bool kValu = false;
#endif
enum {
  kTrEntry = 0,     // kernel entry (s_memrealtime, 100 MHz)
  kTrTables,        // lengths and unit offsets in LDS
  kTrFirstUnit,     // first unit's logits and softmax done (its K has arrived)
  kTrStreamEnd,     // streamer's last unit done
  kTrStoresIssued,  // fused append: new rows' stores issued
  kTrHelperEnd,     // helper wave done (last merge written)
  kTrXcc,           // XCC (XCD) id of the workgroup
  kTrUnits,         // units the streamer processed
  kTrPieces,        // cut pieces handed to the helper
  kTrMerges,        // runs the helper merged
  kTrHwId,          // HW_ID register (CU, SIMD) of the streamer
  kTrRingWait,      // streamer: ticks waiting for room in the ring to the helper
  kTrHelperBusy,    // helper: ticks in rounds (pieces written, counted, merged)
  kTrHelperRounds,  // helper: rounds
  kTrLastIters = 16,  // streamer: durations (ticks) of its last 8 iterations, oldest first
};

size_t decode_workspace_bytes(int64_t S, int64_t Hkv, int64_t D, int64_t workers);
// The decode attends up to 4 sub-groups per pass over the units (16 query
// rows, the columns of 16x16 MFMA tiles) and then needs one share slot per
// worker and sub-group of a pass; a count above 4 is rounded up to a
// multiple of 4 (empty sub-groups at the end), one copy of the batch per 4.
// The vector-ALU measurement build takes one sub-group per pass (one copy of
// the batch each).
inline int decode_split(int kv_split) {
  return (kv_split > 4 && !kValu) ? (kv_split + 3) / 4 * 4 : kv_split;
}
inline bool decode_wide(int split) { return split > 1 && !kValu; }
// share slots per worker: one per sub-group a pass attends
inline int decode_slot_factor(int split) { return decode_wide(split) ? (split < 4 ? split : 4) : 1; }
// Bytes of arrival counters a launch over S sequences keeps against the end
// of its workspace.
size_t decode_control_bytes(int64_t S, int64_t Hkv);

// The allocation-free decode takes its workspace from a file-scope device
// array of this size (one per GPU, held until the process ends).  Its last
// kStaticControlBytes, where the arrival counters live, are zeroed on the
// first call on each device.
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
constexpr size_t kStaticControlBytes = (size_t)1 << 20;
// The device address of the current device's array (looked up once per
// device; the first call also enqueues the counters' clear on `stream`).
hipError_t decode_static_scratch(hipStream_t stream, void** ptr);
// The layout of one launch in a workspace of `bytes` >= decode_workspace_bytes.
DecodeWorkspace decode_workspace_carve(void* base, size_t bytes, int64_t S, int64_t Hkv, int64_t D,
                                       int64_t workers);

hipError_t launch_reshape_and_cache(const half_t* k, const half_t* v, half_t* k_cache,
                                    half_t* v_cache, const int64_t* slot_mapping,
                                    int64_t num_tokens, int num_kv_heads, int head_dim,
                                    int block_size, int64_t num_blocks, hipStream_t stream);

// Whole-block copies from block src of (src_k, src_v) to block dst of
// (dst_k, dst_v); same_pool: one pool (copy-on-write), where src == dst is a
// no-op.
hipError_t launch_copy_blocks(const half_t* src_k, const half_t* src_v, half_t* dst_k,
                              half_t* dst_v, const int64_t* block_mapping, int64_t num_pairs,
                              int num_kv_heads, int head_dim, int block_size, int64_t src_blocks,
                              int64_t dst_blocks, bool same_pool, hipStream_t stream);

struct DecodeArgs {
  half_t* out;
  const half_t* q;
  const half_t* k_cache;
  const half_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float scale_log2;  // softmax scale times log2(e)
  int num_seqs;      // virtual sequences: one copy of the batch per sub-group
  int num_q_heads, num_kv_heads;
  int kv_split;      // query-head sub-groups per KV head: decode_split(ceil(G / kMaxGroup))
  int head_dim;
  int block_size;  // 8, 16 or 32
  int max_blocks_per_seq;
  int64_t num_blocks;
  int max_context_len;
  int num_workers;        // grid size: persistent workgroups sharing the work
  int spin_limit;         // bound on the waits between a worker's waves (kSpinLimit)
  DecodeWorkspace ws;
  // Fused append (null when plain decode): token s's new K and V rows
  // ([S][Hkv][D]), its slot, and writable views of the pools.  Position
  // context_lens[s] - 1 is then taken from these rows, not from the pools,
  // and the rows are stored into the slot.
  const half_t* k_new;
  const half_t* v_new;
  const int64_t* slot_mapping;
  half_t* k_cache_w;
  half_t* v_cache_w;
  // Batches whose sequences share prefix blocks (null otherwise): the
  // prefix pass attended positions [0, pre_len[s]) of sequence s for every
  // query head, in prefix_chunks(pre_len[s]) chunks, each a normalised row
  // and a log-sum-exp (DecodeWorkspace); the decode covers the positions
  // from pre_len[s] on and folds the pieces together.
  const int* pre_len;
  const half_t* pre_o;
  const float* pre_lse;
};

// Read-bandwidth probe (sequential when order is null, else num_tiles tiles
// of tile_bytes in the given order); grid workgroups of 256 lanes.
hipError_t launch_read_probe(const void* buf, int64_t bytes, const int32_t* order,
                             int64_t num_tiles, int32_t tile_bytes, uint32_t* sink, int grid,
                             hipStream_t stream, hipEvent_t start, hipEvent_t stop);

// One launch over a.num_seqs <= kMaxSeqsPerLaunch sequences.  Non-null
// events are bound to the kernel itself (its start and end times).
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream, hipEvent_t start,
                         hipEvent_t stop);

// Multi-query paged attention (chunked prefill).  One wave per tile of
// kPrefillWaveRows rows of one (sequence, KV head); a workgroup holds
// kPrefillWaves such tiles, and tile_groups workgroups cover the longest
// chunk: ceil(max_query_len * G / (kPrefillWaves kPrefillWaveRows)).
struct PrefillArgs {
  half_t* out;
  const half_t* q;
  const half_t* k_cache;
  const half_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;
  int num_tokens;    // rows of q and out
  float scale_log2;  // |softmax scale| times log2(e), at least 1e-30
  int negate_q;      // the scale is negative: q enters with its sign flipped
  int num_seqs, num_q_heads, num_kv_heads, head_dim;
  int block_size;    // 8, 16 or 32
  int max_blocks_per_seq;
  int64_t num_blocks;
  int max_context_len, max_query_len;
  int tile_groups;
};

// 32-key K/V steps a prefill workgroup keeps in its LDS ring (64 KiB at D = 128)
constexpr int kPrefillStages = 4;
constexpr int kPrefillWaveRows = 32;  // query rows of one wave
constexpr int kPrefillWaves = 4;      // waves of one workgroup

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

// Shared prefixes of a decode batch (pa_prefix.hip).  Sequences are taken
// in windows of kPrefixWindow; a group is a run of at least two consecutive
// sequences of one window, each holding its first 64-token units in the same
// physical blocks as the one before, and its prefix P the multiple of 64
// tokens they all hold so, short of every member's last position.  The pass
// attends each group's query rows (members x heads of a KV group, at most 32)
// to its P keys in prefix_chunks(P) chunks of prefix_chunk_len(P) keys (the
// last shorter), one workgroup of kPrefixWaves waves per (chunk, window, KV
// head).
constexpr int kPrefixWindow = 8;
constexpr int kPrefixWaves = 8;
constexpr int kPrefixMaxChunks = 4;
constexpr int kPrefixChunkKeys = 1024;  // chunk length while fewer than kPrefixMaxChunks
__host__ __device__ inline int prefix_chunks(int P) {
  if (P <= 0) return 0;
  const int c = (P + kPrefixChunkKeys - 1) / kPrefixChunkKeys;
  return c < kPrefixMaxChunks ? c : kPrefixMaxChunks;
}
__host__ __device__ inline int prefix_chunk_len(int P) {  // a multiple of kPrefixWaves x 32 keys
  constexpr int q = kPrefixWaves * 32;
  const int c = prefix_chunks(P);
  return c ? ((P + c - 1) / c + q - 1) / q * q : 0;
}
struct PrefixArgs {
  const half_t* q;
  const half_t* k_cache;
  const half_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float scale_log2;  // softmax scale times log2(e)
  int num_seqs, num_q_heads;
  int num_kv_heads;  // KV heads x kv_split: each query-head sub-group counts as a head
  int kv_split;      // sub-groups (of up to kMaxGroup query heads) per KV head
  int head_dim;
  int block_size;
  int max_blocks_per_seq;
  int64_t num_blocks;
  int max_context_len;
  int max_chunks;  // chunks of the longest possible prefix (grid dimension)
  int* pre_len;    // [S] out
  half_t* pre_o;   // out, as DecodeWorkspace
  float* pre_lse;  // out, as DecodeWorkspace
};
// `start`, when not null, is an event bound to this launch's start.
hipError_t launch_prefix(const PrefixArgs& a, hipStream_t stream, hipEvent_t start);

}  // namespace pa
