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

constexpr int kBlockSize = 16;    // token slots per block (the default; 8 and 32 also built)
constexpr int kChunk = 8;         // fp16 elements per 16-byte chunk
constexpr int kGroupTokens = 64;  // tokens one wave handles per step of its loop (a "unit")
constexpr int kWorkersPerCU = 2;  // decode waves per compute unit
constexpr int kMaxWorkers = 1 << 16;
// Sequences one decode launch takes (their unit offsets and lengths sit in
// LDS, 8 bytes each); the host splits larger batches into several launches.
constexpr int kMaxSeqsPerLaunch = 4096;

// Work split of one decode launch (see decode_kernel).  Every (sequence, KV
// head) run of n 64-token units keeps its first floor(n * F / 16) units (its
// head) in the static part, cut into one equal share per worker; the rest of
// the run (its tail) is cut, from its end, into dynamic chunks of 1, 1, 2, 4
// and then M units ("classes" 0, 1, 2, 3, 4, ...), that workers claim largest
// class first.  M >= 8 keeps the classes below kMaxClasses.  F defaults to
// kStaticSixteenths (all static: measured fastest while the claims' atomics
// share the streaming wave's in-order memory queue); the environment variable
// PA_DECODE_STATIC_SIXTEENTHS (0..16) overrides it per call.
constexpr int kStaticSixteenths = 16;
constexpr int kMaxClasses = 256;

// Claim counters of the dynamic chunks: kClaimPools of them, kClaimStride
// ints (4 KiB) apart so that they sit in different memory channels.
constexpr int kClaimPools = 8;
constexpr int kClaimStride = 1024;
constexpr size_t kClaimBytes = (size_t)kClaimPools * kClaimStride * sizeof(int);

// LDS exchange between a decode workgroup's three waves: cut pieces the
// streamer hands to the merger (a ring of kRing), chunks the claimer has
// claimed for the streamer (at most kClaimDepth queued, claimed on the
// streamer's request), and the control words.
constexpr int kRing = 4;
constexpr int kClaimDepth = 2;
enum { kCtlRingMade = 0, kCtlRingTaken, kCtlClaimsMade, kCtlClaimsTaken, kCtlClaimsWanted, kCtlDone };
// Bound on every wait between the waves (about 0.5 s of s_sleep): a wait
// that long means a broken invariant, and the kernel then ends with wrong
// results rather than never.
constexpr int kSpinLimit = 1 << 23;

// Dynamic chunks of one run with a tail of b units when the top chunks are M
// units long.
__host__ __device__ inline int tail_chunks(int b, int M) {
  return b <= 2 ? b : b <= 4 ? 3 : b <= 8 ? 4 : 4 + (b - 8 + M - 1) / M;
}

// Decode workspace: one arrival counter per (sequence, KV head) run, the
// claim counters of the dynamic chunks, then the partial slots: one per run
// (the first piece of its head), one per worker (a piece that starts its
// share) and one per dynamic chunk, each holding for 4 query-head rows a
// (max, sum) pair and a D-vector of unnormalised fp32 output.
struct DecodeWorkspace {
  int* counters;  // [S][Hkv], zero between calls
  int* claims;    // [kClaimPools * kClaimStride], zero between calls
  float* ml;      // [slots][4][2]
  float* o;       // [slots][4][D]
};

// Partial slots a launch over S sequences of at most max_len tokens can use.
int64_t decode_max_slots(int64_t S, int64_t Hkv, int64_t max_len, int64_t workers);
size_t decode_workspace_bytes(int64_t S, int64_t Hkv, int64_t D, int64_t max_len, int64_t workers);
DecodeWorkspace decode_workspace_carve(void* base, int64_t S, int64_t Hkv, int64_t max_len,
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
  int num_seqs, num_q_heads, num_kv_heads, head_dim;
  int block_size;  // 8, 16 or 32
  int max_blocks_per_seq;
  int64_t num_blocks;
  int max_context_len;
  int num_workers;        // grid size: persistent waves sharing the work
  int static_sixteenths;  // static share of each run, in sixteenths (0..16)
  DecodeWorkspace ws;
};

// One launch over a.num_seqs <= kMaxSeqsPerLaunch sequences.  Non-null
// events are bound to the kernel itself (its start and end times).
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream, hipEvent_t start,
                         hipEvent_t stop);

// Multi-query paged attention (chunked prefill).  One wave per tile of 32
// rows of one (sequence, KV head); a workgroup holds 4 such tiles, and
// tile_groups workgroups cover the longest chunk: ceil(max_query_len * G / 128).
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

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

}  // namespace pa
