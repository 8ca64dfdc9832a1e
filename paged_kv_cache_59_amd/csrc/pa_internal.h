// Internal declarations shared by the library's translation units (not ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef _Float16 half_t;
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kBlockSize = 16;   // token slots per block
constexpr int kChunk = 8;        // fp16 elements per 16-byte chunk
constexpr int kGroupTokens = 64; // tokens one wave handles per step of its loop
constexpr int kWorkersPerCU = 2;  // decode waves per compute unit
constexpr int kMaxWorkers = 1 << 20;

// Decode workspace: one arrival counter per (sequence, KV head) run, then two
// partial slots per worker, each holding for 4 query-head rows a (max, sum)
// pair and a D-vector of unnormalised fp32 output.
struct DecodeWorkspace {
  int* counters;  // [S][Hkv], zero between calls
  float* ml;      // [2*workers][4][2]
  float* o;       // [2*workers][4][D]
};

size_t decode_workspace_bytes(int64_t S, int64_t Hkv, int64_t D, int64_t workers);
DecodeWorkspace decode_workspace_carve(void* base, int64_t S, int64_t Hkv, int64_t workers);

hipError_t launch_reshape_and_cache(const half_t* k, const half_t* v, half_t* k_cache,
                                    half_t* v_cache, const int64_t* slot_mapping,
                                    int64_t num_tokens, int num_kv_heads, int head_dim,
                                    int64_t num_blocks, hipStream_t stream);

hipError_t launch_copy_blocks(half_t* k_cache, half_t* v_cache, const int64_t* block_mapping,
                              int64_t num_pairs, int num_kv_heads, int head_dim,
                              int64_t num_blocks, hipStream_t stream);

struct DecodeArgs {
  half_t* out;
  const half_t* q;
  const half_t* k_cache;
  const half_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float scale_log2;  // softmax scale times log2(e)
  int num_seqs, num_q_heads, num_kv_heads, head_dim;
  int max_blocks_per_seq;
  int64_t num_blocks;
  int max_context_len;
  int num_workers;  // grid size: persistent waves sharing the work
  DecodeWorkspace ws;
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

}  // namespace pa
