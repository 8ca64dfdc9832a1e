/*
 * pa.h -- C ABI of the paged KV-cache decode library for AMD Instinct MI355X
 * (gfx950).
 *
 * The library implements the decode-step hot path of paged attention: the KV
 * cache of every sequence lives in fixed blocks of token slots that may sit
 * anywhere in one shared pool, and a per-sequence block table maps logical
 * block j to its physical block.  Sources (web pages, by title and section):
 *
 *   [AQ] "PagedAttention and Continuous Batching Explained (2026)", aquanode.io
 *        - "PagedAttention: a block table for the KV cache": 16-token blocks,
 *          per-request block table, the kernel reads through the table, blocks
 *          need not be contiguous, blocks are shared with copy-on-write.
 *        - "Why the KV cache is the problem": one K and one V vector per layer
 *          per token; the cache grows by one entry per token ("TL;DR").
 *        - "FAQ": the attention computed is the ordinary one.
 *   [TT] "KV Cache in Serving Engines: PagedAttention, Continuous Batching, and
 *        Prefix Caching", ttlab - section 2 "Blocks and Block Tables" (a block
 *        is taken only when the last is full; only the last block is partly
 *        empty; the computation is that of a contiguous array) and "Sharing
 *        Blocks" (reference counts; copy when a holder appends).
 *   [AG] "Continuous batching and paged attention", abhi-g.dev - "Paged
 *        attention": K and V are gathered through the block table.
 *   [CB] "Continuous batching, paged attention, prefix caching",
 *        backplane.click - "Prefix caching": one stored copy of a prompt
 *        prefix serves every request that starts with it.
 *
 * Departures from the plain decode interface (pa_reshape_and_cache,
 * pa_copy_blocks, pa_decode_workspace_size(num_seqs, num_q_heads, head_dim,
 * max_context_len), pa_decode without a pool size or worker count, pools
 * [NB][Hkv][16][D]), each for a reason stated where it applies:
 *  - the pools are tiled inside each (block, head) tile (layout below): the
 *    tile stays BS*D contiguous elements, and the order inside it gives the
 *    kernels' 16-byte loads the operand layouts of their matrix instructions;
 *  - pa_decode and pa_copy_blocks take num_blocks, the pool size (as
 *    pa_reshape_and_cache does), so that ids outside the pool are skipped
 *    instead of read or written out of bounds; token and pair counts are
 *    int64;
 *  - pa_decode takes num_workers (0 = automatic), the size of its
 *    persistent grid, and pa_decode_workspace_size takes num_kv_heads and
 *    num_workers besides num_q_heads: the workspace holds one partial
 *    result per (sequence, KV head) run and one per worker;
 *  - the library keeps two pieces of state: a per-device cache of the
 *    compute-unit count and the device array of pa_decode_append_noalloc;
 *  - further entry points: the timed variants, the fused append
 *    (pa_decode_append, with the shared-prefix flag, and its allocation-free
 *    form), block swaps, the multi-query (chunked prefill) kernel, and
 *    pa_read_probe, which is for measurement only and not part of the path.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Element types: K, V, q and out are IEEE fp16; block tables and context
 *    lengths int32; slot indices and block pairs int64; scale fp32.
 *  - Block size BS: 16 token slots by default ([AQ], [TT]); 8 and 32 are the
 *    variants ([AQ] "FAQ": smaller blocks waste less of the last block but
 *    cost more table entries).  Each entry point states the sizes it takes.
 *  - Pool layout (part of this ABI).  With NB physical blocks, Hkv KV heads
 *    and head dimension D (64 or 128):
 *        K pool: fp16 [NB][Hkv][D/8][BS][8]
 *                element (block b, head h, slot offset o, dim d) at
 *                ((((b*Hkv + h)*(D/8) + d/8)*BS + o)*8 + d%8)
 *        V pool: fp16 [NB][Hkv][BS/8][D][8]
 *                element (b, h, o, d) at ((((b*Hkv + h)*(BS/8) + o/8)*D + d)*8 + o%8)
 *    so one (block, head) tile is BS*D contiguous elements in both pools.
 *  - A slot index is  physical_block * BS + offset  (offset < BS).
 *  - Pointers are device pointers unless stated; all buffers are owned and
 *    allocated by the caller.  The library allocates nothing and keeps no
 *    state beyond a per-device cache of the compute-unit count and the
 *    device array of pa_decode_append_noalloc; it never synchronises and
 *    never reads device data on the host.
 *  - Every call only enqueues work on `stream` (0 = the null stream) and
 *    returns.  Faults inside a kernel surface at the caller's next
 *    synchronisation.  The library clears the HIP error state on entry.
 *  - Return value: PA_OK (0) or a negative PA_ERR_* code; argument errors are
 *    detected on the host before anything is enqueued.
 *  - Data preconditions that the host cannot check (slot and block ids inside
 *    the pool, table entries valid for every block a length covers, distinct
 *    slots, non-overlapping copy pairs) are the caller's.  The kernels never
 *    access memory outside the pools for ids outside [0, NB): such slots,
 *    pairs and blocks are skipped, which leaves results undefined but safe.
 */
#ifndef PAGED_KV_PA_H
#define PAGED_KV_PA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1, /* null pointer, negative or inconsistent size     */
  PA_ERR_UNSUPPORTED = -2, /* head_dim not 64/128, block size, sizes > 2^31 */
  PA_ERR_WORKSPACE = -3,   /* workspace missing, misaligned or too small      */
  PA_ERR_HIP = -4,         /* a HIP call or kernel launch failed              */
  PA_ERR_SCRATCH_LIMIT = -5, /* pa_decode_append_noalloc: batch above its array */
};

#define PA_BLOCK_SIZE 16 /* the default block size; 8 and 32 are also accepted */

/*
 * Append: write each new token's K and V rows into its slot ([AQ] "TL;DR",
 * [TT] "Blocks and Block Tables").
 *
 *   k, v          fp16 [num_tokens][num_kv_heads][head_dim], contiguous
 *   k_cache       K pool (layout above), v_cache V pool
 *   slot_mapping  int64 [num_tokens]; token t goes to slot slot_mapping[t];
 *                 negative = padding, skipped; >= num_blocks*BS is skipped
 *   Two tokens with the same non-negative slot in one call race (precondition).
 *   The write is a bit copy.  num_tokens == 0 is a no-op.  block_size 8, 16, 32.
 */
int pa_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int64_t num_tokens,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int64_t num_blocks, hipStream_t stream);

/*
 * Copy-on-write: for each pair (src, dst) copy the whole block, K and V, all
 * KV heads ([TT] "Sharing Blocks"; [AQ] sharing bullet of "PagedAttention:
 * a block table for the KV cache").
 *
 *   block_mapping int64 [num_pairs][2] = (src, dst), device memory
 *   Pairs with src == dst, or an id outside [0, num_blocks), are skipped.
 *   Preconditions: dsts distinct and none of them is also a src.
 *   Reference counting and the decision to copy are the caller's
 *   (pa_block_manager.h makes both).  block_size 8, 16 or 32.
 */
int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping,
                   int64_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int64_t num_blocks, hipStream_t stream);

/*
 * Swap: copy whole blocks, K and V, all KV heads, between two pools of the
 * same layout -- a request's blocks out to host memory when it is preempted
 * and back when it resumes ("Continuous batching and paged attention",
 * "Why they depend on each other": preemption by recomputation or by swap
 * to host memory).
 *
 *   src_k, src_v  source pools (src_num_blocks blocks), dst_k, dst_v the
 *                 destination pools (dst_num_blocks); either side may be host
 *                 memory from hipHostMalloc (pinned, device-accessible): the
 *                 kernel reads or writes it directly over the host link
 *   block_mapping int64 [num_pairs][2] = (src block, dst block), in device
 *                 memory or pinned host memory
 *   Pairs with an id outside its pool are skipped.  Destination blocks must be
 *   distinct.  The pools must differ (within one pool use pa_copy_blocks).
 *   block_size 8, 16 or 32.  The copy is a bit copy.
 */
int pa_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                   const int64_t* block_mapping, int64_t num_pairs, int32_t num_kv_heads,
                   int32_t head_dim, int32_t block_size, int64_t src_num_blocks,
                   int64_t dst_num_blocks, hipStream_t stream);

/*
 * Number of decode workers pa_decode uses when it is passed num_workers == 0:
 * 2 per compute unit of the current HIP device.  A worker is one workgroup of
 * two 64-lane wavefronts: one streams K and V, one writes and merges the
 * partial results of cut sequences.
 * Returns a negative PA_ERR_* code if the device cannot be queried.
 */
int32_t pa_decode_num_workers(void);

/*
 * Workspace bytes pa_decode needs for these sizes; max_context_len and
 * num_workers as for pa_decode (0 workers = automatic, on the current
 * device).  Returns 0 for invalid sizes (num_q_heads not a multiple of
 * num_kv_heads included).  The workspace holds, from its start, the partial
 * results of sequences cut between workers (one per (sequence, KV head)
 * run and one per worker, 4 query-head rows each; with G > 4 query heads
 * per KV head each sequence counts ceil(G / 4) times, above 4 rounded up to
 * a multiple of 4, here and below, and each worker min(ceil(G / 4), 4)
 * times), then
 * the shared-prefix pass's results (PA_DECODE_SHARED_BLOCKS: per sequence
 * its prefix length, per (chunk, sequence, query head) up to 4 normalised
 * fp16 rows and their log-sum-exps) and, against its end, one arrival
 * counter per (sequence, KV head).  The size does not depend on
 * max_context_len (kept for a stable signature).
 * Batches above 4096 sequences need no more than 4096 do (they run as
 * several launches).
 */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_context_len, int32_t num_workers);

/*
 * Decode attention through the block table ([AQ] "PagedAttention: a block
 * table for the KV cache" and "FAQ"; [TT] "Blocks and Block Tables"; [AG]
 * "Paged attention").  For sequence s and query head h, with
 * G = num_q_heads / num_kv_heads and KV head kh = h / G:
 *
 *   out[s][h] = softmax_i( scale * q[s][h] . K_s[kh][i] ) V_s[kh][i],
 *               i = 0 .. context_lens[s]-1,
 *
 * where position i of sequence s is slot offset i%BS of physical block
 * block_tables[s][i/BS] (BS = block_size: 8, 16 or 32).  The unused tail of
 * the last block never enters the result, whatever it holds (NaN included).
 * A length of 0 gives a zero row.
 *
 *   out               fp16 [num_seqs][num_q_heads][head_dim]
 *   q                 fp16 [num_seqs][num_q_heads][head_dim]
 *   block_tables      int32 [num_seqs][max_blocks_per_seq] (row stride
 *                     max_blocks_per_seq); entries past ceil(len/BS) unread
 *   context_lens      int32 [num_seqs]; values are clamped to [0, max_context_len]
 *   scale             softmax scale (e.g. 1/sqrt(head_dim)), finite
 *   max_context_len   host-known upper bound of context_lens, at most
 *                     max_blocks_per_seq*BS
 *   num_workers       0 = automatic (pa_decode_num_workers()); else the number
 *                     of persistent workgroups that share the work.  Every
 *                     (sequence, KV head) is cut into 64-token units; all
 *                     units, end to end, go into equal contiguous shares,
 *                     one per worker.  A sequence cut into several pieces
 *                     is merged by the last piece to finish (log-sum-exp
 *                     rescaling).
 *   workspace         device buffer of at least pa_decode_workspace_size(
 *                     num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
 *                     num_workers) bytes, 256-byte aligned, ZERO-FILLED before
 *                     its first use; each call leaves its counters at zero
 *                     again, so a workspace is reusable without clearing,
 *                     also by calls of smaller shapes.  Two calls
 *                     that overlap in time must not share one workspace.
 *                     Its last int32 is a status word: 0, or 1 once a
 *                     bounded wait between a worker's two waves (about
 *                     0.5 s; a broken invariant) gave up.  The kernel then
 *                     still ends, with that call's results undefined and
 *                     counters possibly non-zero: the caller, reading the
 *                     word after its synchronisation, zeroes the workspace
 *                     before reusing it.  (PA_DECODE_SPIN_LIMIT=n in the
 *                     environment lowers the bound to n polls, for tests.)
 *
 * Accumulation is fp32 (products of fp16 inputs; the softmax weights enter
 * the value product rounded to fp16); out is rounded to nearest even fp16.
 * Any G >= 1: the grouped query heads of a KV head share each K and V load.
 * Up to 4 are the rows of a 4x4x4 matrix instruction; a group of G > 4 is
 * taken as ceil(G / 4) sub-groups of up to 4 query heads, up to 16 query
 * heads per pass over K and V, as the columns of 16x16x32 matrix tiles.
 * Above 16 the passes are copies of the batch in the same launch, whose
 * reads of one block fall at the same time (the L2 serves most repeats).
 * num_seqs == 0 is a no-op.
 */
int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens, float scale,
              int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads,
              int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
              int64_t num_blocks, int32_t max_context_len, int32_t num_workers,
              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pa_decode with timing: identical work and results; in addition the caller's
 * events (created with timing enabled, either may be NULL) are bound to the
 * kernel itself through hipExtLaunchKernel, so hipEventElapsedTime(start,
 * stop) is the decode kernel's execution time (first launch's start to last
 * launch's end for batches above 4096 sequences), without the queueing and
 * dispatch latency that events recorded around the call also include.  For
 * profiling callers; num_seqs == 0 leaves both events untouched.
 */
int pa_decode_timed(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens, float scale,
                    int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads,
                    int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                    int64_t num_blocks, int32_t max_context_len, int32_t num_workers,
                    void* workspace, size_t workspace_bytes, hipStream_t stream,
                    hipEvent_t kernel_start, hipEvent_t kernel_stop);

/*
 * Append and decode in one launch: the same results as
 *     pa_reshape_and_cache(k_new, v_new, k_cache, v_cache, slot_mapping,
 *                          num_tokens = num_seqs, ...)
 * followed by pa_decode(...) with the same pools, when token s is sequence
 * s's new token at position context_lens[s] - 1 (the decode step of [AQ]
 * "TL;DR": one new K and V entry per sequence, then attention over the whole
 * cache) and slot_mapping[s] is the slot the block table gives that position.
 *
 *   k_new, v_new   fp16 [num_seqs][num_kv_heads][head_dim], 16-byte aligned
 *   slot_mapping   int64 [num_seqs]: the slot of token s; negative (or past
 *                  the pool) = the row is attended but not stored
 *   flags          0, or PA_DECODE_SHARED_BLOCKS when sequences of the batch
 *                  share blocks (prefix caching, forks; [TT] "Sharing
 *                  Blocks", [CB] "Prefix caching"); any other bit is
 *                  PA_ERR_INVALID_ARG.  With the flag a prefix pass runs
 *                  first: in each aligned window of 8 consecutive
 *                  sequences, runs of at least two sequences whose tables
 *                  start with the same physical blocks form a group, whose
 *                  prefix P is the multiple of 64 tokens every member holds
 *                  in those blocks short of its last position (the new
 *                  token's).  The pass attends all the group's query rows
 *                  (members x up to 4 query heads of a KV head, at most
 *                  32; larger groups of query heads in sub-groups) to
 *                  those P positions once, and the decode covers each
 *                  member's positions from P on, starting its online
 *                  softmax from that result.  Results equal the flagless
 *                  ones up to rounding.  Measured on MI355X (256 sequences
 *                  in 32 groups of 8 sharing 1,024-token prefixes): 104 us
 *                  for both kernels, 1.11x the distinct K/V bytes read from
 *                  HBM, against 171 us and 2.78x when every sequence read
 *                  its prefix.
 *   the rest       as pa_decode; k_cache and v_cache are written (the new
 *                  rows only)
 *
 * The attention takes position context_lens[s] - 1 from k_new / v_new, not
 * from the pools, so nothing in the launch reads what it writes.  A sequence
 * with context length 0 appends nothing and gets a zero row.  Errors as
 * pa_decode, and PA_ERR_INVALID_ARG for a null or misaligned new row.
 *
 * One launch: each worker stores the new rows of the runs that end in its
 * share after its last unit (scattered partial-line writes, slow to
 * complete; a worker's memory operations complete in order, so inside its
 * stream they would hold back its K/V loads).  Measured on MI355X
 * (Llama-3.1-8B layer, 64 sequences): 59.1 us per step, against 62.7 us for
 * pa_reshape_and_cache then pa_decode.
 */
#define PA_DECODE_SHARED_BLOCKS 1u /* flag: sequences share blocks (prefix caching, forks) */
int pa_decode_append(void* out, const void* q, const void* k_new, const void* v_new,
                     const int64_t* slot_mapping, void* k_cache, void* v_cache,
                     const int32_t* block_tables, const int32_t* context_lens, float scale,
                     int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads,
                     int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                     int64_t num_blocks, int32_t max_context_len, int32_t num_workers,
                     uint32_t flags, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/*
 * pa_decode_append for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, work and results as pa_decode_append, without the
 * workspace: the partial results and arrival counters live in a device array
 * of 32 MiB that the library holds in each GPU's memory from its first use
 * until the process ends (a file-scope __device__ array, reached through
 * hipGetSymbolAddress once per device).  Nothing here allocates or frees.
 *
 *   - The first call on a device also enqueues, on `stream`, a kernel that
 *     zeroes the array's last 1 MiB, where the counters live (a graph
 *     captured around that first call replays it: harmless).  Every call
 *     leaves the counters at zero again.
 *   - All calls on one GPU share the array: calls that overlap in time on one
 *     GPU (different streams, or concurrent graph replays) race and give
 *     wrong results.  Serialise them, or use pa_decode_append with a
 *     workspace per stream.
 *   - A batch whose workspace (pa_decode_workspace_size of the same sizes)
 *     exceeds 32 MiB returns PA_ERR_SCRATCH_LIMIT before anything is enqueued
 *     (e.g. a 128-sequence batch of 40 KV heads at 512 workers needs 12 MB).
 *   - Other errors as pa_decode_append.
 */
int pa_decode_append_noalloc(void* out, const void* q, const void* k_new, const void* v_new,
                             const int64_t* slot_mapping, void* k_cache, void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens,
                             float scale, int32_t num_kv_heads, int32_t num_seqs,
                             int32_t num_q_heads, int32_t head_dim, int32_t block_size,
                             int32_t max_blocks_per_seq, int64_t num_blocks,
                             int32_t max_context_len, int32_t num_workers, uint32_t flags,
                             hipStream_t stream);

/* pa_decode_append with the kernel-bound timing events of pa_decode_timed. */
int pa_decode_append_timed(void* out, const void* q, const void* k_new, const void* v_new,
                           const int64_t* slot_mapping, void* k_cache, void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens, float scale,
                           int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads,
                           int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                           int64_t num_blocks, int32_t max_context_len, int32_t num_workers,
                           uint32_t flags, void* workspace, size_t workspace_bytes,
                           hipStream_t stream, hipEvent_t kernel_start, hipEvent_t kernel_stop);

/*
 * Read-bandwidth probe, for measurement: the HBM read rate this device
 * reaches with the loads the decode kernel issues (16-byte non-temporal
 * vector loads), to read a kernel's rate against it beside the part's
 * nominal peak.  Not part of the decode path.
 *
 *   buf, bytes     device buffer, 16-byte aligned, bytes a multiple of 16
 *   tile_order     NULL: read buf once, sequentially.  Else int32
 *                  [num_tiles] on the device: read tiles of tile_bytes
 *                  (a multiple of 16) at byte offsets tile_order[t] *
 *                  tile_bytes, in that order (an entry outside buf reads
 *                  tile 0)
 *   sink           device uint32, zeroed by the caller: receives the XOR of
 *                  every 32-bit word read, so no read is skipped
 *   kernel_start/stop  optional timing events bound to the kernel, as in
 *                  pa_decode_timed
 */
int pa_read_probe(const void* buf, int64_t bytes, const int32_t* tile_order, int64_t num_tiles,
                  int32_t tile_bytes, uint32_t* sink, hipStream_t stream, hipEvent_t kernel_start,
                  hipEvent_t kernel_stop);

/*
 * Multi-query paged attention: each sequence's chunk of new query tokens
 * attends causally to its paged context -- chunked prefill ("KV Cache in
 * Serving Engines", section 3 "New Problem: Long Prefills Pause Decoding")
 * and the continuation after a prefix-cache hit (same page, section 4;
 * "PagedAttention and Continuous Batching Explained (2026)", "Prefix
 * caching").  The chunk's K and V must already be in the cache
 * (pa_reshape_and_cache).  With n = context_lens[s] and n_q its chunk length,
 * chunk row i sits at position p = n - n_q + i and, for query head h with KV
 * head kh = h / G,
 *
 *   out[t][h] = softmax_j( scale * q[t][h] . K_s[kh][j] ) V_s[kh][j],
 *               j = 0 .. p,   t = query_start[s] + i.
 *
 * A decode step is the case n_q = 1.
 *
 *   out, q            fp16 [num_tokens][num_q_heads][head_dim]
 *   query_start       int32 [num_seqs + 1], device memory, non-decreasing from 0:
 *                     rows query_start[s] .. query_start[s+1]-1 are sequence s's chunk
 *   num_tokens        rows of q and out (query_start[num_seqs] when consistent)
 *   block_tables, context_lens, scale, pools: as for pa_decode (context_lens
 *                     clamped to [0, max_context_len])
 *   max_query_len     host-known upper bound of every chunk length, at most
 *                     max_context_len; 0 = nothing to do
 * block_size 8, 16 or 32.  Any G = num_q_heads / num_kv_heads is accepted.  A chunk longer than its
 * context or than max_query_len, or reaching past num_tokens, is a broken
 * precondition: its rows are left unwritten (nothing outside q and out is
 * touched).  Accumulation is fp32; softmax weights enter the value product
 * rounded to fp16; out is rounded to nearest even.  No workspace.
 */
int pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, const int32_t* context_lens,
               const int32_t* query_start, int32_t num_tokens, float scale,
               int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
               int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
               int32_t max_context_len, int32_t max_query_len, hipStream_t stream);

/* Text for a PA_* code (static storage, never NULL). */
const char* pa_strerror(int code);

/* Library version: major*10000 + minor*100 + patch. */
int pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_PA_H */
