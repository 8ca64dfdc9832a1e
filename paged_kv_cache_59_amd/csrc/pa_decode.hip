// Decode attention through the block table, for gfx950 (CDNA4, wave64).
//
// What is computed ("PagedAttention and Continuous Batching Explained (2026)",
// sections "PagedAttention: a block table for the KV cache" and "FAQ";
// "KV Cache in Serving Engines ...", section 2 "Blocks and Block Tables";
// "Continuous batching and paged attention", section "Paged attention"):
// for each sequence and query head, softmax(scale * q . K) V over the
// sequence's positions, where position i lives at slot i % 16 of physical
// block block_tables[s][i / 16].  The result is the ordinary attention; only
// the addresses of K and V come from the table.
//
// Design (the pages give none; decode reads every K/V byte once, so HBM
// bandwidth bounds it):
//  * Units and shares.  Each (sequence, KV head) pair is a run of 64-token
//    units (4 blocks each); all runs are laid end to end in (sequence, head)
//    order and cut into one equal contiguous share per worker of a fixed grid
//    of persistent workers.  Each worker finds its units through a prefix
//    sum of the lengths it keeps in LDS; the host never reads the lengths.
//    (Shares balanced at run time, by claimed chunks or by taking units from
//    slower workers' shares, were measured slower on MI355X: the claims'
//    lookahead, the extra cut pieces and their merges at the kernel's end
//    cost more than the per-XCD speed spread they remove.)
//  * A run cut between shares is merged by the last of its pieces to
//    arrive: each piece writes (max, sum, unnormalised output) through to
//    memory and adds its units to the run's counter; the piece that
//    completes the count merges with the log-sum-exp rescale and resets the
//    counter.  A piece that finds every other unit of its run already
//    counted merges at once, without counting.  Merges therefore happen
//    inside the stream, not after it.  One launch per decode.
//  * Consecutive shares run on one XCD (workgroups are handed to the 8 XCDs
//    in turn), so neighbouring runs, e.g. sequences sharing prefix blocks,
//    meet in the same L2.
//  * The grouped query heads of one KV head (G <= 4) are the 4 rows of the
//    4x4x4 16-block MFMA, so every K and V element loaded serves all G heads;
//    the G q rows stay in 1 KiB of LDS for the whole run (in registers they
//    would cost 64 per lane and halve the waves a SIMD holds).  A larger
//    group (Wide) is taken as kv_split = ceil(G / 4) sub-groups of up to 4
//    query heads, up to 4 of them (16 rows) per pass: the logits are
//    S^T = K Q^T on 16x16x32 MFMA tiles (16 tokens x 16 query rows), the
//    products O^T += V^T P^T on the same tiles (16 dims x 16 rows), so each
//    lane carries one query row's softmax state and the unit's VALU work
//    does not grow with G.  The merger sees kv_split x S virtual sequences,
//    sub-group j's copy of sequence s at j S + s, and a pass hands it one
//    piece per sub-group.  Above 4 sub-groups the count is rounded up to a
//    multiple of 4 and the unit order holds one copy of the batch per 4;
//    copy c's units lie exactly c / copies of the way along, so with equal
//    shares the workers that read one block for different copies read it at
//    the same time, and (for an even split of the workers into runs of 32
//    per XCD) on the same XCD, whose L2 serves the repeats.
//  * q . K: lane l owns token l of the 64; it loads its 16-byte chunks of the
//    K row (K pool [NB][Hkv][D/8][16][8]: for a fixed chunk the 64 lanes read
//    four contiguous 256-byte runs) and feeds them as the B operand, so the
//    dot products reduce inside the MFMA, with no cross-lane sums.
//  * Online softmax: running max per head (wave max per unit, DPP within rows
//    of 16), per-lane partial sums (one wave sum per run piece).
//  * The fp16 probabilities are transposed through 512 bytes of LDS so lane
//    4c+g holds head g's weights of tokens 4c..4c+3; the MFMA broadcast
//    (CBSZ=4, ABID=c) hands that quad to all 16 blocks.
//  * P . V: lane l owns output dims l and l+64; V pool [NB][Hkv][2][D][8] puts
//    8 consecutive tokens of one dim in 16 bytes, so for a fixed (block, half)
//    the 64 lanes read 1 KiB contiguous.
//  * Software pipeline: the next unit's K loads are issued once this unit's
//    logits are formed, its V loads once this unit's P.V is done, the table
//    entries two units ahead one iteration earlier still; every unit issues
//    the same loads (block ids past a run's end re-read its last block).  K
//    and V are read with non-temporal loads (each byte is used once).
//  * Positions at or past the length are removed by selection (logit -inf,
//    V element 0), never by multiplication, so NaN or huge values in the
//    unused tail of the last block cannot leak.
#include <mutex>
#include <type_traits>

#include <hip/hip_ext.h>

#include "pa_internal.h"

namespace pa {

namespace {


template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}

// Max within each row of 16 lanes, in every lane of the row (DPP: swap pairs,
// swap pairs of pairs, mirror halves, mirror the row).
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp<0x140>(x));  // row_mirror
  return x;
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}

// Max over the 64 lanes, in every lane: the four row results read out as scalars.
__device__ __forceinline__ float wave_max(float x) {
  x = row_max16(x);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Sum over the 64 lanes, in every lane (same pattern as wave_max).
__device__ __forceinline__ float wave_sum(float x) {
  x = row_sum16(x);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef _Float16 half2x __attribute__((ext_vector_type(2)));
__device__ __forceinline__ half4_t lo4(half8_t v) { return __builtin_shufflevector(v, v, 0, 1, 2, 3); }
__device__ __forceinline__ half4_t hi4(half8_t v) { return __builtin_shufflevector(v, v, 4, 5, 6, 7); }

__device__ __forceinline__ half8_t load_nt(const half_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const half8_t*>(p));
}

// K/V tile loads: non-temporal, every block is read once (measured 9-12%
// faster than loads through the caches on batches that share nothing).
// Prefix blocks that sequences share are read by the prefix pass instead.
__device__ __forceinline__ half8_t load_kv(const half_t* p) { return load_nt(p); }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Max and sum over lanes l, l ^ 16, l ^ 32 and l ^ 48 (the four lanes that
// hold one query row of a 16x16 tile), with the gfx950 cross-row swaps; all
// four lanes end with the same bits.
__device__ __forceinline__ float max_row4(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float sum_row4(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
__device__ __forceinline__ float4_t mfma16(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Measurement builds: a 100 MHz timestamp (the same clock on every CU), and
// the XCC_ID / HW_ID hardware registers of the wave.
__device__ __forceinline__ uint64_t stamp_now() {
  if constexpr (kTrace) return __builtin_amdgcn_s_memrealtime();
  else return 0;
}
[[maybe_unused]] __device__ __forceinline__ uint64_t xcc_id() {
  if constexpr (kTrace) return (uint64_t)__builtin_amdgcn_s_getreg((20) | (0 << 6) | (15 << 11));
  else return 0;
}
[[maybe_unused]] __device__ __forceinline__ uint64_t hw_id() {
  if constexpr (kTrace) return (uint64_t)__builtin_amdgcn_s_getreg((4) | (0 << 6) | (31 << 11));
  else return 0;
}

// A compiler-only ordering point for LDS exchanged between the waves of a
// workgroup.  The DS instructions of one wave execute in program order, so
// keeping the compiler from reordering (or caching) the accesses is enough;
// volatile or fenced accesses would instead make the compiler wait for every
// outstanding memory operation, draining the streamer's K/V pipeline.
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

// Loads and stores of the partial results, coherent across XCDs: stores write
// through to memory, loads bypass the caches (system scope, sc0 sc1).
__device__ __forceinline__ void store_through(float* p, float x) {
  __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ float load_through(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ int load_through_i(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
// 16 bytes at byte offset `off` of the buffer starting at `base` (uniform).
__device__ __forceinline__ float4_t load_through16(const float* base, int off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, 0x7fffffff, 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 17);  // sc0 sc1
}

}  // namespace

// Shared: the batch's shared prefixes were attended by the prefix pass (one
// pass per group over its common blocks, results in out and pre_lse); each
// run covers its sequence's positions from a.pre_len[s] on, and its result
// is folded together with the prefix pass's.
// Wide (more than 4 query heads per KV head): one pass over a unit attends
// up to 4 sub-groups, 16 query rows, as the columns of 16x16x32 MFMA tiles;
// the units enumerate one copy of the batch per 4 sub-groups (kv_split <= 4:
// the batch once), and each piece is handed to the merger once per
// sub-group, as the pieces of the sub-groups' copies (virtual sequences
// j Sr + s) would be.
template <int D, int BS, bool Fused, bool Shared, bool Wide>
__global__ __launch_bounds__(128) void decode_kernel(const DecodeArgs a) {
  constexpr int kChunks = D / kChunk;  // 16-byte chunks in one K row
  constexpr int kSets = D / 64;        // 64-dim ranges a lane covers in P.V
  constexpr int kF = D / 16;           // floats per lane of one partial in a merge
  constexpr int64_t kTile = (int64_t)BS * D;
  constexpr int NBU = kGroupTokens / BS;  // blocks per 64-token unit (8, 4 or 2)
  constexpr int kGroups = BS / kChunk;    // 8-token V groups per block
  static_assert(NBU * BS == kGroupTokens && kGroups * kChunk == BS, "block size 8, 16 or 32");
  static_assert(kChunks * kChunk == D && kSets * 64 == D, "head_dim must be 64 or 128");

  // measurement builds: this worker's stamps, written at its end
  uint64_t tr[kTraceSlots] = {};
  tr[kTrEntry] = stamp_now();
  // [S] units (per KV head) of the sequences before s, [S] its length
  extern __shared__ int seq_lds[];
  // Rows padded so that the 4 rows of one access fall in different LDS banks
  // (unpadded, rows 128 and 256 bytes apart share banks: 4-way conflicts).
  constexpr int kQRow = D + 8;  // halves per q row
  // (Wide: 16 rows of 64 weights, 144 bytes apart, so that the 16 rows of a
  // 16-byte access fall in distinct banks)
  constexpr int kPRow = Wide ? 64 + 8 : 64 + 16;  // halves per softmax-weight row
  constexpr int kRows = Wide ? 16 : 4;  // query rows a unit is attended for
  constexpr int kSub = Wide ? 4 : 1;    // sub-groups of 4 rows a pass can attend
  constexpr int kWT = D / 16;           // Wide: 16-dim tiles of the output and of V
  constexpr int kWK = D / 32;           // Wide: 32-dim steps of the logits
  static_assert(!(Wide && kValu), "the vector-ALU measurement build attends 4 rows");
  __shared__ __attribute__((aligned(16))) half_t p_lds[kRows * kPRow];
  __shared__ __attribute__((aligned(16))) half_t q_lds[kRows * kQRow];
  // streamer -> merger: cut pieces, a ring of kRing entries
  __shared__ __attribute__((aligned(16))) float ring_o[kRing][4 * D];
  __shared__ float ring_ml[kRing][8];
  __shared__ int ring_meta[kRing][4];  // sequence, KV head, partial slot, units
  __shared__ int ctl[4];  // ring produced/consumed, streamer done

  // Wave 0 streams the units.  Wave 1 takes every operation whose latency
  // would stall the streamer's in-order memory queue: it writes cut pieces
  // through, counts their arrivals and merges.
  const int role = threadIdx.x >> 6;
  const bool streamer = role == 0;
  const int lane = threadIdx.x & 63;
  const int nw = gridDim.x;
  // Logical worker numbering: runs of up to 32 consecutive logical workers
  // on one XCD (workgroup i runs on XCD i % 8), the runs dealt to the XCDs in
  // turn.  Consecutive shares then meet in one L2 (sequences that share
  // prefix blocks are adjacent), while every XCD still draws on the whole
  // batch (its speed then depends less on which sequences it holds).
  const int bx = (int)blockIdx.x;
  int kw = 1;  // run length: the largest power of two <= 32 dividing nw / 8
  if (nw % 8 == 0) {
    const int per_xcd = nw / 8;
    kw = min(per_xcd & -per_xcd, 32);
  }
  const int w = (nw % 8 == 0) ? ((bx / 8) / kw) * 8 * kw + (bx % 8) * kw + (bx / 8) % kw : bx;
  const int Sv = a.num_seqs;          // virtual sequences (slots, counters)
  const int Hkv = a.num_kv_heads;
  const int Hq = a.num_q_heads;
  // Sub-groups: a KV head with more than 4 query heads is taken as kv_split
  // sub-groups of up to 4 query heads; the merger, its counters and the
  // partial slots see Sv virtual sequences, sub-group s / Sr of sequence
  // s % Sr.
  const int split = a.kv_split;
  const int Sr = Sv / split;  // sequences of the batch (lengths, tables, new rows)
  // sequences in unit order (the unit tables); Wide: one copy of the batch
  // per 4 sub-groups (a split above 4 is a multiple of 4)
  const int S = !Wide ? Sv : split <= kSub ? Sr : Sv / kSub;
  const int n_sub = Wide ? min(split, kSub) : 1;  // sub-groups a pass attends
  const int G = Hq / Hkv;    // query heads per KV head
  auto sub_of = [&](int s) { return split == 1 ? 0 : s / Sr; };
  auto real_of = [&](int s) { return split == 1 ? s : s - s / Sr * Sr; };
  // (an empty sub-group, which rounds a count above 4 up to a multiple of 4,
  // has none)
  auto q_rows = [&](int s) { return split == 1 ? G : max(0, min(4, G - sub_of(s) * 4)); };
  // the q / out row of the first query head of run (s, h)
  auto q_row0 = [&](int s, int h) -> int64_t {
    return (int64_t)real_of(s) * Hq + h * G + sub_of(s) * 4;
  };
  // a virtual sequence's entry in the unit tables
  auto tab = [&](int s) {
    if constexpr (Wide) return split <= kSub ? real_of(s) : sub_of(s) / kSub * Sr + real_of(s);
    else return s;
  };
  // Wide: the first of the sub-groups a table entry's pass attends (kv_split
  // <= 4: the table holds the batch once, no division), the sequence of the
  // batch at table entry t, and the virtual sequence of the pass's sub-group u
  auto pass_sub0 = [&](int t) { return split <= kSub ? 0 : kSub * (t / Sr); };
  auto seq_of = [&](int t) {
    if constexpr (Wide) return split <= kSub ? t : t - t / Sr * Sr;
    else return real_of(t);
  };
  auto pass_seq = [&](int t, int u) { return (pass_sub0(t) + u) * Sr + seq_of(t); };
  int* const off_lds = seq_lds;
  int* const len_lds = seq_lds + S;
  int* const base_lds = seq_lds + 2 * S;  // Shared: the positions before unit 0 of s's runs

  auto units_for = [](int c) { return (c + kGroupTokens - 1) / kGroupTokens; };
  // units of each of s's runs (Shared: of the positions after its prefix pass's)
  auto run_units = [&](int s) {
    return units_for(Shared ? len_lds[s] - base_lds[s] : len_lds[s]);
  };

  // ---- lengths into LDS; zero the rows of empty sequences ----------------
  // (the lengths of up to 4 x 64 sequences are loaded at once: one memory
  // latency per 256 sequences rather than per 64)
  constexpr int kLenBatch = 4;
  int carry = 0;  // uniform
  for (int cb = 0; cb < S; cb += 64 * kLenBatch) {
    int len_in[kLenBatch], pre_in[kLenBatch];
#pragma unroll
    for (int b = 0; b < kLenBatch; ++b) {
      const int s = cb + 64 * b + lane;
      len_in[b] = s < S ? a.context_lens[seq_of(s)] : 0;
      pre_in[b] = (Shared && s < S) ? a.pre_len[seq_of(s)] : 0;
    }
#pragma unroll
    for (int b = 0; b < kLenBatch; ++b) {
      const int c0 = cb + 64 * b;
      if (c0 >= S) break;
      const int s = c0 + lane;
      const int c = s < S ? min(max(len_in[b], 0), a.max_context_len) : 0;
      // Shared: positions [0, pre) were attended by the prefix pass (pre <= c - 1)
      const int pre = (Shared && s < S) ? min(max(pre_in[b], 0), max(c - 1, 0)) : 0;
      const int n = units_for(c - pre);
      const int incl = wave_inclusive_scan(n, lane);
      if (streamer && s < S) {
        off_lds[s] = carry + incl - n;
        len_lds[s] = c;
        if constexpr (Shared) base_lds[s] = pre;
      }
      carry += __builtin_amdgcn_readlane(incl, 63);
      // (the first sub-group's copy clears every row of the sequence)
      uint64_t empty = streamer ? __ballot(s < Sr && n == 0 && (s % nw) == w) : 0;
      while (empty) {
        const int se = c0 + __builtin_ctzll(empty);
        empty &= empty - 1;
        half_t* o = a.out + (int64_t)se * Hq * D;
        for (int e = lane; e < Hq * D; e += 64) o[e] = (half_t)0.0f;
      }
    }
  }
  const int U = carry * Hkv;  // all units (the host bounds this below 2^31)
  if (U == 0) return;
  const int P = min(nw, U);  // active workers: one share each
  if (w >= P) return;
  if (streamer && lane < 4) ctl[lane] = 0;
  __syncthreads();  // the LDS tables are complete
  tr[kTrTables] = stamp_now();
  auto write_trace = [&](int first, int last) {
    if constexpr (kTrace) {
      if (lane == 0 && a.ws.trace)
        for (int i = first; i <= last; ++i) a.ws.trace[(int64_t)w * kTraceSlots + i] = tr[i];
    }
  };

  // the sequence holding head index `key`: the last s with off[s] <= key (a
  // 64-ary search over the LDS prefix sums)
  auto find_head = [&](int key) {
    int stride = 1;
    while (stride * 64 < S) stride *= 64;
    int lo = 0;
    while (true) {
      const int idx = lo + lane * stride;
      const bool ok = idx < S && off_lds[idx] <= key;
      lo += (__popcll(__ballot(ok)) - 1) * stride;
      if (stride == 1) break;
      stride >>= 6;
    }
    return uniform(lo);
  };

  // ---- shares ------------------------------------------------------------------
  // The streamer's time goes to units and, at the end of each run, to the
  // run's sums, its hand-over to the merger and the next run's q rows (on
  // batches of short runs about 2.4 us per unit and 1.1 us per run end).
  // With more runs than workers, shares are equal in that cost, kUnitCost
  // per unit and kRunCost per run:
  // unit g of run (s, h) sits at position
  //   Hkv (kUnitCost off[s] + kRunCost s) + h (kUnitCost n_s + kRunCost) + kRunCost + kUnitCost g
  // of a total C, and share j holds the units at positions in
  // [ceil(j C / P), ceil((j + 1) C / P)), in (sequence, head, unit) order.
  // Otherwise (a few long runs per worker at most, where the run ends weigh
  // little) shares are equal in units, share j = [floor(j U / P),
  // floor((j + 1) U / P)), which costs the workers less to find.
  const bool by_cost = S * Hkv > P;
  constexpr int kUnitCost = 4, kRunCost = 2;
  const int64_t C = (int64_t)kUnitCost * U + (int64_t)kRunCost * S * Hkv;
  // 32-bit arithmetic when j C and pos P fit (64-bit division is emulated,
  // several times slower)
  const bool narrow = (int64_t)P * C < ((int64_t)1 << 31);
  auto seq_pos = [&](int s) -> int64_t {
    return (int64_t)Hkv * ((int64_t)kUnitCost * uniform(off_lds[s]) + (int64_t)kRunCost * s);
  };
  // the last sequences s with seq_pos(s) <= T0 and <= T1 (one pass of the
  // 64-ary search of find_head for both)
  auto find_pos2 = [&](int64_t T0, int64_t T1, int& s0, int& s1) {
    int stride = 1;
    while (stride * 64 < S) stride *= 64;
    int lo0 = 0, lo1 = 0;
    while (true) {
      const int i0 = lo0 + lane * stride, i1 = lo1 + lane * stride;
      const int64_t p0 = i0 < S ? (int64_t)Hkv * ((int64_t)kUnitCost * off_lds[i0] + (int64_t)kRunCost * i0) : T0 + 1;
      const int64_t p1 = i1 < S ? (int64_t)Hkv * ((int64_t)kUnitCost * off_lds[i1] + (int64_t)kRunCost * i1) : T1 + 1;
      lo0 += (__popcll(__ballot(p0 <= T0)) - 1) * stride;
      lo1 += (__popcll(__ballot(p1 <= T1)) - 1) * stride;
      if (stride == 1) break;
      stride >>= 6;
    }
    s0 = uniform(lo0);
    s1 = uniform(lo1);
  };
  // the first unit at cost position >= T inside sequence s (the last with
  // seq_pos(s) <= T), or the next sequence's first: unit u = (s, h, g), or
  // h = Hkv / g = n_s when it is the next run's (the caller's cursor steps)
  struct ShareStart {
    int u, h, g;
  };
  auto start_in = [&](int64_t T, int s) -> ShareStart {
    const int n_s = uniform(run_units(s));
    const int u_s = Hkv * uniform(off_lds[s]);
    if (n_s == 0) return {u_s, Hkv, 0};  // (the next sequence's first unit)
    const int t1 = (int)(T - seq_pos(s));  // < Hkv (kUnitCost n_s + kRunCost)
    const int cr = kUnitCost * n_s + kRunCost;
    const int h = (int)((unsigned)t1 / (unsigned)cr);
    const int t2 = t1 - h * cr;
    const int g = t2 <= kRunCost ? 0 : (t2 - kRunCost + kUnitCost - 1) / kUnitCost;
    return {g >= n_s ? u_s + (h + 1) * n_s : u_s + h * n_s + g, h, g};
  };
  auto share_pos = [&](int j) -> int64_t {  // ceil(j C / P)
    return narrow ? (int64_t)(((unsigned)j * (unsigned)C + P - 1) / (unsigned)P)
                  : ((int64_t)j * C + P - 1) / P;
  };
  // the share holding unit u
  const bool narrow_u = (int64_t)U * P < ((int64_t)1 << 31);
  auto share_of = [&](int u) -> int {
    if (!by_cost)
      return narrow_u ? (int)((unsigned)((u + 1) * P - 1) / (unsigned)U)
                      : (int)(((int64_t)(u + 1) * P - 1) / U);
    const int s = find_head(u / Hkv);
    const int n_s = uniform(run_units(s));
    const int r = u - Hkv * uniform(off_lds[s]);
    const int h = r / n_s, g = r - h * n_s;
    const int64_t pos = seq_pos(s) + (int64_t)h * (kUnitCost * n_s + kRunCost) + kRunCost + kUnitCost * g;
    return narrow ? (int)((unsigned)pos * (unsigned)P / (unsigned)C) : (int)(pos * P / C);
  };
  // this worker's share [my_first, my_end) (a share can come out empty when
  // C / P is small)
  auto unit_sb = [&](int j) -> int {
    return narrow_u ? (int)((unsigned)(j * U) / (unsigned)P) : (int)((int64_t)j * U / P);
  };
  int first_s = -1;
  ShareStart first{0, Hkv, 0};
  int my_first, my_end;
  if (by_cost) {
    int end_s;
    const int64_t T_first = share_pos(w), T_end = share_pos(w + 1);
    find_pos2(T_first, w + 1 < P ? T_end : T_first, first_s, end_s);
    first = start_in(T_first, first_s);
    my_first = first.u;
    my_end = w + 1 < P ? start_in(T_end, end_s).u : U;
  } else {
    my_first = unit_sb(w);
    my_end = unit_sb(w + 1);
  }
  if (my_first >= my_end) return;
  // Partial slots: [0, R) the piece that starts run r, R + j the piece that
  // starts share j inside a run.
  // (Wide: slot R + u nw + j for sub-group u of a pass)
  const int R = Sv * Hkv;

  // ---- cursors over units --------------------------------------------------
  struct Cursor {
    int s, h, g;   // sequence, KV head, unit of the run
    int n_s, len;  // units and length of s
    int base;      // positions before the run's unit 0 (Shared: its prefix pass's)
    int left;      // units of the worker's share from this one on
    bool valid;    // false past the worker's last unit (then a copy of it)
  };
  auto set_seq = [&](Cursor& c, int s) {
    c.s = s;
    c.len = uniform(len_lds[s]);
    c.base = Shared ? uniform(base_lds[s]) : 0;
    c.n_s = units_for(c.len - c.base);
  };
  auto locate = [&](int u) {
    Cursor c;
    set_seq(c, find_head(u / Hkv));
    const int r = u - Hkv * uniform(off_lds[c.s]);
    c.h = r / c.n_s;
    c.g = r - c.h * c.n_s;
    c.left = 1;
    c.valid = true;
    return c;
  };
  // the next unit in (sequence, head, unit) order
  auto step = [&](Cursor c) {
    --c.left;
    if (c.g + 1 < c.n_s) {
      ++c.g;
      return c;
    }
    c.g = 0;
    if (c.h + 1 < Hkv) {
      ++c.h;
    } else {
      c.h = 0;
      int s = c.s;
      do {
        s = min(s + 1, S - 1);
        set_seq(c, s);
      } while (c.n_s == 0 && s + 1 < S);
    }
    return c;
  };

  auto lds_ld = [](const int* p) {
    lds_order();
    const int v = *p;
    lds_order();
    return uniform(v);
  };
  auto lds_st = [&](int* p, int v) {
    lds_order();
    if (lane == 0) *p = v;
    lds_order();
  };
  auto next = [&](Cursor c) -> Cursor {
    if (!c.valid) return c;
    if (c.left > 1) return step(c);
    c.valid = false;
    return c;
  };

  const int my_blk = lane / BS;  // which of a unit's blocks holds this lane's token
  const int g_lane = lane & 3;   // q head of the group this lane's MFMA row carries
  const int64_t block_stride = (int64_t)Hkv * kTile;

  // Table entries of unit c's NBU blocks: one vector load, lane i reads
  // entry NBU g + i % NBU.  Blocks past the sequence's last re-read its last
  // block, so every unit issues the same loads; positions past the end are
  // removed later by position.
  auto load_table = [&](const Cursor& c) {
    const int32_t* row = a.block_tables + (int64_t)seq_of(c.s) * a.max_blocks_per_seq;
    const int last = (c.len + BS - 1) / BS - 1;
    return row[min(c.base / BS + NBU * c.g + (lane % NBU), last)];
  };
  // The NBU physical ids (uniform) from such a load; an id outside the pool
  // (a broken table) reads pool block 0 instead.
  auto blocks_of = [&](int tbl, int (&pb)[NBU]) {
#pragma unroll
    for (int i = 0; i < NBU; ++i) {
      const int e = __builtin_amdgcn_readlane(tbl, i);
      pb[i] = (e >= 0 && e < a.num_blocks) ? e : 0;
    }
  };

  half8_t kreg[kChunks];  // (Wide: [tile kt][32-dim step j], kt * kWK + j)
  half8_t vreg[8][kSets];  // 8-token group g of the unit, 64-dim range st
  half8_t vw[kWT][2];      // Wide: V^T operand of 16-dim tile i, 32-token step kk
  // Wide: lane 16 wq + wm holds column wm (query row wm, or token wm of a
  // tile) and k-slice wq of the 16x16x32 operands
  const int wq = lane >> 4, wm = lane & 15;
  // q rows of a run: load i, lane r*kChunks + c: 16-byte chunk c of row
  // i * 64 / kChunks + r
  constexpr int kQLoads = (kRows * kChunks + 63) / 64;
  half8_t qreg[kQLoads];
  // K of unit c: lane l's token lies in the unit's block l / BS, whose table
  // entry lane l / BS of the table load tbl holds (a cross-lane read, not a
  // register-indexed select, which the compiler would turn into scratch)
  auto load_k = [&](const Cursor& c, int tbl, const int (&pb)[NBU]) {
    if constexpr (Wide) {
      // A operand of the logits: tile kt holds tokens 16 kt .. 16 kt + 15 of
      // the unit as its rows; for the 32-dim step j lane 16 wq + wm loads
      // 16-byte chunk 4 j + wq of token 16 kt + wm (with blocks of 16, one
      // load reads 1 KiB contiguous)
      auto tile = [&](int kt) {
        int phys, slot;
        if constexpr (BS >= 16) {
          phys = pb[16 * kt / BS];
          slot = 16 * kt % BS + wm;
        } else {
          phys = (wm >> 3) ? pb[2 * kt + 1] : pb[2 * kt];
          slot = wm & 7;
        }
        return a.k_cache + (int64_t)phys * block_stride + (int64_t)c.h * kTile +
               (int64_t)(wq * BS + slot) * kChunk;
      };
      if constexpr (Fused) {
        const int tn = c.len - 1 - (c.base + c.g * kGroupTokens);
        if (tn < kGroupTokens) {  // (uniform) the new token's lanes read k_new
          const half_t* np = a.k_new + ((int64_t)seq_of(c.s) * Hkv + c.h) * D + wq * kChunk;
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) {
            const half_t* kp = tile(kt);
            const bool mine = 16 * kt + wm == tn;
#pragma unroll
            for (int j = 0; j < kWK; ++j)
              kreg[kt * kWK + j] = load_kv(mine ? np + j * 4 * kChunk : kp + j * 4 * BS * kChunk);
          }
          return;
        }
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const half_t* kp = tile(kt);
#pragma unroll
        for (int j = 0; j < kWK; ++j) kreg[kt * kWK + j] = load_kv(kp + j * 4 * BS * kChunk);
      }
      return;
    }
    const int e = __shfl(tbl, my_blk);
    const int phys = (e >= 0 && e < a.num_blocks) ? e : 0;
    const half_t* kp = a.k_cache + (int64_t)phys * block_stride + (int64_t)c.h * kTile +
                       (lane % BS) * kChunk;
    if constexpr (Fused) {
      // the run's last unit holds the new token (position len - 1, which the
      // pools do not hold yet): its lane reads the K row from k_new
      const int tn = c.len - 1 - (c.base + c.g * kGroupTokens);
      if (tn < kGroupTokens) {  // (uniform)
        const half_t* np = a.k_new + ((int64_t)seq_of(c.s) * Hkv + c.h) * D;
        const bool mine = lane == tn;
#pragma unroll
        for (int cc = 0; cc < kChunks; ++cc)
          kreg[cc] = load_kv(mine ? np + cc * kChunk : kp + cc * (BS * kChunk));
        return;
      }
    }
#pragma unroll
    for (int cc = 0; cc < kChunks; ++cc) kreg[cc] = load_kv(kp + cc * (BS * kChunk));
  };
  // V group g (tokens 8g..8g+7 of the unit) is group g % kGroups of the
  // unit's block g / kGroups: for a fixed 64-dim range one 1 KiB load
  auto load_v = [&](const Cursor& c, const int (&pb)[NBU]) {
    if constexpr (Wide) {
      // A operand of the products (V^T): for the 32-token step kk lane
      // 16 wq + wm loads dim 16 i + wm of the unit's 8-token group 4 kk + wq
      // (16 bytes), for each 16-dim tile i
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        int phys;
        if constexpr (kGroups == 4) phys = pb[kk];
        else if constexpr (kGroups == 2) phys = (wq >> 1) ? pb[2 * kk + 1] : pb[2 * kk];
        else
          phys = wq == 0 ? pb[4 * kk] : wq == 1 ? pb[4 * kk + 1] : wq == 2 ? pb[4 * kk + 2] : pb[4 * kk + 3];
        const half_t* vp = a.v_cache + (int64_t)phys * block_stride + (int64_t)c.h * kTile +
                           (int64_t)(((4 * kk + wq) % kGroups) * D + wm) * kChunk;
#pragma unroll
        for (int i = 0; i < kWT; ++i) vw[i][kk] = load_kv(vp + i * 16 * kChunk);
      }
      return;
    }
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const half_t* vp = a.v_cache + (int64_t)pb[g / kGroups] * block_stride +
                         (int64_t)c.h * kTile + (int64_t)(g % kGroups) * D * kChunk;
#pragma unroll
      for (int st = 0; st < kSets; ++st) vreg[g][st] = load_kv(vp + (st * 64 + lane) * kChunk);
    }
  };
  // q rows of c's run; every lane loads (rows past the head's and lanes past
  // the rows re-read row 0 and are zeroed at the LDS write) so the load is
  // unconditional
  // (Wide: rows 0..15 of the 16 are query heads h G + q0 + 0..15 of the
  // sequence, q0 the pass's first, rows past G zero; one load covers
  // 64 / kChunks rows)
  const int q_row = lane / kChunks, q_chunk = lane % kChunks;
  bool q_ok[kQLoads];  // this lane's row of each load holds a query head
  auto load_q = [&](const Cursor& c) {
#pragma unroll
    for (int i = 0; i < kQLoads; ++i) {
      const int r = i * (64 / kChunks) + q_row;
      int64_t row;
      if constexpr (Wide) {
        const int q0 = 4 * pass_sub0(c.s);  // the pass's first query head of the group
        q_ok[i] = q0 + r < G;
        row = (int64_t)seq_of(c.s) * Hq + c.h * G + q0 + (q_ok[i] ? r : 0);
      } else {
        q_ok[i] = r < q_rows(c.s);
        row = q_row0(c.s, c.h) + (q_ok[i] ? r : 0);
      }
      qreg[i] = *reinterpret_cast<const half8_t*>(a.q + row * D + q_chunk * kChunk);
    }
  };
  // Shared: the prefix pass's first chunk for a run, loaded for a unit that
  // starts the run one iteration ahead, ahead of that unit's K (rows: dims
  // 64 st + lane of head g; lane g < rows: head g's log-sum-exp).  A piece that
  // starts a run begins from it, a piece of weight 1 at its log-sum-exp,
  // instead of from nothing: the run's online softmax then takes the prefix
  // in with no fold afterwards.  (Further chunks, of prefixes above one
  // chunk, are folded by the merger.)
  // (Wide: lane 16 wq + wm, the pass's query row wm, dims 16 i + 4 wq .. + 3)
  half_t pre_o[kSub][4][kSets];
  float pre_m[kSub];
  half4_t pre_w[kWT];
  float pre_mw = -INFINITY;
  auto load_pre = [&](const Cursor& c) {
    if constexpr (Shared && Wide) {
      const int q0 = 4 * pass_sub0(c.s);
      const bool ok = q0 + wm < G;
      const int64_t row = (int64_t)seq_of(c.s) * Hq + c.h * G + q0 + (ok ? wm : 0);
#pragma unroll
      for (int i = 0; i < kWT; ++i) {
        const half4_t v = *reinterpret_cast<const half4_t*>(a.pre_o + row * D + 16 * i + 4 * wq);
        pre_w[i] = ok ? v : half4_t{};
      }
      const float lse = a.pre_lse[row];
      pre_mw = ok ? lse : -INFINITY;
    } else if constexpr (Shared) {
#pragma unroll
      for (int u = 0; u < kSub; ++u) {
        const int sv = c.s;
        const int64_t row0 = q_row0(sv, c.h);
        const int nr = q_rows(sv);
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int st = 0; st < kSets; ++st)
            pre_o[u][g][st] = g < nr ? a.pre_o[(row0 + g) * D + st * 64 + lane] : (half_t)0.0f;
        pre_m[u] = nr > 0 ? a.pre_lse[row0 + min(lane, nr - 1)] : -INFINITY;
      }
    }
  };
  auto starts_with_pre = [&](const Cursor& c) { return Shared && c.valid && c.g == 0 && c.base > 0; };
  auto store_q = [&]() {
#pragma unroll
    for (int i = 0; i < kQLoads; ++i) {
      const int r = i * (64 / kChunks) + q_row;
      if (r < kRows) {
        const half8_t v = q_ok[i] ? qreg[i] : half8_t{};
        *reinterpret_cast<half8_t*>(q_lds + r * kQRow + q_chunk * kChunk) = v;
      }
    }
  };
  // Fused append: the new token of sequence s sits at position len - 1, in
  // the last unit of each of s's runs, where it takes part in the unit's
  // logits and weights like any other position: its lane's K row comes from
  // k_new (load_k), and its V element is put into the unit's V tile from
  // v_new.  The V row is loaded with every unit (lane l: dims 64 st + l), so
  // that every iteration issues the same loads.
  auto load_new = [&](const Cursor& c, half_t (&vn)[kSets]) {
    if constexpr (Fused) {
      const int64_t row = ((int64_t)seq_of(c.s) * Hkv + c.h) * D;
#pragma unroll
      for (int st = 0; st < kSets; ++st) vn[st] = a.v_new[row + st * 64 + lane];
    }
  };
  // The stores of the new rows, after the worker's last unit: scattered
  // partial-line writes are slow to complete, and a wave's memory operations
  // complete in order, so inside the loop each would hold back the K/V loads
  // issued after it.  The runs whose last unit lies in this worker's share
  // [first, end) are walked in order and stored 4 at a time: lane 16 i + c
  // moves 16-byte chunk c (8 dims) of the i-th run's K and V rows, K to
  // [chunk][slot][8], V as 8 elements at [slot / 8][dim][slot % 8].
  auto store_new_rows = [&]() {
    if constexpr (Fused) {
      const int first = my_first, end = my_end;
      const int ch = lane & 15;
      int my_s = -1, my_h = 0, grp = 0;
      auto flush = [&]() {
        if (my_s >= 0 && ch < kChunks) {
          const int64_t slot = a.slot_mapping[my_s];
          const int64_t row = ((int64_t)my_s * Hkv + my_h) * D + ch * kChunk;
          const half8_t kr = *reinterpret_cast<const half8_t*>(a.k_new + row);
          const half8_t vr = *reinterpret_cast<const half8_t*>(a.v_new + row);
          if (slot >= 0 && slot < a.num_blocks * BS) {
            const int64_t b = slot / BS;
            const int o = (int)(slot - b * BS);
            const int64_t tile = (b * Hkv + my_h) * kTile;
            *reinterpret_cast<half8_t*>(a.k_cache_w + tile + ((int64_t)ch * BS + o) * kChunk) = kr;
            half_t* vp = a.v_cache_w + tile + ((int64_t)(o / kChunk) * D + ch * kChunk) * kChunk +
                         o % kChunk;
#pragma unroll
            for (int e = 0; e < kChunk; ++e) vp[e * kChunk] = vr[e];
          }
        }
        my_s = -1;
        grp = 0;
      };
      Cursor c = locate(first);
      while (true) {
        const int run0 = Hkv * uniform(off_lds[c.s]) + c.h * c.n_s;  // the run's first unit
        if (run0 >= end) break;
        const int last = run0 + c.n_s - 1;
        // (the first sub-group's copy of the sequence stores its rows)
        if (last >= first && last < end && c.s < Sr) {
          if ((lane >> 4) == grp) {
            my_s = c.s;
            my_h = c.h;
          }
          if (++grp == 4) flush();
        }
        if (run0 + c.n_s >= end) break;  // no further run starts in the share
        c.g = c.n_s - 1;  // step to the next run
        c.left = 2;
        c = step(c);
      }
      if (grp > 0) flush();
    }
  };

  // ---- merge of a cut run ----------------------------------------------------
  // Run r = (s, kvh) holds units [u0, u0 + n); its pieces are its overlaps
  // with the shares v it meets: slot r for the one that starts the run, slot
  // R + v for a piece that starts share v.  Lane 16*gq + pq handles head gq:
  // for a batch of up to 16 pieces it loads (max, sum) of piece pq and output
  // dims pq*kF .. +kF of head gq of every piece (one round trip); batches
  // combine with the running-max rescale into (mx, lsum, acc): mx the running
  // max of head gq, lsum this lane's part of the weighted sum, acc the
  // weighted output dims.
  struct Merged {
    float mx, lsum;
    float acc[kF];
  };
  const int gq = lane >> 4, pq = lane & 15;
  // one batch of nb <= B pieces whose slot lane pq holds in sl (lanes past
  // the batch repeat its last), B = 2, 4 or 16 so that small batches load
  // only what they use
  // (own_slot >= 0: the piece of that slot is not in the workspace but in
  // ring entry own_k, where the merger still holds it)
  auto absorb = [&](auto batch, Merged& m, int sl, int nb, int own_slot, int own_k, int nr) {
    constexpr int B = decltype(batch)::value;
    const bool valid = pq < nb && gq < nr;
    const bool own = sl == own_slot;
    float m_p = valid ? load_through(a.ws.ml + (int64_t)sl * 8 + 2 * gq) : -INFINITY;
    float l_p = valid ? load_through(a.ws.ml + (int64_t)sl * 8 + 2 * gq + 1) : 0.0f;
    if (own_slot >= 0) {
      const float mo = ring_ml[own_k][2 * (gq & 3)], lo = ring_ml[own_k][2 * (gq & 3) + 1];
      m_p = (valid && own) ? mo : m_p;
      l_p = (valid && own) ? lo : l_p;
    }
    float ov[B][kF];
#pragma unroll
    for (int qi = 0; qi < B; ++qi) {
      const int sq = __builtin_amdgcn_readlane(sl, qi);
      if (sq == own_slot) {
#pragma unroll
        for (int j = 0; j < kF; ++j) ov[qi][j] = ring_o[own_k][(gq & 3) * D + pq * kF + j];
      } else {
        const float* base = a.ws.o + (int64_t)sq * 4 * D;
#pragma unroll
        for (int st = 0; st < kSets; ++st) {
          const float4_t x = load_through16(base, ((gq & 3) * D + pq * kF + st * 4) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[qi][st * 4 + e] = x[e];
        }
      }
    }
    const float m_new = fmaxf(m.mx, row_max16(m_p));
    const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2(m.mx - m_new);
    const float wt = valid ? fast_exp2(m_p - m_new) : 0.0f;
    m.lsum = m.lsum * alpha + wt * l_p;
    m.mx = m_new;
#pragma unroll
    for (int j = 0; j < kF; ++j) m.acc[j] *= alpha;
#pragma unroll
    for (int qi = 0; qi < B; ++qi) {
      const float wq = __shfl(wt, (lane & 48) | qi);  // 0 for pieces past the batch
#pragma unroll
      for (int j = 0; j < kF; ++j) m.acc[j] += wq * ov[qi][j];
    }
  };
  // all pieces of run (s, kvh)
  auto merge_pieces = [&](int s, int kvh, int own_slot, int own_k) {
    Merged m;
    m.mx = -INFINITY;
    m.lsum = 0.0f;
#pragma unroll
    for (int j = 0; j < kF; ++j) m.acc[j] = 0.0f;
    const int ts = tab(s);
    const int n = uniform(run_units(ts));
    const int u0 = Hkv * uniform(off_lds[ts]) + kvh * n;
    const int r = s * Hkv + kvh;
    // the slot of a piece that starts share v inside the run (Wide: each
    // sub-group of a pass has slots of its own)
    const int r_share = Wide ? R + (sub_of(s) & (kSub - 1)) * nw : R;
    const int nr = q_rows(s);
    const int64_t q0 = q_row0(s, kvh) - (int64_t)real_of(s) * Hq;  // (its first query head)
    // Shared: the prefix pass's chunks 1.. of the run's rows (the piece that
    // starts the run began from chunk 0), loaded before the pieces so that
    // the two round trips overlap
    constexpr int NC = Shared ? kPrefixMaxChunks : 1;
    typedef half_t hvec_t __attribute__((ext_vector_type(kF)));
    float m_c[NC];
    hvec_t o_c[NC];
    int nch = 0;
    if constexpr (Shared) {
      nch = prefix_chunks(uniform(base_lds[ts]));
      const bool valid = gq < nr;
#pragma unroll
      for (int c = 1; c < NC; ++c) {
        const int64_t qrow = ((int64_t)min(c, max(nch - 1, 0)) * Sr + real_of(s)) * Hq + q0 + (valid ? gq : 0);
        m_c[c] = (c < nch && valid) ? a.pre_lse[qrow] : -INFINITY;
        o_c[c] = c < nch ? *reinterpret_cast<const hvec_t*>(a.pre_o + qrow * D + pq * kF) : hvec_t{};
      }
    }
    const int va = share_of(u0), vb = share_of(u0 + n - 1);
    const int np_all = vb - va + 1;
    for (int p0 = 0; p0 < np_all; p0 += 16) {
      const int nb = min(16, np_all - p0);
      // piece p0 + pq (pieces past the batch repeat its last)
      const int p = p0 + min(pq, nb - 1);
      const int v = va + p;
      const int sl = v == va ? r : r_share + v;
      if (nb <= 2)
        absorb(std::integral_constant<int, 2>{}, m, sl, nb, own_slot, own_k, nr);
      else if (nb <= 4)
        absorb(std::integral_constant<int, 4>{}, m, sl, nb, own_slot, own_k, nr);
      else
        absorb(std::integral_constant<int, 16>{}, m, sl, nb, own_slot, own_k, nr);
    }
    // Shared: each chunk a piece of weight 1 (in lane pq = 0 of each row)
    // at its log-sum-exp
    if constexpr (Shared) {
#pragma unroll
      for (int c = 1; c < NC; ++c) {
        if (c < nch) {
          const float m_new = fmaxf(m.mx, m_c[c]);
          const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2(m.mx - m_new);
          const float wt = gq < nr ? fast_exp2(m_c[c] - m_new) : 0.0f;
          m.lsum = m.lsum * alpha + (pq == 0 ? wt : 0.0f);
          m.mx = m_new;
#pragma unroll
          for (int j = 0; j < kF; ++j) m.acc[j] = m.acc[j] * alpha + wt * (float)o_c[c][j];
        }
      }
    }
    return m;
  };
  // the output rows of run (s, kvh) from its merged pieces; clears the run's
  // counter for the next call
  auto merge_out = [&](int s, int kvh, const Merged& m) {
    const float inv = 1.0f / row_sum16(m.lsum);
    if (gq < q_rows(s)) {
      half_t* o = a.out + (q_row0(s, kvh) + gq) * D + pq * kF;
#pragma unroll
      for (int j = 0; j < kF; ++j) o[j] = (half_t)(m.acc[j] * inv);
    }
    if (lane == 0)
      __hip_atomic_store(a.ws.counters + s * Hkv + kvh, 0, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  };

  // per-piece softmax state
  // (one set per sub-group the pass attends)
  float m_run[kSub][4], l_lane[kSub][4];
  float4_t acc_o[kSub][kSets];
  // (Wide: lane 16 wq + wm holds query row wm: its running max, its part of
  // the sum, and dims 16 i + 4 wq .. + 3 of its unnormalised output, tile i)
  float w_m = -INFINITY, w_l = 0.0f;
  float4_t w_acc[kWT];
  auto reset_run = [&]() {
    if constexpr (Wide) {
      w_m = -INFINITY;
      w_l = 0.0f;
#pragma unroll
      for (int i = 0; i < kWT; ++i) w_acc[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
      return;
    }
#pragma unroll
    for (int u = 0; u < kSub; ++u) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        m_run[u][g] = -INFINITY;
        l_lane[u][g] = 0.0f;
      }
#pragma unroll
      for (int st = 0; st < kSets; ++st) acc_o[u][st] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
  };
  // a piece that starts a run with a prefix: begin from its first chunk
  // (nr[u]: query rows of sub-group u)
  auto seed_pre = [&](const int (&nr)[kSub]) {
    if constexpr (Wide) {  // (rows past the group: max -inf, nothing)
      w_m = pre_mw;
      w_l = (wq == 0 && pre_mw != -INFINITY) ? 1.0f : 0.0f;
#pragma unroll
      for (int i = 0; i < kWT; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) w_acc[i][e] = (float)pre_w[i][e];
      return;
    }
#pragma unroll
    for (int u = 0; u < kSub; ++u)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (g < nr[u]) {
          m_run[u][g] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pre_m[u]), g));
          l_lane[u][g] = lane == 0 ? 1.0f : 0.0f;
#pragma unroll
          for (int st = 0; st < kSets; ++st) acc_o[u][st][g] = (float)pre_o[u][g][st];
        }
      }
  };

  // ---- the merger wave --------------------------------------------------------
  if (!streamer) {
    // The merger works in rounds: take every finished piece from the ring (up
    // to kRing); read their runs' counters and write the pieces through to
    // their slots; wait once.  A piece whose run already has every other
    // unit in is the last: it merges at once, without being counted.  The
    // others count their arrivals (one lane each, by units); wait once; the
    // piece that completes its run's count merges.
    int cons = 0;
    // Shared: chunks 1.. of a whole run's prefix (the streamer began the run
    // from chunk 0), loaded when the run comes
    half_t pf_o[kPrefixMaxChunks][4][kSets];  // dims 64 st + lane of head g, chunk c
    float pf_m[kPrefixMaxChunks];             // lane g < rows: head g's log-sum-exp, chunk c
    auto load_pieces = [&](int s, int hh, int nch) {
#pragma unroll
      for (int c = 1; c < kPrefixMaxChunks; ++c) {
        const int64_t row0 = ((int64_t)c * Sr + real_of(s)) * Hq + hh * G + sub_of(s) * 4;
        const int nr = q_rows(s);
        pf_m[c] = (c < nch && nr > 0) ? a.pre_lse[row0 + min(lane, nr - 1)] : -INFINITY;
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int st = 0; st < kSets; ++st)
            pf_o[c][g][st] = (c < nch && g < nr) ? a.pre_o[(row0 + g) * D + st * 64 + lane] : (half_t)0.0f;
      }
    };
    int idle = 0;
    for (; idle < a.spin_limit;) {
      const int avail = min(lds_ld(&ctl[kCtlRingMade]) - cons, kRing);
      if (avail == 0) {
        // the streamer writes its last entry before its done flag: once the
        // flag is seen, one more look at the ring is final
        if (lds_ld(&ctl[kCtlDone]) && cons == lds_ld(&ctl[kCtlRingMade])) break;
        __builtin_amdgcn_s_sleep(2);
        ++idle;
        continue;
      }
      idle = 0;
      const uint64_t t_round = stamp_now();
      int ps[kRing], ph[kRing], pu[kRing];
      int64_t pslot[kRing];
#pragma unroll
      for (int i = 0; i < kRing; ++i) {
        if (i < avail) {
          const int k = (cons + i) % kRing;
          ps[i] = lds_ld(&ring_meta[k][0]);
          ph[i] = lds_ld(&ring_meta[k][1]);
          pslot[i] = lds_ld(&ring_meta[k][2]);
          pu[i] = lds_ld(&ring_meta[k][3]);
        }
      }
      // lane i < avail: piece i's run counter and units (whole runs: none)
      int ci = 0, ui = 0, seen = 0;
      bool counted = false;
      if (lane < avail) {
        int si = ps[0], hi = ph[0];
        int64_t sli = pslot[0];
        ui = pu[0];
#pragma unroll
        for (int i = 1; i < kRing; ++i)
          if (lane == i) si = ps[i], hi = ph[i], ui = pu[i], sli = pslot[i];
        ci = si * Hkv + hi;
        counted = sli >= 0;
        if (counted) seen = load_through_i(a.ws.counters + ci);
      }
      // the entries into registers, then release them
      float pv[kRing][4][kSets], pml[kRing];
#pragma unroll
      for (int i = 0; i < kRing; ++i) {
        if (i < avail) {
          const int k = (cons + i) % kRing;
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int st = 0; st < kSets; ++st) pv[i][g][st] = ring_o[k][g * D + st * 64 + lane];
          pml[i] = lane < 8 ? ring_ml[k][lane] : 0.0f;
        }
      }
      // Pieces that complete their run, known at this point (every other
      // unit of the run already counted): merged straight from the ring,
      // neither written through nor counted.  Their ring entries are released
      // after the merge, the others' at once.
      const bool last_known = counted && seen + ui == run_units(tab(ci / Hkv));
      const uint64_t fast = __ballot(last_known);  // bit i: piece i
      const int cons0 = cons;
      cons += avail;
      if (!fast) lds_st(&ctl[kCtlRingTaken], cons);  // (the ring reads above precede this write)
#pragma unroll
      for (int i = 0; i < kRing; ++i) {
        if (i < avail && pslot[i] < 0) {
          // a whole run: its output rows (Shared: with the prefix pass's
          // chunks 1.. folded in, each a piece of weight 1 at its log-sum-exp)
          const int s_i = ps[i];
          const int nch = Shared ? prefix_chunks(uniform(base_lds[tab(s_i)])) : 0;
          if (Shared && nch > 1) load_pieces(s_i, ph[i], nch);
          const int nr = q_rows(s_i);
          const int64_t row_0 = q_row0(s_i, ph[i]);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            if (g < nr) {
              const float mr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pml[i]), 2 * g));
              const float lt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pml[i]), 2 * g + 1));
              const int64_t row = row_0 + g;
              float v[kSets], den = lt;
#pragma unroll
              for (int st = 0; st < kSets; ++st) v[st] = pv[i][g][st];
              if (Shared && nch > 1) {
                float mp[kPrefixMaxChunks], mx = mr;
#pragma unroll
                for (int c = 1; c < kPrefixMaxChunks; ++c) {
                  mp[c] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pf_m[c]), g));
                  mx = fmaxf(mx, mp[c]);
                }
                const float a1 = fast_exp2(mr - mx);
                den = lt * a1;
#pragma unroll
                for (int st = 0; st < kSets; ++st) v[st] *= a1;
#pragma unroll
                for (int c = 1; c < kPrefixMaxChunks; ++c) {
                  const float wc = c < nch ? fast_exp2(mp[c] - mx) : 0.0f;
                  den += wc;
#pragma unroll
                  for (int st = 0; st < kSets; ++st) v[st] += wc * (float)pf_o[c][g][st];
                }
              }
              const float inv = 1.0f / den;
              half_t* o = a.out + row * D;
#pragma unroll
              for (int st = 0; st < kSets; ++st) o[st * 64 + lane] = (half_t)(v[st] * inv);
            }
          }
          if constexpr (kTrace) ++tr[kTrMerges];
        } else if (i < avail && !((fast >> i) & 1)) {
          // a cut piece: written through to its slot
          float* po = a.ws.o + pslot[i] * 4 * D;
          const int nr = q_rows(ps[i]);
#pragma unroll
          for (int g = 0; g < 4; ++g)
            if (g < nr)
#pragma unroll
              for (int st = 0; st < kSets; ++st)
                store_through(po + g * D + st * 64 + lane, pv[i][g][st]);
          if (lane < 2 * nr) store_through(a.ws.ml + pslot[i] * 8 + lane, pml[i]);
        }
      }
      // the slots are written through before they are counted (a round
      // without pieces to count waits for nothing)
      if (__ballot(counted && !last_known)) __builtin_amdgcn_s_waitcnt(0);
      int arr = 0;
      if (counted && !last_known)
        arr = __hip_atomic_fetch_add(a.ws.counters + ci, ui, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int i = 0; i < kRing; ++i) {
        if (i < avail && pslot[i] >= 0) {
          const bool fi = (fast >> i) & 1;
          const int n = uniform(run_units(tab(ps[i])));
          if (fi || __builtin_amdgcn_readlane(arr, i) + pu[i] == n) {
            merge_out(ps[i], ph[i],
                      merge_pieces(ps[i], ph[i], fi ? (int)pslot[i] : -1, (cons0 + i) % kRing));
            if constexpr (kTrace) ++tr[kTrMerges];
          }
        }
      }
      if (fast) lds_st(&ctl[kCtlRingTaken], cons);  // (after the merges read the ring)
      if constexpr (kTrace) {
        __builtin_amdgcn_s_waitcnt(0);
        tr[kTrHelperBusy] += stamp_now() - t_round;
        ++tr[kTrHelperRounds];
      }
    }
    // the streamer never said it was done: give up (reported in the status word)
    if (idle >= a.spin_limit && lane == 0)
      __hip_atomic_store(a.ws.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if constexpr (kTrace) {
      __builtin_amdgcn_s_waitcnt(0);
      tr[kTrHelperEnd] = stamp_now();
      write_trace(kTrHelperEnd, kTrHelperEnd);
      write_trace(kTrMerges, kTrMerges);
      write_trace(kTrHelperBusy, kTrHelperRounds);
    }
    return;
  }

  // ---- the streamer wave -----------------------------------------------------
  int ring_made = 0;
  __builtin_amdgcn_s_setprio(1);
  // the streamer is done: the merger finishes what is queued and stops
  auto finish = [&]() { lds_st(&ctl[kCtlDone], 1); };

  // ---- prologue: first unit's loads, next unit's table entries ------------
  // Lookahead: cur is computed, nxt has its K/V loads in flight and its ids in
  // pb_nxt, nxt2 has its table entries loading into tbl_nxt2.
  // the first unit: the start of this worker's share
  Cursor cur;
  if (first_s >= 0 && first.h < Hkv && first.g < uniform(run_units(first_s))) {
    set_seq(cur, first_s);  // (found by the share search)
    cur.h = first.h;
    cur.g = first.g;
    cur.valid = true;
  } else {
    cur = locate(my_first);
  }
  cur.left = my_end - my_first;
  Cursor nxt = next(cur);
  Cursor nxt2 = next(nxt);
  int pb_cur[NBU], pb_nxt[NBU];
  const int tbl_cur = load_table(cur);
  int tbl_nxt = load_table(nxt);
  load_q(cur);
  if (starts_with_pre(cur)) load_pre(cur);
  blocks_of(tbl_cur, pb_cur);
  // keep the prologue in loop order (all K loads, then all V loads): the
  // wait counts at the loop head are merged over both ways in
  __builtin_amdgcn_sched_barrier(0);
  half_t vn_cur[kSets] = {}, vn_nxt[kSets] = {};
  load_k(cur, tbl_cur, pb_cur);
  load_new(cur, vn_cur);
  __builtin_amdgcn_sched_barrier(0);
  load_v(cur, pb_cur);
  __builtin_amdgcn_sched_barrier(0);
  store_q();
  __builtin_amdgcn_wave_barrier();
  reset_run();
  // query rows of each sub-group a pass over (cur.s, .) attends
  auto rows_of = [&](int s, int (&nr)[kSub]) {
    if constexpr (Wide) {
      const int q0 = 4 * pass_sub0(s);
#pragma unroll
      for (int u = 0; u < kSub; ++u) nr[u] = max(0, min(4, G - q0 - 4 * u));
    } else {
      nr[0] = q_rows(s);
    }
  };
  {
    int nr0[kSub];
    rows_of(cur.s, nr0);
    if (starts_with_pre(cur)) seed_pre(nr0);
  }
  uint64_t t_iter = stamp_now();
  int piece_g0 = cur.g;  // unit of the run where the piece began
  bool q_pending = false;  // a new piece starts: its q rows go to LDS first

  while (cur.valid) {
    const int t0 = cur.base + cur.g * kGroupTokens;  // position of the unit's first token
    int nrs[kSub];  // query rows of each sub-group of the run
    rows_of(cur.s, nrs);
    const int nr = nrs[0];
    // q rows of a piece that starts here.  Their load was issued one
    // iteration ago, before this unit's K: waiting for it here costs nothing,
    // as the logits wait for that K anyway.
    if (q_pending) {
      store_q();
      if (starts_with_pre(cur)) seed_pre(nrs);
    }
    q_pending = false;

    // logits: S[g][token lane] = q_g . K_token  (rows = heads, columns = tokens)
    float4_t sacc_u[kSub];
#pragma unroll
    for (int u = 0; u < kSub; ++u) sacc_u[u] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float4_t& sacc = sacc_u[0];
    if constexpr (Wide) {
      // S^T = K Q^T, one 16x16 tile per 16 tokens: sacc_u[kt] holds, in lane
      // 16 wq + wm, query row wm's logits at tokens 16 kt + 4 wq + 0..3
#pragma unroll
      for (int j = 0; j < kWK; ++j) {
        const half8_t qb = *reinterpret_cast<const half8_t*>(q_lds + wm * kQRow + 32 * j + 8 * wq);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) sacc_u[kt] = mfma16(kreg[kt * kWK + j], qb, sacc_u[kt]);
      }
    } else if constexpr (kValu) {
      // (measurement build) lane = token: its K row against each head's q
      // row, read from LDS by every lane at once, in pairs of dims
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (g < nr) {
          float acc = 0.0f;
#pragma unroll
          for (int c = 0; c < kChunks; ++c) {
            const half8_t qv = *reinterpret_cast<const half8_t*>(q_lds + g * kQRow + c * kChunk);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc = __builtin_amdgcn_fdot2(half2x{qv[2 * i], qv[2 * i + 1]},
                                           half2x{kreg[c][2 * i], kreg[c][2 * i + 1]}, acc, false);
          }
          sacc[g] = acc;
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
#pragma unroll
        for (int u = 0; u < kSub; ++u) {
          const half8_t qv =
              *reinterpret_cast<const half8_t*>(q_lds + (4 * u + g_lane) * kQRow + c * kChunk);
          sacc_u[u] = __builtin_amdgcn_mfma_f32_4x4x4f16(lo4(qv), lo4(kreg[c]), sacc_u[u], 0, 0, 0);
          sacc_u[u] = __builtin_amdgcn_mfma_f32_4x4x4f16(hi4(qv), hi4(kreg[c]), sacc_u[u], 0, 0, 0);
        }
      }
    }
    // keep the next unit's address work below the logits: hoisted above
    // them it would wait for this unit's whole K (and table) first
    __builtin_amdgcn_sched_barrier(0);
    // the next unit's prefix piece when it starts a run (issued ahead of its
    // K, so that the waits for that K stay the same on both ways)
    if (starts_with_pre(nxt)) load_pre(nxt);
    __builtin_amdgcn_sched_barrier(0);
    // table entries two units ahead, then the next unit's K and q
    const int tbl_nxt2 = load_table(nxt2);
    blocks_of(tbl_nxt, pb_nxt);
    load_k(nxt, tbl_nxt, pb_nxt);
    load_q(nxt);
    load_new(nxt, vn_nxt);
    // the unit after nxt2, computed while this unit's V is in flight
    const Cursor nxt3 = next(nxt2);

    // online softmax over these 64 positions
    // (every unit holds at least one position: its first, t0 < len)
    if constexpr (Wide) {
      // lane 16 wq + wm: query row wm at positions t0 + 16 kt + 4 wq + e; the
      // row's max over the unit from its four lanes
      float z[4][4];
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          z[kt][e] = t0 + 16 * kt + 4 * wq + e < cur.len ? sacc_u[kt][e] * a.scale_log2 : -INFINITY;
          mx = fmaxf(mx, z[kt][e]);
        }
      const float m_new = fmaxf(w_m, max_row4(mx));
      const float alpha = fast_exp2(w_m - m_new);  // 0 at the piece's first unit
      const half2x one = {(half_t)1.0f, (half_t)1.0f};
      float ls = 0.0f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        half4_t ph;
#pragma unroll
        for (int e = 0; e < 4; ++e) ph[e] = (half_t)fast_exp2(z[kt][e] - m_new);
        ls = __builtin_amdgcn_fdot2(half2x{ph[0], ph[1]}, one, ls, false);
        ls = __builtin_amdgcn_fdot2(half2x{ph[2], ph[3]}, one, ls, false);
        *reinterpret_cast<half4_t*>(p_lds + wm * kPRow + 16 * kt + 4 * wq) = ph;
      }
      w_l = w_l * alpha + ls;
#pragma unroll
      for (int i = 0; i < kWT; ++i) w_acc[i] *= alpha;
      w_m = m_new;
    } else {
    const bool live = (t0 + lane) < cur.len;
#pragma unroll
    for (int u = 0; u < kSub; ++u)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        half_t ph = (half_t)0.0f;
        if (g < nrs[u]) {
          const float z = live ? sacc_u[u][g] * a.scale_log2 : -INFINITY;
          const float m_new = fmaxf(m_run[u][g], wave_max(z));
          const float alpha = fast_exp2(m_run[u][g] - m_new);  // 0 at the piece's first unit
          ph = (half_t)fast_exp2(z - m_new);
          l_lane[u][g] = l_lane[u][g] * alpha + (float)ph;
#pragma unroll
          for (int st = 0; st < kSets; ++st) acc_o[u][st][g] *= alpha;
          m_run[u][g] = m_new;
        }
        p_lds[(4 * u + g) * kPRow + lane] = ph;
      }
    }

    if constexpr (kTrace) {
      if (tr[kTrUnits]++ == 0) tr[kTrFirstUnit] = stamp_now();
    }
    // The run's last unit: positions past the end (the tail of the last
    // block, and blocks past it re-read) hold any bits, NaN included, and
    // 0 * NaN is not 0, so their V elements are cleared; a fused append's
    // new token (offset tn) takes its V element from v_new.  Lane l holds
    // dim 64 st + l of 8 positions per 8-position group, two per 32-bit
    // word, so each word takes one mask (uniform) and at most one insert.
    const int t_end = cur.len - t0;  // positions of the unit (uniform)
    if (Fused ? t_end <= kGroupTokens : t_end < kGroupTokens) {
      const int tn = Fused ? t_end - 1 : kGroupTokens;
      const int keep_end = Fused ? tn : t_end;  // positions < keep_end come from the pools
      if constexpr (Wide) {
        // lane 16 wq + wm holds positions 32 kk + 8 wq + 2 x, + 1 of dim
        // 16 i + wm in word x of vw[i][kk] (masks per lane); the new token's
        // V element comes from the lane of v_new's load that holds the dim
        uint32_t vnw[kWT] = {};
        if constexpr (Fused) {
#pragma unroll
          for (int i = 0; i < kWT; ++i) {
            const int bits = __shfl((int)__builtin_bit_cast(uint16_t, vn_cur[i / 4]), 16 * (i % 4) + wm);
            vnw[i] = ((uint32_t)bits & 0xffffu) << (16 * (tn & 1));
          }
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int p0 = 32 * kk + 8 * wq + 2 * x;
            const uint32_t keep = (p0 < keep_end ? 0x0000ffffu : 0u) | (p0 + 1 < keep_end ? 0xffff0000u : 0u);
            const bool put = Fused && p0 == (tn & ~1);
#pragma unroll
            for (int i = 0; i < kWT; ++i) {
              uint4_t wv = __builtin_bit_cast(uint4_t, vw[i][kk]);
              wv[x] = (wv[x] & keep) | (put ? vnw[i] : 0u);
              vw[i][kk] = __builtin_bit_cast(half8_t, wv);
            }
          }
      } else {
      uint32_t vnw[kSets];
#pragma unroll
      for (int st = 0; st < kSets; ++st)
        vnw[st] = (uint32_t)__builtin_bit_cast(uint16_t, vn_cur[st]) << (16 * (tn & 1));
      static_for<0, 32>([&](auto iw) {
        constexpr int word = decltype(iw)::value;  // word w: positions 2w, 2w + 1
        constexpr int g = word / 4, i = word % 4;
        const uint32_t keep = (2 * word < keep_end ? 0x0000ffffu : 0u) |
                              (2 * word + 1 < keep_end ? 0xffff0000u : 0u);
        const bool put = Fused && word == (tn >> 1);
#pragma unroll
        for (int st = 0; st < kSets; ++st) {
          uint4_t w = __builtin_bit_cast(uint4_t, vreg[g][st]);
          w[i] = (w[i] & keep) | (put ? vnw[st] : 0u);
          vreg[g][st] = __builtin_bit_cast(half8_t, w);
        }
      });
      }
    }

    __builtin_amdgcn_wave_barrier();
    if constexpr (Wide) {
      // O^T tile i += V^T (dims 16 i .., tokens 32 kk ..) P^T: lane 16 wq + wm
      // takes query row wm's weights of tokens 32 kk + 8 wq .. + 7
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const half8_t pb8 = *reinterpret_cast<const half8_t*>(p_lds + wm * kPRow + 32 * kk + 8 * wq);
#pragma unroll
        for (int i = 0; i < kWT; ++i) w_acc[i] = mfma16(vw[i][kk], pb8, w_acc[i]);
      }
    } else if constexpr (kValu) {
      // (measurement build) lane = dim 64 st + lane: each head's weights,
      // read from LDS by every lane at once, against its 8-token V groups, in
      // pairs of tokens
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (g < nr) {
#pragma unroll
          for (int grp = 0; grp < 8; ++grp) {
            const half8_t pv = *reinterpret_cast<const half8_t*>(p_lds + g * kPRow + grp * 8);
#pragma unroll
            for (int st = 0; st < kSets; ++st)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                acc_o[0][st][g] = __builtin_amdgcn_fdot2(
                    half2x{pv[2 * i], pv[2 * i + 1]},
                    half2x{vreg[grp][st][2 * i], vreg[grp][st][2 * i + 1]}, acc_o[0][st][g], false);
          }
        }
      }
    } else {
      // lane 4c+g: weights of head g for tokens 4c..4c+3
      half4_t pfrag[kSub];
#pragma unroll
      for (int u = 0; u < kSub; ++u)
        pfrag[u] = *reinterpret_cast<const half4_t*>(p_lds + (4 * u + (lane & 3)) * kPRow +
                                                     (lane >> 2) * 4);

      // out[g][d] += sum_t P[g][t] V[t][d]; chunk c = tokens 4c..4c+3 of the unit
      static_for<0, 16>([&](auto ic) {
        constexpr int c = decltype(ic)::value;
        constexpr int g = c / 2, half = c % 2;  // 8-token group, its half
#pragma unroll
        for (int st = 0; st < kSets; ++st) {
          const half4_t vf = half ? hi4(vreg[g][st]) : lo4(vreg[g][st]);
#pragma unroll
          for (int u = 0; u < kSub; ++u)
            acc_o[u][st] = __builtin_amdgcn_mfma_f32_4x4x4f16(pfrag[u], vf, acc_o[u][st], 4, c, 0);
        }
      });
    }
    load_v(nxt, pb_nxt);
    __builtin_amdgcn_wave_barrier();

    // ---- end of a piece: the run or the share ends ------------------------
    const bool run_end = cur.g + 1 == cur.n_s;
    if (run_end || !nxt.valid) {
      float l_tot[kSub][4];
      float lt_w = 0.0f;  // Wide: query row wm's sum
      if constexpr (Wide) {
        lt_w = sum_row4(w_l);
      } else {
#pragma unroll
        for (int u = 0; u < kSub; ++u)
#pragma unroll
          for (int g = 0; g < 4; ++g) l_tot[u][g] = (g < nrs[u]) ? wave_sum(l_lane[u][g]) : 1.0f;
      }
      // The piece goes to the merger through the LDS ring (wait while the
      // ring is full, which the merger rarely lets happen): a whole run
      // (slot -1), which the merger normalises and stores, or a cut piece: a
      // piece that starts a run goes to slot r, the piece that starts this
      // worker's share inside a run to slot R + w.  The streamer itself
      // stores nothing inside the loop: a wave's memory operations complete
      // in order, so a store here would hold back the K/V loads issued after
      // it, a memory latency at every run end.
      // (Wide: one entry per sub-group of the pass, as the pieces of the
      // sub-groups' copies of the batch: sequence u Sr + s and share slot
      // R + u nw + w for sub-group u)
      const uint64_t t_ring = stamp_now();
      for (int spin = 0; ring_made - lds_ld(&ctl[kCtlRingTaken]) > kRing - n_sub; ++spin) {
        if (spin >= a.spin_limit) {  // give up (reported in the status word)
          if (lane == 0)
            __hip_atomic_store(a.ws.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if constexpr (kTrace) tr[kTrRingWait] += stamp_now() - t_ring;
      if constexpr (Wide) {
        // lane u < n_sub describes entry u; lane 16 wq + wm writes query row
        // wm's part into entry wm / 4, as its row wm % 4
        if (lane < n_sub) {
          const int sv = pass_seq(cur.s, lane);
          const int k = (ring_made + lane) % kRing;
          ring_meta[k][0] = sv;
          ring_meta[k][1] = cur.h;
          ring_meta[k][2] = (piece_g0 == 0 && run_end) ? -1
                            : piece_g0 == 0            ? sv * Hkv + cur.h
                                                       : R + lane * nw + w;
          ring_meta[k][3] = cur.g - piece_g0 + 1;
        }
        const int u = wm >> 2, g = wm & 3;
        if (u < n_sub) {
          const int k = (ring_made + u) % kRing;
#pragma unroll
          for (int i = 0; i < kWT; ++i)
            *reinterpret_cast<float4_t*>(&ring_o[k][g * D + 16 * i + 4 * wq]) = w_acc[i];
          if (wq == 0) {
            ring_ml[k][2 * g] = w_m;
            ring_ml[k][2 * g + 1] = lt_w;
          }
        }
      } else {
#pragma unroll
      for (int u = 0; u < kSub; ++u) {
        const int sv = cur.s;
        const int slot = (piece_g0 == 0 && run_end) ? -1
                         : piece_g0 == 0            ? sv * Hkv + cur.h
                                                    : R + u * nw + w;
        const int k = (ring_made + u) % kRing;
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int st = 0; st < kSets; ++st)
            ring_o[k][g * D + st * 64 + lane] = acc_o[u][st][g];
        if (lane < 8) {  // (max, sum) of head lane/2
          const int gi = lane >> 1;
          const float mv = gi == 0   ? m_run[u][0]
                           : gi == 1 ? m_run[u][1]
                           : gi == 2 ? m_run[u][2]
                                     : m_run[u][3];
          const float lv = gi == 0   ? l_tot[u][0]
                           : gi == 1 ? l_tot[u][1]
                           : gi == 2 ? l_tot[u][2]
                                     : l_tot[u][3];
          ring_ml[k][lane] = (lane & 1) ? lv : mv;
        }
        if (lane == 0) {
          ring_meta[k][0] = sv;
          ring_meta[k][1] = cur.h;
          ring_meta[k][2] = slot;
          ring_meta[k][3] = cur.g - piece_g0 + 1;
        }
      }
      }
      ring_made += n_sub;
      lds_st(&ctl[kCtlRingMade], ring_made);
      if constexpr (kTrace) ++tr[kTrPieces];
      reset_run();
      q_pending = true;
      piece_g0 = nxt.g;
    }

    // ---- shift the lookahead -------------------------------------------
    cur = nxt;
    nxt = nxt2;
    tbl_nxt = tbl_nxt2;
    if constexpr (Fused) {
#pragma unroll
      for (int st = 0; st < kSets; ++st) vn_cur[st] = vn_nxt[st];
    }
    nxt2 = nxt3;
    if constexpr (kTrace) {
      const uint64_t now = stamp_now();
      for (int i = 0; i < 7; ++i) tr[kTrLastIters + i] = tr[kTrLastIters + i + 1];
      tr[kTrLastIters + 7] = now - t_iter;
      t_iter = now;
    }
    __builtin_amdgcn_wave_barrier();
  }

  tr[kTrStreamEnd] = stamp_now();
  finish();
  store_new_rows();
  if constexpr (kTrace) {
    tr[kTrStoresIssued] = stamp_now();
    tr[kTrXcc] = xcc_id();
    tr[kTrHwId] = hw_id();
    write_trace(kTrEntry, kTrStoresIssued);  // (the helper writes its own slots)
    write_trace(kTrXcc, kTrPieces);
    write_trace(kTrHwId, kTrRingWait);
    write_trace(kTrLastIters, kTrLastIters + 7);
  }
}

namespace {
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Partial slots at the front, the arrival counters at the back of the
// workspace.  A call places its counters against the workspace's end: calls
// of any shape sharing one workspace then find only counters there, which
// every call leaves at zero, and never another call's partial results.
struct WorkspaceLayout {
  int64_t slots;
  size_t ml, o, partial;  // partial slots: offsets, end
  size_t pre_len, pre_lse, pre_o, end;  // shared-prefix area (DecodeWorkspace)
  size_t control;         // arrival counters: size
};

WorkspaceLayout workspace_layout(int64_t S, int64_t Hkv, int64_t D, int64_t workers) {
  WorkspaceLayout l;
  l.slots = S * Hkv + workers;
  // measurement builds: per-worker stamps first
  l.ml = kTrace ? align256((size_t)workers * kTraceSlots * sizeof(uint64_t)) : 0;
  l.o = l.ml + align256((size_t)(l.slots * 8) * sizeof(float));
  l.partial = l.o + align256((size_t)(l.slots * 4 * D) * sizeof(float));
  const size_t pre_rows = (size_t)kPrefixMaxChunks * S * Hkv * kMaxGroup;
  l.pre_len = l.partial;
  l.pre_lse = l.pre_len + align256((size_t)S * sizeof(int));
  l.pre_o = l.pre_lse + align256(pre_rows * sizeof(float));
  l.end = l.pre_o + align256(pre_rows * D * sizeof(half_t));
  l.control = decode_control_bytes(S, Hkv);
  return l;
}
}  // namespace

size_t decode_workspace_bytes(int64_t S, int64_t Hkv, int64_t D, int64_t workers) {
  const WorkspaceLayout l = workspace_layout(S, Hkv, D, workers);
  return l.end + l.control;
}

// arrival counters, then 256 bytes whose last 4 are the status word
size_t decode_control_bytes(int64_t S, int64_t Hkv) {
  return align256((size_t)(S * Hkv) * sizeof(int)) + 256;
}

// ---- the allocation-free decode's workspace --------------------------------
// For callers that cannot allocate device memory (code under graph capture,
// tight serving loops).  Every call on one GPU uses this same array; calls
// that overlap in time on one GPU race.  In host code its name is only a
// stand-in: kernels get the device address from hipGetSymbolAddress.
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
__global__ void zero_words_kernel(uint32_t* p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0;
}

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_static_scratch(hipStream_t stream, void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255)) return hipErrorInvalidSymbol;
    // the arrival counters must start at zero (every call leaves them so);
    // a fill kernel rather than a memset, so that a caller's graph capture
    // may hold it
    uint32_t* control = reinterpret_cast<uint32_t*>(static_cast<char*>(p) + kStaticScratchBytes -
                                                    kStaticControlBytes);
    hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, stream, control,
                       (int64_t)(kStaticControlBytes / sizeof(uint32_t)));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    scratch_ptr[dev] = p;
  }
  *ptr = scratch_ptr[dev];
  return hipSuccess;
}

DecodeWorkspace decode_workspace_carve(void* base, size_t bytes, int64_t S, int64_t Hkv, int64_t D,
                                       int64_t workers) {
  const WorkspaceLayout l = workspace_layout(S, Hkv, D, workers);
  char* p = reinterpret_cast<char*>(base);
  DecodeWorkspace w;
  w.trace = kTrace ? reinterpret_cast<uint64_t*>(p) : nullptr;
  w.ml = reinterpret_cast<float*>(p + l.ml);
  w.o = reinterpret_cast<float*>(p + l.o);
  w.counters = reinterpret_cast<int*>(p + ((bytes - l.control) & ~(size_t)255));
  w.pre_len = reinterpret_cast<int*>(p + l.pre_len);
  w.pre_lse = reinterpret_cast<float*>(p + l.pre_lse);
  w.pre_o = reinterpret_cast<half_t*>(p + l.pre_o);
  w.status = reinterpret_cast<int*>(p + (bytes & ~(size_t)3)) - 1;
  return w;
}

template <int D, int BS, bool Fused, bool Shared, bool Wide>
void launch_decode_f(const DecodeArgs& a, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  const dim3 grid((unsigned)a.num_workers);
  const uint32_t lds = (uint32_t)((size_t)a.num_seqs * (Shared ? 3 : 2) * sizeof(int));
  if (!start && !stop)
    hipLaunchKernelGGL((decode_kernel<D, BS, Fused, Shared, Wide>), grid, dim3(128), lds, stream, a);
  else  // the events take the kernel's own start and end times
    hipExtLaunchKernelGGL((decode_kernel<D, BS, Fused, Shared, Wide>), grid, dim3(128), lds,
                          stream, start, stop, 0, a);
}

template <int D, int BS, bool Wide>
void launch_decode_p(const DecodeArgs& a, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (a.k_new && a.pre_len)
    launch_decode_f<D, BS, true, true, Wide>(a, stream, start, stop);
  else if (a.k_new)
    launch_decode_f<D, BS, true, false, Wide>(a, stream, start, stop);
  else
    launch_decode_f<D, BS, false, false, Wide>(a, stream, start, stop);
}

template <int D, int BS>
void launch_decode_t(const DecodeArgs& a, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if constexpr (!kValu) {
    if (decode_wide(a.kv_split)) {
      launch_decode_p<D, BS, true>(a, stream, start, stop);
      return;
    }
  }
  launch_decode_p<D, BS, false>(a, stream, start, stop);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream, hipEvent_t start,
                         hipEvent_t stop) {
#define PA_DECODE(D, BS) \
  if (a.head_dim == D && a.block_size == BS) launch_decode_t<D, BS>(a, stream, start, stop);
  PA_DECODE(128, 16) PA_DECODE(64, 16) PA_DECODE(128, 8) PA_DECODE(64, 8) PA_DECODE(128, 32)
  PA_DECODE(64, 32)
#undef PA_DECODE
  return hipGetLastError();
}

}  // namespace pa
