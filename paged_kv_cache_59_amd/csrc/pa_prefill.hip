// Multi-query paged attention for gfx950: a chunk of new query tokens per
// sequence attends causally to the sequence's paged context (chunked prefill,
// and the continuation after a prefix-cache hit).
//
// Sources (web pages, by title and section):
//  - "KV Cache in Serving Engines: PagedAttention, Continuous Batching, and
//    Prefix Caching", section 3 "New Problem: Long Prefills Pause Decoding":
//    a long prefill is cut into chunks spread over steps; section 4 "Prefix
//    Caching": blocks found in the cache skip their prefill.
//  - "PagedAttention and Continuous Batching Explained (2026)", "Prefix
//    caching": on a hit only the tokens after the cached full blocks remain;
//    "FAQ": the attention itself is the ordinary one.
// A chunk of n_q rows is the last n_q positions of the sequence's context
// (their K/V already appended); the row at position p sees positions 0..p.
//
// Work: one wave computes a tile of 32 rows of one (sequence, KV head) --
// rows enumerate (chunk token, query head of the group) -- against the keys
// 0 .. (its last row's position), 32 keys per step:
//   S^T = K . Q^T  (v_mfma_f32_16x16x32_f16, A = 16 keys x 32 dims of K,
//                   B = 32 dims x 16 rows of Q^T)
//   O^T += V^T . P^T (A = 16 dims x 32 keys of V^T, B = 32 keys x 16 rows)
// With lane l = 16 j + c: the A/B operand of lane l covers k-slots
// 8j..8j+7 of row/column c, and the result of lane l is rows 4j..4j+3 of
// column c.  Key k-row m of S^T sub-tile kt is loaded as key
// 8 (m / 4) + 4 kt + m % 4 of the 32-key step, so lane l's 8 logits of its
// row c are the keys 8j..8j+7 in order: exactly its P^T operand.  Those are
// 8 consecutive tokens of one 8-token V group, so its V^T operand is one
// 16-byte load, and the O^T result of lane l is its own row c, the row whose
// softmax state it holds.
//
// K and V reach the waves through LDS: a workgroup's 4 waves (128 rows of
// one (sequence, KV head)) share every 32-key step, which the waves copy
// from memory into a ring of kStages steps with LDS-DMA loads
// (global_load_lds_dwordx4, 1 KiB per wave instruction), kStages - 1 steps
// ahead.  Read straight from L2 into each wave's registers, every step's
// K/V would cross the L2-to-CU path 4 times, which bounds the MFMA rate at
// about half of peak (a 32-row wave needs 1/32 byte of K/V per flop).  In LDS
// the K tile is stored in the MFMA's key order and the V tile by 8-key group,
// so that each 16-lane group of a wave reads 256 contiguous bytes.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "pa_internal.h"

namespace pa {
namespace {

typedef float float4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half8_t ld16(const half_t* p) {
  return *reinterpret_cast<const half8_t*>(p);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));

// sum of the 8 halves of v, accumulated in fp32 (v_dot2_f32_f16 against ones)
__device__ __forceinline__ float sum8(half8_t v) {
  const half2v one = {(half_t)1.0f, (half_t)1.0f};
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    acc = __builtin_amdgcn_fdot2(half2v{v[2 * i], v[2 * i + 1]}, one, acc, false);
  return acc;
}

// Max over lanes l, l ^ 16, l ^ 32, l ^ 48 (the 4 k-slot groups of one row)
// of two values at once (the two row sub-tiles' maxima), with the gfx950
// cross-row swaps, three in all: (m0, m1) -> rows 0..3 hold the maxima of
// rows (0, 1) of m0, (0, 1) of m1, (2, 3) of m0, (2, 3) of m1; then the
// halves are combined; then each result is spread over all four rows.
__device__ __forceinline__ void max_rows2(float& m0, float& m1) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(m0), __float_as_uint(m1), false, false);
  const float x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float z = fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(z), __float_as_uint(z), false, false);
  m0 = __uint_as_float(r[0]);
  m1 = __uint_as_float(r[1]);
}

__device__ __forceinline__ float4v mfma16x16x32(half8_t a, half8_t b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

}  // namespace

template <int D, int BS>
__global__ __launch_bounds__(256, 2) void prefill_kernel(const PrefillArgs a) {
  constexpr int KS = D / 32;             // 32-dim steps of the contraction over D
  constexpr int DT = D / 16;             // 16-dim tiles of the output
  constexpr int64_t kTile = (int64_t)BS * D;
  constexpr int NBS = 32 / BS;           // blocks per 32-key step (4, 2 or 1)
  static_assert(NBS * BS == 32, "block size 8, 16 or 32");
  static_assert(kPrefillWaves == 4 && kPrefillWaveRows == 32, "4 waves of 32 rows");
  constexpr float kStale = 8.0f;         // see the rescale below
  constexpr float kFloor = -1.0e30f;     // initial reference max (log2 units)
  constexpr int kTileBytes = 32 * D * 2;        // K (or V) of one 32-key step
  constexpr int kStepBytes = 2 * kTileBytes;    // K then V
  constexpr int kDmaPerTile = kTileBytes / 4096;  // wave instructions per tile and wave
  constexpr int kDmaPerStep = 2 * kDmaPerTile;
  static_assert(kDmaPerTile * 4096 == kTileBytes, "head_dim must be 64 or 128");
  extern __shared__ __attribute__((aligned(16))) char kv_lds[];  // [kPrefillStages][kStepBytes]
  constexpr int kStages = kPrefillStages;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15;  // column of the MFMA operands / results: this lane's row
  const int j = lane >> 4;    // k-slot group

  // Workgroup i runs on XCD i % 8.  (sequence, KV head) pairs are dealt to
  // the XCDs round-robin (XCD x takes pairs x, x + 8, ...), so that the KV
  // heads of one sequence -- equal work -- spread over the XCDs while all
  // workgroups of one pair share one L2; within a pair the tile groups go
  // last first, the ones with the most keys (causal) dispatched first.
  const int xcd = (int)(blockIdx.x % 8);
  const int m = (int)(blockIdx.x / 8);
  const int sh = 8 * (m / a.tile_groups) + xcd;
  if (sh >= a.num_seqs * a.num_kv_heads) return;
  const int s = sh / a.num_kv_heads;
  const int h = sh - s * a.num_kv_heads;
  const int group = a.tile_groups - 1 - m % a.tile_groups;
  const int tile = group * 4 + wave;

  const int Hq = a.num_q_heads;
  const int G = Hq / a.num_kv_heads;
  const int t0 = a.query_start[s];
  const int nq = a.query_start[s + 1] - t0;
  const int len = min(max(a.context_lens[s], 0), a.max_context_len);
  // an empty chunk, or one that breaks a precondition (longer than its
  // context or than the bound, or rows outside q): nothing to do (the whole
  // workgroup leaves together)
  if (nq <= 0 || nq > len || nq > a.max_query_len || t0 < 0 || t0 + nq > a.num_tokens) return;
  const int rows = nq * G;
  if (group * 128 >= rows) return;
  // steps of the workgroup: keys 0 .. the position of its last row; every
  // wave takes part in all of them (the ring's barriers), and computes those
  // up to its own last row
  const int wg_last_row = min(group * 128 + 127, rows - 1);
  const int nsteps = (len - nq + wg_last_row / G) / 32 + 1;
  const bool active = tile * 32 < rows;  // (uniform per wave)

  // this lane's two rows (sub-tiles rt = 0, 1)
  int tok[2], grp[2], pos[2];
  bool valid[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int r = tile * 32 + rt * 16 + c16;
    valid[rt] = r < rows;
    const int rr = valid[rt] ? r : rows - 1;
    tok[rt] = rr / G;
    grp[rt] = rr - tok[rt] * G;
    pos[rt] = valid[rt] ? len - nq + tok[rt] : -1;
  }
  const int last_row = active ? min(tile * 32 + 31, rows - 1) : rows - 1;
  const int pos_first = len - nq + (min(tile * 32, rows - 1)) / G;  // the tile's first position
  const int my_steps = active ? (len - nq + last_row / G) / 32 + 1 : 0;

  // Q^T operands, held for the whole loop
  half8_t qf[2][KS];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const half_t* qp = a.q + ((int64_t)(t0 + tok[rt]) * Hq + h * G + grp[rt]) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[rt][ks] = ld16(qp + ks * 32 + j * 8);
      if (a.negate_q) qf[rt][ks] = -qf[rt][ks];  // exact: a sign flip
    }
  }

  const int32_t* row = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const int last_blk = (len + BS - 1) / BS - 1;
  const int64_t hoff = (int64_t)h * kTile;
  // elements per physical block (all heads); below 2^32, so a block's
  // offset is one 32 x 32 -> 64-bit product
  const uint32_t bstride = (uint32_t)a.num_kv_heads * (uint32_t)kTile;
  // ids at or past the pool's end (or negative) are broken entries
  const uint32_t nblk = (uint32_t)min(a.num_blocks, (int64_t)0x7fffffff);
  // physical block of logical block lb (clamped to the sequence's last): a
  // scalar load, whose wait (lgkmcnt) does not drain the loads in flight
  // (read through the constant address space: a scalar load, which the LDS
  // copies in flight cannot be taken to alias)
  const __attribute__((address_space(4))) int32_t* crow =
      (const __attribute__((address_space(4))) int32_t*)row;
  auto phys_of = [&](int lb) -> int {
    const int e = crow[__builtin_amdgcn_readfirstlane(min(lb, last_blk))];
    return (uint32_t)e < nblk ? e : 0;  // a broken table entry reads block 0
  };
  // The NBS blocks of a step (keys i BS .. i BS + BS - 1 in block i), as
  // separate scalars (uniform): a lane picks its own with selects.  (Held
  // in a struct or an array across the loop, the compiler indexes them in
  // scratch memory.)
  int nb0 = 0, nb1 = 0, nb2 = 0, nb3 = 0;  // the next step to issue
  auto fetch_blocks = [&](int st) {
    st = min(st, nsteps - 1);  // steps past the end re-read the last one
    nb0 = phys_of(NBS * st);
    if (NBS > 1) nb1 = phys_of(NBS * st + 1);
    if (NBS > 2) {
      nb2 = phys_of(NBS * st + 2);
      nb3 = phys_of(NBS * st + 3);
    }
  };
  // Per-lane constant parts of the copies (element offsets inside a block's
  // head tile, and which block of the step a lane's K piece lies in); per
  // step only the blocks' offsets (uniform, scalar) and a select remain.
  //   K tile: [chunk c of 8 dims][slot 16 kt + c][8 dims]; slot (kt, c)
  //           holds key 8 (c / 4) + 4 kt + c % 4 (the MFMA's key order).
  //   V tile: [8-key group jj][dim][8 keys].
  int k_off[kDmaPerTile], k_blk[kDmaPerTile], v_off[kDmaPerTile], v_blk[kDmaPerTile];
#pragma unroll
  for (int i = 0; i < kDmaPerTile; ++i) {
    const int ci = wave * kDmaPerTile + i;
    const int c = 2 * ci + (lane >> 5), slot = lane & 31;
    const int cs = slot & 15, key = 8 * (cs >> 2) + (cs & 3) + 4 * (slot >> 4);
    k_blk[i] = key / BS;
    k_off[i] = (c * BS + key % BS) * 8;
    const int e = ci * 64 + lane, jj = e / D, d = e % D;
    v_blk[i] = __builtin_amdgcn_readfirstlane((8 * jj) / BS);  // uniform per instruction
    v_off[i] = ((8 * jj % BS) / 8 * D + d) * 8;
  }

  // One step's K and V into ring stage `stage`: each wave writes its
  // kDmaPerTile KiB of each tile; lane L of wave instruction ci writes 16
  // bytes at ci KiB + 16 L.
  auto issue = [&](int b0, int b1, int b2, int b3, int stage) {
    char* base = kv_lds + stage * kStepBytes;
    // the step's blocks' offsets (uniform) and a lane's pick among them.
    // Selects work on the index's bits (a compare chain on one index becomes
    // a table the compiler keeps in scratch memory).  With two blocks per
    // step the lane selects between two 64-bit offsets; with four it selects
    // the block id and multiplies.  Each form measured the faster at its
    // block size (at 8: 317 against 329 us; at 16: 287 against 299 us).
    auto boff = [&](int b) { return (int64_t)((uint64_t)(uint32_t)b * bstride) + hoff; };
    const int64_t o0 = boff(b0), o1 = boff(b1);
    auto sel = [&](int i) -> int64_t {
      if constexpr (NBS == 1) return o0;
      else if constexpr (NBS == 2) return (i & 1) ? o1 : o0;
      else {
        const int lo = (i & 1) ? b1 : b0, hi = (i & 1) ? b3 : b2;
        return boff((i & 2) ? hi : lo);
      }
    };
#pragma unroll
    for (int i = 0; i < kDmaPerTile; ++i) {
      const int ci = wave * kDmaPerTile + i;
      const half_t* src = a.k_cache + sel(k_blk[i]) + k_off[i];
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(base + ci * 1024),
                                       16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kDmaPerTile; ++i) {
      const int ci = wave * kDmaPerTile + i;
      const half_t* src = a.v_cache + sel(v_blk[i]) + v_off[i];
      __builtin_amdgcn_global_load_lds(
          src, (__attribute__((address_space(3))) void*)(base + kTileBytes + ci * 1024), 16, 0, 0);
    }
  };
  half8_t kf[2][KS], vf[DT];
  auto read_k = [&](int stage) {
    const char* base = kv_lds + stage * kStepBytes;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[kt][ks] = *reinterpret_cast<const half8_t*>(base + ((4 * ks + j) * 32 + kt * 16 + c16) * 16);
  };
  auto read_v = [&](int stage) {
    const char* base = kv_lds + stage * kStepBytes + kTileBytes;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      vf[dt] = *reinterpret_cast<const half8_t*>(base + (j * D + dt * 16 + c16) * 16);
  };
  // s_waitcnt for "at most n vector memory operations of this wave in
  // flight" (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt
  // left at their maxima, i.e. not waited for)
  auto wait_vm = [](auto n) {
    constexpr int N = decltype(n)::value;
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
  };

  float4v o[2][DT];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[rt][dt] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
  // Reference max per row, log2 units.  It starts at a finite floor far
  // below any logit, so exp2(z - m) is 0 for removed keys (z = -inf) without
  // a select, and the first key raises it (the rescale below).
  float m_run[2] = {kFloor, kFloor};
  float l_lane[2] = {0.0f, 0.0f};

  // Ring: steps 0 .. kStages - 2 are issued first; at step st the waves
  // wait for their own copies of step st, meet at a barrier (then every
  // wave's copy has landed, and every wave is done with stage (st - 1) %
  // kStages), and issue step st + kStages - 1 into that stage.  Every step
  // issues the same loads (past the end they re-read the last step), so the
  // wait counts are exact.  Table entries are read one issue ahead.
  fetch_blocks(0);
#pragma unroll
  for (int p = 0; p < kStages - 1; ++p) {
    const int b0 = nb0, b1 = nb1, b2 = nb2, b3 = nb3;
    fetch_blocks(p + 1);
    issue(b0, b1, b2, b3, p);
  }
  for (int st = 0; st < nsteps; ++st) {
    const int stage = st % kStages;
    wait_vm(std::integral_constant<int, kDmaPerStep * (kStages - 2)>{});
    __builtin_amdgcn_s_barrier();
    {
      const int b0 = nb0, b1 = nb1, b2 = nb2, b3 = nb3;
      fetch_blocks(st + kStages);
      issue(b0, b1, b2, b3, (st + kStages - 1) % kStages);
    }
    if (st >= my_steps) continue;  // past this wave's last row (uniform)

    read_k(stage);
    // logits of both row sub-tiles
    float4v sacc[2][2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        sacc[rt][kt] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          sacc[rt][kt] = mfma16x16x32(kf[kt][ks], qf[rt][ks], sacc[rt][kt]);
      }
    __builtin_amdgcn_s_setprio(1);
    read_v(stage);

    // raw logits of keys 32 st + 8 j + e, e = 4 kt + i, of this lane's row.
    // The scale c > 0 (the host folds a negative scale into q's sign) enters
    // through the row max, max(c z) = c max(z), and the exponent's fma.
    float z[2][8], mt[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int e = 0; e < 8; ++e) z[rt][e] = sacc[rt][e >> 2][e & 3];
    // Only the steps that reach past the tile's first position can hold keys
    // past a row's position (removed: z = -inf) or past the context (V := 0
    // by selection: the last block's tail holds any bits, NaN included, and
    // 0 * NaN would not be 0).  One uniform branch for both.
    if (st * 32 + 31 > pos_first) {  // (uniform: st and pos_first are)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kp = st * 32 + 8 * j + e;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) z[rt][e] = kp <= pos[rt] ? z[rt][e] : -INFINITY;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vf[dt][e] = kp >= len ? (half_t)0.0f : vf[dt][e];
      }
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      mt[rt] = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) mt[rt] = fmaxf(mt[rt], z[rt][e]);
    }
    max_rows2(mt[0], mt[1]);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) mt[rt] *= a.scale_log2;
    // The reference max m_run is raised only when a row's max passes it by
    // more than kStale (log2 units); otherwise the weights exp2(z - m_run)
    // stay below 2^kStale, well inside fp16, and O and l need no rescale.
    // The result O / l does not depend on the reference.
    if (__any(mt[0] > m_run[0] + kStale || mt[1] > m_run[1] + kStale)) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const float m_new = fmaxf(m_run[rt], mt[rt]);
        const float alpha = exp2_fast(m_run[rt] - m_new);  // 0 when leaving the floor
        l_lane[rt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[rt][dt] *= alpha;
        m_run[rt] = m_new;
      }
    }
    half8_t pf[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float2v w = {exp2_fast(__builtin_fmaf(z[rt][e], a.scale_log2, -m_run[rt])),
                           exp2_fast(__builtin_fmaf(z[rt][e + 1], a.scale_log2, -m_run[rt]))};
        const half2v hw = __builtin_convertvector(w, half2v);  // round to nearest even
        pf[rt][e] = hw[0];
        pf[rt][e + 1] = hw[1];
      }
      l_lane[rt] += sum8(pf[rt]);
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[rt][dt] = mfma16x16x32(vf[dt], pf[rt], o[rt][dt]);
    __builtin_amdgcn_s_setprio(0);
  }
  wait_vm(std::integral_constant<int, 0>{});  // the ring's last copies land before the wave ends
  if (!active) return;

  // out[row][dims 16 dt + 4 j .. +3] = O^T / l
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    float l = l_lane[rt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (!valid[rt]) continue;
    const float inv = 1.0f / l;
    half_t* op = a.out + ((int64_t)(t0 + tok[rt]) * Hq + h * G + grp[rt]) * D + 4 * j;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      half4_t r;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = (half_t)(o[rt][dt][i] * inv);
      *reinterpret_cast<half4_t*>(op + dt * 16) = r;
    }
  }
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const int64_t pairs = (int64_t)a.num_seqs * a.num_kv_heads;
  const int64_t padded = (pairs + 7) / 8 * 8 * a.tile_groups;  // 8 XCDs x pairs/8 x tile groups
  const dim3 grid((unsigned)padded);
#define PA_PREFILL(D, BS)                                                             \
  if (a.head_dim == D && a.block_size == BS)                                         \
    hipLaunchKernelGGL((prefill_kernel<D, BS>), grid, dim3(256),                     \
                       (size_t)kPrefillStages * 2 * 32 * D * sizeof(half_t), stream, a);
  PA_PREFILL(128, 16) PA_PREFILL(64, 16) PA_PREFILL(128, 8) PA_PREFILL(64, 8) PA_PREFILL(128, 32)
  PA_PREFILL(64, 32)
#undef PA_PREFILL
  return hipGetLastError();
}

}  // namespace pa
