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
//  * Work balance.  Each (sequence, KV head) pair is a run of 64-token units
//    (4 blocks each).  All runs are laid end to end in (sequence, head) order
//    and a fixed grid of persistent workers (one wave each, 8 per compute
//    unit) takes equal contiguous shares, so ragged lengths cost nothing in
//    tail.  Each worker finds its share from a prefix sum of the lengths that
//    it computes itself (no host knowledge of the lengths is needed).
//  * A run cut between workers is finished by the last of them to arrive: each
//    writes (max, sum, unnormalised output) to the workspace, bumps a counter,
//    and the one that sees the count complete merges with the log-sum-exp
//    rescale and resets the counter.  One launch per decode.
//  * Consecutive workers are placed on one XCD (workgroups are handed to the 8
//    XCDs in turn), so neighbouring runs, e.g. sequences sharing prefix blocks,
//    meet in the same L2.
//  * The grouped query heads of one KV head (G <= 4) are the 4 rows of the
//    4x4x4 16-block MFMA, so every K and V element loaded serves all G heads;
//    the G q rows stay in 1 KiB of LDS for the whole run (in registers they
//    would cost 64 per lane and halve the waves a SIMD holds).
//  * q . K: lane l owns token l of the 64; it loads its 16-byte chunks of the
//    K row (K pool [NB][Hkv][D/8][16][8]: for a fixed chunk the 64 lanes read
//    four contiguous 256-byte runs) and feeds them as the B operand, so the
//    dot products reduce inside the MFMA, with no cross-lane sums.
//  * Online softmax: running max per head (wave max per unit, DPP within rows
//    of 16), per-lane partial sums (one wave sum per run).
//  * The fp16 probabilities are transposed through 512 bytes of LDS so lane
//    4c+g holds head g's weights of tokens 4c..4c+3; the MFMA broadcast
//    (CBSZ=4, ABID=c) hands that quad to all 16 blocks.
//  * P . V: lane l owns output dims l and l+64; V pool [NB][Hkv][2][D][8] puts
//    8 consecutive tokens of one dim in 16 bytes, so for a fixed (block, half)
//    the 64 lanes read 1 KiB contiguous.
//  * Software pipeline: the next unit's K loads are issued once this unit's
//    logits are formed, its V loads once this unit's P.V is done; every unit
//    but a run's last issues the same 32 loads (block ids past the run's end
//    re-read its last block) so the hardware wait counts stay exact.  K and V
//    are read with non-temporal loads (each byte is used once).
//  * Positions at or past the length are removed by selection (logit -inf,
//    V element 0), never by multiplication, so NaN or huge values in the
//    unused tail of the last block cannot leak.
#include <type_traits>

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

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ int wave_sum_int(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
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

// Max over the 64 lanes, in every lane: DPP within each row of 16 (swap
// pairs, swap pairs of pairs, mirror halves, mirror the row), then the four
// row results read out as scalars.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp<0x140>(x));  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Sum over the 64 lanes, in every lane (same pattern as wave_max).
__device__ __forceinline__ float wave_sum_dpp(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ half4_t lo4(half8_t v) { return __builtin_shufflevector(v, v, 0, 1, 2, 3); }
__device__ __forceinline__ half4_t hi4(half8_t v) { return __builtin_shufflevector(v, v, 4, 5, 6, 7); }

__device__ __forceinline__ half8_t load_nt(const half_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const half8_t*>(p));
}

// The work share of worker w among nw over `total` units: [begin(w), begin(w+1)).
__device__ __forceinline__ int64_t share_begin(int64_t w, int64_t nw, int64_t total) {
  return w * total / nw;
}
// The worker whose share holds unit u.
__device__ __forceinline__ int64_t share_owner(int64_t u, int64_t nw, int64_t total) {
  return ((u + 1) * nw - 1) / total;
}

}  // namespace

template <int D>
__global__ __launch_bounds__(64) void decode_kernel(const DecodeArgs a) {
  constexpr int kChunks = D / kChunk;  // 16-byte chunks in one K row
  constexpr int kSets = D / 64;        // 64-dim ranges a lane covers in P.V
  constexpr int64_t kTile = (int64_t)kBlockSize * D;
  constexpr int kLenRegs = 4;          // lengths of the first 256 sequences stay in registers
  static_assert(kChunks * kChunk == D && kSets * 64 == D, "head_dim must be 64 or 128");
  static_assert(kLenRegs == 4, "four length registers");

  const int lane = threadIdx.x;
  const int nw = gridDim.x;
  // consecutive logical workers on one XCD (workgroup i runs on XCD i % 8)
  const int w = (nw % 8 == 0) ? (int)(blockIdx.x % 8) * (nw / 8) + (int)(blockIdx.x / 8)
                              : (int)blockIdx.x;
  const int S = a.num_seqs;
  const int Hkv = a.num_kv_heads;
  const int Hq = a.num_q_heads;
  const int G = Hq / Hkv;

  auto clamp_len = [&](int c) { return min(max(c, 0), a.max_context_len); };
  auto units_for = [](int c) { return (c + kGroupTokens - 1) / kGroupTokens; };

  // ---- lengths: total units; zero the rows of empty sequences ------------
  // clamped length of sequence 64*k + lane, k < kLenRegs (separate variables,
  // never an indexed array: that would live in scratch memory)
  int len0 = 0, len1 = 0, len2 = 0, len3 = 0;
  int64_t seq_units = 0;  // sum over sequences of ceil(len / 64)
  for (int c0 = 0, k = 0; c0 < S; c0 += 64, ++k) {
    const int s = c0 + lane;
    const int c = s < S ? clamp_len(a.context_lens[s]) : 0;
    if (k == 0) len0 = c;
    if (k == 1) len1 = c;
    if (k == 2) len2 = c;
    if (k == 3) len3 = c;
    const int n = units_for(c);
    seq_units += wave_sum_int(n);
    uint64_t empty = __ballot(s < S && n == 0 && (s % nw) == w);
    while (empty) {
      const int se = c0 + __builtin_ctzll(empty);
      empty &= empty - 1;
      half_t* o = a.out + (int64_t)se * Hq * D;
      for (int e = lane; e < Hq * D; e += 64) o[e] = (half_t)0.0f;
    }
  }
  // clamped length of sequence s (s uniform; the result is uniform): from
  // registers when it can
  auto len_of = [&](int s) {
    const int k = s >> 6, l = s & 63;
    int c;
    if (k == 0) c = __builtin_amdgcn_readlane(len0, l);
    else if (k == 1) c = __builtin_amdgcn_readlane(len1, l);
    else if (k == 2) c = __builtin_amdgcn_readlane(len2, l);
    else if (k == 3) c = __builtin_amdgcn_readlane(len3, l);
    else c = clamp_len(a.context_lens[s]);
    return __builtin_amdgcn_readfirstlane(c);
  };

  // the sums are equal in every lane; say so, so that all the work-share
  // arithmetic below is scalar
  seq_units = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(seq_units >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((int)seq_units));
  const int64_t total = seq_units * Hkv;
  if (total == 0) return;
  const int64_t nwa = min((int64_t)nw, total);  // active workers: each gets >= 1 unit
  if (w >= nwa) return;
  const int64_t u_begin = share_begin(w, nwa, total);
  const int64_t u_end = share_begin(w + 1, nwa, total);

  // ---- the unit u_begin: its sequence by a prefix sum of the units --------
  // units of sequence s are [Hkv*O_s, Hkv*O_{s+1}), ordered (head, unit)
  struct Cursor {
    int s, h, g, n_s, len;
    int64_t o_s;  // units of the sequences before s
  };
  Cursor cur{};
  {
    const int64_t key = u_begin / Hkv;
    int64_t base = 0;
    for (int c0 = 0, k = 0; c0 < S; c0 += 64, ++k) {
      const int s = c0 + lane;
      const int c = k == 0 ? len0 : k == 1 ? len1 : k == 2 ? len2 : k == 3 ? len3
                  : (s < S ? clamp_len(a.context_lens[s]) : 0);
      const int n = s < S ? units_for(c) : 0;
      const int incl = wave_inclusive_scan(n, lane);
      const uint64_t hit = __ballot(s < S && base + incl > key);
      if (hit) {
        const int l = __builtin_ctzll(hit);
        cur.s = __builtin_amdgcn_readfirstlane(c0 + l);
        cur.n_s = __builtin_amdgcn_readfirstlane(__shfl(n, l));
        cur.len = __builtin_amdgcn_readfirstlane(__shfl(c, l));
        const int64_t o = base + __builtin_amdgcn_readfirstlane(__shfl(incl, l)) - cur.n_s;
        cur.o_s = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(o >> 32)) << 32) |
                            (uint32_t)__builtin_amdgcn_readfirstlane((int)o));
        break;
      }
      base += __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
    }
  }
  if (cur.n_s == 0) return;  // unreachable for consistent lengths; never divide by 0
  {
    const int64_t r = u_begin - (int64_t)Hkv * cur.o_s;
    cur.h = (int)(r / cur.n_s);
    cur.g = (int)(r - (int64_t)cur.h * cur.n_s);
  }
  // the unit after c in (sequence, head, unit) order; empty sequences skipped
  auto advance = [&](Cursor c) {
    if (c.g + 1 < c.n_s) {
      ++c.g;
    } else if (c.h + 1 < Hkv) {
      ++c.h;
      c.g = 0;
    } else {
      c.o_s += c.n_s;
      c.h = 0;
      c.g = 0;
      do {
        ++c.s;
        c.len = c.s < S ? len_of(c.s) : 0;
        c.n_s = units_for(c.len);
      } while (c.n_s == 0 && c.s < S);
    }
    return c;
  };

  __shared__ half_t p_lds[4 * 64];
  __shared__ __attribute__((aligned(16))) half_t q_lds[4 * D];
  const int my_blk = lane >> 4;  // which of a unit's 4 blocks holds this lane's token
  const int g_lane = lane & 3;   // q head of the group this lane's MFMA row carries
  const int64_t block_stride = (int64_t)Hkv * kTile;

  // Table entries of unit c's 4 blocks: one vector load, lane i & 3 reads
  // entry 4g + (i & 3).  Blocks past the sequence's last re-read its last
  // block, so every unit issues the same loads; positions past the end are
  // removed later by position.
  auto load_table = [&](const Cursor& c) {
    const int32_t* row = a.block_tables + (int64_t)c.s * a.max_blocks_per_seq;
    const int last = (c.len + kBlockSize - 1) / kBlockSize - 1;
    return row[min(4 * c.g + (lane & 3), last)];
  };
  // The 4 physical ids (uniform) from such a load; an id outside the pool (a
  // broken table) reads pool block 0 instead.
  auto blocks_of = [&](int tbl, int (&pb)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = __builtin_amdgcn_readlane(tbl, i);
      pb[i] = (e >= 0 && e < a.num_blocks) ? e : 0;
    }
  };

  half8_t kreg[kChunks];
  half8_t vreg[4][kSets][2];
  half8_t qreg;  // lane g*kChunks + c: 16-byte chunk c of q row g of a run
  auto load_k = [&](const Cursor& c, const int (&pb)[4]) {
    const int phys = my_blk == 0 ? pb[0] : my_blk == 1 ? pb[1] : my_blk == 2 ? pb[2] : pb[3];
    const half_t* kp = a.k_cache + (int64_t)phys * block_stride + (int64_t)c.h * kTile +
                       (lane & 15) * kChunk;
#pragma unroll
    for (int cc = 0; cc < kChunks; ++cc) kreg[cc] = load_nt(kp + cc * (kBlockSize * kChunk));
  };
  auto load_v = [&](const Cursor& c, const int (&pb)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const half_t* vp = a.v_cache + (int64_t)pb[i] * block_stride + (int64_t)c.h * kTile;
#pragma unroll
      for (int st = 0; st < kSets; ++st)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          vreg[i][st][hh] = load_nt(vp + ((int64_t)hh * D + st * 64 + lane) * kChunk);
    }
  };
  // q rows of c's run; every lane loads (rows past G and lanes past the rows
  // re-read row 0 and are zeroed at the LDS write) so the load is unconditional
  const int q_row = lane / kChunks, q_chunk = lane % kChunks;
  auto load_q = [&](const Cursor& c) {
    const int row = (q_row < G && q_row < 4) ? q_row : 0;
    qreg = *reinterpret_cast<const half8_t*>(a.q + ((int64_t)c.s * Hq + c.h * G + row) * D +
                                             q_chunk * kChunk);
  };
  auto store_q = [&]() {
    if (q_row < 4) {
      const half8_t v = q_row < G ? qreg : half8_t{};
      *reinterpret_cast<half8_t*>(q_lds + q_row * D + q_chunk * kChunk) = v;
    }
  };

  // per-run softmax state
  float m_run[4], l_lane[4];
  float4_t acc_o[kSets];
  auto reset_run = [&]() {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      m_run[g] = -INFINITY;
      l_lane[g] = 0.0f;
    }
#pragma unroll
    for (int st = 0; st < kSets; ++st) acc_o[st] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  };

  // cut runs of this share (its first and its last), merged after the stream
  int cut_n = 0;
  int cut_s[2] = {0, 0}, cut_h[2] = {0, 0}, cut_ns[2] = {0, 0};
  int64_t cut_os[2] = {0, 0};

  // ---- prologue: first unit's loads, next unit's table entries ------------
  // Lookahead: cur is computed, nxt has its K/V loads in flight and its ids in
  // pb_nxt, nxt2 has its table entries loading into tbl_nxt2.  Past the end of
  // the share the cursors stay on the last unit (harmless re-reads).
  const int64_t n_units = u_end - u_begin;
  Cursor nxt = cur;
  if (n_units > 1) nxt = advance(cur);
  Cursor nxt2 = nxt;
  if (n_units > 2) nxt2 = advance(nxt);
  int pb_cur[4], pb_nxt[4];
  const int tbl_cur = load_table(cur);
  int tbl_nxt = load_table(nxt);
  load_q(cur);
  blocks_of(tbl_cur, pb_cur);
  // keep the prologue in loop order (all K loads, then all V loads): the
  // wait counts at the loop head are merged over both ways in
  __builtin_amdgcn_sched_barrier(0);
  load_k(cur, pb_cur);
  __builtin_amdgcn_sched_barrier(0);
  load_v(cur, pb_cur);
  __builtin_amdgcn_sched_barrier(0);
  store_q();
  __syncthreads();
  reset_run();
  int piece_first_g = cur.g;  // first unit of the current run in this share
  bool first_piece = true;

  for (int64_t ui = 0; ui < n_units; ++ui) {
    const bool last_unit = ui + 1 == n_units;
    // the next unit's loads go to nxt (the current unit again past the share)
    const int t0 = cur.g * kGroupTokens;

    // logits: S[g][token lane] = q_g . K_token  (rows = heads, columns = tokens)
    float4_t sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const half8_t qv = *reinterpret_cast<const half8_t*>(q_lds + g_lane * D + c * kChunk);
      sacc = __builtin_amdgcn_mfma_f32_4x4x4f16(lo4(qv), lo4(kreg[c]), sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_4x4x4f16(hi4(qv), hi4(kreg[c]), sacc, 0, 0, 0);
    }
    // table entries two units ahead, then the next unit's K and q
    const int tbl_nxt2 = load_table(nxt2);
    blocks_of(tbl_nxt, pb_nxt);
    load_k(nxt, pb_nxt);
    load_q(nxt);

    // online softmax over these 64 positions
    const bool live = (t0 + lane) < cur.len;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      half_t ph = (half_t)0.0f;
      if (g < G) {
        const float z = live ? sacc[g] * a.scale_log2 : -INFINITY;
        const float m_new = fmaxf(m_run[g], wave_max(z));
        const float alpha = fast_exp2(m_run[g] - m_new);
        ph = (half_t)fast_exp2(z - m_new);
        l_lane[g] = l_lane[g] * alpha + (float)ph;
#pragma unroll
        for (int st = 0; st < kSets; ++st) acc_o[st][g] *= alpha;
        m_run[g] = m_new;
      }
      p_lds[g * 64 + lane] = ph;
    }

    // positions past the end (tail of the last block, and re-read blocks past
    // it) in the sequence's last unit: V element := 0
    if (t0 + kGroupTokens > cur.len) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int e = 0; e < kChunk; ++e) {
            const bool dead = t0 + i * kBlockSize + hh * kChunk + e >= cur.len;
#pragma unroll
            for (int st = 0; st < kSets; ++st)
              vreg[i][st][hh][e] = dead ? (half_t)0.0f : vreg[i][st][hh][e];
          }
    }

    __syncthreads();
    // lane 4c+g: weights of head g for tokens 4c..4c+3
    const half4_t pfrag =
        *reinterpret_cast<const half4_t*>(p_lds + (lane & 3) * 64 + (lane >> 2) * 4);

    // out[g][d] += sum_t P[g][t] V[t][d]; chunk c = tokens 4c..4c+3 of the unit
    static_for<0, 16>([&](auto ic) {
      constexpr int c = decltype(ic)::value;
      constexpr int i = c / 4, hh = (c % 4) / 2, sub = c % 2;
#pragma unroll
      for (int st = 0; st < kSets; ++st) {
        const half4_t vf = sub ? hi4(vreg[i][st][hh]) : lo4(vreg[i][st][hh]);
        acc_o[st] = __builtin_amdgcn_mfma_f32_4x4x4f16(pfrag, vf, acc_o[st], 4, c, 0);
      }
    });
    load_v(nxt, pb_nxt);
    __syncthreads();

    // ---- end of a run piece: finish it ---------------------------------
    const bool run_ends = last_unit || cur.g + 1 == cur.n_s;
    if (run_ends) {
      float l_tot[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) l_tot[g] = (g < G) ? wave_sum_dpp(l_lane[g]) : 1.0f;
      if (piece_first_g == 0 && cur.g + 1 == cur.n_s) {
        // the whole run is this worker's
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if (g < G) {
            const float inv = 1.0f / l_tot[g];
            half_t* o = a.out + ((int64_t)cur.s * Hq + cur.h * G + g) * D;
#pragma unroll
            for (int st = 0; st < kSets; ++st) o[st * 64 + lane] = (half_t)(acc_o[st][g] * inv);
          }
        }
      } else {
        // partial: slot 2w for this worker's first run, 2w+1 for its last,
        // written through to memory (system-scope relaxed stores) so a worker
        // on another XCD can read it; merged after the stream
        const int64_t slot = 2 * (int64_t)w + (first_piece ? 0 : 1);
        float* po = a.ws.o + slot * 4 * D;
        float* pml = a.ws.ml + slot * 8;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if (g < G) {
#pragma unroll
            for (int st = 0; st < kSets; ++st)
              __hip_atomic_store(po + g * D + st * 64 + lane, acc_o[st][g], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_SYSTEM);
            if (lane == 0) {
              __hip_atomic_store(pml + 2 * g, m_run[g], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_SYSTEM);
              __hip_atomic_store(pml + 2 * g + 1, l_tot[g], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_SYSTEM);
            }
          }
        }
        const int ci = cut_n < 2 ? cut_n : 1;
        cut_s[ci] = cur.s;
        cut_h[ci] = cur.h;
        cut_ns[ci] = cur.n_s;
        cut_os[ci] = cur.o_s;
        cut_n = ci + 1;
      }
      reset_run();
      first_piece = false;
      piece_first_g = 0;
      store_q();  // q rows of the next run (the current run's q reads are done)
    }

    // ---- shift the lookahead -------------------------------------------
    cur = nxt;
    nxt = nxt2;
    tbl_nxt = tbl_nxt2;
    if (ui + 3 < n_units) nxt2 = advance(nxt2);
    __syncthreads();
  }

  // ---- counters and merges of the cut runs ---------------------------------
  if (cut_n == 0) return;
  __builtin_amdgcn_s_waitcnt(0);  // every partial store above has completed
  for (int ci = 0; ci < cut_n; ++ci) {
    const int s = cut_s[ci], kvh = cut_h[ci], n_s = cut_ns[ci];
    const int64_t ua = (int64_t)Hkv * cut_os[ci] + (int64_t)kvh * n_s;  // the run's first unit
    const int64_t wa = share_owner(ua, nwa, total);
    const int64_t wb = share_owner(ua + n_s - 1, nwa, total);
    int* counter = a.ws.counters + (int64_t)s * Hkv + kvh;
    int arrived = 0;
    if (lane == 0)
      arrived = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    arrived = __shfl(arrived, 0);
    if (arrived != (int)(wb - wa)) continue;
    // last to arrive: merge the run's np partials.  Part p (0-based) is worker
    // wa + p's slot: its last-run slot for p = 0 unless the run starts its
    // share, its first-run slot otherwise.  Reads bypass the caches.
    auto ld = [](const float* p) {
      return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    };
    const int np = (int)(wb - wa + 1);
    const bool wa_first = ua == share_begin(wa, nwa, total);
    auto slot_of = [&](int p) { return 2 * (wa + p) + ((p == 0 && !wa_first) ? 1 : 0); };
    // Parts in batches of 16: lane 4p+g loads part p's (max, sum) of head g
    // and, with them, every lane loads the batch's output vectors (all these
    // loads are independent: one round trip per batch).  Batches combine
    // with the running-max rescale.
    const int gq = lane & 3;
    float mx = -INFINITY, lsum = 0.0f;  // per head gq
    float acc[4][kSets];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int st = 0; st < kSets; ++st) acc[g][st] = 0.0f;
    for (int p0 = 0; p0 < np; p0 += 16) {
      const int p = p0 + (lane >> 2);
      const bool valid = p < np && gq < G;
      const int64_t sp = slot_of(valid ? p : p0);
      const float m_p = valid ? ld(a.ws.ml + sp * 8 + 2 * gq) : -INFINITY;
      const float l_p = valid ? ld(a.ws.ml + sp * 8 + 2 * gq + 1) : 0.0f;
      const int nq = min(16, np - p0);
      float ov[16][4][kSets];
#pragma unroll
      for (int qi = 0; qi < 16; ++qi) {
        const int64_t sq = slot_of(p0 + min(qi, nq - 1));
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int st = 0; st < kSets; ++st)
            ov[qi][g][st] = (qi < nq && g < G)
                                ? ld(a.ws.o + sq * 4 * D + g * D + st * 64 + lane) : 0.0f;
      }
      // batch max per head, rescale what was accumulated, add the batch
      float bm = m_p;
#pragma unroll
      for (int o = 4; o < 64; o <<= 1) bm = fmaxf(bm, __shfl_xor(bm, o));
      const float m_new = fmaxf(mx, bm);
      const float alpha = fast_exp2(mx - m_new);   // 0 for the first batch
      const float wt = valid ? fast_exp2(m_p - m_new) : 0.0f;
      lsum = lsum * alpha + wt * l_p;
      mx = m_new;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (g < G) {
          const float al = __shfl(alpha, g);
#pragma unroll
          for (int st = 0; st < kSets; ++st) acc[g][st] *= al;
#pragma unroll
          for (int qi = 0; qi < 16; ++qi) {
            const float wq = __shfl(wt, 4 * qi + g);
#pragma unroll
            for (int st = 0; st < kSets; ++st) acc[g][st] += wq * ov[qi][g][st];
          }
        }
      }
    }
#pragma unroll
    for (int o = 4; o < 64; o <<= 1) lsum += __shfl_xor(lsum, o);  // per head
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (g < G) {
        const float inv = 1.0f / __shfl(lsum, g);
        half_t* o = a.out + ((int64_t)s * Hq + kvh * G + g) * D;
#pragma unroll
        for (int st = 0; st < kSets; ++st) o[st * 64 + lane] = (half_t)(acc[g][st] * inv);
      }
    }
    if (lane == 0)  // ready for the next call
      __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

size_t decode_workspace_bytes(int64_t S, int64_t Hkv, int64_t D, int64_t workers) {
  const size_t cnt = ((size_t)(S * Hkv) * sizeof(int) + 255) & ~(size_t)255;
  const size_t ml = ((size_t)(2 * workers * 8) * sizeof(float) + 255) & ~(size_t)255;
  return cnt + ml + (size_t)(2 * workers * 4 * D) * sizeof(float);
}

DecodeWorkspace decode_workspace_carve(void* base, int64_t S, int64_t Hkv, int64_t workers) {
  const size_t cnt = ((size_t)(S * Hkv) * sizeof(int) + 255) & ~(size_t)255;
  const size_t ml = ((size_t)(2 * workers * 8) * sizeof(float) + 255) & ~(size_t)255;
  char* p = reinterpret_cast<char*>(base);
  DecodeWorkspace w;
  w.counters = reinterpret_cast<int*>(p);
  w.ml = reinterpret_cast<float*>(p + cnt);
  w.o = reinterpret_cast<float*>(p + cnt + ml);
  return w;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.num_workers);
  if (a.head_dim == 128)
    hipLaunchKernelGGL(decode_kernel<128>, grid, dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_kernel<64>, grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
