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
  static_assert(kChunks * kChunk == D && kSets * 64 == D, "head_dim must be 64 or 128");

  const int lane = threadIdx.x;
  const int nw = gridDim.x;
  // consecutive logical workers on one XCD (workgroup i runs on XCD i % 8)
  const int w = (nw % 8 == 0) ? (int)(blockIdx.x % 8) * (nw / 8) + (int)(blockIdx.x / 8)
                              : (int)blockIdx.x;
  const int S = a.num_seqs;
  const int Hkv = a.num_kv_heads;
  const int Hq = a.num_q_heads;
  const int G = Hq / Hkv;

  auto units_of = [&](int s) {
    int c = a.context_lens[s];
    c = min(max(c, 0), a.max_context_len);
    return (c + kGroupTokens - 1) / kGroupTokens;
  };

  // ---- pass 1: total units; zero the rows of empty sequences ------------
  int64_t seq_units = 0;  // sum over sequences of ceil(len / 64)
  for (int c0 = 0; c0 < S; c0 += 64) {
    const int s = c0 + lane;
    const int n = s < S ? units_of(s) : 0;
    seq_units += wave_sum_int(n);
    uint64_t empty = __ballot(s < S && n == 0 && (s % nw) == w);
    while (empty) {
      const int se = c0 + __builtin_ctzll(empty);
      empty &= empty - 1;
      half_t* o = a.out + (int64_t)se * Hq * D;
      for (int e = lane; e < Hq * D; e += 64) o[e] = (half_t)0.0f;
    }
  }
  const int64_t total = seq_units * Hkv;
  if (total == 0) return;
  const int64_t nwa = min((int64_t)nw, total);  // active workers: each gets >= 1 unit
  if (w >= nwa) return;
  const int64_t u_begin = share_begin(w, nwa, total);
  const int64_t u_end = share_begin(w + 1, nwa, total);

  // ---- pass 2: the sequence holding u_begin ------------------------------
  // units of sequence s are [Hkv*O_s, Hkv*O_{s+1}), ordered (head, unit)
  const int64_t key = u_begin / Hkv;
  int s_cur = 0, n_s = 0;
  int64_t o_s = 0;  // O_s: units of the sequences before s_cur
  {
    int64_t base = 0;
    for (int c0 = 0; c0 < S; c0 += 64) {
      const int s = c0 + lane;
      const int n = s < S ? units_of(s) : 0;
      const int incl = wave_inclusive_scan(n, lane);
      const uint64_t hit = __ballot(s < S && base + incl > key);
      if (hit) {
        const int l = __builtin_ctzll(hit);
        s_cur = c0 + l;
        n_s = __shfl(n, l);
        o_s = base + __shfl(incl, l) - n_s;
        break;
      }
      base += __shfl(incl, 63);
    }
  }
  if (n_s == 0) return;  // unreachable for consistent lengths; never divide by 0
  int64_t rem_in_seq = u_begin - (int64_t)Hkv * o_s;
  int h = (int)(rem_in_seq / n_s);
  int g_first = (int)(rem_in_seq - (int64_t)h * n_s);
  int64_t remaining = u_end - u_begin;
  bool first_run = true;

  __shared__ half_t p_lds[4 * 64];
  __shared__ __attribute__((aligned(16))) half_t q_lds[4 * D];
  const int my_blk = lane >> 4;  // which of a unit's 4 blocks holds this lane's token
  const int g_lane = lane & 3;   // q head of the group this lane's MFMA row carries
  const int64_t block_stride = (int64_t)Hkv * kTile;

  while (remaining > 0) {
    const int g_last = (int)min((int64_t)n_s - 1, (int64_t)g_first + remaining - 1);
    const int s = s_cur;
    const int kvh = h;
    int ctx = a.context_lens[s];
    ctx = min(max(ctx, 0), a.max_context_len);
    const int start = g_first * kGroupTokens;
    const int end = min((g_last + 1) * kGroupTokens, ctx);

    // q rows of this KV head's group into LDS (rows >= G are 0): row g, 16-byte
    // chunk c is held by lane g * kChunks + c
    if (lane < 4 * kChunks) {
      const int g = lane / kChunks, c = lane % kChunks;
      half8_t v = half8_t{};
      if (g < G) v = *reinterpret_cast<const half8_t*>(a.q + ((int64_t)s * Hq + kvh * G + g) * D + c * kChunk);
      *reinterpret_cast<half8_t*>(q_lds + g * D + c * kChunk) = v;
    }
    __syncthreads();

    float m_run[4], l_lane[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      m_run[g] = -INFINITY;
      l_lane[g] = 0.0f;
    }
    float4_t acc_o[kSets];
#pragma unroll
    for (int st = 0; st < kSets; ++st) acc_o[st] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
    const int64_t kv_head_off = (int64_t)kvh * kTile;
    const int jb0 = start / kBlockSize;
    const int nblk = (end - start + kBlockSize - 1) / kBlockSize;  // blocks with live tokens

    // Physical id of the run's block j (a uniform scalar load); j past the
    // live blocks re-reads the last live one; an id outside the pool (a
    // broken table) reads pool block 0 instead.
    auto entry = [&](int j) {
      const int e = table[jb0 + min(j, nblk - 1)];
      return (e >= 0 && e < a.num_blocks) ? e : 0;
    };

    half8_t kreg[kChunks];
    half8_t vreg[4][kSets][2];
    auto load_k = [&](const int (&pb)[4]) {
      const int phys = my_blk == 0 ? pb[0] : my_blk == 1 ? pb[1] : my_blk == 2 ? pb[2] : pb[3];
      const half_t* kp = a.k_cache + (int64_t)phys * block_stride + kv_head_off + (lane & 15) * kChunk;
#pragma unroll
      for (int c = 0; c < kChunks; ++c) kreg[c] = load_nt(kp + c * (kBlockSize * kChunk));
    };
    auto load_v = [&](const int (&pb)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const half_t* vp = a.v_cache + (int64_t)pb[i] * block_stride + kv_head_off;
#pragma unroll
        for (int st = 0; st < kSets; ++st)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
            vreg[i][st][hh] = load_nt(vp + ((int64_t)hh * D + st * 64 + lane) * kChunk);
      }
    };

    int pb_nxt[4];
    {
      int pb0[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb0[i] = entry(i);
        pb_nxt[i] = entry(4 + i);
      }
      // keep the prologue in loop order (all K loads, then all V loads): the
      // wait counts at the loop head are merged over both ways in
      __builtin_amdgcn_sched_barrier(0);
      load_k(pb0);
      __builtin_amdgcn_sched_barrier(0);
      load_v(pb0);
      __builtin_amdgcn_sched_barrier(0);
    }

    // One 64-token unit starting at position t0; with kNext the next unit's
    // loads are issued inside it.
    int ui = 0;
    auto unit = [&](int t0, auto next_tag) {
      constexpr bool kNext = decltype(next_tag)::value;
      // logits: S[g][token lane] = q_g . K_token  (rows = heads, columns = tokens)
      // (lane l's MFMA row is q head l % 4, read from LDS chunk by chunk)
      float4_t sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        const half8_t qv = *reinterpret_cast<const half8_t*>(q_lds + g_lane * D + c * kChunk);
        sacc = __builtin_amdgcn_mfma_f32_4x4x4f16(lo4(qv), lo4(kreg[c]), sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_4x4x4f16(hi4(qv), hi4(kreg[c]), sacc, 0, 0, 0);
      }
      if constexpr (kNext) load_k(pb_nxt);

      // online softmax over these 64 positions
      const bool live = (t0 + lane) < end;
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

      // positions past the end (tail of the last live block, and re-read
      // blocks past it): V element := 0
      if constexpr (!kNext) {
        if (t0 + kGroupTokens > end) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
              for (int e = 0; e < kChunk; ++e) {
                const bool dead = t0 + i * kBlockSize + hh * kChunk + e >= end;
#pragma unroll
                for (int st = 0; st < kSets; ++st)
                  vreg[i][st][hh][e] = dead ? (half_t)0.0f : vreg[i][st][hh][e];
              }
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
      if constexpr (kNext) {
        load_v(pb_nxt);
#pragma unroll
        for (int i = 0; i < 4; ++i) pb_nxt[i] = entry(4 * (ui + 2) + i);
      }
      __syncthreads();
    };

    int t0 = start;
    for (; t0 + kGroupTokens < end; t0 += kGroupTokens, ++ui) unit(t0, std::true_type{});
    unit(t0, std::false_type{});

    // ---- finish the run ---------------------------------------------------
    float l_tot[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) l_tot[g] = (g < G) ? wave_sum(l_lane[g]) : 1.0f;

    if (g_first == 0 && g_last == n_s - 1) {
      // the whole run is this worker's
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (g < G) {
          const float inv = 1.0f / l_tot[g];
          half_t* o = a.out + ((int64_t)s * Hq + kvh * G + g) * D;
#pragma unroll
          for (int st = 0; st < kSets; ++st) o[st * 64 + lane] = (half_t)(acc_o[st][g] * inv);
        }
      }
    } else {
      // partial: slot 2w for this worker's first run, 2w+1 for its last.
      // Hand-off without whole-cache maintenance: the partial goes out with
      // write-through stores (system-scope relaxed atomics), is complete
      // before the counter moves (wait for all stores), and the merging
      // worker reads the slots with cache-bypassing loads (same kind of
      // atomics), so workers on different XCDs (separate L2s) agree.
      const int64_t slot = 2 * (int64_t)w + (first_run ? 0 : 1);
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
            __hip_atomic_store(pml + 2 * g, m_run[g], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            __hip_atomic_store(pml + 2 * g + 1, l_tot[g], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_SYSTEM);
          }
        }
      }
      const int64_t ua = (int64_t)Hkv * o_s + (int64_t)kvh * n_s;  // the run's first unit
      const int64_t wa = share_owner(ua, nwa, total);
      const int64_t wb = share_owner(ua + n_s - 1, nwa, total);
      int* counter = a.ws.counters + (int64_t)s * Hkv + kvh;
      __builtin_amdgcn_s_waitcnt(0);  // every store above has completed
      int arrived = 0;
      if (lane == 0)
        arrived = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      arrived = __shfl(arrived, 0);
      if (arrived == (int)(wb - wa)) {
        // last to arrive: merge the run's partials in worker order
        auto ld = [](const float* p) {
          return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        };
        const bool wa_first = ua == share_begin(wa, nwa, total);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if (g < G) {
            float mx = -INFINITY;
            for (int64_t p = wa; p <= wb; ++p) {
              const int64_t sp = p == wa ? 2 * p + (wa_first ? 0 : 1) : 2 * p;
              mx = fmaxf(mx, ld(a.ws.ml + sp * 8 + 2 * g));
            }
            float lsum = 0.0f;
            float acc[kSets];
#pragma unroll
            for (int st = 0; st < kSets; ++st) acc[st] = 0.0f;
            for (int64_t p = wa; p <= wb; ++p) {
              const int64_t sp = p == wa ? 2 * p + (wa_first ? 0 : 1) : 2 * p;
              const float wt = fast_exp2(ld(a.ws.ml + sp * 8 + 2 * g) - mx);
              lsum += wt * ld(a.ws.ml + sp * 8 + 2 * g + 1);
#pragma unroll
              for (int st = 0; st < kSets; ++st)
                acc[st] += wt * ld(a.ws.o + sp * 4 * D + g * D + st * 64 + lane);
            }
            const float inv = 1.0f / lsum;
            half_t* o = a.out + ((int64_t)s * Hq + kvh * G + g) * D;
#pragma unroll
            for (int st = 0; st < kSets; ++st) o[st * 64 + lane] = (half_t)(acc[st] * inv);
          }
        }
        if (lane == 0)  // ready for the next call
          __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }

    // ---- next run ----------------------------------------------------------
    remaining -= g_last - g_first + 1;
    first_run = false;
    g_first = 0;
    if (remaining > 0 && ++h == Hkv) {
      h = 0;
      do {
        o_s += n_s;
        ++s_cur;
        n_s = s_cur < S ? units_of(s_cur) : 0;
      } while (n_s == 0 && s_cur < S);
      if (n_s == 0) break;  // unreachable for consistent lengths
    }
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
