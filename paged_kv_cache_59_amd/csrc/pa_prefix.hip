// Shared prefixes of a decode batch, for gfx950: the groups, and each
// group's query rows attended to its common prefix once.
//
// Sequences that hold the same physical blocks hold the same keys and values
// there ("Continuous batching, paged attention, prefix caching", "Prefix
// caching": one stored copy of a prompt prefix serves every request that
// starts with it; "KV Cache in Serving Engines ...", section 2 "Sharing
// Blocks").  A decode over such a batch reads each shared prefix block once:
// this pass attends all the query rows of a group of sequences to their
// common prefix, in a few chunks of keys, and writes per chunk a normalised
// row and its log-sum-exp; the decode kernel covers each sequence's remaining
// positions and folds those pieces in (the log-sum-exp merge of flash
// decoding's split keys).
//
// Groups (pa_internal.h): runs of consecutive sequences inside windows of 8,
// each sharing at least one 64-token unit of blocks with the one before.
// Each workgroup finds its window's groups itself from the block tables
// (seven comparisons of table rows), so no pass over the whole batch comes
// first.
//
// Work: one workgroup per (chunk, window, KV head); its 8 waves take equal
// slices of the chunk's keys, 32 keys per step, each wave reading its own
// slice straight into registers, for the group's
// rows (members x query heads of the KV group, at most 32):
//   S^T = K . Q^T   (v_mfma_f32_16x16x32_f16: 16 keys x 32 dims of K against
//                    32 dims x 16 rows of Q^T)
//   O^T += V^T . P^T (16 dims x 32 keys of V^T against 32 keys x 16 rows)
// With lane l = 16 j + c, an operand of lane l covers k-slots 8j..8j+7 of row
// (column) c and its result rows 4j..4j+3 of column c.  The K operand's row
// m of sub-tile kt is key 8 (m / 4) + 4 kt + m % 4 of the step, so the eight
// logits lane l holds for its row c are keys 8j..8j+7 in order: its P^T
// operand as they stand, and one 8-key group of V, one 16-byte load per dim.
// The waves then combine their (max, sum, rows) through LDS.
#include <climits>

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pa {
namespace {

typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kRows = 32;  // a group's rows: 8 members x at most 4 query heads

__device__ __forceinline__ float4v mfma16(half8_t a, half8_t b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// K/V tiles: read once, non-temporal
__device__ __forceinline__ half8_t load_tile(const half_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const half8_t*>(p));
}
// max and sum over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four 8-key slices of a row)
__device__ __forceinline__ float max4(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float sum4(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}
template <int D, int BS>
__global__ __launch_bounds__(64 * kPrefixWaves, 1) void prefix_kernel(const PrefixArgs a) {
  constexpr int W = kPrefixWaves;
  constexpr int KS = D / 32;  // 32-dim steps of the contraction over D
  constexpr int DT = D / 16;  // 16-dim tiles of the output
  constexpr int NBS = 32 / BS;  // blocks per 32-key step
  static_assert(NBS * BS == 32 && KS * 32 == D, "block size 8, 16 or 32; head_dim 64 or 128");
  constexpr int64_t kTile = (int64_t)BS * D;
  constexpr int kORow = D + 4;  // floats per row of the waves' partial outputs in LDS
  extern __shared__ __attribute__((aligned(16))) float comb_lds[];  // [W][kRows][kORow], [W][kRows][2]
  constexpr int kQRow = D + 8;  // halves per query row in LDS
  __shared__ __attribute__((aligned(16))) half_t q_lds[kRows * kQRow];
  __shared__ int len_lds[kPrefixWindow];
  __shared__ int sh_lds[kPrefixWindow];  // tokens sequence i holds in the blocks of i - 1

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15;  // operand / result column: this lane's row of a sub-tile
  const int j = lane >> 4;    // k-slot group
  const int S = a.num_seqs, Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  // (a KV head of more than 4 query heads is taken as kv_split heads, one
  // per sub-group of up to 4 query heads; Hkv counts them)
  const int split = a.kv_split, Hkr = Hkv / split;
  // workgroup -> (chunk, window, KV head), the chunk slowest: chunks that
  // turn out empty (past a group's prefix) are dispatched last
  const int bid = (int)blockIdx.x;
  const int per_chunk = (int)(gridDim.x / a.max_chunks);
  const int chunk = bid / per_chunk;
  const int h = bid % Hkv;
  const int hr = h / split;                                          // KV head of the pools
  const int G = split == 1 ? Hq / Hkv : min(4, Hq / Hkr - h % split * 4);  // query rows per member
  const int qh0 = hr * (Hq / Hkr) + h % split * 4;                   // their first query head
  const int s0 = (bid % per_chunk) / Hkv * kPrefixWindow;
  const int n = min(kPrefixWindow, S - s0);

  // ---- the window's groups ---------------------------------------------------
  if ((int)threadIdx.x < n)
    len_lds[threadIdx.x] = min(max(a.context_lens[s0 + threadIdx.x], 0), a.max_context_len);
  __syncthreads();
  // pair (p - 1, p): the leading table entries they agree on, up to the
  // blocks both hold (wave w takes p = w + 1)
  for (int p = 1 + wave; p < n; p += W) {
    const int la = len_lds[p - 1], lb = len_lds[p];
    const int nblk = (min(la, lb) + BS - 1) / BS;
    const int32_t* ra = a.block_tables + (int64_t)(s0 + p - 1) * a.max_blocks_per_seq;
    const int32_t* rb = ra + a.max_blocks_per_seq;
    int common = nblk;
    for (int j0 = 0; j0 < nblk; j0 += 256) {
      int x[4], y[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = j0 + 64 * u + lane;
        x[u] = idx < nblk ? ra[idx] : 0;
        y[u] = idx < nblk ? rb[idx] : 0;
      }
      int first = -1;  // (uniform)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint64_t d = __ballot(x[u] != y[u]);
        if (first < 0 && d) first = j0 + 64 * u + __builtin_ctzll(d);
      }
      if (first >= 0) {
        common = first;
        break;
      }
    }
    // the last position of each is not in the pools yet (a fused append brings it)
    if (lane == 0) sh_lds[p] = max(0, min(common * BS, min(la, lb) - 1));
  }
  __syncthreads();

  // ---- one group's chunk ----------------------------------------------------
  auto attend = [&](int gf, int M, int P) {
    const int rows = M * G;
    const int cl = prefix_chunk_len(P);
    const int k0 = chunk * cl, k1 = min(k0 + cl, P);
    const int wk0 = k0 + wave * (cl / W);  // this wave's keys: [wk0, wk1), whole 32-key steps
    const int wk1 = min(wk0 + cl / W, k1);
    const int nsteps = wk1 > wk0 ? (wk1 - wk0) / 32 : 0;

    // the group's query rows into LDS (rows past the group: zero), read as
    // the Q^T operands at every step (held in registers they would crowd
    // out the second step in flight)
    __syncthreads();  // (the previous group's steps have read q_lds)
    for (int e = threadIdx.x; e < kRows * (D / 8); e += 64 * W) {
      const int r = e / (D / 8), c = e % (D / 8);
      half8_t v = {};
      if (r < rows)
        v = *reinterpret_cast<const half8_t*>(
            a.q + ((int64_t)(s0 + gf + r / G) * Hq + qh0 + r % G) * D + 8 * c);
      *reinterpret_cast<half8_t*>(q_lds + r * kQRow + 8 * c) = v;
    }
    __syncthreads();

    // The group's blocks, from its first member's table (the members hold
    // the same ones below P).  Scalar loads, through the constant address
    // space: their wait (lgkmcnt) does not drain the K/V loads in flight.
    const __attribute__((address_space(4))) int32_t* crow =
        (const __attribute__((address_space(4))) int32_t*)(a.block_tables +
                                                            (int64_t)(s0 + gf) * a.max_blocks_per_seq);
    auto blk = [&](int lb) {
      const int e = crow[__builtin_amdgcn_readfirstlane(lb)];
      return (e >= 0 && e < a.num_blocks) ? e : 0;  // a broken entry reads block 0
    };
    int n0 = 0, n1 = 0, n2 = 0, n3 = 0;  // the next step's blocks (uniform)
    auto fetch = [&](int t) {
      const int lb = (wk0 + 32 * min(t, nsteps - 1)) / BS;
      n0 = blk(lb);
      if constexpr (NBS > 1) n1 = blk(lb + 1);
      if constexpr (NBS > 2) {
        n2 = blk(lb + 2);
        n3 = blk(lb + 3);
      }
    };
    // per-lane parts of the addresses: the K operand's 8-key group c16 / 4
    // and the V operand's 8-key group j, each in block (8 group) / BS of the
    // step, at element offsets inside that block's head tile
    // (K: chunk 4 ks + j of the key's 8 dims, slot (8 gk) % BS + 4 kt + c16 % 4;
    // V: 8-key group (8 j) % BS / 8, dim 16 dt + c16; the ks, kt and dt
    // parts are constant offsets)
    const int gk = c16 >> 2;
    const int bk = (8 * gk) / BS, bv = (8 * j) / BS;
    const int klane = (j * BS + (8 * gk) % BS + (c16 & 3)) * 8;
    const int vlane = (((8 * j) % BS) / 8 * D + c16) * 8;
    const int64_t hoff = (int64_t)hr * kTile, bstride = (int64_t)Hkr * kTile;
    auto pick = [&](int sel, int b0, int b1, int b2, int b3) {
      if constexpr (NBS == 1) return b0;
      else if constexpr (NBS == 2) return sel ? b1 : b0;
      else return (sel & 2) ? ((sel & 1) ? b3 : b2) : ((sel & 1) ? b1 : b0);
    };

    // One step's K and V in registers: the next step's K is issued as soon
    // as this step's logits have read the K registers, its V once P.V has
    // read the V registers (the other waves of the compute unit keep the
    // memory busy in between).
    half8_t kf[2][KS], vf[DT];
    auto issue_k = [&](int b0, int b1, int b2, int b3) {
      const half_t* kb = a.k_cache + (int64_t)pick(bk, b0, b1, b2, b3) * bstride + hoff + klane;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[kt][ks] = load_tile(kb + (4 * ks * BS + 4 * kt) * 8);
    };
    auto issue_v = [&](int b0, int b1, int b2, int b3) {
      const half_t* vb = a.v_cache + (int64_t)pick(bv, b0, b1, b2, b3) * bstride + hoff + vlane;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) vf[dt] = load_tile(vb + 16 * dt * 8);
    };

    float4v o[2][DT];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[rt][dt] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run[2] = {-INFINITY, -INFINITY}, l_part[2] = {0.0f, 0.0f};
    if (nsteps > 0) {
      fetch(0);
      issue_k(n0, n1, n2, n3);
      issue_v(n0, n1, n2, n3);
      fetch(1);
    }
    for (int t = 0; t < nsteps; ++t) {
      const int b0 = n0, b1 = n1, b2 = n2, b3 = n3;  // step t + 1's blocks
      const bool more = t + 1 < nsteps;
      // logits of both 16-row sub-tiles: S^T = K . Q^T
      // (the Q offset passes through an empty asm so that the compiler does
      // not hoist the Q reads out of the loop into registers)
      int qoff = c16 * kQRow + 8 * j;
      asm volatile("" : "+v"(qoff));
      float4v sacc[2][2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        sacc[rt][0] = sacc[rt][1] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          // Q^T operand: row 16 rt + c16, dims 32 ks + 8 j ..
          const half8_t qv = *reinterpret_cast<const half8_t*>(q_lds + qoff + 16 * rt * kQRow + 32 * ks);
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) sacc[rt][kt] = mfma16(kf[kt][ks], qv, sacc[rt][kt]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (more) {
        fetch(t + 2);
        issue_k(b0, b1, b2, b3);
      }
      __builtin_amdgcn_sched_barrier(0);
      // the online softmax; keys 8j + e of the step, e = 4 kt + i, for this lane's rows
      half8_t pf[2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        float z[8], mt = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          z[e] = sacc[rt][e >> 2][e & 3] * a.scale_log2;
          mt = fmaxf(mt, z[e]);
        }
        const float m_new = fmaxf(m_run[rt], max4(mt));
        const float alpha = __builtin_amdgcn_exp2f(m_run[rt] - m_new);  // 0 at the first step
        m_run[rt] = m_new;
        float ls = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pf[rt][e] = (half_t)__builtin_amdgcn_exp2f(z[e] - m_new);
          ls += (float)pf[rt][e];
        }
        l_part[rt] = l_part[rt] * alpha + ls;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[rt][dt] *= alpha;
      }
      // O^T += V^T . P^T
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[rt][dt] = mfma16(vf[dt], pf[rt], o[rt][dt]);
      __builtin_amdgcn_sched_barrier(0);
      if (more) issue_v(b0, b1, b2, b3);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- the waves' pieces combined through LDS -------------------------------
    float* o_lds = comb_lds;
    float* ml_lds = comb_lds + W * kRows * kORow;
    __syncthreads();  // (the previous group's combine has read the LDS)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int r = 16 * rt + c16;
      const float l = sum4(l_part[rt]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<float4v*>(o_lds + (wave * kRows + r) * kORow + 16 * dt + 4 * j) = o[rt][dt];
      if (j == 0) {
        ml_lds[(wave * kRows + r) * 2] = m_run[rt];
        ml_lds[(wave * kRows + r) * 2 + 1] = l;
      }
    }
    __syncthreads();
    // wave w: rows kRW w .. + kRW - 1; lane: row kRW w + lane / kLR, dims
    // kDL (lane % kLR) ..
    constexpr int kRW = kRows / W;   // rows per wave
    constexpr int kLR = 64 / kRW;    // lanes per row
    constexpr int kDL = D / kLR;     // dims per lane (a multiple of 4)
    const int r = kRW * wave + lane / kLR;
    const int d0 = (lane % kLR) * kDL;
    float mw[W], mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      mw[w] = ml_lds[(w * kRows + r) * 2];
      mx = fmaxf(mx, mw[w]);
    }
    float L = 0.0f, acc[kDL];
#pragma unroll
    for (int d = 0; d < kDL; ++d) acc[d] = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float wt = mx == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw[w] - mx);  // 0 for a wave without keys
      L += wt * ml_lds[(w * kRows + r) * 2 + 1];
#pragma unroll
      for (int d = 0; d < kDL; d += 4) {
        const float4v x = *reinterpret_cast<const float4v*>(o_lds + (w * kRows + r) * kORow + d0 + d);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[d + i] += wt * x[i];
      }
    }
    if (r < rows) {
      const int64_t ro = ((int64_t)chunk * S + (s0 + gf + r / G)) * Hq + qh0 + r % G;
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
      for (int d = 0; d < kDL; d += 4) {
        half4_t v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (half_t)(acc[d + i] * inv);
        *reinterpret_cast<half4_t*>(a.pre_o + ro * D + d0 + d) = v;
      }
      if (lane % kLR == 0) a.pre_lse[ro] = L > 0.0f ? mx + __builtin_log2f(L) : -INFINITY;
    }
  };

  // runs of the window (uniform: every thread reads the same LDS values)
  int gf = 0;
  for (int p = 1; p <= n; ++p) {
    if (p < n && sh_lds[p] >= kGroupTokens) continue;  // p joins the run
    const int M = p - gf;
    int P = 0;
    if (M >= 2) {
      int m = INT_MAX;
      for (int i = gf + 1; i < p; ++i) m = min(m, sh_lds[i]);
      P = m / kGroupTokens * kGroupTokens;
      if (chunk < prefix_chunks(P)) attend(gf, M, P);
    }
    if (h == 0 && chunk == 0 && (int)threadIdx.x >= gf && (int)threadIdx.x < p)
      a.pre_len[s0 + threadIdx.x] = P;
    gf = p;
  }
}

}  // namespace

hipError_t launch_prefix(const PrefixArgs& a, hipStream_t stream, hipEvent_t start) {
  const int64_t windows = (a.num_seqs + kPrefixWindow - 1) / kPrefixWindow;
  const dim3 grid((unsigned)(windows * a.num_kv_heads * a.max_chunks));
#define PA_PREFIX(D, BS)                                                                       \
  if (a.head_dim == D && a.block_size == BS) {                                                \
    const size_t lds = (size_t)kPrefixWaves * kRows * ((D + 4) + 2) * sizeof(float);          \
    if (!start)                                                                                \
      hipLaunchKernelGGL((prefix_kernel<D, BS>), grid, dim3(64 * kPrefixWaves), lds, stream, a); \
    else                                                                                       \
      hipExtLaunchKernelGGL((prefix_kernel<D, BS>), grid, dim3(64 * kPrefixWaves), lds, stream,    \
                            start, nullptr, 0, a);                                             \
  }
  PA_PREFIX(128, 16) PA_PREFIX(64, 16) PA_PREFIX(128, 8) PA_PREFIX(64, 8) PA_PREFIX(128, 32)
  PA_PREFIX(64, 32)
#undef PA_PREFIX
  return hipGetLastError();
}

}  // namespace pa
