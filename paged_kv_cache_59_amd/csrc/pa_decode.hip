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
// Design (none is given on the pages; decode reads every K/V byte once, so
// HBM bandwidth bounds it):
//  * one wave (64 lanes) per (sequence, KV head, context partition); a wave
//    walks its partition 64 tokens = 4 blocks at a time;
//  * the grouped query heads of one KV head (G <= 4) are the 4 rows of the
//    4x4x4 16-block MFMA, so every K and V element loaded is used by all G
//    heads; q stays in registers for the whole partition;
//  * q . K: lane l owns token l of the 64; it loads its 16-byte chunks of the
//    K row (K pool [NB][Hkv][D/8][16][8]: for a fixed chunk the 64 lanes read
//    four contiguous 256-byte runs) and feeds them as the B operand, so the
//    dot products reduce inside the MFMA, with no cross-lane sums;
//  * the online softmax keeps a running max per head (wave max per 64
//    tokens) and per-lane partial sums (one wave sum at the end);
//  * the fp16 probabilities are transposed through 512 bytes of LDS so lane
//    4c+g holds head g's weights of tokens 4c..4c+3; the MFMA broadcast
//    (CBSZ=4, ABID=c) hands that quad to all 16 blocks;
//  * P . V: lane l owns output dim l (and l+64); V pool [NB][Hkv][2][D][8]
//    puts 8 consecutive tokens of one dim in 16 bytes, so for a fixed
//    (block, half) the 64 lanes read 1 KiB contiguous;
//  * positions at or past the length are removed by selection (logit set to
//    -inf, V element set to 0), never by multiplication, so NaN or huge
//    values in the unused tail of the last block cannot leak;
//  * long contexts: partitions write (max, sum, unnormalised output) to the
//    workspace and a second kernel merges them with the log-sum-exp rescale.
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

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ half4_t lo4(half8_t v) { return __builtin_shufflevector(v, v, 0, 1, 2, 3); }
__device__ __forceinline__ half4_t hi4(half8_t v) { return __builtin_shufflevector(v, v, 4, 5, 6, 7); }

}  // namespace

template <int D>
__global__ __launch_bounds__(64) void decode_partition_kernel(const DecodeArgs a) {
  constexpr int kChunks = D / kChunk;  // 16-byte chunks in one K row
  constexpr int kSets = D / 64;        // 64-dim ranges a lane covers in P.V
  constexpr int64_t kTile = (int64_t)kBlockSize * D;
  static_assert(kChunks * kChunk == D && kSets * 64 == D, "head_dim must be 64 or 128");

  const int lane = threadIdx.x;
  const int part = blockIdx.x;
  const int kvh = blockIdx.y;
  const int s = blockIdx.z;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int P = a.partition_size;

  int ctx = a.context_lens[s];
  ctx = min(max(ctx, 0), a.max_context_len);
  const int start = part * P;
  if (ctx == 0) {
    if (part == 0) {
      for (int g = 0; g < G; ++g) {
        half_t* o = a.out + ((int64_t)s * a.num_q_heads + kvh * G + g) * D;
#pragma unroll
        for (int st = 0; st < kSets; ++st) o[st * 64 + lane] = (half_t)0.0f;
      }
    }
    return;
  }
  if (start >= ctx) return;
  const int end = min(start + P, ctx);
  const int nparts_seq = (ctx + P - 1) / P;

  // q rows: lane l holds head g = l % 4 of this KV head's group (rows >= G are 0)
  const int g_lane = lane & 3;
  half8_t qreg[kChunks];
  if (g_lane < G) {
    const half_t* qp = a.q + ((int64_t)s * a.num_q_heads + kvh * G + g_lane) * D;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) qreg[c] = *reinterpret_cast<const half8_t*>(qp + c * kChunk);
  } else {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) qreg[c] = half8_t{};
  }

  float m_run[4], l_lane[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    m_run[g] = -INFINITY;
    l_lane[g] = 0.0f;
  }
  float4_t acc_o[kSets];
#pragma unroll
  for (int st = 0; st < kSets; ++st) acc_o[st] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  __shared__ half_t p_lds[4 * 64];

  const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const int64_t kv_head_off = (int64_t)kvh * kTile;
  const int64_t block_stride = (int64_t)a.num_kv_heads * kTile;

  for (int t0 = start; t0 < end; t0 += kGroupTokens) {
    const int jb = t0 / kBlockSize;
    const int nvb = min(4, (end - t0 + kBlockSize - 1) / kBlockSize);  // blocks with live tokens
    const int my_blk = lane >> 4;
    int phys = -1;
    if (my_blk < nvb) phys = table[jb + my_blk];
    if (phys >= a.num_blocks) phys = -1;

    // K: token t0 + lane, i.e. slot lane % 16 of block my_blk
    half8_t kreg[kChunks];
    if (phys >= 0) {
      const half_t* kp = a.k_cache + (int64_t)phys * block_stride + kv_head_off + (lane & 15) * kChunk;
#pragma unroll
      for (int c = 0; c < kChunks; ++c)
        kreg[c] = *reinterpret_cast<const half8_t*>(kp + c * (kBlockSize * kChunk));
    } else {
#pragma unroll
      for (int c = 0; c < kChunks; ++c) kreg[c] = half8_t{};
    }

    // V: every lane reads its dims of all live blocks, 8 tokens per 16 bytes
    half8_t vreg[4][kSets][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pb = __builtin_amdgcn_readlane(phys, i * 16);
      if (pb >= 0) {
        const half_t* vp = a.v_cache + (int64_t)pb * block_stride + kv_head_off;
#pragma unroll
        for (int st = 0; st < kSets; ++st)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
            vreg[i][st][hh] =
                *reinterpret_cast<const half8_t*>(vp + ((int64_t)hh * D + st * 64 + lane) * kChunk);
      } else {
#pragma unroll
        for (int st = 0; st < kSets; ++st)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) vreg[i][st][hh] = half8_t{};
      }
    }

    // logits: S[g][token lane] = q_g . K_token  (rows = heads, columns = tokens)
    float4_t sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      sacc = __builtin_amdgcn_mfma_f32_4x4x4f16(lo4(qreg[c]), lo4(kreg[c]), sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_4x4x4f16(hi4(qreg[c]), hi4(kreg[c]), sacc, 0, 0, 0);
    }

    // online softmax over this group of 64 positions
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

    // positions past the end inside the last live block: V element := 0
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

    __syncthreads();
    // lane 4c+g: weights of head g for tokens 4c..4c+3
    const half4_t pfrag = *reinterpret_cast<const half4_t*>(p_lds + (lane & 3) * 64 + (lane >> 2) * 4);

    // out[g][d] += sum_t P[g][t] V[t][d]; chunk c = tokens 4c..4c+3 of the group
    static_for<0, 16>([&](auto ic) {
      constexpr int c = decltype(ic)::value;
      constexpr int i = c / 4, hh = (c % 4) / 2, sub = c % 2;
#pragma unroll
      for (int st = 0; st < kSets; ++st) {
        const half4_t vf = sub ? hi4(vreg[i][st][hh]) : lo4(vreg[i][st][hh]);
        acc_o[st] = __builtin_amdgcn_mfma_f32_4x4x4f16(pfrag, vf, acc_o[st], 4, c, 0);
      }
    });
    __syncthreads();
  }

  float l_tot[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) l_tot[g] = (g < G) ? wave_sum(l_lane[g]) : 1.0f;

  if (nparts_seq == 1) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (g < G) {
        const float inv = 1.0f / l_tot[g];
        half_t* o = a.out + ((int64_t)s * a.num_q_heads + kvh * G + g) * D;
#pragma unroll
        for (int st = 0; st < kSets; ++st) o[st * 64 + lane] = (half_t)(acc_o[st][g] * inv);
      }
    }
  } else {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (g < G) {
        const int64_t idx = ((int64_t)s * a.num_q_heads + kvh * G + g) * a.num_partitions + part;
#pragma unroll
        for (int st = 0; st < kSets; ++st) a.ws.o[idx * D + st * 64 + lane] = acc_o[st][g];
        if (lane == 0) {
          a.ws.ml[idx * 2] = m_run[g];
          a.ws.ml[idx * 2 + 1] = l_tot[g];
        }
      }
    }
  }
}

// Merge the partitions of one (sequence, q head):
//   M = max_p m_p,  w_p = 2^(m_p - M),  out = (sum_p w_p o_p) / (sum_p w_p l_p)
// with m_p in log2 units (the logits were scaled by scale * log2 e).
template <int D>
__global__ __launch_bounds__(64) void decode_reduce_kernel(const DecodeArgs a) {
  constexpr int kSets = D / 64;
  const int lane = threadIdx.x;
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  int ctx = a.context_lens[s];
  ctx = min(max(ctx, 0), a.max_context_len);
  const int np = (ctx + a.partition_size - 1) / a.partition_size;
  if (np <= 1) return;

  __shared__ float w_lds[kMaxPartitions];
  const int64_t base = ((int64_t)s * a.num_q_heads + h) * a.num_partitions;
  float mx = -INFINITY;
  for (int p = lane; p < np; p += 64) mx = fmaxf(mx, a.ws.ml[(base + p) * 2]);
  mx = wave_max(mx);
  float lsum = 0.0f;
  for (int p = lane; p < np; p += 64) {
    const float w = fast_exp2(a.ws.ml[(base + p) * 2] - mx);
    w_lds[p] = w;
    lsum += w * a.ws.ml[(base + p) * 2 + 1];
  }
  lsum = wave_sum(lsum);
  __syncthreads();

  float acc[kSets];
#pragma unroll
  for (int st = 0; st < kSets; ++st) acc[st] = 0.0f;
  for (int p = 0; p < np; ++p) {
    const float w = w_lds[p];
    const float* o = a.ws.o + (base + p) * D;
#pragma unroll
    for (int st = 0; st < kSets; ++st) acc[st] += w * o[st * 64 + lane];
  }
  const float inv = 1.0f / lsum;
  half_t* out = a.out + ((int64_t)s * a.num_q_heads + h) * D;
#pragma unroll
  for (int st = 0; st < kSets; ++st) out[st * 64 + lane] = (half_t)(acc[st] * inv);
}

size_t decode_workspace_bytes(int64_t S, int64_t Hq, int64_t D, int64_t NP) {
  const size_t ml = (size_t)(S * Hq * NP * 2) * sizeof(float);
  const size_t ml_aligned = (ml + 255) & ~(size_t)255;
  return ml_aligned + (size_t)(S * Hq * NP * D) * sizeof(float);
}

DecodeWorkspace decode_workspace_carve(void* base, int64_t S, int64_t Hq, int64_t NP) {
  const size_t ml = (size_t)(S * Hq * NP * 2) * sizeof(float);
  const size_t ml_aligned = (ml + 255) & ~(size_t)255;
  DecodeWorkspace w;
  w.ml = reinterpret_cast<float*>(base);
  w.o = reinterpret_cast<float*>(reinterpret_cast<char*>(base) + ml_aligned);
  return w;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.num_partitions, (unsigned)a.num_kv_heads, (unsigned)a.num_seqs);
  if (a.head_dim == 128)
    hipLaunchKernelGGL(decode_partition_kernel<128>, grid, dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_partition_kernel<64>, grid, dim3(64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_partitions <= 1) return e;
  const dim3 rgrid((unsigned)a.num_q_heads, (unsigned)a.num_seqs);
  if (a.head_dim == 128)
    hipLaunchKernelGGL(decode_reduce_kernel<128>, rgrid, dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_reduce_kernel<64>, rgrid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
