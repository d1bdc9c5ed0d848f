// Paged BF16 decode attention: the all-BF16 cache that an INT2 history is measured against.
//
// The OSCAR write-ups state the system gains of the rotated INT2 history relative to keeping the
// history in BF16: about 8x less KV memory, up to 3x faster batch-1 decoding at 100k context
// with a full prefix-cache hit, up to 7x throughput at large batch under the same memory budget
// ("超越TurboQuant！OSCAR：面向真实服务的2-bit KV Cache量化" and its repost, evaluation part;
// "OSCAR: Offline Spectral Covariance-Aware Rotation for 2-bit KV Cache Quantization", Abstract).
// This file is that baseline on the same page table: every cached token of a sequence, from
// position 0, sits in a BF16 page.
//
// Page block (one page of 64 tokens, one KV head), 32 KiB in matrix-core operand order: 32 rows
// of 64 lanes x 16 bytes; row 16 h + 4 tt + s holds, for lane 16 j + n, key channels
// 32 s + 8 j .. + 7 of token 32 h + 16 tt + n, and row 16 h + 8 + nt holds, for lane 16 j + n,
// value channel 16 nt + n of tokens 32 h + 8 j .. + 7.  Every load instruction of a wave then
// reads 1 KiB of contiguous memory, and each 8-byte group of bf16 elements is one lane's operand.
//
// Launch order on one stream:
//   1. bf16_attn_kernel   split-KV: block = 4 waves on pages [p0, p1) of one (sequence, KV head);
//                         per 32-token chunk: scores as v_mfma_f32_16x16x32_bf16 (exact bf16
//                         products, fp32 sums), online softmax, p split into bf16 hi + lo parts
//                         transposed through the wave's LDS tile, values as bf16 MFMAs;
//                         -> (m, l, acc) per split;
//   2. bf16_merge_kernel  log-sum-exp merge of the splits and normalisation.
// Softmax statistics are kept in the log2 domain (scores scaled by sm_scale * log2 e).
#include "device_common.h"
#include "oscar_internal.h"

namespace oscar {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));

constexpr float kLog2eBf = 1.4426950408889634f;
constexpr int kRsrcWord3 = 0x00020000;   // last buffer-descriptor word: raw 32-bit elements
constexpr int kAuxStream = 2;            // non-temporal cache policy of a buffer load

__device__ __forceinline__ v8bf as_bf8(u4v x) { return __builtin_bit_cast(v8bf, x); }

// One 32-token chunk of a page, as this lane's matrix-core operands: k[tt][s] = key row
// 16 tt + n, channels 32 s + 8 j .. + 7; v[nt] = value channel 16 nt + n, tokens 8 j .. + 7.
struct Chunk {
  u4v k[2][4];
  u4v v[8];
};

// Scores D[row][token] = sum_k A[row][k] B[k][token]: A row r holds query head r % G (all 16
// rows used, so lane (n, j) register i carries head (4 j + i) % G); B = 16 keys.  Values
// D[row][ch] = sum_t P[row][t] V[t][ch]: P rows 0-7 hold the bf16 hi part of p for head r % G,
// rows 8-15 the lo part (p - hi), so row groups j = 0, 1 hold hi and j = 2, 3 lo sums of the
// same heads, and one swap of wave halves adds them.
// STREAM: non-temporal page loads, chosen when the launch holds one sequence (no page can be read
// twice); with several sequences shared prefix pages may be read again and cached loads let the
// later readers hit.
template <int G, bool STREAM>
__global__ __launch_bounds__(256, 2) void bf16_attn_kernel(Bf16DecodeArgs a, Bf16Plan p) {
  __shared__ __attribute__((aligned(16))) __bf16 ptile[4][16][32];
  __shared__ __attribute__((aligned(16))) float red_acc[4][G][kHeadDim];
  __shared__ float red_m[4][G], red_l[4][G];
  const int kv = static_cast<int>(blockIdx.x) % p.hkv;
  const int split = static_cast<int>(blockIdx.x) / p.hkv;
  const int b = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = dev::lane_id();
  const int n = lane & 15, j = lane >> 4;
  const int p0 = split * p.pages_per_split;
  // page ids of this wave's pages p0 + wave + 4 i, one per lane i (a split covers at most 256
  // pages), read before the sequence length is known; the index stays inside the table row
  static_assert(kMaxPagesPerSplit <= 4 * 64, "one page id per lane and wave");
  const int wave_ids = a.page_table[static_cast<int64_t>(b) * a.max_pages_per_seq +
                                    min(p0 + wave + 4 * lane, a.max_pages_per_seq - 1)];
  const int L = a.seq_lens[b];
  const int n_pages = (L + kPage - 1) / kPage;
  if (p0 >= n_pages) return;
  const int p1 = min(p0 + p.pages_per_split, n_pages);
  const int head0 = b * p.hq + kv * G;
  const float scale_log2 = a.sm_scale * kLog2eBf;

  // query operands: lane (row n, k block j) holds q[head n % G][32 s + 8 j .. + 7]
  v8bf qa[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    qa[s] = *reinterpret_cast<const v8bf*>(a.q + static_cast<int64_t>(head0 + n % G) * kHeadDim +
                                           32 * s + 8 * j);

  float m_run[4], l_run[4];
  v4f acc[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_run[i] = -INFINITY;   // a wave without pages keeps -inf (its partial weighs nothing)
    l_run[i] = 0.f;
  }
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) acc[nt] = v4f{0.f, 0.f, 0.f, 0.f};

  const int n_wave_pages = max(0, (p1 - p0 - wave + 3) / 4);
  const int n_chunks = 2 * n_wave_pages;
  const int loff = lane * 16;   // the lane's 16 bytes in each 1 KiB row of the block
  auto load_chunk = [&](int ci, Chunk& c) {
    ci = min(ci, n_chunks - 1);   // clamped prefetch: the same loads every round
    const int half = ci & 1;
    const int pid = __builtin_amdgcn_readlane(wave_ids, ci >> 1);
    const uint8_t* blk = a.pool + (static_cast<int64_t>(pid) * p.hkv + kv) * kBf16Block;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(blk), 0, kBf16Block, kRsrcWord3);
    constexpr int aux = STREAM ? kAuxStream : 0;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        c.k[tt][s] = __builtin_amdgcn_raw_buffer_load_b128(rs, loff,
                                                           (16 * half + 4 * tt + s) * 1024, aux);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
      c.v[nt] = __builtin_amdgcn_raw_buffer_load_b128(rs, loff, (16 * half + 8 + nt) * 1024, aux);
  };
  auto process_chunk = [&](int ci, Chunk& c) {
    const int tok0 = (p0 + wave + 4 * (ci >> 1)) * kPage + 32 * (ci & 1);
    v4f sc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      v4f d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], as_bf8(c.k[tt][s]), d, 0, 0, 0);
      sc[tt] = d;
    }
    // logits of tokens past the sequence are -inf (their key bits are never used); the chunk's
    // first token is valid for the wave's first chunk, so the running maximum is finite after it
    const bool v0 = tok0 + n < L, v1 = tok0 + 16 + n < L;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x0 = v0 ? sc[0][i] * scale_log2 : -INFINITY;
      const float x1 = v1 ? sc[1][i] * scale_log2 : -INFINITY;
      const float mn = fmaxf(m_run[i], dev::row16_max(fmaxf(x0, x1)));
      const float al = __builtin_amdgcn_exp2f(m_run[i] - mn);
      m_run[i] = mn;
      const float q0 = __builtin_amdgcn_exp2f(x0 - mn), q1 = __builtin_amdgcn_exp2f(x1 - mn);
      l_run[i] = fmaf(l_run[i], al, q0 + q1);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) acc[nt][i] *= al;
      const __bf16 h0 = static_cast<__bf16>(q0), h1 = static_cast<__bf16>(q1);
      const __bf16 w0 = j < 2 ? h0 : static_cast<__bf16>(q0 - static_cast<float>(h0));
      const __bf16 w1 = j < 2 ? h1 : static_cast<__bf16>(q1 - static_cast<float>(h1));
      ptile[wave][4 * j + i][n] = w0;
      ptile[wave][4 * j + i][16 + n] = w1;
    }
    // LDS operations of one wave execute in order: the read below sees the writes above
    __builtin_amdgcn_wave_barrier();
    const v8bf pa = *reinterpret_cast<const v8bf*>(&ptile[wave][n][8 * j]);
    // value slots past the sequence may hold any bits (NaN included): zero them
    if (tok0 + 32 > L) {
      const int vc = min(max(L - (tok0 + 8 * j), 0), 8);   // valid tokens of this lane's octet
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t keep = 2 * d + 1 < vc ? 0xFFFFFFFFu : (2 * d < vc ? 0x0000FFFFu : 0u);
          c.v[nt][d] &= keep;
        }
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, as_bf8(c.v[nt]), acc[nt], 0, 0, 0);
    __builtin_amdgcn_wave_barrier();
  };

  // Two chunk register sets used in turn: the next chunk's loads are in flight while one is
  // processed; the loop over full rounds has a single exit so the wait counts stay exact.
  if (n_chunks > 0) {
    Chunk r[2];
    load_chunk(0, r[0]);
    load_chunk(1, r[1]);
    process_chunk(0, r[0]);
    int ci = 1;
    for (; ci + 1 < n_chunks; ci += 2) {
      load_chunk(ci + 1, r[0]);
      process_chunk(ci, r[1]);
      __builtin_amdgcn_sched_barrier(0);
      load_chunk(ci + 2, r[1]);
      process_chunk(ci + 1, r[0]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (ci < n_chunks) process_chunk(ci, r[1]);
  }

  // ---- the wave's (m, l, acc) per head; hi + lo rows met by one swap of wave halves
#pragma unroll
  for (int i = 0; i < 4; ++i) l_run[i] = dev::row16_sum(l_run[i]);
#pragma unroll
  for (int nt = 0; nt < 8; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x = __float_as_uint(acc[nt][i]);
      const auto sw = __builtin_amdgcn_permlane32_swap(x, x, false, false);
      acc[nt][i] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
  if (j < (G + 3) / 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * j + i;
      if (h < G) {
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) red_acc[wave][h][16 * nt + n] = acc[nt][i];
        if (n == 0) {
          red_m[wave][h] = m_run[i];
          red_l[wave][h] = l_run[i];
        }
      }
    }
  }
  __syncthreads();
  // ---- combine the four waves (wave 0 always has a page, so the maximum is finite)
  float* ml = reinterpret_cast<float*>(a.workspace + p.off_ml);
  float* pacc = reinterpret_cast<float*>(a.workspace + p.off_acc);
  if (threadIdx.x < G * kHeadDim / 4) {
    const int h = threadIdx.x / (kHeadDim / 4), q4 = threadIdx.x % (kHeadDim / 4);
    float mw[4], lw[4];
    float4 aw[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      mw[w] = red_m[w][h];
      lw[w] = red_l[w][h];
      aw[w] = reinterpret_cast<const float4*>(red_acc[w][h])[q4];
    }
    const float mm = fmaxf(fmaxf(mw[0], mw[1]), fmaxf(mw[2], mw[3]));
    float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = __builtin_amdgcn_exp2f(mw[w] - mm);
      s4.x = fmaf(aw[w].x, f, s4.x);
      s4.y = fmaf(aw[w].y, f, s4.y);
      s4.z = fmaf(aw[w].z, f, s4.z);
      s4.w = fmaf(aw[w].w, f, s4.w);
      l = fmaf(lw[w], f, l);
    }
    const int64_t prow = static_cast<int64_t>(head0 + h) * p.num_splits + split;
    reinterpret_cast<float4*>(pacc + prow * kHeadDim)[q4] = s4;
    if (q4 == 0) reinterpret_cast<float2*>(ml)[prow] = make_float2(mm, l);
  }
}

// One 128-thread block per (sequence, query head); thread c owns output channel c.  The split
// statistics go through LDS (one load per thread and round), the accumulators are loaded eight
// splits at a time so that their round trips overlap.  Splits the sequence does not reach were
// never written and are skipped.
__global__ __launch_bounds__(128) void bf16_merge_kernel(Bf16DecodeArgs a, Bf16Plan p) {
  __shared__ float2 st[kMaxSplits];
  __shared__ float red[2];
  const int row = blockIdx.x;   // b * hq + head
  const int b = row / p.hq;
  const int c = threadIdx.x;
  const int L = a.seq_lens[b];
  const int n_pages = (L + kPage - 1) / kPage;
  const int n_valid = (n_pages + p.pages_per_split - 1) / p.pages_per_split;
  const float2* ml = reinterpret_cast<const float2*>(a.workspace + p.off_ml) +
                     static_cast<int64_t>(row) * p.num_splits;
  const float* pacc = reinterpret_cast<const float*>(a.workspace + p.off_acc) +
                      static_cast<int64_t>(row) * p.num_splits * kHeadDim;
  float m = -INFINITY;
  for (int s = c; s < n_valid; s += 128) {
    const float2 v = ml[s];
    st[s] = v;
    m = fmaxf(m, v.x);
  }
  m = dev::wave_max(m);
  if ((c & 63) == 0) red[c >> 6] = m;
  __syncthreads();
  m = fmaxf(red[0], red[1]);
  float l = 0.f, o = 0.f;
  int s = 0;
  for (; s + 8 <= n_valid; s += 8) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = pacc[static_cast<int64_t>(s + i) * kHeadDim + c];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float f = __builtin_amdgcn_exp2f(st[s + i].x - m);
      l = fmaf(st[s + i].y, f, l);
      o = fmaf(v[i], f, o);
    }
  }
  for (; s < n_valid; ++s) {
    const float f = __builtin_amdgcn_exp2f(st[s].x - m);
    l = fmaf(st[s].y, f, l);
    o = fmaf(pacc[static_cast<int64_t>(s) * kHeadDim + c], f, o);
  }
  a.out[static_cast<int64_t>(row) * kHeadDim + c] = o / l;
  if (a.lse != nullptr && c == 0) a.lse[row] = (m + log2f(l)) * 0.6931471805599453f;
}

// Token i of sequence b goes to position start_pos[b] + i, slot pos % 64 of page
// page_table[b][pos / 64], in the operand order of the block (see the top of this file).  One
// wave per (token, KV head, sequence); lane l moves channels 2 l and 2 l + 1.
__global__ __launch_bounds__(64) void bf16_store_kernel(Bf16StoreArgs a) {
  const int i = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int l = threadIdx.x;
  const int pos = a.start_pos[b] + i;
  const int pid = a.page_table[static_cast<int64_t>(b) * a.max_pages_per_seq + pos / kPage];
  const int slot = pos % kPage;
  uint8_t* blk = a.pool + (static_cast<int64_t>(pid) * a.hkv + kv) * kBf16Block;
  const int64_t src = b * a.stride_b + i * a.stride_t + kv * a.stride_h + 2 * l;
  const uint32_t k0 = a.k_src[src], k1 = a.k_src[src + 1];
  const int h = slot >> 5, tt = (slot >> 4) & 1, tn = slot & 15;
  const int c = 2 * l;   // key: channels c, c + 1 = elements (c % 8), (c % 8) + 1 of one lane
  const int krow = 16 * h + 4 * tt + (c >> 5), klane = 16 * ((c & 31) >> 3) + tn;
  reinterpret_cast<uint32_t*>(blk + krow * 1024 + klane * 16)[(c & 7) >> 1] = k0 | (k1 << 16);
  uint16_t* v = reinterpret_cast<uint16_t*>(blk);
  const int vj = (slot & 31) >> 3, ve = slot & 7;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int ch = c + e;
    const int vrow = 16 * h + 8 + (ch >> 4), vlane = 16 * vj + (ch & 15);
    v[(vrow * 1024 + vlane * 16) / 2 + ve] = a.v_src[src + e];
  }
}

}  // namespace

hipError_t launch_bf16_decode(const Bf16DecodeArgs& a, const Bf16Plan& p, hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  if (p.num_splits > 0) {
    const dim3 grid(p.num_splits * p.hkv, 1, p.batch);
    const bool st = a.stream_loads != 0;
    switch (p.gqa) {
      case 1:
        if (st) hipLaunchKernelGGL((bf16_attn_kernel<1, true>), grid, dim3(256), 0, stream, a, p);
        else hipLaunchKernelGGL((bf16_attn_kernel<1, false>), grid, dim3(256), 0, stream, a, p);
        break;
      case 2:
        if (st) hipLaunchKernelGGL((bf16_attn_kernel<2, true>), grid, dim3(256), 0, stream, a, p);
        else hipLaunchKernelGGL((bf16_attn_kernel<2, false>), grid, dim3(256), 0, stream, a, p);
        break;
      case 4:
        if (st) hipLaunchKernelGGL((bf16_attn_kernel<4, true>), grid, dim3(256), 0, stream, a, p);
        else hipLaunchKernelGGL((bf16_attn_kernel<4, false>), grid, dim3(256), 0, stream, a, p);
        break;
      case 8:
        if (st) hipLaunchKernelGGL((bf16_attn_kernel<8, true>), grid, dim3(256), 0, stream, a, p);
        else hipLaunchKernelGGL((bf16_attn_kernel<8, false>), grid, dim3(256), 0, stream, a, p);
        break;
      default: return hipErrorInvalidValue;
    }
  }
  hipLaunchKernelGGL(bf16_merge_kernel, dim3(p.batch * p.hq), dim3(128), 0, stream, a, p);
  return hipGetLastError();
}

hipError_t launch_bf16_store(const Bf16StoreArgs& a, hipStream_t stream) {
  if (a.batch == 0 || a.n_tokens == 0) return hipSuccess;
  hipLaunchKernelGGL(bf16_store_kernel, dim3(a.n_tokens, a.hkv, a.batch), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace oscar
