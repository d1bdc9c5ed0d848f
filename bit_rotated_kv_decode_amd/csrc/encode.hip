// Everything that rotates and encodes: bulk demotion of keys / values into the rotated INT2
// history, and the per-step preparation launch (the decode-step append with the demotion of the
// token that leaves the recent window, and the query rotation for the INT2 pass).
//
// The steps follow the OSCAR write-up "超越TurboQuant！OSCAR：面向真实服务的2-bit KV Cache量化",
// section OSCAR 的设计: the token leaving the BF16 recent window is rotated by R = U * Hadamard *
// bit-reversal, clipped, quantised with a per-group scale and zero point and packed four 2-bit
// codes to a byte; the query is rotated by the same R_k so that scores can be taken against the
// stored rotated keys.  One 64-lane wave encodes one (token, KV head, K|V) vector: lane l owns
// rotated channels l and l + 64.  The rotation runs in fp64 (x U as a matrix-vector product, the
// Hadamard as cross-lane butterflies), the rotated vector is rounded once to fp32 and every step
// that decides a code (clip, group min / max, (max - min) / 3, fp16 rounding, (x - z) / s, rint)
// runs in IEEE fp32.
#include "device_common.h"
#include "oscar_internal.h"

namespace oscar {
namespace {

constexpr int kWaves = 4;

struct LaneCodes {
  uint32_t c0, c1;     // codes of channels lane and lane + 64
  uint32_t meta[2];    // per group: fp16 scale in bits 0..15, fp16 zero in bits 16..31
};

// Clip and quantise the rotated channels (lane, lane + 64) of one vector; all lanes of the wave
// must call this together (the group min / max are wave reductions).
__device__ __forceinline__ LaneCodes quantize_lane(double r0, double r1, float clip,
                                                   int n_groups) {
  float x0 = static_cast<float>(r0);
  float x1 = static_cast<float>(r1);
  x0 = fminf(fmaxf(x0, -clip), clip);
  x1 = fminf(fmaxf(x1, -clip), clip);
  float mn[2], mx[2];
  if (n_groups == 1) {
    mn[0] = mn[1] = dev::wave_min(fminf(x0, x1));
    mx[0] = mx[1] = dev::wave_max(fmaxf(x0, x1));
  } else {
    // group 0 = channels 0..63 (slot 0 of every lane), group 1 = channels 64..127 (slot 1)
    mn[0] = dev::wave_min(x0);
    mx[0] = dev::wave_max(x0);
    mn[1] = dev::wave_min(x1);
    mx[1] = dev::wave_max(x1);
  }
  LaneCodes out;
  float sf[2], zf[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const float s32 = (mx[m] - mn[m]) / 3.0f;
    const __half s16 = __float2half_rn(s32);
    const __half z16 = __float2half_rn(mn[m]);
    sf[m] = __half2float(s16);
    zf[m] = __half2float(z16);
    out.meta[m] = static_cast<uint32_t>(__half_as_ushort(s16)) |
                  (static_cast<uint32_t>(__half_as_ushort(z16)) << 16);
  }
  auto code = [](float x, float s, float z) -> uint32_t {
    if (s == 0.0f) return 0u;
    const float t = rintf((x - z) / s);
    return static_cast<uint32_t>(fminf(fmaxf(t, 0.0f), 3.0f));
  };
  out.c0 = code(x0, sf[0], zf[0]);
  out.c1 = code(x1, sf[1], zf[1]);
  return out;
}

__device__ __forceinline__ uint8_t* page_block(uint8_t* pool, const int32_t* page_table,
                                               int max_pages_per_seq, int b, int hist_idx, int hkv,
                                               int h, int blk_bytes) {
  const int page = page_table[static_cast<int64_t>(b) * max_pages_per_seq + hist_idx / kPage];
  return pool + (static_cast<int64_t>(page) * hkv + h) * blk_bytes;
}

// Key codes are packed along channels: word w of a token holds channels 16w..16w+15, and the
// words sit in the tiled order of k_word_index.
__device__ __forceinline__ void store_key_row(uint8_t* blk, int slot, uint32_t c0, uint32_t c1) {
  const int lane = dev::lane_id();
  uint32_t v0 = c0 << (2 * (lane & 15));
  uint32_t v1 = c1 << (2 * (lane & 15));
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) {
    v0 |= __shfl_xor(v0, m);
    v1 |= __shfl_xor(v1, m);
  }
  if ((lane & 15) == 0) {
    uint32_t* words = reinterpret_cast<uint32_t*>(blk + kKCodesOff);
    words[k_word_index(slot, lane >> 4)] = v0;
    words[k_word_index(slot, 4 + (lane >> 4))] = v1;
  }
}

// Per-token meta: key groups first, then value groups (tensor 0 = K, 1 = V).
__device__ __forceinline__ void store_meta(uint8_t* blk, int tensor, int slot, int n_groups,
                                           const LaneCodes& q) {
  if (dev::lane_id() == 0) {
    uint32_t* m = reinterpret_cast<uint32_t*>(blk + kMetaOff + slot * meta_bytes_per_token(n_groups)) +
                  tensor * n_groups;
    for (int g = 0; g < n_groups; ++g) m[g] = q.meta[g];
  }
}

// Replace the bits under `mask` of a pool dword that other waves may update concurrently.
__device__ __forceinline__ void merge_bits(uint32_t* p, uint32_t mask, uint32_t bits) {
  uint32_t old = *p;
  while (true) {
    const uint32_t want = (old & ~mask) | bits;
    const uint32_t prev = atomicCAS(p, old, want);
    if (prev == old) break;
    old = prev;
  }
}

// ------------------------------------------------------------------------------------------
// Bulk demotion.  A wave encodes the tokens of one 16-slot run of a page (history indices
// [16k, 16k + 16) that the call covers) for one (sequence, KV head, K|V).  The 16 slots share the
// value-code dwords, which a full run writes with plain stores; a partly covered run merges its
// bits with compare-and-swap.
constexpr int kRun = 16;

__global__ __launch_bounds__(256) void demote_kernel(DemoteArgs a, int runs_per_seq) {
  __shared__ float xs[kWaves][kRun * kHeadDim];
  const int wave = threadIdx.x >> 6;
  const int lane = dev::lane_id();
  int64_t wid = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
  const int tensor = static_cast<int>(wid % 2);
  wid /= 2;
  const int h = static_cast<int>(wid % a.hkv);
  wid /= a.hkv;
  const int run = static_cast<int>(wid % runs_per_seq);
  const int b = static_cast<int>(wid / runs_per_seq);
  if (b >= a.batch) return;

  const int hs = a.hist_start[b];
  const int first = (hs / kRun + run) * kRun;   // first history index of this run
  const int lo = max(first, hs);
  const int hi = min(first + kRun, hs + a.n_tokens);
  if (lo >= hi) return;

  const uint16_t* src = tensor == 0 ? a.k_src : a.v_src;
  float* x = xs[wave];
  for (int t = 0; t < kRun; ++t) {
    const int idx = first + t;
    float v0 = 0.0f, v1 = 0.0f;
    if (idx >= lo && idx < hi) {
      const uint16_t* row = src + b * a.stride_b + static_cast<int64_t>(idx - hs) * a.stride_t +
                            static_cast<int64_t>(h) * a.stride_h;
      v0 = dev::bf16_to_f32(row[lane]);
      v1 = dev::bf16_to_f32(row[lane + 64]);
    }
    x[t * kHeadDim + lane] = v0;
    x[t * kHeadDim + lane + 64] = v1;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

  const float* u = (tensor == 0 ? a.u_k : a.u_v) + static_cast<int64_t>(h) * kHeadDim * kHeadDim;
  const float clip = (tensor == 0 ? a.clip_k : a.clip_v)[h];
  double r[kRun][2];
  dev::rotate_fp64<kRun>(x, u, r);

  const int blk_bytes = block_bytes(a.n_groups);
  uint8_t* blk = page_block(a.pool, a.page_table, a.max_pages_per_seq, b, first, a.hkv, h,
                            blk_bytes);
  const int slot0 = first % kPage;
  uint32_t vword0 = 0, vword1 = 0, vmask = 0;
#pragma unroll
  for (int t = 0; t < kRun; ++t) {
    const LaneCodes q = quantize_lane(r[t][0], r[t][1], clip, a.n_groups);
    const int idx = first + t;
    if (idx < lo || idx >= hi) continue;
    if (tensor == 0) {
      store_key_row(blk, slot0 + t, q.c0, q.c1);
    } else {
      vword0 |= q.c0 << (2 * t);
      vword1 |= q.c1 << (2 * t);
      vmask |= 3u << (2 * t);
    }
    store_meta(blk, tensor, slot0 + t, a.n_groups, q);
  }
  if (tensor == 1) {
    // value codes of channel j for this run: word (j, slot0 / 16) of the value region
    uint32_t* vc = reinterpret_cast<uint32_t*>(blk + kVCodesOff);
    const int uw = slot0 / kRun;
    uint32_t* w0 = &vc[v_word_index(lane, uw)];
    uint32_t* w1 = &vc[v_word_index(lane + 64, uw)];
    if (vmask == 0xFFFFFFFFu) {
      *w0 = vword0;
      *w1 = vword1;
    } else {
      merge_bits(w0, vmask, vword0);
      merge_bits(w1, vmask, vword1);
    }
  }
}

// ------------------------------------------------------------------------------------------
// Step preparation: one 256-thread block per work item.  Items [0, n_query) rotate one query
// row each (sequence b, query head); the following batch * hkv * 2 items append one new token
// per (sequence, KV head, K|V).  Both kinds start their U loads before anything else.
//
// Append: the token at position pos goes to the sink (pos < 64) or to ring row pos % 256; once
// the ring is full the row's previous token (position pos - 256, history index pos - 320) is
// first rotated, quantised and stored in its page slot.  Waves 2 and 3 overwrite the ring row
// after the old row is staged; wave 0 quantises and stores.  The value-code bits of the slot are
// replaced with a pair of no-return atomics (and, then or), which needs no read: no other writer
// touches the word during the launch, since a sequence appends one token per call and a page is
// written by its own sequence only.
//
// Query: q' = q R_k for the row's KV head, split for the INT2 pass into int8 hi / lo parts
// (q' ~ a (hi + lo / 256), a = max |q'| / 127) stored in MFMA operand order, and per row the
// score scale a / 256 * sm_scale * log2(e) and the per-group sums of the quantised q' (exact, in
// units of a / 256) that the zero points multiply.
__device__ __forceinline__ void append_item(const AppendArgs& a, int item, unsigned char* smem) {
  float* x = reinterpret_cast<float*>(smem);
  double (*red)[kHeadDim] = reinterpret_cast<double (*)[kHeadDim]>(smem + 4 * kHeadDim);
  const int tid = threadIdx.x;
  const int tensor = item & 1;
  const int h = (item >> 1) % a.hkv;
  const int b = (item >> 1) / a.hkv;
  const int pos = a.seq_lens[b];
  const int64_t slot = a.seq_slot[b];
  const uint16_t* nw = (tensor == 0 ? a.k_new : a.v_new) +
                       (static_cast<int64_t>(b) * a.hkv + h) * kHeadDim;
  if (pos < kSink) {
    if (tid < kHeadDim) {
      uint16_t* row = (tensor == 0 ? a.sink_k : a.sink_v) +
                      ((slot * a.hkv + h) * kSink + pos) * kHeadDim;
      row[tid] = nw[tid];
    }
    return;
  }
  uint16_t* ring = (tensor == 0 ? a.recent_k : a.recent_v) +
                   ((slot * a.hkv + h) * kRecent + pos % kRecent) * kHeadDim;
  const uint16_t nv = tid >= 128 ? nw[tid - 128] : 0;
  if (pos < kSink + kRecent) {
    if (tid >= 128) ring[tid - 128] = nv;
    return;
  }
  dev::URows ur;
  dev::load_u_rows((tensor == 0 ? a.u_k : a.u_v) + static_cast<int64_t>(h) * kHeadDim * kHeadDim,
                   ur);
  if (tid < kHeadDim) x[tid] = dev::bf16_to_f32(ring[tid]);
  __syncthreads();   // the old row is staged: waves 2 and 3 may overwrite it
  if (tid >= 128) ring[tid - 128] = nv;
  double r0, r1;
  if (dev::rotate1_block(x, ur, red, r0, r1)) {
    const float clip = (tensor == 0 ? a.clip_k : a.clip_v)[h];
    const LaneCodes q = quantize_lane(r0, r1, clip, a.n_groups);
    const int idx = pos - kSink - kRecent;
    uint8_t* blk = page_block(a.pool, a.page_table, a.max_pages_per_seq, b, idx, a.hkv, h,
                              block_bytes(a.n_groups));
    const int slot_in_page = idx % kPage;
    const int lane = dev::lane_id();
    if (tensor == 0) {
      store_key_row(blk, slot_in_page, q.c0, q.c1);
    } else {
      uint32_t* vc = reinterpret_cast<uint32_t*>(blk + kVCodesOff);
      const int u = slot_in_page / 16;
      const int sh = 2 * (slot_in_page % 16);
      uint32_t* w0 = &vc[v_word_index(lane, u)];
      uint32_t* w1 = &vc[v_word_index(lane + 64, u)];
      __hip_atomic_fetch_and(w0, ~(3u << sh), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_and(w1, ~(3u << sh), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_or(w0, q.c0 << sh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_or(w1, q.c1 << sh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    store_meta(blk, tensor, slot_in_page, a.n_groups, q);
  }
}

__device__ __forceinline__ void query_item(const QueryArgs& a, int row, unsigned char* smem) {
  float* x = reinterpret_cast<float*>(smem);
  double (*red)[kHeadDim] = reinterpret_cast<double (*)[kHeadDim]>(smem + 4 * kHeadDim);
  const int kv = (row % a.hq) / a.gqa;
  dev::URows ur;
  dev::load_u_rows(a.u_k + static_cast<int64_t>(kv) * kHeadDim * kHeadDim, ur);
  if (threadIdx.x < kHeadDim)
    x[threadIdx.x] = dev::bf16_to_f32(a.q[static_cast<int64_t>(row) * kHeadDim + threadIdx.x]);
  __syncthreads();
  double r0, r1;
  if (!dev::rotate1_block(x, ur, red, r0, r1)) return;
  const int lane = dev::lane_id();
  const float f0 = static_cast<float>(r0);   // rotated channel lane
  const float f1 = static_cast<float>(r1);   // rotated channel lane + 64
  const float amax = dev::wave_max(fmaxf(fabsf(f0), fabsf(f1)));
  const float sa = amax > 0.f ? amax / 127.f : 1.f;
  auto split = [sa](float v, int& hi, int& lo) {
    hi = static_cast<int>(rintf(v / sa));
    const float r = fmaf(-static_cast<float>(hi), sa, v);
    lo = static_cast<int>(fminf(fmaxf(rintf(r * 256.f / sa), -127.f), 127.f));
  };
  int h0, l0, h1, l1;
  split(f0, h0, l0);
  split(f1, h1, l1);
  // MFMA operand order: channel j = 16 qd + 4 b + k sits at byte 16 qd + 4 k + b
  auto opos = [](int j) { return (j >> 4) * 16 + (j & 3) * 4 + ((j >> 2) & 3); };
  int8_t* dst = a.qpack + static_cast<int64_t>(row) * 256;
  dst[opos(lane)] = static_cast<int8_t>(h0);
  dst[opos(lane + 64)] = static_cast<int8_t>(h1);
  dst[128 + opos(lane)] = static_cast<int8_t>(l0);
  dst[128 + opos(lane + 64)] = static_cast<int8_t>(l1);
  // sums of the quantised q' per group, in units of a / 256 (exact in int32)
  const int e0 = 256 * h0 + l0, e1 = 256 * h1 + l1;
  int s0, s1;
  if (a.n_groups == 1) {
    s0 = dev::wave_sum_i(e0 + e1);
    s1 = 0;
  } else {
    s0 = dev::wave_sum_i(e0);
    s1 = dev::wave_sum_i(e1);
  }
  if (lane == 0) {
    float* m = a.qmeta + static_cast<int64_t>(row) * 4;
    m[0] = sa / 256.f * a.scale_log2;
    m[1] = static_cast<float>(s0);
    m[2] = static_cast<float>(s1);
    m[3] = 0.f;
  }
}

// x0 + blockIdx.x < n_query: query row; else append item x0 + blockIdx.x - n_query.
__global__ __launch_bounds__(256) void prep_kernel(AppendArgs ap, QueryArgs qa, int n_query,
                                                   int x0) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * kHeadDim + 4 * 8 * kHeadDim];
  const int item = x0 + blockIdx.x;
  if (item < n_query)
    query_item(qa, item, smem);
  else
    append_item(ap, item - n_query, smem);
}

}  // namespace

hipError_t launch_demote(const DemoteArgs& a, hipStream_t stream) {
  if (a.batch == 0 || a.n_tokens == 0) return hipSuccess;
  const int runs_per_seq = (a.n_tokens + kRun - 1) / kRun + 1;
  const int64_t waves = static_cast<int64_t>(a.batch) * runs_per_seq * a.hkv * 2;
  const int64_t blocks = (waves + kWaves - 1) / kWaves;
  hipLaunchKernelGGL(demote_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a,
                     runs_per_seq);
  return hipGetLastError();
}

hipError_t launch_prep(const AppendArgs* ap, const QueryArgs* qa, hipStream_t stream) {
  const int n_query = qa ? qa->batch * qa->hq : 0;
  const int n_append = ap ? ap->batch * ap->hkv * 2 : 0;
  const int x0 = qa ? 0 : n_query;
  const int n = n_query + n_append - x0;
  if (n == 0) return hipSuccess;
  const AppendArgs a0 = ap ? *ap : AppendArgs{};
  const QueryArgs q0 = qa ? *qa : QueryArgs{};
  hipLaunchKernelGGL(prep_kernel, dim3(static_cast<unsigned>(n)), dim3(256), 0, stream, a0, q0,
                     n_query, x0);
  return hipGetLastError();
}

}  // namespace oscar
