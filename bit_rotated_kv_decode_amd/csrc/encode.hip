// Everything that rotates and encodes: bulk demotion of keys / values into the rotated INT2
// history, and the per-step preparation launch (the decode-step append with the demotion of the
// token that leaves the recent window, and the query rotation for the INT2 pass).
//
// The steps follow the OSCAR write-up "超越TurboQuant！OSCAR：面向真实服务的2-bit KV Cache量化",
// section OSCAR 的设计: the token leaving the BF16 recent window is rotated by R = U * Hadamard *
// bit-reversal, clipped, quantised with a per-group scale and zero point and packed four 2-bit
// codes to a byte; the query is rotated by the same R_k so that scores can be taken against the
// stored rotated keys.  One 64-lane wave encodes one (token, KV head, K|V) vector: lane l owns
// rotated channels l and l + 64.  The history's rotation runs in fp64 (x U as a matrix-vector
// product, the Hadamard as cross-lane butterflies), the rotated vector is rounded once to fp32 and
// every step that decides a code (clip, group min / max, (max - min) / 3, fp16 rounding,
// (x - z) / s, rint) runs in IEEE fp32.  The query's rotation for the four-head pass runs in fp32
// (it decides no code; dev::query_partials / query_finish, shared with the decode step's segment
// launch, which repeats it); the other passes' query rotation is the fp64 one.
#include "device_common.h"
#include "encode_common.h"
#include "oscar_internal.h"

namespace oscar {
namespace {

using namespace enc;

constexpr int kWaves = 4;

// ------------------------------------------------------------------------------------------
// Bulk demotion.  A wave encodes the 16 slots of one value-word group of a page, the slots
// 16 s + 4 u + j (s, j = 0..3) whose value codes share one word per channel, for one (sequence,
// KV head, K|V), taking the ones the call covers.  A fully covered group writes its value-code
// words with plain stores; a partly covered one merges its bits with compare-and-swap.
constexpr int kRun = 16;
constexpr int kGroupsPerPage = kPage / kRun;

__device__ __forceinline__ int group_slot(int u, int t) { return 16 * (t >> 2) + 4 * u + (t & 3); }

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
  const int first = (hs / kPage + run / kGroupsPerPage) * kPage;   // history index of slot 0
  const int ug = run % kGroupsPerPage;
  const int lo = hs, hi = hs + a.n_tokens;
  bool any = false;
#pragma unroll
  for (int t = 0; t < kRun; ++t) {
    const int idx = first + group_slot(ug, t);
    any |= idx >= lo && idx < hi;
  }
  if (!any) return;

  const uint16_t* src = tensor == 0 ? a.k_src : a.v_src;
  float* x = xs[wave];
  for (int t = 0; t < kRun; ++t) {
    const int idx = first + group_slot(ug, t);
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
  const float* lvp = tensor == 0 ? a.levels_k : a.levels_v;
  const float lv_lo = lvp ? lvp[2 * h] : 0.0f;
  const float lv_step = lvp ? lvp[2 * h + 1] : 1.0f;
  double r[kRun][2];
  dev::rotate_fp64<kRun>(x, u, r);

  const int blk_bytes = block_bytes(a.n_groups);
  uint8_t* blk = page_block(a.pool, a.page_table, a.max_pages_per_seq, b, first, a.hkv, h,
                            blk_bytes);
  uint32_t vword0 = 0, vword1 = 0, vmask = 0;
#pragma unroll
  for (int t = 0; t < kRun; ++t) {
    const LaneCodes q = quantize_lane(r[t][0], r[t][1], clip, a.n_groups, lv_lo, lv_step,
                                     a.levels_kind);
    const int slot = group_slot(ug, t);
    const int idx = first + slot;
    if (idx < lo || idx >= hi) continue;
    if (tensor == 0) {
      store_key_row(blk, slot, q.c0, q.c1);
    } else {
      const int sh = 2 * v_code_pos(slot);
      vword0 |= q.c0 << sh;
      vword1 |= q.c1 << sh;
      vmask |= 3u << sh;
    }
    store_meta(blk, tensor, slot, a.n_groups, q);
  }
  if (tensor == 1) {
    // value codes of channel j for this group: word (j, ug) of the value region
    uint32_t* vc = reinterpret_cast<uint32_t*>(blk + kVCodesOff);
    uint32_t* w0 = &vc[v_word_index(lane, ug)];
    uint32_t* w1 = &vc[v_word_index(lane + 64, ug)];
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
// row each (sequence b, query head); the following batch * 2 * hkv items append one new token
// per (sequence, K|V, KV head).  Both kinds start their U loads before anything else.
//
// Append: the token at position pos goes to the sink (pos < 64) or to ring row pos % 256; once
// the ring is full the row's previous token (position pos - 256, history index pos - 320) is
// first rotated, quantised and stored in its page slot.  Waves 2 and 3 overwrite the ring row
// after the old row is staged; wave 0 quantises and stores.  The value-code bits of the slot are
// replaced with a pair of no-return atomics (and, then or), which needs no read: no other writer
// touches the word during the launch, since a sequence appends one token per call and a page is
// written by its own sequence only.
//
// Query: q' = q R_k for the row's KV head, scaled by sm_scale * log2(e) and written as the key
// operand of the INT2 pass the shape takes: fp8 parts with E8M0 row scales (up to four heads,
// one group) or int8 hi / lo parts (otherwise), with the per-group sums the zero points multiply.
__device__ __forceinline__ void append_item(const AppendArgs& a, int item, unsigned char* smem) {
  float* x = reinterpret_cast<float*>(smem);
  double (*red)[kHeadDim] = reinterpret_cast<double (*)[kHeadDim]>(smem + 4 * kHeadDim);
  const int tid = threadIdx.x;
  const int h = item % a.hkv;
  const int tensor = (item / a.hkv) & 1;
  const int b = item / a.hkv / 2;
  // the U slice is read before anything else (it does not depend on the position), so its loads
  // overlap the round trips for the position and the ring row
  dev::URows ur;
  dev::load_u_rows((tensor == 0 ? a.u_k : a.u_v) + static_cast<int64_t>(h) * kHeadDim * kHeadDim,
                   ur);
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
  // the slot's page and the clip threshold are fetched alongside the old row
  const int idx = pos - kSink - kRecent;
  uint8_t* blk = page_block(a.pool, a.page_table, a.max_pages_per_seq, b, idx, a.hkv, h,
                            block_bytes(a.n_groups));
  const float clip = (tensor == 0 ? a.clip_k : a.clip_v)[h];
  const float* lvp = tensor == 0 ? a.levels_k : a.levels_v;
  const float lv_lo = lvp ? lvp[2 * h] : 0.0f;
  const float lv_step = lvp ? lvp[2 * h + 1] : 1.0f;
  if (tid < kHeadDim) x[tid] = dev::bf16_to_f32(ring[tid]);
  __syncthreads();   // the old row is staged: waves 2 and 3 may overwrite it
  if (tid >= 128) ring[tid - 128] = nv;
  double r0, r1;
  if (dev::rotate1_block(x, ur, red, r0, r1)) {
    const LaneCodes q = quantize_lane(r0, r1, clip, a.n_groups, lv_lo, lv_step, a.levels_kind);
    store_token(blk, tensor, idx % kPage, a.n_groups, q);
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
  if (!int2_fp8_pass(a.gqa, a.n_groups)) {
    double r0, r1;
    if (!dev::rotate1_block(x, ur, red, r0, r1)) return;
    split_query(r0, r1, a.n_groups, a.scale_log2, a.qpack + static_cast<int64_t>(row) * 256,
                a.qmeta + static_cast<int64_t>(row) * 4);
    return;
  }
  // the fp8 pass: the fp32 rotation the segment launch of a fused decode step also runs
  float (*redf)[kHeadDim] = reinterpret_cast<float (*)[kHeadDim]>(smem + 4 * kHeadDim);
  float y[4];
  dev::query_partials(x, ur, y);
#pragma unroll
  for (int e = 0; e < 4; ++e) redf[threadIdx.x >> 5][4 * (threadIdx.x & 31) + e] = y[e];
  __syncthreads();
  if ((threadIdx.x >> 6) != 0) return;
  float o0, o1;
  dev::query_finish(redf, o0, o1);
  const int b = row / a.hq, hd = (row % a.hq) % a.gqa;
  const int64_t op = (static_cast<int64_t>(b) * a.hkv + kv) * key_tiles(a.gqa) * a.n_groups;
  query_operands(o0, o1, a.n_groups, a.gqa, hd, a.scale_log2, a.qops + op * 2048,
                 a.qscales + op * 64, a.qmeta + static_cast<int64_t>(row) * 4);
}

// x0 + blockIdx.x < n_query: query row; else append item x0 + blockIdx.x - n_query.
__global__ __launch_bounds__(256) void prep_kernel(AppendArgs ap, QueryArgs qa, int n_query,
                                                   int x0) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * kHeadDim +
                                                           dev::kRotGroups * 8 * kHeadDim];
  // Items are numbered with the KV head fastest: consecutive blocks go to the eight dies in turn,
  // so the items of one KV head (which share its U) run on one die, as do that head's attention
  // blocks (block x of the attention grid serves KV head x mod Hkv).
  const int item = x0 + blockIdx.x;
  if (item < n_query) {
    const int kv = item % qa.hkv, r = item / qa.hkv;
    query_item(qa, (r / qa.gqa) * qa.hq + kv * qa.gqa + r % qa.gqa, smem);
  } else {
    append_item(ap, item - n_query, smem);
  }
}

}  // namespace

hipError_t launch_demote(const DemoteArgs& a, hipStream_t stream) {
  if (a.batch == 0 || a.n_tokens == 0) return hipSuccess;
  // value-word groups of the pages a call can touch: at most ceil(n / 64) + 1 pages
  const int runs_per_seq = ((a.n_tokens + kPage - 1) / kPage + 1) * kGroupsPerPage;
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
