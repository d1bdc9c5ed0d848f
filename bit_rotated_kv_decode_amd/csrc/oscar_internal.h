// Internal interface between the C-ABI host layer (oscar_api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "oscar.h"

namespace oscar {

constexpr int kHeadDim = 128;
constexpr int kPage = 64;
constexpr int kSink = 64;
constexpr int kRecent = 256;
constexpr int kBf16Chunks = (kSink + kRecent) / 64;  // 64-token chunks of the BF16 segments
constexpr int kMaxGqa = 8;
constexpr int kMaxPagesPerSplit = 256;    // history pages one INT2 work item may cover
constexpr int kMaxSplits = 1024;          // INT2 work items per (sequence, KV head)
constexpr int kMergeSplits = 96;          // splits per row the merge loads at once
constexpr int kInt2Items = 512;           // blocks per launch the plan aims at (2 per compute unit)
constexpr int kComputeUnits = 256;        // compute units of an MI355X (gfx950)
// Shared-prefix cascade: a cascade block takes kCascPages pages of the shared prefix of one KV head
// (staged in LDS) for a group of kCascGroup sequences, four waves taking kCascGroup / 4 each.
constexpr int kCascPages = 12;
constexpr int kCascGroup = 16;
// The INT2 pass a (query heads per KV head, groups per head) shape takes: the fp8 x FP4 pass for
// tiles of up to four heads and one group, the int8 / bf16 pass otherwise.  The preparation
// launch writes the query operand that pass reads.
__host__ __device__ constexpr bool int2_fp8_pass(int gqa, int n_groups) {
  return gqa <= 4 && n_groups == 1;
}

// Byte offsets inside one (page, KV head) block for head_dim 128 (see include/oscar.h).
constexpr int kKCodesOff = 0;
constexpr int kVCodesOff = kPage * kHeadDim / 4;              // 2048
constexpr int kMetaOff = kVCodesOff + kHeadDim * kPage / 4;   // 4096
// per token: fp16 (scale, zero) of each key group, then of each value group
__host__ __device__ inline int meta_bytes_per_token(int n_groups) { return 8 * n_groups; }
__host__ __device__ inline int block_bytes(int n_groups) {
  return kMetaOff + kPage * meta_bytes_per_token(n_groups);
}
// Tiled word order of the code regions: a word holds 16 two-bit codes, and each 1 KiB row of a
// region is 64 lanes x 16 bytes, so that one 16-byte load per lane fetches the words of that lane's
// MFMA operands.  Key word (token t = 16 st + n, channels 16 w .. 16 w + 15 with w = 4 hf + q):
// lane 16 q + n of chunk row st / 2, entry 2 (st % 2) + hf.  Value word (channel c = 16 nt + n,
// token group u): lane 16 u + n of chunk row nt / 4, entry nt % 4; it holds the codes of the 16
// tokens 16 s + 4 u + j (s, j = 0..3), token (s, j) at code position v_code_pos.
__host__ __device__ inline int k_word_index(int t, int w) {
  return (((t >> 5) * 64 + (w & 3) * 16 + (t & 15)) << 2) + (((t >> 4) & 1) << 1) + (w >> 2);
}
__host__ __device__ inline int v_word_index(int c, int u) {
  return (((c >> 6) * 64 + u * 16 + (c & 15)) << 2) + ((c >> 4) & 3);
}
// value-code word group and code position of page slot t = 16 s + 4 u + j
__host__ __device__ inline int v_code_group(int t) { return (t >> 2) & 3; }
__host__ __device__ inline int v_code_pos(int t) {
  return 8 * ((t >> 1) & 1) + 2 * (t >> 4) + (t & 1);
}

// Work plan of one decode-attention call, and the carve-up of its workspace.
struct Plan {
  int batch = 0, hq = 0, hkv = 0, gqa = 0, n_groups = 0;
  int max_pages = 0;         // history pages of the longest sequence
  int pages_per_split = 1;   // history pages per INT2 work item
  int num_splits = 0;        // work items per (sequence, KV head)
  int casc_chunks = 0;       // shared-prefix chunks of kCascPages pages taken by cascade blocks
  int casc_groups = 0;       // sequence groups of kCascGroup per cascade chunk
  int slots = 0;             // INT2 partials per (sequence, query head): casc_chunks + num_splits
  size_t off_qrot = 0;       // int8 [B][Hq][2][128] rotated queries, hi / lo parts (int8 pass)
  size_t off_qops = 0;       // fp8 key operands [B][Hkv][tiles][groups][64 lanes][32 B]
  size_t off_qscale = 0;     // int32 E8M0 row scales [B][Hkv][tiles][groups][64 lanes]
  size_t off_sigma = 0;      // fp32 [B][Hq][4] per-group sums of the rotated, scaled query
  size_t off_int2_ml = 0;    // fp32 [B][Hq][slots][2] (m, l) of INT2 partials (log2 domain):
                             // cascade chunks first, then the splits
  size_t off_int2_acc = 0;   // fp32 [B][Hq][slots][128] rotated-space accumulators
  size_t off_bf16_ml = 0;    // fp32 [B][Hq][5][2]
  size_t off_bf16_acc = 0;   // fp32 [B][Hq][5][128]
  size_t off_flags = 0;      // int32 [B][Hkv] at offset 0: a fused decode step's displaced-token
                             // flags, zero between calls
  size_t total = 0;
};

// prefix_pages: pages of a shared prefix a cascade may take (0: none).
Plan make_plan(const oscar_layout& lay, int batch, int max_seq_len, int prefix_pages = 0);

// History pages of a sequence that the cascade chunks of plan p take: the whole chunks within
// both its full history pages (n_hist tokens) and its first `shared` pages (those of its
// page-table row that are the shared prefix's).
__host__ __device__ inline int cascade_pages(const Plan& p, int n_hist, int shared) {
  const int held = n_hist / kPage < shared ? n_hist / kPage : shared;
  const int chunks = held / kCascPages;
  return kCascPages * (chunks < p.casc_chunks ? chunks : p.casc_chunks);
}

struct DemoteArgs {
  uint8_t* pool;
  const int32_t* page_table;
  int max_pages_per_seq;
  int hkv;
  int n_groups;
  const float* u_k;
  const float* u_v;
  const float* clip_k;
  const float* clip_v;
  const float* levels_k;   // [hkv][2] (lo, step) of an equally spaced codebook, (l0, l1) of a
  const float* levels_v;   // symmetric one (levels_kind 1), or NULL
  int levels_kind;
  const uint16_t* k_src;
  const uint16_t* v_src;
  int64_t stride_b, stride_t, stride_h;
  const int32_t* hist_start;
  int batch;
  int n_tokens;
};

struct AppendArgs {
  uint8_t* pool;
  const int32_t* page_table;
  int max_pages_per_seq;
  int hkv;
  int n_groups;
  uint16_t* sink_k;
  uint16_t* sink_v;
  uint16_t* recent_k;
  uint16_t* recent_v;
  const float* u_k;
  const float* u_v;
  const float* clip_k;
  const float* clip_v;
  const float* levels_k;   // as in DemoteArgs
  const float* levels_v;
  int levels_kind;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int32_t* seq_slot;
  const int32_t* seq_lens;
  int batch;
};

struct DecodeArgs {
  const uint8_t* pool;
  const int32_t* page_table;
  int max_pages_per_seq;
  const uint16_t* sink_k;
  const uint16_t* sink_v;
  const uint16_t* recent_k;
  const uint16_t* recent_v;
  const int32_t* seq_slot;
  const int32_t* seq_lens;
  const uint16_t* q;
  const float* u_k;
  const float* u_v;
  float sm_scale;
  float* out;
  float* lse;
  uint8_t* workspace;
  int len_add;            // added to seq_lens[b] (1 when seq_lens holds the new token's position)
  // [hkv][2] (l0, l1) of the symmetric codebooks the history was encoded with (levels
  // (l0, l1, 3 - l1, 3 - l0)), or NULL for the grid {0, 1, 2, 3}
  const float* cb_k;
  const float* cb_v;
  // physical ids of the shared prefix's pages (plan.casc_chunks * kCascPages of them are read) and,
  // per sequence, how many leading pages of its page-table row are those; NULL without a cascade
  const int32_t* prefix_ids;
  const int32_t* shared_pages;
  // fuse != 0: a decode step whose append and query rotation run inside the segment launch (the
  // fp8 pass without codebooks or a cascade); `ap` holds the step's append arguments and
  // seq_lens[b] the new token's position (len_add 1)
  int fuse;
  AppendArgs ap;
};

struct QueryArgs {
  const uint16_t* q;      // bf16 [batch][hq][128]
  const float* u_k;
  int batch, hq, hkv, gqa, n_groups;
  float scale_log2;       // sm_scale * log2(e)
  int8_t* qpack;          // workspace: int8 [batch][hq][2][128] (int8 pass)
  uint8_t* qops;          // workspace: key operands [batch][hkv][tiles][groups][64][32] (fp8)
  int32_t* qscales;       // workspace: their E8M0 row scales [batch][hkv][tiles][groups][64]
  float* qmeta;           // workspace: fp32 [batch][hq][4]: fp8 pass: per-group sums of the
                          // operand's q''; int8 pass: score scale, per-group sums of hi / lo
};

// Key-operand tiles per (sequence, KV head): four query heads per matrix-core tile.
__host__ __device__ inline int key_tiles(int gqa) { return gqa > 4 ? 2 : 1; }

// ---- paged BF16 baseline: every cached token in a BF16 page block of 64 tokens and one KV head
// (keys and values, 32 KiB, in matrix-core operand order: see bf16_decode.hip).
constexpr int kBf16Block = 2 * kPage * kHeadDim * 2;   // 32768

struct Bf16Plan {
  int batch = 0, hq = 0, hkv = 0, gqa = 0;
  int max_pages = 0;         // pages of the longest sequence
  int pages_per_split = 1;   // pages per work item
  int num_splits = 0;        // work items per (sequence, KV head)
  size_t off_ml = 0;         // fp32 [B][Hq][S][2] (m, l), log2 domain
  size_t off_acc = 0;        // fp32 [B][Hq][S][128]
  size_t total = 0;
};

Bf16Plan make_bf16_plan(const oscar_layout& lay, int batch, int max_seq_len);

struct Bf16DecodeArgs {
  const uint8_t* pool;
  const int32_t* page_table;
  int max_pages_per_seq;
  const int32_t* seq_lens;
  const uint16_t* q;
  float sm_scale;
  float* out;
  float* lse;
  uint8_t* workspace;
  int stream_loads;       // non-temporal page loads (one sequence: no page is read twice)
};

struct Bf16StoreArgs {
  uint8_t* pool;
  const int32_t* page_table;
  int max_pages_per_seq;
  int hkv;
  const uint16_t* k_src;
  const uint16_t* v_src;
  int64_t stride_b, stride_t, stride_h;
  const int32_t* start_pos;
  int batch;
  int n_tokens;
};

hipError_t launch_bf16_decode(const Bf16DecodeArgs& a, const Bf16Plan& plan, hipStream_t stream);
hipError_t launch_bf16_store(const Bf16StoreArgs& a, hipStream_t stream);

hipError_t launch_demote(const DemoteArgs& a, hipStream_t stream);
hipError_t launch_probe_read(const void* buf, size_t bytes, uint32_t* sink, int blocks,
                             hipStream_t stream);
hipError_t launch_probe_gather(const void* pool, const int32_t* table, int n_pages, int hkv,
                               int block_bytes, int pages_per_split, int sets, int work, uint32_t* sink,
                               hipStream_t stream);
// Library-owned decode workspace of oscar_decode_step_noalloc (noalloc.hip): one array of this
// many bytes per GPU, its device address looked up once per device.
constexpr size_t kScratchBytes = size_t(16) << 20;
hipError_t scratch_on_current_device(void** ptr);
// One launch for the append items (ap) and the query rows (qa); either may be null.
hipError_t launch_prep(const AppendArgs* ap, const QueryArgs* qa, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, const Plan& plan, uint32_t stages,
                         hipStream_t stream);

}  // namespace oscar
