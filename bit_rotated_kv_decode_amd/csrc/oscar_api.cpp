// C-ABI entry points of liboscar: argument validation (host only, before any HIP call), work
// planning and kernel launches.  See include/oscar.h for the contract of every function.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <unordered_map>
#include <unordered_set>

#include "oscar.h"
#include "oscar_internal.h"

namespace {

thread_local std::string g_last_error;

oscar_status fail(oscar_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

oscar_status ok() {
  g_last_error.clear();
  return OSCAR_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

oscar_status check_layout(const oscar_layout* l) {
  if (l == nullptr) return fail(OSCAR_ERR_NULL, "layout is NULL");
  if (l->head_dim != oscar::kHeadDim)
    return fail(OSCAR_ERR_SHAPE, "head_dim %d unsupported (must be 128)", l->head_dim);
  if (l->group_size != 128 && l->group_size != 64)
    return fail(OSCAR_ERR_SHAPE, "group_size %d unsupported (must be 64 or 128)", l->group_size);
  if (l->num_q_heads <= 0 || l->num_kv_heads <= 0 || l->num_q_heads % l->num_kv_heads != 0)
    return fail(OSCAR_ERR_SHAPE, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                l->num_q_heads, l->num_kv_heads);
  const int gqa = l->num_q_heads / l->num_kv_heads;
  if (gqa != 1 && gqa != 2 && gqa != 4 && gqa != 8)
    return fail(OSCAR_ERR_SHAPE, "query heads per KV head %d unsupported (1, 2, 4 or 8)", gqa);
  if (l->page_tokens != oscar::kPage || l->sink_tokens != oscar::kSink ||
      l->recent_tokens != oscar::kRecent)
    return fail(OSCAR_ERR_SHAPE, "page/sink/recent tokens must be 64/64/256 (got %d/%d/%d)",
                l->page_tokens, l->sink_tokens, l->recent_tokens);
  if (l->num_pages < 0 || l->max_seqs < 0 || l->max_pages_per_seq < 0)
    return fail(OSCAR_ERR_SHAPE, "negative num_pages / max_seqs / max_pages_per_seq");
  if (l->levels_kind != 0 && l->levels_kind != 1)
    return fail(OSCAR_ERR_SHAPE, "levels_kind %d unsupported (0 or 1)", l->levels_kind);
  return OSCAR_OK;
}

// A history encoded with symmetric codebooks (levels_kind 1) needs their levels to encode and
// to decode.
oscar_status check_codebook(const oscar_layout* l, const float* levels_k, const float* levels_v,
                            const char* what) {
  if (l->levels_kind == 1 && (levels_k == nullptr || levels_v == nullptr))
    return fail(OSCAR_ERR_NULL, "%s: levels_kind 1 needs levels_k and levels_v", what);
  return OSCAR_OK;
}

int n_groups(const oscar_layout* l) { return oscar::kHeadDim / l->group_size; }

oscar_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(OSCAR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

namespace oscar {

Plan make_plan(const oscar_layout& lay, int batch, int max_seq_len, int prefix_pages) {
  Plan p;
  p.batch = batch;
  p.hq = lay.num_q_heads;
  p.hkv = lay.num_kv_heads;
  p.gqa = p.hq / p.hkv;
  p.n_groups = kHeadDim / lay.group_size;
  const int64_t n_hist = std::max<int64_t>(0, int64_t{max_seq_len} - kSink - kRecent);
  p.max_pages = static_cast<int>((n_hist + kPage - 1) / kPage);
  // Aim for one round of two blocks per compute unit: a grid that leaves some units a third
  // block finishes when those do.  The INT2 work items share the launch with the BF16 chunk
  // blocks.  At least one page per wave, within the per-item page and per-head item limits.
  const long long slots = kInt2Items;
  const long long bf16_blocks = static_cast<long long>(kBf16Chunks) * batch * p.hkv;
  const long long target = bf16_blocks * 2 <= slots ? slots - bf16_blocks : slots;
  const long long items = static_cast<long long>(p.max_pages) * batch * p.hkv;
  long long pps = std::max<long long>(4, (items + target - 1) / target);
  pps = std::max<long long>(pps, (p.max_pages + kMaxSplits - 1) / kMaxSplits);
  p.pages_per_split = static_cast<int>(std::min<long long>(pps, kMaxPagesPerSplit));
  // The four-head single-group pass takes a wave's pages two at a time, so items get a multiple of
  // eight pages (whole pairs per wave: a pair step costs the same with one page) while the grid
  // keeps three quarters of its blocks.  Then one INT2 block per compute unit (each wave alone on
  // its SIMD) replaces the two per unit when a wave gets at least four pairs that way, or when
  // two per unit leave a wave less than one pair.  Measured on MI355X: 100k tokens, Hkv 8: 56
  // pages per item (224 blocks) 13.6 us against 14.5 us at 32 pages (392 blocks); Hkv 1: 8 pages
  // 7.0 us against 8.8 us at 4; 32k tokens, Hkv 8: 9 pages (456 blocks) 8.8 us against 16 pages
  // (254 blocks) 9.1 us.  A grid that leaves some units two INT2 blocks and others one runs at the
  // slower units' pace (48 pages at 100k: 264 blocks, 16.4 us).  Histories with symmetric codebooks
  // keep the plan above: their pass holds more registers (two value accumulators per tile) and ran
  // slower with one block per unit (100k: 22.9 us at 56 pages against 20.0 us at 27).
  if (int2_fp8_pass(p.gqa, p.n_groups) && lay.levels_kind == 0 && items > 0) {
    const long long up = std::min<long long>(kMaxPagesPerSplit, (p.pages_per_split + 7) / 8 * 8);
    if (4 * ((items + up - 1) / up) >= 3 * std::min(target, (items + p.pages_per_split - 1) /
                                                             p.pages_per_split))
      p.pages_per_split = static_cast<int>(up);
    const long long one = std::min<long long>(
        kMaxPagesPerSplit, ((items + kComputeUnits - 1) / kComputeUnits + 7) / 8 * 8);
    if ((items + one - 1) / one <= kComputeUnits && one >= p.pages_per_split &&
        (one >= 32 || p.pages_per_split < 8))
      p.pages_per_split = static_cast<int>(one);
    // At most kMergeSplits splits per row: the merge takes that many at once and any further ones
    // in rounds of dependent loads.  Measured (one KV head at 100k tokens, decode steps/s): 8
    // pages per item (196 splits) 1,440; 16 pages 1,651; 24 pages (65 splits) 1,660.
    const long long cap = std::min<long long>(
        kMaxPagesPerSplit, ((p.max_pages + kMergeSplits - 1) / kMergeSplits + 7) / 8 * 8);
    if (cap > p.pages_per_split) p.pages_per_split = static_cast<int>(cap);
  }
  p.num_splits = p.max_pages ? (p.max_pages + p.pages_per_split - 1) / p.pages_per_split : 0;
  // whole cascade chunks of the shared prefix (the cascade runs on the four-head single-group pass)
  if (prefix_pages > 0 && int2_fp8_pass(p.gqa, p.n_groups)) {
    p.casc_chunks = std::min(prefix_pages, p.max_pages) / kCascPages;
    p.casc_groups =
        p.casc_chunks ? static_cast<int>((int64_t{batch} + kCascGroup - 1) / kCascGroup) : 0;
  }
  p.slots = p.casc_chunks + p.num_splits;
  auto al = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  const size_t rows = static_cast<size_t>(batch) * p.hq;
  size_t off = 0;
  const size_t ops = static_cast<size_t>(batch) * p.hkv * key_tiles(p.gqa) * p.n_groups;
  // the fused step's flag words first: a plan of up to 64 (sequence, KV head) pairs keeps them
  // in the first 256 bytes, where no other region of any plan lies
  p.off_flags = off;
  off = al(off + static_cast<size_t>(batch) * p.hkv * 4);
  p.off_qrot = off;
  off = al(off + rows * 256);
  p.off_qops = off;
  off = al(off + ops * 64 * 32);
  p.off_qscale = off;
  off = al(off + ops * 64 * 4);
  p.off_sigma = off;
  off = al(off + rows * 4 * 4);
  p.off_int2_ml = off;
  off = al(off + rows * std::max(p.slots, 1) * 2 * 4);
  p.off_int2_acc = off;
  off = al(off + rows * std::max(p.slots, 1) * kHeadDim * 4);
  p.off_bf16_ml = off;
  off = al(off + rows * kBf16Chunks * 2 * 4);
  p.off_bf16_acc = off;
  off = al(off + rows * kBf16Chunks * kHeadDim * 4);
  p.total = off;
  return p;
}

Bf16Plan make_bf16_plan(const oscar_layout& lay, int batch, int max_seq_len) {
  Bf16Plan p;
  p.batch = batch;
  p.hq = lay.num_q_heads;
  p.hkv = lay.num_kv_heads;
  p.gqa = p.hq / p.hkv;
  p.max_pages = static_cast<int>((std::max<int64_t>(0, max_seq_len) + kPage - 1) / kPage);
  // one round of two blocks per compute unit, as for the INT2 pass; at least one page per wave
  const long long items = static_cast<long long>(p.max_pages) * batch * p.hkv;
  long long pps = std::max<long long>(4, (items + kInt2Items - 1) / kInt2Items);
  pps = std::max<long long>(pps, (p.max_pages + kMaxSplits - 1) / kMaxSplits);
  p.pages_per_split = static_cast<int>(std::min<long long>(pps, kMaxPagesPerSplit));
  p.num_splits = p.max_pages ? (p.max_pages + p.pages_per_split - 1) / p.pages_per_split : 0;
  auto al = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  const size_t rows = static_cast<size_t>(batch) * p.hq;
  p.off_ml = 0;
  p.off_acc = al(rows * std::max(p.num_splits, 1) * 2 * 4);
  p.total = al(p.off_acc + rows * std::max(p.num_splits, 1) * kHeadDim * 4);
  return p;
}

}  // namespace oscar

namespace {

oscar_status make_append_args(const oscar_layout* l, void* pool, const int32_t* page_table,
                              void* sink_k, void* sink_v, void* recent_k, void* recent_v,
                              const float* u_k, const float* u_v, const float* clip_k,
                              const float* clip_v, const float* levels_k, const float* levels_v,
                              const void* k_new, const void* v_new, const int32_t* seq_slot,
                              const int32_t* seq_lens, int32_t batch, oscar::AppendArgs& a) {
  oscar_status st = check_layout(l);
  if (st != OSCAR_OK) return st;
  if (batch < 0) return fail(OSCAR_ERR_RANGE, "negative batch");
  if (batch == 0) return ok();
  if (l->max_seqs == 0) return fail(OSCAR_ERR_SHAPE, "layout has no sequence slots");
  if (!pool || !page_table || !sink_k || !sink_v || !recent_k || !recent_v || !u_k || !u_v ||
      !clip_k || !clip_v || !k_new || !v_new || !seq_slot || !seq_lens)
    return fail(OSCAR_ERR_NULL, "append: a required pointer is NULL");
  st = check_codebook(l, levels_k, levels_v, "append");
  if (st != OSCAR_OK) return st;
  if (!aligned(pool, 16) || !aligned(sink_k, 16) || !aligned(sink_v, 16) ||
      !aligned(recent_k, 16) || !aligned(recent_v, 16))
    return fail(OSCAR_ERR_ALIGN, "pool and BF16 segments must be 16-byte aligned");
  if (!aligned(k_new, 2) || !aligned(v_new, 2) || !aligned(u_k, 4) || !aligned(u_v, 4) ||
      !aligned(clip_k, 4) || !aligned(clip_v, 4) || !aligned(levels_k, 4) ||
      !aligned(levels_v, 4) || !aligned(seq_slot, 4) || !aligned(seq_lens, 4) ||
      !aligned(page_table, 4))
    return fail(OSCAR_ERR_ALIGN, "append: misaligned pointer");
  a.pool = static_cast<uint8_t*>(pool);
  a.page_table = page_table;
  a.max_pages_per_seq = l->max_pages_per_seq;
  a.hkv = l->num_kv_heads;
  a.n_groups = n_groups(l);
  a.sink_k = static_cast<uint16_t*>(sink_k);
  a.sink_v = static_cast<uint16_t*>(sink_v);
  a.recent_k = static_cast<uint16_t*>(recent_k);
  a.recent_v = static_cast<uint16_t*>(recent_v);
  a.u_k = u_k;
  a.u_v = u_v;
  a.clip_k = clip_k;
  a.clip_v = clip_v;
  a.levels_k = levels_k;
  a.levels_v = levels_v;
  a.levels_kind = l->levels_kind;
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.seq_slot = seq_slot;
  a.seq_lens = seq_lens;
  a.batch = batch;
  return ok();
}

oscar_status make_decode_args(const oscar_layout* l, const void* pool, const int32_t* page_table,
                              const void* sink_k, const void* sink_v, const void* recent_k,
                              const void* recent_v, const int32_t* seq_slot,
                              const int32_t* seq_lens, const void* q, const float* u_k,
                              const float* u_v, float sm_scale, float* out, float* lse,
                              void* workspace, size_t workspace_bytes, int32_t batch,
                              int32_t max_seq_len, oscar::DecodeArgs& a, oscar::QueryArgs& qa,
                              oscar::Plan& plan, const int32_t* prefix_ids = nullptr,
                              const int32_t* shared_pages = nullptr, int32_t prefix_pages = 0) {
  oscar_status st = check_layout(l);
  if (st != OSCAR_OK) return st;
  if (batch < 0) return fail(OSCAR_ERR_RANGE, "negative batch");
  if (prefix_pages < 0) return fail(OSCAR_ERR_RANGE, "negative prefix_pages");
  if (prefix_pages > 0) {
    if (prefix_ids == nullptr || shared_pages == nullptr)
      return fail(OSCAR_ERR_NULL, "decode: a shared prefix needs prefix_ids and shared_pages");
    if (!aligned(prefix_ids, 4) || !aligned(shared_pages, 4))
      return fail(OSCAR_ERR_ALIGN, "decode: misaligned prefix_ids or shared_pages");
    if (prefix_pages > l->num_pages || prefix_pages > l->max_pages_per_seq)
      return fail(OSCAR_ERR_RANGE, "prefix_pages %d exceeds the pool or the page-table rows",
                  prefix_pages);
    if (l->levels_kind != 0)
      return fail(OSCAR_ERR_SHAPE, "decode: the shared-prefix cascade runs on histories without "
                  "symmetric codebooks (levels_kind 0)");
  }
  if (batch == 0) return ok();
  if (max_seq_len < 1) return fail(OSCAR_ERR_RANGE, "max_seq_len %d < 1", max_seq_len);
  plan = oscar::make_plan(*l, batch, max_seq_len, prefix_pages);
  if (plan.max_pages > l->max_pages_per_seq)
    return fail(OSCAR_ERR_RANGE, "max_seq_len %d needs %d pages > max_pages_per_seq %d",
                max_seq_len, plan.max_pages, l->max_pages_per_seq);
  if (plan.num_splits > oscar::kMaxSplits)
    return fail(OSCAR_ERR_RANGE, "max_seq_len %d needs %d INT2 work items per head > %d",
                max_seq_len, plan.num_splits, oscar::kMaxSplits);
  if ((plan.max_pages > 0 && (!pool || !page_table)) || !sink_k || !sink_v || !recent_k ||
      !recent_v || !seq_slot || !seq_lens || !q || !u_k || !u_v || !out)
    return fail(OSCAR_ERR_NULL, "decode: a required pointer is NULL");
  if (workspace == nullptr || workspace_bytes < plan.total)
    return fail(OSCAR_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes,
                plan.total);
  if (!aligned(workspace, 256)) return fail(OSCAR_ERR_ALIGN, "workspace must be 256-byte aligned");
  if ((pool && !aligned(pool, 16)) || !aligned(sink_k, 16) || !aligned(sink_v, 16) ||
      !aligned(recent_k, 16) || !aligned(recent_v, 16))
    return fail(OSCAR_ERR_ALIGN, "pool and BF16 segments must be 16-byte aligned");
  if (!aligned(q, 4) || !aligned(u_k, 4) || !aligned(u_v, 4) || !aligned(out, 4) ||
      (lse && !aligned(lse, 4)) || !aligned(seq_slot, 4) || !aligned(seq_lens, 4) ||
      (page_table && !aligned(page_table, 4)))
    return fail(OSCAR_ERR_ALIGN, "decode: misaligned pointer");
  a.pool = static_cast<const uint8_t*>(pool);
  a.page_table = page_table;
  a.max_pages_per_seq = l->max_pages_per_seq;
  a.sink_k = static_cast<const uint16_t*>(sink_k);
  a.sink_v = static_cast<const uint16_t*>(sink_v);
  a.recent_k = static_cast<const uint16_t*>(recent_k);
  a.recent_v = static_cast<const uint16_t*>(recent_v);
  a.seq_slot = seq_slot;
  a.seq_lens = seq_lens;
  a.q = static_cast<const uint16_t*>(q);
  a.u_k = u_k;
  a.u_v = u_v;
  a.sm_scale = sm_scale > 0.f ? sm_scale : 0.08838834764831845f;
  a.out = out;
  a.lse = lse;
  a.workspace = static_cast<uint8_t*>(workspace);
  a.len_add = 0;
  a.cb_k = nullptr;
  a.cb_v = nullptr;
  a.prefix_ids = plan.casc_chunks > 0 ? prefix_ids : nullptr;
  a.shared_pages = plan.casc_chunks > 0 ? shared_pages : nullptr;
  a.fuse = 0;
  a.ap = oscar::AppendArgs{};
  qa.q = a.q;
  qa.u_k = u_k;
  qa.batch = batch;
  qa.hq = plan.hq;
  qa.hkv = plan.hkv;
  qa.gqa = plan.gqa;
  qa.n_groups = plan.n_groups;
  qa.scale_log2 = a.sm_scale * 1.4426950408889634f;
  qa.qpack = reinterpret_cast<int8_t*>(a.workspace + plan.off_qrot);
  qa.qops = a.workspace + plan.off_qops;
  qa.qscales = reinterpret_cast<int32_t*>(a.workspace + plan.off_qscale);
  qa.qmeta = reinterpret_cast<float*>(a.workspace + plan.off_sigma);
  return ok();
}

}  // namespace

extern "C" {

uint32_t oscar_abi_version(void) { return OSCAR_ABI_VERSION; }

const char* oscar_status_string(oscar_status s) {
  switch (s) {
    case OSCAR_OK: return "ok";
    case OSCAR_ERR_NULL: return "null pointer";
    case OSCAR_ERR_SHAPE: return "unsupported or inconsistent shape";
    case OSCAR_ERR_ALIGN: return "misaligned pointer or stride";
    case OSCAR_ERR_RANGE: return "value out of range";
    case OSCAR_ERR_WORKSPACE: return "workspace missing or too small";
    case OSCAR_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* oscar_last_error(void) { return g_last_error.c_str(); }

oscar_status oscar_layout_check(const oscar_layout* layout) {
  const oscar_status st = check_layout(layout);
  return st == OSCAR_OK ? ok() : st;
}

size_t oscar_page_block_bytes(const oscar_layout* l) {
  if (check_layout(l) != OSCAR_OK) return 0;
  return static_cast<size_t>(oscar::block_bytes(n_groups(l)));
}

size_t oscar_page_bytes(const oscar_layout* l) {
  if (check_layout(l) != OSCAR_OK) return 0;
  return static_cast<size_t>(oscar::block_bytes(n_groups(l))) * l->num_kv_heads;
}

size_t oscar_pool_bytes(const oscar_layout* l) {
  if (check_layout(l) != OSCAR_OK) return 0;
  return oscar_page_bytes(l) * static_cast<size_t>(l->num_pages);
}

size_t oscar_sink_bytes(const oscar_layout* l) {
  if (check_layout(l) != OSCAR_OK) return 0;
  return static_cast<size_t>(l->max_seqs) * l->num_kv_heads * oscar::kSink * oscar::kHeadDim * 2;
}

size_t oscar_recent_bytes(const oscar_layout* l) {
  if (check_layout(l) != OSCAR_OK) return 0;
  return static_cast<size_t>(l->max_seqs) * l->num_kv_heads * oscar::kRecent * oscar::kHeadDim *
         2;
}

size_t oscar_decode_workspace_bytes(const oscar_layout* l, int32_t batch, int32_t max_seq_len) {
  if (check_layout(l) != OSCAR_OK || batch < 0 || max_seq_len < 0) return 0;
  return oscar::make_plan(*l, batch, max_seq_len).total;
}

int32_t oscar_decode_splits(const oscar_layout* l, int32_t batch, int32_t max_seq_len,
                            int32_t* pages_per_split) {
  if (check_layout(l) != OSCAR_OK || batch < 0 || max_seq_len < 0) return -1;
  const oscar::Plan p = oscar::make_plan(*l, batch, max_seq_len);
  if (pages_per_split != nullptr) *pages_per_split = p.pages_per_split;
  return p.num_splits;
}

oscar_status oscar_check_page_table(const oscar_layout* l, const int32_t* table,
                                    const int32_t* seq_lens, int32_t batch, int32_t extra) {
  oscar_status st = check_layout(l);
  if (st != OSCAR_OK) return st;
  if (batch < 0 || extra < 0) return fail(OSCAR_ERR_RANGE, "negative batch or extra_tokens");
  if (batch > 0 && (table == nullptr || seq_lens == nullptr))
    return fail(OSCAR_ERR_NULL, "page table or seq_lens is NULL");
  // page id -> (sequence, logical page) of its first user
  std::unordered_map<int32_t, std::pair<int32_t, int32_t>> owner;
  std::unordered_set<int32_t> shared;   // page ids used by more than one sequence
  for (int32_t b = 0; b < batch; ++b) {
    const long long len = static_cast<long long>(seq_lens[b]) + extra;
    if (seq_lens[b] < 0) return fail(OSCAR_ERR_RANGE, "seq_lens[%d] = %d < 0", b, seq_lens[b]);
    const long long hist = std::max(0LL, len - oscar::kSink - oscar::kRecent);
    const long long pages = (hist + oscar::kPage - 1) / oscar::kPage;
    if (pages > l->max_pages_per_seq)
      return fail(OSCAR_ERR_RANGE, "sequence %d needs %lld pages > max_pages_per_seq %d", b,
                  pages, l->max_pages_per_seq);
    const int32_t* row = table + static_cast<size_t>(b) * l->max_pages_per_seq;
    for (int32_t p = 0; p < pages; ++p) {
      const int32_t id = row[p];
      if (id < 0 || id >= l->num_pages)
        return fail(OSCAR_ERR_RANGE, "page_table[%d][%d] = %d outside [0, %d)", b, p, id,
                    l->num_pages);
      auto it = owner.find(id);
      if (it == owner.end()) {
        owner.emplace(id, std::make_pair(b, p));
        continue;
      }
      const int32_t ob = it->second.first, op = it->second.second;
      if (ob == b || op != p)
        return fail(OSCAR_ERR_RANGE, "page %d used by (%d,%d) and (%d,%d)", id, ob, op, b, p);
      const int32_t* orow = table + static_cast<size_t>(ob) * l->max_pages_per_seq;
      for (int32_t q = 0; q <= p; ++q)
        if (orow[q] != row[q])
          return fail(OSCAR_ERR_RANGE, "shared page %d of sequences %d and %d is not part of a "
                      "common prefix", id, ob, b);
      shared.insert(id);
    }
  }
  // pages the next extra_tokens decode steps write (history indices [L - 320, L + extra - 320)
  // of each sequence) must belong to that sequence alone: a shared page holds another sequence's
  // tokens, and its copy must be made private (copy-on-write) before the first write
  if (extra > 0) {
    const long long bf16 = oscar::kSink + oscar::kRecent;
    for (int32_t b = 0; b < batch; ++b) {
      const long long first = std::max(0LL, static_cast<long long>(seq_lens[b]) - bf16);
      const long long end = static_cast<long long>(seq_lens[b]) + extra - bf16;   // exclusive
      const int32_t* row = table + static_cast<size_t>(b) * l->max_pages_per_seq;
      if (end <= first) continue;
      for (long long p = first / oscar::kPage; p <= (end - 1) / oscar::kPage; ++p) {
        if (shared.count(row[p]))
          return fail(OSCAR_ERR_RANGE, "sequence %d writes history page %lld (page id %d), "
                      "which other sequences share (give the sequence a private copy first)",
                      b, p, row[p]);
      }
    }
  }
  return ok();
}

oscar_status oscar_demote(const oscar_layout* l, void* pool, const int32_t* page_table,
                          const float* u_k, const float* u_v, const float* clip_k,
                          const float* clip_v, const float* levels_k, const float* levels_v,
                          const void* k_src, const void* v_src,
                          int64_t stride_b, int64_t stride_t, int64_t stride_h,
                          const int32_t* hist_start, int32_t batch, int32_t n_tokens,
                          void* stream) {
  oscar_status st = check_layout(l);
  if (st != OSCAR_OK) return st;
  if (batch < 0 || n_tokens < 0) return fail(OSCAR_ERR_RANGE, "negative batch or n_tokens");
  if (batch == 0 || n_tokens == 0) return ok();
  if (!pool || !page_table || !u_k || !u_v || !clip_k || !clip_v || !k_src || !v_src ||
      !hist_start)
    return fail(OSCAR_ERR_NULL, "oscar_demote: a required pointer is NULL");
  st = check_codebook(l, levels_k, levels_v, "oscar_demote");
  if (st != OSCAR_OK) return st;
  if (stride_b < 0 || stride_t < 0 || stride_h < 0)
    return fail(OSCAR_ERR_RANGE, "negative source stride");
  if (!aligned(pool, 16)) return fail(OSCAR_ERR_ALIGN, "pool must be 16-byte aligned");
  if (!aligned(k_src, 2) || !aligned(v_src, 2) || !aligned(u_k, 4) || !aligned(u_v, 4) ||
      !aligned(clip_k, 4) || !aligned(clip_v, 4) || !aligned(levels_k, 4) ||
      !aligned(levels_v, 4) || !aligned(page_table, 4) || !aligned(hist_start, 4))
    return fail(OSCAR_ERR_ALIGN, "oscar_demote: misaligned pointer");
  oscar::DemoteArgs a;
  a.pool = static_cast<uint8_t*>(pool);
  a.page_table = page_table;
  a.max_pages_per_seq = l->max_pages_per_seq;
  a.hkv = l->num_kv_heads;
  a.n_groups = n_groups(l);
  a.u_k = u_k;
  a.u_v = u_v;
  a.clip_k = clip_k;
  a.clip_v = clip_v;
  a.levels_k = levels_k;
  a.levels_v = levels_v;
  a.levels_kind = l->levels_kind;
  a.k_src = static_cast<const uint16_t*>(k_src);
  a.v_src = static_cast<const uint16_t*>(v_src);
  a.stride_b = stride_b;
  a.stride_t = stride_t;
  a.stride_h = stride_h;
  a.hist_start = hist_start;
  a.batch = batch;
  a.n_tokens = n_tokens;
  return hip_status(oscar::launch_demote(a, static_cast<hipStream_t>(stream)), "oscar_demote");
}

oscar_status oscar_append(const oscar_layout* l, void* pool, const int32_t* page_table,
                          void* sink_k, void* sink_v, void* recent_k, void* recent_v,
                          const float* u_k, const float* u_v, const float* clip_k,
                          const float* clip_v, const float* levels_k, const float* levels_v,
                          const void* k_new, const void* v_new, const int32_t* seq_slot,
                          const int32_t* seq_lens, int32_t batch, void* stream) {
  oscar::AppendArgs a;
  const oscar_status st = make_append_args(l, pool, page_table, sink_k, sink_v, recent_k, recent_v,
                                           u_k, u_v, clip_k, clip_v, levels_k, levels_v,
                                           k_new, v_new, seq_slot, seq_lens, batch, a);
  if (st != OSCAR_OK || batch == 0) return st;
  return hip_status(oscar::launch_prep(&a, nullptr, static_cast<hipStream_t>(stream)),
                    "oscar_append");
}

oscar_status oscar_decode_attn(const oscar_layout* l, const void* pool, const int32_t* page_table,
                               const void* sink_k, const void* sink_v, const void* recent_k,
                               const void* recent_v, const int32_t* seq_slot,
                               const int32_t* seq_lens, const void* q, const float* u_k,
                               const float* u_v, float sm_scale, float* out, float* lse,
                               void* workspace, size_t workspace_bytes, int32_t batch,
                               int32_t max_seq_len, void* stream) {
  return oscar_decode_attn_stages(l, pool, page_table, sink_k, sink_v, recent_k, recent_v,
                                  seq_slot, seq_lens, q, u_k, u_v, sm_scale, out, lse, workspace,
                                  workspace_bytes, batch, max_seq_len, OSCAR_STAGE_ALL, stream);
}

namespace {

// The symmetric-codebook attention runs on the fp8 x FP4 pass only.
oscar_status check_codebook_attention(const oscar_layout* l, const float* levels_k,
                                      const float* levels_v, const char* what) {
  if (l == nullptr || l->levels_kind != 1) return OSCAR_OK;
  oscar_status st = check_codebook(l, levels_k, levels_v, what);
  if (st != OSCAR_OK) return st;
  if (!aligned(levels_k, 4) || !aligned(levels_v, 4))
    return fail(OSCAR_ERR_ALIGN, "%s: misaligned levels", what);
  if (!oscar::int2_fp8_pass(l->num_q_heads / l->num_kv_heads, n_groups(l)))
    return fail(OSCAR_ERR_SHAPE, "%s: codebook attention supports up to 4 query heads per KV head "
                "and group_size 128", what);
  return OSCAR_OK;
}

oscar_status decode_attn_impl(const oscar_layout* l, const void* pool, const int32_t* page_table,
                              const void* sink_k, const void* sink_v, const void* recent_k,
                              const void* recent_v, const int32_t* seq_slot,
                              const int32_t* seq_lens, const void* q, const float* u_k,
                              const float* u_v, const float* cb_k, const float* cb_v,
                              float sm_scale, float* out, float* lse, void* workspace,
                              size_t workspace_bytes, int32_t batch, int32_t max_seq_len,
                              uint32_t stages, void* stream, const int32_t* prefix_ids = nullptr,
                              const int32_t* shared_pages = nullptr, int32_t prefix_pages = 0) {
  if (stages == 0 || (stages & ~OSCAR_STAGE_ALL) != 0)
    return fail(OSCAR_ERR_RANGE, "stage mask 0x%x invalid", stages);
  oscar::DecodeArgs a;
  oscar::QueryArgs qa;
  oscar::Plan plan;
  const oscar_status st = make_decode_args(l, pool, page_table, sink_k, sink_v, recent_k,
                                           recent_v, seq_slot, seq_lens, q, u_k, u_v, sm_scale,
                                           out, lse, workspace, workspace_bytes, batch,
                                           max_seq_len, a, qa, plan, prefix_ids, shared_pages,
                                           prefix_pages);
  if (st != OSCAR_OK || batch == 0) return st;
  a.cb_k = cb_k;
  a.cb_v = cb_v;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (stages & OSCAR_STAGE_QUERY) {
    const hipError_t e = oscar::launch_prep(nullptr, &qa, s);
    if (e != hipSuccess) return hip_status(e, "oscar_decode_attn");
  }
  return hip_status(oscar::launch_decode(a, plan, stages, s), "oscar_decode_attn");
}

}  // namespace

oscar_status oscar_decode_attn_stages(const oscar_layout* l, const void* pool,
                                      const int32_t* page_table, const void* sink_k,
                                      const void* sink_v, const void* recent_k,
                                      const void* recent_v, const int32_t* seq_slot,
                                      const int32_t* seq_lens, const void* q, const float* u_k,
                                      const float* u_v, float sm_scale, float* out, float* lse,
                                      void* workspace, size_t workspace_bytes, int32_t batch,
                                      int32_t max_seq_len, uint32_t stages, void* stream) {
  if (l != nullptr && l->levels_kind == 1)
    return fail(OSCAR_ERR_SHAPE, "oscar_decode_attn: a layout with levels_kind 1 needs the "
                "codebook levels (oscar_decode_attn_codebook)");
  return decode_attn_impl(l, pool, page_table, sink_k, sink_v, recent_k, recent_v, seq_slot,
                          seq_lens, q, u_k, u_v, nullptr, nullptr, sm_scale, out, lse, workspace,
                          workspace_bytes, batch, max_seq_len, stages, stream);
}

oscar_status oscar_decode_attn_codebook(const oscar_layout* l, const void* pool,
                                        const int32_t* page_table, const void* sink_k,
                                        const void* sink_v, const void* recent_k,
                                        const void* recent_v, const int32_t* seq_slot,
                                        const int32_t* seq_lens, const void* q, const float* u_k,
                                        const float* u_v, const float* levels_k,
                                        const float* levels_v, float sm_scale, float* out,
                                        float* lse, void* workspace, size_t workspace_bytes,
                                        int32_t batch, int32_t max_seq_len, uint32_t stages,
                                        void* stream) {
  const oscar_status st =
      check_codebook_attention(l, levels_k, levels_v, "oscar_decode_attn_codebook");
  if (st != OSCAR_OK) return st;
  const bool cb = l != nullptr && l->levels_kind == 1;
  return decode_attn_impl(l, pool, page_table, sink_k, sink_v, recent_k, recent_v, seq_slot,
                          seq_lens, q, u_k, u_v, cb ? levels_k : nullptr, cb ? levels_v : nullptr,
                          sm_scale, out, lse, workspace, workspace_bytes, batch, max_seq_len,
                          stages, stream);
}

namespace {

// Whether a decode step's segment launch appends the token and rotates the query itself: the
// fp8 pass (at most four query heads per KV head, one group) without codebooks or a cascade, when
// its INT2 blocks all run at once (at most one per compute unit) with at least kFusePages pages
// each.  Every such block then repeats the query rotation (about 4.5 us of dependent loads and
// fp64 arithmetic before its pages stream), which pays only where a wave's pages take long enough
// to hide it.  Measured on MI355X (steps/s, fused against three launches): Hkv 8 at 64k tokens
// (256 blocks of 32 pages) 1,328 against 1,294, at 80k (40 pages) 1,275 against 1,228, at 100k
// (224 blocks of 56 pages) 1,283 against 1,232; 100k, Hkv 1 (8 pages) 1,383 against 1,458;
// batch 64 at 8k-128k tokens (4,096 blocks) 71.9 against 76.1; 32k, Hkv 8 (9 pages) 27,921
// against 28,412.
constexpr int kFusePages = 32;

bool step_fused(const oscar::Plan& plan, int levels_kind) {
  return oscar::int2_fp8_pass(plan.gqa, plan.n_groups) && plan.casc_chunks == 0 &&
         levels_kind == 0 && plan.pages_per_split >= kFusePages &&
         static_cast<long long>(plan.batch) * plan.hkv * plan.num_splits <= oscar::kComputeUnits;
}

// The launches of one decode step (those `stages` selects): fused, the segment launch and the
// merge; otherwise the preparation launch (OSCAR_STAGE_QUERY), the segment launch and the merge.
hipError_t launch_step(oscar::DecodeArgs& a, const oscar::QueryArgs& qa,
                       const oscar::AppendArgs& ap, const oscar::Plan& plan, uint32_t stages,
                       hipStream_t s) {
  const uint32_t rest = stages & (OSCAR_STAGE_INT2 | OSCAR_STAGE_BF16 | OSCAR_STAGE_MERGE);
  if (step_fused(plan, ap.levels_kind)) {
    a.fuse = 1;
    a.ap = ap;
  } else if (stages & OSCAR_STAGE_QUERY) {
    const hipError_t e = oscar::launch_prep(&ap, &qa, s);
    if (e != hipSuccess) return e;
  }
  return rest ? oscar::launch_decode(a, plan, rest, s) : hipSuccess;
}

oscar_status decode_step_impl(const oscar_layout* l, void* pool, const int32_t* page_table,
                              void* sink_k, void* sink_v, void* recent_k, void* recent_v,
                              const float* u_k, const float* u_v, const float* clip_k,
                              const float* clip_v, const float* levels_k,
                              const float* levels_v, const void* k_new, const void* v_new,
                              const int32_t* seq_slot, const int32_t* seq_pos, const void* q,
                              float sm_scale, float* out, float* lse, void* workspace,
                              size_t workspace_bytes, int32_t batch, int32_t max_seq_len,
                              void* stream, const int32_t* prefix_ids,
                              const int32_t* shared_pages, int32_t prefix_pages,
                              uint32_t stages = OSCAR_STAGE_ALL) {
  if (stages == 0 || (stages & ~OSCAR_STAGE_ALL) != 0)
    return fail(OSCAR_ERR_RANGE, "oscar_decode_step: stage mask 0x%x invalid", stages);
  oscar::AppendArgs ap;
  oscar_status st = make_append_args(l, pool, page_table, sink_k, sink_v, recent_k, recent_v,
                                     u_k, u_v, clip_k, clip_v, levels_k, levels_v, k_new, v_new,
                                     seq_slot, seq_pos, batch, ap);
  if (st != OSCAR_OK) return st;
  oscar::DecodeArgs a;
  oscar::QueryArgs qa;
  oscar::Plan plan;
  st = make_decode_args(l, pool, page_table, sink_k, sink_v, recent_k, recent_v, seq_slot, seq_pos,
                        q, u_k, u_v, sm_scale, out, lse, workspace, workspace_bytes, batch,
                        max_seq_len, a, qa, plan, prefix_ids, shared_pages, prefix_pages);
  if (st != OSCAR_OK || batch == 0) return st;
  st = check_codebook_attention(l, levels_k, levels_v, "oscar_decode_step");
  if (st != OSCAR_OK) return st;
  if (l->levels_kind == 1) {
    a.cb_k = levels_k;
    a.cb_v = levels_v;
  }
  a.len_add = 1;   // attention sees the appended token
  constexpr uint32_t kSeg = OSCAR_STAGE_INT2 | OSCAR_STAGE_BF16;
  if (step_fused(plan, l->levels_kind) && (stages & kSeg) != 0 && (stages & kSeg) != kSeg)
    return fail(OSCAR_ERR_RANGE, "oscar_decode_step: this step's segment launch also appends; "
                "stages INT2 and BF16 go together (mask 0x%x)", stages);
  return hip_status(launch_step(a, qa, ap, plan, stages, static_cast<hipStream_t>(stream)),
                    "oscar_decode_step");
}

}  // namespace

oscar_status oscar_decode_step(const oscar_layout* l, void* pool, const int32_t* page_table,
                               void* sink_k, void* sink_v, void* recent_k, void* recent_v,
                               const float* u_k, const float* u_v, const float* clip_k,
                               const float* clip_v, const float* levels_k,
                               const float* levels_v, const void* k_new, const void* v_new,
                               const int32_t* seq_slot, const int32_t* seq_pos, const void* q,
                               float sm_scale, float* out, float* lse, void* workspace,
                               size_t workspace_bytes, int32_t batch, int32_t max_seq_len,
                               void* stream) {
  return decode_step_impl(l, pool, page_table, sink_k, sink_v, recent_k, recent_v, u_k, u_v,
                          clip_k, clip_v, levels_k, levels_v, k_new, v_new, seq_slot, seq_pos, q,
                          sm_scale, out, lse, workspace, workspace_bytes, batch, max_seq_len,
                          stream, nullptr, nullptr, 0);
}

int32_t oscar_decode_step_launches(const oscar_layout* l, int32_t batch, int32_t max_seq_len) {
  if (check_layout(l) != OSCAR_OK || batch < 1 || max_seq_len < 1) return 0;
  return step_fused(oscar::make_plan(*l, batch, max_seq_len), l->levels_kind) ? 2 : 3;
}

oscar_status oscar_decode_step_stages(const oscar_layout* l, void* pool,
                                      const int32_t* page_table, void* sink_k, void* sink_v,
                                      void* recent_k, void* recent_v, const float* u_k,
                                      const float* u_v, const float* clip_k, const float* clip_v,
                                      const float* levels_k, const float* levels_v,
                                      const void* k_new, const void* v_new,
                                      const int32_t* seq_slot, const int32_t* seq_pos,
                                      const void* q, float sm_scale, float* out, float* lse,
                                      void* workspace, size_t workspace_bytes, int32_t batch,
                                      int32_t max_seq_len, uint32_t stages, void* stream) {
  return decode_step_impl(l, pool, page_table, sink_k, sink_v, recent_k, recent_v, u_k, u_v,
                          clip_k, clip_v, levels_k, levels_v, k_new, v_new, seq_slot, seq_pos, q,
                          sm_scale, out, lse, workspace, workspace_bytes, batch, max_seq_len,
                          stream, nullptr, nullptr, 0, stages);
}

oscar_status oscar_decode_step_prefix(const oscar_layout* l, void* pool,
                                      const int32_t* page_table, void* sink_k, void* sink_v,
                                      void* recent_k, void* recent_v, const float* u_k,
                                      const float* u_v, const float* clip_k, const float* clip_v,
                                      const void* k_new, const void* v_new,
                                      const int32_t* seq_slot, const int32_t* seq_pos,
                                      const void* q, const int32_t* prefix_ids,
                                      const int32_t* shared_pages, int32_t prefix_pages,
                                      float sm_scale, float* out, float* lse, void* workspace,
                                      size_t workspace_bytes, int32_t batch, int32_t max_seq_len,
                                      void* stream) {
  if (l != nullptr && l->levels_kind != 0)
    return fail(OSCAR_ERR_SHAPE, "oscar_decode_step_prefix: the shared-prefix path takes layouts "
                "with levels_kind 0 only");
  return decode_step_impl(l, pool, page_table, sink_k, sink_v, recent_k, recent_v, u_k, u_v,
                          clip_k, clip_v, nullptr, nullptr, k_new, v_new, seq_slot, seq_pos, q,
                          sm_scale, out, lse, workspace, workspace_bytes, batch, max_seq_len,
                          stream, prefix_ids, shared_pages, prefix_pages);
}

oscar_status oscar_decode_attn_prefix(const oscar_layout* l, const void* pool,
                                      const int32_t* page_table, const void* sink_k,
                                      const void* sink_v, const void* recent_k,
                                      const void* recent_v, const int32_t* seq_slot,
                                      const int32_t* seq_lens, const void* q, const float* u_k,
                                      const float* u_v, const int32_t* prefix_ids,
                                      const int32_t* shared_pages, int32_t prefix_pages,
                                      float sm_scale, float* out, float* lse, void* workspace,
                                      size_t workspace_bytes, int32_t batch, int32_t max_seq_len,
                                      uint32_t stages, void* stream) {
  if (l != nullptr && l->levels_kind != 0)
    return fail(OSCAR_ERR_SHAPE, "oscar_decode_attn_prefix: the shared-prefix path takes layouts "
                "with levels_kind 0 only");
  return decode_attn_impl(l, pool, page_table, sink_k, sink_v, recent_k, recent_v, seq_slot,
                          seq_lens, q, u_k, u_v, nullptr, nullptr, sm_scale, out, lse, workspace,
                          workspace_bytes, batch, max_seq_len, stages, stream, prefix_ids,
                          shared_pages, prefix_pages);
}

size_t oscar_decode_workspace_bytes_prefix(const oscar_layout* l, int32_t batch,
                                           int32_t max_seq_len, int32_t prefix_pages) {
  if (check_layout(l) != OSCAR_OK || batch < 0 || max_seq_len < 0 || prefix_pages < 0) return 0;
  return oscar::make_plan(*l, batch, max_seq_len, prefix_pages).total;
}

oscar_status oscar_check_shared_prefix(const oscar_layout* l, const int32_t* page_table,
                                       int32_t batch, const int32_t* prefix_ids,
                                       const int32_t* shared_pages, int32_t prefix_pages) {
  oscar_status st = check_layout(l);
  if (st != OSCAR_OK) return st;
  if (batch < 0 || prefix_pages < 0 || prefix_pages > l->max_pages_per_seq)
    return fail(OSCAR_ERR_RANGE, "check_shared_prefix: batch %d or prefix_pages %d out of range",
                batch, prefix_pages);
  if ((batch > 0 && (!page_table || !shared_pages)) || (prefix_pages > 0 && !prefix_ids))
    return fail(OSCAR_ERR_NULL, "check_shared_prefix: NULL pointer");
  for (int j = 0; j < prefix_pages; ++j)
    if (prefix_ids[j] < 0 || prefix_ids[j] >= l->num_pages)
      return fail(OSCAR_ERR_RANGE, "prefix page %d has id %d outside [0, %d)", j, prefix_ids[j],
                  l->num_pages);
  for (int b = 0; b < batch; ++b) {
    const int n = shared_pages[b];
    if (n < 0 || n > prefix_pages)
      return fail(OSCAR_ERR_RANGE, "sequence %d: shared_pages %d outside [0, %d]", b, n,
                  prefix_pages);
    const int32_t* row = page_table + static_cast<int64_t>(b) * l->max_pages_per_seq;
    for (int j = 0; j < n; ++j)
      if (row[j] != prefix_ids[j])
        return fail(OSCAR_ERR_SHAPE, "sequence %d: page %d is %d, not the shared prefix's %d", b,
                    j, row[j], prefix_ids[j]);
  }
  return ok();
}

oscar_status oscar_decode_step_noalloc(const oscar_layout* l, void* pool,
                                       const int32_t* page_table, void* sink_k, void* sink_v,
                                       void* recent_k, void* recent_v, const float* u_k,
                                       const float* u_v, const float* clip_k, const float* clip_v,
                                       const float* levels_k, const float* levels_v,
                                       const void* k_new, const void* v_new,
                                       const int32_t* seq_slot, const int32_t* seq_pos,
                                       const void* q, float sm_scale, float* out, float* lse,
                                       int32_t batch, int32_t max_seq_len, void* stream) {
  oscar::AppendArgs ap;
  oscar_status st = make_append_args(l, pool, page_table, sink_k, sink_v, recent_k, recent_v,
                                     u_k, u_v, clip_k, clip_v, levels_k, levels_v, k_new, v_new,
                                     seq_slot, seq_pos, batch, ap);
  if (st != OSCAR_OK) return st;
  st = check_codebook_attention(l, levels_k, levels_v, "oscar_decode_step_noalloc");
  if (st != OSCAR_OK) return st;
  if (batch > 0 && max_seq_len >= 1 && check_layout(l) == OSCAR_OK) {
    const size_t need = oscar::make_plan(*l, batch, max_seq_len).total;
    if (need > oscar::kScratchBytes)
      return fail(OSCAR_ERR_WORKSPACE, "oscar_decode_step_noalloc: %d sequences of up to %d "
                  "tokens need %zu bytes of workspace, more than its %zu-byte scratch array "
                  "(use oscar_decode_step with a caller workspace)", batch, max_seq_len, need,
                  oscar::kScratchBytes);
  }
  // every host check first, against an aligned stand-in of the scratch array's size; the
  // device address is looked up only once they all pass
  oscar::DecodeArgs a;
  oscar::QueryArgs qa;
  oscar::Plan plan;
  st = make_decode_args(l, pool, page_table, sink_k, sink_v, recent_k, recent_v, seq_slot, seq_pos,
                        q, u_k, u_v, sm_scale, out, lse, reinterpret_cast<void*>(uintptr_t{256}),
                        oscar::kScratchBytes, batch, max_seq_len, a, qa, plan);
  if (st != OSCAR_OK || batch == 0) return st;
  void* ws = nullptr;
  hipError_t e = oscar::scratch_on_current_device(&ws);
  if (e != hipSuccess) return hip_status(e, "oscar_decode_step_noalloc: scratch address");
  a.workspace = static_cast<uint8_t*>(ws);
  qa.qpack = reinterpret_cast<int8_t*>(a.workspace + plan.off_qrot);
  qa.qops = a.workspace + plan.off_qops;
  qa.qscales = reinterpret_cast<int32_t*>(a.workspace + plan.off_qscale);
  qa.qmeta = reinterpret_cast<float*>(a.workspace + plan.off_sigma);
  if (l->levels_kind == 1) {
    a.cb_k = levels_k;
    a.cb_v = levels_v;
  }
  a.len_add = 1;   // attention sees the appended token
  return hip_status(launch_step(a, qa, ap, plan, OSCAR_STAGE_ALL,
                                static_cast<hipStream_t>(stream)),
                    "oscar_decode_step_noalloc");
}

size_t oscar_bf16_page_block_bytes(const oscar_layout* l) {
  if (check_layout(l) != OSCAR_OK) return 0;
  return static_cast<size_t>(oscar::kBf16Block);
}

size_t oscar_bf16_page_bytes(const oscar_layout* l) {
  if (check_layout(l) != OSCAR_OK) return 0;
  return static_cast<size_t>(oscar::kBf16Block) * l->num_kv_heads;
}

size_t oscar_bf16_pool_bytes(const oscar_layout* l) {
  if (check_layout(l) != OSCAR_OK) return 0;
  return oscar_bf16_page_bytes(l) * static_cast<size_t>(l->num_pages);
}

size_t oscar_bf16_decode_workspace_bytes(const oscar_layout* l, int32_t batch,
                                         int32_t max_seq_len) {
  if (check_layout(l) != OSCAR_OK || batch < 0 || max_seq_len < 0) return 0;
  return oscar::make_bf16_plan(*l, batch, max_seq_len).total;
}

oscar_status oscar_bf16_store(const oscar_layout* l, void* pool, const int32_t* page_table,
                              const void* k_src, const void* v_src, int64_t stride_b,
                              int64_t stride_t, int64_t stride_h, const int32_t* start_pos,
                              int32_t batch, int32_t n_tokens, void* stream) {
  oscar_status st = check_layout(l);
  if (st != OSCAR_OK) return st;
  if (batch < 0 || n_tokens < 0) return fail(OSCAR_ERR_RANGE, "negative batch or n_tokens");
  if (batch == 0 || n_tokens == 0) return ok();
  if (!pool || !page_table || !k_src || !v_src || !start_pos)
    return fail(OSCAR_ERR_NULL, "oscar_bf16_store: a required pointer is NULL");
  if (stride_b < 0 || stride_t < 0 || stride_h < 0)
    return fail(OSCAR_ERR_RANGE, "negative source stride");
  if (!aligned(pool, 16)) return fail(OSCAR_ERR_ALIGN, "pool must be 16-byte aligned");
  if (!aligned(k_src, 2) || !aligned(v_src, 2) || !aligned(page_table, 4) ||
      !aligned(start_pos, 4))
    return fail(OSCAR_ERR_ALIGN, "oscar_bf16_store: misaligned pointer");
  oscar::Bf16StoreArgs a;
  a.pool = static_cast<uint8_t*>(pool);
  a.page_table = page_table;
  a.max_pages_per_seq = l->max_pages_per_seq;
  a.hkv = l->num_kv_heads;
  a.k_src = static_cast<const uint16_t*>(k_src);
  a.v_src = static_cast<const uint16_t*>(v_src);
  a.stride_b = stride_b;
  a.stride_t = stride_t;
  a.stride_h = stride_h;
  a.start_pos = start_pos;
  a.batch = batch;
  a.n_tokens = n_tokens;
  return hip_status(oscar::launch_bf16_store(a, static_cast<hipStream_t>(stream)),
                    "oscar_bf16_store");
}

oscar_status oscar_bf16_decode_attn(const oscar_layout* l, const void* pool,
                                    const int32_t* page_table, const int32_t* seq_lens,
                                    const void* q, float sm_scale, float* out, float* lse,
                                    void* workspace, size_t workspace_bytes, int32_t batch,
                                    int32_t max_seq_len, void* stream) {
  oscar_status st = check_layout(l);
  if (st != OSCAR_OK) return st;
  if (batch < 0) return fail(OSCAR_ERR_RANGE, "negative batch");
  if (batch == 0) return ok();
  if (max_seq_len < 1) return fail(OSCAR_ERR_RANGE, "max_seq_len %d < 1", max_seq_len);
  const oscar::Bf16Plan plan = oscar::make_bf16_plan(*l, batch, max_seq_len);
  if (plan.max_pages > l->max_pages_per_seq)
    return fail(OSCAR_ERR_RANGE, "max_seq_len %d needs %d pages > max_pages_per_seq %d",
                max_seq_len, plan.max_pages, l->max_pages_per_seq);
  if (plan.num_splits > oscar::kMaxSplits)
    return fail(OSCAR_ERR_RANGE, "max_seq_len %d needs %d work items per head > %d",
                max_seq_len, plan.num_splits, oscar::kMaxSplits);
  if (!pool || !page_table || !seq_lens || !q || !out)
    return fail(OSCAR_ERR_NULL, "oscar_bf16_decode_attn: a required pointer is NULL");
  if (workspace == nullptr || workspace_bytes < plan.total)
    return fail(OSCAR_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes,
                plan.total);
  if (!aligned(workspace, 256)) return fail(OSCAR_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (!aligned(pool, 16) || !aligned(q, 16))
    return fail(OSCAR_ERR_ALIGN, "pool and q must be 16-byte aligned");
  if (!aligned(out, 4) || (lse && !aligned(lse, 4)) || !aligned(seq_lens, 4) ||
      !aligned(page_table, 4))
    return fail(OSCAR_ERR_ALIGN, "oscar_bf16_decode_attn: misaligned pointer");
  oscar::Bf16DecodeArgs a;
  a.pool = static_cast<const uint8_t*>(pool);
  a.page_table = page_table;
  a.max_pages_per_seq = l->max_pages_per_seq;
  a.seq_lens = seq_lens;
  a.q = static_cast<const uint16_t*>(q);
  a.sm_scale = sm_scale > 0.f ? sm_scale : 0.08838834764831845f;
  a.out = out;
  a.lse = lse;
  a.workspace = static_cast<uint8_t*>(workspace);
  a.stream_loads = batch == 1 ? 1 : 0;
  return hip_status(oscar::launch_bf16_decode(a, plan, static_cast<hipStream_t>(stream)),
                    "oscar_bf16_decode_attn");
}

oscar_status oscar_probe_read(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words,
                              int32_t blocks, void* stream) {
  if (buf == nullptr || sink == nullptr) return fail(OSCAR_ERR_NULL, "probe_read: NULL pointer");
  if (!aligned(buf, 16) || bytes % 16 != 0 || !aligned(sink, 4))
    return fail(OSCAR_ERR_ALIGN, "probe_read: buffer and size must be 16-byte aligned");
  if (blocks < 1 || blocks > 65536)
    return fail(OSCAR_ERR_RANGE, "probe_read: blocks %d outside [1, 65536]", blocks);
  if (sink_words < static_cast<size_t>(blocks))
    return fail(OSCAR_ERR_SHAPE, "probe_read: sink of %zu words < %d blocks", sink_words, blocks);
  if (bytes == 0) return ok();
  return hip_status(oscar::launch_probe_read(buf, bytes, sink, blocks,
                                             static_cast<hipStream_t>(stream)),
                    "oscar_probe_read");
}

oscar_status oscar_probe_gather(const oscar_layout* l, const void* pool,
                                const int32_t* page_table_row, int32_t n_pages,
                                int32_t pages_per_split, int32_t sets, int32_t work,
                                uint32_t* sink, size_t sink_words, void* stream) {
  oscar_status st = check_layout(l);
  if (st != OSCAR_OK) return st;
  if (!pool || !page_table_row || !sink) return fail(OSCAR_ERR_NULL, "probe_gather: NULL pointer");
  if (!aligned(pool, 16) || !aligned(page_table_row, 4) || !aligned(sink, 4))
    return fail(OSCAR_ERR_ALIGN, "probe_gather: misaligned pointer");
  if (n_pages < 0 || n_pages > l->num_pages || n_pages > l->max_pages_per_seq)
    return fail(OSCAR_ERR_RANGE, "probe_gather: n_pages %d outside [0, min(num_pages, "
                "max_pages_per_seq)]", n_pages);
  if (pages_per_split < 1 || pages_per_split > oscar::kMaxPagesPerSplit || sets < 1 || sets > 4 ||
      work < 0 || work > (1 << 20))
    return fail(OSCAR_ERR_RANGE, "probe_gather: pages_per_split %d outside [1, %d], sets %d "
                "outside [1, 4] or work %d outside [0, 2^20]", pages_per_split,
                oscar::kMaxPagesPerSplit, sets, work);
  const long long blocks =
      static_cast<long long>((n_pages + pages_per_split - 1) / pages_per_split) * l->num_kv_heads;
  if (blocks > (1LL << 30)) return fail(OSCAR_ERR_RANGE, "probe_gather: grid too large");
  if (sink_words < static_cast<size_t>(4 * blocks))
    return fail(OSCAR_ERR_SHAPE, "probe_gather: sink of %zu words < %lld", sink_words, 4 * blocks);
  if (n_pages == 0) return ok();
  return hip_status(oscar::launch_probe_gather(pool, page_table_row, n_pages, l->num_kv_heads,
                                               oscar::block_bytes(n_groups(l)), pages_per_split,
                                               sets, work, sink,
                                               static_cast<hipStream_t>(stream)),
                    "oscar_probe_gather");
}

}  // extern "C"
