// Decode attention over the three-segment cache (BF16 sink | rotated INT2 history | BF16 recent).
//
// Structure after the OSCAR write-up "超越TurboQuant！OSCAR：面向真实服务的2-bit KV Cache量化",
// section OSCAR 的设计: the INT2 history and the BF16 segments are processed separately and then
// combined with an online-softmax merge.  Launch order on one stream (after the preparation
// launch of encode.hip, which rotates the query and writes it as the fp8 operand of the key
// contraction, q'' = q' * sm_scale * log2(e) in four parts, plus its per-group sums -- or, for a
// decode step on the fp8 pass, with that preparation and the step's append inside attn_kernel:
// see step_prologue and displace_token):
//   1. attn_kernel   both segment passes in one grid:
//                    INT2 blocks: split-KV over history pages on the matrix cores, the codes as
//                    FP4 operands: scores s (q'' . codes) + z sum(q''), a softmax reference per
//                    page pair, values p * s_v (fp8 parts) against the value codes, accumulated
//                    in the rotated frame -> (m, l, acc') partials;
//                    BF16 blocks: 64-token chunks of the BF16 sink and recent ring -> (m, l, acc);
//   2. merge_kernel  log-sum-exp merge of the INT2 partials, un-rotation acc' R_v^T, merge with
//                    the BF16 partials, normalisation.
// Softmax statistics are kept in the log2 domain: scores are scaled by sm_scale * log2(e).
#include "device_common.h"
#include "encode_common.h"
#include "oscar_internal.h"

namespace oscar {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
// Buffer resources: the last descriptor word for raw 32-bit-element access on gfx9-family parts,
// and the cache-policy bit of a non-temporal access.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kNonTemporal = 2;

// ------------------------------------------------------------------------------------------
// 2. INT2 split-KV decode on the matrix cores.
//
// Block = 4 waves on pages [p0, p1) of one (sequence, KV head).  Wave w takes pages
// p0 + w + 4 i in pairs (i = 2 j, 2 j + 1); the next pair's loads are in flight while a pair is
// processed (two register sets used in turn).
//
// Both contractions are v_mfma_scale_f32_16x16x128_f8f6f4 with the stored 2-bit codes as the FP4
// operand B -- a code c zero-extended to a nibble is the E2M1 value c / 2, so a 32-bit word of 16
// codes becomes two operand dwords with one mask and one shift-and-mask -- and an fp8 (e4m3)
// operand A in several parts whose E8M0 row scales restore the magnitudes:
//   keys:   D[(head, part)][token] = sum over 128 channels of the parts of q'' = q' * sm_scale *
//           log2(e) (written by the preparation launch, four parts, about 16 bits) times the key
//           codes of 16 tokens; a lane (g, n) then holds head 4 ht + g of token 16 st + n in its
//           four accumulators (one per part), so the logit is s (d0 + d1 + d2 + d3) + z sum(q'');
//   values: D[(head, part)][channel] = sum over the 128 tokens of a page pair of the parts of
//           x = p * s_v (four parts, about 20 bits, bytes transposed through the wave's own LDS
//           tile) times the value codes; the accumulators sum the parts once, at the end.
// The matrix cores add the products of one contraction with a precision set by its largest
// product: smaller ones are truncated toward zero, so terms of one sign spread over many
// binades come out low.  Every x and code is non-negative; at 100k tokens, where the output is
// a small average of large terms, such a bias shows as up to 1e-3 of the output.  The leading
// parts are therefore integers on fixed grids (products that are multiples of one step sum
// exactly): the query's first part, and x's first two (steps 16 and 1); only small remainders,
// of either sign, go through the floating parts.
// Softmax: each pair takes its own reference, the integer ceil(m_pair) of the head's largest
// logit in the pair, so every p = 2^(logit - m_pair + 8 - e_v) lies in (0, 2^(8 - e_v)] and
// x = p * s_v < 256 (e_v: the pair's largest value scale is below 2^e_v) -- the range of e4m3
// with room for the parts' remainders.  The pair's weight relative to the wave's reference m_ref,
// 2^(m_pair - 8 + e_v - m_ref), is a power of two: it is the value operand's E8M0 row scale and
// one multiply for the sums of p and p * z_v.  m_ref is the first pair's m_pair and moves (with an
// exact power-of-two rescale of the accumulators) only when a later pair's exceeds it by 32.
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef short v2s __attribute__((ext_vector_type(2)));

constexpr uint32_t kNibbles = 0x33333333u;
constexpr int kScaleTwo = 128;          // E8M0 2^1: FP4 holds a 2-bit code c as c / 2
constexpr float kRescaleSpan = 32.0f;   // m_ref moves once a pair's reference passes it by this

__device__ __forceinline__ v4f mfma_f8_f4(const v8i& a, const v8i& b, v4f c, int scale_a) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, scale_a, 0, kScaleTwo);
}
// 32 codes (two words) as an FP4 operand: even codes of w0, odd codes of w0, then of w1
__device__ __forceinline__ v8i fp4_operand(uint32_t w0, uint32_t w1) {
  return v8i{static_cast<int>(w0 & kNibbles), static_cast<int>((w0 >> 2) & kNibbles),
             static_cast<int>(w1 & kNibbles), static_cast<int>((w1 >> 2) & kNibbles), 0, 0, 0, 0};
}
// The high bits (c >> 1) of the same 32 codes, in the same element order, as an FP4 operand
// (a bit b zero-extended to a nibble is the E2M1 value b / 2)
__device__ __forceinline__ v8i fp4_high_bits(uint32_t w0, uint32_t w1) {
  constexpr uint32_t kOnes = 0x11111111u;
  return v8i{static_cast<int>((w0 >> 1) & kOnes), static_cast<int>((w0 >> 3) & kOnes),
             static_cast<int>((w1 >> 1) & kOnes), static_cast<int>((w1 >> 3) & kOnes), 0, 0, 0, 0};
}
__device__ __forceinline__ float lo_half(uint32_t w) {
  return __half2float(__ushort_as_half(static_cast<uint16_t>(w & 0xFFFF)));
}
__device__ __forceinline__ float hi_half(uint32_t w) {
  return __half2float(__ushort_as_half(static_cast<uint16_t>(w >> 16)));
}

// LDS carve-up of an INT2 block: per wave and value operand (tile ht, group g) one fp8 operand
// tile of 64 lanes x 32 bytes, and apart from them the per-wave rows the block combines at the end.
template <int G, int NG>
struct Int2Lds {
  static constexpr int NT = G > 4 ? 2 : 1;                    // head tiles of four heads
  static constexpr int NA = NT * NG;                          // fp8 operands per contraction
  static constexpr int PT = 0;                                // [wave][NA][64][32] bytes
  static constexpr int RED = PT + 4 * NA * 2048;              // [wave][head][ch] fp32
  static constexpr int RED_M = RED + 4 * G * kHeadDim * 4;    // [wave][8] fp32
  static constexpr int RED_L = RED_M + 4 * 8 * 4;
  static constexpr int TOTAL = RED_L + 4 * 8 * 4;
  // cascade blocks: the chunk's kCascPages page blocks of one KV head, staged once for all waves
  static constexpr int STAGE = (TOTAL + 15) & ~15;
  static constexpr int CASC_TOTAL = STAGE + kCascPages * (kMetaOff + kPage * 8 * NG);
  // a decode step's own query rotation (step_prologue), apart from everything the page loop
  // uses: the G query rows (fp32 [G][128]), their rotation partials (fp32 [G][8][128]) and the
  // query operands the block builds: NA tiles, their E8M0 row scales and the per-head sums
  static constexpr int FX = (TOTAL + 15) & ~15;
  static constexpr int FRED = FX + G * kHeadDim * 4;
  static constexpr int FOPS = FRED + G * dev::kRotGroups * kHeadDim * 4;
  static constexpr int FSC = FOPS + NA * 2048;
  static constexpr int FSIG = FSC + NA * 64 * 4;
  static constexpr int FUSED_TOTAL = FSIG + G * 4 * 4;
};

// Whether a page pair may be a wave's last one (a compile-time flag of the pair step).
template <bool B>
struct PairKind {
  static constexpr bool value = B;
};

// ------------------------------------------------------------------------------------------
// A decode step's own preparation inside the segment launch (fp8 pass, one group, no codebooks),
// with the arithmetic of the preparation launch (encode.hip) in the same order, so both give the
// same bytes:
//  - every INT2 split block rotates the G query rows of its KV head and builds their key operands
//    in LDS (step_prologue);
//  - once the new token at position pos >= 320 displaces the ring row of position pos - 256
//    (history index pos - 320, in the history's last page), one BF16 block of that (sequence,
//    KV head), that of chunk kDisplaceChunk, moves the row into its page slot -- rotation,
//    quantiser, store -- gives the ring slot to the new token and then sets the pair's flag to
//    pos + 1 (displace_token);
//  - the one wave that reads that page waits for the flag before it loads its last page pair,
//    and clears it.  The BF16 block has the lower workgroup number, so it is dispatched first and
//    never waits for anything; the wait is bounded all the same, and a wave that gives up poisons
//    its partial (the output turns NaN).
constexpr int kFlagSpins = 1 << 19;   // polls of about 0.2 us each
// The BF16 chunk whose block demotes: the last one.  The launch's workgroups beyond one per
// compute unit (the last INT2 splits, which hold the demoted tokens' pages) share units with the
// first ones, the sink chunks; measured at 100k tokens, Hkv 8, with the sink chunk demoting, the
// demoting blocks and the last splits slowed each other (1.5 us longer preparations).
constexpr int kDisplaceChunk = kBf16Chunks - 1;

// step_prologue: every thread of the block; on return the query operands are in LDS.  U_k's
// slices and the query rows are requested first, `prefetch0` (the first page pair's loads) once
// they have arrived -- issued earlier, the page loads would queue ahead of them at the memory and
// hold up the whole preparation -- and `prefetch1` (the second pair's) once U_k's registers are
// free.  One pass over U_k's slices serves all rows (thread t: the partial sums over rows
// 16 (t / 32) .. + 15 of U for columns 4 (t % 32) .. + 3); wave w then sums the eight partials of
// row w in order and applies the Hadamard transform and the operand split.
template <int G, typename Prefetch0, typename Prefetch1>
__device__ __forceinline__ void step_prologue(const DecodeArgs& a, const Plan& p, int b, int kv,
                                              unsigned char* smem, Prefetch0&& prefetch0,
                                              Prefetch1&& prefetch1) {
  using S = Int2Lds<G, 1>;
  float* xs = reinterpret_cast<float*>(smem + S::FX);
  float (*red)[dev::kRotGroups][kHeadDim] =
      reinterpret_cast<float (*)[dev::kRotGroups][kHeadDim]>(smem + S::FRED);
  const int tid = threadIdx.x;
  constexpr int kQ = (G * kHeadDim + 255) / 256;   // query values per thread
  dev::URows uk;
  dev::load_u_rows(a.u_k + static_cast<int64_t>(kv) * kHeadDim * kHeadDim, uk);
  const uint16_t* qrow = a.q + static_cast<int64_t>(b * p.hq + kv * G) * kHeadDim;
  uint16_t qv[kQ];
#pragma unroll
  for (int j = 0; j < kQ; ++j) qv[j] = tid + 256 * j < G * kHeadDim ? qrow[tid + 256 * j] : 0;
#pragma unroll
  for (int j = 0; j < kQ; ++j)
    if (tid + 256 * j < G * kHeadDim) xs[tid + 256 * j] = dev::bf16_to_f32(qv[j]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < 16; ++k) asm volatile("" ::"v"(uk.v[k].x));
  __builtin_amdgcn_sched_barrier(0);
  prefetch0();
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();   // query rows staged
  const int g = tid >> 5, c = tid & 31;
#pragma unroll
  for (int r = 0; r < G; ++r) {
    float y[4];
    dev::query_partials(xs + r * kHeadDim, uk, y);
#pragma unroll
    for (int e = 0; e < 4; ++e) red[r][g][4 * c + e] = y[e];
  }
  __builtin_amdgcn_sched_barrier(0);
  prefetch1();   // U_k's registers are free again
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  const int wave = tid >> 6;
  if (wave < G) {
    float o0, o1;
    dev::query_finish(red[wave], o0, o1);
    enc::query_operands(o0, o1, 1, G, wave, a.sm_scale * kLog2e, smem + S::FOPS,
                        reinterpret_cast<int32_t*>(smem + S::FSC),
                        reinterpret_cast<float*>(smem + S::FSIG) + 4 * wave);
  }
  __syncthreads();   // the query operands
}

// displace_token: the whole BF16 block of chunk kDisplaceChunk, before its own work, in the
// first 9 KiB of its LDS (every read of them is done when it returns).  Per tensor (K, then V)
// the rotation of the preparation launch's append: the block's fp64 partial sums, wave 0 adding
// them and quantising (one group, the equally spaced levels of levels_kind 0) and storing the
// token.  Wave 0 then makes its stores visible at agent scope before it sets the flag.
__device__ __forceinline__ void displace_token(const DecodeArgs& a, const Plan& p, int b, int kv,
                                               int pos, int64_t slot, unsigned char* lds) {
  const AppendArgs& ap = a.ap;
  int32_t* flag = reinterpret_cast<int32_t*>(a.workspace + p.off_flags) + b * p.hkv + kv;
  // cleared first (the reader waits for this call's value, which is written last)
  if (threadIdx.x == 0) __hip_atomic_store(flag, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  float* x = reinterpret_cast<float*>(lds);                                // [2][128]
  double (*red)[kHeadDim] = reinterpret_cast<double (*)[kHeadDim]>(lds + 2 * kHeadDim * 4);
  const int tid = threadIdx.x;
  constexpr int64_t kU = kHeadDim * kHeadDim;
  dev::URows ur;
  dev::load_u_rows(ap.u_k + kv * kU, ur);
  // thread t < 128: key channel t, else value channel t - 128
  const int tensor = tid >> 7, ch = tid & (kHeadDim - 1);
  uint16_t* ring = (tensor == 0 ? ap.recent_k : ap.recent_v) +
                   ((slot * p.hkv + kv) * kRecent + pos % kRecent) * kHeadDim + ch;
  const uint16_t nw =
      (tensor == 0 ? ap.k_new : ap.v_new)[(static_cast<int64_t>(b) * p.hkv + kv) * kHeadDim + ch];
  x[tensor * kHeadDim + ch] = dev::bf16_to_f32(*ring);
  const int idx = pos - kSink - kRecent;
  uint8_t* blk = enc::page_block(ap.pool, ap.page_table, ap.max_pages_per_seq, b, idx, p.hkv,
                                 kv, block_bytes(1));
  __syncthreads();   // the displaced rows are staged: their ring slot takes the new token
  *ring = nw;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (t == 1) dev::load_u_rows(ap.u_v + kv * kU, ur);
    double r0, r1;
    if (dev::rotate1_block(x + t * kHeadDim, ur, red, r0, r1)) {
      const float* lvp = t == 0 ? ap.levels_k : ap.levels_v;
      const float lv_lo = lvp ? lvp[2 * kv] : 0.0f;
      const float lv_step = lvp ? lvp[2 * kv + 1] : 1.0f;
      const enc::LaneCodes q = enc::quantize_lane(r0, r1, (t == 0 ? ap.clip_k : ap.clip_v)[kv],
                                                  1, lv_lo, lv_step, 0);
      enc::store_token(blk, t, idx % kPage, 1, q);
    }
    __syncthreads();   // wave 0 has read the partials before they are written again
  }
  if ((tid >> 6) == 0) {
    __threadfence();
    if (tid == 0) __hip_atomic_store(flag, pos + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The reader's side: wait (bounded) until the flag of (b, kv) reads pos + 1, then clear it.
// Returns false if it never did.
__device__ __forceinline__ bool wait_displaced(const DecodeArgs& a, const Plan& p, int b, int kv,
                                               int pos) {
  int32_t* flag = reinterpret_cast<int32_t*>(a.workspace + p.off_flags) + b * p.hkv + kv;
  bool seen = false;
  for (int it = 0; it < kFlagSpins && !seen; ++it) {
    seen = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == pos + 1;
    if (!seen) __builtin_amdgcn_s_sleep(8);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if (dev::lane_id() == 0) __hip_atomic_store(flag, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return seen;
}

// STREAM: history pages are fetched with non-temporal loads.  Chosen when the launch holds one
// sequence, so no page is read twice in it; with several sequences pages may be shared (a prefix
// cache), and cached loads let the second reader hit.
// CASC: a cascade block -- chunk `split` of a shared prefix (kCascPages pages of KV head kv, the
// physical ids in a.prefix_ids) for the sequences of group `grp` (kCascGroup of them).  The
// chunk's pages are staged in LDS once; each wave then takes its sequences in turn (those whose
// history wholly holds the chunk), runs the same page-pair arithmetic as a split block against
// the staged pages and writes the sequence's partial for the chunk itself.
// PCASC: the plan has cascade chunks (a split block then skips the pages they took).
// FUSE: a decode step whose preparation the block runs itself (step_prologue); the query operands
// then come from LDS.
template <int G, int NG, bool STREAM, bool CB, bool CASC = false, bool PCASC = CASC,
          bool FUSE = false>
__device__ __forceinline__ void int2_block(const DecodeArgs& a, const Plan& p, int split, int kv,
                                           int grp, unsigned char* smem) {
  static_assert(!FUSE || (NG == 1 && !CB && !CASC && !PCASC), "fp8 pass without extras");
  using S = Int2Lds<G, NG>;
  constexpr int NT = S::NT, NA = S::NA;
  constexpr int BLK = kMetaOff + kPage * 8 * NG;
  float* red_acc = reinterpret_cast<float*>(smem + S::RED);
  float (*red_m)[8] = reinterpret_cast<float (*)[8]>(smem + S::RED_M);
  float (*red_l)[8] = reinterpret_cast<float (*)[8]>(smem + S::RED_L);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = dev::lane_id();
  const int gq = lane >> 4, n = lane & 15;
  int b = grp;                 // the sequence (a cascade block sets it per sequence)
  int head0 = b * p.hq + kv * G;
  // Wave w takes the contiguous pages [w0, w0 + qw) of the item, from wa = max(w0, the pages the
  // cascade took) on.  Its first eight page ids are read with scalar loads, before anything else:
  // they return through the scalar cache, not behind the page streams of the unit's other waves,
  // which a vector load's return would queue after.  Indices stay inside the table row; ids of
  // pages past the sequence's end are read, never used.  A cascade block's pages are the staged
  // chunk: local indices 0 .. kCascPages - 1, all of them history.
  static_assert((kMaxPagesPerSplit + 3) / 4 <= 8 + 64, "eight scalar ids and one per lane");
  int w0 = 0, w1 = kCascPages, wa = 0, n_hist = 1 << 30;
  bool demote = false;   // FUSE: the split holds the page the displaced token goes to
  int owner = -1;        // FUSE: the wave whose pages include it
  int ids[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int more_ids = 0;
  if constexpr (!CASC) {
    const int p0 = split * p.pages_per_split;
    const int qw = (p.pages_per_split + 3) >> 2;
    w0 = p0 + wave * qw;
    const int* trow = a.page_table + static_cast<int64_t>(b) * a.max_pages_per_seq;
    const int tmax = a.max_pages_per_seq - 1;
#pragma unroll
    for (int j = 0; j < 8; ++j) ids[j] = trow[min(w0 + j, tmax)];
    const int L = a.seq_lens[b] + a.len_add;
    // ids of the wave's pages from the ninth on, one per lane, issued ahead of every page load so
    // that waiting for it later never waits for those
    more_ids = trow[min(w0 + 8 + lane, tmax)];
    __builtin_amdgcn_sched_barrier(0);
    // all of the above are issued before the first wait
    asm volatile("" ::"s"(ids[0]), "s"(ids[1]), "s"(ids[2]), "s"(ids[3]), "s"(ids[4]),
                 "s"(ids[5]), "s"(ids[6]), "s"(ids[7]), "s"(L));
    n_hist = max(0, L - kSink - kRecent);
    const int n_pages = (n_hist + kPage - 1) / kPage;
    if (p0 >= n_pages) return;
    const int p1 = min(p0 + p.pages_per_split, n_pages);
    if constexpr (FUSE) {
      demote = p1 == n_pages;
      owner = (n_pages - 1 - p0) / qw;
    }
    // pages of a shared prefix that cascade blocks took for this sequence are not this item's
    int cend = 0;
    if constexpr (PCASC) cend = cascade_pages(p, n_hist, a.shared_pages[b]);
    if (p1 <= cend) return;
    w1 = min(w0 + qw, p1);   // w1 <= w0: a wave without pages (it still combines)
    wa = max(w0, cend);
  }

  // ---- key operands of the query (registers, the same for every page) and, per lane, the sums
  // of q'' of its head in each tile (head 4 ht + gq; a head the group does not have gets -inf
  // logits); loaded after the first pages' loads are issued (see the pair loop)
  int64_t op0 = (static_cast<int64_t>(b) * p.hkv + kv) * NA;
  v8i aq[NA];
  int sq[NA];
  float sig[NT][NG], hbias[NT];
  auto load_query = [&]() {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const uint4* src =
          FUSE ? reinterpret_cast<const uint4*>(smem + S::FOPS + i * 2048 + lane * 32)
               : reinterpret_cast<const uint4*>(a.workspace + p.off_qops + (op0 + i) * 2048 +
                                                lane * 32);
      const uint4 x = src[0], y = src[1];
      aq[i] = v8i{static_cast<int>(x.x), static_cast<int>(x.y), static_cast<int>(x.z),
                  static_cast<int>(x.w), static_cast<int>(y.x), static_cast<int>(y.y),
                  static_cast<int>(y.z), static_cast<int>(y.w)};
      sq[i] = FUSE ? reinterpret_cast<const int32_t*>(smem + S::FSC)[i * 64 + lane]
                   : reinterpret_cast<const int32_t*>(a.workspace +
                                                      p.off_qscale)[(op0 + i) * 64 + lane];
    }
    const float* qmeta = reinterpret_cast<const float*>(a.workspace + p.off_sigma);
#pragma unroll
    for (int ht = 0; ht < NT; ++ht) {
      const int hd = 4 * ht + gq;
      const float* m = FUSE ? reinterpret_cast<const float*>(smem + S::FSIG) + min(hd, G - 1) * 4
                            : qmeta + static_cast<int64_t>(head0 + min(hd, G - 1)) * 4;
#pragma unroll
      for (int g = 0; g < NG; ++g) sig[ht][g] = hd < G ? m[g] : 0.f;
      hbias[ht] = hd < G ? 0.f : -INFINITY;
    }
  };

  // ---- this wave's fp8 operand tiles for the values.  The value codes' K order: in the FP4
  // operand of lane group u, element 8 r + i is the code at position 2 i + (r & 1) of the word of
  // page r >> 1, i.e. token 16 s + 4 u + j with s = i & 3, j = 2 (i >> 2) + (r & 1).  So the fp8
  // operand's four consecutive bytes 16 (u >> 1) + 8 (j & 1) + 4 (j >> 1) + s, s = 0..3, of lane
  // 16 (2 (u & 1) + P) + 4 g + pt (row: head g, part pt) hold part pt of the four sub-tiles of
  // token 4 u + j of page P -- the four logits lane (g, n = 4 u + j) holds: one dword store per
  // (page, part).
  uint8_t* ptile = smem + S::PT + wave * NA * 2048;
  uint8_t* pbase = ptile + (32 * ((n >> 2) & 1) + 4 * gq) * 32 + 16 * (n >> 3) + 8 * (n & 1) +
                   4 * ((n >> 1) & 1);
  // E8M0 row scales of the value operand come from the row's head, whose reference lives in
  // lane group (lane & 15) >> 2
  const int src_lane4 = 4 * 16 * ((lane & 15) >> 2);
  const int row_part = lane & 3;

  // CB: the history's codes name the levels (l0, l1, 3 - l1, 3 - l0) of symmetric codebooks,
  // i.e. a + b c + d (c >> 1): a key's dot product is b q''.c + d q''.(c >> 1) + a sum(q''), a
  // value's weighted sum b x.c + d x.(c >> 1) + a sum(x) -- one more matrix-core contraction of
  // the codes' high bits for each, and a second set of value accumulators (accb).
  float cbk_a = 0.f, cbk_b = 1.f, cbk_d = 0.f, cbv_a = 0.f, cbv_b = 1.f, cbv_d = 0.f;
  if constexpr (CB) {
    const float k0 = a.cb_k[2 * kv], k1 = a.cb_k[2 * kv + 1];
    const float v0 = a.cb_v[2 * kv], v1 = a.cb_v[2 * kv + 1];
    cbk_a = k0;
    cbk_b = k1 - k0;
    cbk_d = 3.f + k0 - 3.f * k1;
    cbv_a = v0;
    cbv_b = v1 - v0;
    cbv_d = 3.f + v0 - 3.f * v1;
  }
  constexpr int NB = CB ? NT : 0;
  float m_ref[NT], l_run[NT], z_run[NT][NG];
  v4f acc[NT][8];
  v4f accb[NB > 0 ? NB : 1][8];
#pragma unroll
  for (int ht = 0; ht < NT; ++ht) {
    m_ref[ht] = -INFINITY;   // a wave without pages leaves -inf (its partial weighs nothing)
    l_run[ht] = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) z_run[ht][g] = 0.f;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[ht][nt] = v4f{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int ht = 0; ht < NB; ++ht)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) accb[ht][nt] = v4f{0.f, 0.f, 0.f, 0.f};
  auto reset_state = [&]() {
#pragma unroll
    for (int ht = 0; ht < NT; ++ht) {
      m_ref[ht] = -INFINITY;
      l_run[ht] = 0.f;
#pragma unroll
      for (int g = 0; g < NG; ++g) z_run[ht][g] = 0.f;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) acc[ht][nt] = v4f{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ht = 0; ht < NB; ++ht)
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) accb[ht][nt] = v4f{0.f, 0.f, 0.f, 0.f};
  };

  // One page's operands, fetched with 16-byte loads from the tiled block (one chunk row = 64 lanes
  // x 16 bytes): key chunk row j holds this lane's words of sub-tiles 2j and 2j + 1, value chunk
  // row j those of channel tiles 4j .. 4j + 3; m[st]: the meta of token 16 st + n, the token whose
  // logits the lane holds in sub-tile st (key groups, then value groups; the four lanes of one n
  // read the same bytes).
  struct PageRegs {
    uint4 k[2];
    uint4 v[2];
    uint32_t m[4][2 * NG];
  };
  auto kword = [](const PageRegs& r, int st, int hf) {
    const uint4& c = r.k[st >> 1];
    const int e = ((st & 1) << 1) + hf;
    return e == 0 ? c.x : e == 1 ? c.y : e == 2 ? c.z : c.w;
  };
  auto vword = [](const PageRegs& r, int nt) {
    const uint4& c = r.v[nt >> 2];
    const int e = nt & 3;
    return e == 0 ? c.x : e == 1 ? c.y : e == 2 ? c.z : c.w;
  };
  // the first eight ids in lanes 0..7 of one register (no memory wait: written from the scalars)
  int first_ids = ids[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) first_ids = lane == j ? ids[j] : first_ids;
  auto page_id = [&](int pg) {
    const int j = pg - w0;
    if (j < 8) return __builtin_amdgcn_readlane(first_ids, j);
    return __builtin_amdgcn_readlane(more_ids, j - 8);
  };
  // Buffer loads over the page's block: the block address in scalar registers, the lane's
  // offsets in loop-invariant registers.  A slot past the wave's pages (a clamped prefetch index)
  // gets a zero-length range, so its loads return zeros without touching memory and every round
  // still issues the same loads.
  auto load_page = [&](int pg, PageRegs& r) {
    if constexpr (CASC) {
      const uint8_t* blk = smem + S::STAGE + pg * BLK;
      r.k[0] = *reinterpret_cast<const uint4*>(blk + kKCodesOff + lane * 16);
      r.k[1] = *reinterpret_cast<const uint4*>(blk + kKCodesOff + 1024 + lane * 16);
      r.v[0] = *reinterpret_cast<const uint4*>(blk + kVCodesOff + lane * 16);
      r.v[1] = *reinterpret_cast<const uint4*>(blk + kVCodesOff + 1024 + lane * 16);
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int w = 0; w < 2 * NG; ++w)
          r.m[st][w] = reinterpret_cast<const uint32_t*>(blk + kMetaOff + n * 8 * NG +
                                                         st * 16 * 8 * NG)[w];
      return;
    }
    const int pid = page_id(min(pg, w1 - 1));
    const uint8_t* blk = a.pool + (static_cast<int64_t>(pid) * p.hkv + kv) * BLK;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(blk), 0, pg < w1 ? BLK : 0, kBufferWord3);
    const int cp = STREAM ? kNonTemporal : 0;
    r.k[0] = dev::to_uint4(__builtin_amdgcn_raw_buffer_load_b128(rs, kKCodesOff + lane * 16, 0, cp));
    r.k[1] = dev::to_uint4(
        __builtin_amdgcn_raw_buffer_load_b128(rs, kKCodesOff + 1024 + lane * 16, 0, cp));
    r.v[0] = dev::to_uint4(__builtin_amdgcn_raw_buffer_load_b128(rs, kVCodesOff + lane * 16, 0, cp));
    r.v[1] = dev::to_uint4(
        __builtin_amdgcn_raw_buffer_load_b128(rs, kVCodesOff + 1024 + lane * 16, 0, cp));
    const int moff = kMetaOff + n * 8 * NG;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      if constexpr (NG == 1) {
        const uint2 w = dev::to_uint2(
            __builtin_amdgcn_raw_buffer_load_b64(rs, moff + st * 16 * 8 * NG, 0, cp));
        r.m[st][0] = w.x;
        r.m[st][1] = w.y;
      } else {
        const uint4 w = dev::to_uint4(
            __builtin_amdgcn_raw_buffer_load_b128(rs, moff + st * 16 * 8 * NG, 0, cp));
        r.m[st][0] = w.x;
        r.m[st][1] = w.y;
        r.m[st][2] = w.z;
        r.m[st][3] = w.w;
      }
    }
  };
  // pair q: pages wa + 2 q and wa + 2 q + 1
  auto load_pair = [&](int q, PageRegs* rr) {
    load_page(wa + 2 * q, rr[0]);
    load_page(wa + 2 * q + 1, rr[1]);
  };

  // ---- one pair of pages.  `last` (a PairKind): only a wave's last pair can hold a slot past
  // the history or a page past the wave's range, so only that pair carries the checks.
  auto process_pair = [&](int q, PageRegs* rr, bool first, auto last) {
    const int pgs[2] = {wa + 2 * q, wa + 2 * q + 1};
    // a slot past the history (or a page past the wave's range) holds arbitrary bytes: its meta
    // becomes zero (no value contribution, finite products) and its logit -inf
    const bool tail = decltype(last)::value && (pgs[1] >= w1 || (pgs[1] + 1) * kPage > n_hist);
    if (tail) {
#pragma unroll
      for (int P = 0; P < 2; ++P)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const bool ok = pgs[P] < w1 && pgs[P] * kPage + 16 * st + n < n_hist;
#pragma unroll
          for (int w = 0; w < 2 * NG; ++w) rr[P].m[st][w] = ok ? rr[P].m[st][w] : 0u;
        }
    }
    // meta of token 16 st + n of page P
    uint32_t km[2][NG][4], vm[2][NG][4];
#pragma unroll
    for (int P = 0; P < 2; ++P)
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          km[P][g][st] = rr[P].m[st][g];
          vm[P][g][st] = rr[P].m[st][NG + g];
        }
    // the pair's largest value scale (positive fp16 bits order like their values): over the
    // lane's 8 tokens, then over the 16 lanes of its row (each row holds all 128 tokens)
    uint32_t smax = 0;
#pragma unroll
    for (int P = 0; P < 2; ++P)
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int st = 0; st < 4; ++st) smax = max(smax, vm[P][g][st] & 0xFFFFu);
    smax = max(smax, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(smax), 0xB1, 0xF, 0xF, 0)));
    smax = max(smax, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(smax), 0x4E, 0xF, 0xF, 0)));
    smax = max(smax, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(smax), 0x124, 0xF, 0xF, 0)));
    smax = max(smax, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(smax), 0x128, 0xF, 0xF, 0)));
    int ev = 0;
    if (smax != 0) frexpf(__half2float(__ushort_as_half(static_cast<uint16_t>(smax))), &ev);

    // ---- logits of head 4 ht + gq for token 16 st + n of page P
    float lg[NT][2][4];
    // without codebooks, a page's four sub-tile contractions are issued back to back (four
    // independent results) before their sums are read
    v4f dk[4][NT * NG];
#pragma unroll
    for (int P = 0; P < 2; ++P) {
      if constexpr (!CB) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const v8i bk = fp4_operand(kword(rr[P], st, 0), kword(rr[P], st, 1));
#pragma unroll
          for (int i = 0; i < NT * NG; ++i)
            dk[st][i] = mfma_f8_f4(aq[i], bk, v4f{0.f, 0.f, 0.f, 0.f}, sq[i]);
        }
      }
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const uint32_t kw0 = kword(rr[P], st, 0), kw1 = kword(rr[P], st, 1);
        float sc[NT][NG];
#pragma unroll
        for (int ht = 0; ht < NT; ++ht)
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            v4f d;
            if constexpr (CB)
              d = mfma_f8_f4(aq[ht * NG + g], fp4_operand(kw0, kw1), v4f{0.f, 0.f, 0.f, 0.f},
                             sq[ht * NG + g]);
            else
              d = dk[st][ht * NG + g];
            sc[ht][g] = (d[0] + d[1]) + (d[2] + d[3]);
          }
        if constexpr (CB) {
          const v8i bh = fp4_high_bits(kw0, kw1);
#pragma unroll
          for (int ht = 0; ht < NT; ++ht)
#pragma unroll
            for (int g = 0; g < NG; ++g) {
              const v4f d =
                  mfma_f8_f4(aq[ht * NG + g], bh, v4f{0.f, 0.f, 0.f, 0.f}, sq[ht * NG + g]);
              sc[ht][g] = fmaf(cbk_d, (d[0] + d[1]) + (d[2] + d[3]), cbk_b * sc[ht][g]);
            }
        }
#pragma unroll
        for (int ht = 0; ht < NT; ++ht) {
          float t = hbias[ht];
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            const float ks = lo_half(km[P][g][st]);
            const float kz = CB ? fmaf(cbk_a, ks, hi_half(km[P][g][st])) : hi_half(km[P][g][st]);
            t = fmaf(kz, sig[ht][g], t);
            t = fmaf(ks, sc[ht][g], t);
          }
          lg[ht][P][st] = t;
        }
      }
    }
    if (tail) {
#pragma unroll
      for (int P = 0; P < 2; ++P)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const bool ok = pgs[P] < w1 && pgs[P] * kPage + 16 * st + n < n_hist;
#pragma unroll
          for (int ht = 0; ht < NT; ++ht) lg[ht][P][st] = ok ? lg[ht][P][st] : -INFINITY;
        }
    }
    // ---- the pair's reference per head, and the wave's
    float mp[NT];
#pragma unroll
    for (int ht = 0; ht < NT; ++ht) {
      float v = lg[ht][0][0];
#pragma unroll
      for (int P = 0; P < 2; ++P)
#pragma unroll
        for (int st = 0; st < 4; ++st) v = fmaxf(v, lg[ht][P][st]);
      v = dev::row16_max(v);
      mp[ht] = v == -INFINITY ? 0.f : ceilf(v);   // -inf: a head the group does not have
      if (first) m_ref[ht] = mp[ht];
    }
    if (!first) {
      bool up = false;
#pragma unroll
      for (int ht = 0; ht < NT; ++ht) up |= mp[ht] > m_ref[ht] + kRescaleSpan;
      if (__builtin_amdgcn_ballot_w64(up) != 0) {
#pragma unroll
        for (int ht = 0; ht < NT; ++ht) {
          const float d = mp[ht] > m_ref[ht] + kRescaleSpan ? m_ref[ht] - mp[ht] : 0.f;
          const int di = static_cast<int>(d);
          l_run[ht] = ldexpf(l_run[ht], di);
#pragma unroll
          for (int g = 0; g < NG; ++g) z_run[ht][g] = ldexpf(z_run[ht][g], di);
#pragma unroll
          for (int nt = 0; nt < 8; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[ht][nt][i] = ldexpf(acc[ht][nt][i], di);
          if constexpr (CB) {
#pragma unroll
            for (int nt = 0; nt < 8; ++nt)
#pragma unroll
              for (int i = 0; i < 4; ++i) accb[ht][nt][i] = ldexpf(accb[ht][nt][i], di);
          }
          if (mp[ht] > m_ref[ht] + kRescaleSpan) m_ref[ht] = mp[ht];
        }
      }
    }
    // ---- probabilities against the pair's reference, sums, the value operand parts
    int sv[NT];
#pragma unroll
    for (int ht = 0; ht < NT; ++ht) {
      const float nb = 8.f - static_cast<float>(ev) - mp[ht];
      const int dexp = static_cast<int>(mp[ht] - m_ref[ht]) - 8 + ev;   // pair weight 2^dexp
      const float wgt = ldexpf(1.f, dexp);
      float lp = 0.f, zp[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) zp[g] = 0.f;
      float x[NG][2][4];
#pragma unroll
      for (int P = 0; P < 2; ++P)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const float pr = __builtin_amdgcn_exp2f(lg[ht][P][st] + nb);   // 0 for -inf
          lp += pr;
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            const float vs = lo_half(vm[P][g][st]);
            const float vz = CB ? fmaf(cbv_a, vs, hi_half(vm[P][g][st])) : hi_half(vm[P][g][st]);
            zp[g] = fmaf(pr, vz, zp[g]);
            x[g][P][st] = pr * vs;
          }
        }
      l_run[ht] = fmaf(lp, wgt, l_run[ht]);
#pragma unroll
      for (int g = 0; g < NG; ++g) z_run[ht][g] = fmaf(zp[g], wgt, z_run[ht][g]);
      // parts of x, bytes to the tile: part 0 the integer i0 = rint(x / 16) in [0, 16], part 1 the
      // integer i1 = rint(x - 16 i0) in [-8, 8] (rows of multiples of one step, which the matrix
      // cores sum exactly), parts 2 and 3 e4m3 values of the remainder (|r| <= 1/2) scaled by 16
      // and 256 in the conversion.  The matrix cores truncate the small products of a sum whose
      // terms span many binades, and p of a token far below its pair's maximum is tiny: kept in
      // an e4m3 part of up to 8, such positive terms biased every value sum low (up to 1e-3 of
      // the output at 100k tokens); below 1/2 the bias is sixteen times smaller.
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        uint8_t* tb = pbase + (ht * NG + g) * 2048;
#pragma unroll
        for (int P = 0; P < 2; ++P) {
          float r[4];
#pragma unroll
          for (int st = 0; st < 4; ++st) r[st] = x[g][P][st];
#pragma unroll
          for (int pt = 0; pt < 4; ++pt) {
            float in[4];
            if (pt == 0) {
#pragma unroll
              for (int st = 0; st < 4; ++st) {
                in[st] = rintf(r[st] * 0.0625f);
                r[st] = fmaf(in[st], -16.f, r[st]);
              }
            } else if (pt == 1) {
#pragma unroll
              for (int st = 0; st < 4; ++st) {
                in[st] = rintf(r[st]);
                r[st] -= in[st];
              }
            } else {
#pragma unroll
              for (int st = 0; st < 4; ++st) in[st] = r[st];
            }
            const float div = pt <= 1 ? 1.f : pt == 2 ? 0.0625f : 0.00390625f;
            // both halves of the dword are written: the first conversion's other half may be any
            v2s w00;
            w00 = __builtin_nondeterministic_value(w00);
            v2s w01 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w00, in[0], in[1], div, false);
            const v2s w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w01, in[2], in[3], div, true);
            uint32_t pk;
            __builtin_memcpy(&pk, &w, 4);
            *reinterpret_cast<uint32_t*>(tb + P * 512 + pt * 32) = pk;   // bytes: st 0..3
            if (pt == 2) {
              const v2f b01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(static_cast<int>(pk), div, false);
              const v2f b23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(static_cast<int>(pk), div, true);
              r[0] -= b01[0];
              r[1] -= b01[1];
              r[2] -= b23[0];
              r[3] -= b23[1];
            }
          }
        }
      }
      // row scale of this lane's value-operand row (head (lane & 15) >> 2, part lane & 3)
      const int rd = __builtin_amdgcn_ds_bpermute(src_lane4, dexp);
      sv[ht] = min(max(127 + rd + (row_part == 0 ? 4 : 4 - 4 * row_part), 0), 254);
    }
    // LDS operations of one wave execute in order, so the reads below see the writes above
    __builtin_amdgcn_wave_barrier();
    v8i pa[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const uint4* src = reinterpret_cast<const uint4*>(ptile + i * 2048 + lane * 32);
      const uint4 x0 = src[0], x1 = src[1];
      pa[i] = v8i{static_cast<int>(x0.x), static_cast<int>(x0.y), static_cast<int>(x0.z),
                  static_cast<int>(x0.w), static_cast<int>(x1.x), static_cast<int>(x1.y),
                  static_cast<int>(x1.z), static_cast<int>(x1.w)};
    }
    // ---- values: channel tile nt of both pages against the pair's probability parts
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const uint32_t vw0 = vword(rr[0], nt), vw1 = vword(rr[1], nt);
      const v8i bv = fp4_operand(vw0, vw1);
      const int g = NG == 2 ? nt / 4 : 0;
#pragma unroll
      for (int ht = 0; ht < NT; ++ht)
        acc[ht][nt] = mfma_f8_f4(pa[ht * NG + g], bv, acc[ht][nt], sv[ht]);
      if constexpr (CB) {
        const v8i bh = fp4_high_bits(vw0, vw1);
#pragma unroll
        for (int ht = 0; ht < NB; ++ht)
          accb[ht][nt] = mfma_f8_f4(pa[ht * NG + g], bh, accb[ht][nt], sv[ht]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  // Pairs of this wave: pages wa + 2 q and + 1.  Two register sets used in turn: while one pair
  // is processed, the next pair's loads are in flight.  Every load of a round is issued whether
  // or not its page is the wave's (slots past the wave's pages read nothing), so the wait before
  // a pair never covers a later one's.  The query operands are loaded between the first two
  // pairs' loads: the first pair waits on them and on its own pages only.
  const int npairs = w1 > wa ? (w1 - wa + 1) / 2 : 0;
  // FUSE: the wave that reads the displaced token's page takes its last pair after the loop,
  // once the token is there (the same pairs as without FUSE, so the same arithmetic)
  const bool last_apart = FUSE && demote && wave == owner;
  const int nl = last_apart ? npairs - 1 : npairs;   // pairs of the loop
  // pairs before a wave's last one skip the checks
  using Inner = PairKind<false>;
  // Issue priority by the pairs a wave has left: two blocks share a compute unit, and the arbiter
  // otherwise favours the older one throughout, so the younger one would end its pages alone.
  auto set_prio = [&](int q) {
    const int rem = nl - q;
    if (rem >= 3)
      __builtin_amdgcn_s_setprio(3);
    else if (rem >= 2)
      __builtin_amdgcn_s_setprio(2);
    else
      __builtin_amdgcn_s_setprio(1);
  };
  float* ml = reinterpret_cast<float*>(a.workspace + p.off_int2_ml);
  float* pacc = reinterpret_cast<float*>(a.workspace + p.off_int2_acc);
  if constexpr (CASC) {
    // stage the chunk's page blocks of this KV head (cached loads: the other groups' blocks read
    // the same pages)
    constexpr int kChunks16 = BLK / 16;
    for (int i = threadIdx.x; i < kCascPages * kChunks16; i += 256) {
      const int pg = i / kChunks16, o = i - pg * kChunks16;
      const int pid = a.prefix_ids[split * kCascPages + pg];
      reinterpret_cast<uint4*>(smem + S::STAGE + pg * BLK)[o] = reinterpret_cast<const uint4*>(
          a.pool + (static_cast<int64_t>(pid) * p.hkv + kv) * BLK)[o];
    }
    __syncthreads();
    // wave w: sequences grp * kCascGroup + w + 4 i of the group for which the chunk is one of the
    // cascade's (the chunk lies in their full history pages and their shared pages); each one's
    // partial goes to slot `split` (the chunk) of its rows
    for (int i = 0; i < kCascGroup / 4; ++i) {
      b = grp * kCascGroup + wave + 4 * i;
      if (b >= p.batch) break;
      const int nh = max(0, a.seq_lens[b] + a.len_add - kSink - kRecent);
      if (cascade_pages(p, nh, a.shared_pages[b]) < (split + 1) * kCascPages) continue;
      head0 = b * p.hq + kv * G;
      op0 = (static_cast<int64_t>(b) * p.hkv + kv) * NA;
      reset_state();
      load_query();
      for (int q = 0; q < kCascPages / 2; ++q) {
        PageRegs rr[2];
        load_pair(q, rr);
        process_pair(q, rr, q == 0, PairKind<false>{});   // staged pages: all history
      }
#pragma unroll
      for (int ht = 0; ht < NT; ++ht) {
        const int hd = 4 * ht + gq;
        const float l = dev::row16_sum(l_run[ht]);
        float zs[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) zs[g] = dev::row16_sum(z_run[ht][g]);
        if (hd < G) {
          const int64_t prow = static_cast<int64_t>(head0 + hd) * p.slots + split;
#pragma unroll
          for (int nt = 0; nt < 8; ++nt) {
            float v = (acc[ht][nt][0] + acc[ht][nt][1]) + (acc[ht][nt][2] + acc[ht][nt][3]);
            if constexpr (CB) {
              const float h =
                  (accb[ht][nt][0] + accb[ht][nt][1]) + (accb[ht][nt][2] + accb[ht][nt][3]);
              v = fmaf(cbv_d, h, cbv_b * v);
            }
            pacc[prow * kHeadDim + 16 * nt + n] = v + zs[NG == 2 ? nt / 4 : 0];
          }
          if (n == 0) reinterpret_cast<float2*>(ml)[prow] = make_float2(m_ref[ht], l);
        }
      }
    }
    return;
  }
  PageRegs r0[2], r1[2];
  // FUSE: the first pair's loads are in flight during the query rotation
  if constexpr (FUSE) step_prologue<G>(a, p, b, kv, smem, [&]() {
      if (nl > 0) load_pair(0, r0);
    }, [&]() {
      if (nl > 1) load_pair(1, r1);
    });
  if (nl > 0) {
    set_prio(0);
    if (!FUSE) load_pair(0, r0);
    __builtin_amdgcn_sched_barrier(0);
    load_query();
    __builtin_amdgcn_sched_barrier(0);
    if (!FUSE) load_pair(1, r1);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (CB) {
      // one pair step with the checks throughout (the codebook pass's registers are at the
      // limit; more inlined steps spill)
      process_pair(0, r0, true, PairKind<true>{});
      int q = 1, rest = npairs - 1;
      for (; rest >= 2; rest -= 2) {
        set_prio(q);
        load_pair(q + 1, r0);
        process_pair(q, r1, false, PairKind<true>{});
        ++q;
        __builtin_amdgcn_sched_barrier(0);
        set_prio(q);
        load_pair(q + 1, r1);
        process_pair(q, r0, false, PairKind<true>{});
        ++q;
        __builtin_amdgcn_sched_barrier(0);
      }
      if (rest == 1) {
        set_prio(q);
        process_pair(q, r1, false, PairKind<true>{});
      }
    } else {
    if (nl == 1)
      process_pair(0, r0, true, PairKind<true>{});
    else
      process_pair(0, r0, true, Inner{});
    int q = 1, rest = nl - 1;
    // rounds of two pairs while a later pair remains; the wave's last pair (the only one with
    // checks) in the round or single pair after the loop
    for (; rest >= 3; rest -= 2) {
      set_prio(q);
      load_pair(q + 1, r0);
      process_pair(q, r1, false, Inner{});
      ++q;
      __builtin_amdgcn_sched_barrier(0);
      set_prio(q);
      load_pair(q + 1, r1);
      process_pair(q, r0, false, Inner{});
      ++q;
      __builtin_amdgcn_sched_barrier(0);
    }
    if (rest == 2) {
      set_prio(q);
      load_pair(q + 1, r0);
      process_pair(q, r1, false, Inner{});
      ++q;
      __builtin_amdgcn_sched_barrier(0);
      set_prio(q);
      process_pair(q, r0, false, PairKind<true>{});
    } else if (rest == 1) {
      set_prio(q);
      process_pair(q, r1, false, PairKind<true>{});
    }
    }
    __builtin_amdgcn_s_setprio(0);
  }
  if constexpr (FUSE) {
    if (last_apart) {
      // the displaced token's page is read once the demoting BF16 block has stored the token
      const bool ok = wait_displaced(a, p, b, kv, n_hist + kSink + kRecent - 1);
      if (nl == 0) load_query();
      PageRegs rr[2];
      load_pair(nl, rr);
      process_pair(nl, rr, nl == 0, PairKind<true>{});
#pragma unroll
      for (int ht = 0; ht < NT; ++ht) l_run[ht] = ok ? l_run[ht] : NAN;
    }
  }

  // ---- finish the wave: l and z summed over the 16 lanes of each head; each accumulator row as
  // the sum of its parts plus z; rows to the wave's own LDS rows [wave][head][ch], apart from
  // every operand tile, so a single barrier orders them before the combine.
#pragma unroll
  for (int ht = 0; ht < NT; ++ht) {
    const int hd = 4 * ht + gq;
    const float l = dev::row16_sum(l_run[ht]);
    float zs[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) zs[g] = dev::row16_sum(z_run[ht][g]);
    if (hd < G) {
      if (n == 0) {
        red_m[wave][hd] = m_ref[ht];
        red_l[wave][hd] = l;
      }
      float* red_w = red_acc + (wave * G + hd) * kHeadDim;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        float v = (acc[ht][nt][0] + acc[ht][nt][1]) + (acc[ht][nt][2] + acc[ht][nt][3]);
        if constexpr (CB) {
          const float h = (accb[ht][nt][0] + accb[ht][nt][1]) + (accb[ht][nt][2] + accb[ht][nt][3]);
          v = fmaf(cbv_d, h, cbv_b * v);
        }
        red_w[16 * nt + n] = v + zs[NG == 2 ? nt / 4 : 0];
      }
    }
  }
  __syncthreads();
  // ---- combine the 4 waves and write this split's partial:
  // acc'[h][ch] = sum_w f_w acc_w[h][ch] with f_w = 2^(m_w - m).  Every wave has written its rows
  // (a wave without pages: m = -inf, l = 0, zero rows, so f_w = 0), and every LDS read below is
  // issued before the first one is used.
  // thread i: head i / 32, channels 4 (i % 32) .. 4 (i % 32) + 3 (one 16-byte store)
  static_assert(G * kHeadDim / 4 <= 256, "one round of outputs");
  if (threadIdx.x < G * kHeadDim / 4) {
    const int h = threadIdx.x / (kHeadDim / 4), jq = threadIdx.x % (kHeadDim / 4);
    float mw[4], lw[4];
    float4 aw[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      mw[w] = red_m[w][h];
      lw[w] = red_l[w][h];
      aw[w] = reinterpret_cast<const float4*>(red_acc + (w * G + h) * kHeadDim)[jq];
    }
    const float mm = fmaxf(fmaxf(mw[0], mw[1]), fmaxf(mw[2], mw[3]));   // finite: a wave has pages
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
    const int64_t prow = static_cast<int64_t>(head0 + h) * p.slots + p.casc_chunks + split;
    reinterpret_cast<float4*>(pacc + prow * kHeadDim)[jq] = s4;
    if (jq == 0) reinterpret_cast<float2*>(ml)[prow] = make_float2(mm, l);
  }
}

// ------------------------------------------------------------------------------------------
// 2b. the int8 / bf16 INT2 pass (eight-head or two-group tiles)
#include "int2_i8.h"

// ------------------------------------------------------------------------------------------
// 3. BF16 segments: one 256-thread block per (64-token chunk, kv head, sequence), launched in the
// same grid as the INT2 blocks so the two segment passes run side by side.  Chunk 0 = sink rows
// 0..63, chunk c >= 1 = recent ring rows 64(c-1) .. 64c-1.  Every global load is issued up front:
// thread (token t, quarter) holds key row t, channels 32 quarter .. +31, for the scores (summed
// over the four lanes of a quad); thread (channel pair, wave) holds the value pairs of rows
// 16 wave .. 16 wave + 15 for the weighted sum.  Rows that hold no cached token count as -inf.
template <int G>
struct Bf16Lds {
  static constexpr int Q = 0;                                // fp32 [G][128]
  static constexpr int P = Q + G * kHeadDim * 4;             // fp32 [G][64]
  static constexpr int RM = P + G * kPage * 4;               // fp32 [4][G] wave maxima
  static constexpr int RL = RM + 4 * G * 4;                  // fp32 [4][G] wave sums
  static constexpr int RACC = RL + 4 * G * 4;                // fp32 [4][G][128]
  static constexpr int TOTAL = RACC + 4 * G * kHeadDim * 4;
};

// FUSE: a decode step whose append the segment launch runs: the new token's key and value rows
// are read from k_new / v_new in place of their row of the sink or ring, and the chunk that holds
// that row writes them there unless the token displaces a ring row (position >= 320: the block
// of chunk kDisplaceChunk, which demotes the displaced row first, writes the slot after reading
// it).
template <int G, bool FUSE = false>
__device__ __forceinline__ void bf16_block(const DecodeArgs& a, const Plan& p, float scale_log2,
                                           int chunk, int kv, int b, unsigned char* smem) {
  using S = Bf16Lds<G>;
  float (*q_s)[kHeadDim] = reinterpret_cast<float (*)[kHeadDim]>(smem + S::Q);
  float (*p_s)[kPage] = reinterpret_cast<float (*)[kPage]>(smem + S::P);
  float (*red_m)[G] = reinterpret_cast<float (*)[G]>(smem + S::RM);
  float (*red_l)[G] = reinterpret_cast<float (*)[G]>(smem + S::RL);
  float* red_acc = reinterpret_cast<float*>(smem + S::RACC);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = dev::lane_id();
  const int L = a.seq_lens[b] + a.len_add;
  const int64_t slot = a.seq_slot[b];
  if constexpr (FUSE) {
    if (chunk == kDisplaceChunk && L - 1 >= kSink + kRecent)
      displace_token(a, p, b, kv, L - 1, slot, smem);   // done with its LDS on return
  }
  const int head0 = b * p.hq + kv * G;
  const int64_t row0 = chunk == 0 ? (slot * p.hkv + kv) * kSink
                                   : (slot * p.hkv + kv) * kRecent + (chunk - 1) * 64;
  const uint16_t* krows = (chunk == 0 ? a.sink_k : a.recent_k) + row0 * kHeadDim;
  const uint16_t* vrows = (chunk == 0 ? a.sink_v : a.recent_v) + row0 * kHeadDim;
  const int n_recent = min(kRecent, max(0, L - kSink));
  auto row_valid = [&](int t) {
    if (chunk == 0) return t < min(L, kSink);
    const int r = (chunk - 1) * 64 + t;   // ring row
    const int start = L - n_recent;
    const int posr = start + (((r - start) % kRecent) + kRecent) % kRecent;
    return n_recent > 0 && posr < L;
  };
  // FUSE: the chunk row of the new token (position L - 1), or -1
  int new_row = -1;
  const uint16_t* knew = nullptr;
  const uint16_t* vnew = nullptr;
  if constexpr (FUSE) {
    const int pos = L - 1;
    if (chunk == (pos < kSink ? 0 : 1 + (pos % kRecent) / kPage))
      new_row = pos < kSink ? pos : pos % kPage;
    knew = a.ap.k_new + (static_cast<int64_t>(b) * p.hkv + kv) * kHeadDim;
    vnew = a.ap.v_new + (static_cast<int64_t>(b) * p.hkv + kv) * kHeadDim;
  }
  auto key_row = [&](int r) {
    return FUSE && r == new_row ? knew : krows + static_cast<int64_t>(r) * kHeadDim;
  };
  auto value_row = [&](int r) {
    return FUSE && r == new_row ? vnew : vrows + static_cast<int64_t>(r) * kHeadDim;
  };
  // ---- loads: key quarter rows, value pairs, query
  const int t = tid >> 2, qq = tid & 3;
  const bool kvalid = row_valid(t);
  uint4 kr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    kr[i] = kvalid ? reinterpret_cast<const uint4*>(key_row(t) + 32 * qq)[i]
                   : make_uint4(0, 0, 0, 0);
  uint32_t vr[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int tv = 16 * wave + i;
    vr[i] = row_valid(tv) ? reinterpret_cast<const uint32_t*>(value_row(tv))[lane] : 0u;
  }
  if constexpr (FUSE) {
    if (new_row >= 0 && L - 1 < kSink + kRecent) {
      const int64_t o = row0 * kHeadDim + static_cast<int64_t>(new_row) * kHeadDim;
      uint16_t* kdst = (chunk == 0 ? a.ap.sink_k : a.ap.recent_k) + o;
      uint16_t* vdst = (chunk == 0 ? a.ap.sink_v : a.ap.recent_v) + o;
      if (t == new_row)
#pragma unroll
        for (int i = 0; i < 4; ++i) reinterpret_cast<uint4*>(kdst + 32 * qq)[i] = kr[i];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (16 * wave + i == new_row) reinterpret_cast<uint32_t*>(vdst)[lane] = vr[i];
    }
  }
  for (int i = tid; i < G * kHeadDim; i += 256)
    q_s[i / kHeadDim][i % kHeadDim] =
        dev::bf16_to_f32(a.q[static_cast<int64_t>(head0) * kHeadDim + i]);
  __syncthreads();
  // ---- scores of token t (the four lanes of a quad share it), softmax statistics per head
  float logit[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float acc = 0.f;
    const float* qh = q_s[h] + 32 * qq;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf(qh[8 * i + 2 * e], __uint_as_float(w[e] << 16), acc);
        acc = fmaf(qh[8 * i + 2 * e + 1], __uint_as_float(w[e] & 0xFFFF0000u), acc);
      }
    }
    acc += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc), 0xB1, 0xF, 0xF, 0));
    acc += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc), 0x4E, 0xF, 0xF, 0));
    logit[h] = kvalid ? acc * scale_log2 : -INFINITY;
    const float mw = dev::wave_max(logit[h]);
    if (lane == 0) red_m[wave][h] = mw;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float m = fmaxf(fmaxf(red_m[0][h], red_m[1][h]), fmaxf(red_m[2][h], red_m[3][h]));
    const float pr = kvalid ? exp2f(logit[h] - m) : 0.f;
    if (qq == 0) p_s[h][t] = pr;
    const float lw = dev::wave_sum(qq == 0 ? pr : 0.f);
    if (lane == 0) red_l[wave][h] = lw;
  }
  __syncthreads();
  // ---- weighted values: thread (channel pair lane, wave) over rows 16 wave .. 16 wave + 15
  float acc[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) acc[h][0] = acc[h][1] = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float lo = __uint_as_float(vr[i] << 16);
    const float hi = __uint_as_float(vr[i] & 0xFFFF0000u);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float pr = p_s[h][16 * wave + i];
      acc[h][0] = fmaf(pr, lo, acc[h][0]);
      acc[h][1] = fmaf(pr, hi, acc[h][1]);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    red_acc[(wave * G + h) * kHeadDim + 2 * lane] = acc[h][0];
    red_acc[(wave * G + h) * kHeadDim + 2 * lane + 1] = acc[h][1];
  }
  __syncthreads();
  float* ml = reinterpret_cast<float*>(a.workspace + p.off_bf16_ml);
  float* pacc = reinterpret_cast<float*>(a.workspace + p.off_bf16_acc);
  for (int i = tid; i < G * kHeadDim; i += 256) {
    const int h = i / kHeadDim, j = i % kHeadDim;
    const float v = (red_acc[(0 * G + h) * kHeadDim + j] + red_acc[(1 * G + h) * kHeadDim + j]) +
                    (red_acc[(2 * G + h) * kHeadDim + j] + red_acc[(3 * G + h) * kHeadDim + j]);
    const int64_t prow = static_cast<int64_t>(head0 + h) * kBf16Chunks + chunk;
    pacc[prow * kHeadDim + j] = v;
    if (j == 0) {
      ml[prow * 2] = fmaxf(fmaxf(red_m[0][h], red_m[1][h]), fmaxf(red_m[2][h], red_m[3][h]));
      ml[prow * 2 + 1] = (red_l[0][h] + red_l[1][h]) + (red_l[2][h] + red_l[3][h]);
    }
  }
}

// ------------------------------------------------------------------------------------------
// The segment passes share one launch: blocks x0 + blockIdx.x < kBf16Chunks are BF16 chunks,
// the rest INT2 splits.
template <int G, int NG>
constexpr int attn_lds_bytes() {
  constexpr int i2 = int2_fp8_pass(G, NG) ? Int2Lds<G, NG>::TOTAL : Int2LdsI8<G, NG>::TOTAL;
  return i2 > Bf16Lds<G>::TOTAL ? i2 : Bf16Lds<G>::TOTAL;
}

// CASC: the launch also holds the shared-prefix cascade blocks, one per (prefix chunk, KV head,
// group of kCascGroup sequences): casc_z z-slices of the grid, every casc_step-th slice from the
// first, so that the chip runs them (arithmetic on staged pages) beside the segment blocks
// (streams of private pages) instead of after them.  A cascade block of slice k is number
// k * gridDim.x + blockIdx.x, taken KV head fastest, then group, then chunk: the groups of one
// (chunk, KV head), which read the same pages, are dispatched hkv blocks apart -- with eight KV
// heads, to one XCD and its L2 (workgroups go to the eight XCDs in turn).
// FUSE: a decode step that appends and rotates the query in this launch (see step_prologue).
template <int G, int NG, bool STREAM, bool CB, bool CASC = false, bool FUSE = false>
__global__ __launch_bounds__(256, 2) void attn_kernel(DecodeArgs a, Plan p, float scale_log2,
                                                      int x0, int casc_z, int casc_step) {
  constexpr int kBase = CASC && Int2Lds<G, 1>::CASC_TOTAL > attn_lds_bytes<G, NG>()
                            ? Int2Lds<G, 1>::CASC_TOTAL
                            : attn_lds_bytes<G, NG>();
  constexpr int kLds = FUSE && Int2Lds<G, 1>::FUSED_TOTAL > kBase ? Int2Lds<G, 1>::FUSED_TOTAL
                                                                  : kBase;
  static_assert(!FUSE || kLds >= 2 * kHeadDim * 4 + dev::kRotGroups * kHeadDim * 8,
                "displace_token's rows and partials");
  __shared__ __attribute__((aligned(16))) unsigned char smem[kLds];
  const int x = x0 + static_cast<int>(blockIdx.x) / p.hkv, kv = blockIdx.x % p.hkv;
  int b = blockIdx.z;
  if constexpr (CASC) {
    static_assert(NG == 1 && !CB && !STREAM, "cascade blocks: single-group pass, no codebooks");
    const int k = b / casc_step;
    if (b % casc_step == 0 && k < casc_z) {
      const int ci = k * static_cast<int>(gridDim.x) + static_cast<int>(blockIdx.x);
      if (ci >= p.casc_chunks * p.hkv * p.casc_groups) return;
      const int rest = ci / p.hkv;
      int2_block<G, 1, false, false, true, true>(a, p, rest / p.casc_groups, ci % p.hkv,
                                                 rest % p.casc_groups, smem);
      return;
    }
    b -= min(k + 1, casc_z);
  }
  if (x < kBf16Chunks)
    bf16_block<G, FUSE>(a, p, scale_log2, x, kv, b, smem);
  else if constexpr (int2_fp8_pass(G, NG))
    int2_block<G, NG, STREAM, CB, false, CASC, FUSE>(a, p, x - kBf16Chunks, kv, b, smem);
  else
    int2_block_i8<G, NG, STREAM>(a, p, x - kBf16Chunks, kv, b, smem);
}

// ------------------------------------------------------------------------------------------
// 4. merge: four 256-thread blocks per (sequence, query head) row, block q producing output
// channels [32 q, 32 q + 32) -- or, in launches of at least kMergeRowsOneBlock rows, one block per
// row that produces the four quarters in turn.  Each block combines all INT2 splits of its row
// (the rotated-frame vector is needed whole for the Hadamard transform); a quarter block reads
// only its 32 rows of U_v, so its load volume is about half of one block doing the whole row,
// spread over four times as many compute units.  Every global load is issued before the first reduction and none waits
// on the sequence length (entries of splits the sequence does not reach are read but masked).
//   (1) thread (channel quad, split residue r mod 8) merges its own splits r, r + 8, ... into a
//       local (m, l, acc') with a local maximum;
//   (2) wave 0 merges the eight residue partials (one barrier before), gathers the channels in
//       bit-reversed order and applies H / sqrt(d) as butterflies across the wave;
//   (3) times U_v^T: eight threads per output channel, 16 inputs each, summed across the lanes;
//   (4) merge with the BF16 chunk partials and normalise.
constexpr int kMergePrefetch = 12;   // splits per thread loaded up front (96 splits per row)
static_assert(kMergePrefetch * 8 == kMergeSplits, "the plan caps the splits at what one round takes");
constexpr int kMergeQuarters = 4;    // output-channel quarters of a row (32 channels each)
constexpr int kMergeCols = kHeadDim / kMergeQuarters;
// Rows (sequence, query head) from which a launch gives each row one block that takes all four
// quarters instead of one block per quarter: with enough rows to fill the chip, fewer blocks
// repeat less of the per-row work (the split loads and merges of steps 1 and 2).
constexpr int kMergeRowsOneBlock = 512;

// CASC: the plan has cascade chunks (their slots come first in each row).
template <int PARTS, bool CASC>
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a, Plan p) {
  __shared__ __attribute__((aligned(16))) float part[8][kHeadDim];
  __shared__ float part_m[8], part_l[8];
  __shared__ __attribute__((aligned(16))) float vec[kHeadDim];
  static_assert(PARTS == 1 || PARTS == kMergeQuarters, "one block per row or per quarter");
  // blocks numbered (sequence, head in group, quarter, KV head) with the KV head fastest: the
  // blocks of one KV head (which share its U_v rows) run on one die, as its attention blocks did
  const int kv = blockIdx.x % p.hkv;
  const int q0 = (blockIdx.x / p.hkv) % PARTS;   // first quarter of this block
  const int r = blockIdx.x / p.hkv / PARTS;      // b * gqa + head within the group
  const int b = r / p.gqa;
  const int row = b * p.hq + kv * p.gqa + r % p.gqa;   // b * hq + head
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = dev::lane_id();
  const float2* iml = reinterpret_cast<const float2*>(a.workspace + p.off_int2_ml) +
                      static_cast<int64_t>(row) * p.slots;
  const float4* iacc = reinterpret_cast<const float4*>(a.workspace + p.off_int2_acc) +
                       static_cast<int64_t>(row) * p.slots * (kHeadDim / 4);
  const float* bml = reinterpret_cast<const float*>(a.workspace + p.off_bf16_ml) +
                     static_cast<int64_t>(row) * kBf16Chunks * 2;
  const float* bacc = reinterpret_cast<const float*>(a.workspace + p.off_bf16_acc) +
                      static_cast<int64_t>(row) * kBf16Chunks * kHeadDim;
  const int cq = tid & 31, sr = tid >> 5;     // (1): channel quad, split residue
  const int jl = tid >> 3, ip = tid & 7;      // (3): output channel 32 q + jl, input part

  // ---- loads
  float2 st[kMergePrefetch];
  float4 pa[kMergePrefetch];
#pragma unroll
  for (int i = 0; i < kMergePrefetch; ++i) {
    const int s = sr + 8 * i;
    const bool in = s < p.slots;
    st[i] = in ? iml[s] : make_float2(-INFINITY, 0.f);
    pa[i] = in ? iacc[static_cast<int64_t>(s) * (kHeadDim / 4) + cq]
               : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float4 uv[4];   // U_v[kv][j][16 ip .. 16 ip + 15] of the current quarter's channel j
  float ba[kBf16Chunks];
  auto load_quarter = [&](int j) {
    const float4* u = reinterpret_cast<const float4*>(
        a.u_v + (static_cast<int64_t>(kv) * kHeadDim + j) * kHeadDim + 16 * ip);
#pragma unroll
    for (int c = 0; c < 4; ++c) uv[c] = u[c];
#pragma unroll
    for (int c = 0; c < kBf16Chunks; ++c) ba[c] = ip == 0 ? bacc[c * kHeadDim + j] : 0.f;
  };
  load_quarter(kMergeCols * q0 + jl);
  float bm[kBf16Chunks], bl[kBf16Chunks];
#pragma unroll
  for (int c = 0; c < kBf16Chunks; ++c) {
    bm[c] = bml[2 * c];
    bl[c] = bml[2 * c + 1];
  }
  const int L = a.seq_lens[b] + a.len_add;
  const int n_hist = max(0, L - kSink - kRecent);
  const int n_pages = (n_hist + kPage - 1) / kPage;
  const int n_valid = (n_pages + p.pages_per_split - 1) / p.pages_per_split;
  // slots of the row's partials: cascade chunks [0, casc_chunks) (those its history wholly holds
  // were written), then splits (those holding a page past the cascade's pages and within the
  // history: none when the cascade took every page); without a cascade, the splits [0, n_valid)
  int c_b = 0, s_first = 0, s_end = n_valid;
  if constexpr (CASC) {
    const int cend = cascade_pages(p, n_hist, a.shared_pages[b]);
    c_b = cend / kCascPages;
    s_end = p.casc_chunks + n_valid;
    s_first = cend < n_pages ? p.casc_chunks + cend / p.pages_per_split : s_end;
  }
  // (no short-circuit: one compare per slot, not a branch)
  auto valid = [&](int s) {
    if constexpr (CASC)
      return (s < c_b) | ((s >= s_first) & (s < s_end));
    else
      return s < s_end;
  };

  // ---- (1) this thread's splits (those the sequence reaches), with its own maximum
  float m_loc = -INFINITY, l_loc = 0.f;
  float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);
  auto absorb = [&](const float2* ml, const float4* v, int s0, int n) {
    float mb = -INFINITY;
    for (int i = 0; i < n; ++i)
      if (valid(s0 + 8 * i)) mb = fmaxf(mb, ml[i].x);
    if (mb == -INFINITY) return;
    const float mn = fmaxf(m_loc, mb);
    const float al = exp2f(m_loc - mn);   // 0 while nothing is held yet
    l_loc *= al;
    s4.x *= al;
    s4.y *= al;
    s4.z *= al;
    s4.w *= al;
    m_loc = mn;
    for (int i = 0; i < n; ++i) {
      if (!valid(s0 + 8 * i)) continue;
      const float f = exp2f(ml[i].x - mn);
      l_loc = fmaf(ml[i].y, f, l_loc);
      s4.x = fmaf(v[i].x, f, s4.x);
      s4.y = fmaf(v[i].y, f, s4.y);
      s4.z = fmaf(v[i].z, f, s4.z);
      s4.w = fmaf(v[i].w, f, s4.w);
    }
  };
  absorb(st, pa, sr, kMergePrefetch);
  // slots past the prefetch (more than 96 per row): rounds of four
  for (int s0 = sr + 8 * kMergePrefetch; s0 < s_end; s0 += 32) {
    float2 ml4[4];
    float4 v4[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int s = s0 + 8 * k;
      ml4[k] = s < s_end ? iml[s] : make_float2(-INFINITY, 0.f);
      v4[k] = s < s_end ? iacc[static_cast<int64_t>(s) * (kHeadDim / 4) + cq]
                        : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    absorb(ml4, v4, s0, 4);
  }
  reinterpret_cast<float4*>(part[sr])[cq] = s4;
  if (cq == 0) {
    part_m[sr] = m_loc;
    part_l[sr] = l_loc;
  }
  __syncthreads();
  // ---- (2) merge of the residues, (acc' P) H / sqrt(d) in wave 0: lane holds entries lane and
  // lane + 64
  if (wave == 0) {
    float mi = part_m[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) mi = fmaxf(mi, part_m[r]);
    float w[8], li = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      w[r] = mi == -INFINITY ? 0.f : exp2f(part_m[r] - mi);
      li = fmaf(part_l[r], w[r], li);
    }
    auto gather = [&](int jj) {
      const int src = dev::bitrev7(jj);   // (acc' P)_j = acc'_rev(j)
      float v = 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r) v = fmaf(part[r][src], w[r], v);
      return v;
    };
    float y0 = gather(lane), y1 = gather(lane + 64);
    {
      const float t0 = y0 + y1, t1 = y0 - y1;
      y0 = t0;
      y1 = t1;
    }
    y0 = dev::butterfly<32>(y0);
    y1 = dev::butterfly<32>(y1);
    y0 = dev::butterfly<16>(y0);
    y1 = dev::butterfly<16>(y1);
    y0 = dev::butterfly<8>(y0);
    y1 = dev::butterfly<8>(y1);
    y0 = dev::butterfly<4>(y0);
    y1 = dev::butterfly<4>(y1);
    y0 = dev::butterfly<2>(y0);
    y1 = dev::butterfly<2>(y1);
    y0 = dev::butterfly<1>(y0);
    y1 = dev::butterfly<1>(y1);
    vec[lane] = y0;
    vec[lane + 64] = y1;
    if (lane == 0) {
      part_m[0] = mi;   // every reader of part_m / part_l has passed: only wave 0 read them
      part_l[0] = li;
    }
  }
  __syncthreads();
  const float mi = part_m[0], li = part_l[0];
  for (int qq = 0; qq < kMergeQuarters / PARTS; ++qq) {
    const int j = kMergeCols * (q0 + qq) + jl;
    if (qq > 0) load_quarter(j);
    float o = 0.f;
    {
      const float4 v4[4] = {reinterpret_cast<const float4*>(vec)[4 * ip],
                            reinterpret_cast<const float4*>(vec)[4 * ip + 1],
                            reinterpret_cast<const float4*>(vec)[4 * ip + 2],
                            reinterpret_cast<const float4*>(vec)[4 * ip + 3]};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        o = fmaf(v4[c].x, uv[c].x, o);
        o = fmaf(v4[c].y, uv[c].y, o);
        o = fmaf(v4[c].z, uv[c].z, o);
        o = fmaf(v4[c].w, uv[c].w, o);
      }
      // sum over the eight input parts (lanes 8 jl .. 8 jl + 7 of the wave)
      o += dev::lane_xor_dpp<1>(o);
      o += dev::lane_xor_dpp<2>(o);
      o += dev::lane_xor_dpp<4>(o);
    }
    // ---- (4) merge with the BF16 partials
    if (ip == 0) {
      const float m_int2 = n_valid > 0 ? mi : -INFINITY;
      float mt = m_int2;
#pragma unroll
      for (int c = 0; c < kBf16Chunks; ++c) mt = fmaxf(mt, bm[c]);
      float acc = 0.f, l = 0.f;
      if (m_int2 != -INFINITY) {
        const float f = exp2f(m_int2 - mt);
        acc = o * 0.08838834764831845f * f;
        l = li * f;
      }
#pragma unroll
      for (int c = 0; c < kBf16Chunks; ++c) {
        if (bm[c] == -INFINITY) continue;
        const float f = exp2f(bm[c] - mt);
        acc = fmaf(ba[c], f, acc);
        l = fmaf(bl[c], f, l);
      }
      a.out[static_cast<int64_t>(row) * kHeadDim + j] = acc / l;
      if (a.lse != nullptr && j == 0) a.lse[row] = (mt + log2f(l)) * 0.6931471805599453f;
    }
  }
}

template <int G>
hipError_t launch_g(const DecodeArgs& a, const Plan& p, uint32_t stages, hipStream_t stream) {
  const float scale_log2 = a.sm_scale * kLog2e;
  const int x0 = (stages & OSCAR_STAGE_BF16) ? 0 : kBf16Chunks;
  const int x1 = kBf16Chunks + ((stages & OSCAR_STAGE_INT2) ? p.num_splits : 0);
  bool cb_done = false;
  if ((stages & OSCAR_STAGE_INT2) && p.casc_chunks > 0) {
    // the host admits a cascade on the four-head single-group pass only, without codebooks;
    // its blocks share the segment launch (x1 > x0 here)
    if constexpr (int2_fp8_pass(G, 1)) {
      if (p.n_groups != 1 || a.cb_k != nullptr || a.prefix_ids == nullptr ||
          a.shared_pages == nullptr)
        return hipErrorInvalidValue;
      const int gx = (x1 - x0) * p.hkv;
      const int blocks = p.casc_chunks * p.hkv * p.casc_groups;
      const int cz = (blocks + gx - 1) / gx;
      const int step = (p.batch + cz) / cz;   // >= 1
      hipLaunchKernelGGL((attn_kernel<G, 1, false, false, true>), dim3(gx, 1, p.batch + cz),
                         dim3(256), 0, stream, a, p, scale_log2, x0, cz, step);
      cb_done = true;
    } else {
      return hipErrorInvalidValue;
    }
  }
  if (a.fuse && x1 > x0) {
    // a decode step with its preparation in this launch: every segment block, the fp8 pass
    // without codebooks or a cascade (the host admits no other)
    if constexpr (int2_fp8_pass(G, 1)) {
      if (x0 != 0 || x1 != kBf16Chunks + p.num_splits || p.n_groups != 1 ||
          a.cb_k != nullptr || p.casc_chunks != 0)
        return hipErrorInvalidValue;
      dim3 grid((x1 - x0) * p.hkv, 1, p.batch);
      if (p.batch == 1)
        hipLaunchKernelGGL((attn_kernel<G, 1, true, false, false, true>), grid, dim3(256), 0,
                           stream, a, p, scale_log2, x0, 0, 1);
      else
        hipLaunchKernelGGL((attn_kernel<G, 1, false, false, false, true>), grid, dim3(256), 0,
                           stream, a, p, scale_log2, x0, 0, 1);
      cb_done = true;
    } else {
      return hipErrorInvalidValue;
    }
  }
  if (x1 > x0 && !cb_done) {
    dim3 grid((x1 - x0) * p.hkv, 1, p.batch);
    const bool one = p.batch == 1;
    // a codebook history (cb_k / cb_v) runs on the fp8 pass; the host admits it only there
    const bool cb = a.cb_k != nullptr;
    if constexpr (int2_fp8_pass(G, 1)) {
      if (cb && p.n_groups == 1) {
        if (one)
          hipLaunchKernelGGL((attn_kernel<G, 1, true, true>), grid, dim3(256), 0, stream, a, p,
                             scale_log2, x0, 0, 1);
        else
          hipLaunchKernelGGL((attn_kernel<G, 1, false, true>), grid, dim3(256), 0, stream, a, p,
                             scale_log2, x0, 0, 1);
        cb_done = true;
      }
    }
    if (cb_done)
      ;
    else if (cb)
      return hipErrorInvalidValue;
    else if (p.n_groups == 1 && one)
      hipLaunchKernelGGL((attn_kernel<G, 1, true, false>), grid, dim3(256), 0, stream, a, p,
                         scale_log2, x0, 0, 1);
    else if (p.n_groups == 1)
      hipLaunchKernelGGL((attn_kernel<G, 1, false, false>), grid, dim3(256), 0, stream, a, p,
                         scale_log2, x0, 0, 1);
    else if (one)
      hipLaunchKernelGGL((attn_kernel<G, 2, true, false>), grid, dim3(256), 0, stream, a, p,
                         scale_log2, x0, 0, 1);
    else
      hipLaunchKernelGGL((attn_kernel<G, 2, false, false>), grid, dim3(256), 0, stream, a, p,
                         scale_log2, x0, 0, 1);
  }
  if (stages & OSCAR_STAGE_MERGE) {
    const int rows = p.batch * p.hq;
    const bool casc = p.casc_chunks > 0;
    if (rows >= kMergeRowsOneBlock) {
      if (casc)
        hipLaunchKernelGGL((merge_kernel<1, true>), dim3(rows), dim3(256), 0, stream, a, p);
      else
        hipLaunchKernelGGL((merge_kernel<1, false>), dim3(rows), dim3(256), 0, stream, a, p);
    } else if (casc) {
      hipLaunchKernelGGL((merge_kernel<kMergeQuarters, true>), dim3(rows * kMergeQuarters),
                         dim3(256), 0, stream, a, p);
    } else {
      hipLaunchKernelGGL((merge_kernel<kMergeQuarters, false>), dim3(rows * kMergeQuarters),
                         dim3(256), 0, stream, a, p);
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, const Plan& p, uint32_t stages,
                         hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  switch (p.gqa) {
    case 1: return launch_g<1>(a, p, stages, stream);
    case 2: return launch_g<2>(a, p, stages, stream);
    case 4: return launch_g<4>(a, p, stages, stream);
    case 8: return launch_g<8>(a, p, stages, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace oscar
