// Decode attention over the three-segment cache (BF16 sink | rotated INT2 history | BF16 recent).
//
// Structure after the OSCAR write-up "超越TurboQuant！OSCAR：面向真实服务的2-bit KV Cache量化",
// section OSCAR 的设计: the INT2 history and the BF16 segments are processed separately and then
// combined with an online-softmax merge.  Launch order on one stream:
//   1. query_kernel  q' = q R_k per query head (fp64 rotation), quantised for the INT2 pass into
//                    int8 hi / lo parts (q' ~ a (hi + lo / 256)) laid out as MFMA operands, plus
//                    the per-group sums of the quantised q' that the zero points multiply;
//   2. int2_kernel   split-KV over history pages on the matrix cores: scores s (q' . codes) +
//                    z sum(q') with the dot products as exact int32 i8 MFMAs, online softmax with
//                    lazy rescaling, value accumulation in the rotated frame as bf16 MFMAs ->
//                    (m, l, acc') partials;
//   3. bf16_kernel   64-token chunks of the BF16 sink and recent ring -> (m, l, acc) partials;
//   4. merge_kernel  log-sum-exp merge of the INT2 partials, un-rotation acc' R_v^T, merge with
//                    the BF16 partials, normalisation.
// Softmax statistics are kept in the log2 domain: scores are scaled by sm_scale * log2(e).
#include "device_common.h"
#include "oscar_internal.h"

namespace oscar {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kTau = 8.0f;   // lazy rescaling: exponents up to 2^8 before the max is moved

// ------------------------------------------------------------------------------------------
// 1. query preparation: one 256-thread block per (sequence, query head)
__global__ __launch_bounds__(256) void query_kernel(const uint16_t* __restrict__ q,
                                                    const float* __restrict__ u_k, int hq,
                                                    int gqa, int n_groups, float scale_log2,
                                                    int8_t* __restrict__ qpack,
                                                    float* __restrict__ qmeta) {
  __shared__ float x[kHeadDim];
  __shared__ double red[4][kHeadDim];
  const int row = blockIdx.x;   // b * hq + head
  const int kv = (row % hq) / gqa;
  if (threadIdx.x < kHeadDim)
    x[threadIdx.x] = dev::bf16_to_f32(q[static_cast<int64_t>(row) * kHeadDim + threadIdx.x]);
  __syncthreads();
  double r0, r1;
  const bool lead = dev::rotate1_block(x, u_k + static_cast<int64_t>(kv) * kHeadDim * kHeadDim,
                                       red, r0, r1);
  if (!lead) return;
  const int lane = dev::lane_id();
  const float f0 = static_cast<float>(r0);   // rotated channel lane
  const float f1 = static_cast<float>(r1);   // rotated channel lane + 64
  const float amax = dev::wave_max(fmaxf(fabsf(f0), fabsf(f1)));
  const float a = amax > 0.f ? amax / 127.f : 1.f;
  auto split = [a](float v, int& hi, int& lo) {
    hi = static_cast<int>(rintf(v / a));
    const float r = fmaf(-static_cast<float>(hi), a, v);
    lo = static_cast<int>(fminf(fmaxf(rintf(r * 256.f / a), -127.f), 127.f));
  };
  int h0, l0, h1, l1;
  split(f0, h0, l0);
  split(f1, h1, l1);
  // MFMA operand order: channel j = 16 qd + 4 b + k sits at byte 16 qd + 4 k + b
  auto pos = [](int j) { return (j >> 4) * 16 + (j & 3) * 4 + ((j >> 2) & 3); };
  int8_t* dst = qpack + static_cast<int64_t>(row) * 256;
  dst[pos(lane)] = static_cast<int8_t>(h0);
  dst[pos(lane + 64)] = static_cast<int8_t>(h1);
  dst[128 + pos(lane)] = static_cast<int8_t>(l0);
  dst[128 + pos(lane + 64)] = static_cast<int8_t>(l1);
  // sums of the quantised q' per group, in units of a / 256 (exact in int32)
  const int e0 = 256 * h0 + l0, e1 = 256 * h1 + l1;
  int s0, s1;
  if (n_groups == 1) {
    s0 = dev::wave_sum_i(e0 + e1);
    s1 = 0;
  } else {
    s0 = dev::wave_sum_i(e0);
    s1 = dev::wave_sum_i(e1);
  }
  if (lane == 0) {
    float* m = qmeta + static_cast<int64_t>(row) * 4;
    m[0] = a / 256.f * scale_log2;
    m[1] = static_cast<float>(s0);
    m[2] = static_cast<float>(s1);
    m[3] = 0.f;
  }
}

// FP4 (E2M1) pair in byte B of x -> two bf16; a 2-bit code zero-extended to a nibble encodes
// code / 2, so the scale 2 gives the code itself.
template <int B>
__device__ __forceinline__ v2bf codes_to_bf16(uint32_t x) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, 2.0f, B);
}

// ------------------------------------------------------------------------------------------
// 2. INT2 split-KV decode on the matrix cores.
//
// Block = 4 waves on pages [p0, p1) of one (sequence, KV head).  A wave takes PP consecutive
// pages per step (PP = 2 unless registers do not allow it): wave w's steps start at pages
// p0 + PP (4 i + w), i = 0, 1, ...  The pages of a step are independent chains that the wave
// interleaves, and the next step's loads are in flight while a step is processed (two register
// sets used in turn).
//
// Scores: D[row, token] = sum_k A[row, k] B[k, token] with v_mfma_i32_16x16x64_i8.  B = key codes
// of 16 tokens (lane n + 16 qd holds token n's packed dwords qd and 4 + qd, spread into bytes);
// A = the int8 hi (or lo) part of q' placed in rows 4 st + h (GP = 4) or 8 (st % 2) + h (GP = 8)
// for sub-tile st (zero elsewhere), kept in LDS.  The output rows of one sub-tile land in one
// lane group, so after the page's sub-tiles every lane holds the scores of its own token(s) for
// 4 heads, one per register.
// Values: acc[row, ch] += sum_t P[row, t] V[t, ch] with v_mfma_f32_16x16x32_bf16; P rows are the
// bf16 hi and lo parts of p * s_v for each head, transposed through LDS; V = value codes turned
// into exact bf16 integers by the FP4 conversion path.
template <int G, int NG>
__global__ __launch_bounds__(256, 2) void int2_kernel(DecodeArgs a, Plan p) {
  constexpr int GP = G <= 4 ? 4 : 8;      // padded query heads per KV head
  constexpr int NACC = GP / 4;            // score accumulators (tokens per lane and page)
  constexpr int NPL = 16 / GP;            // operand placements
  constexpr int PP = 1;                    // pages per step
  constexpr int BLK = kMetaOff + kPage * 8 * NG;
  constexpr int QA_BYTES = NPL * 2 * 2 * 64 * 16;             // [pl][hf][hl][lane] int8 x16
  constexpr int PB_BYTES = 4 * PP * NG * 16 * kPage * 2;      // [wave][page][g][row][token] bf16
  constexpr int RED_BYTES = 4 * 2 * GP * kHeadDim * 4;        // [wave][row][ch] fp32, after loop
  constexpr int SMEM = (QA_BYTES + PB_BYTES) > RED_BYTES ? (QA_BYTES + PB_BYTES) : RED_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  __shared__ int page_ids[kMaxPagesPerSplit];
  __shared__ float red_m[4][GP], red_l[4][GP], red_z[4][GP][NG];
  v4i* qa_lds = reinterpret_cast<v4i*>(smem);
  __bf16* pbuf_all = reinterpret_cast<__bf16*>(smem + QA_BYTES);
  float* red_acc = reinterpret_cast<float*>(smem);

  const int split = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int L = a.seq_lens[b];
  const int n_hist = max(0, L - kSink - kRecent);
  const int n_pages = (n_hist + kPage - 1) / kPage;
  const int p0 = split * p.pages_per_split;
  if (p0 >= n_pages) return;
  const int p1 = min(p0 + p.pages_per_split, n_pages);
  const int wave = threadIdx.x >> 6;
  const int lane = dev::lane_id();
  const int gq = lane >> 4, n = lane & 15;
  const int head0 = b * p.hq + kv * G;

  for (int i = threadIdx.x; i < p1 - p0; i += 256)
    page_ids[i] = a.page_table[static_cast<int64_t>(b) * a.max_pages_per_seq + p0 + i];

  // ---- query operands into LDS: operand (pl, hf, hl) is nonzero only in the lanes of placement
  // pl; each wave writes the copy it will read (all four waves hold the same values)
  const int8_t* qpack = reinterpret_cast<const int8_t*>(a.workspace + p.off_qrot);
  const float* qmeta = reinterpret_cast<const float*>(a.workspace + p.off_sigma);
  if (wave == 0) {
    const int pl = n / GP, hd = n % GP;
#pragma unroll
    for (int q = 0; q < NPL; ++q)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int hl = 0; hl < 2; ++hl) {
          v4i v = {0, 0, 0, 0};
          if (q == pl && hd < G)
            v = *reinterpret_cast<const v4i*>(qpack + static_cast<int64_t>(head0 + hd) * 256 +
                                              hl * 128 + (hf * 4 + gq) * 16);
          qa_lds[((q * 2 + hf) * 2 + hl) * 64 + lane] = v;
        }
  }
  // per head-slot constants of this lane: head = hs (GP = 4) or 4 (gq & 1) + hs (GP = 8)
  float kh[4], sq[4][NG];
#pragma unroll
  for (int hs = 0; hs < 4; ++hs) {
    const int hd = GP == 4 ? hs : 4 * (gq & 1) + hs;
    const float* m = qmeta + static_cast<int64_t>(head0 + min(hd, G - 1)) * 4;
    kh[hs] = hd < G ? m[0] : 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) sq[hs][g] = m[1 + g];
  }
  // token (within a page) of this lane's score accumulator pa
  auto tok_of = [&](int pa) { return GP == 4 ? lane : 16 * (2 * pa + (gq >> 1)) + n; };
  // position of a token in a P row; value operands read 8 consecutive entries per lane, which
  // hold tokens 8 k + {0, 2, 4, 6, 1, 3, 5, 7}
  auto ppos = [](int t) { return (t & ~7) | ((t & 7) >> 1) | ((t & 1) << 2); };
  auto pbuf = [&](int pp, int g, int row) -> __bf16* {
    return pbuf_all + ((((wave * PP + pp) * NG + g) * 16 + row) * kPage);
  };
  // rows 2 GP .. 15 of every P tile stay zero (value operands of unused rows)
  for (int i = lane; i < PP * NG * (16 - 2 * GP) * kPage; i += 64) {
    const int per = (16 - 2 * GP) * kPage;
    const int pg2 = i / per, rem = i % per;
    pbuf(pg2 / NG, pg2 % NG, 2 * GP + rem / kPage)[rem % kPage] = static_cast<__bf16>(0.f);
  }
  __syncthreads();

  float m_run[4], l_run[4], z_run[4][NG];
#pragma unroll
  for (int hs = 0; hs < 4; ++hs) {
    m_run[hs] = -INFINITY;
    l_run[hs] = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) z_run[hs][g] = 0.f;
  }
  v4f acc[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) acc[nt] = v4f{0.f, 0.f, 0.f, 0.f};

  // One page's operands, fetched with 16-byte loads from the tiled block (one chunk row = 64 lanes
  // x 16 bytes): key chunk row j holds this lane's words of sub-tiles 2j and 2j + 1, value chunk
  // row j those of channel tiles 4j .. 4j + 3; the meta of a token is (key pairs, value pairs).
  struct PageRegs {
    uint4 k[2];              // k[st / 2] entry 2 (st % 2) + hf: key codes, sub-tile st, half hf
    uint4 v[2];              // v[nt / 4] entry nt % 4: value codes, channel 16 nt + n
    uint32_t km[NACC][NG];   // key meta (scale | zero << 16) of the lane's token(s)
    uint32_t vm[NACC][NG];
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
  auto load_page = [&](int pg, PageRegs& r) {
    const uint8_t* blk = a.pool + (static_cast<int64_t>(page_ids[pg - p0]) * p.hkv + kv) * BLK;
    const uint4* kc = reinterpret_cast<const uint4*>(blk + kKCodesOff);
    const uint4* vc = reinterpret_cast<const uint4*>(blk + kVCodesOff);
    r.k[0] = kc[lane];
    r.k[1] = kc[64 + lane];
    r.v[0] = vc[lane];
    r.v[1] = vc[64 + lane];
#pragma unroll
    for (int pa = 0; pa < NACC; ++pa) {
      const uint8_t* m = blk + kMetaOff + tok_of(pa) * 8 * NG;
      if (NG == 1) {
        const uint2 w = *reinterpret_cast<const uint2*>(m);
        r.km[pa][0] = w.x;
        r.vm[pa][0] = w.y;
      } else {
        const uint4 w = *reinterpret_cast<const uint4*>(m);
        r.km[pa][0] = w.x;
        r.km[pa][NG - 1] = w.y;
        r.vm[pa][0] = w.z;
        r.vm[pa][NG - 1] = w.w;
      }
    }
  };

  // Pages pg .. pg + PP - 1 on register sets r[0 .. PP - 1]; pages past p1 contribute nothing.
  auto process_step = [&](int pg, const PageRegs* r) {
    // ---- scores
    v4i dh[PP][NACC][NG], dl[PP][NACC][NG];
#pragma unroll
    for (int pp = 0; pp < PP; ++pp)
#pragma unroll
      for (int pa = 0; pa < NACC; ++pa)
#pragma unroll
        for (int g = 0; g < NG; ++g) dh[pp][pa][g] = dl[pp][pa][g] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int pa = st / NPL, pl = st % NPL;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const v4i ah = qa_lds[((pl * 2 + hf) * 2 + 0) * 64 + lane];
        const v4i al = qa_lds[((pl * 2 + hf) * 2 + 1) * 64 + lane];
        const int g = NG == 2 ? hf : 0;
#pragma unroll
        for (int pp = 0; pp < PP; ++pp) {
          const uint32_t w = kword(r[pp], st, hf);
          const v4i bk = {static_cast<int>(w & 0x03030303u),
                          static_cast<int>((w >> 2) & 0x03030303u),
                          static_cast<int>((w >> 4) & 0x03030303u),
                          static_cast<int>((w >> 6) & 0x03030303u)};
          dh[pp][pa][g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah, bk, dh[pp][pa][g], 0, 0, 0);
          dl[pp][pa][g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(al, bk, dl[pp][pa][g], 0, 0, 0);
        }
      }
    }
    float logit[PP][NACC][4];
    bool valid[PP][NACC];
    float vs[PP][NACC][NG], vz[PP][NACC][NG];
#pragma unroll
    for (int pp = 0; pp < PP; ++pp)
#pragma unroll
      for (int pa = 0; pa < NACC; ++pa) {
        valid[pp][pa] = (pg + pp) * kPage + tok_of(pa) < n_hist && pg + pp < p1;
        float ks[NG], kz[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const uint32_t km = r[pp].km[pa][g], vm = r[pp].vm[pa][g];
          ks[g] = __half2float(__ushort_as_half(static_cast<uint16_t>(km & 0xFFFF)));
          kz[g] = __half2float(__ushort_as_half(static_cast<uint16_t>(km >> 16)));
          vs[pp][pa][g] = __half2float(__ushort_as_half(static_cast<uint16_t>(vm & 0xFFFF)));
          vz[pp][pa][g] = __half2float(__ushort_as_half(static_cast<uint16_t>(vm >> 16)));
        }
#pragma unroll
        for (int hs = 0; hs < 4; ++hs) {
          float t = 0.f;
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            const int s = (dh[pp][pa][g][hs] << 8) + dl[pp][pa][g][hs];
            t = fmaf(ks[g], static_cast<float>(s), fmaf(kz[g], sq[hs][g], t));
          }
          logit[pp][pa][hs] = valid[pp][pa] ? t * kh[hs] : -INFINITY;
        }
      }
    // ---- online softmax with lazy rescaling (wave-uniform branch)
    bool grow = false;
#pragma unroll
    for (int pp = 0; pp < PP; ++pp)
#pragma unroll
      for (int pa = 0; pa < NACC; ++pa)
#pragma unroll
        for (int hs = 0; hs < 4; ++hs) grow |= logit[pp][pa][hs] > m_run[hs] + kTau;
    if (__any(grow)) {
#pragma unroll
      for (int hs = 0; hs < 4; ++hs) {
        float v = logit[0][0][hs];
#pragma unroll
        for (int pp = 0; pp < PP; ++pp)
#pragma unroll
          for (int pa = 0; pa < NACC; ++pa) v = fmaxf(v, logit[pp][pa][hs]);
        // lanes holding the same head: all 64 (GP = 4) or lane groups of the same parity (GP = 8)
        v = dev::row16_max(v);
        const float r0 = dev::lane_value(v, 0), r1 = dev::lane_value(v, 16);
        const float r2 = dev::lane_value(v, 32), r3 = dev::lane_value(v, 48);
        if (GP == 4)
          v = fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
        else
          v = (gq & 1) ? fmaxf(r1, r3) : fmaxf(r0, r2);
        const float mn = fmaxf(m_run[hs], v);
        const float alpha = __builtin_amdgcn_exp2f(m_run[hs] - mn);
        m_run[hs] = mn;
        l_run[hs] *= alpha;
#pragma unroll
        for (int g = 0; g < NG; ++g) z_run[hs][g] *= alpha;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) acc[nt][hs] *= alpha;
      }
    }
    // ---- probabilities, bf16 hi / lo split of p * s_v, transpose through LDS
#pragma unroll
    for (int pp = 0; pp < PP; ++pp)
#pragma unroll
      for (int pa = 0; pa < NACC; ++pa) {
        const int t = ppos(tok_of(pa));
#pragma unroll
        for (int hs = 0; hs < 4; ++hs) {
          const float pr = __builtin_amdgcn_exp2f(logit[pp][pa][hs] - m_run[hs]);  // 0: invalid
          l_run[hs] += pr;
          const int hd = GP == 4 ? hs : 4 * (gq & 1) + hs;
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            z_run[hs][g] = valid[pp][pa] ? fmaf(pr, vz[pp][pa][g], z_run[hs][g]) : z_run[hs][g];
            const float pt = valid[pp][pa] ? pr * vs[pp][pa][g] : 0.f;
            const __bf16 hi = static_cast<__bf16>(pt);
            const __bf16 lo = static_cast<__bf16>(pt - static_cast<float>(hi));
            pbuf(pp, g, hd)[t] = hi;
            pbuf(pp, g, GP + hd)[t] = lo;
          }
        }
      }
    // LDS operations of one wave execute in order, so the reads below see the writes above; a
    // memory fence here would also wait for the next pages' global loads.
    __builtin_amdgcn_wave_barrier();
    v8bf pa_op[PP][NG][2];
#pragma unroll
    for (int pp = 0; pp < PP; ++pp)
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          pa_op[pp][g][ks] = *reinterpret_cast<const v8bf*>(pbuf(pp, g, n) + 16 * gq + 8 * ks);
    // ---- values
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int g = NG == 2 ? nt / 4 : 0;
#pragma unroll
      for (int pp = 0; pp < PP; ++pp) {
        const uint32_t w = vword(r[pp], nt);
        const uint32_t xs = w & 0x33333333u;          // nibbles: tokens 0, 2, 4, ..., 14
        const uint32_t ys = (w >> 2) & 0x33333333u;   // nibbles: tokens 1, 3, 5, ..., 15
        {
          const v2bf r0 = codes_to_bf16<0>(xs), r1 = codes_to_bf16<1>(xs);
          const v2bf r2 = codes_to_bf16<0>(ys), r3 = codes_to_bf16<1>(ys);
          const v8bf bv = {r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_op[pp][g][0], bv, acc[nt], 0, 0, 0);
        }
        {
          const v2bf r0 = codes_to_bf16<2>(xs), r1 = codes_to_bf16<3>(xs);
          const v2bf r2 = codes_to_bf16<2>(ys), r3 = codes_to_bf16<3>(ys);
          const v8bf bv = {r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_op[pp][g][1], bv, acc[nt], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  // Ping-pong over steps: while one step is processed from one register set, the next step's
  // loads are in flight into the other.  Prefetch indices are clamped to the last
  // page, so every iteration issues the same loads.
  PageRegs x[PP], y[PP];
  int pg = p0 + PP * wave;
  auto load_step = [&](int q, PageRegs* r) {
#pragma unroll
    for (int pp = 0; pp < PP; ++pp) load_page(min(q + pp, p1 - 1), r[pp]);
  };
  if (pg < p1) load_step(pg, x);
  while (pg < p1) {
    load_step(pg + 4 * PP, y);
    process_step(pg, x);
    pg += 4 * PP;
    if (pg >= p1) break;
    load_step(pg + 4 * PP, x);
    process_step(pg, y);
    pg += 4 * PP;
  }

  // ---- finish the wave: sums over lanes of the same head; accumulator rows to LDS (the LDS of
  // the query operands and P tiles is reused, so every wave must be done with it first)
#pragma unroll
  for (int hs = 0; hs < 4; ++hs) {
    // sums over the lanes holding the same head (see the max in the page loop)
    auto head_sum = [&](float v) {
      v = dev::row16_sum(v);
      const float r0 = dev::lane_value(v, 0), r1 = dev::lane_value(v, 16);
      const float r2 = dev::lane_value(v, 32), r3 = dev::lane_value(v, 48);
      return GP == 4 ? (r0 + r1) + (r2 + r3) : ((gq & 1) ? r1 + r3 : r0 + r2);
    };
    const float l = head_sum(l_run[hs]);
    float z[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) z[g] = head_sum(z_run[hs][g]);
    const int hd = GP == 4 ? hs : 4 * (gq & 1) + hs;
    if (n == 0 && gq < GP / 4) {
      red_m[wave][hd] = m_run[hs];
      red_l[wave][hd] = l;
#pragma unroll
      for (int g = 0; g < NG; ++g) red_z[wave][hd][g] = z[g];
    }
  }
  __syncthreads();
#pragma unroll
  for (int nt = 0; nt < 8; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * gq + i;
      if (row < 2 * GP) red_acc[(wave * 2 * GP + row) * kHeadDim + 16 * nt + n] = acc[nt][i];
    }
  __syncthreads();

  // ---- combine the 4 waves and write this split's partial:
  // acc'[h][ch] = sum_w f_w (P_hi row + P_lo row + z_w)  with f_w = 2^(m_w - m)
  float* ml = reinterpret_cast<float*>(a.workspace + p.off_int2_ml);
  float* pacc = reinterpret_cast<float*>(a.workspace + p.off_int2_acc);
  const int nw = min(4, (p1 - p0 + PP - 1) / PP);
  for (int i = threadIdx.x; i < G * kHeadDim; i += 256) {
    const int h = i / kHeadDim, j = i % kHeadDim;
    const int g = NG == 2 ? j / 64 : 0;
    float mm = -INFINITY;
    for (int w = 0; w < nw; ++w) mm = fmaxf(mm, red_m[w][h]);
    float s = 0.f, l = 0.f;
    for (int w = 0; w < nw; ++w) {
      const float f = exp2f(red_m[w][h] - mm);
      s = fmaf(red_acc[(w * 2 * GP + h) * kHeadDim + j] + red_acc[(w * 2 * GP + GP + h) * kHeadDim + j] +
                   red_z[w][h][g],
               f, s);
      l = fmaf(red_l[w][h], f, l);
    }
    const int64_t prow = static_cast<int64_t>(head0 + h) * p.num_splits + split;
    pacc[prow * kHeadDim + j] = s;
    if (j == 0) {
      ml[prow * 2] = mm;
      ml[prow * 2 + 1] = l;
    }
  }
}

// ------------------------------------------------------------------------------------------
// 3. BF16 segments: one 256-thread block per (chunk, kv head, sequence).  Chunk 0 = sink rows
// 0..63, chunk c >= 1 = recent ring rows 64(c-1) .. 64c-1.  The chunk's key and value rows are
// staged in LDS with one round of 16-byte loads (rows that hold no cached token are zeroed: their
// bytes are arbitrary); then thread (token t, head group w) scores heads w, w + 4, ... and thread
// (channel pair c, head group w) accumulates their values.
constexpr int kRowPad = kHeadDim + 8;   // bf16 elements per staged row (breaks bank conflicts)

template <int G>
__global__ __launch_bounds__(256) void bf16_kernel(DecodeArgs a, Plan p, float scale_log2) {
  constexpr int HPW = (G + 3) / 4;   // heads per wave
  __shared__ __attribute__((aligned(16))) uint16_t ks[64][kRowPad];
  __shared__ __attribute__((aligned(16))) uint16_t vsm[64][kRowPad];
  __shared__ float q_s[G][kHeadDim];
  __shared__ float p_s[G][64];
  __shared__ float m_s[G], l_s[G];
  const int chunk = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = dev::lane_id();
  const int L = a.seq_lens[b];
  const int64_t slot = a.seq_slot[b];
  const int head0 = b * p.hq + kv * G;
  const int64_t row0 = chunk == 0 ? (slot * p.hkv + kv) * kSink
                                   : (slot * p.hkv + kv) * kRecent + (chunk - 1) * 64;
  const uint16_t* kb = (chunk == 0 ? a.sink_k : a.recent_k) + row0 * kHeadDim;
  const uint16_t* vb = (chunk == 0 ? a.sink_v : a.recent_v) + row0 * kHeadDim;
  auto row_valid = [&](int t) {
    if (chunk == 0) return t < min(L, kSink);
    const int r = (chunk - 1) * 64 + t;   // ring row
    const int n_recent = min(kRecent, max(0, L - kSink));
    const int start = L - n_recent;
    const int posr = start + (((r - start) % kRecent) + kRecent) % kRecent;
    return n_recent > 0 && posr < L;
  };
  // stage: 64 rows x 16 uint4 per tensor; thread tid takes uint4 c = tid & 15 of rows tid / 16 + 16 i
  {
    uint4 kr[4], vr[4];
    const int c = tid & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = (tid >> 4) + 16 * i;
      const bool ok = row_valid(t);
      kr[i] = ok ? reinterpret_cast<const uint4*>(kb + static_cast<int64_t>(t) * kHeadDim)[c]
                 : make_uint4(0, 0, 0, 0);
      vr[i] = ok ? reinterpret_cast<const uint4*>(vb + static_cast<int64_t>(t) * kHeadDim)[c]
                 : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = (tid >> 4) + 16 * i;
      *reinterpret_cast<uint4*>(&ks[t][8 * c]) = kr[i];
      *reinterpret_cast<uint4*>(&vsm[t][8 * c]) = vr[i];
    }
  }
  for (int i = tid; i < G * kHeadDim; i += 256)
    q_s[i / kHeadDim][i % kHeadDim] =
        dev::bf16_to_f32(a.q[static_cast<int64_t>(head0) * kHeadDim + i]);
  __syncthreads();
  // scores: thread (token lane, wave) for heads wave + 4 j
  const bool valid = row_valid(lane);
  float logit[HPW];
#pragma unroll
  for (int j = 0; j < HPW; ++j) logit[j] = 0.f;
#pragma unroll 4
  for (int c = 0; c < kHeadDim / 8; ++c) {
    const uint4 w = *reinterpret_cast<const uint4*>(&ks[lane][8 * c]);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = __uint_as_float(ws[e] << 16);
      const float hi = __uint_as_float(ws[e] & 0xFFFF0000u);
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        const int h = wave + 4 * j;
        if (h < G) {
          logit[j] = fmaf(q_s[h][8 * c + 2 * e], lo, logit[j]);
          logit[j] = fmaf(q_s[h][8 * c + 2 * e + 1], hi, logit[j]);
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const int h = wave + 4 * j;
    if (h < G) {
      const float lg = valid ? logit[j] * scale_log2 : -INFINITY;
      const float mh = dev::wave_max(lg);
      const float pr = (mh == -INFINITY) ? 0.f : exp2f(lg - mh);
      const float lh = dev::wave_sum(pr);
      p_s[h][lane] = pr;
      if (lane == 0) {
        m_s[h] = mh;
        l_s[h] = lh;
      }
    }
  }
  __syncthreads();
  // values: thread (channel pair lane, wave) for heads wave + 4 j
  float acc[HPW][2];
#pragma unroll
  for (int j = 0; j < HPW; ++j) acc[j][0] = acc[j][1] = 0.f;
#pragma unroll 8
  for (int t = 0; t < 64; ++t) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(&vsm[t][2 * lane]);
    const float lo = __uint_as_float(w << 16);
    const float hi = __uint_as_float(w & 0xFFFF0000u);
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const int h = wave + 4 * j;
      if (h < G) {
        acc[j][0] = fmaf(p_s[h][t], lo, acc[j][0]);
        acc[j][1] = fmaf(p_s[h][t], hi, acc[j][1]);
      }
    }
  }
  float* ml = reinterpret_cast<float*>(a.workspace + p.off_bf16_ml);
  float* pacc = reinterpret_cast<float*>(a.workspace + p.off_bf16_acc);
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const int h = wave + 4 * j;
    if (h < G) {
      const int64_t prow = static_cast<int64_t>(head0 + h) * kBf16Chunks + chunk;
      pacc[prow * kHeadDim + 2 * lane] = acc[j][0];
      pacc[prow * kHeadDim + 2 * lane + 1] = acc[j][1];
      if (lane == 0) {
        ml[prow * 2] = m_s[h];
        ml[prow * 2 + 1] = l_s[h];
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// 4. merge: one 256-thread block per (sequence, query head).
//   (1) weights f_s = 2^(m_s - m) of the INT2 splits (thread s), m and l by block reductions;
//   (2) acc' = sum_s f_s acc'_s with thread (channel quad, split residue mod 8) partial sums;
//   (3) acc'P, then the Hadamard butterflies, then times U_v^T / sqrt(d) (two threads per output);
//   (4) merge with the five BF16 chunk partials and normalise.
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a, Plan p) {
  __shared__ float f_s[kMaxSplits];
  __shared__ __attribute__((aligned(16))) float part[8][kHeadDim];
  __shared__ float vec[kHeadDim];
  __shared__ float outp[2][kHeadDim];
  __shared__ float red[8];
  const int row = blockIdx.x;   // b * hq + head
  const int b = row / p.hq;
  const int kv = (row % p.hq) / p.gqa;
  const int tid = threadIdx.x;
  const int L = a.seq_lens[b];
  const int n_hist = max(0, L - kSink - kRecent);
  const int n_pages = (n_hist + kPage - 1) / kPage;
  const int n_valid = (n_pages + p.pages_per_split - 1) / p.pages_per_split;
  const float* iml = reinterpret_cast<const float*>(a.workspace + p.off_int2_ml) +
                     static_cast<int64_t>(row) * p.num_splits * 2;
  const float* iacc = reinterpret_cast<const float*>(a.workspace + p.off_int2_acc) +
                      static_cast<int64_t>(row) * p.num_splits * kHeadDim;

  // (1) max and weights
  float mloc = -INFINITY;
  for (int s = tid; s < n_valid; s += 256) mloc = fmaxf(mloc, iml[2 * s]);
  mloc = dev::wave_max(mloc);
  if ((tid & 63) == 0) red[tid >> 6] = mloc;
  __syncthreads();
  const float mi = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float lloc = 0.f;
  for (int s = tid; s < n_valid; s += 256) {
    const float f = exp2f(iml[2 * s] - mi);
    f_s[s] = f;
    lloc = fmaf(iml[2 * s + 1], f, lloc);
  }
  lloc = dev::wave_sum(lloc);
  if ((tid & 63) == 0) red[4 + (tid >> 6)] = lloc;
  __syncthreads();
  const float li = red[4] + red[5] + red[6] + red[7];
  // (2) weighted sum of the split accumulators
  {
    const int cq = tid & 31, sr = tid >> 5;
    float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = sr; s < n_valid; s += 8) {
      const float4 v =
          reinterpret_cast<const float4*>(iacc + static_cast<int64_t>(s) * kHeadDim)[cq];
      const float f = f_s[s];
      s4.x = fmaf(v.x, f, s4.x);
      s4.y = fmaf(v.y, f, s4.y);
      s4.z = fmaf(v.z, f, s4.z);
      s4.w = fmaf(v.w, f, s4.w);
    }
    reinterpret_cast<float4*>(part[sr])[cq] = s4;
  }
  __syncthreads();
  if (tid < kHeadDim) {
    // (acc' P)_j = acc'_rev(j)
    const int src = dev::bitrev7(tid);
    float v = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) v += part[r][src];
    vec[tid] = v;
  }
  __syncthreads();
  // (3) Hadamard butterflies, then U_v^T / sqrt(d)
  for (int hs = 1; hs < kHeadDim; hs <<= 1) {
    if (tid < 64) {
      const int i = (tid / hs) * 2 * hs + (tid % hs);
      const float x = vec[i], y = vec[i + hs];
      vec[i] = x + y;
      vec[i + hs] = x - y;
    }
    __syncthreads();
  }
  {
    const int j = tid & 127, half = tid >> 7;
    const float4* u = reinterpret_cast<const float4*>(
        a.u_v + (static_cast<int64_t>(kv) * kHeadDim + j) * kHeadDim + half * 64);
    float o = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const float4 w = u[c];
      const int i = half * 64 + 4 * c;
      o = fmaf(vec[i], w.x, o);
      o = fmaf(vec[i + 1], w.y, o);
      o = fmaf(vec[i + 2], w.z, o);
      o = fmaf(vec[i + 3], w.w, o);
    }
    outp[half][j] = o;
  }
  __syncthreads();
  // (4) merge with the BF16 partials
  if (tid < kHeadDim) {
    const int j = tid;
    const float* bml = reinterpret_cast<const float*>(a.workspace + p.off_bf16_ml) +
                       static_cast<int64_t>(row) * kBf16Chunks * 2;
    const float* bacc = reinterpret_cast<const float*>(a.workspace + p.off_bf16_acc) +
                        static_cast<int64_t>(row) * kBf16Chunks * kHeadDim;
    const float m_int2 = n_valid > 0 ? mi : -INFINITY;
    float mt = m_int2;
    for (int c = 0; c < kBf16Chunks; ++c) mt = fmaxf(mt, bml[2 * c]);
    float acc = 0.f, l = 0.f;
    if (m_int2 != -INFINITY) {
      const float f = exp2f(m_int2 - mt);
      acc = (outp[0][j] + outp[1][j]) * 0.08838834764831845f * f;
      l = li * f;
    }
    for (int c = 0; c < kBf16Chunks; ++c) {
      const float mc = bml[2 * c];
      if (mc == -INFINITY) continue;
      const float f = exp2f(mc - mt);
      acc = fmaf(bacc[c * kHeadDim + j], f, acc);
      l = fmaf(bml[2 * c + 1], f, l);
    }
    a.out[static_cast<int64_t>(row) * kHeadDim + j] = acc / l;
    if (a.lse != nullptr && j == 0) a.lse[row] = (mt + log2f(l)) * 0.6931471805599453f;
  }
}

template <int G>
hipError_t launch_g(const DecodeArgs& a, const Plan& p, uint32_t stages, hipStream_t stream) {
  const float scale_log2 = a.sm_scale * kLog2e;
  if ((stages & OSCAR_STAGE_INT2) && p.max_pages > 0) {
    dim3 grid(p.num_splits, p.hkv, p.batch);
    if (p.n_groups == 1)
      hipLaunchKernelGGL((int2_kernel<G, 1>), grid, dim3(256), 0, stream, a, p);
    else
      hipLaunchKernelGGL((int2_kernel<G, 2>), grid, dim3(256), 0, stream, a, p);
  }
  if (stages & OSCAR_STAGE_BF16)
    hipLaunchKernelGGL((bf16_kernel<G>), dim3(kBf16Chunks, p.hkv, p.batch), dim3(256), 0, stream,
                       a, p, scale_log2);
  if (stages & OSCAR_STAGE_MERGE)
    hipLaunchKernelGGL(merge_kernel, dim3(p.batch * p.hq), dim3(256), 0, stream, a, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, const Plan& p, uint32_t stages,
                         hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  if (stages & OSCAR_STAGE_QUERY) {
    int8_t* qpack = reinterpret_cast<int8_t*>(a.workspace + p.off_qrot);
    float* qmeta = reinterpret_cast<float*>(a.workspace + p.off_sigma);
    hipLaunchKernelGGL(query_kernel, dim3(p.batch * p.hq), dim3(256), 0, stream, a.q, a.u_k, p.hq,
                       p.gqa, p.n_groups, a.sm_scale * kLog2e, qpack, qmeta);
  }
  switch (p.gqa) {
    case 1: return launch_g<1>(a, p, stages, stream);
    case 2: return launch_g<2>(a, p, stages, stream);
    case 4: return launch_g<4>(a, p, stages, stream);
    case 8: return launch_g<8>(a, p, stages, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace oscar
