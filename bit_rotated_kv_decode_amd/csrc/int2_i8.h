// INT2 split-KV pass for tiles of eight query heads or two groups per head: scores as exact int32
// i8 MFMAs (query int8 hi / lo parts written by the preparation launch), values as bf16 MFMAs of
// bf16 hi / lo parts of p * s_v against the codes turned into exact bf16 integers.  Included by
// decode.hip inside its anonymous namespace; the four-head single-group pass is int2_block there.
// For these tiles the fp8 parts of that pass would grow with both the head count and the group
// count, while the bf16 value operand here serves sixteen rows (eight heads, hi and lo) at once.
typedef int v4i __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// The softmax reference of a wave is the maximum logit of its first page; later logits may exceed
// it by up to 2^kRefSpan (p <= 2^64 keeps p * s_v, the value sums and l finite in fp32 / bf16).
constexpr float kRefSpan = 64.0f;
// Pages a wave has in flight or in process: register sets of the page loop.
constexpr int kI8Depth = 2;

// FP4 (E2M1) pair in byte B of x -> two bf16; a 2-bit code zero-extended to a nibble encodes
// code / 2, so the scale 2 gives the code itself.
template <int B>
__device__ __forceinline__ v2bf codes_to_bf16(uint32_t x) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, 2.0f, B);
}

// ------------------------------------------------------------------------------------------
// Block = 4 waves on pages [p0, p1) of one (sequence, KV head).  Wave w takes pages p0 + w + 4 i,
// i = 0, 1, ..., one per step; the next page's loads are in flight while a page is processed
// (two register sets used in turn).
//
// Scores: D[row, token] = sum_k A[row, k] B[k, token] with v_mfma_i32_16x16x64_i8.  B = key codes
// of 16 tokens (lane n + 16 qd holds token n's packed dwords qd and 4 + qd, spread into bytes);
// A = the int8 hi (or lo) part of q' placed in rows 4 st + h (GP = 4) or 8 (st % 2) + h (GP = 8)
// for sub-tile st (zero elsewhere), kept in registers.  The output rows of one sub-tile land in one
// lane group, so after the page's sub-tiles every lane holds the scores of its own token(s) for
// 4 heads, one per register.
// Values: acc[row, ch] += sum_t P[row, t] V[t, ch] with v_mfma_f32_16x16x32_bf16; P rows are the
// bf16 hi and lo parts of p * s_v for each head, transposed through LDS; V = value codes turned
// into exact bf16 integers by the FP4 conversion path.
// LDS carve-up of an INT2 block: per-wave P tiles, and apart from them the per-wave accumulator
// rows and softmax statistics that the block combines at the end.
template <int G, int NG>
struct Int2LdsI8 {
  static constexpr int GP = G <= 4 ? 4 : 8;
  static constexpr int PB = 4 * NG * 16 * kPage * 2;         // [wave][g][row][token] bf16
  static constexpr int RED = PB;                             // [wave][head][ch] fp32
  static constexpr int RED_M = RED + 4 * G * kHeadDim * 4;   // [wave][GP] fp32
  static constexpr int RED_L = RED_M + 4 * 4 * GP;
  static constexpr int TOTAL = RED_L + 4 * 4 * GP;
};

// STREAM: history pages are fetched with non-temporal loads.  Chosen when the launch holds one
// sequence, so no page is read twice in it; with several sequences pages may be shared (a prefix
// cache), and cached loads let the second reader hit.
template <int G, int NG, bool STREAM>
__device__ __forceinline__ void int2_block_i8(const DecodeArgs& a, const Plan& p, int split,
                                              int kv, int b, unsigned char* smem) {
  using S = Int2LdsI8<G, NG>;
  constexpr int GP = S::GP;               // padded query heads per KV head
  constexpr int NACC = GP / 4;            // score accumulators (tokens per lane and page)
  constexpr int PP = 1;                   // pages per step
  constexpr int BLK = kMetaOff + kPage * 8 * NG;
  __bf16* pbuf_all = reinterpret_cast<__bf16*>(smem);
  float* red_acc = reinterpret_cast<float*>(smem + S::RED);
  float (*red_m)[GP] = reinterpret_cast<float (*)[GP]>(smem + S::RED_M);
  float (*red_l)[GP] = reinterpret_cast<float (*)[GP]>(smem + S::RED_L);

  const int p0 = split * p.pages_per_split;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = dev::lane_id();
  const int gq = lane >> 4, n = lane & 15;
  const int head0 = b * p.hq + kv * G;
  // Table entries of this wave's pages p0 + wave + 4 j, one per lane j (at most 64: a split
  // covers at most 256 pages), read before the sequence length is known so that the first page
  // loads wait on one memory round trip only.  The index stays inside the table row; entries of
  // pages past the sequence's end are read but never used.
  static_assert(PP == 1 && kMaxPagesPerSplit <= 4 * 64, "one page id per lane and wave");
  const int wave_ids = a.page_table[static_cast<int64_t>(b) * a.max_pages_per_seq +
                                    min(p0 + wave + 4 * lane, a.max_pages_per_seq - 1)];
  const int L = a.seq_lens[b] + a.len_add;
  const int n_hist = max(0, L - kSink - kRecent);
  const int n_pages = (n_hist + kPage - 1) / kPage;
  if (p0 >= n_pages) return;
  const int p1 = min(p0 + p.pages_per_split, n_pages);

  // ---- query operands (registers, the same for every page).  Score tile rows hold the int8 hi
  // part of a head's q' and, four rows further, its lo part; GP = 4: operand ts (sub-tiles of
  // parity ts) fills rows 8 ts .. 8 ts + 7; GP = 8: rows 0..7 hi and 8..15 lo of heads 0..7.  Lane
  // (k block gq, row n) holds channels [16 gq, 16 gq + 16) of half hf (MFMA operand order).
  const int8_t* qpack = reinterpret_cast<const int8_t*>(a.workspace + p.off_qrot);
  const float* qmeta = reinterpret_cast<const float*>(a.workspace + p.off_sigma);
  v4i qa[GP == 4 ? 2 : 1][2];
  {
    const int ts = GP == 4 ? n / 8 : 0;
    const int hl = GP == 4 ? (n / 4) % 2 : n / 8;
    const int hd = GP == 4 ? n % 4 : n % 8;
#pragma unroll
    for (int t = 0; t < (GP == 4 ? 2 : 1); ++t)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        v4i v = {0, 0, 0, 0};
        if (t == ts && hd < G)
          v = *reinterpret_cast<const v4i*>(qpack + static_cast<int64_t>(head0 + hd) * 256 +
                                            hl * 128 + (hf * 4 + gq) * 16);
        qa[t][hf] = v;
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
  // Combines the per-row results of a 16-lane reduction over the rows holding the same head: all
  // four rows (GP = 4) or rows r and r ^ 2 (GP = 8), with lane swaps; every lane gets the result.
  auto head_reduce = [](float v, auto op) {
    if constexpr (GP == 4) {
      const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
      v = op(__uint_as_float(s16[0]), __uint_as_float(s16[1]));   // rows (0 + 1), (2 + 3)
    }
    const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return op(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
  };
  // token (within a page) of this lane's score vector pa: after the hi / lo lane swap, lane group
  // gq holds sub-tile (0, 2, 1, 3)[gq] (GP = 4) or sub-tile 2 pa + gq / 2 (GP = 8)
  auto tok_of = [&](int pa) {
    return GP == 4 ? 16 * (((gq & 1) << 1) | (gq >> 1)) + n : 16 * (2 * pa + (gq >> 1)) + n;
  };
  // position of a token in a P row.  The value operand of MFMA ks in lane group u holds the codes
  // at word positions 8 ks + {0, 2, 4, 6, 1, 3, 5, 7} of word group u (even positions from the
  // mask, odd ones from the shifted mask), so token t sits at entry 16 u + 8 ks + e of the row,
  // with (u, 8 ks + pos_e) = (v_code_group(t), v_code_pos(t)).
  auto ppos = [](int t) {
    const int pos = v_code_pos(t);
    return 16 * v_code_group(t) + ((pos & 8) | ((pos & 7) >> 1) | ((pos & 1) << 2));
  };
  auto pbuf = [&](int pp, int g, int row) -> __bf16* {
    return pbuf_all + ((((wave * PP + pp) * NG + g) * 16 + row) * kPage);
  };
  // rows 2 GP .. 15 of every P tile stay zero (value operands of unused rows): 8 rows x 64
  // tokens x 2 bytes = 64 lanes x 16 bytes per tile.  The tiles are the wave's own and LDS
  // operations of one wave execute in order, so no barrier is needed before the page loop.
  if constexpr (2 * GP == 8) {
#pragma unroll
    for (int pp = 0; pp < PP; ++pp)
#pragma unroll
      for (int g = 0; g < NG; ++g)
        reinterpret_cast<uint4*>(pbuf(pp, g, 2 * GP))[lane] = make_uint4(0, 0, 0, 0);
  }

  float m_ref[4], m_lim[4], l_run[4], z_run[4][NG];   // m_lim = m_ref + kRefSpan
  v4f acc[8];
  auto reset_sums = [&]() {
#pragma unroll
    for (int hs = 0; hs < 4; ++hs) {
      l_run[hs] = 0.f;
#pragma unroll
      for (int g = 0; g < NG; ++g) z_run[hs][g] = 0.f;
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[nt] = v4f{0.f, 0.f, 0.f, 0.f};
  };
#pragma unroll
  for (int hs = 0; hs < 4; ++hs) {
    m_ref[hs] = -INFINITY;   // a wave without pages leaves -inf (its partial weighs nothing)
    m_lim[hs] = -INFINITY;
  }
  reset_sums();

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
    // lane (pg - p0 - wave) / 4 holds page pg's id; a clamped prefetch index p1 - 1 maps to the
    // wave's last page below p1 (floor division), whose id is valid
    const int pid = __builtin_amdgcn_readlane(wave_ids, (pg - p0 - wave) >> 2);
    const uint8_t* blk = a.pool + (static_cast<int64_t>(pid) * p.hkv + kv) * BLK;
    const uint4* kc = reinterpret_cast<const uint4*>(blk + kKCodesOff);
    const uint4* vc = reinterpret_cast<const uint4*>(blk + kVCodesOff);
    auto ld = [](const auto* q) { return STREAM ? dev::load_stream(q) : *q; };
    r.k[0] = ld(&kc[lane]);
    r.k[1] = ld(&kc[64 + lane]);
    r.v[0] = ld(&vc[lane]);
    r.v[1] = ld(&vc[64 + lane]);
#pragma unroll
    for (int pa = 0; pa < NACC; ++pa) {
      // The meta region lies past the immediate-offset range of a global load, and a global
      // load there takes a per-page 64-bit vector address whose register makes the next page's
      // loads wait for every load in flight; a buffer load over the block takes the block
      // address in scalar registers and the lane's offset in one loop-invariant register.
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(blk), 0, BLK, kBufferWord3);
      const int moff = kMetaOff + tok_of(pa) * 8 * NG;
      if (NG == 1) {
        const uint2 w = dev::to_uint2(__builtin_amdgcn_raw_buffer_load_b64(rs, moff, 0, STREAM ? kNonTemporal : 0));
        r.km[pa][0] = w.x;
        r.vm[pa][0] = w.y;
      } else {
        const uint4 w = dev::to_uint4(__builtin_amdgcn_raw_buffer_load_b128(rs, moff, 0, STREAM ? kNonTemporal : 0));
        r.km[pa][0] = w.x;
        r.km[pa][NG - 1] = w.y;
        r.vm[pa][0] = w.z;
        r.vm[pa][NG - 1] = w.w;
      }
    }
  };

  // Per-page work in two parts: the logits (with the value scales and zero points they come
  // with), then probabilities and values.  Pages pg .. pg + PP - 1 are on register sets
  // r[0 .. PP - 1]; pages past p1 contribute nothing.
  struct Scores {
    float logit[PP][NACC][4];
    float vs[PP][NACC][NG], vz[PP][NACC][NG];
  };
  auto page_scores = [&](int pg, const PageRegs* r, Scores& so) {
    // ---- scores: exact int32 tiles of hi and lo dot products, then one lane swap per register
    // puts hi and lo of the same token in one lane: S = 256 hi + lo
    constexpr int NT = GP == 4 ? 2 : 4;
    int sc[PP][NACC][NG][4];
#pragma unroll
    for (int pp = 0; pp < PP; ++pp) {
      v4i dt[NG][NT];
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int t = 0; t < NT; ++t) dt[g][t] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int g = NG == 2 ? hf : 0;
          const uint32_t w = kword(r[pp], st, hf);
          const v4i bk = {static_cast<int>(w & 0x03030303u),
                          static_cast<int>((w >> 2) & 0x03030303u),
                          static_cast<int>((w >> 4) & 0x03030303u),
                          static_cast<int>((w >> 6) & 0x03030303u)};
          if constexpr (GP == 4)
            dt[g][st >> 1] =
                __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[st & 1][hf], bk, dt[g][st >> 1], 0, 0, 0);
          else
            dt[g][st] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[0][hf], bk, dt[g][st], 0, 0, 0);
        }
#pragma unroll
      for (int pa = 0; pa < NACC; ++pa)
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
          for (int hs = 0; hs < 4; ++hs) {
            // GP = 4: tiles (sub-tiles 0,1) and (2,3) hold rows [hi, lo, hi, lo] per lane group;
            // GP = 8: tiles of sub-tiles 2 pa and 2 pa + 1 hold [hi, hi, lo, lo]
            const uint32_t x = static_cast<uint32_t>(dt[g][GP == 4 ? 0 : 2 * pa][hs]);
            const uint32_t y = static_cast<uint32_t>(dt[g][GP == 4 ? 1 : 2 * pa + 1][hs]);
            const auto sw = GP == 4 ? __builtin_amdgcn_permlane16_swap(x, y, false, false)
                                    : __builtin_amdgcn_permlane32_swap(x, y, false, false);
            sc[pp][pa][g][hs] = (static_cast<int>(sw[0]) << 8) + static_cast<int>(sw[1]);
          }
    }
    bool valid[PP][NACC];
#pragma unroll
    for (int pp = 0; pp < PP; ++pp)
#pragma unroll
      for (int pa = 0; pa < NACC; ++pa) {
        // a slot past the history holds arbitrary bytes: its meta is replaced by zeros (finite
        // scores, no value contribution) and its logit by -inf
        valid[pp][pa] = (pg + pp) * kPage + tok_of(pa) < n_hist && pg + pp < p1;
        float ks[NG], kz[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const uint32_t km = valid[pp][pa] ? r[pp].km[pa][g] : 0u;
          const uint32_t vm = valid[pp][pa] ? r[pp].vm[pa][g] : 0u;
          ks[g] = __half2float(__ushort_as_half(static_cast<uint16_t>(km & 0xFFFF)));
          kz[g] = __half2float(__ushort_as_half(static_cast<uint16_t>(km >> 16)));
          so.vs[pp][pa][g] = __half2float(__ushort_as_half(static_cast<uint16_t>(vm & 0xFFFF)));
          so.vz[pp][pa][g] = __half2float(__ushort_as_half(static_cast<uint16_t>(vm >> 16)));
        }
        const float bias = valid[pp][pa] ? 0.f : -INFINITY;
#pragma unroll
        for (int hs = 0; hs < 4; ++hs) {
          float t = 0.f;
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            t = fmaf(ks[g], static_cast<float>(sc[pp][pa][g][hs]), fmaf(kz[g], sq[hs][g], t));
          }
          so.logit[pp][pa][hs] = fmaf(t, kh[hs], bias);
        }
      }
  };
  // maximum of head slot hs over the page, the same in every lane holding the head
  auto page_max = [&](const Scores& so, int hs) {
    float v = so.logit[0][0][hs];
#pragma unroll
    for (int pp = 0; pp < PP; ++pp)
#pragma unroll
      for (int pa = 0; pa < NACC; ++pa) v = fmaxf(v, so.logit[pp][pa][hs]);
    return head_reduce(dev::row16_max(v), [](float a, float b) { return fmaxf(a, b); });
  };
  auto set_ref = [&](int hs, float m) {
    m_ref[hs] = m;
    m_lim[hs] = m + kRefSpan;
  };
  // lanes holding a logit past the limit, one ballot per compare
  auto over_limit = [&](const Scores& so) {
    uint64_t over = 0;
#pragma unroll
    for (int pp = 0; pp < PP; ++pp)
#pragma unroll
      for (int pa = 0; pa < NACC; ++pa)
#pragma unroll
        for (int hs = 0; hs < 4; ++hs)
          over |= __builtin_amdgcn_ballot_w64(so.logit[pp][pa][hs] > m_lim[hs]);
    return over;
  };
  auto page_values = [&](const PageRegs* r, const Scores& so) {
    // ---- probabilities, bf16 hi / lo split of p * s_v, transpose through LDS
#pragma unroll
    for (int pp = 0; pp < PP; ++pp)
#pragma unroll
      for (int pa = 0; pa < NACC; ++pa) {
        const int t = ppos(tok_of(pa));
#pragma unroll
        for (int hs = 0; hs < 4; ++hs) {
          const float pr = __builtin_amdgcn_exp2f(so.logit[pp][pa][hs] - m_ref[hs]);  // 0: invalid slot
          l_run[hs] += pr;
          const int hd = GP == 4 ? hs : 4 * (gq & 1) + hs;
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            z_run[hs][g] = fmaf(pr, so.vz[pp][pa][g], z_run[hs][g]);
            const float pt = pr * so.vs[pp][pa][g];
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
        const uint32_t xs = w & 0x33333333u;          // nibbles: word positions 0, 2, ..., 14
        const uint32_t ys = (w >> 2) & 0x33333333u;   // nibbles: word positions 1, 3, ..., 15
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


  // kI8Depth register sets used in turn: while one page is processed, the loads of the wave's next
  // kI8Depth - 1 pages are in flight.  Prefetch indices are clamped to the last page, so every round
  // issues the same loads (the wait before a page then never covers a later one's), and the loop
  // over full rounds has a single exit, so the compiler's wait counts stay exact across it.
  // The first page of the wave sets the softmax reference; nothing rescales the accumulators
  // afterwards.  Should a later logit pass the reference by more than 2^kRefSpan, the wave finds
  // its exact maxima in a scores-only pass and takes its pages again from zero (second attempt,
  // which cannot pass them).
  PageRegs r[kI8Depth][PP];
  Scores so;
  auto load_step = [&](int q, PageRegs* rr) {
#pragma unroll
    for (int pp = 0; pp < PP; ++pp) load_page(min(q + pp, p1 - 1), rr[pp]);
  };
  constexpr int WS = 4 * PP;   // page stride of a wave (four waves per block)
  // Issue priority by the pages a wave has left (including the current one): the arbiter
  // otherwise favours the older of the two blocks sharing a compute unit throughout, which then
  // finishes well before the younger one, and the younger one ends its pages alone at one wave
  // per SIMD.  Waves far from their end run first, so the two blocks finish together.
  auto set_prio = [&](int pg_now) {
    const int rem = (p1 - pg_now + WS - 1) / WS;
    if (rem >= 6)
      __builtin_amdgcn_s_setprio(3);
    else if (rem >= 4)
      __builtin_amdgcn_s_setprio(2);
    else if (rem >= 2)
      __builtin_amdgcn_s_setprio(1);
    else
      __builtin_amdgcn_s_setprio(0);
  };
  for (int attempt = 0; p0 + PP * wave < p1; ++attempt) {
    int pg = p0 + PP * wave;
    uint64_t over = 0;
    set_prio(pg);
#pragma unroll
    for (int k = 0; k < kI8Depth; ++k) load_step(pg + k * WS, r[k]);
    page_scores(pg, r[0], so);
    if (attempt == 0) {
#pragma unroll
      for (int hs = 0; hs < 4; ++hs) set_ref(hs, page_max(so, hs));
    }
    page_values(r[0], so);
    pg += WS;
    int rest = (p1 - pg + WS - 1) / WS;   // pages of the wave after the first
    for (; rest >= kI8Depth; rest -= kI8Depth) {
#pragma unroll
      for (int k = 0; k < kI8Depth; ++k) {
        set_prio(pg);
        load_step(pg + (kI8Depth - 1) * WS, r[k]);
        page_scores(pg, r[(k + 1) % kI8Depth], so);
        over |= over_limit(so);
        page_values(r[(k + 1) % kI8Depth], so);
        pg += WS;
        // keep the scheduler from pulling a later page's work (and the wait for its loads)
        // into this one
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int k = 0; k < kI8Depth - 1; ++k) {
      if (k < rest) {
        set_prio(pg);
        page_scores(pg, r[(k + 1) % kI8Depth], so);
        over |= over_limit(so);
        page_values(r[(k + 1) % kI8Depth], so);
        pg += WS;
      }
    }
    if (over == 0) break;
    // exact maxima over the wave's pages, then a second attempt from zero
    float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    for (int q = p0 + PP * wave; q < p1; q += WS) {
      load_step(q, r[0]);
      page_scores(q, r[0], so);
#pragma unroll
      for (int hs = 0; hs < 4; ++hs) mx[hs] = fmaxf(mx[hs], page_max(so, hs));
    }
#pragma unroll
    for (int hs = 0; hs < 4; ++hs) set_ref(hs, mx[hs]);
    reset_sums();
  }

  // ---- finish the wave: l and z summed over the lanes holding each head; each accumulator row
  // as hi + lo + z.  acc[nt][hs] of lane (gq, n) is tile row 4 gq + hs of channel 16 nt + n, the
  // rows being [hi | lo] of heads 0-3 (GP = 4) or [hi 0-7 | lo 0-7] (GP = 8), so one swap of lane
  // groups 0 <-> 1 (GP = 4) or of wave halves (GP = 8) meets each hi row with its lo row.  The
  // rows go to the wave's own LDS rows [wave][head][ch], apart from every P tile, so a single
  // barrier orders them before the combine.
  auto head_sum = [&](float v) {   // over the lanes of one head, as for the max in the page loop
    return head_reduce(dev::row16_sum(v), [](float a, float b) { return a + b; });
  };
  float zs[4][NG];
#pragma unroll
  for (int hs = 0; hs < 4; ++hs) {
    const float l = head_sum(l_run[hs]);
#pragma unroll
    for (int g = 0; g < NG; ++g) zs[hs][g] = head_sum(z_run[hs][g]);
    const int hd = GP == 4 ? hs : 4 * (gq & 1) + hs;
    if (n == 0 && gq < GP / 4) {
      red_m[wave][hd] = m_ref[hs];
      red_l[wave][hd] = l;
    }
  }
#pragma unroll
  for (int nt = 0; nt < 8; ++nt)
#pragma unroll
    for (int hs = 0; hs < 4; ++hs) {
      const uint32_t x = __float_as_uint(acc[nt][hs]);
      const auto sw = GP == 4 ? __builtin_amdgcn_permlane16_swap(x, x, false, false)
                              : __builtin_amdgcn_permlane32_swap(x, x, false, false);
      acc[nt][hs] = (__uint_as_float(sw[0]) + __uint_as_float(sw[1])) +   // hi + lo
                    zs[hs][NG == 2 ? nt / 4 : 0];
    }
  if (gq < GP / 4) {
    float* red_w = red_acc + wave * G * kHeadDim;
#pragma unroll
    for (int hs = 0; hs < 4; ++hs) {
      const int hd = GP == 4 ? hs : 4 * (gq & 1) + hs;
      if (G % 4 == 0 || hd < G) {
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) red_w[hd * kHeadDim + 16 * nt + n] = acc[nt][hs];
      }
    }
  }
  __syncthreads();
  // ---- combine the 4 waves and write this split's partial:
  // acc'[h][ch] = sum_w f_w (P_hi row + P_lo row + z_w)  with f_w = 2^(m_w - m).  Every wave has
  // written its rows (a wave without pages: m = -inf, l = 0, zero rows, so f_w = 0), and every
  // LDS read below is issued before the first one is used.
  float* ml = reinterpret_cast<float*>(a.workspace + p.off_int2_ml);
  float* pacc = reinterpret_cast<float*>(a.workspace + p.off_int2_acc);
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
    const float mm = fmaxf(fmaxf(mw[0], mw[1]), fmaxf(mw[2], mw[3]));   // finite: wave 0 has a page
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

