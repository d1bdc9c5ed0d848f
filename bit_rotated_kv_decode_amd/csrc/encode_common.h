// Encoding steps shared by the bulk demotion and the preparation launch of a decode step: the
// quantiser of a rotated history vector, the stores into the tiled page block, and the rotated
// query's matrix-core operands for the INT2 pass.  Quantiser decisions are
// taken in IEEE fp32 on the rotated vector rounded once from fp64 (steps after the OSCAR write-up
// "超越TurboQuant！OSCAR：面向真实服务的2-bit KV Cache量化", section OSCAR 的设计: clip, per-group
// scale and zero point, four 2-bit codes to a byte).
#pragma once

#include "device_common.h"
#include "oscar_internal.h"

namespace oscar {
namespace enc {

struct LaneCodes {
  uint32_t c0, c1;     // codes of channels lane and lane + 64
  uint32_t meta[2];    // per group: fp16 scale in bits 0..15, fp16 zero in bits 16..31
};

// Clip and quantise the rotated channels (lane, lane + 64) of one vector; all lanes of the wave
// must call this together (the group min / max are wave reductions).  (lv_lo, lv_step) places the
// four levels of an equally spaced codebook at lv_lo + lv_step * c in units of (max - min) / 3
// above the group minimum: the stored scale is (max - min) / 3 * lv_step and the zero point
// min + (max - min) / 3 * lv_lo, every product and sum rounded to fp32 on its own; (0, 1) is the
// plain grid (scale (max - min) / 3, zero point min).  levels_kind 1: (lv_lo, lv_step) = (l0, l1)
// of a codebook symmetric about 1.5, levels (l0, l1, 3 - l1, 3 - l0) in t = (x - z) / s with the
// plain grid's scale and zero point; the code names the nearest level.
__device__ __forceinline__ LaneCodes quantize_lane(double r0, double r1, float clip,
                                                   int n_groups, float lv_lo, float lv_step,
                                                   int levels_kind) {
#pragma clang fp contract(off)
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
  const bool spaced = levels_kind == 0;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const float r3 = (mx[m] - mn[m]) / 3.0f;
    const float s32 = !spaced || lv_step == 1.0f ? r3 : r3 * lv_step;
    const float z32 = !spaced || lv_lo == 0.0f ? mn[m] : mn[m] + r3 * lv_lo;
    const __half s16 = __float2half_rn(s32);
    const __half z16 = __float2half_rn(z32);
    sf[m] = __half2float(s16);
    zf[m] = __half2float(z16);
    out.meta[m] = static_cast<uint32_t>(__half_as_ushort(s16)) |
                  (static_cast<uint32_t>(__half_as_ushort(z16)) << 16);
  }
  if (spaced) {
    auto code = [](float x, float s, float z) -> uint32_t {
      if (s == 0.0f) return 0u;
      const float t = rintf((x - z) / s);
      return static_cast<uint32_t>(fminf(fmaxf(t, 0.0f), 3.0f));
    };
    out.c0 = code(x0, sf[0], zf[0]);
    out.c1 = code(x1, sf[1], zf[1]);
    return out;
  }
  // the number of midpoints strictly below t = (x - z) / s (0 when s is 0): (l0 + l1) / 2, 1.5
  // and 3 - (l0 + l1) / 2 in fp64 (exact from the fp32 levels), so a value on a midpoint takes
  // the lower code
  const double th0 = (static_cast<double>(lv_lo) + static_cast<double>(lv_step)) * 0.5;
  const double th2 = 3.0 - th0;
  auto code = [th0, th2](float x, float s, float z) -> uint32_t {
    const double t = s == 0.0f ? 0.0 : static_cast<double>((x - z) / s);
    return static_cast<uint32_t>(t > th0) + static_cast<uint32_t>(t > 1.5) +
           static_cast<uint32_t>(t > th2);
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
  auto row_or = [](uint32_t v) {   // OR over the 16 lanes of the row (DPP steps)
    v |= dev::dpp<dev::kQuadSwap1>(0u, v);
    v |= dev::dpp<dev::kQuadSwap2>(0u, v);
    v |= dev::dpp<dev::kRowRor4>(0u, v);
    return v | dev::dpp<dev::kRowRor8>(0u, v);
  };
  v0 = row_or(v0);
  v1 = row_or(v1);
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
#pragma unroll
    for (int g = 0; g < 2; ++g)
      if (g < n_groups) m[g] = q.meta[g];
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

// Replace the 2-bit field under `mask` of a value-code word that no other wave writes during the
// launch: a no-return atomic and, then or (same address, same wave: applied in order).
__device__ __forceinline__ void replace_bits(uint32_t* p, uint32_t mask, uint32_t bits) {
  __hip_atomic_fetch_and(p, ~mask, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_fetch_or(p, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Store one token's codes and meta (tensor 0 = K, 1 = V) into its page slot; a whole wave calls
// this with lane l holding rotated channels l and l + 64.
__device__ __forceinline__ void store_token(uint8_t* blk, int tensor, int slot, int n_groups,
                                            const LaneCodes& q) {
  const int lane = dev::lane_id();
  if (tensor == 0) {
    store_key_row(blk, slot, q.c0, q.c1);
  } else {
    uint32_t* vc = reinterpret_cast<uint32_t*>(blk + kVCodesOff);
    const int u = v_code_group(slot);
    const int sh = 2 * v_code_pos(slot);
    replace_bits(&vc[v_word_index(lane, u)], 3u << sh, q.c0 << sh);
    replace_bits(&vc[v_word_index(lane + 64, u)], 3u << sh, q.c1 << sh);
  }
  store_meta(blk, tensor, slot, n_groups, q);
}

// Key operand of the INT2 pass for one query head (lane l holds rotated channels l and l + 64 of
// q' in fp64; a whole wave calls this).  The pass takes q'.codes on the matrix cores as
// v_mfma_scale_f32_16x16x128_f8f6f4 with the query as the fp8 (e4m3) operand A and the stored
// codes as the FP4 operand B.  Rows of A are (head hh of the tile, part p): q'' = q' * scale_log2
// is written as 2^e (16 i + b1 / 16 + b2 / 256 + b3 / 4096) with |q''| / 2^e < 256, i the nearest
// integer to q'' / 2^(e + 4) and each b_p an e4m3 value rounded to nearest from the remainder the
// parts before it leave (q'' to about 2^-16 of its largest element).  Row (hh, 0) holds i with the
// E8M0 row scale 2^(e + 4), row (hh, p) holds b_p with 2^(e - 4 p).  The leading part is an
// integer because the matrix cores add the products of a K-slice with about 16 bits relative to
// the largest one: products that are all multiples of one step sum exactly, and the rows of the
// small remainders lose only bits far below the query's precision.  Channel c sits at the K position its codes take in operand B (key_k_slot).  With
// two groups per vector the tile has one operand per group, the other group's channels zero.
// Also written: the per-group sums of the q'' the parts represent (the zero points multiply them).
// a_ops: the operands of this (sequence, KV head), [tile][group][64 lanes][32 bytes]; scales:
// [tile][group][64 lanes] (E8M0 in byte 0); sig: [group] of this query row.
__device__ __forceinline__ void key_k_slot(int c, int& lane_group, int& byte) {
  // FP4 operand B of the key tile holds, in lane group q, the words of channels 16 q .. 16 q + 15
  // and 64 + 16 q .. as four nibble dwords (even codes, odd codes, even, odd of the second word):
  // K = 32 q + 8 d + m is channel 16 q + 2 m + (d & 1) + 64 (d >> 1).  The fp8 operand A holds K
  // at lane group (K % 64) / 16, byte K % 16 + 16 (K / 64).
  const int q = (c & 63) >> 4, m = (c & 15) >> 1, d = 2 * (c >> 6) + (c & 1);
  const int k = 32 * q + 8 * d + m;
  lane_group = (k & 63) >> 4;
  byte = (k & 15) + 16 * (k >> 6);
}

__device__ __forceinline__ void query_operands(double r0, double r1, int n_groups, int gqa,
                                               int hd, float scale_log2, uint8_t* a_ops,
                                               int32_t* scales, float* sig) {
  typedef float v2f __attribute__((ext_vector_type(2)));
  const int lane = dev::lane_id();
  const int ht = hd >> 2, hh = hd & 3;
  const float f0 = static_cast<float>(r0 * static_cast<double>(scale_log2));
  const float f1 = static_cast<float>(r1 * static_cast<double>(scale_log2));
  const float amax = dev::wave_max(fmaxf(fabsf(f0), fabsf(f1)));
  int ex = 0;
  if (amax > 0.f) {
    frexpf(amax, &ex);   // amax < 2^ex
    ex -= 8;
  }
  ex = max(ex, -110);
  float v0 = ldexpf(f0, -ex), v1 = ldexpf(f1, -ex);
  uint32_t part[4];
  // part 0 on the grid of 16: an integer i in [-16, 16] standing for 16 i (every product of
  // that row is then a multiple of the same step, which the matrix cores sum exactly); parts 1-3
  // are e4m3 values of the remainder scaled by 16, 256 and 4096
  const float i0 = rintf(v0 * 0.0625f), i1 = rintf(v1 * 0.0625f);
  part[0] = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(i0, i1, 0, false)) & 0xFFFFu;
  float rec0 = 16.f * i0, rec1 = 16.f * i1, w = 0.0625f;
  v0 = (v0 - rec0) * 16.f;
  v1 = (v1 - rec1) * 16.f;
#pragma unroll
  for (int p = 1; p < 4; ++p) {
    const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
    const v2f bk = __builtin_amdgcn_cvt_pk_f32_fp8(pk, false);
    part[p] = static_cast<uint32_t>(pk) & 0xFFFFu;
    rec0 = fmaf(bk[0], w, rec0);   // exact: every part has at most 4 significant bits
    rec1 = fmaf(bk[1], w, rec1);
    v0 = (v0 - bk[0]) * 16.f;
    v1 = (v1 - bk[1]) * 16.f;
    w *= 0.0625f;
  }
  const float q0 = ldexpf(rec0, ex), q1 = ldexpf(rec1, ex);
  float s0, s1;
  if (n_groups == 1) {
    s0 = dev::wave_sum(q0 + q1);
    s1 = 0.f;
  } else {
    s0 = dev::wave_sum(q0);
    s1 = dev::wave_sum(q1);
  }
  if (lane == 0) {
    sig[0] = s0;
    sig[1] = s1;
  }
  const int row_head = (lane & 15) >> 2;
  for (int g = 0; g < n_groups; ++g) {
    uint8_t* op = a_ops + static_cast<int64_t>(ht * n_groups + g) * 2048;
    int32_t* sc = scales + (ht * n_groups + g) * 64;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int c = lane + 64 * half;
      const bool in = n_groups == 1 || half == g;
      int lg, e;
      key_k_slot(c, lg, e);
#pragma unroll
      for (int p = 0; p < 4; ++p)
        op[(16 * lg + 4 * hh + p) * 32 + e] =
            in ? static_cast<uint8_t>(part[p] >> (8 * half)) : static_cast<uint8_t>(0);
    }
    if (row_head == hh) {
      const int pt = lane & 3;
      sc[lane] = min(max(127 + ex + (pt == 0 ? 4 : -4 * pt), 0), 254);
    }
    // rows of heads the group does not have (fewer than four query heads per KV head) are zero;
    // the first head writes them
    if (hd == 0 && row_head >= gqa) {
      uint4* z = reinterpret_cast<uint4*>(op + lane * 32);
      z[0] = make_uint4(0, 0, 0, 0);
      z[1] = make_uint4(0, 0, 0, 0);
      sc[lane] = 127;
    }
  }
}

// Split of one rotated query (lane l holds channels l and l + 64, fp64) into the INT2 pass's
// operands: q' ~ a (hi + lo / 256), a = max |q'| / 127, written to dst[0..255] (hi bytes, then lo
// bytes, each in MFMA operand order: channel j = 16 qd + 4 b + k at byte 16 qd + 4 k + b), and
// the query meta (a / 256 * scale_log2, then the per-group sums of 256 hi + lo, exact in int32).
// A whole wave calls this.
__device__ __forceinline__ void split_query(double r0, double r1, int n_groups, float scale_log2,
                                            int8_t* dst, float* meta) {
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
  auto opos = [](int j) { return (j >> 4) * 16 + (j & 3) * 4 + ((j >> 2) & 3); };
  dst[opos(lane)] = static_cast<int8_t>(h0);
  dst[opos(lane + 64)] = static_cast<int8_t>(h1);
  dst[128 + opos(lane)] = static_cast<int8_t>(l0);
  dst[128 + opos(lane + 64)] = static_cast<int8_t>(l1);
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
    meta[0] = sa / 256.f * scale_log2;
    meta[1] = static_cast<float>(s0);
    meta[2] = static_cast<float>(s1);
    meta[3] = 0.f;
  }
}

}  // namespace enc
}  // namespace oscar
