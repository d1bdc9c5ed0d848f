// Encoding steps shared by the bulk demotion and the preparation launch of a decode step: the
// quantiser of a rotated history vector, the stores into the tiled page block, and the split of
// a rotated query into the int8 hi / lo operands of the INT2 pass.  Quantiser decisions are
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
// plain grid (scale (max - min) / 3, zero point min).
__device__ __forceinline__ LaneCodes quantize_lane(double r0, double r1, float clip,
                                                   int n_groups, float lv_lo, float lv_step) {
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
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const float r3 = (mx[m] - mn[m]) / 3.0f;
    const float s32 = lv_step == 1.0f ? r3 : r3 * lv_step;
    const float z32 = lv_lo == 0.0f ? mn[m] : mn[m] + r3 * lv_lo;
    const __half s16 = __float2half_rn(s32);
    const __half z16 = __float2half_rn(z32);
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
    const int u = slot / 16;
    const int sh = 2 * (slot % 16);
    replace_bits(&vc[v_word_index(lane, u)], 3u << sh, q.c0 << sh);
    replace_bits(&vc[v_word_index(lane + 64, u)], 3u << sh, q.c1 << sh);
  }
  store_meta(blk, tensor, slot, n_groups, q);
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
