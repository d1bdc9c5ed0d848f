// Wave-level device helpers for gfx950 (64-lane wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace oscar {
namespace dev {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Loads of data a launch reads once (history pages): non-temporal, so the stream does not
// displace what later launches read again (rotation matrices, partials).
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  const u4 t = __builtin_nontemporal_load(reinterpret_cast<const u4*>(p));
  return make_uint4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ uint2 load_stream(const uint2* p) {
  typedef unsigned int u2 __attribute__((ext_vector_type(2)));
  const u2 t = __builtin_nontemporal_load(reinterpret_cast<const u2*>(p));
  return make_uint2(t[0], t[1]);
}

// Vector results of the buffer-load builtins as HIP vector structs.
__device__ __forceinline__ uint2 to_uint2(unsigned int __attribute__((ext_vector_type(2))) t) {
  return make_uint2(t[0], t[1]);
}
__device__ __forceinline__ uint4 to_uint4(unsigned int __attribute__((ext_vector_type(4))) t) {
  return make_uint4(t[0], t[1], t[2], t[3]);
}

// 7-bit bit reversal of a channel index in [0, 128).
__device__ __forceinline__ int bitrev7(int j) {
  return static_cast<int>(__builtin_bitreverse32(static_cast<uint32_t>(j)) >> 25);
}

// DPP move of a 32-bit value: lane l receives the source lane that `ctrl` selects within its row
// of 16 (row_mask / bank_mask all on; lanes without a source keep `old`).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(old),
                                                           static_cast<int>(v), CTRL, 0xF, 0xF,
                                                           false));
}
constexpr int kQuadSwap1 = 0xB1;   // quad_perm [1, 0, 3, 2]: lane l ^ 1
constexpr int kQuadSwap2 = 0x4E;   // quad_perm [2, 3, 0, 1]: lane l ^ 2
constexpr int kRowShl4 = 0x104;    // lane l + 4 (within the row)
constexpr int kRowShr4 = 0x114;    // lane l - 4
constexpr int kRowRor4 = 0x124;    // lane (l + 4) mod 16
constexpr int kRowRor8 = 0x128;    // lane (l + 8) mod 16 = l ^ 8

// Reduction of a 32-bit value over the whole wave without LDS traffic: DPP steps within each
// row of 16, then the swaps of rows 0 <-> 1, 2 <-> 3 and of the wave halves.  Every lane gets
// the result.  Requires all 64 lanes active.
template <class T, class Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  auto bits = [](T x) { return __builtin_bit_cast(uint32_t, x); };
  auto val = [](uint32_t x) { return __builtin_bit_cast(T, x); };
  v = op(v, val(dpp<kQuadSwap1>(0u, bits(v))));
  v = op(v, val(dpp<kQuadSwap2>(0u, bits(v))));
  v = op(v, val(dpp<kRowRor4>(0u, bits(v))));
  v = op(v, val(dpp<kRowRor8>(0u, bits(v))));
  const auto s16 = __builtin_amdgcn_permlane16_swap(bits(v), bits(v), false, false);
  v = op(val(s16[0]), val(s16[1]));
  const auto s32 = __builtin_amdgcn_permlane32_swap(bits(v), bits(v), false, false);
  return op(val(s32[0]), val(s32[1]));
}

__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}

__device__ __forceinline__ float wave_min(float v) {
  return wave_reduce(v, [](float a, float b) { return fminf(a, b); });
}

__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float a, float b) { return a + b; });
}

// Max / sum over each row of 16 lanes with DPP moves (no LDS traffic): after the call every lane
// holds the result for its row.  Steps: swap neighbours (quad_perm 1,0,3,2), swap pairs
// (quad_perm 2,3,0,1), rotate the row by 4, rotate by 8.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, 0)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, 0)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, 0)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, 0)));
  return v;
}

__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, 0));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, 0));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, 0));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, 0));
  return v;
}

// Value of lane `src` (a constant) of a wave-uniform computation.
__device__ __forceinline__ float lane_value(float v, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

__device__ __forceinline__ int wave_sum_i(int v) {
  return wave_reduce(v, [](int a, int b) { return a + b; });
}

// Value of lane l ^ M for a 64-bit value (M in 1, 2, 4, 8: within the row of 16, by DPP).
template <int M>
__device__ __forceinline__ double lane_xor_dpp(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  uint32_t lo = static_cast<uint32_t>(u), hi = static_cast<uint32_t>(u >> 32);
  if constexpr (M == 1) {
    lo = dpp<kQuadSwap1>(0u, lo);
    hi = dpp<kQuadSwap1>(0u, hi);
  } else if constexpr (M == 2) {
    lo = dpp<kQuadSwap2>(0u, lo);
    hi = dpp<kQuadSwap2>(0u, hi);
  } else if constexpr (M == 8) {
    lo = dpp<kRowRor8>(0u, lo);
    hi = dpp<kRowRor8>(0u, hi);
  } else {
    static_assert(M == 4, "lane distance");
    const bool up = (lane_id() & 4) != 0;
    const uint32_t lo_d = dpp<kRowShr4>(0u, lo), hi_d = dpp<kRowShr4>(0u, hi);
    const uint32_t lo_u = dpp<kRowShl4>(0u, lo), hi_u = dpp<kRowShl4>(0u, hi);
    lo = up ? lo_d : lo_u;
    hi = up ? hi_d : hi_u;
  }
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

// Value of lane l ^ M for a 32-bit value (M in 1, 2, 4, 8: within the row of 16, by DPP).
template <int M>
__device__ __forceinline__ float lane_xor_dpp(float v) {
  const uint32_t u = __float_as_uint(v);
  if constexpr (M == 1) return __uint_as_float(dpp<kQuadSwap1>(0u, u));
  if constexpr (M == 2) return __uint_as_float(dpp<kQuadSwap2>(0u, u));
  if constexpr (M == 8) return __uint_as_float(dpp<kRowRor8>(0u, u));
  static_assert(M == 1 || M == 2 || M == 4 || M == 8, "lane distance");
  const bool up = (lane_id() & 4) != 0;
  const uint32_t d = dpp<kRowShr4>(0u, u), w = dpp<kRowShl4>(0u, u);
  return __uint_as_float(up ? d : w);
}

// The butterfly stage below on a 32-bit value.
template <int H>
__device__ __forceinline__ float butterfly(float y) {
  const bool upper = (lane_id() & H) != 0;
  if constexpr (H >= 16) {
    const uint32_t u = __float_as_uint(y);
    const auto sw = H == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                            : __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float a = __uint_as_float(sw[0]), b = __uint_as_float(sw[1]);
    return upper ? (a - b) : (a + b);
  } else {
    const float p = lane_xor_dpp<H>(y);
    return upper ? (p - y) : (y + p);
  }
}

// One butterfly stage of distance H (a power of two below 64) on a 64-bit value: a lane with bit
// H clear returns y + partner, a lane with it set partner - y.  H = 16 and 32 use the row and
// half-wave swaps (which hand every lane both values of its pair), the others DPP.
template <int H>
__device__ __forceinline__ double butterfly(double y) {
  const bool upper = (lane_id() & H) != 0;
  if constexpr (H >= 16) {
    const uint64_t u = __builtin_bit_cast(uint64_t, y);
    const uint32_t lo = static_cast<uint32_t>(u), hi = static_cast<uint32_t>(u >> 32);
    const auto sl = H == 16 ? __builtin_amdgcn_permlane16_swap(lo, lo, false, false)
                            : __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto sh = H == 16 ? __builtin_amdgcn_permlane16_swap(hi, hi, false, false)
                            : __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    // element [0]: the value of the pair's lower lane, [1]: of its upper lane
    const double a = __builtin_bit_cast(double, (static_cast<uint64_t>(sh[0]) << 32) | sl[0]);
    const double b = __builtin_bit_cast(double, (static_cast<uint64_t>(sh[1]) << 32) | sl[1]);
    return upper ? (a - b) : (a + b);
  } else {
    const double p = lane_xor_dpp<H>(y);
    return upper ? (p - y) : (y + p);
  }
}

// Hadamard butterflies across a wave on the vector held as (y0 = element l, y1 = element l + 64)
// in lane l, followed by the bit-reversal gather and the 1/sqrt(128) scaling: on return lane l
// holds rotated channels l (o0) and l + 64 (o1).  Stage 64 is within the lane; stages 32..1 pair
// lane l with l ^ h.  x'_j = z_rev(j): rev(l) = r is even for l < 64 and rev(l + 64) = r + 1, so
// z[r] sits in lane r & 63 (slot r >> 6) and z[r + 1] in the next lane, same slot.
__device__ __forceinline__ void hadamard_bitrev(double y0, double y1, double& o0, double& o1) {
  const int lane = lane_id();
  {
    const double a = y0 + y1;
    const double b = y0 - y1;
    y0 = a;
    y1 = b;
  }
  y0 = butterfly<32>(y0);
  y1 = butterfly<32>(y1);
  y0 = butterfly<16>(y0);
  y1 = butterfly<16>(y1);
  y0 = butterfly<8>(y0);
  y1 = butterfly<8>(y1);
  y0 = butterfly<4>(y0);
  y1 = butterfly<4>(y1);
  y0 = butterfly<2>(y0);
  y1 = butterfly<2>(y1);
  y0 = butterfly<1>(y0);
  y1 = butterfly<1>(y1);
  const double inv_sqrt_d = 0.08838834764831845;  // 1 / sqrt(128)
  const int r = bitrev7(lane);
  const int src = r & 63;
  const bool hi = (r >> 6) != 0;
  const double a0 = __shfl(y0, src);
  const double a1 = __shfl(y1, src);
  const double b0 = __shfl(y0, src + 1);
  const double b1 = __shfl(y1, src + 1);
  o0 = (hi ? a1 : a0) * inv_sqrt_d;
  o1 = (hi ? b1 : b0) * inv_sqrt_d;
}

// Rotation of one row vector x (fp32 in LDS, 128 entries) by R = U H P / sqrt(128) in fp64 by a
// whole 256-thread block: thread t accumulates rows [16 g, 16 g + 16) (g = t / 32) of x U for
// columns 4 c .. 4 c + 3 (c = t % 32), wave 0 adds the eight partial vectors (staged in `red`) and
// finishes with the Hadamard and the bit reversal.  The U entries a thread needs (16 float4 rows
// slices) are loaded into registers first (load_u_rows), so the loads can be in flight while x
// is still being staged.  Every thread of the block must call rotate1_block (it contains a block
// barrier); it returns true in wave 0, whose lane l then holds rotated channels l and l + 64.
constexpr int kRotGroups = 8;   // row groups of the block rotation (red holds one vector each)

struct URows {
  float4 v[16];   // U[16 g + k][4 c .. 4 c + 3]
};

__device__ __forceinline__ void load_u_rows(const float* __restrict__ u, URows& r) {
  const int g = threadIdx.x >> 5, c = threadIdx.x & 31;
#pragma unroll
  for (int k = 0; k < 16; ++k)
    r.v[k] = reinterpret_cast<const float4*>(u + (16 * g + k) * 128)[c];
}

__device__ __forceinline__ bool rotate1_block(const float* x, const URows& ur,
                                              double (*red)[128], double& o0, double& o1) {
  const int g = threadIdx.x >> 5, c = threadIdx.x & 31;
  double y[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const double xi = static_cast<double>(x[16 * g + k]);
    y[0] = fma(xi, static_cast<double>(ur.v[k].x), y[0]);
    y[1] = fma(xi, static_cast<double>(ur.v[k].y), y[1]);
    y[2] = fma(xi, static_cast<double>(ur.v[k].z), y[2]);
    y[3] = fma(xi, static_cast<double>(ur.v[k].w), y[3]);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) red[g][4 * c + e] = y[e];
  __syncthreads();
  if ((threadIdx.x >> 6) != 0) return false;
  const int lane = lane_id();
  double y0 = red[0][lane], y1 = red[0][lane + 64];
#pragma unroll
  for (int r = 1; r < kRotGroups; ++r) {
    y0 += red[r][lane];
    y1 += red[r][lane + 64];
  }
  hadamard_bitrev(y0, y1, o0, o1);
  return true;
}

// The query's rotation, in fp32 (the query feeds score operands good to about 2^-16 of its
// largest element, far above fp32's rounding; the history's rotation, which decides codes, stays
// fp64).  Partial sums as in rotate1_block -- thread (g, c) = (t / 32, t % 32) sums rows
// 16 g .. 16 g + 15 of x U for columns 4 c .. 4 c + 3, one fmaf chain from zero over the rows in
// order -- then the eight partial vectors added in order of g, the Hadamard butterflies and the
// bit-reversal gather in fp32, and the scaling by 1/sqrt(128) last.  query_partials is one
// thread's part (y[e] for column 4 c + e); query_finish is a wave's: `red` rows [g][128] of one
// vector in, lane l out holding rotated channels l (o0) and l + 64 (o1).
__device__ __forceinline__ void query_partials(const float* x, const URows& ur, float (&y)[4]) {
  const int g = threadIdx.x >> 5;
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const float xi = x[16 * g + k];
    y[0] = fmaf(xi, ur.v[k].x, y[0]);
    y[1] = fmaf(xi, ur.v[k].y, y[1]);
    y[2] = fmaf(xi, ur.v[k].z, y[2]);
    y[3] = fmaf(xi, ur.v[k].w, y[3]);
  }
}

__device__ __forceinline__ void query_finish(const float (*red)[128], float& o0, float& o1) {
  const int lane = lane_id();
  float y0 = red[0][lane], y1 = red[0][lane + 64];
#pragma unroll
  for (int r = 1; r < kRotGroups; ++r) {
    y0 += red[r][lane];
    y1 += red[r][lane + 64];
  }
  {
    const float a = y0 + y1, b = y0 - y1;
    y0 = a;
    y1 = b;
  }
  y0 = butterfly<32>(y0);
  y1 = butterfly<32>(y1);
  y0 = butterfly<16>(y0);
  y1 = butterfly<16>(y1);
  y0 = butterfly<8>(y0);
  y1 = butterfly<8>(y1);
  y0 = butterfly<4>(y0);
  y1 = butterfly<4>(y1);
  y0 = butterfly<2>(y0);
  y1 = butterfly<2>(y1);
  y0 = butterfly<1>(y0);
  y1 = butterfly<1>(y1);
  // as in hadamard_bitrev: x'_j = z_rev(j), z[r] in lane r & 63 (slot r >> 6), z[r + 1] next lane
  const int r = bitrev7(lane);
  const int src = r & 63;
  const bool hi = (r >> 6) != 0;
  const float a0 = __shfl(y0, src), a1 = __shfl(y1, src);
  const float b0 = __shfl(y0, src + 1), b1 = __shfl(y1, src + 1);
  const float inv_sqrt_d = 0.08838834764831845f;   // 1 / sqrt(128)
  o0 = (hi ? a1 : a0) * inv_sqrt_d;
  o1 = (hi ? b1 : b0) * inv_sqrt_d;
}

// Rotation of TPW row vectors x (fp32, staged in LDS as [TPW][128]) by R = U H P / sqrt(128)
// in fp64.  Lane l returns rotated channels l and l+64 of each vector in out[t][0], out[t][1].
// U is fp32 [128][128] row-major in global memory; x U is accumulated in fp64 over i = 0..127,
// the fast Walsh-Hadamard transform runs as butterflies across lanes, and the bit-reversal
// permutation is a lane gather.
template <int TPW>
__device__ __forceinline__ void rotate_fp64(const float* __restrict__ x_lds,
                                            const float* __restrict__ u, double (&out)[TPW][2]) {
  const int lane = lane_id();
  double y0[TPW], y1[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) { y0[t] = 0.0; y1[t] = 0.0; }
#pragma unroll 4
  for (int i = 0; i < 128; ++i) {
    const double u0 = static_cast<double>(u[i * 128 + lane]);
    const double u1 = static_cast<double>(u[i * 128 + lane + 64]);
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const double xi = static_cast<double>(x_lds[t * 128 + i]);
      y0[t] = fma(xi, u0, y0[t]);
      y1[t] = fma(xi, u1, y1[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < TPW; ++t) hadamard_bitrev(y0[t], y1[t], out[t][0], out[t][1]);
}

}  // namespace dev
}  // namespace oscar
