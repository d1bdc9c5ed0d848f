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

// 7-bit bit reversal of a channel index in [0, 128).
__device__ __forceinline__ int bitrev7(int j) {
  return static_cast<int>(__builtin_bitreverse32(static_cast<uint32_t>(j)) >> 25);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fminf(v, __shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
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
  // Hadamard butterflies: stage 64 is within the lane, stages 32..1 pair lane l with l ^ h.
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const double a = y0[t] + y1[t];
    const double b = y0[t] - y1[t];
    y0[t] = a;
    y1[t] = b;
  }
#pragma unroll
  for (int h = 32; h >= 1; h >>= 1) {
    const bool upper = (lane & h) != 0;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const double p0 = __shfl_xor(y0[t], h);
      const double p1 = __shfl_xor(y1[t], h);
      y0[t] = upper ? (p0 - y0[t]) : (y0[t] + p0);
      y1[t] = upper ? (p1 - y1[t]) : (y1[t] + p1);
    }
  }
  // x'_j = z_rev(j) / sqrt(128): rev(l) = r is even for l < 64 and rev(l + 64) = r + 1.  z[r]
  // sits in lane r & 63 (slot r >> 6), z[r + 1] in the next lane, same slot.
  const double inv_sqrt_d = 0.08838834764831845;  // 1 / sqrt(128)
  const int r = bitrev7(lane);
  const int src = r & 63;
  const bool hi = (r >> 6) != 0;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const double a0 = __shfl(y0[t], src);
    const double a1 = __shfl(y1[t], src);
    const double b0 = __shfl(y0[t], src + 1);
    const double b1 = __shfl(y1[t], src + 1);
    out[t][0] = (hi ? a1 : a0) * inv_sqrt_d;
    out[t][1] = (hi ? b1 : b0) * inv_sqrt_d;
  }
}

}  // namespace dev
}  // namespace oscar
