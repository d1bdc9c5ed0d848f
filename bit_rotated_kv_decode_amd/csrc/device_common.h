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
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
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
#pragma unroll
  for (int h = 32; h >= 1; h >>= 1) {
    const bool upper = (lane & h) != 0;
    const double p0 = __shfl_xor(y0, h);
    const double p1 = __shfl_xor(y1, h);
    y0 = upper ? (p0 - y0) : (y0 + p0);
    y1 = upper ? (p1 - y1) : (y1 + p1);
  }
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
// whole 256-thread block: wave w accumulates rows [32w, 32w + 32) of x U, wave 0 adds the four
// partial vectors (staged in `red`) and finishes with the Hadamard and the bit reversal.  The U
// entries a thread needs are loaded into registers first (load_u_rows), so the loads can be in
// flight while x is still being staged.  Every thread of the block must call rotate1_block (it
// contains a block barrier); it returns true in wave 0, whose lane l then holds rotated channels
// l and l + 64.
struct URows {
  float v[32][2];   // U[32 w + k][lane], U[32 w + k][lane + 64]
};

__device__ __forceinline__ void load_u_rows(const float* __restrict__ u, URows& r) {
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const int i = wave * 32 + k;
    r.v[k][0] = u[i * 128 + lane];
    r.v[k][1] = u[i * 128 + lane + 64];
  }
}

__device__ __forceinline__ bool rotate1_block(const float* x, const URows& ur,
                                              double (*red)[128], double& o0, double& o1) {
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  double y0 = 0.0, y1 = 0.0;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const double xi = static_cast<double>(x[wave * 32 + k]);
    y0 = fma(xi, static_cast<double>(ur.v[k][0]), y0);
    y1 = fma(xi, static_cast<double>(ur.v[k][1]), y1);
  }
  red[wave][lane] = y0;
  red[wave][lane + 64] = y1;
  __syncthreads();
  if (wave != 0) return false;
  y0 = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
  y1 = ((red[0][lane + 64] + red[1][lane + 64]) + red[2][lane + 64]) + red[3][lane + 64];
  hadamard_bitrev(y0, y1, o0, o1);
  return true;
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
