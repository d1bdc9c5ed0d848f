// Memory probes: the practical HBM ceilings the attention kernel's roofline is read against.
// Not part of the method -- plain reads with no arithmetic, timed next to the kernels they bound.
//   probe_read_kernel    every 16-byte chunk of a buffer once (non-temporal loads, grid stride,
//                        eight loads in flight per thread): the plain streaming-read ceiling.
//   probe_gather_kernel  the INT2 pool's (page, KV head) blocks through a page table in the
//                        attention kernel's grid and wave order (blocks of four waves on a page
//                        range of one KV head, wave w taking pages p0 + w + 4 i), with DEPTH
//                        pages in flight per wave: what that access pattern alone can reach.
#include "device_common.h"
#include "oscar_internal.h"

namespace oscar {
namespace {

// Folds loaded words into one value and stores it only when it equals a constant no test data
// produces, so the loads stay live without a store per thread.
constexpr uint32_t kNever = 0x9E3779B9u;

__device__ __forceinline__ uint32_t fold(const uint4& v) { return v.x ^ v.y ^ v.z ^ v.w; }

__global__ __launch_bounds__(256) void probe_read_kernel(const uint4* __restrict__ p, size_t n16,
                                                         uint32_t* sink) {
  constexpr int U = 8;
  const size_t stride = static_cast<size_t>(gridDim.x) * 256;
  size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) v[k] = dev::load_stream(p + i + k * stride);
#pragma unroll
    for (int k = 0; k < U; ++k) acc ^= fold(v[k]);
  }
  for (; i < n16; i += stride) acc ^= fold(dev::load_stream(p + i));
  if (acc == kNever) sink[blockIdx.x] = acc;
}

template <int DEPTH>
__global__ __launch_bounds__(256) void probe_gather_kernel(const uint8_t* __restrict__ pool,
                                                           const int32_t* __restrict__ table,
                                                           int n_pages, int hkv, int block_bytes,
                                                           int pages_per_split,
                                                           uint32_t* sink) {
  const int kv = blockIdx.x % hkv, split = blockIdx.x / hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int p0 = split * pages_per_split;
  const int p1 = min(p0 + pages_per_split, n_pages);
  const int meta16 = (block_bytes - kMetaOff) / 16;   // 16-byte chunks of the meta region
  struct Regs {
    uint4 c[4];
    uint4 m;
  };
  auto load = [&](int pg, Regs& r) {
    const uint8_t* blk = pool + (static_cast<int64_t>(table[pg]) * hkv + kv) * block_bytes;
    const uint4* q = reinterpret_cast<const uint4*>(blk);
#pragma unroll
    for (int k = 0; k < 4; ++k) r.c[k] = dev::load_stream(q + 64 * k + lane);
    r.m = lane < meta16 ? dev::load_stream(q + 256 + lane) : make_uint4(0, 0, 0, 0);
  };
  uint32_t acc = 0;
  Regs r[DEPTH];
  int pg = p0 + wave;
#pragma unroll
  for (int k = 0; k < DEPTH; ++k)
    if (pg + 4 * k < p1) load(pg + 4 * k, r[k]);
  for (int i = 0; pg < p1; ++i, pg += 4) {
    // consume the oldest set, then refill it with the page DEPTH steps ahead
#pragma unroll
    for (int k = 0; k < DEPTH; ++k) {
      if (k == i % DEPTH) {
        acc ^= fold(r[k].c[0]) ^ fold(r[k].c[1]) ^ fold(r[k].c[2]) ^ fold(r[k].c[3]) ^
               fold(r[k].m);
        if (pg + 4 * DEPTH < p1) load(pg + 4 * DEPTH, r[k]);
      }
    }
  }
  if (acc == kNever) sink[blockIdx.x * 4 + wave] = acc;
}

}  // namespace

hipError_t launch_probe_read(const void* buf, size_t bytes, uint32_t* sink, int blocks,
                             hipStream_t stream) {
  hipLaunchKernelGGL(probe_read_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const uint4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_probe_gather(const void* pool, const int32_t* table, int n_pages, int hkv,
                               int block_bytes, int pages_per_split, int depth, uint32_t* sink,
                               hipStream_t stream) {
  const int splits = (n_pages + pages_per_split - 1) / pages_per_split;
  const dim3 grid(splits * hkv);
  const uint8_t* p = static_cast<const uint8_t*>(pool);
  switch (depth) {
    case 1: hipLaunchKernelGGL(probe_gather_kernel<1>, grid, dim3(256), 0, stream, p, table,
                               n_pages, hkv, block_bytes, pages_per_split, sink); break;
    case 2: hipLaunchKernelGGL(probe_gather_kernel<2>, grid, dim3(256), 0, stream, p, table,
                               n_pages, hkv, block_bytes, pages_per_split, sink); break;
    case 3: hipLaunchKernelGGL(probe_gather_kernel<3>, grid, dim3(256), 0, stream, p, table,
                               n_pages, hkv, block_bytes, pages_per_split, sink); break;
    default: hipLaunchKernelGGL(probe_gather_kernel<4>, grid, dim3(256), 0, stream, p, table,
                                n_pages, hkv, block_bytes, pages_per_split, sink); break;
  }
  return hipGetLastError();
}

}  // namespace oscar
