// Decode attention over the three-segment cache (BF16 sink | rotated INT2 history | BF16 recent).
//
// Structure after the OSCAR write-up "超越TurboQuant！OSCAR：面向真实服务的2-bit KV Cache量化",
// section OSCAR 的设计: the INT2 history and the BF16 segments are processed separately and then
// combined with an online-softmax merge.  Launch order on one stream:
//   1. qrot_kernel   q' = q R_k per query head (fp64 rotation, stored fp32) and the per-group
//                    sums of q' that the zero points multiply;
//   2. int2_kernel   split-KV over history pages: scores s * (q' . codes) + z * sum(q'), online
//                    softmax, value accumulation in the rotated frame -> (m, l, acc') partials;
//   3. bf16_kernel   64-token chunks of the BF16 sink and recent ring -> (m, l, acc) partials;
//   4. merge_kernel  log-sum-exp merge of the INT2 partials, un-rotation acc' R_v^T, merge with
//                    the BF16 partials, normalisation.
// Softmax statistics are kept in the log2 domain: scores are scaled by sm_scale * log2(e).
#include "device_common.h"
#include "oscar_internal.h"

namespace oscar {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------------------------------------
// 1. query rotation: one wave per (sequence, query head)
__global__ __launch_bounds__(256) void qrot_kernel(const uint16_t* __restrict__ q,
                                                   const float* __restrict__ u_k, int batch,
                                                   int hq, int gqa, int n_groups,
                                                   float* __restrict__ qrot,
                                                   float* __restrict__ sigma) {
  __shared__ float xs[4][kHeadDim];
  const int wave = threadIdx.x >> 6;
  const int lane = dev::lane_id();
  const int row = blockIdx.x * 4 + wave;   // b * hq + head
  if (row >= batch * hq) return;
  const int kv = (row % hq) / gqa;
  float* x = xs[wave];
  x[lane] = dev::bf16_to_f32(q[static_cast<int64_t>(row) * kHeadDim + lane]);
  x[lane + 64] = dev::bf16_to_f32(q[static_cast<int64_t>(row) * kHeadDim + lane + 64]);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  double r[1][2];
  dev::rotate_fp64<1>(x, u_k + static_cast<int64_t>(kv) * kHeadDim * kHeadDim, r);
  const float r0 = static_cast<float>(r[0][0]);
  const float r1 = static_cast<float>(r[0][1]);
  qrot[static_cast<int64_t>(row) * kHeadDim + lane] = r0;
  qrot[static_cast<int64_t>(row) * kHeadDim + lane + 64] = r1;
  // per-group sums of the stored fp32 q'
  if (n_groups == 1) {
    const float s = dev::wave_sum(r0 + r1);
    if (lane == 0) sigma[row * 2] = s;
  } else {
    const float s0 = dev::wave_sum(r0);
    const float s1 = dev::wave_sum(r1);
    if (lane == 0) {
      sigma[row * 2] = s0;
      sigma[row * 2 + 1] = s1;
    }
  }
}

// ------------------------------------------------------------------------------------------
// 2. INT2 split-KV: block (split, kv head, sequence), 4 waves; each wave takes one page at a time
// with lane t = token slot t for the scores and lane j = channels (j, j + 64) for the values.
template <int G, int NG>
__global__ __launch_bounds__(256) void int2_kernel(DecodeArgs a, Plan p, float scale_log2) {
  __shared__ float q_s[G][kHeadDim];
  __shared__ float sig_s[G][2];
  __shared__ float pt_s[4][G][NG][kPage];
  __shared__ float red_m[4][G], red_l[4][G];
  __shared__ float red_acc[4][G][kHeadDim];

  const int split = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int L = a.seq_lens[b];
  const int n_hist = max(0, L - kSink - kRecent);
  const int n_pages = (n_hist + kPage - 1) / kPage;
  const int p0 = split * p.pages_per_split;
  if (p0 >= n_pages) return;
  const int p1 = min(p0 + p.pages_per_split, n_pages);
  const int wave = threadIdx.x >> 6;
  const int lane = dev::lane_id();

  const float* qrot = reinterpret_cast<const float*>(a.workspace + p.off_qrot);
  const float* sigma = reinterpret_cast<const float*>(a.workspace + p.off_sigma);
  const int head0 = b * p.hq + kv * G;
  for (int i = threadIdx.x; i < G * kHeadDim; i += 256)
    q_s[i / kHeadDim][i % kHeadDim] = qrot[static_cast<int64_t>(head0) * kHeadDim + i];
  if (threadIdx.x < G * 2) sig_s[threadIdx.x / 2][threadIdx.x % 2] = sigma[head0 * 2 + threadIdx.x];
  __syncthreads();

  float m[G], lsum[G], acc[G][2], zsum[G][NG];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.f;
    acc[h][0] = acc[h][1] = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) zsum[h][g] = 0.f;
  }
  const int blk_bytes = block_bytes(NG);
  const int vmeta = v_meta_off(NG);
  const int rounds = (p1 - p0 + 3) / 4;
  for (int rd = 0; rd < rounds; ++rd) {
    const int pg = p0 + rd * 4 + wave;
    const bool active = pg < p1;
    const uint8_t* blk = nullptr;
    if (active) {
      const int page = a.page_table[static_cast<int64_t>(b) * a.max_pages_per_seq + pg];
      blk = a.pool + (static_cast<int64_t>(page) * p.hkv + kv) * blk_bytes;
      const bool valid = pg * kPage + lane < n_hist;
      // scores for token slot `lane`
      const uint4* krow = reinterpret_cast<const uint4*>(blk + kKCodesOff + lane * 32);
      const uint4 k0 = krow[0], k1 = krow[1];
      const uint32_t kw[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
      float ks[NG], kz[NG], vs[NG], vz[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const uint32_t km = reinterpret_cast<const uint32_t*>(blk + kKMetaOff)[lane * NG + g];
        const uint32_t vm = reinterpret_cast<const uint32_t*>(blk + vmeta)[lane * NG + g];
        ks[g] = __half2float(__ushort_as_half(static_cast<uint16_t>(km & 0xFFFF)));
        kz[g] = __half2float(__ushort_as_half(static_cast<uint16_t>(km >> 16)));
        vs[g] = __half2float(__ushort_as_half(static_cast<uint16_t>(vm & 0xFFFF)));
        vz[g] = __half2float(__ushort_as_half(static_cast<uint16_t>(vm >> 16)));
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float tot = 0.f;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          float dot = 0.f;
#pragma unroll
          for (int w = g * (8 / NG); w < (g + 1) * (8 / NG); ++w) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
              dot = fmaf(q_s[h][w * 16 + i], static_cast<float>((kw[w] >> (2 * i)) & 3u), dot);
          }
          tot = fmaf(ks[g], dot, fmaf(kz[g], sig_s[h][g], tot));
        }
        const float logit = valid ? tot * scale_log2 : -INFINITY;
        const float pm = dev::wave_max(logit);
        const float mn = fmaxf(m[h], pm);
        const float alpha = exp2f(m[h] - mn);
        const float pr = exp2f(logit - mn);
        m[h] = mn;
        lsum[h] = lsum[h] * alpha + pr;
        acc[h][0] *= alpha;
        acc[h][1] *= alpha;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          // slots past the end of the history hold arbitrary bytes: keep them out entirely
          zsum[h][g] = valid ? fmaf(pr, vz[g], zsum[h][g] * alpha) : zsum[h][g] * alpha;
          pt_s[wave][h][g][lane] = valid ? pr * vs[g] : 0.f;
        }
      }
    }
    __syncthreads();
    if (active) {
      // values: lane owns channels lane (group 0) and lane + 64 (group NG - 1)
      const uint4 va = reinterpret_cast<const uint4*>(blk + kVCodesOff)[lane];
      const uint4 vb = reinterpret_cast<const uint4*>(blk + kVCodesOff)[lane + 64];
      const uint32_t wa[4] = {va.x, va.y, va.z, va.w};
      const uint32_t wb[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll 4
      for (int t = 0; t < kPage; ++t) {
        const float ca = static_cast<float>((wa[t >> 4] >> (2 * (t & 15))) & 3u);
        const float cb = static_cast<float>((wb[t >> 4] >> (2 * (t & 15))) & 3u);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          acc[h][0] = fmaf(pt_s[wave][h][0][t], ca, acc[h][0]);
          acc[h][1] = fmaf(pt_s[wave][h][NG - 1][t], cb, acc[h][1]);
        }
      }
    }
    __syncthreads();
  }
  // finish the wave: lane-local sums -> wave sums; add the zero-point term
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float l = dev::wave_sum(lsum[h]);
    float zt[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) zt[g] = dev::wave_sum(zsum[h][g]);
    if (lane == 0) {
      red_m[wave][h] = m[h];
      red_l[wave][h] = l;
    }
    red_acc[wave][h][lane] = acc[h][0] + zt[0];
    red_acc[wave][h][lane + 64] = acc[h][1] + zt[NG - 1];
  }
  __syncthreads();
  // combine the 4 waves and write the partial of this split
  float* ml = reinterpret_cast<float*>(a.workspace + p.off_int2_ml);
  float* pacc = reinterpret_cast<float*>(a.workspace + p.off_int2_acc);
  for (int i = threadIdx.x; i < G * kHeadDim; i += 256) {
    const int h = i / kHeadDim, j = i % kHeadDim;
    float mm = -INFINITY;
    for (int w = 0; w < 4; ++w) mm = fmaxf(mm, red_m[w][h]);
    float s = 0.f, l = 0.f;
    for (int w = 0; w < 4; ++w) {
      if (red_m[w][h] == -INFINITY) continue;
      const float f = exp2f(red_m[w][h] - mm);
      s = fmaf(red_acc[w][h][j], f, s);
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
// 3. BF16 segments: block (chunk, kv head, sequence), one wave.  Chunk 0 = sink rows 0..63,
// chunk c >= 1 = recent ring rows 64(c-1) .. 64c-1.
template <int G>
__global__ __launch_bounds__(64) void bf16_kernel(DecodeArgs a, Plan p, float scale_log2) {
  __shared__ float q_s[G][kHeadDim];
  __shared__ float p_s[G][64];
  const int chunk = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int lane = dev::lane_id();
  const int L = a.seq_lens[b];
  const int64_t slot = a.seq_slot[b];
  const int head0 = b * p.hq + kv * G;
  for (int i = lane; i < G * kHeadDim; i += 64)
    q_s[i / kHeadDim][i % kHeadDim] =
        dev::bf16_to_f32(a.q[static_cast<int64_t>(head0) * kHeadDim + i]);
  __syncthreads();

  const uint16_t* kbase;
  const uint16_t* vbase;
  bool valid;
  if (chunk == 0) {
    const int64_t off = ((slot * p.hkv + kv) * kSink + lane) * kHeadDim;
    kbase = a.sink_k + off;
    vbase = a.sink_v + off;
    valid = lane < min(L, kSink);
  } else {
    const int r = (chunk - 1) * 64 + lane;   // ring row
    const int64_t off = ((slot * p.hkv + kv) * kRecent + r) * kHeadDim;
    kbase = a.recent_k + off;
    vbase = a.recent_v + off;
    const int n_recent = min(kRecent, max(0, L - kSink));
    const int start = L - n_recent;
    const int posr = start + (((r - start) % kRecent) + kRecent) % kRecent;
    valid = n_recent > 0 && posr < L;
  }
  float logit[G];
#pragma unroll
  for (int h = 0; h < G; ++h) logit[h] = 0.f;
  if (valid) {
    const uint4* kr = reinterpret_cast<const uint4*>(kbase);
#pragma unroll 4
    for (int c = 0; c < 16; ++c) {
      const uint4 w = kr[c];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(ws[e] << 16);
        const float hi = __uint_as_float(ws[e] & 0xFFFF0000u);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          logit[h] = fmaf(q_s[h][c * 8 + 2 * e], lo, logit[h]);
          logit[h] = fmaf(q_s[h][c * 8 + 2 * e + 1], hi, logit[h]);
        }
      }
    }
  }
  float* ml = reinterpret_cast<float*>(a.workspace + p.off_bf16_ml);
  float* pacc = reinterpret_cast<float*>(a.workspace + p.off_bf16_acc);
  float mh[G], lh[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float lg = valid ? logit[h] * scale_log2 : -INFINITY;
    mh[h] = dev::wave_max(lg);
    const float pr = (mh[h] == -INFINITY) ? 0.f : exp2f(lg - mh[h]);
    lh[h] = dev::wave_sum(pr);
    p_s[h][lane] = pr;
  }
  __syncthreads();
  // values: lane owns channels 2*lane, 2*lane + 1
  float acc[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) acc[h][0] = acc[h][1] = 0.f;
  const int64_t vrow0 = (chunk == 0) ? ((slot * p.hkv + kv) * kSink) * kHeadDim
                                     : ((slot * p.hkv + kv) * kRecent + (chunk - 1) * 64) * kHeadDim;
  const uint16_t* vb = (chunk == 0 ? a.sink_v : a.recent_v) + vrow0;
  for (int t = 0; t < 64; ++t) {
    bool any = false;
#pragma unroll
    for (int h = 0; h < G; ++h) any |= p_s[h][t] != 0.f;
    if (!any) continue;
    const uint32_t w = reinterpret_cast<const uint32_t*>(vb + static_cast<int64_t>(t) * kHeadDim)[lane];
    const float lo = __uint_as_float(w << 16);
    const float hi = __uint_as_float(w & 0xFFFF0000u);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      acc[h][0] = fmaf(p_s[h][t], lo, acc[h][0]);
      acc[h][1] = fmaf(p_s[h][t], hi, acc[h][1]);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int64_t prow = static_cast<int64_t>(head0 + h) * kBf16Chunks + chunk;
    pacc[prow * kHeadDim + 2 * lane] = acc[h][0];
    pacc[prow * kHeadDim + 2 * lane + 1] = acc[h][1];
    if (lane == 0) {
      ml[prow * 2] = mh[h];
      ml[prow * 2 + 1] = lh[h];
    }
  }
}

// ------------------------------------------------------------------------------------------
// 4. merge: block (kv head, sequence), 256 threads; thread (hh, j) works on channel j of heads
// hh, hh + 2, ...
template <int G>
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a, Plan p) {
  __shared__ float buf[G][kHeadDim];
  __shared__ float hm[G], hl[G];
  const int kv = blockIdx.x, b = blockIdx.y;
  const int j = threadIdx.x & 127;
  const int hh = threadIdx.x >> 7;
  const int L = a.seq_lens[b];
  const int n_hist = max(0, L - kSink - kRecent);
  const int n_pages = (n_hist + kPage - 1) / kPage;
  const int n_valid = (n_pages + p.pages_per_split - 1) / p.pages_per_split;
  const int head0 = b * p.hq + kv * G;
  const float* iml = reinterpret_cast<const float*>(a.workspace + p.off_int2_ml);
  const float* iacc = reinterpret_cast<const float*>(a.workspace + p.off_int2_acc);
  const float* bml = reinterpret_cast<const float*>(a.workspace + p.off_bf16_ml);
  const float* bacc = reinterpret_cast<const float*>(a.workspace + p.off_bf16_acc);

  // (1) merge the INT2 split partials (rotated frame), P applied on the way into LDS
  for (int h = hh; h < G; h += 2) {
    const int64_t base = static_cast<int64_t>(head0 + h) * p.num_splits;
    float mm = -INFINITY;
    for (int s = 0; s < n_valid; ++s) mm = fmaxf(mm, iml[(base + s) * 2]);
    float acc = 0.f, l = 0.f;
    for (int s = 0; s < n_valid; ++s) {
      const float f = exp2f(iml[(base + s) * 2] - mm);
      acc = fmaf(iacc[(base + s) * kHeadDim + dev::bitrev7(j)], f, acc);
      l = fmaf(iml[(base + s) * 2 + 1], f, l);
    }
    buf[h][j] = acc;   // (acc' P)_j = acc'_rev(j)
    if (j == 0) {
      hm[h] = mm;
      hl[h] = l;
    }
  }
  __syncthreads();
  // (2) Hadamard butterflies on each head's 128-vector
  for (int hs = 1; hs < kHeadDim; hs <<= 1) {
    for (int idx = threadIdx.x; idx < G * 64; idx += 256) {
      const int h = idx / 64, k = idx % 64;
      const int i = (k / hs) * 2 * hs + (k % hs);
      const float x = buf[h][i], y = buf[h][i + hs];
      buf[h][i] = x + y;
      buf[h][i + hs] = x - y;
    }
    __syncthreads();
  }
  // (3) times U_v^T / sqrt(d), merge with the BF16 partials, normalise
  const float* u = a.u_v + static_cast<int64_t>(kv) * kHeadDim * kHeadDim + j * kHeadDim;
  for (int h = hh; h < G; h += 2) {
    float o = 0.f;
    if (n_valid > 0) {
      for (int i = 0; i < kHeadDim; ++i) o = fmaf(buf[h][i], u[i], o);
      o *= 0.08838834764831845f;
    }
    const int64_t bbase = static_cast<int64_t>(head0 + h) * kBf16Chunks;
    float mb = -INFINITY;
    for (int c = 0; c < kBf16Chunks; ++c) mb = fmaxf(mb, bml[(bbase + c) * 2]);
    const float mi = n_valid > 0 ? hm[h] : -INFINITY;
    const float mt = fmaxf(mb, mi);
    float acc = 0.f, l = 0.f;
    if (mi != -INFINITY) {
      const float f = exp2f(mi - mt);
      acc = o * f;
      l = hl[h] * f;
    }
    for (int c = 0; c < kBf16Chunks; ++c) {
      const float mc = bml[(bbase + c) * 2];
      if (mc == -INFINITY) continue;
      const float f = exp2f(mc - mt);
      acc = fmaf(bacc[(bbase + c) * kHeadDim + j], f, acc);
      l = fmaf(bml[(bbase + c) * 2 + 1], f, l);
    }
    a.out[static_cast<int64_t>(head0 + h) * kHeadDim + j] = acc / l;
    if (a.lse != nullptr && j == 0)
      a.lse[head0 + h] = (mt + log2f(l)) * 0.6931471805599453f;
  }
}

template <int G>
hipError_t launch_g(const DecodeArgs& a, const Plan& p, uint32_t stages, hipStream_t stream) {
  const float scale_log2 = a.sm_scale * kLog2e;
  if ((stages & OSCAR_STAGE_INT2) && p.max_pages > 0) {
    dim3 grid(p.num_splits, p.hkv, p.batch);
    if (p.n_groups == 1)
      hipLaunchKernelGGL((int2_kernel<G, 1>), grid, dim3(256), 0, stream, a, p, scale_log2);
    else
      hipLaunchKernelGGL((int2_kernel<G, 2>), grid, dim3(256), 0, stream, a, p, scale_log2);
  }
  if (stages & OSCAR_STAGE_BF16)
    hipLaunchKernelGGL((bf16_kernel<G>), dim3(kBf16Chunks, p.hkv, p.batch), dim3(64), 0, stream,
                       a, p, scale_log2);
  if (stages & OSCAR_STAGE_MERGE)
    hipLaunchKernelGGL((merge_kernel<G>), dim3(p.hkv, p.batch), dim3(256), 0, stream, a, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, const Plan& p, uint32_t stages,
                         hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  if (stages & OSCAR_STAGE_QUERY) {
    float* qrot = reinterpret_cast<float*>(a.workspace + p.off_qrot);
    float* sigma = reinterpret_cast<float*>(a.workspace + p.off_sigma);
    const int rows = p.batch * p.hq;
    hipLaunchKernelGGL(qrot_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, a.q, a.u_k,
                       p.batch, p.hq, p.gqa, p.n_groups, qrot, sigma);
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
