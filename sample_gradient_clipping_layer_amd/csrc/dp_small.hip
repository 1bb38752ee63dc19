// Clip factors and the adaptive per-layer bound (small, latency-bound kernels).
#include "dp_common.hpp"
#include "dp_launch.hpp"
#include "dp_noise.hpp"

namespace dpk {

// norm = sqrt(sqnorm) with negative round-off clamped to 0 (NaN kept);
// c = C / norm when norm > C, else 1 (NaN norm -> NaN; infinite norm -> 0).
// FPC clip_c; SEDP App. C, C_i = min(R/||g_i||, 1).
__global__ __launch_bounds__(256) void k_clip_factors(const float* __restrict__ sqnorm, int64_t B, float C,
                                                      float* __restrict__ c, float* __restrict__ norm) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B) return;
  clip_factor_of(sqnorm[i], C, c + i, norm ? norm + i : nullptr);
}

// The per-sample fold of a norm launch whose samples span several tiles
// (NormSink): one wave per sample. The lanes load 64 tile partials at a time
// (one coalesced load instead of a chain of dependent ones), and the fold
// itself runs in tile order through the lanes' values, the same fp32 additions
// in the same order as norm_sink_finish: each layer's tiles summed from 0, then
// the layers in order onto the starting value.
__global__ __launch_bounds__(64) void k_norm_finish(NormSink sink) {
  const int64_t i = blockIdx.x;
  const int lane = threadIdx.x;
  const int nt = sink.ntiles;
  const float* row = sink.partial + i * nt;
  float v = sink.accumulate ? sink.sqnorm[i] : 0.f;
  float tot = 0.f;
  int l = 0, next = sink.lt[1];
  for (int base = 0; base < nt; base += kWave) {
    const float x = base + lane < nt ? row[base + lane] : 0.f;
#pragma unroll
    for (int j = 0; j < kWave; ++j) {
      const int t = base + j;
      if (t >= nt) break;
      if (t == next) {  // layer l ends before tile t (every layer has at least one tile)
        v = (l == 0 && !sink.accumulate) ? tot : v + tot;
        tot = 0.f;
        next = sink.lt[++l + 1];
      }
      tot += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), j));
    }
  }
  v = (l == 0 && !sink.accumulate) ? tot : v + tot;
  if (lane == 0) {
    sink.sqnorm[i] = v;
    if (sink.clip_c) clip_factor_of(v, sink.C, sink.clip_c + i, sink.clip_norm ? sink.clip_norm + i : nullptr);
  }
}

hipError_t launch_norm_finish(hipStream_t st, const NormSink& sink, int64_t B) {
  if (sink.ntiles == 1) return hipSuccess;  // the tiles wrote sqnorm themselves
  hipLaunchKernelGGL(k_norm_finish, dim3((unsigned)B), dim3(kWave), 0, st, sink);
  return hipGetLastError();
}

// TTP adaptive clipping, one layer: one workgroup of 1024 threads.
//   C_l2   = init ? mean(norm) : beta * C_prev
//   C_next = alpha / B * (sum_i min(norm_i, C_l2) + sigma_l2 * C_l2 * z)
// min(n, C_l2) is written as (n > C_l2 ? C_l2 : n) so that a NaN norm
// propagates, like n / max(1, n / C_l2).
__global__ __launch_bounds__(1024) void k_adaptive_threshold(const float* __restrict__ norm, int64_t B, float C_prev,
                                                             float alpha, float beta, float sigma_l2, int init,
                                                             uint32_t k0, uint32_t k1, uint32_t layer,
                                                             uint32_t step, float* __restrict__ C_next,
                                                             float* __restrict__ C_l2_out) {
  __shared__ float red[1024 / kWave];
  __shared__ float bcast;
  float C_l2;
  if (init) {
    float s = 0.f;
    for (int64_t i = threadIdx.x; i < B; i += blockDim.x) s += norm[i];
    s = block_sum<1024>(s, red);
    if (threadIdx.x == 0) bcast = s / (float)B;
    __syncthreads();
    C_l2 = bcast;
  } else {
    C_l2 = beta * C_prev;
  }
  float s = 0.f;
  for (int64_t i = threadIdx.x; i < B; i += blockDim.x) {
    const float n = norm[i];
    s += (n > C_l2) ? C_l2 : n;
  }
  s = block_sum<1024>(s, red);
  if (threadIdx.x == 0) {
    const f32x4 z = normals4(0u, 2u * layer, step, 1u, k0, k1);
    const float noisy = s + (sigma_l2 * C_l2) * z[0];
    C_next[0] = (alpha / (float)B) * noisy;
    if (C_l2_out) C_l2_out[0] = C_l2;
  }
}

// Virtual step ("Scalable and Efficient Training of Large CNNs with DP",
// Performance section: several physical batches back-propagated before one
// update; App. E, the virtual step): the clipped sums of the physical batches
// add up in fp32, acc[i] = acc[i] + s[i], in batch order.
__global__ __launch_bounds__(256) void k_accumulate(float* __restrict__ acc, const float* __restrict__ s, int64_t n,
                                                    int vec) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (vec) {
    if (4 * t + 3 < n) {
      float4 a = reinterpret_cast<float4*>(acc)[t];
      const float4 b = reinterpret_cast<const float4*>(s)[t];
      a.x = a.x + b.x;
      a.y = a.y + b.y;
      a.z = a.z + b.z;
      a.w = a.w + b.w;
      reinterpret_cast<float4*>(acc)[t] = a;
    } else {
      for (int64_t i = 4 * t; i < n; ++i) acc[i] = acc[i] + s[i];
    }
  } else if (t < n) {
    acc[t] = acc[t] + s[t];
  }
}

// The noise and the mean of a logical batch, once: out = (acc + fl(sigma*C) z)
// * fl(1/denom), z from the same counters as the clipped-sum kernels (weight
// element (m, n): lane m % 4 of group (m/4)*p + n, word 2*layer; bias element
// n: lane n % 4 of group n/4, word 2*layer + 1). One thread per Philox block
// (4 rows of one column); reads its block before writing it, so out may be acc.
// The group index t = q*p + n is below 2^32 (the host checks ceil(d/4)*p <
// 2^32), so q and n come from a 32-bit multiply-shift division by p.
__global__ __launch_bounds__(256) void k_noise_mean(const float* acc, const float* bias_acc, int64_t d, int64_t p,
                                                    FastDiv by_p, NoiseArgs na, float* out, float* bias_out) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nw = ((d + 3) / 4) * p;
  if (t < nw) {
    const uint32_t tt = (uint32_t)t;
    const uint32_t q = fast_div(tt, by_p), n = tt - q * (uint32_t)p;
    const f32x4 z = normals4(tt, 2u * na.layer, na.step, 0u, na.k0, na.k1);
    const int64_t e0 = (int64_t)(4 * (uint64_t)q) * p + n;  // element (4q, n)
    const int rows = d - 4 * (int64_t)q < 4 ? (int)(d - 4 * (int64_t)q) : 4;
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (r < rows) v[r] = acc[e0 + r * p];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (r < rows) out[e0 + r * p] = noised_mean_spec(v[r], na.sc, z[r], na.inv_denom);
  } else if (bias_acc && t < nw + (p + 3) / 4) {
    const int64_t g = t - nw;
    const f32x4 z = normals4((uint32_t)g, 2u * na.layer + 1u, na.step, 0u, na.k0, na.k1);
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * g + r < p) v[r] = bias_acc[4 * g + r];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * g + r < p) bias_out[4 * g + r] = noised_mean_spec(v[r], na.sc, z[r], na.inv_denom);
  }
}

hipError_t launch_accumulate(hipStream_t st, float* acc, const float* s, int64_t n) {
  const int vec = ((reinterpret_cast<uintptr_t>(acc) | reinterpret_cast<uintptr_t>(s)) & 15) == 0;
  const int64_t threads = vec ? (n + 3) / 4 : n;
  hipLaunchKernelGGL(k_accumulate, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, acc, s, n, vec);
  return hipGetLastError();
}

hipError_t launch_noise_mean(hipStream_t st, const float* acc, const float* bias_acc, int64_t d, int64_t p,
                             const NoiseArgs& na, float* out, float* bias_out) {
  const int64_t threads = ((d + 3) / 4) * p + (bias_acc ? (p + 3) / 4 : 0);
  hipLaunchKernelGGL(k_noise_mean, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, acc, bias_acc, d, p,
                     make_fastdiv((uint32_t)p), na, out, bias_out);
  return hipGetLastError();
}

hipError_t launch_clip_factors(hipStream_t st, const float* sqnorm, int64_t B, float C, float* c, float* norm) {
  const dim3 grid((unsigned)((B + 255) / 256));
  hipLaunchKernelGGL(k_clip_factors, grid, dim3(256), 0, st, sqnorm, B, C, c, norm);
  return hipGetLastError();
}

hipError_t launch_adaptive_threshold(hipStream_t st, const float* norm, int64_t B, float C_prev, float alpha,
                                     float beta, float sigma_l2, int init, uint64_t seed, uint32_t layer,
                                     uint32_t step, float* C_next, float* C_l2_out) {
  hipLaunchKernelGGL(k_adaptive_threshold, dim3(1), dim3(1024), 0, st, norm, B, C_prev, alpha, beta, sigma_l2, init,
                     (uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32), layer, step, C_next, C_l2_out);
  return hipGetLastError();
}

}  // namespace dpk
