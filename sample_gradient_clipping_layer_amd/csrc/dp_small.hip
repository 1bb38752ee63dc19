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
  float s = sqnorm[i];
  s = s < 0.0f ? 0.0f : s;
  const float n = sqrt_rn_f32(s);
  float ci;
  if (n > C)
    ci = __fdiv_rn(C, n);
  else
    ci = (n == n) ? 1.0f : n;
  c[i] = ci;
  if (norm) norm[i] = n;
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
