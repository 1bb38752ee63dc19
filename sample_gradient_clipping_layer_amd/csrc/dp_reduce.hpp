// Split-K reduce of the bf16 multi-layer contraction: the arithmetic that
// both the reduce kernels and the contraction kernel's tail workgroups run.
#pragma once

#include "dp_common.hpp"
#include "dp_launch.hpp"
#include "dp_noise.hpp"

namespace dpk {

// The 4 x 4 output block (rows 4 q.., columns 4 cq..) of a split reduce: the
// partials summed in split order per element, then the noise and the mean.
// Same result as k_reduce_noise for d % 4 == 0, p % 4 == 0 and 16-byte
// aligned ws and out: every load is a float4 and the thread keeps 4 splits x
// 4 rows of loads in flight.
// The noise form for a known split count: the partials' loads are issued
// first and the normals drawn while they are in flight; the same operations
// as the general form.
template <int KS>
__device__ __forceinline__ void reduce_noise_block4_ks(const float* __restrict__ ws, int64_t p, int64_t split_stride,
                                                       int64_t q, int64_t cq, const NoiseArgs& na,
                                                       float* __restrict__ out) {
  const float* base = ws + 4 * q * p + 4 * cq;
  float4 v[KS][4];
#pragma unroll
  for (int u = 0; u < KS; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) v[u][r] = *reinterpret_cast<const float4*>(base + u * split_stride + r * p);
  f32x4 z[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) z[k] = normals4((uint32_t)(q * p + 4 * cq + k), 2u * na.layer, na.step, 0u, na.k0, na.k1);
  float4 s[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) s[r] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int u = 0; u < KS; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s[r].x += v[u][r].x;
      s[r].y += v[u][r].y;
      s[r].z += v[u][r].z;
      s[r].w += v[u][r].w;
    }
#pragma unroll
  for (int r = 0; r < 4; ++r)
    *reinterpret_cast<float4*>(out + (4 * q + r) * p + 4 * cq) =
        make_float4(noised_mean_spec(s[r].x, na.sc, z[0][r], na.inv_denom),
                    noised_mean_spec(s[r].y, na.sc, z[1][r], na.inv_denom),
                    noised_mean_spec(s[r].z, na.sc, z[2][r], na.inv_denom),
                    noised_mean_spec(s[r].w, na.sc, z[3][r], na.inv_denom));
}

// With ACC the block's sums are added to out (out = out + S) instead: no
// noise, no mean.
template <bool ACC = false>
__device__ __forceinline__ void reduce_noise_block4(const float* __restrict__ ws, int64_t ks, int64_t p,
                                                    int64_t split_stride, int64_t q, int64_t cq, const NoiseArgs& na,
                                                    float* __restrict__ out) {
  if (!ACC && ks >= 1 && ks <= 4) {
    switch (ks) {
      case 1: reduce_noise_block4_ks<1>(ws, p, split_stride, q, cq, na, out); return;
      case 2: reduce_noise_block4_ks<2>(ws, p, split_stride, q, cq, na, out); return;
      case 3: reduce_noise_block4_ks<3>(ws, p, split_stride, q, cq, na, out); return;
      default: reduce_noise_block4_ks<4>(ws, p, split_stride, q, cq, na, out); return;
    }
  }
  constexpr int U = 4;
  const float* base = ws + 4 * q * p + 4 * cq;
  float4 s[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) s[r] = make_float4(0.f, 0.f, 0.f, 0.f);
  int64_t sp = 0;
  for (; sp + U <= ks; sp += U) {
    float4 v[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) v[u][r] = *reinterpret_cast<const float4*>(base + (sp + u) * split_stride + r * p);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[r].x += v[u][r].x;
        s[r].y += v[u][r].y;
        s[r].z += v[u][r].z;
        s[r].w += v[u][r].w;
      }
  }
  for (; sp < ks; ++sp) {
    float4 v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = *reinterpret_cast<const float4*>(base + sp * split_stride + r * p);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s[r].x += v[r].x;
      s[r].y += v[r].y;
      s[r].z += v[r].z;
      s[r].w += v[r].w;
    }
  }
  if (ACC) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float4* po = reinterpret_cast<float4*>(out + (4 * q + r) * p + 4 * cq);
      float4 a = *po;
      a.x = a.x + s[r].x;
      a.y = a.y + s[r].y;
      a.z = a.z + s[r].z;
      a.w = a.w + s[r].w;
      *po = a;
    }
    return;
  }
  float o[4][4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t n = 4 * cq + k;
    const f32x4 z = normals4((uint32_t)(q * p + n), 2u * na.layer, na.step, 0u, na.k0, na.k1);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float sv = k == 0 ? s[r].x : k == 1 ? s[r].y : k == 2 ? s[r].z : s[r].w;
      o[r][k] = noised_mean_spec(sv, na.sc, z[r], na.inv_denom);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
    *reinterpret_cast<float4*>(out + (4 * q + r) * p + 4 * cq) = make_float4(o[r][0], o[r][1], o[r][2], o[r][3]);
}

// The layers of a grouped reduce: layer k owns the 256-thread blocks
// [blk_begin[k], blk_begin[k + 1]), one thread per 4 x 4 output block.
struct RedGroup {
  SplitReduceLayer L[kDlGroupMax];
  int64_t blk_begin[kDlGroupMax];
  int n;
};

// Whether a layer's reduce may take the vectorised form (else the one-layer
// launch keeps it): d, p multiples of 4, 16-byte aligned partials and output,
// and not the many-splits shape that k_reduce_noise_wide takes.
inline bool split_reduce_vec_ok(const SplitReduceLayer& x) {
  const float* dst = x.acc ? x.acc : x.out;
  return x.d % 4 == 0 && x.p % 4 == 0 && (reinterpret_cast<uintptr_t>(dst) & 15) == 0 &&
         (reinterpret_cast<uintptr_t>(x.ws) & 15) == 0 && !(x.ks >= 64 && (x.d / 4) * (x.p / 4) < 32768);
}

// 256-thread blocks of one layer's vectorised reduce
inline int64_t split_reduce_blocks(const SplitReduceLayer& x) { return ((x.d / 4) * (x.p / 4) + 255) / 256; }

}  // namespace dpk
