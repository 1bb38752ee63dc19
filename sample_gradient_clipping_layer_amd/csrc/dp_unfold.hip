// The unfolding U(a) of a convolution layer's folded input, written to memory.
//
// "Scalable and Efficient Training of Large CNNs with DP", Sec. 2.2, eqs.
// (2.5)-(2.6): a 2-D convolution is the linear layer s = U(a) W on the
// unfolded input, whose row t = ho*Wo + wo holds, in column
// f = (ci*KH + i)*KW + j, a[ci][ho*sh - ph + i*dh][wo*sw - pw + j*dw] (0 in
// the zero padding). The dp_conv_* entry points form these rows on chip; this
// kernel writes them out once, for callers that run the unfolded path (its
// matrix-core kernels read contiguous rows) on a layer they hold folded.
//
// When the kH input rows of all channels that one output row reads fit 48 KB
// of LDS, a workgroup stages them and writes that output row's part of U(a)
// (k_unfold2d_rows); else one thread per element of U(a), gathering from the
// folded input (k_unfold2d; a workgroup covers 256 elements of one sample, so
// the per-sample offsets stay 32-bit).
#include "dp_common.hpp"
#include "dp_launch.hpp"

namespace dpk {

template <typename T>
__global__ __launch_bounds__(256) void k_unfold2d(ConvGeo g, FastDiv by_d, uint32_t blocks_per_sample,
                                                  T* __restrict__ U) {
  const uint32_t b = blockIdx.x / blocks_per_sample;  // wave-uniform
  const uint32_t el = (blockIdx.x - b * blocks_per_sample) * 256u + threadIdx.x;
  const uint32_t n = (uint32_t)g.T * (uint32_t)g.d;  // elements per sample, < 2^31
  if (el >= n) return;
  const uint32_t t = fast_div(el, by_d), f = el - t * (uint32_t)g.d;
  const ConvCol col = conv_col(g, f);
  const uint32_t ho = fast_div(t, g.by_wo), wo = t - ho * (uint32_t)g.Wo;
  const int hi = (int)ho * g.sh - g.ph + col.i * g.dh, wi = (int)wo * g.sw - g.pw + col.j * g.dw;
  T v{};
  if (hi >= 0 && hi < g.H && wi >= 0 && wi < g.W) {
    const T* a = static_cast<const T*>(g.a) + (int64_t)b * g.Cin * g.H * g.W;
    v = a[((int64_t)col.ci * g.H + hi) * g.W + wi];
  }
  U[(int64_t)b * n + el] = v;
}

// One workgroup per (sample b, output row ho): the kH input rows of every
// channel that the row's windows touch are staged in LDS once (zeros for rows
// in the padding), then the workgroup writes the Wo rows of U(a) that this
// output row owns -- one contiguous run of Wo*d elements -- reading the
// window elements from LDS.
template <typename T>
__global__ __launch_bounds__(256) void k_unfold2d_rows(ConvGeo g, FastDiv by_d, FastDiv by_khw_w, FastDiv by_w,
                                                       T* __restrict__ U) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  // [Cin][KH][Wp]: rows padded to an odd pitch, so that lanes reading
  // consecutive channels hit different banks
  T* patch = reinterpret_cast<T*>(lds_raw);
  const uint32_t Wp = (uint32_t)g.W | 1u;
  const uint32_t b = blockIdx.x / (uint32_t)g.Ho, ho = blockIdx.x - b * (uint32_t)g.Ho;
  const T* a = static_cast<const T*>(g.a) + (int64_t)b * g.Cin * g.H * g.W;
  const uint32_t khw = (uint32_t)(g.KH * g.W), npatch = (uint32_t)g.Cin * khw;
  for (uint32_t idx = threadIdx.x; idx < npatch; idx += 256) {
    const uint32_t c = fast_div(idx, by_khw_w), r = idx - c * khw;
    const uint32_t i = fast_div(r, by_w), w = r - i * (uint32_t)g.W;
    const int hi = (int)ho * g.sh - g.ph + (int)i * g.dh;
    T v{};
    if (hi >= 0 && hi < g.H) v = a[((int64_t)c * g.H + hi) * g.W + w];
    patch[(c * (uint32_t)g.KH + i) * Wp + w] = v;
  }
  __syncthreads();
  const uint32_t n = (uint32_t)g.Wo * (uint32_t)g.d;
  T* out = U + ((int64_t)b * g.T + (int64_t)ho * g.Wo) * g.d;
  auto elem = [&](uint32_t wo, int ci, int i, int j) {
    const int wi = (int)wo * g.sw - g.pw + j * g.dw;
    T v{};
    if (wi >= 0 && wi < g.W) v = patch[((uint32_t)ci * (uint32_t)g.KH + (uint32_t)i) * Wp + wi];
    return v;
  };
  constexpr int VEC = 16 / (int)sizeof(T);
  if (g.d % VEC == 0) {
    // VEC consecutive elements of one row per thread, one 16-byte store (the
    // run starts on a 16-byte boundary: U is 16-byte aligned and d % VEC == 0)
    for (uint32_t e = threadIdx.x * VEC; e < n; e += 256 * VEC) {
      const uint32_t wo = fast_div(e, by_d), f = e - wo * (uint32_t)g.d;
      ConvCol col = conv_col(g, f);
      T v[VEC];
#pragma unroll
      for (int k = 0; k < VEC; ++k) {
        v[k] = elem(wo, col.ci, col.i, col.j);
        if (++col.j == g.KW) {  // the next column f + 1
          col.j = 0;
          if (++col.i == g.KH) {
            col.i = 0;
            ++col.ci;
          }
        }
      }
      *reinterpret_cast<uint4*>(out + e) = *reinterpret_cast<const uint4*>(v);
    }
  } else {
    for (uint32_t e = threadIdx.x; e < n; e += 256) {
      const uint32_t wo = fast_div(e, by_d), f = e - wo * (uint32_t)g.d;
      const ConvCol col = conv_col(g, f);
      out[e] = elem(wo, col.ci, col.i, col.j);
    }
  }
}

constexpr int64_t kUnfoldPatchMax = 48 * 1024;  // LDS bytes of the staged rows

hipError_t launch_unfold2d(hipStream_t st, int dtype, const ConvGeo& g, int64_t B, void* U) {
  const int64_t eb = dtype == 1 ? 2 : 4;
  const int64_t patch = (int64_t)g.Cin * g.KH * (g.W | 1) * eb;
  if (patch <= kUnfoldPatchMax && (int64_t)g.Ho * B < (1ll << 31) && (int64_t)g.Wo * g.d < (1ll << 31)) {
    const FastDiv by_d = make_fastdiv((uint32_t)g.d), by_khw_w = make_fastdiv((uint32_t)(g.KH * g.W)),
                  by_w = make_fastdiv((uint32_t)g.W);
    const dim3 grid((unsigned)(g.Ho * B));
    if (dtype == 1)
      hipLaunchKernelGGL(k_unfold2d_rows<bf16s>, grid, dim3(256), (size_t)patch, st, g, by_d, by_khw_w, by_w,
                         static_cast<bf16s*>(U));
    else
      hipLaunchKernelGGL(k_unfold2d_rows<float>, grid, dim3(256), (size_t)patch, st, g, by_d, by_khw_w, by_w,
                         static_cast<float*>(U));
    return hipGetLastError();
  }
  const uint64_t n = (uint64_t)g.T * (uint64_t)g.d;
  if (n == 0 || n >= (1ull << 31)) return hipErrorInvalidValue;
  const uint64_t bps = (n + 255) / 256;
  if (bps * (uint64_t)B >= (1ull << 31)) return hipErrorInvalidValue;
  const FastDiv by_d = make_fastdiv((uint32_t)g.d);
  const dim3 grid((unsigned)(bps * (uint64_t)B));
  if (dtype == 1)
    hipLaunchKernelGGL(k_unfold2d<bf16s>, grid, dim3(256), 0, st, g, by_d, (uint32_t)bps, static_cast<bf16s*>(U));
  else
    hipLaunchKernelGGL(k_unfold2d<float>, grid, dim3(256), 0, st, g, by_d, (uint32_t)bps, static_cast<float*>(U));
  return hipGetLastError();
}

}  // namespace dpk
