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
// One thread per element of U(a): consecutive threads write consecutive
// elements of a row (coalesced stores); the reads are gathers from the folded
// input, which the k*k windows re-read from L2. A workgroup covers 256
// elements of one sample, so the per-sample offsets stay 32-bit.
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

hipError_t launch_unfold2d(hipStream_t st, int dtype, const ConvGeo& g, int64_t B, void* U) {
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
