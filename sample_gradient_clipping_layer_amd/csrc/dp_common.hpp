// Shared device helpers for the clipping kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dpk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
// 16 bytes as a native vector (not HIP's uint4 wrapper class: whole-object
// copies of the wrapper keep register arrays from being promoted out of
// private memory).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// Storage type of a bf16 element (bit pattern); fp32 is plain float.
struct bf16s {
  uint16_t u;
};

template <typename T>
struct elem_traits;
template <>
struct elem_traits<float> {
  static constexpr int bytes = 4;
  static constexpr int per16 = 4;  // elements per 16-byte vector
};
template <>
struct elem_traits<bf16s> {
  static constexpr int bytes = 2;
  static constexpr int per16 = 8;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16s x) { return __uint_as_float((uint32_t)x.u << 16); }

// Raw bits of one element, widened to 32 bits (bf16 -> low 16 bits).
__device__ __forceinline__ uint32_t raw_bits(float x) { return __float_as_uint(x); }
__device__ __forceinline__ uint32_t raw_bits(bf16s x) { return x.u; }

// Sum over the 64 lanes of a wave in a fixed butterfly order. Every lane ends
// with a value; lane 0's is used, and it is the same from run to run.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Sum over the block (NT threads) in a fixed order; valid in thread 0.
// `red` is LDS scratch of NT/64 floats. Contains a barrier: every thread of
// the block must call it.
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  if (threadIdx.x == 0) {
#pragma unroll
    for (int i = 0; i < NT / kWave; ++i) s += red[i];
  }
  return s;
}

// 16-byte load of elements [k, k+per16) of row `row` of an [nrows, K] matrix
// (row-major), zero outside [0, nrows) x [0, K). `vec` says every row starts
// 16-byte aligned (base aligned and K*bytes % 16 == 0), so a full vector
// load is legal when the whole vector is inside the row.
template <typename T>
__device__ __forceinline__ u32x4 load16_rowmajor(const T* __restrict__ X, int64_t nrows, int64_t K,
                                                 int64_t row, int64_t k, bool vec) {
  constexpr int P = elem_traits<T>::per16;
  u32x4 r = {0u, 0u, 0u, 0u};
  if (row < 0 || row >= nrows) return r;
  const T* src = X + row * K;
  if (vec && k + P <= K) {
    r = *reinterpret_cast<const u32x4*>(src + k);
    return r;
  }
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < P; ++e) {
    const int64_t kk = k + e;
    uint32_t bits = 0u;
    if (kk < K) bits = raw_bits(src[kk]);
    if constexpr (P == 8) {
      w[e >> 1] |= bits << (16 * (e & 1));
    } else {
      w[e] = bits;
    }
  }
  r[0] = w[0];
  r[1] = w[1];
  r[2] = w[2];
  r[3] = w[3];
  return r;
}

// Unsigned 32-bit division by a divisor fixed for a launch, as a multiply
// and a shift (Granlund and Montgomery, "Division by Invariant Integers using
// Multiplication", 1994): with s = ceil(log2 d) and
// m = floor(2^32 (2^s - d) / d) + 1, n / d = (hi32(n * m) + n) >> s for every
// 32-bit n (the sum is formed in 64 bits).
struct FastDiv {
  uint32_t m;
  int32_t s;
};
inline FastDiv make_fastdiv(uint32_t d) {
  int s = 0;
  while ((uint64_t{1} << s) < d) ++s;
  const uint64_t num = (uint64_t{1} << 32) * ((uint64_t{1} << s) - d);
  return FastDiv{(uint32_t)(num / d + 1), s};
}
__device__ __forceinline__ uint32_t fast_div(uint32_t n, FastDiv f) {
  return (uint32_t)(((uint64_t)__umulhi(n, f.m) + n) >> f.s);
}

// A 2-D convolution layer given by its folded input a [B, Cin, H, W]: row t of
// sample b's unfolded input U(a) (t = ho*Wo + wo) holds, in column
// f = (ci*KH + i)*KW + j, a[b][ci][ho*sh - ph + i*dh][wo*sw - pw + j*dw], or 0
// in the zero padding ("Scalable and Efficient Training of Large CNNs with
// DP", Sec. 2.2, the unfolding U). T = Ho*Wo rows, d = Cin*KH*KW columns.
// Every size and per-sample offset fits 32 bits: the host checks
// (Cin + 2) * (H + 2ph) * (W + 2pw) < 2^31, which bounds the column offsets,
// the window origins y0*W + x0 and their sums.
struct ConvGeo {
  const void* a;
  int32_t Cin, H, W, KH, KW, sh, sw, ph, pw, dh, dw, Ho, Wo, T, d;
  FastDiv by_khw, by_kw, by_wo, by_t;  // division by KH*KW, KW, Wo and T
};

// Column f0 of U(a) as (channel, kernel row, kernel column).
struct ConvCol {
  int ci, i, j;
};
__device__ __forceinline__ ConvCol conv_col(const ConvGeo& g, int64_t f0) {
  const uint32_t f = (uint32_t)f0;
  const uint32_t ci = fast_div(f, g.by_khw), r = f - ci * (uint32_t)(g.KH * g.KW);
  const uint32_t i = fast_div(r, g.by_kw);
  return ConvCol{(int)ci, (int)i, (int)(r - i * (uint32_t)g.KW)};
}

// A row of U(a) as (sample, output row, output column); next() steps to the
// following flat row b*T + t.
struct ConvRow {
  int64_t b;
  int ho, wo;
  __device__ __forceinline__ void next(const ConvGeo& g) {
    if (++wo == g.Wo) {
      wo = 0;
      if (++ho == g.Ho) {
        ho = 0;
        ++b;
      }
    }
  }
};
__device__ __forceinline__ ConvRow conv_row_at(const ConvGeo& g, int64_t b, int t) {
  const int ho = (int)fast_div((uint32_t)t, g.by_wo);
  return ConvRow{b, ho, t - ho * g.Wo};
}
// Row `flat` = b*T + t of the unfolded input of the whole batch.
__device__ __forceinline__ ConvRow conv_row_flat(const ConvGeo& g, int64_t flat) {
  int64_t b;
  if ((uint64_t)flat <= 0xFFFFFFFFull)
    b = fast_div((uint32_t)flat, g.by_t);
  else
    b = flat / g.T;
  return conv_row_at(g, b, (int)(flat - b * g.T));
}

// The per16 columns [f0, f0 + per16) of U(a), each as its offset in a
// sample's folded input from the window origin, (ci*H + i*dh)*W + j*dw, and its
// tap displacement (i*dh, j*dw); `in` says the column is one of U(a)'s d
// columns, `one` that it is the ones column of the bias.
template <int P>
struct ConvCols {
  int off[P], dy[P], dx[P];
  bool in[P], one[P];
};
template <int P>
__device__ __forceinline__ ConvCols<P> conv_cols(const ConvGeo& g, int64_t f0, int64_t ones_col) {
  ConvCols<P> k;
  const ConvCol c = conv_col(g, f0);
  int ci = c.ci, i = c.i, j = c.j;
#pragma unroll
  for (int e = 0; e < P; ++e) {
    const int64_t f = f0 + e;
    k.in[e] = f < g.d;
    k.one[e] = f == ones_col;
    k.dy[e] = i * g.dh;
    k.dx[e] = j * g.dw;
    k.off[e] = k.in[e] ? (ci * g.H + k.dy[e]) * g.W + k.dx[e] : 0;
    if (++j == g.KW) {
      j = 0;
      if (++i == g.KH) {
        i = 0;
        ++ci;
      }
    }
  }
  return k;
}

// Columns `k` of row `rw` of U(a) as one 16-byte vector: zero in the padding,
// past column d and everywhere when !row_ok; the ones column reads 1. An
// element is read only where its input position (y, x) lies inside the H x W
// input, where its offset equals ((ci*H + y)*W + x).
template <typename T>
__device__ __forceinline__ u32x4 conv_row16(const ConvGeo& g, const ConvRow& rw,
                                            const ConvCols<elem_traits<T>::per16>& k, bool row_ok) {
  constexpr int P = elem_traits<T>::per16;
  constexpr uint32_t one_bits = P == 8 ? 0x3F80u : 0x3F800000u;
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  if (row_ok) {
    const int y0 = rw.ho * g.sh - g.ph, x0 = rw.wo * g.sw - g.pw;
    const int org = y0 * g.W + x0;
    const T* __restrict__ ab = static_cast<const T*>(g.a) + rw.b * (int64_t)g.Cin * g.H * g.W;
#pragma unroll
    for (int e = 0; e < P; ++e) {
      uint32_t bits = k.one[e] ? one_bits : 0u;
      if (k.in[e] && (unsigned)(y0 + k.dy[e]) < (unsigned)g.H && (unsigned)(x0 + k.dx[e]) < (unsigned)g.W)
        bits = raw_bits(ab[k.off[e] + org]);
      if constexpr (P == 8)
        w[e >> 1] |= bits << (16 * (e & 1));
      else
        w[e] = bits;
    }
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// conv_row16 for columns given by their first one (c0 = conv_col(g, f0)),
// stepping the kernel offsets element by element: fewer registers than a
// ConvCols set, which suits kernels that gather several rows per thread with
// little reuse of the column set (the tiled ghost kernel).
template <typename T>
__device__ __forceinline__ u32x4 conv_row16_walk(const ConvGeo& g, const ConvRow& rw, ConvCol c0, int64_t f0,
                                                 bool row_ok) {
  constexpr int P = elem_traits<T>::per16;
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  if (row_ok) {
    const int y0 = rw.ho * g.sh - g.ph, x0 = rw.wo * g.sw - g.pw;
    const T* __restrict__ ab = static_cast<const T*>(g.a) + rw.b * (int64_t)g.Cin * g.H * g.W;
    int ci = c0.ci, i = c0.i, j = c0.j;
#pragma unroll
    for (int e = 0; e < P; ++e) {
      uint32_t bits = 0u;
      if (f0 + e < g.d) {
        const int y = y0 + i * g.dh, x = x0 + j * g.dw;
        if ((unsigned)y < (unsigned)g.H && (unsigned)x < (unsigned)g.W) bits = raw_bits(ab[(ci * g.H + y) * g.W + x]);
      }
      if constexpr (P == 8)
        w[e >> 1] |= bits << (16 * (e & 1));
      else
        w[e] = bits;
      if (++j == g.KW) {
        j = 0;
        if (++i == g.KH) {
          i = 0;
          ++ci;
        }
      }
    }
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// A pointer every lane of the wave holds, taken from lane 0 so that it lives
// in scalar registers (a scalar base for the direct-to-LDS loads). Each half
// goes through uint32_t: readfirstlane returns a signed int, and widening it
// directly would sign-extend a low word with bit 31 set into the high word.
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
}

// D += A * B on one 32x32 output block, K = 16 (bf16 inputs).
__device__ __forceinline__ f32x16 mfma32_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
// D += A * B on one 32x32 output block, K = 2 (fp32 inputs, one per lane).
__device__ __forceinline__ f32x16 mfma32_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Position of accumulator element j of a 32x32 MFMA block held by `lane`:
// column = lane % 32, row = 8*(j/4) + 4*(lane/32) + j%4.
__device__ __forceinline__ int acc_row(int j, int lane) { return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3); }
__device__ __forceinline__ int acc_col(int lane) { return lane & 31; }

// Workgroup -> (group, item) map that keeps all items of one group on one XCD.
// Workgroups are dispatched to the 8 XCDs round robin by their linear id, so
// id % 8 is the XCD. Groups g with g % 8 == xcd are served by that XCD.
__device__ __forceinline__ void xcd_group_map(int64_t bid, int64_t items, int64_t* group, int64_t* item) {
  const int64_t xcd = bid & 7;
  const int64_t local = bid >> 3;
  *item = local % items;
  *group = (local / items) * 8 + xcd;
}

// s_waitcnt with vmcnt(n), expcnt and lgkmcnt left at their maxima (no wait).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Correctly rounded fp32 square root (through the double-precision one).
__device__ __forceinline__ float sqrt_rn_f32(float x) { return (float)__dsqrt_rn((double)x); }

// Clip factor of one sample from its squared norm: norm = sqrt(sq) with
// negative round-off clamped to 0 (NaN kept); c = C / norm when norm > C,
// else 1 (NaN norm -> NaN; infinite norm -> 0). FPC clip_c; SEDP App. C,
// C_i = min(R/||g_i||, 1).
__device__ __forceinline__ void clip_factor_of(float sq, float C, float* c, float* norm) {
  const float s = sq < 0.0f ? 0.0f : sq;
  const float n = sqrt_rn_f32(s);
  float ci;
  if (n > C)
    ci = __fdiv_rn(C, n);
  else
    ci = (n == n) ? 1.0f : n;
  *c = ci;
  if (norm) *norm = n;
}

// Layers one grouped norm launch can take.
constexpr int kNormGroupMax = 8;

// Where a per-sample norm assembled from `ntiles` tile workgroups goes. The
// tiles may belong to several layers (a grouped launch): layer l owns tiles
// [lt[l], lt[l+1]) of each sample, lt[0] = 0, lt[nlayers] = ntiles. Each
// layer's value is the sum of its tile partials in tile order; sqnorm[i]
// then takes the layers in order, as calls with accumulate = 1 after the
// first would: sqnorm[i] = ((start + n_0) + n_1) + ..., start = sqnorm[i]
// when accumulating, else the first layer's value stands alone.
//
// With one tile per sample the tile's workgroup writes sqnorm (and the clip
// factors) itself. With several, each tile stores its partial and the finish
// kernel (k_norm_finish), launched after the tiles' kernel on the same stream,
// folds them: the kernel boundary orders the partials before their reads, so
// no workgroup waits for or signals another.
struct NormSink {
  float* partial;                 // [B][ntiles] (unused when ntiles == 1)
  float* sqnorm;
  int ntiles;
  int accumulate;
  int nlayers;
  int lt[kNormGroupMax + 1];
  float* clip_c;                  // when set: clip factors (and clip_norm, when set) of the final sqnorm
  float* clip_norm;
  float C;
};

// A sink for one layer of `ntiles` tiles per sample.
inline NormSink make_norm_sink(float* partial, float* sqnorm, int ntiles, int accumulate) {
  NormSink k{};
  k.partial = partial;
  k.sqnorm = sqnorm;
  k.ntiles = ntiles;
  k.accumulate = accumulate;
  k.nlayers = 1;
  k.lt[0] = 0;
  k.lt[1] = ntiles;
  return k;
}

// Called by ONE thread per tile workgroup with the tile's partial s.
__device__ __forceinline__ void norm_sink_tile(const NormSink& k, int64_t i, int64_t tile, float s) {
  if (k.ntiles == 1) {
    const float tot = 0.f + s;
    const float v = k.accumulate ? k.sqnorm[i] + tot : tot;
    k.sqnorm[i] = v;
    if (k.clip_c) clip_factor_of(v, k.C, k.clip_c + i, k.clip_norm ? k.clip_norm + i : nullptr);
    return;
  }
  k.partial[i * k.ntiles + tile] = s;
}

// The fold of sample i's tile partials (sink with ntiles > 1), in tile order
// within a layer and layer order across layers, then its clip factor.
__device__ __forceinline__ void norm_sink_finish(const NormSink& k, int64_t i) {
  const float* row = k.partial + i * k.ntiles;
  float v = k.accumulate ? k.sqnorm[i] : 0.f;
  for (int l = 0; l < k.nlayers; ++l) {
    float tot = 0.f;
    for (int t = k.lt[l]; t < k.lt[l + 1]; ++t) tot += row[t];
    v = (l == 0 && !k.accumulate) ? tot : v + tot;
  }
  k.sqnorm[i] = v;
  if (k.clip_c) clip_factor_of(v, k.C, k.clip_c + i, k.clip_norm ? k.clip_norm + i : nullptr);
}

}  // namespace dpk
