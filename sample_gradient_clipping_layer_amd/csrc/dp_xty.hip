// X^T Y engine on MFMA for inputs laid out [rows, features] (features
// contiguous), used twice:
//
//  * explicit norm (per-sample instantiation, SEDP App. C.4; FPC Alg. 2-3):
//    workgroup = (sample i, output tile of A_i^T G_i), K = T; the epilogue
//    squares and sums the tile in registers -- the per-sample gradient is
//    never written to memory.
//  * weighted contraction (SEDP eq. (2.1) weighted gradient sum_i C_i g_i,
//    App. C.5; FPC re-weighted loss): S = A^T diag(c) G over K = B*T. With
//    one K split the noise and the 1/denom are applied in the epilogue and
//    the output is written once; with ks > 1 splits, fp32 partial tiles go to
//    the workspace and a fixed-order reduce adds them and the noise.
//
// A bias is a weight on a constant-1 input feature, so X gets a virtual
// column d of ones (rows inside the sample): row d of X^T Y is then
// sum_t G[t, :], the per-sample bias gradient (FPC bias gradient).
//
// Both operands are K-strided in memory, while MFMA wants K-contiguous
// fragments, so each K chunk is transposed through registers on its way to
// LDS ([feature][k], 144-byte rows: conflict-free b128 fragment reads). The
// next chunk's global loads are in flight while the MFMAs of the current one
// run; LDS is double-buffered so one barrier per chunk suffices. Four waves
// in 2 x 2 own (BM/2) x (BN/2) sub-tiles of 32x32 MFMA blocks.
//
// Clip factors: fp32 inputs scale each G row by c while staging (one fp32
// rounding). bf16 inputs keep the products exact: each sample is accumulated
// in its own register tile and added as acc += c_i * tmp.
#include "dp_common.hpp"
#include "dp_launch.hpp"
#include "dp_noise.hpp"

namespace dpk {

template <typename T>
struct XtyCfg;
template <>
struct XtyCfg<float> {
  static constexpr int KC = 32;  // rows per chunk (128 bytes per feature row)
};
template <>
struct XtyCfg<bf16s> {
  static constexpr int KC = 64;
};
constexpr int kRowB = 144;  // LDS bytes per feature row of a chunk (128 + 16 pad)

template <typename T, int BM, int BN>
struct Xty {
  static constexpr int NT = 256;
  static constexpr int P = elem_traits<T>::per16;
  static constexpr int KC = XtyCfg<T>::KC;
  static constexpr int WMt = BM / 2, WNt = BN / 2;
  static constexpr int NBM = WMt / 32, NBN = WNt / 32;
  static constexpr int UX = (KC / 4) * (BM / P);  // staging units (4 rows x 16 bytes) of X per chunk
  static constexpr int UY = (KC / 4) * (BN / P);
  static constexpr int UT = UX + UY;
  static constexpr int UPT = (UT + NT - 1) / NT;  // units per thread
  static constexpr int BUF = (BM + BN) * kRowB;
  static constexpr int LDS_BYTES = 2 * BUF;

  typedef f32x16 AccT[NBM][NBN];

  struct Regs {
    uint4 v[UPT][4];
    float sc[UPT][4];
  };

  // Global loads of one chunk: rows [row0, row0+KC) of X (features m0..) and
  // Y (features n0..). Rows >= nrows and features past the end are zero; the
  // virtual ones column of X is set on valid rows. fp32: Y rows carry c[row/Tn].
  __device__ __forceinline__ static void load(Regs& R, const T* X, int64_t Kx, bool vecx, int64_t ones_col,
                                              const T* Y, int64_t Ky, bool vecy, int64_t nrows, int64_t row0,
                                              int64_t m0, int64_t n0, const float* c, int64_t Tn) {
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int unit = threadIdx.x + u * NT;
      if (unit < UX) {
        const int rq = unit / (BM / P), cu = unit % (BM / P);
        const int64_t col0 = m0 + cu * P;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t row = row0 + rq * 4 + r;
          uint4 v = load16_rowmajor(X, nrows, Kx, row, col0, vecx);
          if (ones_col >= col0 && ones_col < col0 + P && row < nrows) {
            const int e = (int)(ones_col - col0);
            uint32_t w[4] = {v.x, v.y, v.z, v.w};
            if constexpr (P == 8)
              w[e >> 1] |= 0x3F80u << (16 * (e & 1));
            else
              w[e] = 0x3F800000u;
            v = make_uint4(w[0], w[1], w[2], w[3]);
          }
          R.v[u][r] = v;
          R.sc[u][r] = 1.0f;
        }
      } else if (unit < UT) {
        const int uy = unit - UX;
        const int rq = uy / (BN / P), cu = uy % (BN / P);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t row = row0 + rq * 4 + r;
          R.v[u][r] = load16_rowmajor(Y, nrows, Ky, row, n0 + cu * P, vecy);
          float s = 1.0f;
          if constexpr (P == 4) {
            if (c != nullptr) s = row < nrows ? c[row / Tn] : 0.0f;
          }
          R.sc[u][r] = s;
        }
      }
    }
  }

  // Transposed stores of the loaded chunk into LDS rows [feature][k].
  __device__ __forceinline__ static void store(const Regs& R, unsigned char* buf) {
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int unit = threadIdx.x + u * NT;
      if (unit >= UT) continue;
      int rq, fbase;
      if (unit < UX) {
        rq = unit / (BM / P);
        fbase = (unit % (BM / P)) * P;
      } else {
        const int uy = unit - UX;
        rq = uy / (BN / P);
        fbase = BM + (uy % (BN / P)) * P;
      }
      unsigned char* rows = buf + fbase * kRowB;
      const int k0 = rq * 4;
      if constexpr (P == 4) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          float4 o;
          o.x = __uint_as_float(m == 0 ? R.v[u][0].x : m == 1 ? R.v[u][0].y : m == 2 ? R.v[u][0].z : R.v[u][0].w) * R.sc[u][0];
          o.y = __uint_as_float(m == 0 ? R.v[u][1].x : m == 1 ? R.v[u][1].y : m == 2 ? R.v[u][1].z : R.v[u][1].w) * R.sc[u][1];
          o.z = __uint_as_float(m == 0 ? R.v[u][2].x : m == 1 ? R.v[u][2].y : m == 2 ? R.v[u][2].z : R.v[u][2].w) * R.sc[u][2];
          o.w = __uint_as_float(m == 0 ? R.v[u][3].x : m == 1 ? R.v[u][3].y : m == 2 ? R.v[u][3].z : R.v[u][3].w) * R.sc[u][3];
          *reinterpret_cast<float4*>(rows + m * kRowB + k0 * 4) = o;
        }
      } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const int sh = 16 * (m & 1);
          uint32_t e[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint4& v = R.v[u][r];
            const uint32_t w = (m >> 1) == 0 ? v.x : (m >> 1) == 1 ? v.y : (m >> 1) == 2 ? v.z : v.w;
            e[r] = (w >> sh) & 0xFFFFu;
          }
          *reinterpret_cast<uint2*>(rows + m * kRowB + k0 * 2) = make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
        }
      }
    }
  }

  __device__ __forceinline__ static void compute(const unsigned char* buf, AccT& acc) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const unsigned char* xb = buf;
    const unsigned char* yb = buf + BM * kRowB;
    if constexpr (P == 8) {
#pragma unroll
      for (int ks = 0; ks < KC / 16; ++ks) {
        uint4 a[NBM], b[NBN];
#pragma unroll
        for (int bi = 0; bi < NBM; ++bi)
          a[bi] = *reinterpret_cast<const uint4*>(xb + (wm * WMt + bi * 32 + (lane & 31)) * kRowB + ks * 32 +
                                                  (lane >> 5) * 16);
#pragma unroll
        for (int bj = 0; bj < NBN; ++bj)
          b[bj] = *reinterpret_cast<const uint4*>(yb + (wn * WNt + bj * 32 + (lane & 31)) * kRowB + ks * 32 +
                                                  (lane >> 5) * 16);
#pragma unroll
        for (int bi = 0; bi < NBM; ++bi)
#pragma unroll
          for (int bj = 0; bj < NBN; ++bj) acc[bi][bj] = mfma32_bf16(a[bi], b[bj], acc[bi][bj]);
      }
    } else {
#pragma unroll
      for (int g = 0; g < KC / 8; ++g) {
        float4 a[NBM], b[NBN];
#pragma unroll
        for (int bi = 0; bi < NBM; ++bi)
          a[bi] = *reinterpret_cast<const float4*>(xb + (wm * WMt + bi * 32 + (lane & 31)) * kRowB + g * 32 +
                                                   (lane >> 5) * 16);
#pragma unroll
        for (int bj = 0; bj < NBN; ++bj)
          b[bj] = *reinterpret_cast<const float4*>(yb + (wn * WNt + bj * 32 + (lane & 31)) * kRowB + g * 32 +
                                                   (lane >> 5) * 16);
#pragma unroll
        for (int bi = 0; bi < NBM; ++bi)
#pragma unroll
          for (int bj = 0; bj < NBN; ++bj) {
            acc[bi][bj] = mfma32_f32(a[bi].x, b[bj].x, acc[bi][bj]);
            acc[bi][bj] = mfma32_f32(a[bi].y, b[bj].y, acc[bi][bj]);
            acc[bi][bj] = mfma32_f32(a[bi].z, b[bj].z, acc[bi][bj]);
            acc[bi][bj] = mfma32_f32(a[bi].w, b[bj].w, acc[bi][bj]);
          }
      }
    }
  }

  __device__ __forceinline__ static void zero(AccT& acc) {
#pragma unroll
    for (int bi = 0; bi < NBM; ++bi)
#pragma unroll
      for (int bj = 0; bj < NBN; ++bj)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[bi][bj][j] = 0.f;
  }
};

// ---------------------------------------------------------------- explicit
template <typename T, int BM, int BN>
__global__ __launch_bounds__(256, 2) void k_explicit_tiles(const T* __restrict__ A, const T* __restrict__ G,
                                                           int64_t B, int64_t Tn, int64_t d, int64_t p, int has_bias,
                                                           int mt, int nt, int vecA, int vecG,
                                                           float* __restrict__ partial) {
  using E = Xty<T, BM, BN>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[E::LDS_BYTES];
  __shared__ float red[E::NT / kWave];
  const int ntl = mt * nt;
  int64_t i, tile;
  xcd_group_map(blockIdx.x, ntl, &i, &tile);
  if (i >= B) return;
  const int64_t m0 = (tile / nt) * BM;
  const int64_t n0 = (tile % nt) * BN;
  const T* Xi = A + i * Tn * d;
  const T* Yi = G + i * Tn * p;
  const int64_t ones_col = has_bias ? d : -1;

  typename E::AccT acc;
  E::zero(acc);
  typename E::Regs R;
  const int64_t nq = (Tn + E::KC - 1) / E::KC;
  E::load(R, Xi, d, vecA != 0, ones_col, Yi, p, vecG != 0, Tn, 0, m0, n0, nullptr, Tn);
  for (int64_t q = 0; q < nq; ++q) {
    unsigned char* buf = lds + (q & 1) * E::BUF;
    E::store(R, buf);
    __syncthreads();
    if (q + 1 < nq)
      E::load(R, Xi, d, vecA != 0, ones_col, Yi, p, vecG != 0, Tn, (q + 1) * E::KC, m0, n0, nullptr, Tn);
    E::compute(buf, acc);
  }
  float s = 0.f;
#pragma unroll
  for (int bi = 0; bi < E::NBM; ++bi)
#pragma unroll
    for (int bj = 0; bj < E::NBN; ++bj)
#pragma unroll
      for (int j = 0; j < 16; ++j) s += acc[bi][bj][j] * acc[bi][bj][j];
  s = block_sum<E::NT>(s, red);
  if (threadIdx.x == 0) partial[i * ntl + tile] = s;
}

// ---------------------------------------------------------------- contraction
struct NoiseArgs {
  float sc, denom;
  uint32_t k0, k1, layer, step;
};

// Workgroup = (output tile, K split). FUSED (one split): out and bias_out get
// (S + sc*z)/denom directly. Otherwise ws[split][m][n] (m < d + has_bias).
template <typename T, int BM, int BN, bool FUSED>
__global__ __launch_bounds__(256, 2) void k_contract_tiles(const T* __restrict__ A, const T* __restrict__ G,
                                                           const float* __restrict__ c, int64_t B, int64_t Tn,
                                                           int64_t d, int64_t p, int has_bias, int mt, int nt,
                                                           int64_t units_per_split, int vecA, int vecG,
                                                           float* __restrict__ ws, NoiseArgs na,
                                                           float* __restrict__ out, float* __restrict__ bias_out) {
  using E = Xty<T, BM, BN>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[E::LDS_BYTES];
  const int ntl = mt * nt;
  const int tile = (int)(blockIdx.x % ntl);
  const int64_t split = blockIdx.x / ntl;
  const int64_t m0 = (tile / nt) * BM;
  const int64_t n0 = (tile % nt) * BN;
  const int64_t ones_col = has_bias ? d : -1;
  const int64_t mrows = d + (has_bias ? 1 : 0);

  typename E::AccT acc;
  E::zero(acc);
  typename E::Regs R;
  if constexpr (E::P == 4) {
    // flat K over all B*T rows in chunks of KC rows; G rows scaled by c[row / T]
    const int64_t nrows = B * Tn;
    const int64_t nunits = (nrows + E::KC - 1) / E::KC;
    const int64_t u0 = split * units_per_split;
    const int64_t u1 = u0 + units_per_split < nunits ? u0 + units_per_split : nunits;
    if (u0 < u1) E::load(R, A, d, vecA != 0, ones_col, G, p, vecG != 0, nrows, u0 * E::KC, m0, n0, c, Tn);
    for (int64_t u = u0; u < u1; ++u) {
      unsigned char* buf = lds + ((u - u0) & 1) * E::BUF;
      E::store(R, buf);
      __syncthreads();
      if (u + 1 < u1) E::load(R, A, d, vecA != 0, ones_col, G, p, vecG != 0, nrows, (u + 1) * E::KC, m0, n0, c, Tn);
      E::compute(buf, acc);
    }
  } else {
    // per-sample exact accumulation: acc += c_i * (A_i^T G_i tile)
    const int64_t i0 = split * units_per_split;
    const int64_t i1 = i0 + units_per_split < B ? i0 + units_per_split : B;
    const int64_t cps = (Tn + E::KC - 1) / E::KC;  // chunks per sample
    const int64_t nq = (i1 > i0 ? i1 - i0 : 0) * cps;
    typename E::AccT tmp;
    E::zero(tmp);
    if (nq > 0) E::load(R, A + i0 * Tn * d, d, vecA != 0, ones_col, G + i0 * Tn * p, p, vecG != 0, Tn, 0, m0, n0,
                        nullptr, Tn);
    for (int64_t q = 0; q < nq; ++q) {
      unsigned char* buf = lds + (q & 1) * E::BUF;
      E::store(R, buf);
      __syncthreads();
      if (q + 1 < nq) {
        const int64_t in = i0 + (q + 1) / cps, chn = (q + 1) % cps;
        E::load(R, A + in * Tn * d, d, vecA != 0, ones_col, G + in * Tn * p, p, vecG != 0, Tn, chn * E::KC, m0, n0,
                nullptr, Tn);
      }
      E::compute(buf, tmp);
      if (q % cps == cps - 1) {
        const float ci = c[i0 + q / cps];
#pragma unroll
        for (int bi = 0; bi < E::NBM; ++bi)
#pragma unroll
          for (int bj = 0; bj < E::NBN; ++bj)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              acc[bi][bj][j] += ci * tmp[bi][bj][j];
              tmp[bi][bj][j] = 0.f;
            }
      }
    }
  }

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  if constexpr (FUSED) {
    // lane holds rows 8*j4 + 4*(lane/32) + r (r = 0..3) of column lane%32 in
    // each 32x32 block: one Philox block covers exactly those 4 rows
#pragma unroll
    for (int bi = 0; bi < E::NBM; ++bi)
#pragma unroll
      for (int bj = 0; bj < E::NBN; ++bj)
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          const int64_t mb = m0 + wm * E::WMt + bi * 32 + 8 * j4 + 4 * (lane >> 5);
          const int64_t n = n0 + wn * E::WNt + bj * 32 + (lane & 31);
          if (n >= p) continue;
          if (mb < d) {
            const f32x4 z = normals4((uint32_t)((mb >> 2) * p + n), 2u * na.layer, na.step, 0u, na.k0, na.k1);
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (mb + r < d) out[(mb + r) * p + n] = noised_mean_spec(acc[bi][bj][4 * j4 + r], na.sc, z[r], na.denom);
          }
          if (has_bias && d >= mb && d < mb + 4) {
            const f32x4 zb = normals4((uint32_t)(n >> 2), 2u * na.layer + 1u, na.step, 0u, na.k0, na.k1);
            const int r = (int)(d - mb);
            bias_out[n] = noised_mean_spec(acc[bi][bj][4 * j4 + r], na.sc, zb[(int)(n & 3)], na.denom);
          }
        }
  } else {
    float* wsp = ws + split * mrows * p;
#pragma unroll
    for (int bi = 0; bi < E::NBM; ++bi)
#pragma unroll
      for (int bj = 0; bj < E::NBN; ++bj)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int64_t m = m0 + wm * E::WMt + bi * 32 + acc_row(j, lane);
          const int64_t n = n0 + wn * E::WNt + bj * 32 + acc_col(lane);
          if (m < mrows && n < p) wsp[m * p + n] = acc[bi][bj][j];
        }
  }
}

// ---------------------------------------------------------------- reduce + noise
// Thread = 4 rows x 4 columns of the weight output (rows 4q..4q+3, columns
// 4c..4c+3): sum the ks partials in split order, then each column's 4 rows
// take the 4 normals of one Philox block. Threads past the weight blocks do
// the bias row, 4 columns (one flat block) each.
__global__ __launch_bounds__(256) void k_reduce_noise(const float* __restrict__ ws, int64_t ks, int64_t d, int64_t p,
                                                      int has_bias, int vec, NoiseArgs na, float* __restrict__ out,
                                                      float* __restrict__ bias_out) {
  const int64_t nq = (d + 3) / 4, nc = (p + 3) / 4;
  const int64_t nw = nq * nc;
  const int64_t nb = has_bias ? nc : 0;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= nw + nb) return;
  const int64_t split_stride = (d + (has_bias ? 1 : 0)) * p;
  if (t < nw) {
    const int64_t q = t / nc, cq = t % nc;
    float s[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int k = 0; k < 4; ++k) s[r][k] = 0.f;
    for (int64_t sp = 0; sp < ks; ++sp) {
      const float* base = ws + sp * split_stride;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = 4 * q + r;
        if (m >= d) continue;
        if (vec && 4 * cq + 4 <= p) {
          const float4 v = *reinterpret_cast<const float4*>(base + m * p + 4 * cq);
          s[r][0] += v.x;
          s[r][1] += v.y;
          s[r][2] += v.z;
          s[r][3] += v.w;
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (4 * cq + k < p) s[r][k] += base[m * p + 4 * cq + k];
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t n = 4 * cq + k;
      if (n >= p) continue;
      const f32x4 z = normals4((uint32_t)(q * p + n), 2u * na.layer, na.step, 0u, na.k0, na.k1);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = 4 * q + r;
        if (m < d) s[r][k] = noised_mean_spec(s[r][k], na.sc, z[r], na.denom);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = 4 * q + r;
      if (m >= d) continue;
      if (vec && 4 * cq + 4 <= p) {
        *reinterpret_cast<float4*>(out + m * p + 4 * cq) = make_float4(s[r][0], s[r][1], s[r][2], s[r][3]);
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (4 * cq + k < p) out[m * p + 4 * cq + k] = s[r][k];
      }
    }
  } else {
    const int64_t cq = t - nw;
    const f32x4 z = normals4((uint32_t)cq, 2u * na.layer + 1u, na.step, 0u, na.k0, na.k1);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t n = 4 * cq + k;
      if (n >= p) continue;
      float s = 0.f;
      for (int64_t sp = 0; sp < ks; ++sp) s += ws[sp * split_stride + d * p + n];
      bias_out[n] = noised_mean_spec(s, na.sc, z[k], na.denom);
    }
  }
}

// ---------------------------------------------------------------- plans
static int pick_tile(int64_t n) {
  // 64 or 128, whichever pads n less (ties -> 128)
  const int64_t p64 = (n + 63) / 64 * 64, p128 = (n + 127) / 128 * 128;
  return p64 < p128 ? 64 : 128;
}

ContractPlan contract_plan(int dtype, int64_t B, int64_t Tn, int64_t d, int64_t p, int has_bias) {
  ContractPlan pl;
  const int64_t mrows = d + (has_bias ? 1 : 0);
  pl.bm = pick_tile(mrows);
  pl.bn = pick_tile(p);
  pl.mt = (int)((mrows + pl.bm - 1) / pl.bm);
  pl.nt = (int)((p + pl.bn - 1) / pl.bn);
  const int64_t kc = dtype == 1 ? XtyCfg<bf16s>::KC : XtyCfg<float>::KC;
  const int64_t units = dtype == 1 ? B : (B * Tn + kc - 1) / kc;
  const int64_t ntl = (int64_t)pl.mt * pl.nt;
  // about two workgroups per CU (256 CUs); no split once the tiles alone fill most of the chip
  int64_t ks = ntl >= 192 ? 1 : (512 + ntl - 1) / ntl;
  if (ks > units) ks = units;
  if (ks < 1) ks = 1;
  pl.units_per_split = (units + ks - 1) / ks;
  pl.ks = (units + pl.units_per_split - 1) / pl.units_per_split;
  return pl;
}

ExplicitPlan explicit_plan(int64_t d, int64_t p, int has_bias) {
  ExplicitPlan pl;
  pl.bm = pick_tile(d + (has_bias ? 1 : 0));
  pl.bn = pick_tile(p);
  pl.mt = (int)((d + (has_bias ? 1 : 0) + pl.bm - 1) / pl.bm);
  pl.nt = (int)((p + pl.bn - 1) / pl.bn);
  return pl;
}

// ---------------------------------------------------------------- launchers
template <typename T, int BM, int BN>
static hipError_t launch_explicit_t(hipStream_t st, const void* A, const void* G, int64_t B, int64_t Tn, int64_t d,
                                    int64_t p, int has_bias, const ExplicitPlan& pl, float* partial) {
  const int eb = elem_traits<T>::bytes;
  const int vecA = ((reinterpret_cast<uintptr_t>(A) & 15) == 0) && ((d * eb) % 16 == 0);
  const int vecG = ((reinterpret_cast<uintptr_t>(G) & 15) == 0) && ((p * eb) % 16 == 0);
  const int64_t ntl = (int64_t)pl.mt * pl.nt;
  const dim3 grid((unsigned)((B + 7) / 8 * 8 * ntl));
  hipLaunchKernelGGL((k_explicit_tiles<T, BM, BN>), grid, dim3(256), 0, st, static_cast<const T*>(A),
                     static_cast<const T*>(G), B, Tn, d, p, has_bias, pl.mt, pl.nt, vecA, vecG, partial);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_explicit_d(hipStream_t st, const void* A, const void* G, int64_t B, int64_t Tn, int64_t d,
                                    int64_t p, int has_bias, const ExplicitPlan& pl, float* partial) {
  if (pl.bm == 64 && pl.bn == 64) return launch_explicit_t<T, 64, 64>(st, A, G, B, Tn, d, p, has_bias, pl, partial);
  if (pl.bm == 64) return launch_explicit_t<T, 64, 128>(st, A, G, B, Tn, d, p, has_bias, pl, partial);
  if (pl.bn == 64) return launch_explicit_t<T, 128, 64>(st, A, G, B, Tn, d, p, has_bias, pl, partial);
  return launch_explicit_t<T, 128, 128>(st, A, G, B, Tn, d, p, has_bias, pl, partial);
}

hipError_t launch_explicit(hipStream_t st, int dtype, const void* A, const void* G, int64_t B, int64_t Tn, int64_t d,
                           int64_t p, int has_bias, float* partial) {
  const ExplicitPlan pl = explicit_plan(d, p, has_bias);
  if (dtype == 1) return launch_explicit_d<bf16s>(st, A, G, B, Tn, d, p, has_bias, pl, partial);
  return launch_explicit_d<float>(st, A, G, B, Tn, d, p, has_bias, pl, partial);
}

template <typename T, int BM, int BN>
static hipError_t launch_contract_t(hipStream_t st, const void* A, const void* G, const float* c, int64_t B,
                                    int64_t Tn, int64_t d, int64_t p, int has_bias, const ContractPlan& pl,
                                    float* ws, const NoiseArgs& na, float* out, float* bias_out) {
  const int eb = elem_traits<T>::bytes;
  const int vecA = ((reinterpret_cast<uintptr_t>(A) & 15) == 0) && ((d * eb) % 16 == 0);
  const int vecG = ((reinterpret_cast<uintptr_t>(G) & 15) == 0) && ((p * eb) % 16 == 0);
  const dim3 grid((unsigned)((int64_t)pl.mt * pl.nt * pl.ks));
  if (pl.ks == 1) {
    hipLaunchKernelGGL((k_contract_tiles<T, BM, BN, true>), grid, dim3(256), 0, st, static_cast<const T*>(A),
                       static_cast<const T*>(G), c, B, Tn, d, p, has_bias, pl.mt, pl.nt, pl.units_per_split, vecA,
                       vecG, ws, na, out, bias_out);
  } else {
    hipLaunchKernelGGL((k_contract_tiles<T, BM, BN, false>), grid, dim3(256), 0, st, static_cast<const T*>(A),
                       static_cast<const T*>(G), c, B, Tn, d, p, has_bias, pl.mt, pl.nt, pl.units_per_split, vecA,
                       vecG, ws, na, out, bias_out);
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_contract_d(hipStream_t st, const void* A, const void* G, const float* c, int64_t B,
                                    int64_t Tn, int64_t d, int64_t p, int has_bias, const ContractPlan& pl,
                                    float* ws, const NoiseArgs& na, float* out, float* bias_out) {
  if (pl.bm == 64 && pl.bn == 64)
    return launch_contract_t<T, 64, 64>(st, A, G, c, B, Tn, d, p, has_bias, pl, ws, na, out, bias_out);
  if (pl.bm == 64) return launch_contract_t<T, 64, 128>(st, A, G, c, B, Tn, d, p, has_bias, pl, ws, na, out, bias_out);
  if (pl.bn == 64) return launch_contract_t<T, 128, 64>(st, A, G, c, B, Tn, d, p, has_bias, pl, ws, na, out, bias_out);
  return launch_contract_t<T, 128, 128>(st, A, G, c, B, Tn, d, p, has_bias, pl, ws, na, out, bias_out);
}

hipError_t launch_clipped_sum(hipStream_t st, int dtype, const void* A, const void* G, const float* c, int64_t B,
                              int64_t Tn, int64_t d, int64_t p, const ContractPlan& pl, float* ws, float sc,
                              float denom, uint64_t seed, uint32_t layer, uint32_t step, float* out,
                              float* bias_out) {
  const int has_bias = bias_out != nullptr ? 1 : 0;
  NoiseArgs na;
  na.sc = sc;
  na.denom = denom;
  na.k0 = (uint32_t)(seed & 0xFFFFFFFFu);
  na.k1 = (uint32_t)(seed >> 32);
  na.layer = layer;
  na.step = step;
  hipError_t e = dtype == 1 ? launch_contract_d<bf16s>(st, A, G, c, B, Tn, d, p, has_bias, pl, ws, na, out, bias_out)
                            : launch_contract_d<float>(st, A, G, c, B, Tn, d, p, has_bias, pl, ws, na, out, bias_out);
  if (e != hipSuccess || pl.ks == 1) return e;
  const int vec = (p % 4 == 0) && ((reinterpret_cast<uintptr_t>(out) & 15) == 0);
  const int64_t threads = ((d + 3) / 4) * ((p + 3) / 4) + (has_bias ? (p + 3) / 4 : 0);
  const dim3 grid((unsigned)((threads + 255) / 256));
  hipLaunchKernelGGL(k_reduce_noise, grid, dim3(256), 0, st, ws, pl.ks, d, p, has_bias, vec, na, out, bias_out);
  return hipGetLastError();
}

}  // namespace dpk
