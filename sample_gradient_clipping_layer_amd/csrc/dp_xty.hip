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
  static constexpr int RU = 4;   // rows per staging unit (4 x 4 floats, transposed)
};
template <>
struct XtyCfg<bf16s> {
  static constexpr int KC = 64;
  static constexpr int RU = 8;   // rows per staging unit (8 x 8 bf16, transposed)
};
constexpr int kRowB = 144;  // LDS bytes per feature row of a chunk (128 + 16 pad)

// Where chunk rows come from: X rows at xp, Y rows at yp (row r of the chunk at
// xp + r*Kx), rv of the KC rows valid; fp32 rows are scaled by c[(r0 + r) / Tn].
template <typename T>
struct ChunkSrc {
  const T* xp;
  const T* yp;
  int rv;
  int64_t r0;  // flat row index of chunk row 0 (for the clip factor)
};

template <typename T, int BM, int BN>
struct Xty {
  static constexpr int NT = 256;
  static constexpr int P = elem_traits<T>::per16;
  static constexpr int KC = XtyCfg<T>::KC;
  static constexpr int RU = XtyCfg<T>::RU;
  static constexpr int WMt = BM / 2, WNt = BN / 2;
  static constexpr int NBM = WMt / 32, NBN = WNt / 32;
  static constexpr int UX = (KC / RU) * (BM / P);  // staging units (RU rows x 16 bytes) of X per chunk
  static constexpr int UY = (KC / RU) * (BN / P);
  static constexpr int UT = UX + UY;
  static constexpr int UPT = (UT + NT - 1) / NT;  // units per thread
  static constexpr int BUF = (BM + BN) * kRowB;
  static constexpr int LDS_BYTES = 2 * BUF;
  static_assert(KC / RU == 8, "eight row groups per chunk");

  typedef f32x16 AccT[NBM][NBN];

  struct Regs {
    uint4 v[UPT][RU];
  };

  // Unit u of an operand -> (row group rr, 16-byte column vector cc). The map
  // makes every 16-lane pass of the transposed LDS stores hit 16 distinct
  // 4-bank groups, and keeps global loads of one row contiguous across lanes.
  __device__ __forceinline__ static void unit_rc(int u, int* rr, int* cc) {
    if constexpr (P == 8) {
      *rr = u & 7;
      *cc = u >> 3;
    } else {
      *rr = (u & 3) + 4 * ((u >> 4) & 1);
      *cc = ((u >> 2) & 3) + 4 * (u >> 5);
    }
  }

  // Load one chunk into registers. x_full/y_full: the whole tile width is
  // inside the matrix and rows are 16-byte aligned (no per-element checks).
  __device__ __forceinline__ static void load(Regs& R, const ChunkSrc<T>& cs, int64_t Kx, int64_t Ky, int64_t m0,
                                              int64_t n0, bool x_full, bool y_full, bool vecx, bool vecy,
                                              int64_t ones_col) {
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int unit = threadIdx.x + u * NT;
      if (unit >= UT) continue;
      const bool isx = unit < UX;
      int rr, cc;
      unit_rc(isx ? unit : unit - UX, &rr, &cc);
      const T* base = isx ? cs.xp : cs.yp;
      const int64_t K = isx ? Kx : Ky;
      const int64_t col = (isx ? m0 : n0) + cc * P;
      const bool full = (isx ? x_full : y_full) && cs.rv == KC;
      if (full) {
        const T* src = base + (int64_t)(rr * RU) * K + col;
#pragma unroll
        for (int r = 0; r < RU; ++r) R.v[u][r] = *reinterpret_cast<const uint4*>(src + (int64_t)r * K);
      } else {
#pragma unroll
        for (int r = 0; r < RU; ++r) {
          const int row = rr * RU + r;
          uint4 v = load16_rowmajor(base, (int64_t)cs.rv, K, (int64_t)row, col, isx ? vecx : vecy);
          if (isx && ones_col >= col && ones_col < col + P && row < cs.rv) {
            const int e = (int)(ones_col - col);
            uint32_t w[4] = {v.x, v.y, v.z, v.w};
            if constexpr (P == 8)
              w[e >> 1] |= 0x3F80u << (16 * (e & 1));
            else
              w[e] = 0x3F800000u;
            v = make_uint4(w[0], w[1], w[2], w[3]);
          }
          R.v[u][r] = v;
        }
      }
    }
  }

  // Transposed stores: feature f = cc*P + m gets the RU k-values of the unit
  // as one 16-byte write at k offset rr*RU. fp32 G rows are scaled by c.
  __device__ __forceinline__ static void store(const Regs& R, unsigned char* buf, const ChunkSrc<T>& cs,
                                               const float* c, int64_t Tn) {
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int unit = threadIdx.x + u * NT;
      if (unit >= UT) continue;
      const bool isx = unit < UX;
      int rr, cc;
      unit_rc(isx ? unit : unit - UX, &rr, &cc);
      unsigned char* dst = buf + ((isx ? 0 : BM) + cc * P) * kRowB + rr * 16;
      if constexpr (P == 4) {
        float sc[4] = {1.0f, 1.0f, 1.0f, 1.0f};
        if (!isx && c != nullptr) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = rr * 4 + r;
            sc[r] = row < cs.rv ? c[(cs.r0 + row) / Tn] : 0.0f;
          }
        }
        const uint4* v = R.v[u];
        *reinterpret_cast<float4*>(dst + 0 * kRowB) = make_float4(__uint_as_float(v[0].x) * sc[0], __uint_as_float(v[1].x) * sc[1], __uint_as_float(v[2].x) * sc[2], __uint_as_float(v[3].x) * sc[3]);
        *reinterpret_cast<float4*>(dst + 1 * kRowB) = make_float4(__uint_as_float(v[0].y) * sc[0], __uint_as_float(v[1].y) * sc[1], __uint_as_float(v[2].y) * sc[2], __uint_as_float(v[3].y) * sc[3]);
        *reinterpret_cast<float4*>(dst + 2 * kRowB) = make_float4(__uint_as_float(v[0].z) * sc[0], __uint_as_float(v[1].z) * sc[1], __uint_as_float(v[2].z) * sc[2], __uint_as_float(v[3].z) * sc[3]);
        *reinterpret_cast<float4*>(dst + 3 * kRowB) = make_float4(__uint_as_float(v[0].w) * sc[0], __uint_as_float(v[1].w) * sc[1], __uint_as_float(v[2].w) * sc[2], __uint_as_float(v[3].w) * sc[3]);
      } else {
        // 8 x 8 bf16 transpose: out[m] packs rows (2kp, 2kp+1) of column m
        const uint4* v = R.v[u];
#pragma unroll
        for (int mp = 0; mp < 4; ++mp) {  // column pair (2mp, 2mp+1) lives in dword mp of every row
          uint32_t w[8];
#pragma unroll
          for (int r = 0; r < 8; ++r) w[r] = mp == 0 ? v[r].x : mp == 1 ? v[r].y : mp == 2 ? v[r].z : v[r].w;
          uint4 even, odd;
          even.x = (w[0] & 0xFFFFu) | (w[1] << 16);
          even.y = (w[2] & 0xFFFFu) | (w[3] << 16);
          even.z = (w[4] & 0xFFFFu) | (w[5] << 16);
          even.w = (w[6] & 0xFFFFu) | (w[7] << 16);
          odd.x = (w[0] >> 16) | (w[1] & 0xFFFF0000u);
          odd.y = (w[2] >> 16) | (w[3] & 0xFFFF0000u);
          odd.z = (w[4] >> 16) | (w[5] & 0xFFFF0000u);
          odd.w = (w[6] >> 16) | (w[7] & 0xFFFF0000u);
          *reinterpret_cast<uint4*>(dst + (2 * mp) * kRowB) = even;
          *reinterpret_cast<uint4*>(dst + (2 * mp + 1) * kRowB) = odd;
        }
      }
    }
  }

  __device__ __forceinline__ static void compute(const unsigned char* buf, AccT& acc) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const unsigned char* xb = buf + (wm * WMt + (lane & 31)) * kRowB + (lane >> 5) * 16;
    const unsigned char* yb = buf + (BM + wn * WNt + (lane & 31)) * kRowB + (lane >> 5) * 16;
    if constexpr (P == 8) {
#pragma unroll
      for (int ks = 0; ks < KC / 16; ++ks) {
        uint4 a[NBM], b[NBN];
#pragma unroll
        for (int bi = 0; bi < NBM; ++bi) a[bi] = *reinterpret_cast<const uint4*>(xb + bi * 32 * kRowB + ks * 32);
#pragma unroll
        for (int bj = 0; bj < NBN; ++bj) b[bj] = *reinterpret_cast<const uint4*>(yb + bj * 32 * kRowB + ks * 32);
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
        for (int bi = 0; bi < NBM; ++bi) a[bi] = *reinterpret_cast<const float4*>(xb + bi * 32 * kRowB + g * 32);
#pragma unroll
        for (int bj = 0; bj < NBN; ++bj) b[bj] = *reinterpret_cast<const float4*>(yb + bj * 32 * kRowB + g * 32);
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
  const bool x_full = vecA && (m0 + BM <= d);
  const bool y_full = vecG && (n0 + BN <= p);
  const int64_t nq = (Tn + E::KC - 1) / E::KC;
  auto src = [&](int64_t q) {
    ChunkSrc<T> cs;
    cs.xp = Xi + q * E::KC * d;
    cs.yp = Yi + q * E::KC * p;
    const int64_t left = Tn - q * E::KC;
    cs.rv = (int)(left < E::KC ? left : E::KC);
    cs.r0 = 0;
    return cs;
  };
  ChunkSrc<T> cs = src(0);
  E::load(R, cs, d, p, m0, n0, x_full, y_full, vecA != 0, vecG != 0, ones_col);
  for (int64_t q = 0; q < nq; ++q) {
    unsigned char* buf = lds + (q & 1) * E::BUF;
    E::store(R, buf, cs, nullptr, Tn);
    __syncthreads();
    if (q + 1 < nq) {
      cs = src(q + 1);
      E::load(R, cs, d, p, m0, n0, x_full, y_full, vecA != 0, vecG != 0, ones_col);
    }
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
  float sc, inv_denom;  // sigma*C and the fp32 reciprocal of denom
  uint32_t k0, k1, layer, step;
};

// Workgroup = (output tile, K split). FUSED (one split): out and bias_out get
// (S + sc*z) * (1/denom) directly. Otherwise ws[split][m][n] (m < d + has_bias).
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
  const bool x_full = vecA && (m0 + BM <= d);
  const bool y_full = vecG && (n0 + BN <= p);
  if constexpr (E::P == 4) {
    // flat K over all B*T rows in chunks of KC rows; G rows scaled by c[row / T]
    const int64_t nrows = B * Tn;
    const int64_t nunits = (nrows + E::KC - 1) / E::KC;
    const int64_t u0 = split * units_per_split;
    const int64_t u1 = u0 + units_per_split < nunits ? u0 + units_per_split : nunits;
    auto src = [&](int64_t u) {
      ChunkSrc<T> cs;
      cs.r0 = u * E::KC;
      cs.xp = A + cs.r0 * d;
      cs.yp = G + cs.r0 * p;
      const int64_t left = nrows - cs.r0;
      cs.rv = (int)(left < E::KC ? left : E::KC);
      return cs;
    };
    ChunkSrc<T> cs = src(u0);
    if (u0 < u1) E::load(R, cs, d, p, m0, n0, x_full, y_full, vecA != 0, vecG != 0, ones_col);
    for (int64_t u = u0; u < u1; ++u) {
      unsigned char* buf = lds + ((u - u0) & 1) * E::BUF;
      E::store(R, buf, cs, c, Tn);
      __syncthreads();
      if (u + 1 < u1) {
        cs = src(u + 1);
        E::load(R, cs, d, p, m0, n0, x_full, y_full, vecA != 0, vecG != 0, ones_col);
      }
      E::compute(buf, acc);
    }
  } else {
    // per-sample exact accumulation: acc += c_i * (A_i^T G_i tile)
    const int64_t i0 = split * units_per_split;
    const int64_t i1 = i0 + units_per_split < B ? i0 + units_per_split : B;
    const int cps = (int)((Tn + E::KC - 1) / E::KC);  // chunks per sample
    typename E::AccT tmp;
    E::zero(tmp);
    auto src = [&](int64_t i, int ch) {
      ChunkSrc<T> cs;
      const int64_t row = i * Tn + (int64_t)ch * E::KC;
      cs.xp = A + row * d;
      cs.yp = G + row * p;
      const int64_t left = Tn - (int64_t)ch * E::KC;
      cs.rv = (int)(left < E::KC ? left : E::KC);
      cs.r0 = row;
      return cs;
    };
    int64_t i = i0;
    int ch = 0;
    ChunkSrc<T> cs = src(i, ch);
    if (i0 < i1) E::load(R, cs, d, p, m0, n0, x_full, y_full, vecA != 0, vecG != 0, ones_col);
    int64_t q = 0;
    while (i < i1) {
      unsigned char* buf = lds + (q & 1) * E::BUF;
      E::store(R, buf, cs, nullptr, Tn);
      __syncthreads();
      const bool last = (ch == cps - 1);
      const int64_t in = last ? i + 1 : i;
      const int chn = last ? 0 : ch + 1;
      if (in < i1) {
        cs = src(in, chn);
        E::load(R, cs, d, p, m0, n0, x_full, y_full, vecA != 0, vecG != 0, ones_col);
      }
      E::compute(buf, tmp);
      if (last) {
        const float ci = c[i];
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
      i = in;
      ch = chn;
      ++q;
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
              if (mb + r < d) out[(mb + r) * p + n] = noised_mean_spec(acc[bi][bj][4 * j4 + r], na.sc, z[r], na.inv_denom);
          }
          if (has_bias && d >= mb && d < mb + 4) {
            const f32x4 zb = normals4((uint32_t)(n >> 2), 2u * na.layer + 1u, na.step, 0u, na.k0, na.k1);
            const int r = (int)(d - mb);
            bias_out[n] = noised_mean_spec(acc[bi][bj][4 * j4 + r], na.sc, zb[(int)(n & 3)], na.inv_denom);
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
        if (m < d) s[r][k] = noised_mean_spec(s[r][k], na.sc, z[r], na.inv_denom);
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
      bias_out[n] = noised_mean_spec(s, na.sc, z[k], na.inv_denom);
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
  na.inv_denom = 1.0f / denom;
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
