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
#include "dp_reduce.hpp"

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
  int64_t r0;    // flat row index of chunk row 0 (for the clip factor)
  int64_t xrow;  // row of the unfolded input (b*T + t) of chunk row 0, for X = U(a) formed from a folded input
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
    u32x4 v[UPT][RU];
    float sc[UPT][RU];  // fp32: clip factor of each staged G row (loaded with the rows)
  };

  // Index of the sample that flat row `row` belongs to (T rows per sample).
  __device__ __forceinline__ static int64_t sample_of(int64_t row, int64_t Tn) {
    if (Tn == 1) return row;
    if ((uint64_t)row <= 0xFFFFFFFFull && (uint64_t)Tn <= 0xFFFFFFFFull)
      return (int64_t)((uint32_t)row / (uint32_t)Tn);
    return row / Tn;
  }

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

  // Load one chunk into registers. FULL: every chunk row is valid, the whole
  // tile width is inside both matrices and rows are 16-byte aligned, so the
  // loads need no checks (and the compiled loop has no per-element fallback).
  // IM2COL: X is the unfolded input of the convolution `geo`, its rows formed
  // element by element from the folded input.
  template <bool FULL, bool IM2COL = false>
  __device__ __forceinline__ static void load(Regs& R, const ChunkSrc<T>& cs, int64_t Kx, int64_t Ky, int64_t m0,
                                              int64_t n0, bool vecx, bool vecy, int64_t ones_col,
                                              const float* c = nullptr, int64_t Tn = 1,
                                              const ConvGeo* geo = nullptr) {
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int unit = threadIdx.x + u * NT;
      if (UT % NT != 0 && unit >= UT) continue;
      const bool isx = unit < UX;
      int rr, cc;
      unit_rc(isx ? unit : unit - UX, &rr, &cc);
      if constexpr (P == 4) {
        if (!isx && c != nullptr) {
#pragma unroll
          for (int r = 0; r < RU; ++r) {
            const int row = rr * RU + r;
            R.sc[u][r] = row < cs.rv ? c[sample_of(cs.r0 + row, Tn)] : 0.0f;
          }
        }
      }
      const T* base = isx ? cs.xp : cs.yp;
      const int64_t K = isx ? Kx : Ky;
      const int64_t col = (isx ? m0 : n0) + cc * P;
      if constexpr (IM2COL) {
        static_assert(!FULL, "unfolded rows are formed with checks");
        if (isx) {
          // the unit's RU consecutive rows: one division for the first, then steps
          const ConvCols<P> kc = conv_cols<P>(*geo, col, ones_col);
          ConvRow rw = conv_row_flat(*geo, cs.xrow + rr * RU);
#pragma unroll
          for (int r = 0; r < RU; ++r) {
            R.v[u][r] = conv_row16<T>(*geo, rw, kc, rr * RU + r < cs.rv);
            rw.next(*geo);
          }
          continue;
        }
      }
      if constexpr (FULL) {
        const T* src = base + (int64_t)(rr * RU) * K + col;
#pragma unroll
        for (int r = 0; r < RU; ++r) R.v[u][r] = *reinterpret_cast<const u32x4*>(src + (int64_t)r * K);
      } else {
#pragma unroll
        for (int r = 0; r < RU; ++r) {
          const int row = rr * RU + r;
          u32x4 v = load16_rowmajor(base, (int64_t)cs.rv, K, (int64_t)row, col, isx ? vecx : vecy);
          if (isx && ones_col >= col && ones_col < col + P && row < cs.rv) {
            const int e = (int)(ones_col - col);
            if constexpr (P == 8)
              v[e >> 1] |= 0x3F80u << (16 * (e & 1));
            else
              v[e] = 0x3F800000u;
          }
          R.v[u][r] = v;
        }
      }
    }
  }

  // Per-thread byte-free element offsets of its staging units inside a chunk
  // (row group rr, column vector cc), for the unchecked loads of kloop_full.
  struct Offs {
    int64_t off[UPT];
    bool isx[UPT];
    int row[UPT];  // first chunk row of the unit
  };
  __device__ __forceinline__ static void full_offsets(Offs& O, int64_t Kx, int64_t Ky, int64_t m0, int64_t n0) {
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int unit = threadIdx.x + u * NT;
      const bool isx = unit < UX;
      int rr, cc;
      unit_rc(isx ? unit : unit - UX, &rr, &cc);
      O.isx[u] = isx;
      O.row[u] = rr * RU;
      O.off[u] = isx ? (int64_t)(rr * RU) * Kx + m0 + cc * P : (int64_t)(rr * RU) * Ky + n0 + cc * P;
    }
  }
  // Unchecked loads of chunk q: rows [q*KC, q*KC + KC) of X = A and Y = G.
  __device__ __forceinline__ static void load_full(Regs& R, const Offs& O, const T* A, const T* G, int64_t Kx,
                                                   int64_t Ky, int64_t q, const float* c = nullptr,
                                                   int64_t Tn = 1) {
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      if (UT % NT != 0 && threadIdx.x + u * NT >= UT) continue;
      if constexpr (P == 4) {
        if (!O.isx[u] && c != nullptr) {
#pragma unroll
          for (int r = 0; r < RU; ++r) R.sc[u][r] = c[sample_of(q * (int64_t)KC + O.row[u] + r, Tn)];
        }
      }
      const int64_t K = O.isx[u] ? Kx : Ky;
      const T* src = (O.isx[u] ? A : G) + q * (int64_t)KC * K + O.off[u];
#pragma unroll
      for (int r = 0; r < RU; ++r) R.v[u][r] = *reinterpret_cast<const u32x4*>(src + (int64_t)r * K);
    }
  }

  // Transposed stores: feature f = cc*P + m gets the RU k-values of the unit
  // as one 16-byte write at k offset rr*RU. fp32 G rows are scaled by c (the
  // factors were loaded with the rows; `scaled` says whether they were).
  __device__ __forceinline__ static void store(const Regs& R, unsigned char* buf, bool scaled) {
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int unit = threadIdx.x + u * NT;
      if (UT % NT != 0 && unit >= UT) continue;
      const bool isx = unit < UX;
      int rr, cc;
      unit_rc(isx ? unit : unit - UX, &rr, &cc);
      unsigned char* dst = buf + ((isx ? 0 : BM) + cc * P) * kRowB + rr * 16;
      if constexpr (P == 4) {
        float sc[4] = {1.0f, 1.0f, 1.0f, 1.0f};
        if (!isx && scaled) {
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[r] = R.sc[u][r];
        }
        const u32x4* v = R.v[u];
        *reinterpret_cast<float4*>(dst + 0 * kRowB) = make_float4(__uint_as_float(v[0].x) * sc[0], __uint_as_float(v[1].x) * sc[1], __uint_as_float(v[2].x) * sc[2], __uint_as_float(v[3].x) * sc[3]);
        *reinterpret_cast<float4*>(dst + 1 * kRowB) = make_float4(__uint_as_float(v[0].y) * sc[0], __uint_as_float(v[1].y) * sc[1], __uint_as_float(v[2].y) * sc[2], __uint_as_float(v[3].y) * sc[3]);
        *reinterpret_cast<float4*>(dst + 2 * kRowB) = make_float4(__uint_as_float(v[0].z) * sc[0], __uint_as_float(v[1].z) * sc[1], __uint_as_float(v[2].z) * sc[2], __uint_as_float(v[3].z) * sc[3]);
        *reinterpret_cast<float4*>(dst + 3 * kRowB) = make_float4(__uint_as_float(v[0].w) * sc[0], __uint_as_float(v[1].w) * sc[1], __uint_as_float(v[2].w) * sc[2], __uint_as_float(v[3].w) * sc[3]);
      } else {
        // 8 x 8 bf16 transpose: out[m] packs rows (2kp, 2kp+1) of column m
        const u32x4* v = R.v[u];
#pragma unroll
        for (int mp = 0; mp < 4; ++mp) {  // column pair (2mp, 2mp+1) lives in dword mp of every row
          uint32_t w[8];
#pragma unroll
          for (int r = 0; r < 8; ++r) w[r] = v[r][mp];
          // byte permutes: even = low halves of rows (2kp, 2kp+1), odd = high halves
          u32x4 even, odd;
          even[0] = __builtin_amdgcn_perm(w[1], w[0], 0x05040100u);
          even[1] = __builtin_amdgcn_perm(w[3], w[2], 0x05040100u);
          even[2] = __builtin_amdgcn_perm(w[5], w[4], 0x05040100u);
          even[3] = __builtin_amdgcn_perm(w[7], w[6], 0x05040100u);
          odd[0] = __builtin_amdgcn_perm(w[1], w[0], 0x07060302u);
          odd[1] = __builtin_amdgcn_perm(w[3], w[2], 0x07060302u);
          odd[2] = __builtin_amdgcn_perm(w[5], w[4], 0x07060302u);
          odd[3] = __builtin_amdgcn_perm(w[7], w[6], 0x07060302u);
          *reinterpret_cast<u32x4*>(dst + (2 * mp) * kRowB) = even;
          *reinterpret_cast<u32x4*>(dst + (2 * mp + 1) * kRowB) = odd;
        }
      }
    }
  }

  // acc += X^T Y of the chunk in buf. FRESH: acc is overwritten (the first
  // MFMA of each block starts from zero instead of acc).
  template <bool FRESH = false>
  __device__ __forceinline__ static void compute(const unsigned char* buf, AccT& acc) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const unsigned char* xb = buf + (wm * WMt + (lane & 31)) * kRowB + (lane >> 5) * 16;
    const unsigned char* yb = buf + (BM + wn * WNt + (lane & 31)) * kRowB + (lane >> 5) * 16;
    if constexpr (P == 8) {
#pragma unroll
      for (int ks = 0; ks < KC / 16; ++ks) {
        u32x4 a[NBM], b[NBN];
#pragma unroll
        for (int bi = 0; bi < NBM; ++bi) a[bi] = *reinterpret_cast<const u32x4*>(xb + bi * 32 * kRowB + ks * 32);
#pragma unroll
        for (int bj = 0; bj < NBN; ++bj) b[bj] = *reinterpret_cast<const u32x4*>(yb + bj * 32 * kRowB + ks * 32);
#pragma unroll
        for (int bi = 0; bi < NBM; ++bi)
#pragma unroll
          for (int bj = 0; bj < NBN; ++bj) {
            if (FRESH && ks == 0) {
              const f32x16 zero = {};
              acc[bi][bj] = mfma32_bf16(a[bi], b[bj], zero);
            } else {
              acc[bi][bj] = mfma32_bf16(a[bi], b[bj], acc[bi][bj]);
            }
          }
      }
    } else {
      static_assert(!FRESH, "fp32 path accumulates directly");
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

// ---------------------------------------------------------------- K loops
// Software pipeline with prefetch distance 2: chunk q is stored from register
// stage q&1 into LDS buffer q&1, then (after one barrier) the global loads of
// chunk q+2 are issued into the freed register stage while the MFMAs of chunk
// q run; the loads of chunk q+1 are in flight too. One barrier per chunk
// suffices with two LDS buffers: a wave reaching the store of chunk q+1 has
// passed the barrier of chunk q, so every wave has finished chunk q-1.
//
// Desc(q) returns the ChunkSrc of chunk q; Epi(q, acc-kind) is called after
// the MFMAs of chunk q (per-sample scaling for bf16).
template <typename T, int BM, int BN, bool FULL, bool PER_SAMPLE, bool IM2COL, typename Desc>
__device__ __forceinline__ void kloop(typename Xty<T, BM, BN>::AccT& acc, unsigned char* lds, int64_t nq, Desc desc,
                                      int cps, const float* cs_sample, int64_t d, int64_t p, int64_t m0, int64_t n0,
                                      bool vecA, bool vecG, int64_t ones_col, const float* c_rows, int64_t Tn,
                                      const ConvGeo* geo = nullptr) {
  using E = Xty<T, BM, BN>;
  if (nq <= 0) return;
  typename E::Regs R[2];
  ChunkSrc<T> cs[2];
  cs[0] = desc(0);
  E::template load<FULL, IM2COL>(R[0], cs[0], d, p, m0, n0, vecA, vecG, ones_col, c_rows, Tn, geo);
  if (nq > 1) {
    cs[1] = desc(1);
    E::template load<FULL, IM2COL>(R[1], cs[1], d, p, m0, n0, vecA, vecG, ones_col, c_rows, Tn, geo);
  }
  typename E::AccT tmp;
  if constexpr (!PER_SAMPLE) (void)tmp;
  for (int64_t q0 = 0; q0 < nq; q0 += 2) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int64_t q = q0 + st;
      if (q < nq) {
        unsigned char* buf = lds + st * E::BUF;
        E::store(R[st], buf, c_rows != nullptr);
        __syncthreads();
        if (q + 2 < nq) {
          cs[st] = desc(q + 2);
          E::template load<FULL, IM2COL>(R[st], cs[st], d, p, m0, n0, vecA, vecG, ones_col, c_rows, Tn, geo);
        }
        if constexpr (PER_SAMPLE) {
          const int ch = (int)(q % cps);
          if (ch == 0)
            E::template compute<true>(buf, tmp);
          else
            E::template compute<false>(buf, tmp);
          if (ch == cps - 1) {
            const float ci = cs_sample[q / cps];
#pragma unroll
            for (int bi = 0; bi < E::NBM; ++bi)
#pragma unroll
              for (int bj = 0; bj < E::NBN; ++bj)
#pragma unroll
                for (int j = 0; j < 16; ++j) acc[bi][bj][j] += ci * tmp[bi][bj][j];
          }
        } else {
          E::template compute<false>(buf, acc);
        }
      }
    }
  }
}

// Pipeline for the common case: every chunk is KC full rows of the flattened
// [B*T] row space and the whole tile is inside both matrices, so chunk q is
// simply rows [q*KC, q*KC + KC) and the loads need no checks. Two named
// register stages keep the loads of chunks q+1 and q+2 in flight; the loads
// of the last two iterations re-read the final chunk (clamped index) so the
// loop body stays straight-line. PER_SAMPLE (bf16, T % KC == 0): chunks never
// straddle samples; each sample's chunks go to tmp, then acc += c_i * tmp.
// fp32: G rows are scaled by c[row / T] while staging.
template <typename T, int BM, int BN, bool PER_SAMPLE>
__device__ __forceinline__ void kloop_full(typename Xty<T, BM, BN>::AccT& acc, unsigned char* lds, const T* A,
                                           const T* G, const float* c, int64_t q0, int64_t nq, int64_t Tn,
                                           int64_t d, int64_t p, int64_t m0, int64_t n0) {
  using E = Xty<T, BM, BN>;
  if (nq <= 0) return;
  typename E::Offs O;
  E::full_offsets(O, d, p, m0, n0);
  const int64_t qlast = q0 + nq - 1;
  typename E::Regs R0, R1;
  const float* c_rows = PER_SAMPLE ? nullptr : c;  // fp32: G rows scaled while staging
  E::load_full(R0, O, A, G, d, p, q0, c_rows, Tn);
  E::load_full(R1, O, A, G, d, p, q0 + 1 <= qlast ? q0 + 1 : qlast, c_rows, Tn);
  typename E::AccT tmp;
  const int cps = (int)(Tn / E::KC);             // chunks per sample (PER_SAMPLE)
  int ch = PER_SAMPLE ? (int)(q0 % cps) : 0;     // chunk index inside its sample
  int64_t sample = PER_SAMPLE ? q0 / cps : 0;
  unsigned char* buf0 = lds;
  unsigned char* buf1 = lds + E::BUF;

  auto run = [&](typename E::Regs& R, unsigned char* buf, int64_t q) {
    E::store(R, buf, c_rows != nullptr);
    __syncthreads();
    const int64_t qn = q + 2 <= qlast ? q + 2 : qlast;
    E::load_full(R, O, A, G, d, p, qn, c_rows, Tn);
    if constexpr (PER_SAMPLE) {
      if (ch == 0)
        E::template compute<true>(buf, tmp);
      else
        E::template compute<false>(buf, tmp);
      if (ch == cps - 1) {
        const float ci = c[sample];
#pragma unroll
        for (int bi = 0; bi < E::NBM; ++bi)
#pragma unroll
          for (int bj = 0; bj < E::NBN; ++bj)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[bi][bj][j] += ci * tmp[bi][bj][j];
        ch = 0;
        ++sample;
      } else {
        ++ch;
      }
    } else {
      E::template compute<false>(buf, acc);
    }
  };

  int64_t q = q0;
  for (; q + 1 <= qlast; q += 2) {
    run(R0, buf0, q);
    run(R1, buf1, q + 1);
  }
  if (q == qlast) run(R0, buf0, q);
}

// Chunk q of a row range [q*KC, ...) of nrows rows starting at X/Y.
template <typename T, int KC>
struct RowDesc {
  const T* X;
  const T* Y;
  int64_t nrows, d, p, q_base;
  int64_t xrow_base;  // unfolded-input row of row 0 of X
  __device__ __forceinline__ ChunkSrc<T> operator()(int64_t q) const {
    ChunkSrc<T> cs;
    cs.r0 = (q + q_base) * KC;
    cs.xp = X + cs.r0 * d;
    cs.yp = Y + cs.r0 * p;
    cs.xrow = xrow_base + cs.r0;
    const int64_t left = nrows - cs.r0;
    cs.rv = (int)(left < KC ? left : KC);
    return cs;
  }
};

// Chunk q of samples i0.. : sample i0 + q / cps, chunk q % cps of that sample.
template <typename T, int KC>
struct SampleDesc {
  const T* A;
  const T* G;
  int64_t Tn, d, p, i0;
  int cps;
  __device__ __forceinline__ ChunkSrc<T> operator()(int64_t q) const {
    ChunkSrc<T> cs;
    const int64_t i = i0 + q / cps;
    const int ch = (int)(q % cps);
    const int64_t row = i * Tn + (int64_t)ch * KC;
    cs.xp = A + row * d;
    cs.yp = G + row * p;
    const int64_t left = Tn - (int64_t)ch * KC;
    cs.rv = (int)(left < KC ? left : KC);
    cs.r0 = row;
    cs.xrow = row;
    return cs;
  }
};

// ---------------------------------------------------------------- explicit
// IM2COL: A is unused and the rows of the unfolded input of `geo` are formed
// from its folded input.
template <typename T, int BM, int BN, bool IM2COL>
__global__ __launch_bounds__(256, 2) void k_explicit_tiles(const T* __restrict__ A, const T* __restrict__ G,
                                                           int64_t B, int64_t Tn, int64_t d, int64_t p, int has_bias,
                                                           int mt, int nt, int vecA, int vecG, NormSink sink,
                                                           ConvGeo geo) {
  using E = Xty<T, BM, BN>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[E::LDS_BYTES];
  __shared__ float red[E::NT / kWave];
  const int ntl = mt * nt;
  int64_t i, tile;
  xcd_group_map(blockIdx.x, ntl, &i, &tile);
  if (i >= B) return;
  const int64_t m0 = (tile / nt) * BM;
  const int64_t n0 = (tile % nt) * BN;
  const int64_t ones_col = has_bias ? d : -1;
  const bool full = !IM2COL && vecA && vecG && (m0 + BM <= d) && (n0 + BN <= p) && (Tn % E::KC == 0);
  const int64_t nq = (Tn + E::KC - 1) / E::KC;
  typename E::AccT acc;
  E::zero(acc);
  const RowDesc<T, E::KC> desc{IM2COL ? A : A + i * Tn * d, G + i * Tn * p, Tn, d, p, 0, i * Tn};
  if (full)
    kloop_full<T, BM, BN, false>(acc, lds, A + i * Tn * d, G + i * Tn * p, nullptr, 0, nq, Tn, d, p, m0, n0);
  else
    kloop<T, BM, BN, false, false, IM2COL>(acc, lds, nq, desc, 1, nullptr, d, p, m0, n0, vecA != 0, vecG != 0,
                                           ones_col, nullptr, Tn, &geo);
  float s = 0.f;
#pragma unroll
  for (int bi = 0; bi < E::NBM; ++bi)
#pragma unroll
    for (int bj = 0; bj < E::NBN; ++bj)
#pragma unroll
      for (int j = 0; j < 16; ++j) s += acc[bi][bj][j] * acc[bi][bj][j];
  s = block_sum<E::NT>(s, red);
  if (threadIdx.x == 0) norm_sink_tile(sink, i, tile, s);
}

// ---------------------------------------------------------------- contraction
// Workgroups per CU the register budget is sized for: the bf16 128x128 tile
// carries a second accumulator set (per-sample exact scaling), so it runs one
// workgroup per CU with the full register file; the others run two.
template <typename T, int BM, int BN>
struct ContractOcc {
  static constexpr int value = (elem_traits<T>::per16 == 8 && BM == 128 && BN == 128) ? 1 : 2;
};

// Workgroup = (output tile, K split). FUSED (one split): out and bias_out get
// (S + sc*z) * (1/denom) directly. Otherwise ws[split][m][n] (m < d + has_bias).
// IM2COL: A is the folded input of `geo`, whose unfolded rows are formed on chip.
template <typename T, int BM, int BN, bool FUSED, bool IM2COL>
__global__ __launch_bounds__(256, (ContractOcc<T, BM, BN>::value)) void k_contract_tiles(const T* __restrict__ A, const T* __restrict__ G,
                                                           const float* __restrict__ c, int64_t B, int64_t Tn,
                                                           int64_t d, int64_t p, int has_bias, int mt, int nt,
                                                           int64_t units_per_split, int64_t nitems, int vecA,
                                                           int vecG, float* __restrict__ ws, NoiseArgs na,
                                                           float* __restrict__ out, float* __restrict__ bias_out,
                                                           ConvGeo geo) {
  using E = Xty<T, BM, BN>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[E::LDS_BYTES];
  // Work items (split, column block, row block), row block fastest; XCD x
  // (blockIdx % 8) takes the contiguous items [x * per, (x + 1) * per), so the
  // row blocks that read one slice of G (one column block and split) run
  // together on one XCD and share that slice in its L2. The grid is a
  // multiple of 8; surplus workgroups return before any barrier.
  const int64_t per = gridDim.x / 8;
  const int64_t item = (int64_t)(blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (item >= nitems) return;
  const int ntl = mt * nt;
  const int64_t split = item / ntl;
  const int tile = (int)(item - split * ntl);
  const int64_t m0 = (tile % mt) * BM;
  const int64_t n0 = (tile / mt) * BN;
  const int64_t ones_col = has_bias ? d : -1;
  const int64_t mrows = d + (has_bias ? 1 : 0);
  const bool wide = !IM2COL && vecA && vecG && (m0 + BM <= d) && (n0 + BN <= p);

  typename E::AccT acc;
  E::zero(acc);
  if constexpr (E::P == 4) {
    // flat K over all B*T rows in chunks of KC rows; G rows scaled by c[row / T]
    const int64_t nrows = B * Tn;
    const int64_t nunits = (nrows + E::KC - 1) / E::KC;
    const int64_t u0 = split * units_per_split;
    const int64_t u1 = u0 + units_per_split < nunits ? u0 + units_per_split : nunits;
    const RowDesc<T, E::KC> desc{A, G, nrows, d, p, u0, 0};
    const int64_t nq = u1 > u0 ? u1 - u0 : 0;
    if (wide && (u1 < nunits || nrows % E::KC == 0))
      kloop_full<T, BM, BN, false>(acc, lds, A, G, c, u0, nq, Tn, d, p, m0, n0);
    else
      kloop<T, BM, BN, false, false, IM2COL>(acc, lds, nq, desc, 1, nullptr, d, p, m0, n0, vecA != 0, vecG != 0,
                                             ones_col, c, Tn, &geo);
  } else {
    const int64_t i0 = split * units_per_split;
    const int64_t i1 = i0 + units_per_split < B ? i0 + units_per_split : B;
    const int cps = (int)((Tn + E::KC - 1) / E::KC);
    const SampleDesc<T, E::KC> desc{A, G, Tn, d, p, i0, cps};
    const int64_t nq = i1 > i0 ? (i1 - i0) * cps : 0;
    if (wide && Tn % E::KC == 0)
      kloop_full<T, BM, BN, true>(acc, lds, A, G, c, i0 * cps, nq, Tn, d, p, m0, n0);
    else
      kloop<T, BM, BN, false, true, IM2COL>(acc, lds, nq, desc, cps, c + i0, d, p, m0, n0, vecA != 0, vecG != 0,
                                            ones_col, nullptr, Tn, &geo);
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

// One thread per 4 x 4 output block (reduce_noise_block4), then one per 4
// bias columns.
__global__ __launch_bounds__(256) void k_reduce_noise_vec(const float* __restrict__ ws, int64_t ks, int64_t d,
                                                          int64_t p, int has_bias, NoiseArgs na,
                                                          float* __restrict__ out, float* __restrict__ bias_out) {
  const int64_t nq = d / 4, nc = p / 4;
  const int64_t nw = nq * nc;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t split_stride = (d + (has_bias ? 1 : 0)) * p;
  if (t < nw) {
    reduce_noise_block4(ws, ks, p, split_stride, t / nc, t % nc, na, out);
  } else if (has_bias && t < nw + nc) {
    const int64_t cq = t - nw;
    const float* base = ws + d * p + 4 * cq;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int64_t sp = 0; sp < ks; ++sp) {
      const float4 v = *reinterpret_cast<const float4*>(base + sp * split_stride);
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    const f32x4 z = normals4((uint32_t)cq, 2u * na.layer + 1u, na.step, 0u, na.k0, na.k1);
    bias_out[4 * cq + 0] = noised_mean_spec(s.x, na.sc, z[0], na.inv_denom);
    bias_out[4 * cq + 1] = noised_mean_spec(s.y, na.sc, z[1], na.inv_denom);
    bias_out[4 * cq + 2] = noised_mean_spec(s.z, na.sc, z[2], na.inv_denom);
    bias_out[4 * cq + 3] = noised_mean_spec(s.w, na.sc, z[3], na.inv_denom);
  }
}

// The split reduces of several layers in one launch: each layer owns a
// contiguous range of workgroups, one thread per 4 x 4 output block, with the
// arithmetic of k_reduce_noise_vec (no bias rows).
template <bool ACC>
__global__ __launch_bounds__(256) void k_reduce_noise_group(RedGroup g) {
  int k = 0;
#pragma unroll
  for (int j = 1; j < kDlGroupMax; ++j)
    if (j < g.n && (int64_t)blockIdx.x >= g.blk_begin[j]) k = j;
  const SplitReduceLayer L = g.L[k];
  const int64_t nc = L.p / 4, nw = (L.d / 4) * nc;
  const int64_t t = ((int64_t)blockIdx.x - g.blk_begin[k]) * blockDim.x + threadIdx.x;
  if (t >= nw) return;
  reduce_noise_block4<ACC>(L.ws, L.ks, L.p, L.d * L.p, t / nc, t % nc, L.na, ACC ? L.acc : L.out);
}

// Many splits, small output. A workgroup takes a block of 4 weight rows x 16
// columns: thread (lane sl = t / 16, element e = t % 16 = row r x column
// quad) sums the float4 partials of splits sl, sl + 16, ... in split order;
// the 16 lane sums are then added in lane order through LDS and each of 16
// threads takes one column (4 rows = one Philox block) and writes the noised
// mean. Blocks past the weight rows do the bias row, 64 columns each.
// Requires p % 4 == 0 and 16-byte aligned ws (float4 partial rows).
__global__ __launch_bounds__(256) void k_reduce_noise_wide(const float* __restrict__ ws, int64_t ks, int64_t d,
                                                           int64_t p, int has_bias, NoiseArgs na,
                                                           float* __restrict__ out, float* __restrict__ bias_out) {
  __shared__ float4 part[16][16];
  const int64_t split_stride = (d + (has_bias ? 1 : 0)) * p;
  const int64_t nq = (d + 3) / 4, nc16 = (p + 15) / 16;
  const int64_t nwb = nq * nc16;
  const int t = threadIdx.x, sl = t >> 4, e = t & 15;
  const bool bias_blk = (int64_t)blockIdx.x >= nwb;
  int64_t m, cq;  // row and column quad this thread sums
  bool valid;
  if (!bias_blk) {
    const int64_t q = blockIdx.x / nc16, c16 = blockIdx.x % nc16;
    m = 4 * q + (e >> 2);
    cq = 4 * c16 + (e & 3);
    valid = m < d && 4 * cq < p;
  } else {
    m = d;
    cq = 16 * ((int64_t)blockIdx.x - nwb) + e;
    valid = 4 * cq < p;
  }
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  if (valid) {
    const float* base = ws + m * p + 4 * cq;
    int64_t sp = sl;
    for (; sp + 48 < ks; sp += 64) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const float4*>(base + (sp + 16 * u) * split_stride);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        s.x += v[u].x;
        s.y += v[u].y;
        s.z += v[u].z;
        s.w += v[u].w;
      }
    }
    for (; sp < ks; sp += 16) {
      const float4 v = *reinterpret_cast<const float4*>(base + sp * split_stride);
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
  }
  part[sl][e] = s;
  __syncthreads();
  if (t >= 16) return;
  if (!bias_blk) {
    // thread t: column 4 * (4 * c16 + t / 4) + t % 4 of rows 4q .. 4q+3
    const int64_t q = blockIdx.x / nc16, c16 = blockIdx.x % nc16;
    const int qi = t >> 2, comp = t & 3;
    const int64_t n = 4 * (4 * c16 + qi) + comp;
    if (n >= p) return;
    float r4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float acc = 0.f;
      for (int l = 0; l < 16; ++l) {
        const float4 v = part[l][4 * r + qi];
        acc += comp == 0 ? v.x : comp == 1 ? v.y : comp == 2 ? v.z : v.w;
      }
      r4[r] = acc;
    }
    const f32x4 z = normals4((uint32_t)(q * p + n), 2u * na.layer, na.step, 0u, na.k0, na.k1);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * q + r < d) out[(4 * q + r) * p + n] = noised_mean_spec(r4[r], na.sc, z[r], na.inv_denom);
  } else {
    const int64_t cqb = 16 * ((int64_t)blockIdx.x - nwb) + t;
    if (4 * cqb >= p) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int l = 0; l < 16; ++l) {
      const float4 v = part[l][t];
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    const f32x4 z = normals4((uint32_t)cqb, 2u * na.layer + 1u, na.step, 0u, na.k0, na.k1);
    bias_out[4 * cqb + 0] = noised_mean_spec(acc.x, na.sc, z[0], na.inv_denom);
    bias_out[4 * cqb + 1] = noised_mean_spec(acc.y, na.sc, z[1], na.inv_denom);
    bias_out[4 * cqb + 2] = noised_mean_spec(acc.z, na.sc, z[2], na.inv_denom);
    bias_out[4 * cqb + 3] = noised_mean_spec(acc.w, na.sc, z[3], na.inv_denom);
  }
}

// ---------------------------------------------------------------- plans
static int pick_tile(int64_t n) {
  // 64 or 128, whichever pads n less (ties -> 128)
  const int64_t p64 = (n + 63) / 64 * 64, p128 = (n + 127) / 128 * 128;
  return p64 < p128 ? 64 : 128;
}

ContractPlan contract_plan(int dtype, int64_t B, int64_t Tn, int64_t d, int64_t p, int has_bias) {
  if (dl_eligible(dtype, B, Tn, d, p, has_bias)) return dl_plan(B, Tn, d, p);
  if (dl32_eligible(dtype, B, Tn, d, p, has_bias)) return dl32_plan(B, Tn, d, p, has_bias);
  return tiles_plan(dtype, B, Tn, d, p, has_bias, false);
}

ContractPlan tiles_plan(int dtype, int64_t B, int64_t Tn, int64_t d, int64_t p, int has_bias, bool folded) {
  ContractPlan pl;
  pl.engine = 0;
  const int64_t mrows = d + (has_bias ? 1 : 0);
  // folded conv inputs with p >= 128: 128-row tiles, so that each gathered
  // input element feeds 128 x 128 outputs (measured faster despite the padding)
  pl.bm = folded && p >= 128 && mrows >= 128 ? 128 : pick_tile(mrows);
  pl.bn = pick_tile(p);
  pl.mt = (int)((mrows + pl.bm - 1) / pl.bm);
  pl.nt = (int)((p + pl.bn - 1) / pl.bn);
  const bool bf16 = dtype == 1;
  const int64_t kc = bf16 ? XtyCfg<bf16s>::KC : XtyCfg<float>::KC;
  // K units: whole samples (bf16, exact per-sample scaling) or KC-row chunks (fp32)
  const int64_t units = bf16 ? B : (B * Tn + kc - 1) / kc;
  const double rows_per_unit = bf16 ? (double)((Tn + kc - 1) / kc * kc) : (double)kc;
  const int64_t ntl = (int64_t)pl.mt * pl.nt;
  const int occ = (bf16 && pl.bm == 128 && pl.bn == 128) ? 1 : 2;
  const int64_t slots = 256 * (int64_t)occ;  // 256 CUs
  // cost model (seconds): MFMA rounds x per-split work on one CU, plus the
  // split-K partial traffic (write + read of ks tiles) and a reduce launch
  const double cu_rate = bf16 ? 4.0e12 : 0.27e12;  // sustained flop/s per CU at ~50% of peak
  const double tile_unit_flops = 2.0 * pl.bm * pl.bn * rows_per_unit;
  double best = 1e300;
  int64_t best_ks = 1;
  const int64_t ks_max = units < 1024 ? units : 1024;
  for (int64_t ks = 1; ks <= ks_max; ++ks) {
    const int64_t ups = (units + ks - 1) / ks;
    const int64_t ks_eff = (units + ups - 1) / ups;
    if (ks_eff != ks) continue;
    const int64_t wgs = ntl * ks;
    const double rounds = (double)((wgs + slots - 1) / slots);
    const double t_mfma = rounds * (double)ups * tile_unit_flops / (cu_rate / occ);
    const double t_red = ks > 1 ? (2.0 * ks + 1.0) * (double)mrows * (double)p * 4.0 / 5.0e12 + 4.0e-6 : 0.0;
    const double t = t_mfma + t_red;
    if (t < best * 0.999) {
      best = t;
      best_ks = ks;
    }
  }
  pl.units_per_split = (units + best_ks - 1) / best_ks;
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
// geo != nullptr: a convolution layer, A is its folded input (the IM2COL
// kernels); otherwise A is [B, T, d].
template <typename T, int BM, int BN>
static hipError_t launch_explicit_t(hipStream_t st, const void* A, const void* G, int64_t B, int64_t Tn, int64_t d,
                                    int64_t p, int has_bias, const ExplicitPlan& pl, const NormSink& sink,
                                    const ConvGeo* geo) {
  const int eb = elem_traits<T>::bytes;
  const int vecA = ((reinterpret_cast<uintptr_t>(A) & 15) == 0) && ((d * eb) % 16 == 0);
  const int vecG = ((reinterpret_cast<uintptr_t>(G) & 15) == 0) && ((p * eb) % 16 == 0);
  const int64_t ntl = (int64_t)pl.mt * pl.nt;
  const dim3 grid((unsigned)((B + 7) / 8 * 8 * ntl));
  if (geo)
    hipLaunchKernelGGL((k_explicit_tiles<T, BM, BN, true>), grid, dim3(256), 0, st, static_cast<const T*>(A),
                       static_cast<const T*>(G), B, Tn, d, p, has_bias, pl.mt, pl.nt, 0, vecG, sink, *geo);
  else
    hipLaunchKernelGGL((k_explicit_tiles<T, BM, BN, false>), grid, dim3(256), 0, st, static_cast<const T*>(A),
                       static_cast<const T*>(G), B, Tn, d, p, has_bias, pl.mt, pl.nt, vecA, vecG, sink, ConvGeo{});
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_explicit_d(hipStream_t st, const void* A, const void* G, int64_t B, int64_t Tn, int64_t d,
                                    int64_t p, int has_bias, const ExplicitPlan& pl, const NormSink& sink,
                                    const ConvGeo* geo) {
  if (pl.bm == 64 && pl.bn == 64) return launch_explicit_t<T, 64, 64>(st, A, G, B, Tn, d, p, has_bias, pl, sink, geo);
  if (pl.bm == 64) return launch_explicit_t<T, 64, 128>(st, A, G, B, Tn, d, p, has_bias, pl, sink, geo);
  if (pl.bn == 64) return launch_explicit_t<T, 128, 64>(st, A, G, B, Tn, d, p, has_bias, pl, sink, geo);
  return launch_explicit_t<T, 128, 128>(st, A, G, B, Tn, d, p, has_bias, pl, sink, geo);
}

hipError_t launch_explicit(hipStream_t st, int dtype, const void* A, const void* G, int64_t B, int64_t Tn, int64_t d,
                           int64_t p, int has_bias, const NormSink& sink) {
  const ExplicitPlan pl = explicit_plan(d, p, has_bias);
  if (dtype == 1) return launch_explicit_d<bf16s>(st, A, G, B, Tn, d, p, has_bias, pl, sink, nullptr);
  return launch_explicit_d<float>(st, A, G, B, Tn, d, p, has_bias, pl, sink, nullptr);
}

hipError_t launch_explicit_conv(hipStream_t st, int dtype, const ConvGeo& geo, const void* G, int64_t B, int64_t p,
                                int has_bias, const NormSink& sink) {
  const ExplicitPlan pl = explicit_plan(geo.d, p, has_bias);
  if (dtype == 1) return launch_explicit_d<bf16s>(st, geo.a, G, B, geo.T, geo.d, p, has_bias, pl, sink, &geo);
  return launch_explicit_d<float>(st, geo.a, G, B, geo.T, geo.d, p, has_bias, pl, sink, &geo);
}

template <typename T, int BM, int BN, bool FUSED>
static void launch_contract_k(hipStream_t st, dim3 grid, const void* A, const void* G, const float* c, int64_t B,
                              int64_t Tn, int64_t d, int64_t p, int has_bias, const ContractPlan& pl, int vecA,
                              int vecG, float* ws, const NoiseArgs& na, float* out, float* bias_out,
                              const ConvGeo* geo) {
  const int64_t nitems = (int64_t)pl.mt * pl.nt * pl.ks;
  if (geo)
    hipLaunchKernelGGL((k_contract_tiles<T, BM, BN, FUSED, true>), grid, dim3(256), 0, st, static_cast<const T*>(A),
                       static_cast<const T*>(G), c, B, Tn, d, p, has_bias, pl.mt, pl.nt, pl.units_per_split, nitems,
                       0, vecG, ws, na, out, bias_out, *geo);
  else
    hipLaunchKernelGGL((k_contract_tiles<T, BM, BN, FUSED, false>), grid, dim3(256), 0, st, static_cast<const T*>(A),
                       static_cast<const T*>(G), c, B, Tn, d, p, has_bias, pl.mt, pl.nt, pl.units_per_split, nitems,
                       vecA, vecG, ws, na, out, bias_out, ConvGeo{});
}

template <typename T, int BM, int BN>
static hipError_t launch_contract_t(hipStream_t st, const void* A, const void* G, const float* c, int64_t B,
                                    int64_t Tn, int64_t d, int64_t p, int has_bias, const ContractPlan& pl,
                                    float* ws, const NoiseArgs& na, float* out, float* bias_out,
                                    const ConvGeo* geo) {
  const int eb = elem_traits<T>::bytes;
  const int vecA = ((reinterpret_cast<uintptr_t>(A) & 15) == 0) && ((d * eb) % 16 == 0);
  const int vecG = ((reinterpret_cast<uintptr_t>(G) & 15) == 0) && ((p * eb) % 16 == 0);
  const dim3 grid((unsigned)(((int64_t)pl.mt * pl.nt * pl.ks + 7) / 8 * 8));  // whole XCD rounds
  if (pl.ks == 1)
    launch_contract_k<T, BM, BN, true>(st, grid, A, G, c, B, Tn, d, p, has_bias, pl, vecA, vecG, ws, na, out,
                                       bias_out, geo);
  else
    launch_contract_k<T, BM, BN, false>(st, grid, A, G, c, B, Tn, d, p, has_bias, pl, vecA, vecG, ws, na, out,
                                        bias_out, geo);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_contract_d(hipStream_t st, const void* A, const void* G, const float* c, int64_t B,
                                    int64_t Tn, int64_t d, int64_t p, int has_bias, const ContractPlan& pl,
                                    float* ws, const NoiseArgs& na, float* out, float* bias_out,
                                    const ConvGeo* geo = nullptr) {
  if (pl.bm == 64 && pl.bn == 64)
    return launch_contract_t<T, 64, 64>(st, A, G, c, B, Tn, d, p, has_bias, pl, ws, na, out, bias_out, geo);
  if (pl.bm == 64)
    return launch_contract_t<T, 64, 128>(st, A, G, c, B, Tn, d, p, has_bias, pl, ws, na, out, bias_out, geo);
  if (pl.bn == 64)
    return launch_contract_t<T, 128, 64>(st, A, G, c, B, Tn, d, p, has_bias, pl, ws, na, out, bias_out, geo);
  return launch_contract_t<T, 128, 128>(st, A, G, c, B, Tn, d, p, has_bias, pl, ws, na, out, bias_out, geo);
}

// Split partials in ws -> out (and bias_out) with the noise and the mean.
static hipError_t launch_reduce_noise(hipStream_t st, const ContractPlan& pl, float* ws, int64_t d, int64_t p,
                                      int has_bias, const NoiseArgs& na, float* out, float* bias_out) {
  const int64_t std_threads = ((d + 3) / 4) * ((p + 3) / 4);
  if (p % 4 == 0 && pl.ks >= 64 && std_threads < 32768) {
    // many splits, few outputs: split lanes in parallel
    const int64_t blocks = ((d + 3) / 4) * ((p + 15) / 16) + (has_bias ? (p + 63) / 64 : 0);
    hipLaunchKernelGGL(k_reduce_noise_wide, dim3((unsigned)blocks), dim3(256), 0, st, ws, pl.ks, d, p, has_bias, na,
                       out, bias_out);
    return hipGetLastError();
  }
  const int vec = (p % 4 == 0) && ((reinterpret_cast<uintptr_t>(out) & 15) == 0);
  if (vec && d % 4 == 0) {
    const int64_t threads = (d / 4) * (p / 4) + (has_bias ? p / 4 : 0);
    const dim3 grid((unsigned)((threads + 255) / 256));
    hipLaunchKernelGGL(k_reduce_noise_vec, grid, dim3(256), 0, st, ws, pl.ks, d, p, has_bias, na, out, bias_out);
    return hipGetLastError();
  }
  const int64_t threads = ((d + 3) / 4) * ((p + 3) / 4) + (has_bias ? (p + 3) / 4 : 0);
  const dim3 grid((unsigned)((threads + 255) / 256));
  hipLaunchKernelGGL(k_reduce_noise, grid, dim3(256), 0, st, ws, pl.ks, d, p, has_bias, vec, na, out, bias_out);
  return hipGetLastError();
}

hipError_t launch_split_reduce(hipStream_t st, int64_t ks, float* ws, int64_t d, int64_t p, const NoiseArgs& na,
                               float* out) {
  ContractPlan pl{};
  pl.ks = ks;
  return launch_reduce_noise(st, pl, ws, d, p, 0, na, out, nullptr);
}

hipError_t launch_split_reduce_group(hipStream_t st, const SplitReduceLayer* layers, int n) {
  if (n < 0 || n > kDlGroupMax) return hipErrorInvalidValue;
  RedGroup g{};
  int64_t blocks = 0;
  const bool acc = n > 0 && layers[0].acc != nullptr;
  for (int l = 0; l < n; ++l) {
    const SplitReduceLayer& x = layers[l];
    if ((x.acc != nullptr) != acc) return hipErrorInvalidValue;  // one kind of reduce per group
    const int64_t blocks_l = split_reduce_blocks(x);
    // layers the one-layer launch would not give to the vectorised kernel keep that launch
    if (!split_reduce_vec_ok(x) || blocks_l == 0) {
      hipError_t e = launch_split_reduce(st, x.ks, const_cast<float*>(x.ws), x.d, x.p, x.na, x.out);
      if (e == hipSuccess && x.acc) e = launch_accumulate(st, x.acc, x.out, x.d * x.p);
      if (e != hipSuccess) return e;
      continue;
    }
    g.L[g.n] = x;
    g.blk_begin[g.n] = blocks;
    blocks += blocks_l;
    ++g.n;
  }
  if (g.n == 0) return hipSuccess;
  if (blocks >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  if (acc)
    hipLaunchKernelGGL(k_reduce_noise_group<true>, dim3((unsigned)blocks), dim3(256), 0, st, g);
  else
    hipLaunchKernelGGL(k_reduce_noise_group<false>, dim3((unsigned)blocks), dim3(256), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_clipped_sum_conv(hipStream_t st, int dtype, const ConvGeo& geo, const void* G, const float* c,
                                   int64_t B, int64_t p, const ContractPlan& pl, float* ws, float sc, float denom,
                                   uint64_t seed, uint32_t layer, uint32_t step, float* out, float* bias_out) {
  const int has_bias = bias_out != nullptr ? 1 : 0;
  const NoiseArgs na = make_noise_args(sc, denom, seed, layer, step);
  hipError_t e;
  if (dtype == 1)
    e = launch_contract_d<bf16s>(st, geo.a, G, c, B, geo.T, geo.d, p, has_bias, pl, ws, na, out, bias_out, &geo);
  else
    e = launch_contract_d<float>(st, geo.a, G, c, B, geo.T, geo.d, p, has_bias, pl, ws, na, out, bias_out, &geo);
  if (e != hipSuccess || pl.ks == 1) return e;
  return launch_reduce_noise(st, pl, ws, geo.d, p, has_bias, na, out, bias_out);
}

hipError_t launch_clipped_sum(hipStream_t st, int dtype, const void* A, const void* G, const float* c, int64_t B,
                              int64_t Tn, int64_t d, int64_t p, const ContractPlan& pl, float* ws, float sc,
                              float denom, uint64_t seed, uint32_t layer, uint32_t step, float* out,
                              float* bias_out) {
  const int has_bias = bias_out != nullptr ? 1 : 0;
  const NoiseArgs na = make_noise_args(sc, denom, seed, layer, step);
  hipError_t e;
  if (pl.engine == 1)
    e = launch_contract_dl(st, A, G, c, B, Tn, d, p, pl, ws, na, out);
  else if (pl.engine == 2)
    e = launch_contract_dl32(st, A, G, c, B, Tn, d, p, pl, ws, na, out, bias_out);
  else if (dtype == 1)
    e = launch_contract_d<bf16s>(st, A, G, c, B, Tn, d, p, has_bias, pl, ws, na, out, bias_out);
  else
    e = launch_contract_d<float>(st, A, G, c, B, Tn, d, p, has_bias, pl, ws, na, out, bias_out);
  if (e != hipSuccess || (pl.ks == 1 && !pl.partials)) return e;
  return launch_reduce_noise(st, pl, ws, d, p, has_bias, na, out, bias_out);
}

}  // namespace dpk
