// Per-example gradient norms of one layer (three paths) and their per-sample
// reduction.
//
//  * closed form, T = 1: ||a_i (x) g_i||_F^2 = ||a_i||^2 ||g_i||^2 (FPC eq. (6));
//    with a bias the input gains a constant-1 feature: (||a_i||^2 + 1) ||g_i||^2.
//  * ghost: ||A_i^T G_i||_F^2 = <A_i A_i^T, G_i G_i^T> (SEDP eq. (2.7), Sec. 3.1)
//    on LDS-staged Gram tiles computed by MFMA; the Grams never leave
//    registers. With a bias, A_i A_i^T + 1 1^T.
//  * explicit (per-sample instantiation, SEDP App. C.4) lives in dp_xty.hip.
//
// Reductions are fixed-order (no atomics), so results are bitwise
// reproducible.
#include "dp_common.hpp"

#include "dp_launch.hpp"

namespace dpk {

// ---------------------------------------------------------------- T == 1
template <typename T>
__device__ __forceinline__ float row_sqsum(const T* __restrict__ row, int64_t n, int lane) {
  constexpr int P = elem_traits<T>::per16;
  float s0 = 0.f, s1 = 0.f;
  const bool vec = ((reinterpret_cast<uintptr_t>(row) & 15) == 0);
  int64_t nv = vec ? (n / P) : 0;
  const u32x4* rv = reinterpret_cast<const u32x4*>(row);
  for (int64_t q = lane; q < nv; q += kWave) {
    const u32x4 v = rv[q];
    const uint32_t w[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (P == 8) {
        const float lo = __uint_as_float(w[e] << 16);
        const float hi = __uint_as_float(w[e] & 0xFFFF0000u);
        s0 += lo * lo;
        s1 += hi * hi;
      } else {
        const float x = __uint_as_float(w[e]);
        if (e & 1)
          s1 += x * x;
        else
          s0 += x * x;
      }
    }
  }
  for (int64_t k = nv * P + lane; k < n; k += kWave) {
    const float x = to_f32(row[k]);
    s0 += x * x;
  }
  return s0 + s1;
}

// One wave per sample, four samples per workgroup.
template <typename T>
__global__ __launch_bounds__(256) void k_norm_t1(const T* __restrict__ A, const T* __restrict__ G, int64_t B,
                                                 int64_t d, int64_t p, int has_bias, int accumulate,
                                                 float* __restrict__ sqnorm) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= B) return;
  float sa = wave_sum(row_sqsum(A + i * d, d, lane));
  float sg = wave_sum(row_sqsum(G + i * p, p, lane));
  if (lane == 0) {
    const float v = (sa + (has_bias ? 1.0f : 0.0f)) * sg;
    sqnorm[i] = accumulate ? sqnorm[i] + v : v;
  }
}

// ---------------------------------------------------------------- ghost tiles
// Workgroup = (sample i, Gram tile (sb, tb), sb <= tb) of TS x TS. Four waves
// in 2 x 2, each a (TS/2)^2 sub-tile of 32x32 MFMA blocks. The K loop stages
// 256-byte row chunks of the two row blocks (one if diagonal) into a
// double-buffered LDS, with the next chunk's global loads in flight during
// the MFMAs of this one: first the chunks of A_i (K = d, Gram of A), then
// those of G_i (K = p, Gram of G). The epilogue forms sum (GA + bias) .* GG,
// doubled off the diagonal. Samples of at most TS/2 rows are stacked, up to
// kGhostPackMax consecutive samples per tile (their rows are consecutive in
// memory): the workgroup then takes one diagonal tile of all of them, and the
// epilogue keeps only the entries of two rows of one sample, per sample.
#ifndef GHOST64_GROUPS
#define GHOST64_GROUPS 2
#endif
constexpr int kGhost64Groups = GHOST64_GROUPS;
// At most this many samples share one Gram tile (samples of T <= TS / 2 rows).
constexpr int kGhostPackMax = 4;

template <typename T, int TS>
struct GhostCfg {
  // 64-row tiles: KW groups of 4 waves taking interleaved MFMA k-steps of
  // every chunk (more waves per SIMD to hide LDS latency; the groups'
  // partial Grams are added before the Frobenius product); 128-row tiles: 4
  // waves
  static constexpr int KW = TS == 64 ? kGhost64Groups : 1;  // wave groups sharing a chunk's k-steps
  static constexpr int NT = 256 * KW;
  static constexpr int P = elem_traits<T>::per16;
  static constexpr int CB = TS == 64 ? 256 : 128;  // bytes per staged row chunk (8 vectors/thread either way)
  static constexpr int V = CB / 16;                // 16-byte vectors per row chunk
  static constexpr int KC = V * P;                 // elements per staged row chunk
  static constexpr int ROWB = CB + 16;             // LDS row stride (bytes), conflict-free b128 reads
  static constexpr int BUF = 2 * TS * ROWB;        // one buffer: both row blocks
  static constexpr int WM = TS / 2;
  static constexpr int NB = WM / 32;
  static constexpr int PIECES = 2 * TS * V;        // 16-byte pieces of one chunk of both row blocks
  static constexpr int PPT = PIECES / NT;
  static_assert(PIECES % NT == 0, "tile/threads mismatch");
  struct Regs {
    u32x4 v[PPT];
  };
};

template <typename T, int TS>
__device__ __forceinline__ void ghost_load(typename GhostCfg<T, TS>::Regs& regs, const T* __restrict__ Xi, int64_t Tn,
                                           int64_t K, bool vec, int sb, int tb, int64_t chunk) {
  using Cfg = GhostCfg<T, TS>;
  const bool diag = (sb == tb);
#pragma unroll
  for (int r = 0; r < Cfg::PPT; ++r) {
    const int q = threadIdx.x + r * Cfg::NT;
    const int h = q / (TS * Cfg::V);
    const int row = (q / Cfg::V) % TS;
    const int c16 = q % Cfg::V;
    if (diag && h == 1) {
      regs.v[r] = u32x4{0u, 0u, 0u, 0u};
    } else {
      const int64_t grow = (int64_t)(h == 0 ? sb : tb) * TS + row;
      regs.v[r] = load16_rowmajor(Xi, Tn, K, grow, chunk * Cfg::KC + c16 * Cfg::P, vec);
    }
  }
}

// ghost_load of a chunk of A_i = U(a_i), the unfolded input of convolution
// `g`, formed from sample i of its folded input.
template <typename T, int TS>
__device__ __forceinline__ void ghost_load_conv(typename GhostCfg<T, TS>::Regs& regs, const ConvGeo& g, int64_t i,
                                                int sb, int tb, int64_t chunk) {
  using Cfg = GhostCfg<T, TS>;
  static_assert(Cfg::NT % Cfg::V == 0, "a thread keeps one column vector");
  const bool diag = (sb == tb);
  // every piece of this thread covers the same columns
  const int64_t col = chunk * Cfg::KC + (threadIdx.x % Cfg::V) * Cfg::P;
  const ConvCol c0 = conv_col(g, col);
#pragma unroll
  for (int r = 0; r < Cfg::PPT; ++r) {
    const int q = threadIdx.x + r * Cfg::NT;
    const int h = q / (TS * Cfg::V);
    const int row = (q / Cfg::V) % TS;
    if (diag && h == 1) {
      regs.v[r] = u32x4{0u, 0u, 0u, 0u};
    } else {
      const int grow = (h == 0 ? sb : tb) * TS + row;
      const bool ok = grow < g.T;
      regs.v[r] = conv_row16_walk<T>(g, conv_row_at(g, i, ok ? grow : 0), c0, col, ok);
    }
  }
}

template <typename T, int TS>
__device__ __forceinline__ void ghost_store(const typename GhostCfg<T, TS>::Regs& regs, unsigned char* buf, bool diag) {
  using Cfg = GhostCfg<T, TS>;
#pragma unroll
  for (int r = 0; r < Cfg::PPT; ++r) {
    const int q = threadIdx.x + r * Cfg::NT;
    const int h = q / (TS * Cfg::V);
    const int row = (q / Cfg::V) % TS;
    const int c16 = q % Cfg::V;
    if (!(diag && h == 1)) *reinterpret_cast<u32x4*>(buf + (h * TS + row) * Cfg::ROWB + c16 * 16) = regs.v[r];
  }
}

template <typename T, int TS>
__device__ __forceinline__ void ghost_compute(const unsigned char* buf, bool diag,
                                              f32x16 (&acc)[GhostCfg<T, TS>::NB][GhostCfg<T, TS>::NB]) {
  using Cfg = GhostCfg<T, TS>;
  constexpr int NB = Cfg::NB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wq = wave & 3, kg = wave >> 2;  // sub-tile, and share of the chunk's k-steps
  static_assert(Cfg::KC / 16 % Cfg::KW == 0 && Cfg::KC / 8 % Cfg::KW == 0, "k-steps split evenly");
  const int wm = wq & 1, wn = wq >> 1;
  const unsigned char* sbase = buf;
  const unsigned char* tbase = buf + (diag ? 0 : TS * Cfg::ROWB);
  if constexpr (Cfg::P == 8) {
#pragma unroll
    for (int kj = 0; kj < Cfg::KC / 16 / Cfg::KW; ++kj) {
      const int ks = kj * Cfg::KW + kg;
      u32x4 a[NB], b[NB];
#pragma unroll
      for (int bi = 0; bi < NB; ++bi) {
        const int row = wm * Cfg::WM + bi * 32 + (lane & 31);
        a[bi] = *reinterpret_cast<const u32x4*>(sbase + row * Cfg::ROWB + ks * 32 + (lane >> 5) * 16);
      }
#pragma unroll
      for (int bj = 0; bj < NB; ++bj) {
        const int row = wn * Cfg::WM + bj * 32 + (lane & 31);
        b[bj] = *reinterpret_cast<const u32x4*>(tbase + row * Cfg::ROWB + ks * 32 + (lane >> 5) * 16);
      }
#pragma unroll
      for (int bi = 0; bi < NB; ++bi)
#pragma unroll
        for (int bj = 0; bj < NB; ++bj) acc[bi][bj] = mfma32_bf16(a[bi], b[bj], acc[bi][bj]);
    }
  } else {
#pragma unroll
    for (int gj = 0; gj < Cfg::KC / 8 / Cfg::KW; ++gj) {
      const int g = gj * Cfg::KW + kg;
      float4 a[NB], b[NB];
#pragma unroll
      for (int bi = 0; bi < NB; ++bi) {
        const int row = wm * Cfg::WM + bi * 32 + (lane & 31);
        a[bi] = *reinterpret_cast<const float4*>(sbase + row * Cfg::ROWB + g * 32 + (lane >> 5) * 16);
      }
#pragma unroll
      for (int bj = 0; bj < NB; ++bj) {
        const int row = wn * Cfg::WM + bj * 32 + (lane & 31);
        b[bj] = *reinterpret_cast<const float4*>(tbase + row * Cfg::ROWB + g * 32 + (lane >> 5) * 16);
      }
#pragma unroll
      for (int bi = 0; bi < NB; ++bi)
#pragma unroll
        for (int bj = 0; bj < NB; ++bj) {
          acc[bi][bj] = mfma32_f32(a[bi].x, b[bj].x, acc[bi][bj]);
          acc[bi][bj] = mfma32_f32(a[bi].y, b[bj].y, acc[bi][bj]);
          acc[bi][bj] = mfma32_f32(a[bi].z, b[bj].z, acc[bi][bj]);
          acc[bi][bj] = mfma32_f32(a[bi].w, b[bj].w, acc[bi][bj]);
        }
    }
  }
}

// Unchecked pipeline for interior tiles: both row blocks inside the sample
// and d, p multiples of the chunk. Chunk c < nA comes from A_i (Gram of A),
// the rest from G_i. Two named register stages keep the loads of chunks c+1
// and c+2 in flight (the last loads re-read the final chunk: a clamped index
// keeps the body straight-line). Piece slot r of a thread belongs to row
// block r / PPB (a compile-time constant), so diagonal tiles skip the second
// block's slots without divergence.
template <typename T, int TS, bool DIAG>
struct GhostFull {
  using Cfg = GhostCfg<T, TS>;
  static constexpr int PPB = Cfg::PPT / 2;             // pieces per thread per row block
  static constexpr int NPS = DIAG ? PPB : Cfg::PPT;    // piece slots in use (one block if diagonal)

  // slot r of this thread: row block r / PPB, piece pb = tid + (r % PPB) * NT
  __device__ __forceinline__ static void load(typename Cfg::Regs& R, const T* base, int64_t K, int64_t k0, int sb,
                                              int tb) {
#pragma unroll
    for (int r = 0; r < NPS; ++r) {
      const int pb = (int)threadIdx.x + (r % PPB) * Cfg::NT;
      const int64_t row = (int64_t)((r / PPB) == 0 ? sb : tb) * TS + pb / Cfg::V;
      R.v[r] = *reinterpret_cast<const u32x4*>(base + row * K + k0 + (pb % Cfg::V) * Cfg::P);
    }
  }
  __device__ __forceinline__ static void store(const typename Cfg::Regs& R, unsigned char* buf) {
#pragma unroll
    for (int r = 0; r < NPS; ++r) {
      const int pb = (int)threadIdx.x + (r % PPB) * Cfg::NT;
      *reinterpret_cast<u32x4*>(buf + ((r / PPB) * TS + pb / Cfg::V) * Cfg::ROWB + (pb % Cfg::V) * 16) = R.v[r];
    }
  }
  __device__ __forceinline__ static void load_chunk(typename Cfg::Regs& R, const T* Ai, const T* Gi, int64_t d,
                                                    int64_t p, int64_t nA, int64_t c, int sb, int tb) {
    const bool isA = c < nA;
    load(R, isA ? Ai : Gi, isA ? d : p, (isA ? c : c - nA) * Cfg::KC, sb, tb);
  }
  __device__ __forceinline__ static void step(typename Cfg::Regs& R, unsigned char* buf, const T* Ai, const T* Gi,
                                              int64_t d, int64_t p, int64_t nA, int64_t c, int64_t last, int sb,
                                              int tb, f32x16 (&acc_a)[Cfg::NB][Cfg::NB],
                                              f32x16 (&acc_g)[Cfg::NB][Cfg::NB]) {
    store(R, buf);
    __syncthreads();
    load_chunk(R, Ai, Gi, d, p, nA, c + 2 <= last ? c + 2 : last, sb, tb);
    if (c < nA)
      ghost_compute<T, TS>(buf, DIAG, acc_a);
    else
      ghost_compute<T, TS>(buf, DIAG, acc_g);
  }
  // Unchecked pipeline for interior tiles: both row blocks inside the sample
  // and d, p multiples of the chunk. Chunk c < nA comes from A_i (Gram of
  // A), the rest from G_i. Two register stages keep the loads of chunks c+1
  // and c+2 in flight (the last loads re-read the final chunk: a clamped
  // index keeps the body straight-line).
  __device__ __forceinline__ static void run(const T* Ai, const T* Gi, int64_t d, int64_t p, int sb, int tb,
                                             unsigned char* lds, f32x16 (&acc_a)[Cfg::NB][Cfg::NB],
                                             f32x16 (&acc_g)[Cfg::NB][Cfg::NB]) {
    const int64_t nA = d / Cfg::KC, n = nA + p / Cfg::KC;
    const int64_t last = n - 1;
    typename Cfg::Regs R0, R1;
    load_chunk(R0, Ai, Gi, d, p, nA, 0, sb, tb);
    load_chunk(R1, Ai, Gi, d, p, nA, 1 <= last ? 1 : last, sb, tb);
    int64_t c = 0;
    for (; c + 1 <= last; c += 2) {
      step(R0, lds, Ai, Gi, d, p, nA, c, last, sb, tb, acc_a, acc_g);
      step(R1, lds + Cfg::BUF, Ai, Gi, d, p, nA, c + 1, last, sb, tb, acc_a, acc_g);
    }
    if (c == last) step(R0, lds, Ai, Gi, d, p, nA, c, last, sb, tb, acc_a, acc_g);
  }
};

// One layer of a ghost launch: its operands and sizes, the first workgroup
// of its range in the grid (a multiple of 8, so that a workgroup's id mod 8
// is still its XCD within the range) and its first tile in the sink.
template <typename T>
struct GhostLayer {
  const T* A;
  const T* G;
  int64_t Tn, d, p;
  int pack;  // samples stacked in one tile (T <= TS / 2), else 1
  int64_t wg_begin;
  int nb, ntiles, tile_base, vecA, vecG, has_bias;
};
// The layers of one launch, ordered by wg_begin.
template <typename T>
struct GhostGroup {
  GhostLayer<T> L[kNormGroupMax];
  int n;
  ConvGeo conv;  // IM2COL launches (one layer): A_i is formed from conv's folded input
};

template <typename T, int TS, bool IM2COL>
__global__ __launch_bounds__((GhostCfg<T, TS>::NT)) void k_ghost_tiles(GhostGroup<T> grp, int64_t B, NormSink sink) {
  using Cfg = GhostCfg<T, TS>;
  constexpr int NB = Cfg::NB;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  __shared__ float red[Cfg::NT / kWave];

  // the layer whose workgroup range holds this workgroup (a uniform choice
  // among compile-time entries: no indexing into the argument block)
  GhostLayer<T> L = grp.L[0];
#pragma unroll
  for (int k = 1; k < kNormGroupMax; ++k)
    if (k < grp.n && (int64_t)blockIdx.x >= grp.L[k].wg_begin) L = grp.L[k];
  const T* __restrict__ A = L.A;
  const T* __restrict__ G = L.G;
  const int64_t Tn = L.Tn, d = L.d, p = L.p;
  const int nb = L.nb, vecA = L.vecA, vecG = L.vecG, has_bias = L.has_bias;

  int64_t grp_i, tile;
  xcd_group_map((int64_t)blockIdx.x - L.wg_begin, L.ntiles, &grp_i, &tile);
  // samples i0 .. i0 + nvalid - 1 (one unless the layer packs several short samples per tile)
  const int pack = L.pack;
  const int64_t i0 = grp_i * pack;
  if (i0 >= B) return;
  const int nvalid = (int)(B - i0 < pack ? B - i0 : pack);
  const int64_t rows = nvalid * Tn;  // valid tile rows: consecutive rows of consecutive samples
  int sb = 0;
  int rem = (int)tile;
  while (rem >= nb - sb) {
    rem -= nb - sb;
    ++sb;
  }
  const int tb = sb + rem;
  const bool diag = (sb == tb);

  f32x16 acc_a[NB][NB], acc_g[NB][NB];
#pragma unroll
  for (int bi = 0; bi < NB; ++bi)
#pragma unroll
    for (int bj = 0; bj < NB; ++bj)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        acc_a[bi][bj][j] = 0.f;
        acc_g[bi][bj][j] = 0.f;
      }

  const T* Ai = IM2COL ? A : A + i0 * Tn * d;
  const T* Gi = G + i0 * Tn * p;
  const bool full =
      !IM2COL && vecA && vecG && (int64_t)(tb + 1) * TS <= rows && d % Cfg::KC == 0 && p % Cfg::KC == 0;
  if (full && sb == tb) {
    GhostFull<T, TS, true>::run(Ai, Gi, d, p, sb, tb, lds, acc_a, acc_g);
  } else if (full) {
    GhostFull<T, TS, false>::run(Ai, Gi, d, p, sb, tb, lds, acc_a, acc_g);
  } else {
  const int64_t nA = (d + Cfg::KC - 1) / Cfg::KC;
  const int64_t nG = (p + Cfg::KC - 1) / Cfg::KC;
  const int64_t n = nA + nG;
  typename Cfg::Regs regs;
  if constexpr (IM2COL)
    ghost_load_conv<T, TS>(regs, grp.conv, i0, sb, tb, 0);  // pack == 1
  else
    ghost_load<T, TS>(regs, Ai, rows, d, vecA != 0, sb, tb, 0);
  for (int64_t c = 0; c < n; ++c) {
    unsigned char* buf = lds + (c & 1) * Cfg::BUF;
    ghost_store<T, TS>(regs, buf, diag);
    __syncthreads();
    const int64_t cn = c + 1;
    if (cn < nA) {
      if constexpr (IM2COL)
        ghost_load_conv<T, TS>(regs, grp.conv, i0, sb, tb, cn);
      else
        ghost_load<T, TS>(regs, Ai, rows, d, vecA != 0, sb, tb, cn);
    } else if (cn < n)
      ghost_load<T, TS>(regs, Gi, rows, p, vecG != 0, sb, tb, cn - nA);
    if (c < nA)
      ghost_compute<T, TS>(buf, diag, acc_a);
    else
      ghost_compute<T, TS>(buf, diag, acc_g);
  }
  }

  bool owner = true;  // this wave holds complete Gram entries
  if constexpr (Cfg::KW > 1) {
    // the groups' partial Grams are added pairwise through LDS (groups
    // [h, 2h) into [0, h), h = KW/2 .. 1), entry-major ([entry][sub-tile][lane]:
    // consecutive lanes, consecutive words)
    constexpr int PER = 2 * NB * NB * 16;
    constexpr int REGION = PER * 256;  // floats of one group
    static_assert((Cfg::KW / 2) * REGION * 4 <= 2 * Cfg::BUF, "exchange fits the staging buffers");
    float* xch = reinterpret_cast<float*>(lds);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int grp = wave >> 2, slot = (wave & 3) * 64 + lane;
#pragma unroll
    for (int h = Cfg::KW / 2; h >= 1; h /= 2) {
      __syncthreads();  // every wave is done with the staging buffers / the previous round
      if (grp >= h && grp < 2 * h) {
        float* dst = xch + (grp - h) * REGION;
        int e = 0;
#pragma unroll
        for (int bi = 0; bi < NB; ++bi)
#pragma unroll
          for (int bj = 0; bj < NB; ++bj)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              dst[(e++) * 256 + slot] = acc_a[bi][bj][j];
              dst[(e++) * 256 + slot] = acc_g[bi][bj][j];
            }
      }
      __syncthreads();
      if (grp < h) {
        const float* src = xch + grp * REGION;
        int e = 0;
#pragma unroll
        for (int bi = 0; bi < NB; ++bi)
#pragma unroll
          for (int bj = 0; bj < NB; ++bj)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              acc_a[bi][bj][j] += src[(e++) * 256 + slot];
              acc_g[bi][bj][j] += src[(e++) * 256 + slot];
            }
      }
    }
    owner = grp == 0;
  }

  const float one = has_bias ? 1.0f : 0.0f;
  if (pack > 1) {
    // one diagonal tile of stacked samples: only entries of two rows of the
    // same sample count, summed per sample (row r belongs to sample r / T)
    __shared__ float red4[kGhostPackMax * (Cfg::NT / kWave)];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wq = wave & 3, wm = wq & 1, wn = wq >> 1;
    float sk[kGhostPackMax];
#pragma unroll
    for (int k = 0; k < kGhostPackMax; ++k) sk[k] = 0.f;
    if (owner) {
#pragma unroll
      for (int bi = 0; bi < NB; ++bi)
#pragma unroll
        for (int bj = 0; bj < NB; ++bj)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int r = wm * Cfg::WM + bi * 32 + acc_row(j, lane);
            const int c = wn * Cfg::WM + bj * 32 + acc_col(lane);
            const int kr = r / (int)Tn, kc = c / (int)Tn;
            const float v = (acc_a[bi][bj][j] + one) * acc_g[bi][bj][j];
#pragma unroll
            for (int k = 0; k < kGhostPackMax; ++k)
              if (kr == k && kc == k) sk[k] += v;
          }
    }
#pragma unroll
    for (int k = 0; k < kGhostPackMax; ++k) sk[k] = wave_sum(sk[k]);
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < kGhostPackMax; ++k) red4[k * (Cfg::NT / kWave) + wave] = sk[k];
    }
    __syncthreads();
    if ((int)threadIdx.x < nvalid) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < Cfg::NT / kWave; ++w) v += red4[threadIdx.x * (Cfg::NT / kWave) + w];
      norm_sink_tile(sink, i0 + threadIdx.x, L.tile_base + tile, v);
    }
    return;
  }
  float s = 0.f;
  if (owner) {
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
#pragma unroll
      for (int bj = 0; bj < NB; ++bj)
#pragma unroll
        for (int j = 0; j < 16; ++j) s += (acc_a[bi][bj][j] + one) * acc_g[bi][bj][j];
  }
  if (!diag) s *= 2.0f;
  s = block_sum<Cfg::NT>(s, red);
  if (threadIdx.x == 0) norm_sink_tile(sink, i0, L.tile_base + tile, s);
}

// ---------------------------------------------------------------- launchers
template <typename T>
hipError_t launch_norm_t1_t(hipStream_t st, const void* A, const void* G, int64_t B, int64_t d, int64_t p,
                            int has_bias, int accumulate, float* sqnorm) {
  const dim3 grid((unsigned)((B + 3) / 4));
  hipLaunchKernelGGL(k_norm_t1<T>, grid, dim3(256), 0, st, static_cast<const T*>(A), static_cast<const T*>(G), B, d,
                     p, has_bias, accumulate, sqnorm);
  return hipGetLastError();
}

hipError_t launch_norm_t1(hipStream_t st, int dtype, const void* A, const void* G, int64_t B, int64_t d, int64_t p,
                          int has_bias, int accumulate, float* sqnorm) {
  if (dtype == 1) return launch_norm_t1_t<bf16s>(st, A, G, B, d, p, has_bias, accumulate, sqnorm);
  return launch_norm_t1_t<float>(st, A, G, B, d, p, has_bias, accumulate, sqnorm);
}

int ghost_tile_size(int64_t T) { return T <= 384 ? 64 : 128; }

int64_t ghost_tiled_ntiles(int64_t T) {
  const int64_t ts = ghost_tile_size(T);
  const int64_t nb = (T + ts - 1) / ts;
  return nb * (nb + 1) / 2;
}

int64_t ghost_ntiles(int dtype, int64_t T, int64_t d, int64_t p) {
  if (ghost_wide_eligible(dtype, T, d, p)) return ghost_wide_ntiles(T);
  return ghost_tiled_ntiles(T);
}

template <typename T>
static GhostLayer<T> ghost_layer(const GhostLayerDesc& x, int ts, bool folded) {
  const int eb = elem_traits<T>::bytes;
  GhostLayer<T> L{};
  L.A = static_cast<const T*>(x.A);
  L.G = static_cast<const T*>(x.G);
  L.Tn = x.Tn;
  L.d = x.d;
  L.p = x.p;
  L.nb = (int)((x.Tn + ts - 1) / ts);
  L.ntiles = L.nb * (L.nb + 1) / 2;
  // samples of at most half a tile share one tile (up to kGhostPackMax): the
  // loads then fill the tile's rows instead of one sample's few. Not for
  // folded convolution inputs: their rows are gathered element by element
  // whatever the tile holds, and packing only removes workgroups.
  const int64_t fit = ts / x.Tn;
  L.pack = !folded && fit >= 2 ? (int)(fit < kGhostPackMax ? fit : kGhostPackMax) : 1;
  L.vecA = ((reinterpret_cast<uintptr_t>(x.A) & 15) == 0) && ((x.d * eb) % 16 == 0);
  L.vecG = ((reinterpret_cast<uintptr_t>(x.G) & 15) == 0) && ((x.p * eb) % 16 == 0);
  L.has_bias = x.has_bias;
  return L;
}

// Layers are laid out in the grid by decreasing work per tile (the largest
// tiles start first and the short ones fill the tail); tile_base follows the
// caller's order, which is the order of the sink's fold.
template <typename T, int TS>
hipError_t launch_ghost_t(hipStream_t st, const GhostLayerDesc* layers, int n, int64_t B, const NormSink& sink,
                          const ConvGeo* conv = nullptr) {
  GhostGroup<T> grp{};
  int order[kNormGroupMax];
  int base = 0;
  for (int l = 0; l < n; ++l) {
    grp.L[l] = ghost_layer<T>(layers[l], TS, conv != nullptr);
    grp.L[l].tile_base = base;
    base += grp.L[l].ntiles;
    order[l] = l;
  }
  for (int a = 1; a < n; ++a)  // stable insertion sort by d + p, largest first
    for (int b = a; b > 0 && layers[order[b]].d + layers[order[b]].p > layers[order[b - 1]].d + layers[order[b - 1]].p;
         --b) {
      const int t = order[b];
      order[b] = order[b - 1];
      order[b - 1] = t;
    }
  GhostGroup<T> sorted{};
  int64_t wg = 0;
  for (int k = 0; k < n; ++k) {
    sorted.L[k] = grp.L[order[k]];
    sorted.L[k].wg_begin = wg;
    const int64_t units = (B + sorted.L[k].pack - 1) / sorted.L[k].pack;  // samples or sample packs
    wg += (units + 7) / 8 * 8 * sorted.L[k].ntiles;
  }
  sorted.n = n;
  const size_t lds_bytes = 2 * GhostCfg<T, TS>::BUF;
  if (conv) {
    sorted.conv = *conv;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_ghost_tiles<T, TS, true>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_ghost_tiles<T, TS, true>), dim3((unsigned)wg), dim3(GhostCfg<T, TS>::NT), lds_bytes, st,
                       sorted, B, sink);
    return hipGetLastError();
  }
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_ghost_tiles<T, TS, false>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_ghost_tiles<T, TS, false>), dim3((unsigned)wg), dim3(GhostCfg<T, TS>::NT), lds_bytes, st,
                     sorted, B, sink);
  return hipGetLastError();
}

int ghost_group_key(int dtype, int64_t Tn, int64_t d, int64_t p) {
  if (ghost_wide_eligible(dtype, Tn, d, p)) return 1;
  return 2 * ghost_tile_size(Tn) + (dtype == 1 ? 1 : 0);
}

hipError_t launch_ghost_group(hipStream_t st, int dtype, const GhostLayerDesc* layers, int n, int64_t B,
                              const NormSink& sink) {
  if (ghost_wide_eligible(dtype, layers[0].Tn, layers[0].d, layers[0].p))
    return launch_ghost_wide_group(st, layers, n, B, sink);
  const int ts = ghost_tile_size(layers[0].Tn);
  if (dtype == 1) {
    if (ts == 64) return launch_ghost_t<bf16s, 64>(st, layers, n, B, sink);
    return launch_ghost_t<bf16s, 128>(st, layers, n, B, sink);
  }
  if (ts == 64) return launch_ghost_t<float, 64>(st, layers, n, B, sink);
  return launch_ghost_t<float, 128>(st, layers, n, B, sink);
}

hipError_t launch_ghost(hipStream_t st, int dtype, const void* A, const void* G, int64_t B, int64_t Tn, int64_t d,
                        int64_t p, int has_bias, const NormSink& sink) {
  if (ghost_wide_eligible(dtype, Tn, d, p)) return launch_ghost_wide(st, A, G, B, Tn, d, p, has_bias, sink);
  const GhostLayerDesc x{A, G, Tn, d, p, has_bias};
  return launch_ghost_group(st, dtype, &x, 1, B, sink);
}

hipError_t launch_ghost_conv(hipStream_t st, int dtype, const ConvGeo& geo, const void* G, int64_t B, int64_t p,
                             int has_bias, const NormSink& sink) {
  const GhostLayerDesc x{geo.a, G, geo.T, geo.d, p, has_bias};
  const int ts = ghost_tile_size(geo.T);
  if (dtype == 1) {
    if (ts == 64) return launch_ghost_t<bf16s, 64>(st, &x, 1, B, sink, &geo);
    return launch_ghost_t<bf16s, 128>(st, &x, 1, B, sink, &geo);
  }
  if (ts == 64) return launch_ghost_t<float, 64>(st, &x, 1, B, sink, &geo);
  return launch_ghost_t<float, 128>(st, &x, 1, B, sink, &geo);
}

}  // namespace dpk
