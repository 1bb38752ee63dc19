// Ghost norm of a bf16 layer of more than 64 rows per sample, direct-to-LDS
// engine.
//
// The per-example squared norm of "Scalable and Efficient Training of Large
// CNNs with DP", eq. (2.7) / Sec. 3.1 (ghost clipping):
// n_i^2 = <A_i A_i^T, G_i G_i^T>_F, plus the bias term through
// A_i A_i^T + 1 1^T, without forming A_i^T G_i. Both Grams are symmetric, so
// only entries s <= t are computed; entries s < t count twice.
//
// Eligible layers: bf16, T > 64, d and p multiples of 64 (samples of at most
// 64 rows are stacked in the tiled kernel's 64-row tiles instead). At
// T <= 128 a sample is one 128 x 128 tile: each row is read once, by one
// workgroup.
//
// Work item = (sample i, Gram tile (r, c)): rows s in [256 r, 256 r + 256) x
// columns t in [128 c, 128 c + 128), c >= 2r (every entry with s <= t lies in
// such a tile). A T x T Gram has sum over r of (ceil(T/128) - 2r) tiles.
// When the column block lies inside the row block (c = 2r or 2r + 1) its
// rows are read from the row block's stage instead of being loaded again;
// for c = 2r only the first 128 rows of the row block hold entries s <= t, and
// only they are loaded. A wave whose 64 x 64 sub-tile lies wholly below the
// diagonal (or past T) has weight 0 everywhere and skips its reads and MFMAs.
//
// gfx950 mapping:
// - Features are streamed in chunks of 64: a chunk holds the tile's rows
//   (256 + 128, 256 or 128) x 128 bytes and goes from HBM straight to LDS with
//   16-byte global_load_lds; the 16-byte pieces of row R are XOR-swizzled by
//   (R / 2) % 8, so that the 16 rows a ds_read_b128 serves per pass land on
//   64 distinct banks. The chunks of A_i come first (Gram of A), then those
//   of G_i (Gram of G).
// - A Gram product only needs row-major operands: an MFMA 32x32x16 operand
//   is 8 consecutive features of one row, one ds_read_b128 (no transposes).
// - 8 waves on the 4 x 2 grid of 64 x 64 sub-tiles (assignment in
//   gw_item); each lane holds both Grams' 64-entry accumulators until the
//   epilogue forms
//   sum_{s,t} w(s,t) (GA + bias) GG with w = 2 (s < t), 1 (s = t), 0 (s > t
//   or past T).
// - LDS stages: 3 for the 384- and 256-row tiles, 4 for the 128-row tile
//   (its chunks are a third the size); one barrier per chunk; each tile
//   stores its part and the finish kernel sums a sample's parts in tile
//   order (NormSink).
// - Operand reads run half a chunk (two k-steps) ahead of the MFMAs, across
//   the barrier into the next chunk.
// - Work items are XCD-grouped by sample: the tiles of one sample run on one
//   XCD and share its rows in that XCD's L2.
#include "dp_common.hpp"
#include "dp_launch.hpp"
#include "dp_lds.hpp"

namespace dpk {

namespace gw {
constexpr int BM = 256, BN = 128;  // Gram tile rows x columns
constexpr int KC = 64;             // features per chunk
constexpr int ROWB = KC * 2;       // LDS bytes per row and chunk
constexpr int NW = 8, NT = 64 * NW;
constexpr int STAGES = 3;
constexpr int STAGE_MAX = (BM + BN) * ROWB;  // 48 KB
constexpr int LDS = STAGES * STAGE_MAX;
constexpr int WGM = 4, WGN = 2;              // wave grid
constexpr int WM = BM / WGM, WN = BN / WGN;  // 64 x 64
static_assert(WM == 64 && WN == 64, "two 32-blocks per operand and wave");
static_assert(LDS <= 160 * 1024, "LDS budget");

// Tile kinds: 0 = column block outside the row block (BM + BN rows loaded);
// 1 = column block inside it, c = 2r + 1 (BM rows); 2 = c = 2r, where rows
// past the first BN are wholly below the diagonal (BN rows).
#ifndef GW_STAGES0
#define GW_STAGES0 3
#endif
#ifndef GW_STAGES1
#define GW_STAGES1 3
#endif
#ifndef GW_STAGES2
#define GW_STAGES2 4
#endif
template <int KIND>
struct Cfg {
  static constexpr int ROWS = KIND == 0 ? BM + BN : (KIND == 1 ? BM : BN);
  static constexpr int STAGE = ROWS * ROWB;
  // LDS stages of this kind's chunks in the launch's allocation: the smaller
  // tiles keep more chunks in flight
  static constexpr int STAGES = KIND == 0 ? GW_STAGES0 : (KIND == 1 ? GW_STAGES1 : GW_STAGES2);
  static constexpr int LPC = STAGE / (1024 * NW);  // 1 KB loads per wave per chunk
  static_assert(LPC * 1024 * NW == STAGE, "whole 1 KB loads per wave");
  static_assert(STAGES >= 3 && STAGES * STAGE <= LDS, "stages fit the allocation");
  static_assert(LPC * (STAGES - 2) <= 63, "vmcnt range");
};
}  // namespace gw

struct GwArgs {
  int64_t B, Tn, d, p;
  int has_bias;
  int nbc;     // column blocks: ceil(T / 128)
  int ntiles;  // tiles per sample
};

// Row block r and column block c of tile `tile` (r-major, c from 2r).
__device__ __forceinline__ void gw_tile_rc(int tile, int nbc, int* r, int* c) {
  int rr = 0, rem = tile;
  while (rem >= nbc - 2 * rr) {
    rem -= nbc - 2 * rr;
    ++rr;
  }
  *r = rr;
  *c = 2 * rr + rem;
}

template <int KIND>
__device__ __forceinline__ float gw_item(const bf16s* __restrict__ Ai, const bf16s* __restrict__ Gi, const GwArgs& a,
                                         int r, int c, unsigned char* lds) {
  using C = gw::Cfg<KIND>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // sub-tile (wm, wn) of wave w: (0,0) (0,1) (1,1) (1,0) (2,0) (2,1) (3,0) (3,1). Wave w runs
  // on SIMD w % 4, so the sub-tiles that diagonal tiles keep ((0,0), (0,1), (1,1) for c = 2r,
  // all but (3,0) for c = 2r + 1) sit on different SIMDs where they can.
  const int wm = wave >> 1, wn = (wave & 1) ^ (wm == 1 ? 1 : 0);
  const int64_t row0 = (int64_t)r * gw::BM;       // first Gram row of the tile
  const int64_t col0 = (int64_t)c * gw::BN;       // first Gram column of the tile
  const int toff = KIND == 0 ? gw::BM : (int)(col0 - row0);  // stage row of the column block's first row
  // every entry of the wave's sub-tile has s > t or lies past T: weight 0, nothing to compute
  const int64_t sr0 = row0 + wm * gw::WM, sc0 = col0 + wn * gw::WN;
  const bool idle = sr0 > sc0 + (gw::WN - 1) || sr0 >= a.Tn || sc0 >= a.Tn;
  const int64_t nA = a.d / gw::KC, nG = a.p / gw::KC, n = nA + nG;

  // ---- this lane's 16-byte pieces: load i of the wave covers stage rows
  // R = 8 (wave + 8 i) + lane / 8, slot lane % 8, which holds logical piece
  // slot ^ ((R / 2) % 8) -- the same piece for every i. grow[i] is the Gram
  // row (clamped: rows past T hold finite values and get weight 0).
  const uint32_t piece16 = (uint32_t)(((lane & 7) ^ ((4 * wave + (lane >> 4)) & 7)) * 16);
  uint32_t grow[C::LPC];
#pragma unroll
  for (int i = 0; i < C::LPC; ++i) {
    const int R = 8 * (wave + gw::NW * i) + (lane >> 3);
    int64_t g = R < gw::BM ? row0 + R : col0 + (R - gw::BM);
    if (g > a.Tn - 1) g = a.Tn - 1;
    grow[i] = (uint32_t)g;
  }
  const uint32_t rowbA = (uint32_t)(a.d * 2), rowbG = (uint32_t)(a.p * 2);  // row bytes
  auto issue = [&](int64_t q, int stage) {
    const uint32_t sl = lds_addr(lds) + stage * C::STAGE + wave * 1024;
    const bool inA = q < nA;
    const bf16s* g = inA ? Ai + q * gw::KC : Gi + (q - nA) * gw::KC;
    const uint32_t rowb = inA ? rowbA : rowbG;
#pragma unroll
    for (int i = 0; i < C::LPC; ++i) dma16(g, grow[i] * rowb + piece16, sl + 1024 * gw::NW * i);
  };

  // ---- per-lane LDS read offsets: row j = lane % 32 of a 32-row block,
  // logical piece 2 kk + lane / 32 for k-step kk (16 features); the swizzle
  // term depends on j only (block starts are multiples of 16 rows)
  const int j = lane & 31, h = lane >> 5;
  uint32_t rd[gw::KC / 16];
#pragma unroll
  for (int kk = 0; kk < gw::KC / 16; ++kk) rd[kk] = j * gw::ROWB + (((2 * kk + h) ^ ((j >> 1) & 7)) * 16);
  const int ra0 = wm * gw::WM, rg0 = toff + wn * gw::WN;  // stage rows of the wave's operand blocks

  f32x16 accA[2][2], accG[2][2];
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        accA[bi][bj][e] = 0.f;
        accG[bi][bj][e] = 0.f;
      }

  // The operands of half a chunk (k-steps 2 hh and 2 hh + 1), and its MFMAs.
  struct Half {
    u32x4 a[2][2], b[2][2];
  };
  auto read_half = [&](uint32_t sb, int hh, Half& F) {
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        F.a[k2][b] = *(const lds_u32x4*)(uintptr_t)(sb + rd[2 * hh + k2] + (ra0 + 32 * b) * gw::ROWB);
        F.b[k2][b] = *(const lds_u32x4*)(uintptr_t)(sb + rd[2 * hh + k2] + (rg0 + 32 * b) * gw::ROWB);
      }
  };
  auto mfma_half = [&](const Half& F, f32x16 (&acc)[2][2]) {
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) acc[bi][bj] = mfma32_bf16(F.a[k2][bi], F.b[k2][bj], acc[bi][bj]);
  };
  static_assert(gw::KC == 64, "two halves of two k-steps per chunk");

  // ---- pipeline: chunk q in stage q % S; loads for chunk q+S-1 go out once
  // every wave is past chunk q-1 (the barrier), while chunk q is computed.
  // Two loops (A chunks, then G chunks) so that each body updates one
  // accumulator set.
  constexpr int S = C::STAGES;
  auto step = [&](int64_t q) -> uint32_t {
    // chunks q+1 .. q+S-2 (those issued) may still be in flight
    const int later = n - 1 - q < S - 2 ? (int)(n - 1 - q) : S - 2;
    wait_chunks<C::LPC, S - 2>(later);
    lds_barrier();
    if (q + S - 1 < n) issue(q + S - 1, (int)((q + S - 1) % S));
    return lds_addr(lds) + (uint32_t)((q % S) * C::STAGE);
  };
#pragma unroll
  for (int q = 0; q < S - 1; ++q)
    if (q < n) issue(q, q);
  if (idle) {  // wave-uniform: the wave still loads its share and meets every barrier
    for (int64_t q = 0; q < n; ++q) (void)step(q);
    return 0.0f;
  }
  // Software-pipelined by half chunks: the second half of chunk q is read
  // while the first half's MFMAs run, and the first half of chunk q+1 right
  // after the barrier that makes it visible, while the second half's MFMAs
  // run. n >= 2 (d, p >= 64); the last chunk (of G) is peeled off the loops,
  // so that every path into a half's MFMAs passes the barrier, which waits
  // for this wave's earlier reads, and the compiler's wait insertion does not
  // make them wait for the reads just issued.
  uint32_t sb = step(0);
  Half h0, h1;
  read_half(sb, 0, h0);
  auto body = [&](int64_t q, f32x16 (&acc)[2][2]) {  // chunk q < n - 1
    read_half(sb, 1, h1);
    mfma_half(h0, acc);
    sb = step(q + 1);
    read_half(sb, 0, h0);
    mfma_half(h1, acc);
  };
  for (int64_t q = 0; q < nA; ++q) body(q, accA);
  for (int64_t q = nA; q < n - 1; ++q) body(q, accG);
  read_half(sb, 1, h1);
  mfma_half(h0, accG);
  mfma_half(h1, accG);

  // ---- epilogue: weighted Frobenius product of the tile
  const float one = a.has_bias ? 1.0f : 0.0f;
  const bool above = row0 + gw::BM <= col0 && col0 + gw::BN <= a.Tn;  // every entry s < t < T
  float s = 0.f;
  if (above) {
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int bj = 0; bj < 2; ++bj)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += (accA[bi][bj][e] + one) * accG[bi][bj][e];
    s *= 2.0f;
  } else {
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int bj = 0; bj < 2; ++bj)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t srow = row0 + ra0 + 32 * bi + acc_row(e, lane);
          const int64_t tcol = col0 + wn * gw::WN + 32 * bj + acc_col(lane);
          const float w = (srow >= a.Tn || tcol >= a.Tn || srow > tcol) ? 0.0f : (srow == tcol ? 1.0f : 2.0f);
          s += w * ((accA[bi][bj][e] + one) * accG[bi][bj][e]);
        }
  }
  return s;
}

// One layer of a wide-ghost launch (workgroup range a multiple of 8, first tile in the sink).
struct GwLayer {
  const bf16s* A;
  const bf16s* G;
  GwArgs a;
  int64_t wg_begin;
  int tile_base;
};
struct GwGroup {
  GwLayer L[kNormGroupMax];
  int n;
};

__global__ __launch_bounds__(gw::NT, 1) void k_ghost_wide(GwGroup g, NormSink sink) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char lds[];
  __shared__ float red[gw::NW];
  // the layer whose workgroup range holds this workgroup (uniform choice among compile-time entries)
  GwLayer L = g.L[0];
#pragma unroll
  for (int k = 1; k < kNormGroupMax; ++k)
    if (k < g.n && (int64_t)blockIdx.x >= g.L[k].wg_begin) L = g.L[k];
  const GwArgs& a = L.a;
  int64_t i, tile;
  xcd_group_map((int64_t)blockIdx.x - L.wg_begin, a.ntiles, &i, &tile);
  if (i >= a.B) return;  // whole workgroup, before any barrier
  int r, c;
  gw_tile_rc((int)tile, a.nbc, &r, &c);
  // the sample's bases are wave-uniform; readfirstlane lets them live in SGPRs
  // (the direct-to-LDS loads take a scalar base)
  const bf16s* Ai = uniform_ptr(L.A + i * a.Tn * a.d);
  const bf16s* Gi = uniform_ptr(L.G + i * a.Tn * a.p);
  float s = c >= 2 * r + 2 ? gw_item<0>(Ai, Gi, a, r, c, lds)
            : (c == 2 * r + 1 ? gw_item<1>(Ai, Gi, a, r, c, lds) : gw_item<2>(Ai, Gi, a, r, c, lds));
  s = block_sum<gw::NT>(s, red);
  if (threadIdx.x == 0) norm_sink_tile(sink, i, L.tile_base + tile, s);
}

bool ghost_wide_eligible(int dtype, int64_t Tn, int64_t d, int64_t p) {
  // per-sample byte offsets are 32-bit: T * max(d, p) * 2 < 2^32
  return dtype == 1 && Tn > 64 && d % gw::KC == 0 && p % gw::KC == 0 &&
         Tn * (d > p ? d : p) * 2 < (1ll << 32) - 4096;
}

int64_t ghost_wide_ntiles(int64_t Tn) {
  const int64_t nbc = (Tn + gw::BN - 1) / gw::BN;
  int64_t n = 0;
  for (int64_t r = 0; 2 * r < nbc; ++r) n += nbc - 2 * r;
  return n;
}

// Layers laid out in the grid by decreasing d + p (largest tiles first);
// tile_base follows the caller's order, the order of the sink's fold.
hipError_t launch_ghost_wide_group(hipStream_t st, const GhostLayerDesc* layers, int n, int64_t B,
                                   const NormSink& sink) {
  GwGroup g{};
  int order[kNormGroupMax];
  int base[kNormGroupMax];
  int tb = 0;
  for (int l = 0; l < n; ++l) {
    order[l] = l;
    base[l] = tb;
    tb += (int)ghost_wide_ntiles(layers[l].Tn);
  }
  for (int x = 1; x < n; ++x)  // stable insertion sort by d + p, largest first
    for (int y = x; y > 0 && layers[order[y]].d + layers[order[y]].p > layers[order[y - 1]].d + layers[order[y - 1]].p;
         --y) {
      const int t = order[y];
      order[y] = order[y - 1];
      order[y - 1] = t;
    }
  const int64_t groups8 = (B + 7) / 8;
  int64_t wg = 0;
  for (int k = 0; k < n; ++k) {
    const GhostLayerDesc& x = layers[order[k]];
    GwLayer& L = g.L[k];
    L.A = static_cast<const bf16s*>(x.A);
    L.G = static_cast<const bf16s*>(x.G);
    L.a.B = B;
    L.a.Tn = x.Tn;
    L.a.d = x.d;
    L.a.p = x.p;
    L.a.has_bias = x.has_bias;
    L.a.nbc = (int)((x.Tn + gw::BN - 1) / gw::BN);
    L.a.ntiles = (int)ghost_wide_ntiles(x.Tn);
    L.wg_begin = wg;
    L.tile_base = base[order[k]];
    wg += groups8 * 8 * L.a.ntiles;
  }
  g.n = n;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_ghost_wide),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, gw::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_ghost_wide, dim3((unsigned)wg), dim3(gw::NT), gw::LDS, st, g, sink);
  return hipGetLastError();
}

hipError_t launch_ghost_wide(hipStream_t st, const void* A, const void* G, int64_t B, int64_t Tn, int64_t d,
                             int64_t p, int has_bias, const NormSink& sink) {
  const GhostLayerDesc x{A, G, Tn, d, p, has_bias};
  return launch_ghost_wide_group(st, &x, 1, B, sink);
}

}  // namespace dpk
