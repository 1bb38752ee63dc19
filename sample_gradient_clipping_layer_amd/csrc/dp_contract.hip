// Weighted contraction S = A^T diag(c) G of a bf16 layer, direct-to-LDS engine.
//
// Computes the clipped sum of "Scaling up DP Deep Learning with Fast
// Per-Example Gradient Clipping" (re-weighted loss) and "Scalable and
// Efficient Training of Large CNNs with DP" eq. (2.1) / Sec. 3.2: the sum over
// samples of c_i * A_i^T G_i as ONE contraction over K = B*T rows of the
// flattened [B*T, d] and [B*T, p] views, plus the Gaussian noise and the mean
// in the epilogue.
//
// Eligible layers: bf16, no bias row, T a multiple of 64 (a 64-row K chunk
// never straddles two samples, so one clip factor covers a chunk), d and p
// multiples of 8 (16-byte rows).
//
// gfx950 mapping:
// - Operand chunks [64 k-rows x BM (or BN) features] go from HBM straight to
//   LDS with 16-byte global_load_lds (no staging registers, no VALU), stored
//   row-major [k][feature] with the 16-byte pieces of row r XOR-swizzled by
//   4*(r % 4).
// - MFMA 32x32x16 bf16 operands are read with ds_read_b64_tr_b16: within a
//   16-lane group, the lane at (row k0+j, features f0+4a..f0+4a+3) supplies,
//   and lane 4a+b receives feature f0+4a+b of rows k0..k0+3, i.e. the lane's
//   half of an operand that holds 8 consecutive k of one feature. The swizzle
//   puts the 4 rows x 64 bytes a half-wave reads on 64 distinct banks.
// - Each sample's partial A_i^T G_i is accumulated unscaled in a second set of
//   accumulators and folded in as acc += c_i * partial in fp32: the clip
//   factor is applied exactly.
// - STAGES LDS buffers: loads for chunk q+STAGES-1 are in flight while chunk q
//   is computed; one barrier per chunk.
// - Workgroups are mapped so that each XCD (blockIdx % 8) owns a contiguous
//   range of (split, tile) work items, ordered with the shorter tile dimension
//   fastest, so concurrently running workgroups of one XCD share operand tiles
//   in its L2.
#include "dp_common.hpp"
#include "dp_launch.hpp"
#include "dp_lds.hpp"
#include "dp_noise.hpp"

#include <type_traits>

namespace dpk {


// K rows per chunk and LDS stages of the pipeline
#ifndef DL_KC
#define DL_KC 64
#endif
#ifndef DL_STAGES
#define DL_STAGES 3
#endif
constexpr int kDlKC = DL_KC;
constexpr int kDlStages = DL_STAGES;
static_assert(kDlKC % 16 == 0 && kDlStages >= 3, "chunk of whole MFMA k-steps; at least 3 stages");

template <int BM, int BN, int STAGES, int NW, int KC_ = kDlKC>
struct DlCfg {
  static constexpr int KC = KC_;                  // K rows per chunk
  static constexpr int NT = 64 * NW;              // threads
  static constexpr int RA = BM * 2, RG = BN * 2;  // LDS row bytes
  static constexpr int A_BYTES = KC * RA, G_BYTES = KC * RG;
  static constexpr int STAGE = A_BYTES + G_BYTES;
  static constexpr int LDS = STAGES * STAGE;
  static constexpr int WGM = NW / 2, WGN = 2;     // wave grid
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int NBM = WM / 32, NBN = WN / 32;
  static constexpr int LA = A_BYTES / (1024 * NW);  // 1 KB loads per wave per chunk
  static constexpr int LG = G_BYTES / (1024 * NW);
  static constexpr int LPC = LA + LG;
  static_assert(LA * 1024 * NW == A_BYTES && LG * 1024 * NW == G_BYTES, "whole 1 KB loads per wave");
  static_assert(NBM >= 1 && NBN >= 1 && WM % 32 == 0 && WN % 32 == 0, "32x32 blocks");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(LPC * (STAGES - 2) <= 63, "vmcnt range");
};


// One MFMA operand (8 consecutive k of one feature per lane) from a swizzled
// stage: two transposing reads 4 rows apart. `addr` is an LDS byte address;
// the constant offsets fold into the instructions' offset fields.
__device__ __forceinline__ u32x4 frag_tr(uint32_t addr, int off, int four_rows) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(addr + off));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(addr + off + four_rows));
  u32x4 r;
  r[0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
  r[1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
  r[2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
  r[3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
  return r;
}

// k-steps whose operand reads are grouped ahead of their MFMAs
#ifndef DL_READ_GROUP
#define DL_READ_GROUP 1
#endif
constexpr int kDlReadGroup = DL_READ_GROUP;

struct DlArgs {
  int64_t d, p;
  int64_t cps;              // chunks per sample (T / KC)
  int mt, nt;
  int64_t ks;               // K splits
  int64_t chunks_per_split;
  int64_t nchunks;          // B * T / KC
  int m_fast;               // work-item order: tile row index fastest
  NoiseArgs na;
};



// RATIO (one accumulator set, for wave tiles too large for two): acc holds
// the clipped sum so far divided by the current sample's clip factor; at the
// first chunk of a sample with c_i != 0 it is rescaled by c_prev / c_i, and
// at the end multiplied by the last c. One fp32 rounding per sample instead
// of the exact fold; samples with c_i = 0 contribute exactly nothing and are
// skipped; a NaN factor still propagates. The partial tile is written to the
// workspace straight from registers (FUSED is not used).
template <int BM, int BN, int STAGES, int NW, bool FUSED, int KCK = kDlKC, bool RATIO = false>
__global__ __launch_bounds__(64 * NW, 1) void k_contract_dl(const bf16s* __restrict__ A, const bf16s* __restrict__ G,
                                                            const float* __restrict__ c, float* __restrict__ ws,
                                                            float* __restrict__ out, DlArgs a) {
  using C = DlCfg<BM, BN, STAGES, NW, KCK>;
  static_assert(!(RATIO && FUSED), "the single-accumulator variant writes partials");
  extern __shared__ __attribute__((aligned(1024))) unsigned char lds[];

  // ---- work item (XCD-contiguous)
  const int64_t ntl = (int64_t)a.mt * a.nt;
  const int64_t nitems = ntl * a.ks;
  const int64_t per = (nitems + 7) / 8;
  const int64_t w = (int64_t)(blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (w >= nitems) return;  // whole workgroup, before any barrier
  const int64_t split = w / ntl;
  const int64_t t = w - split * ntl;
  const int tm = a.m_fast ? (int)(t % a.mt) : (int)(t / a.nt);
  const int tn = a.m_fast ? (int)(t / a.mt) : (int)(t % a.nt);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t q0 = split * a.chunks_per_split;
  const int64_t q1 = q0 + a.chunks_per_split < a.nchunks ? q0 + a.chunks_per_split : a.nchunks;
  const int nq = (int)(q1 - q0);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave % C::WGM, wn = wave / C::WGM;

  // ---- per-lane global byte offsets of this lane's 16-byte pieces within a chunk
  // (< KC * max(d, p) * 2 < 2^32)
  uint32_t offA[C::LA], offG[C::LG];
#pragma unroll
  for (int i = 0; i < C::LA; ++i) {
    const int byte = (wave + NW * i) * 1024 + 16 * lane;
    const int r = byte / C::RA, slot = (byte % C::RA) / 16;
    int64_t col = m0 + 8 * (slot ^ (4 * (r & 3)));
    if (col > a.d - 8) col = a.d - 8;  // columns past d only feed unwritten output rows
    offA[i] = (uint32_t)((r * a.d + col) * 2);
  }
#pragma unroll
  for (int i = 0; i < C::LG; ++i) {
    const int byte = (wave + NW * i) * 1024 + 16 * lane;
    const int r = byte / C::RG, slot = (byte % C::RG) / 16;
    int64_t col = n0 + 8 * (slot ^ (4 * (r & 3)));
    if (col > a.p - 8) col = a.p - 8;
    offG[i] = (uint32_t)((r * a.p + col) * 2);
  }

  auto issue = [&](int64_t q, int stage) {
    const bf16s* ga = A + q * (int64_t)C::KC * a.d;
    const bf16s* gg = G + q * (int64_t)C::KC * a.p;
    const uint32_t sa = lds_addr(lds) + stage * C::STAGE + wave * 1024;
    const uint32_t sg = sa + C::A_BYTES;
#pragma unroll
    for (int i = 0; i < C::LA; ++i) dma16(ga, offA[i], sa + 1024 * NW * i);
#pragma unroll
    for (int i = 0; i < C::LG; ++i) dma16(gg, offG[i], sg + 1024 * NW * i);
  };

  // ---- per-lane LDS read offsets (transposing reads)
  const int s = lane & 15;
  const int lo = 2 * ((lane >> 4) & 1) + ((s & 3) >> 1);
  int rdA[C::NBM], rdG[C::NBN];
#pragma unroll
  for (int bi = 0; bi < C::NBM; ++bi) {
    const int piece0 = (wm * C::WM + bi * 32) / 8;
    rdA[bi] = (8 * (lane >> 5) + (s >> 2)) * C::RA + 16 * ((piece0 ^ (4 * (s >> 2))) + lo) + 8 * (s & 1);
  }
#pragma unroll
  for (int bj = 0; bj < C::NBN; ++bj) {
    const int piece0 = (wn * C::WN + bj * 32) / 8;
    rdG[bj] = C::A_BYTES + (8 * (lane >> 5) + (s >> 2)) * C::RG + 16 * ((piece0 ^ (4 * (s >> 2))) + lo) +
              8 * (s & 1);
  }

  // acc: the clipped sum so far; tmp: the current sample segment's unscaled
  // partial (a segment is the part of one sample inside this split), restarted
  // by the segment's first MFMA and folded in as acc += c_i * tmp in fp32 at
  // the segment's last chunk, so the clip factor is applied exactly.
  f32x16 acc[C::NBM][C::NBN];
  f32x16 tmp_[RATIO ? 1 : C::NBM][RATIO ? 1 : C::NBN];
  auto& tmp = [&]() -> auto& {
    if constexpr (RATIO)
      return acc;
    else
      return tmp_;
  }();
#pragma unroll
  for (int bi = 0; bi < C::NBM; ++bi)
#pragma unroll
    for (int bj = 0; bj < C::NBN; ++bj)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[bi][bj][j] = 0.f;

  auto compute = [&](uint32_t sbase, auto fresh) {
    uint32_t ra[C::NBM], rg[C::NBN];
#pragma unroll
    for (int bi = 0; bi < C::NBM; ++bi) ra[bi] = sbase + rdA[bi];
#pragma unroll
    for (int bj = 0; bj < C::NBN; ++bj) rg[bj] = sbase + rdG[bj];
    // operand reads of KG k-steps are issued together, ahead of their MFMAs
    constexpr int KG = kDlReadGroup;
#pragma unroll
    for (int k0 = 0; k0 < C::KC / 16; k0 += KG) {
      u32x4 fa[KG][C::NBM], fg[KG][C::NBN];
#pragma unroll
      for (int kk = 0; kk < KG; ++kk) {
#pragma unroll
        for (int bi = 0; bi < C::NBM; ++bi) fa[kk][bi] = frag_tr(ra[bi], (k0 + kk) * 16 * C::RA, 4 * C::RA);
#pragma unroll
        for (int bj = 0; bj < C::NBN; ++bj) fg[kk][bj] = frag_tr(rg[bj], (k0 + kk) * 16 * C::RG, 4 * C::RG);
      }
      if constexpr (KG > 1) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < KG; ++kk)
#pragma unroll
        for (int bi = 0; bi < C::NBM; ++bi)
#pragma unroll
          for (int bj = 0; bj < C::NBN; ++bj) {
            if (decltype(fresh)::value && k0 + kk == 0)
              tmp[bi][bj] = mfma32_bf16(fa[kk][bi], fg[kk][bj], f32x16{});
            else
              tmp[bi][bj] = mfma32_bf16(fa[kk][bi], fg[kk][bj], tmp[bi][bj]);
          }
    }
  };

  // ---- pipeline: chunk q in stage q % STAGES; loads for chunk it+STAGES-1
  // go out once every wave is past chunk it-1 (the barrier), while chunk it
  // is computed.
  int64_t sample = q0 / a.cps;
  int64_t in_sample = q0 - sample * a.cps;
  float cur = 0.0f, prev = 0.0f;  // RATIO: current and last nonzero clip factor
  bool have_prev = false;
#pragma unroll
  for (int c = 0; c < STAGES - 1; ++c)
    if (c < nq) issue(q0 + c, c);
  for (int it = 0; it < nq; ++it) {
    // chunks it+1 .. it+STAGES-2 (those issued) may still be in flight
    const int later = nq - 1 - it < STAGES - 2 ? nq - 1 - it : STAGES - 2;
    wait_chunks<C::LPC, STAGES - 2>(later);
    lds_barrier();  // chunk it landed for every wave; every wave is done with chunk it-1
    if (it + STAGES - 1 < nq) issue(q0 + it + STAGES - 1, (it + STAGES - 1) % STAGES);

    const uint32_t sb = lds_addr(lds) + (uint32_t)((it % STAGES) * C::STAGE);
    if constexpr (RATIO) {
      if (it == 0 || in_sample == 0) {
        cur = c[sample];
        if (cur != 0.0f) {  // a NaN factor is not 0: it propagates
          if (have_prev) {
            const float r = prev / cur;
#pragma unroll
            for (int bi = 0; bi < C::NBM; ++bi)
#pragma unroll
              for (int bj = 0; bj < C::NBN; ++bj)
#pragma unroll
                for (int j = 0; j < 16; ++j) acc[bi][bj][j] *= r;
          }
          prev = cur;
          have_prev = true;
        }
      }
      if (cur != 0.0f) compute(sb, std::false_type{});
      if (++in_sample == a.cps) {
        in_sample = 0;
        ++sample;
      }
      continue;
    } else {
      if (it == 0 || in_sample == 0)
        compute(sb, std::true_type{});
      else
        compute(sb, std::false_type{});
    }
    if (++in_sample == a.cps || it + 1 == nq) {
      const float ci = c[sample];
#pragma unroll
      for (int bi = 0; bi < C::NBM; ++bi)
#pragma unroll
        for (int bj = 0; bj < C::NBN; ++bj)
#pragma unroll
          for (int j = 0; j < 16; ++j) acc[bi][bj][j] = __builtin_fmaf(ci, tmp[bi][bj][j], acc[bi][bj][j]);
      if (in_sample == a.cps) {
        in_sample = 0;
        ++sample;
      }
    }
  }

  if constexpr (RATIO) {
    // ---- epilogue: undo the last sample's division and write the partial
    // tile [m][n] (m < d, n < p) straight from the accumulators
    const float last = have_prev ? prev : 0.0f;
    float* wsp = ws + split * a.d * a.p;
#pragma unroll
    for (int bi = 0; bi < C::NBM; ++bi)
#pragma unroll
      for (int bj = 0; bj < C::NBN; ++bj)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int64_t m = m0 + wm * C::WM + bi * 32 + acc_row(j, lane);
          const int64_t n = n0 + wn * C::WN + bj * 32 + acc_col(lane);
          if (m < a.d && n < a.p) wsp[m * a.p + n] = have_prev ? acc[bi][bj][j] * last : 0.0f;
        }
    return;
  } else {
  // ---- epilogue: the output tile goes through LDS ([BM][BN + 8] fp32; the
  // stages are free once every wave passed the barrier), then each thread
  // takes whole Philox blocks (4 rows of one column) or float4 row pieces,
  // with consecutive threads on consecutive columns.
  constexpr int TP = BN + 8;
  static_assert(BM * TP * 4 <= C::LDS, "epilogue tile fits the stages");
  float* tile = reinterpret_cast<float*>(lds);
  lds_barrier();
#pragma unroll
  for (int bi = 0; bi < C::NBM; ++bi)
#pragma unroll
    for (int bj = 0; bj < C::NBN; ++bj)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        tile[(wm * C::WM + bi * 32 + acc_row(j, lane)) * TP + wn * C::WN + bj * 32 + acc_col(lane)] = acc[bi][bj][j];
  lds_barrier();
  if constexpr (FUSED) {
#pragma unroll 1
    for (int b = threadIdx.x; b < (BM / 4) * BN; b += C::NT) {
      const int rq = b / BN, nn = b % BN;
      const int64_t m = m0 + 4 * rq, n = n0 + nn;
      if (m >= a.d || n >= a.p) continue;
      const f32x4 z = normals4((uint32_t)((m >> 2) * a.p + n), 2u * a.na.layer, a.na.step, 0u, a.na.k0, a.na.k1);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (m + r < a.d)
          out[(m + r) * a.p + n] = noised_mean_spec(tile[(4 * rq + r) * TP + nn], a.na.sc, z[r], a.na.inv_denom);
    }
  } else {
    float* wsp = ws + split * a.d * a.p;
#pragma unroll 1
    for (int e = threadIdx.x; e < BM * (BN / 4); e += C::NT) {
      const int row = e / (BN / 4), c4 = e % (BN / 4);
      const int64_t m = m0 + row, n = n0 + 4 * c4;
      if (m >= a.d || n >= a.p) continue;
      const float4 v = *reinterpret_cast<const float4*>(tile + row * TP + 4 * c4);
      // p % 8 == 0 and n % 4 == 0: the four columns are all in range and 16-byte aligned
      *reinterpret_cast<float4*>(wsp + m * a.p + n) = v;
    }
  }
  }
}

// ---------------------------------------------------------------- plan
bool dl_eligible(int dtype, int64_t B, int64_t Tn, int64_t d, int64_t p, int has_bias) {
  (void)B;
  return dtype == 1 && !has_bias && Tn % kDlKC == 0 && d % 8 == 0 && p % 8 == 0 &&
         kDlKC * (d > p ? d : p) < (1ll << 31);
}

// Tile and K split for the direct-load engine from a cost model: rounds of
// one workgroup per CU (256 CUs) x the chunks each item runs at a per-CU
// MFMA rate that grows with the tile (fewer LDS bytes per flop), plus the
// write and re-read of split partials and a reduce launch.
// The 256 x 256 tile (64 x 128 wave tiles, single accumulator set) streams
// 32-row chunks through four stages and always writes partials.
constexpr int kDlWideKC = 32, kDlWideStages = 4;

// Tile and K split from a cost model fitted to MI355X measurements of this
// engine: rounds of one workgroup per CU (256 CUs) x (the item's chunks at a
// sustained fraction of the bf16 MFMA peak + a fixed cost per item: fill and
// the partial tile's write), plus the write and re-read of split partials by
// the reduce kernel and its launch.
ContractPlan dl_plan(int64_t B, int64_t Tn, int64_t d, int64_t p) {
  static const int tiles[3][2] = {{128, 128}, {256, 128}, {256, 256}};
  static const double eff[3] = {0.30, 0.35, 0.47};        // of the bf16 peak, in the K loop
  static const double fixed_s[3] = {6e-6, 8e-6, 13.5e-6};  // per item
  static const int kcs[3] = {kDlKC, kDlKC, kDlWideKC};
  const double cu_peak = 2.5e15 / 256.0;
  ContractPlan best{};
  double best_t = 1e300;
  for (int ti = 0; ti < 3; ++ti) {
    const int bm = tiles[ti][0], bn = tiles[ti][1];
    const bool wide = bn == 256;
    if (Tn % kcs[ti] != 0) continue;
    const int64_t nchunks = B * Tn / kcs[ti];
    const int64_t mt = (d + bm - 1) / bm, nt = (p + bn - 1) / bn;
    const double chunk_s = 2.0 * bm * bn * kcs[ti] / (cu_peak * eff[ti]);
    const int64_t ks_max = nchunks < 512 ? nchunks : 512;
    for (int64_t ks = 1; ks <= ks_max; ++ks) {
      const int64_t cpsplit = (nchunks + ks - 1) / ks;
      if ((nchunks + cpsplit - 1) / cpsplit != ks) continue;
      // the wide tile pays off with long K ranges per item; on short ones its
      // larger partial tiles cost more than the model sees once other
      // layers' calls run beside it
      if (wide && cpsplit < 64) continue;
      const int64_t items = mt * nt * ks;
      const double rounds = (double)((items + 255) / 256);
      double t = rounds * ((double)cpsplit * chunk_s + fixed_s[ti]);
      if (ks > 1 || wide) t += (2.0 * ks + 1.0) * (double)d * (double)p * 4.0 / 8.0e12 + 4.0e-6;
      if (t < best_t * 0.999) {
        best_t = t;
        best.bm = bm;
        best.bn = bn;
        best.mt = (int)mt;
        best.nt = (int)nt;
        best.ks = ks;
        best.units_per_split = cpsplit;
        best.partials = wide ? 1 : 0;
      }
    }
  }
  best.engine = 1;
  return best;
}

// ---------------------------------------------------------------- launch
struct DlPtrs {
  const bf16s* A;
  const bf16s* G;
  const float* c;
  float* ws;
  float* out;
};

template <int BM, int BN, int NW>
static hipError_t launch_dl_t(hipStream_t st, const DlPtrs& P, const DlArgs& a, int64_t items) {
  constexpr int S = kDlStages;
  using C = DlCfg<BM, BN, S, NW>;
  const int64_t per = (items + 7) / 8;
  const dim3 grid((unsigned)(per * 8));
  // more than 64 KB of dynamic LDS must be allowed per kernel (per call:
  // cheap, and correct whichever device is current)
  if (a.ks == 1) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_contract_dl<BM, BN, S, NW, true>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_contract_dl<BM, BN, S, NW, true>), grid, dim3(C::NT), C::LDS, st, P.A, P.G, P.c, P.ws, P.out, a);
  } else {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_contract_dl<BM, BN, S, NW, false>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_contract_dl<BM, BN, S, NW, false>), grid, dim3(C::NT), C::LDS, st, P.A, P.G, P.c, P.ws, P.out, a);
  }
  return hipGetLastError();
}

hipError_t launch_contract_dl(hipStream_t st, const void* A, const void* G, const float* c, int64_t B, int64_t Tn,
                              int64_t d, int64_t p, const ContractPlan& pl, float* ws, const NoiseArgs& na,
                              float* out) {
  const DlPtrs P{static_cast<const bf16s*>(A), static_cast<const bf16s*>(G), c, ws, out};
  const bool wide = pl.bn == 256;
  const int kc = wide ? kDlWideKC : kDlKC;
  DlArgs a;
  a.d = d;
  a.p = p;
  a.cps = Tn / kc;
  a.mt = pl.mt;
  a.nt = pl.nt;
  a.ks = pl.ks;
  a.chunks_per_split = pl.units_per_split;
  a.nchunks = B * Tn / kc;
  a.m_fast = pl.mt <= pl.nt ? 1 : 0;
  a.na = na;
  const int64_t items = (int64_t)pl.mt * pl.nt * pl.ks;
  if (wide) {
    constexpr int S = kDlWideStages, KCW = kDlWideKC;
    using C = DlCfg<256, 256, S, 8, KCW>;
    const int64_t per = (items + 7) / 8;
    const dim3 grid((unsigned)(per * 8));
    auto kern = &k_contract_dl<256, 256, S, 8, false, KCW, true>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(C::NT), C::LDS, st, P.A, P.G, P.c, P.ws, P.out, a);
    return hipGetLastError();
  }
  if (pl.bm == 128 && pl.bn == 128) return launch_dl_t<128, 128, 8>(st, P, a, items);
  return launch_dl_t<256, 128, 8>(st, P, a, items);
}

}  // namespace dpk
