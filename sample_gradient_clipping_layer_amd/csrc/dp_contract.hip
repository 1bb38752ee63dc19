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
// - 128x128 and 256x128 tiles: each sample's partial A_i^T G_i is accumulated
//   unscaled in a second set of accumulators and folded in as
//   acc += c_i * partial in fp32 (the clip factor applied exactly). 256x256
//   tiles keep one set and rescale it by c_prev / c_i at each sample (one
//   more fp32 rounding per sample; see RATIO below).
// - STAGES LDS buffers: loads for chunk q+STAGES-1 are in flight while chunk q
//   is computed; one barrier per chunk. The 256x256 tile (two k-steps per
//   chunk) reads the next chunk's first k-step right after that chunk's
//   barrier, while this chunk's second k-step runs on the matrix cores.
// - One launch takes up to kDlGroupMax layers (one tile shape, a K split per
//   layer). Each XCD (blockIdx % 8) owns a contiguous range of every layer's
//   (split, tile) work items, ordered with the shorter tile dimension fastest,
//   so concurrently running workgroups of one XCD share operand tiles in its
//   L2.
// - A split output tile (or any 256x256 tile) leaves its partial in the
//   workspace; the reduce kernel adds the partials in split order and applies
//   the noise and the mean.
#include "dp_common.hpp"
#include "dp_launch.hpp"
#include "dp_lds.hpp"
#include "dp_noise.hpp"
#include "dp_reduce.hpp"

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

// One layer of a contraction launch.
struct DlLayer {
  const bf16s* A;
  const bf16s* G;
  float* ws;                  // partial tiles [ks][d][p] (when ks > 1 or the tile always writes partials)
  float* out;
  int64_t d, p;
  int64_t cps;                // chunks per sample (T / KC)
  int64_t ks;                 // K splits
  int64_t chunks_per_split;
  int64_t nchunks;            // B * T / KC
  int64_t per;                // work items per XCD: ceil(mt * nt * ks / 8)
  int mt, nt;
  int m_fast;                 // work-item order: tile row index fastest
  NoiseArgs na;
};
// The layers of one launch, in dispatch order, and the tail work: the split
// reduce of the previous launch of the same call, which the workgroups past
// the work items (ids >= wgs_main) run on the CUs that the last round of
// items leaves idle.
struct DlGroup {
  DlLayer L[kDlGroupMax];
  int n;
  int64_t wgs_main;
  int64_t tail_blocks;  // 256-thread blocks of the tail reduce (0: none)
  RedGroup tail;
};

// RATIO (one accumulator set, for wave tiles too large for two): acc holds
// the clipped sum so far divided by the current sample's clip factor; at the
// first chunk of a sample with c_i != 0 it is rescaled by c_prev / c_i, and
// at the end multiplied by the last c. One fp32 rounding per sample instead
// of the exact fold; samples with c_i = 0 contribute exactly nothing and are
// skipped; a NaN factor still propagates. The partial tile is written to the
// workspace straight from registers.
//
// The units of acc must not drift far from the factors it holds: were a
// factor 2^-100 to follow factors near 1, acc = sum / c_i would overflow. So
// when c_i lies outside [ref * 2^-32, ref * 2^32], ref being the factor of
// the first sample since the last such event, acc * c_prev is flushed into
// this split's partial tile in the workspace (added to what earlier flushes
// left there; each lane owns its elements) and acc restarts from zero with
// ref = c_i. Within the window the rescale factor is at most 2^32 and every
// term of acc is c_j * P_j / c_i with c_j / c_i <= 2^64 (P_j the unscaled
// per-sample product), which stays finite for clipped terms |c_j P_j| <= C
// whenever C / c_i does. The epilogue adds the flushed part first.
//
// Work items: XCD x (blockIdx % 8) takes items [x * per_l, (x+1) * per_l) of
// every layer l in turn, so that each XCD holds a share of every layer and
// its concurrently running workgroups share operand tiles in its L2.
template <int BM, int BN, int STAGES, int NW, int KCK = kDlKC, bool RATIO = false>
__global__ __launch_bounds__(64 * NW, 1) void k_contract_dl(const float* __restrict__ c, DlGroup g) {
  using C = DlCfg<BM, BN, STAGES, NW, KCK>;
  extern __shared__ __attribute__((aligned(1024))) unsigned char lds[];

  // ---- tail workgroups: the previous launch's split reduce, two 256-thread
  // blocks per pass, blocks strided over the tail workgroups
  if ((int64_t)blockIdx.x >= g.wgs_main) {
    const int64_t ntail = (int64_t)gridDim.x - g.wgs_main, e = (int64_t)blockIdx.x - g.wgs_main;
    const int64_t half = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8);
    const int tid = threadIdx.x & 255;
    for (int64_t vb = 2 * e + half; vb < g.tail_blocks; vb += 2 * ntail) {
      int k = 0;
#pragma unroll
      for (int j = 1; j < kDlGroupMax; ++j)
        if (j < g.tail.n && vb >= g.tail.blk_begin[j]) k = j;
      const SplitReduceLayer R = g.tail.L[k];
      const int64_t nc = R.p / 4, nw = (R.d / 4) * nc;
      const int64_t t = (vb - g.tail.blk_begin[k]) * 256 + tid;
      if (t < nw) reduce_noise_block4(R.ws, R.ks, R.p, R.d * R.p, t / nc, t % nc, R.na, R.out);
    }
    return;  // whole workgroup, no barrier
  }

  // ---- layer and work item
  const int64_t xcd = blockIdx.x & 7;
  const int64_t local = blockIdx.x >> 3;
  int li = -1;
  int64_t first = 0, acc_per = 0;
#pragma unroll
  for (int k = 0; k < kDlGroupMax; ++k)
    if (k < g.n && li < 0) {
      if (local < acc_per + g.L[k].per) {
        li = k;
        first = acc_per;
      }
      acc_per += g.L[k].per;
    }
  if (li < 0) return;  // whole workgroup, before any barrier
  DlLayer L = g.L[0];
#pragma unroll
  for (int k = 1; k < kDlGroupMax; ++k)
    if (k == li) L = g.L[k];
  const bf16s* __restrict__ A = L.A;
  const bf16s* __restrict__ G = L.G;
  const int64_t ntl = (int64_t)L.mt * L.nt;
  const int64_t w = xcd * L.per + (local - first);
  if (w >= ntl * L.ks) return;
  const int64_t split = w / ntl;
  const int64_t t = w - split * ntl;
  const int tm = L.m_fast ? (int)(t % L.mt) : (int)(t / L.nt);
  const int tn = L.m_fast ? (int)(t / L.mt) : (int)(t % L.nt);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t q0 = split * L.chunks_per_split;
  const int64_t q1 = q0 + L.chunks_per_split < L.nchunks ? q0 + L.chunks_per_split : L.nchunks;
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
    if (col > L.d - 8) col = L.d - 8;  // columns past d only feed unwritten output rows
    offA[i] = (uint32_t)((r * L.d + col) * 2);
  }
#pragma unroll
  for (int i = 0; i < C::LG; ++i) {
    const int byte = (wave + NW * i) * 1024 + 16 * lane;
    const int r = byte / C::RG, slot = (byte % C::RG) / 16;
    int64_t col = n0 + 8 * (slot ^ (4 * (r & 3)));
    if (col > L.p - 8) col = L.p - 8;
    offG[i] = (uint32_t)((r * L.p + col) * 2);
  }

  auto issue = [&](int64_t q, int stage) {
    const bf16s* ga = A + q * (int64_t)C::KC * L.d;
    const bf16s* gg = G + q * (int64_t)C::KC * L.p;
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

  // RATIO: one k-step's operands of the chunk in stage base sbase, and its MFMAs
  struct Frags {
    u32x4 a[C::NBM], g[C::NBN];
  };
  auto read_kstep = [&](uint32_t sbase, int k, Frags& f) {
#pragma unroll
    for (int bi = 0; bi < C::NBM; ++bi) f.a[bi] = frag_tr(sbase + rdA[bi], k * 16 * C::RA, 4 * C::RA);
#pragma unroll
    for (int bj = 0; bj < C::NBN; ++bj) f.g[bj] = frag_tr(sbase + rdG[bj], k * 16 * C::RG, 4 * C::RG);
  };
  auto mfma_kstep = [&](const Frags& f) {
#pragma unroll
    for (int bi = 0; bi < C::NBM; ++bi)
#pragma unroll
      for (int bj = 0; bj < C::NBN; ++bj) acc[bi][bj] = mfma32_bf16(f.a[bi], f.g[bj], acc[bi][bj]);
  };

  // ---- pipeline: chunk q in stage q % STAGES; loads for chunk it+STAGES-1
  // go out once every wave is past chunk it-1 (the barrier), while chunk it
  // is computed.
  int64_t sample = q0 / L.cps;
  int64_t in_sample = q0 - sample * L.cps;
  float cur = 0.0f, prev = 0.0f;  // RATIO: current and last nonzero clip factor
  float ref = 0.0f;               // RATIO: factor of the first sample since the last flush
  bool have_prev = false, flushed = false;
  // RATIO: acc element (bi, bj, j) of this lane sits at row lrow + bi*32 + 8*(j/4) + j%4
  // and column lcol + bj*32 of the split's partial tile; `f(elem, ptr)` is called for the
  // elements inside [0, d) x [0, p) (flushes and the epilogue; the offsets past the lane's
  // base are compile-time constants times p).
  auto for_tile_elems = [&](auto f) {
    // an opaque copy of the row stride: the element addresses are formed where
    // they are used instead of being computed ahead of the (rare) flushes and
    // held in registers through the whole K loop
    int64_t ps = L.p;
    asm volatile("" : "+s"(ps));
    const int64_t lrow = m0 + wm * C::WM + 4 * (lane >> 5), lcol = n0 + wn * C::WN + (lane & 31);
    float* const base = L.ws + split * L.d * ps + lrow * ps + lcol;
    const int64_t rem_r = L.d - lrow, rem_c = L.p - lcol;
#pragma unroll
    for (int bi = 0; bi < C::NBM; ++bi)
#pragma unroll
      for (int bj = 0; bj < C::NBN; ++bj)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int ro = bi * 32 + 8 * (j >> 2) + (j & 3), co = bj * 32;
          if (ro < rem_r && co < rem_c) f(acc[bi][bj][j], base + ro * ps + co);
        }
  };
#pragma unroll
  for (int c = 0; c < STAGES - 1; ++c)
    if (c < nq) issue(q0 + c, c);
  if constexpr (RATIO) {
    // Two k-steps per chunk, software-pipelined across chunks: chunk it+1's
    // first k-step is read right after the barrier that makes it visible,
    // while chunk it's second k-step runs on the matrix cores. The barrier
    // for chunk it+1 also finds every wave done reading chunk it, whose stage
    // then takes the loads of chunk it+STAGES.
    static_assert(C::KC == 32, "two k-steps per chunk");
    auto stage_of = [&](int it) { return lds_addr(lds) + (uint32_t)((it % STAGES) * C::STAGE); };
    auto arrive = [&](int it) {  // chunk it landed for every wave; issue chunk it + STAGES - 1
      const int later = nq - 1 - it < STAGES - 2 ? nq - 1 - it : STAGES - 2;
      wait_chunks<C::LPC, STAGES - 2>(later);
      lds_barrier();
      if (it + STAGES - 1 < nq) issue(q0 + it + STAGES - 1, (it + STAGES - 1) % STAGES);
    };
    // The last chunk is peeled off the loop, so that every path into the
    // second k-step's MFMAs passes the barrier, which waits for this wave's
    // reads: the compiler's wait insertion then tracks only the next chunk's
    // first-k-step reads as pending there, and the MFMAs do not wait for them.
    auto begin_chunk = [&](int it) {  // the chunk's clip factor: rescale (or flush) at a sample's start
      if (it == 0 || in_sample == 0) {
        cur = c[sample];
        if (cur != 0.0f) {  // a NaN factor is not 0: it propagates
          if (have_prev) {
            const float mag = fabsf(cur), rmag = fabsf(ref);
            float r;
            if (mag < rmag * 0x1p-32f || mag > rmag * 0x1p32f) {
              // flush: partial tile (+)= acc * c_prev; acc restarts (times 0) in units of c_i
              for_tile_elems([&](float a, float* dst) {
                const float v = a * prev;
                *dst = flushed ? *dst + v : v;
              });
              flushed = true;
              ref = cur;
              r = 0.0f;
            } else {
              r = prev / cur;
            }
#pragma unroll
            for (int bi = 0; bi < C::NBM; ++bi)
#pragma unroll
              for (int bj = 0; bj < C::NBN; ++bj)
#pragma unroll
                for (int j = 0; j < 16; ++j) acc[bi][bj][j] *= r;
          } else {
            ref = cur;
          }
          prev = cur;
          have_prev = true;
        }
      }
    };
    auto end_chunk = [&]() {
      if (++in_sample == L.cps) {
        in_sample = 0;
        ++sample;
      }
    };
    Frags f0, f1;
    if (nq > 0) {
      arrive(0);
      read_kstep(stage_of(0), 0, f0);
    }
    for (int it = 0; it + 1 < nq; ++it) {
      begin_chunk(it);
      read_kstep(stage_of(it), 1, f1);
      if (cur != 0.0f) mfma_kstep(f0);
      arrive(it + 1);  // also: this wave's reads of chunk it are done (lgkmcnt)
      read_kstep(stage_of(it + 1), 0, f0);
      if (cur != 0.0f) mfma_kstep(f1);
      end_chunk();
    }
    if (nq > 0) {
      begin_chunk(nq - 1);
      read_kstep(stage_of(nq - 1), 1, f1);
      if (cur != 0.0f) {
        mfma_kstep(f0);
        mfma_kstep(f1);
      }
      end_chunk();
    }
  } else
  for (int it = 0; it < nq; ++it) {
    // chunks it+1 .. it+STAGES-2 (those issued) may still be in flight
    const int later = nq - 1 - it < STAGES - 2 ? nq - 1 - it : STAGES - 2;
    wait_chunks<C::LPC, STAGES - 2>(later);
    lds_barrier();  // chunk it landed for every wave; every wave is done with chunk it-1
    if (it + STAGES - 1 < nq) issue(q0 + it + STAGES - 1, (it + STAGES - 1) % STAGES);

    const uint32_t sb = lds_addr(lds) + (uint32_t)((it % STAGES) * C::STAGE);
    if (it == 0 || in_sample == 0)
      compute(sb, std::true_type{});
    else
      compute(sb, std::false_type{});
    if (++in_sample == L.cps || it + 1 == nq) {
      const float ci = c[sample];
#pragma unroll
      for (int bi = 0; bi < C::NBM; ++bi)
#pragma unroll
        for (int bj = 0; bj < C::NBN; ++bj)
#pragma unroll
          for (int j = 0; j < 16; ++j) acc[bi][bj][j] = __builtin_fmaf(ci, tmp[bi][bj][j], acc[bi][bj][j]);
      if (in_sample == L.cps) {
        in_sample = 0;
        ++sample;
      }
    }
  }

  if constexpr (RATIO) {
    // ---- epilogue: undo the last sample's division, write the partial tile
    // [m][n] (m < d, n < p) straight from the accumulators (for the reduce)
    const float last = have_prev ? prev : 0.0f;
    for_tile_elems([&](float a, float* dst) {
      const float v = have_prev ? a * last : 0.0f;
      *dst = flushed ? *dst + v : v;
    });
    return;
  } else {
  // ---- epilogue: the output tile goes through LDS ([BM][BN + 8] fp32; the
  // stages are free once every wave passed the barrier). With one K split the
  // noise and the mean are applied here: each thread takes whole Philox
  // blocks (4 rows of one column), consecutive threads on consecutive
  // columns. Otherwise the partial tile goes to ws[split] (16-byte pieces
  // of consecutive columns) for the reduce kernel.
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
  if (L.ks == 1) {
#pragma unroll 1
    for (int b = threadIdx.x; b < (BM / 4) * BN; b += C::NT) {
      const int rq = b / BN, nn = b % BN;
      const int64_t m = m0 + 4 * rq, n = n0 + nn;
      if (m >= L.d || n >= L.p) continue;
      const f32x4 z = normals4((uint32_t)((m >> 2) * L.p + n), 2u * L.na.layer, L.na.step, 0u, L.na.k0, L.na.k1);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (m + r < L.d)
          L.out[(m + r) * L.p + n] = noised_mean_spec(tile[(4 * rq + r) * TP + nn], L.na.sc, z[r], L.na.inv_denom);
    }
    return;
  }
  float* wsp = L.ws + split * L.d * L.p;
#pragma unroll 1
  for (int e = threadIdx.x; e < BM * (BN / 4); e += C::NT) {
    const int row = e / (BN / 4), c4 = e % (BN / 4);
    const int64_t m = m0 + row, n = n0 + 4 * c4;
    if (m >= L.d || n >= L.p) continue;
    // p % 8 == 0 and n % 4 == 0: the four columns are all in range and 16-byte aligned
    *reinterpret_cast<float4*>(wsp + m * L.p + n) = *reinterpret_cast<const float4*>(tile + row * TP + 4 * c4);
  }
  }
}

// ---------------------------------------------------------------- plan
bool dl_eligible(int dtype, int64_t B, int64_t Tn, int64_t d, int64_t p, int has_bias) {
  (void)B;
  return dtype == 1 && !has_bias && Tn % kDlKC == 0 && d % 8 == 0 && p % 8 == 0 &&
         kDlKC * (d > p ? d : p) < (1ll << 31);
}

// The 256 x 256 tile (64 x 128 wave tiles, single accumulator set) streams
// 32-row chunks through four stages and always writes partials.
constexpr int kDlWideKC = 32, kDlWideStages = 4;

// tiles the planner may choose (bit i: kTileBM/kTileBN[i])
#ifndef DL_TILE_MASK
#define DL_TILE_MASK 7
#endif

namespace {
constexpr int kTiles = 3;
const int kTileBM[kTiles] = {128, 256, 256}, kTileBN[kTiles] = {128, 128, 256};
const int kTileKC[kTiles] = {kDlKC, kDlKC, kDlWideKC};
// Cost model fitted to MI355X measurements of this engine: a work item runs
// its chunks at a sustained fraction of the bf16 MFMA peak of one CU, plus a
// fixed cost (pipeline fill, epilogue); one workgroup per CU (LDS). Split
// tiles cost the reduce kernel that follows the launch: it reads every
// partial and writes the output.
const double kTileEff[kTiles] = {0.30, 0.35, 0.47};
const double kTileFixed[kTiles] = {6e-6, 8e-6, 13.5e-6};
constexpr double kCuPeak = 2.5e15 / 256.0;
constexpr int kCusPerXcd = 32;

struct LayerChoice {
  int64_t ks, cps, mt, nt, per;
  double item_s, reduce_s;
};

// Split of one layer into items of about `target` chunks; false when the
// tile cannot take it.
bool choose_split(int ti, int64_t B, int64_t Tn, int64_t d, int64_t p, int64_t target, LayerChoice* o) {
  const int kc = kTileKC[ti];
  if (Tn % kc != 0) return false;
  const int64_t nchunks = B * Tn / kc;
  int64_t ks = (nchunks + target - 1) / target;
  if (ks < 1) ks = 1;
  if (ks > 512) ks = 512;
  const int64_t cps = (nchunks + ks - 1) / ks;
  ks = (nchunks + cps - 1) / cps;
  if (kTileBN[ti] == 256 && cps < 64) return false;  // the wide tile needs long K ranges per item
  o->ks = ks;
  o->cps = cps;
  o->mt = (d + kTileBM[ti] - 1) / kTileBM[ti];
  o->nt = (p + kTileBN[ti] - 1) / kTileBN[ti];
  o->per = (o->mt * o->nt * ks + 7) / 8;
  const double chunk_s = 2.0 * kTileBM[ti] * kTileBN[ti] * kc / (kCuPeak * kTileEff[ti]);
  const bool partials = ks > 1 || kTileBN[ti] == 256;
  o->item_s = (double)cps * chunk_s + kTileFixed[ti];
  // the reduce kernel writes the output after reading every partial
  o->reduce_s = partials ? (2.0 * ks + 1.0) * (double)d * (double)p * 4.0 / 8.0e12 + 4.0e-6 : 0.0;
  return true;
}

// Makespan of one XCD's share (the first XCD holds the most): its 32 CUs
// take the items in dispatch order, each as soon as one is free. A layer's
// items are alike: whole rounds go to every CU, the rest to the least loaded
// (the loads stay sorted: two sorted runs merged).
double xcd_makespan(const LayerChoice* ch, const int* order, int n) {
  double cu[kCusPerXcd] = {}, nx[kCusPerXcd];  // ascending
  for (int k = 0; k < n; ++k) {
    const LayerChoice& x = ch[order[k]];
    const int64_t full = x.per / kCusPerXcd;
    const int rem = (int)(x.per % kCusPerXcd);
    const double add = (double)full * x.item_s;
    int i = rem, j = 0, o = 0;  // run 1: cu[rem..] + add; run 2: cu[..rem) + add + item
    while (o < kCusPerXcd) {
      const bool take1 = j >= rem || (i < kCusPerXcd && cu[i] <= cu[j] + x.item_s);
      nx[o++] = take1 ? cu[i++] + add : cu[j++] + add + x.item_s;
    }
    for (int u = 0; u < kCusPerXcd; ++u) cu[u] = nx[u];
  }
  return cu[kCusPerXcd - 1];
}
}  // namespace

// Tile (shared by the launch) and per-layer K splits: over the three tiles
// and a range of target item lengths, the smallest simulated makespan.
// Layers go in dispatch order by decreasing item time.
DlGroupPlan dl_group_plan(const int64_t* B, const int64_t* Tn, const int64_t* d, const int64_t* p, int n) {
  static const int64_t targets[] = {4, 6, 8, 12, 16, 24, 32, 48, 64, 96, 128, 192, 256, 384, 512, 768, 1024,
                                    1536, 2048, 4096, 8192, 1ll << 40};
  DlGroupPlan best{};
  best.n = 0;
  double best_t = 1e300;
  for (int ti = 0; ti < kTiles; ++ti) {
    if (!((DL_TILE_MASK >> ti) & 1)) continue;
    int64_t prev_ks[kDlGroupMax] = {};
    for (int64_t target : targets) {
      LayerChoice ch[kDlGroupMax];
      bool ok = true;
      for (int l = 0; l < n && ok; ++l) ok = choose_split(ti, B[l], Tn[l], d[l], p[l], target, &ch[l]);
      if (!ok) continue;
      bool same = true;  // the splits of the previous target: nothing new
      for (int l = 0; l < n; ++l) {
        same = same && ch[l].ks == prev_ks[l];
        prev_ks[l] = ch[l].ks;
      }
      if (same) continue;
      int order[kDlGroupMax];
      for (int l = 0; l < n; ++l) order[l] = l;
      for (int a = 1; a < n; ++a)  // stable, by decreasing item time
        for (int b = a; b > 0 && ch[order[b]].item_s > ch[order[b - 1]].item_s; --b) {
          const int tmp = order[b];
          order[b] = order[b - 1];
          order[b - 1] = tmp;
        }
      double t = xcd_makespan(ch, order, n);
      for (int l = 0; l < n; ++l) t += ch[l].reduce_s;
      if (t < best_t * 0.999) {
        best_t = t;
        best.n = n;
        best.bm = kTileBM[ti];
        best.bn = kTileBN[ti];
        best.kc = kTileKC[ti];
        best.seconds = t;
        for (int l = 0; l < n; ++l) {
          best.ks[l] = ch[l].ks;
          best.cps[l] = ch[l].cps;
          best.mt[l] = (int)ch[l].mt;
          best.nt[l] = (int)ch[l].nt;
          best.order[l] = order[l];
        }
      }
    }
  }
  return best;
}

ContractPlan dl_plan(int64_t B, int64_t Tn, int64_t d, int64_t p) {
  const DlGroupPlan g = dl_group_plan(&B, &Tn, &d, &p, 1);
  ContractPlan pl{};
  pl.bm = g.bm;
  pl.bn = g.bn;
  pl.mt = g.mt[0];
  pl.nt = g.nt[0];
  pl.ks = g.ks[0];
  pl.units_per_split = g.cps[0];
  pl.partials = (g.ks[0] > 1 || g.bn == 256) ? 1 : 0;
  pl.engine = 1;
  return pl;
}

DlGroupPlan dl_single_plan(const ContractPlan& pl) {
  DlGroupPlan g{};
  g.n = 1;
  g.bm = pl.bm;
  g.bn = pl.bn;
  g.kc = pl.bn == 256 ? kDlWideKC : kDlKC;
  g.ks[0] = pl.ks;
  g.cps[0] = pl.units_per_split;
  g.mt[0] = pl.mt;
  g.nt[0] = pl.nt;
  g.order[0] = 0;
  return g;
}

size_t dl_layer_ws_bytes(const DlGroupPlan& g, int l, int64_t d, int64_t p) {
  if (g.ks[l] == 1 && g.bn != 256) return 0;
  const size_t part = (size_t)g.ks[l] * (size_t)d * (size_t)p * sizeof(float);
  return (part + 255) / 256 * 256;
}

// ---------------------------------------------------------------- launch
template <int BM, int BN, int S, int KC, bool RATIO>
static hipError_t launch_dl_t(hipStream_t st, const float* c, const DlGroup& grp, int64_t wgs) {
  using C = DlCfg<BM, BN, S, 8, KC>;
  static_assert(C::NT == 512, "tail workgroups run two 256-thread reduce blocks");
  auto kern = &k_contract_dl<BM, BN, S, 8, KC, RATIO>;
  // more than 64 KB of dynamic LDS must be allowed per kernel (per call:
  // cheap, and correct whichever device is current)
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     C::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(C::NT), C::LDS, st, c, grp);
  return hipGetLastError();
}

hipError_t launch_contract_dl_group(hipStream_t st, const DlLaunchLayer* layers, int n, const float* c,
                                    const DlGroupPlan& g, const SplitReduceLayer* tail, int ntail, bool* tail_taken) {
  if (tail_taken) *tail_taken = false;
  DlGroup grp{};
  grp.n = n;
  int64_t per_sum = 0;
  for (int k = 0; k < n; ++k) {
    const int l = g.order[k];
    const DlLaunchLayer& x = layers[l];
    DlLayer& L = grp.L[k];
    L.A = static_cast<const bf16s*>(x.A);
    L.G = static_cast<const bf16s*>(x.G);
    L.out = x.out;
    L.d = x.d;
    L.p = x.p;
    L.cps = x.Tn / g.kc;
    L.ks = g.ks[l];
    L.chunks_per_split = g.cps[l];
    L.nchunks = x.B * x.Tn / g.kc;
    L.mt = g.mt[l];
    L.nt = g.nt[l];
    L.per = ((int64_t)L.mt * L.nt * L.ks + 7) / 8;
    L.m_fast = L.mt <= L.nt ? 1 : 0;
    L.na = x.na;
    L.ws = x.ws;
    per_sum += L.per;
  }
  const int64_t wgs = 8 * per_sum;
  grp.wgs_main = wgs;
  int64_t extra = 0;
  if (tail && ntail > 0 && ntail <= kDlGroupMax && tail_taken) {
    // the CUs of each XCD (32) that the last round of items leaves idle take the
    // tail, when its vectorised reduce (VALU-bound: about 5 us per pass of two
    // blocks on a CU) fits in about 80 % of that round
    const int64_t rounds = (per_sum + kCusPerXcd - 1) / kCusPerXcd;
    const int64_t idle = 8 * (rounds * kCusPerXcd - per_sum);
    bool ok = idle > 0 && (wgs + idle) * 512 < ((int64_t)1 << 32);
    int64_t blocks = 0;
    for (int k = 0; ok && k < ntail; ++k) {
      ok = tail[k].acc == nullptr && split_reduce_vec_ok(tail[k]) && split_reduce_blocks(tail[k]) > 0;
      grp.tail.L[k] = tail[k];
      grp.tail.blk_begin[k] = blocks;
      blocks += split_reduce_blocks(tail[k]);
    }
    const double round_s = g.seconds / (double)(rounds > 0 ? rounds : 1);
    const double tail_s = (double)((blocks + 2 * idle - 1) / (2 * (idle > 0 ? idle : 1))) * 5.0e-6;
    if (ok && tail_s <= 0.8 * round_s) {
      grp.tail.n = ntail;
      grp.tail_blocks = blocks;
      extra = idle;
      *tail_taken = true;
    }
  }
  if ((wgs + extra) * 512 >= ((int64_t)1 << 32)) return hipErrorInvalidValue;  // work-items counted in 32 bits
  const int64_t grid = wgs + extra;
  if (g.bn == 256) return launch_dl_t<256, 256, kDlWideStages, kDlWideKC, true>(st, c, grp, grid);
  if (g.bm == 256) return launch_dl_t<256, 128, kDlStages, kDlKC, false>(st, c, grp, grid);
  return launch_dl_t<128, 128, kDlStages, kDlKC, false>(st, c, grp, grid);
}

hipError_t launch_contract_dl(hipStream_t st, const void* A, const void* G, const float* c, int64_t B, int64_t Tn,
                              int64_t d, int64_t p, const ContractPlan& pl, float* ws, const NoiseArgs& na,
                              float* out) {
  const DlGroupPlan g = dl_single_plan(pl);
  const DlLaunchLayer x{A, G, B, Tn, d, p, ws, out, na};
  return launch_contract_dl_group(st, &x, 1, c, g, nullptr, 0, nullptr);
}

}  // namespace dpk
