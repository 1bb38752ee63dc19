// Weighted contraction S = A^T diag(c) G of an fp32 layer, direct-to-LDS engine.
//
// The clipped sum of "Scaling up DP Deep Learning with Fast Per-Example
// Gradient Clipping" (gradient of the re-weighted loss sum_i c_i L_i) and
// "Scalable and Efficient Training of Large CNNs with DP" eq. (2.1) /
// Sec. 3.2, as ONE contraction over the K = B*T rows of the flattened
// [B*T, d] and [B*T, p] views (each row scaled by the clip factor of its
// sample), with the Gaussian noise and the mean in the epilogue, or in the
// split-K reduce. With a bias, S_b = sum_rows c_row G[row, :] (the bias
// gradient is the row sum of G over the sample's T rows).
//
// Eligible layers: fp32, d and p multiples of 4 and >= 128 (16-byte rows),
// B*T a multiple of 32 (whole 32-row chunks).
//
// gfx950 mapping:
// - 32-row K chunks of the A tile (BM features) and the G tile (BN features)
//   go from HBM straight to LDS with 16-byte global_load_lds, row-major
//   [k][feature]; the 32 clip factors of the chunk's rows land next to them
//   (one 4-byte global_load_lds per wave, 4 rows each).
// - v_mfma_f32_32x32x2_f32 takes one element of each operand per lane
//   (feature lane % 32, k = lane / 32). A wave's 64x64 sub-tile is two 32-row
//   blocks of each operand with the features interleaved (block b holds
//   features 2j + b), so one 8-byte LDS read gives a lane both blocks'
//   operands; a half-wave reads 256 contiguous bytes of one k-row (all 64
//   banks). The G operand is scaled by its row's clip factor in registers.
// - Tiles that hold output row 0 also accumulate the bias sum on the VALU
//   from the staged G rows.
// - Three LDS stages: the loads of chunk q+2 are in flight while chunk q is
//   computed; one barrier per chunk. Work items are XCD-contiguous as in the
//   bf16 engine.
#include "dp_common.hpp"
#include "dp_launch.hpp"
#include "dp_lds.hpp"
#include "dp_noise.hpp"

namespace dpk {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) f32x2 lds_f32x2;
typedef __attribute__((address_space(3))) float lds_f32;

template <int BM, int BN, int NW>
struct Dl32Cfg {
  static constexpr int KC = 32;                   // K rows per chunk
  static constexpr int STAGES = 3;
  static constexpr int NT = 64 * NW;
  static constexpr int RA = BM * 4, RG = BN * 4;  // LDS row bytes
  static constexpr int A_BYTES = KC * RA, G_BYTES = KC * RG;
  static constexpr int C_OFF = A_BYTES + G_BYTES;  // KC clip factors
  static constexpr int STAGE = C_OFF + KC * 4;
  static constexpr int LDS = STAGES * STAGE;
  static constexpr int WGM = NW / 2, WGN = 2;     // wave grid
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int LA = A_BYTES / (1024 * NW);  // 1 KB loads per wave per chunk
  static constexpr int LG = G_BYTES / (1024 * NW);
  static constexpr int LPC = LA + LG + 1;           // + the clip-factor load
  static constexpr int TP = BN + 8;                 // epilogue tile row (floats)
  static_assert(WM == 64 && WN == 64, "64x64 wave sub-tiles (two interleaved 32-blocks per operand)");
  static_assert(LA * 1024 * NW == A_BYTES && LG * 1024 * NW == G_BYTES, "whole 1 KB loads per wave");
  static_assert(KC == 4 * NW, "each wave loads the clip factors of four chunk rows");
  static_assert(NT == 4 * BN && KC % 4 == 0, "bias sum: four row groups of KC/4 rows x BN columns");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(BM * TP * 4 + 4 * BN * 4 <= LDS, "epilogue tile + bias partials fit the stages");
  static_assert(LPC * (STAGES - 1) <= 63, "vmcnt range");
};

struct Dl32Args {
  int64_t d, p, Tn;
  int mt, nt;
  int64_t ks;
  int64_t chunks_per_split;
  int64_t nchunks;  // B * T / 32
  int m_fast;
  int has_bias;
  NoiseArgs na;
};

// 4 bytes per lane from the lane's own global address into LDS at
// lds_base + 4*lane (global_load_lds_dword, base in M0).
__device__ __forceinline__ void dma4(const void* gaddr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(gaddr), "s"(lds_base)
               : "memory", "m0");
}

__device__ __forceinline__ f32x2 lds_f2(uint32_t addr) { return *(const lds_f32x2*)(uintptr_t)addr; }
__device__ __forceinline__ float lds_f1(uint32_t addr) { return *(const lds_f32*)(uintptr_t)addr; }

__device__ __forceinline__ int64_t row_sample(int64_t row, int64_t Tn) {
  if (Tn == 1) return row;
  if ((uint64_t)row <= 0xFFFFFFFFull && (uint64_t)Tn <= 0xFFFFFFFFull) return (int64_t)((uint32_t)row / (uint32_t)Tn);
  return row / Tn;
}

template <int BM, int BN, int NW, bool FUSED>
__global__ __launch_bounds__(64 * NW, 1) void k_contract_dl32(const float* __restrict__ A, const float* __restrict__ G,
                                                              const float* __restrict__ c, float* __restrict__ ws,
                                                              float* __restrict__ out, float* __restrict__ bias_out,
                                                              Dl32Args a) {
  using C = Dl32Cfg<BM, BN, NW>;
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
  const bool bias_tile = a.has_bias && tm == 0;  // workgroup-uniform

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave % C::WGM, wn = wave / C::WGM;

  // ---- per-lane global byte offsets of this lane's 16-byte pieces within a chunk
  // (< 32 * max(d, p) * 4 < 2^31)
  uint32_t offA[C::LA], offG[C::LG];
#pragma unroll
  for (int i = 0; i < C::LA; ++i) {
    const int byte = (wave + NW * i) * 1024 + 16 * lane;
    const int r = byte / C::RA;
    int64_t col = m0 + (byte % C::RA) / 4;
    if (col > a.d - 4) col = a.d - 4;  // columns past d only feed unwritten output rows
    offA[i] = (uint32_t)((r * a.d + col) * 4);
  }
#pragma unroll
  for (int i = 0; i < C::LG; ++i) {
    const int byte = (wave + NW * i) * 1024 + 16 * lane;
    const int r = byte / C::RG;
    int64_t col = n0 + (byte % C::RG) / 4;
    if (col > a.p - 4) col = a.p - 4;
    offG[i] = (uint32_t)((r * a.p + col) * 4);
  }

  auto issue = [&](int64_t q, int stage) {
    const float* ga = A + q * (int64_t)C::KC * a.d;
    const float* gg = G + q * (int64_t)C::KC * a.p;
    const uint32_t st = lds_addr(lds) + stage * C::STAGE;
    const uint32_t sa = st + wave * 1024;
    const uint32_t sg = st + C::A_BYTES + wave * 1024;
#pragma unroll
    for (int i = 0; i < C::LA; ++i) dma16(ga, offA[i], sa + 1024 * NW * i);
#pragma unroll
    for (int i = 0; i < C::LG; ++i) dma16(gg, offG[i], sg + 1024 * NW * i);
    const uint32_t sc = st + C::C_OFF + 16 * wave;
    if (lane < 4) dma4(c + row_sample(q * C::KC + 4 * wave + lane, a.Tn), sc);
  };

  // ---- per-lane LDS read offsets: lane (j = lane % 32, h = lane / 32) reads
  // k-row h (+2 per MFMA step) at features 2j, 2j+1 of its wave's sub-tile
  const int j32 = lane & 31, h = lane >> 5;
  const uint32_t rdA = h * C::RA + (wm * C::WM + 2 * j32) * 4;
  const uint32_t rdG = C::A_BYTES + h * C::RG + (wn * C::WN + 2 * j32) * 4;
  const uint32_t rdC = C::C_OFF + 4 * h;

  f32x16 acc[2][2];
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[bi][bj][e] = 0.f;
  float bsum = 0.f;  // bias tiles: sum over this thread's rows of c_row * G[row][n]
  const int bn_col = threadIdx.x % BN, bn_grp = threadIdx.x / BN;

  auto compute = [&](uint32_t sb) {
#pragma unroll
    for (int s = 0; s < C::KC / 2; ++s) {
      const f32x2 av = lds_f2(sb + rdA + 2 * s * C::RA);
      f32x2 gv = lds_f2(sb + rdG + 2 * s * C::RG);
      const float cv = lds_f1(sb + rdC + 8 * s);
      gv.x *= cv;
      gv.y *= cv;
      acc[0][0] = mfma32_f32(av.x, gv.x, acc[0][0]);
      acc[0][1] = mfma32_f32(av.x, gv.y, acc[0][1]);
      acc[1][0] = mfma32_f32(av.y, gv.x, acc[1][0]);
      acc[1][1] = mfma32_f32(av.y, gv.y, acc[1][1]);
    }
  };
  auto bias_step = [&](uint32_t sb) {
#pragma unroll
    for (int r = 0; r < C::KC / 4; ++r) {
      const int row = (C::KC / 4) * bn_grp + r;
      const float g = lds_f1(sb + C::A_BYTES + row * C::RG + bn_col * 4);
      const float cv = lds_f1(sb + C::C_OFF + row * 4);
      bsum = __builtin_fmaf(cv, g, bsum);
    }
  };

  // ---- pipeline: chunk q in stage q % 3; loads for chunk it+2 go out once
  // every wave is past chunk it-1 (the barrier), while chunk it is computed.
  if (nq > 0) issue(q0, 0);
  if (nq > 1) issue(q0 + 1, 1);
  for (int it = 0; it < nq; ++it) {
    if (it + 1 < nq)
      wait_vmcnt<C::LPC>();
    else
      wait_vmcnt<0>();
    lds_barrier();  // chunk it landed for every wave; every wave is done with chunk it-1
    if (it + 2 < nq) issue(q0 + it + 2, (it + 2) % 3);
    const uint32_t sb = lds_addr(lds) + (uint32_t)((it % 3) * C::STAGE);
    compute(sb);
    if (bias_tile) bias_step(sb);
  }

  // ---- epilogue: the output tile goes through LDS ([BM][BN + 8] fp32; block
  // (bi, bj) element (m, n) is feature row wm*64 + 2m + bi, column
  // wn*64 + 2n + bj), then whole Philox blocks (4 rows of one column) or
  // float4 row pieces per thread.
  constexpr int TP = C::TP;
  float* tile = reinterpret_cast<float*>(lds);
  float* bpart = tile + BM * TP;  // [4][BN] bias partials
  lds_barrier();
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        tile[(wm * C::WM + 2 * acc_row(e, lane) + bi) * TP + wn * C::WN + 2 * acc_col(lane) + bj] = acc[bi][bj][e];
  if (bias_tile) bpart[bn_grp * BN + bn_col] = bsum;
  lds_barrier();
  const int64_t split_stride = (a.d + (a.has_bias ? 1 : 0)) * a.p;
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
    if (bias_tile && threadIdx.x < BN) {
      const int64_t n = n0 + threadIdx.x;
      if (n < a.p) {
        const float sbias = ((bpart[threadIdx.x] + bpart[BN + threadIdx.x]) + bpart[2 * BN + threadIdx.x]) +
                            bpart[3 * BN + threadIdx.x];
        const f32x4 zb = normals4((uint32_t)(n >> 2), 2u * a.na.layer + 1u, a.na.step, 0u, a.na.k0, a.na.k1);
        bias_out[n] = noised_mean_spec(sbias, a.na.sc, zb[(int)(n & 3)], a.na.inv_denom);
      }
    }
  } else {
    float* wsp = ws + split * split_stride;
#pragma unroll 1
    for (int e = threadIdx.x; e < BM * (BN / 4); e += C::NT) {
      const int row = e / (BN / 4), c4 = e % (BN / 4);
      const int64_t m = m0 + row, n = n0 + 4 * c4;
      if (m >= a.d || n >= a.p) continue;
      const float4 v = *reinterpret_cast<const float4*>(tile + row * TP + 4 * c4);
      // p % 4 == 0 and n % 4 == 0: the four columns are all in range and 16-byte aligned
      *reinterpret_cast<float4*>(wsp + m * a.p + n) = v;
    }
    if (bias_tile && threadIdx.x < BN) {
      const int64_t n = n0 + threadIdx.x;
      if (n < a.p)
        wsp[a.d * a.p + n] = ((bpart[threadIdx.x] + bpart[BN + threadIdx.x]) + bpart[2 * BN + threadIdx.x]) +
                             bpart[3 * BN + threadIdx.x];
    }
  }
}

// ---------------------------------------------------------------- plan
bool dl32_eligible(int dtype, int64_t B, int64_t Tn, int64_t d, int64_t p, int has_bias) {
  (void)has_bias;
  return dtype == 0 && (B * Tn) % 32 == 0 && d % 4 == 0 && p % 4 == 0 && d >= 128 && p >= 128 &&
         32 * 4 * (d > p ? d : p) < (1ll << 31);
}

// K split from a cost model: rounds of one workgroup per CU (256 CUs) x the
// chunks each item runs at a sustained per-CU fp32 MFMA rate, plus the write
// and re-read of split partials and a reduce launch.
ContractPlan dl32_plan(int64_t B, int64_t Tn, int64_t d, int64_t p, int has_bias) {
  constexpr int BM = 256, BN = 128;
  const double cu_rate = 157.3e12 / 256.0 * 0.8;
  const int64_t nchunks = B * Tn / 32;
  const int64_t mt = (d + BM - 1) / BM, nt = (p + BN - 1) / BN;
  const double chunk_s = 2.0 * BM * BN * 32 / cu_rate;
  const int64_t mrows = d + (has_bias ? 1 : 0);
  ContractPlan best{};
  double best_t = 1e300;
  const int64_t ks_max = nchunks < 512 ? nchunks : 512;
  for (int64_t ks = 1; ks <= ks_max; ++ks) {
    const int64_t cpsplit = (nchunks + ks - 1) / ks;
    if ((nchunks + cpsplit - 1) / cpsplit != ks) continue;
    const int64_t items = mt * nt * ks;
    const double rounds = (double)((items + 255) / 256);
    double tt = rounds * (double)cpsplit * chunk_s + 3.0e-6;
    if (ks > 1) tt += (2.0 * ks + 1.0) * (double)mrows * (double)p * 4.0 / 5.0e12 + 4.0e-6;
    if (tt < best_t * 0.999) {
      best_t = tt;
      best.ks = ks;
      best.units_per_split = cpsplit;
    }
  }
  best.bm = BM;
  best.bn = BN;
  best.mt = (int)mt;
  best.nt = (int)nt;
  best.engine = 2;
  return best;
}

// ---------------------------------------------------------------- launch
hipError_t launch_contract_dl32(hipStream_t st, const void* A, const void* G, const float* c, int64_t B, int64_t Tn,
                                int64_t d, int64_t p, const ContractPlan& pl, float* ws, const NoiseArgs& na,
                                float* out, float* bias_out) {
  constexpr int BM = 256, BN = 128, NW = 8;
  using Cf = Dl32Cfg<BM, BN, NW>;
  Dl32Args a;
  a.d = d;
  a.p = p;
  a.Tn = Tn;
  a.mt = pl.mt;
  a.nt = pl.nt;
  a.ks = pl.ks;
  a.chunks_per_split = pl.units_per_split;
  a.nchunks = B * Tn / 32;
  a.m_fast = pl.mt <= pl.nt ? 1 : 0;
  a.has_bias = bias_out != nullptr ? 1 : 0;
  a.na = na;
  const int64_t items = (int64_t)pl.mt * pl.nt * pl.ks;
  const int64_t per = (items + 7) / 8;
  const dim3 grid((unsigned)(per * 8));
  const float* Af = static_cast<const float*>(A);
  const float* Gf = static_cast<const float*>(G);
  if (pl.ks == 1) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_contract_dl32<BM, BN, NW, true>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, Cf::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_contract_dl32<BM, BN, NW, true>), grid, dim3(Cf::NT), Cf::LDS, st, Af, Gf, c, ws, out,
                       bias_out, a);
  } else {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_contract_dl32<BM, BN, NW, false>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, Cf::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_contract_dl32<BM, BN, NW, false>), grid, dim3(Cf::NT), Cf::LDS, st, Af, Gf, c, ws, out,
                       bias_out, a);
  }
  return hipGetLastError();
}

}  // namespace dpk
