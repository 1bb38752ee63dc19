// Host-side launchers of the clipping kernels (internal to libdpclip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dp_common.hpp"

namespace dpk {

struct ContractPlan {
  int bm, bn;               // output tile
  int mt, nt;               // tiles along d (+1 bias row) and p
  int64_t ks;               // K splits (partial tiles summed by the reduce)
  int64_t units_per_split;  // engine 0: samples (bf16) or KC-row chunks (fp32); 1: 64-row, 2: 32-row chunks
  int engine;               // 0 register-staged (any shape), 1 direct-to-LDS bf16, 2 direct-to-LDS fp32
  int partials = 0;         // the contraction writes partials even with one split
};
// Noise + mean applied in a contraction epilogue or reduce: out = (S + sc*z) * inv_denom.
struct NoiseArgs {
  float sc, inv_denom;  // sigma*C and the fp32 reciprocal of denom
  uint32_t k0, k1, layer, step;
};
// out = (S + fl(sigma*C) * z) * fl(1/denom); noise key (seed lo32, seed hi32).
inline NoiseArgs make_noise_args(float sc, float denom, uint64_t seed, uint32_t layer, uint32_t step) {
  NoiseArgs na;
  na.sc = sc;
  na.inv_denom = 1.0f / denom;
  na.k0 = (uint32_t)(seed & 0xFFFFFFFFu);
  na.k1 = (uint32_t)(seed >> 32);
  na.layer = layer;
  na.step = step;
  return na;
}
struct ExplicitPlan {
  int bm, bn, mt, nt;
};

ContractPlan contract_plan(int dtype, int64_t B, int64_t Tn, int64_t d, int64_t p, int has_bias);
// direct-to-LDS bf16 engine: layers it takes, its plan, its launch (partials in ws when pl.ks > 1)
bool dl_eligible(int dtype, int64_t B, int64_t Tn, int64_t d, int64_t p, int has_bias);
ContractPlan dl_plan(int64_t B, int64_t Tn, int64_t d, int64_t p);
hipError_t launch_contract_dl(hipStream_t st, const void* A, const void* G, const float* c, int64_t B, int64_t Tn,
                              int64_t d, int64_t p, const ContractPlan& pl, float* ws, const NoiseArgs& na,
                              float* out);
// Launches of the direct-to-LDS bf16 engine: up to kDlGroupMax eligible
// layers in one kernel launch, one tile shape for all of them, K splits per
// layer. Split tiles (and the 256x256 tile's) leave partials in the layer's
// workspace region for the reduce kernel (launch_split_reduce).
constexpr int kDlGroupMax = 8;
struct DlLaunchLayer {
  const void* A;
  const void* G;
  int64_t B, Tn, d, p;
  float* ws;  // this layer's workspace region (dl_layer_ws_bytes), or nullptr when that is 0
  float* out;
  NoiseArgs na;
};
struct DlGroupPlan {
  int n;
  int bm, bn, kc;                 // tile and K rows per chunk
  int64_t ks[kDlGroupMax];        // per layer (caller's order)
  int64_t cps[kDlGroupMax];       // chunks per split
  int mt[kDlGroupMax], nt[kDlGroupMax];
  int order[kDlGroupMax];         // dispatch order (layer indices)
  double seconds;                 // modelled time
};
DlGroupPlan dl_group_plan(const int64_t* B, const int64_t* Tn, const int64_t* d, const int64_t* p, int n);
size_t dl_layer_ws_bytes(const DlGroupPlan& g, int l, int64_t d, int64_t p);
// The one-layer group plan of a single-layer engine-1 plan.
DlGroupPlan dl_single_plan(const ContractPlan& pl);
struct SplitReduceLayer;
// tail (may be null): the split reduce of the previous launch of the same
// call (noise form, ntail layers); the launch takes it on its idle CUs when it
// fits, and says so in *tail_taken; else the caller launches that reduce.
hipError_t launch_contract_dl_group(hipStream_t st, const DlLaunchLayer* layers, int n, const float* c,
                                    const DlGroupPlan& g, const SplitReduceLayer* tail, int ntail,
                                    bool* tail_taken);
// The split partials [ks][d][p] a launch left in ws (no bias row) -> out,
// with the noise and the mean: the reduce kernel of the split contractions.
hipError_t launch_split_reduce(hipStream_t st, int64_t ks, float* ws, int64_t d, int64_t p, const NoiseArgs& na,
                               float* out);
// One layer's split partials [ks][d][p] (no bias row) and its output; with
// acc set, the partials' sum S is added to acc instead (acc = acc + S, no
// noise) and out is left alone.
struct SplitReduceLayer {
  const float* ws;
  int64_t ks, d, p;
  NoiseArgs na;
  float* out;
  float* acc;
};
// The split reduces of up to kDlGroupMax layers, each layer's output the same
// as launch_split_reduce's (for an acc layer: as launch_split_reduce with no
// noise and a mean of 1, then launch_accumulate): one launch for the layers
// the vectorised reduce takes, launches of their own for the others. Either
// every layer has acc set or none.
hipError_t launch_split_reduce_group(hipStream_t st, const SplitReduceLayer* layers, int n);
// direct-to-LDS fp32 engine (bias row accumulated on the side, partials [ks][d + bias][p] in ws)
bool dl32_eligible(int dtype, int64_t B, int64_t Tn, int64_t d, int64_t p, int has_bias);
ContractPlan dl32_plan(int64_t B, int64_t Tn, int64_t d, int64_t p, int has_bias);
hipError_t launch_contract_dl32(hipStream_t st, const void* A, const void* G, const float* c, int64_t B, int64_t Tn,
                                int64_t d, int64_t p, const ContractPlan& pl, float* ws, const NoiseArgs& na,
                                float* out, float* bias_out);
ExplicitPlan explicit_plan(int64_t d, int64_t p, int has_bias);
int ghost_tile_size(int64_t T);
// Gram tiles per sample of the ghost kernel that dp_ghost_norm runs for this layer
int64_t ghost_ntiles(int dtype, int64_t T, int64_t d, int64_t p);
// Gram tiles per sample of the tiled ghost kernel (the kernel convolution
// layers given by their folded input take, whatever the shape).
int64_t ghost_tiled_ntiles(int64_t T);
// bf16 long-sequence ghost engine (256 x 128 Gram tiles, direct-to-LDS)
bool ghost_wide_eligible(int dtype, int64_t Tn, int64_t d, int64_t p);
int64_t ghost_wide_ntiles(int64_t Tn);
hipError_t launch_ghost_wide(hipStream_t st, const void* A, const void* G, int64_t B, int64_t Tn, int64_t d,
                             int64_t p, int has_bias, const NormSink& sink);

hipError_t launch_norm_t1(hipStream_t st, int dtype, const void* A, const void* G, int64_t B, int64_t d, int64_t p,
                          int has_bias, int accumulate, float* sqnorm);
// One layer handed to a grouped ghost launch.
struct GhostLayerDesc {
  const void* A;
  const void* G;
  int64_t Tn, d, p;
  int has_bias;
};
// Layers of one ghost launch share ghost_group_key: the tiled kernel's tile
// size and dtype, or the long-sequence bf16 engine.
int ghost_group_key(int dtype, int64_t Tn, int64_t d, int64_t p);
// Up to kNormGroupMax groupable layers with one key in one launch (the tiled
// kernel, or the long-sequence bf16 engine); the sink spans the tiles of all
// of them (lt[] in the order of `layers`).
hipError_t launch_ghost_group(hipStream_t st, int dtype, const GhostLayerDesc* layers, int n, int64_t B,
                              const NormSink& sink);
hipError_t launch_ghost_wide_group(hipStream_t st, const GhostLayerDesc* layers, int n, int64_t B,
                                   const NormSink& sink);
// Norm kernels whose sample spans several tile workgroups store per-tile
// partials; launch_norm_finish (after the tiles' launch, same stream) folds
// them per sample (NormSink in dp_common.hpp). A no-op for one tile per sample.
hipError_t launch_norm_finish(hipStream_t st, const NormSink& sink, int64_t B);
hipError_t launch_ghost(hipStream_t st, int dtype, const void* A, const void* G, int64_t B, int64_t Tn, int64_t d,
                        int64_t p, int has_bias, const NormSink& sink);
hipError_t launch_explicit(hipStream_t st, int dtype, const void* A, const void* G, int64_t B, int64_t Tn, int64_t d,
                           int64_t p, int has_bias, const NormSink& sink);
// Weighted contraction + noise + 1/denom: one kernel when pl.ks == 1, else
// partial tiles in ws and a reduce kernel. bias_out != nullptr <=> bias row.
// Convolution layers given by their folded input (ConvGeo): the unfolded
// rows are formed on chip by the tiled ghost, explicit and register-staged
// contraction kernels; G is [B, geo.T, p]. The contraction plan is tiles_plan.
// `folded`: the plan of a folded-input convolution.
ContractPlan tiles_plan(int dtype, int64_t B, int64_t Tn, int64_t d, int64_t p, int has_bias, bool folded);
// U(a) [B, T, d] of a folded input a (geometry g) written to U: the unfolding of dp_conv_*.
hipError_t launch_unfold2d(hipStream_t st, int dtype, const ConvGeo& g, int64_t B, void* U);
hipError_t launch_ghost_conv(hipStream_t st, int dtype, const ConvGeo& geo, const void* G, int64_t B, int64_t p,
                             int has_bias, const NormSink& sink);
hipError_t launch_explicit_conv(hipStream_t st, int dtype, const ConvGeo& geo, const void* G, int64_t B, int64_t p,
                                int has_bias, const NormSink& sink);
hipError_t launch_clipped_sum_conv(hipStream_t st, int dtype, const ConvGeo& geo, const void* G, const float* c,
                                   int64_t B, int64_t p, const ContractPlan& pl, float* ws, float sc, float denom,
                                   uint64_t seed, uint32_t layer, uint32_t step, float* out, float* bias_out);
hipError_t launch_clipped_sum(hipStream_t st, int dtype, const void* A, const void* G, const float* c, int64_t B,
                              int64_t Tn, int64_t d, int64_t p, const ContractPlan& pl, float* ws, float sc,
                              float denom, uint64_t seed, uint32_t layer, uint32_t step, float* out,
                              float* bias_out);
hipError_t launch_clip_factors(hipStream_t st, const float* sqnorm, int64_t B, float C, float* c, float* norm);
// Virtual step: acc += s (n floats); out = (acc + sc z) * inv_denom with the clipped sums' noise counters.
hipError_t launch_accumulate(hipStream_t st, float* acc, const float* s, int64_t n);
hipError_t launch_noise_mean(hipStream_t st, const float* acc, const float* bias_acc, int64_t d, int64_t p,
                             const NoiseArgs& na, float* out, float* bias_out);
hipError_t launch_adaptive_threshold(hipStream_t st, const float* norm, int64_t B, float C_prev, float alpha,
                                     float beta, float sigma_l2, int init, uint64_t seed, uint32_t layer,
                                     uint32_t step, float* C_next, float* C_l2_out);

}  // namespace dpk
