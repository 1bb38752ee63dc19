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
  int partials = 0;         // the contraction writes partials (and a reduce adds the noise) even with one split
};
// Noise + mean applied in a contraction epilogue or reduce: out = (S + sc*z) * inv_denom.
struct NoiseArgs {
  float sc, inv_denom;  // sigma*C and the fp32 reciprocal of denom
  uint32_t k0, k1, layer, step;
};
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
// Layers that the tiled ghost kernel takes (the long-sequence bf16 engine
// runs one layer per launch); layers of one launch share ghost_group_key.
bool ghost_groupable(int dtype, int64_t Tn, int64_t d, int64_t p);
int ghost_group_key(int dtype, int64_t Tn);
// Workgroups of a grouped launch (the caller keeps it below 2^32).
int64_t ghost_group_grid(int64_t B, const GhostLayerDesc* layers, int n);
// Up to kNormGroupMax groupable layers with one key in one launch; the sink
// spans the tiles of all of them (lt[] in the order of `layers`).
hipError_t launch_ghost_group(hipStream_t st, int dtype, const GhostLayerDesc* layers, int n, int64_t B,
                              const NormSink& sink);
// Norm kernels whose sample spans several tile workgroups finish each
// sample in its last-arriving tile (NormSink in dp_common.hpp).
hipError_t launch_ghost(hipStream_t st, int dtype, const void* A, const void* G, int64_t B, int64_t Tn, int64_t d,
                        int64_t p, int has_bias, const NormSink& sink);
hipError_t launch_explicit(hipStream_t st, int dtype, const void* A, const void* G, int64_t B, int64_t Tn, int64_t d,
                           int64_t p, int has_bias, const NormSink& sink);
// Tag of one call for its arrival counters: 48 bits, never 0, distinct per call in the process.
uint64_t next_epoch();
// Weighted contraction + noise + 1/denom: one kernel when pl.ks == 1,
// else partial tiles in ws and a reduce kernel. bias_out != nullptr <=> bias row.
hipError_t launch_clipped_sum(hipStream_t st, int dtype, const void* A, const void* G, const float* c, int64_t B,
                              int64_t Tn, int64_t d, int64_t p, const ContractPlan& pl, float* ws, float sc,
                              float denom, uint64_t seed, uint32_t layer, uint32_t step, float* out,
                              float* bias_out);
hipError_t launch_clip_factors(hipStream_t st, const float* sqnorm, int64_t B, float C, float* c, float* norm);
hipError_t launch_adaptive_threshold(hipStream_t st, const float* norm, int64_t B, float C_prev, float alpha,
                                     float beta, float sigma_l2, int init, uint64_t seed, uint32_t layer,
                                     uint32_t step, float* C_next, float* C_l2_out);

}  // namespace dpk
