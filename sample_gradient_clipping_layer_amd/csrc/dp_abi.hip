// extern "C" entry points of libdpclip.so (declared in include/dpclip.h).
// Every argument is validated before the first HIP call; then the kernels of
// the chosen path are enqueued on the caller's stream, without synchronising.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/dpclip.h"
#include "dp_launch.hpp"

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;    // each of B, T, d+1, p below 2^31
constexpr int64_t kMaxElems = (int64_t)1 << 50;  // B*T*(d+1), B*T*p
constexpr int64_t kMaxNoise = (int64_t)1 << 32;  // ceil(d/4)*p: noise group index fits 32 bits

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }
bool finite(float x) { return isfinite(x) != 0; }

dp_status check_shape(int64_t B, int64_t T, int64_t d, int64_t p) {
  if (B < 1 || T < 1 || d < 1 || p < 1) return DP_ERR_SHAPE;
  if (B >= kMaxDim || T >= kMaxDim || d + 1 >= kMaxDim || p >= kMaxDim) return DP_ERR_SHAPE;
  if (B * T >= kMaxDim * 8) return DP_ERR_SHAPE;
  const int64_t bt = B * T;
  if (bt > kMaxElems / (d + 1) || bt > kMaxElems / p) return DP_ERR_SHAPE;
  if ((d + 3) / 4 >= kMaxNoise / p) return DP_ERR_SHAPE;
  return DP_OK;
}

dp_status check_layer(const void* A, const void* G, dp_dtype dtype, int64_t B, int64_t T, int64_t d, int64_t p) {
  if (!A || !G) return DP_ERR_NULL;
  dp_status s = check_shape(B, T, d, p);
  if (s != DP_OK) return s;
  if (dtype != DP_F32 && dtype != DP_BF16) return DP_ERR_DTYPE;
  if (!aligned(A, 16) || !aligned(G, 16)) return DP_ERR_ALIGN;
  return DP_OK;
}

dp_status device_ready() {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n < 1) return DP_ERR_NO_DEVICE;
  return DP_OK;
}

int path_of(int64_t T, int64_t d, int64_t p, dp_mode mode, int32_t kappa) {
  if (mode == DP_MODE_EXPLICIT) return DP_PATH_EXPLICIT;
  if (T == 1) return DP_PATH_T1;
  if (mode == DP_MODE_GHOST) return DP_PATH_GHOST;
  if (mode == DP_MODE_TIME) {
    // per-sample matrix-core work: instantiation 2Tdp + 2dp, ghost T(T+1)(d+p) + 2T^2 (long double: exact here)
    const long double Tl = (long double)T, dl = (long double)d, pl = (long double)p;
    const long double expl = 2.0L * Tl * dl * pl + 2.0L * dl * pl;
    const long double ghost = Tl * (Tl + 1.0L) * (dl + pl) + 2.0L * Tl * Tl;
    return expl < ghost ? DP_PATH_EXPLICIT : DP_PATH_GHOST;
  }
  // p*d < kappa*T^2 -> instantiate; compared in long double to stay exact for large sizes
  const long double pd = (long double)p * (long double)d;
  const long double t2 = (long double)kappa * (long double)T * (long double)T;
  return pd < t2 ? DP_PATH_EXPLICIT : DP_PATH_GHOST;
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// A dispatch's work-items (workgroups x threads) are counted in 32 bits; the
// kernels run at most 512 threads per workgroup.
constexpr uint64_t kMaxWorkgroups = (1ull << 32) / 512;
bool grid_fits(uint64_t workgroups) { return workgroups < kMaxWorkgroups; }

// tiles per sample of one norm call (the documented DP_ERR_SHAPE limit)
constexpr int64_t kMaxTilesPerSample = 65535;

int64_t norm_ntiles(int dtype, int path, int64_t T, int64_t d, int64_t p, int has_bias) {
  if (path == DP_PATH_T1) return 1;
  if (path == DP_PATH_GHOST) return dpk::ghost_ntiles(dtype, T, d, p);
  const dpk::ExplicitPlan pl = dpk::explicit_plan(d, p, has_bias);
  return (int64_t)pl.mt * pl.nt;
}

// tile partials [B][ntiles] fp32
size_t norm_partial_bytes(int64_t B, int64_t ntiles) { return round256((size_t)B * (size_t)ntiles * sizeof(float)); }

size_t norm_ws_bytes(int dtype, int path, int64_t B, int64_t T, int64_t d, int64_t p, int has_bias) {
  const int64_t ntiles = norm_ntiles(dtype, path, T, d, p, has_bias);
  if (ntiles == 1) return 0;
  return norm_partial_bytes(B, ntiles);
}

size_t contract_ws_for(const dpk::ContractPlan& pl, int64_t d, int64_t p, int has_bias) {
  if (pl.engine == 1) return dpk::dl_layer_ws_bytes(dpk::dl_single_plan(pl), 0, d, p);
  if (pl.ks == 1 && !pl.partials) return 0;  // one K split: the epilogue writes the output directly
  return round256((size_t)pl.ks * (size_t)(d + (has_bias ? 1 : 0)) * (size_t)p * sizeof(float));
}

size_t contract_ws_bytes(dp_dtype dtype, int64_t B, int64_t T, int64_t d, int64_t p, int has_bias) {
  return contract_ws_for(dpk::contract_plan(dtype, B, T, d, p, has_bias), d, p, has_bias);
}

dp_status hip_status(hipError_t e) { return e == hipSuccess ? DP_OK : DP_ERR_HIP; }

// Clip factors (and norms) to form from the final squared norms of a call.
struct ClipOut {
  float C;
  float* c;
  float* norm;  // may be null
};

// Launches the norm kernels of one layer whose arguments are validated; with
// `clip`, also the clip factors of the resulting squared norms (in the
// kernel's per-sample sink, or by the clip kernel after the closed form).
hipError_t launch_layer_norm(hipStream_t st, int dtype, const void* A, const void* G, int64_t B, int64_t T, int64_t d,
                             int64_t p, int hb, int path, void* workspace, float* sqnorm, int acc,
                             const ClipOut* clip = nullptr) {
  if (path == DP_PATH_T1) {
    hipError_t e = dpk::launch_norm_t1(st, dtype, A, G, B, d, p, hb, acc, sqnorm);
    if (e == hipSuccess && clip) e = dpk::launch_clip_factors(st, sqnorm, B, clip->C, clip->c, clip->norm);
    return e;
  }
  const int64_t ntiles = norm_ntiles(dtype, path, T, d, p, hb);
  dpk::NormSink sink = dpk::make_norm_sink(static_cast<float*>(workspace), sqnorm, (int)ntiles, acc);
  if (clip) {
    sink.clip_c = clip->c;
    sink.clip_norm = clip->norm;
    sink.C = clip->C;
  }
  const hipError_t e = path == DP_PATH_GHOST ? dpk::launch_ghost(st, dtype, A, G, B, T, d, p, hb, sink)
                                             : dpk::launch_explicit(st, dtype, A, G, B, T, d, p, hb, sink);
  return e == hipSuccess ? dpk::launch_norm_finish(st, sink, B) : e;
}

// Per-layer limits of dp_ghost_norm: tiles per sample (kMaxTilesPerSample)
// and the ghost grid (32-bit workgroup ids).
bool layer_fits(int dtype, int path, int64_t B, int64_t T, int64_t d, int64_t p, int hb) {
  const int64_t nt = norm_ntiles(dtype, path, T, d, p, hb);
  if (!grid_fits((uint64_t)((B + 7) / 8 * 8) * (uint64_t)nt)) return false;  // ghost / explicit grids
  return nt <= kMaxTilesPerSample;
}

// Consecutive layers of a multi-layer norm call that share one launch.
struct NormRun {
  int first, count;
  bool grouped;       // ghost layers of one kernel, one launch for all of them
  int64_t ntiles;     // tiles per sample over the run
};

constexpr int32_t kMaxNormLayers = 4096;

// The layer list itself: count, pointers, shapes, dtype, reserved fields.
dp_status check_layer_list(const dp_layer* layers, int32_t n, dp_dtype dtype, int64_t B) {
  if (!layers) return DP_ERR_NULL;
  if (n < 1 || n > kMaxNormLayers) return DP_ERR_SHAPE;
  for (int32_t l = 0; l < n; ++l) {
    const dp_layer& x = layers[l];
    const dp_status s = check_layer(x.A, x.G, dtype, B, x.T, x.d, x.p);
    if (s != DP_OK) return s;
    if (x.reserved != 0) return DP_ERR_VALUE;
  }
  return DP_OK;
}

dp_status check_norm_layers(const dp_layer* layers, int32_t n, dp_dtype dtype, int64_t B, dp_mode mode,
                            int32_t kappa) {
  const dp_status s = check_layer_list(layers, n, dtype, B);
  if (s != DP_OK) return s;
  if (mode < DP_MODE_MIXED || mode > DP_MODE_TIME || kappa < 1) return DP_ERR_VALUE;
  for (int32_t l = 0; l < n; ++l) {
    const dp_layer& x = layers[l];
    const int path = path_of(x.T, x.d, x.p, mode, kappa);
    if (!layer_fits(dtype, path, B, x.T, x.d, x.p, x.has_bias ? 1 : 0)) return DP_ERR_SHAPE;
  }
  return DP_OK;
}

// Runs in layer order: a run of ghost layers grows while the next layer takes
// the same ghost kernel (the tiled one with the same tile size, or the
// long-sequence bf16 engine) and the run stays within one launch's limits
// (kNormGroupMax layers, the sample's tile count, the grid); every other
// layer is a run of its own.
int plan_norm_runs(const dp_layer* layers, int32_t n, dp_dtype dtype, int64_t B, dp_mode mode, int32_t kappa,
                   NormRun* runs) {
  int nr = 0;
  for (int32_t l = 0; l < n; ++l) {
    const dp_layer& x = layers[l];
    const int hb = x.has_bias ? 1 : 0;
    const int path = path_of(x.T, x.d, x.p, mode, kappa);
    const int64_t nt = norm_ntiles(dtype, path, x.T, x.d, x.p, hb);
    const bool groupable = path == DP_PATH_GHOST;
    if (groupable && nr > 0) {
      NormRun& r = runs[nr - 1];
      const dp_layer& f = layers[r.first];
      if (r.grouped && r.count < dpk::kNormGroupMax &&
          dpk::ghost_group_key(dtype, f.T, f.d, f.p) == dpk::ghost_group_key(dtype, x.T, x.d, x.p) &&
          r.ntiles + nt <= kMaxTilesPerSample &&
          grid_fits((uint64_t)((B + 7) / 8 * 8) * (uint64_t)(r.ntiles + nt))) {
        r.count += 1;
        r.ntiles += nt;
        continue;
      }
    }
    runs[nr++] = NormRun{(int)l, 1, groupable, nt};
  }
  return nr;
}

size_t run_ws_bytes(const NormRun& r, const dp_layer* layers, int dtype, int64_t B, dp_mode mode, int32_t kappa) {
  if (r.grouped) {
    if (r.ntiles == 1) return 0;
    return norm_partial_bytes(B, r.ntiles);
  }
  const dp_layer& x = layers[r.first];
  return norm_ws_bytes(dtype, path_of(x.T, x.d, x.p, mode, kappa), B, x.T, x.d, x.p, x.has_bias ? 1 : 0);
}

// ---- multi-layer clipped sums
// Layers the direct-to-LDS bf16 engine takes go, in the caller's order, in
// launches of up to kDlGroupMax layers (each layer's workspace region after
// the previous one's); the others, and an eligible layer left alone, get
// single-layer launches. Launches follow one
// another on the stream, so every launch starts again at the workspace base.
struct SumLaunch {
  int first[dpk::kDlGroupMax];
  int count;
  bool grouped;
};

std::vector<SumLaunch> plan_sum_launches(const dp_layer* layers, int32_t n, dp_dtype dtype, int64_t B) {
  std::vector<SumLaunch> out;
  SumLaunch cur{};
  for (int32_t l = 0; l < n; ++l) {
    const dp_layer& x = layers[l];
    const int hb = x.has_bias ? 1 : 0;
    if (dpk::dl_eligible(dtype, B, x.T, x.d, x.p, hb)) {  // the engine contract_plan picks first
      cur.grouped = true;
      cur.first[cur.count++] = (int)l;
      if (cur.count == dpk::kDlGroupMax) {
        out.push_back(cur);
        cur = SumLaunch{};
      }
    } else {
      SumLaunch one{};
      one.first[0] = (int)l;
      one.count = 1;
      one.grouped = false;
      out.push_back(one);
    }
  }
  if (cur.count > 0) out.push_back(cur);
  // one eligible layer alone: the single-layer path (its split tiles go to the reduce kernel)
  for (SumLaunch& g : out)
    if (g.count == 1) g.grouped = false;
  return out;
}

dpk::DlGroupPlan group_plan_of(const SumLaunch& g, const dp_layer* layers, int64_t B) {
  int64_t Bv[dpk::kDlGroupMax], Tv[dpk::kDlGroupMax], dv[dpk::kDlGroupMax], pv[dpk::kDlGroupMax];
  for (int k = 0; k < g.count; ++k) {
    const dp_layer& x = layers[g.first[k]];
    Bv[k] = B;
    Tv[k] = x.T;
    dv[k] = x.d;
    pv[k] = x.p;
  }
  return dpk::dl_group_plan(Bv, Tv, dv, pv, g.count);
}

size_t sum_launch_ws_bytes(const SumLaunch& g, const dp_layer* layers, dp_dtype dtype, int64_t B) {
  if (!g.grouped) {
    const dp_layer& x = layers[g.first[0]];
    return contract_ws_bytes(dtype, B, x.T, x.d, x.p, x.has_bias ? 1 : 0);
  }
  const dpk::DlGroupPlan pl = group_plan_of(g, layers, B);
  size_t w = 0;
  for (int k = 0; k < g.count; ++k) w += dpk::dl_layer_ws_bytes(pl, k, layers[g.first[k]].d, layers[g.first[k]].p);
  return w;
}

// Workspace of a multi-layer clipped-sum call: the split partials of the
// shared launches take two regions in turn, each as large as the largest
// launch's (a launch's partials stay intact while the next launch reduces
// them on its idle CUs); a single-layer launch uses the start.
struct SumWsLayout {
  size_t region = 0;  // one region of the shared launches' partials
  bool two = false;   // at least two shared launches leave partials
  size_t total = 0;
};
static SumWsLayout sum_ws_layout(const std::vector<size_t>& grouped_ws, size_t single_ws) {
  SumWsLayout o;
  int n_part = 0;
  for (size_t w : grouped_ws) {
    o.region = std::max(o.region, round256(w));
    if (w > 0) ++n_part;
  }
  o.two = n_part >= 2;
  o.total = std::max(single_ws, o.two ? 2 * o.region : o.region);
  return o;
}

size_t sum_layers_ws_bytes(const dp_layer* layers, int32_t n, dp_dtype dtype, int64_t B) {
  std::vector<size_t> grouped;
  size_t single = 0;
  for (const SumLaunch& g : plan_sum_launches(layers, n, dtype, B)) {
    if (g.grouped)
      grouped.push_back(sum_launch_ws_bytes(g, layers, dtype, B));
    else
      single = std::max(single, sum_launch_ws_bytes(g, layers, dtype, B));
  }
  return sum_ws_layout(grouped, single).total;
}

// ---- convolution layers given by their folded input
constexpr int64_t kMaxConv = (int64_t)1 << 31;

// Geometry, shapes and limits of a folded-input convolution layer: every size
// >= 1 (padding >= 0) and below 2^31, one sample's folded input and the
// window offsets within 32-bit indexing, and the unfolded shape (T, d) within
// dp_ghost_norm's limits.
dp_status check_conv(const void* a, const void* G, const dp_conv2d* cv, dp_dtype dtype, int64_t B, int64_t p,
                     dpk::ConvGeo* geo) {
  if (!a || !G || !cv) return DP_ERR_NULL;
  if (dtype != DP_F32 && dtype != DP_BF16) return DP_ERR_DTYPE;
  const int64_t v[] = {cv->C_in, cv->H, cv->W, cv->kh, cv->kw, cv->stride_h, cv->stride_w, cv->dil_h, cv->dil_w};
  for (int64_t x : v)
    if (x < 1 || x >= kMaxConv) return DP_ERR_SHAPE;
  if (cv->pad_h < 0 || cv->pad_w < 0 || cv->pad_h >= kMaxConv || cv->pad_w >= kMaxConv) return DP_ERR_SHAPE;
  if (cv->C_in * cv->H >= kMaxConv || cv->C_in * cv->H * cv->W >= kMaxConv) return DP_ERR_SHAPE;
  if (cv->kh * cv->kw >= kMaxConv || cv->C_in * cv->kh * cv->kw >= kMaxConv) return DP_ERR_SHAPE;
  const int64_t span_h = cv->dil_h * (cv->kh - 1) + 1, span_w = cv->dil_w * (cv->kw - 1) + 1;
  const int64_t ext_h = cv->H + 2 * cv->pad_h, ext_w = cv->W + 2 * cv->pad_w;
  if (span_h > ext_h || span_w > ext_w || ext_h >= kMaxConv || ext_w >= kMaxConv) return DP_ERR_SHAPE;
  // 32-bit offsets in the kernels: column offsets, window origins and their sums
  if ((cv->C_in + 2) * ext_h >= kMaxConv || (cv->C_in + 2) * ext_h * ext_w >= kMaxConv) return DP_ERR_SHAPE;
  const int64_t Ho = (ext_h - span_h) / cv->stride_h + 1, Wo = (ext_w - span_w) / cv->stride_w + 1;
  // window positions ho*stride - pad + i*dil, and Ho*Wo, within int32
  if ((Ho - 1) * cv->stride_h + span_h >= kMaxConv || (Wo - 1) * cv->stride_w + span_w >= kMaxConv) return DP_ERR_SHAPE;
  if (Ho * Wo >= kMaxConv) return DP_ERR_SHAPE;
  const int64_t T = Ho * Wo, d = cv->C_in * cv->kh * cv->kw;
  dp_status s = check_shape(B, T, d, p);
  if (s != DP_OK) return s;
  const uintptr_t eb = dtype == DP_BF16 ? 2 : 4;
  if (!aligned(a, eb) || !aligned(G, 16)) return DP_ERR_ALIGN;
  if (geo) {
    *geo = dpk::ConvGeo{a, (int32_t)cv->C_in, (int32_t)cv->H, (int32_t)cv->W, (int32_t)cv->kh, (int32_t)cv->kw,
                        (int32_t)cv->stride_h, (int32_t)cv->stride_w, (int32_t)cv->pad_h, (int32_t)cv->pad_w,
                        (int32_t)cv->dil_h, (int32_t)cv->dil_w, (int32_t)Ho, (int32_t)Wo, (int32_t)T, (int32_t)d,
                        dpk::make_fastdiv((uint32_t)(cv->kh * cv->kw)), dpk::make_fastdiv((uint32_t)cv->kw),
                        dpk::make_fastdiv((uint32_t)Wo), dpk::make_fastdiv((uint32_t)T)};
  }
  return DP_OK;
}

// The path of a folded-input conv layer: dp_ghost_norm's rule, with the
// ghost kernel for T = 1 (the closed form reads unfolded rows).
int conv_path(int64_t T, int64_t d, int64_t p, dp_mode mode, int32_t kappa) {
  const int path = path_of(T, d, p, mode, kappa);
  return path == DP_PATH_T1 ? DP_PATH_GHOST : path;
}

int64_t conv_norm_ntiles(int path, int64_t T, int64_t d, int64_t p, int has_bias) {
  if (path == DP_PATH_GHOST) return dpk::ghost_tiled_ntiles(T);
  const dpk::ExplicitPlan pl = dpk::explicit_plan(d, p, has_bias);
  return (int64_t)pl.mt * pl.nt;
}

size_t conv_norm_ws_bytes(int path, int64_t B, int64_t T, int64_t d, int64_t p, int has_bias) {
  const int64_t nt = conv_norm_ntiles(path, T, d, p, has_bias);
  if (nt == 1) return 0;
  return norm_partial_bytes(B, nt);
}

size_t conv_sum_ws_bytes(const dpk::ContractPlan& pl, int64_t d, int64_t p, int has_bias) {
  if (pl.ks == 1) return 0;
  return round256((size_t)pl.ks * (size_t)(d + (has_bias ? 1 : 0)) * (size_t)p * sizeof(float));
}

// ---- scratch of the entry point that allocates nothing
// (dp_ghost_norm_clip_layers_noalloc): a fixed device array that every call on
// a GPU shares (each GPU holds its own copy until the process ends). It holds
// the norm kernels' tile partials. Nothing in it must start at zero: every
// partial is written by its tile before the finish kernel reads it. Calls
// that overlap on one GPU (different streams) race on it.
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;
constexpr int32_t kNoAllocMaxLayers = 1024;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// The device address of `scratch` on the current device: looked up once per
// device with that device current, then reused. The array's host-side name
// is only a stand-in for the symbol and is never passed to a kernel.
dp_status noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DP_ERR_NO_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DP_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return DP_OK;
}

}  // namespace

extern "C" {

int32_t dp_abi_version(void) { return DP_ABI_VERSION; }

const char* dp_status_string(dp_status status) {
  switch (status) {
    case DP_OK: return "ok";
    case DP_ERR_NULL: return "a required pointer is NULL";
    case DP_ERR_SHAPE: return "a size is < 1 or too large";
    case DP_ERR_DTYPE: return "unknown dtype";
    case DP_ERR_VALUE: return "a scalar argument is out of range";
    case DP_ERR_WORKSPACE: return "workspace too small";
    case DP_ERR_HIP: return "HIP call or kernel launch failed";
    case DP_ERR_NO_DEVICE: return "no usable GPU device";
    case DP_ERR_ALIGN: return "pointer not aligned as required";
    default: return "unknown status";
  }
}

int32_t dp_choose_path(int64_t T, int64_t d, int64_t p, dp_mode mode, int32_t kappa) {
  if (T < 1 || d < 1 || p < 1 || mode < DP_MODE_MIXED || mode > DP_MODE_TIME || kappa < 1) return -1;
  return path_of(T, d, p, mode, kappa);
}

size_t dp_workspace_bytes(dp_dtype dtype, int64_t B, int64_t T, int64_t d, int64_t p, dp_mode mode, int32_t kappa) {
  if (check_shape(B, T, d, p) != DP_OK) return 0;
  if (dtype != DP_F32 && dtype != DP_BF16) return 0;
  if (mode < DP_MODE_MIXED || mode > DP_MODE_TIME || kappa < 1) return 0;
  const int path = path_of(T, d, p, mode, kappa);
  size_t w = 0;
  for (int hb = 0; hb <= 1; ++hb) {
    const size_t a = norm_ws_bytes(dtype, path, B, T, d, p, hb);
    const size_t b = contract_ws_bytes(dtype, B, T, d, p, hb);
    if (a > w) w = a;
    if (b > w) w = b;
  }
  return w;
}

dp_status dp_ghost_norm(void* stream, const void* A, const void* G, dp_dtype dtype, int64_t B, int64_t T, int64_t d,
                        int64_t p, int32_t has_bias, dp_mode mode, int32_t kappa, void* workspace, size_t ws_bytes,
                        float* sqnorm, int32_t accumulate, int32_t* path_out) {
  dp_status s = check_layer(A, G, dtype, B, T, d, p);
  if (s != DP_OK) return s;
  if (!sqnorm) return DP_ERR_NULL;
  if (!aligned(sqnorm, 4)) return DP_ERR_ALIGN;
  if (mode < DP_MODE_MIXED || mode > DP_MODE_TIME || kappa < 1) return DP_ERR_VALUE;
  const int hb = has_bias ? 1 : 0;
  const int path = path_of(T, d, p, mode, kappa);
  const size_t need = norm_ws_bytes(dtype, path, B, T, d, p, hb);
  if (need > 0) {
    if (!workspace) return DP_ERR_NULL;
    if (ws_bytes < need) return DP_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return DP_ERR_ALIGN;
  }
  if (!layer_fits(dtype, path, B, T, d, p, hb)) return DP_ERR_SHAPE;
  s = device_ready();
  if (s != DP_OK) return s;
  if (path_out) *path_out = path;
  return hip_status(launch_layer_norm(static_cast<hipStream_t>(stream), dtype, A, G, B, T, d, p, hb, path, workspace,
                                      sqnorm, accumulate ? 1 : 0));
}

size_t dp_layers_workspace_bytes(const dp_layer* layers, int32_t n_layers, dp_dtype dtype, int64_t B, dp_mode mode,
                                 int32_t kappa) {
  if (check_norm_layers(layers, n_layers, dtype, B, mode, kappa) != DP_OK) return 0;
  std::vector<NormRun> runs((size_t)n_layers);
  const int nr = plan_norm_runs(layers, n_layers, dtype, B, mode, kappa, runs.data());
  size_t w = sum_layers_ws_bytes(layers, n_layers, dtype, B);
  for (int r = 0; r < nr; ++r) w = std::max(w, run_ws_bytes(runs[r], layers, dtype, B, mode, kappa));
  return w;
}

// The multi-layer norm calls; `runs` has room for n_layers runs (the caller's
// buffer, so that an entry point can keep it off the heap).
static dp_status norm_layers_impl(void* stream, const dp_layer* layers, int32_t n_layers, dp_dtype dtype, int64_t B,
                                  dp_mode mode, int32_t kappa, void* workspace, size_t ws_bytes, float* sqnorm,
                                  int32_t accumulate, int32_t* paths_out, const ClipOut* clip, NormRun* runs) {
  dp_status s = check_norm_layers(layers, n_layers, dtype, B, mode, kappa);
  if (s != DP_OK) return s;
  if (!sqnorm) return DP_ERR_NULL;
  if (!aligned(sqnorm, 4)) return DP_ERR_ALIGN;
  const int nr = plan_norm_runs(layers, n_layers, dtype, B, mode, kappa, runs);
  size_t need = 0;
  for (int r = 0; r < nr; ++r) need = std::max(need, run_ws_bytes(runs[r], layers, dtype, B, mode, kappa));
  if (need > 0) {
    if (!workspace) return DP_ERR_NULL;
    if (ws_bytes < need) return DP_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return DP_ERR_ALIGN;
  }
  s = device_ready();
  if (s != DP_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int32_t l = 0; l < n_layers; ++l)
    if (paths_out) paths_out[l] = path_of(layers[l].T, layers[l].d, layers[l].p, mode, kappa);
  for (int r = 0; r < nr; ++r) {
    const NormRun& run = runs[r];
    const int acc = (run.first == 0 && !accumulate) ? 0 : 1;
    hipError_t e;
    if (run.grouped) {
      dpk::GhostLayerDesc desc[dpk::kNormGroupMax];
      dpk::NormSink sink = dpk::make_norm_sink(static_cast<float*>(workspace), sqnorm, (int)run.ntiles, acc);
      sink.nlayers = run.count;
      if (clip && r == nr - 1) {  // the last run's sink holds each sample's final value
        sink.clip_c = clip->c;
        sink.clip_norm = clip->norm;
        sink.C = clip->C;
      }
      sink.lt[0] = 0;
      for (int k = 0; k < run.count; ++k) {
        const dp_layer& x = layers[run.first + k];
        desc[k] = dpk::GhostLayerDesc{x.A, x.G, x.T, x.d, x.p, x.has_bias ? 1 : 0};
        sink.lt[k + 1] = sink.lt[k] + (int)norm_ntiles(dtype, DP_PATH_GHOST, x.T, x.d, x.p, desc[k].has_bias);
      }
      e = dpk::launch_ghost_group(st, dtype, desc, run.count, B, sink);
      if (e == hipSuccess) e = dpk::launch_norm_finish(st, sink, B);
    } else {
      const dp_layer& x = layers[run.first];
      const int hb = x.has_bias ? 1 : 0;
      e = launch_layer_norm(st, dtype, x.A, x.G, B, x.T, x.d, x.p, hb, path_of(x.T, x.d, x.p, mode, kappa),
                            workspace, sqnorm, acc, r == nr - 1 ? clip : nullptr);
    }
    if (e != hipSuccess) return DP_ERR_HIP;
  }
  return DP_OK;
}

dp_status dp_ghost_norm_layers(void* stream, const dp_layer* layers, int32_t n_layers, dp_dtype dtype, int64_t B,
                               dp_mode mode, int32_t kappa, void* workspace, size_t ws_bytes, float* sqnorm,
                               int32_t accumulate, int32_t* paths_out) {
  if (n_layers < 1 || n_layers > kMaxNormLayers) return layers ? DP_ERR_SHAPE : DP_ERR_NULL;
  std::vector<NormRun> runs((size_t)n_layers);
  return norm_layers_impl(stream, layers, n_layers, dtype, B, mode, kappa, workspace, ws_bytes, sqnorm, accumulate,
                          paths_out, nullptr, runs.data());
}

dp_status dp_ghost_norm_clip_layers(void* stream, const dp_layer* layers, int32_t n_layers, dp_dtype dtype, int64_t B,
                                    dp_mode mode, int32_t kappa, void* workspace, size_t ws_bytes, float* sqnorm,
                                    int32_t accumulate, float C, float* c, float* norm, int32_t* paths_out) {
  if (!c) return DP_ERR_NULL;
  if (!aligned(c, 4) || (norm && !aligned(norm, 4))) return DP_ERR_ALIGN;
  if (!finite(C) || !(C > 0.0f)) return DP_ERR_VALUE;
  if (n_layers < 1 || n_layers > kMaxNormLayers) return layers ? DP_ERR_SHAPE : DP_ERR_NULL;
  std::vector<NormRun> runs((size_t)n_layers);
  const ClipOut clip{C, c, norm};
  return norm_layers_impl(stream, layers, n_layers, dtype, B, mode, kappa, workspace, ws_bytes, sqnorm, accumulate,
                          paths_out, &clip, runs.data());
}

dp_status dp_ghost_norm_clip_layers_noalloc(void* stream, const dp_layer* layers, int32_t n_layers, dp_dtype dtype,
                                            int64_t B, dp_mode mode, int32_t kappa, float* sqnorm,
                                            int32_t accumulate, float C, float* c, float* norm,
                                            int32_t* paths_out) {
  if (!c) return DP_ERR_NULL;
  if (!aligned(c, 4) || (norm && !aligned(norm, 4))) return DP_ERR_ALIGN;
  if (!finite(C) || !(C > 0.0f)) return DP_ERR_VALUE;
  if (!layers) return DP_ERR_NULL;
  if (n_layers < 1 || n_layers > kNoAllocMaxLayers) return DP_ERR_SHAPE;
  dp_status s = check_norm_layers(layers, n_layers, dtype, B, mode, kappa);
  if (s != DP_OK) return s;
  if (!sqnorm) return DP_ERR_NULL;
  if (!aligned(sqnorm, 4)) return DP_ERR_ALIGN;
  NormRun runs[kNoAllocMaxLayers];  // on the stack: no heap either
  const int nr = plan_norm_runs(layers, n_layers, dtype, B, mode, kappa, runs);
  size_t need = 0;
  for (int r = 0; r < nr; ++r) need = std::max(need, run_ws_bytes(runs[r], layers, dtype, B, mode, kappa));
  if (need > kNoAllocScratchBytes) return DP_ERR_WORKSPACE;
  s = device_ready();
  if (s != DP_OK) return s;
  void* ws = nullptr;
  s = noalloc_scratch(&ws);
  if (s != DP_OK) return s;
  const ClipOut clip{C, c, norm};
  return norm_layers_impl(stream, layers, n_layers, dtype, B, mode, kappa, ws, kNoAllocScratchBytes, sqnorm,
                          accumulate, paths_out, &clip, runs);
}

// The multi-layer clipped sums. With accs, a layer whose split partials go
// through the grouped reduce has them added to accs[l] there (acc = acc + S,
// no noise, outs[l] untouched) and acc_done[l] is set; the caller adds the
// other layers' outs[l].
static dp_status sum_layers_impl(void* stream, const dp_layer* layers, int32_t n_layers, dp_dtype dtype, int64_t B,
                                 const float* c, float C, float sigma, float denom, uint64_t seed,
                                 const uint32_t* layer_ids, uint32_t step, void* workspace, size_t ws_bytes,
                                 float* const* outs, float* const* bias_outs, float* const* accs, char* acc_done) {
  dp_status s = check_layer_list(layers, n_layers, dtype, B);
  if (s != DP_OK) return s;
  if (!c || !outs) return DP_ERR_NULL;
  if (!aligned(c, 4)) return DP_ERR_ALIGN;
  if (!finite(C) || !(C > 0.0f) || !finite(sigma) || sigma < 0.0f || !finite(denom) || !(denom > 0.0f))
    return DP_ERR_VALUE;
  for (int32_t l = 0; l < n_layers; ++l) {
    const dp_layer& x = layers[l];
    if (!outs[l]) return DP_ERR_NULL;
    if (!aligned(outs[l], 4)) return DP_ERR_ALIGN;
    if (x.has_bias) {
      if (!bias_outs || !bias_outs[l]) return DP_ERR_NULL;
      if (!aligned(bias_outs[l], 4)) return DP_ERR_ALIGN;
    }
  }
  // plans of every launch, made once (the grouped launches check their own grid size)
  const std::vector<SumLaunch> launches = plan_sum_launches(layers, n_layers, dtype, B);
  std::vector<dpk::DlGroupPlan> gplans(launches.size());
  std::vector<dpk::ContractPlan> splans(launches.size());
  std::vector<size_t> grouped_ws;
  size_t single_ws = 0;
  for (size_t k = 0; k < launches.size(); ++k) {
    const SumLaunch& g = launches[k];
    const dp_layer& x0 = layers[g.first[0]];
    if (g.grouped) {
      gplans[k] = group_plan_of(g, layers, B);
      size_t w = 0;
      for (int j = 0; j < g.count; ++j)
        w += dpk::dl_layer_ws_bytes(gplans[k], j, layers[g.first[j]].d, layers[g.first[j]].p);
      grouped_ws.push_back(w);
    } else {
      const int hb = x0.has_bias ? 1 : 0;
      splans[k] = dpk::contract_plan(dtype, B, x0.T, x0.d, x0.p, hb);
      if (!grid_fits((uint64_t)splans[k].mt * splans[k].nt * splans[k].ks)) return DP_ERR_SHAPE;
      single_ws = std::max(single_ws, contract_ws_for(splans[k], x0.d, x0.p, hb));
    }
  }
  const SumWsLayout wl = sum_ws_layout(grouped_ws, single_ws);
  const size_t need = wl.total;
  if (need > 0) {
    if (!workspace) return DP_ERR_NULL;
    if (ws_bytes < need) return DP_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return DP_ERR_ALIGN;
  }
  s = device_ready();
  if (s != DP_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const float sc = sigma * C;
  auto lid = [&](int l) { return layer_ids ? layer_ids[l] : (uint32_t)l; };
  // The split reduce of the last shared launch, not yet issued (noise form):
  // the next shared launch runs it on its idle CUs when it can, else it is
  // issued on its own before the workspace region it reads is written again.
  dpk::SplitReduceLayer pend[dpk::kDlGroupMax];
  int npend = 0;
  auto flush = [&]() -> hipError_t {
    const hipError_t e = npend > 0 ? dpk::launch_split_reduce_group(st, pend, npend) : hipSuccess;
    npend = 0;
    return e;
  };
  int parts = 0;  // shared launches so far that left partials
  for (size_t k = 0; k < launches.size(); ++k) {
    const SumLaunch& g = launches[k];
    hipError_t e;
    if (g.grouped) {
      const dpk::DlGroupPlan& pl = gplans[k];
      dpk::DlLaunchLayer ll[dpk::kDlGroupMax];
      unsigned char* base = static_cast<unsigned char*>(workspace) + (wl.two ? (size_t)(parts % 2) * wl.region : 0);
      size_t off = 0;
      for (int k = 0; k < g.count; ++k) {
        const int l = g.first[k];
        const dp_layer& x = layers[l];
        const size_t wb = dpk::dl_layer_ws_bytes(pl, k, x.d, x.p);
        float* wsl = wb ? reinterpret_cast<float*>(base + off) : nullptr;
        off += wb;
        ll[k] = dpk::DlLaunchLayer{x.A, x.G, B, x.T, x.d, x.p, wsl, outs[l],
                                   dpk::make_noise_args(sc, denom, seed, lid(l), step)};
      }
      bool taken = false;
      e = dpk::launch_contract_dl_group(st, ll, g.count, c, pl, npend > 0 ? pend : nullptr, npend, &taken);
      if (taken) npend = 0;
      if (e == hipSuccess) e = flush();  // not taken: the pending reduce reads the other region
      // the split tiles' partials (and the 256x256 tiles') -> outputs, one reduce launch for the
      // group: issued now in the accumulating form, else left pending for the next launch
      dpk::SplitReduceLayer rl[dpk::kDlGroupMax];
      int nr = 0;
      for (int k = 0; k < g.count; ++k)
        if (pl.ks[k] > 1 || pl.bn == 256) {
          float* acc = accs ? accs[g.first[k]] : nullptr;
          rl[nr++] = dpk::SplitReduceLayer{ll[k].ws, pl.ks[k], ll[k].d, ll[k].p, ll[k].na, ll[k].out, acc};
          if (acc) acc_done[g.first[k]] = 1;
        }
      if (nr > 0) ++parts;
      if (e == hipSuccess && nr > 0) {
        if (accs) {
          e = dpk::launch_split_reduce_group(st, rl, nr);
        } else {
          for (int r = 0; r < nr; ++r) pend[r] = rl[r];
          npend = nr;
        }
      }
    } else {
      e = flush();  // the single-layer launch writes the start of the workspace
      if (e != hipSuccess) return DP_ERR_HIP;
      const int l = g.first[0];
      const dp_layer& x = layers[l];
      const int hb = x.has_bias ? 1 : 0;
      e = dpk::launch_clipped_sum(st, dtype, x.A, x.G, c, B, x.T, x.d, x.p, splans[k], static_cast<float*>(workspace), sc,
                                  denom, seed, lid(l), step, outs[l], hb ? bias_outs[l] : nullptr);
    }
    if (e != hipSuccess) return DP_ERR_HIP;
  }
  if (flush() != hipSuccess) return DP_ERR_HIP;
  return DP_OK;
}

dp_status dp_clipped_sum_noise_layers(void* stream, const dp_layer* layers, int32_t n_layers, dp_dtype dtype,
                                      int64_t B, const float* c, float C, float sigma, float denom, uint64_t seed,
                                      const uint32_t* layer_ids, uint32_t step, void* workspace, size_t ws_bytes,
                                      float* const* outs, float* const* bias_outs) {
  return sum_layers_impl(stream, layers, n_layers, dtype, B, c, C, sigma, denom, seed, layer_ids, step, workspace,
                         ws_bytes, outs, bias_outs, nullptr, nullptr);
}

dp_status dp_clip_factors(void* stream, const float* sqnorm, int64_t B, float C, float* c, float* norm) {
  if (!sqnorm || !c) return DP_ERR_NULL;
  if (B < 1 || B >= kMaxDim) return DP_ERR_SHAPE;
  if (!finite(C) || !(C > 0.0f)) return DP_ERR_VALUE;
  if (!aligned(sqnorm, 4) || !aligned(c, 4) || (norm && !aligned(norm, 4))) return DP_ERR_ALIGN;
  dp_status s = device_ready();
  if (s != DP_OK) return s;
  return hip_status(dpk::launch_clip_factors(static_cast<hipStream_t>(stream), sqnorm, B, C, c, norm));
}

dp_status dp_clipped_sum_noise(void* stream, const void* A, const void* G, dp_dtype dtype, int64_t B, int64_t T,
                               int64_t d, int64_t p, const float* c, float C, float sigma, float denom, uint64_t seed,
                               uint32_t layer_id, uint32_t step, void* workspace, size_t ws_bytes, float* out,
                               float* bias_out) {
  dp_status s = check_layer(A, G, dtype, B, T, d, p);
  if (s != DP_OK) return s;
  if (!c || !out) return DP_ERR_NULL;
  if (!aligned(c, 4) || !aligned(out, 4) || (bias_out && !aligned(bias_out, 4))) return DP_ERR_ALIGN;
  if (!finite(C) || !(C > 0.0f) || !finite(sigma) || sigma < 0.0f || !finite(denom) || !(denom > 0.0f))
    return DP_ERR_VALUE;
  const int hb = bias_out ? 1 : 0;
  const dpk::ContractPlan pl = dpk::contract_plan(dtype, B, T, d, p, hb);
  const size_t need = contract_ws_for(pl, d, p, hb);
  if (need > 0) {
    if (!workspace) return DP_ERR_NULL;
    if (ws_bytes < need) return DP_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return DP_ERR_ALIGN;
  }
  if (!grid_fits((uint64_t)pl.mt * pl.nt * pl.ks)) return DP_ERR_SHAPE;
  s = device_ready();
  if (s != DP_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const float sc = sigma * C;
  return hip_status(dpk::launch_clipped_sum(st, dtype, A, G, c, B, T, d, p, pl, static_cast<float*>(workspace), sc,
                                            denom, seed, layer_id, step, out, bias_out));
}

size_t dp_conv_workspace_bytes(const dp_conv2d* conv, dp_dtype dtype, int64_t B, int64_t p, int32_t has_bias,
                               dp_mode mode, int32_t kappa) {
  alignas(16) static const float probe[4] = {};  // stands in for the data pointers: only the shapes are checked
  dpk::ConvGeo g;
  if (!conv || check_conv(probe, probe, conv, dtype, B, p, &g) != DP_OK) return 0;
  if (mode < DP_MODE_MIXED || mode > DP_MODE_TIME || kappa < 1) return 0;
  const int hb = has_bias ? 1 : 0;
  const size_t a = conv_norm_ws_bytes(conv_path(g.T, g.d, p, mode, kappa), B, g.T, g.d, p, hb);
  const size_t b = conv_sum_ws_bytes(dpk::tiles_plan(dtype, B, g.T, g.d, p, hb, true), g.d, p, hb);
  return std::max(a, b);
}

dp_status dp_conv_norm(void* stream, const void* a, const void* G, const dp_conv2d* conv, dp_dtype dtype, int64_t B,
                       int64_t p, int32_t has_bias, dp_mode mode, int32_t kappa, void* workspace, size_t ws_bytes,
                       float* sqnorm, int32_t accumulate, int32_t* path_out) {
  dpk::ConvGeo g;
  dp_status s = check_conv(a, G, conv, dtype, B, p, &g);
  if (s != DP_OK) return s;
  if (!sqnorm) return DP_ERR_NULL;
  if (!aligned(sqnorm, 4)) return DP_ERR_ALIGN;
  if (mode < DP_MODE_MIXED || mode > DP_MODE_TIME || kappa < 1) return DP_ERR_VALUE;
  const int hb = has_bias ? 1 : 0;
  const int path = conv_path(g.T, g.d, p, mode, kappa);
  const int64_t nt = conv_norm_ntiles(path, g.T, g.d, p, hb);
  if (nt > kMaxTilesPerSample) return DP_ERR_SHAPE;
  if (!grid_fits((uint64_t)((B + 7) / 8 * 8) * (uint64_t)nt)) return DP_ERR_SHAPE;
  const size_t need = conv_norm_ws_bytes(path, B, g.T, g.d, p, hb);
  if (need > 0) {
    if (!workspace) return DP_ERR_NULL;
    if (ws_bytes < need) return DP_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return DP_ERR_ALIGN;
  }
  s = device_ready();
  if (s != DP_OK) return s;
  if (path_out) *path_out = path;
  const dpk::NormSink sink = dpk::make_norm_sink(static_cast<float*>(workspace), sqnorm, (int)nt, accumulate ? 1 : 0);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = path == DP_PATH_GHOST ? dpk::launch_ghost_conv(st, dtype, g, G, B, p, hb, sink)
                                             : dpk::launch_explicit_conv(st, dtype, g, G, B, p, hb, sink);
  return hip_status(e == hipSuccess ? dpk::launch_norm_finish(st, sink, B) : e);
}

dp_status dp_unfold2d(void* stream, const void* a, const dp_conv2d* conv, dp_dtype dtype, int64_t B, void* U) {
  dpk::ConvGeo g;
  // U stands where the conv calls take G: non-NULL and 16-byte aligned
  dp_status s = check_conv(a, U, conv, dtype, B, 1, &g);
  if (s != DP_OK) return s;
  if ((int64_t)g.T * g.d >= kMaxConv || (((int64_t)g.T * g.d + 255) / 256) * B >= kMaxConv) return DP_ERR_SHAPE;
  s = device_ready();
  if (s != DP_OK) return s;
  return hip_status(dpk::launch_unfold2d(static_cast<hipStream_t>(stream), dtype, g, B, U));
}

dp_status dp_conv_clipped_sum_noise(void* stream, const void* a, const void* G, const dp_conv2d* conv, dp_dtype dtype,
                                    int64_t B, int64_t p, const float* c, float C, float sigma, float denom,
                                    uint64_t seed, uint32_t layer_id, uint32_t step, void* workspace, size_t ws_bytes,
                                    float* out, float* bias_out) {
  dpk::ConvGeo g;
  dp_status s = check_conv(a, G, conv, dtype, B, p, &g);
  if (s != DP_OK) return s;
  if (!c || !out) return DP_ERR_NULL;
  if (!aligned(c, 4) || !aligned(out, 4) || (bias_out && !aligned(bias_out, 4))) return DP_ERR_ALIGN;
  if (!finite(C) || !(C > 0.0f) || !finite(sigma) || sigma < 0.0f || !finite(denom) || !(denom > 0.0f))
    return DP_ERR_VALUE;
  const int hb = bias_out ? 1 : 0;
  const dpk::ContractPlan pl = dpk::tiles_plan(dtype, B, g.T, g.d, p, hb, true);
  const size_t need = conv_sum_ws_bytes(pl, g.d, p, hb);
  if (need > 0) {
    if (!workspace) return DP_ERR_NULL;
    if (ws_bytes < need) return DP_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return DP_ERR_ALIGN;
  }
  if (!grid_fits((uint64_t)pl.mt * pl.nt * pl.ks)) return DP_ERR_SHAPE;
  s = device_ready();
  if (s != DP_OK) return s;
  return hip_status(dpk::launch_clipped_sum_conv(static_cast<hipStream_t>(stream), dtype, g, G, c, B, p, pl,
                                                 static_cast<float*>(workspace), sigma * C, denom, seed, layer_id,
                                                 step, out, bias_out));
}

size_t dp_layers_accumulate_workspace_bytes(const dp_layer* layers, int32_t n_layers, dp_dtype dtype, int64_t B) {
  if (check_layer_list(layers, n_layers, dtype, B) != DP_OK) return 0;
  size_t w = round256(sum_layers_ws_bytes(layers, n_layers, dtype, B));
  for (int32_t l = 0; l < n_layers; ++l)
    w += round256((size_t)(layers[l].d + (layers[l].has_bias ? 1 : 0)) * (size_t)layers[l].p * sizeof(float));
  return w;
}

dp_status dp_clipped_sum_accumulate_layers(void* stream, const dp_layer* layers, int32_t n_layers, dp_dtype dtype,
                                           int64_t B, const float* c, void* workspace, size_t ws_bytes,
                                           float* const* accs, float* const* bias_accs, int32_t accumulate) {
  dp_status s = check_layer_list(layers, n_layers, dtype, B);
  if (s != DP_OK) return s;
  if (!c || !accs) return DP_ERR_NULL;
  const size_t sum_ws = round256(sum_layers_ws_bytes(layers, n_layers, dtype, B));
  // the physical batch's clipped sums, exactly: (S + 0*z) * 1 = S
  if (!accumulate)
    return dp_clipped_sum_noise_layers(stream, layers, n_layers, dtype, B, c, 1.0f, 0.0f, 1.0f, 0, nullptr, 0,
                                       workspace, ws_bytes, accs, bias_accs);
  for (int32_t l = 0; l < n_layers; ++l) {
    if (!accs[l]) return DP_ERR_NULL;
    if (!aligned(accs[l], 4)) return DP_ERR_ALIGN;
    if (layers[l].has_bias && (!bias_accs || !bias_accs[l])) return DP_ERR_NULL;
    if (layers[l].has_bias && !aligned(bias_accs[l], 4)) return DP_ERR_ALIGN;
  }
  const size_t need = dp_layers_accumulate_workspace_bytes(layers, n_layers, dtype, B);
  if (!workspace) return DP_ERR_NULL;
  if (ws_bytes < need) return DP_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return DP_ERR_ALIGN;
  // per layer: its sum (and bias sum) after the clipped sums' own workspace
  std::vector<float*> sums((size_t)n_layers), bsums((size_t)n_layers, nullptr);
  size_t off = sum_ws;
  for (int32_t l = 0; l < n_layers; ++l) {
    float* base = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + off);
    sums[l] = base;
    if (layers[l].has_bias) bsums[l] = base + layers[l].d * layers[l].p;
    off += round256((size_t)(layers[l].d + (layers[l].has_bias ? 1 : 0)) * (size_t)layers[l].p * sizeof(float));
  }
  // split partials that go through the grouped reduce are added to accs there
  std::vector<char> done((size_t)n_layers, 0);
  s = sum_layers_impl(stream, layers, n_layers, dtype, B, c, 1.0f, 0.0f, 1.0f, 0, nullptr, 0, workspace, sum_ws,
                      sums.data(), bsums.data(), accs, done.data());
  if (s != DP_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int32_t l = 0; l < n_layers; ++l) {
    hipError_t e = done[l] ? hipSuccess : dpk::launch_accumulate(st, accs[l], sums[l], layers[l].d * layers[l].p);
    if (e == hipSuccess && layers[l].has_bias) e = dpk::launch_accumulate(st, bias_accs[l], bsums[l], layers[l].p);
    if (e != hipSuccess) return DP_ERR_HIP;
  }
  return DP_OK;
}

size_t dp_accumulate_workspace_bytes(dp_dtype dtype, int64_t B, int64_t T, int64_t d, int64_t p, int32_t has_bias) {
  if (check_shape(B, T, d, p) != DP_OK) return 0;
  if (dtype != DP_F32 && dtype != DP_BF16) return 0;
  const int hb = has_bias ? 1 : 0;
  return round256(contract_ws_bytes(dtype, B, T, d, p, hb)) + round256((size_t)(d + hb) * (size_t)p * sizeof(float));
}

dp_status dp_clipped_sum_accumulate(void* stream, const void* A, const void* G, dp_dtype dtype, int64_t B, int64_t T,
                                    int64_t d, int64_t p, const float* c, void* workspace, size_t ws_bytes,
                                    float* acc, float* bias_acc, int32_t accumulate) {
  dp_status s = check_layer(A, G, dtype, B, T, d, p);
  if (s != DP_OK) return s;
  if (!c || !acc) return DP_ERR_NULL;
  if (!aligned(c, 4) || !aligned(acc, 4) || (bias_acc && !aligned(bias_acc, 4))) return DP_ERR_ALIGN;
  const int hb = bias_acc ? 1 : 0;
  const dpk::ContractPlan pl = dpk::contract_plan(dtype, B, T, d, p, hb);
  if (!grid_fits((uint64_t)pl.mt * pl.nt * pl.ks)) return DP_ERR_SHAPE;
  const size_t cws = round256(contract_ws_for(pl, d, p, hb));
  const size_t need = accumulate ? cws + round256((size_t)(d + hb) * (size_t)p * sizeof(float)) : cws;
  if (need > 0) {
    if (!workspace) return DP_ERR_NULL;
    if (ws_bytes < need) return DP_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return DP_ERR_ALIGN;
  }
  s = device_ready();
  if (s != DP_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* ws = static_cast<float*>(workspace);
  // the physical batch's clipped sum, exactly: (S + 0*z) * 1 = S
  if (!accumulate)
    return hip_status(dpk::launch_clipped_sum(st, dtype, A, G, c, B, T, d, p, pl, ws, 0.0f, 1.0f, 0, 0, 0, acc,
                                              bias_acc));
  float* sum = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + cws);
  float* bias_sum = hb ? sum + d * p : nullptr;
  hipError_t e = dpk::launch_clipped_sum(st, dtype, A, G, c, B, T, d, p, pl, ws, 0.0f, 1.0f, 0, 0, 0, sum, bias_sum);
  if (e == hipSuccess) e = dpk::launch_accumulate(st, acc, sum, d * p);
  if (e == hipSuccess && hb) e = dpk::launch_accumulate(st, bias_acc, bias_sum, p);
  return hip_status(e);
}

dp_status dp_noise_mean(void* stream, const float* acc, const float* bias_acc, int64_t d, int64_t p, float C,
                        float sigma, float denom, uint64_t seed, uint32_t layer_id, uint32_t step, float* out,
                        float* bias_out) {
  if (!acc || !out) return DP_ERR_NULL;
  if ((bias_acc != nullptr) != (bias_out != nullptr)) return DP_ERR_NULL;
  if (check_shape(1, 1, d, p) != DP_OK) return DP_ERR_SHAPE;
  if (!aligned(acc, 4) || !aligned(out, 4) || (bias_acc && (!aligned(bias_acc, 4) || !aligned(bias_out, 4))))
    return DP_ERR_ALIGN;
  if (!finite(C) || !(C > 0.0f) || !finite(sigma) || sigma < 0.0f || !finite(denom) || !(denom > 0.0f))
    return DP_ERR_VALUE;
  dp_status s = device_ready();
  if (s != DP_OK) return s;
  return hip_status(dpk::launch_noise_mean(static_cast<hipStream_t>(stream), acc, bias_acc, d, p,
                                           dpk::make_noise_args(sigma * C, denom, seed, layer_id, step), out,
                                           bias_out));
}

dp_status dp_adaptive_threshold(void* stream, const float* norm, int64_t B, float C_prev, float alpha, float beta,
                                float sigma_l2, int32_t init, uint64_t seed, uint32_t layer_id, uint32_t step,
                                float* C_next, float* C_l2_out) {
  if (!norm || !C_next) return DP_ERR_NULL;
  if (B < 1 || B >= kMaxDim) return DP_ERR_SHAPE;
  if (!aligned(norm, 4) || !aligned(C_next, 4) || (C_l2_out && !aligned(C_l2_out, 4))) return DP_ERR_ALIGN;
  if (!finite(alpha) || !(alpha > 0.0f) || !finite(beta) || !(beta > 0.0f) || !finite(sigma_l2) || sigma_l2 < 0.0f)
    return DP_ERR_VALUE;
  if (!init && (!finite(C_prev) || !(C_prev > 0.0f))) return DP_ERR_VALUE;
  dp_status s = device_ready();
  if (s != DP_OK) return s;
  return hip_status(dpk::launch_adaptive_threshold(static_cast<hipStream_t>(stream), norm, B, C_prev, alpha, beta,
                                                   sigma_l2, init ? 1 : 0, seed, layer_id, step, C_next, C_l2_out));
}

}  // extern "C"
