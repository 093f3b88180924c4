// Dispatch of the weight-streaming MFMA kernels (their templates are in
// gemm_stream_kernels.hpp, instantiated per format in gemm_stream_<format>.hip):
// launch geometry, the K-split plan and the choice of kernel for a shape.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "common.hpp"
#include "gemm_stream_geom.hpp"
#include "internal.hpp"

namespace qg {
namespace {

// y[bi][16 t + r] = sum over parts, in part order, of slot (part, t) output
// 16 bi + r; rounded once to fp16.  Each thread adds four consecutive
// outputs (four weight rows of one batch row).
__global__ void __launch_bounds__(256)
split_finish_kernel(const float* __restrict__ ws, _Float16* __restrict__ y, SplitGeom sg) {
  const StreamGeom& g = sg.s;
  const uint32_t i = (blockIdx.x * 256u + threadIdx.x) * 4u;
  const uint32_t vals = (uint32_t)sg.vals;
  if (i >= (uint32_t)g.tiles * vals) return;
  const uint32_t t = i / vals, j = i % vals;
  f4 sum = f4{0.0f, 0.0f, 0.0f, 0.0f};
  const size_t stride = (size_t)g.tiles * vals;
  const f4* src = reinterpret_cast<const f4*>(ws + (size_t)t * vals + j);
  for (int p = 0; p < sg.parts; ++p) sum += src[(size_t)p * stride / 4];
  const int bi = (int)(j >> 4), row = (int)(t * 16u + (j & 15u));
  const __amdgpu_buffer_rsrc_t yrs = make_rsrc(y, g.y_bytes);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t off = (bi < g.b && row + e < g.n) ? ((uint32_t)bi * (uint32_t)g.n + (uint32_t)(row + e)) * 2u
                                                      : 0xFFFFFF00u;
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)sum[e]), yrs, off, 0, 0);
  }
}

// Finish for the lane-order slots of the LDS form: thread j adds the four
// batch rows 16 t + 4 q + i (i = 0..3) of weight row r16 over the parts.
__global__ void __launch_bounds__(256)
split_finish_lane_kernel(const float* __restrict__ ws, _Float16* __restrict__ y, SplitGeom sg) {
  const StreamGeom& g = sg.s;
  const uint32_t i = (blockIdx.x * 256u + threadIdx.x) * 4u;
  const uint32_t vals = (uint32_t)sg.vals;
  if (i >= (uint32_t)g.tiles * vals) return;
  const uint32_t tile = i / vals, j = i % vals;
  f4 sum = f4{0.0f, 0.0f, 0.0f, 0.0f};
  const size_t stride = (size_t)g.tiles * vals;
  const f4* src = reinterpret_cast<const f4*>(ws + (size_t)tile * vals + j);
  for (int p = 0; p < sg.parts; ++p) sum += src[(size_t)p * stride / 4];
  const uint32_t t = j >> 8, l = (j >> 2) & 63;
  const int row = (int)(tile * 16u + (l & 15u)), b0 = (int)(16u * t + 4u * (l >> 4));
  const __amdgpu_buffer_rsrc_t yrs = make_rsrc(y, g.y_bytes);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t off = (b0 + e < g.b && row < g.n) ? ((uint32_t)(b0 + e) * (uint32_t)g.n + (uint32_t)row) * 2u
                                                      : 0xFFFFFF00u;
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)sum[e]), yrs, off, 0, 0);
  }
}

// MFMA steps per group (group / 32) for the group formats; 4 otherwise.
int stream_gs(const WeightView& w) {
  const bool grouped = w.fmt == Q_INT4_ASYM || w.fmt == Q_FP4_E2M1 || is_razer(w.fmt) || is_afpq(w.fmt);
  return grouped ? w.group / 32 : 4;
}

// Byte geometry shared by both launchers.
void fill_geom(const WeightView& w, int b, StreamGeom& g) {
  g.n = w.n;
  g.k = w.k;
  g.b = b;
  g.batch_tiles = (b + 15) / 16;
  g.tiles = (w.n + 15) / 16;
  g.chunks = (w.k + 127) / 128;
  g.gshift = ilog2(w.group);
  const int G = w.k / w.group;
  const uint64_t n = (uint64_t)w.n;
  g.codes_row = (uint32_t)(w.fmt == Q_INT8 ? w.k : is_fp3(w.fmt) ? w.k / 32 * 12 : w.k / 2);
  g.hi_row = (uint32_t)(w.k / 4);
  g.scales_row = (uint32_t)(w.fmt == Q_INT8 ? 2 : G * (is_afpq(w.fmt) ? 4 : 2));
  g.aux_row = (uint32_t)(w.fmt == Q_INT4_ASYM ? (G + 7) / 8 * 4 : is_razer(w.fmt) ? (G + 15) / 16 * 4 : w.k / 16);
  // whole allocations, pad included: a metadata run that starts off a
  // 4-byte boundary is read from the boundary below and may end in the pad
  g.codes_bytes = (uint32_t)buffer_bytes(w.fmt, w.n, w.k, w.group, Q_BUF_CODES);
  g.hi_bytes = (uint32_t)buffer_bytes(w.fmt, w.n, w.k, w.group, Q_BUF_CODES_HI);
  g.scales_bytes = (uint32_t)buffer_bytes(w.fmt, w.n, w.k, w.group, Q_BUF_SCALES);
  g.aux_bytes = (uint32_t)buffer_bytes(w.fmt, w.n, w.k, w.group, Q_BUF_AUX);
  g.x_bytes = (uint32_t)(b * w.k * 2);
  g.y_bytes = (uint32_t)((uint64_t)b * n * 2u);
}

struct SplitPlan {
  int kc, parts;
  uint64_t ws_bytes;
};

// Smallest batch at which the split form runs by default, from
// measurements on MI355X.  The split pays a second launch and a workspace
// round trip (about 3.5 us); it gains where the full-K kernel streams the
// activations with the weights (k > 8192: from b = 4 for groups of 32,
// whose full-K slices decode the most groups, b = 8 for groups of 128 and
// 256, b = 16 otherwise), where its batch tiles each re-read a large weight
// matrix (two batch tiles or more, b > 16, on 16 MiB and more, AFPQ
// included), and for the block formats, whose full-K slices carry the
// heaviest activation prologue.
int split_min_b_default(const WeightView& w) {
  if (w.fmt == Q_BFP6 || w.fmt == Q_BFP4) return 8;
  if (w.k > 8192) {
    if (is_afpq(w.fmt) || w.fmt == Q_INT8) return 16;
    return w.group <= 32 ? 4 : w.group == 64 ? 16 : 8;
  }
  if (is_afpq(w.fmt)) return 17;
  size_t bytes = 0;
  for (int which = Q_BUF_CODES; which <= Q_BUF_AUX; ++which) bytes += buffer_bytes(w.fmt, w.n, w.k, w.group, which);
  return bytes >= ((size_t)16 << 20) ? 17 : Q_MAX_BATCH + 1;
}

// Chunks per wave of the split form: two for groups of 256 (a group spans
// two chunks).  Two also, from measurements on MI355X, where halving the
// parts -- and with them the per-tile LDS reduction per weight byte, the
// workspace and the finishing reads -- gains 5-14%: one batch tile
// (b <= 16) of INT4, E2M1 and RaZeR at K above 8192; more batch tiles of
// those and INT8 at K above 8192 or 32 MiB of packed weights.  AFPQ, the
// block formats and smaller matrices lose.  QGEMV_SPLIT_KC = 1 or 2
// overrides the choice (tuning).
int split_kc(const WeightView& w, int b, int gs) {
  if (gs == 8) return 2;
  const int forced = tuning(kTuneSplitKc, 0);
  if (forced == 1 || forced == 2) return forced;
  const bool plain4 = w.fmt == Q_INT4_ASYM || w.fmt == Q_FP4_E2M1 || w.fmt == Q_FP4_RAZER;
  if (b <= 16) return plain4 && w.k > 8192 ? 2 : 1;
  size_t bytes = 0;
  for (int which = Q_BUF_CODES; which <= Q_BUF_AUX; ++which) bytes += buffer_bytes(w.fmt, w.n, w.k, w.group, which);
  const bool large = w.k > 8192 || bytes >= ((size_t)32 << 20);
  return (plain4 || w.fmt == Q_INT8) && large ? 2 : 1;
}

// The K-split plan for (w, b), or false when the call runs the full-K kernel:
// batches below the minimum (QGEMV_SPLIT_MIN_B overrides the default above;
// 0 disables the split), a K that one workgroup covers whole, or a workspace
// past 32-bit offsets.
bool split_plan(const WeightView& w, int b, SplitPlan& plan) {
  const int min_b = tuning(kTuneSplitMinB, split_min_b_default(w));
  if (min_b <= 0 || b < min_b || b > Q_MAX_BATCH) return false;
  const int chunks = (w.k + 127) / 128;
  const int gs = stream_gs(w);
  plan.kc = split_kc(w, b, gs);
  plan.parts = (chunks + kSplitWaves * plan.kc - 1) / (kSplitWaves * plan.kc);
  if (plan.parts < 2) return false;
  const uint64_t tiles = (uint64_t)((w.n + 15) / 16);
  plan.ws_bytes = (uint64_t)plan.parts * tiles * (uint64_t)((b + 15) / 16) * 256u * 4u;
  return plan.ws_bytes <= 0xFFFFFF00u;
}

}  // namespace

bool gemm_stream_supported(const WeightView& w, int b) {
  const int chunks = (w.k + 127) / 128;  // up to 8 waves of 16 chunks (k <= Q_MAX_K)
  return b >= 1 && b <= Q_MAX_BATCH && chunks <= 8 * 16 && (uint64_t)b * (uint64_t)w.n * 2u <= 0xFFFFFF00u;
}

size_t gemm_split_workspace(const WeightView& w, int b) {
  SplitPlan plan;
  return split_plan(w, b, plan) ? (size_t)plan.ws_bytes : 0;
}

hipError_t launch_gemm_split(const WeightView& w, const _Float16* x, _Float16* y, int b, void* ws, size_t ws_bytes,
                             hipStream_t s) {
  SplitPlan plan;
  if (!split_plan(w, b, plan) || ws == nullptr || ws_bytes < plan.ws_bytes) return hipErrorInvalidValue;
  SplitGeom sg;
  fill_geom(w, b, sg.s);
  sg.parts = plan.parts;
  sg.vals = sg.s.batch_tiles * 256;
  sg.ws_bytes = (uint32_t)plan.ws_bytes;
  const int gs = stream_gs(w);
  SplitKernelFn fn;
  const int bt = sg.s.batch_tiles;
  // the LDS form for AFPQ (its 4-byte scale pairs of 64-element groups make
  // the register form's per-chunk metadata loads the costliest), else the
  // register form; QGEMV_SPLIT_LDS = 0 / 1 forces one (tuning and tests)
  const bool lds = tuning(kTuneSplitLds, is_afpq(w.fmt) ? 1 : 0) != 0 && plan.kc == 1;
  switch (w.fmt) {
    case Q_INT4_ASYM: fn = split_kernel_for<Q_INT4_ASYM>(gs, bt, plan.kc, lds); break;
    case Q_FP4_E2M1: fn = split_kernel_for<Q_FP4_E2M1>(gs, bt, plan.kc, lds); break;
    case Q_FP4_RAZER: fn = split_kernel_for<Q_FP4_RAZER>(gs, bt, plan.kc, lds); break;
    case Q_FP4_AFPQ: fn = split_kernel_for<Q_FP4_AFPQ>(gs, bt, plan.kc, lds); break;
    case Q_BFP6: fn = split_kernel_for<Q_BFP6>(gs, bt, plan.kc, lds); break;
    case Q_BFP4: fn = split_kernel_for<Q_BFP4>(gs, bt, plan.kc, lds); break;
    case Q_INT8: fn = split_kernel_for<Q_INT8>(gs, bt, plan.kc, lds); break;
    case Q_FP3_RAZER: fn = split_kernel_for<Q_FP3_RAZER>(gs, bt, plan.kc, lds); break;
    case Q_FP3_AFPQ: fn = split_kernel_for<Q_FP3_AFPQ>(gs, bt, plan.kc, lds); break;
    default: return hipErrorInvalidValue;
  }
  // one persistent workgroup of 8 waves per compute unit, split evenly over
  // the parts (QGEMV_SPLIT_GRID_ROWS overrides the workgroups per part)
  int grid_rows = device_cu_count() / plan.parts;
  const int rows_env = tuning(kTuneSplitGridRows, 0);
  if (rows_env > 0) grid_rows = rows_env;
  if (grid_rows < 1) grid_rows = 1;
  if (grid_rows > sg.s.tiles) grid_rows = sg.s.tiles;
  // (the LDS form walks tiles per wave: no more workgroups than 8 tiles each)
  if (lds && grid_rows * kSplitWaves > sg.s.tiles) grid_rows = (sg.s.tiles + kSplitWaves - 1) / kSplitWaves;
  sg.grid_rows = grid_rows;
  float* wsf = static_cast<float*>(ws);
  hipLaunchKernelGGL(fn, dim3(grid_rows * plan.parts), dim3(64 * kSplitWaves), 0, s, w, x, wsf, sg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint64_t quads = (uint64_t)sg.s.tiles * (uint64_t)sg.vals / 4;
  if (lds)
    hipLaunchKernelGGL(split_finish_lane_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, s, wsf, y, sg);
  else
    hipLaunchKernelGGL(split_finish_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, s, wsf, y, sg);
  return hipGetLastError();
}

hipError_t launch_gemm_stream(const WeightView& w, const _Float16* x, _Float16* y, int b, hipStream_t s) {
  if (!gemm_stream_supported(w, b)) return hipErrorInvalidValue;
  StreamGeom g;
  fill_geom(w, b, g);
  const int gs = stream_gs(w);
  const bool xs = g.chunks > 8 * 8;  // slices of x too large for registers: stream them
  // chunks per wave: the smallest slice that keeps the workgroup within
  // max_waves (QGEMV_STREAM_MAX_WAVES, up to 16, trades registers for
  // waves); groups of 256 span two chunks, so their slices hold at least two
  // defaults from sweeps on MI355X: one tile in flight; up to 16 waves for
  // the block formats (their decode is the heaviest), 8 otherwise
  const bool block = w.fmt == Q_BFP6 || w.fmt == Q_BFP4;
  int max_waves = tuning(kTuneStreamMaxWaves, block ? 16 : 8);
  if (max_waves < 1 || max_waves > kStreamMaxWaves) max_waves = 8;
  int depth = 1;  // tiles in flight (two measured no faster)
  int kc = gs == 8 ? 2 : 1;
  if (xs) {
    kc = 16;  // 16 chunks per wave, up to 8 waves (k <= Q_MAX_K)
    if ((g.chunks + kc - 1) / kc > 8) return hipErrorInvalidValue;
  } else {
    while (kc < 8 && (g.chunks + kc - 1) / kc > std::min(max_waves, stream_max_waves(kc, gs, depth))) kc *= 2;
    const int kc_env = tuning(kTuneStreamKc, 0);  // tuning override: 1, 2, 4 or 8
    if ((kc_env == 1 || kc_env == 2 || kc_env == 4 || kc_env == 8) && kc_env > kc) kc = kc_env;
    if (kc >= 8) depth = 1;
    if ((g.chunks + kc - 1) / kc > stream_max_waves(kc, gs, depth)) return hipErrorInvalidValue;
  }
  const int ks = (g.chunks + kc - 1) / kc;
  StreamKernelFn fn;
  switch (w.fmt) {
    case Q_INT4_ASYM: fn = stream_kernel_for<Q_INT4_ASYM>(kc, gs, depth, xs); break;
    case Q_FP4_E2M1: fn = stream_kernel_for<Q_FP4_E2M1>(kc, gs, depth, xs); break;
    case Q_FP4_RAZER: fn = stream_kernel_for<Q_FP4_RAZER>(kc, gs, depth, xs); break;
    case Q_FP4_AFPQ: fn = stream_kernel_for<Q_FP4_AFPQ>(kc, gs, depth, xs); break;
    case Q_BFP6: fn = stream_kernel_for<Q_BFP6>(kc, gs, depth, xs); break;
    case Q_BFP4: fn = stream_kernel_for<Q_BFP4>(kc, gs, depth, xs); break;
    case Q_INT8: fn = stream_kernel_for<Q_INT8>(kc, gs, depth, xs); break;
    case Q_FP3_RAZER: fn = stream_kernel_for<Q_FP3_RAZER>(kc, gs, depth, xs); break;
    case Q_FP3_AFPQ: fn = stream_kernel_for<Q_FP3_AFPQ>(kc, gs, depth, xs); break;
    default: return hipErrorInvalidValue;
  }
  // persistent workgroups: QGEMV_STREAM_WAVES_PER_CU waves per compute unit
  // (default 8: one workgroup per compute unit does best)
  const int waves_per_cu = tuning(kTuneStreamWavesPerCu, 8);
  int per_cu = waves_per_cu / ks;
  if (per_cu < 1) per_cu = 1;
  // (counted over all batch tiles: each gets an equal share of the grid)
  int grid_rows = device_cu_count() * per_cu / g.batch_tiles;
  if (grid_rows > 8) grid_rows -= grid_rows % 8;  // XCD-aligned row groups (see batch_tile_of)
  const int rows_env = tuning(kTuneStreamGridRows, 0);  // tuning override
  if (rows_env > 0) grid_rows = rows_env;
  if (grid_rows < 1) grid_rows = 1;
  if (grid_rows > g.tiles) grid_rows = g.tiles;
  hipLaunchKernelGGL(fn, dim3(grid_rows * g.batch_tiles), dim3(64 * ks), 0, s, w, x, y, g);
  return hipGetLastError();
}

}  // namespace qg
