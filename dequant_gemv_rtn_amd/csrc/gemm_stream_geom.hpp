// Launch geometry of the weight-streaming MFMA kernels, shared by their
// dispatch (gemm_stream.hip) and the per-format units that instantiate them
// (gemm_stream_<format>.hip, from the templates in gemm_stream_kernels.hpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace qg {

constexpr int kStreamMaxWaves = 16;
constexpr int kSplitWaves = 8;

struct StreamGeom {
  int n, k, b;
  int batch_tiles;  // ceil(b / 16)
  int tiles;   // ceil(n / 16)
  int chunks;  // ceil(k / 128)
  int gshift;  // log2(group) for the group formats
  uint32_t codes_row, hi_row, scales_row, aux_row;  // bytes per weight row
  uint32_t codes_bytes, hi_bytes, scales_bytes, aux_bytes, x_bytes, y_bytes;
};

struct SplitGeom {
  StreamGeom s;
  int parts;      // K-parts: workgroups per row tile
  int grid_rows;  // workgroups per part; workgroup id = rg * parts + part
  int vals;       // outputs of one (part, row tile) slot: batch_tiles * 256
  uint32_t ws_bytes;
};

// Workgroups of up to 16 waves, except where the registers of a slice leave
// room for two waves per SIMD only: 8-chunk slices, and 4-chunk slices with a
// ring two tiles deep or extra metadata (groups shorter than a chunk).
__host__ __device__ constexpr int stream_max_waves(int kc, int gs, int depth) {
  return (kc >= 8 || (kc == 4 && (gs < 4 || depth > 1))) ? 8 : kStreamMaxWaves;
}

typedef void (*StreamKernelFn)(WeightView, const _Float16*, _Float16*, StreamGeom);
typedef void (*SplitKernelFn)(WeightView, const _Float16*, float*, SplitGeom);

// The kernel that serves format FMT at a launch shape.  Defined in
// gemm_stream_kernels.hpp and instantiated once per format, each in its own
// translation unit (they compile in parallel).
//   stream_kernel_for: full-K kernel; kc chunks per wave, gs MFMA steps per
//     group, depth tiles in flight (1; 2 only for kc < 8), xs = activations
//     streamed with the weights (k > 8192)
//   split_kernel_for: K-split kernel; bt batch tiles, kc chunks per wave,
//     lds = the form with the K-part of x in LDS
template <int FMT>
StreamKernelFn stream_kernel_for(int kc, int gs, int depth, bool xs);
template <int FMT>
SplitKernelFn split_kernel_for(int gs, int bt, int kc, bool lds);

}  // namespace qg
