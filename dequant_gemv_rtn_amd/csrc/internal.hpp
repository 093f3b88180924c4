// Host-side launchers shared between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace qg {

// Largest k accepted by every kernel (the vector-ALU GEMV keeps x slices in
// registers and spreads a row over at most 8 waves).
constexpr int kMaxK = Q_MAX_K;

// Launch the RTN quantize-and-pack kernel for every row of W.
hipError_t launch_pack(const WeightView& w, const _Float16* src, hipStream_t s);

// b in [1, 8]: vector-ALU fused-dequant GEMV.
hipError_t launch_gemv_valu(const WeightView& w, const _Float16* x, _Float16* y, int b, hipStream_t s);

// b in [9, 64]: MFMA fused-dequant skinny GEMM.
hipError_t launch_gemm_mfma(const WeightView& w, const _Float16* x, _Float16* y, int b, hipStream_t s);

// Compute units of the current device (cached per device).
int device_cu_count();

}  // namespace qg
