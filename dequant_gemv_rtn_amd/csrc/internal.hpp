// Host-side launchers shared between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace qg {

// Largest k accepted by every kernel (the vector-ALU GEMV keeps x slices in
// registers and spreads a row over at most 8 waves).
constexpr int kMaxK = Q_MAX_K;

// Launch the RTN quantize-and-pack kernel for every row of W.
// clip_candidates > 1: the per-group clipping search (INT4 asym, E2M1 only)
hipError_t launch_pack(const WeightView& w, const _Float16* src, hipStream_t s, int clip_candidates = 1);

// b in [1, 8]: vector-ALU fused-dequant GEMV.
hipError_t launch_gemv_valu(const WeightView& w, const _Float16* x, _Float16* y, int b, hipStream_t s);

// b in [1, 64], k <= Q_MAX_K: weight-streaming MFMA kernel.
bool gemm_stream_supported(const WeightView& w, int b);
hipError_t launch_gemm_stream(const WeightView& w, const _Float16* x, _Float16* y, int b, hipStream_t s);

// K-split MFMA kernel plus the kernel that sums its parts.  Workspace bytes
// it needs for (w, b), 0 when (w, b) runs the full-K kernel instead.
size_t gemm_split_workspace(const WeightView& w, int b);
hipError_t launch_gemm_split(const WeightView& w, const _Float16* x, _Float16* y, int b, void* ws, size_t ws_bytes,
                             hipStream_t s);

// Decode attention over FP4-quantized K and V caches (head_dim 128): the
// workspace bytes for a shape, and the split + combine launch.
size_t attn_workspace_bytes(int batch, int q_heads, int kv_heads, int max_len);
hipError_t launch_attn_decode(const WeightView& k, const WeightView& v, const _Float16* q, const int32_t* seq_lens,
                              _Float16* out, int batch, int q_heads, int kv_heads, int max_len, float scale, void* ws,
                              hipStream_t s);

// W8A8 product over an INT8 weight: workspace bytes (activation codes and
// scales) and the quantize + integer-MFMA launch.
size_t w8a8_workspace_bytes(int b, int k);
int w8a8_waves(int n, int k, int b);  // waves per workgroup of the W8A8 product
hipError_t launch_w8a8(const WeightView& w, const _Float16* x, const float* smooth, _Float16* y, int b, void* ws,
                       hipStream_t s);

// Debug export: W_deq [n][k] as fp16 (each value exact in fp32, rounded once).
hipError_t launch_dequant(const WeightView& w, _Float16* out, hipStream_t s);

// Every packed buffer is allocated as its packed bytes rounded up to a
// multiple of kBufferPad, the pad zero-filled by q_pack, so that 16-byte
// loads starting inside a buffer never end outside it.
constexpr size_t kBufferPad = 16;

// Bytes of packed contents of buffer `which` (q_buffer), before padding.
size_t packed_bytes_logical(int32_t format, int32_t n, int32_t k, int32_t group, int32_t which);

// Allocated size of buffer `which`: packed_bytes_logical rounded up to kBufferPad.
size_t buffer_bytes(int32_t format, int32_t n, int32_t k, int32_t group, int32_t which);

// Compute units of the current device (cached per device).
int device_cu_count();

// Integer tuning override from the environment, or dflt when unset.
int env_int(const char* name, int dflt);

// Smallest r with (1 << r) >= v.
int ilog2(int v);

}  // namespace qg
