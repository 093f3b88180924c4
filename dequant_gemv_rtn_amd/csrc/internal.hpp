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
// scales) and the launch (one fused kernel for b <= 4 on short tile walks,
// else quantize + integer-MFMA).
size_t w8a8_workspace_bytes(int b, int k);
int w8a8_waves(int n, int k, int b);  // waves per workgroup of the W8A8 product
hipError_t launch_w8a8(const WeightView& w, const _Float16* x, const float* smooth, _Float16* y, int b, void* ws,
                       hipStream_t s);

// Decode stack (b = 1, one launch for a sequence of linears): plan bytes,
// the plan writer (host only; views are the checked entries' weights), and
// the launch over a plan copied to the device.
size_t stack_plan_bytes(int count);
int stack_plan(const q_stack_entry* entries, int count, const WeightView* views, void* out, size_t out_bytes);
hipError_t launch_stack(const void* plan_device, bool chain, hipStream_t s);

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

// Launch-shape tuning overrides, for measurement and for the tests that force
// every kernel form.  Each key is unset unless q_tuning_set gave it a value,
// or the environment variable of the same name (QGEMV_...) was set when the
// library first read its tuning table: once per process, so the plan that
// sizes a workspace and the plan that launches always agree.
enum TuneKey : int {
  kTunePath = 0,          // QGEMV_PATH: 1 vector-ALU (b <= 8), 2 streaming MFMA
  kTuneSplitMinB,         // QGEMV_SPLIT_MIN_B: smallest b of the K-split form (0 = never)
  kTuneSplitKc,           // QGEMV_SPLIT_KC: chunks per wave of the K-split form (1 or 2)
  kTuneSplitLds,          // QGEMV_SPLIT_LDS: K-split form with x in LDS (0 or 1)
  kTuneSplitGridRows,     // QGEMV_SPLIT_GRID_ROWS: workgroups per K-part
  kTuneStreamMaxWaves,    // QGEMV_STREAM_MAX_WAVES: waves per full-K workgroup (1..16)
  kTuneStreamKc,          // QGEMV_STREAM_KC: chunks per wave of the full-K kernel
  kTuneStreamWavesPerCu,  // QGEMV_STREAM_WAVES_PER_CU
  kTuneStreamGridRows,    // QGEMV_STREAM_GRID_ROWS
  kTuneValuCpl,           // QGEMV_VALU_CPL: 32-element pieces per lane (cap)
  kTuneValuRows,          // QGEMV_VALU_ROWS: rows per register stage at b = 1 (1 or 2)
  kTuneValuShare,         // QGEMV_VALU_SHARE: row walkers sharing one LDS copy of x (1, 4, 8)
  kTuneValuStrided,       // QGEMV_VALU_STRIDED: walkers stride over row blocks (1) or take ranges (0)
  kTuneValuWavesPerCu,    // QGEMV_VALU_WAVES_PER_CU
  kTuneAttnMfma,          // QGEMV_ATTN_MFMA: decode attention products on the matrix cores (0 or 1)
  kTuneW8a8Waves,         // QGEMV_W8A8_WAVES
  kTuneW8a8Joint,         // QGEMV_W8A8_JOINT
  kTuneW8a8WavesPerCu,    // QGEMV_W8A8_WAVES_PER_CU
  kTuneW8a8FuseMaxB,      // QGEMV_W8A8_FUSE_MAX_B: largest b of the fused quantize + product (0 = never)
  kTuneW8a8Dot,           // QGEMV_W8A8_DOT: the vector-ALU (dot4) forms of the W8A8 product for b <= this (0 = off)
  kTuneW8a8DotWavesPerCu, // QGEMV_W8A8_DOT_WAVES_PER_CU
  kTuneW8a8DotP,          // QGEMV_W8A8_DOT_P: KiB of a row per stage of the dot4 form (2 or 4)
  kTuneW8a8DotS,          // QGEMV_W8A8_DOT_S: stages in flight per wave of the dot4 form (2 or 4)
  kTuneW8a8DotSplit,      // QGEMV_W8A8_DOT_SPLIT: rows over several waves in the dot4 form (1: every k > 8192, 0: never)
  kTuneW8a8DotWalkersPerCu, // QGEMV_W8A8_DOT_WALKERS_PER_CU: row walkers of the split dot4 form per CU
  kTuneCount
};

// The override of `key`, or dflt when it is unset.
int tuning(TuneKey key, int dflt);

// Smallest r with (1 << r) >= v.
int ilog2(int v);

}  // namespace qg
