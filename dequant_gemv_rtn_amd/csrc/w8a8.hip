// W8A8 product: INT8 activations per token times INT8 weights per output
// channel, on the int8 matrix cores ("A Method for Layer Bit-Width
// Allocation in LLM Quantization via Performance Maximization Under a
// Quality-Degradation Constraint", abstract: W8A8 variants whose integer
// arithmetic pays for quantizing and dequantizing in the FFN and lm_head).
//
// Two kernels on the caller's stream:
// * w8a8_quantize_kernel, one workgroup of 1024 lanes per activation row b
//   (16 bytes of x per lane per load, the row kept in registers between the
//   absmax pass and the coding pass, k <= 16384):
//     a[k] = x[k] / m[k]   (m: optional per-input-channel smoothing factors)
//     s    = max_k |a[k]| / 127
//     q[k] = clamp(rne(a[k] / s), -127, 127)   (0 when s = 0)
//   every division the correctly rounded binary32 one (__fdiv_rn), so the
//   codes are a function of the inputs alone.  Codes int8 [b][k] and scales
//   fp32 [b] go to the workspace.
// * w8a8_gemm_kernel: v_mfma_i32_16x16x64_i8 with 16 activation rows as A
//   (rows past b read as zero through the buffer bound) and 16 weight rows
//   as B.  A step is 128 k: lane l (row l % 16, quarter q = l / 16) loads
//   bytes 32 q .. 32 q + 31 of the step as two 16-byte pieces, so the four
//   quarters of a row read one whole 128-byte line, and MFMA h of the step
//   takes piece h of every lane (the same k-pattern on both operands, so
//   each product pairs equal k).  Exact int32 sums, then
//   y = f16((s_x * s_w) * f32(acc)): two binary32 multiplies, each rounded
//   to binary32, then the rounding to fp16.
//   A workgroup of W waves (W = 4, 8 or 16: one step or more each) owns a
//   16-row weight tile at a time, its row group striding over the tiles
//   (persistent workgroups, 16 waves per compute unit); wave w takes the S
//   steps w, w + W, ... of every tile, its activation slice held in
//   registers for the launch, and loads the tile's weights in rounds of up
//   to 4 steps, the next tile's first round in flight while the W partial
//   tiles meet in LDS (integer adds give the same sum in any order).  One
//   workgroup serves every batch tile where their slices fit in registers
//   (the weights are then read once), else one per batch tile, XCD-aligned.
//   The activation scales of the workgroup's rows sit in LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "common.hpp"
#include "internal.hpp"

namespace qg {
namespace {

typedef int i4v __attribute__((ext_vector_type(4)));
typedef unsigned u4v __attribute__((ext_vector_type(4)));

constexpr int kQuantThreads = 1024;
constexpr int kQuantChunks = 2;   // 16-byte pieces of x per lane: 1024 * 2 * 8 = 16384 >= k
constexpr int kW8MaxWaves = 16;
constexpr uint32_t kNone = 0xFFFFFF00u;  // a buffer offset past every range: loads give 0, stores drop

__device__ __forceinline__ float lo_h(uint32_t w) { return h2f((uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float hi_h(uint32_t w) { return h2f((uint16_t)(w >> 16)); }

__global__ void __launch_bounds__(kQuantThreads)
w8a8_quantize_kernel(const _Float16* __restrict__ x, const float* __restrict__ smooth, int k,
                     int8_t* __restrict__ xq, float* __restrict__ sx) {
  __shared__ float red[kQuantThreads / 64];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunks = k / 8;
  const _Float16* xr = x + (size_t)b * k;
  float a[kQuantChunks][8];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < kQuantChunks; ++c) {
    const int idx = tid + c * kQuantThreads;
    if (idx < chunks) {
      const u4v v = *reinterpret_cast<const u4v*>(xr + 8 * idx);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[c][2 * e] = lo_h(v[e]);
        a[c][2 * e + 1] = hi_h(v[e]);
      }
      if (smooth) {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[c][e] = __fdiv_rn(a[c][e], smooth[8 * idx + e]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(a[c][e]));
    }
  }
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if (lane == 0) red[wave] = amax;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kQuantThreads / 64; ++w) amax = fmaxf(amax, red[w]);
  const float s = __fdiv_rn(amax, 127.0f);
  if (tid == 0) sx[b] = s;
  int8_t* qr = xq + (size_t)b * k;
#pragma unroll
  for (int c = 0; c < kQuantChunks; ++c) {
    const int idx = tid + c * kQuantThreads;
    if (idx < chunks) {
      uint32_t packed[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float r = s > 0.0f ? fminf(fmaxf(rintf(__fdiv_rn(a[c][e], s)), -127.0f), 127.0f) : 0.0f;
        packed[e >> 2] |= ((uint32_t)(int)r & 0xFFu) << (8 * (e & 3));
      }
      *reinterpret_cast<uint2*>(qr + 8 * idx) = make_uint2(packed[0], packed[1]);
    }
  }
}

struct W8Geom {
  int n, k, b, batch_tiles, tiles, ksteps;
  uint32_t codes_bytes, scales_bytes, xq_bytes, sx_bytes, y_bytes;
};

template <int WAVES, int S, int NBT>
__global__ void __launch_bounds__(64 * WAVES)
w8a8_gemm_kernel(const int8_t* __restrict__ wq, const _Float16* __restrict__ sw, const int8_t* __restrict__ xq,
                 const float* __restrict__ sx, _Float16* __restrict__ y, W8Geom g) {
  constexpr int RW = S < 4 ? S : S == 4 ? 4 : 2;  // steps per round of weight loads (registers: 8 per step)
  constexpr int NR = S / RW;         // rounds per tile
  __shared__ i4v red[WAVES][NBT][64];
  __shared__ float sxs[NBT * 16];  // activation scales of the workgroup's batch rows
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, q = lane >> 4;
  // this workgroup serves batch tiles NBT btg .. NBT btg + NBT - 1
  int btg, t0;
  const int groups = g.batch_tiles / NBT;
  const int grid_rows = (int)gridDim.x / groups;
  batch_tile_of(groups, grid_rows, btg, t0);
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(wq, g.codes_bytes);
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(sw, g.scales_bytes);
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(xq, g.xq_bytes);
  const __amdgpu_buffer_rsrc_t sxr = make_rsrc(sx, g.sx_bytes);
  const __amdgpu_buffer_rsrc_t yrs = make_rsrc(y, g.y_bytes);
  // piece h of step j of this wave: k offset of its first byte, or kNone
  // when the piece lies past the row (k is a multiple of 32, so a 16-byte
  // piece is wholly inside or wholly past) or the step past the last one
  auto piece = [&](int j, int h) -> uint32_t {
    const int st = wave + WAVES * j;
    const uint32_t ko = (uint32_t)st * 128u + 32u * q + 16u * h;
    return st < g.ksteps && ko < (uint32_t)g.k ? ko : kNone;
  };
  // the wave's activation slices, loaded once for the launch (rows past b: 0)
  i4v xv[NBT][S][2];
  if (threadIdx.x < NBT * 16) {
    const int brow = 16 * NBT * btg + threadIdx.x;
    sxs[threadIdx.x] = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(sxr, brow < g.b ? (uint32_t)brow * 4u : kNone, 0, 0));
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < NBT; ++u) {
    const int xr = 16 * (NBT * btg + u) + r16;
#pragma unroll
    for (int j = 0; j < S; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t ko = piece(j, h);
        xv[u][j][h] = __builtin_bit_cast(
            i4v, __builtin_amdgcn_raw_buffer_load_b128(
                     xrs, ko != kNone && xr < g.b ? (uint32_t)xr * (uint32_t)g.k + ko : kNone, 0, 0));
      }
  }
  i4v wv[RW][2];
  auto load_w = [&](int t, int r) {
    const uint32_t wbase = (uint32_t)min(16 * t + r16, g.n - 1) * (uint32_t)g.k;  // rows past n: a real row, never stored
#pragma unroll
    for (int j = 0; j < RW; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t ko = piece(r * RW + j, h);
        wv[j][h] = __builtin_bit_cast(
            i4v, __builtin_amdgcn_raw_buffer_load_b128(wrs, ko != kNone ? wbase + ko : kNone, 0, 0));
      }
  };
  if (t0 < g.tiles) load_w(t0, 0);
  for (int t = t0; t < g.tiles; t += grid_rows) {
    const int wrow = min(16 * t + r16, g.n - 1);
    const uint16_t swbits = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(srs, (uint32_t)wrow * 2u, 0, 0);
    i4v acc[NBT];
#pragma unroll
    for (int u = 0; u < NBT; ++u) acc[u] = i4v{0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      if (r > 0) load_w(t, r);
#pragma unroll
      for (int j = 0; j < RW; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int u = 0; u < NBT; ++u)
            acc[u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xv[u][r * RW + j][h], wv[j][h], acc[u], 0, 0, 0);
    }
    // the next tile's first round is in flight while this one is reduced
    if (t + grid_rows < g.tiles) load_w(t + grid_rows, 0);
    if constexpr (WAVES > 1) {
#pragma unroll
      for (int u = 0; u < NBT; ++u) red[wave][u][lane] = acc[u];
      __syncthreads();
    }
    if (wave == 0) {
      const int n = 16 * t + r16;
      const float swf = h2f(swbits);
#pragma unroll
      for (int u = 0; u < NBT; ++u) {
      i4v sum = acc[u];
      if constexpr (WAVES > 1) {
        sum = red[0][u][lane];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) sum += red[w][u][lane];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int brow = 16 * (NBT * btg + u) + 4 * q + i;
        const bool live = brow < g.b && n < g.n;
        float v = (sxs[16 * u + 4 * q + i] * swf) * (float)sum[i];  // scale of row D[4 q + i]
        // v is the binary32 product: without this empty register barrier
        // the multiply and the fp16 conversion fuse into v_fma_mixlo_f16,
        // which rounds once, and differs where v falls on an fp16 tie
        asm volatile("" : "+v"(v));
        const uint32_t off = live ? ((uint32_t)brow * (uint32_t)g.n + (uint32_t)n) * 2u : kNone;
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)v), yrs, off, 0, 0);
      }
      }
    }
    if constexpr (WAVES > 1) __syncthreads();  // red is rewritten by the next tile
  }
}

size_t round16(size_t v) { return (v + 15) / 16 * 16; }

template <int WAVES>
void* pick_w8a8(int steps, int nbt) {
  // several batch tiles per workgroup only where their slices fit: steps *
  // nbt <= 8, and with 16 waves steps <= 2 (launch_w8a8 asks for no other)
  if (steps == 1 && nbt == 2) return reinterpret_cast<void*>(w8a8_gemm_kernel<WAVES, 1, 2>);
  if (steps == 1 && nbt == 3) return reinterpret_cast<void*>(w8a8_gemm_kernel<WAVES, 1, 3>);
  if (steps == 1 && nbt == 4) return reinterpret_cast<void*>(w8a8_gemm_kernel<WAVES, 1, 4>);
  if (steps == 2 && nbt == 2) return reinterpret_cast<void*>(w8a8_gemm_kernel<WAVES, 2, 2>);
  if (steps == 2 && nbt == 3) return reinterpret_cast<void*>(w8a8_gemm_kernel<WAVES, 2, 3>);
  if (steps == 2 && nbt == 4) return reinterpret_cast<void*>(w8a8_gemm_kernel<WAVES, 2, 4>);
  if constexpr (WAVES < 16) {  // (16 waves: 128 VGPRs are not enough for it)
    if (steps == 4 && nbt == 2) return reinterpret_cast<void*>(w8a8_gemm_kernel<WAVES, 4, 2>);
  }
  switch (steps) {
    case 1: return reinterpret_cast<void*>(w8a8_gemm_kernel<WAVES, 1, 1>);
    case 2: return reinterpret_cast<void*>(w8a8_gemm_kernel<WAVES, 2, 1>);
    case 4: return reinterpret_cast<void*>(w8a8_gemm_kernel<WAVES, 4, 1>);
    default: return reinterpret_cast<void*>(w8a8_gemm_kernel<WAVES, 8, 1>);
  }
}

int pow2_at_least(int v) {
  int p = 1;
  while (p < v) p *= 2;
  return p;
}

}  // namespace

size_t w8a8_workspace_bytes(int b, int k) { return round16((size_t)b * (size_t)k) + round16((size_t)b * 4u); }

int w8a8_waves(int n, int k, int b) {
  (void)n;
  (void)b;
  const int ksteps = (k + 127) / 128;
  const int forced = tuning(kTuneW8a8Waves, 0);
  if ((forced == 4 || forced == 8 || forced == 16) && forced * 8 >= ksteps) return forced;
  // one step or more per wave, at most 16 waves (the slice of k <= 16384
  // then takes at most 8 steps)
  const int waves = pow2_at_least(ksteps);
  return waves < 4 ? 4 : waves > kW8MaxWaves ? kW8MaxWaves : waves;
}

hipError_t launch_w8a8(const WeightView& w, const _Float16* x, const float* smooth, _Float16* y, int b, void* ws,
                       hipStream_t s) {
  auto* xq = static_cast<int8_t*>(ws);
  auto* sx = reinterpret_cast<float*>(static_cast<char*>(ws) + round16((size_t)b * (size_t)w.k));
  hipLaunchKernelGGL(w8a8_quantize_kernel, dim3(b), dim3(kQuantThreads), 0, s, x, smooth, w.k, xq, sx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  W8Geom g;
  g.n = w.n;
  g.k = w.k;
  g.b = b;
  g.batch_tiles = (b + 15) / 16;
  g.tiles = (w.n + 15) / 16;
  g.ksteps = (w.k + 127) / 128;
  g.codes_bytes = (uint32_t)buffer_bytes(Q_INT8, w.n, w.k, w.k, Q_BUF_CODES);
  g.scales_bytes = (uint32_t)buffer_bytes(Q_INT8, w.n, w.k, w.k, Q_BUF_SCALES);
  g.xq_bytes = (uint32_t)((size_t)b * (size_t)w.k);
  g.sx_bytes = (uint32_t)(b * 4);
  g.y_bytes = (uint32_t)((size_t)b * (size_t)w.n * 2u);
  const int waves = w8a8_waves(w.n, w.k, b);
  const int steps = pow2_at_least((g.ksteps + waves - 1) / waves);  // waves * steps >= ksteps
  // one workgroup serves every batch tile where their activation slices fit
  // in registers (steps * batch tiles <= 8, and steps <= 2 with 16 waves,
  // whose lanes have 128 VGPRs): the weights are then read once; else one
  // workgroup per batch tile (QGEMV_W8A8_JOINT=0 forces that)
  int nbt_wg = 1;
  if (g.batch_tiles > 1 && steps * g.batch_tiles <= 8 && (waves < 16 || steps <= 2) &&
      tuning(kTuneW8a8Joint, 1) != 0)
    nbt_wg = g.batch_tiles;
  const int groups = g.batch_tiles / nbt_wg;
  // persistent workgroups: QGEMV_W8A8_WAVES_PER_CU waves per compute unit
  // counted over all batch-tile groups (all resident at once: at most 128
  // VGPRs per lane leave room for 16); the row groups are XCD-aligned
  // (batch_tile_of)
  const int waves_per_cu = tuning(kTuneW8a8WavesPerCu, 16);
  const int per_cu = waves_per_cu / waves > 1 ? waves_per_cu / waves : 1;
  int grid_rows = device_cu_count() * per_cu / groups;
  if (grid_rows > 8) grid_rows -= grid_rows % 8;
  if (grid_rows < 1) grid_rows = 1;
  if (grid_rows > g.tiles) grid_rows = g.tiles;
  void* fn = waves == 4   ? pick_w8a8<4>(steps, nbt_wg)
             : waves == 8 ? pick_w8a8<8>(steps, nbt_wg)
                          : pick_w8a8<16>(steps, nbt_wg);
  const int8_t* wc = reinterpret_cast<const int8_t*>(w.codes);
  const _Float16* wsc = static_cast<const _Float16*>(w.scales);
  const int8_t* xqc = xq;
  const float* sxc = sx;
  void* args[] = {&wc, &wsc, &xqc, &sxc, &y, &g};
  return hipLaunchKernel(fn, dim3(grid_rows * groups), dim3(64 * waves), args, 0, s);
}

}  // namespace qg
