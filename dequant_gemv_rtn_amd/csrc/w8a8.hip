// W8A8 product: INT8 activations per token times INT8 weights per output
// channel, on the int8 matrix cores ("A Method for Layer Bit-Width
// Allocation in LLM Quantization via Performance Maximization Under a
// Quality-Degradation Constraint", abstract: W8A8 variants whose integer
// arithmetic pays for quantizing and dequantizing in the FFN and lm_head).
//
// Two kernels on the caller's stream:
// * w8a8_quantize_kernel, one workgroup per activation row b:
//     a[k] = x[k] / m[k]   (m: optional per-input-channel smoothing factors)
//     s    = max_k |a[k]| / 127
//     q[k] = clamp(rne(a[k] / s), -127, 127)   (0 when s = 0)
//   every division the correctly rounded binary32 one (__fdiv_rn), so the
//   codes are a function of the inputs alone.  Codes int8 [b][k] and scales
//   fp32 [b] go to the workspace.
// * w8a8_gemm_kernel: v_mfma_i32_16x16x64_i8 with 16 activation rows as A
//   (rows past b read as zero through the buffer bound) and 16 weight rows
//   as B, both as 16 contiguous bytes per lane (lane l: row l % 16, bytes
//   16 (l / 16) .. + 15 of the 64-element step; the same k-pattern on both
//   operands, so each product pairs equal k).  Exact int32 sums, then
//   y = f16((s_x * s_w) * f32(acc)): two binary32 multiplies, each rounded
//   to binary32, then the rounding to fp16.
//   A workgroup of 4 waves owns row tiles of 16 weight rows (strided over
//   the grid); wave w takes the 64-element steps w, w + 4, ..., four steps
//   of loads in flight at a time; the four partial tiles meet in LDS, where
//   integer adds give the same sum in any order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"
#include "internal.hpp"

namespace qg {
namespace {

typedef int i4v __attribute__((ext_vector_type(4)));

constexpr int kW8Waves = 4;
constexpr int kW8Steps = 4;  // 64-element steps per wave per batch of loads
constexpr int kQuantThreads = 256;

__global__ void __launch_bounds__(kQuantThreads)
w8a8_quantize_kernel(const _Float16* __restrict__ x, const float* __restrict__ smooth, int k,
                     int8_t* __restrict__ xq, float* __restrict__ sx) {
  __shared__ float red[kQuantThreads / 64];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const _Float16* xr = x + (size_t)b * k;
  float amax = 0.0f;
  for (int i = tid; i < k; i += kQuantThreads) {
    const float a = smooth ? __fdiv_rn((float)xr[i], smooth[i]) : (float)xr[i];
    amax = fmaxf(amax, fabsf(a));
  }
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if (lane == 0) red[wave] = amax;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kQuantThreads / 64; ++w) amax = fmaxf(amax, red[w]);
  const float s = __fdiv_rn(amax, 127.0f);
  if (tid == 0) sx[b] = s;
  int8_t* qr = xq + (size_t)b * k;
  for (int i = tid; i < k; i += kQuantThreads) {
    const float a = smooth ? __fdiv_rn((float)xr[i], smooth[i]) : (float)xr[i];
    const float r = s > 0.0f ? fminf(fmaxf(rintf(__fdiv_rn(a, s)), -127.0f), 127.0f) : 0.0f;
    qr[i] = (int8_t)(int)r;
  }
}

struct W8Geom {
  int n, k, b, tiles, ksteps;
  uint32_t codes_bytes, scales_bytes, xq_bytes, sx_bytes, y_bytes;
};

template <int BT>
__global__ void __launch_bounds__(64 * kW8Waves)
w8a8_gemm_kernel(const int8_t* __restrict__ wq, const _Float16* __restrict__ sw, const int8_t* __restrict__ xq,
                 const float* __restrict__ sx, _Float16* __restrict__ y, W8Geom g) {
  __shared__ i4v red[kW8Waves][BT][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, q = lane >> 4;
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(wq, g.codes_bytes);
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(sw, g.scales_bytes);
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(xq, g.xq_bytes);
  const __amdgpu_buffer_rsrc_t sxr = make_rsrc(sx, g.sx_bytes);
  const __amdgpu_buffer_rsrc_t yrs = make_rsrc(y, g.y_bytes);
  // activation rows of this lane in each batch tile (rows past b: offsets
  // past the codes, which read as zero)
  uint32_t xrow[BT];
#pragma unroll
  for (int bt = 0; bt < BT; ++bt) {
    const int row = 16 * bt + r16;
    xrow[bt] = row < g.b ? (uint32_t)row * (uint32_t)g.k + 16u * q : 0xFFFFFF00u;
  }
  for (int t = blockIdx.x; t < g.tiles; t += gridDim.x) {
    const int wrow = min(16 * t + r16, g.n - 1);  // rows past n: a real row, never stored
    const uint32_t wbase = (uint32_t)wrow * (uint32_t)g.k + 16u * q;
    i4v acc[BT];
#pragma unroll
    for (int bt = 0; bt < BT; ++bt) acc[bt] = i4v{0, 0, 0, 0};
    for (int s0 = wave; s0 < g.ksteps; s0 += kW8Waves * kW8Steps) {
      i4v wv[kW8Steps], xv[kW8Steps][BT];
#pragma unroll
      for (int j = 0; j < kW8Steps; ++j) {
        const int st = s0 + kW8Waves * j;
        const uint32_t ko = (uint32_t)st * 64u;
        // this lane's 16 bytes lie inside the row (k is a multiple of 16,
        // so a last half step leaves lanes 32-63 out, reading zero)
        const bool in = st < g.ksteps && ko + 16u * (uint32_t)q < (uint32_t)g.k;
        wv[j] = __builtin_bit_cast(i4v, __builtin_amdgcn_raw_buffer_load_b128(wrs, in ? wbase + ko : 0xFFFFFF00u, 0, 0));
#pragma unroll
        for (int bt = 0; bt < BT; ++bt)
          xv[j][bt] = __builtin_bit_cast(
              i4v, __builtin_amdgcn_raw_buffer_load_b128(xrs, in && xrow[bt] != 0xFFFFFF00u ? xrow[bt] + ko : 0xFFFFFF00u,
                                                         0, 0));
      }
#pragma unroll
      for (int j = 0; j < kW8Steps; ++j)
#pragma unroll
        for (int bt = 0; bt < BT; ++bt) acc[bt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xv[j][bt], wv[j], acc[bt], 0, 0, 0);
    }
#pragma unroll
    for (int bt = 0; bt < BT; ++bt) red[wave][bt][lane] = acc[bt];
    __syncthreads();
    if (wave == 0) {
      const int n = 16 * t + r16;
      const float swf = h2f((uint16_t)__builtin_amdgcn_raw_buffer_load_b16(srs, (uint32_t)wrow * 2u, 0, 0));
#pragma unroll
      for (int bt = 0; bt < BT; ++bt) {
        i4v sum = red[0][bt][lane];
#pragma unroll
        for (int w = 1; w < kW8Waves; ++w) sum += red[w][bt][lane];
        // D[4 q + i][r16]: activation row 16 bt + 4 q + i, weight row n
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int brow = 16 * bt + 4 * q + i;
          const bool live = brow < g.b && n < g.n;
          const float sxf = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(sxr, live ? (uint32_t)brow * 4u : 0xFFFFFF00u, 0, 0));
          float v = (sxf * swf) * (float)sum[i];
          // v is the binary32 product: without this empty register barrier
          // the multiply and the fp16 conversion fuse into v_fma_mixlo_f16,
          // which rounds once, and differs where v falls on an fp16 tie
          asm volatile("" : "+v"(v));
          const uint32_t off = live ? ((uint32_t)brow * (uint32_t)g.n + (uint32_t)n) * 2u : 0xFFFFFF00u;
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)v), yrs, off, 0, 0);
        }
      }
    }
    __syncthreads();  // red is rewritten by the next tile
  }
}

size_t round16(size_t v) { return (v + 15) / 16 * 16; }

}  // namespace

size_t w8a8_workspace_bytes(int b, int k) { return round16((size_t)b * (size_t)k) + round16((size_t)b * 4u); }

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
  g.tiles = (w.n + 15) / 16;
  g.ksteps = w.k / 64 + (w.k % 64 ? 1 : 0);
  g.codes_bytes = (uint32_t)buffer_bytes(Q_INT8, w.n, w.k, w.k, Q_BUF_CODES);
  g.scales_bytes = (uint32_t)buffer_bytes(Q_INT8, w.n, w.k, w.k, Q_BUF_SCALES);
  g.xq_bytes = (uint32_t)((size_t)b * (size_t)w.k);
  g.sx_bytes = (uint32_t)(b * 4);
  g.y_bytes = (uint32_t)((size_t)b * (size_t)w.n * 2u);
  // persistent workgroups: QGEMV_W8A8_WG_PER_CU per compute unit (tuning)
  const int per_cu = env_int("QGEMV_W8A8_WG_PER_CU", 4);
  int grid = device_cu_count() * (per_cu > 0 ? per_cu : 4);
  if (grid > g.tiles) grid = g.tiles;
  const int bt = (b + 15) / 16;
  auto fn = bt == 1 ? w8a8_gemm_kernel<1> : bt == 2 ? w8a8_gemm_kernel<2> : bt == 3 ? w8a8_gemm_kernel<3>
                                                                                   : w8a8_gemm_kernel<4>;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(64 * kW8Waves), 0, s, reinterpret_cast<const int8_t*>(w.codes),
                     static_cast<const _Float16*>(w.scales), xq, sx, y, g);
  return hipGetLastError();
}

}  // namespace qg
