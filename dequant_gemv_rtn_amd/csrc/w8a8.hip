// W8A8 product: INT8 activations per token times INT8 weights per output
// channel, on the int8 matrix cores ("A Method for Layer Bit-Width
// Allocation in LLM Quantization via Performance Maximization Under a
// Quality-Degradation Constraint", abstract: W8A8 variants whose integer
// arithmetic pays for quantizing and dequantizing in the FFN and lm_head).
//
// Two forms.  For b <= 4, w8a8_small_kernel (further down) quantizes and
// multiplies in one launch where it applies; otherwise two kernels on the
// caller's stream:
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

// ---- fused form for a few activation rows -------------------------------------
//
// w8a8_small_kernel: the quantizer and the product in one launch, for b <= 4.
// Every workgroup quantizes the b activation rows itself (a few KB, from L2
// after the first touch) with the binary32 steps of w8a8_quantize_kernel,
// so its codes and scales are the same bits:
//   1. the lane's 8-element pieces of x (and of m) are loaded first, then the
//      first kSmallRing steps of weight loads are put in flight behind them;
//   2. per-row absmax: lane maxima, wave shuffles, one LDS slot per wave;
//      s = absmax / 127, computed by every lane from the same maxima;
//   3. the quotients are formed again and coded into LDS as int8 [b + 1][kp]
//      (kp: k rounded up to a step; bytes past k, and row b, are zeros).
// The product keeps the codes in LDS instead of registers, so each wave's
// registers hold a ring of weight steps in flight: slot (m, j) holds step j
// of the workgroup's tile m tiles ahead (M = kSmallRing / S tiles, at least
// one), refilled as soon as its MFMAs have read it.  (Deeper rings, up to
// 8 steps per wave, measured no faster: 14336 x 4096 at b = 1 ran 13.7 us
// with 2 steps, 14.1 with 4 and 16.1 with 8.)  Slots and steps are
// compile-time indices (the tile loop is unrolled M times); a step past the
// last one is skipped by a wave-uniform branch, load and MFMA alike.  Lanes
// of rows r16 >= b read the zero row.  Pieces of the last step that lie past
// k load the next row's bytes (or zeros past the buffer) against zero codes.
// With b <= 4 every live output sits in lanes 0..15 (D rows 0..3), so the
// per-tile reduction moves 16 lanes per wave through a double-buffered LDS
// slot with one barrier (lds_barrier waits for LDS only, so the ring stays
// in flight).

constexpr int kSmallMaxB = 4;    // activation rows of the fused form
constexpr int kSmallChunks = 2;  // 8-element pieces of x per lane held through the prologue
constexpr int kSmallRing = 2;    // steps of weight loads in flight per wave (at least one tile's S)
constexpr int kSmallScales = 2;  // weight-row scales per lane loaded by the prologue
constexpr int kSmallMaxVisits = 8;  // tiles per workgroup (rounded up to the ring's M) of the fused form

struct W8Small {
  int n, k, b, tiles, ksteps, kp;
  uint32_t codes_bytes, scales_bytes, x_bytes, m_bytes, y_bytes;
};

// Pieces of x the fused prologue holds per lane; its launcher requires
// b * k / 8 <= that many times the workgroup's lanes.
__host__ __device__ constexpr int small_chunks(int steps) { return steps < kSmallChunks ? steps : kSmallChunks; }

template <int WAVES, int S, bool SMOOTH>
__global__ void __launch_bounds__(64 * WAVES, 4)
w8a8_small_kernel(const int8_t* __restrict__ wq, const _Float16* __restrict__ sw, const _Float16* __restrict__ x,
                  const float* __restrict__ smooth, _Float16* __restrict__ y, W8Small g) {
  constexpr int M = kSmallRing > S ? kSmallRing / S : 1;  // tiles of weight loads in flight
  constexpr int NT = 64 * WAVES;
  constexpr int CH = small_chunks(S);
  extern __shared__ __attribute__((aligned(16))) int8_t xs[];  // activation codes [b + 1][kp]
  __shared__ i4v red[2][WAVES][16];
  __shared__ float amx[WAVES][kSmallMaxB];
  __shared__ uint16_t sws[kSmallScales * NT];  // scales of the workgroup's weight rows, tile by tile
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, q = lane >> 4;
  const int stride = (int)gridDim.x, t0 = (int)blockIdx.x;
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(wq, g.codes_bytes);
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(sw, g.scales_bytes);
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, g.x_bytes);
  const __amdgpu_buffer_rsrc_t mrs = make_rsrc(smooth, g.m_bytes);
  const __amdgpu_buffer_rsrc_t yrs = make_rsrc(y, g.y_bytes);
  const int kc = g.k >> 3, pieces = g.b * kc;
  // piece c = tid + NT i: elements 8 (c - r kc) .. + 7 of row r = c / kc;
  // the rows are contiguous, so it starts at byte 16 c of x
  auto row_of = [&](int c) { return (int)(c >= kc) + (int)(c >= 2 * kc) + (int)(c >= 3 * kc); };
  u4v xraw[CH];
  u4v mraw[CH][2];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = tid + NT * i;
    const bool live = c < pieces;
    xraw[i] = __builtin_bit_cast(u4v, __builtin_amdgcn_raw_buffer_load_b128(xrs, live ? (uint32_t)c * 16u : kNone, 0, 0));
    if constexpr (SMOOTH) {
      const uint32_t mo = (uint32_t)(c - row_of(c) * kc) * 32u;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        mraw[i][h] = __builtin_bit_cast(u4v, __builtin_amdgcn_raw_buffer_load_b128(mrs, live ? mo + 16u * h : kNone, 0, 0));
    }
  }
  // the fp16 scales of the workgroup's weight rows: entry 16 i + r is row r
  // of its i-th tile (the launcher guarantees 16 tiles per lane cover them)
  const int mine = t0 < g.tiles ? (g.tiles - 1 - t0) / stride + 1 : 0;
  uint32_t swv[kSmallScales];
#pragma unroll
  for (int i = 0; i < kSmallScales; ++i) {
    const int e = tid + NT * i, n = 16 * (t0 + (e >> 4) * stride) + (e & 15);
    swv[i] = __builtin_amdgcn_raw_buffer_load_b16(srs, (e >> 4) < mine && n < g.n ? (uint32_t)n * 2u : kNone, 0, 0);
  }
  // the weight ring; rows past n read row n - 1 (never stored), tiles past
  // the workgroup's last load nothing
  i4v wr[M][S][2];
  // (every load is issued, with an offset past the buffer where it has
  // nothing to read, so that the compiler counts loads in flight exactly)
  auto fill = [&](int m, int t) {
    const bool tl = t < g.tiles;
    const int wrow = min(16 * t + r16, g.n - 1);
    const uint32_t vb = (uint32_t)wrow * (uint32_t)g.k + (uint32_t)(128 * wave + 32 * q);
#pragma unroll
    for (int j = 0; j < S; ++j) {
      const bool ok = tl && wave + WAVES * j < g.ksteps;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        wr[m][j][h] = __builtin_bit_cast(
            i4v, __builtin_amdgcn_raw_buffer_load_b128(wrs, ok ? vb + (uint32_t)(128 * WAVES * j + 16 * h) : kNone, 0, 0));
    }
  };
#pragma unroll
  for (int m = 0; m < M; ++m) fill(m, t0 + m * stride);

  // prologue: per-row absmax, the scales, the codes into LDS
  auto quotients = [&](int i, float* a) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[2 * e] = lo_h(xraw[i][e]);
      a[2 * e + 1] = hi_h(xraw[i][e]);
    }
    if constexpr (SMOOTH) {
      // (each factor is copied out of its vector first: a bit_cast taken
      // straight from a vector element read element 0 in this compiler)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t mb = mraw[i][e >> 2][e & 3];
        a[e] = __fdiv_rn(a[e], __builtin_bit_cast(float, mb));
      }
    }
  };
  float am[kSmallMaxB];
#pragma unroll
  for (int r = 0; r < kSmallMaxB; ++r) am[r] = 0.0f;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = tid + NT * i;
    if (c < pieces) {
      float a[8];
      quotients(i, a);
      float mx = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(a[e]));
      const int r = row_of(c);
#pragma unroll
      for (int rr = 0; rr < kSmallMaxB; ++rr)
        if (r == rr) am[rr] = fmaxf(am[rr], mx);
    }
  }
#pragma unroll
  for (int rr = 0; rr < kSmallMaxB; ++rr) {
    float v = am[rr];
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    if (lane == 0) amx[wave][rr] = v;
  }
#pragma unroll
  for (int i = 0; i < kSmallScales; ++i) sws[tid + NT * i] = (uint16_t)swv[i];
  // zeros: bytes k .. kp of every row, and the whole row b
  // (fewer than 8 pieces of 16 bytes lie past k in a row: k is a multiple of 32)
  if (tid < 8 * g.b && g.k + 16 * (tid & 7) < g.kp)
    *reinterpret_cast<i4v*>(xs + (tid >> 3) * g.kp + g.k + 16 * (tid & 7)) = i4v{0, 0, 0, 0};
  for (int z = 16 * tid; z < g.kp; z += 16 * NT) *reinterpret_cast<i4v*>(xs + g.b * g.kp + z) = i4v{0, 0, 0, 0};
  lds_barrier();
  // lane l takes the maximum of wave l / 4 for row l % 4; shuffles fold
  // the waves, and every lane takes row rr's result from lane rr
  float s[kSmallMaxB];
  {
    float v = lane / kSmallMaxB < WAVES ? amx[lane / kSmallMaxB][lane % kSmallMaxB] : 0.0f;
    for (int off = kSmallMaxB; off < 64; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
#pragma unroll
    for (int rr = 0; rr < kSmallMaxB; ++rr) s[rr] = __fdiv_rn(__shfl(v, rr, 64), 127.0f);
  }
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = tid + NT * i;
    if (c < pieces) {
      const int r = row_of(c);
      float sr = s[0];
#pragma unroll
      for (int rr = 1; rr < kSmallMaxB; ++rr)
        if (r == rr) sr = s[rr];
      float a[8];
      quotients(i, a);
      uint32_t packed[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = sr > 0.0f ? fminf(fmaxf(rintf(__fdiv_rn(a[e], sr)), -127.0f), 127.0f) : 0.0f;
        packed[e >> 2] |= ((uint32_t)(int)v & 0xFFu) << (8 * (e & 3));
      }
      *reinterpret_cast<uint2*>(xs + r * g.kp + 8 * (c - r * kc)) = make_uint2(packed[0], packed[1]);
    }
  }
  lds_barrier();

  // the product: this workgroup's tiles t0, t0 + stride, ..., in groups
  // of M (a group's tiles past the last load nothing and store nothing)
  const int xbase = (r16 < g.b ? r16 : g.b) * g.kp + 32 * q + 128 * wave;
  for (int it = 0; it < mine; it += M) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      {
        const int t = t0 + (it + m) * stride;
        int xo = xbase;
        asm volatile("" : "+v"(xo));  // the code reads stay in the loop (registers go to the ring)
        i4v acc = i4v{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < S; ++j)
          if (wave + WAVES * j < g.ksteps) {
            const i4v a0 = *reinterpret_cast<const i4v*>(xs + xo + 128 * WAVES * j);
            const i4v a1 = *reinterpret_cast<const i4v*>(xs + xo + 128 * WAVES * j + 16);
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, wr[m][j][0], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, wr[m][j][1], acc, 0, 0, 0);
          }
        fill(m, t + M * stride);
        const int p = (it + m) & 1;
        if (q == 0) red[p][wave][r16] = acc;
        lds_barrier();
        if (wave == 0) {  // lane (r16, q): output column r16 of activation row q
          const int* rp = reinterpret_cast<const int*>(&red[p][0][r16]) + q;
          int sum = 0;
#pragma unroll
          for (int w = 0; w < WAVES; ++w) sum += rp[64 * w];
          const int n = 16 * t + r16;
          float sq = s[0];
#pragma unroll
          for (int i = 1; i < kSmallMaxB; ++i)
            if (q == i) sq = s[i];
          float v = (sq * h2f(sws[16 * (it + m) + r16])) * (float)sum;
          asm volatile("" : "+v"(v));  // two binary32 roundings, then fp16 (as in w8a8_gemm_kernel)
          const uint32_t off = q < g.b && n < g.n ? ((uint32_t)q * (uint32_t)g.n + (uint32_t)n) * 2u : kNone;
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)v), yrs, off, 0, 0);
        }
      }
    }
  }
}

// ---- b <= 2 on the vector ALU -------------------------------------------------
//
// w8a8_dot_kernel: the quantizer and the product in one launch for one or two
// activation rows.  At b <= 2 a matrix-core step uses at most two of its 16
// activation rows; here each product is v_dot4_i32_i8 (four int8 x int8
// products added to an int32, exact), one instruction per 4 weight bytes and
// activation row.
//   * Prologue (every workgroup, on its own copy of x): the binary32 steps of
//     w8a8_quantize_kernel, so the codes and the scales are the same bits: a
//     = x / m (or x), per-row absmax by lane maxima, wave shuffles and one LDS
//     slot per wave and row, s = absmax / 127, codes into LDS as int8
//     [B][ldr] (ldr: k rounded up to a stage; the bytes past k are zeros).
//   * Product: a wave owns whole rows (rows gw, gw + TW, ...), each cut into
//     stages of P KiB: lane l loads bytes 1024 p + 16 l of the stage (p < P,
//     P wave loads of 1 KiB) and reads the same bytes of each activation
//     row's codes from LDS.  P is 4 (2 as a tuning override).  A ring of S
//     stages keeps S P KiB per wave in flight; a slot is refilled with the
//     stage S ahead as soon as its dots have read it.  At a row's last stage
//     the wave sums its lanes' int32 partials with DPP (exact in any order)
//     and lane r writes y[r] = f16((s_r * s_w) * acc_r), two binary32
//     multiplies, as the other forms.
constexpr int kDotThreads = 256;          // 4 waves per workgroup
constexpr int kDotMaxB = 2;               // activation rows of the dot4 forms
// 8-element pieces of x per lane: b k <= 16384 (b = 2 with k <= 8192)
constexpr int kDotPieces = 16384 / 8 / kDotThreads;

struct W8Dot {
  int n, k, b, kp, spr;  // spr: stages per row = kp / (1024 P)
  uint32_t codes_bytes, scales_bytes, x_bytes, m_bytes, y_bytes;
};

__device__ __forceinline__ int dpp_i32_add(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast15 into rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast31 into rows 2 and 3
  return __builtin_amdgcn_readlane(v, 63);
}

// The prologue of the dot4 forms.  x is [B][k] fp16, so piece c (8 elements)
// starts at byte 16 c and belongs to row c / kc; the thread's pieces are
// tid + NT i.  dot_load_x issues the loads (the oldest in flight);
// dot_quantize codes them into xs [B][ldr] and returns each row's scale.
template <bool SMOOTH, int B, int NT, int XP>
__device__ __forceinline__ void dot_load_x(u4v* xraw, u4v (*mraw)[2], __amdgpu_buffer_rsrc_t xrs,
                                           __amdgpu_buffer_rsrc_t mrs, int kc) {
#pragma unroll
  for (int i = 0; i < XP; ++i) {
    const int c = (int)threadIdx.x + NT * i;
    const bool live = c < B * kc;
    xraw[i] = __builtin_bit_cast(u4v, __builtin_amdgcn_raw_buffer_load_b128(xrs, live ? (uint32_t)c * 16u : kNone, 0, 0));
    if constexpr (SMOOTH) {
      const uint32_t e = (uint32_t)(c >= kc ? c - kc : c);  // piece within its row (B <= 2)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        mraw[i][h] = __builtin_bit_cast(
            u4v, __builtin_amdgcn_raw_buffer_load_b128(mrs, live ? e * 32u + 16u * h : kNone, 0, 0));
    }
  }
}

template <bool SMOOTH, int B, int NT, int XP>
__device__ __forceinline__ void dot_quantize(const u4v* xraw, const u4v (*mraw)[2], int kc, int k, int ldr,
                                             int8_t* xs, float* amx, float* s) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto quotients = [&](int i, float* a) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[2 * e] = lo_h(xraw[i][e]);
      a[2 * e + 1] = hi_h(xraw[i][e]);
    }
    if constexpr (SMOOTH) {
      // (each factor is copied out of its vector first: a bit_cast taken
      // straight from a vector element read element 0 in this compiler)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t mb = mraw[i][e >> 2][e & 3];
        a[e] = __fdiv_rn(a[e], __builtin_bit_cast(float, mb));
      }
    }
  };
  float am[B];
#pragma unroll
  for (int r = 0; r < B; ++r) am[r] = 0.0f;
#pragma unroll
  for (int i = 0; i < XP; ++i) {
    const int c = tid + NT * i;
    if (c < B * kc) {
      float a[8];
      quotients(i, a);
      float mx = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(a[e]));
      const int r = c >= kc ? 1 : 0;
#pragma unroll
      for (int rr = 0; rr < B; ++rr)
        if (r == rr) am[rr] = fmaxf(am[rr], mx);
    }
  }
#pragma unroll
  for (int r = 0; r < B; ++r) {
    float v = am[r];
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    if (lane == 0) amx[wave * B + r] = v;
  }
  // zeros past k in every row (ldr - k < a stage, in 16-byte pieces)
#pragma unroll
  for (int r = 0; r < B; ++r)
    for (int z = k + 16 * tid; z < ldr; z += 16 * NT) *reinterpret_cast<i4v*>(xs + r * ldr + z) = i4v{0, 0, 0, 0};
  lds_barrier();
#pragma unroll
  for (int r = 0; r < B; ++r) {
    float mx = amx[r];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) mx = fmaxf(mx, amx[w * B + r]);
    s[r] = __fdiv_rn(mx, 127.0f);
  }
#pragma unroll
  for (int i = 0; i < XP; ++i) {
    const int c = tid + NT * i;
    if (c < B * kc) {
      const int r = c >= kc ? 1 : 0;
      const float sr = r ? s[B - 1] : s[0];
      float a[8];
      quotients(i, a);
      uint32_t packed[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = sr > 0.0f ? fminf(fmaxf(rintf(__fdiv_rn(a[e], sr)), -127.0f), 127.0f) : 0.0f;
        packed[e >> 2] |= ((uint32_t)(int)v & 0xFFu) << (8 * (e & 3));
      }
      *reinterpret_cast<uint2*>(xs + r * ldr + 8 * (c - r * kc)) = make_uint2(packed[0], packed[1]);
    }
  }
  lds_barrier();
}

template <bool SMOOTH, int P, int S, int B>
__global__ void __launch_bounds__(kDotThreads)
w8a8_dot_kernel(const int8_t* __restrict__ wq, const _Float16* __restrict__ sw, const _Float16* __restrict__ x,
                const float* __restrict__ smooth, _Float16* __restrict__ y, W8Dot g) {
  constexpr int STAGE = 1024 * P;  // bytes of a row per stage
  extern __shared__ __attribute__((aligned(16))) int8_t xs[];  // activation codes [B][kp]
  __shared__ float amx[kDotThreads / 64 * B];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(wq, g.codes_bytes);
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(sw, g.scales_bytes);
  const __amdgpu_buffer_rsrc_t yrs = make_rsrc(y, g.y_bytes);
  const int kc = g.k >> 3;  // 8-element pieces of an activation row

  u4v xraw[kDotPieces];
  u4v mraw[kDotPieces][2];
  dot_load_x<SMOOTH, B, kDotThreads, kDotPieces>(xraw, mraw, make_rsrc(x, g.x_bytes), make_rsrc(smooth, g.m_bytes), kc);

  // rows of this wave: gw, gw + tw, ...; a stage is (row, st) with st < spr.
  // The fill and consume positions advance one stage per call (wave-uniform
  // counters, no division); every load is issued (past the wave's last
  // row, or past k, at an offset the range check turns into zeros), so the
  // compiler counts the loads in flight exactly.
  const int gw = (int)blockIdx.x * (kDotThreads / 64) + wave, tw = (int)gridDim.x * (kDotThreads / 64);
  int f_row = gw, f_st = 0;
  i4v wr[S][P];
  uint32_t swr[S];
  auto fill = [&](int m) {
    const bool live = f_row < g.n;
    const uint32_t base = (uint32_t)f_row * (uint32_t)g.k;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const uint32_t kb = (uint32_t)(STAGE * f_st + 1024 * p + 16 * lane);
      wr[m][p] = __builtin_bit_cast(
          i4v, __builtin_amdgcn_raw_buffer_load_b128(wrs, live && kb < (uint32_t)g.k ? base + kb : kNone, 0, 0));
    }
    swr[m] = __builtin_amdgcn_raw_buffer_load_b16(srs, live ? (uint32_t)f_row * 2u : kNone, 0, 0);
    if (++f_st == g.spr) {
      f_st = 0;
      f_row += tw;
    }
  };
#pragma unroll
  for (int m = 0; m < S; ++m) {
    fill(m);
    __builtin_amdgcn_sched_barrier(0);
  }

  float s[B];
  dot_quantize<SMOOTH, B, kDotThreads, kDotPieces>(xraw, mraw, kc, g.k, g.kp, xs, amx, s);

  // the product
  int acc[B];
#pragma unroll
  for (int r = 0; r < B; ++r) acc[r] = 0;
  int c_row = gw, c_st = 0;
  auto consume = [&](int m) {
    const int8_t* xb = xs + STAGE * c_st + 16 * lane;
#pragma unroll
    for (int p = 0; p < P; ++p) {
#pragma unroll
      for (int r = 0; r < B; ++r) {
        const i4v xv = *reinterpret_cast<const i4v*>(xb + r * g.kp + 1024 * p);
#pragma unroll
        for (int d = 0; d < 4; ++d) acc[r] = __builtin_amdgcn_sdot4(wr[m][p][d], xv[d], acc[r], false);
      }
    }
    const float ws = h2f((uint16_t)swr[m]);
    fill(m);
    // a row ends here: the wave's int32 sums, then y[r] from lane r (a store
    // is issued on every stage, dropped where there is nothing to write, so
    // that no wait count depends on the path)
    float v = 0.0f;
    uint32_t off = kNone;
    if (c_st == g.spr - 1) {
      int sum = 0;
#pragma unroll
      for (int r = 0; r < B; ++r) {
        const int t = dpp_i32_add(acc[r]);
        acc[r] = 0;
        if (lane == r) {
          sum = t;
          v = (s[r] * ws) * (float)sum;
        }
      }
      asm volatile("" : "+v"(v));  // two binary32 roundings, then fp16 (as in w8a8_gemm_kernel)
      if (lane < B) off = ((uint32_t)lane * (uint32_t)g.n + (uint32_t)c_row) * 2u;
    }
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)v), yrs, off, 0, 0);
    if (++c_st == g.spr) {
      c_st = 0;
      c_row += tw;
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  while (c_row < g.n) {
#pragma unroll
    for (int m = 0; m < S; ++m)
      if (c_row < g.n) consume(m);
  }
}

// w8a8_dot_split_kernel: the same product for 8192 < k <= 16384, each row
// split over KS = ceil(k / 2048) waves.  One wave alone on such a row
// streams up to 16 KiB through a short ring (the 4096 x 14336 down gives
// each of 3072 waves one or two rows), so here a workgroup is one row
// walker of KS waves: wave h takes bytes 2048 h .. 2048 h + 2047 of every
// row it visits (lane l: 16 bytes at 1024 p + 16 l, p = 0, 1), holding its
// 32 bytes of each activation row's codes in registers for the launch.  S
// rows are in flight per wave.  Each wave sums its lanes' int32 partials
// with DPP and writes the row's partials to an LDS slot; after every M rows
// one barrier, and lane B j + r of wave 0 adds the KS partials of row j,
// activation row r (integer adds: exact in any order), and writes y with
// the same two binary32 multiplies.
constexpr int kSplitRing = 4;   // rows in flight per wave
constexpr int kSplitBatch = 16; // rows per LDS batch

template <bool SMOOTH, int KS, int B>
__global__ void __launch_bounds__(64 * KS)
w8a8_dot_split_kernel(const int8_t* __restrict__ wq, const _Float16* __restrict__ sw, const _Float16* __restrict__ x,
                      const float* __restrict__ smooth, _Float16* __restrict__ y, W8Dot g) {
  constexpr int NT = 64 * KS;
  constexpr int XP = (B * 16384 / 8 + NT - 1) / NT;  // 8-element pieces of x per lane (k <= 16384)
  constexpr int S = kSplitRing, M = kSplitBatch;
  constexpr int LDR = KS * 2048;  // bytes per activation row of codes
  __shared__ __attribute__((aligned(16))) int8_t xs[B * LDR];  // activation codes, zeros past k
  __shared__ float amx[KS * B];
  __shared__ int red[2][M][B][KS];
  __shared__ float rsc[2][M];
  const int tid = threadIdx.x, lane = tid & 63;
  const int h = __builtin_amdgcn_readfirstlane(tid >> 6);
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(wq, g.codes_bytes);
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(sw, g.scales_bytes);
  const __amdgpu_buffer_rsrc_t yrs = make_rsrc(y, g.y_bytes);
  const int kc = g.k >> 3;

  u4v xraw[XP];
  u4v mraw[XP][2];
  dot_load_x<SMOOTH, B, NT, XP>(xraw, mraw, make_rsrc(x, g.x_bytes), make_rsrc(smooth, g.m_bytes), kc);

  // this workgroup's rows: blockIdx.x, + gridDim.x, ...
  const int first = (int)blockIdx.x, stride = (int)gridDim.x;
  const int count = first < g.n ? (g.n - 1 - first) / stride + 1 : 0;
  const uint32_t kb0 = (uint32_t)(2048 * h + 16 * lane);
  i4v wr[S][2];
  uint32_t swr[S];
  // every load is issued (rows past the walker's last at an offset the
  // range check turns into zeros), so the compiler counts them exactly
  auto fill = [&](int m, int i) {
    const bool live = i < count;
    const uint32_t base = (uint32_t)(first + i * stride) * (uint32_t)g.k;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const uint32_t kb = kb0 + 1024u * p;
      wr[m][p] = __builtin_bit_cast(
          i4v, __builtin_amdgcn_raw_buffer_load_b128(wrs, live && kb < (uint32_t)g.k ? base + kb : kNone, 0, 0));
    }
    swr[m] = __builtin_amdgcn_raw_buffer_load_b16(srs, live ? (uint32_t)(first + i * stride) * 2u : kNone, 0, 0);
  };
#pragma unroll
  for (int m = 0; m < S; ++m) {
    fill(m, m);
    __builtin_amdgcn_sched_barrier(0);
  }

  float s[B];
  dot_quantize<SMOOTH, B, NT, XP>(xraw, mraw, kc, g.k, LDR, xs, amx, s);
  i4v xv[B][2];
#pragma unroll
  for (int r = 0; r < B; ++r)
#pragma unroll
    for (int p = 0; p < 2; ++p) xv[r][p] = *reinterpret_cast<const i4v*>(xs + r * LDR + kb0 + 1024u * p);

  // the product, S rows per round, an LDS batch every M rows
  for (int it = 0; it < count; it += S) {
#pragma unroll
    for (int m = 0; m < S; ++m) {
      const int i = it + m;  // (workgroup-uniform)
      if (i < count) {
#pragma unroll
        for (int r = 0; r < B; ++r) {
          int acc = __builtin_amdgcn_sdot4(wr[m][0][0], xv[r][0][0], 0, false);
#pragma unroll
          for (int d = 1; d < 4; ++d) acc = __builtin_amdgcn_sdot4(wr[m][0][d], xv[r][0][d], acc, false);
#pragma unroll
          for (int d = 0; d < 4; ++d) acc = __builtin_amdgcn_sdot4(wr[m][1][d], xv[r][1][d], acc, false);
          const int sum = dpp_i32_add(acc);
          if (lane == 0) red[(i / M) & 1][i % M][r][h] = sum;
        }
        const float ws = h2f((uint16_t)swr[m]);
        if (lane == 0 && h == 0) rsc[(i / M) & 1][i % M] = ws;
      }
      fill(m, i + S);
      __builtin_amdgcn_sched_barrier(0);
    }
    if ((it + S) % M == 0 || it + S >= count) {
      lds_barrier();
      if (h == 0) {
        const int b0 = it / M * M, buf = (it / M) & 1;
        const int j = lane / B, r = lane % B;
        float v = 0.0f;
        uint32_t off = kNone;
        if (j < M && b0 + j < count) {
          int total = 0;
#pragma unroll
          for (int w = 0; w < KS; ++w) total += red[buf][j][r][w];
          v = ((r ? s[B - 1] : s[0]) * rsc[buf][j]) * (float)total;
          asm volatile("" : "+v"(v));  // two binary32 roundings, then fp16 (as in w8a8_gemm_kernel)
          off = ((uint32_t)r * (uint32_t)g.n + (uint32_t)(first + (b0 + j) * stride)) * 2u;
        }
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)v), yrs, off, 0, 0);
      }
    }
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

namespace {

template <int WAVES, int S>
void* pick_small(bool smooth) {
  return smooth ? reinterpret_cast<void*>(w8a8_small_kernel<WAVES, S, true>)
                : reinterpret_cast<void*>(w8a8_small_kernel<WAVES, S, false>);
}

// The fused form where it applies (b <= 4, the rows' pieces fit the
// prologue's registers, QGEMV_W8A8_FUSE_MAX_B not below b); returns false
// without launching otherwise.
bool launch_small(const WeightView& w, const _Float16* x, const float* smooth, _Float16* y, int b, hipStream_t s,
                  hipError_t& err) {
  const int fuse_max = tuning(kTuneW8a8FuseMaxB, kSmallMaxB);
  if (b > fuse_max || b > kSmallMaxB) return false;
  const int ksteps = (w.k + 127) / 128;
  int waves = pow2_at_least(ksteps);
  waves = waves < 4 ? 4 : waves > 16 ? 16 : waves;
  const int steps = pow2_at_least((ksteps + waves - 1) / waves);  // 1 where waves < 16; at most 8 (k <= 16384)
  if ((long)b * (w.k / 8) > (long)small_chunks(steps) * 64 * waves) return false;
  W8Small g;
  g.n = w.n;
  g.k = w.k;
  g.b = b;
  g.tiles = (w.n + 15) / 16;
  g.ksteps = ksteps;
  g.kp = ksteps * 128;
  g.codes_bytes = (uint32_t)buffer_bytes(Q_INT8, w.n, w.k, w.k, Q_BUF_CODES);
  g.scales_bytes = (uint32_t)buffer_bytes(Q_INT8, w.n, w.k, w.k, Q_BUF_SCALES);
  g.x_bytes = (uint32_t)(b * w.k * 2);
  g.m_bytes = smooth ? (uint32_t)(w.k * 4) : 0u;
  g.y_bytes = (uint32_t)((size_t)b * (size_t)w.n * 2u);
  // persistent: 16 waves per compute unit
  int grid = device_cu_count() * (16 / waves);
  if (grid > g.tiles) grid = g.tiles;
  // the prologue loads the scales of every tile a workgroup visits (its
  // tiles rounded up to the ring's M) into LDS: 16 per tile.  Long tile
  // walks keep the two-kernel form: measured on 128256 x 4096 at b = 1
  // (31 tiles per workgroup), its loop with the activations in registers
  // ran 91 us against 95 us fused, while on 14336 x 4096 (3.5 tiles) the
  // fused form ran 13.7 us against 16.5 us
  const int ring_tiles = kSmallRing > steps ? kSmallRing / steps : 1;
  const int visits = ((g.tiles + grid - 1) / grid + ring_tiles - 1) / ring_tiles * ring_tiles;
  if (visits > kSmallMaxVisits || 16 * visits > kSmallScales * 64 * waves) return false;
  const bool sm = smooth != nullptr;
  void* fn = waves == 4    ? pick_small<4, 1>(sm)
             : waves == 8  ? pick_small<8, 1>(sm)
             : steps == 1  ? pick_small<16, 1>(sm)
             : steps == 2  ? pick_small<16, 2>(sm)
             : steps == 4  ? pick_small<16, 4>(sm)
                           : pick_small<16, 8>(sm);
  const int8_t* wc = reinterpret_cast<const int8_t*>(w.codes);
  const _Float16* wsc = static_cast<const _Float16*>(w.scales);
  void* args[] = {&wc, &wsc, &x, &smooth, &y, &g};
  err = hipLaunchKernel(fn, dim3(grid), dim3(64 * waves), args, (size_t)(b + 1) * (size_t)g.kp, s);
  return true;
}

}  // namespace

namespace {

template <int P, int S, int B>
void* pick_dot(bool smooth) {
  return smooth ? reinterpret_cast<void*>(w8a8_dot_kernel<true, P, S, B>)
                : reinterpret_cast<void*>(w8a8_dot_kernel<false, P, S, B>);
}

template <int KS, int B>
void* pick_dot_split(bool smooth) {
  return smooth ? reinterpret_cast<void*>(w8a8_dot_split_kernel<true, KS, B>)
                : reinterpret_cast<void*>(w8a8_dot_split_kernel<false, KS, B>);
}

template <int B>
void* pick_dot_split_ks(int ks, bool smooth) {
  return ks <= 5 ? pick_dot_split<5, B>(smooth) : ks == 6 ? pick_dot_split<6, B>(smooth)
         : ks == 7 ? pick_dot_split<7, B>(smooth) : pick_dot_split<8, B>(smooth);
}

void fill_dot_geom(const WeightView& w, int b, const float* smooth, W8Dot& g) {
  g.n = w.n;
  g.k = w.k;
  g.b = b;
  g.codes_bytes = (uint32_t)buffer_bytes(Q_INT8, w.n, w.k, w.k, Q_BUF_CODES);
  g.scales_bytes = (uint32_t)buffer_bytes(Q_INT8, w.n, w.k, w.k, Q_BUF_SCALES);
  g.x_bytes = (uint32_t)(b * w.k * 2);
  g.m_bytes = smooth ? (uint32_t)(w.k * 4) : 0u;
  g.y_bytes = (uint32_t)((size_t)b * (size_t)w.n * 2u);
}

// k > 8192: each row over KS = ceil(k / 2048) waves.  At b = 1 by default
// from k > 12288, two row walkers per compute unit (MI355X, graph replay,
// b = 1: 4096 x 14336 13.4 us against 14.0 with one wave per row, 8192 x
// 14336 21.4 against 23.3; 4096 x 12288 12.7 against 12.2, so not there);
// at b = 2 for every k > 8192, where one wave per row would hold too many
// activation pieces.  QGEMV_W8A8_DOT_SPLIT=1 takes it at b = 1 for every
// k > 8192, 0 never.
hipError_t launch_dot_split(const WeightView& w, const _Float16* x, const float* smooth, _Float16* y, int b,
                            hipStream_t s) {
  const int ks = (w.k + 2047) / 2048;  // 5..8
  W8Dot g;
  fill_dot_geom(w, b, smooth, g);
  g.kp = ks * 2048;
  g.spr = 1;
  // row walkers (one per workgroup) per compute unit: 2 at b = 1, 1 at b = 2,
  // whose workgroups each quantize twice the activations (4096 x 14336 at
  // b = 2: 17.1 us against 19.6 with 2); QGEMV_W8A8_DOT_WALKERS_PER_CU
  const int per_cu = std::max(1, tuning(kTuneW8a8DotWalkersPerCu, b == 1 ? 2 : 1));
  int grid = device_cu_count() * per_cu;
  if (grid > w.n) grid = w.n;
  const bool sm = smooth != nullptr;
  void* fn = b == 1 ? pick_dot_split_ks<1>(ks, sm) : pick_dot_split_ks<2>(ks, sm);
  const int8_t* wc = reinterpret_cast<const int8_t*>(w.codes);
  const _Float16* wsc = static_cast<const _Float16*>(w.scales);
  void* args[] = {&wc, &wsc, &x, &smooth, &y, &g};
  return hipLaunchKernel(fn, dim3(grid), dim3(64 * ks), args, 0, s);
}

// The dot4 forms for b <= 2 (k <= 16384).
hipError_t launch_dot(const WeightView& w, const _Float16* x, const float* smooth, _Float16* y, int b, hipStream_t s) {
  const int split = tuning(kTuneW8a8DotSplit, -1);
  if (w.k > 8192 && (b == 2 || split > 0 || (split < 0 && w.k > 12288)))
    return launch_dot_split(w, x, smooth, y, b, s);
  // stages of P = 4 KiB of a row, two of them in flight per wave, 12 waves
  // per compute unit: the best of P = 2 / 4 / 7, S = 2 / 4 and 4-16 waves
  // per CU on the Llama-3-8B FFN and lm_head shapes (MI355X, graph replay,
  // b = 1: 14336 x 4096 11.3 us, 4096 x 14336 13.8, 128256 x 4096 85-87).
  // P = 2 (QGEMV_W8A8_DOT_P) and S = 4 (QGEMV_W8A8_DOT_S) stay for the tests.
  int P = tuning(kTuneW8a8DotP, 4);
  if (P != 2) P = 4;
  int S = tuning(kTuneW8a8DotS, 2);
  if (S != 4) S = 2;
  W8Dot g;
  fill_dot_geom(w, b, smooth, g);
  g.kp = (w.k + 1024 * P - 1) / (1024 * P) * (1024 * P);
  g.spr = g.kp / (1024 * P);
  // persistent: QGEMV_W8A8_DOT_WAVES_PER_CU waves per compute unit, 12, or 8
  // on long row walks (128256 x 4096 at b = 1: 85.0-85.7 us against
  // 87.3-89.9 with 12)
  const int wpc = tuning(kTuneW8a8DotWavesPerCu, w.n > 65536 ? 8 : 12);
  const int per_cu = wpc / (kDotThreads / 64) > 1 ? wpc / (kDotThreads / 64) : 1;
  int grid = device_cu_count() * per_cu;
  const int need = (w.n + kDotThreads / 64 - 1) / (kDotThreads / 64);  // one row per wave at least
  if (grid > need) grid = need;
  const bool sm = smooth != nullptr;
  void* fn;
  if (b == 1)
    fn = P == 4 ? (S == 2 ? pick_dot<4, 2, 1>(sm) : pick_dot<4, 4, 1>(sm))
                : (S == 2 ? pick_dot<2, 2, 1>(sm) : pick_dot<2, 4, 1>(sm));
  else
    fn = P == 4 ? (S == 2 ? pick_dot<4, 2, 2>(sm) : pick_dot<4, 4, 2>(sm))
                : (S == 2 ? pick_dot<2, 2, 2>(sm) : pick_dot<2, 4, 2>(sm));
  const int8_t* wc = reinterpret_cast<const int8_t*>(w.codes);
  const _Float16* wsc = static_cast<const _Float16*>(w.scales);
  void* args[] = {&wc, &wsc, &x, &smooth, &y, &g};
  return hipLaunchKernel(fn, dim3(grid), dim3(kDotThreads), args, (size_t)b * (size_t)g.kp, s);
}

}  // namespace

hipError_t launch_w8a8(const WeightView& w, const _Float16* x, const float* smooth, _Float16* y, int b, void* ws,
                       hipStream_t s) {
  // the dot4 forms: by default at b = 1, and at b = 2 unless the rows are
  // many (128256 x 4096 at b = 2: 90.1 us against 88.3 for the two-kernel
  // form; 14336 x 4096: 12.8 against 14.7 fused, 4096 x 14336: 17.1 against
  // 19.5); QGEMV_W8A8_DOT = d forces them for b <= d (0 turns them off)
  const int dot_max = tuning(kTuneW8a8Dot, -1);
  const bool dot = dot_max >= 0 ? b <= std::min(dot_max, kDotMaxB) : (b == 1 || (b == 2 && w.n <= 65536));
  if (dot) return launch_dot(w, x, smooth, y, b, s);
  hipError_t fused;
  if (launch_small(w, x, smooth, y, b, s, fused)) return fused;
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
