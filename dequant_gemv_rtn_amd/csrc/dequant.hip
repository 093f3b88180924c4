// Debug export: packed weights back to fp16 W_deq [n][k].
//
// Each thread decodes the 8 consecutive elements of one row that share a
// 32-bit code word (two words for int8), element by element from the packed
// layout, forms the exact value in fp32 and rounds it once to fp16.  The
// product kernels never materialize W_deq; this path exists so that tests can
// compare a layout decode on the device bit for bit with the reference.
//
// Values (the format definitions the product kernels decode as well):
//   int4_asym  (q - z) * s                     per group of g
//   fp4_e2m1   (-1)^sign * M[idx] * s           M = {0, .5, 1, 1.5, 2, 3, 4, 6}
//   fp4_razer  as e2m1, but code 8 (-0) is the group's special value v * s
//   fp4_afpq   +M * s+ for sign 0, -M * s- for sign 1
//   bfp6/bfp4  m * 2^(E - 127 - Mb + 1), m the two's complement mantissa
//   int8       q * s_row
//   fp3_razer  (-1)^sign * M3[idx] * s, M3 = {0, 1, 2, 4}; code 4 (-0) is the
//              group's special value v * s, v in {+3, -3, +8, -8}
//   fp3_afpq   +M3 * s+ for sign 0, -M3 * s- for sign 1
// Every product is exact in fp32 (at most 19 significant bits).  3-bit codes
// are read element by element from their bit positions in the piece's three
// words (the layout in qgemv.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"
#include "internal.hpp"

namespace qg {
namespace {

struct DequantGeom {
  int n, k, group, groups;   // groups per row (k / group) for the group formats
  uint32_t aux_row_words;    // u32 words per row of int4 zeros / razer selectors
};

__device__ __forceinline__ float half_at(const void* p, uint64_t i) {
  return h2f(static_cast<const uint16_t*>(p)[i]);
}

__device__ __forceinline__ float e2m1_magnitude(uint32_t idx) {
  // {0, 0.5, 1, 1.5, 2, 3, 4, 6}: 2^(e-1) (1 + m/2) for e >= 1, m / 2 for e = 0
  const uint32_t e = idx >> 1, m = idx & 1u;
  return e == 0 ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, (int)e - 1);
}

template <int FMT>
__global__ void __launch_bounds__(256) dequant_kernel(WeightView W, _Float16* __restrict__ out, DequantGeom g) {
  const uint64_t words_row = (uint64_t)g.k / 8;
  const uint64_t total = (uint64_t)g.n * words_row;
  for (uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (uint64_t)gridDim.x * blockDim.x) {
    const uint64_t row = t / words_row;
    const uint32_t word = (uint32_t)(t % words_row);
    const uint32_t k0 = word * 8u;
    float v[8];
    if constexpr (FMT == Q_INT8) {
      const uint32_t* c = W.codes + row * ((uint64_t)g.k / 4) + 2u * word;
      const float s = half_at(W.scales, row);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int8_t q = (int8_t)((c[e >> 2] >> (8 * (e & 3))) & 0xFFu);
        v[e] = (float)q * s;
      }
    } else if constexpr (is_fp3(FMT)) {
      // these 8 elements are the q-th group of eight of their 32-element piece
      const uint32_t* piece = W.codes + row * ((uint64_t)g.k / 32) * 3 + (uint64_t)(word / 4) * 3;
      const uint32_t q = word % 4;
      const uint32_t iw = piece[q / 2], sg = piece[2];
      const uint32_t gi = k0 / (uint32_t)g.group;
      const uint64_t gidx = row * (uint64_t)g.groups + gi;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const uint32_t b0 = (q & 1u) ? 4u * r + 3u : 4u * r + 1u;
        const uint32_t b1 = (q & 1u) ? (4u * r + 4u) & 31u : 4u * r + 2u;
        const uint32_t idx = ((iw >> b0) & 1u) | (((iw >> b1) & 1u) << 1);
        const uint32_t sign = (sg >> (4u * r + 3u - q)) & 1u;
        const float mag = idx == 0 ? 0.0f : ldexpf(1.0f, (int)idx - 1);
        if constexpr (FMT == Q_FP3_AFPQ) {
          v[r] = sign ? -mag * half_at(W.scales, 2 * gidx + 1) : mag * half_at(W.scales, 2 * gidx);
        } else {
          const float s = half_at(W.scales, gidx);
          float val = sign ? -mag * s : mag * s;
          if (sign && idx == 0) {
            const uint32_t sw = static_cast<const uint32_t*>(W.aux)[row * g.aux_row_words + gi / 16];
            val = razer_special_of<Q_FP3_RAZER>((int)((sw >> (2 * (gi % 16))) & 3u)) * s;
          }
          v[r] = val;
        }
      }
    } else {
      const uint32_t c = W.codes[row * words_row + word];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t k = k0 + (uint32_t)e;
        const uint32_t code = (c >> (4 * e)) & 0xFu;
        if constexpr (FMT == Q_BFP4 || FMT == Q_BFP6) {
          constexpr int mb = FMT == Q_BFP6 ? 5 : 3;
          const uint64_t blk = row * ((uint64_t)g.k / 16) + k / 16;
          int m;
          if constexpr (FMT == Q_BFP6) {
            const uint32_t eb = k % 16;
            const uint32_t pos = 16u * ((eb % 8) / 4) + 8u * (eb / 8) + 2u * (eb % 4);
            const uint32_t hi = (W.codes_hi[blk] >> pos) & 3u;
            const int c6 = (int)(code | (hi << 4));
            m = c6 >= 32 ? c6 - 64 : c6;
          } else {
            m = code >= 8 ? (int)code - 16 : (int)code;
          }
          const int E = static_cast<const uint8_t*>(W.aux)[blk];
          v[e] = E ? (float)m * ldexpf(1.0f, E - 127 - mb + 1) : 0.0f;
        } else {
          const uint32_t gi = k / (uint32_t)g.group;
          const uint64_t gidx = row * (uint64_t)g.groups + gi;
          if constexpr (FMT == Q_INT4_ASYM) {
            const uint32_t zw = static_cast<const uint32_t*>(W.aux)[row * g.aux_row_words + gi / 8];
            const int z = (int)((zw >> (4 * (gi % 8))) & 0xFu);
            v[e] = (float)((int)code - z) * half_at(W.scales, gidx);
          } else if constexpr (FMT == Q_FP4_AFPQ) {
            const float mag = e2m1_magnitude(code & 7u);
            v[e] = (code & 8u) ? -mag * half_at(W.scales, 2 * gidx + 1) : mag * half_at(W.scales, 2 * gidx);
          } else {
            const float s = half_at(W.scales, gidx);
            float val = e2m1_magnitude(code & 7u) * s;
            if (code & 8u) val = -val;
            if constexpr (FMT == Q_FP4_RAZER) {
              if (code == 8u) {
                const uint32_t sw = static_cast<const uint32_t*>(W.aux)[row * g.aux_row_words + gi / 16];
                val = razer_special((int)((sw >> (2 * (gi % 16))) & 3u)) * s;
              }
            }
            v[e] = val;
          }
        }
      }
    }
    uint32_t packed[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const _Float16 a = (_Float16)v[2 * i], b = (_Float16)v[2 * i + 1];
      packed[i] = (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
    }
    *reinterpret_cast<uint4*>(out + row * (uint64_t)g.k + k0) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  }
}

}  // namespace

hipError_t launch_dequant(const WeightView& w, _Float16* out, hipStream_t s) {
  DequantGeom g;
  g.n = w.n;
  g.k = w.k;
  g.group = w.group;
  g.groups = w.k / w.group;
  g.aux_row_words = (uint32_t)(w.fmt == Q_INT4_ASYM ? (g.groups + 7) / 8 : (g.groups + 15) / 16);
  const uint64_t total = (uint64_t)w.n * (uint64_t)(w.k / 8);
  uint64_t blocks = (total + 255) / 256;
  const uint64_t cap = (uint64_t)device_cu_count() * 16;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks), block(256);
  switch (w.fmt) {
    case Q_INT4_ASYM: hipLaunchKernelGGL(dequant_kernel<Q_INT4_ASYM>, grid, block, 0, s, w, out, g); break;
    case Q_FP4_E2M1: hipLaunchKernelGGL(dequant_kernel<Q_FP4_E2M1>, grid, block, 0, s, w, out, g); break;
    case Q_FP4_RAZER: hipLaunchKernelGGL(dequant_kernel<Q_FP4_RAZER>, grid, block, 0, s, w, out, g); break;
    case Q_FP4_AFPQ: hipLaunchKernelGGL(dequant_kernel<Q_FP4_AFPQ>, grid, block, 0, s, w, out, g); break;
    case Q_BFP6: hipLaunchKernelGGL(dequant_kernel<Q_BFP6>, grid, block, 0, s, w, out, g); break;
    case Q_BFP4: hipLaunchKernelGGL(dequant_kernel<Q_BFP4>, grid, block, 0, s, w, out, g); break;
    case Q_INT8: hipLaunchKernelGGL(dequant_kernel<Q_INT8>, grid, block, 0, s, w, out, g); break;
    case Q_FP3_RAZER: hipLaunchKernelGGL(dequant_kernel<Q_FP3_RAZER>, grid, block, 0, s, w, out, g); break;
    case Q_FP3_AFPQ: hipLaunchKernelGGL(dequant_kernel<Q_FP3_AFPQ>, grid, block, 0, s, w, out, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qg
