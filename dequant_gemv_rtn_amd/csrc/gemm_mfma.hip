// MFMA fused-dequantization skinny GEMM for 9 <= b <= 64 activation rows.
//
// With 16 or more activation rows the product is a dense contraction, so it
// runs on the matrix cores: v_mfma_f32_16x16x32_f16 with the weight tile as
// the A operand (16 output rows x 32 k) and the activations as B (32 k x 16
// batch rows), fp32 accumulation.  Each wave owns 16 output rows; a
// workgroup of 4 waves owns 64 rows and walks k in slices whose activations
// are staged once in LDS (in the decoders' pair order) for all four waves.
//
// A operand: lane l loads 16 contiguous bytes of row (l mod 16) -- a
// coalesced 128-bit load -- and decodes them into A fragments.
//  * Group formats (int4_asym, fp4_e2m1, fp4_razer, fp4_afpq): the four
//    16-lane groups exchange words so that every MFMA step covers 32
//    consecutive k of one group; A holds exact unscaled values and the group
//    scale multiplies the fp32 partial (gemm_mfma_group_kernel).
//  * Block formats: the power-of-two block step is folded into the fp16 A
//    values (exact while the block maximum is at least 2^-20).
//  * int8: A holds the exact integers; the row scale multiplies the result.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"
#include "internal.hpp"

namespace qg {
namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWg = 16 * kWaves;

__device__ __forceinline__ uint32_t pk_mul(uint32_t a, h2 s) { return as_u32(as_h2(a) * s); }

// Per-lane metadata of one piece: fp16 scale pair for the A operand.
struct AMeta {
  h2 s0, s1;  // int4: (s,s),(1024+z,..); e2m1: (s,s); razer: (s,s),(v,v); afpq: (s+,s+),(s-,s-); bfp: block steps
};

template <int FMT>
__device__ __forceinline__ AMeta load_ameta(const WeightView& W, int row, int kk) {
  AMeta m;
  m.s0 = h2{(_Float16)0.0f, (_Float16)0.0f};
  m.s1 = m.s0;
  if constexpr (FMT == Q_INT8) {
    (void)W; (void)row; (void)kk;
  } else if constexpr (FMT == Q_BFP6 || FMT == Q_BFP4) {
    constexpr int mb = FMT == Q_BFP6 ? 5 : 3;
    const uint16_t e2 = *reinterpret_cast<const uint16_t*>(
        reinterpret_cast<const uint8_t*>(W.aux) + (size_t)row * (W.k / 16) + kk / 16);
    const _Float16 a = (_Float16)((e2 & 0xFF) ? ldexpf(1.0f, (int)(e2 & 0xFF) - 127 - mb + 1) : 0.0f);
    const _Float16 b = (_Float16)((e2 >> 8) ? ldexpf(1.0f, (int)(e2 >> 8) - 127 - mb + 1) : 0.0f);
    m.s0 = h2{a, a};
    m.s1 = h2{b, b};
  } else {
    const int groups = W.k / W.group;
    const int gi = kk / W.group;
    if constexpr (FMT == Q_FP4_AFPQ) {
      const uint32_t pr = reinterpret_cast<const uint32_t*>(W.scales)[(size_t)row * groups + gi];
      m.s0 = as_h2((pr & 0xFFFFu) * 0x00010001u);
      m.s1 = as_h2((pr >> 16) * 0x00010001u);
    } else {
      const uint32_t sb = reinterpret_cast<const uint16_t*>(W.scales)[(size_t)row * groups + gi];
      m.s0 = as_h2(sb * 0x00010001u);
      if constexpr (FMT == Q_INT4_ASYM) {
        const int zw = (groups + 7) / 8;
        const uint32_t z = reinterpret_cast<const uint32_t*>(W.aux)[(size_t)row * zw + gi / 8];
        const _Float16 zb = (_Float16)(1024.0f + (float)((z >> (4 * (gi & 7))) & 0xFu));
        m.s1 = h2{zb, zb};
      } else if constexpr (FMT == Q_FP4_RAZER) {
        const int sw = (groups + 15) / 16;
        const uint32_t sl = reinterpret_cast<const uint32_t*>(W.aux)[(size_t)row * sw + gi / 16];
        const _Float16 v = (_Float16)razer_special((int)((sl >> (2 * (gi & 15))) & 3u));
        m.s1 = h2{v, v};
      }
    }
  }
  return m;
}

// Decode one code word (8 elements; int8: two words -> one fragment) into the
// fp16 A fragment of one MFMA step, scale folded in.
template <int FMT>
__device__ __forceinline__ h8 decode_fragment(uint32_t w, uint32_t w2, uint32_t hi, int hsh, const AMeta& m,
                                              int block) {
  if constexpr (FMT == Q_FP4_E2M1 || FMT == Q_FP4_RAZER || FMT == Q_FP4_AFPQ) {
    uint32_t d[4] = {as_u32(fp4_pair<0>(w)), as_u32(fp4_pair<1>(w)), as_u32(fp4_pair<2>(w)),
                     as_u32(fp4_pair<3>(w))};
    if constexpr (FMT == Q_FP4_RAZER) {
      const uint32_t sm = special_mask(w, 0x88888888u);
      const uint32_t e[4] = {as_u32(fp4_pair<0>(sm)), as_u32(fp4_pair<1>(sm)), as_u32(fp4_pair<2>(sm)),
                             as_u32(fp4_pair<3>(sm))};
#pragma unroll
      for (int j = 0; j < 4; ++j) d[j] = as_u32(as_h2(e[j]) * m.s1 + as_h2(d[j]));  // exact
    }
    if constexpr (FMT == Q_FP4_AFPQ) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // per half: negative values take s-, others s+
        const uint32_t neg = (d[j] & 0x80008000u) >> 15;       // 1 in the low bit of each negative half
        const uint32_t mask = neg * 0xFFFFu;                      // 0xFFFF per negative half
        const uint32_t sc = (as_u32(m.s1) & mask) | (as_u32(m.s0) & ~mask);
        d[j] = pk_mul(d[j], as_h2(sc));
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) d[j] = pk_mul(d[j], m.s0);
    }
    return make_h8(d[0], d[1], d[2], d[3]);
  } else if constexpr (FMT == Q_INT4_ASYM || FMT == Q_BFP4 || FMT == Q_BFP6) {
    uint32_t t[4];
    if constexpr (FMT == Q_BFP6) {
      hi ^= 0xAAAAAAAAu;  // offset binary: flip the top bit of every 6-bit field
      t[0] = six_bit_magic<0>(w, hi, hsh);
      t[1] = six_bit_magic<1>(w, hi, hsh);
      t[2] = six_bit_magic<2>(w, hi, hsh);
      t[3] = six_bit_magic<3>(w, hi, hsh);
    } else {
      const uint32_t c = FMT == Q_BFP4 ? w ^ 0x88888888u : w;
      t[0] = nibble_magic<0>(c);
      t[1] = nibble_magic<1>(c);
      t[2] = nibble_magic<2>(c);
      t[3] = nibble_magic<3>(c);
    }
    h2 bias, scale;
    if constexpr (FMT == Q_INT4_ASYM) {
      bias = m.s1;
      scale = m.s0;
    } else {
      constexpr float kb = FMT == Q_BFP4 ? 1032.0f : 1056.0f;
      bias = h2{(_Float16)kb, (_Float16)kb};
      scale = block ? m.s1 : m.s0;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) t[j] = as_u32((as_h2(t[j]) - bias) * scale);
    return make_h8(t[0], t[1], t[2], t[3]);
  } else {  // int8: exact integers, row scale applied to the result
    const h2 bias = h2{(_Float16)1152.0f, (_Float16)1152.0f};
    const uint32_t u0 = w ^ 0x80808080u, u1 = w2 ^ 0x80808080u;
    return make_h8(as_u32(as_h2(byte_magic_lo(u0)) - bias), as_u32(as_h2(byte_magic_hi(u0)) - bias),
                   as_u32(as_h2(byte_magic_lo(u1)) - bias), as_u32(as_h2(byte_magic_hi(u1)) - bias));
  }
}

// KS: k elements per LDS slice; NB: 16-row activation blocks.
template <int FMT, int NB, int KS>
__global__ void __launch_bounds__(64 * kWaves)
gemm_mfma_kernel(WeightView W, const _Float16* __restrict__ x, _Float16* __restrict__ y, int batch) {
  constexpr int ORDER = FmtTraits<FMT>::order;
  constexpr bool kInt8 = FMT == Q_INT8;
  constexpr int KT = kInt8 ? 64 : 128;       // k per 16-byte load of every lane (one K-tile)
  constexpr int STEPS = KT / 32;             // MFMA steps per K-tile
  constexpr int TILES = KS / KT;
  constexpr int LSTRIDE = KS + 8;            // halves per LDS activation row (+16 B pad)
  __shared__ __attribute__((aligned(16))) _Float16 xl[NB * 16 * LSTRIDE];

  const int K = W.k, N = W.n;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, q = lane >> 4;
  const int row = blockIdx.x * kRowsPerWg + wave * 16 + r16;
  const bool row_ok = row < N;
  const int piece = KT / 4;  // k per lane per K-tile (32, or 16 for int8)

  f4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int ks = 0; ks < K; ks += KS) {
    lds_barrier();
    // Stage activations x[b][ks .. ks+KS) for all 16*NB rows (zeros past
    // `batch` and past K), permuted into decoder order, 16 bytes per store.
    constexpr int GROUPS = NB * 16 * (KS / 8);
    for (int gidx = threadIdx.x; gidx < GROUPS; gidx += 64 * kWaves) {
      const int b = gidx / (KS / 8);
      const int kk = (gidx % (KS / 8)) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (b < batch && ks + kk < K) v = *reinterpret_cast<const uint4*>(x + (size_t)b * K + ks + kk);
      *reinterpret_cast<uint4*>(&xl[b * LSTRIDE + kk]) = permute8<ORDER>(v);
    }
    lds_barrier();
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      const int kt = ks + t * KT;
      if (kt >= K) break;
      const int kk = kt + q * piece;  // this lane's first k
      uint4 cv = make_uint4(0, 0, 0, 0);
      uint2 hv = make_uint2(0, 0);
      AMeta m;
      m.s0 = h2{(_Float16)0.0f, (_Float16)0.0f};
      m.s1 = m.s0;
      if (row_ok && kk < K) {  // k % 32 == 0: a piece is wholly inside or outside the row
        if constexpr (kInt8) {
          cv = *reinterpret_cast<const uint4*>(reinterpret_cast<const int8_t*>(W.codes) + (size_t)row * K + kk);
        } else {
          cv = *reinterpret_cast<const uint4*>(W.codes + (size_t)row * (K / 8) + kk / 8);
          if constexpr (FMT == Q_BFP6) hv = *reinterpret_cast<const uint2*>(W.codes_hi + (size_t)row * (K / 16) + kk / 16);
        }
        m = load_ameta<FMT>(W, row, kk);
      }
      const uint32_t cw[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
      for (int i = 0; i < STEPS; ++i) {
        h8 a;
        if constexpr (kInt8) a = decode_fragment<FMT>(cw[2 * i], cw[2 * i + 1], 0, 0, m, 0);
        else a = decode_fragment<FMT>(cw[i], 0, i < 2 ? hv.x : hv.y, 8 * (i & 1), m, i >> 1);
        // B fragment: activations of batch row (nb*16 + r16), the same 8 k
        // (in decoder order) that lane group q holds in A.
        const int koff = t * KT + q * piece + 8 * i;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const h8 bx = *reinterpret_cast<const h8*>(&xl[(nb * 16 + r16) * LSTRIDE + koff]);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bx, acc[nb], 0, 0, 0);
        }
      }
    }
  }
  // D fragment: lane holds rows 4q..4q+3 of the wave's 16, batch column r16.
  const int orow0 = blockIdx.x * kRowsPerWg + wave * 16 + 4 * q;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int b = nb * 16 + r16;
    if (b >= batch) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int orow = orow0 + i;
      if (orow < N) {
        float v = acc[nb][i];
        if constexpr (kInt8) v *= h2f(reinterpret_cast<const uint16_t*>(W.scales)[orow]);
        y[(size_t)b * N + orow] = (_Float16)v;
      }
    }
  }
}

// ---- group formats: exact per-group scaling ---------------------------------
//
// For int4_asym, fp4_e2m1, fp4_razer and fp4_afpq every MFMA step covers 32
// consecutive k, i.e. one group piece per row, so A holds exact unscaled
// values (q - z; E2M1 magnitudes with sign; RaZeR's special) and the group
// scale multiplies the fp32 partial product of its steps.  Lane l still loads
// 16 contiguous bytes (words 4q..4q+3 of its row's 128-element tile, q = l/16);
// a 4x4 transpose across the four 16-lane rows (two permlane32 and two
// permlane16 swaps) gives lane group q the words 4i+q that step i needs.

// Transpose words across lane groups: after it, register i of lane group q
// holds what register q of lane group i held.
__device__ __forceinline__ void transpose_lane_groups(uint32_t* r) {
  // swap the high bit of the lane group with the high bit of the register index
  for (int d = 0; d < 2; ++d) {
    const auto t = __builtin_amdgcn_permlane32_swap(r[d], r[2 + d], false, false);
    r[d] = t[0];
    r[2 + d] = t[1];
  }
  // then the low bits
  for (int c = 0; c < 2; ++c) {
    const auto t = __builtin_amdgcn_permlane16_swap(r[2 * c], r[2 * c + 1], false, false);
    r[2 * c] = t[0];
    r[2 * c + 1] = t[1];
  }
}

// Exact A fragment (no scale) of one code word.  int4: q - z; e2m1: M;
// razer: M, or the special v for code 8; afpq: signed M in a, |M| in mag.
template <int FMT>
__device__ __forceinline__ h8 exact_fragment(uint32_t w, h2 a_meta, h8* mag) {
  if constexpr (FMT == Q_INT4_ASYM) {
    const uint32_t t0 = nibble_magic<0>(w), t1 = nibble_magic<1>(w), t2 = nibble_magic<2>(w), t3 = nibble_magic<3>(w);
    // (1024 + q) - (1024 + z): exact integers
    return make_h8(as_u32(as_h2(t0) - a_meta), as_u32(as_h2(t1) - a_meta), as_u32(as_h2(t2) - a_meta),
                   as_u32(as_h2(t3) - a_meta));
  } else {
    uint32_t d[4] = {as_u32(fp4_pair<0>(w)), as_u32(fp4_pair<1>(w)), as_u32(fp4_pair<2>(w)), as_u32(fp4_pair<3>(w))};
    if constexpr (FMT == Q_FP4_RAZER) {
      const uint32_t sm = special_mask(w, 0x88888888u);
      const uint32_t e[4] = {as_u32(fp4_pair<0>(sm)), as_u32(fp4_pair<1>(sm)), as_u32(fp4_pair<2>(sm)),
                             as_u32(fp4_pair<3>(sm))};
#pragma unroll
      for (int j = 0; j < 4; ++j) d[j] = as_u32(as_h2(e[j]) * a_meta + as_h2(d[j]));  // -0 + v, or M + 0
    }
    if constexpr (FMT == Q_FP4_AFPQ) {
      *mag = make_h8(d[0] & 0x7FFF7FFFu, d[1] & 0x7FFF7FFFu, d[2] & 0x7FFF7FFFu, d[3] & 0x7FFF7FFFu);
    }
    return make_h8(d[0], d[1], d[2], d[3]);
  }
}

// A-layout metadata (row of this lane, group gi): int4 (1024 + z); razer v.
template <int FMT>
__device__ __forceinline__ h2 load_a_meta(const WeightView& W, int row, int gi, int groups) {
  if constexpr (FMT == Q_INT4_ASYM) {
    const int zw = (groups + 7) / 8;
    const uint32_t z = reinterpret_cast<const uint32_t*>(W.aux)[(size_t)row * zw + gi / 8];
    const _Float16 zb = (_Float16)(1024.0f + (float)((z >> (4 * (gi & 7))) & 0xFu));
    return h2{zb, zb};
  } else if constexpr (FMT == Q_FP4_RAZER) {
    const int sw = (groups + 15) / 16;
    const uint32_t sl = reinterpret_cast<const uint32_t*>(W.aux)[(size_t)row * sw + gi / 16];
    const _Float16 v = (_Float16)razer_special((int)((sl >> (2 * (gi & 15))) & 3u));
    return h2{v, v};
  } else {
    (void)W; (void)row; (void)gi; (void)groups;
    return h2{(_Float16)0.0f, (_Float16)0.0f};
  }
}

// SPG: MFMA steps per group within a 128-element tile (1, 2 or 4).
template <int FMT, int NB, int KS, int SPG>
__global__ void __launch_bounds__(64 * kWaves)
gemm_mfma_group_kernel(WeightView W, const _Float16* __restrict__ x, _Float16* __restrict__ y, int batch,
                       int gshift) {
  constexpr int ORDER = FmtTraits<FMT>::order;
  constexpr int KT = 128;
  constexpr int TILES = KS / KT;
  constexpr int LSTRIDE = KS + 8;
  constexpr bool kAfpq = FMT == Q_FP4_AFPQ;
  __shared__ __attribute__((aligned(16))) _Float16 xl[NB * 16 * LSTRIDE];

  const int K = W.k, N = W.n;
  const int groups = K >> gshift;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, q = lane >> 4;
  const int row0 = blockIdx.x * kRowsPerWg + wave * 16;
  const int row = row0 + r16;                   // A-layout row of this lane
  const int arow = min(row, N - 1);             // clamped for metadata loads
  int crow[4];                                  // C-layout rows of this lane
#pragma unroll
  for (int j = 0; j < 4; ++j) crow[j] = min(row0 + 4 * q + j, N - 1);

  f4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  const f4 zero4 = f4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int ks = 0; ks < K; ks += KS) {
    lds_barrier();
    constexpr int GROUPS8 = NB * 16 * (KS / 8);
    for (int gidx = threadIdx.x; gidx < GROUPS8; gidx += 64 * kWaves) {
      const int b = gidx / (KS / 8);
      const int kk = (gidx % (KS / 8)) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (b < batch && ks + kk < K) v = *reinterpret_cast<const uint4*>(x + (size_t)b * K + ks + kk);
      *reinterpret_cast<uint4*>(&xl[b * LSTRIDE + kk]) = permute8<ORDER>(v);
    }
    lds_barrier();
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      const int kt = ks + t * KT;
      if (kt >= K) break;
      uint4 cv = make_uint4(0, 0, 0, 0);
      if (row < N && kt + 32 * q < K)
        cv = *reinterpret_cast<const uint4*>(W.codes + (size_t)row * (K / 8) + (kt + 32 * q) / 8);
      uint32_t wd[4] = {cv.x, cv.y, cv.z, cv.w};
      transpose_lane_groups(wd);  // wd[i] = word 4i + q of the tile
#pragma unroll
      for (int gg = 0; gg < 4 / SPG; ++gg) {
        const int gi = min((kt + 32 * gg * SPG) >> gshift, groups - 1);
        const h2 am = load_a_meta<FMT>(W, arow, gi, groups);
        f4 part[NB], partm[NB];
#pragma unroll
        for (int s = 0; s < SPG; ++s) {
          const int i = gg * SPG + s;
          h8 mag;
          const h8 a = exact_fragment<FMT>(wd[i], am, &mag);
          const int koff = t * KT + 32 * i + 8 * q;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const h8 bx = *reinterpret_cast<const h8*>(&xl[(nb * 16 + r16) * LSTRIDE + koff]);
            part[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bx, s == 0 ? zero4 : part[nb], 0, 0, 0);
            if constexpr (kAfpq)
              partm[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(mag, bx, s == 0 ? zero4 : partm[nb], 0, 0, 0);
          }
        }
        // group scales of this lane's C rows
        float sc[4], sc2[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const size_t gidx = (size_t)crow[j] * groups + gi;
          if constexpr (kAfpq) {
            const uint32_t pr = reinterpret_cast<const uint32_t*>(W.scales)[gidx];
            const float sp = h2f((uint16_t)(pr & 0xFFFFu)), sn = h2f((uint16_t)(pr >> 16));
            sc[j] = 0.5f * (sp + sn);   // weight of the signed sum
            sc2[j] = 0.5f * (sp - sn);  // weight of the magnitude sum
          } else {
            sc[j] = h2f(reinterpret_cast<const uint16_t*>(W.scales)[gidx]);
            sc2[j] = 0.0f;
          }
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[nb][j] += sc[j] * part[nb][j];
            if constexpr (kAfpq) acc[nb][j] += sc2[j] * partm[nb][j];
          }
      }
    }
  }
  const int orow0 = row0 + 4 * q;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int b = nb * 16 + r16;
    if (b >= batch) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (orow0 + j < N) y[(size_t)b * N + orow0 + j] = (_Float16)acc[nb][j];
  }
}

typedef void (*KernelFn)(WeightView, const _Float16*, _Float16*, int);
typedef void (*GroupKernelFn)(WeightView, const _Float16*, _Float16*, int, int);

template <int FMT>
KernelFn pick(int nb) {
  switch (nb) {
    case 1: return gemm_mfma_kernel<FMT, 1, 512>;
    case 2: return gemm_mfma_kernel<FMT, 2, 512>;
    case 3: return gemm_mfma_kernel<FMT, 3, 256>;
    default: return gemm_mfma_kernel<FMT, 4, 256>;
  }
}

template <int FMT, int SPG>
GroupKernelFn pick_group_nb(int nb) {
  switch (nb) {
    case 1: return gemm_mfma_group_kernel<FMT, 1, 512, SPG>;
    case 2: return gemm_mfma_group_kernel<FMT, 2, 512, SPG>;
    case 3: return gemm_mfma_group_kernel<FMT, 3, 256, SPG>;
    default: return gemm_mfma_group_kernel<FMT, 4, 256, SPG>;
  }
}

template <int FMT>
GroupKernelFn pick_group(int nb, int group) {
  if (group == 32) return pick_group_nb<FMT, 1>(nb);
  if (group == 64) return pick_group_nb<FMT, 2>(nb);
  return pick_group_nb<FMT, 4>(nb);
}

}  // namespace

hipError_t launch_gemm_mfma(const WeightView& w, const _Float16* x, _Float16* y, int b, hipStream_t s) {
  const int nb = (b + 15) / 16;
  const int grid = (w.n + kRowsPerWg - 1) / kRowsPerWg;
  int gshift = 0;
  while ((1 << gshift) < w.group) ++gshift;
  GroupKernelFn gfn = nullptr;
  KernelFn fn = nullptr;
  switch (w.fmt) {
    case Q_INT4_ASYM: gfn = pick_group<Q_INT4_ASYM>(nb, w.group); break;
    case Q_FP4_E2M1: gfn = pick_group<Q_FP4_E2M1>(nb, w.group); break;
    case Q_FP4_RAZER: gfn = pick_group<Q_FP4_RAZER>(nb, w.group); break;
    case Q_FP4_AFPQ: gfn = pick_group<Q_FP4_AFPQ>(nb, w.group); break;
    case Q_BFP6: fn = pick<Q_BFP6>(nb); break;
    case Q_BFP4: fn = pick<Q_BFP4>(nb); break;
    case Q_INT8: fn = pick<Q_INT8>(nb); break;
    default: return hipErrorInvalidValue;
  }
  if (gfn) hipLaunchKernelGGL(gfn, dim3(grid), dim3(64 * kWaves), 0, s, w, x, y, b, gshift);
  else hipLaunchKernelGGL(fn, dim3(grid), dim3(64 * kWaves), 0, s, w, x, y, b);
  return hipGetLastError();
}

}  // namespace qg
