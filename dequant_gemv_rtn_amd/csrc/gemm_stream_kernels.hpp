// Weight-streaming MFMA kernel for 1 <= b <= 64 activation rows.
//
// y[b][n] = sum_k W_deq[n][k] x[b][k] as v_mfma_f32_16x16x32_f16 with the
// activations as the A operand (16 batch rows x 32 k, rows past b are zero)
// and the decoded weights as the B operand (32 k x 16 weight rows).  Each
// workgroup serves one tile of 16 activation rows; with b > 16 the tiles'
// workgroups share the weight stream through the last-level cache.  With the
// weights on the B side, lane l of the 16x16 result holds four batch values
// of ONE weight row (l mod 16), so a group scale is one scalar per lane and
// multiplies the fp32 partial of its group exactly once: B holds exact
// unscaled values (INT4 q - z, E2M1 magnitudes with sign, INT8 integers).
//
// Work split.  K is cut into 128-element chunks; a workgroup of KS waves owns
// a 16-row tile at a time and wave w handles chunks [w*KC, (w+1)*KC) of every
// tile it visits.  The wave's activation slice (KC chunks x 4 MFMA steps)
// is loaded once, permuted into the decoder's element order, and stays in
// registers for the whole launch.  Workgroups are persistent and stride over
// the tiles; each wave keeps the next tile's chunks in flight (one 16-byte
// code load per lane per chunk, plus metadata) while it decodes the current
// one.  The KS partial tiles are summed through LDS and stored as fp16.
//
// Metadata (group scales, INT4 zero-points, RaZeR selectors, block
// exponents, the INT8 row scale) is loaded once per tile: each lane reads its
// row's run for the wave's whole K-slice in a few wide loads.  Loading it per
// chunk instead takes many tiny loads that each touch 16 rows, and those, not
// the arithmetic, bound the kernel.
//
// Element order inside an MFMA step.  Lane (r, q) = (l mod 16, l / 16) loads
// 16 contiguous bytes of row r: k = 32q .. 32q+31 of the chunk.  MFMA step s
// then pairs word s of every lane (k = 32q + 8s + e), which is consistent on
// both operands.  When a group is shorter than the chunk (g = 32, 64) a 4x4
// transpose across the four lane groups makes step s cover the 32
// consecutive k 32s .. 32s+31 instead, so every step stays inside one group.
#include <hip/hip_runtime.h>
#include <stdint.h>
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "gemm_stream_geom.hpp"
#include "internal.hpp"

namespace qg {
namespace {


template <int FMT>
struct StreamFmt {
  static constexpr int words = FMT == Q_INT8 ? 8 : 4;  // code words per lane per chunk
  static constexpr bool two = is_afpq(FMT);             // a second MFMA chain per step
  // bytes of one lane's 32-element piece: 16 (4-bit), 12 (3-bit), 32 (int8)
  static constexpr uint32_t piece_bytes = FMT == Q_INT8 ? 32u : is_fp3(FMT) ? 12u : 16u;
  static constexpr bool grouped =
      FMT == Q_INT4_ASYM || FMT == Q_FP4_E2M1 || is_razer(FMT) || is_afpq(FMT);
  static constexpr bool block = FMT == Q_BFP6 || FMT == Q_BFP4;
  static constexpr int order = FmtTraits<FMT>::order;
};

// Shape of one wave's K-slice: KC chunks; GS = MFMA steps per group
// (group / 32) for the group formats.
template <int FMT, int KC, int GS>
struct Slice {
  static constexpr bool grouped = StreamFmt<FMT>::grouped;
  static constexpr int seg = grouped ? (GS < 4 ? GS : 4) : 4;          // steps per scale segment
  static constexpr int groups = grouped ? (GS <= 4 ? KC * 4 / GS : KC / 2) : 0;
  static constexpr int sb = is_afpq(FMT) ? 4 : 2;                       // bytes per group scale
  static constexpr int meta_bytes = grouped ? groups * sb : FMT == Q_INT8 ? 2 : StreamFmt<FMT>::block ? KC * 8 : 0;
  static constexpr int meta_words = (meta_bytes + 3) / 4;
  static constexpr bool aligned = is_afpq(FMT);                         // rows and slices start on 4 bytes
  static constexpr int raw_words = meta_words + (aligned ? 0 : 1);
  static constexpr int aux_words = FMT == Q_INT4_ASYM ? (groups >= 8 ? groups / 8 : 1)
                                 : is_razer(FMT) ? (groups >= 16 ? groups / 16 : 1) : 1;
};


struct StreamRes {
  __amdgpu_buffer_rsrc_t codes, hi, scales, aux;
};

// One lane's code words for one chunk of one weight row.
template <int FMT>
struct ChunkRegs {
  uint32_t cw[StreamFmt<FMT>::words];
  uint32_t hw[2];  // bfp6 high plane (32 elements)
};

// One lane's metadata for its row over the wave's K-slice.
template <int FMT, int KC, int GS>
struct TileMeta {
  using S = Slice<FMT, KC, GS>;
  uint32_t raw[S::raw_words > 0 ? S::raw_words : 1];  // scales / int8 row scale / block exponents
  uint32_t aux[S::aux_words];                         // int4 zero-points, razer selectors
  uint32_t shift;                                     // byte misalignment of raw, in bits
};

// Per-lane parts of the byte offsets (the wave-uniform parts go in soffset).
struct LaneOff {
  uint32_t code, hi;
};

template <int N>
__device__ __forceinline__ void load_words(uint32_t* dst, __amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff) {
  int i = 0;
#pragma unroll
  for (; i + 4 <= N; i += 4) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 4u * i, soff, 0);
    dst[i] = v.x; dst[i + 1] = v.y; dst[i + 2] = v.z; dst[i + 3] = v.w;
  }
  if constexpr (N % 4 >= 2) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, voff + 4u * i, soff, 0);
    dst[i] = v.x; dst[i + 1] = v.y;
    i += 2;
  }
  if constexpr (N % 2 == 1) dst[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff + 4u * i, soff, 0);
}

template <int FMT>
__device__ __forceinline__ void load_chunk(ChunkRegs<FMT>& r, const StreamRes& rs, const StreamGeom& g,
                                           const LaneOff& lo, uint32_t row0, uint32_t cc) {
  if constexpr (FMT == Q_INT8) {
    load_words<8>(r.cw, rs.codes, lo.code, row0 * g.codes_row + cc * 128u);
  } else {
    if constexpr (is_fp3(FMT)) {  // three dwords per lane, expanded when consumed
      const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(rs.codes, lo.code, row0 * g.codes_row + cc * 48u, 0);
      r.cw[0] = v.x; r.cw[1] = v.y; r.cw[2] = v.z; r.cw[3] = 0u;
    } else {
      load_words<4>(r.cw, rs.codes, lo.code, row0 * g.codes_row + cc * 64u);
    }
  }
  if constexpr (FMT == Q_BFP6) load_words<2>(r.hw, rs.hi, lo.hi, row0 * g.hi_row + cc * 32u);
}

// Metadata of row r16 of the tile at row0 for the slice starting at chunk
// c_begin.  Runs that may start off a 4-byte boundary are read from the
// boundary below with one extra word and realigned at use.
template <int FMT, int KC, int GS>
__device__ __forceinline__ void load_meta(TileMeta<FMT, KC, GS>& m, const StreamRes& rs, const StreamGeom& g,
                                          uint32_t r16, uint32_t row0, uint32_t c_begin) {
  using S = Slice<FMT, KC, GS>;
  if constexpr (S::meta_bytes > 0) {
    __amdgpu_buffer_rsrc_t src;
    uint32_t row_bytes, start;
    if constexpr (S::grouped) {
      src = rs.scales; row_bytes = g.scales_row; start = ((c_begin * 128u) >> g.gshift) * (uint32_t)S::sb;
    } else if constexpr (FMT == Q_INT8) {
      src = rs.scales; row_bytes = 2u; start = 0u;
    } else {
      src = rs.aux; row_bytes = g.aux_row; start = c_begin * 8u;
    }
    const uint32_t off = (r16 + row0) * row_bytes + start;
    load_words<S::raw_words>(m.raw, src, off & ~3u, 0u);
    m.shift = (off & 3u) * 8u;
  }
  if constexpr (FMT == Q_INT4_ASYM || is_razer(FMT)) {
    const uint32_t gfirst = (c_begin * 128u) >> g.gshift;
    const uint32_t word = FMT == Q_INT4_ASYM ? gfirst >> 3 : gfirst >> 4;
    load_words<S::aux_words>(m.aux, rs.aux, (r16 + row0) * g.aux_row + word * 4u, 0u);
  }
}

// Meta word i, realigned.
template <int FMT, int KC, int GS>
__device__ __forceinline__ uint32_t meta_word(const TileMeta<FMT, KC, GS>& m, int i) {
  if constexpr (Slice<FMT, KC, GS>::aligned) return m.raw[i];
  else return __builtin_amdgcn_alignbit(m.raw[i + 1], m.raw[i], m.shift);
}

// Transpose words across lane groups: afterwards register i of lane group q
// holds what register q of lane group i held.
__device__ __forceinline__ void transpose4(uint32_t* r) {
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const auto t = __builtin_amdgcn_permlane32_swap(r[d], r[2 + d], false, false);
    r[d] = t[0];
    r[2 + d] = t[1];
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const auto t = __builtin_amdgcn_permlane16_swap(r[2 * c], r[2 * c + 1], false, false);
    r[2 * c] = t[0];
    r[2 * c + 1] = t[1];
  }
}

__device__ __forceinline__ uint32_t h2bits(uint32_t half_bits) { return half_bits | (half_bits << 16); }

// Nibble fields of u in stride-4 pair order, exact: fields 0, 2 (and 4, 6) as
// 1024 + n, fields 1, 3 (and 5, 7) as 64 + n -- the field sits in the low
// mantissa bits of an fp16 whose exponent gives it unit weight.
__device__ __forceinline__ void nibble_fields(uint32_t u, uint32_t* t) {
  uint32_t lo = 0x000F000Fu, hi = 0x00F000F0u, k1024 = 0x64006400u, k64 = 0x54005400u;
  asm("" : "+v"(lo), "+v"(hi), "+v"(k1024), "+v"(k64));
  const uint32_t u8 = u >> 8;
  t[0] = and_or(u, lo, k1024);   // (e0, e4)
  t[1] = and_or(u, hi, k64);     // (e1, e5)
  t[2] = and_or(u8, lo, k1024);  // (e2, e6)
  t[3] = and_or(u8, hi, k64);    // (e3, e7)
}

// Consume chunk C of the slice: decode the B operand of its four MFMA steps
// once and accumulate its product with each of the BT batch tiles xa[t]
// into acc[t] (group formats: per-group partials scaled once).
template <int FMT, int KC, int GS, int C, int BT>
__device__ __forceinline__ void consume_chunk(ChunkRegs<FMT> r, const TileMeta<FMT, KC, GS>& m,
                                              const h8 (*xa)[4], f4* acc, uint32_t gfirst, int q, int eref) {
  using S = Slice<FMT, KC, GS>;
  constexpr int SEG = S::seg;
  const f4 zero4 = f4{0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (is_fp3(FMT)) {  // 3-bit piece -> the four E2M1 code words of the same values
    uint32_t e[4];
    expand_fp3(r.cw[0], r.cw[1], r.cw[2], e);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.cw[i] = e[i];
  }
  if constexpr (S::grouped && GS < 4) transpose4(r.cw);
  if constexpr (S::grouped) {
#pragma unroll
    for (int seg = 0; seg < 4 / SEG; ++seg) {
      const int gs = (C * 4 + seg * SEG) / GS;  // group within the slice (compile-time)
      const uint32_t gi = gfirst + (uint32_t)gs;
      float sa, sb = 0.0f;
      uint32_t z1024 = 0, z64 = 0;
      h2 special = h2{(_Float16)0.0f, (_Float16)0.0f};
      if constexpr (is_afpq(FMT)) {
        const uint32_t pr = meta_word(m, gs);
        const float sp = h2f((uint16_t)(pr & 0xFFFFu)), sn = h2f((uint16_t)(pr >> 16));
        sa = 0.5f * (sp + sn);  // weight of the signed partial
        sb = 0.5f * (sp - sn);  // weight of the magnitude partial
      } else {
        sa = h2f((uint16_t)((meta_word(m, gs >> 1) >> (16 * (gs & 1))) & 0xFFFFu));
      }
      if constexpr (FMT == Q_INT4_ASYM) {
        const uint32_t z = (m.aux[S::groups >= 8 ? gs / 8 : 0] >> (4u * (gi & 7u))) & 0xFu;
        z1024 = h2bits(0x6400u | z);       // 1024 + z
        z64 = h2bits(0x5400u | (z << 4));  // 64 + z
      }
      if constexpr (is_razer(FMT)) {
        const _Float16 v = (_Float16)razer_special_of<FMT>((int)((m.aux[S::groups >= 16 ? gs / 16 : 0] >> (2u * (gi & 15u))) & 3u));
        special = h2{v, v};
      }
      f4 p[BT], p2[BT];
#pragma unroll
      for (int t = 0; t < BT; ++t) { p[t] = zero4; p2[t] = zero4; }
#pragma unroll
      for (int ss = 0; ss < SEG; ++ss) {
        const int s = seg * SEG + ss;
        const uint32_t w = r.cw[s];
        h8 b1, b2;
        if constexpr (FMT == Q_INT4_ASYM) {
          uint32_t t[4];
          nibble_fields(w, t);
          b1 = make_h8(as_u32(as_h2(t[0]) - as_h2(z1024)), as_u32(as_h2(t[1]) - as_h2(z64)),
                       as_u32(as_h2(t[2]) - as_h2(z1024)), as_u32(as_h2(t[3]) - as_h2(z64)));
        } else {
          const uint32_t d0 = as_u32(fp4_pair<0>(w)), d1 = as_u32(fp4_pair<1>(w));
          const uint32_t d2 = as_u32(fp4_pair<2>(w)), d3 = as_u32(fp4_pair<3>(w));
          b1 = make_h8(d0, d1, d2, d3);
          if constexpr (is_razer(FMT)) {
            // code 8 decodes to -0 and its mask element to 1: -0 + v * 1 = v,
            // and every other element keeps its value (x + v * 0), exactly
            uint32_t m8 = 0x88888888u;
            asm("" : "+v"(m8));
            const uint32_t sm = special_mask(w, m8);
            b1 = make_h8(as_u32(fp4_pair<0>(sm) * special + as_h2(d0)), as_u32(fp4_pair<1>(sm) * special + as_h2(d1)),
                         as_u32(fp4_pair<2>(sm) * special + as_h2(d2)), as_u32(fp4_pair<3>(sm) * special + as_h2(d3)));
          }
          if constexpr (is_afpq(FMT)) {
            uint32_t mm = 0x7FFF7FFFu;
            asm("" : "+v"(mm));
            b2 = make_h8(d0 & mm, d1 & mm, d2 & mm, d3 & mm);
          }
        }
#pragma unroll
        for (int t = 0; t < BT; ++t) {
          p[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[t][s], b1, p[t], 0, 0, 0);
          if constexpr (StreamFmt<FMT>::two)
            p2[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[t][s], b2, p2[t], 0, 0, 0);
        }
      }
#pragma unroll
      for (int t = 0; t < BT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[t][i] += sa * p[t][i];
          if constexpr (StreamFmt<FMT>::two) acc[t][i] += sb * p2[t][i];
        }
    }
  } else if constexpr (FMT == Q_INT8) {
    const h2 bias = h2{(_Float16)1152.0f, (_Float16)1152.0f};  // 1024 + offset-binary 128
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t u0 = r.cw[2 * s] ^ 0x80808080u, u1 = r.cw[2 * s + 1] ^ 0x80808080u;
      const h8 b1 = make_h8(as_u32(as_h2(byte_magic_lo(u0)) - bias), as_u32(as_h2(byte_magic_hi(u0)) - bias),
                            as_u32(as_h2(byte_magic_lo(u1)) - bias), as_u32(as_h2(byte_magic_hi(u1)) - bias));
#pragma unroll
      for (int t = 0; t < BT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[t][s], b1, acc[t], 0, 0, 0);
    }
  } else {
    // block formats: the block step relative to the row slice's largest,
    // 2^(E - eref) <= 1, is folded into the fp16 operand (the tile applies
    // 2^(eref - 127 - mb + 1) in fp32).  Exact for blocks down to 2^-24 of
    // the slice's largest step; smaller ones are below fp32 accumulation
    // error anyway.  Step s of lane group q covers k = 32q + 8s + e, i.e.
    // block 2q + s/2 of the chunk; its two exponent bytes sit at byte
    // 8C + 2q of the slice run.
    const uint32_t pair_word = q >= 2 ? meta_word(m, 2 * C + 1) : meta_word(m, 2 * C);
    const uint32_t exps = pair_word >> (16 * (q & 1));
    h2 step[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = (int)((exps >> (8 * h)) & 0xFFu);
      const _Float16 v = (_Float16)(e ? ldexpf(1.0f, e - eref) : 0.0f);
      step[h] = h2{v, v};
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t w = r.cw[s];
      uint32_t t[4];
      h2 bias_even, bias_odd;
      if constexpr (FMT == Q_BFP4) {
        nibble_fields(w ^ 0x88888888u, t);  // offset binary m + 8
        bias_even = h2{(_Float16)1032.0f, (_Float16)1032.0f};
        bias_odd = h2{(_Float16)72.0f, (_Float16)72.0f};
      } else {
        const uint32_t hi = r.hw[s >> 1] ^ 0xAAAAAAAAu;  // offset binary m + 32
        const int hsh = 8 * (s & 1);
        t[0] = six_bit_magic<0>(w, hi, hsh);
        t[1] = six_bit_magic<1>(w, hi, hsh);
        t[2] = six_bit_magic<2>(w, hi, hsh);
        t[3] = six_bit_magic<3>(w, hi, hsh);
        bias_even = bias_odd = h2{(_Float16)1056.0f, (_Float16)1056.0f};
      }
      const h2 st = step[s >> 1];
      const h8 b1 = make_h8(as_u32((as_h2(t[0]) - bias_even) * st), as_u32((as_h2(t[1]) - bias_odd) * st),
                            as_u32((as_h2(t[2]) - bias_even) * st), as_u32((as_h2(t[3]) - bias_odd) * st));
#pragma unroll
      for (int t = 0; t < BT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[t][s], b1, acc[t], 0, 0, 0);
    }
  }
}

// Block formats: the largest block exponent of this lane's row over the
// wave's K-slice (every lane of the row holds the same run), and the fp32
// factor 2^(eref - 127 - mb + 1) that turns the rescaled partials into
// output units.  Other formats: 0 and 1.
template <int FMT, int KC, int GS>
__device__ __forceinline__ int slice_eref(const TileMeta<FMT, KC, GS>& m) {
  if constexpr (StreamFmt<FMT>::block) {
    uint32_t mx = 0;  // two 16-bit lanes of byte maxima
#pragma unroll
    for (int i = 0; i < 2 * KC; ++i) {
      const uint32_t w = meta_word(m, i);
      mx = __builtin_elementwise_max(mx, w & 0x00FF00FFu);
      mx = __builtin_elementwise_max(mx, (w >> 8) & 0x00FF00FFu);
    }
    // (per-halfword maxima: the two halves are combined below)
    const uint32_t lo = mx & 0xFFFFu, hi = mx >> 16;
    return (int)(lo > hi ? lo : hi);
  }
  return 0;
}

template <int FMT>
__device__ __forceinline__ float slice_scale(int eref) {
  if constexpr (StreamFmt<FMT>::block) {
    constexpr int mb = FMT == Q_BFP6 ? 5 : 3;
    return ldexpf(1.0f, eref - 127 - mb + 1);
  }
  return 1.0f;
}

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Sum the nw partial tiles in red and store the 16 x 16 output tile t of
// batch tile bt: output block i (64 outputs) is summed by wave i mod nw
// (SPREAD), or by wave 0 alone where registers are tight (spreading the sums
// made the streamed-activation kernel spill).  Every wave issues the same
// four stores -- outputs that are not its own, past b or past n go to an
// offset the range check drops -- so the count of memory operations in
// flight is the same in every wave and on every path.
template <bool SPREAD>
__device__ __forceinline__ void store_tile(const float (*red)[256], int nw, int wave, int lane, int t, int bt,
                                           int bt_rows, const StreamGeom& g, __amdgpu_buffer_rsrc_t yrs) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int o = 64 * i + lane, bi = o >> 4, row = t * 16 + (o & 15);
    const bool mine = SPREAD ? i % nw == wave : wave == 0;
    float sum = 0.0f;
    if (mine)
      for (int w = 0; w < nw; ++w) sum += red[w][o];
    const uint32_t off = (mine && bi < bt_rows && row < g.n)
                             ? ((uint32_t)(16 * bt + bi) * (uint32_t)g.n + (uint32_t)row) * 2u : 0xFFFFFF00u;
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)sum), yrs, off, 0, 0);
  }
}


template <int FMT, int KC, int GS, int D>
__global__ void __launch_bounds__(64 * stream_max_waves(KC, GS, D))
gemm_stream_kernel(WeightView W, const _Float16* __restrict__ x, _Float16* __restrict__ y, StreamGeom g) {
  using S = Slice<FMT, KC, GS>;
  constexpr int ORDER = StreamFmt<FMT>::order;
  constexpr bool kTranspose = S::grouped && GS < 4;
  __shared__ float red[2][kStreamMaxWaves][256];

  const int nw = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, q = lane >> 4;

  StreamRes rs;
  rs.codes = make_rsrc(W.codes, g.codes_bytes);
  rs.hi = make_rsrc(W.codes_hi, g.hi_bytes);
  rs.scales = make_rsrc(W.scales, g.scales_bytes);
  rs.aux = make_rsrc(W.aux, g.aux_bytes);
  const __amdgpu_buffer_rsrc_t yrs = make_rsrc(y, g.y_bytes);

  LaneOff lo;
  lo.code = (uint32_t)r16 * g.codes_row + StreamFmt<FMT>::piece_bytes * q;
  lo.hi = (uint32_t)r16 * g.hi_row + 8u * q;

  // this wave's chunks, clamped to the last real chunk for loads (the
  // activations of chunks past k are zero, so they add nothing)
  const int c_begin = __builtin_amdgcn_readfirstlane(wave * KC);
  const uint32_t c_meta = (uint32_t)min(c_begin, g.chunks - 1);
  uint32_t ccl[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) ccl[c] = (uint32_t)min(c_begin + c, g.chunks - 1);
  const uint32_t gfirst = S::grouped ? (c_meta * 128u) >> g.gshift : 0u;

  // batch tile of this workgroup (16 activation rows) and its row group
  int bt, t_first;
  const int nbt = g.batch_tiles;
  const int grid_rows = (int)gridDim.x / nbt;
  batch_tile_of(nbt, grid_rows, bt, t_first);
  const int count = t_first < g.tiles ? (g.tiles - 1 - t_first) / grid_rows + 1 : 0;
  const int bt_rows = min(16, g.b - 16 * bt);  // activation rows of this batch tile

  // activation fragments of this wave's K-slice, in decoder order
  h8 xa[KC][1][4];
  {
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, g.x_bytes);
    const uint32_t xrow = (uint32_t)(16 * bt + r16) * (uint32_t)g.k * 2u;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int k = (c_begin + c) * 128 + (kTranspose ? 32 * s + 8 * q : 32 * q + 8 * s);
        // rows past b fall outside the buffer and read as zero; so do k past the end
        const uint32_t off = (k < g.k && r16 < bt_rows) ? xrow + (uint32_t)k * 2u : 0xFFFFFF00u;
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0);
        const uint4 p = permute8<ORDER>(make_uint4(v.x, v.y, v.z, v.w));
        xa[c][0][s] = make_h8(p.x, p.y, p.z, p.w);
      }
    }
  }

  // ring of D tiles: slot d holds tile it + d.  A consumed chunk is reloaded
  // with the same chunk of tile it + d + D, and the metadata after the last
  // chunk, so every load has D - 1 whole tile times (plus the rest of the
  // current one) to arrive.
  ChunkRegs<FMT> ring[D][KC];
  TileMeta<FMT, KC, GS> meta[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const uint32_t row0 = (uint32_t)(d < count ? t_first + d * grid_rows : t_first) * 16u;
    // the same memory operations, in the same order, as a tile issues: the
    // code loads, the metadata, then four output stores (dropped here).  The
    // compiler's wait at the loop head serves both the first tile and every
    // later one; a different prologue sequence makes it wait for far more
    // than the tile's own loads.
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      load_chunk<FMT>(ring[d][c], rs, g, lo, row0, ccl[c]);
      __builtin_amdgcn_sched_barrier(0);
    }
    load_meta<FMT, KC, GS>(meta[d], rs, g, (uint32_t)r16, row0, c_meta);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)0, yrs, 0xFFFFFF00u, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }

  // resolve the activation loads here (the first tiles' weight loads are
  // already in flight behind them): left to their first use inside the
  // tile loop, the wait for them would be merged into the loop head and
  // drain the weight prefetch on every tile
#pragma unroll
  for (int c = 0; c < KC; ++c)
#pragma unroll
    for (int s = 0; s < 4; ++s) asm volatile("" : "+v"(xa[c][0][s]));

  // One tile: decode + MFMA every chunk of slot d (reloading when `reload`),
  // then sum the waves' partial tiles through LDS and store.
  auto tile = [&](auto dc, int it, bool reload) {
    constexpr int d = decltype(dc)::value;
    const int t = t_first + it * grid_rows;
    const uint32_t row_load = (uint32_t)(it + D < count ? t + D * grid_rows : t_first) * 16u;
    f4 acc = f4{0.0f, 0.0f, 0.0f, 0.0f};
    const int eref = slice_eref<FMT, KC, GS>(meta[d]);
    float rowscale = slice_scale<FMT>(eref);
    if constexpr (FMT == Q_INT8) rowscale = h2f((uint16_t)(meta_word(meta[d], 0) & 0xFFFFu));
    static_for<0, KC>([&](auto cc) {
      constexpr int C = decltype(cc)::value;
      consume_chunk<FMT, KC, GS, C, 1>(ring[d][C], meta[d], xa[C], &acc, gfirst, q, eref);
      if (reload) load_chunk<FMT>(ring[d][C], rs, g, lo, row_load, ccl[C]);
      // keep the prefetch where it is: left alone, the scheduler sinks the
      // next tile's loads below the last chunk's MFMAs, and the wait at the
      // top of the loop then drains them
      __builtin_amdgcn_sched_barrier(0);
    });
    if (reload) load_meta<FMT, KC, GS>(meta[d], rs, g, (uint32_t)r16, row_load, c_meta);
    __builtin_amdgcn_sched_barrier(0);
    // lane (r16, q) holds batch rows 4q..4q+3 of weight row r16
    float* red_w = red[it & 1][wave];
#pragma unroll
    for (int i = 0; i < 4; ++i) red_w[(4 * q + i) * 16 + r16] = rowscale * acc[i];
    lds_barrier();
    store_tile<true>(red[it & 1], nw, wave, lane, t, bt, bt_rows, g, yrs);
  };

  // main loop: D tiles per iteration, every load unconditional (past the
  // end they re-read this workgroup's first tile); the last count % D tiles
  // run after it without reloading
  int it = 0;
  for (; it + D <= count; it += D) {
    tile(std::integral_constant<int, 0>{}, it, true);
    if constexpr (D > 1) tile(std::integral_constant<int, 1>{}, it + 1, true);
  }
  if constexpr (D > 1)
    if (it < count) tile(std::integral_constant<int, 0>{}, it, false);
}

// Activation fragments of chunk cc for lane (r16, q) of batch tile bt, in
// decoder order (zeros past b and past k).
template <int ORDER, bool TRANSPOSE>
__device__ __forceinline__ void load_x_chunk(u32x4* raw, __amdgpu_buffer_rsrc_t xrs, const StreamGeom& g, uint32_t xrow,
                                             bool row_ok, int cc, int q) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int k = cc * 128 + (TRANSPOSE ? 32 * s + 8 * q : 32 * q + 8 * s);
    const uint32_t off = (k < g.k && row_ok) ? xrow + (uint32_t)k * 2u : 0xFFFFFF00u;
    raw[s] = __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0);
  }
}

// The same product for k > 8192, where a wave's activation slice no longer
// fits in registers: the activation fragments of each chunk are loaded with
// its code words (from the cache: every tile re-reads the same slice), and
// the ring holds SR chunks instead of whole tiles.  Metadata alternates
// between two slots, one per tile parity, so the next tile's is loaded
// while the current one is in use.
template <int FMT, int KC, int GS, int SR>
__global__ void __launch_bounds__(64 * 8)
gemm_stream_xs_kernel(WeightView W, const _Float16* __restrict__ x, _Float16* __restrict__ y, StreamGeom g) {
  static_assert(KC % SR == 0, "ring slots must divide the slice");
  using S = Slice<FMT, KC, GS>;
  constexpr int ORDER = StreamFmt<FMT>::order;
  constexpr bool kTranspose = S::grouped && GS < 4;
  __shared__ float red[2][kStreamMaxWaves][256];

  const int nw = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, q = lane >> 4;

  StreamRes rs;
  rs.codes = make_rsrc(W.codes, g.codes_bytes);
  rs.hi = make_rsrc(W.codes_hi, g.hi_bytes);
  rs.scales = make_rsrc(W.scales, g.scales_bytes);
  rs.aux = make_rsrc(W.aux, g.aux_bytes);
  const __amdgpu_buffer_rsrc_t yrs = make_rsrc(y, g.y_bytes);
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, g.x_bytes);

  LaneOff lo;
  lo.code = (uint32_t)r16 * g.codes_row + StreamFmt<FMT>::piece_bytes * q;
  lo.hi = (uint32_t)r16 * g.hi_row + 8u * q;

  const int c_begin = __builtin_amdgcn_readfirstlane(wave * KC);
  const uint32_t c_meta = (uint32_t)min(c_begin, g.chunks - 1);
  uint32_t ccl[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) ccl[c] = (uint32_t)min(c_begin + c, g.chunks - 1);
  const uint32_t gfirst = S::grouped ? (c_meta * 128u) >> g.gshift : 0u;

  int bt, t_first;
  const int nbt = g.batch_tiles;
  const int grid_rows = (int)gridDim.x / nbt;
  batch_tile_of(nbt, grid_rows, bt, t_first);
  const int count = t_first < g.tiles ? (g.tiles - 1 - t_first) / grid_rows + 1 : 0;
  const int bt_rows = min(16, g.b - 16 * bt);
  const uint32_t xrow = (uint32_t)(16 * bt + r16) * (uint32_t)g.k * 2u;
  const bool xrow_ok = r16 < bt_rows;

  struct Slot {
    ChunkRegs<FMT> w;
    u32x4 xr[4];
  };
  Slot ring[SR];
  TileMeta<FMT, KC, GS> meta[2];
  auto tile_row = [&](int it) { return (uint32_t)(it < count ? t_first + it * grid_rows : t_first) * 16u; };

  // prologue, in the issue order of a tile's end: metadata of tile 0, the
  // first SR chunks of tile 0, metadata of tile 1, then four output stores
  // (dropped here), so that the compiler's waits in the first tile equal
  // those of every later one
  load_meta<FMT, KC, GS>(meta[0], rs, g, (uint32_t)r16, tile_row(0), c_meta);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < SR; ++c) {
    load_chunk<FMT>(ring[c].w, rs, g, lo, tile_row(0), ccl[c]);
    load_x_chunk<ORDER, kTranspose>(ring[c].xr, xrs, g, xrow, xrow_ok, c_begin + c, q);
    __builtin_amdgcn_sched_barrier(0);
  }
  load_meta<FMT, KC, GS>(meta[1], rs, g, (uint32_t)r16, tile_row(1), c_meta);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 4; ++i) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)0, yrs, 0xFFFFFF00u, 0, 0);
  __builtin_amdgcn_sched_barrier(0);

  auto tile = [&](auto mc, int it, bool reload) {
    constexpr int m = decltype(mc)::value;
    const int t = t_first + it * grid_rows;
    const uint32_t row_next = tile_row(it + 1), row_meta = tile_row(it + 2);
    f4 acc = f4{0.0f, 0.0f, 0.0f, 0.0f};
    const int eref = slice_eref<FMT, KC, GS>(meta[m]);
    float rowscale = slice_scale<FMT>(eref);
    if constexpr (FMT == Q_INT8) rowscale = h2f((uint16_t)(meta_word(meta[m], 0) & 0xFFFFu));
    static_for<0, KC>([&](auto cc) {
      constexpr int C = decltype(cc)::value;
      constexpr int slot = C % SR;
      h8 xa[1][4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 v = ring[slot].xr[s];
        const uint4 p = permute8<ORDER>(make_uint4(v.x, v.y, v.z, v.w));
        xa[0][s] = make_h8(p.x, p.y, p.z, p.w);
      }
      consume_chunk<FMT, KC, GS, C, 1>(ring[slot].w, meta[m], xa, &acc, gfirst, q, eref);
      // refill the slot with the chunk SR further on: later in this tile, or
      // at the start of the next one
      constexpr int NC = C + SR < KC ? C + SR : C + SR - KC;
      const bool same_tile = C + SR < KC;
      if (same_tile || reload) {
        load_chunk<FMT>(ring[slot].w, rs, g, lo, same_tile ? tile_row(it) : row_next, ccl[NC]);
        load_x_chunk<ORDER, kTranspose>(ring[slot].xr, xrs, g, xrow, xrow_ok, c_begin + NC, q);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    if (reload) load_meta<FMT, KC, GS>(meta[m], rs, g, (uint32_t)r16, row_meta, c_meta);
    __builtin_amdgcn_sched_barrier(0);
    float* red_w = red[it & 1][wave];
#pragma unroll
    for (int i = 0; i < 4; ++i) red_w[(4 * q + i) * 16 + r16] = rowscale * acc[i];
    lds_barrier();
    store_tile<false>(red[it & 1], nw, wave, lane, t, bt, bt_rows, g, yrs);
  };

  // two tiles per iteration (metadata slots 0 and 1), loads unconditional;
  // an odd last tile runs after the loop without refills
  int it = 0;
  for (; it + 2 <= count; it += 2) {
    tile(std::integral_constant<int, 0>{}, it, true);
    tile(std::integral_constant<int, 1>{}, it + 1, true);
  }
  if (it < count) tile(std::integral_constant<int, 0>{}, it, false);
}

// ---------------------------------------------------------------------------
// K-split variant for larger batches.  The full-K kernel above holds each
// workgroup's activations for the whole of K, so every workgroup pulls
// b * k * 2 bytes of x through the cache, and with b > 16 the workgroups of
// the batch tiles each re-read the weights.  Here a workgroup owns one K-part
// (8 waves x KC chunks) of ALL batch tiles: its activations stay in
// registers, each weight chunk is read and decoded once and feeds the MFMAs
// of every batch tile.  A workgroup sums its waves' partial tiles through LDS
// and stores the fp32 result to its own slot of a workspace, one slot per
// (part, row tile); a second kernel adds the slots of each row tile in part
// order and rounds to fp16.  Deterministic: no atomics, and the order of
// every addition is fixed.



template <int FMT, int KC, int GS, int BT, int D>
__global__ void __launch_bounds__(64 * kSplitWaves)
gemm_split_kernel(WeightView W, const _Float16* __restrict__ x, float* __restrict__ ws, SplitGeom sg) {
  using S = Slice<FMT, KC, GS>;
  constexpr int ORDER = StreamFmt<FMT>::order;
  constexpr bool kTranspose = S::grouped && GS < 4;
  constexpr int VALS = BT * 256;
  constexpr int VPL = (VALS + 64 * kSplitWaves - 1) / (64 * kSplitWaves);  // outputs per lane in the reduction
  __shared__ float red[2][kSplitWaves][VALS];

  const StreamGeom& g = sg.s;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, q = lane >> 4;

  StreamRes rs;
  rs.codes = make_rsrc(W.codes, g.codes_bytes);
  rs.hi = make_rsrc(W.codes_hi, g.hi_bytes);
  rs.scales = make_rsrc(W.scales, g.scales_bytes);
  rs.aux = make_rsrc(W.aux, g.aux_bytes);
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(ws, sg.ws_bytes);

  LaneOff lo;
  lo.code = (uint32_t)r16 * g.codes_row + StreamFmt<FMT>::piece_bytes * q;
  lo.hi = (uint32_t)r16 * g.hi_row + 8u * q;

  // this workgroup's K-part and row group; the wave's chunks in the part
  // (clamped to the last real chunk for loads: activations past k are zero)
  const int part = (int)blockIdx.x % sg.parts, rg = (int)blockIdx.x / sg.parts;
  const int c_begin = __builtin_amdgcn_readfirstlane((part * kSplitWaves + wave) * KC);
  const uint32_t c_meta = (uint32_t)min(c_begin, g.chunks - 1);
  uint32_t ccl[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) ccl[c] = (uint32_t)min(c_begin + c, g.chunks - 1);
  const uint32_t gfirst = S::grouped ? (c_meta * 128u) >> g.gshift : 0u;
  const int count = rg < g.tiles ? (g.tiles - 1 - rg) / sg.grid_rows + 1 : 0;

  // activation fragments of every batch tile over the wave's chunks
  h8 xa[KC][BT][4];
  {
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, g.x_bytes);
#pragma unroll
    for (int c = 0; c < KC; ++c)
#pragma unroll
      for (int t = 0; t < BT; ++t) {
        const int row = 16 * t + r16;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int k = (c_begin + c) * 128 + (kTranspose ? 32 * s + 8 * q : 32 * q + 8 * s);
          const uint32_t off = (k < g.k && row < g.b) ? ((uint32_t)row * (uint32_t)g.k + (uint32_t)k) * 2u : 0xFFFFFF00u;
          const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0);
          const uint4 pm = permute8<ORDER>(make_uint4(v.x, v.y, v.z, v.w));
          xa[c][t][s] = make_h8(pm.x, pm.y, pm.z, pm.w);
        }
      }
  }

  // ring of D row tiles, as in the full-K kernel
  ChunkRegs<FMT> ring[D][KC];
  TileMeta<FMT, KC, GS> meta[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    // a unit's memory operations in a unit's order (codes, metadata, then
    // the workspace stores, dropped here): see the full-K kernel
    const uint32_t row0 = (uint32_t)(d < count ? rg + d * sg.grid_rows : rg) * 16u;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      load_chunk<FMT>(ring[d][c], rs, g, lo, row0, ccl[c]);
      __builtin_amdgcn_sched_barrier(0);
    }
    load_meta<FMT, KC, GS>(meta[d], rs, g, (uint32_t)r16, row0, c_meta);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int v = 0; v < VPL; ++v) __builtin_amdgcn_raw_buffer_store_b32(0u, wrs, 0xFFFFFF00u, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int c = 0; c < KC; ++c)
#pragma unroll
    for (int t = 0; t < BT; ++t)
#pragma unroll
      for (int s = 0; s < 4; ++s) asm volatile("" : "+v"(xa[c][t][s]));

  auto unit = [&](auto dc, int it, bool reload) {
    constexpr int d = decltype(dc)::value;
    const int tile = rg + it * sg.grid_rows;
    const uint32_t row_load = (uint32_t)(it + D < count ? tile + D * sg.grid_rows : rg) * 16u;
    f4 acc[BT];
#pragma unroll
    for (int t = 0; t < BT; ++t) acc[t] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    const int eref = slice_eref<FMT, KC, GS>(meta[d]);
    float rowscale = slice_scale<FMT>(eref);
    if constexpr (FMT == Q_INT8) rowscale = h2f((uint16_t)(meta_word(meta[d], 0) & 0xFFFFu));
    static_for<0, KC>([&](auto cc) {
      constexpr int C = decltype(cc)::value;
      consume_chunk<FMT, KC, GS, C, BT>(ring[d][C], meta[d], xa[C], acc, gfirst, q, eref);
      if (reload) load_chunk<FMT>(ring[d][C], rs, g, lo, row_load, ccl[C]);
      __builtin_amdgcn_sched_barrier(0);
    });
    if (reload) load_meta<FMT, KC, GS>(meta[d], rs, g, (uint32_t)r16, row_load, c_meta);
    __builtin_amdgcn_sched_barrier(0);
    // lane (r16, q) holds batch rows 16t + 4q .. 16t + 4q + 3 of weight row
    // r16: stored in lane order, four consecutive floats per lane and tile
    float* rw = red[it & 1][wave];
#pragma unroll
    for (int t = 0; t < BT; ++t) {
      const f4 v = rowscale * acc[t];
      *reinterpret_cast<f4*>(rw + t * 256 + lane * 4) = v;
    }
    lds_barrier();
    // output j of the slot is batch row j / 16, weight row j % 16 of the
    // tile; lane handles j = (v * 8 + wave) * 64 + lane.  Slots past VALS
    // (a whole wave's worth) store nowhere.
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int jw = v * kSplitWaves + wave;  // 64-output block of this wave
      const int j = jw * 64 + lane;
      const int bi = min(j >> 4, 16 * BT - 1), r = j & 15;  // (clamped for the unused slots)
      const int idx = (bi >> 4) * 256 + (((bi & 15) >> 2) * 16 + r) * 4 + (bi & 3);
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < kSplitWaves; ++w) sum += red[it & 1][w][idx];
      const uint32_t off = jw < 4 * BT
                               ? (((uint32_t)part * (uint32_t)g.tiles + (uint32_t)tile) * (uint32_t)VALS + (uint32_t)j) * 4u
                               : 0xFFFFFF00u;
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sum), wrs, off, 0, 0);
    }
  };

  int it = 0;
  for (; it + D <= count; it += D)
    static_for<0, D>([&](auto dc) { unit(dc, it + decltype(dc)::value, true); });
  static_for<0, D - 1>([&](auto dc) {
    if (it + decltype(dc)::value < count) unit(dc, it + decltype(dc)::value, false);
  });
}


// LDS form of the split product.  The workgroup's K-part of the activations
// (8 chunks, every batch tile) lives in LDS, laid out as the MFMA A-fragments
// themselves: block (chunk, batch tile, step) is 1 KiB, lane l's 16 bytes at
// 16 l, so every fragment is one conflict-free ds_read_b128.  Each wave then
// owns whole row tiles over the part -- its own 8-chunk register ring,
// refilled chunk by chunk with the next tile -- and stores its fp32 partial
// tile straight to the workspace: no cross-wave reduction and no barrier
// after the prologue.  Slot (part, tile) holds the tile in lane order:
// float 256 t + 4 l + i is batch row 16 t + 4 (l / 16) + i, weight row l % 16.
constexpr int kLdsChunks = 8;

template <int FMT, int GS, int BT>
__global__ void __launch_bounds__(64 * kSplitWaves)
gemm_split_lds_kernel(WeightView W, const _Float16* __restrict__ x, float* __restrict__ ws, SplitGeom sg) {
  constexpr int KC = kLdsChunks;
  using S = Slice<FMT, KC, GS>;
  constexpr int ORDER = StreamFmt<FMT>::order;
  constexpr bool kTranspose = S::grouped && GS < 4;
  __shared__ u32x4 xlds[KC * BT * 4 * 64];  // 32 KiB per batch tile

  const StreamGeom& g = sg.s;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, q = lane >> 4;

  StreamRes rs;
  rs.codes = make_rsrc(W.codes, g.codes_bytes);
  rs.hi = make_rsrc(W.codes_hi, g.hi_bytes);
  rs.scales = make_rsrc(W.scales, g.scales_bytes);
  rs.aux = make_rsrc(W.aux, g.aux_bytes);
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(ws, sg.ws_bytes);

  LaneOff lo;
  lo.code = (uint32_t)r16 * g.codes_row + StreamFmt<FMT>::piece_bytes * q;
  lo.hi = (uint32_t)r16 * g.hi_row + 8u * q;

  // part and row group of the workgroup; the wave walks row tiles
  // wave_id, wave_id + waves_per_part, ... of the part
  const int part = (int)blockIdx.x % sg.parts, rg = (int)blockIdx.x / sg.parts;
  const int c_begin = part * KC;
  const uint32_t c_meta = (uint32_t)min(c_begin, g.chunks - 1);
  uint32_t ccl[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) ccl[c] = (uint32_t)min(c_begin + c, g.chunks - 1);
  const uint32_t gfirst = S::grouped ? (c_meta * 128u) >> g.gshift : 0u;
  const int first = __builtin_amdgcn_readfirstlane(rg * kSplitWaves + wave);
  const int stride = sg.grid_rows * kSplitWaves;
  const int count = first < g.tiles ? (g.tiles - 1 - first) / stride + 1 : 0;
  auto tile_row = [&](int it) { return (uint32_t)(it < count ? first + it * stride : min(first, g.tiles - 1)) * 16u; };

  // the first tile's weights go out first, then the activations
  ChunkRegs<FMT> ring[KC];
  TileMeta<FMT, KC, GS> meta;
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    load_chunk<FMT>(ring[c], rs, g, lo, tile_row(0), ccl[c]);
    __builtin_amdgcn_sched_barrier(0);
  }
  load_meta<FMT, KC, GS>(meta, rs, g, (uint32_t)r16, tile_row(0), c_meta);
  __builtin_amdgcn_sched_barrier(0);
  {
    // activation fragment block b = (c * BT + t) * 4 + s, blocks dealt to
    // the waves in turn
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, g.x_bytes);
    constexpr int NB = KC * BT * 4, PER = (NB + kSplitWaves - 1) / kSplitWaves;
    u32x4 v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int blk = i * kSplitWaves + wave;
      const int s = blk & 3, t = (blk >> 2) % BT, c = (blk >> 2) / BT;
      const int row = 16 * t + r16;
      const int k = (c_begin + c) * 128 + (kTranspose ? 32 * s + 8 * q : 32 * q + 8 * s);
      const uint32_t off = (blk < NB && k < g.k && row < g.b) ? ((uint32_t)row * (uint32_t)g.k + (uint32_t)k) * 2u
                                                             : 0xFFFFFF00u;
      v[i] = __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int blk = i * kSplitWaves + wave;
      const uint4 pm = permute8<ORDER>(make_uint4(v[i].x, v[i].y, v[i].z, v[i].w));
      if (blk < NB) xlds[blk * 64 + lane] = u32x4{pm.x, pm.y, pm.z, pm.w};
    }
  }
  __syncthreads();

  for (int it = 0; it < count; ++it) {
    const uint32_t row_next = tile_row(it + 1);
    f4 acc[BT];
#pragma unroll
    for (int t = 0; t < BT; ++t) acc[t] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    const int eref = slice_eref<FMT, KC, GS>(meta);
    float rowscale = slice_scale<FMT>(eref);
    if constexpr (FMT == Q_INT8) rowscale = h2f((uint16_t)(meta_word(meta, 0) & 0xFFFFu));
    static_for<0, KC>([&](auto cc) {
      constexpr int C = decltype(cc)::value;
      h8 xa[BT][4];
#pragma unroll
      for (int t = 0; t < BT; ++t)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const u32x4 v = xlds[((C * BT + t) * 4 + s) * 64 + lane];
          xa[t][s] = make_h8(v.x, v.y, v.z, v.w);
        }
      consume_chunk<FMT, KC, GS, C, BT>(ring[C], meta, xa, acc, gfirst, q, eref);
      load_chunk<FMT>(ring[C], rs, g, lo, row_next, ccl[C]);
      __builtin_amdgcn_sched_barrier(0);
    });
    load_meta<FMT, KC, GS>(meta, rs, g, (uint32_t)r16, row_next, c_meta);
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t base = ((uint32_t)part * (uint32_t)g.tiles + (uint32_t)(first + it * stride)) * (uint32_t)(BT * 256);
#pragma unroll
    for (int t = 0; t < BT; ++t) {
      const f4 v = rowscale * acc[t];
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), wrs, (base + (uint32_t)(t * 256 + lane * 4)) * 4u,
                                             0, 0);
    }
  }
}



template <int FMT, int GS>
SplitKernelFn pick_split_lds_bt(int bt) {
  switch (bt) {
    case 1: return gemm_split_lds_kernel<FMT, GS, 1>;
    case 2: return gemm_split_lds_kernel<FMT, GS, 2>;
    case 3: return gemm_split_lds_kernel<FMT, GS, 3>;
    default: return gemm_split_lds_kernel<FMT, GS, 4>;
  }
}

template <int FMT>
SplitKernelFn pick_split_lds(int gs, int bt) {
  if constexpr (StreamFmt<FMT>::grouped) {
    switch (gs) {
      case 1: return pick_split_lds_bt<FMT, 1>(bt);
      case 2: return pick_split_lds_bt<FMT, 2>(bt);
      case 8: return pick_split_lds_bt<FMT, 8>(bt);
      default: return pick_split_lds_bt<FMT, 4>(bt);
    }
  }
  return pick_split_lds_bt<FMT, 4>(bt);
}



// (a ring of two row tiles: three and four measured no faster)
template <int FMT, int KC, int GS, int BT>
SplitKernelFn pick_split_depth(int) {
  return gemm_split_kernel<FMT, KC, GS, BT, 2>;
}

template <int FMT, int KC, int GS>
SplitKernelFn pick_split_bt(int bt, int depth) {
  switch (bt) {
    case 1: return pick_split_depth<FMT, KC, GS, 1>(depth);
    case 2: return pick_split_depth<FMT, KC, GS, 2>(depth);
    case 3: return pick_split_depth<FMT, KC, GS, 3>(depth);
    default: return pick_split_depth<FMT, KC, GS, 4>(depth);
  }
}

// One chunk per wave (two for groups of 256, a group spans two chunks, and
// when the plan asks for two)
template <int FMT>
SplitKernelFn pick_split(int gs, int bt, int depth, int kc) {
  if (kc == 2 && bt == 1) {
    if constexpr (StreamFmt<FMT>::grouped) {
      switch (gs) {
        case 1: return pick_split_depth<FMT, 2, 1, 1>(depth);
        case 2: return pick_split_depth<FMT, 2, 2, 1>(depth);
        case 8: return pick_split_depth<FMT, 2, 8, 1>(depth);
        default: return pick_split_depth<FMT, 2, 4, 1>(depth);
      }
    }
    return pick_split_depth<FMT, 2, 4, 1>(depth);
  }
  if (kc == 2 && bt >= 2) {
    if constexpr (StreamFmt<FMT>::grouped) {
      switch (gs) {
        case 1: return bt == 2 ? pick_split_depth<FMT, 2, 1, 2>(depth) : bt == 3 ? pick_split_depth<FMT, 2, 1, 3>(depth) : pick_split_depth<FMT, 2, 1, 4>(depth);
        case 2: return bt == 2 ? pick_split_depth<FMT, 2, 2, 2>(depth) : bt == 3 ? pick_split_depth<FMT, 2, 2, 3>(depth) : pick_split_depth<FMT, 2, 2, 4>(depth);
        case 8: return bt == 2 ? pick_split_depth<FMT, 2, 8, 2>(depth) : bt == 3 ? pick_split_depth<FMT, 2, 8, 3>(depth) : pick_split_depth<FMT, 2, 8, 4>(depth);
        default: return bt == 2 ? pick_split_depth<FMT, 2, 4, 2>(depth) : bt == 3 ? pick_split_depth<FMT, 2, 4, 3>(depth) : pick_split_depth<FMT, 2, 4, 4>(depth);
      }
    }
    return bt == 2 ? pick_split_depth<FMT, 2, 4, 2>(depth) : bt == 3 ? pick_split_depth<FMT, 2, 4, 3>(depth) : pick_split_depth<FMT, 2, 4, 4>(depth);
  }
  if constexpr (StreamFmt<FMT>::grouped) {
    switch (gs) {
      case 1: return pick_split_bt<FMT, 1, 1>(bt, depth);
      case 2: return pick_split_bt<FMT, 1, 2>(bt, depth);
      case 8: return pick_split_bt<FMT, 2, 8>(bt, depth);
      default: return pick_split_bt<FMT, 1, 4>(bt, depth);
    }
  }
  return pick_split_bt<FMT, 1, 4>(bt, depth);
}


// (one tile in flight: two measured no faster)
template <int FMT, int GS>
StreamKernelFn pick_kc(int kc, int) {
  switch (kc) {
    case 1: return gemm_stream_kernel<FMT, 1, GS, 1>;
    case 2: return gemm_stream_kernel<FMT, 2, GS, 1>;
    case 4: return gemm_stream_kernel<FMT, 4, GS, 1>;
    default: return gemm_stream_kernel<FMT, 8, GS, 1>;
  }
}

template <int FMT, int GS>
StreamKernelFn pick_xs(int) {
  return gemm_stream_xs_kernel<FMT, 16, GS, 4>;
}

template <int FMT>
StreamKernelFn pick_stream_xs(int kc, int gs) {
  if constexpr (StreamFmt<FMT>::grouped) {
    switch (gs) {
      case 1: return pick_xs<FMT, 1>(kc);
      case 2: return pick_xs<FMT, 2>(kc);
      case 8: return pick_xs<FMT, 8>(kc);
      default: return pick_xs<FMT, 4>(kc);
    }
  }
  return pick_xs<FMT, 4>(kc);
}


template <int FMT>
StreamKernelFn pick_stream(int kc, int gs, int depth) {
  if constexpr (StreamFmt<FMT>::grouped) {
    switch (gs) {
      case 1: return pick_kc<FMT, 1>(kc, depth);
      case 2: return pick_kc<FMT, 2>(kc, depth);
      case 8: return pick_kc<FMT, 8>(kc, depth);
      default: return pick_kc<FMT, 4>(kc, depth);
    }
  }
  return pick_kc<FMT, 4>(kc, depth);
}


}  // namespace

template <int FMT>
StreamKernelFn stream_kernel_for(int kc, int gs, int depth, bool xs) {
  return xs ? pick_stream_xs<FMT>(kc, gs) : pick_stream<FMT>(kc, gs, depth);
}

template <int FMT>
SplitKernelFn split_kernel_for(int gs, int bt, int kc, bool lds) {
  return lds ? pick_split_lds<FMT>(gs, bt) : pick_split<FMT>(gs, bt, 2, kc);
}

}  // namespace qg
