// Vector-ALU decode-and-dot building blocks shared by the b <= 8 GEMV
// (gemv_valu.hip) and the decode-stack kernel (stack.hip): the per-piece
// metadata, the fused decode + v_dot2 of one 32-element piece, and the DPP
// wave reduction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace qg {

struct Meta {
  float a, b;  // format-specific: (s, z) int4; (s, -) e2m1; (s, v) razer; (s+, s-) afpq; block exps; int8 unused
};

// Raw metadata of one piece as loaded (bits only; decoded at use so that no
// instruction waits on the load right after issuing it).
struct RawMeta {
  uint32_t a, b;
};

// Decode raw metadata into the two per-piece factors used by piece_dot.
template <int FMT>
__device__ __forceinline__ Meta decode_meta(const RawMeta& r) {
  Meta m{0.0f, 0.0f};
  if constexpr (FMT == Q_BFP6 || FMT == Q_BFP4) {
    constexpr int mb = FMT == Q_BFP6 ? 5 : 3;
    const int e0 = (int)(r.a & 0xFFu), e1 = (int)((r.a >> 8) & 0xFFu);
    m.a = e0 ? ldexpf(1.0f, e0 - 127 - mb + 1) : 0.0f;
    m.b = e1 ? ldexpf(1.0f, e1 - 127 - mb + 1) : 0.0f;
  } else if constexpr (is_afpq(FMT)) {
    m.a = h2f((uint16_t)(r.a & 0xFFFFu));
    m.b = h2f((uint16_t)(r.a >> 16));
  } else if constexpr (FMT != Q_INT8) {
    m.a = h2f((uint16_t)(r.a & 0xFFFFu));
    if constexpr (FMT == Q_INT4_ASYM) m.b = (float)(r.b & 0xFu);
    else if constexpr (is_razer(FMT)) m.b = razer_special_of<FMT>((int)(r.b & 3u));
  }
  return m;
}

// Operands of the 4-bit decode (the AND-OR masks and the fp16 magic
// number), held in VGPRs: a caller that creates them once, outside its
// loops, saves rebuilding them for every piece.
struct NibbleMasks {
  uint32_t lo, hi, magic, bytes;  // bytes: the int8 decode's byte mask
};
__device__ __forceinline__ NibbleMasks nibble_masks() {
  NibbleMasks m{0x000F000Fu, 0x00F000F0u, 0x64006400u, 0x00FF00FFu};
  asm("" : "+v"(m.lo), "+v"(m.hi), "+v"(m.magic), "+v"(m.bytes));
  return m;
}

// The first product of an accumulator chain: v_dot2_f32_f16 with an inline
// zero addend.  (The builtin with a zero addend becomes a move of 0 and the
// accumulating v_dot2c form.)
__device__ __forceinline__ float dot2_first(h2 a, uint32_t b) {
  float r;
  asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Dot products of one 32-element piece with the B activation slices.
// `cw` holds the piece's code words (4, 3 for the 3-bit formats, or 8 for
// int8), `hw` the bfp6 high plane words, `xr[b]` the 16 activation pairs in
// decoder order, `xsum` the piece's activation sums (int4: 1024 X_even +
// 64 X_odd and X_even + X_odd, or with HALF_SUMS the even and odd sums of
// each 16-element half, as for bfp4; int8: 1152 X, or nothing with
// HALF_SUMS; unused by the other formats).
template <int FMT, int B, bool HALF_SUMS = false>
__device__ __forceinline__ void piece_dot(const uint32_t* cw_in, const uint32_t* hw, const RawMeta& raw,
                                          const uint32_t (*xr)[16], const float* xsum, float* acc,
                                          const NibbleMasks& nm) {
  const Meta m = decode_meta<FMT>(raw);
  uint32_t cw3[4];
  const uint32_t* cw = cw_in;
  if constexpr (is_fp3(FMT)) {  // three words -> four E2M1 code words of the same values
    expand_fp3(cw_in[0], cw_in[1], cw_in[2], cw3);
    cw = cw3;
  }
  if constexpr (FMT == Q_FP4_E2M1 || is_razer(FMT) || is_afpq(FMT)) {
    // two accumulator chains per sum (words 0-1 and 2-3) for instruction-level parallelism
    float p[2][B], q[2][B];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int b = 0; b < B; ++b) { p[h][b] = 0.0f; q[h][b] = 0.0f; }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int h = w >> 1;
      const h2 d[4] = {fp4_pair<0>(cw[w]), fp4_pair<1>(cw[w]), fp4_pair<2>(cw[w]), fp4_pair<3>(cw[w])};
      if constexpr (is_razer(FMT)) {
        uint32_t m8 = 0x88888888u;
        asm("" : "+v"(m8));
        const uint32_t sm = special_mask(cw[w], m8);
        const h2 e[4] = {fp4_pair<0>(sm), fp4_pair<1>(sm), fp4_pair<2>(sm), fp4_pair<3>(sm)};
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int b = 0; b < B; ++b) q[h][b] = __builtin_amdgcn_fdot2(e[j], as_h2(xr[b][4 * w + j]), q[h][b], false);
      }
      if constexpr (is_afpq(FMT)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const h2 mag = as_h2(as_u32(d[j]) & 0x7FFF7FFFu);
#pragma unroll
          for (int b = 0; b < B; ++b) q[h][b] = __builtin_amdgcn_fdot2(mag, as_h2(xr[b][4 * w + j]), q[h][b], false);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int b = 0; b < B; ++b) p[h][b] = __builtin_amdgcn_fdot2(d[j], as_h2(xr[b][4 * w + j]), p[h][b], false);
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float ps = p[0][b] + p[1][b], qs = q[0][b] + q[1][b];
      if constexpr (FMT == Q_FP4_E2M1) acc[b] += m.a * ps;
      else if constexpr (is_razer(FMT)) acc[b] += m.a * (ps + m.b * qs);
      else {
        // ps = P - Q (signed), qs = P + Q (magnitudes); y += s+ P - s- Q
        const float P = 0.5f * (qs + ps);
        const float Q = 0.5f * (qs - ps);
        acc[b] += m.a * P - m.b * Q;
      }
    }
  } else if constexpr (FMT == Q_INT4_ASYM || FMT == Q_BFP4) {
    // Fields j = 0, 2 of a word (even elements) decode to 1024 + u and fields
    // j = 1, 3 (odd elements) to 1024 + 16 u, each with one AND-OR on the word
    // or on the word shifted by 8; the 1024 * x part is removed per piece
    // with the activation sums (xsum).  u is the stored nibble (int4: q;
    // bfp4: offset binary m + 8).  Each accumulator chain starts from its
    // first product (no zeroed register to add it to).
    float a[2][B], c[2][B];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t u = FMT == Q_BFP4 ? cw[w] ^ 0x88888888u : cw[w];
      const uint32_t u8 = u >> 8;
      const h2 t0 = as_h2(and_or(u, nm.lo, nm.magic));
      const h2 t1 = as_h2(and_or(u, nm.hi, nm.magic));
      const h2 t2 = as_h2(and_or(u8, nm.lo, nm.magic));
      const h2 t3 = as_h2(and_or(u8, nm.hi, nm.magic));
      const int h = w >> 1;
#pragma unroll
      for (int b = 0; b < B; ++b) {
        if (w & 1) {
          a[h][b] = __builtin_amdgcn_fdot2(t0, as_h2(xr[b][4 * w + 0]), a[h][b], false);
          c[h][b] = __builtin_amdgcn_fdot2(t1, as_h2(xr[b][4 * w + 1]), c[h][b], false);
        } else {
          a[h][b] = dot2_first(t0, xr[b][4 * w + 0]);
          c[h][b] = dot2_first(t1, xr[b][4 * w + 1]);
        }
        a[h][b] = __builtin_amdgcn_fdot2(t2, as_h2(xr[b][4 * w + 2]), a[h][b], false);
        c[h][b] = __builtin_amdgcn_fdot2(t3, as_h2(xr[b][4 * w + 3]), c[h][b], false);
      }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float* xsb = xsum + 4 * b;
      if constexpr (FMT == Q_INT4_ASYM) {
        // sum (q - z) x = A + C/16 - (1024 + z) X_even - (64 + z) X_odd
        //              = A + C/16 - K1 - z K2,  K1 = 1024 X_even + 64 X_odd, K2 = X_even + X_odd
        const float A = a[0][b] + a[1][b], C = c[0][b] + c[1][b];
        float k1 = xsb[0], k2 = xsb[1];
        if constexpr (HALF_SUMS) {
          const float xe = xsb[0] + xsb[2], xo = xsb[1] + xsb[3];
          k1 = 1024.0f * xe + 64.0f * xo;
          k2 = xe + xo;
        }
        acc[b] += m.a * (((A + 0.0625f * C) - k1) - m.b * k2);
      } else {  // {even, odd} sums of halves 0 and 1
        // per 16-element block: sum (u - 8) x = A + C/16 - 1032 X_even - 72 X_odd
        const float v0 = (a[0][b] + 0.0625f * c[0][b]) - 1032.0f * xsb[0] - 72.0f * xsb[1];
        const float v1 = (a[1][b] + 0.0625f * c[1][b]) - 1032.0f * xsb[2] - 72.0f * xsb[3];
        acc[b] += m.a * v0 + m.b * v1;
      }
    }
  } else if constexpr (FMT == Q_BFP6) {
    const h2 bias = h2{(_Float16)1056.0f, (_Float16)1056.0f};  // 1024 + offset-binary bias 32
    float p[2][B];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int b = 0; b < B; ++b) p[h][b] = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t lo = cw[w];
      const uint32_t hi = hw[w >> 1] ^ 0xAAAAAAAAu;  // offset binary: flip the field's top bit
      const int hsh = 8 * (w & 1);
      const uint32_t t[4] = {six_bit_magic<0>(lo, hi, hsh), six_bit_magic<1>(lo, hi, hsh),
                             six_bit_magic<2>(lo, hi, hsh), six_bit_magic<3>(lo, hi, hsh)};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const h2 v = as_h2(t[j]) - bias;  // exact small integers
#pragma unroll
        for (int b = 0; b < B; ++b)
          p[w >> 1][b] = __builtin_amdgcn_fdot2(v, as_h2(xr[b][4 * w + j]), p[w >> 1][b], false);
      }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] += m.a * p[0][b] + m.b * p[1][b];
  } else if constexpr (HALF_SUMS) {  // Q_INT8: 8 words of 4 bytes, the bias removed per element
    const h2 bias = h2{(_Float16)1152.0f, (_Float16)1152.0f};
    float p[B];
#pragma unroll
    for (int b = 0; b < B; ++b) p[b] = 0.0f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint32_t u = cw[w] ^ 0x80808080u;
      const h2 v0 = as_h2(byte_magic_lo(u)) - bias;
      const h2 v1 = as_h2(byte_magic_hi(u)) - bias;
#pragma unroll
      for (int b = 0; b < B; ++b) {
        p[b] = __builtin_amdgcn_fdot2(v0, as_h2(xr[b][2 * w + 0]), p[b], false);
        p[b] = __builtin_amdgcn_fdot2(v1, as_h2(xr[b][2 * w + 1]), p[b], false);
      }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] += p[b];
  } else {  // Q_INT8: the bytes as 1152 + q (exact fp16 integers), the bias removed per piece
    float p[2][B];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint32_t u = cw[w] ^ 0x80808080u;
      const h2 v0 = as_h2(and_or(u, nm.bytes, nm.magic));
      const h2 v1 = as_h2(and_or(u >> 8, nm.bytes, nm.magic));
      const int h = w >> 2;
#pragma unroll
      for (int b = 0; b < B; ++b) {
        p[h][b] = (w & 3) ? __builtin_amdgcn_fdot2(v0, as_h2(xr[b][2 * w + 0]), p[h][b], false)
                          : dot2_first(v0, xr[b][2 * w + 0]);
        p[h][b] = __builtin_amdgcn_fdot2(v1, as_h2(xr[b][2 * w + 1]), p[h][b], false);
      }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] += (p[0][b] + p[1][b]) - xsum[4 * b];
  }
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xF, false));
}

// piece_dot with the 4-bit decode's operands built at the call.
template <int FMT, int B, bool HALF_SUMS = false>
__device__ __forceinline__ void piece_dot(const uint32_t* cw_in, const uint32_t* hw, const RawMeta& raw,
                                          const uint32_t (*xr)[16], const float* xsum, float* acc) {
  piece_dot<FMT, B, HALF_SUMS>(cw_in, hw, raw, xr, xsum, acc, nibble_masks());
}

// Sum over each 16-lane row with DPP: afterwards every lane holds the sum of
// its own row.
__device__ __forceinline__ float row_total(float v) {
  v += dpp_f32<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141, 0xF>(v);  // row_half_mirror
  v += dpp_f32<0x140, 0xF>(v);  // row_mirror
  return v;
}

// Full 64-lane sum with DPP row operations; the total is returned uniformly.
__device__ __forceinline__ float wave_total(float v) {
  v = row_total(v);
  v += dpp_f32<0x142, 0xA>(v);  // row_bcast15 into rows 1 and 3
  v += dpp_f32<0x143, 0xC>(v);  // row_bcast31 into rows 2 and 3: lane 63 holds the total
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

}  // namespace qg
