// RTN quantize-and-pack kernel: fp16 weights [n][k] -> packed codes and
// per-group metadata, bit-identical to the layout documented in qgemv.h.
//
// One workgroup (256 lanes) per row; each lane owns 8 consecutive elements
// (one 32-bit code word) per pass over the row.  Group statistics are reduced
// across the g/8 lanes of a group with cross-lane shuffles.
//
// Exactness: every scale is one fp32 operation sequence rounded once to fp16;
// every code decision compares |w| with c * s where c has at most 9
// significant bits, so c * s is exact in fp32 and the comparison is exact.
// FMA contraction is disabled so each product and sum rounds on its own.
// The pragma does not stop the backend from fusing a multiply with a
// following fp16 conversion (v_fma_mixlo_f16, one rounding instead of two);
// the only such fusion here is a division of an absmax by 8, which is an
// exact power-of-two scaling, so one and two roundings agree.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"
#include "internal.hpp"

#pragma clang fp contract(off)

namespace qg {
namespace {

constexpr int kPackThreads = 256;

__device__ __forceinline__ float to_f16_f32(float v) { return (float)(_Float16)v; }

// round-half-even(a / s) for s > 0 with a, s fp16 values.  The fp32 quotient
// is at most one step off; the exact boundaries (r +- 0.5) * s settle it.
__device__ __forceinline__ float rne_div(float a, float s) {
  float r = rintf(a / s);
  const float up = (r + 0.5f) * s;
  const float dn = (r - 0.5f) * s;
  const bool odd = (((int)r) & 1) != 0;
  if (a > up || (a == up && odd)) r += 1.0f;
  else if (a < dn || (a == dn && odd)) r -= 1.0f;
  return r;
}

// Clipping search: candidate c shrinks a range bound v by the ratio
// (kClipDenom - c) / kClipDenom: v * (20 - c) is exact for an fp16 value v,
// then one correctly rounded division; c = 0 returns v.
constexpr int kClipDenom = 20;
__device__ __forceinline__ float clip_bound(float v, int c) {
  return (v * (float)(kClipDenom - c)) / (float)kClipDenom;
}

// Nearest E2M1 magnitude index of a >= 0 under scale s, ties to even index.
// Midpoints 0.25 0.75 1.25 1.75 2.5 3.5 5 (times s); at an odd-indexed
// midpoint the upper (even) neighbour wins the tie.
__device__ __forceinline__ int e2m1_index(float a, float s) {
  if (s == 0.0f) return 0;
  int i = 0;
  i += a > 0.25f * s;
  i += a >= 0.75f * s;
  i += a > 1.25f * s;
  i += a >= 1.75f * s;
  i += a > 2.5f * s;
  i += a >= 3.5f * s;
  i += a > 5.0f * s;
  return i;
}

__device__ __forceinline__ float e2m1_magnitude(int idx) {
  const int e = idx >> 1, m = idx & 1;
  return e == 0 ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, e - 1);
}

// Nearest FP3 (E2M0) magnitude index of a >= 0 under scale s, ties to even
// index: midpoints 0.5, 1.5, 3 (times s); at 1.5 the upper (even) neighbour
// wins, at 0.5 and 3 the lower.
__device__ __forceinline__ int fp3_index(float a, float s) {
  if (s == 0.0f) return 0;
  return (int)(a > 0.5f * s) + (int)(a >= 1.5f * s) + (int)(a > 3.0f * s);
}

__device__ __forceinline__ float fp3_magnitude(int idx) { return idx == 0 ? 0.0f : ldexpf(1.0f, idx - 1); }

// Whether x lies strictly inside the interval where the 3-bit RaZeR special
// of candidate c (+3, -3, +8, -8 times s) is nearer than every FP3 value.
__device__ __forceinline__ bool fp3_special(float x, float s, int c) {
  bool sp;
  if (c == 0) sp = x > 2.5f * s && x < 3.5f * s;
  else if (c == 1) sp = x < -2.5f * s && x > -3.5f * s;
  else if (c == 2) sp = x > 6.0f * s;
  else sp = x < -6.0f * s;
  return sp && s != 0.0f;  // a zero scale makes every value 0
}

template <int L>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int off = L / 2; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
template <int L>
__device__ __forceinline__ float group_min(float v) {
#pragma unroll
  for (int off = L / 2; off >= 1; off >>= 1) v = fminf(v, __shfl_xor(v, off, 64));
  return v;
}

// Sum of squared errors over a group, in the fixed order a <- a[:h] + a[h:]
// (fp64).  Lane j of the group holds elements 8j..8j+7 in sq[0..7].  The
// result is valid in every lane of the group.
template <int L>
__device__ __forceinline__ double group_sse(double sq[8], int lane) {
#pragma unroll
  for (int h = L / 2; h >= 1; h >>= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) sq[i] = sq[i] + __shfl_xor(sq[i], h, 64);
  }
#pragma unroll
  for (int h = 4; h >= 1; h >>= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < h) sq[i] = sq[i] + sq[i + h];
  }
  const int leader = lane & ~(L - 1);
  return __shfl(sq[0], leader, 64);
}

// ---------------------------------------------------------------- formats --

// Groups of g = 8*L elements (L lanes), 4-bit codes plus fp16 scale.
// nclip > 1 (the grouped 4-bit formats): each group keeps the clipping
// candidate c < nclip whose RTN codes give the smallest fp64 SSE (ties:
// smaller c; RaZeR tries its four specials under each c).
template <int FMT, int L>
__device__ void pack_row_grouped(const WeightView& W, const _Float16* __restrict__ src, int row,
                                 uint8_t* lds_meta, int nclip) {
  const int k = W.k;
  const int lane = threadIdx.x & 63;
  const int groups = k / (8 * L);
  uint32_t* codes = const_cast<uint32_t*>(W.codes) + (size_t)row * (k / 8);
  for (int base = 0; base < k; base += kPackThreads * 8) {
    const int e0 = base + threadIdx.x * 8;
    const bool active = e0 < k;  // k % 32 == 0, so a lane is all in or all out
    float w[8];
    if (active) {
      const uint4 raw = *reinterpret_cast<const uint4*>(src + e0);
      const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[2 * i] = h2f((uint16_t)(rw[i] & 0xFFFFu));
        w[2 * i + 1] = h2f((uint16_t)(rw[i] >> 16));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = 0.0f;
    }
    // Inactive lanes are whole groups (k is a multiple of 32 and of g), so
    // their zeros never mix with real data in a group reduction.
    const int gi = e0 / (8 * L);
    const bool leader = (lane & (L - 1)) == 0;
    uint32_t word = 0;
    if constexpr (FMT == Q_INT4_ASYM) {
      float lo = 0.0f, hi = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) { lo = fminf(lo, w[i]); hi = fmaxf(hi, w[i]); }
      lo = group_min<L>(lo);
      hi = group_max<L>(hi);
      if (nclip > 1) {
        double best_sse = 0.0;
        int best = 0;
        for (int c = 0; c < nclip; ++c) {
          const float lc = clip_bound(lo, c), hc = clip_bound(hi, c);
          const float s = to_f16_f32((hc - lc) / 15.0f);
          int z = 0;
          if (s != 0.0f) z = (int)fminf(fmaxf(rne_div(-lc, s), 0.0f), 15.0f);
          double sq[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            int q = 0;
            if (s != 0.0f) q = (int)fminf(fmaxf((float)z + rne_div(w[i], s), 0.0f), 15.0f);
            const double d = (double)w[i] - (double)((float)(q - z) * s);
            sq[i] = d * d;
          }
          const double sse = group_sse<L>(sq, lane);
          if (c == 0 || sse < best_sse) { best_sse = sse; best = c; }
        }
        lo = clip_bound(lo, best);
        hi = clip_bound(hi, best);
      }
      const float s = to_f16_f32((hi - lo) / 15.0f);
      int z = 0;
      if (s != 0.0f) z = (int)fminf(fmaxf(rne_div(-lo, s), 0.0f), 15.0f);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int q = 0;
        if (s != 0.0f) q = (int)fminf(fmaxf((float)z + rne_div(w[i], s), 0.0f), 15.0f);
        word |= (uint32_t)q << (4 * i);
      }
      if (active && leader) {
        reinterpret_cast<_Float16*>(const_cast<void*>(W.scales))[(size_t)row * groups + gi] = (_Float16)s;
        lds_meta[gi] = (uint8_t)z;
      }
    } else if constexpr (FMT == Q_FP4_E2M1) {
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(w[i]));
      a = group_max<L>(a);
      if (nclip > 1) {
        double best_sse = 0.0;
        int best = 0;
        for (int c = 0; c < nclip; ++c) {
          const float s = to_f16_f32(clip_bound(a, c) / 6.0f);
          double sq[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float mag = e2m1_magnitude(e2m1_index(fabsf(w[i]), s)) * s;
            const double d = (double)w[i] - (double)(w[i] < 0.0f ? -mag : mag);
            sq[i] = d * d;
          }
          const double sse = group_sse<L>(sq, lane);
          if (c == 0 || sse < best_sse) { best_sse = sse; best = c; }
        }
        a = clip_bound(a, best);
      }
      const float s = to_f16_f32(a / 6.0f);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int idx = e2m1_index(fabsf(w[i]), s);
        const int code = (w[i] < 0.0f && idx > 0) ? (8 | idx) : idx;
        word |= (uint32_t)code << (4 * i);
      }
      if (active && leader)
        reinterpret_cast<_Float16*>(const_cast<void*>(W.scales))[(size_t)row * groups + gi] = (_Float16)s;
    } else if constexpr (FMT == Q_FP4_RAZER) {
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(w[i]));
      a = group_max<L>(a);
      double best_sse = 0.0;
      int best = 0, best_clip = 0;
      for (int cc = 0; cc < nclip; ++cc) {  // clipping candidates (1: plain RTN)
      const float ac = clip_bound(a, cc);
      const float s6 = to_f16_f32(ac / 6.0f);
      const float s8 = to_f16_f32(ac / 8.0f);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float v = razer_special(c);
        const float s = (c & 2) ? s8 : s6;
        double sq[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float x = w[i];
          const int idx = e2m1_index(fabsf(x), s);
          const float mag = e2m1_magnitude(idx) * s;
          float deq = (x < 0.0f) ? -mag : mag;
          bool special;
          if (c == 0) special = x > 4.5f * s && x < 5.5f * s;
          else if (c == 1) special = x < -4.5f * s && x > -5.5f * s;
          else if (c == 2) special = x > 7.0f * s;
          else special = x < -7.0f * s;
          special = special && s != 0.0f;  // a zero scale makes every value 0
          if (special) deq = v * s;
          const double d = (double)x - (double)deq;
          sq[i] = d * d;
        }
        const double sse = group_sse<L>(sq, lane);
        if ((cc == 0 && c == 0) || sse < best_sse) { best_sse = sse; best = c; best_clip = cc; }
      }
      }
      const float ab = clip_bound(a, best_clip);
      const float s = (best & 2) ? to_f16_f32(ab / 8.0f) : to_f16_f32(ab / 6.0f);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = w[i];
        bool special;
        if (best == 0) special = x > 4.5f * s && x < 5.5f * s;
        else if (best == 1) special = x < -4.5f * s && x > -5.5f * s;
        else if (best == 2) special = x > 7.0f * s;
        else special = x < -7.0f * s;
        special = special && s != 0.0f;
        int code;
        if (special) code = 8;
        else {
          const int idx = e2m1_index(fabsf(x), s);
          code = (x < 0.0f && idx > 0) ? (8 | idx) : idx;
        }
        word |= (uint32_t)code << (4 * i);
      }
      if (active && leader) {
        reinterpret_cast<_Float16*>(const_cast<void*>(W.scales))[(size_t)row * groups + gi] = (_Float16)s;
        lds_meta[gi] = (uint8_t)best;
      }
    } else if constexpr (FMT == Q_FP4_AFPQ) {
      float p = 0.0f, m = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) { p = fmaxf(p, w[i]); m = fmaxf(m, -w[i]); }
      p = group_max<L>(p);
      m = group_max<L>(m);
      if (nclip > 1) {  // both one-sided ranges shrink by the same ratio
        double best_sse = 0.0;
        int best = 0;
        for (int c = 0; c < nclip; ++c) {
          const float sp = to_f16_f32(clip_bound(p, c) / 6.0f);
          const float sn = to_f16_f32(clip_bound(m, c) / 6.0f);
          double sq[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float x = w[i];
            float deq = 0.0f;
            if (x > 0.0f) deq = e2m1_magnitude(e2m1_index(x, sp)) * sp;
            else if (x < 0.0f) deq = -(e2m1_magnitude(e2m1_index(-x, sn)) * sn);
            const double d = (double)x - (double)deq;
            sq[i] = d * d;
          }
          const double sse = group_sse<L>(sq, lane);
          if (c == 0 || sse < best_sse) { best_sse = sse; best = c; }
        }
        p = clip_bound(p, best);
        m = clip_bound(m, best);
      }
      const float sp = to_f16_f32(p / 6.0f);
      const float sn = to_f16_f32(m / 6.0f);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int code = 0;
        if (w[i] > 0.0f) code = e2m1_index(w[i], sp);
        else if (w[i] < 0.0f) {
          const int idx = e2m1_index(-w[i], sn);
          code = idx ? (8 | idx) : 0;
        }
        word |= (uint32_t)code << (4 * i);
      }
      if (active && leader) {
        const uint32_t pair = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)sp) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)sn) << 16);
        reinterpret_cast<uint32_t*>(const_cast<void*>(W.scales))[(size_t)row * groups + gi] = pair;
      }
    } else if constexpr (FMT == Q_FP3_RAZER) {
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(w[i]));
      a = group_max<L>(a);
      const float s4 = to_f16_f32(a / 4.0f);
      const float s8 = to_f16_f32(a / 8.0f);
      double best_sse = 0.0;
      int best = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float v = razer_special_of<Q_FP3_RAZER>(c);
        const float s = (c & 2) ? s8 : s4;
        double sq[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float x = w[i];
          const float mag = fp3_magnitude(fp3_index(fabsf(x), s)) * s;
          const float deq = fp3_special(x, s, c) ? v * s : (x < 0.0f ? -mag : mag);
          const double d = (double)x - (double)deq;
          sq[i] = d * d;
        }
        const double sse = group_sse<L>(sq, lane);
        if (c == 0 || sse < best_sse) { best_sse = sse; best = c; }
      }
      const float s = (best & 2) ? s8 : s4;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = w[i];
        int code = 4;
        if (!fp3_special(x, s, best)) {
          const int idx = fp3_index(fabsf(x), s);
          code = (x < 0.0f && idx > 0) ? (4 | idx) : idx;
        }
        word |= (uint32_t)code << (4 * i);  // 3-bit codes in nibbles; laid out below
      }
      if (active && leader) {
        reinterpret_cast<_Float16*>(const_cast<void*>(W.scales))[(size_t)row * groups + gi] = (_Float16)s;
        lds_meta[gi] = (uint8_t)best;
      }
    } else if constexpr (FMT == Q_FP3_AFPQ) {
      float p = 0.0f, m = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) { p = fmaxf(p, w[i]); m = fmaxf(m, -w[i]); }
      p = group_max<L>(p);
      m = group_max<L>(m);
      const float sp = to_f16_f32(p / 4.0f);
      const float sn = to_f16_f32(m / 4.0f);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int code = 0;
        if (w[i] > 0.0f) code = fp3_index(w[i], sp);
        else if (w[i] < 0.0f) {
          const int idx = fp3_index(-w[i], sn);
          code = idx ? (4 | idx) : 0;
        }
        word |= (uint32_t)code << (4 * i);  // 3-bit codes in nibbles; laid out below
      }
      if (active && leader) {
        const uint32_t pair = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)sp) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)sn) << 16);
        reinterpret_cast<uint32_t*>(const_cast<void*>(W.scales))[(size_t)row * groups + gi] = pair;
      }
    }
    if constexpr (is_fp3(FMT)) {
      // Lane q = 0..3 of a 32-element piece holds its elements 8q .. 8q+7
      // (3-bit codes, one per nibble of `word`).  Its index bits go to word
      // q/2 (bits 4r+1, 4r+2 for even q; 4r+3, (4r+4) mod 32 for odd q) and
      // its signs to word 2 (bit 4r + 3 - q); the four lanes OR their parts.
      const int q = lane & 3;
      uint32_t iw = 0, sw = 0;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const uint32_t c = (word >> (4 * r)) & 7u;
        const uint32_t i0 = c & 1u, i1 = (c >> 1) & 1u;
        if (q & 1) iw |= (i0 << (4 * r + 3)) | (i1 << ((4 * r + 4) & 31));
        else iw |= (i0 << (4 * r + 1)) | (i1 << (4 * r + 2));
        sw |= ((c >> 2) & 1u) << (4 * r + 3 - q);
      }
      iw |= __shfl_xor(iw, 1, 64);
      sw |= __shfl_xor(sw, 1, 64);
      sw |= __shfl_xor(sw, 2, 64);
      if (active && q != 3) {
        uint32_t* piece = const_cast<uint32_t*>(W.codes) + (size_t)row * (k / 32) * 3 + (size_t)(e0 / 32) * 3;
        piece[q == 0 ? 0 : q == 2 ? 1 : 2] = q == 1 ? sw : iw;
      }
    } else {
      if (active) codes[e0 / 8] = word;
    }
  }
}

// Block formats: 16 elements (2 lanes) share one exponent byte.
template <int MB>
__device__ void pack_row_block(const WeightView& W, const _Float16* __restrict__ src, int row) {
  const int k = W.k;
  const int lane = threadIdx.x & 63;
  uint32_t* codes = const_cast<uint32_t*>(W.codes) + (size_t)row * (k / 8);
  uint32_t* codes_hi = const_cast<uint32_t*>(W.codes_hi) + (size_t)row * (k / 16);
  uint8_t* exps = reinterpret_cast<uint8_t*>(const_cast<void*>(W.aux)) + (size_t)row * (k / 16);
  const int mmax = (1 << MB) - 1;
  for (int base = 0; base < k; base += kPackThreads * 8) {
    const int e0 = base + threadIdx.x * 8;
    const bool active = e0 < k;
    float w[8];
    if (active) {
      const uint4 raw = *reinterpret_cast<const uint4*>(src + e0);
      const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[2 * i] = h2f((uint16_t)(rw[i] & 0xFFFFu));
        w[2 * i + 1] = h2f((uint16_t)(rw[i] >> 16));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = 0.0f;
    }
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(w[i]));
    a = group_max<2>(a);
    int E = 0;
    if (a > 0.0f) E = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;
    uint32_t lo = 0, hi = 0;
    const int half = lane & 1;  // which 8 of the 16-element block
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int m = 0;
      if (a > 0.0f) {
        m = (int)rintf(ldexpf(fabsf(w[i]), -(E - MB + 1)));
        m = m > mmax ? mmax : m;
      }
      const int val = w[i] < 0.0f ? -m : m;
      const uint32_t field = (uint32_t)val & ((1u << (MB + 1)) - 1u);
      lo |= (field & 0xFu) << (4 * i);
      if constexpr (MB == 5) hi |= (field >> 4) << (16 * (i >> 2) + 8 * half + 2 * (i & 3));
    }
    if constexpr (MB == 5) hi |= __shfl_xor(hi, 1, 64);
    if (active) {
      codes[e0 / 8] = lo;
      if (half == 0) {
        if constexpr (MB == 5) codes_hi[e0 / 16] = hi;
        exps[e0 / 16] = a > 0.0f ? (uint8_t)(E + 127) : (uint8_t)0;
      }
    }
  }
}

__device__ void pack_row_int8(const WeightView& W, const _Float16* __restrict__ src, int row, float* lds_red) {
  const int k = W.k;
  float a = 0.0f;
  for (int e0 = threadIdx.x * 8; e0 < k; e0 += kPackThreads * 8) {
    const uint4 raw = *reinterpret_cast<const uint4*>(src + e0);
    const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a = fmaxf(a, fabsf(h2f((uint16_t)(rw[i] & 0xFFFFu))));
      a = fmaxf(a, fabsf(h2f((uint16_t)(rw[i] >> 16))));
    }
  }
  a = group_max<64>(a);
  if ((threadIdx.x & 63) == 0) lds_red[threadIdx.x >> 6] = a;
  __syncthreads();
  a = fmaxf(fmaxf(lds_red[0], lds_red[1]), fmaxf(lds_red[2], lds_red[3]));
  const float s = to_f16_f32(a / 127.0f);
  int8_t* codes = reinterpret_cast<int8_t*>(const_cast<uint32_t*>(W.codes)) + (size_t)row * k;
  for (int e0 = threadIdx.x * 8; e0 < k; e0 += kPackThreads * 8) {
    const uint4 raw = *reinterpret_cast<const uint4*>(src + e0);
    const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
    uint32_t out[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = h2f((uint16_t)(i & 1 ? rw[i / 2] >> 16 : rw[i / 2] & 0xFFFFu));
      int q = 0;
      if (s != 0.0f) q = (int)fminf(fmaxf(rne_div(x, s), -127.0f), 127.0f);
      out[i / 4] |= ((uint32_t)q & 0xFFu) << (8 * (i & 3));
    }
    *reinterpret_cast<uint2*>(codes + e0) = make_uint2(out[0], out[1]);
  }
  if (threadIdx.x == 0)
    reinterpret_cast<_Float16*>(const_cast<void*>(W.scales))[row] = (_Float16)s;
}

// Packs the per-group 4-bit zero-points / 2-bit selectors staged in LDS.
__device__ void store_sub_byte_meta(const WeightView& W, int row, const uint8_t* lds_meta, int bits) {
  const int groups = W.k / W.group;
  const int per = 32 / bits;
  const int words = (groups + per - 1) / per;
  uint32_t* aux = reinterpret_cast<uint32_t*>(const_cast<void*>(W.aux)) + (size_t)row * words;
  for (int wi = threadIdx.x; wi < words; wi += kPackThreads) {
    uint32_t v = 0;
    for (int j = 0; j < per; ++j) {
      const int gi = wi * per + j;
      if (gi < groups) v |= (uint32_t)lds_meta[gi] << (bits * j);
    }
    aux[wi] = v;
  }
}

template <int FMT>
__global__ void __launch_bounds__(kPackThreads) pack_kernel(WeightView W, const _Float16* __restrict__ src,
                                                             int nclip) {
  __shared__ uint8_t lds_meta[kMaxK / 32];
  __shared__ float lds_red[4];
  const int row = blockIdx.x;
  const _Float16* rsrc = src + (size_t)row * W.k;
  if constexpr (FMT == Q_INT8) {
    pack_row_int8(W, rsrc, row, lds_red);
  } else if constexpr (FMT == Q_BFP6) {
    pack_row_block<5>(W, rsrc, row);
  } else if constexpr (FMT == Q_BFP4) {
    pack_row_block<3>(W, rsrc, row);
  } else {
    switch (W.group) {
      case 32: pack_row_grouped<FMT, 4>(W, rsrc, row, lds_meta, nclip); break;
      case 64: pack_row_grouped<FMT, 8>(W, rsrc, row, lds_meta, nclip); break;
      case 128: pack_row_grouped<FMT, 16>(W, rsrc, row, lds_meta, nclip); break;
      default: pack_row_grouped<FMT, 32>(W, rsrc, row, lds_meta, nclip); break;
    }
    if constexpr (FMT == Q_INT4_ASYM || is_razer(FMT)) {
      __syncthreads();
      store_sub_byte_meta(W, row, lds_meta, FMT == Q_INT4_ASYM ? 4 : 2);
    }
  }
}

}  // namespace

// Zero the pad bytes at the end of each packed buffer (fewer than
// kBufferPad each), so the buffers are a deterministic function of W.
struct PadJob {
  uint8_t* p[4];
  uint32_t from[4], to[4];
};

__global__ void zero_pad_kernel(PadJob job) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t at = job.from[i] + threadIdx.x;
    if (job.p[i] && at < job.to[i]) job.p[i][at] = 0;
  }
}

hipError_t launch_pack(const WeightView& w, const _Float16* src, hipStream_t s, int clip_candidates) {
  PadJob job;
  const void* bufs[4] = {w.codes, w.codes_hi, w.scales, w.aux};
  bool any = false;
  for (int i = 0; i < 4; ++i) {
    const size_t logical = packed_bytes_logical(w.fmt, w.n, w.k, w.group, i);
    const size_t padded = buffer_bytes(w.fmt, w.n, w.k, w.group, i);
    job.p[i] = (logical < padded && bufs[i]) ? static_cast<uint8_t*>(const_cast<void*>(bufs[i])) : nullptr;
    job.from[i] = (uint32_t)logical;
    job.to[i] = (uint32_t)padded;
    any = any || job.p[i];
  }
  if (any) zero_pad_kernel<<<1, (int)kBufferPad, 0, s>>>(job);
  const dim3 grid(w.n), block(kPackThreads);
  switch (w.fmt) {
    case Q_INT4_ASYM: pack_kernel<Q_INT4_ASYM><<<grid, block, 0, s>>>(w, src, clip_candidates); break;
    case Q_FP4_E2M1: pack_kernel<Q_FP4_E2M1><<<grid, block, 0, s>>>(w, src, clip_candidates); break;
    case Q_FP4_RAZER: pack_kernel<Q_FP4_RAZER><<<grid, block, 0, s>>>(w, src, clip_candidates); break;
    case Q_FP4_AFPQ: pack_kernel<Q_FP4_AFPQ><<<grid, block, 0, s>>>(w, src, clip_candidates); break;
    case Q_BFP6: pack_kernel<Q_BFP6><<<grid, block, 0, s>>>(w, src, clip_candidates); break;
    case Q_BFP4: pack_kernel<Q_BFP4><<<grid, block, 0, s>>>(w, src, clip_candidates); break;
    case Q_INT8: pack_kernel<Q_INT8><<<grid, block, 0, s>>>(w, src, clip_candidates); break;
    case Q_FP3_RAZER: pack_kernel<Q_FP3_RAZER><<<grid, block, 0, s>>>(w, src, clip_candidates); break;
    case Q_FP3_AFPQ: pack_kernel<Q_FP3_AFPQ><<<grid, block, 0, s>>>(w, src, clip_candidates); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qg
