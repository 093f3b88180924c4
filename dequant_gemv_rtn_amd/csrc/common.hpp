// Device-side building blocks shared by the pack, GEMV and MFMA kernels:
// vector types, the packed-weight view, and the per-format code decoders.
//
// Decoders turn one 32-bit word of packed codes into fp16 pairs with pure bit
// manipulation (plus the gfx950 FP4 conversion for the E2M1 family).  They
// return pairs in a format-specific element order; the activation registers
// or LDS tiles are permuted the same way once, so the dot products need no
// shuffles (a K-reduction does not care about order).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qgemv.h"

namespace qg {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

// Packed weights as the kernels see them (all device pointers).
struct WeightView {
  int fmt, n, k, group;
  const uint32_t* codes;
  const uint32_t* codes_hi;
  const void* scales;
  const void* aux;
};

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

__device__ __forceinline__ float h2f(uint16_t bits) {
  return (float)__builtin_bit_cast(_Float16, bits);
}

// Element-pair orders produced by the decoders, for 8 consecutive elements
// e0..e7 of one code word (4-bit formats) or 4 elements of one int8 word:
//   kPairAdjacent: (e0,e1) (e2,e3) (e4,e5) (e6,e7)   -- FP4 conversion
//   kPairStride4:  (e0,e4) (e1,e5) (e2,e6) (e3,e7)   -- nibble magic numbers
//   kPairStride2:  (e0,e2) (e1,e3)                   -- byte magic numbers
enum PairOrder { kPairAdjacent = 0, kPairStride4 = 1, kPairStride2 = 2 };

template <int FMT>
struct FmtTraits;
template <> struct FmtTraits<Q_INT4_ASYM> { static constexpr int order = kPairStride4; static constexpr int chunk_bytes = 16; };
template <> struct FmtTraits<Q_FP4_E2M1>  { static constexpr int order = kPairAdjacent; static constexpr int chunk_bytes = 16; };
template <> struct FmtTraits<Q_FP4_RAZER> { static constexpr int order = kPairAdjacent; static constexpr int chunk_bytes = 16; };
template <> struct FmtTraits<Q_FP4_AFPQ>  { static constexpr int order = kPairAdjacent; static constexpr int chunk_bytes = 16; };
template <> struct FmtTraits<Q_BFP6>      { static constexpr int order = kPairStride4; static constexpr int chunk_bytes = 16; };
template <> struct FmtTraits<Q_BFP4>      { static constexpr int order = kPairStride4; static constexpr int chunk_bytes = 16; };
template <> struct FmtTraits<Q_INT8>      { static constexpr int order = kPairStride2; static constexpr int chunk_bytes = 32; };
// 3-bit formats: 12 bytes per 32-element piece, expanded to E2M1 code words
// (expand_fp3) and then decoded like their 4-bit counterparts
template <> struct FmtTraits<Q_FP3_RAZER> { static constexpr int order = kPairAdjacent; static constexpr int chunk_bytes = 12; };
template <> struct FmtTraits<Q_FP3_AFPQ>  { static constexpr int order = kPairAdjacent; static constexpr int chunk_bytes = 12; };

// Host and device: whether a format stores 3-bit codes.
__host__ __device__ constexpr bool is_fp3(int fmt) { return fmt == Q_FP3_RAZER || fmt == Q_FP3_AFPQ; }
// The RaZeR family (a remapped -0 code with a per-group special value) and
// the AFPQ family (separate positive and negative scales).
__host__ __device__ constexpr bool is_razer(int fmt) { return fmt == Q_FP4_RAZER || fmt == Q_FP3_RAZER; }
__host__ __device__ constexpr bool is_afpq(int fmt) { return fmt == Q_FP4_AFPQ || fmt == Q_FP3_AFPQ; }

// Rearrange 32 activations held as 16 natural pairs (2i, 2i+1) into the pair
// order a decoder emits.  `nat` and `out` are 16 words each.
template <int ORDER>
__device__ __forceinline__ void pair_activations(const uint32_t* nat, uint32_t* out) {
  if constexpr (ORDER == kPairAdjacent) {
#pragma unroll
    for (int i = 0; i < 16; ++i) out[i] = nat[i];
  } else if constexpr (ORDER == kPairStride4) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t n0 = nat[4 * w + 0], n1 = nat[4 * w + 1];
      const uint32_t n2 = nat[4 * w + 2], n3 = nat[4 * w + 3];
      out[4 * w + 0] = (n0 & 0xFFFFu) | (n2 << 16);          // (e0, e4)
      out[4 * w + 1] = (n0 >> 16) | (n2 & 0xFFFF0000u);      // (e1, e5)
      out[4 * w + 2] = (n1 & 0xFFFFu) | (n3 << 16);          // (e2, e6)
      out[4 * w + 3] = (n1 >> 16) | (n3 & 0xFFFF0000u);      // (e3, e7)
    }
  } else {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint32_t n0 = nat[2 * w + 0], n1 = nat[2 * w + 1];
      out[2 * w + 0] = (n0 & 0xFFFFu) | (n1 << 16);          // (e0, e2)
      out[2 * w + 1] = (n0 >> 16) | (n1 & 0xFFFF0000u);      // (e1, e3)
    }
  }
}

// Permute one 8-element activation group (4 natural pairs, as loaded) into
// the pair order a decoder emits; every MFMA path uses it on its activations.
template <int ORDER>
__device__ __forceinline__ uint4 permute8(uint4 v) {
  if constexpr (ORDER == kPairAdjacent) {
    return v;
  } else if constexpr (ORDER == kPairStride4) {
    return make_uint4((v.x & 0xFFFFu) | (v.z << 16), (v.x >> 16) | (v.z & 0xFFFF0000u),
                      (v.y & 0xFFFFu) | (v.w << 16), (v.y >> 16) | (v.w & 0xFFFF0000u));
  } else {
    return make_uint4((v.x & 0xFFFFu) | (v.y << 16), (v.x >> 16) | (v.y & 0xFFFF0000u),
                      (v.z & 0xFFFFu) | (v.w << 16), (v.z >> 16) | (v.w & 0xFFFF0000u));
  }
}

__device__ __forceinline__ h8 make_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint4 u = make_uint4(a, b, c, d);
  return __builtin_bit_cast(h8, u);
}

// ---- decoders --------------------------------------------------------------

// E2M1 codes of byte `sel` of w -> (low nibble, high nibble) as fp16, unit scale.
template <int SEL>
__device__ __forceinline__ h2 fp4_pair(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}

// Unsigned nibbles j and j+4 of w as fp16 (1024 + nibble): the 4-bit field is
// placed in the low mantissa bits of an fp16 whose exponent encodes 1024.
template <int J>
__device__ __forceinline__ uint32_t nibble_magic(uint32_t w) {
  return ((w >> (4 * J)) & 0x000F000Fu) | 0x64006400u;
}

// bfp6: 6-bit offset-binary field (low 4 bits from w, top 2 bits from hi at
// the positions of the codes_hi layout) of elements j and j+4, as 1024 + u.
// `hsh` is 8 * (word index within the 16-element block pair).
template <int J>
__device__ __forceinline__ uint32_t six_bit_magic(uint32_t w, uint32_t hi, int hsh) {
  const uint32_t top = ((hi >> (hsh + 2 * J)) & 0x00030003u) << 4;
  return ((w >> (4 * J)) & 0x000F000Fu) | top | 0x64006400u;
}

// int8: bytes (b0, b2) and (b1, b3) of u (already XOR 0x80) as 1024 + byte.
__device__ __forceinline__ uint32_t byte_magic_lo(uint32_t u) { return (u & 0x00FF00FFu) | 0x64006400u; }
__device__ __forceinline__ uint32_t byte_magic_hi(uint32_t u) { return ((u >> 8) & 0x00FF00FFu) | 0x64006400u; }

// (a & b) | c in one instruction (v_and_or_b32 with every operand in a
// register; the compiler otherwise splits it when both constants are literals).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// a & b & c in one instruction (v_bitop3_b32 with truth table 0x80: the
// output bit is set only when all three input bits are set).
__device__ __forceinline__ uint32_t and3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x80);
}

// For each nibble equal to 0b1000 (RaZeR's remapped negative zero), the E2M1
// code 0b0010 (value 1.0); every other nibble becomes 0.  `m8` holds
// 0x88888888 in a register.  8 - (n & 7) has bit 3 set exactly when the low
// three bits of n are zero (no borrow crosses a nibble).
__device__ __forceinline__ uint32_t special_mask(uint32_t w, uint32_t m8) {
  const uint32_t low3_zero = 0x88888888u - (w & 0x77777777u);
  return and3(low3_zero, w, m8) >> 2;
}

__device__ __forceinline__ float razer_special(int sel) {
  // selector 0..3 -> +5, -5, +8, -8
  const float mag = (sel & 2) ? 8.0f : 5.0f;
  return (sel & 1) ? -mag : mag;
}

// The special value of a RaZeR-family format: 4-bit selector 0..3 -> +5, -5,
// +8, -8; 3-bit -> +3, -3, +8, -8.
template <int FMT>
__device__ __forceinline__ float razer_special_of(int sel) {
  const float mag = (sel & 2) ? 8.0f : (FMT == Q_FP3_RAZER ? 3.0f : 5.0f);
  return (sel & 1) ? -mag : mag;
}

// One 3-bit piece (words p0, p1 and the sign word sg; 32 codes) as the four
// E2M1 code words of its elements 8q .. 8q+7 (q = 0..3): code s<<2 | i
// becomes s<<3 | i<<1, the E2M1 code of the same magnitude {0, 1, 2, 4}.
__device__ __forceinline__ void expand_fp3(uint32_t p0, uint32_t p1, uint32_t sg, uint32_t* out) {
  uint32_t m6 = 0x66666666u, m8 = 0x88888888u;
  asm("" : "+v"(m6), "+v"(m8));
  out[0] = (p0 & m6) | (sg & m8);
  out[1] = (__builtin_amdgcn_alignbit(p0, p0, 2) & m6) | ((sg << 1) & m8);
  out[2] = (p1 & m6) | ((sg << 2) & m8);
  out[3] = (__builtin_amdgcn_alignbit(p1, p1, 2) & m6) | ((sg << 3) & m8);
}

// ---- buffer resources -----------------------------------------------------------

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Raw (untyped) buffer resource over `bytes` bytes at `base`.  Loads take a
// per-lane 32-bit offset plus a wave-uniform scalar offset; loads past the
// end return zeros instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// ---- workgroup barrier -------------------------------------------------------

// Barrier that orders LDS traffic only.  __syncthreads() also carries a
// workgroup release fence, which waits for every outstanding global load of
// the wave (vmcnt(0)) and so drains the prefetched weight loads the GEMV
// kernels keep in flight across tiles.  Here the wave waits for its own LDS
// (and scalar) operations, then meets the others at s_barrier; the memory
// clobber keeps the compiler from moving memory accesses across it.  Use it
// only where the barrier guards LDS data.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---- wave-level reductions ---------------------------------------------------

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Batch tile `bt` and row group `rg` (first row tile; the group then strides
// by grid_rows) of this workgroup.  The workgroups of one row group -- one
// per batch tile, all reading the same weights -- get IDs that are equal
// modulo 8: workgroups are dealt round-robin to the 8 XCDs, so these land on
// one XCD, launch close together and share its L2.  Needs grid_rows to be a
// multiple of 8 (else the IDs are split plainly).
__device__ __forceinline__ void batch_tile_of(int nbt, int grid_rows, int& bt, int& rg) {
  const int id = (int)blockIdx.x;
  if (nbt > 1 && grid_rows % 8 == 0) {
    const int xcd = id & 7, slot = id >> 3;
    bt = slot % nbt;
    rg = (slot / nbt) * 8 + xcd;
  } else {
    bt = id % nbt;
    rg = id / nbt;
  }
}

}  // namespace qg
