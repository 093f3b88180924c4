// Decode attention over a KV cache quantized with the FP4 formats (E2M1 and
// RaZeR, one weight-style row per cached vector, groups along head_dim).
//
// One new token per sequence: o[b, h] = softmax_t(scale <q[b, h], K[b, kv, t]>)
// weighted sum of V[b, kv, t], kv = h / (Hq / Hkv).  Split over the sequence:
// attn_split_kernel takes one (sequence, KV head, query-head group, token
// range) per workgroup and writes the range's max score, weight sum and
// weighted value sum to the workspace; attn_combine_kernel rescales and adds
// the ranges and rounds once to fp16.
//
// Inside a workgroup (4 waves):
// * scores: a key row is 64 bytes of codes; four lanes take 16 bytes (32
//   elements) each, so one 16-byte load per lane covers 16 rows.  Decode as
//   in the weight kernels (RaZeR: the special value folded into the fp16
//   operand, exactly).  With one group per row (128) the products are four
//   MFMAs per 16 rows, query heads as A and keys as B, times the row scale;
//   with smaller groups v_dot2 against the query slice, times the group
//   scale, and a two-step reduction inside each four-lane group;
// * softmax over the range through LDS (max, exp, sum);
// * lane reductions inside a row of 16 lanes are DPP row operations (an
//   LDS-routed swizzle costs a round trip through the LDS pipe each);
// * both passes keep loads in flight in register rings; the workgroup's
//   barriers wait for LDS only (a __syncthreads would also wait for every
//   load in flight);
// * values, one group per row: on the matrix cores.  32-token blocks are
//   decoded exactly to fp16 into an LDS tile; transposing LDS reads
//   (ds_read_b64_tr_b16) give the MFMA its token-by-column operand, and the
//   softmax weights times the row scales, shifted by a power of two and
//   split into an fp16 hi + lo pair, are the other;
// * values, smaller groups: eight lanes per row, two code words (16
//   elements) each, so the weighted sum needs no reduction until the end:
//   fp32 sums per lane, then three cross-lane steps and one pass through LDS
//   over the waves.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace qg {
namespace {

constexpr int kHeadDim = 128;     // elements per cached vector
constexpr int kRowBytes = 64;     // 4-bit codes of one vector
constexpr int kAttnWaves = 4;
constexpr int kMaxSplitLen = 1024;

struct AttnGeom {
  int batch, q_heads, kv_heads, max_len;
  int gq;           // query heads per KV head
  int head_groups;  // workgroups per KV head (gq / heads per workgroup)
  int split_len, splits;
  int gshift, groups;  // log2(group), groups per vector
  float scale;
  uint32_t codes_bytes, scales_bytes, aux_bytes, q_bytes;
};

template <int FMT>
__device__ __forceinline__ void decode_word(uint32_t w, h2 special, uint32_t* out) {
  const h2 d[4] = {fp4_pair<0>(w), fp4_pair<1>(w), fp4_pair<2>(w), fp4_pair<3>(w)};
  if constexpr (FMT == Q_FP4_RAZER) {
    // code 8 decodes to -0 and its mask element to 1: -0 + v * 1 = v, every
    // other element x + v * 0 = x, exactly
    uint32_t m8 = 0x88888888u;
    asm("" : "+v"(m8));
    const uint32_t sm = special_mask(w, m8);
    out[0] = as_u32(fp4_pair<0>(sm) * special + d[0]);
    out[1] = as_u32(fp4_pair<1>(sm) * special + d[1]);
    out[2] = as_u32(fp4_pair<2>(sm) * special + d[2]);
    out[3] = as_u32(fp4_pair<3>(sm) * special + d[3]);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = as_u32(d[j]);
  }
}

// Raw metadata of group grp of cache row `row`: the fp16 scale bits and the
// RaZeR selector word; rows that are not valid read as 0 (scale 0).
struct RowMeta {
  uint32_t scale_bits, sel_word;
};

template <int FMT>
__device__ __forceinline__ RowMeta load_row_meta(const AttnGeom& g, __amdgpu_buffer_rsrc_t srs,
                                                 __amdgpu_buffer_rsrc_t ars, uint32_t row, int grp, bool valid) {
  RowMeta m;
  const uint32_t soff = valid ? (row * (uint32_t)g.groups + (uint32_t)grp) * 2u : 0xFFFFFF00u;
  m.scale_bits = __builtin_amdgcn_raw_buffer_load_b16(srs, soff, 0, 0);
  m.sel_word = 0;
  if constexpr (FMT == Q_FP4_RAZER) {
    // selectors: 2 bits per group, ceil(groups / 16) words per row
    const uint32_t words = (uint32_t)(g.groups + 15) / 16u;
    const uint32_t aoff = valid ? (row * words + (uint32_t)(grp >> 4)) * 4u : 0xFFFFFF00u;
    m.sel_word = __builtin_amdgcn_raw_buffer_load_b32(ars, aoff, 0, 0);
  }
  return m;
}

// Scale (fp32) and RaZeR special value (fp16 pair) from raw metadata.
template <int FMT>
__device__ __forceinline__ void decode_row_meta(const RowMeta& m, int grp, float* s, h2* special) {
  *s = h2f((uint16_t)m.scale_bits);
  *special = h2{(_Float16)0.0f, (_Float16)0.0f};
  if constexpr (FMT == Q_FP4_RAZER) {
    const _Float16 v = (_Float16)razer_special((int)((m.sel_word >> (2 * (grp & 15))) & 3u));
    *special = h2{v, v};
  }
}

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// x combined with another lane's x by a DPP row operation (every lane valid)
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kHalfMirror = 0x141;  // lane 7 - i within each half row
constexpr int kRowMirror = 0x140;   // lane 15 - i within each row
constexpr int kRowRor8 = 0x128;     // lane (i + 8) mod 16 within each row: lane ^ 8

// Maximum / sum over the 64 lanes, in every lane: four DPP steps make each
// 16-lane row's total, two swizzles join the rows.
__device__ __forceinline__ float wave_max(float m) {
  m = fmaxf(m, dpp_f32<kQuadXor1>(m));
  m = fmaxf(m, dpp_f32<kQuadXor2>(m));
  m = fmaxf(m, dpp_f32<kHalfMirror>(m));
  m = fmaxf(m, dpp_f32<kRowMirror>(m));
  m = fmaxf(m, __shfl_xor(m, 16, 64));
  return fmaxf(m, __shfl_xor(m, 32, 64));
}
__device__ __forceinline__ float wave_sum(float l) {
  l += dpp_f32<kQuadXor1>(l);
  l += dpp_f32<kQuadXor2>(l);
  l += dpp_f32<kHalfMirror>(l);
  l += dpp_f32<kRowMirror>(l);
  l += __shfl_xor(l, 16, 64);
  return l + __shfl_xor(l, 32, 64);
}

// Key and value loads in flight per wave (register rings).
constexpr int kKeyRing = 4, kValRing = 3;

// MF: scores on the matrix cores (groups of 128, one scale per key row):
// v_mfma_f32_16x16x32_f16 with the query heads as A (16 rows, GH of them
// non-zero) and 16 key rows as B, four MFMAs per 16-token step.  Otherwise
// (groups of 32 and 64, several scales per row) v_dot2 per group.
template <int FMT, int GH, bool MF>
__global__ void __launch_bounds__(64 * kAttnWaves)
attn_split_kernel(WeightView K, WeightView V, const _Float16* __restrict__ q, const int32_t* __restrict__ seq_lens,
                  float* __restrict__ ws, AttnGeom g) {
  __shared__ float sc[kMaxSplitLen][GH];  // scores, then weights
  __shared__ float red[kAttnWaves][GH];
  // value tile of each wave (MF: 32 rows of fp16, rows 4 banks apart); the
  // per-wave weighted values [GH][128] go to part(wave): with MF the start of
  // the wave's own tile, which the wave has finished reading by then, so the
  // workgroup fits three to a CU
  constexpr int kVPitch = kHeadDim + 8;
  __shared__ __attribute__((aligned(16))) _Float16 vt[MF ? kAttnWaves : 1][32][kVPitch];
  __shared__ float part_own[MF ? 1 : kAttnWaves][GH][kHeadDim];
  auto part = [&](int w) -> float* {
    return MF ? reinterpret_cast<float*>(&vt[w][0][0]) : &part_own[w][0][0];
  };

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int split = blockIdx.x;
  const int hg = (int)blockIdx.y % g.head_groups, kv = (int)blockIdx.y / g.head_groups;
  const int b = blockIdx.z;
  const int len = seq_lens ? min(max(seq_lens[b], 0), g.max_len) : g.max_len;
  const int t_begin = split * g.split_len;
  const int t_end = min(t_begin + g.split_len, len);
  const int h0 = kv * g.gq + hg * GH;  // first query head of the workgroup
  const uint32_t row0 = (uint32_t)(b * g.kv_heads + kv) * (uint32_t)g.max_len;

  const __amdgpu_buffer_rsrc_t kcs = make_rsrc(K.codes, g.codes_bytes), vcs = make_rsrc(V.codes, g.codes_bytes);
  const __amdgpu_buffer_rsrc_t kss = make_rsrc(K.scales, g.scales_bytes), vss = make_rsrc(V.scales, g.scales_bytes);
  const __amdgpu_buffer_rsrc_t kas = make_rsrc(K.aux, g.aux_bytes), vas = make_rsrc(V.aux, g.aux_bytes);

  // ---- scores: lane (t, c) takes elements 32c .. 32c + 31 of key row t of
  // the step: t = lane / 4, c = lane % 4 for v_dot2; t = lane % 16,
  // c = lane / 16 for the MFMAs (B operand: column t, k-slots of lane group
  // c), so a step's 16 rows are one contiguous 1 KiB either way
  const int c4 = MF ? lane >> 4 : lane & 3;
  const int tl = MF ? lane & 15 : lane >> 2;
  uint32_t qv[MF ? 1 : GH][16];  // v_dot2: the GH heads' elements 32c .. 32c + 31
  h8 qa[MF ? 4 : 1];             // MFMA A operand m: head lane % 16, elements 32c + 8m .. + 7 (0 past GH)
  {
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(q, g.q_bytes);
    if constexpr (MF) {
      const int h = lane & 15;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t off =
            h < GH ? ((uint32_t)(b * g.q_heads + h0 + h) * kHeadDim + 32u * c4 + 8u * m) * 2u : 0xFFFFFF00u;
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0);
        qa[m] = make_h8(v.x, v.y, v.z, v.w);
      }
    } else {
#pragma unroll
      for (int h = 0; h < GH; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t off = ((uint32_t)(b * g.q_heads + h0 + h) * kHeadDim + 32u * c4 + 8u * i) * 2u;
          const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0);
          qv[h][4 * i] = v.x; qv[h][4 * i + 1] = v.y; qv[h][4 * i + 2] = v.z; qv[h][4 * i + 3] = v.w;
        }
    }
  }
  const int grp_k = (32 * c4) >> g.gshift;
  // key step i covers local tokens 64 i + 16 wave .. + 15, lane's token t_k(i)
  const int nk = g.split_len / (16 * kAttnWaves);
  auto t_k = [&](int i) { return 64 * i + 16 * wave + tl; };
  struct KSlot {
    u32x4 cw;
    RowMeta m;
  };
  auto kload = [&](int i, KSlot& sl) {
    const int tok = t_begin + t_k(i);
    const bool valid = i < nk && tok < t_end;
    const uint32_t row = row0 + (uint32_t)tok;
    sl.cw = __builtin_amdgcn_raw_buffer_load_b128(kcs, valid ? row * kRowBytes + 16u * c4 : 0xFFFFFF00u, 0, 0);
    sl.m = load_row_meta<FMT>(g, kss, kas, row, grp_k, valid);
  };
  auto kuse = [&](int i, const KSlot& sl) {
    const int t = t_k(i);
    const bool valid = t_begin + t < t_end;
    float s;
    h2 special;
    decode_row_meta<FMT>(sl.m, grp_k, &s, &special);
    const uint32_t words[4] = {sl.cw.x, sl.cw.y, sl.cw.z, sl.cw.w};
    if constexpr (MF) {
      // D[head][token]: lanes 0-15 (token = lane) hold heads 0-3 in order
      f4 d4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint32_t d[4];
        decode_word<FMT>(words[m], special, d);
        d4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[m], make_h8(d[0], d[1], d[2], d[3]), d4, 0, 0, 0);
      }
      if (lane < 16) {
#pragma unroll
        for (int h = 0; h < GH; ++h) sc[t][h] = valid ? d4[h] * s * g.scale : -INFINITY;
      }
    } else {
      float dot[GH];
#pragma unroll
      for (int h = 0; h < GH; ++h) dot[h] = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t d[4];
        decode_word<FMT>(words[w], special, d);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int h = 0; h < GH; ++h) dot[h] = __builtin_amdgcn_fdot2(as_h2(d[j]), as_h2(qv[h][4 * w + j]), dot[h], false);
      }
#pragma unroll
      for (int h = 0; h < GH; ++h) {
        float v = dot[h] * s;
        v += dpp_f32<kQuadXor1>(v);  // the four lanes of a key row
        v += dpp_f32<kQuadXor2>(v);
        if (c4 == 0) sc[t][h] = valid ? v * g.scale : -INFINITY;
      }
    }
  };
  KSlot kr[kKeyRing];
  static_for<0, kKeyRing>([&](auto dc) { kload(decltype(dc)::value, kr[decltype(dc)::value]); });
  int ik = 0;
  for (; ik + kKeyRing <= nk; ik += kKeyRing)
    static_for<0, kKeyRing>([&](auto dc) {
      constexpr int d = decltype(dc)::value;
      kuse(ik + d, kr[d]);
      kload(ik + d + kKeyRing, kr[d]);
    });
  static_for<0, kKeyRing>([&](auto dc) {
    constexpr int d = decltype(dc)::value;
    if (ik + d < nk) kuse(ik + d, kr[d]);
  });

  // value geometry (the value pass follows the softmax)
  const int w8 = lane & 7;
  const int grp_v = (16 * w8) >> g.gshift;
  const int nv = g.split_len / (8 * kAttnWaves);
  auto t_v = [&](int i) { return 32 * i + 8 * wave + (lane >> 3); };
  struct VSlot {
    u32x2 cw;
    RowMeta m;
  };
  auto vload = [&](int i, VSlot& sl) {
    const int tok = t_begin + t_v(i);
    const bool valid = i < nv && tok < t_end;
    const uint32_t row = row0 + (uint32_t)tok;
    sl.cw = __builtin_amdgcn_raw_buffer_load_b64(vcs, valid ? row * kRowBytes + 8u * w8 : 0xFFFFFF00u, 0, 0);
    sl.m = load_row_meta<FMT>(g, vss, vas, row, grp_v, valid);
  };
  lds_barrier();

  // ---- softmax over the range
  float mx[GH], sum[GH];
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    float m = -INFINITY;
    for (int t = tid; t < g.split_len; t += 64 * kAttnWaves) m = fmaxf(m, sc[t][h]);
    m = wave_max(m);
    if (lane == 0) red[wave][h] = m;
  }
  lds_barrier();
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    float m = red[0][h];
#pragma unroll
    for (int w = 1; w < kAttnWaves; ++w) m = fmaxf(m, red[w][h]);
    mx[h] = m;
  }
  lds_barrier();  // every wave has read red before it is reused
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    float l = 0.0f;
    for (int t = tid; t < g.split_len; t += 64 * kAttnWaves) {
      const float v = sc[t][h];
      const float e = v == -INFINITY ? 0.0f : __expf(v - mx[h]);
      sc[t][h] = e;
      l += e;
    }
    l = wave_sum(l);
    if (lane == 0) red[wave][h] = l;
  }
  lds_barrier();
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    float l = 0.0f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) l += red[w][h];
    sum[h] = l;
  }

  if constexpr (MF) {
    // ---- values on the matrix cores (one scale per row).  The wave takes
    // 32-token blocks kAttnWaves * i + wave of the range.  Lane (r, hf) =
    // (lane / 2, lane % 2) decodes elements 64 hf .. 64 hf + 63 of the
    // block's row r exactly to fp16 into the wave's LDS tile vt, and turns the
    // row's softmax weights times its scale (times the shift below) into
    // fp16 hi + lo (error about 2^-22 of the product) for heads 2 hf and
    // 2 hf + 1.  Per 16 columns two
    // MFMAs (hi, lo) then take A = weights [head][token] and B = the tile's
    // columns, read with ds_read_b64_tr_b16: in each 16-lane group q, lane
    // 4 j + m reads row 8 q + j (then 8 q + 4 + j), columns 4 m .. 4 m + 3,
    // and lane i of the group receives column i of those four rows.
    __shared__ __attribute__((aligned(16))) _Float16 wt[kAttnWaves][2][GH][32];
    typedef short s4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s4* lds_s4;
    const int r = lane >> 1, hf = lane & 1;
    const int hq = lane & 15, qg = lane >> 4, jr = (lane & 15) >> 2, mc = lane & 3;
    const int nvb = g.split_len / (32 * kAttnWaves);  // blocks per wave (ranges are 128 tokens or more)
    struct VBlk {
      u32x4 c0, c1;
      RowMeta m;
    };
    auto vbload = [&](int i, VBlk& sl) {
      const int tok = t_begin + 32 * (kAttnWaves * i + wave) + r;
      const bool valid = i < nvb && tok < t_end;
      const uint32_t row = row0 + (uint32_t)tok;
      const uint32_t off = row * kRowBytes + 32u * hf;
      sl.c0 = __builtin_amdgcn_raw_buffer_load_b128(vcs, valid ? off : 0xFFFFFF00u, 0, 0);
      sl.c1 = __builtin_amdgcn_raw_buffer_load_b128(vcs, valid ? off + 16u : 0xFFFFFF00u, 0, 0);
      sl.m = load_row_meta<FMT>(g, vss, vas, row, 0, valid);
    };
    // Power-of-two shift 2^k of the weights: the range's largest value scale
    // s_max sets k = 14 - e (s_max in [2^e, 2^(e+1))), so every weight
    // times its scale times 2^k stays below 2^15 -- no fp16 overflow -- and
    // weights down to 2^-38 of s_max stay out of fp16's subnormal range.
    // The sums are multiplied back by 2^-k, exactly.
    __shared__ float smax_w[kAttnWaves];
    float smax = 0.0f;
#pragma unroll
    for (int u = 0; u < kMaxSplitLen / (64 * kAttnWaves); ++u) {
      const int tok = t_begin + tid + 64 * kAttnWaves * u;
      const bool valid = tid + 64 * kAttnWaves * u < g.split_len && tok < t_end;
      const uint32_t soff = valid ? (row0 + (uint32_t)tok) * (uint32_t)g.groups * 2u : 0xFFFFFF00u;
      smax = fmaxf(smax, h2f((uint16_t)__builtin_amdgcn_raw_buffer_load_b16(vss, soff, 0, 0)));
    }
    smax = wave_max(smax);
    if (lane == 0) smax_w[wave] = smax;
    lds_barrier();
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) smax = fmaxf(smax, smax_w[w]);
    const int ke = smax > 0.0f ? 14 - ((int)((__builtin_bit_cast(uint32_t, smax) >> 23) & 255u) - 127) : 0;
    const float wshift = __builtin_bit_cast(float, (uint32_t)(127 + ke) << 23);
    const float wunshift = __builtin_bit_cast(float, (uint32_t)(127 - ke) << 23);
    f4 vacc[kHeadDim / 16];
#pragma unroll
    for (int nb = 0; nb < kHeadDim / 16; ++nb) vacc[nb] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    auto vbuse = [&](int i, const VBlk& sl) {
      const int tl = 32 * (kAttnWaves * i + wave) + r;  // token within the range
      float s;
      h2 special;
      decode_row_meta<FMT>(sl.m, 0, &s, &special);
      const uint32_t words[8] = {sl.c0.x, sl.c0.y, sl.c0.z, sl.c0.w, sl.c1.x, sl.c1.y, sl.c1.z, sl.c1.w};
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        uint32_t d[4];
        decode_word<FMT>(words[w], special, d);
        *reinterpret_cast<u32x4*>(&vt[wave][r][64 * hf + 8 * w]) = u32x4{d[0], d[1], d[2], d[3]};
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int h = 2 * hf + u;
        if (h < GH) {
          const float pw = sc[tl][h] * s * wshift;
          const _Float16 hi = (_Float16)pw;
          wt[wave][0][h][r] = hi;
          wt[wave][1][h][r] = (_Float16)(pw - (float)hi);
        }
      }
      h8 ahi = h8{}, alo = h8{};
      if (hq < GH) {
        ahi = *reinterpret_cast<const h8*>(&wt[wave][0][hq][8 * qg]);
        alo = *reinterpret_cast<const h8*>(&wt[wave][1][hq][8 * qg]);
      }
#pragma unroll
      for (int nb = 0; nb < kHeadDim / 16; ++nb) {
        const s4 ba = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)&vt[wave][8 * qg + jr][16 * nb + 4 * mc]);
        const s4 bb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)&vt[wave][8 * qg + 4 + jr][16 * nb + 4 * mc]);
        const h8 bv = __builtin_bit_cast(h8, u32x4{__builtin_bit_cast(u32x2, ba).x, __builtin_bit_cast(u32x2, ba).y,
                                                   __builtin_bit_cast(u32x2, bb).x, __builtin_bit_cast(u32x2, bb).y});
        vacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bv, vacc[nb], 0, 0, 0);
        vacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bv, vacc[nb], 0, 0, 0);
      }
    };
    VBlk vb[kValRing];
    static_for<0, kValRing>([&](auto dc) { vbload(decltype(dc)::value, vb[decltype(dc)::value]); });
    int ib = 0;
    for (; ib + kValRing <= nvb; ib += kValRing)
      static_for<0, kValRing>([&](auto dc) {
        constexpr int d = decltype(dc)::value;
        vbuse(ib + d, vb[d]);
        vbload(ib + d + kValRing, vb[d]);
      });
    static_for<0, kValRing>([&](auto dc) {
      constexpr int d = decltype(dc)::value;
      if (ib + d < nvb) vbuse(ib + d, vb[d]);
    });
    // D[head][column]: lanes 0-15 hold heads 0-3 (register h), column 16 nb + lane
    if (lane < 16) {
#pragma unroll
      for (int nb = 0; nb < kHeadDim / 16; ++nb)
#pragma unroll
        for (int h = 0; h < GH; ++h) part(wave)[h * kHeadDim + 16 * nb + lane] = vacc[nb][h] * wunshift;
    }
  } else {
    // ---- values: lane (t = lane / 8, w = lane % 8) takes elements 16w .. 16w + 15
    VSlot vr[kValRing];
    static_for<0, kValRing>([&](auto dc) { vload(decltype(dc)::value, vr[decltype(dc)::value]); });
    float acc[GH][16];
  #pragma unroll
    for (int h = 0; h < GH; ++h)
  #pragma unroll
      for (int e = 0; e < 16; ++e) acc[h][e] = 0.0f;
    auto vuse = [&](int i, const VSlot& sl) {
      const int t = t_v(i);
      float s;
      h2 special;
      decode_row_meta<FMT>(sl.m, grp_v, &s, &special);
      uint32_t d[8];
      decode_word<FMT>(sl.cw.x, special, d);
      decode_word<FMT>(sl.cw.y, special, d + 4);
  #pragma unroll
      for (int h = 0; h < GH; ++h) {
        const float ps = sc[t][h] * s;
  #pragma unroll
        for (int j = 0; j < 8; ++j) {
          const h2 p = as_h2(d[j]);
          acc[h][2 * j] += ps * (float)p.x;
          acc[h][2 * j + 1] += ps * (float)p.y;
        }
      }
    };
    int iv = 0;
    for (; iv + kValRing <= nv; iv += kValRing)
      static_for<0, kValRing>([&](auto dc) {
        constexpr int d = decltype(dc)::value;
        vuse(iv + d, vr[d]);
        vload(iv + d + kValRing, vr[d]);
      });
    static_for<0, kValRing>([&](auto dc) {
      constexpr int d = decltype(dc)::value;
      if (iv + d < nv) vuse(iv + d, vr[d]);
    });
  #pragma unroll
    for (int h = 0; h < GH; ++h)
  #pragma unroll
      for (int e = 0; e < 16; ++e) {
        float v = acc[h][e];
        v += dpp_f32<kRowRor8>(v);
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        if (lane < 8) part(wave)[h * kHeadDim + 16 * w8 + e] = v;
      }
  }
  lds_barrier();

  // ---- range result: [max, sum, weighted values] per query head
  for (int i = tid; i < GH * kHeadDim; i += 64 * kAttnWaves) {
    const int h = i / kHeadDim, d = i % kHeadDim;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) v += part(w)[h * kHeadDim + d];
    float* dst = ws + ((size_t)(b * g.q_heads + h0 + h) * g.splits + split) * (kHeadDim + 2);
    dst[2 + d] = v;
    if (d == 0) {
      dst[0] = mx[h];
      dst[1] = sum[h];
    }
  }
}

// o[b, h, d] = sum_s e^(m_s - M) a_s[d] / sum_s e^(m_s - M) l_s over the
// ranges s of the sequence (M the largest m_s); 0 for an empty sequence.
// Every load that does not depend on another goes out at once: thread d's
// value of each of the first kCombinePre ranges, and the maxima and sums of
// ranges d, d + 128, ... (at most 8 each); loads past the range count read
// zeros through the buffer range check (issuing each under its own branch
// was slower: 11.5 against 10.9 us at b = 1, 4096 tokens).  The range weights are then found
// once in LDS, and thread d adds the ranges' values for its d in range
// order (ranges past the first kCombinePre are loaded in that loop).
constexpr int kMaxSplits = 1024;
constexpr int kCombinePre = 32;

__global__ void __launch_bounds__(kHeadDim)
attn_combine_kernel(const float* __restrict__ ws, _Float16* __restrict__ out, AttnGeom g) {
  __shared__ float wgt[kMaxSplits];
  __shared__ float red[kHeadDim / 64][2];
  constexpr uint32_t RS = kHeadDim + 2;  // floats per range: max, sum, values
  constexpr uint32_t kNoLoad = 0xFFFFFF00u;
  const int bh = blockIdx.x, d = threadIdx.x, lane = d & 63, wave = d >> 6;
  const int ns = g.splits;
  const __amdgpu_buffer_rsrc_t srs =
      make_rsrc(ws + (size_t)bh * (size_t)ns * RS, (uint32_t)ns * RS * 4u);
  auto ld = [&](int s, uint32_t e) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                         srs, s < ns ? ((uint32_t)s * RS + e) * 4u : kNoLoad, 0, 0));
  };
  // (two uniform tests skip the second half of the prefetch and the ranges
  // past 128 when there are none)
  float v[kCombinePre];
#pragma unroll
  for (int j = 0; j < kCombinePre / 2; ++j) v[j] = ld(j, 2u + (uint32_t)d);
  if (ns > kCombinePre / 2) {
#pragma unroll
    for (int j = kCombinePre / 2; j < kCombinePre; ++j) v[j] = ld(j, 2u + (uint32_t)d);
  } else {
#pragma unroll
    for (int j = kCombinePre / 2; j < kCombinePre; ++j) v[j] = 0.0f;
  }
  float mo[kMaxSplits / kHeadDim], lo[kMaxSplits / kHeadDim];
  mo[0] = ld(d, 0u);
  lo[0] = ld(d, 1u);
#pragma unroll
  for (int i = 1; i < kMaxSplits / kHeadDim; ++i) mo[i] = lo[i] = 0.0f;
  if (ns > kHeadDim) {
#pragma unroll
    for (int i = 1; i < kMaxSplits / kHeadDim; ++i) {
      mo[i] = ld(d + kHeadDim * i, 0u);
      lo[i] = ld(d + kHeadDim * i, 1u);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMaxSplits / kHeadDim; ++i)
    if (d + kHeadDim * i < ns) M = fmaxf(M, mo[i]);
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  if (lane == 0) red[wave][0] = M;
  __syncthreads();
  M = fmaxf(red[0][0], red[1][0]);
  float L = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxSplits / kHeadDim; ++i) {
    const int s = d + kHeadDim * i;
    if (s < ns) {
      const float w = (mo[i] == -INFINITY || M == -INFINITY) ? 0.0f : __expf(mo[i] - M);
      wgt[s] = w;
      L += w * lo[i];
    }
  }
  for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off, 64);
  if (lane == 0) red[wave][1] = L;
  __syncthreads();
  L = red[0][1] + red[1][1];
  float o = 0.0f;
#pragma unroll
  for (int j = 0; j < kCombinePre; ++j)
    if (j < ns) o += wgt[j] * v[j];
#pragma unroll 8
  for (int s = kCombinePre; s < ns; ++s) o += wgt[s] * ld(s, 2u + (uint32_t)d);
  out[(size_t)bh * kHeadDim + d] = (_Float16)(L > 0.0f ? o / L : 0.0f);
}

typedef void (*AttnKernelFn)(WeightView, WeightView, const _Float16*, const int32_t*, float*, AttnGeom);

template <int FMT>
AttnKernelFn pick_attn(int gh, bool mf) {
  switch (gh) {
    case 1: return mf ? attn_split_kernel<FMT, 1, true> : attn_split_kernel<FMT, 1, false>;
    case 2: return mf ? attn_split_kernel<FMT, 2, true> : attn_split_kernel<FMT, 2, false>;
    default: return mf ? attn_split_kernel<FMT, 4, true> : attn_split_kernel<FMT, 4, false>;
  }
}

// Heads per workgroup (1, 2 or 4, dividing the query-head group) and the
// tokens per range: a power of two from 128 to 1024 that gives about 512
// workgroups.  Depends on the shape only.
void attn_plan(int batch, int q_heads, int kv_heads, int max_len, AttnGeom& g) {
  g.gq = q_heads / kv_heads;
  const int gh = g.gq % 4 == 0 ? 4 : g.gq % 2 == 0 ? 2 : 1;
  g.head_groups = g.gq / gh;
  const long units = (long)batch * kv_heads * g.head_groups;
  const long want = (512 + units - 1) / units;  // ranges per sequence
  long per = (max_len + want - 1) / want;
  int split = 128;
  while (split < per && split < kMaxSplitLen) split *= 2;
  g.split_len = split;
  g.splits = (max_len + split - 1) / split;
}

}  // namespace

size_t attn_workspace_bytes(int batch, int q_heads, int kv_heads, int max_len) {
  AttnGeom g;
  attn_plan(batch, q_heads, kv_heads, max_len, g);
  return (size_t)batch * q_heads * g.splits * (kHeadDim + 2) * sizeof(float);
}

hipError_t launch_attn_decode(const WeightView& k, const WeightView& v, const _Float16* q, const int32_t* seq_lens,
                              _Float16* out, int batch, int q_heads, int kv_heads, int max_len, float scale, void* ws,
                              hipStream_t s) {
  AttnGeom g;
  g.batch = batch;
  g.q_heads = q_heads;
  g.kv_heads = kv_heads;
  g.max_len = max_len;
  attn_plan(batch, q_heads, kv_heads, max_len, g);
  g.gshift = ilog2(k.group);
  g.groups = kHeadDim / k.group;
  g.scale = scale;
  g.codes_bytes = (uint32_t)buffer_bytes(k.fmt, k.n, k.k, k.group, Q_BUF_CODES);
  g.scales_bytes = (uint32_t)buffer_bytes(k.fmt, k.n, k.k, k.group, Q_BUF_SCALES);
  g.aux_bytes = (uint32_t)buffer_bytes(k.fmt, k.n, k.k, k.group, Q_BUF_AUX);
  g.q_bytes = (uint32_t)((size_t)batch * q_heads * kHeadDim * 2);
  const int gh = g.gq / g.head_groups;
  // scores on the matrix cores for one scale per key row (QGEMV_ATTN_MFMA=0 turns it off, for tuning)
  const bool mf = k.group == kHeadDim && tuning(kTuneAttnMfma, 1) != 0;
  AttnKernelFn fn = k.fmt == Q_FP4_RAZER ? pick_attn<Q_FP4_RAZER>(gh, mf) : pick_attn<Q_FP4_E2M1>(gh, mf);
  float* wsf = static_cast<float*>(ws);
  hipLaunchKernelGGL(fn, dim3(g.splits, kv_heads * g.head_groups, batch), dim3(64 * kAttnWaves), 0, s, k, v, q,
                     seq_lens, wsf, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(batch * q_heads), dim3(kHeadDim), 0, s, wsf, out, g);
  return hipGetLastError();
}

}  // namespace qg
