// Vector-ALU fused-dequantization GEMV for 1 <= b <= 8 activation rows.
//
// y[b][n] = sum_k W_deq[n][k] x[b][k].  The weight stream is the only large
// operand, so the kernel is laid out for HBM: lane l of a wave reads 16-byte
// code pieces l, l+64, ... of a row, so every wave load is 1 KiB contiguous;
// several rows' pieces are issued before any is consumed to keep bytes in
// flight.  Each lane keeps its fixed K-slice of x in registers for all rows
// it visits (x is read once per workgroup), paired in the order the decoder
// emits so the inner loop is decode + v_dot2 (fp16 products, fp32 sums).
//
// Scales are applied exactly once per 32-element piece in fp32:
//   int4_asym  s * (sum q x - z * sum x)      (q from a magic-number decode)
//   fp4_e2m1   s * sum M x                     (hardware FP4 -> fp16 convert)
//   fp4_razer  s * (sum M x + v * sum_{code 8} x)
//   fp4_afpq   s+ * P - s- * Q with P, Q from a signed and a magnitude dot
//   bfp6/bfp4  2^(E - Mb + 1) * sum m x per block of 16
//   int8       s_row * sum q x
// so, apart from fp32 summation order, the result is the exact product.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "common.hpp"
#include "internal.hpp"
#include "valu_dot.hpp"

namespace qg {
namespace {

constexpr int kMaxWaves = 8;

// Per-launch layout constants: byte sizes of each buffer and of one row of it.
struct Geometry {
  int pieces;           // 32-element pieces per row (k / 32)
  int gshift;           // log2(group), 4-bit group formats
  uint32_t codes_row;   // bytes per row of codes
  uint32_t hi_row;      // bytes per row of the bfp6 high plane
  uint32_t scales_row;  // bytes per row of scales
  uint32_t aux_row;     // bytes per row of zero-points / selectors / exponents
  uint32_t codes_bytes, hi_bytes, scales_bytes, aux_bytes;
  int ksw;              // waves that split one row's K (1..8); when 1, the
                        // workgroup's waves walk rows independently
};

// Per-lane, loop-invariant byte offsets of a piece inside one row of each
// buffer, plus the bit position of its zero-point / selector.
struct PieceOffsets {
  uint32_t code, hi, scale, aux;
  uint32_t shift;
};

template <int FMT>
__device__ __forceinline__ PieceOffsets piece_offsets(const Geometry& g, int pc) {
  PieceOffsets o;
  o.code = (uint32_t)pc * (uint32_t)FmtTraits<FMT>::chunk_bytes;
  o.hi = (uint32_t)pc * 8u;
  o.scale = 0; o.aux = 0; o.shift = 0;
  if constexpr (FMT == Q_BFP6 || FMT == Q_BFP4) {
    o.aux = (uint32_t)pc * 2u;  // two exponent bytes per piece
  } else if constexpr (FMT != Q_INT8) {
    const uint32_t gi = ((uint32_t)pc * 32u) >> g.gshift;
    o.scale = gi * (is_afpq(FMT) ? 4u : 2u);
    if constexpr (FMT == Q_INT4_ASYM) { o.aux = (gi >> 3) * 4u; o.shift = 4u * (gi & 7u); }
    if constexpr (is_razer(FMT)) { o.aux = (gi >> 4) * 4u; o.shift = 2u * (gi & 15u); }
  }
  return o;
}

// Codes and raw metadata of R rows x CPL pieces, held in registers.
template <int FMT, int CPL, int R>
struct Stage {
  static constexpr int CW = FmtTraits<FMT>::chunk_bytes / 4;
  uint32_t cw[R][CPL][CW];
  uint32_t hw[R][CPL][2];
  RawMeta meta[R][CPL];
  uint32_t rs[R];  // int8 row scale bits
};

struct Resources {
  __amdgpu_buffer_rsrc_t codes, hi, scales, aux;
};

// Issue every load of one stage, with no control flow: rows past the end are
// clamped to the last row (their results are never stored) and pieces past
// the end of k to the last piece (their activations are zero, so they add
// nothing).  Row offsets are wave-uniform scalar offsets.
template <int FMT, int CPL, int R>
__device__ __forceinline__ void load_stage(Stage<FMT, CPL, R>& st, const Resources& rs, const Geometry& g,
                                           const PieceOffsets* po, int n, int row0) {
  constexpr int CB = FmtTraits<FMT>::chunk_bytes;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    // wave-uniform: keep it in an SGPR so the row offset is a scalar offset
    const uint32_t row = (uint32_t)__builtin_amdgcn_readfirstlane(min(row0 + r, n - 1));
    const uint32_t so_codes = row * g.codes_row;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      if constexpr (CB == 12) {  // a 3-bit piece: three dwords, expanded at decode
        const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(rs.codes, po[c].code, so_codes, 0);
        st.cw[r][c][0] = v.x; st.cw[r][c][1] = v.y; st.cw[r][c][2] = v.z;
      } else {
#pragma unroll
        for (int i = 0; i < CB / 16; ++i) {
          const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs.codes, po[c].code + 16u * i, so_codes, 0);
          st.cw[r][c][4 * i + 0] = v.x; st.cw[r][c][4 * i + 1] = v.y;
          st.cw[r][c][4 * i + 2] = v.z; st.cw[r][c][4 * i + 3] = v.w;
        }
      }
      if constexpr (FMT == Q_BFP6) {
        const u32x2 h = __builtin_amdgcn_raw_buffer_load_b64(rs.hi, po[c].hi, row * g.hi_row, 0);
        st.hw[r][c][0] = h.x; st.hw[r][c][1] = h.y;
      } else {
        st.hw[r][c][0] = st.hw[r][c][1] = 0;
      }
      RawMeta m{0u, 0u};
      if constexpr (FMT == Q_BFP6 || FMT == Q_BFP4) {
        m.a = __builtin_amdgcn_raw_buffer_load_b16(rs.aux, po[c].aux, row * g.aux_row, 0);
      } else if constexpr (is_afpq(FMT)) {
        m.a = __builtin_amdgcn_raw_buffer_load_b32(rs.scales, po[c].scale, row * g.scales_row, 0);
      } else if constexpr (FMT != Q_INT8) {
        m.a = __builtin_amdgcn_raw_buffer_load_b16(rs.scales, po[c].scale, row * g.scales_row, 0);
        if constexpr (FMT == Q_INT4_ASYM || is_razer(FMT))
          m.b = __builtin_amdgcn_raw_buffer_load_b32(rs.aux, po[c].aux, row * g.aux_row, 0) >> po[c].shift;
      }
      st.meta[r][c] = m;
    }
    st.rs[r] = 0x3C00u;  // 1.0
    if constexpr (FMT == Q_INT8) st.rs[r] = __builtin_amdgcn_raw_buffer_load_b16(rs.scales, 0u, row * 2u, 0);
  }
}

// Decode + dot the staged rows and reduce across the wave.  Lane r * B + b
// receives this wave's total for (row r, batch b) in *t and the row's scale
// in *scale.
template <int FMT, int B, int CPL, int R>
__device__ __forceinline__ void stage_result(const Stage<FMT, CPL, R>& st, const uint32_t (*xr)[B][16],
                                             const float (*xs)[B * 4], const NibbleMasks& nm, float* t,
                                             float* scale) {
  const int lane = threadIdx.x & 15;  // position in the lane's 16-lane row
  const int r = lane / B;
  float acc[R][B];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
#pragma unroll
    for (int bb = 0; bb < B; ++bb) acc[rr][bb] = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      piece_dot<FMT, B>(st.cw[rr][c], st.hw[rr][c], st.meta[rr][c], xr[c], xs[c], acc[rr], nm);
  }
#pragma unroll
  for (int rr = 0; rr < R; ++rr)
#pragma unroll
    for (int bb = 0; bb < B; ++bb) acc[rr][bb] = row_total(acc[rr][bb]);
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    if (rr == r) *scale = h2f((uint16_t)st.rs[rr]);
#pragma unroll
    for (int bb = 0; bb < B; ++bb)
      if (rr * B + bb == lane) *t = acc[rr][bb];
  }
}

// One stage's contribution: for each of the stage's R x B outputs, this
// wave's four scaled 16-lane row sums go to its LDS slot (lane 16 q + j
// writes entry q * R * B + j; stopping at row sums saves the broadcasts and
// the lane read of a full wave total, and the batch end adds the four).  A
// stage past the end of its walker's range (live == false) skips the
// arithmetic and writes zeros.
template <int FMT, int B, int CPL, int R>
__device__ __forceinline__ void finish_stage(const Stage<FMT, CPL, R>& st, const uint32_t (*xr)[B][16],
                                             const float (*xs)[B * 4], const NibbleMasks& nm, bool live,
                                             float* slot) {
  const int lane = threadIdx.x & 63, j = lane & 15;
  float t = 0.0f, scale = 1.0f;
  if (live) stage_result<FMT, B, CPL, R>(st, xr, xs, nm, &t, &scale);
  if (j < R * B) slot[(lane >> 4) * (R * B) + j] = scale * t;
}

// Each row walker owns a strided (or contiguous) set of row blocks and walks
// it with a ring of S register stages: the loads of the next blocks are in
// flight while one block is decoded and reduced.  A walker is g.ksw waves
// splitting the row's K.  For b <= 2 a workgroup holds several walkers,
// which share one copy of the activations staged through LDS (each wave
// holding its own copy costs as much load traffic as the weights of a small
// layer, and shows up directly in the time per call).
template <int FMT, int B, int CPL, int R, int S, bool SHX>
__global__ void __launch_bounds__(64 * kMaxWaves)
gemv_valu_kernel(WeightView W, const _Float16* __restrict__ x, _Float16* __restrict__ y, int nrb, Geometry g,
                 int strided) {
  constexpr int ORDER = FmtTraits<FMT>::order;
  // SHX: the workgroup's row walkers share the activations through LDS
  // (launched only with b <= 2 and b * k * 2 within the XMAX cooperative
  // 16-byte loads per lane of the workgroup).  A compile-time choice: with
  // both paths in one kernel the compiler's waits for the direct loads also
  // land on the shared path and drain the weight stages there.
  static_assert(!SHX || B <= 2, "shared activations are instantiated for b <= 2 only");
  constexpr int XMAX = 4;
  extern __shared__ __attribute__((aligned(16))) uint8_t xlds[];
  const int K = W.k;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nwg = blockDim.x >> 6;
  const int ksw = g.ksw;
  const int kwave = wave % ksw;
  const int walkers = nwg / ksw;
  const uint32_t xbytes = (uint32_t)(B * K * 2);
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, xbytes);

  // Shared activations: every wave of the workgroup loads its share first
  // (the oldest loads in flight, so writing them to LDS waits for nothing
  // else).
  u32x4 xl[XMAX];
  if constexpr (SHX) {
#pragma unroll
    for (int i = 0; i < XMAX; ++i)
      xl[i] = __builtin_amdgcn_raw_buffer_load_b128(xrs, ((uint32_t)(i * nwg * 64) + threadIdx.x) * 16u, 0u, 0);
  }

  int pc[CPL];
  bool valid[CPL];
  PieceOffsets po[CPL];
  Resources rs;
  rs.codes = make_rsrc(W.codes, g.codes_bytes);
  rs.hi = make_rsrc(W.codes_hi, g.hi_bytes);
  rs.scales = make_rsrc(W.scales, g.scales_bytes);
  rs.aux = make_rsrc(W.aux, g.aux_bytes);
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    pc[c] = (kwave * CPL + c) * 64 + lane;
    valid[c] = pc[c] < g.pieces;
    po[c] = piece_offsets<FMT>(g, valid[c] ? pc[c] : g.pieces - 1);
  }

  // Row blocks of this walker: block(i) for i in [0, count).  Strided:
  // walker + i * walkers_total, so that at any moment all walkers stream one
  // contiguous window of the matrix; otherwise a contiguous range each.
  const int vb = (int)blockIdx.x * walkers + wave / ksw;
  const int G = (int)gridDim.x * walkers;
  const int rb_begin = strided ? vb : (int)(((long long)vb * nrb) / G);
  const int count = strided ? max(0, (nrb - vb + G - 1) / G) : (int)(((long long)(vb + 1) * nrb) / G) - rb_begin;
  // trip count shared by the workgroup's walkers (their counts differ by at
  // most one), so that the per-row barriers of ksw > 1 line up.  Strided,
  // the workgroup's first walker has the most row blocks.
  int count_wg = 0;
  if (strided) {
    const int v0 = (int)blockIdx.x * walkers;
    count_wg = v0 < nrb ? (nrb - v0 + G - 1) / G : 0;
  } else {
    for (int w = 0; w < walkers; ++w) {
      const int v = (int)blockIdx.x * walkers + w;
      count_wg = max(count_wg, (int)(((long long)(v + 1) * nrb) / G) - (int)(((long long)v * nrb) / G));
    }
  }
  const int step = strided ? G : 1;
  // Prefetches past the end of this walker's range re-read its own first
  // row block (already in cache; a block shared by every walker would put
  // all of them on one cache channel at once).
  const int dummy = min(rb_begin, nrb - 1) * R;
  // The first S weight stages go out before the activations are staged: a
  // ring of S register stages keeps up to S row blocks in flight per wave.
  Stage<FMT, CPL, R> st[S];
  // (one scheduling barrier per stage: the issue order has to match the
  // steady state, because the wait at the loop head serves the first
  // iteration and every later one)
#pragma unroll
  for (int i = 0; i < S; ++i) {
    load_stage<FMT, CPL, R>(st[i], rs, g, po, W.n, i < count ? (rb_begin + i * step) * R : dummy);
    __builtin_amdgcn_sched_barrier(0);
  }

  if constexpr (SHX) {
#pragma unroll
    for (int i = 0; i < XMAX; ++i) {
      const uint32_t o = ((uint32_t)(i * nwg * 64) + threadIdx.x) * 16u;
      if (o < xbytes) *reinterpret_cast<u32x4*>(xlds + o) = xl[i];
    }
    lds_barrier();
  }

  // This lane's activation slices, paired in decoder order.  Pieces past the
  // end of k read as zeros.
  uint32_t xr[CPL][B][16];
  float xs[CPL][B * 4];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      uint32_t nat[16];
      if constexpr (SHX) {
        const uint32_t xo = (uint32_t)(b * K * 2) + (uint32_t)pc[c] * 64u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x4 v = {0u, 0u, 0u, 0u};
          if (valid[c]) v = *reinterpret_cast<const u32x4*>(xlds + xo + 16u * i);
          nat[4 * i + 0] = v.x; nat[4 * i + 1] = v.y; nat[4 * i + 2] = v.z; nat[4 * i + 3] = v.w;
        }
      } else {
        // the whole offset is per-lane (no scalar part), so an invalid
        // piece's offset stays past the end of the buffer
        const uint32_t xoff = valid[c] ? (uint32_t)(b * K * 2) + (uint32_t)pc[c] * 64u : 0xFFFFFF00u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(xrs, xoff + 16u * i, 0u, 0);
          nat[4 * i + 0] = v.x; nat[4 * i + 1] = v.y; nat[4 * i + 2] = v.z; nat[4 * i + 3] = v.w;
        }
      }
      pair_activations<ORDER>(nat, xr[c][b]);
#pragma unroll
      for (int i = 0; i < 4; ++i) xs[c][4 * b + i] = 0.0f;
      if constexpr (FMT == Q_BFP4) {  // sums of the even and odd elements of each 16-element half
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float se = 0.0f, so = 0.0f;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const h2 v = as_h2(nat[8 * h + i]);
            se += (float)v[0];
            so += (float)v[1];
          }
          xs[c][4 * b + 2 * h + 0] = se;
          xs[c][4 * b + 2 * h + 1] = so;
        }
      }
      // int4: 1024 X_even + 64 X_odd and X_even + X_odd over the piece's
      // natural pairs; int8: 1152 X.  One dot2 per pair and sum (the
      // products with these constants are exact in fp32).
      if constexpr (FMT == Q_INT4_ASYM) {
        const h2 w0 = h2{(_Float16)1024.0f, (_Float16)64.0f}, w1 = h2{(_Float16)1.0f, (_Float16)1.0f};
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s0 = __builtin_amdgcn_fdot2(as_h2(nat[i]), w0, s0, false);
          s1 = __builtin_amdgcn_fdot2(as_h2(nat[i]), w1, s1, false);
        }
        xs[c][4 * b + 0] = s0;
        xs[c][4 * b + 1] = s1;
      }
      if constexpr (FMT == Q_INT8) {
        const h2 w0 = h2{(_Float16)1152.0f, (_Float16)1152.0f};
        float s0 = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) s0 = __builtin_amdgcn_fdot2(as_h2(nat[i]), w0, s0, false);
        xs[c][4 * b + 0] = s0;
      }
    }
  }

  // Resolve the activations before the loop: left to their first use inside
  // it, the wait for them would be merged into the loop head and drain the
  // weight stages on every iteration.
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(xr[c][b][i]));

  // Outputs are reduced and stored in batches of M stages: each stage's
  // per-wave row sums go to an LDS slot, and after every M stages (and at the
  // end) lane (slot, r, b) of each walker's first wave sums the 4 x ksw
  // partials of its output and stores it.  The two slot buffers alternate, so a batch
  // needs one barrier (and none when one wave covers a row).  The store is
  // issued on every iteration, with an offset past the end of y unless it
  // has something to write: a store issued only on some paths makes the
  // compiler's wait for the next stage cover it as well, and every stage
  // would then wait for the previous write to complete.
  constexpr int RB = R * B;
  constexpr int M = (64 / RB) / S * S;  // stages per batch: M * RB <= 64 lanes
  static_assert(M >= S, "a batch holds at least one iteration");
  static_assert(RB <= 16, "a stage's outputs fit one 16-lane row");
  __shared__ float red[2][M][kMaxWaves][4 * RB];
  // b * n * 2 <= 0xFFFFFF00 (checked by the caller), so the dropped-store
  // offset lies past the end of y
  const __amdgpu_buffer_rsrc_t yrs = make_rsrc(y, (uint32_t)B * (uint32_t)W.n * 2u);

  // Loads are issued unconditionally (past the range they re-read this
  // walker's first block, which is in cache), so no wait ever has to cover
  // a load that only some paths issued.  The scheduling barriers keep each
  // refill ahead of the decode it is meant to overlap.
  const NibbleMasks nm = nibble_masks();  // once, outside the loop
  for (int it = 0; it < count_wg; it += S) {
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const int stage = it + i;
      finish_stage<FMT, B, CPL, R>(st[i], xr, xs, nm, stage < count, &red[(stage / M) & 1][stage % M][wave][0]);
      load_stage<FMT, CPL, R>(st[i], rs, g, po, W.n,
                              stage + S < count ? (rb_begin + (stage + S) * step) * R : dummy);
      __builtin_amdgcn_sched_barrier(0);
    }
    float val = 0.0f;
    uint32_t off = 0xFFFFFF00u;
    if ((it + S) % M == 0 || it + S >= count_wg) {  // workgroup-uniform
      if (ksw > 1) lds_barrier();
      const int b0 = it / M * M, buf = (it / M) & 1;
      const int slot = lane / RB, j = lane % RB;
      const int stage = b0 + slot;
      if (kwave == 0 && slot < M && stage < count) {
        float v = 0.0f;
        for (int w = 0; w < ksw; ++w)
#pragma unroll
          for (int q = 0; q < 4; ++q) v += red[buf][slot][wave + w][q * RB + j];
        const int row = (rb_begin + stage * step) * R + j / B;
        if (row < W.n) {
          val = v;
          off = ((uint32_t)(j % B) * (uint32_t)W.n + (uint32_t)row) * 2u;
        }
      }
    }
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)val), yrs, off, 0, 0);
  }
}

// ------------------------------------------------------------- dispatch --

typedef void (*KernelFn)(WeightView, const _Float16*, _Float16*, int, Geometry, int);

template <int FMT, int R, bool SHX>
KernelFn pick_b1(int cpl) {
  switch (cpl) {
    case 1: return gemv_valu_kernel<FMT, 1, 1, R, 2, SHX>;
    case 2: return gemv_valu_kernel<FMT, 1, 2, R, 2, SHX>;
    default: return gemv_valu_kernel<FMT, 1, 4, 1, 2, SHX>;  // more rows per stage would spill
  }
}

template <int FMT>
KernelFn pick_batch(int b, int cpl, int r1, bool shx) {
  switch (b) {
    case 1:
      if (shx) return r1 == 1 ? pick_b1<FMT, 1, true>(cpl) : pick_b1<FMT, 2, true>(cpl);
      return r1 == 1 ? pick_b1<FMT, 1, false>(cpl) : pick_b1<FMT, 2, false>(cpl);
    case 2:
      if (shx) return cpl == 1 ? gemv_valu_kernel<FMT, 2, 1, 2, 2, true> : gemv_valu_kernel<FMT, 2, 2, 2, 2, true>;
      return cpl == 1 ? gemv_valu_kernel<FMT, 2, 1, 2, 2, false> : gemv_valu_kernel<FMT, 2, 2, 2, 2, false>;
    case 3: return gemv_valu_kernel<FMT, 3, 1, 2, 2, false>;
    case 4: return gemv_valu_kernel<FMT, 4, 1, 2, 2, false>;
    case 5: return gemv_valu_kernel<FMT, 5, 1, 2, 2, false>;
    // b >= 6 stages one row at a time: two would spill for int4 and bfp4
    case 6: return gemv_valu_kernel<FMT, 6, 1, 1, 2, false>;
    case 7: return gemv_valu_kernel<FMT, 7, 1, 1, 2, false>;
    default: return gemv_valu_kernel<FMT, 8, 1, 1, 2, false>;
  }
}

}  // namespace

hipError_t launch_gemv_valu(const WeightView& w, const _Float16* x, _Float16* y, int b, hipStream_t s) {
  // Pieces of 32 elements per lane: enough to cover k with at most 8 waves,
  // bounded by the register budget of the b activation slices.
  const int cpl_max = b == 1 ? 4 : (b == 2 ? 2 : 1);
  const int need = (w.k + 2047) / 2048;  // pieces per lane if one wave covered the row
  int cpl = need < cpl_max ? need : cpl_max;
  // rows that need several waves anyway split into 2-piece slices (more
  // waves per row, measured faster: k = 14336 int4 9.9 vs 11.1 us)
  if (need > cpl_max && b == 1) cpl = 2;
  const int cpl_env = tuning(kTuneValuCpl, 0);  // tuning override, capped like the default
  if (cpl_env > 0 && cpl_env < cpl) cpl = cpl_env;
  if (cpl == 3) cpl = 4;
  const int nw = (w.k + 2048 * cpl - 1) / (2048 * cpl);
  if (nw > kMaxWaves) return hipErrorInvalidValue;
  // b = 1: rows per stage (QGEMV_VALU_ROWS, 1 or 2) is tunable; the
  // default, from measurements, is two rows per stage for AFPQ and one for
  // the rest.  Two register stages are in flight (more measured
  // slower: the memory system does best with about 8 MB in flight over the
  // whole chip).
  const int r1_default = is_afpq(w.fmt) ? 2 : 1;
  int r1 = tuning(kTuneValuRows, r1_default);
  if (r1 != 1) r1 = 2;
  if (cpl == 4) r1 = 1;  // the 4-piece kernel stages one row at a time
  const int rows = b == 1 ? r1 : (b >= 6 ? 1 : 2);  // as instantiated in pick_batch
  const int nrb = (w.n + rows - 1) / rows;
  // For b <= 2 several row walkers share a workgroup and one LDS copy of the
  // activations: QGEMV_VALU_SHARE (1, 4 or 8; default 4, measured best) when
  // one wave covers a row, else as many as fit 8 waves.  The kernel's
  // cooperative load covers 4 KiB per wave of the workgroup; without room
  // for b * k * 2 bytes the walkers keep their own copies.
  int walkers = 1;
  if (b <= 2) {
    if (nw == 1) {
      walkers = tuning(kTuneValuShare, 4);
      if (walkers != 1 && walkers != 8) walkers = 4;
    } else {
      walkers = kMaxWaves / nw;
    }
  }
  const uint32_t xbytes = (uint32_t)(b * w.k * 2);
  if (xbytes > (uint32_t)(nw * walkers * 1024 * 4)) walkers = 1;
  const bool shx = walkers > 1;
  KernelFn fn;
  switch (w.fmt) {
    case Q_INT4_ASYM: fn = pick_batch<Q_INT4_ASYM>(b, cpl, r1, shx); break;
    case Q_FP4_E2M1: fn = pick_batch<Q_FP4_E2M1>(b, cpl, r1, shx); break;
    case Q_FP4_RAZER: fn = pick_batch<Q_FP4_RAZER>(b, cpl, r1, shx); break;
    case Q_FP4_AFPQ: fn = pick_batch<Q_FP4_AFPQ>(b, cpl, r1, shx); break;
    case Q_BFP6: fn = pick_batch<Q_BFP6>(b, cpl, r1, shx); break;
    case Q_BFP4: fn = pick_batch<Q_BFP4>(b, cpl, r1, shx); break;
    case Q_INT8: fn = pick_batch<Q_INT8>(b, cpl, r1, shx); break;
    case Q_FP3_RAZER: fn = pick_batch<Q_FP3_RAZER>(b, cpl, r1, shx); break;
    case Q_FP3_AFPQ: fn = pick_batch<Q_FP3_AFPQ>(b, cpl, r1, shx); break;
    default: return hipErrorInvalidValue;
  }
  Geometry g;
  g.pieces = w.k / 32;
  g.gshift = ilog2(w.group);
  const int groups = (w.fmt == Q_BFP6 || w.fmt == Q_BFP4 || w.fmt == Q_INT8) ? 1 : w.k / w.group;
  g.codes_row = (uint32_t)(w.fmt == Q_INT8 ? w.k : is_fp3(w.fmt) ? w.k / 32 * 12 : w.k / 2);
  g.hi_row = (uint32_t)(w.k / 4);
  g.scales_row = (uint32_t)(w.fmt == Q_INT8 ? 2 : groups * (is_afpq(w.fmt) ? 4 : 2));
  g.aux_row = (uint32_t)(w.fmt == Q_INT4_ASYM ? (groups + 7) / 8 * 4
                         : is_razer(w.fmt) ? (groups + 15) / 16 * 4 : w.k / 16);
  const uint64_t n = (uint64_t)w.n;
  g.codes_bytes = (uint32_t)(n * g.codes_row);
  g.hi_bytes = w.fmt == Q_BFP6 ? (uint32_t)(n * g.hi_row) : 0u;
  g.scales_bytes = (w.fmt == Q_BFP6 || w.fmt == Q_BFP4) ? 0u : (uint32_t)(n * g.scales_row);
  g.aux_bytes = (w.fmt == Q_INT4_ASYM || is_razer(w.fmt) || w.fmt == Q_BFP6 || w.fmt == Q_BFP4)
                    ? (uint32_t)(n * g.aux_row) : 0u;
  g.ksw = nw;
  // Persistent workgroups: QGEMV_VALU_WAVES_PER_CU resident waves per compute
  // unit, each row walker striding over the row blocks.  Default 8; 4 for
  // INT8 at b = 1 when one wave covers a row, whose stages carry twice the
  // bytes of the 4-bit formats' (measured on MI355X: Llama-3-8B-shaped q|k|v
  // 6.97 vs 7.39 us, o 5.61 vs 6.24, lm_head 85.5 vs 87.5; the memory system
  // does best with about 8 MB in flight over the chip).
  const int waves_per_cu = tuning(kTuneValuWavesPerCu, (w.fmt == Q_INT8 && b == 1 && nw == 1) ? 4 : 8);
  const int per_wg = nw * walkers;
  int grid = (device_cu_count() * waves_per_cu + per_wg - 1) / per_wg;
  const int grid_max = (nrb + walkers - 1) / walkers;
  if (grid > grid_max) grid = grid_max;
  if (grid < 1) grid = 1;
  const int strided = tuning(kTuneValuStrided, 1);
  hipLaunchKernelGGL(fn, dim3(grid), dim3(64 * per_wg), walkers > 1 ? xbytes : 0u, s, w, x, y, nrb, g, strided);
  return hipGetLastError();
}

}  // namespace qg
