// Decode-stack kernel: every quantized linear of one decode step (b = 1) in
// one persistent launch.
//
// A decode step runs a fixed sequence of matrix-vector products: per decoder
// layer q|k|v, o, gate|up and down, then the output head, with INT4 or INT8
// weights ("Is (Selective) Round-To-Nearest Quantization All You Need?",
// abstract: RTN on fused-dequant kernels, selective up-precision; "A Method
// for Layer Bit-Width Allocation ...", English abstract: the FFN and lm_head
// layers carry the gain).  Launched one kernel per linear, every launch pays
// the ramp of a fresh grid, the first loads' latency and the tail of its
// slowest wave.  Here one grid of resident workgroups walks all the
// matrices in order and keeps its register ring of weight loads running
// across matrix boundaries, so those costs are paid once per step.
//
// Work unit.  A unit is 2 KiB of packed codes of one row: 64 lanes x two
// 16-byte pieces (4-bit formats, 4096 elements) or one 32-byte piece (INT8,
// 2048 elements).  Each lane also loads four metadata dwords (group scales,
// zero-points or selectors of its pieces; the INT8 row scale).  Every unit
// issues the same six vector loads whatever its format, so the compiler's
// waits for the ring are the same on every path.  Rows longer than a unit
// (k = 14336) take several consecutive units of the same wave, which
// accumulates their partial sums in registers.
//
// Stages.  Entries that read the same activations form a stage (q|k|v of a
// layer; gate|up).  Rows of a stage are dealt to the waves of the grid
// round-robin (wave w takes rows w, w + W, ...).  The stage's activations
// are staged once per workgroup in LDS, in the decoder's pair order and laid
// out so that a wave's 16-byte reads are contiguous (no bank conflicts),
// with the per-piece even/odd sums INT4 needs.
//
// Dependent stages (Q_STACK_CHAIN).  In a decoder each stage reads what the
// one before produced (through attention, norms and the activation, which are
// not part of this path).  With the flag, outputs are written through to the
// device coherence point, each workgroup counts its arrival at the end of a
// stage once its waves' stores have completed, and no workgroup reads the
// next stage's activations (with device-coherent loads) before every
// workgroup has arrived.  The weight loads of the next stage are issued
// before that wait: weights do not depend on activations.  Without the flag
// the stages only share the grid.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <vector>

#include "common.hpp"
#include "internal.hpp"
#include "valu_dot.hpp"

namespace qg {
namespace {

constexpr int kStackWaves = 8;                // compute waves per workgroup (plus one producer)
constexpr int kStackRing = 2;                 // units in flight per compute wave
constexpr int kStackPieces = Q_MAX_K / 32;    // staged x pieces (512 x 32 elements)
constexpr uint32_t kPlanMagic = 0x4B415453u;  // "STAK"
constexpr uint32_t kPlanVersion = 2;
constexpr int kMaxGrid = 1024;                // workgroups a launch may use
// Plan layout: StackHeader (64 bytes) | counters | StackStage[nstages] |
// StackLayer[nlayers].  Counters (uint32): the launch's finished workgroups,
// the abort flag, the launch count, the relay's release word, then one
// arrival word per workgroup.  Arrival and release words hold epochs that
// grow across launches (launch count * stages + stage + 1), so nothing has
// to be returned to zero between launches except the finished count.
constexpr int kCtrDone = 0, kCtrAbort = 1, kCtrLaunch = 2, kCtrGo = 3, kCtrArr = 4;
constexpr uint32_t kCtrOff = 64;
static_assert(kCtrOff + 4 * kCtrAbort == Q_STACK_ABORT_OFFSET, "abort word offset");
// poll budget of one stage wait: beyond it the kernel sets the abort flag and
// stops waiting (every wave then runs to the end; results are undefined)
constexpr uint32_t kSpinLimit = 1u << 22;

struct StackHeader {
  uint32_t magic, version;
  int32_t nstages, nlayers;
  uint32_t stages_off, layers_off, ctr_off, total_bytes;
  int32_t pad[8];
};
static_assert(sizeof(StackHeader) == 64, "plan header layout");

struct StackStage {
  const _Float16* x;  // fp16 [k]
  int32_t k, pieces;  // pieces = k / 32
  int32_t rows;       // rows of the stage over all its layers
  int32_t layer_begin, layer_end;
  int32_t units;      // units per row
  int32_t order;      // decoder pair order of the staged activations
  int32_t xsum;       // 1: stage the per-piece even/odd activation sums (INT4)
  int32_t fmt;
  int32_t pad[5];
};
static_assert(sizeof(StackStage) == 64, "plan stage layout");

struct StackLayer {
  const uint32_t* codes;
  const void* scales;
  const void* aux;
  _Float16* y;
  int32_t fmt, n, k, gshift;
  int32_t row_begin, row_end;  // global rows of the stage held by this layer
  uint32_t codes_row, scales_row, aux_row;
  uint32_t codes_bytes, scales_bytes, aux_bytes, y_bytes;
  int32_t pad[1];
};
static_assert(sizeof(StackLayer) == 88, "plan layer layout");


// The kernel reads the plan's tables through the constant address space:
// they are never written during a launch (the counters, which are, sit in
// their own bytes and are only touched with atomics), and constant loads
// stay scalar (s_load) even after the kernel's own vector stores, which
// plain global loads would not (they would then be vector loads whose waits
// drain the weight ring).
typedef const __attribute__((address_space(4))) StackHeader CHeader;
typedef const __attribute__((address_space(4))) StackStage CStage;
typedef const __attribute__((address_space(4))) StackLayer CLayer;

struct Plan {
  CHeader* h;
  CStage* st;
  CLayer* ly;
  int nst;
};

// Position of a wave in its stream of units, with the fields of its stage
// and layer that loads and decoding need kept in scalar registers: they are
// re-read from the plan only when the cursor moves to another stage or
// layer.  Past the end of the stream (done) the fields are layer 0's, which
// the dummy loads of the ring use.  Wave-uniform.
struct Cursor {
  int stage, layer, grow, unit;
  bool done;
  int units, rows;                   // of the stage
  int layer_end, row_begin, fmt, pieces, gshift;
  const uint32_t* codes;
  const void* scales;
  const void* aux;
  _Float16* y;
  uint32_t codes_row, scales_row, aux_row, codes_bytes, scales_bytes, aux_bytes, y_bytes;
};

__device__ __forceinline__ void cursor_layer(Cursor& c, const Plan& p) {
  CLayer* q = p.ly + c.layer;
  c.layer_end = q->row_end; c.row_begin = q->row_begin; c.fmt = q->fmt; c.pieces = q->k >> 5; c.gshift = q->gshift;
  c.codes = q->codes; c.scales = q->scales; c.aux = q->aux; c.y = q->y;
  c.codes_row = q->codes_row; c.scales_row = q->scales_row; c.aux_row = q->aux_row;
  c.codes_bytes = q->codes_bytes; c.scales_bytes = q->scales_bytes; c.aux_bytes = q->aux_bytes; c.y_bytes = q->y_bytes;
}

// Enter the first stage at or after c.stage that has row c.grow (the wave's
// own first row), or finish the stream.
__device__ __forceinline__ void cursor_enter(Cursor& c, const Plan& p) {
  while (c.stage < p.nst && c.grow >= p.st[c.stage].rows) ++c.stage;
  if (c.stage >= p.nst) {
    c.done = true;
    c.stage = p.nst;
    c.layer = 0;
    c.unit = 0;
    c.units = 1;
    c.rows = 0;
    cursor_layer(c, p);
    return;
  }
  c.units = p.st[c.stage].units;
  c.rows = p.st[c.stage].rows;
  c.layer = p.st[c.stage].layer_begin;
  while (c.grow >= p.ly[c.layer].row_end) ++c.layer;
  cursor_layer(c, p);
}

// First unit of wave wid: row wid of the first stage that has one.
__device__ __forceinline__ void cursor_first(Cursor& c, const Plan& p, int wid) {
  c.stage = 0;
  c.grow = wid;
  c.unit = 0;
  c.done = false;
  cursor_enter(c, p);
}

__device__ __forceinline__ void cursor_next(Cursor& c, const Plan& p, int wid, int W) {
  if (c.done) return;
  if (++c.unit < c.units) return;
  c.unit = 0;
  c.grow += W;
  if (c.grow >= c.rows) {
    c.grow = wid;
    ++c.stage;
    cursor_enter(c, p);
    return;
  }
  if (c.grow >= c.layer_end) {
    do ++c.layer;
    while (c.grow >= p.ly[c.layer].row_end);
    cursor_layer(c, p);
  }
}

// One unit's loads, held in registers: 8 code words and 4 metadata dwords.
struct Unit {
  uint32_t cw[8];
  uint32_t md[4];
};

template <int FMT>
struct UnitShape {
  static constexpr int cpl = FMT == Q_INT8 ? 1 : 2;  // pieces per lane
};

// Issue the six loads of the unit under cursor c (past the end of the
// stream, the same six loads of row 0 of layer 0, whose results are unused).
// Metadata dword j: 4-bit formats -- j = 0, 1 the dword holding the scale
// (AFPQ: the scale pair) of piece j, j = 2, 3 the zero-point / selector
// dword of piece j - 2; INT8 -- the dword holding the row scale.
__device__ __forceinline__ void load_unit(Unit& u, const Cursor& c, int lane) {
  const int lrow = c.done ? 0 : c.grow - c.row_begin;
  const int unit = c.done ? 0 : c.unit;
  const bool int8 = c.fmt == Q_INT8;
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(c.codes, c.codes_bytes);
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(c.scales, c.scales_bytes);
  const __amdgpu_buffer_rsrc_t ars = make_rsrc(c.aux, c.aux_bytes);  // 0 bytes: loads return 0
  const uint32_t so_codes = (uint32_t)lrow * c.codes_row;
  uint32_t coff[2], moff[4];
  if (int8) {
    const int pc = min(unit * 64 + lane, c.pieces - 1);
    coff[0] = (uint32_t)pc * 32u;
    coff[1] = coff[0] + 16u;
    const uint32_t so = (uint32_t)lrow * 2u;
    moff[0] = moff[1] = moff[2] = moff[3] = so & ~3u;
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int pc = min(unit * 128 + j * 64 + lane, c.pieces - 1);
      coff[j] = (uint32_t)pc * 16u;
      const uint32_t gi = ((uint32_t)pc * 32u) >> c.gshift;
      const uint32_t sb = c.fmt == Q_FP4_AFPQ ? gi * 4u : gi * 2u;
      moff[j] = ((uint32_t)lrow * c.scales_row + sb) & ~3u;
      const uint32_t aw = c.fmt == Q_INT4_ASYM ? (gi >> 3) : (gi >> 4);
      moff[2 + j] = (uint32_t)lrow * c.aux_row + aw * 4u;
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(crs, coff[j], so_codes, 0);
    u.cw[4 * j + 0] = v.x; u.cw[4 * j + 1] = v.y; u.cw[4 * j + 2] = v.z; u.cw[4 * j + 3] = v.w;
  }
  u.md[0] = __builtin_amdgcn_raw_buffer_load_b32(srs, moff[0], 0u, 0);
  u.md[1] = __builtin_amdgcn_raw_buffer_load_b32(srs, moff[1], 0u, 0);
  u.md[2] = __builtin_amdgcn_raw_buffer_load_b32(int8 ? srs : ars, moff[2], 0u, 0);
  u.md[3] = __builtin_amdgcn_raw_buffer_load_b32(int8 ? srs : ars, moff[3], 0u, 0);
}

struct StageLds {
  u32x4 xq[4][kStackPieces];  // x piece p, quarter i (16 bytes) at xq[i][p]
  f4 xs[kStackPieces];        // per piece: even/odd sums of its two 16-element halves
};

// This lane's activations for the unit under c, in decoder pair order: the
// pieces it decodes (two for 4-bit formats, one for INT8) and, for INT4,
// their even/odd half sums.
struct LaneX {
  uint32_t xr[2][16];
  float xs[2][4];
};

__device__ __forceinline__ void load_lane_x(LaneX& x, const Cursor& c, const StageLds& lds, int lane) {
  const int cpl = c.fmt == Q_INT8 ? 1 : 2;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (j < cpl) {
      const int pc = c.unit * 64 * cpl + j * 64 + lane;  // < kStackPieces (k <= Q_MAX_K)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 v = lds.xq[i][pc];
        x.xr[j][4 * i + 0] = v.x; x.xr[j][4 * i + 1] = v.y; x.xr[j][4 * i + 2] = v.z; x.xr[j][4 * i + 3] = v.w;
      }
      if (c.fmt == Q_INT4_ASYM) {
        const f4 s = lds.xs[pc];
        x.xs[j][0] = s[0]; x.xs[j][1] = s[1]; x.xs[j][2] = s[2]; x.xs[j][3] = s[3];
      }
    }
  }
}

// Decode + dot of the unit under cursor c; adds the lane's partial to *acc.
template <int FMT>
__device__ __forceinline__ void compute_unit(const Unit& u, const Cursor& c, const LaneX& x, int lane, float* acc) {
  constexpr int CPL = UnitShape<FMT>::cpl;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    RawMeta raw{0u, 0u};
    if constexpr (FMT != Q_INT8) {
      const int pcc = min(c.unit * 128 + j * 64 + lane, c.pieces - 1);
      const uint32_t gi = ((uint32_t)pcc * 32u) >> c.gshift;
      if constexpr (FMT == Q_FP4_AFPQ) {
        raw.a = u.md[j];
      } else {
        const uint32_t off = (uint32_t)(c.grow - c.row_begin) * c.scales_row + gi * 2u;
        raw.a = (u.md[j] >> (8u * (off & 2u))) & 0xFFFFu;
      }
      if constexpr (FMT == Q_INT4_ASYM) raw.b = u.md[2 + j] >> (4u * (gi & 7u));
      if constexpr (FMT == Q_FP4_RAZER) raw.b = u.md[2 + j] >> (2u * (gi & 15u));
    }
    const uint32_t(*xrp)[16] = &x.xr[j];
    // (the staged sums are the halves' even/odd sums: folding them at the
    // stage boundary measured slower, as that work is on the chained path)
    piece_dot<FMT, 1, true>(u.cw + (FMT == Q_INT8 ? 0 : 4 * j), nullptr, raw, xrp, x.xs[j], acc);
  }
}

// Stage s's activations into LDS, `nthreads` threads from `t0`: thread t
// handles pieces t, t + nthreads, ... (pieces past k read zeros through the
// buffer range check), issuing up to four pieces' loads before it waits.
// CHAIN: device-coherent loads (the activations may be what another
// workgroup has just written).
template <bool CHAIN>
__device__ __forceinline__ void stage_x(const Plan& p, int s, StageLds& lds, int t0, int nthreads) {
  CStage* S = p.st + s;
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(S->x, (uint32_t)S->k * 2u);
  constexpr int kAux = CHAIN ? 16 : 0;  // sc1: coherent at device scope
  const int order = S->order, xsum = S->xsum;
  // pieces the stage's units read: units * (128 or 64) per row
  const int span = S->units * (S->fmt == Q_INT8 ? 64 : 128);
  for (int base = 0; base < span; base += 4 * nthreads) {
    uint32_t nat[4][16];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = base + r * nthreads + t0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(xrs, (uint32_t)t * 64u + 16u * i, 0u, kAux);
        nat[r][4 * i + 0] = v.x; nat[r][4 * i + 1] = v.y; nat[r][4 * i + 2] = v.z; nat[r][4 * i + 3] = v.w;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = base + r * nthreads + t0;
      if (t < span) {
        uint32_t out[16];
        if (order == kPairStride4) pair_activations<kPairStride4>(nat[r], out);
        else if (order == kPairStride2) pair_activations<kPairStride2>(nat[r], out);
        else pair_activations<kPairAdjacent>(nat[r], out);
#pragma unroll
        for (int i = 0; i < 4; ++i) lds.xq[i][t] = u32x4{out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]};
        if (xsum) {
          f4 s4 = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const h2 v = as_h2(nat[r][8 * h + i]);
              s4[2 * h + 0] += (float)v[0];
              s4[2 * h + 1] += (float)v[1];
            }
          lds.xs[t] = s4;
        }
      }
    }
  }
}

// Producer side of the end of stage s under CHAIN: publish this workgroup's
// arrival (its compute waves' stores have completed: they waited before the
// barrier that precedes this) and wait until every workgroup has arrived.
// A relay: every workgroup stores the stage's epoch in its arrival word;
// workgroup 0 waits until all arrival words hold it and then stores it in the
// release word, which the others wait for.  255 pollers of one word and one
// poller of the compact arrival array load the memory system far less than
// 256 pollers of one counter that every workgroup increments (measured on its
// own: 3.1 against 7.2 us per stage).  Bounded: past kSpinLimit polls the
// abort flag is set and nobody waits any more (results are then undefined,
// but every wave runs to the end).
__device__ __forceinline__ void arrive_and_wait(uint32_t* ctrs, uint32_t epoch, int lane) {
  uint32_t* abort_flag = ctrs + kCtrAbort;
  if (lane == 0) __hip_atomic_store(ctrs + kCtrArr + blockIdx.x, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int nwg = (int)gridDim.x;
  uint32_t spins = 0;
  if (blockIdx.x == 0) {
    while (true) {
      bool ok = true;
      for (int w = lane; w < kMaxGrid; w += 64) {
        if (w < nwg) {
          const uint32_t v = __hip_atomic_load(ctrs + kCtrArr + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = ok && (int)(v - epoch) >= 0;
        }
      }
      if (__builtin_amdgcn_ballot_w64(!ok) == 0) break;
      if ((++spins & 63u) == 0) {
        if (__hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) break;
        if (spins >= kSpinLimit) {
          __hip_atomic_store(abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
    if (lane == 0) __hip_atomic_store(ctrs + kCtrGo, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    while ((int)((uint32_t)__builtin_amdgcn_readfirstlane(
                     (int)__hip_atomic_load(ctrs + kCtrGo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) - epoch) < 0) {
      if ((++spins & 63u) == 0) {
        if (__hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) break;
        if (spins >= kSpinLimit) {
          __hip_atomic_store(abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
  }
}

// Workgroup: NW compute waves and one producer wave.  The compute waves'
// stream of memory operations is their ring's weight loads and their output
// stores, the same at every step; the producer stages activations into a
// double-buffered LDS copy and, under CHAIN, handles the stage arrivals.
//
// Barriers (every wave executes each of them once): B0 after the first
// stage's activations; per stage boundary s -> s + 1 without CHAIN, A_s (the
// compute waves are done with stage s and the producer has staged stage
// s + 1 into the other buffer, during stage s); under CHAIN, A_s (the
// compute waves are done with stage s and their stores have completed),
// B_s (every workgroup has arrived) and C_s (all waves of the workgroup
// have staged stage s + 1, one piece per thread).
template <bool CHAIN, int NW, int S>
__global__ void __launch_bounds__(64 * (NW + 1)) stack_kernel(const uint8_t* __restrict__ plan_bytes) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  StageLds* lds = reinterpret_cast<StageLds*>(smem);  // [2]
  Plan p;
  const __attribute__((address_space(4))) uint8_t* cplan = (const __attribute__((address_space(4))) uint8_t*)plan_bytes;
  p.h = (CHeader*)cplan;
  p.st = (CStage*)(cplan + p.h->stages_off);
  p.ly = (CLayer*)(cplan + p.h->layers_off);
  p.nst = p.h->nstages;
  uint32_t* ctrs = reinterpret_cast<uint32_t*>(const_cast<uint8_t*>(plan_bytes) + kCtrOff);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nst = p.nst;
  constexpr int kThreads = 64 * (NW + 1);

  if (wave == NW) {
    // ---- producer wave
    // epochs of this launch's stages: past every epoch an earlier launch wrote
    const uint32_t launch = CHAIN ? __hip_atomic_load(ctrs + kCtrLaunch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
    stage_x<CHAIN>(p, 0, lds[0], lane, 64);
    lds_barrier();  // B0
    for (int s = 0; s + 1 < nst; ++s) {
      if constexpr (CHAIN) {
        lds_barrier();  // A_s
        arrive_and_wait(ctrs, launch * (uint32_t)nst + (uint32_t)s + 1u, lane);
        lds_barrier();  // B_s
        stage_x<CHAIN>(p, s + 1, lds[(s + 1) & 1], (int)threadIdx.x, kThreads);
        lds_barrier();  // C_s
      } else {
        stage_x<CHAIN>(p, s + 1, lds[(s + 1) & 1], lane, 64);
        lds_barrier();  // A_s
      }
    }
  } else {
    // ---- compute waves
    const int W = (int)gridDim.x * NW;
    const int wid = (int)blockIdx.x * NW + wave;
    // the ring: slot i holds unit t with t mod S == i
    Cursor ld, cp;
    cursor_first(ld, p, wid);
    cp = ld;
    Unit ring[S];
    // (the prologue issues its loads in the steady state's order: the wait
    // at the loop head serves its first iteration as well)
#pragma unroll
    for (int i = 0; i < S; ++i) {
      load_unit(ring[i], ld, lane);
      cursor_next(ld, p, wid, W);
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_barrier();  // B0
    int cur = 0;                  // stage whose activations the compute uses
    int x_stage = -1, x_unit = -1;  // what `lx` holds
    LaneX lx;
    float acc = 0.0f;             // this lane's partial of the current row
    constexpr int kStoreAux = CHAIN ? 16 : 0;  // sc1: write through to device scope

    // One step: cross into the unit's stage if needed, compute the unit,
    // store the row at its last unit (every step issues one store: a
    // dropped one otherwise), then refill the slot.  The store and the S
    // slots' refill loads are pinned in issue order, so when the next step
    // crosses a stage boundary under CHAIN, vmcnt(6) -- vector memory
    // operations retire in issue order -- means every store of this wave has
    // completed while the refill stays in flight.
    auto step = [&](Unit& rx) {
      while (cur < cp.stage && cur + 1 < nst) {
        if constexpr (CHAIN) {
          asm volatile("s_waitcnt vmcnt(6)" ::: "memory");  // this wave's stores have completed
          lds_barrier();  // A_cur
          lds_barrier();  // B_cur
          stage_x<CHAIN>(p, cur + 1, lds[(cur + 1) & 1], (int)threadIdx.x, kThreads);
          lds_barrier();  // C_cur
        } else {
          lds_barrier();  // A_cur
        }
        ++cur;
      }
      // Past the end of the stream the step still issues its store (dropped)
      // and its refill (dummy loads), so that every path through the loop
      // issues the same memory operations in the same order and no wait
      // ever covers more than the ring needs.
      const bool live = !cp.done;
      float val = 0.0f;
      uint32_t off = 0xFFFFFF00u;
      if (live) {
        if (cur != x_stage || cp.unit != x_unit) {
          load_lane_x(lx, cp, lds[cur & 1], lane);
          x_stage = cur;
          x_unit = cp.unit;
        }
        if (cp.unit == 0) acc = 0.0f;
        switch (cp.fmt) {
          case Q_INT4_ASYM: compute_unit<Q_INT4_ASYM>(rx, cp, lx, lane, &acc); break;
          case Q_FP4_E2M1: compute_unit<Q_FP4_E2M1>(rx, cp, lx, lane, &acc); break;
          case Q_FP4_RAZER: compute_unit<Q_FP4_RAZER>(rx, cp, lx, lane, &acc); break;
          case Q_FP4_AFPQ: compute_unit<Q_FP4_AFPQ>(rx, cp, lx, lane, &acc); break;
          default: compute_unit<Q_INT8>(rx, cp, lx, lane, &acc); break;
        }
        if (cp.unit + 1 == cp.units) {  // the row's last unit
          val = wave_total(acc);
          if (cp.fmt == Q_INT8) {
            const uint32_t sw = rx.md[0] >> (8u * ((uint32_t)((cp.grow - cp.row_begin) * 2) & 2u));
            val *= h2f((uint16_t)(sw & 0xFFFFu));
          }
          if (lane == 0) off = (uint32_t)(cp.grow - cp.row_begin) * 2u;
        }
      }
      const __amdgpu_buffer_rsrc_t yrs = make_rsrc(cp.y, cp.y_bytes);
      __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)val), yrs, off, 0, kStoreAux);
      __builtin_amdgcn_sched_barrier(0);
      cursor_next(cp, p, wid, W);
      load_unit(rx, ld, lane);
      cursor_next(ld, p, wid, W);
      __builtin_amdgcn_sched_barrier(0);
    };

    // S steps per trip and no exit in between: every path into a step then
    // carries the same loads in the same order.  A trip past the end of the
    // stream makes the remaining stage changes (every wave meets every
    // barrier once) and issues dummy loads and dropped stores.
    do {
#pragma unroll
      for (int i = 0; i < S; ++i) step(ring[i]);
    } while (!cp.done || cur + 1 < nst);
  }

  if constexpr (CHAIN) {
    // the last workgroup to finish advances the launch count, which moves
    // the next launch's epochs past every word this one wrote (stream order
    // makes it visible to the next launch)
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t launch = __hip_atomic_load(ctrs + kCtrLaunch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t old = __hip_atomic_fetch_add(ctrs + kCtrDone, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old + 1u == gridDim.x) {
        __hip_atomic_store(ctrs + kCtrDone, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ctrs + kCtrLaunch, launch + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

int pair_order(int fmt) { return fmt == Q_INT8 ? kPairStride2 : fmt == Q_INT4_ASYM ? kPairStride4 : kPairAdjacent; }

// LDS per workgroup: the staged activations, rounded up so that one
// workgroup fits a compute unit (160 KB), which spreads the grid over every
// compute unit.
constexpr uint32_t kStackLds = 84 * 1024;
static_assert(2 * sizeof(StageLds) <= kStackLds, "stack LDS");

}  // namespace

// Byte offset of the stage table: after the header and the counters.
size_t stages_offset(int) { return (kCtrOff + (size_t)(kCtrArr + kMaxGrid) * 4u + 15) / 16 * 16; }

size_t stack_plan_bytes(int count) {
  if (count < 1) return 0;
  return stages_offset(count) + (size_t)count * (sizeof(StackStage) + sizeof(StackLayer));
}

int stack_plan(const q_stack_entry* e, int count, const WeightView* views, void* out, size_t out_bytes) {
  // stages: runs of entries with the same stage id (ids non-decreasing),
  // each run sharing x, k and format
  std::vector<int> stage_first;
  for (int i = 0; i < count; ++i) {
    if (i > 0 && e[i].stage < e[i - 1].stage) return Q_ERR_SHAPE;
    if (i == 0 || e[i].stage != e[i - 1].stage) {
      stage_first.push_back(i);
    } else {
      const int f = stage_first.back();
      if (e[i].x != e[f].x || views[i].k != views[f].k) return Q_ERR_SHAPE;
      if (views[i].fmt != views[f].fmt) return Q_ERR_FORMAT;
    }
  }
  const int nst = (int)stage_first.size();
  uint8_t* base = static_cast<uint8_t*>(out);
  memset(base, 0, out_bytes < stack_plan_bytes(count) ? out_bytes : stack_plan_bytes(count));
  StackHeader h{};
  h.magic = kPlanMagic;
  h.version = kPlanVersion;
  h.nstages = nst;
  h.nlayers = count;
  h.ctr_off = kCtrOff;
  h.stages_off = (uint32_t)stages_offset(nst);
  h.layers_off = h.stages_off + (uint32_t)(nst * sizeof(StackStage));
  h.total_bytes = h.layers_off + (uint32_t)(count * sizeof(StackLayer));
  for (int si = 0; si < nst; ++si) {
    const int f = stage_first[si], l_end = si + 1 < nst ? stage_first[si + 1] : count;
    const WeightView& v = views[f];
    StackStage st{};
    st.x = static_cast<const _Float16*>(e[f].x);
    st.k = v.k;
    st.pieces = v.k / 32;
    st.layer_begin = f;
    st.layer_end = l_end;
    st.fmt = v.fmt;
    const int span = v.fmt == Q_INT8 ? 64 : 128;  // pieces per unit
    st.units = (st.pieces + span - 1) / span;
    st.order = pair_order(v.fmt);
    st.xsum = v.fmt == Q_INT4_ASYM ? 1 : 0;
    int64_t rows = 0;
    for (int i = f; i < l_end; ++i) {
      const WeightView& w = views[i];
      StackLayer L{};
      L.codes = w.codes;
      L.scales = w.scales;
      L.aux = w.aux;
      L.y = static_cast<_Float16*>(e[i].y);
      L.fmt = w.fmt;
      L.n = w.n;
      L.k = w.k;
      L.gshift = ilog2(w.group);
      L.row_begin = (int32_t)rows;
      rows += w.n;
      if (rows > (int64_t)INT32_MAX / 2) return Q_ERR_SHAPE;
      L.row_end = (int32_t)rows;
      const int G = w.k / w.group;
      L.codes_row = (uint32_t)(w.fmt == Q_INT8 ? w.k : w.k / 2);
      L.scales_row = (uint32_t)(w.fmt == Q_INT8 ? 2 : G * (w.fmt == Q_FP4_AFPQ ? 4 : 2));
      L.aux_row = (uint32_t)(w.fmt == Q_INT4_ASYM ? (G + 7) / 8 * 4 : w.fmt == Q_FP4_RAZER ? (G + 15) / 16 * 4 : 0);
      L.codes_bytes = (uint32_t)buffer_bytes(w.fmt, w.n, w.k, w.group, Q_BUF_CODES);
      L.scales_bytes = (uint32_t)buffer_bytes(w.fmt, w.n, w.k, w.group, Q_BUF_SCALES);
      L.aux_bytes = L.aux_row ? (uint32_t)buffer_bytes(w.fmt, w.n, w.k, w.group, Q_BUF_AUX) : 0u;
      L.y_bytes = (uint32_t)w.n * 2u;
      memcpy(base + h.layers_off + i * sizeof(StackLayer), &L, sizeof(L));
    }
    st.rows = (int32_t)rows;
    memcpy(base + h.stages_off + si * sizeof(StackStage), &st, sizeof(st));
  }
  memcpy(base, &h, sizeof(h));
  return Q_OK;
}

hipError_t launch_stack(const void* plan_device, bool chain, hipStream_t s) {
  static bool attr_set[2] = {false, false};
  auto fn = chain ? stack_kernel<true, kStackWaves, kStackRing> : stack_kernel<false, kStackWaves, kStackRing>;
  if (!attr_set[chain]) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kStackLds);
    if (e != hipSuccess) return e;
    attr_set[chain] = true;
  }
  // one workgroup per compute unit: under CHAIN every workgroup must be
  // resident at once
  const int grid = device_cu_count() < kMaxGrid ? device_cu_count() : kMaxGrid;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(64 * (kStackWaves + 1)), kStackLds, s,
                     static_cast<const uint8_t*>(plan_device));
  return hipGetLastError();
}

}  // namespace qg
