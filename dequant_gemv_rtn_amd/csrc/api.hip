// C ABI entry points (declared in include/qgemv.h): host-side validation and
// dispatch to the pack, vector-ALU GEMV and MFMA skinny-GEMM kernels.
// Validation runs before any HIP call, so argument errors never touch the
// device.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <stdlib.h>

#include <string.h>

#include <atomic>
#include <cmath>
#include <mutex>
#include <vector>

#include "common.hpp"
#include "internal.hpp"
#include "qgemv.h"

namespace qg {

namespace {

// Names of the tuning keys (TuneKey order): the environment variables read
// once, and the names q_tuning_set accepts.
const char* const kTuneNames[kTuneCount] = {
    "QGEMV_PATH",           "QGEMV_SPLIT_MIN_B",    "QGEMV_SPLIT_KC",          "QGEMV_SPLIT_LDS",
    "QGEMV_SPLIT_GRID_ROWS", "QGEMV_STREAM_MAX_WAVES", "QGEMV_STREAM_KC",     "QGEMV_STREAM_WAVES_PER_CU",
    "QGEMV_STREAM_GRID_ROWS", "QGEMV_VALU_CPL",      "QGEMV_VALU_ROWS",         "QGEMV_VALU_SHARE",
    "QGEMV_VALU_STRIDED",   "QGEMV_VALU_WAVES_PER_CU", "QGEMV_ATTN_MFMA",      "QGEMV_W8A8_WAVES",
    "QGEMV_W8A8_JOINT",     "QGEMV_W8A8_WAVES_PER_CU", "QGEMV_W8A8_FUSE_MAX_B", "QGEMV_W8A8_DOT",
    "QGEMV_W8A8_DOT_WAVES_PER_CU", "QGEMV_W8A8_DOT_P", "QGEMV_W8A8_DOT_S", "QGEMV_W8A8_DOT_SPLIT",
    "QGEMV_W8A8_DOT_WALKERS_PER_CU"};

struct TuneTable {
  std::atomic<int> value[kTuneCount];
  std::atomic<bool> set[kTuneCount];
  TuneTable() {
    for (int i = 0; i < kTuneCount; ++i) {
      const char* v = getenv(kTuneNames[i]);
      set[i].store(v && *v);
      value[i].store(v && *v ? atoi(v) : 0);
    }
  }
};

// Built on first use (C++ guarantees one thread-safe initialisation).
TuneTable& tune_table() {
  static TuneTable t;
  return t;
}

int tune_index(const char* name) {
  for (int i = 0; i < kTuneCount; ++i)
    if (strcmp(name, kTuneNames[i]) == 0) return i;
  return -1;
}

}  // namespace

int tuning(TuneKey key, int dflt) {
  TuneTable& t = tune_table();
  return t.set[key].load(std::memory_order_relaxed) ? t.value[key].load(std::memory_order_relaxed) : dflt;
}

int ilog2(int v) {
  int r = 0;
  while ((1 << r) < v) ++r;
  return r;
}

int device_cu_count() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

size_t packed_bytes_logical(int32_t format, int32_t n, int32_t k, int32_t group, int32_t which) {
  const size_t N = (size_t)n, K = (size_t)k;
  const size_t G = K / (size_t)group;
  switch (which) {
    case Q_BUF_CODES:
      if (format == Q_INT8) return N * K;
      if (is_fp3(format)) return N * (K / 32) * 12;
      return N * (K / 8) * 4;
    case Q_BUF_CODES_HI:
      return format == Q_BFP6 ? N * (K / 16) * 4 : 0;
    case Q_BUF_SCALES:
      if (format == Q_INT8) return N * 2;
      if (format == Q_BFP6 || format == Q_BFP4) return 0;
      return N * G * 2 * (format == Q_FP4_AFPQ || format == Q_FP3_AFPQ ? 2 : 1);
    case Q_BUF_AUX:
      if (format == Q_INT4_ASYM) return N * ((G + 7) / 8) * 4;
      if (format == Q_FP4_RAZER || format == Q_FP3_RAZER) return N * ((G + 15) / 16) * 4;
      if (format == Q_BFP6 || format == Q_BFP4) return N * (K / 16);
      return 0;
    default:
      return 0;
  }
}

size_t buffer_bytes(int32_t format, int32_t n, int32_t k, int32_t group, int32_t which) {
  const size_t v = packed_bytes_logical(format, n, k, group, which);
  return (v + kBufferPad - 1) / kBufferPad * kBufferPad;
}

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_group(int32_t format, int32_t n, int32_t k, int32_t group) {
  if (format < Q_INT4_ASYM || format > Q_FP3_AFPQ) return Q_ERR_FORMAT;
  if (n < 1 || k < 32 || k % 32 != 0 || k > Q_MAX_K) return Q_ERR_SHAPE;
  switch (format) {
    case Q_INT4_ASYM:
    case Q_FP4_E2M1:
    case Q_FP4_RAZER:
    case Q_FP4_AFPQ:
    case Q_FP3_RAZER:
    case Q_FP3_AFPQ:
      if (group != 32 && group != 64 && group != 128 && group != 256) return Q_ERR_FORMAT;
      if (k % group != 0) return Q_ERR_SHAPE;
      return Q_OK;
    case Q_BFP6:
    case Q_BFP4:
      return group == 16 ? Q_OK : Q_ERR_FORMAT;
    default:  // Q_INT8
      return group == k ? Q_OK : Q_ERR_FORMAT;
  }
}

// Shape and group rules, plus the addressing limit of the kernels: every
// packed buffer is read through a buffer resource with 32-bit byte offsets.
int check_shape(int32_t format, int32_t n, int32_t k, int32_t group) {
  const int st = check_group(format, n, k, group);
  if (st != Q_OK) return st;
  for (int which = Q_BUF_CODES; which <= Q_BUF_AUX; ++which)
    if (buffer_bytes(format, n, k, group, which) > (size_t)UINT32_MAX) return Q_ERR_SHAPE;
  return Q_OK;
}

// Checks the descriptor and its buffers; fills `view` on success.
int check_weight(const q_weight* w, WeightView* view) {
  if (!w) return Q_ERR_NULL;
  const int st = check_shape(w->format, w->n, w->k, w->group);
  if (st != Q_OK) return st;
  const int f = w->format;
  const bool need_scales = !(f == Q_BFP6 || f == Q_BFP4);
  const bool need_aux = f == Q_INT4_ASYM || f == Q_FP4_RAZER || f == Q_FP3_RAZER || f == Q_BFP6 || f == Q_BFP4;
  const bool need_hi = f == Q_BFP6;
  if (!w->codes || (need_scales && !w->scales) || (need_aux && !w->aux) || (need_hi && !w->codes_hi))
    return Q_ERR_NULL;
  if (!aligned16(w->codes) || (need_scales && !aligned16(w->scales)) || (need_aux && !aligned16(w->aux)) ||
      (need_hi && !aligned16(w->codes_hi)))
    return Q_ERR_ALIGN;
  view->fmt = f;
  view->n = w->n;
  view->k = w->k;
  view->group = w->group;
  view->codes = static_cast<const uint32_t*>(w->codes);
  view->codes_hi = need_hi ? static_cast<const uint32_t*>(w->codes_hi) : nullptr;
  view->scales = need_scales ? w->scales : nullptr;
  view->aux = need_aux ? w->aux : nullptr;
  return Q_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? Q_OK : Q_ERR_HIP; }

}  // namespace
}  // namespace qg

// Scratch of q_gemm_skinny_noalloc: the K-split form's fp32 part slots, in
// device memory the library owns, so that the call allocates nothing.  Every
// device the library runs on holds one copy until the process ends.  Host
// code never names this array directly (the host-side name is a stand-in,
// not a device address): it takes each device's address once, with
// hipGetSymbolAddress, and passes that.
static __device__ __align__(256) uint8_t scratch[Q_NOALLOC_SCRATCH_BYTES];

namespace qg {
namespace {

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // per device id; null until first taken

// Device address of the current device's scratch, taken once per device
// with that device current.
int scratch_of_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return Q_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return Q_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return Q_OK;
}

}  // namespace
}  // namespace qg

extern "C" {

size_t q_packed_bytes(int32_t format, int32_t n, int32_t k, int32_t group, int32_t which) {
  if (qg::check_shape(format, n, k, group) != Q_OK) return 0;
  if (which < Q_BUF_CODES || which > Q_BUF_AUX) return 0;
  return qg::buffer_bytes(format, n, k, group, which);
}

int q_pack(const q_weight* w, const void* w_fp16, void* stream) {
  qg::WeightView v;
  const int st = qg::check_weight(w, &v);
  if (st != Q_OK) return st;
  if (!w_fp16) return Q_ERR_NULL;
  if (!qg::aligned16(w_fp16)) return Q_ERR_ALIGN;
  return qg::from_hip(qg::launch_pack(v, static_cast<const _Float16*>(w_fp16), static_cast<hipStream_t>(stream)));
}

int q_pack_clip(const q_weight* w, const void* w_fp16, int32_t candidates, void* stream) {
  qg::WeightView v;
  const int st = qg::check_weight(w, &v);
  if (st != Q_OK) return st;
  if (v.fmt != Q_INT4_ASYM && v.fmt != Q_FP4_E2M1 && v.fmt != Q_FP4_RAZER && v.fmt != Q_FP4_AFPQ)
    return Q_ERR_FORMAT;
  if (candidates < 1 || candidates > Q_MAX_CLIP_CANDIDATES) return Q_ERR_SHAPE;
  if (!w_fp16) return Q_ERR_NULL;
  if (!qg::aligned16(w_fp16)) return Q_ERR_ALIGN;
  return qg::from_hip(
      qg::launch_pack(v, static_cast<const _Float16*>(w_fp16), static_cast<hipStream_t>(stream), candidates));
}

size_t q_workspace_bytes(const q_weight* w, int32_t b) {
  qg::WeightView v;
  if (qg::check_weight(w, &v) != Q_OK || b < 1 || b > Q_MAX_BATCH) return 0;
  return qg::gemm_split_workspace(v, b);
}

// Batches 2 and 3 on the vector-ALU kernel where it measured faster than the
// streaming MFMA kernel on MI355X (graph us, vector-ALU / streaming): at
// b = 2 INT8 (Llama-3-8B-shaped q|k|v 9.5 / 11.1, gate|up 23.8 / 27.3,
// down 15.7 / 17.4, lm_head 95.8 / 99.2), E2M1 (11008x4096 g32 8.8 / 11.6),
// BFP6 (13824x5120 22.7 / 23.9) and INT4 from 20 M elements (6144x4096
// 7.5 / 7.8, 28672x4096 15.7 / 17.8, 4096x14336 12.4 / 14.4; 4096x4096
// 6.3 / 5.9); at b = 3 INT8 with k <= 8192 (gate|up 24.4 / 27.4) and E2M1
// (10.4 / 11.8).  RaZeR, AFPQ and BFP4 stay on the streaming kernel.
static bool valu_small_batch(const qg::WeightView& v, int b) {
  if (b == 2) {
    if (v.fmt == Q_INT8 || v.fmt == Q_FP4_E2M1 || v.fmt == Q_BFP6) return true;
    return v.fmt == Q_INT4_ASYM && (uint64_t)v.n * (uint64_t)v.k >= ((uint64_t)20 << 20);
  }
  if (b == 3) return (v.fmt == Q_INT8 && v.k <= 8192) || v.fmt == Q_FP4_E2M1;
  return false;
}

int q_gemm_skinny_ws(const q_weight* w, const void* x_fp16, void* y_fp16, int32_t b, void* workspace,
                     size_t workspace_bytes, void* stream) {
  qg::WeightView v;
  const int st = qg::check_weight(w, &v);
  if (st != Q_OK) return st;
  if (b < 1 || b > Q_MAX_BATCH) return Q_ERR_BATCH;
  if (!x_fp16 || !y_fp16) return Q_ERR_NULL;
  if (!qg::aligned16(x_fp16) || !qg::aligned16(y_fp16)) return Q_ERR_ALIGN;
  if (workspace && !qg::aligned16(workspace)) return Q_ERR_ALIGN;
  // y is written through a buffer resource too; offsets from 0xFFFFFF00 up
  // are reserved for stores that the range check drops
  if ((uint64_t)b * (uint64_t)v.n * 2u > 0xFFFFFF00u) return Q_ERR_SHAPE;
  const auto* x = static_cast<const _Float16*>(x_fp16);
  auto* y = static_cast<_Float16*>(y_fp16);
  const auto s = static_cast<hipStream_t>(stream);
  // Routing, from measurements on MI355X: b = 1 runs the vector-ALU kernel,
  // and so do the small batches where it measured faster (valu_small_batch);
  // otherwise the streaming MFMA kernel, in its K-split form when a large
  // enough workspace is given and the plan asks for it (see
  // q_workspace_bytes), else in its full-K form (which serves every shape
  // that passed the checks above).  QGEMV_PATH (tuning and tests) forces
  // one: 1 = vector-ALU (b <= 8), 2 = streaming MFMA.
  const int path = qg::tuning(qg::kTunePath, 0);
  const bool valu = path == 1 ? b <= 8 : path == 2 ? false : (b == 1 || valu_small_batch(v, b));
  if (valu) return qg::from_hip(qg::launch_gemv_valu(v, x, y, b, s));
  const size_t need = qg::gemm_split_workspace(v, b);
  if (need > 0 && workspace && workspace_bytes >= need)
    return qg::from_hip(qg::launch_gemm_split(v, x, y, b, workspace, workspace_bytes, s));
  if (!qg::gemm_stream_supported(v, b)) return Q_ERR_SHAPE;
  return qg::from_hip(qg::launch_gemm_stream(v, x, y, b, s));
}

int q_gemm_skinny(const q_weight* w, const void* x_fp16, void* y_fp16, int32_t b, void* stream) {
  return q_gemm_skinny_ws(w, x_fp16, y_fp16, b, nullptr, 0, stream);
}

int q_gemm_skinny_noalloc(const q_weight* w, const void* x_fp16, void* y_fp16, int32_t b, void* stream) {
  qg::WeightView v;
  const int st = qg::check_weight(w, &v);
  if (st != Q_OK) return st;
  if (b < 1 || b > Q_MAX_BATCH) return Q_ERR_BATCH;
  if (!x_fp16 || !y_fp16) return Q_ERR_NULL;
  if (!qg::aligned16(x_fp16) || !qg::aligned16(y_fp16)) return Q_ERR_ALIGN;
  if ((uint64_t)b * (uint64_t)v.n * 2u > 0xFFFFFF00u) return Q_ERR_SHAPE;
  const size_t need = qg::gemm_split_workspace(v, b);
  if (need > (size_t)Q_NOALLOC_SCRATCH_BYTES) return Q_ERR_SCRATCH;
  if (need == 0) return q_gemm_skinny_ws(w, x_fp16, y_fp16, b, nullptr, 0, stream);
  void* ws = nullptr;
  const int sst = qg::scratch_of_current_device(&ws);
  if (sst != Q_OK) return sst;
  // the same validation and kernels as q_gemm_skinny_ws with a workspace of
  // exactly the scratch's size
  return q_gemm_skinny_ws(w, x_fp16, y_fp16, b, ws, (size_t)Q_NOALLOC_SCRATCH_BYTES, stream);
}

size_t q_w8a8_workspace_bytes(int32_t b, int32_t k) {
  if (b < 1 || b > Q_MAX_BATCH || k < 32 || k > Q_MAX_K || k % 32 != 0) return 0;
  return qg::w8a8_workspace_bytes(b, k);
}

int q_gemm_w8a8(const q_weight* w, const void* x_fp16, const float* smooth, void* y_fp16, int32_t b, void* workspace,
                size_t workspace_bytes, void* stream) {
  qg::WeightView v;
  const int st = qg::check_weight(w, &v);
  if (st != Q_OK) return st;
  if (v.fmt != Q_INT8) return Q_ERR_FORMAT;
  if (b < 1 || b > Q_MAX_BATCH) return Q_ERR_BATCH;
  if (!x_fp16 || !y_fp16 || !workspace) return Q_ERR_NULL;
  if (!qg::aligned16(x_fp16) || !qg::aligned16(y_fp16) || !qg::aligned16(workspace) ||
      (reinterpret_cast<uintptr_t>(smooth) & 3u) != 0)
    return Q_ERR_ALIGN;
  // y is written through a buffer resource; offsets from 0xFFFFFF00 up are
  // reserved for stores that the range check drops
  if ((uint64_t)b * (uint64_t)v.n * 2u > 0xFFFFFF00u) return Q_ERR_SHAPE;
  if (workspace_bytes < qg::w8a8_workspace_bytes(b, v.k)) return Q_ERR_SHAPE;
  return qg::from_hip(qg::launch_w8a8(v, static_cast<const _Float16*>(x_fp16), smooth, static_cast<_Float16*>(y_fp16),
                                      b, workspace, static_cast<hipStream_t>(stream)));
}

size_t q_stack_plan_bytes(int32_t count) {
  if (count < 1 || count > Q_MAX_STACK_ENTRIES) return 0;
  return qg::stack_plan_bytes(count);
}

int q_stack_plan(const q_stack_entry* entries, int32_t count, void* plan, size_t plan_bytes) {
  if (count < 1 || count > Q_MAX_STACK_ENTRIES) return Q_ERR_SHAPE;
  if (!entries || !plan) return Q_ERR_NULL;
  std::vector<qg::WeightView> views((size_t)count);
  for (int i = 0; i < count; ++i) {
    const int st = qg::check_weight(&entries[i].w, &views[i]);
    if (st != Q_OK) return st;
    const int f = views[i].fmt;
    if (f == Q_BFP6 || f == Q_BFP4 || qg::is_fp3(f)) return Q_ERR_FORMAT;
    if (!entries[i].x || !entries[i].y) return Q_ERR_NULL;
    if (!qg::aligned16(entries[i].x) || !qg::aligned16(entries[i].y)) return Q_ERR_ALIGN;
    if ((uint64_t)views[i].n * 2u > 0xFFFFFF00u) return Q_ERR_SHAPE;
  }
  if (plan_bytes < qg::stack_plan_bytes(count)) return Q_ERR_SHAPE;
  return qg::stack_plan(entries, count, views.data(), plan, plan_bytes);
}

int q_gemv_stack(const void* plan_device, int32_t flags, void* stream) {
  if (!plan_device) return Q_ERR_NULL;
  if (!qg::aligned16(plan_device)) return Q_ERR_ALIGN;
  if (flags & ~Q_STACK_CHAIN) return Q_ERR_ARG;
  return qg::from_hip(qg::launch_stack(plan_device, (flags & Q_STACK_CHAIN) != 0, static_cast<hipStream_t>(stream)));
}

int q_gemv(const q_weight* w, const void* x_fp16, void* y_fp16, void* stream) {
  return q_gemm_skinny(w, x_fp16, y_fp16, 1, stream);
}

int q_dequant(const q_weight* w, void* out_fp16, void* stream) {
  qg::WeightView v;
  const int st = qg::check_weight(w, &v);
  if (st != Q_OK) return st;
  if (!out_fp16) return Q_ERR_NULL;
  if (!qg::aligned16(out_fp16)) return Q_ERR_ALIGN;
  return qg::from_hip(qg::launch_dequant(v, static_cast<_Float16*>(out_fp16), static_cast<hipStream_t>(stream)));
}

// Shape rules shared by the two attention calls.
static int check_attn_shape(int32_t batch, int32_t q_heads, int32_t kv_heads, int32_t max_len) {
  // (at most 2^20 cached tokens: 1024 ranges of up to 1024 tokens)
  if (batch < 1 || kv_heads < 1 || q_heads < kv_heads || q_heads % kv_heads != 0 || max_len < 1 || max_len > (1 << 20))
    return Q_ERR_SHAPE;
  // (q and out are addressed with 32-bit byte offsets: batch * q_heads * 256 < 4 GiB)
  if ((int64_t)batch * q_heads >= (1 << 24) || (int64_t)batch * kv_heads * max_len > INT32_MAX) return Q_ERR_SHAPE;
  return Q_OK;
}

size_t q_attn_workspace_bytes(int32_t batch, int32_t q_heads, int32_t kv_heads, int32_t max_len) {
  if (check_attn_shape(batch, q_heads, kv_heads, max_len) != Q_OK) return 0;
  return qg::attn_workspace_bytes(batch, q_heads, kv_heads, max_len);
}

int q_attn_decode(const q_weight* k_cache, const q_weight* v_cache, const void* q_fp16, void* out_fp16,
                  int32_t batch, int32_t q_heads, int32_t kv_heads, int32_t max_len, const int32_t* seq_lens,
                  float scale, void* workspace, size_t workspace_bytes, void* stream) {
  qg::WeightView kv, vv;
  int st = qg::check_weight(k_cache, &kv);
  if (st != Q_OK) return st;
  st = qg::check_weight(v_cache, &vv);
  if (st != Q_OK) return st;
  if (kv.fmt != Q_FP4_RAZER && kv.fmt != Q_FP4_E2M1) return Q_ERR_FORMAT;
  if (vv.fmt != kv.fmt || vv.group != kv.group) return Q_ERR_FORMAT;
  if (kv.group > 128) return Q_ERR_FORMAT;
  st = check_attn_shape(batch, q_heads, kv_heads, max_len);
  if (st != Q_OK) return st;
  const int64_t rows = (int64_t)batch * kv_heads * max_len;
  if (kv.k != 128 || vv.k != 128 || kv.n != rows || vv.n != rows) return Q_ERR_SHAPE;
  if (!q_fp16 || !out_fp16 || !workspace) return Q_ERR_NULL;
  if (!qg::aligned16(q_fp16) || !qg::aligned16(out_fp16) || !qg::aligned16(workspace) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u) != 0)
    return Q_ERR_ALIGN;
  if (!std::isfinite(scale)) return Q_ERR_SHAPE;
  if (workspace_bytes < qg::attn_workspace_bytes(batch, q_heads, kv_heads, max_len)) return Q_ERR_SHAPE;
  return qg::from_hip(qg::launch_attn_decode(kv, vv, static_cast<const _Float16*>(q_fp16), seq_lens,
                                             static_cast<_Float16*>(out_fp16), batch, q_heads, kv_heads, max_len,
                                             scale, workspace, static_cast<hipStream_t>(stream)));
}

const char* q_strerror(int status) {
  switch (status) {
    case Q_OK: return "ok";
    case Q_ERR_NULL: return "a required pointer is NULL";
    case Q_ERR_SHAPE: return "bad shape: need n >= 1, 32 <= k <= Q_MAX_K, k % 32 == 0, group dividing k, "
                             "every packed buffer and the output below 4 GiB";
    case Q_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case Q_ERR_FORMAT: return "unknown format or group size not allowed for the format";
    case Q_ERR_BATCH: return "batch outside [1, 64]";
    case Q_ERR_HIP: return "HIP runtime error (no device or launch failure)";
    case Q_ERR_ARG: return "unknown tuning name or flag";
    case Q_ERR_SCRATCH: return "the call needs more scratch than Q_NOALLOC_SCRATCH_BYTES (use q_gemm_skinny_ws)";
    default: return "unknown status";
  }
}

int q_tuning_set(const char* name, int32_t value) {
  if (!name) return Q_ERR_NULL;
  const int i = qg::tune_index(name);
  if (i < 0) return Q_ERR_ARG;
  qg::TuneTable& t = qg::tune_table();
  t.value[i].store(value);
  t.set[i].store(true);
  return Q_OK;
}

int q_tuning_clear(const char* name) {
  qg::TuneTable& t = qg::tune_table();
  if (!name) {
    for (int i = 0; i < qg::kTuneCount; ++i) t.set[i].store(false);
    return Q_OK;
  }
  const int i = qg::tune_index(name);
  if (i < 0) return Q_ERR_ARG;
  t.set[i].store(false);
  return Q_OK;
}

int q_version(void) { return 200; }

}  // extern "C"
