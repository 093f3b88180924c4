/*
 * qgemv.h -- C ABI of the MI355X (gfx950) library for group-wise round-to-
 * nearest (RTN) low-bit weight quantization and the fused-dequantization
 * matrix-vector / skinny matrix product that consumes the packed weights.
 *
 * What the calls compute, and where the pages define it:
 *   - q_pack: one-shot, data-free RTN of fp16 weights onto a low-bit format
 *     ("Is (Selective) Round-To-Nearest Quantization All You Need?", abstract:
 *     RTN is cheap to apply; "Revisiting Block-based Quantisation", abstract:
 *     no data calibration).  Formats: asymmetric INT4 with per-group scale and
 *     zero-point (the comparison format of "The Power of Negative Zero" and the
 *     storage baseline of "AFPQ"); FP4 E2M1 in sign-magnitude form; RaZeR, which
 *     remaps E2M1's negative-zero code to a special value chosen per group
 *     ("The Power of Negative Zero", abstract and method section); AFPQ with
 *     separate positive and negative scales ("AFPQ: Asymmetric Floating Point
 *     Quantization for LLMs", abstract); block formats sharing one exponent
 *     across 16 packed numbers ("Revisiting Block-based Quantisation",
 *     abstract); INT8 per output channel for selectively up-precisioned layers
 *     ("Is (Selective) Round-To-Nearest Quantization All You Need?", abstract).
 *   - q_gemv / q_gemm_skinny: y = x * W_deq^T with dequantization fused into
 *     the product ("The Power of Negative Zero", abstract: a GEMV kernel with
 *     fused dequantization; Kogan, abstract: RTN on Marlin-style kernels).
 *
 * Conventions shared by every call:
 *   - W is [n, k] row-major fp16 (row = output channel), groups run along k.
 *     x is [b, k] fp16 row-major, y is [b, n] fp16 row-major.
 *   - Every pointer is a device pointer owned by the caller; the library never
 *     allocates, frees or retains memory and keeps no state between calls.
 *     Sizes of the packed buffers come from q_packed_bytes.
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL is the
 *     null stream) and returns without synchronizing.  Calls are reentrant.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     negative q_status is returned and nothing runs.  A HIP launch failure
 *     returns Q_ERR_HIP.  No exception crosses the ABI.
 *   - Every pointer must be 16-byte aligned.
 *   - Preconditions not checked on the device: W and x are finite and every
 *     y value fits in fp16.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight formats.  Allowed `group` values:
 *   Q_INT4_ASYM, Q_FP4_E2M1, Q_FP4_RAZER, Q_FP4_AFPQ,
 *   Q_FP3_RAZER, Q_FP3_AFPQ: 32, 64, 128 or 256
 *   Q_BFP6, Q_BFP4: 16 (one shared exponent per 16 elements along k)
 *   Q_INT8: k (one scale per output row)
 * The 3-bit formats ("The Power of Negative Zero", abstract: RaZeR at 3 and
 * 4 bits; "AFPQ", abstract: asymmetric FP below 4 bits) use FP3 = E2M0, the
 * E2M1 grid without its mantissa bit: magnitudes {0, 1, 2, 4} times the
 * scale.  Q_FP3_RAZER remaps the -0 code to a per-group special value in
 * {+3, -3, +8, -8} (selector 0..3; scale absmax / max(4, |v|)); Q_FP3_AFPQ
 * has separate scales max+/4 and max-/4. */
typedef enum q_format {
  Q_INT4_ASYM = 1,
  Q_FP4_E2M1 = 2,
  Q_FP4_RAZER = 3,
  Q_FP4_AFPQ = 4,
  Q_BFP6 = 5,
  Q_BFP4 = 6,
  Q_INT8 = 7,
  Q_FP3_RAZER = 8,
  Q_FP3_AFPQ = 9
} q_format;

typedef enum q_status {
  Q_OK = 0,
  Q_ERR_NULL = -1,   /* a required pointer is NULL */
  Q_ERR_SHAPE = -2,  /* n < 1, k < 32, k % 32 != 0, k > Q_MAX_K, group does not divide k,
                        a packed buffer would reach 4 GiB, or (q_gemm_skinny) the
                        output b * n * 2 bytes would exceed 0xFFFFFF00 (the kernels
                        address each buffer with 32-bit byte offsets) */
  Q_ERR_ALIGN = -3,  /* a pointer is not 16-byte aligned */
  Q_ERR_FORMAT = -4, /* unknown format, or group not allowed for the format */
  Q_ERR_BATCH = -5,  /* b outside [1, Q_MAX_BATCH] */
  Q_ERR_HIP = -6,    /* the HIP runtime reported an error (no device, launch failure) */
  Q_ERR_ARG = -7,    /* unknown tuning name (q_tuning_set / q_tuning_clear) or flag */
  Q_ERR_SCRATCH = -8 /* q_gemm_skinny_noalloc: the call needs more than Q_NOALLOC_SCRATCH_BYTES */
} q_status;

#define Q_MAX_K 16384
#define Q_MAX_BATCH 64

/* Buffer selector for q_packed_bytes. */
typedef enum q_buffer {
  Q_BUF_CODES = 0,    /* codes: 4-bit formats uint32 [n][k/8], element j of a word in
                         bits 4j..4j+3; Q_BFP6 its low 4 bits likewise; Q_INT8 int8 [n][k];
                         3-bit formats uint32 [n][k/32][3]: element e = 8q + r of a
                         32-element piece (code = s<<2 | i1<<1 | i0) has i0, i1 in word
                         q/2 at bits 4r+1, 4r+2 (q even) or 4r+3, (4r+4) mod 32 (q odd),
                         and its sign s in word 2 at bit 4r + 3 - q */
  Q_BUF_CODES_HI = 1, /* Q_BFP6 only: top 2 bits of each 6-bit field, uint32 [n][k/16] */
  Q_BUF_SCALES = 2,   /* fp16 [n][k/group]; Q_FP4_AFPQ, Q_FP3_AFPQ fp16 [n][k/group][2] as (s+, s-);
                         Q_INT8 fp16 [n]; none for block formats */
  Q_BUF_AUX = 3       /* Q_INT4_ASYM zero-points, 4-bit, uint32 [n][ceil(G/8)];
                         Q_FP4_RAZER, Q_FP3_RAZER special-value selectors, 2-bit,
                         uint32 [n][ceil(G/16)];
                         block formats: exponent bytes uint8 [n][k/16] (E + 127, 0 for an
                         all-zero block); G = k/group */
} q_buffer;

/* Descriptor of one packed weight matrix.  The library reads it and the
 * buffers it points to; the caller owns all of them. */
typedef struct q_weight {
  int32_t format; /* q_format */
  int32_t n;      /* output rows */
  int32_t k;      /* input columns */
  int32_t group;  /* see q_format */
  void* codes;
  void* codes_hi; /* Q_BFP6 only, else ignored */
  void* scales;   /* ignored by block formats */
  void* aux;      /* Q_INT4_ASYM, Q_FP4_RAZER, Q_FP3_RAZER, Q_BFP6, Q_BFP4; else ignored */
} q_weight;

/* Utility (the pages define no such call; it sizes the caller's
 * allocations for the layouts above).
 * Byte size to allocate for buffer `which` (q_buffer) for the given shape,
 * or 0 when the format has no such buffer or the arguments are invalid.
 * Host-only.  It is the packed contents (layouts above) rounded up to a
 * multiple of 16 bytes; q_pack writes zeros to the pad, and the product calls
 * may read it (16-byte loads that start inside a buffer end inside it). */
size_t q_packed_bytes(int32_t format, int32_t n, int32_t k, int32_t group, int32_t which);

/* Quantize fp16 weights w_fp16 [n][k] (device) by RTN and write the packed
 * buffers named by *w.  Output is a deterministic function of the input bits.
 * Rounding: every scale is computed in fp32 and rounded once to fp16; each
 * element takes the nearest value its format can represent under that stored
 * scale, ties to the even integer / even E2M1 magnitude index; RaZeR keeps the
 * special value only when strictly nearer, and picks per group the special in
 * {+5, -5, +8, -8} (selector 0..3) with the least fp64 squared error. */
int q_pack(const q_weight* w, const void* w_fp16, void* stream);

/* q_pack with a data-free clipping search per group, for Q_INT4_ASYM,
 * Q_FP4_E2M1, Q_FP4_AFPQ and Q_FP4_RAZER ("The Power of Negative Zero",
 * abstract, names clipping as a method RaZeR combines with, without fixing a
 * procedure; the ratio grid and the selection rule below are this library's
 * own reading).  Candidate c = 0 .. candidates - 1 shrinks
 * the group's range bounds (INT4: min(w,0) and max(w,0); E2M1 and RaZeR: the
 * absmax; AFPQ: max(w,0) and max(-w,0)) to (v * (20 - c)) / 20 in fp32,
 * quantizes the group by RTN on that range exactly as q_pack does (values
 * beyond it saturate; RaZeR tries its four specials under each c), and the
 * candidate with the smallest fp64 sum of squared errors against the fp16
 * weights is stored (equal sums: the smaller c, then the earlier RaZeR
 * special).  The packed layout is q_pack's: every product
 * call reads it unchanged.  candidates = 1 gives q_pack's output.
 * Errors: Q_ERR_FORMAT (another format), Q_ERR_SHAPE (candidates outside
 * 1 .. Q_MAX_CLIP_CANDIDATES), and q_pack's. */
#define Q_MAX_CLIP_CANDIDATES 10
int q_pack_clip(const q_weight* w, const void* w_fp16, int32_t candidates, void* stream);

/* y[n] = sum_k W_deq[n][k] * x[k]; x fp16 [k], y fp16 [n]; fp32 accumulation.
 * Identical to q_gemm_skinny with b = 1. */
int q_gemv(const q_weight* w, const void* x_fp16, void* y_fp16, void* stream);

/* y[b][n] = sum_k W_deq[n][k] * x[b][k] for b in [0, b); 1 <= b <= 64.
 * b = 1 runs a vector-ALU kernel, and so do b = 2 and 3 for the formats
 * and shapes where it measured faster (INT8, E2M1, BFP6 and large INT4 at
 * b = 2; INT8 with k <= 8192 and E2M1 at b = 3); the other batches run a
 * weight-streaming MFMA kernel.  Both multiply fp16 activations by exact unscaled codes with fp32
 * accumulation and apply each group scale once to the fp32 partial of its
 * group.  The MFMA kernel folds the block formats' power-of-two step,
 * relative to the largest block of the row's slice, into the fp16 operand
 * and applies the rest in fp32: exact for blocks down to 2^-24 of that
 * largest one.  The output is rounded once to fp16. */
int q_gemm_skinny(const q_weight* w, const void* x_fp16, void* y_fp16, int32_t b, void* stream);

/* Bytes of device workspace that q_gemm_skinny_ws uses for (w, b), or 0
 * when that call needs none (it then runs the same kernels as
 * q_gemm_skinny).  Host-only; 0 also for invalid arguments. */
size_t q_workspace_bytes(const q_weight* w, int32_t b);

/* q_gemm_skinny with a caller-owned device workspace (16-byte aligned).
 * With workspace_bytes >= q_workspace_bytes(w, b) the streaming MFMA kernel
 * runs in its K-split form: each workgroup covers one part of K for all b
 * activation rows, so the weights are read and decoded once whatever b, and
 * writes fp32 partial results to the workspace; a second kernel on the same
 * stream adds the parts of each output in a fixed order and rounds once to
 * fp16.  The result is deterministic; it may differ from q_gemm_skinny's in
 * the last fp16 place (another fp32 summation order).  The workspace needs
 * no initialization and holds scratch afterwards.  Two calls that may run at
 * the same time (other streams) must not share a workspace.  A NULL or too
 * small workspace runs q_gemm_skinny's kernels.  Same status codes as
 * q_gemm_skinny, plus Q_ERR_ALIGN for a misaligned workspace. */
int q_gemm_skinny_ws(const q_weight* w, const void* x_fp16, void* y_fp16, int32_t b, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Decode stack: every linear of one decode step at b = 1 in one launch.
 * A decode step runs a fixed sequence of fused-dequant matrix-vector
 * products -- per decoder layer q|k|v, o, gate|up and down, then the output
 * head, INT4 for most layers and INT8 for the selectively up-precisioned
 * ones ("Is (Selective) Round-To-Nearest Quantization All You Need?",
 * abstract: selective RTN and token-generation throughput on fused-dequant
 * kernels; "A Method for Layer Bit-Width Allocation ...", English abstract:
 * the FFN and lm_head layers).  Each entry computes y[n] = sum_k W_deq[n][k]
 * x[k] exactly as q_gemv does (same decode, fp32 sums per piece and group,
 * one fp16 rounding; only the fp32 summation order differs).
 *
 * Entries: weights in Q_INT4_ASYM, Q_FP4_E2M1, Q_FP4_RAZER, Q_FP4_AFPQ or
 * Q_INT8 (not the block formats); x fp16 [k] and y fp16 [n], device,
 * 16-byte aligned.  Consecutive entries with the same `stage` form a stage:
 * they must read the same x (same pointer, same k) and share a format;
 * stage ids are non-decreasing.  Outputs of different entries must not
 * overlap, and no entry's x may overlap an output of its own stage. */
typedef struct q_stack_entry {
  q_weight w;
  const void* x;
  void* y;
  int32_t stage;
  int32_t reserved; /* 0 */
} q_stack_entry;

#define Q_MAX_STACK_ENTRIES 65536
/* q_gemv_stack flag: each stage waits for the previous stage's outputs (a
 * stage's x may then be an output of an earlier stage).  Outputs are written
 * through to device scope and every workgroup of the launch meets at the end
 * of each stage; the next stage's weight loads are issued before that wait.
 * Without the flag stages do not wait for each other, and no x may be an
 * output of the same launch. */
#define Q_STACK_CHAIN 1
#define Q_STACK_ABORT_OFFSET 68

/* Bytes of the plan for `count` entries (0 outside 1 .. Q_MAX_STACK_ENTRIES).
 * Host-only. */
size_t q_stack_plan_bytes(int32_t count);

/* Validate the entries and write the plan into `plan` (host memory, at least
 * q_stack_plan_bytes(count) bytes).  Host-only: no HIP call.  The caller
 * copies the plan unchanged to device memory (16-byte aligned) and keeps it,
 * and every buffer it names, alive while launches may use it; the plan holds
 * the entries' device pointers.  Errors: Q_ERR_NULL, Q_ERR_SHAPE (count,
 * plan size, stage ids decreasing, a stage mixing x or k, an output past
 * 32-bit offsets), Q_ERR_FORMAT (a block format, a stage mixing formats),
 * Q_ERR_ALIGN, and q_gemv's checks of each weight. */
int q_stack_plan(const q_stack_entry* entries, int32_t count, void* plan, size_t plan_bytes);

/* Run every entry of a plan (its device copy) in one launch on `stream`:
 * one resident workgroup per compute unit walks the entries in order.
 * flags: 0 or Q_STACK_CHAIN.  The plan's device copy also holds the
 * launch's stage counters: launches that share a plan copy must not overlap
 * (other streams).  With Q_STACK_CHAIN every workgroup of the launch must be
 * resident at once, which holds while no other kernel occupies the device's
 * compute units; a stage wait that sees no progress for about a second gives
 * up, sets the plan copy's abort word (uint32 at byte offset
 * Q_STACK_ABORT_OFFSET of the plan, 0 as written by q_stack_plan; the caller
 * may read it after the launch) and leaves the outputs undefined.  Errors: Q_ERR_NULL, Q_ERR_ALIGN, Q_ERR_ARG (unknown
 * flag), Q_ERR_HIP. */
int q_gemv_stack(const void* plan_device, int32_t flags, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * q_gemm_skinny_ws with the library's own static scratch in place of a
 * caller workspace.  Same result, kernels and status codes as
 * q_gemm_skinny_ws given a workspace of Q_NOALLOC_SCRATCH_BYTES bytes; the
 * caller still owns x and y.  The scratch is one fixed device array of
 * Q_NOALLOC_SCRATCH_BYTES per device (64 MiB), held from the first call on
 * that device until the process ends; its address is taken once per device
 * on that first call, with the device current.  The call itself allocates
 * and frees nothing.  The K-split form writes every scratch slot it reads in
 * the same call, so nothing needs to start at zero.  All calls on one device
 * share its scratch and it keeps the last call's contents: calls that may
 * run at the same time on one device (other streams, other threads' streams)
 * race on it and must be serialized by the caller.  Errors: those of
 * q_gemm_skinny_ws, Q_ERR_SCRATCH when q_workspace_bytes(w, b) exceeds
 * Q_NOALLOC_SCRATCH_BYTES (nothing is launched), Q_ERR_HIP when the
 * scratch's address cannot be taken. */
#define Q_NOALLOC_SCRATCH_BYTES (64u << 20)
int q_gemm_skinny_noalloc(const q_weight* w, const void* x_fp16, void* y_fp16, int32_t b, void* stream);

/* Decode attention over a quantized KV cache: the KV cache quantized with
 * RaZeR as for weights ("The Power of Negative Zero", abstract: the datatype
 * applies to weight and KV-cache quantization).  Each cached key or value
 * vector -- one token of one KV head, head_dim = 128 elements -- is one row
 * of a q_weight made by q_pack: format Q_FP4_RAZER (or Q_FP4_E2M1), group
 * 32, 64 or 128 along head_dim, n = batch * kv_heads * max_len rows in the
 * order ((b * kv_heads) + kv) * max_len + t, k = 128.  k_cache and v_cache
 * must share format and group.
 *
 * For one new token per sequence, query head h of sequence b (q_fp16 fp16
 * [batch][q_heads][128]) attends to the first seq_lens[b] cached tokens of
 * KV head h / (q_heads / kv_heads):
 *   out[b][h] = sum_t p_t V_deq[b][kv][t],
 *   p = softmax_t(scale * <q[b][h], K_deq[b][kv][t]>)
 * with fp32 scores, exponentials and sums, rounded once to fp16 into
 * out_fp16 [batch][q_heads][128].  With group 128 the value sum runs on the
 * matrix cores: each weight p_t times its value row's scale, shifted by a
 * power of two that keeps the range's products below 2^15, enters as an fp16
 * pair (hi + lo), within about 2^-22 of the product.  seq_lens: device int32 [batch] (values
 * clamped to [0, max_len]; 0 gives a zero output), or NULL for max_len
 * everywhere.  workspace: caller-owned device memory of at least
 * q_attn_workspace_bytes bytes, no initialization needed, not shared by calls
 * that may overlap.  max_len is at most 2^20.  Errors: Q_ERR_FORMAT (format or group), Q_ERR_SHAPE
 * (shapes, a non-finite scale, a short workspace), Q_ERR_NULL, Q_ERR_ALIGN
 * (16 bytes; seq_lens 4), Q_ERR_HIP. */
size_t q_attn_workspace_bytes(int32_t batch, int32_t q_heads, int32_t kv_heads, int32_t max_len);
int q_attn_decode(const q_weight* k_cache, const q_weight* v_cache, const void* q_fp16, void* out_fp16,
                  int32_t batch, int32_t q_heads, int32_t kv_heads, int32_t max_len, const int32_t* seq_lens,
                  float scale, void* workspace, size_t workspace_bytes, void* stream);

/* W8A8 product over an INT8 weight (format Q_INT8): INT8 activations per
 * token times INT8 weights per output channel, on the vector ALU's int8 dot
 * products for b <= 2 (b = 2 up to 65536 rows) and on the int8 matrix cores
 * otherwise; every form gives the same bits
 * ("A Method for Layer Bit-Width Allocation in LLM Quantization via
 * Performance Maximization Under a Quality-Degradation Constraint",
 * abstract: W8A8 variants, integer arithmetic, a SmoothQuant
 * implementation).  For each activation row b, in IEEE binary32 with
 * round-to-nearest-even, one operation per step:
 *   a[k] = x[b][k] / smooth[k]   (a = x when smooth is NULL)
 *   s_x  = max_k |a[k]| / 127
 *   q[k] = clamp(rne(a[k] / s_x), -127, 127)   (0 when s_x = 0)
 *   y[b][n] = f16((s_x * s_w[n]) * f32(sum_k q[k] * q_w[n][k]))
 * with the integer sum exact and each product rounded to binary32 before
 * the one rounding to fp16 (the library matches this bit for bit).
 * smooth: optional device fp32 [k], positive
 * per-input-channel factors (4-byte aligned); the caller folds them into
 * the weights (W[n][k] * smooth[k]) before q_pack.  x fp16 [b][k], y fp16
 * [b][n], 1 <= b <= 64; x, y and workspace 16-byte aligned.  workspace:
 * caller-owned device memory of at least q_w8a8_workspace_bytes(b, k) bytes
 * (round16(b k) bytes of activation codes, then round16(4 b) bytes of fp32
 * scales; 0 is returned for b or k outside the limits), no initialization
 * needed, rewritten by every call that runs as two kernels (the b <= 4
 * calls that quantize inside the product leave it untouched; by default every
 * b = 1 call does), not shared by calls that may overlap.
 * Errors:
 * Q_ERR_FORMAT (not Q_INT8), Q_ERR_BATCH, Q_ERR_NULL, Q_ERR_ALIGN, Q_ERR_SHAPE
 * (shapes, a short workspace), Q_ERR_HIP.  Asynchronous on stream. */
size_t q_w8a8_workspace_bytes(int32_t b, int32_t k);
int q_gemm_w8a8(const q_weight* w, const void* x_fp16, const float* smooth, void* y_fp16, int32_t b, void* workspace,
                size_t workspace_bytes, void* stream);

/* Debug export: write W_deq [n][k] (fp16, row-major, 16-byte aligned,
 * caller-owned) decoded from the packed buffers of *w, each value formed
 * exactly in fp32 from its code and metadata (the value definitions listed
 * under q_pack) and rounded once to fp16.  The product calls never build this
 * matrix; it lets tests check a layout decode on the device against a
 * reference bit for bit.  Same status codes as q_pack; asynchronous on
 * stream. */
int q_dequant(const q_weight* w, void* out_fp16, void* stream);

/* Utility (not defined by the pages): static message for a q_status value. */
const char* q_strerror(int status);

/* Utility (not defined by the pages): library version as
 * major*10000 + minor*100 + patch. */
int q_version(void);

/* Utility for measurement and tests (not defined by the pages): launch-shape
 * overrides that force a kernel form or tile shape.  The library reads the
 * environment variables of these names (QGEMV_PATH, QGEMV_SPLIT_MIN_B,
 * QGEMV_SPLIT_KC, QGEMV_SPLIT_LDS, QGEMV_VALU_SHARE, QGEMV_ATTN_MFMA, ...)
 * once per process, at its first launch; q_tuning_set overrides one for
 * every later call, and q_tuning_clear(name) returns it to the library's
 * default (NULL: all of them), over any environment setting.  Results of
 * the product calls are the same whatever the tuning, up to fp32 summation
 * order.  Host-only, thread-safe; a change does not affect work already
 * enqueued, and a workspace must be sized (q_workspace_bytes) under the same
 * tuning as the call that uses it.  Errors: Q_ERR_NULL, Q_ERR_ARG. */
int q_tuning_set(const char* name, int32_t value);
int q_tuning_clear(const char* name);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
