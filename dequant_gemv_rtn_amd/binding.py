"""Thin ctypes binding over libqgemv.so (C ABI in include/qgemv.h).

Argument marshalling only: torch provides device memory and the current HIP
stream; every computation runs in the library's kernels.  There is no CPU
fallback -- a missing library or a CPU tensor raises.
"""

from __future__ import annotations

import contextlib
import ctypes
import os
import threading
from typing import Dict, Optional

import torch

from . import FORMATS

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqgemv.so")
_lib = None
_lock = threading.Lock()

BUFFERS = ("codes", "codes_hi", "scales", "aux")  # q_buffer order
Q_OK = 0


class QWeightDesc(ctypes.Structure):
    """Mirror of ``q_weight``."""

    _fields_ = [
        ("format", ctypes.c_int32),
        ("n", ctypes.c_int32),
        ("k", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("codes", ctypes.c_void_p),
        ("codes_hi", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("aux", ctypes.c_void_p),
    ]


class QStackEntry(ctypes.Structure):
    """Mirror of ``q_stack_entry``."""

    _fields_ = [
        ("w", QWeightDesc),
        ("x", ctypes.c_void_p),
        ("y", ctypes.c_void_p),
        ("stage", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


Q_STACK_CHAIN = 1
Q_STACK_ABORT_OFFSET = 68


class QError(RuntimeError):
    def __init__(self, call: str, status: int):
        super().__init__(f"{call} failed: {strerror(status)} (status {status})")
        self.status = status


def lib(build_if_missing: bool = True) -> ctypes.CDLL:
    """Load libqgemv.so, building it first if it is absent."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            if not build_if_missing:
                raise FileNotFoundError(f"{_LIB_PATH} is not built")
            from .build import build

            build(verbose=False)
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        L.q_packed_bytes.argtypes = [i32, i32, i32, i32, i32]
        L.q_packed_bytes.restype = ctypes.c_size_t
        L.q_pack.argtypes = [ctypes.POINTER(QWeightDesc), vp, vp]
        L.q_pack.restype = ctypes.c_int
        L.q_pack_clip.argtypes = [ctypes.POINTER(QWeightDesc), vp, ctypes.c_int32, vp]
        L.q_pack_clip.restype = ctypes.c_int
        L.q_gemv.argtypes = [ctypes.POINTER(QWeightDesc), vp, vp, vp]
        L.q_gemv.restype = ctypes.c_int
        L.q_gemm_skinny.argtypes = [ctypes.POINTER(QWeightDesc), vp, vp, i32, vp]
        L.q_gemm_skinny.restype = ctypes.c_int
        L.q_workspace_bytes.argtypes = [ctypes.POINTER(QWeightDesc), i32]
        L.q_workspace_bytes.restype = ctypes.c_size_t
        L.q_gemm_skinny_ws.argtypes = [ctypes.POINTER(QWeightDesc), vp, vp, i32, vp, ctypes.c_size_t, vp]
        L.q_gemm_skinny_ws.restype = ctypes.c_int
        L.q_gemm_skinny_noalloc.argtypes = [ctypes.POINTER(QWeightDesc), vp, vp, i32, vp]
        L.q_gemm_skinny_noalloc.restype = ctypes.c_int
        L.q_attn_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.q_attn_workspace_bytes.restype = ctypes.c_size_t
        L.q_attn_decode.argtypes = [ctypes.POINTER(QWeightDesc), ctypes.POINTER(QWeightDesc), vp, vp, i32, i32, i32,
                                    i32, vp, ctypes.c_float, vp, ctypes.c_size_t, vp]
        L.q_attn_decode.restype = ctypes.c_int
        L.q_w8a8_workspace_bytes.argtypes = [i32, i32]
        L.q_w8a8_workspace_bytes.restype = ctypes.c_size_t
        L.q_gemm_w8a8.argtypes = [ctypes.POINTER(QWeightDesc), vp, vp, vp, i32, vp, ctypes.c_size_t, vp]
        L.q_gemm_w8a8.restype = ctypes.c_int
        L.q_dequant.argtypes = [ctypes.POINTER(QWeightDesc), vp, vp]
        L.q_dequant.restype = ctypes.c_int
        L.q_strerror.argtypes = [ctypes.c_int]
        L.q_strerror.restype = ctypes.c_char_p
        L.q_version.argtypes = []
        L.q_version.restype = ctypes.c_int
        L.q_stack_plan_bytes.argtypes = [i32]
        L.q_stack_plan_bytes.restype = ctypes.c_size_t
        L.q_stack_plan.argtypes = [ctypes.POINTER(QStackEntry), i32, vp, ctypes.c_size_t]
        L.q_stack_plan.restype = ctypes.c_int
        L.q_gemv_stack.argtypes = [vp, i32, vp]
        L.q_gemv_stack.restype = ctypes.c_int
        L.q_tuning_set.argtypes = [ctypes.c_char_p, i32]
        L.q_tuning_set.restype = ctypes.c_int
        L.q_tuning_clear.argtypes = [ctypes.c_char_p]
        L.q_tuning_clear.restype = ctypes.c_int
        _lib = L
        return L


def lib_path() -> str:
    return _LIB_PATH


def strerror(status: int) -> str:
    return lib().q_strerror(int(status)).decode()


def set_tuning(name: str, value: int) -> None:
    """Override one launch-shape tuning key (q_tuning_set), e.g.
    set_tuning("QGEMV_PATH", 2) forces the streaming MFMA kernel."""
    st = lib().q_tuning_set(name.encode(), int(value))
    if st != Q_OK:
        raise QError("q_tuning_set", st)


def clear_tuning(name: Optional[str] = None) -> None:
    """Return one tuning key (None: all) to the library default."""
    st = lib().q_tuning_clear(None if name is None else name.encode())
    if st != Q_OK:
        raise QError("q_tuning_clear", st)


@contextlib.contextmanager
def tuning(**keys):
    """Context manager: tuning(QGEMV_PATH=2, QGEMV_SPLIT_MIN_B=0) sets the
    keys for the block and returns them to the default afterwards."""
    try:
        for name, value in keys.items():
            set_tuning(name, value)
        yield
    finally:
        for name in keys:
            clear_tuning(name)


def format_id(fmt) -> int:
    if isinstance(fmt, int):
        return fmt
    try:
        return FORMATS[fmt]
    except KeyError:
        raise ValueError(f"unknown format {fmt!r}; known: {sorted(FORMATS)}") from None


def packed_bytes(fmt, n: int, k: int, group: int) -> Dict[str, int]:
    f = format_id(fmt)
    return {name: int(lib().q_packed_bytes(f, n, k, group, i)) for i, name in enumerate(BUFFERS)}


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _require_device_fp16(t: torch.Tensor, what: str):
    if not t.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor (the library has no CPU path)")
    if t.dtype != torch.float16:
        raise ValueError(f"{what} must be float16")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")


class QWeight:
    """Packed weights: the descriptor plus the device buffers that own them."""

    def __init__(self, fmt, n: int, k: int, group: int, device="cuda", buffers=None):
        self.fmt = fmt if isinstance(fmt, str) else {v: s for s, v in FORMATS.items()}[fmt]
        self.n, self.k, self.group = int(n), int(k), int(group)
        self.device = torch.device(device)
        sizes = packed_bytes(self.fmt, self.n, self.k, self.group)
        if sizes["codes"] == 0:
            raise ValueError(f"invalid shape/format: {self.fmt} n={n} k={k} group={group}")
        self.sizes = sizes
        if buffers is None:
            buffers = {name: (torch.empty(sz, dtype=torch.uint8, device=self.device) if sz else None)
                       for name, sz in sizes.items()}
        self.buffers = buffers

    def desc(self) -> QWeightDesc:
        b = self.buffers
        return QWeightDesc(format_id(self.fmt), self.n, self.k, self.group,
                           _ptr(b["codes"]), _ptr(b["codes_hi"]), _ptr(b["scales"]), _ptr(b["aux"]))

    def nbytes(self) -> int:
        return sum(self.sizes.values())

    def to_host(self) -> Dict[str, Optional[torch.Tensor]]:
        return {k: (None if v is None else v.cpu()) for k, v in self.buffers.items()}


def _check_out_weight(out: QWeight, w: torch.Tensor, fmt, group: int) -> None:
    """A given output QWeight must describe exactly the weights being packed:
    the kernel reads out.n x out.k values of w in out's format."""
    if (out.n, out.k) != tuple(w.shape):
        raise ValueError(f"out is {out.n}x{out.k}, w is {tuple(w.shape)}")
    if format_id(out.fmt) != format_id(fmt) or out.group != int(group):
        raise ValueError(f"out is {out.fmt} group {out.group}, asked for {fmt} group {group}")
    for name, t in out.buffers.items():
        if t is not None and t.device != w.device:
            raise ValueError(f"out buffer {name} is on {t.device}, w on {w.device}")


def pack(w: torch.Tensor, fmt, group: int, out: Optional[QWeight] = None) -> QWeight:
    """RTN-quantize fp16 weights [n, k] on the GPU into a new (or given) QWeight."""
    _require_device_fp16(w, "w")
    if w.dim() != 2:
        raise ValueError("w must be [n, k]")
    n, k = w.shape
    if out is not None:
        _check_out_weight(out, w, fmt, group)
    qw = out if out is not None else QWeight(fmt, n, k, group, device=w.device)
    d = qw.desc()
    st = lib().q_pack(ctypes.byref(d), ctypes.c_void_p(w.data_ptr()), _stream(w.device))
    if st != Q_OK:
        raise QError("q_pack", st)
    return qw


def pack_clip(w: torch.Tensor, fmt, group: int, candidates: int, out: Optional[QWeight] = None) -> QWeight:
    """pack() with the per-group clipping search over `candidates` range
    ratios (20 - c) / 20 (the grouped 4-bit formats; 1 is plain pack)."""
    _require_device_fp16(w, "w")
    if w.dim() != 2:
        raise ValueError("w must be [n, k]")
    n, k = w.shape
    if out is not None:
        _check_out_weight(out, w, fmt, group)
    qw = out if out is not None else QWeight(fmt, n, k, group, device=w.device)
    d = qw.desc()
    st = lib().q_pack_clip(ctypes.byref(d), ctypes.c_void_p(w.data_ptr()), int(candidates), _stream(w.device))
    if st != Q_OK:
        raise QError("q_pack_clip", st)
    return qw


def workspace_bytes(qw: QWeight, b: int) -> int:
    """Device workspace bytes the K-split product uses for (qw, b); 0 when
    the call needs none."""
    d = qw.desc()
    return int(lib().q_workspace_bytes(ctypes.byref(d), int(b)))


# Eager calls without a workspace of their own share one per (device,
# stream), grown as needed: calls on one stream run in order, so they never
# overlap.  Calls under graph capture take a fresh one from the capture's
# pool instead (a cached buffer could outlive the graph's memory).
_ws_cache: Dict[tuple, torch.Tensor] = {}


def _cached_workspace(need: int, device: torch.device) -> torch.Tensor:
    if torch.cuda.is_current_stream_capturing():
        return torch.empty(need, dtype=torch.uint8, device=device)
    key = (device.index if device.index is not None else torch.cuda.current_device(),
           torch.cuda.current_stream(device).cuda_stream)
    with _lock:
        t = _ws_cache.get(key)
        if t is None or t.numel() < need:
            t = torch.empty(need, dtype=torch.uint8, device=device)
            _ws_cache[key] = t
        return t


def gemm_skinny(qw: QWeight, x: torch.Tensor, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[b, n] = sum_k W_deq[n, k] x[b, k] for x fp16 [b, k], 1 <= b <= 64.

    Where the library asks for a workspace (workspace_bytes > 0) one is used
    from a per-stream cache (eager calls) or torch's allocator (graph
    capture), unless `workspace` (a uint8 device tensor) is given; pass an
    empty tensor to run without one."""
    _require_device_fp16(x, "x")
    if x.dim() != 2 or x.shape[1] != qw.k:
        raise ValueError(f"x must be [b, {qw.k}]")
    b = x.shape[0]
    y = out if out is not None else torch.empty((b, qw.n), dtype=torch.float16, device=x.device)
    _require_device_fp16(y, "out")
    if tuple(y.shape) != (b, qw.n):
        raise ValueError("out has the wrong shape")
    if y.device != x.device:
        raise ValueError("out must be on x's device")
    d = qw.desc()
    if workspace is None:
        need = int(lib().q_workspace_bytes(ctypes.byref(d), b))
        workspace = _cached_workspace(need, x.device) if need else None
    elif not workspace.is_cuda or workspace.device != x.device:
        raise ValueError("workspace must be a GPU tensor on x's device")
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None and workspace.numel() else None
    ws_len = workspace.numel() * workspace.element_size() if ws_ptr is not None else 0
    st = lib().q_gemm_skinny_ws(ctypes.byref(d), ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                                b, ws_ptr, ws_len, _stream(x.device))
    if st != Q_OK:
        raise QError("q_gemm_skinny_ws", st)
    return y


def gemm_skinny_noalloc(qw: QWeight, x: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    """gemm_skinny on the library's static scratch (q_gemm_skinny_noalloc):
    for callers that cannot allocate; `out` must be given."""
    _require_device_fp16(x, "x")
    _require_device_fp16(out, "out")
    if x.dim() != 2 or x.shape[1] != qw.k or tuple(out.shape) != (x.shape[0], qw.n) or out.device != x.device:
        raise ValueError(f"x must be [b, {qw.k}] and out [b, {qw.n}] on x's device")
    d = qw.desc()
    st = lib().q_gemm_skinny_noalloc(ctypes.byref(d), ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                     x.shape[0], _stream(x.device))
    if st != Q_OK:
        raise QError("q_gemm_skinny_noalloc", st)
    return out


class StackPlan:
    """A decode stack run in one launch (q_stack_plan / q_gemv_stack).

    ``entries``: (QWeight, x fp16 [k], y fp16 [n], stage) in order; entries
    of one stage share x.  The plan is written on the host and copied once to
    x's device; it names the entries' device buffers, which this object keeps
    alive."""

    def __init__(self, entries):
        if not entries:
            raise ValueError("empty stack")
        L = lib()
        n = len(entries)
        arr = (QStackEntry * n)()
        self.refs = []
        dev = entries[0][1].device
        for i, (qw, x, y, stage) in enumerate(entries):
            _require_device_fp16(x, "x")
            _require_device_fp16(y, "y")
            if x.numel() != qw.k or y.numel() != qw.n or x.device != dev or y.device != dev:
                raise ValueError(f"entry {i}: x must hold {qw.k} and y {qw.n} values on {dev}")
            arr[i] = QStackEntry(qw.desc(), x.data_ptr(), y.data_ptr(), int(stage), 0)
            self.refs.append((qw, x, y))
        nbytes = int(L.q_stack_plan_bytes(n))
        if nbytes == 0:
            raise ValueError(f"{n} entries: outside 1 .. Q_MAX_STACK_ENTRIES")
        host = (ctypes.c_uint8 * nbytes)()
        st = L.q_stack_plan(arr, n, ctypes.cast(host, ctypes.c_void_p), nbytes)
        if st != Q_OK:
            raise QError("q_stack_plan", st)
        self.host = bytes(host)
        self.device = dev
        self.plan = torch.frombuffer(bytearray(self.host), dtype=torch.uint8).to(dev)

    def run(self, chain: bool = False) -> None:
        """One launch over every entry, on the current stream of the plan's
        device (chain: each stage waits for the one before)."""
        st = lib().q_gemv_stack(ctypes.c_void_p(self.plan.data_ptr()), Q_STACK_CHAIN if chain else 0,
                                _stream(self.device))
        if st != Q_OK:
            raise QError("q_gemv_stack", st)

    def aborted(self) -> bool:
        """Whether a chained launch gave up a stage wait (synchronizes)."""
        word = self.plan[Q_STACK_ABORT_OFFSET:Q_STACK_ABORT_OFFSET + 4].cpu().numpy().view("<u4")[0]
        return int(word) != 0


def w8a8_workspace_bytes(b: int, k: int) -> int:
    return int(lib().q_w8a8_workspace_bytes(int(b), int(k)))


def gemm_w8a8(qw: QWeight, x: torch.Tensor, smooth: Optional[torch.Tensor] = None,
              out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """W8A8 product over an INT8 weight: x fp16 [b, k] quantized per token
    to INT8 (after division by the optional fp32 [k] smoothing factors),
    integer products, y fp16 [b, n] (q_gemm_w8a8).  Unless `workspace` is
    given, the per-stream cache of gemm_skinny (eager calls) or torch's
    allocator (graph capture) provides it."""
    _require_device_fp16(x, "x")
    if x.dim() != 2 or x.shape[1] != qw.k:
        raise ValueError(f"x must be [b, {qw.k}]")
    b = x.shape[0]
    if smooth is not None and (not smooth.is_cuda or smooth.dtype != torch.float32 or tuple(smooth.shape) != (qw.k,)
                               or not smooth.is_contiguous()):
        raise ValueError(f"smooth must be a contiguous float32 GPU tensor of shape [{qw.k}]")
    y = out if out is not None else torch.empty((b, qw.n), dtype=torch.float16, device=x.device)
    _require_device_fp16(y, "out")
    if tuple(y.shape) != (b, qw.n):
        raise ValueError("out has the wrong shape")
    if workspace is None:
        workspace = _cached_workspace(max(1, w8a8_workspace_bytes(b, qw.k)), x.device)
    elif not workspace.is_cuda:
        raise ValueError("workspace must be a GPU tensor")
    d = qw.desc()
    st = lib().q_gemm_w8a8(ctypes.byref(d), ctypes.c_void_p(x.data_ptr()),
                           ctypes.c_void_p(smooth.data_ptr()) if smooth is not None else None,
                           ctypes.c_void_p(y.data_ptr()), b, ctypes.c_void_p(workspace.data_ptr()),
                           workspace.numel() * workspace.element_size(), _stream(x.device))
    if st != Q_OK:
        raise QError("q_gemm_w8a8", st)
    return y


def attn_workspace_bytes(batch: int, q_heads: int, kv_heads: int, max_len: int) -> int:
    return int(lib().q_attn_workspace_bytes(batch, q_heads, kv_heads, max_len))


def pack_kv(cache: torch.Tensor, fmt="fp4_razer", group: int = 128) -> QWeight:
    """Quantize a KV cache fp16 [B, Hkv, L, 128] with q_pack, one row per
    cached vector (row ((b * Hkv) + kv) * L + t)."""
    _require_device_fp16(cache, "cache")
    if cache.dim() != 4 or cache.shape[-1] != 128:
        raise ValueError("cache must be [B, Hkv, L, 128]")
    return pack(cache.reshape(-1, 128), fmt, group)


def _check_attn_io(q: torch.Tensor, y: torch.Tensor, k_cache: QWeight, v_cache: QWeight,
                   seq_lens: Optional[torch.Tensor], workspace: torch.Tensor) -> None:
    """q_attn_decode writes B * Hq * 128 fp16 values to y and reads the caches,
    seq_lens and the workspace: all must be on q's device, y shaped as q."""
    if tuple(y.shape) != tuple(q.shape) or y.device != q.device:
        raise ValueError(f"out must be [B, Hq, 128] = {tuple(q.shape)} on q's device")
    for name, cache in (("k_cache", k_cache), ("v_cache", v_cache)):
        for t in cache.buffers.values():
            if t is not None and t.device != q.device:
                raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    if seq_lens is not None and (seq_lens.dtype != torch.int32 or seq_lens.numel() != q.shape[0]
                                 or seq_lens.device != q.device):
        raise ValueError("seq_lens must be an int32 tensor of B entries on q's device")
    if workspace.device != q.device:
        raise ValueError("workspace must be on q's device")


def attn_decode(k_cache: QWeight, v_cache: QWeight, q: torch.Tensor, kv_heads: int, max_len: int,
                seq_lens: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[b, h] = softmax_t(scale <q[b, h], K[b, kv, t]>) . V[b, kv, t] over the
    first seq_lens[b] tokens, kv = h // (Hq // kv_heads); q fp16 [B, Hq, 128];
    caches from pack_kv; scale defaults to 1 / sqrt(128)."""
    _require_device_fp16(q, "q")
    if q.dim() != 3 or q.shape[2] != 128:
        raise ValueError("q must be [B, Hq, 128]")
    B, Hq, _ = q.shape
    y = out if out is not None else torch.empty_like(q)
    _require_device_fp16(y, "out")
    if workspace is None:
        workspace = torch.empty(attn_workspace_bytes(B, Hq, kv_heads, max_len), dtype=torch.uint8, device=q.device)
    _check_attn_io(q, y, k_cache, v_cache, seq_lens, workspace)
    kd, vd = k_cache.desc(), v_cache.desc()
    st = lib().q_attn_decode(ctypes.byref(kd), ctypes.byref(vd), ctypes.c_void_p(q.data_ptr()),
                             ctypes.c_void_p(y.data_ptr()), B, Hq, kv_heads, max_len,
                             None if seq_lens is None else ctypes.c_void_p(seq_lens.data_ptr()),
                             float(128 ** -0.5 if scale is None else scale), ctypes.c_void_p(workspace.data_ptr()),
                             workspace.numel(), _stream(q.device))
    if st != Q_OK:
        raise QError("q_attn_decode", st)
    return y


def gemv(qw: QWeight, x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[n] = sum_k W_deq[n, k] x[k] for x fp16 [k]."""
    _require_device_fp16(x, "x")
    if x.dim() != 1 or x.shape[0] != qw.k:
        raise ValueError(f"x must be [{qw.k}]")
    y = out if out is not None else torch.empty((qw.n,), dtype=torch.float16, device=x.device)
    _require_device_fp16(y, "out")
    d = qw.desc()
    st = lib().q_gemv(ctypes.byref(d), ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                      _stream(x.device))
    if st != Q_OK:
        raise QError("q_gemv", st)
    return y


def dequant(qw: QWeight, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """W_deq [n, k] fp16 decoded on the device from the packed buffers (a
    debug and test aid; the product calls never build this matrix)."""
    dev = qw.buffers["codes"].device
    y = out if out is not None else torch.empty((qw.n, qw.k), dtype=torch.float16, device=dev)
    _require_device_fp16(y, "out")
    if tuple(y.shape) != (qw.n, qw.k):
        raise ValueError("out has the wrong shape")
    d = qw.desc()
    st = lib().q_dequant(ctypes.byref(d), ctypes.c_void_p(y.data_ptr()), _stream(dev))
    if st != Q_OK:
        raise QError("q_dequant", st)
    return y


def linear(x: torch.Tensor, qw: QWeight, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = x W_deq^T for x fp16 [..., k] with at most 64 rows in the leading
    dimensions (flattened); the result has shape [..., n]."""
    lead = x.shape[:-1]
    x2 = x.reshape(-1, x.shape[-1])
    y2 = gemm_skinny(qw, x2, out=None if out is None else out.view(-1, qw.n))
    return y2.view(*lead, qw.n)
