"""Host-side checks of the C-ABI library (no GPU needed, no compute calls).

* libqgemv.so loads and exports every function include/qgemv.h declares;
* q_packed_bytes agrees with the oracle's buffer sizes for every format
  (packed bytes rounded up to a multiple of 16);
* argument validation returns the documented status before touching HIP
  (fake, never-dereferenced pointers are enough for that).
"""

from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest
import torch

import oracle
from dequant_gemv_rtn_amd import FORMATS, binding, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemv.h")

Q_OK, Q_ERR_NULL, Q_ERR_SHAPE, Q_ERR_ALIGN, Q_ERR_FORMAT, Q_ERR_BATCH, Q_ERR_HIP = 0, -1, -2, -3, -4, -5, -6


def _header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\*?\s+\*?(q_[a-z0-9_]+)\(", text, re.M)))


def test_header_declares_the_boundary():
    fns = _header_functions()
    for name in ("q_pack", "q_gemv", "q_gemm_skinny", "q_gemm_skinny_ws", "q_workspace_bytes", "q_dequant",
                 "q_packed_bytes", "q_strerror", "q_version", "q_attn_workspace_bytes", "q_attn_decode",
                 "q_w8a8_workspace_bytes", "q_gemm_w8a8", "q_pack_clip", "q_tuning_set", "q_tuning_clear"):
        assert name in fns


def test_library_exports_every_declared_symbol():
    L = binding.lib()
    for name in _header_functions():
        assert hasattr(L, name), name


def test_header_enums_match_binding():
    text = open(HEADER).read()
    for name, val in (("Q_INT4_ASYM", 1), ("Q_FP4_E2M1", 2), ("Q_FP4_RAZER", 3), ("Q_FP4_AFPQ", 4),
                      ("Q_BFP6", 5), ("Q_BFP4", 6), ("Q_INT8", 7), ("Q_FP3_RAZER", 8), ("Q_FP3_AFPQ", 9)):
        assert re.search(rf"{name}\s*=\s*{val}\b", text)
    assert FORMATS == {"int4_asym": 1, "fp4_e2m1": 2, "fp4_razer": 3, "fp4_afpq": 4,
                       "bfp6": 5, "bfp4": 6, "int8": 7, "fp3_razer": 8, "fp3_afpq": 9}


SHAPES = [(1, 32), (7, 96), (33, 4096), (11008, 4096), (28672, 8192), (13824, 5120), (128256, 4096), (5, 16384)]


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_packed_bytes_match_oracle(fmt):
    for n, k in SHAPES:
        groups = {"bfp6": [16], "bfp4": [16], "int8": [k]}.get(fmt, [32, 64, 128, 256])
        for g in groups:
            if k % g:
                assert binding.packed_bytes(fmt, n, k, g)["codes"] == 0
                continue
            got = binding.packed_bytes(fmt, n, k, g)
            assert got == oracle.buffer_nbytes(fmt, n, k, g), (fmt, n, k, g)
            for name, v in got.items():
                assert v % 16 == 0 and v - oracle.packed_nbytes(fmt, n, k, g)[name] < 16


def test_packed_bytes_rejects_bad_arguments():
    L = binding.lib()
    assert L.q_packed_bytes(99, 4, 128, 128, 0) == 0
    assert L.q_packed_bytes(1, 0, 128, 128, 0) == 0
    assert L.q_packed_bytes(1, 4, 100, 4, 0) == 0       # k % 32
    assert L.q_packed_bytes(1, 4, 32768, 128, 0) == 0   # k > Q_MAX_K
    assert L.q_packed_bytes(1, 4, 128, 48, 0) == 0      # group not allowed
    assert L.q_packed_bytes(5, 4, 128, 32, 0) == 0      # block formats need 16
    assert L.q_packed_bytes(7, 4, 128, 64, 0) == 0      # int8 needs group == k
    assert L.q_packed_bytes(1, 4, 128, 128, 4) == 0     # no such buffer
    # every packed buffer must stay below 4 GiB (32-bit buffer offsets)
    assert L.q_packed_bytes(7, 262143, 16384, 16384, 0) == 262143 * 16384
    assert L.q_packed_bytes(7, 262144, 16384, 16384, 0) == 0
    assert L.q_packed_bytes(7, 262144, 16384, 16384, 2) == 0
    assert L.q_packed_bytes(1, 524287, 16384, 128, 0) == 524287 * 8192
    assert L.q_packed_bytes(1, 524288, 16384, 128, 0) == 0


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation returns first


def _desc(fmt=1, n=4, k=128, g=128, codes=FAKE, hi=None, scales=FAKE, aux=FAKE):
    return binding.QWeightDesc(fmt, n, k, g, codes, hi, scales, aux)


def _gemm(desc, x=FAKE, y=FAKE, b=1):
    return binding.lib().q_gemm_skinny(None if desc is None else ctypes.byref(desc), x, y, b, None)


def test_validation_statuses():
    L = binding.lib()
    assert _gemm(None) == Q_ERR_NULL
    assert _gemm(_desc(fmt=0)) == Q_ERR_FORMAT
    assert _gemm(_desc(fmt=10)) == Q_ERR_FORMAT
    assert _gemm(_desc(n=0)) == Q_ERR_SHAPE
    assert _gemm(_desc(k=100, g=4)) == Q_ERR_SHAPE
    assert _gemm(_desc(k=160, g=64)) == Q_ERR_SHAPE     # group does not divide k
    assert _gemm(_desc(k=32768, g=128)) == Q_ERR_SHAPE  # above Q_MAX_K
    assert _gemm(_desc(n=262144, k=16384, g=16384, fmt=7)) == Q_ERR_SHAPE  # 4 GiB of int8 codes
    # the output is addressed with 32-bit offsets as well: b * n * 2 <= 0xFFFFFF00
    assert _gemm(_desc(n=1 << 26, k=32, g=32), b=32) == Q_ERR_SHAPE
    assert _gemm(_desc(g=48)) == Q_ERR_FORMAT
    assert _gemm(_desc(fmt=5, g=32)) == Q_ERR_FORMAT
    assert _gemm(_desc(fmt=7, g=64)) == Q_ERR_FORMAT
    assert _gemm(_desc(codes=None)) == Q_ERR_NULL
    assert _gemm(_desc(scales=None)) == Q_ERR_NULL
    assert _gemm(_desc(aux=None)) == Q_ERR_NULL             # int4 needs zero-points
    assert _gemm(_desc(fmt=5, g=16, hi=None)) == Q_ERR_NULL  # bfp6 needs the high plane
    assert _gemm(_desc(codes=FAKE + 4)) == Q_ERR_ALIGN
    assert _gemm(_desc(), x=FAKE + 2) == Q_ERR_ALIGN
    assert _gemm(_desc(), y=None) == Q_ERR_NULL
    assert _gemm(_desc(), b=0) == Q_ERR_BATCH
    assert _gemm(_desc(), b=65) == Q_ERR_BATCH
    assert L.q_gemv(None, FAKE, FAKE, None) == Q_ERR_NULL
    assert L.q_dequant(None, FAKE, None) == Q_ERR_NULL
    assert L.q_dequant(ctypes.byref(_desc()), None, None) == Q_ERR_NULL
    assert L.q_dequant(ctypes.byref(_desc()), FAKE + 2, None) == Q_ERR_ALIGN
    assert L.q_dequant(ctypes.byref(_desc(fmt=10)), FAKE, None) == Q_ERR_FORMAT
    assert L.q_dequant(ctypes.byref(_desc(k=100, g=4)), FAKE, None) == Q_ERR_SHAPE
    assert L.q_pack(ctypes.byref(_desc()), None, None) == Q_ERR_NULL
    assert L.q_pack(ctypes.byref(_desc()), FAKE + 8, None) == Q_ERR_ALIGN
    assert L.q_pack(ctypes.byref(_desc(fmt=10)), FAKE, None) == Q_ERR_FORMAT


def _ws_bytes(desc, b):
    return binding.lib().q_workspace_bytes(None if desc is None else ctypes.byref(desc), b)


def test_workspace_bytes_plan(tune):
    """The K-split plan: one fp32 slot of 256 outputs per batch tile, row tile
    and K-part, a part being 8 chunks of 128 (16 for groups of 256); no
    workspace below the minimum batch (here forced to 16), for K within one
    part, or for invalid arguments."""
    tune.set("QGEMV_SPLIT_MIN_B", "16")
    razer = _desc(fmt=3, n=11008, k=4096, g=128)
    assert [_ws_bytes(razer, b) for b in (1, 8, 15)] == [0, 0, 0]
    assert _ws_bytes(razer, 16) == 4 * 688 * 1 * 1024
    assert _ws_bytes(razer, 17) == 4 * 688 * 2 * 1024
    assert _ws_bytes(razer, 64) == 4 * 688 * 4 * 1024
    assert _ws_bytes(_desc(fmt=1, n=100, k=1024, g=128), 64) == 0           # one part
    assert _ws_bytes(_desc(fmt=1, n=100, k=1056, g=32), 64) == 2 * 7 * 4 * 1024
    assert _ws_bytes(_desc(fmt=1, n=40, k=5120, g=256), 32) == 3 * 3 * 2 * 1024  # 2 chunks per wave
    assert _ws_bytes(_desc(fmt=7, n=19, k=14336, g=14336), 16) == 14 * 2 * 1024
    # 2 chunks per wave: INT4 / E2M1 / RaZeR above k = 8192; from two batch
    # tiles INT8 too, and 32 MiB of packed weights
    int4_long = _desc(fmt=1, n=19, k=14336, g=128)
    assert _ws_bytes(int4_long, 16) == 7 * 2 * 1024
    assert _ws_bytes(int4_long, 17) == 7 * 2 * 2 * 1024
    assert _ws_bytes(int4_long, 64) == 7 * 2 * 4 * 1024
    int8_long = _desc(fmt=7, n=19, k=14336, g=14336)
    assert _ws_bytes(int8_long, 16) == 14 * 2 * 1024 and _ws_bytes(int8_long, 32) == 7 * 2 * 2 * 1024
    assert _ws_bytes(razer, 32) == 4 * 688 * 2 * 1024                       # 22.5 MiB: one chunk
    int4_big = _desc(fmt=1, n=28672, k=4096, g=128)                           # 58.7 MiB
    assert _ws_bytes(int4_big, 16) == 4 * 1792 * 1024 and _ws_bytes(int4_big, 32) == 2 * 1792 * 2 * 1024
    assert _ws_bytes(int4_big, 64) == 2 * 1792 * 4 * 1024
    assert _ws_bytes(razer, 64) == 4 * 688 * 4 * 1024                       # 22.5 MiB: one chunk
    tune.set("QGEMV_SPLIT_KC", "1")
    assert _ws_bytes(int4_long, 16) == 14 * 2 * 1024 and _ws_bytes(int4_big, 32) == 4 * 1792 * 2 * 1024
    tune.set("QGEMV_SPLIT_KC", "2")
    assert _ws_bytes(razer, 16) == 2 * 688 * 1024 and _ws_bytes(razer, 32) == 2 * 688 * 2 * 1024
    assert _ws_bytes(razer, 33) == 2 * 688 * 3 * 1024
    tune.clear("QGEMV_SPLIT_KC")
    assert _ws_bytes(None, 16) == 0
    assert _ws_bytes(razer, 0) == 0 and _ws_bytes(razer, 65) == 0
    assert _ws_bytes(_desc(fmt=3, n=11008, k=4096, g=48), 16) == 0
    tune.set("QGEMV_SPLIT_MIN_B", "0")
    assert _ws_bytes(razer, 64) == 0
    tune.set("QGEMV_SPLIT_MIN_B", "2")
    assert _ws_bytes(razer, 2) == 4 * 688 * 1024 and _ws_bytes(razer, 1) == 0


def test_workspace_default_routing(tune):
    """Default minimum batch of the split form: block formats from b = 8;
    K above 8192 from b = 16 for AFPQ and INT8, else from b = 4, 16 and 8 for
    groups of 32, 64 and 128 or more; AFPQ from b = 17 (two batch tiles);
    other formats from b = 17 when the packed matrix holds 16 MiB or more,
    else never."""
    tune.clear("QGEMV_SPLIT_MIN_B")
    tune.clear("QGEMV_SPLIT_KC")

    def first_b(desc):
        return next((b for b in range(1, 65) if _ws_bytes(desc, b)), None)

    assert first_b(_desc(fmt=5, n=13824, k=5120, g=16, hi=FAKE)) == 8
    assert first_b(_desc(fmt=6, n=100, k=2048, g=16)) == 8
    assert first_b(_desc(fmt=1, n=4096, k=14336, g=128)) == 8
    assert first_b(_desc(fmt=3, n=5120, k=13824, g=32)) == 4
    assert first_b(_desc(fmt=2, n=4096, k=14336, g=64)) == 16
    assert first_b(_desc(fmt=4, n=4096, k=14336, g=64)) == 16
    assert first_b(_desc(fmt=7, n=4096, k=14336, g=14336)) == 16
    assert first_b(_desc(fmt=4, n=28672, k=8192, g=64)) == 17
    assert first_b(_desc(fmt=3, n=11008, k=4096, g=128)) == 17   # 22.5 MiB
    assert first_b(_desc(fmt=7, n=128256, k=4096, g=4096)) == 17
    assert first_b(_desc(fmt=1, n=6144, k=4096, g=128)) is None  # 12.6 MiB
    assert first_b(_desc(fmt=1, n=4096, k=1024, g=128)) is None  # one part


def test_workspace_call_statuses():
    L = binding.lib()
    ws = lambda desc, **kw: L.q_gemm_skinny_ws(  # noqa: E731
        None if desc is None else ctypes.byref(desc), kw.get("x", FAKE), kw.get("y", FAKE), kw.get("b", 16),
        kw.get("ws", FAKE), kw.get("nbytes", 1 << 20), None)
    assert ws(None) == Q_ERR_NULL
    assert ws(_desc(fmt=0)) == Q_ERR_FORMAT
    assert ws(_desc(), b=0) == Q_ERR_BATCH
    assert ws(_desc(), x=None) == Q_ERR_NULL
    assert ws(_desc(), ws=FAKE + 4) == Q_ERR_ALIGN
    assert ws(_desc(n=1 << 26, k=32, g=32), b=32) == Q_ERR_SHAPE


def test_attention_workspace_and_statuses():
    """Attention: workspace = B * Hq * ranges * (128 + 2) floats, ranges of a
    power of two from 128 to 1024 tokens aiming at 512 workgroups; argument
    errors return their status before any device work."""
    L = binding.lib()
    # B=1, Hq=32, Hkv=8 (4 heads per workgroup): 8 units -> 64 ranges wanted -> 128-token floor -> 32 ranges
    assert L.q_attn_workspace_bytes(1, 32, 8, 4096) == 1 * 32 * 32 * 130 * 4
    # B=8: 64 units -> 8 ranges wanted -> 512-token ranges
    assert L.q_attn_workspace_bytes(8, 32, 8, 4096) == 8 * 32 * 8 * 130 * 4
    # long sequences cap the range at 1024 tokens
    assert L.q_attn_workspace_bytes(64, 32, 8, 32768) == 64 * 32 * 32 * 130 * 4
    for bad in ((0, 8, 8, 16), (1, 6, 4, 16), (1, 2, 4, 16), (1, 8, 8, 0), (1, 8, 8, (1 << 20) + 1)):
        assert L.q_attn_workspace_bytes(*bad) == 0
    B, Hq, Hkv, T = 2, 8, 2, 64
    rows = B * Hkv * T
    k = _desc(fmt=3, n=rows, k=128, g=128)
    v = _desc(fmt=3, n=rows, k=128, g=128)

    def call(kd=k, vd=v, q=FAKE, out=FAKE, b=B, hq=Hq, hkv=Hkv, t=T, lens=None, scale=0.1, ws=FAKE, nb=1 << 20):
        return L.q_attn_decode(None if kd is None else ctypes.byref(kd), None if vd is None else ctypes.byref(vd),
                               q, out, b, hq, hkv, t, lens, ctypes.c_float(scale), ws, nb, None)

    assert call(kd=None) == Q_ERR_NULL
    assert call(kd=_desc(fmt=1, n=rows, k=128, g=128)) == Q_ERR_FORMAT          # INT4 cache
    assert call(vd=_desc(fmt=2, n=rows, k=128, g=128)) == Q_ERR_FORMAT          # formats differ
    assert call(kd=_desc(fmt=3, n=rows, k=256, g=256), vd=_desc(fmt=3, n=rows, k=256, g=256)) == Q_ERR_FORMAT
    assert call(kd=_desc(fmt=3, n=rows + 1, k=128, g=128)) == Q_ERR_SHAPE        # rows != B*Hkv*T
    assert call(hq=7) == Q_ERR_SHAPE                                              # not a multiple of Hkv
    assert call(q=None) == Q_ERR_NULL
    assert call(ws=None) == Q_ERR_NULL
    assert call(out=FAKE + 2) == Q_ERR_ALIGN
    assert call(lens=FAKE + 2) == Q_ERR_ALIGN
    assert call(scale=float("inf")) == Q_ERR_SHAPE
    assert call(nb=L.q_attn_workspace_bytes(B, Hq, Hkv, T) - 1) == Q_ERR_SHAPE


def test_strerror_and_version():
    for st in (Q_OK, Q_ERR_NULL, Q_ERR_SHAPE, Q_ERR_ALIGN, Q_ERR_FORMAT, Q_ERR_BATCH, Q_ERR_HIP):
        assert binding.strerror(st)
    assert binding.strerror(-99) == "unknown status"
    assert binding.lib().q_version() >= 100


def test_binding_refuses_cpu_tensors():
    import torch
    w = torch.zeros((4, 128), dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        binding.pack(w, "int4_asym", 128)


def test_oracle_and_library_share_no_code():
    """The oracle imports nothing from the product package and vice versa."""
    pkg = os.path.join(ROOT, "dequant_gemv_rtn_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", text, re.M), f
                assert "oracle/" not in text, f
    for dirpath, _, files in os.walk(os.path.join(ROOT, "oracle")):
        for f in files:
            if f.endswith(".py"):
                text = open(os.path.join(dirpath, f)).read()
                assert "dequant_gemv_rtn_amd" not in text, f
    # the oracle module itself is numpy-only
    assert np is not None


def test_stack_fusion_groups_shared_input_linears():
    from dequant_gemv_rtn_amd import stack, synth
    layers = synth.WORKLOADS["llama3_8b_decode_stack"].layers
    groups = stack.fuse_layers(layers)
    assert len(groups) == 32 * 4 + 1  # q|k|v, o, gate|up, down per layer, plus lm_head
    names = [n for n, _ in groups]
    assert names[:4] == ["l0.q_k_v", "l0.o", "l0.gate_up", "l0.down"] and names[-1] == "lm_head"
    flat = [m.name for _, ms in groups for m in ms]
    assert flat == [l.name for l in layers]  # every linear once, in order
    for _, ms in groups:
        assert len({(m.k, m.fmt, m.group) for m in ms}) == 1


def test_precision_map_reproduces_the_stack_workload():
    """The decode-stack workload's per-linear formats follow the selective
    rule that PrecisionMap states (first/last two decoder layers and the
    output head in INT8 per channel, INT4 g128 elsewhere)."""
    from dequant_gemv_rtn_amd import stack

    pm = stack.PrecisionMap()
    layers = synth.WORKLOADS["llama3_8b_decode_stack"].layers
    assert len(layers) == 32 * 7 + 1
    for l in layers:
        assert pm.for_layer(l.name, l.k) == (l.fmt, l.group), l.name
    assert sum(pm.is_high(l.name) for l in layers) == 4 * 7 + 1


def test_w8a8_workspace_and_statuses():
    """W8A8: workspace = b * k activation codes then b fp32 scales, each part
    rounded up to 16 bytes; argument errors return their status before any
    device work."""
    L = binding.lib()
    assert L.q_w8a8_workspace_bytes(1, 4096) == 4096 + 16
    assert L.q_w8a8_workspace_bytes(3, 4128) == (3 * 4128 + 15) // 16 * 16 + 16
    assert L.q_w8a8_workspace_bytes(64, 16384) == 64 * 16384 + 256
    for bad in ((0, 4096), (65, 4096), (1, 16), (1, 4100), (1, 16416)):
        assert L.q_w8a8_workspace_bytes(*bad) == 0
    w = _desc(fmt=7, n=100, k=4096, g=4096)

    def call(wd=w, x=FAKE, sm=None, y=FAKE, b=4, ws=FAKE, nb=1 << 20):
        return L.q_gemm_w8a8(None if wd is None else ctypes.byref(wd), x, sm, y, b, ws, nb, None)

    assert call(wd=None) == Q_ERR_NULL
    assert call(wd=_desc(fmt=1, n=100, k=4096, g=128)) == Q_ERR_FORMAT      # not INT8
    assert call(b=0) == Q_ERR_BATCH and call(b=65) == Q_ERR_BATCH
    assert call(x=None) == Q_ERR_NULL and call(y=None) == Q_ERR_NULL and call(ws=None) == Q_ERR_NULL
    assert call(x=FAKE + 2) == Q_ERR_ALIGN and call(ws=FAKE + 8) == Q_ERR_ALIGN
    assert call(sm=FAKE + 2) == Q_ERR_ALIGN                                   # smoothing factors: 4 bytes
    assert call(nb=4 * 4096) == Q_ERR_SHAPE                                    # the scales' 16 bytes short


def test_noalloc_statuses():
    """q_gemm_skinny_noalloc: q_gemm_skinny_ws's argument checks, and
    Q_ERR_SCRATCH, before anything is launched, for a call whose K-split
    workspace would exceed Q_NOALLOC_SCRATCH_BYTES (64 MiB)."""
    L = binding.lib()
    Q_ERR_SCRATCH = -8
    assert "Q_NOALLOC_SCRATCH_BYTES (64u << 20)" in open(HEADER).read()

    def call(wd, b=64, x=FAKE, y=FAKE):
        return L.q_gemm_skinny_noalloc(None if wd is None else ctypes.byref(wd), x, y, b, None)

    big = _desc(fmt=7, n=65536, k=16384, g=16384)  # 8 parts x 4096 tiles x 4 batch tiles x 1 KiB = 128 MiB
    assert _ws_bytes(big, 64) > (64 << 20)
    assert call(big) == Q_ERR_SCRATCH
    assert call(None) == Q_ERR_NULL
    assert call(_desc(fmt=3, n=11008, k=4096, g=128), b=0) == Q_ERR_BATCH
    assert call(_desc(fmt=3, n=11008, k=4096, g=128), b=65) == Q_ERR_BATCH
    assert call(_desc(fmt=3, n=11008, k=4096, g=48)) == Q_ERR_FORMAT
    assert call(_desc(fmt=3, n=11008, k=4096, g=128), x=None) == Q_ERR_NULL
    assert call(_desc(fmt=3, n=11008, k=4096, g=128), y=FAKE + 2) == Q_ERR_ALIGN


def test_pack_clip_statuses():
    """q_pack_clip: the grouped 4-bit formats only, 1 .. Q_MAX_CLIP_CANDIDATES
    candidates; argument errors return their status before any device work."""
    L = binding.lib()

    def call(wd, cands=4, src=FAKE):
        return L.q_pack_clip(None if wd is None else ctypes.byref(wd), src, cands, None)

    w4 = _desc(fmt=1, n=100, k=4096, g=128)
    assert call(None) == Q_ERR_NULL
    for fmt in (5, 6, 7):  # the block formats, INT8
        g = {5: 16, 6: 16, 7: 4096}.get(fmt, 128)
        assert call(_desc(fmt=fmt, n=100, k=4096, g=g, hi=FAKE if fmt == 5 else None)) == Q_ERR_FORMAT
    assert call(w4, cands=0) == Q_ERR_SHAPE and call(w4, cands=11) == Q_ERR_SHAPE
    assert call(w4, src=None) == Q_ERR_NULL and call(w4, src=FAKE + 2) == Q_ERR_ALIGN
    for fmt in (2, 3, 4):  # E2M1, RaZeR, AFPQ: accepted up to the pointer check
        assert call(_desc(fmt=fmt, n=100, k=4096, g=128), src=None) == Q_ERR_NULL


Q_ERR_ARG = -7


def test_tuning_calls(tune):
    """q_tuning_set / q_tuning_clear: unknown names and NULL return their
    status; a set key changes the plan every later call sees (here the
    K-split workspace), and clearing returns the default."""
    L = binding.lib()
    assert L.q_tuning_set(b"QGEMV_NO_SUCH_KEY", 1) == Q_ERR_ARG
    assert L.q_tuning_clear(b"QGEMV_NO_SUCH_KEY") == Q_ERR_ARG
    assert L.q_tuning_set(None, 1) == Q_ERR_NULL
    razer = _desc(fmt=3, n=11008, k=4096, g=128)
    default = _ws_bytes(razer, 16)
    tune.set("QGEMV_SPLIT_MIN_B", 2)
    assert _ws_bytes(razer, 2) == 4 * 688 * 1024
    tune.set("QGEMV_SPLIT_MIN_B", 0)
    assert _ws_bytes(razer, 16) == 0
    tune.clear("QGEMV_SPLIT_MIN_B")
    assert _ws_bytes(razer, 16) == default
    with binding.tuning(QGEMV_SPLIT_MIN_B=2):
        assert _ws_bytes(razer, 2) > 0
    assert _ws_bytes(razer, 2) == 0
    assert L.q_tuning_clear(None) == Q_OK


def test_pack_out_must_match_the_weights():
    """pack(w, out=...) rejects an output QWeight of another shape, format,
    group or device (the kernel reads out.n x out.k values of w in out's
    format).  Checked on CPU tensors: the check runs before any device work."""
    w = torch.zeros((64, 256), dtype=torch.float16)
    ok = binding.QWeight("int4_asym", 64, 256, 128, device="cpu")
    binding._check_out_weight(ok, w, "int4_asym", 128)
    for bad, fmt, g in ((binding.QWeight("int4_asym", 128, 256, 128, device="cpu"), "int4_asym", 128),
                        (binding.QWeight("int4_asym", 64, 512, 128, device="cpu"), "int4_asym", 128),
                        (ok, "fp4_e2m1", 128),
                        (ok, "int4_asym", 64)):
        with pytest.raises(ValueError):
            binding._check_out_weight(bad, w, fmt, g)
    with pytest.raises(ValueError):
        binding._check_out_weight(ok, w.to("meta"), "int4_asym", 128)


def test_attn_io_checks():
    """attn_decode rejects an output of another shape or device, and caches,
    lengths or workspace on another device than q."""
    q = torch.zeros((2, 8, 128), dtype=torch.float16)
    kc = binding.QWeight("fp4_razer", 2 * 2 * 16, 128, 128, device="cpu")
    vc = binding.QWeight("fp4_razer", 2 * 2 * 16, 128, 128, device="cpu")
    lens = torch.tensor([16, 3], dtype=torch.int32)
    ws = torch.empty(64, dtype=torch.uint8)
    binding._check_attn_io(q, torch.empty_like(q), kc, vc, lens, ws)
    cases = [dict(y=torch.empty((2, 4, 128), dtype=torch.float16)),
             dict(y=torch.empty_like(q).to("meta")),
             dict(kc=binding.QWeight("fp4_razer", 64, 128, 128, device="meta")),
             dict(lens=torch.tensor([16], dtype=torch.int32)),
             dict(lens=lens.to("meta")),
             dict(ws=ws.to("meta"))]
    for c in cases:
        with pytest.raises(ValueError):
            binding._check_attn_io(q, c.get("y", torch.empty_like(q)), c.get("kc", kc), vc, c.get("lens", lens),
                                   c.get("ws", ws))


_NO_DEVICE_PROBE = r"""
import ctypes, sys
hip = ctypes.CDLL("libamdhip64.so")
count = ctypes.c_int(0)
if hip.hipGetDeviceCount(ctypes.byref(count)) == 0 and count.value > 0:
    sys.exit(77)  # a device is visible: nothing is launched
from dequant_gemv_rtn_amd import binding
L = binding.lib(build_if_missing=False)
d = binding.QWeightDesc(1, 64, 128, 128, 0x10000, None, 0x20000, 0x30000)
print(L.q_gemv(ctypes.byref(d), ctypes.c_void_p(0x40000), ctypes.c_void_p(0x50000), None),
      L.q_pack(ctypes.byref(d), ctypes.c_void_p(0x40000), None))
"""


def test_no_device_returns_hip_error():
    """With no device visible (HIP_VISIBLE_DEVICES=-1 set before the library
    loads, in a fresh process), calls whose arguments pass validation return
    Q_ERR_HIP.  Skipped when a device is visible anyway: nothing launches."""
    import subprocess
    import sys

    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    res = subprocess.run([sys.executable, "-c", _NO_DEVICE_PROBE], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=120)
    if res.returncode == 77:
        pytest.skip("a device is visible despite HIP_VISIBLE_DEVICES=-1")
    assert res.returncode == 0, res.stderr
    assert res.stdout.split() == [str(Q_ERR_HIP), str(Q_ERR_HIP)]


def _stack_entry(fmt=1, n=64, k=4096, g=128, x=FAKE, y=FAKE, stage=0):
    return binding.QStackEntry(_desc(fmt=fmt, n=n, k=k, g=g), x, y, stage, 0)


def test_stack_plan_statuses_and_layout():
    """q_stack_plan (host only): argument statuses, and the plan it writes --
    stages as runs of equal stage ids, rows of a stage's entries numbered
    consecutively, units of 2 KiB of codes per row (two 16-byte pieces per
    lane for 4-bit formats, one 32-byte piece for INT8), the counters zero."""
    import struct

    L = binding.lib()
    assert L.q_stack_plan_bytes(0) == 0 and L.q_stack_plan_bytes(65537) == 0
    specs = [_stack_entry(n=300, stage=0), _stack_entry(n=77, stage=0), _stack_entry(n=129, k=14336, stage=1, x=FAKE + 64),
             _stack_entry(fmt=7, n=200, k=5120, g=5120, stage=2, x=FAKE + 128),
             _stack_entry(fmt=4, n=5, k=1056, g=32, stage=5, x=FAKE + 256)]
    arr = (binding.QStackEntry * len(specs))(*specs)
    nbytes = L.q_stack_plan_bytes(len(specs))
    buf = (ctypes.c_uint8 * nbytes)()
    assert L.q_stack_plan(arr, len(specs), ctypes.cast(buf, ctypes.c_void_p), nbytes) == Q_OK
    raw = bytes(buf)
    magic, version, nst, nly, st_off, ly_off, ctr_off, total = struct.unpack_from("<IIiiIIII", raw, 0)
    assert (magic, version, nst, nly, ctr_off) == (0x4B415453, 2, 4, 5, 64) and total <= nbytes
    assert st_off == 64 + (4 + 1024) * 4  # done, abort, launch count, release word, 1024 arrival words
    assert raw[64:st_off] == bytes(st_off - 64)  # counters (abort word at byte 68) start at zero
    assert binding.Q_STACK_ABORT_OFFSET == 68
    stages = [struct.unpack_from("<Qiiiiiiiii", raw, st_off + 64 * i) for i in range(nst)]
    # (x, k, pieces, rows, layer_begin, layer_end, units, order, xsum, fmt)
    assert [s[1:] for s in stages] == [(4096, 128, 377, 0, 2, 1, 1, 1, 1), (14336, 448, 129, 2, 3, 4, 1, 1, 1),
                                       (5120, 160, 200, 3, 4, 3, 2, 0, 7), (1056, 33, 5, 4, 5, 1, 0, 0, 4)]
    assert [s[0] for s in stages] == [FAKE, FAKE + 64, FAKE + 128, FAKE + 256]
    layers = [struct.unpack_from("<QQQQiiiiii", raw, ly_off + 88 * i) for i in range(nly)]
    assert [l[8:10] for l in layers] == [(0, 300), (300, 377), (0, 129), (0, 200), (0, 5)]
    assert [l[4] for l in layers] == [1, 1, 1, 7, 4] and [l[7] for l in layers] == [7, 7, 7, 13, 5]  # (INT8: log2 rounded up, unused)

    def call(specs, nbytes=1 << 20, plan=True):
        a = (binding.QStackEntry * len(specs))(*specs)
        b = (ctypes.c_uint8 * nbytes)()
        return L.q_stack_plan(a, len(specs), ctypes.cast(b, ctypes.c_void_p) if plan else None, nbytes)

    assert call([_stack_entry()], plan=False) == Q_ERR_NULL
    assert L.q_stack_plan(None, 1, ctypes.cast(buf, ctypes.c_void_p), nbytes) == Q_ERR_NULL
    assert call([_stack_entry()], nbytes=16) == Q_ERR_SHAPE
    assert call([_stack_entry(stage=1), _stack_entry(stage=0)]) == Q_ERR_SHAPE          # stage ids decrease
    assert call([_stack_entry(), _stack_entry(x=FAKE + 16)]) == Q_ERR_SHAPE            # a stage mixing x
    assert call([_stack_entry(), _stack_entry(fmt=2)]) == Q_ERR_FORMAT                 # a stage mixing formats
    assert call([binding.QStackEntry(_desc(fmt=6, n=64, k=4096, g=16), FAKE, FAKE, 0, 0)]) == Q_ERR_FORMAT
    assert call([_stack_entry(x=None)]) == Q_ERR_NULL and call([_stack_entry(y=None)]) == Q_ERR_NULL
    assert call([_stack_entry(x=FAKE + 2)]) == Q_ERR_ALIGN
    assert call([_stack_entry(g=48)]) == Q_ERR_FORMAT
    assert L.q_gemv_stack(None, 0, None) == Q_ERR_NULL
    assert L.q_gemv_stack(FAKE + 8, 0, None) == Q_ERR_ALIGN
    assert L.q_gemv_stack(FAKE, 2, None) == Q_ERR_ARG
