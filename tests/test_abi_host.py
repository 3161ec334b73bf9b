"""The C-ABI library on the CPU: it loads, exports every function the header
declares, sizes workspaces, and validates record headers (host-only logic;
no GPU calls)."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    import quantized_routed_expert_bit_amd as q
    if not os.path.exists(q.LIB_PATH):
        from quantized_routed_expert_bit_amd import build
        build.build()
    return q.load()


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", src)))


def test_exports_every_declared_function(lib):
    from quantized_routed_expert_bit_amd import _lib
    names = _declared()
    assert set(names) == set(_lib.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_strerror(lib):
    for code in range(0, -7, -1):
        assert lib.moe_strerror(code)
    assert lib.moe_strerror(-99) == b"unknown status"


def _cfg(**kw):
    from quantized_routed_expert_bit_amd import make_config
    d = dict(hidden=2816, n_experts=128, top_k=8, inter=704, shared_inter=2112, max_tokens=16)
    d.update(kw)
    return make_config(**d)


def test_workspace_bytes_and_config_checks(lib):
    c = _cfg()
    ws = lib.moe_workspace_bytes(ctypes.byref(c))
    # at least the per-slot fp32 expert outputs and fp16 intermediates
    assert ws >= (16 * 8 + 16) * 2816 * 4 + (16 * 8 * 704 + 16 * 2112) * 2
    assert ws % 256 == 0
    for bad in (dict(hidden=100), dict(inter=0), dict(top_k=0), dict(top_k=129),
                dict(top_k=33, n_experts=64), dict(n_experts=2000), dict(max_tokens=0),
                dict(shared_inter=65)):
        cb = _cfg(**bad)
        assert lib.moe_workspace_bytes(ctypes.byref(cb)) == 0, bad
        out = ctypes.c_void_p()
        assert lib.moe_open(ctypes.byref(cb), ctypes.byref(out)) == -2, bad
    c2 = _cfg()
    c2.group = 32
    assert lib.moe_workspace_bytes(ctypes.byref(c2)) == 0
    c3 = _cfg()
    c3.struct_size = 4
    out = ctypes.c_void_p()
    assert lib.moe_open(ctypes.byref(c3), ctypes.byref(out)) == -1


def _check(lib, hdr, cfg, eid, stride):
    buf = np.ascontiguousarray(hdr, dtype=np.uint8)
    return lib.moe_check_record_header(buf.ctypes.data_as(ctypes.c_void_p), buf.size,
                                       ctypes.byref(cfg), eid, stride)


def test_record_header_validation(lib):
    cfg = _cfg()
    rec = synth.make_record(0, 1, 0, 5, 2816, 704)
    stride = len(rec)
    assert _check(lib, rec[:256], cfg, 5, stride) == 0
    assert _check(lib, rec[:256], cfg, 4, stride) == -4          # wrong expert id
    assert _check(lib, rec[:256], cfg, 5, stride - 4096) == -4   # stride too small
    assert _check(lib, rec[:100], cfg, 5, stride) == -1          # short buffer
    assert _check(lib, rec[:256], cfg, 128, stride) == -1        # id out of range
    sh = synth.make_record(0, 1, 0, 0, 2816, 2112, shared=True)
    assert _check(lib, sh[:256], cfg, -1, len(sh)) == 0
    assert _check(lib, sh[:256], cfg, 0, len(sh)) == -4
    # each header field corrupted on its own is refused
    for off in list(range(0, 64, 4)) + [100, 255]:
        bad = rec[:256].copy()
        bad[off] ^= 0x01
        assert _check(lib, bad, cfg, 5, stride) == -4, off


def test_record_header_fuzz(lib):
    """Random byte mutations never pass the header check unless they leave the
    header unchanged or touch only the payload checksum's value (which only
    the payload verification can decide)."""
    cfg = _cfg()
    rec = synth.make_record(0, 1, 0, 9, 2816, 704)[:256].copy()
    rng = np.random.default_rng(0)
    n_crc_only = 0
    for _ in range(600):
        bad = rec.copy()
        n = int(rng.integers(1, 6))
        pos = rng.integers(0, 256, n)
        if rng.random() < 0.2:
            pos = rng.integers(64, 68, n)                     # the checksum value only
        bad[pos] = rng.integers(0, 256, n).astype(np.uint8)
        rc = _check(lib, bad, cfg, 9, 3346432)
        changed = np.nonzero(bad != rec)[0]
        if changed.size == 0 or (changed.min() >= 64 and changed.max() < 68):
            n_crc_only += changed.size > 0
            assert rc == 0
        else:
            assert rc == -4
    assert n_crc_only > 50


def test_checksum_field_rules(lib):
    """hflags 0 requires a zero checksum; hflags above 1 is refused; a record
    without a checksum (hflags 0) passes the header check."""
    import struct
    cfg = _cfg()
    rec = synth.make_record(0, 1, 0, 9, 2816, 704)
    stride = len(rec)
    assert struct.unpack_from("<II", bytes(rec[64:72]))[1] == 1
    plain = synth.make_record(0, 1, 0, 9, 2816, 704, checksum=False)
    assert _check(lib, plain[:256], cfg, 9, stride) == 0
    h = rec[:256].copy()
    h[68:72] = 0                                          # flag cleared, checksum left
    assert _check(lib, h, cfg, 9, stride) == -4
    h = rec[:256].copy()
    h[68] = 3
    assert _check(lib, h, cfg, 9, stride) == -4


def test_generator_checksum_is_zlib_crc32():
    """The record generator's checksum is zlib's CRC-32 of [gate_off, end_off)."""
    import struct
    import zlib
    rec = synth.make_record(0, 0, 0, 3, 512, 256)
    lay = synth.record_layout(512, 256)
    crc, flags = struct.unpack_from("<II", bytes(rec[64:72]))
    assert flags == 1 and crc == zlib.crc32(bytes(rec[lay["gate"]:lay["end"]]))
    # a single flipped payload bit changes it
    rec2 = rec.copy()
    rec2[lay["down"] + 1000] ^= 4
    assert zlib.crc32(bytes(rec2[lay["gate"]:lay["end"]])) != crc


def test_rvq_workspace_bytes(lib):
    """The residual-VQ workspace holds the fp32 partial outputs of every K
    group of 256 columns; invalid shapes size 0."""
    T, K, R, n = 3, 7168, 4096, 16
    ws = lib.moe_rvq_workspace_bytes(T, K, R, n)
    assert ws % 256 == 0
    assert ws >= (K // 256) * n * T * R * 4
    for bad in ((1, 96, 64, 1), (1, 64, 96, 1), (1, 0, 64, 1), (1, 64, 0, 1), (-1, 64, 64, 1),
                (1, 64, 64, 0), (65536, 64, 64, 1), (64, 64, 1 << 20, 1 << 12),
                (1, 1 << 24, 1 << 14, 1 << 10)):
        assert lib.moe_rvq_workspace_bytes(*bad) == 0, bad
