"""Hand placement of codes and (scale, bias) pairs into tiled matrices, written
directly from the record-format text in include/moe.h, independent of both the
oracle's reader and the generator.  Used only to build pin fixtures."""
import struct

import numpy as np


def q4_tiles(q: np.ndarray, s_bits: np.ndarray, b_bits: np.ndarray) -> bytearray:
    """q int [R, C] in 0..15; s_bits, b_bits uint16 [R, C/64] (fp16 bit patterns)."""
    R, C = q.shape
    out = bytearray((R // 64) * (C // 64) * 2304)
    for rb in range(R // 64):
        for g in range(C // 64):
            base = (rb * (C // 64) + g) * 2304
            for r in range(64):
                row = rb * 64 + r
                for h in range(2):
                    for j in range(16):
                        c0 = g * 64 + h * 32 + 2 * j
                        out[base + h * 1024 + r * 16 + j] = int(q[row, c0]) | (int(q[row, c0 + 1]) << 4)
                struct.pack_into("<HH", out, base + 2048 + 4 * r, int(s_bits[row, g]), int(b_bits[row, g]))
    return out


def q8_tiles(q: np.ndarray, s_bits: np.ndarray, b_bits: np.ndarray) -> bytearray:
    R, C = q.shape
    out = bytearray((R // 64) * (C // 64) * 4352)
    for rb in range(R // 64):
        for g in range(C // 64):
            base = (rb * (C // 64) + g) * 4352
            for r in range(64):
                row = rb * 64 + r
                for c4 in range(4):
                    for j in range(16):
                        out[base + c4 * 1024 + r * 16 + j] = int(q[row, g * 64 + c4 * 16 + j])
                struct.pack_into("<HH", out, base + 4096 + 4 * r, int(s_bits[row, g]), int(b_bits[row, g]))
    return out


def f16bits(v) -> np.ndarray:
    return np.asarray(v, dtype=np.float16).view(np.uint16)


def record(expert_id: int, hidden: int, inter: int, gate: bytes, up: bytes, down: bytes) -> np.ndarray:
    sec = (inter // 64) * (hidden // 64) * 2304
    assert len(gate) == len(up) == len(down) == sec
    end = 256 + 3 * sec
    stride = -(-end // 4096) * 4096
    buf = bytearray(stride)
    struct.pack_into("<IIiIIIII4Q", buf, 0, 0x58455251, 1, expert_id, hidden, inter, 64, 4, 64,
                     256, 256 + sec, 256 + 2 * sec, end)
    buf[256:256 + sec] = gate
    buf[256 + sec:256 + 2 * sec] = up
    buf[256 + 2 * sec:end] = down
    return np.frombuffer(bytes(buf), dtype=np.uint8)
