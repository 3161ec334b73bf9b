"""Plain fp64 reference of the 3-bit residual vector-quantized matrices.

TEST INFRASTRUCTURE ONLY: imported by tests/ and bench.py's cpu_baseline leg,
never by the GPU library.

Source: WASTE page ("Kimi K3'ü 29 GB RAM'de 0,50 tok/sn hızla çalıştırmak"),
section "Quantization ve doğruluk": expert weights are stored as residual
vector quantization in three stages over 8-dimensional vectors, each stage a
256-entry codebook, which is 3.00 bits per weight (three 8-bit indices per 8
weights).  The oracle is the definition: every 8-weight run of a row is the
sum of one entry from each stage's codebook, and the product is the plain
matrix product of the reconstructed matrix.  (The GPU instead builds partial
inner-product tables per input row and sums three lookups per run, which the
same page describes; the results agree up to rounding.)

Storage (normative text in include/moe.h): a matrix of R rows by K columns
(both multiples of 64) is (R/64) * (K/64) tiles in row-block-major order, each
1536 bytes: byte s*512 + r*8 + j is the stage-s index of row r's run j (the
columns 8j .. 8j+7 of the tile).  Codebooks: fp16 [3][256][8].
"""
from __future__ import annotations

import numpy as np

__all__ = ["RVQ_TILE_BYTES", "rvq_codebooks_f64", "rvq_indices", "rvq_reconstruct", "rvq_gemv"]

RVQ_TILE_BYTES = 1536


def rvq_codebooks_f64(cb_bits) -> np.ndarray:
    """fp16 bit patterns [3, 256, 8] -> fp64 (exact)."""
    return np.asarray(cb_bits, dtype=np.uint16).view(np.float16).astype(np.float64).reshape(3, 256, 8)


def rvq_indices(buf, offset: int, rows: int, cols: int) -> np.ndarray:
    """Stage indices [3, rows, cols / 8] from the tiled bytes."""
    if rows % 64 or cols % 64:
        raise ValueError("rows and cols must be multiples of 64")
    n_rb, n_g = rows // 64, cols // 64
    t = np.asarray(buf[offset: offset + n_rb * n_g * RVQ_TILE_BYTES], dtype=np.uint8)
    t = t.reshape(n_rb, n_g, 3, 64, 8)                    # [rb, g, s, r, j]
    return t.transpose(2, 0, 3, 1, 4).reshape(3, rows, cols // 8)


def rvq_reconstruct(buf, offset: int, rows: int, cols: int, cb_bits) -> np.ndarray:
    """W [rows, cols] in fp64: W[r, 8j + d] = sum over stages s of C_s[i_s(r, j)][d]."""
    idx = rvq_indices(buf, offset, rows, cols)
    cb = rvq_codebooks_f64(cb_bits)
    w = np.zeros((rows, cols // 8, 8))
    for s in range(3):
        w += cb[s][idx[s]]
    return w.reshape(rows, cols)


def rvq_gemv(buf, offset: int, rows: int, cols: int, cb_bits, x: np.ndarray) -> np.ndarray:
    """y [T, rows] = x [T, cols] @ W^T, in fp64."""
    return np.asarray(x, dtype=np.float64) @ rvq_reconstruct(buf, offset, rows, cols, cb_bits).T
