"""Seeded generators for the layer's inputs, written in the storage format.

Storage format (normative text: ``include/moe.h``, "Record format"):

* A 4-bit matrix of R rows (outputs) by C columns (inputs) is a row-block-major
  sequence of tiles.  Each tile covers 64 rows by one group of 64 columns and is
  2304 bytes: 2048 bytes of codes followed by 64 (scale, bias) fp16 pairs.
* An 8-bit matrix uses the same tiling with 4096 code bytes per tile (4352 B).
* An expert record is a 256-byte header, then the gate, up and down matrices,
  padded to a multiple of 4096 bytes.  Host-generated records carry the
  payload's CRC-32 in the header; device-generated banks (``gpu_bank``) do
  not.

Value recipe (the workloads' own description of the synthetic layer):

* codes: uniform random bytes.  A uniform byte is two independent uniform
  nibbles, so 4-bit codes are uniform on 0..15 and 8-bit codes on 0..255.
* expert scales: fp16(|z| * 0.02 / 8), z ~ N(0, 1); bias = -8 * scale (exact).
* router scales: fp16(|z| * 0.02 / 128); bias = -128 * scale (exact).
  fp16 subnormal scales are kept.
* hidden states: bf16 (round-to-nearest-even of the fp32 value) of N(0, 1).
* router logit bias: none, N(0, 0.5) per expert (std 0.5), or the log of a
  Zipf(1.1) prior over a seeded permutation of the experts.

Everything is drawn from numpy's PCG64 with a SeedSequence whose spawn key is
(config, layer, tensor, expert-or-tag), so one record can be regenerated
without generating the bank around it.
"""
from __future__ import annotations

import struct
import zlib
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "GROUP", "TILE_ROWS", "Q4_TILE_BYTES", "Q4_CODE_BYTES", "Q8_TILE_BYTES",
    "Q8_CODE_BYTES", "HEADER_BYTES", "RECORD_ALIGN", "MAGIC", "VERSION",
    "SHARED_ID", "LayerShape", "Workload", "WORKLOADS", "record_layout",
    "record_stride", "router_bytes_len", "make_record", "set_payload_crc32", "make_router",
    "make_router_bias", "make_hidden", "bf16_bits_from_f32", "LayerInputs",
]

GROUP = 64
TILE_ROWS = 64
Q4_CODE_BYTES = 2048
Q4_TILE_BYTES = Q4_CODE_BYTES + 4 * TILE_ROWS      # 2304
Q8_CODE_BYTES = 4096
Q8_TILE_BYTES = Q8_CODE_BYTES + 4 * TILE_ROWS      # 4352
HEADER_BYTES = 256
RECORD_ALIGN = 4096
MAGIC = 0x58455251          # bytes "QREX" read as a little-endian u32
VERSION = 1
SHARED_ID = -1

# tensor ids used in seed spawn keys
_T_ROUTER, _T_RBIAS, _T_EXPERT, _T_SHARED, _T_HIDDEN = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class LayerShape:
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    shared_inter: int = 0   # 0: no shared expert

    @property
    def has_shared(self) -> bool:
        return self.shared_inter > 0


@dataclass(frozen=True)
class Workload:
    """One of the five synthetic workloads (index = its position in the list)."""
    index: int
    name: str
    shape: LayerShape
    batches: tuple
    bias: str | None = None        # None | "normal0.5" | "zipf1.1"
    layers: int = 1
    chunk: int = 0                 # prefill chunk size (0: not chunked)
    notes: str = ""


WORKLOADS = [
    Workload(0, "tiny", LayerShape(512, 16, 4, 256, 0), (4,)),
    Workload(1, "decode", LayerShape(2816, 128, 8, 704, 2112), (1, 4, 16)),
    Workload(2, "prefill", LayerShape(2816, 128, 8, 704, 2112), (2048,),
             bias="normal0.5", chunk=128),
    Workload(3, "large_decode", LayerShape(7168, 512, 16, 2048, 2048), (1, 8, 64)),
    Workload(4, "stack", LayerShape(7168, 512, 16, 2048, 2048), (256,),
             bias="zipf1.1", layers=8),
]


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def _round_up(v: int, a: int) -> int:
    return (v + a - 1) // a * a


def record_layout(hidden: int, inter: int) -> dict:
    """Byte offsets of the three matrices inside one expert record."""
    n_tiles = (inter // TILE_ROWS) * (hidden // GROUP)   # same count for all three
    sec = n_tiles * Q4_TILE_BYTES
    gate = HEADER_BYTES
    up = gate + sec
    down = up + sec
    end = down + sec
    return dict(gate=gate, up=up, down=down, end=end, tiles=n_tiles,
                stride=_round_up(end, RECORD_ALIGN))


def record_stride(hidden: int, inter: int) -> int:
    return record_layout(hidden, inter)["stride"]


def router_bytes_len(hidden: int, n_experts: int) -> int:
    rows = _round_up(n_experts, TILE_ROWS)
    return (rows // TILE_ROWS) * (hidden // GROUP) * Q8_TILE_BYTES


def _fill_tiles(dst: np.ndarray, n_tiles: int, code_bytes: int, tile_bytes: int,
                rng: np.random.Generator, scale_div: float, zero_code: float) -> None:
    """Random codes, then (scale, bias) fp16 pairs, in storage order."""
    tiles = dst[: n_tiles * tile_bytes].reshape(n_tiles, tile_bytes)
    tiles[:, :code_bytes] = np.frombuffer(rng.bytes(n_tiles * code_bytes),
                                          dtype=np.uint8).reshape(n_tiles, code_bytes)
    z = rng.standard_normal(n_tiles * TILE_ROWS)
    s = (np.abs(z) * 0.02 / scale_div).astype(np.float16)
    b = (-zero_code * s.astype(np.float64)).astype(np.float16)
    sb = np.empty((n_tiles * TILE_ROWS, 2), dtype=np.float16)
    sb[:, 0] = s
    sb[:, 1] = b
    tiles[:, code_bytes:] = sb.view(np.uint8).reshape(n_tiles, tile_bytes - code_bytes)


def _pack_header(buf: np.ndarray, expert_id: int, hidden: int, inter: int, lay: dict) -> None:
    hdr = struct.pack("<IIiIIIII4Q", MAGIC, VERSION, expert_id, hidden, inter, GROUP, 4,
                      TILE_ROWS, lay["gate"], lay["up"], lay["down"], lay["end"])
    buf[: len(hdr)] = np.frombuffer(hdr, dtype=np.uint8)


def set_payload_crc32(buf: np.ndarray) -> np.ndarray:
    """Write the header's payload checksum (CRC-32 of bytes [gate_off, end_off),
    zlib's) and set hflags bit 0; returns buf."""
    gate, end = struct.unpack_from("<Q", bytes(buf[32:40]))[0], struct.unpack_from("<Q", bytes(buf[56:64]))[0]
    crc = zlib.crc32(memoryview(np.ascontiguousarray(buf[gate:end])))
    buf[64:72] = np.frombuffer(struct.pack("<II", crc, 1), dtype=np.uint8)
    return buf


def make_record(seed: int, cfg: int, layer: int, expert: int, hidden: int, inter: int,
                shared: bool = False, checksum: bool = True) -> np.ndarray:
    """One expert record (uint8, record_stride bytes).  ``shared`` selects the
    always-on expert's stream and marks its header with expert id -1; with
    ``checksum`` the header carries the payload's CRC-32."""
    lay = record_layout(hidden, inter)
    buf = np.zeros(lay["stride"], dtype=np.uint8)
    rng = _rng(seed, cfg, layer, _T_SHARED if shared else _T_EXPERT, 0 if shared else expert)
    _pack_header(buf, SHARED_ID if shared else expert, hidden, inter, lay)
    sec = lay["tiles"] * Q4_TILE_BYTES
    for off in (lay["gate"], lay["up"], lay["down"]):
        _fill_tiles(buf[off: off + sec], lay["tiles"], Q4_CODE_BYTES, Q4_TILE_BYTES,
                    rng, 8.0, 8.0)
    return set_payload_crc32(buf) if checksum else buf


def make_router(seed: int, cfg: int, layer: int, hidden: int, n_experts: int) -> np.ndarray:
    """The 8-bit router matrix (rows = experts padded to 64; padding rows hold
    random bytes and are ignored by definition)."""
    n = router_bytes_len(hidden, n_experts)
    buf = np.zeros(n, dtype=np.uint8)
    rng = _rng(seed, cfg, layer, _T_ROUTER, 0)
    _fill_tiles(buf, n // Q8_TILE_BYTES, Q8_CODE_BYTES, Q8_TILE_BYTES, rng, 128.0, 128.0)
    return buf


def make_router_bias(seed: int, cfg: int, layer: int, n_experts: int, kind: str | None):
    """float32 [E] additive router logit bias, or None."""
    if kind is None:
        return None
    rng = _rng(seed, cfg, layer, _T_RBIAS, 0)
    if kind == "normal0.5":
        return (rng.standard_normal(n_experts) * 0.5).astype(np.float32)
    if kind == "zipf1.1":
        rank = 1 + rng.permutation(n_experts)
        return (-1.1 * np.log(rank.astype(np.float64))).astype(np.float32)
    raise ValueError(kind)


def bf16_bits_from_f32(v: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def make_hidden(seed: int, cfg: int, n_tokens: int, hidden: int, tag: int = 0) -> np.ndarray:
    """bf16 bits [T, H] of N(0, 1) hidden states."""
    rng = _rng(seed, cfg, 0, _T_HIDDEN, n_tokens * 1000 + tag)
    z = rng.standard_normal((n_tokens, hidden)).astype(np.float32)
    return bf16_bits_from_f32(z)


@dataclass
class LayerInputs:
    """Lazy view of one layer's inputs: records are regenerated on demand."""
    seed: int
    cfg: int
    layer: int
    shape: LayerShape
    bias_kind: str | None = None
    _router: np.ndarray | None = field(default=None, repr=False)

    @property
    def stride(self) -> int:
        return record_stride(self.shape.hidden, self.shape.inter)

    def router(self) -> np.ndarray:
        if self._router is None:
            self._router = make_router(self.seed, self.cfg, self.layer, self.shape.hidden,
                                       self.shape.n_experts)
        return self._router

    def router_bias(self):
        return make_router_bias(self.seed, self.cfg, self.layer, self.shape.n_experts,
                                self.bias_kind)

    def record(self, e: int) -> np.ndarray:
        return make_record(self.seed, self.cfg, self.layer, e, self.shape.hidden,
                           self.shape.inter)

    def shared_record(self):
        if not self.shape.has_shared:
            return None
        return make_record(self.seed, self.cfg, self.layer, 0, self.shape.hidden,
                           self.shape.shared_inter, shared=True)

    def bank(self) -> np.ndarray:
        """All E records back to back (only for banks that fit host memory)."""
        return np.concatenate([self.record(e) for e in range(self.shape.n_experts)])


def layer_inputs(wl: Workload, layer: int = 0, seed: int = 0) -> LayerInputs:
    return LayerInputs(seed, wl.index, layer, wl.shape, wl.bias)


__all__.append("layer_inputs")


# ---------------------------------------------------------------------------
# Device-side generation for banks too large to generate on the host in
# reasonable time (tens to hundreds of GB).  Same value recipe as above, drawn
# with torch's seeded device generator instead of PCG64, so the bytes differ
# from make_record's; the header layout is identical.  A consumer that needs a
# record on the host (the oracle) copies it back from the bank.
# ---------------------------------------------------------------------------

def gpu_bank(seed: int, cfg: int, layer: int, hidden: int, inter: int, n_records: int,
             device, shared: bool = False):
    """A bank of n_records expert records (uint8 device tensor) and its stride.
    With shared=True, one record with expert id -1 (n_records must be 1)."""
    import torch
    lay = record_layout(hidden, inter)
    stride, n_tiles = lay["stride"], lay["tiles"]
    bank = torch.zeros(n_records * stride, dtype=torch.uint8, device=device)
    gen = torch.Generator(device=device)
    gen.manual_seed(((seed * 1000003 + cfg) * 1000003 + layer) * 8 + (_T_SHARED if shared else _T_EXPERT))
    rec = bank.view(n_records, stride)
    sec = n_tiles * Q4_TILE_BYTES
    for e in range(n_records):
        hdr = np.zeros(HEADER_BYTES, dtype=np.uint8)
        _pack_header(hdr, SHARED_ID if shared else e, hidden, inter, lay)
        rec[e, :HEADER_BYTES].copy_(torch.from_numpy(hdr))
        for off in (lay["gate"], lay["up"], lay["down"]):
            tiles = rec[e, off: off + sec].view(n_tiles, Q4_TILE_BYTES)
            tiles[:, :Q4_CODE_BYTES] = torch.randint(0, 256, (n_tiles, Q4_CODE_BYTES), generator=gen,
                                                     device=device, dtype=torch.uint8)
            z = torch.randn(n_tiles * TILE_ROWS, generator=gen, device=device, dtype=torch.float64)
            s = (z.abs() * 0.02 / 8.0).to(torch.float16)
            b = (-8.0 * s.to(torch.float64)).to(torch.float16)
            sb = torch.stack([s, b], dim=1).contiguous().view(torch.uint8)
            tiles[:, Q4_CODE_BYTES:] = sb.view(n_tiles, Q4_TILE_BYTES - Q4_CODE_BYTES)
    return bank, stride


__all__.append("gpu_bank")


# ---------------------------------------------------------------------------
# 3-bit residual-VQ matrices (the WASTE page's expert codec): indices are
# uniform random bytes; the three codebooks hold N(0, sigma_s) entries with
# sigma = 0.02, 0.005, 0.00125 (each stage refines the one before), as fp16.
# ---------------------------------------------------------------------------

RVQ_TILE_BYTES = 1536
_T_RVQ = 5


def rvq_bytes(rows: int, cols: int) -> int:
    """Bytes of a tiled RVQ matrix: three 8-bit indices per 8 weights."""
    return (rows // 64) * (cols // 64) * RVQ_TILE_BYTES


def make_rvq_codebooks(seed: int, tag: int = 0) -> np.ndarray:
    """fp16 bit patterns [3, 256, 8]."""
    rng = _rng(seed, 0, 0, _T_RVQ, 1000 + tag)
    sig = np.array([0.02, 0.005, 0.00125])[:, None, None]
    return (rng.standard_normal((3, 256, 8)) * sig).astype(np.float16).view(np.uint16)


def make_rvq_matrix(seed: int, rows: int, cols: int, tag: int = 0) -> np.ndarray:
    """Tiled RVQ matrix bytes (uniform random indices)."""
    rng = _rng(seed, 0, 0, _T_RVQ, tag)
    return np.frombuffer(rng.bytes(rvq_bytes(rows, cols)), dtype=np.uint8).copy()


__all__ += ["RVQ_TILE_BYTES", "rvq_bytes", "make_rvq_codebooks", "make_rvq_matrix"]

