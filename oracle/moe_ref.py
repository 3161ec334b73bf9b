"""Plain, slow, fp64 reference of the routed-expert MoE layer.

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by
bench.py's cpu_baseline leg, never by the GPU library.

What it computes, step by step, and where each step comes from:

* dequantization, W = s * q + b with group 64 along the input axis, 4-bit
  experts and an 8-bit router -- TurboFieldfare page, section "Belleği azaltan
  çalışma yapısı" (MLX affine 4-bit with group 64; router 8-bit).  The byte
  layout is the record format written out in include/moe.h.
* router logits from resident weights, then the top-k expert ids -- same page,
  section "Token üretim süreci" (top-8 ids per layer); WASTE page, section
  "Önceden okuma ve router tahmini" (16 expert ids per layer).
* softmax over the selected logits, SwiGLU expert FFN, shared expert added
  with weight 1 -- readings of the workload description and of "shared and
  routed outputs are combined" (Token üretim süreci).
* residual stack r_{l+1} = r_l + y_l, and lookahead = the next layer's router
  on the current residual -- WASTE page, "Önceden okuma ve router tahmini"
  (the next router runs one residual ahead; the real router decides, so the
  output is unchanged).

Every value is carried in fp64; the fp16 scales/biases and bf16 inputs convert
to fp64 exactly, and s*q+b is exact in fp64.  Each function states its pins in
tests/test_oracle_pins.py.
"""
from __future__ import annotations

import struct

import numpy as np

__all__ = [
    "f16_bits_to_f64", "bf16_bits_to_f64", "read_record_header", "dequant_tiled",
    "expert_matrices", "router_matrix", "router_logits", "select_topk",
    "softmax_selected", "silu", "expert_ffn", "OracleLayer", "oracle_stack", "rms_normalize",
]

_GROUP = 64
_ROWS = 64


def f16_bits_to_f64(bits) -> np.ndarray:
    """IEEE binary16 bit patterns -> fp64 (exact, subnormals kept)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns -> fp64 (exact: bf16 is the top half of an fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def read_record_header(rec) -> dict:
    """Decode the 256-byte record header (field list in include/moe.h)."""
    raw = bytes(np.asarray(rec[:64], dtype=np.uint8))
    f = struct.unpack("<IIiIIIII4Q", raw)
    keys = ("magic", "version", "expert_id", "hidden", "inter", "group", "bits",
            "tile_rows", "gate_off", "up_off", "down_off", "end_off")
    return dict(zip(keys, f))


def dequant_tiled(buf, offset: int, rows: int, cols: int, bits: int) -> np.ndarray:
    """W[r, c] = s[r, c//64] * q[r, c] + b[r, c//64] for a tiled matrix.

    Tile (rb, g) starts at offset + (rb*(cols/64) + g) * tile_bytes.
    4-bit: byte h*1024 + r*16 + j holds columns h*32+2j (low nibble) and
    h*32+2j+1 (high nibble).  8-bit: byte c4*1024 + r*16 + j holds column
    c4*16 + j.  Then 64 (s, b) fp16 pairs, row r at code_bytes + 4r.
    """
    if rows % _ROWS or cols % _GROUP:
        raise ValueError("rows and cols must be multiples of 64")
    code_bytes = 2048 if bits == 4 else 4096
    tile_bytes = code_bytes + 4 * _ROWS
    n_rb, n_g = rows // _ROWS, cols // _GROUP
    t = np.asarray(buf[offset: offset + n_rb * n_g * tile_bytes], dtype=np.uint8)
    t = t.reshape(n_rb, n_g, tile_bytes)
    if bits == 4:
        c = t[:, :, :code_bytes].reshape(n_rb, n_g, 2, _ROWS, 16)       # [rb, g, h, r, j]
        q = np.stack([c & 0x0F, c >> 4], axis=-1)                        # [rb, g, h, r, j, lo/hi]
        q = q.reshape(n_rb, n_g, 2, _ROWS, 32)                           # col within half = 2j + nib
        q = q.transpose(0, 3, 1, 2, 4).reshape(rows, cols)               # [rb, r, g, h, 32]
    elif bits == 8:
        c = t[:, :, :code_bytes].reshape(n_rb, n_g, 4, _ROWS, 16)       # [rb, g, c4, r, j]
        q = c.transpose(0, 3, 1, 2, 4).reshape(rows, cols)
    else:
        raise ValueError("bits must be 4 or 8")
    sb = np.ascontiguousarray(t[:, :, code_bytes:]).view(np.uint16).reshape(n_rb, n_g, _ROWS, 2)
    s = f16_bits_to_f64(sb[..., 0]).transpose(0, 2, 1).reshape(rows, n_g, 1)   # [row, g, 1]
    b = f16_bits_to_f64(sb[..., 1]).transpose(0, 2, 1).reshape(rows, n_g, 1)
    w = q.reshape(rows, n_g, _GROUP) * s + b          # column c = g*64 + (c % 64)
    return w.reshape(rows, cols)


def expert_matrices(rec, hidden: int, inter: int):
    """(Wg [I,H], Wu [I,H], Wd [H,I]) in fp64 from one record."""
    h = read_record_header(rec)
    if h["magic"] != 0x58455251 or h["hidden"] != hidden or h["inter"] != inter:
        raise ValueError(f"record header does not match the layer: {h}")
    wg = dequant_tiled(rec, h["gate_off"], inter, hidden, 4)
    wu = dequant_tiled(rec, h["up_off"], inter, hidden, 4)
    wd = dequant_tiled(rec, h["down_off"], hidden, inter, 4)
    return wg, wu, wd


def router_matrix(router_buf, hidden: int, n_experts: int) -> np.ndarray:
    """Wr [E, H] fp64 (padding rows dropped)."""
    rows = -(-n_experts // _ROWS) * _ROWS
    return dequant_tiled(router_buf, 0, rows, hidden, 8)[:n_experts]


def router_logits(x: np.ndarray, wr: np.ndarray, beta=None) -> np.ndarray:
    """l[t, e] = sum_h x[t, h] Wr[e, h] + beta[e]."""
    lg = x @ wr.T
    if beta is not None:
        lg = lg + np.asarray(beta, dtype=np.float64)[None, :]
    return lg


def select_topk(logits: np.ndarray, k: int):
    """ids [T, k]: experts ordered by (logit descending, index ascending), first k.
    gap [T]: k-th minus (k+1)-th largest logit (+inf when k == E)."""
    t, e = logits.shape
    ids = np.empty((t, k), dtype=np.int64)
    gap = np.full(t, np.inf)
    idx = np.arange(e)
    for i in range(t):
        order = np.lexsort((idx, -logits[i]))     # primary: -logit, secondary: index
        ids[i] = order[:k]
        if k < e:
            gap[i] = logits[i, order[k - 1]] - logits[i, order[k]]
    return ids, gap


def softmax_selected(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """p[t, j] = exp(l[t, ids[t,j]]) / sum_j' exp(l[t, ids[t,j']])."""
    sel = np.take_along_axis(logits, ids, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def expert_ffn(x: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """SwiGLU FFN on rows of x: Wd (SiLU(Wg x) * (Wu x))."""
    g = x @ wg.T
    u = x @ wu.T
    return (silu(g) * u) @ wd.T


class OracleLayer:
    """One MoE layer.  ``get_record(e)`` returns expert e's record bytes, so a
    bank that does not fit host memory is regenerated one record at a time."""

    def __init__(self, hidden, n_experts, top_k, inter, shared_inter, router_buf,
                 router_bias, get_record, shared_record=None):
        self.hidden, self.n_experts, self.top_k = hidden, n_experts, top_k
        self.inter, self.shared_inter = inter, shared_inter
        self.wr = router_matrix(router_buf, hidden, n_experts)
        self.beta = None if router_bias is None else np.asarray(router_bias, np.float64)
        self.get_record = get_record
        self.shared_record = shared_record

    def logits(self, x: np.ndarray) -> np.ndarray:
        return router_logits(x, self.wr, self.beta)

    def forward(self, x: np.ndarray, logits=None, force_ids=None, pool=None) -> dict:
        """x fp64 [T, H] -> dict(y, ids, p, gap, logits).

        ``force_ids`` [T, k] replaces the top-k selection (the layer evaluated
        on a given selection; p is still the softmax of the oracle's logits of
        those experts).  Used where the top-k is not unique within a tolerance.
        ``pool`` (an executor with ``map``) evaluates the experts concurrently;
        each expert's rows are computed on their own either way, so the result
        is the same."""
        x = np.asarray(x, dtype=np.float64)
        t = x.shape[0]
        lg = self.logits(x) if logits is None else logits
        ids, gap = select_topk(lg, self.top_k)
        if force_ids is not None:
            ids = np.asarray(force_ids, dtype=np.int64).reshape(t, self.top_k)
        p = softmax_selected(lg, ids)
        # out[t, j] = FFN_{ids[t,j]}(x[t]); tokens sharing an expert are one matmul
        out = np.zeros((t, self.top_k, self.hidden))

        def one(e):
            rows, cols = np.nonzero(ids == e)
            wg, wu, wd = expert_matrices(self.get_record(int(e)), self.hidden, self.inter)
            return rows, cols, expert_ffn(x[rows], wg, wu, wd)
        for rows, cols, o in (pool.map if pool is not None else map)(one, np.unique(ids)):
            out[rows, cols] = o
        y = np.zeros((t, self.hidden))
        for j in range(self.top_k):                      # fixed order: j ascending
            y += p[:, j:j + 1] * out[:, j]
        if self.shared_record is not None:               # shared expert last, weight 1
            wg, wu, wd = expert_matrices(self.shared_record, self.hidden, self.shared_inter)
            y += expert_ffn(x, wg, wu, wd)
        return dict(y=y, ids=ids, p=p, gap=gap, logits=lg)


def rms_normalize(x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) per row (a parameter-free RMS norm)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)


def oracle_stack(layers, x0: np.ndarray, lookahead_k: int | None = None,
                 norm: bool = False, pool=None, force_ids=None) -> dict:
    """r_0 = x0; y_l = layer_l(n(r_l)); r_{l+1} = r_l + y_l, with n the RMS norm
    when ``norm`` (else the identity).  With lookahead_k, also the next layer's
    router on n(r_l) (its top-lookahead_k ids), for reporting only: it never
    feeds back into the result.  ``pool`` is passed to each layer's forward;
    ``force_ids`` (one [T, k] selection per layer, or None) evaluates each
    layer on a given selection, as forward(force_ids=...) does."""
    r = np.asarray(x0, dtype=np.float64)
    per_layer = []
    for li, layer in enumerate(layers):
        xin = rms_normalize(r) if norm else r
        res = layer.forward(xin, pool=pool,
                            force_ids=None if force_ids is None else force_ids[li])
        res["input"] = r
        if lookahead_k is not None and li + 1 < len(layers):
            pred, _ = select_topk(layers[li + 1].logits(xin), lookahead_k)
            res["lookahead_ids"] = pred
        per_layer.append(res)
        r = r + res["y"]
    return dict(layers=per_layer, out=r)
