"""ORACLE: test infrastructure, not product code.

Symmetric per-row int8 weights for small-batch decode, as a definition the
HIP path's int8 route is checked against.  Only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
it; it shares no code with the HIP library.

Source: the Albatross article (RWKV-Runner backend, "boundaries and follow-up
route") lists int8 quantised weights among the performance items its first
version leaves out; it gives no scheme.  At one token per step a decode step
streams every weight once, so halving the bytes per weight is the lever.
Reading, the plainest symmetric scheme:

* the source is the fp16 weight (the values the fp16 path packs);
* per output unit of a projection (a row of the PyTorch-style [out, in]
  matrix), over its inputs: m = max |w| and the scale s = m / 127, both in
  fp32;
* code q = rint(w / s) (fp32 division, ties to even), clamped to
  [-127, 127]; q = 0 where s = 0;
* the weight used is q * s.

The channel-mix value projection is read row by row of its hidden units on
the sparse path (each active hidden unit adds its row), so its "rows" are the
hidden units: scales run over the columns of ffn.value.weight [C, F].

Matrices on the int8 route: the r / k / v / output projections, the first
stage of the four low-rank adapters (w1, a1, v1, g1), the channel-mix key
and value, and the head.  The adapters' second stage and the embedding stay
as they are.

Pins: tests/test_oracle_quant.py (rows on the grid come back exactly, the
error bound s/2, the extreme element at +-127, zero rows, ties to even, the
column orientation of the value matrix).
"""
from __future__ import annotations

from typing import Dict, Tuple

import numpy as np

INT8_ROWWISE = ("att.receptance.weight", "att.key.weight", "att.value.weight", "att.output.weight",
                "att.w1", "att.a1", "att.v1", "att.g1", "ffn.key.weight")


def quantize_rows(w) -> Tuple[np.ndarray, np.ndarray]:
    """Codes int8 [rows, K] and fp32 scales [rows] of a [rows, K] matrix, per
    the definition above (the input is rounded to fp16 first)."""
    w32 = np.asarray(w).astype(np.float16).astype(np.float32)
    m = np.max(np.abs(w32), axis=1)
    s = (m / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = np.rint((w32 / safe[:, None]).astype(np.float32))
    q = np.where(s[:, None] > 0, np.clip(q, -127, 127), 0).astype(np.int8)
    return q, s


def dequantize_rows(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    return q.astype(np.float64) * s.astype(np.float64)[:, None]


def int8_weights(weights: Dict[str, np.ndarray], n_layer: int) -> Dict[str, np.ndarray]:
    """A copy of the weight table with every int8-route matrix replaced by its
    dequantised values (float64)."""
    out = dict(weights)
    for l in range(n_layer):
        p = f"blocks.{l}."
        for n in INT8_ROWWISE:
            out[p + n] = dequantize_rows(*quantize_rows(weights[p + n]))
        wv = weights[p + "ffn.value.weight"]                   # [C, F]: hidden units are columns
        out[p + "ffn.value.weight"] = dequantize_rows(*quantize_rows(np.asarray(wv).T)).T
    out["head.weight"] = dequantize_rows(*quantize_rows(weights["head.weight"]))
    return out


class Int8View:
    """The weight table of int8_weights, dequantising each int8-route matrix
    when it is read (for shapes whose fp64 copies would not fit at once)."""

    def __init__(self, weights: Dict[str, np.ndarray], n_layer: int):
        self.w = weights
        self.rowwise = {f"blocks.{l}.{n}" for l in range(n_layer) for n in INT8_ROWWISE} | {"head.weight"}
        self.colwise = {f"blocks.{l}.ffn.value.weight" for l in range(n_layer)}

    def __getitem__(self, name: str) -> np.ndarray:
        if name in self.rowwise:
            return dequantize_rows(*quantize_rows(self.w[name]))
        if name in self.colwise:
            return dequantize_rows(*quantize_rows(np.asarray(self.w[name]).T)).T
        return self.w[name]

    def __contains__(self, name: str) -> bool:
        return name in self.w
