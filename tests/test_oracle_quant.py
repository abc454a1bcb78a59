"""Pins of the oracle's int8 weight definition (oracle/quant.py) against what
the definition and arithmetic fix: rows already on the grid come back exactly,
every weight is within s/2 (plus the fp32 rounding of w/s) of its
dequantised value, the largest |w| of a row maps to +-127, zero rows give zero
scales and codes, exact halves round to even, and the value matrix is
scaled per hidden unit (per column of ffn.value.weight).  CPU only."""
import numpy as np

import synth
from oracle import quant as Q


def test_grid_rows_round_trip_exactly():
    rng = np.random.default_rng(0)
    s = np.float32(2.0 ** -9)
    q = rng.integers(-127, 128, size=(6, 64))
    q[:, 0] = np.where(rng.random(6) < 0.5, 127, -127)     # the row maximum sits on the grid
    w = (q * s).astype(np.float16)                          # exact in fp16 (|q| s < 1, 9 fraction bits)
    qq, ss = Q.quantize_rows(w)
    assert np.array_equal(qq, q.astype(np.int8))
    assert np.all(ss == np.float32(127 * s / 127))
    assert np.array_equal(Q.dequantize_rows(qq, ss), w.astype(np.float64))


def test_error_bound_and_extremes():
    rng = np.random.default_rng(1)
    w = (rng.normal(size=(40, 256)) * rng.uniform(0.01, 3, size=(40, 1))).astype(np.float16)
    q, s = Q.quantize_rows(w)
    w64 = w.astype(np.float64)
    err = np.abs(Q.dequantize_rows(q, s) - w64)
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 1e-6) + np.abs(w64) * 2.0 ** -23)
    m = np.abs(w64).max(axis=1)
    assert np.all(s == (m.astype(np.float32) / np.float32(127)))
    arg = np.abs(w64).argmax(axis=1)
    assert np.all(np.abs(q[np.arange(40), arg].astype(int)) == 127)
    assert q.min() >= -127


def test_zero_row_and_ties_to_even():
    s = np.float32(2.0 ** -7)
    row = np.zeros(16, np.float32)
    row[0] = 127 * s
    row[1:6] = np.array([0.5, 1.5, 2.5, -2.5, -3.5]) * s    # exact halves of the step
    w = np.stack([row, np.zeros(16, np.float32)]).astype(np.float16)
    q, sc = Q.quantize_rows(w)
    assert q[0, :6].tolist() == [127, 0, 2, 2, -2, -4]
    assert sc[1] == 0 and not q[1].any()


def test_value_matrix_is_scaled_per_hidden_unit():
    s = synth.TINY
    rng = np.random.default_rng(2)
    w = {}
    for l in range(s.n_layer):
        p = f"blocks.{l}."
        for n in Q.INT8_ROWWISE:
            w[p + n] = rng.normal(size=(8, 32)).astype(np.float16)
        # columns with very different magnitudes: a per-row scale would flatten the small ones to 0
        w[p + "ffn.value.weight"] = (rng.normal(size=(16, 24)) * np.geomspace(1e-3, 1, 24)).astype(np.float16)
    w["head.weight"] = rng.normal(size=(10, 32)).astype(np.float16)
    w["emb.weight"] = rng.normal(size=(10, 32)).astype(np.float16)
    out = Q.int8_weights(w, s.n_layer)
    assert out["emb.weight"] is w["emb.weight"]
    for l in range(s.n_layer):
        v = out[f"blocks.{l}.ffn.value.weight"]
        src = w[f"blocks.{l}.ffn.value.weight"].astype(np.float64)
        col_max = np.abs(src).max(axis=0)
        # each column keeps its own extreme and is accurate to half its own step
        assert np.allclose(np.abs(v).max(axis=0), col_max, rtol=1e-6)
        assert np.all(np.abs(v - src) <= col_max / 127 * 0.5 * (1 + 1e-5))
        r = out[f"blocks.{l}.att.key.weight"]
        assert np.array_equal(r, Q.dequantize_rows(*Q.quantize_rows(w[f"blocks.{l}.att.key.weight"])))


def test_lazy_view_equals_table():
    s = synth.TINY
    w = synth.make_weights(s)
    full = Q.int8_weights(w, s.n_layer)
    lazy = Q.Int8View(w, s.n_layer)
    for name in ("head.weight", "blocks.1.ffn.value.weight", "blocks.0.att.g1", "blocks.0.att.g2", "emb.weight"):
        assert np.array_equal(np.asarray(lazy[name], np.float64), np.asarray(full[name], np.float64)), name
