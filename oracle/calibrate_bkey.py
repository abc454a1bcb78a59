"""ORACLE-side script: calibrate the synthetic channel-mix key bias.

Test infrastructure.  For each model shape, runs the fp64 oracle over the
seeded 64-token calibration stream, layer by layer, and sets layer l's key
bias to minus the 0.85-quantile of that layer's key pre-activations (bias of
earlier layers already applied), so that about 85 % of the ReLU^2 outputs
are zero.  Writes synth/bkey.json, which the input generator only reads.

    python -m oracle.calibrate_bkey tiny 2.9b 7.2b
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

from . import rwkv7 as O

_HERE = os.path.dirname(os.path.abspath(__file__))
_OUT = os.path.join(os.path.dirname(_HERE), "synth", "bkey.json")
QUANTILE = 0.85


def calibrate(shape_name: str) -> dict:
    sys.path.insert(0, os.path.dirname(_HERE))
    import synth
    s = synth.SHAPES[shape_name]
    zeros = [0.0] * s.n_layer
    tokens = synth.calibration_stream(s, 64)
    T = len(tokens)
    H = s.n_head
    glob = synth.make_weights(s, zeros, ["emb.weight", "ln0.weight", "ln0.bias"])
    W = O.Weights(s, glob, cache=True)
    x = O.embed(W, tokens)
    state = O.State(s)
    v_first = None
    bkey, sparsity = [], []
    for l in range(s.n_layer):
        t0 = time.time()
        names = [n for n, _, _ in synth.tensor_specs(s) if n.startswith(f"blocks.{l}.")]
        layer = synth.make_weights(s, zeros, names)
        W = O.Weights(s, {**glob, **layer}, cache=True)
        u = O.layer_norm(x, W.L(l, "ln1.weight"), W.L(l, "ln1.bias"))
        prev = np.concatenate([state.att_shift[l][None, :], u[:-1]], axis=0)
        p = O.tmix_inputs(W, l, u, prev, v_first)
        v_first = p["v_first"]
        a = -O.heads_view(p["kappa_hat"], H)
        bb = O.heads_view(p["kappa_hat"] * p["alpha"], H)
        r, d, kt, v = (O.heads_view(p[n], H) for n in ("r", "d", "k_tilde", "v"))
        S = state.S[l]
        ys = np.empty((T, H, s.head_size))
        for t in range(T):
            S, ys[t] = O.wkv_update(S, r[t], d[t], kt[t], v[t], a[t], bb[t])
        x = x + O.tmix_output(W, l, ys.reshape(T, -1), p)
        u2 = O.layer_norm(x, W.L(l, "ln2.weight"), W.L(l, "ln2.bias"))
        prev2 = np.concatenate([state.ffn_shift[l][None, :], u2[:-1]], axis=0)
        z = O.cmix_key(W, l, u2, prev2)
        b = -float(np.quantile(z, QUANTILE))
        bkey.append(b)
        # the model holds the bias at the weight dtype
        layer["blocks.%d.ffn.key.bias" % l] = np.full(s.ffn, b, np.float32).astype(s.np_dtype)
        W = O.Weights(s, {**glob, **layer}, cache=True)
        sparsity.append(float(np.mean(z + W.L(l, "ffn.key.bias") <= 0.0)))
        x = x + O.cmix_value(W, l, z, sparse=False)
        print(f"[{shape_name}] layer {l}: bkey={b:.6f} zero-frac={sparsity[-1]:.4f} "
              f"({time.time() - t0:.1f}s)", flush=True)
    return {"bkey": bkey, "quantile": QUANTILE, "calib_tokens": int(T),
            "zero_fraction": sparsity}


def main(argv):
    names = argv or ["tiny"]
    tab = {}
    if os.path.exists(_OUT):
        with open(_OUT) as f:
            tab = json.load(f)
    for n in names:
        tab[n] = calibrate(n)
        with open(_OUT, "w") as f:
            json.dump(tab, f, indent=1)
    print("wrote", _OUT)


if __name__ == "__main__":
    main(sys.argv[1:])
