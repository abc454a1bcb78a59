"""Pins of the oracle's layer assembly against a hand-worked two-layer model.

``tests/golden/layer_n2.json`` holds a two-layer RWKV-7 with C = N = 2, one
head, F = 2, V = 2, adapter ranks 1/1/1/2, and two tokens worked out by hand
in exact rationals (its "design" notes say how each nonlinearity was made to
land on a rational value).  The oracle's decode step, its sequence path and
its pieces (time-mix inputs and output, channel-mix key and value, head) must
reproduce every listed value to 1e-12.

The planted-slip tests then change one term of the oracle's source at a time
(the sign of a, b without alpha, k~ with k_k, the value-residual direction,
bonus and gate placement, the key bias outside the ReLU, ...), load the
changed source as a separate module and show that the fixture rejects it.
CPU only.
"""
import inspect
import json
import os
import types
from fractions import Fraction

import numpy as np
import pytest

from oracle import rwkv7 as O

GOLD = os.path.join(os.path.dirname(__file__), "golden", "layer_n2.json")
RTOL = 1e-12


def _num(x):
    if isinstance(x, list):
        return [_num(y) for y in x]
    if isinstance(x, str):
        return float(Fraction(x))
    return float(x)


def _arr(x):
    return np.array(_num(x), dtype=np.float64)


@pytest.fixture(scope="module")
def fx():
    with open(GOLD) as f:
        return json.load(f)


def _model(mod, fx):
    shape = types.SimpleNamespace(name="layer_n2", **fx["shape"])
    tensors = {k: _arr(v) for k, v in fx["weights"].items()}
    return shape, mod.Weights(shape, tensors, cache=True)


def _close(got, want, what):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    scale = max(float(np.abs(want).max()), 1e-300)
    err = float(np.abs(got - want).max()) / scale
    assert err <= RTOL, f"{what}: max |got - want| / max |want| = {err:.3e}"


def _deviation(mod, fx) -> float:
    """Largest relative deviation of the module's step and sequence paths from
    the fixture (logits after each token, state after each token)."""
    shape, W = _model(mod, fx)
    worst = 0.0

    def dev(got, want):
        want = np.asarray(want, np.float64)
        got = np.asarray(got, np.float64)
        if got.shape != want.shape or not np.all(np.isfinite(got)):
            return np.inf
        return float(np.abs(got - want).max()) / max(float(np.abs(want).max()), 1e-300)

    st = mod.State(shape)
    for t, tok in enumerate(fx["tokens"]):
        lg = mod.step(W, [st], [tok])[0]
        ref = fx["state_after_token"][t]
        worst = max(worst, dev(lg, _arr(fx["logits"][t])), dev(st.S[:, 0], _arr(ref["S"])),
                    dev(st.att_shift, _arr(ref["att_shift"])), dev(st.ffn_shift, _arr(ref["ffn_shift"])))
    sq = mod.State(shape)
    lg = mod.seq(W, sq, fx["tokens"])
    ref = fx["state_after_token"][-1]
    worst = max(worst, dev(lg, _arr(fx["logits"])), dev(sq.S[:, 0], _arr(ref["S"])))
    return worst


# ---------------------------------------------------------------- the oracle as it stands
def test_step_matches_fixture(fx):
    shape, W = _model(O, fx)
    st = O.State(shape)
    for t, tok in enumerate(fx["tokens"]):
        lg = O.step(W, [st], [tok])[0]
        ref = fx["state_after_token"][t]
        _close(lg, _arr(fx["logits"][t]), f"logits after token {t + 1}")
        _close(st.S[:, 0], _arr(ref["S"]), f"S after token {t + 1}")
        _close(st.att_shift, _arr(ref["att_shift"]), f"att_shift after token {t + 1}")
        _close(st.ffn_shift, _arr(ref["ffn_shift"]), f"ffn_shift after token {t + 1}")
        assert st.t == t + 1


@pytest.mark.parametrize("sparse", [False, True])
def test_seq_matches_fixture(fx, sparse):
    shape, W = _model(O, fx)
    st = O.State(shape)
    lg = O.seq(W, st, fx["tokens"], sparse=sparse)
    _close(lg, _arr(fx["logits"]), "sequence logits")
    ref = fx["state_after_token"][-1]
    _close(st.S[:, 0], _arr(ref["S"]), "sequence state")
    _close(st.att_shift, _arr(ref["att_shift"]), "sequence att_shift")
    _close(st.ffn_shift, _arr(ref["ffn_shift"]), "sequence ffn_shift")
    assert st.t == 2


def test_pieces_match_fixture(fx):
    """Each piece on the fixture's inputs: embedding, time-mix inputs (r, k~,
    kappa_hat, alpha, v, g, d), time-mix output, channel-mix key and value,
    head."""
    shape, W = _model(O, fx)
    _close(O.embed(W, fx["tokens"]), _arr(fx["x0"]), "LN0(E[token])")
    v_first = None
    for l in range(shape.n_layer):
        u = W.L(l, "ln1.bias")[None, :]
        u2 = W.L(l, "ln2.bias")[None, :]
        for t in range(2):
            want = fx["layers"][l][t]
            prev = np.zeros_like(u) if t == 0 else u
            vf = None if l == 0 else _arr(fx["layers"][0][t]["v_first"])[None, :]
            p = O.tmix_inputs(W, l, u, prev, vf)
            for name in ("r", "k_tilde", "kappa_hat", "alpha", "v", "g", "d"):
                _close(p[name][0], _arr(want[name]), f"layer {l} token {t + 1} {name}")
            if l == 0:
                _close(p["v_first"][0], _arr(want["v_first"]), f"token {t + 1} v_first")
            y = _arr(want["y"])[None, :]
            _close(O.tmix_output(W, l, y, p)[0], _arr(want["tmix_delta"]), f"layer {l} token {t + 1} tmix")
            prev2 = np.zeros_like(u2) if t == 0 else u2
            z = O.cmix_key(W, l, u2, prev2)
            _close(z[0], _arr(want["key_pre"]), f"layer {l} token {t + 1} key")
            for sparse in (False, True):
                _close(O.cmix_value(W, l, z, sparse)[0], _arr(want["cmix_delta"]),
                       f"layer {l} token {t + 1} value (sparse={sparse})")
    for t in range(2):
        _close(O.head_logits(W, _arr(fx["x_final"][t])[None, :])[0], _arr(fx["logits"][t]), "head")


def test_wkv_update_on_fixture_vectors(fx):
    """The fixture's per-token vectors through wkv_update land on its states
    and readouts (a = -kappa_hat and b = kappa_hat*alpha as listed)."""
    for l in range(2):
        S = np.zeros((2, 2))
        for t in range(2):
            w = fx["layers"][l][t]
            S, y = O.wkv_update(S, _arr(w["r"]), _arr(w["d"]), _arr(w["k_tilde"]), _arr(w["v"]),
                                _arr(w["a"]), _arr(w["b"]))
            _close(S, _arr(w["S"]), f"layer {l} token {t + 1} S")
            _close(y, _arr(w["y"]), f"layer {l} token {t + 1} y")
            _close(_arr(w["a"]), -_arr(w["kappa_hat"]), "a = -kappa_hat")
            _close(_arr(w["b"]), _arr(w["kappa_hat"]) * _arr(w["alpha"]), "b = kappa_hat*alpha")


# ---------------------------------------------------------------- planted slips
_SRC = inspect.getsource(O)

# (name, [(old, new), ...]); every `old` must occur in the oracle's source.
SLIPS = [
    ("a_sign_flipped_in_step_and_seq",
     [('a = -heads_view(p["kappa_hat"], H)', 'a = heads_view(p["kappa_hat"], H)')]),
    ("b_without_alpha",
     [('bb = heads_view(p["kappa_hat"] * p["alpha"], H)', 'bb = heads_view(p["kappa_hat"], H)')]),
    ("k_tilde_with_k_k",
     [('k * (1.0 + (alpha - 1.0) * W.L(l, "att.k_a"))', 'k * (1.0 + (alpha - 1.0) * W.L(l, "att.k_k"))')]),
    ("k_tilde_without_alpha",
     [('k * (1.0 + (alpha - 1.0) * W.L(l, "att.k_a"))', 'k')]),
    ("kappa_not_normalised",
     [('kappa_hat = l2_normalize_heads(k * W.L(l, "att.k_k"), H)', 'kappa_hat = k * W.L(l, "att.k_k")')]),
    ("kappa_without_k_k",
     [('kappa_hat = l2_normalize_heads(k * W.L(l, "att.k_k"), H)', 'kappa_hat = l2_normalize_heads(k, H)')]),
    ("value_residual_reversed",
     [('v = v + (v_first - v) * gate_v', 'v = v_first + (v - v_first) * gate_v')]),
    ("value_residual_dropped",
     [('v = v + (v_first - v) * gate_v', 'v = v')]),
    ("v_first_reset_every_layer",
     [('if l == 0:\n        v_first = v', 'if True:\n        v_first = v')]),
    ("bonus_after_gate",
     [('o = o + (bonus * p["v"].reshape(rk.shape[:-1] + (H, N))).reshape(rk.shape)\n'
       '    return (o * p["g"]) @ W.L(l, "att.output.weight").T',
       'o = o * p["g"] + (bonus * p["v"].reshape(rk.shape[:-1] + (H, N))).reshape(rk.shape)\n'
       '    return o @ W.L(l, "att.output.weight").T')]),
    ("bonus_before_groupnorm",
     [('o = head_group_norm(y, W.L(l, "att.ln_x.weight"), W.L(l, "att.ln_x.bias"), H)\n'
       '    rk = (p["r"] * p["k_tilde"] * W.L(l, "att.r_k").reshape(-1))\n'
       '    bonus = rk.reshape(rk.shape[:-1] + (H, N)).sum(axis=-1, keepdims=True)\n'
       '    o = o + (bonus * p["v"].reshape(rk.shape[:-1] + (H, N))).reshape(rk.shape)',
       'rk = (p["r"] * p["k_tilde"] * W.L(l, "att.r_k").reshape(-1))\n'
       '    bonus = rk.reshape(rk.shape[:-1] + (H, N)).sum(axis=-1, keepdims=True)\n'
       '    y = y + (bonus * p["v"].reshape(rk.shape[:-1] + (H, N))).reshape(rk.shape)\n'
       '    o = head_group_norm(y, W.L(l, "att.ln_x.weight"), W.L(l, "att.ln_x.bias"), H)')]),
    ("bonus_with_k_not_k_tilde",
     [('rk = (p["r"] * p["k_tilde"] * W.L(l, "att.r_k").reshape(-1))',
       'rk = (p["r"] * p["kappa_hat"] * W.L(l, "att.r_k").reshape(-1))')]),
    ("bonus_without_r_k",
     [('rk = (p["r"] * p["k_tilde"] * W.L(l, "att.r_k").reshape(-1))', 'rk = (p["r"] * p["k_tilde"])')]),
    ("gate_before_groupnorm",
     [('o = head_group_norm(y, W.L(l, "att.ln_x.weight"), W.L(l, "att.ln_x.bias"), H)',
       'o = head_group_norm(y * p["g"], W.L(l, "att.ln_x.weight"), W.L(l, "att.ln_x.bias"), H)'),
      ('return (o * p["g"]) @ W.L(l, "att.output.weight").T', 'return o @ W.L(l, "att.output.weight").T')]),
    ("gate_sigmoid_outside",
     [('g = sigmoid(xq["g"] @ W.L(l, "att.g1").T) @ W.L(l, "att.g2").T',
       'g = sigmoid(xq["g"] @ W.L(l, "att.g1").T @ W.L(l, "att.g2").T)')]),
    ("key_bias_outside_relu",
     [('h = np.maximum(pre, 0.0) ** 2', 'h = np.maximum(z, 0.0) ** 2 + W.L(l, "ffn.key.bias")')]),
    ("relu_not_squared",
     [('h = np.maximum(pre, 0.0) ** 2', 'h = np.maximum(pre, 0.0)')]),
    ("lerp_reversed",
     [('return u + (prev - u) * mu', 'return prev + (u - prev) * mu')]),
    ("decay_offset_sign",
     [('np.exp(-np.exp(-softplus(-z) - 0.5))', 'np.exp(-np.exp(-softplus(-z) + 0.5))')]),
    ("w_adapter_without_tanh",
     [('np.tanh(xq["w"] @ W.L(l, "att.w1").T)', '(xq["w"] @ W.L(l, "att.w1").T)')]),
    ("alpha_without_a0",
     [('alpha = sigmoid(W.L(l, "att.a0") + ', 'alpha = sigmoid(0.0 + ')]),
    ("readout_from_old_state",
     [('y = np.matmul(S_new, r[..., :, None])[..., 0]', 'y = np.matmul(S, r[..., :, None])[..., 0]')]),
    ("att_shift_stores_residual",
     [('st.att_shift[l] = u[b]', 'st.att_shift[l] = x[b]'),
      ('state.att_shift[l] = u[-1]', 'state.att_shift[l] = x[-1]')]),
    ("ffn_shift_not_updated",
     [('st.ffn_shift[l] = u2[b]', 'pass'),
      ('state.ffn_shift[l] = u2[-1]', 'pass')]),
]


def _slipped(edits):
    src = _SRC
    for old, new in edits:
        assert old in src, f"slip target not in the oracle's source: {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType("oracle_with_slip")
    exec(compile(src, "oracle_with_slip", "exec"), mod.__dict__)
    return mod


def test_unchanged_source_reloads_clean(fx):
    """The reload route itself changes nothing: the copy matches the fixture."""
    assert _deviation(_slipped([]), fx) <= RTOL


@pytest.mark.parametrize("name,edits", SLIPS, ids=[s[0] for s in SLIPS])
def test_planted_slip_is_caught(fx, name, edits):
    with np.errstate(all="ignore"):
        dev = _deviation(_slipped(edits), fx)
    assert dev > 1e-6, f"slip {name} went unnoticed (deviation {dev:.3e})"
