"""Pins of the oracle's elementary pieces against things other than itself:
torch's fp64 library routines, closed forms, hand-worked fixtures and brute
force.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import rwkv7 as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- norms
def test_layer_norm_matches_torch():
    g = _rng(0)
    x = g.standard_normal((5, 256)) * 3 + 1.5
    gam = 1 + 0.1 * g.standard_normal(256)
    bet = 0.1 * g.standard_normal(256)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (256,), torch.from_numpy(gam),
                                         torch.from_numpy(bet), eps=1e-5).numpy()
    np.testing.assert_allclose(O.layer_norm(x, gam, bet), ref, rtol=1e-12, atol=1e-12)


def test_layer_norm_constant_row_gives_beta():
    bet = np.linspace(-1, 1, 64)
    out = O.layer_norm(np.full((1, 64), 0.37), np.ones(64) * 2.0, bet)
    np.testing.assert_allclose(out[0], bet, atol=1e-9)


def test_layer_norm_moments():
    g = _rng(1)
    x = g.standard_normal((3, 512)) * 7 - 2
    y = O.layer_norm(x, np.ones(512), np.zeros(512))
    np.testing.assert_allclose(y.mean(-1), 0, atol=1e-12)
    var = x.var(-1)
    np.testing.assert_allclose(y.var(-1), var / (var + 1e-5), rtol=1e-12)


def test_group_norm_matches_torch():
    g = _rng(2)
    H, N = 4, 64
    y = g.standard_normal((3, H * N)) * 50
    gam = 1 + 0.1 * g.standard_normal(H * N)
    bet = 0.1 * g.standard_normal(H * N)
    ref = torch.nn.functional.group_norm(torch.from_numpy(y), H, torch.from_numpy(gam),
                                         torch.from_numpy(bet), eps=64e-5).numpy()
    np.testing.assert_allclose(O.head_group_norm(y, gam, bet, H), ref, rtol=1e-11, atol=1e-12)


def test_l2_normalize_matches_torch():
    g = _rng(3)
    H, N = 4, 64
    x = g.standard_normal((2, H * N))
    x[1, :N] = 0.0  # a zero head stays zero (clamped norm)
    ref = torch.nn.functional.normalize(torch.from_numpy(x).view(2, H, N), p=2.0, dim=-1,
                                        eps=1e-12).view(2, -1).numpy()
    np.testing.assert_allclose(O.l2_normalize_heads(x, H), ref, rtol=1e-13, atol=0)
    assert np.all(O.l2_normalize_heads(x, H)[1, :N] == 0.0)


# ---------------------------------------------------------------- decay / lerp
def test_decay_closed_form():
    # z = 0: d = exp(-e^-0.5 * 1/2)
    assert O.decay(np.array([0.0]))[0] == pytest.approx(0.7384031, abs=5e-8)
    z = np.linspace(-30, 30, 1001)
    sig = 1 / (1 + np.exp(-z))
    np.testing.assert_allclose(O.decay(z), np.exp(-math.exp(-0.5) * sig), rtol=1e-13)
    # range (exp(-e^-0.5), 1)
    lo = math.exp(-math.exp(-0.5))
    assert lo == pytest.approx(0.545239, abs=1e-6)
    d = O.decay(np.array([-40.0, 40.0]))
    assert d[0] == pytest.approx(1.0, abs=1e-15) and d[1] == pytest.approx(lo, rel=1e-12)
    assert np.all((O.decay(z) > lo - 1e-15) & (O.decay(z) <= 1.0))


def test_token_shift_fresh_slot_closed_form():
    g = _rng(4)
    u = g.standard_normal(32)
    mu = g.random(32)
    np.testing.assert_allclose(O.token_shift_mix(u, np.zeros(32), mu), u * (1 - mu), rtol=1e-13, atol=1e-15)
    prev = g.standard_normal(32)
    np.testing.assert_array_equal(O.token_shift_mix(u, prev, np.zeros(32)), u)
    np.testing.assert_allclose(O.token_shift_mix(u, prev, np.ones(32)), prev, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- WKV closed forms
def test_wkv_golden_n2():
    with open(os.path.join(GOLD, "wkv_n2.json")) as f:
        gold = json.load(f)
    for c in gold["cases"]:
        A = {k: np.array(v, dtype=np.float64) for k, v in c.items() if k != "note"}
        S_new, y = O.wkv_update(A["S"], A["r"], A["d"], A["k_tilde"], A["v"], A["a"], A["b"])
        np.testing.assert_array_equal(S_new, A["S_new"])
        np.testing.assert_array_equal(y, A["y"])


def test_wkv_first_token_from_zero_state():
    g = _rng(5)
    N = 64
    r, d, kt, v = (g.standard_normal(N) for _ in range(4))
    a, b = g.standard_normal(N), g.standard_normal(N)
    S_new, y = O.wkv_update(np.zeros((N, N)), r, np.abs(d), kt, v, a, b)
    np.testing.assert_allclose(S_new, np.outer(v, kt), rtol=1e-15)
    np.testing.assert_allclose(y, v * (kt @ r), rtol=1e-12, atol=1e-13)


def test_wkv_pure_decay_pins_decay_axis():
    g = _rng(6)
    N, T = 64, 20
    S0 = g.standard_normal((N, N))
    S = S0.copy()
    ds = 0.5 + 0.5 * g.random((T, N))
    z = np.zeros(N)
    for t in range(T):
        S, _ = O.wkv_update(S, z, ds[t], z, z, z, z)
    np.testing.assert_allclose(S, S0 * np.prod(ds, axis=0)[None, :], rtol=1e-12)


def test_wkv_delta_rule_recall():
    """d = 1, alpha = 1: a = -k, b = k, k~ = k (unit) => S' k = v exactly."""
    g = _rng(7)
    N = 64
    S = g.standard_normal((N, N))
    for t in range(5):
        k = g.standard_normal(N)
        k /= np.linalg.norm(k)
        v = g.standard_normal(N)
        S, _ = O.wkv_update(S, np.zeros(N), np.ones(N), k, v, -k, k)
        np.testing.assert_allclose(S @ k, v, rtol=1e-10, atol=1e-11)


def test_wkv_value_row_permutation():
    g = _rng(8)
    N = 64
    S = g.standard_normal((N, N))
    r, kt, v, a, b = (g.standard_normal(N) for _ in range(5))
    d = g.random(N)
    perm = g.permutation(N)
    S1, y1 = O.wkv_update(S, r, d, kt, v, a, b)
    S2, y2 = O.wkv_update(S[perm], r, d, kt, v[perm], a, b)
    np.testing.assert_allclose(S2, S1[perm], rtol=1e-13)
    np.testing.assert_allclose(y2, y1[perm], rtol=1e-12)


# ---------------------------------------------------------------- greedy
def _brute_greedy(logits, occ, pres, freq, dec):
    """Brute force: score every index with Python float32 scalars, keep the first best."""
    f32 = np.float32
    best, best_i = None, None
    scores = []
    for i in range(len(logits)):
        l = f32(logits[i])
        if occ[i] > 0:
            l = f32(l - f32(f32(f32(freq) * f32(occ[i])) + f32(pres)))
        scores.append(l)
        if np.isnan(l):
            continue
        if best is None or l > best:
            best, best_i = l, i
    err = best_i is None
    if err:
        best_i = 0
    new = [f32(f32(o) * f32(dec)) for o in occ]
    new[best_i] = f32(new[best_i] + f32(1))
    return best_i, np.array(new, dtype=np.float32), err


def test_greedy_golden():
    with open(os.path.join(GOLD, "greedy_penalty.json")) as f:
        gold = json.load(f)
    rows = gold["rows"]
    conv = lambda a: np.array([float(x) for x in a], dtype=np.float32)
    L = np.stack([conv(r["logits"]) for r in rows])
    occ = np.stack([conv(r["occ"]) for r in rows])
    ids, occ_new, err = O.greedy_penalized(L, occ, [r["presence"] for r in rows],
                                           [r["frequency"] for r in rows], [r["decay"] for r in rows])
    for b, r in enumerate(rows):
        assert ids[b] == r["id"], r["note"]
        assert err[b] == r["error"], r["note"]
        np.testing.assert_array_equal(occ_new[b], conv(r["occ_new"]), err_msg=r["note"])


def test_greedy_brute_force_small():
    g = _rng(9)
    for trial in range(200):
        V = int(g.integers(1, 12))
        L = (g.integers(-3, 4, size=V) * 0.5).astype(np.float32)  # many ties
        if trial % 7 == 0:
            L[g.integers(0, V)] = np.nan
        occ = (g.integers(0, 3, size=V) * g.random(V)).astype(np.float32)
        pres, freq, dec = float(g.random()), float(g.random() * 2), float(0.9 + 0.1 * g.random())
        ids, new, err = O.greedy_penalized(L[None], occ[None], [pres], [freq], [dec])
        bi, bnew, berr = _brute_greedy(L, occ, pres, freq, dec)
        assert ids[0] == bi and err[0] == berr
        np.testing.assert_array_equal(new[0], bnew)
