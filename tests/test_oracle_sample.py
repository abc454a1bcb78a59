"""Pins of the oracle's sampler (oracle.rwkv7.sample_penalized) against what
the mathematics fixes: the inverse-CDF draw over a fine grid of uniforms
reproduces softmax(l'/T), restricted and renormalised to the top-k or nucleus
(top-p) support; the degenerate settings reduce to the penalised greedy pick
(pinned separately); a hand-worked four-token example pins the order of equal
logits and the top-p cut.  CPU only."""
import numpy as np
import pytest

from oracle import rwkv7 as O


def draw(logits, u, T=1.0, p=1.0, k=0, forbidden=None, occ=None, pres=0.0, freq=0.0):
    """ids for one row of logits over the uniforms u."""
    logits = np.asarray(logits, dtype=np.float32)[None, :]
    occ = np.zeros_like(logits) if occ is None else np.asarray(occ, dtype=np.float32)[None, :]
    out = []
    for x in u:
        ids, _, err = O.sample_penalized(logits, occ, [pres], [freq], [1.0], [T], [p], [k], forbidden, [x])
        assert not err[0]
        out.append(int(ids[0]))
    return np.array(out)


def freqs(logits, n=20000, **kw):
    u = (np.arange(n) + 0.5) / n
    ids = draw(logits, u, **kw)
    return np.bincount(ids, minlength=len(logits)) / n


def softmax(x):
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


def test_hand_worked_four_tokens():
    # probabilities 1/2, 1/4, 1/8, 1/8; tokens 2 and 3 tie and go in index order
    lg = np.log(np.array([4.0, 2.0, 1.0, 1.0])).astype(np.float32)
    assert draw(lg, [0.49, 0.51, 0.74, 0.76, 0.87, 0.88, 0.99]).tolist() == [0, 1, 1, 2, 2, 3, 3]
    # top-p 0.6: 1/2 < 0.6 <= 3/4 keeps tokens 0 and 1, renormalised to 2/3, 1/3
    assert draw(lg, [0.6, 0.66, 0.67, 0.9], p=0.6).tolist() == [0, 0, 1, 1]
    # top-p 0.5 keeps token 0 alone (its mass reaches the threshold exactly)
    assert draw(lg, [0.0, 0.5, 0.999], p=0.5).tolist() == [0, 0, 0]
    # top-k 3: the tie is broken by index, so token 3 is out
    assert set(draw(lg, np.linspace(0, 0.999, 50), k=3).tolist()) == {0, 1, 2}


@pytest.mark.parametrize("T", [1.0, 0.5, 2.0])
def test_draw_follows_softmax(T):
    rng = np.random.default_rng(1)
    lg = rng.normal(size=24).astype(np.float32)
    f = freqs(lg, T=T)
    ref = softmax(np.float64(lg) / np.float64(np.float32(T)))
    assert np.abs(f - ref).max() < 2e-4


def test_top_k_support_and_renormalisation():
    rng = np.random.default_rng(2)
    lg = rng.normal(size=30).astype(np.float32)
    k = 5
    f = freqs(lg, k=k)
    top = np.argsort(-lg)[:k]
    assert set(np.nonzero(f)[0]) == set(top)
    ref = np.zeros(30)
    ref[top] = softmax(lg[top])
    assert np.abs(f - ref).max() < 2e-4


def test_top_p_nucleus():
    lg = np.log(np.array([0.05, 0.30, 0.10, 0.25, 0.20, 0.10])).astype(np.float32)
    # sorted masses 0.30, 0.25, 0.20, ...: p = 0.7 needs 0.30 + 0.25 + 0.20 = 0.75
    f = freqs(lg, p=0.7)
    assert set(np.nonzero(f)[0]) == {1, 3, 4}
    ref = np.zeros(6)
    ref[[1, 3, 4]] = np.array([0.30, 0.25, 0.20]) / 0.75
    assert np.abs(f - ref).max() < 2e-4


def test_degenerate_settings_are_greedy():
    rng = np.random.default_rng(3)
    B, V = 6, 200
    lg = rng.normal(size=(B, V)).astype(np.float32)
    occ = (rng.random((B, V)) < 0.1).astype(np.float32) * rng.integers(1, 4, (B, V)).astype(np.float32)
    pres, freq, dec = np.full(B, 1.0), np.full(B, 1.0), np.full(B, 0.996)
    g_ids, g_occ, _ = O.greedy_penalized(lg, occ, pres, freq, dec)
    u = rng.random(B).astype(np.float32)
    for T, p, k in ((0.0, 1.0, 0), (float("nan"), 0.3, 0), (1.0, 1.0, 1), (0.7, 1e-9, 0)):
        ids, new_occ, err = O.sample_penalized(lg, occ, pres, freq, dec, np.full(B, T, np.float32),
                                               np.full(B, p, np.float32), np.full(B, k), None, u)
        assert not err.any()
        assert ids.tolist() == g_ids.tolist(), (T, p, k)
        assert np.array_equal(new_occ, g_occ)


def test_forbidden_and_penalties():
    lg = np.array([5.0, 4.0, 0.0, -1.0], dtype=np.float32)
    forb = np.array([True, False, False, False])
    u = np.linspace(0, 0.999, 200)
    assert 0 not in set(draw(lg, u, forbidden=forb).tolist())
    assert draw(lg, [0.5], k=1, forbidden=forb).tolist() == [1]
    # presence penalty 10 on token 1 (occ > 0) drops it below token 2
    assert draw(lg, [0.5], k=1, forbidden=forb, occ=[0, 1, 0, 0], pres=10.0).tolist() == [2]
    # every token forbidden: id 0 and the error flag, occ still decays
    ids, occ, err = O.sample_penalized(lg[None], np.ones((1, 4), np.float32), [0.0], [0.0], [0.5], [1.0],
                                       [1.0], [0], np.ones(4, bool), [0.3])
    assert ids[0] == 0 and err[0] and occ[0].tolist() == [1.5, 0.5, 0.5, 0.5]


def test_uniform_is_clamped_and_occ_updated():
    lg = np.log(np.array([1.0, 1.0, 2.0])).astype(np.float32)
    assert draw(lg, [-3.0, float("nan")]).tolist() == [2, 2]          # u -> 0: the heaviest token
    assert draw(lg, [1.0, 7.0]).tolist() == [1, 1]                    # u -> 1 - 2^-24: the last in order
    ids, occ, _ = O.sample_penalized(lg[None], np.array([[2.0, 0.0, 1.0]], np.float32), [0.0], [0.0],
                                     [0.5], [1.0], [1.0], [0], None, [0.0])
    assert ids[0] == 2 and occ[0].tolist() == [1.0, 0.0, 1.5]


def _exp_exact(t):
    """exp(t) to 40 digits (decimal), rounded to float64 (a correctly rounded exp)."""
    from decimal import Decimal, getcontext
    getcontext().prec = 40
    return float(Decimal(float(t)).exp())


def _exp_points():
    rng = np.random.default_rng(11)
    ln2 = np.log(2.0)
    special = [0.0, -0.0, -1e-300, -2.0 ** -60, -ln2 / 2, -ln2, -21.487, -21.5, -22.0]
    special += [-k * ln2 for k in range(1, 32)] + [-(k + 0.5) * ln2 for k in range(31)]
    return np.concatenate([special, -rng.uniform(0, 22, 3000), -rng.uniform(0, 1e-3, 200)])


def test_exp_fixed_is_exp_to_2_ulp():
    """The weights' exp (a fixed float64 operation sequence, so that any
    implementation of the same sequence matches bit for bit) against a
    correctly rounded exp: within 2 ulp over [-22, 0]; exactly 1 at 0 and 0
    below -22."""
    t = _exp_points()
    e = O.exp_fixed(t)
    ref = np.array([_exp_exact(x) for x in t])
    ulp = np.abs(e - ref) / np.spacing(ref)
    assert ulp.max() <= 2.0, (t[np.argmax(ulp)], ulp.max())
    assert O.exp_fixed(np.array([0.0]))[0] == 1.0 and O.exp_fixed(np.array([-0.0]))[0] == 1.0
    assert (O.exp_fixed(np.array([-22.000001, -50.0, -1e30, -np.inf])) == 0.0).all()


def test_sample_weights_fixed_point():
    """floor(exp(z - m) * 2^31): 2^31 at the maximum, 2^(31-k) at z = m - k ln2
    within one unit, 0 once exp(z - m) < 2^-31 (z - m < -21.4875...), and equal
    to the floor of the correctly rounded value except where that value is
    within 1e-6 of an integer."""
    z = np.float32([3.0, 2.5, -18.4, -19.0])
    assert O.sample_weights(z, np.float32(3.0))[0] == 2 ** 31
    ln2 = np.log(2.0)
    for k in range(1, 31):
        zk = np.float32(3.0 - k * ln2)
        w = int(O.sample_weights(np.array([zk]), np.float32(3.0))[0])
        exact = _exp_exact(float(np.float64(zk) - 3.0)) * 2.0 ** 31
        assert w == int(np.floor(exact)) and abs(w - 2.0 ** (31 - k)) <= 2.0 ** (31 - k) * 1e-6 + 1
    assert O.sample_weights(np.float32([-21.48]), np.float32(0.0))[0] == 1
    assert O.sample_weights(np.float32([-21.49]), np.float32(0.0))[0] == 0
    rng = np.random.default_rng(5)
    zs = rng.normal(0, 4, 4000).astype(np.float32)
    m = zs.max()
    w = O.sample_weights(zs, m)
    exact = np.array([_exp_exact(float(np.float64(x) - np.float64(m))) for x in zs]) * 2.0 ** 31
    fl = np.floor(exact)
    near = np.abs(exact - np.round(exact)) < 1e-6
    assert np.array_equal(w[~near], fl[~near].astype(np.int64))
    assert near.sum() <= 2


@pytest.mark.parametrize("slip", ["lo", "degree", "hi"])
def test_exp_fixed_pins_catch_slips(monkeypatch, slip):
    """A dropped low part of ln2, a polynomial two degrees short or ln2_hi
    rounded to fewer bits each break the 2-ulp bound."""
    if slip == "lo":
        monkeypatch.setattr(O, "_EXP_LN2_LO", 0.0)
    elif slip == "degree":
        monkeypatch.setattr(O, "_EXP_TAYLOR", O._EXP_TAYLOR[:12] + [0.0, 0.0])
    else:
        monkeypatch.setattr(O, "_EXP_LN2_HI", float(np.float32(O._EXP_LN2_HI)))
    t = _exp_points()
    e = O.exp_fixed(t)
    ref = np.array([_exp_exact(x) for x in t])
    assert (np.abs(e - ref) / np.spacing(ref)).max() > 2.0
