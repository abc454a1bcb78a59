"""rwkv7_sample (penalised temperature / top-k / top-p sampling) through the
C ABI against the oracle's sampler on the same logits and uniforms: ids and
the updated occurrence rows bit for bit (every decision is integer
arithmetic on fixed-point weights from a fixed sequence of fp64 operations,
the penalties separately rounded fp32 ops).  Peaky and nearly flat logits
(tens of thousands of tokens inside the nucleus), a whole row inside one
top-level bin, every split of a row over workgroups, penalties (with ties
that a fused multiply-add would break), a forbidden mask, the greedy special
case against rwkv7_greedy, the all-forbidden error and the host-side checks."""
import numpy as np
import pytest
import torch

from oracle import rwkv7 as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def R():
    import rwkv_linear_attention_decode_amd as R
    return R


def run(R, logits, occ_rows, pres, freq, dec, T, p, k, forb, u):
    """One rwkv7_sample call over B rows (slot b = row b of a fresh occ pool)."""
    B, V = logits.shape
    dev = "cuda"
    f = lambda x: torch.tensor(np.asarray(x, np.float32), device=dev)
    occ = f(occ_rows).contiguous()
    ids = torch.zeros(B, dtype=torch.int32, device=dev)
    ws = torch.zeros(R.rwkv7_sample_workspace_bytes(B, V), dtype=torch.uint8, device=dev)
    fb = None if forb is None else torch.tensor(np.asarray(forb, np.uint8), device=dev)
    R.rwkv7_sample(f(logits), occ, B, torch.arange(B, dtype=torch.int32, device=dev), f(pres), f(freq), f(dec),
                   f(T), f(p), torch.tensor(np.asarray(k, np.int32), device=dev), fb, f(u), ids, ws)
    err = R.rwkv7_poll_error(ws)
    return ids.cpu().numpy(), occ.cpu().numpy(), err


def case(seed, B, V, scale, T, p, k, with_occ=True, forb_frac=0.0):
    rng = np.random.default_rng(seed)
    lg = (rng.normal(size=(B, V)) * scale).astype(np.float32)
    occ = np.zeros((B, V), np.float32)
    if with_occ:
        m = rng.random((B, V)) < 0.02
        occ[m] = rng.integers(1, 5, m.sum()).astype(np.float32) * np.float32(0.996)
    forb = (rng.random(V) < forb_frac) if forb_frac else None
    u = rng.random(B).astype(np.float32)
    return (lg, occ, np.full(B, 1.0), np.full(B, 1.0), np.full(B, 0.996), np.full(B, T), np.full(B, p),
            np.full(B, k), forb, u)


@pytest.mark.parametrize("V", [1024, 65536])
@pytest.mark.parametrize("scale,T,p,k", [(3.0, 1.0, 0.3, 0), (3.0, 0.7, 0.9, 50), (0.1, 1.0, 0.3, 0),
                                         (0.1, 1.3, 1.0, 0), (1.0, 1.0, 1.0, 7), (2.0, 0.5, 0.05, 0)])
def test_sample_matches_oracle(R, V, scale, T, p, k):
    args = case(int(scale * 10 + T * 100 + p * 1000 + k + V), 5, V, scale, T, p, k, forb_frac=0.01)
    ids, occ, err = run(R, *args)
    o_ids, o_occ, o_err = O.sample_penalized(*args)
    assert err == 0 and not o_err.any()
    assert ids.tolist() == o_ids.tolist()
    assert np.array_equal(occ, o_occ)


def test_sample_many_uniforms_flat_row(R):
    """A nearly flat 65536-token row: the nucleus holds tens of thousands of
    tokens; 64 uniforms across [0, 1) on copies of the row."""
    rng = np.random.default_rng(7)
    V, B = 65536, 64
    row = (rng.normal(size=V) * 0.05).astype(np.float32)
    lg = np.tile(row, (B, 1))
    occ = np.zeros((B, V), np.float32)
    u = ((np.arange(B) + rng.random(B)) / B).astype(np.float32)
    args = (lg, occ, np.zeros(B), np.zeros(B), np.ones(B), np.ones(B), np.full(B, 0.3), np.zeros(B, int), None, u)
    ids, _, err = run(R, *args)
    o_ids, _, _ = O.sample_penalized(*args)
    assert err == 0
    assert ids.tolist() == o_ids.tolist()
    assert len(set(ids.tolist())) > 32


@pytest.mark.parametrize("B,V", [(1, 1000), (1, 4097), (3, 65535), (37, 65536), (300, 4097)])
def test_sample_chunking(R, B, V):
    """Row counts and vocabulary sizes that give every split of a row over
    workgroups (64 down to 1), ragged chunks, and rows whose maximum is the
    last token."""
    rng = np.random.default_rng(B * 100003 + V)
    lg = (rng.normal(size=(B, V)) * 2.0).astype(np.float32)
    lg[::3, V - 1] = 9.0
    occ = np.zeros((B, V), np.float32)
    m = rng.random((B, V)) < 0.05
    occ[m] = rng.integers(1, 4, m.sum()).astype(np.float32)
    T = rng.choice([0.0, 0.8, 1.0, 1.5], B)
    p = rng.choice([0.1, 0.3, 0.95, 1.0], B)
    k = rng.choice([0, 0, 1, 40], B)
    args = (lg, occ, np.full(B, 0.3), np.full(B, 0.7), np.full(B, 0.99), T, p, k,
            rng.random(V) < 0.02, rng.random(B).astype(np.float32))
    ids, occ_g, err = run(R, *args)
    o_ids, o_occ, o_err = O.sample_penalized(*args)
    assert err == 0 and not o_err.any()
    assert ids.tolist() == o_ids.tolist()
    assert np.array_equal(occ_g, o_occ)


@pytest.mark.parametrize("kind", ["one_bin", "all_equal"])
def test_sample_crowded_top_bin(R, kind):
    """Every token in one top-level bin (more than the 4096 the selection
    gathers into LDS): z in [0.5, 0.5625), or all logits equal so that only
    the index orders them."""
    V, B = 65536, 8
    rng = np.random.default_rng(21)
    row = (0.5 + rng.uniform(0, 0.06, V)).astype(np.float32) if kind == "one_bin" else np.zeros(V, np.float32)
    lg = np.tile(row, (B, 1))
    u = ((np.arange(B) + rng.random(B)) / B).astype(np.float32)
    args = (lg, np.zeros((B, V), np.float32), np.zeros(B), np.zeros(B), np.ones(B), np.ones(B),
            np.array([0.3, 1.0, 0.05, 0.5, 0.9, 1.0, 0.3, 0.7]), np.array([0, 0, 0, 100, 0, 5000, 9000, 0]),
            None, u)
    ids, occ, err = run(R, *args)
    o_ids, o_occ, _ = O.sample_penalized(*args)
    assert err == 0
    assert ids.tolist() == o_ids.tolist()
    assert np.array_equal(occ, o_occ)


def _penalty_cases(n, seed):
    """float32 (frequency, occurrence, presence) with frequency * occurrence +
    presence rounded once (an FMA) different from the product rounded and then
    the sum rounded (more than 0.6 ulp between the exact value and the latter)."""
    from fractions import Fraction
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        f, o, p = rng.uniform(0.1, 2.0, 3).astype(np.float32)
        two = np.float32(np.float32(f * o) + p)
        exact = Fraction(float(f)) * Fraction(float(o)) + Fraction(float(p))
        if abs(exact - Fraction(float(two))) > Fraction(float(np.spacing(two))) * Fraction(6, 10):
            out.append((f, o, p, two))
    return out


def test_penalty_rounded_per_operation(R):
    """The penalty l - (frequency * occ + presence) takes three separately
    rounded fp32 operations in both selections.  Each case is a tie: row A
    penalises token 0 (logit 0) against token 1 whose logit is the separately
    rounded penalised value; row B swaps them.  The lower index wins a tie, so
    the pick is 0 in both rows; a fused multiply-add moves token 0 (row A) or
    token 1 (row B) by an ulp and picks 1 in one of them."""
    cases = _penalty_cases(32, 3)
    V, B = 256, 2 * len(cases)
    lg = np.full((B, V), -50.0, np.float32)
    occ = np.zeros((B, V), np.float32)
    pres, freq = np.zeros(B, np.float32), np.zeros(B, np.float32)
    for i, (f, o, p, two) in enumerate(cases):
        a, b = 2 * i, 2 * i + 1
        lg[a, 0], occ[a, 0], lg[a, 1] = 0.0, o, -two
        lg[b, 0], lg[b, 1], occ[b, 1] = -two, 0.0, o
        pres[a] = pres[b] = p
        freq[a] = freq[b] = f
    dec = np.full(B, 0.75, np.float32)
    for T, k in ((0.0, 0), (1.0, 1)):
        args = (lg, occ, pres, freq, dec, np.full(B, T), np.ones(B), np.full(B, k), None, np.full(B, 0.5))
        o_ids, o_occ, _ = O.sample_penalized(*args)
        assert (o_ids == 0).all()
        ids, occ_g, err = run(R, *args)
        assert err == 0 and ids.tolist() == o_ids.tolist(), T
        assert np.array_equal(occ_g, o_occ)
    dev = "cuda"
    f = lambda x: torch.tensor(np.asarray(x, np.float32), device=dev)
    g_occ, g_ids = f(occ), torch.zeros(B, dtype=torch.int32, device=dev)
    ws = torch.zeros(R.rwkv7_greedy_workspace_bytes(B, V), dtype=torch.uint8, device=dev)
    R.rwkv7_greedy(f(lg), g_occ, B, torch.arange(B, dtype=torch.int32, device=dev), f(pres), f(freq), f(dec),
                   g_ids, ws)
    assert g_ids.cpu().tolist() == [0] * B
    assert np.array_equal(g_occ.cpu().numpy(), o_occ)


def test_greedy_special_case_and_determinism(R):
    args = list(case(11, 6, 4096, 2.0, 0.0, 0.3, 0))
    ids, occ, _ = run(R, *args)
    # T = 0: the penalised greedy pick, as rwkv7_greedy computes it
    lg, occ0 = args[0], args[1]
    B, V = lg.shape
    g_ids = torch.zeros(B, dtype=torch.int32, device="cuda")
    g_occ = torch.tensor(occ0, device="cuda")
    ws = torch.zeros(R.rwkv7_greedy_workspace_bytes(B, V), dtype=torch.uint8, device="cuda")
    f = lambda x: torch.tensor(np.asarray(x, np.float32), device="cuda")
    R.rwkv7_greedy(f(lg), g_occ, B, torch.arange(B, dtype=torch.int32, device="cuda"), f(args[2]), f(args[3]),
                   f(args[4]), g_ids, ws)
    assert ids.tolist() == g_ids.cpu().tolist()
    assert np.array_equal(occ, g_occ.cpu().numpy())
    # same inputs twice: same picks
    args2 = list(case(12, 6, 65536, 0.5, 1.0, 0.3, 0))
    a, _, _ = run(R, *args2)
    b, _, _ = run(R, *args2)
    assert a.tolist() == b.tolist()


def test_all_forbidden_flags_error(R):
    B, V = 2, 512
    lg = np.zeros((B, V), np.float32)
    args = (lg, np.zeros((B, V), np.float32), np.zeros(B), np.zeros(B), np.ones(B), np.ones(B), np.ones(B),
            np.zeros(B, int), np.ones(V, bool), np.full(B, 0.5))
    ids, occ, err = run(R, *args)
    assert ids.tolist() == [0, 0]
    assert err & R.ERR_ALL_NAN
    assert occ[:, 0].tolist() == [1.0, 1.0]


def test_sample_host_errors(R):
    dev = "cuda"
    V = 70000
    lg = torch.zeros(1, V, device=dev)
    one = torch.ones(1, device=dev)
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device=dev)
    sl = torch.zeros(1, dtype=torch.int32, device=dev)
    with pytest.raises(R.RWKV7Error):
        R.rwkv7_sample(lg, torch.zeros(1, V, device=dev), 1, sl, one, one, one, one, one,
                       torch.zeros(1, dtype=torch.int32, device=dev), None, one, sl, ws)
    lg = torch.zeros(4, 4096, device=dev)
    with pytest.raises(R.RWKV7Error):
        R.rwkv7_sample(lg, torch.zeros(4, 4096, device=dev), 4, torch.arange(4, dtype=torch.int32, device=dev),
                       *(torch.ones(4, device=dev),) * 5, torch.zeros(4, dtype=torch.int32, device=dev), None,
                       torch.ones(4, device=dev) * 0.5, torch.zeros(4, dtype=torch.int32, device=dev),
                       torch.zeros(64, dtype=torch.uint8, device=dev))
