"""rwkv7_sample (penalised temperature / top-k / top-p sampling) through the
C ABI against the oracle's sampler on the same logits and uniforms: ids and
the updated occurrence rows bit for bit (every decision is integer
arithmetic on fp64 fixed-point weights, the penalties separately rounded
fp32 ops).  Peaky and nearly flat logits (tens of thousands of tokens inside
the nucleus), penalties, a forbidden mask, the greedy special case against
rwkv7_greedy, the all-forbidden error and the host-side checks."""
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
