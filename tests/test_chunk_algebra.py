"""The chunked (WY-form) evaluation of the WKV-7 recurrence that the prefill
chunk kernels implement, written out in fp64 NumPy and checked against the
token-by-token recurrence S_t = S_{t-1} (diag(d_t) + a_t b_t^T) + v_t k_t^T,
y_t = S_t r_t (RWKV-Server article, section 2: prefill as an O(n) scan that
must land on the decode state).  CPU only; independent of the oracle and of
the HIP path."""
import numpy as np
import pytest

L = 16


def serial(S0, a, b, k, v, r, d):
    S = S0.copy()
    ys = []
    for t in range(a.shape[0]):
        S = S * d[t][None, :] + np.outer(S @ a[t], b[t]) + np.outer(v[t], k[t])
        ys.append(S @ r[t])
    return S, np.array(ys)


def chunked(S0, a, b, k, v, r, d, slip=False):
    T, N = a.shape
    S = S0.copy()
    ys = []
    for c0 in range(0, T, L):
        n = min(L, T - c0)
        blk = [x[c0:c0 + n] for x in (a, b, k, v, r, d)]
        if n < L:   # padding tokens: d = 1, zero vectors (identity transitions)
            blk = [np.vstack([x, np.full((L - n, N), 1.0 if i == 5 else 0.0)]) for i, x in enumerate(blk)]
        A, B, K, V, R, D = blk
        ell = np.cumsum(np.log(D), axis=0)
        ellm1 = np.vstack([np.zeros((1, N)), ell[:-1]])
        eL = ell[-1][None, :]
        abar, rbar = A * np.exp(ellm1), R * np.exp(ell)
        bhat, khat = B * np.exp(-ell), K * np.exp(-ell)
        btil, ktil = B * np.exp(eL - ell), K * np.exp(eL - ell)
        Cm = np.tril(abar @ bhat.T, -1)
        Em = np.tril(abar @ khat.T, -1)
        Fm = np.tril(rbar @ bhat.T)
        Hm = np.tril(rbar @ khat.T)
        A2 = np.linalg.solve(np.eye(L) - Cm, abar)
        G = np.linalg.solve(np.eye(L) - Cm, Em)
        K2 = ktil + G.T @ btil
        Q = rbar + Fm @ A2
        Z = Fm @ G + Hm
        ys.append((S @ Q.T + (Z @ V).T).T[:n])
        S = S * np.exp(eL) + (S @ (Q if slip else A2).T) @ btil + V.T @ K2
    return S, np.vstack(ys)


def inputs(T, seed, repeat_keys=False, fast_decay=False):
    rng = np.random.default_rng(seed)
    N = 64
    kap = rng.normal(size=(T, N))
    if repeat_keys:
        kap[1::2] = kap[0::2][: T // 2]
    kap /= np.linalg.norm(kap, axis=1, keepdims=True)
    alpha = 1.0 / (1.0 + np.exp(-rng.normal(size=(T, N))))
    z = rng.normal(size=(T, N)) * 2.0 + (8.0 if fast_decay else 0.0)
    d = np.exp(-np.exp(-0.5) / (1.0 + np.exp(-z)))     # (0.545, 1), as the decay of the model
    return (rng.normal(size=(N, N)), -kap, kap * alpha, rng.normal(size=(T, N)) * 0.5,
            rng.normal(size=(T, N)), rng.normal(size=(T, N)), d)


@pytest.mark.parametrize("T,seed,rep,fast", [(1, 0, False, False), (5, 1, False, False), (16, 2, False, False),
                                              (37, 3, False, False), (100, 4, True, False), (64, 5, False, True)])
def test_chunked_equals_serial(T, seed, rep, fast):
    S0, a, b, k, v, r, d = inputs(T, seed, rep, fast)
    Ss, ys = serial(S0, a, b, k, v, r, d)
    Sc, yc = chunked(S0, a, b, k, v, r, d)
    rel = lambda x, y: np.linalg.norm(x - y) / np.linalg.norm(y)
    assert rel(Sc, Ss) < 1e-12
    assert rel(yc, ys) < 1e-12


def test_chunked_catches_a_wrong_term():
    """A plausible slip (the update's low-rank term built from Q instead of A2)
    is visible, so the comparison above has teeth."""
    S0, a, b, k, v, r, d = inputs(40, 9)
    Ss, _ = serial(S0, a, b, k, v, r, d)
    Sc, _ = chunked(S0, a, b, k, v, r, d)
    Sx, _ = chunked(S0, a, b, k, v, r, d, slip=True)
    assert np.linalg.norm(Sc - Ss) / np.linalg.norm(Ss) < 1e-12
    assert np.linalg.norm(Sx - Ss) / np.linalg.norm(Ss) > 1e-2
