"""ORACLE: test infrastructure, not product code.

A plain, slow fp64 NumPy forward of RWKV-7 ("Goose", x070).  It exists only to
check the HIP path.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with
the HIP library and does not import it.

What it computes, and where that comes from:

* RWKV-Server article (gitcode.csdn.net, "RWKV 批量推理中 Prefill 的正确打开方式"),
  section 2 table: decode is a single-token O(1) state update, prefill an O(n)
  linear scan over the prompt.  Section 3 lists the parts of a layer:
  LayerNorm, the time-mix "mix6" token-shift lerps, the r/k/v projections, the
  channel-mix key/value, and the per-sequence state
  ``(shift_state, wkv_state, elapsed_t)`` (section 5, Task.prefill listing).
* The pages never write the layer equations out.  The equations below are
  the public RWKV-7 x070 definition: token-shift lerps, r/k/v/o linears,
  low-rank w/a/v/g adapters, decay ``exp(-exp(-softplus(-z) - 0.5))``,
  per-head L2-normalised removal key, rank-1 ``(S a) b^T`` update with
  ``a = -kappa_hat`` and ``b = kappa_hat * alpha``, write ``v k~^T``, readout
  ``S r``, per-head GroupNorm (eps 64e-5), the ``(r . k~ . r_k) v`` bonus, the
  gate, and the ReLU^2 channel-mix.
* One addition that RWKV-7 does not have: a channel-mix key bias, used only
  to make ~85 % of the ReLU^2 outputs zero (the synthetic-weight recipe).

Where the pages are silent, the plainest reading is taken and stated at the function that takes it.

Pins (tests/test_oracle_*.py): LayerNorm / GroupNorm / L2-normalise against
torch's fp64 library routines; decay closed form; WKV closed forms (first
token from zero state, pure decay, delta-rule recall, row permutation) and a
hand-worked N=2 example (tests/golden/wkv_n2.json); a hand-worked two-layer,
two-token model in exact rationals (tests/golden/layer_n2.json) that fixes
the layer assembly -- tmix_inputs (adapters, alpha, kappa_hat, k~, the
v_first residual), tmix_output (GroupNorm, bonus, gate), the key bias inside
the ReLU^2, the a = -kappa_hat / b = kappa_hat*alpha wiring of step and seq,
the shifts and the head -- with planted slips in each that the fixture
rejects; sparse = dense channel-mix; whole-model invariants (sequence =
steps, batch = singles, prefix split, slot permutation, bounded state);
greedy brute force and a hand-worked penalty example
(tests/golden/greedy_penalty.json); the sampler against softmax frequencies
and its exp_fixed against a correctly rounded exp.  Parity against any third party is
unpinned: the pages print no logits, states or weights.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

LN_EPS = 1e-5
GN_EPS = 64e-5
L2_EPS = 1e-12

TMIX_MIX = ("r", "w", "k", "v", "a", "g")


# --------------------------------------------------------------------------
# elementary pieces
# --------------------------------------------------------------------------
def layer_norm(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float = LN_EPS) -> np.ndarray:
    """LayerNorm over the last axis, population variance."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * gamma + beta


def head_group_norm(y: np.ndarray, gamma: np.ndarray, beta: np.ndarray, n_head: int,
                    eps: float = GN_EPS) -> np.ndarray:
    """GroupNorm with one group per head over the last axis ([..., H*N])."""
    shp = y.shape
    yh = y.reshape(shp[:-1] + (n_head, shp[-1] // n_head))
    mu = yh.mean(axis=-1, keepdims=True)
    var = ((yh - mu) ** 2).mean(axis=-1, keepdims=True)
    return ((yh - mu) / np.sqrt(var + eps)).reshape(shp) * gamma + beta


def l2_normalize_heads(x: np.ndarray, n_head: int, eps: float = L2_EPS) -> np.ndarray:
    """x_h / max(||x_h||_2, eps) per head."""
    shp = x.shape
    xh = x.reshape(shp[:-1] + (n_head, shp[-1] // n_head))
    nrm = np.sqrt((xh * xh).sum(axis=-1, keepdims=True))
    return (xh / np.maximum(nrm, eps)).reshape(shp)


def sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


def softplus(z: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, z)


def decay(z: np.ndarray) -> np.ndarray:
    """Per-channel decay from the decay logit z: exp(-exp(-softplus(-z) - 0.5))."""
    return np.exp(-np.exp(-softplus(-z) - 0.5))


def token_shift_mix(u: np.ndarray, prev: np.ndarray, mu: np.ndarray) -> np.ndarray:
    """Token-shift lerp: u + (prev - u) * mu."""
    return u + (prev - u) * mu


def wkv_update(S: np.ndarray, r: np.ndarray, d: np.ndarray, k_tilde: np.ndarray,
               v: np.ndarray, a: np.ndarray, b: np.ndarray):
    """One WKV-7 step for states S[..., i(value), j(key)].

    S' = S diag(d) + (S a) b^T + v k~^T, all terms from the old S; y = S' r.
    Works for any head size N (the last two axes of S).
    """
    Sa = np.matmul(S, a[..., :, None])                       # [..., N, 1]
    S_new = S * d[..., None, :] + Sa * b[..., None, :] + v[..., :, None] * k_tilde[..., None, :]
    y = np.matmul(S_new, r[..., :, None])[..., 0]
    return S_new, y


# --------------------------------------------------------------------------
# model weights (upcast to fp64 on use)
# --------------------------------------------------------------------------
class Weights:
    """Read-only view over the synthetic weight dict, upcasting to fp64.

    ``cache=True`` keeps the fp64 copies (fine for the tiny shape; the large
    shapes upcast per use to bound host memory).
    """

    def __init__(self, shape, tensors: Dict[str, np.ndarray], cache: bool = True):
        self.s = shape
        self.t = tensors
        self.cache = cache
        self._c: Dict[str, np.ndarray] = {}

    def __call__(self, name: str) -> np.ndarray:
        if name in self._c:
            return self._c[name]
        src = self.t[name]
        if src.dtype == np.float16:
            # exact widening; torch's CPU conversion is ~25x faster than NumPy's
            import torch
            a = torch.from_numpy(np.ascontiguousarray(src)).to(torch.float64).numpy()
        else:
            a = np.asarray(src, dtype=np.float64)
        if self.cache:
            self._c[name] = a
        return a

    def L(self, l: int, name: str) -> np.ndarray:
        return self(f"blocks.{l}.{name}")


# --------------------------------------------------------------------------
# state: per sequence, fp64
# --------------------------------------------------------------------------
class State:
    """att_shift[L][C], ffn_shift[L][C], S[L][H][N][N] and the step counter."""

    def __init__(self, shape):
        L, C, H, N = shape.n_layer, shape.n_embd, shape.n_head, shape.head_size
        self.att_shift = np.zeros((L, C))
        self.ffn_shift = np.zeros((L, C))
        self.S = np.zeros((L, H, N, N))
        self.t = 0

    def copy(self) -> "State":
        c = State.__new__(State)
        c.att_shift = self.att_shift.copy()
        c.ffn_shift = self.ffn_shift.copy()
        c.S = self.S.copy()
        c.t = self.t
        return c

    def flat(self) -> np.ndarray:
        """Per layer: att_shift | ffn_shift | S row-major [h][i][j]  -> [L, 2C + H N N]."""
        L = self.S.shape[0]
        return np.concatenate([self.att_shift, self.ffn_shift, self.S.reshape(L, -1)], axis=1)

    @staticmethod
    def from_flat(shape, flat: np.ndarray, t: int = 0) -> "State":
        L, C, H, N = shape.n_layer, shape.n_embd, shape.n_head, shape.head_size
        f = np.asarray(flat, dtype=np.float64).reshape(L, 2 * C + H * N * N)
        st = State(shape)
        st.att_shift = f[:, :C].copy()
        st.ffn_shift = f[:, C:2 * C].copy()
        st.S = f[:, 2 * C:].reshape(L, H, N, N).copy()
        st.t = t
        return st


# --------------------------------------------------------------------------
# layer pieces over R rows (decode rows, or the T tokens of one sequence)
# --------------------------------------------------------------------------
def embed(W: Weights, tokens: Sequence[int]) -> np.ndarray:
    """x = LN0(E[token]) for each token."""
    E = W.t["emb.weight"]
    x = np.asarray(E[np.asarray(tokens, dtype=np.int64)], dtype=np.float64)
    return layer_norm(x, W("ln0.weight"), W("ln0.bias"))


def tmix_inputs(W: Weights, l: int, u: np.ndarray, prev: np.ndarray, v_first: Optional[np.ndarray]):
    """Projections and adapters of the time-mix for rows u (prev = shifted rows).

    Returns a dict with r, k~, kappa_hat, alpha, v (after the value residual),
    g, the decay d, and v_first.
    """
    s = W.s
    H = s.n_head
    xq = {q: token_shift_mix(u, prev, W.L(l, f"att.x_{q}")) for q in TMIX_MIX}
    r = xq["r"] @ W.L(l, "att.receptance.weight").T
    k = xq["k"] @ W.L(l, "att.key.weight").T
    v = xq["v"] @ W.L(l, "att.value.weight").T
    z = W.L(l, "att.w0") + np.tanh(xq["w"] @ W.L(l, "att.w1").T) @ W.L(l, "att.w2").T
    d = decay(z)
    alpha = sigmoid(W.L(l, "att.a0") + (xq["a"] @ W.L(l, "att.a1").T) @ W.L(l, "att.a2").T)
    if l == 0:
        v_first = v
    else:
        gate_v = sigmoid(W.L(l, "att.v0") + (xq["v"] @ W.L(l, "att.v1").T) @ W.L(l, "att.v2").T)
        v = v + (v_first - v) * gate_v
    g = sigmoid(xq["g"] @ W.L(l, "att.g1").T) @ W.L(l, "att.g2").T
    kappa_hat = l2_normalize_heads(k * W.L(l, "att.k_k"), H)
    k_tilde = k * (1.0 + (alpha - 1.0) * W.L(l, "att.k_a"))
    return dict(r=r, k_tilde=k_tilde, kappa_hat=kappa_hat, alpha=alpha, v=v, g=g, d=d,
                v_first=v_first)


def tmix_output(W: Weights, l: int, y: np.ndarray, p: dict) -> np.ndarray:
    """GroupNorm(y) + bonus, gated, through the output projection: the residual delta."""
    s = W.s
    H, N = s.n_head, s.head_size
    o = head_group_norm(y, W.L(l, "att.ln_x.weight"), W.L(l, "att.ln_x.bias"), H)
    rk = (p["r"] * p["k_tilde"] * W.L(l, "att.r_k").reshape(-1))
    bonus = rk.reshape(rk.shape[:-1] + (H, N)).sum(axis=-1, keepdims=True)
    o = o + (bonus * p["v"].reshape(rk.shape[:-1] + (H, N))).reshape(rk.shape)
    return (o * p["g"]) @ W.L(l, "att.output.weight").T


def heads_view(x: np.ndarray, H: int) -> np.ndarray:
    return x.reshape(x.shape[:-1] + (H, x.shape[-1] // H))


def cmix_key(W: Weights, l: int, u: np.ndarray, prev: np.ndarray) -> np.ndarray:
    """Key pre-activation W_key x_k (before the bias)."""
    xk = token_shift_mix(u, prev, W.L(l, "ffn.x_k"))
    return xk @ W.L(l, "ffn.key.weight").T


def cmix_value(W: Weights, l: int, z: np.ndarray, sparse: bool) -> np.ndarray:
    """Value projection of h = relu(z + b_key)^2 (the residual delta).

    ``sparse`` sums only the hidden units whose pre-activation is positive;
    both forms are the same sum.
    """
    pre = z + W.L(l, "ffn.key.bias")
    h = np.maximum(pre, 0.0) ** 2
    Wv = W.L(l, "ffn.value.weight")            # [C, F]
    if not sparse:
        return h @ Wv.T
    out = np.zeros(h.shape[:-1] + (Wv.shape[0],))
    for idx in np.ndindex(h.shape[:-1]):
        nz = np.nonzero(pre[idx] > 0.0)[0]
        out[idx] = Wv[:, nz] @ h[idx][nz]
    return out


def active_set(W: Weights, l: int, z: np.ndarray) -> np.ndarray:
    """Sorted indices f with z_f + b_key_f > 0 (one row)."""
    return np.nonzero(z + W.L(l, "ffn.key.bias") > 0.0)[0]


def head_logits(W: Weights, x: np.ndarray) -> np.ndarray:
    xo = layer_norm(x, W("ln_out.weight"), W("ln_out.bias"))
    return xo @ W("head.weight").T


# --------------------------------------------------------------------------
# decode: one token for each of B independent sequences
# --------------------------------------------------------------------------
def step(W: Weights, states: List[State], tokens: Sequence[int], sparse: bool = False,
         want_logits: bool = True) -> Optional[np.ndarray]:
    """One decode step for B rows (row b uses states[b]); states are updated.

    Returns logits [B, V] (fp64).
    """
    s = W.s
    H = s.n_head
    B = len(states)
    assert len(tokens) == B
    x = embed(W, tokens)
    v_first = None
    for l in range(s.n_layer):
        u = layer_norm(x, W.L(l, "ln1.weight"), W.L(l, "ln1.bias"))
        prev = np.stack([st.att_shift[l] for st in states])
        for b, st in enumerate(states):
            st.att_shift[l] = u[b]
        p = tmix_inputs(W, l, u, prev, v_first)
        v_first = p["v_first"]
        S = np.stack([st.S[l] for st in states])              # [B, H, N, N]
        a = -heads_view(p["kappa_hat"], H)
        bb = heads_view(p["kappa_hat"] * p["alpha"], H)
        S_new, y = wkv_update(S, heads_view(p["r"], H), heads_view(p["d"], H),
                              heads_view(p["k_tilde"], H), heads_view(p["v"], H), a, bb)
        for b, st in enumerate(states):
            st.S[l] = S_new[b]
        x = x + tmix_output(W, l, y.reshape(B, -1), p)
        u2 = layer_norm(x, W.L(l, "ln2.weight"), W.L(l, "ln2.bias"))
        prev2 = np.stack([st.ffn_shift[l] for st in states])
        for b, st in enumerate(states):
            st.ffn_shift[l] = u2[b]
        z = cmix_key(W, l, u2, prev2)
        x = x + cmix_value(W, l, z, sparse)
    for st in states:
        st.t += 1
    return head_logits(W, x) if want_logits else None


# --------------------------------------------------------------------------
# prefill: T tokens of one sequence
# --------------------------------------------------------------------------
def seq(W: Weights, state: State, tokens: Sequence[int], want_logits: bool = True,
        sparse: bool = False) -> Optional[np.ndarray]:
    """Forward T tokens of one sequence from ``state`` (updated in place).

    Projections run over all T rows as matrix products; the token shift of
    row t takes row t-1 (the stored shift for t = 0); the WKV recurrence is a
    loop over t.  Returns logits [T, V] when asked.
    """
    s = W.s
    H = s.n_head
    T = len(tokens)
    if T == 0:
        return np.zeros((0, s.vocab)) if want_logits else None
    x = embed(W, tokens)
    v_first = None
    for l in range(s.n_layer):
        u = layer_norm(x, W.L(l, "ln1.weight"), W.L(l, "ln1.bias"))
        prev = np.concatenate([state.att_shift[l][None, :], u[:-1]], axis=0)
        state.att_shift[l] = u[-1]
        p = tmix_inputs(W, l, u, prev, v_first)
        v_first = p["v_first"]
        a = -heads_view(p["kappa_hat"], H)
        bb = heads_view(p["kappa_hat"] * p["alpha"], H)
        r, d, kt, v = (heads_view(p[n], H) for n in ("r", "d", "k_tilde", "v"))
        S = state.S[l]
        ys = np.empty((T, H, s.head_size))
        for t in range(T):
            S, ys[t] = wkv_update(S, r[t], d[t], kt[t], v[t], a[t], bb[t])
        state.S[l] = S
        x = x + tmix_output(W, l, ys.reshape(T, -1), p)
        u2 = layer_norm(x, W.L(l, "ln2.weight"), W.L(l, "ln2.bias"))
        prev2 = np.concatenate([state.ffn_shift[l][None, :], u2[:-1]], axis=0)
        state.ffn_shift[l] = u2[-1]
        z = cmix_key(W, l, u2, prev2)
        x = x + cmix_value(W, l, z, sparse)
    state.t += T
    return head_logits(W, x) if want_logits else None


# --------------------------------------------------------------------------
# presence / frequency penalty + greedy selection, in IEEE float32
# --------------------------------------------------------------------------
def greedy_penalized(logits: np.ndarray, occ: np.ndarray, presence, frequency, decay_):
    """Penalised greedy pick per row, with the occurrence update.

    Albatross article (RWKV-Runner): decode rows get presence / frequency
    penalties before selection, with a per-step penalty decay (defaults
    frequency penalty 1, decay 0.996).  Reading of the order of operations,
    each a separately rounded float32 op:
      t = freq * occ; p = t + pres; l' = l - p where occ > 0, else l;
      id = lowest index of the maximum of l' (NaN never wins; an all-NaN row
      gives id 0 and an error flag); occ = occ * decay; occ[id] = occ[id] + 1.

    logits, occ: float32 [B, V] (occ rows of the listed slots).  Returns
    (ids int32 [B], new occ float32 [B, V], error bool [B]).
    """
    logits = np.asarray(logits, dtype=np.float32)
    occ = np.asarray(occ, dtype=np.float32)
    B, V = logits.shape
    ids = np.zeros(B, dtype=np.int32)
    err = np.zeros(B, dtype=bool)
    occ_new = np.empty_like(occ)
    for b in range(B):
        f32 = np.float32
        t = np.multiply(f32(frequency[b]), occ[b], dtype=np.float32)
        pen = np.add(t, f32(presence[b]), dtype=np.float32)
        lp = np.where(occ[b] > 0, np.subtract(logits[b], pen, dtype=np.float32), logits[b])
        ok = ~np.isnan(lp)
        if not ok.any():
            best = 0
            err[b] = True
        else:
            m = lp[ok].max()
            best = int(np.nonzero(ok & (lp == m))[0][0])
        ids[b] = best
        o = np.multiply(occ[b], f32(decay_[b]), dtype=np.float32)
        o[best] = np.add(o[best], f32(1.0), dtype=np.float32)
        occ_new[b] = o
    return ids, occ_new, err


def _order_key(z: np.ndarray) -> np.ndarray:
    """float32 -> uint32 increasing with the IEEE total order (-0 before +0)."""
    bits = z.astype(np.float32).view(np.uint32).astype(np.uint64)
    return np.where(bits >> 31, (~bits) & 0xFFFFFFFF, bits | 0x80000000)


# exp for the sampling weights, evaluated by a fixed sequence of IEEE float64
# operations (each rounded to nearest even, none fused), so that any
# implementation that performs the same operations gets the same bits:
# Cody and Waite's argument reduction t = n ln2 + r with ln2 split in two
# (ln2_hi has 40 fractional bits, so n * ln2_hi is exact for |n| <= 32),
# then the degree-13 Taylor polynomial of exp(r), |r| <= ln2 / 2, by Horner's
# rule, scaled by 2**n.  Truncation error < 5e-18 relative; the rounding of
# the 30 operations adds a few ulp.
_EXP_INV_LN2 = float.fromhex("0x1.71547652b82fep+0")     # 1/ln2 rounded to float64
_EXP_LN2_HI = float.fromhex("0x1.62e42fefa4000p-1")      # ln2 rounded to a multiple of 2**-40
_EXP_LN2_LO = float.fromhex("-0x1.8432a1b0e2634p-43")    # ln2 - ln2_hi rounded to float64
_EXP_TAYLOR = [1.0 / math.factorial(k) for k in range(14)]   # 1/k! rounded to float64


def exp_fixed(t) -> np.ndarray:
    """exp(t) for float64 t in [-22, 0] (see the comment above); 0 below -22."""
    t = np.asarray(t, dtype=np.float64)
    inside = t >= -22.0
    ti = np.where(inside, t, 0.0)
    n = np.rint(np.multiply(ti, _EXP_INV_LN2))
    r = np.subtract(np.subtract(ti, np.multiply(n, _EXP_LN2_HI)), np.multiply(n, _EXP_LN2_LO))
    p = np.full_like(ti, _EXP_TAYLOR[13])
    for k in range(12, -1, -1):
        p = np.add(_EXP_TAYLOR[k], np.multiply(r, p))
    return np.where(inside, np.ldexp(p, n.astype(np.int32)), 0.0)


def sample_weights(z: np.ndarray, m) -> np.ndarray:
    """The sampler's fixed-point weights floor(exp(z - m) * 2**31) as int64
    (z float32 candidates, m their maximum): z - m in float64 (exact operands,
    one rounding), exp by exp_fixed, the scaling by 2**31 exact."""
    t = np.subtract(np.asarray(z, dtype=np.float32).astype(np.float64), np.float64(m))
    return np.floor(exp_fixed(t) * 2.0 ** 31).astype(np.int64)


def sample_penalized(logits: np.ndarray, occ: np.ndarray, presence, frequency, decay_, temperature,
                     top_p, top_k, forbidden, uniform):
    """Penalised temperature / top-k / top-p sampling per row, with the occurrence update.

    Albatross article (RWKV-Runner): the adapter inherits the sampling
    defaults temperature 1.0, top_p 0.3, top_k 0 with the penalty defaults of
    greedy_penalized, and the worker masks forbidden tokens, applies the
    presence / frequency penalties and samples the decode rows as one batch.
    The pages give no formulas.  Reading: plain temperature, top-k and nucleus
    sampling, defined so that every decision is exact integer arithmetic:
      l' as in greedy_penalized (float32); z = l' / T (float32);
      candidates: tokens not forbidden with z finite;
      order: z descending (IEEE total order, -0 after +0), then index ascending;
      weight: W = floor(exp(z - max z) * 2**31) (0 .. 2**31), z - max z in
        float64 and exp by exp_fixed (a fixed sequence of float64 operations);
      top-k (0 < k < candidates): the first k candidates in that order;
      top-p (p < 1): the shortest non-empty prefix of those whose weight sum
        reaches ceil(p * S_k) (float64 product, S_k = their weight sum);
      draw: u clamped to [0, 1 - 2**-24]; target = floor(u * S) (float64, S the
        kept weight sum); the first kept token whose running weight sum
        exceeds target;
      T not > 0 (or NaN): z = l' and k = 1 (the penalised greedy pick);
      occ = occ * decay; occ[id] += 1.
    A row with no candidate gives id 0 and an error flag (occ is still updated).

    logits, occ: float32 [B, V] (occ rows of the listed slots); presence,
    frequency, decay_, temperature, top_p, uniform: float32 [B]; top_k: int
    [B]; forbidden: bool [V] or None.  Returns (ids int32 [B], new occ float32
    [B, V], error bool [B]).
    """
    logits = np.asarray(logits, dtype=np.float32)
    occ = np.asarray(occ, dtype=np.float32)
    B, V = logits.shape
    f32 = np.float32
    ids = np.zeros(B, dtype=np.int32)
    err = np.zeros(B, dtype=bool)
    occ_new = np.empty_like(occ)
    idx = np.arange(V, dtype=np.uint64)
    for b in range(B):
        t = np.multiply(f32(frequency[b]), occ[b], dtype=np.float32)
        pen = np.add(t, f32(presence[b]), dtype=np.float32)
        lp = np.where(occ[b] > 0, np.subtract(logits[b], pen, dtype=np.float32), logits[b])
        T = f32(temperature[b])
        greedy = not (T > 0)
        with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
            z = lp if greedy else np.divide(lp, T, dtype=np.float32)
        cand = np.isfinite(z)
        if forbidden is not None:
            cand &= ~np.asarray(forbidden, dtype=bool)
        best = 0
        if not cand.any():
            err[b] = True
        else:
            ci = np.nonzero(cand)[0]
            zc = z[ci]
            comp = (_order_key(zc) << np.uint64(16)) | (np.uint64(0xFFFF) - idx[ci])
            order = ci[np.argsort(comp)[::-1]]                       # descending, unique keys
            m = np.float64(zc.max())
            w = sample_weights(z[order], m)
            n = len(order)
            k = 1 if greedy else int(top_k[b])
            kk = n if (k <= 0 or k >= n) else k
            csum = np.cumsum(w[:kk])
            p = np.float64(f32(top_p[b]))
            keep = kk
            if p < 1.0:
                goal = max(int(np.ceil(p * np.float64(csum[-1]))), 1)
                keep = int(np.searchsorted(csum, goal, side="left")) + 1
            S = int(csum[keep - 1])
            u = f32(uniform[b])
            if not (u >= 0):
                u = f32(0.0)
            if u >= 1:
                u = f32(1.0 - 2.0 ** -24)
            target = int(np.floor(np.float64(u) * np.float64(S)))
            j = int(np.searchsorted(csum[:keep], target, side="right"))   # first running sum > target
            best = int(order[j])
        ids[b] = best
        o = np.multiply(occ[b], f32(decay_[b]), dtype=np.float32)
        o[best] = np.add(o[best], f32(1.0), dtype=np.float32)
        occ_new[b] = o
    return ids, occ_new, err
