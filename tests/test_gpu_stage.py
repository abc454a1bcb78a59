"""Stage check of the WKV step on its own, ahead of the output projection.

A one-layer model with the 2.9B shape's layer 0 (C 2560, 40 heads, adapter
ranks 64/64/32/320, fp16 weights) is decoded for one step after 24
single-token steps.  The time-mix output before W_o -- (GroupNorm(S r) + bonus * v) * g,
read from the workspace through rwkv7_debug_wkv_out -- and the layer's WKV
state after the step are compared with the fp64 oracle's pieces: the
time-mix inputs, the WKV update (a = -kappa_hat, b = kappa_hat * alpha) and
the time-mix output taken with an identity output matrix.  The GEMV path
(B = 1, fp32 activations) is held to 1e-4; the MFMA path (B = 8, projection
inputs and this output stored in fp16) to 2e-3.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle import rwkv7 as O

pytestmark = pytest.mark.gpu

S32 = synth.R7_2B9
S1 = dataclasses.replace(S32, name="2.9b-layer0", n_layer=1)


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def dev(x):
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device="cuda")


@pytest.fixture(scope="module")
def weights():
    names = [n for n, _, _ in synth.tensor_specs(S32)
             if not n.startswith("blocks.") or n.startswith("blocks.0.")]
    return synth.make_weights(S32, names=names)


@pytest.fixture(scope="module")
def model(weights):
    import rwkv_linear_attention_decode_amd as R
    m = R.Model.from_numpy(S1, weights, n_slots=16, max_B=8, max_T=64)
    yield m
    m.close()


def oracle_stage(W, W_id, st, tok):
    """(time-mix output before W_o [C], layer-0 S after the step [H, N, N])."""
    H = S1.n_head
    x = O.embed(W, [tok])
    u = O.layer_norm(x, W.L(0, "ln1.weight"), W.L(0, "ln1.bias"))
    p = O.tmix_inputs(W, 0, u, st.att_shift[0][None, :], None)
    kh = O.heads_view(p["kappa_hat"], H)
    S_new, y = O.wkv_update(st.S[0][None], O.heads_view(p["r"], H), O.heads_view(p["d"], H),
                            O.heads_view(p["k_tilde"], H), O.heads_view(p["v"], H), -kh,
                            O.heads_view(p["kappa_hat"] * p["alpha"], H))
    og = O.tmix_output(W_id, 0, y.reshape(1, -1), p)[0]
    return og, S_new[0]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("B,tol", [(1, 1e-4), (8, 2e-3)])
def test_wkv_stage_before_output_projection(model, weights, B, tol):
    import rwkv_linear_attention_decode_amd as R
    W = O.Weights(S1, weights, cache=True)
    eye = np.eye(S1.n_embd, dtype=np.float64)
    W_id = O.Weights(S1, dict(weights, **{"blocks.0.att.output.weight": eye}), cache=True)
    rng = np.random.default_rng(100 + B)
    slots = list(range(B))
    prompts = [rng.integers(0, S1.vocab, 24) for _ in slots]
    toks = [int(t) for t in rng.integers(0, S1.vocab, B)]
    model.reset(dev(slots))
    states = []
    one = torch.empty(1, S1.vocab, device="cuda")
    for b in slots:
        # the state before the checked step comes from 24 single-token steps
        # (fp32 activations), so that the comparison measures the step itself
        for tok in prompts[b]:
            model.decode_step(dev([b]), dev([int(tok)]), one)
        st = O.State(S1)
        O.seq(W, st, prompts[b], want_logits=False)
        states.append(st)
    logits = torch.empty(B, S1.vocab, device="cuda")
    model.decode_step(dev(slots), dev(toks), logits)
    addr, f16 = R.rwkv7_debug_wkv_out(model.handle, model.ws, B)
    assert f16 == (B > R.rwkv7_get_option(model.handle, R.OPT_GEMV_MAX_B))
    C = S1.n_embd
    off = addr - model.ws.data_ptr()
    nbytes = B * C * (2 if f16 else 4)
    raw = model.ws[off:off + nbytes].clone()
    got = (raw.view(torch.float16) if f16 else raw.view(torch.float32)).double().cpu().numpy().reshape(B, C)
    assert model.poll_error() == 0
    H, N = S1.n_head, S1.head_size
    worst_y = worst_s = 0.0
    for b in slots:
        og, S_new = oracle_stage(W, W_id, states[b], toks[b])
        gs = model.slot_state(b).cpu().double().numpy()[0, 2 * C:].reshape(H, N, N)
        worst_y = max(worst_y, rel(got[b], og))
        worst_s = max(worst_s, rel(gs, S_new))
    print(f"layer-0 WKV stage, B={B} ({'fp16' if f16 else 'fp32'} output): time-mix output before W_o "
          f"rel L2 {worst_y:.3e}, state after the step {worst_s:.3e}")
    assert worst_y <= tol
    assert worst_s <= tol
