"""GPU parity at the 7.2B shape (32 layers, C 4096, 64 heads, F 16384,
adapter ranks 128/128/64/480, V 65536, fp16 weights) in the launch
configuration bench.py times for it: B = 256 decode on the MFMA path.

Every 8th row of a B = 256 step is compared with the same row stepped alone
on the B = 1 GEMV path; one row is compared with the fp64 oracle (a pass of
the oracle takes tens of seconds at this size, so it is sampled).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import rwkv7 as O

pytestmark = pytest.mark.gpu

S = synth.R7_7B2
TOL = 1e-2


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def dev(x):
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device="cuda")


@pytest.fixture(scope="module")
def weights():
    return synth.make_weights(S)


@pytest.fixture(scope="module")
def model(weights):
    import rwkv_linear_attention_decode_amd as R
    m = R.Model.from_numpy(S, weights, n_slots=288, max_B=256, max_T=64)
    yield m
    m.close()


@pytest.mark.timeout(1200)
def test_b256_rows_vs_b1_and_oracle(model, weights):
    B = 256
    wl = synth.WORKLOADS["decode_b256_7.2b"]
    prompts = [synth.prompt_tokens(wl, b, 4) for b in range(B)]
    checked = list(range(0, B, 8))
    model.reset(dev(list(range(B + len(checked)))))
    for b in range(B):
        model.prefill(b, dev(prompts[b][:-1]))
    for i, b in enumerate(checked):
        model.prefill(B + i, dev(prompts[b][:-1]))
    toks = [int(p[-1]) for p in prompts]
    logits = torch.empty(B, S.vocab, device="cuda")
    one = torch.empty(1, S.vocab, device="cuda")
    model.decode_step(dev(list(range(B))), dev(toks), logits)
    L = logits.cpu().numpy()
    worst = 0.0
    for i, b in enumerate(checked):
        model.decode_step(dev([B + i]), dev([toks[b]]), one)
        worst = max(worst, rel(L[b], one.cpu().numpy()[0]))
    print(f"7.2B B=256 vs B=1 rows: worst logits rel L2 {worst:.3e}")
    assert worst <= TOL
    assert model.poll_error() == 0

    W = O.Weights(S, weights, cache=False)
    b = 77
    st = O.State(S)
    O.seq(W, st, prompts[b][:-1], want_logits=False)
    ref = O.step(W, [st], [toks[b]])[0]
    e = rel(L[b], ref)
    es = rel(model.slot_state(b).cpu().double().numpy(), st.flat())
    print(f"7.2B B=256 row {b} vs oracle: logits {e:.3e}, state {es:.3e}")
    assert e <= TOL
    assert es <= TOL
