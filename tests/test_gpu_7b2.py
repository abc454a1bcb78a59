"""GPU parity at the 7.2B shape (32 layers, C 4096, 64 heads, F 16384,
adapter ranks 128/128/64/480, V 65536, fp16 weights) in the launch
configuration bench.py times for it: B = 256 decode on the MFMA path, slots
prefilled from the workload's 20-2000-token prompt mix in 512-token chunks.

Two seeded slots whose prompts hold 64-512 tokens (so their prefill takes
the chunked WKV scan with the 7.2B adapter ranks) are prefilled by the fp64
oracle and followed for 16 teacher-forced steps of the B = 256 batch:
per-step logits and the states afterwards.  The first step is also
compared, every 8th row, with the same rows stepped alone on the B = 1
path.
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
    m = R.Model.from_numpy(S, weights, n_slots=288, max_B=256, max_T=512)
    yield m
    m.close()


STEPS = 16


@pytest.mark.timeout(1500)
def test_b256_protocol_16_steps(model, weights):
    B = 256
    wl = synth.WORKLOADS["decode_b256_7.2b"]
    lengths = synth.prompt_lengths(wl)
    prompts = [synth.prompt_tokens(wl, b, int(lengths[b])) for b in range(B)]
    feeds = [np.concatenate([p[-1:], synth.teacher_stream(wl, b, STEPS - 1)]).astype(np.int32)
             for b, p in enumerate(prompts)]
    cand = [b for b in range(B) if 64 <= lengths[b] <= 512]
    sub = sorted(int(x) for x in np.random.default_rng(72).choice(cand, 2, replace=False))
    checked = list(range(0, B, 8))
    model.reset(dev(list(range(B + len(checked)))))
    for b in range(B):
        model.prefill(b, dev(prompts[b][:-1]))
    for i, b in enumerate(checked):
        model.prefill(B + i, dev(prompts[b][:-1]))
    logits = torch.empty(B, S.vocab, device="cuda")
    one = torch.empty(1, S.vocab, device="cuda")
    got = np.empty((STEPS, len(sub), S.vocab), np.float32)
    for t in range(STEPS):
        model.decode_step(dev(list(range(B))), dev([int(f[t]) for f in feeds]), logits)
        L = logits.cpu().numpy()
        got[t] = L[sub]
        if t == 0:
            worst = 0.0
            for i, b in enumerate(checked):
                model.decode_step(dev([B + i]), dev([int(feeds[b][0])]), one)
                worst = max(worst, rel(L[b], one.cpu().numpy()[0]))
            print(f"7.2B B=256 vs B=1 rows: worst logits rel L2 {worst:.3e}")
            assert worst <= TOL
    gstates = [model.slot_state(b).cpu().double().numpy() for b in sub]
    assert model.poll_error() == 0

    W = O.Weights(S, weights, cache=True)
    states = []
    for b in sub:
        st = O.State(S)
        O.seq(W, st, prompts[b][:-1], want_logits=False)
        states.append(st)
        print(f"[oracle] slot {b}: {len(prompts[b]) - 1} prompt tokens prefilled", flush=True)
    errs = np.zeros((STEPS, len(sub)))
    for t in range(STEPS):
        ref = O.step(W, states, [int(feeds[b][t]) for b in sub])
        for i in range(len(sub)):
            errs[t, i] = rel(got[t, i], ref[i])
        if t % 4 == 3:
            print(f"[oracle] {t + 1} batched steps", flush=True)
    es = [rel(g, st.flat()) for g, st in zip(gstates, states)]
    print(f"7.2B B=256 slots {sub} (prompts {[int(lengths[b]) for b in sub]} tokens): logits rel L2 over "
          f"{STEPS} steps max {errs.max():.3e} mean {errs.mean():.3e}; state after {STEPS} steps {es}")
    assert errs.max() <= TOL
    assert max(es) <= TOL
