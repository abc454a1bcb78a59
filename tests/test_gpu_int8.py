"""The int8 weight route (rwkv7_quantize_int8 + RWKV7_OPT_INT8) against the
oracle's int8 definition (oracle/quant.py).

* Codes and scales of every int8 matrix of the tiny model equal the oracle's,
  bit for bit (both sides take the rounding decision in fp32), and the
  padding rows of the fused input matrix are zero.
* Decode at B = 1 and 2 with int8 on matches the oracle whose int8-route
  matrices are replaced by their dequantised values (the prefill before it
  stays on the fp16 weights, as on the GPU), step by step within the logits
  tolerance; the route is really taken (its logits differ from the fp16
  route's by the quantisation noise).  B = 3 falls back to the fp16 path.
* The 2.9B shape at B = 1, the configuration the bench times, for a few
  teacher-forced steps."""
import numpy as np
import pytest
import torch

import synth
from oracle import quant as Q
from oracle import rwkv7 as O

pytestmark = pytest.mark.gpu
TOL = 1e-2


@pytest.fixture(scope="module")
def R():
    import rwkv_linear_attention_decode_amd as R
    return R


@pytest.fixture(scope="module")
def weights():
    return synth.make_weights(synth.TINY)


@pytest.fixture(scope="module")
def tiny(weights, R):
    S = synth.TINY
    m = R.Model.from_numpy(S, weights, n_slots=8, max_B=4, max_T=64)
    buf = torch.empty(R.rwkv7_int8_bytes(m.cfg), dtype=torch.uint8, device="cuda")
    R.rwkv7_quantize_int8(m.handle, buf)
    torch.cuda.synchronize()
    yield m, buf
    m.close()


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def dev(x):
    return torch.as_tensor(np.asarray(x, np.int32), device="cuda")


def read_matrix(R, m, buf, layer, which):
    c, s, rows, K = R.rwkv7_debug_int8_matrix(m.handle, layer, which)
    base = buf.data_ptr()
    codes = buf[c - base: c - base + rows * K].cpu().numpy().reshape(rows, K).astype(np.int16) - 128
    sc = buf[s - base: s - base + rows * 4].cpu().view(torch.float32).numpy()
    return codes, sc


def test_codes_and_scales_bit_exact(R, tiny, weights):
    m, buf = tiny
    S = synth.TINY
    C = S.n_embd
    for l in range(S.n_layer):
        p = f"blocks.{l}."
        codes, sc = read_matrix(R, m, buf, l, 0)
        row = 0
        for name, n in (("att.receptance.weight", C), ("att.key.weight", C), ("att.value.weight", C),
                        ("att.w1", S.d_w), ("att.a1", S.d_a), ("att.v1", S.d_v), ("att.g1", S.d_g)):
            q, s = Q.quantize_rows(weights[p + name])
            assert np.array_equal(codes[row:row + n], q), (l, name)
            assert np.array_equal(sc[row:row + n], s), (l, name)
            pad = (n + 63) // 64 * 64
            assert not codes[row + n:row + pad].any() and not sc[row + n:row + pad].any()
            row += pad
        assert row == codes.shape[0]
        for which, name, tr in ((1, "att.output.weight", False), (2, "ffn.key.weight", False),
                                (3, "ffn.value.weight", True)):
            codes, sc = read_matrix(R, m, buf, l, which)
            w = weights[p + name]
            q, s = Q.quantize_rows(np.asarray(w).T if tr else w)
            assert np.array_equal(codes, q) and np.array_equal(sc, s), (l, name)
    codes, sc = read_matrix(R, m, buf, 0, 4)
    q, s = Q.quantize_rows(weights["head.weight"])
    assert np.array_equal(codes, q) and np.array_equal(sc, s)


@pytest.mark.parametrize("B", [1, 2])
def test_int8_decode_matches_oracle(R, tiny, weights, B):
    m, _ = tiny
    S = synth.TINY
    W = O.Weights(S, weights)
    W8 = O.Weights(S, Q.int8_weights(weights, S.n_layer))
    rng = np.random.default_rng(30 + B)
    slots = list(range(B))
    m.reset(dev(slots))
    states = []
    for b in range(B):
        pr = rng.integers(0, S.vocab, 9 + 4 * b)
        m.prefill(b, dev(pr))
        st = O.State(S)
        O.seq(W, st, pr.tolist(), want_logits=False)
        states.append(st)
    logits = torch.empty(B, S.vocab, device="cuda")
    worst = 0.0
    R.rwkv7_set_option(m.handle, R.OPT_INT8, 1)
    for t in range(12):
        toks = rng.integers(0, S.vocab, B)
        m.decode_step(dev(slots), dev(toks), logits)
        got = logits.cpu().numpy().copy()
        ref = O.step(W8, states, toks.tolist())
        for b in range(B):
            e = rel(got[b], ref[b])
            worst = max(worst, e)
            assert e <= TOL, (t, b, e)
    print(f"B={B}: worst logits rel error vs the int8 oracle {worst:.2e}")
    for b in range(B):
        g = m.slot_state(b).cpu().double().numpy()
        assert rel(g, states[b].flat()) <= TOL
    # the route is taken: the fp16 route gives visibly different logits on the same state
    snap = m.pool.clone()
    R.rwkv7_set_option(m.handle, R.OPT_INT8, 0)
    toks = dev(rng.integers(0, S.vocab, B))
    m.decode_step(dev(slots), toks, logits)
    l16 = logits.cpu().numpy().copy()
    m.pool.copy_(snap)
    R.rwkv7_set_option(m.handle, R.OPT_INT8, 1)
    m.decode_step(dev(slots), toks, logits)
    l8 = logits.cpu().numpy().copy()
    R.rwkv7_set_option(m.handle, R.OPT_INT8, 0)
    assert rel(l8, l16) > 1e-4


def test_int8_b3_keeps_fp16_and_option_checks(R, tiny, weights):
    m, buf = tiny
    S = synth.TINY
    slots = dev([0, 1, 2])
    m.reset(slots)
    snap = m.pool.clone()
    toks = dev([3, 4, 5])
    out = []
    for flag in (0, 1):
        m.pool.copy_(snap)
        R.rwkv7_set_option(m.handle, R.OPT_INT8, flag)
        logits = torch.empty(3, S.vocab, device="cuda")
        m.decode_step(slots, toks, logits)
        out.append(logits.cpu().numpy())
    R.rwkv7_set_option(m.handle, R.OPT_INT8, 0)
    assert np.array_equal(out[0], out[1])
    m2 = R.Model.from_numpy(S, weights, n_slots=2, max_B=2, max_T=16)
    with pytest.raises(R.RWKV7Error):
        R.rwkv7_set_option(m2.handle, R.OPT_INT8, 1)
    with pytest.raises(R.RWKV7Error):
        R.rwkv7_quantize_int8(m2.handle, buf[:1024])
    m2.close()


@pytest.mark.timeout(900)
def test_int8_2b9_b1_steps(R):
    S = synth.R7_2B9
    w = synth.make_weights(S)
    m = R.Model.from_numpy(S, w, n_slots=1, max_B=1, max_T=64)
    buf = torch.empty(R.rwkv7_int8_bytes(m.cfg), dtype=torch.uint8, device="cuda")
    R.rwkv7_quantize_int8(m.handle, buf)
    R.rwkv7_set_option(m.handle, R.OPT_INT8, 1)
    wl = synth.WORKLOADS["decode_b1_2.9b"]
    p = synth.prompt_tokens(wl, 0, 16)
    feeds = np.concatenate([p[15:16], synth.teacher_stream(wl, 0, 3)]).astype(np.int32)
    m.reset(dev([0]))
    m.prefill(0, dev(p[:15]))
    out = torch.empty(len(feeds), S.vocab, device="cuda")
    for t, tok in enumerate(feeds):
        m.decode_step(dev([0]), dev([tok]), out[t:t + 1])
    got = out.cpu().numpy()
    # oracle: fp16 weights for the prefill, the int8 definition for the steps
    st = O.State(S)
    O.seq(O.Weights(S, w, cache=False), st, p[:15].tolist(), want_logits=False)
    ref = O.seq(O.Weights(S, Q.Int8View(w, S.n_layer), cache=False), st, feeds.tolist())
    errs = [rel(got[t], ref[t]) for t in range(len(feeds))]
    print("2.9B int8 B=1 logits rel errors:", ["%.2e" % e for e in errs])
    assert max(errs) <= TOL
    m.close()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("shape,B", [("2.9b", 2), ("7.2b", 1)])
def test_int8_full_shapes(R, shape, B):
    """The other GEMV instantiations at full size: B = 2 at K = 2560 and B = 1
    at K = 4096 (the 7.2B shape), a few teacher-forced steps after short
    prefills, against the int8 oracle."""
    S = synth.R7_2B9 if shape == "2.9b" else synth.R7_7B2
    w = synth.make_weights(S)
    m = R.Model.from_numpy(S, w, n_slots=B, max_B=B, max_T=64)
    buf = torch.empty(R.rwkv7_int8_bytes(m.cfg), dtype=torch.uint8, device="cuda")
    R.rwkv7_quantize_int8(m.handle, buf)
    R.rwkv7_set_option(m.handle, R.OPT_INT8, 1)
    rng = np.random.default_rng(77)
    prompts = [rng.integers(0, S.vocab, 6 + 3 * b) for b in range(B)]
    feeds = rng.integers(0, S.vocab, (2, B))
    m.reset(dev(list(range(B))))
    for b in range(B):
        m.prefill(b, dev(prompts[b]))
    out = torch.empty(B, S.vocab, device="cuda")
    got = []
    for t in range(len(feeds)):
        m.decode_step(dev(list(range(B))), dev(feeds[t]), out)
        got.append(out.cpu().numpy().copy())
    W16 = O.Weights(S, w, cache=False)
    W8 = O.Weights(S, Q.Int8View(w, S.n_layer), cache=False)
    errs = []
    for b in range(B):
        st = O.State(S)
        O.seq(W16, st, prompts[b].tolist(), want_logits=False)
        ref = O.seq(W8, st, [int(feeds[t][b]) for t in range(len(feeds))])
        errs += [rel(got[t][b], ref[t]) for t in range(len(feeds))]
    print(f"{shape} int8 B={B} logits rel errors:", ["%.2e" % e for e in errs])
    assert max(errs) <= TOL
    m.close()
