"""GPU parity of the HIP path against the fp64 oracle on the tiny shape
(2 layers, C=256, 4 heads, F=1024, V=1024), through the C ABI.

Tolerances: per-step logits relative L2 <= 1e-2, slot-state relative L2
<= 1e-2; greedy ids, occurrence updates, slot bookkeeping and sparse
active sets bit-exact.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import rwkv7 as O

pytestmark = pytest.mark.gpu

S = synth.TINY
TOL = 1e-2
NSLOT = 16


@pytest.fixture(scope="module")
def weights():
    return synth.make_weights(S)


@pytest.fixture(scope="module")
def W(weights):
    return O.Weights(S, weights)


@pytest.fixture(scope="module")
def R():
    import rwkv_linear_attention_decode_amd as R
    return R


@pytest.fixture(scope="module")
def model(weights, R):
    m = R.Model.from_numpy(S, weights, n_slots=NSLOT, max_B=8, max_T=64)
    yield m
    m.close()


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def dev(x):
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device="cuda")


def gstate(m, slot):
    torch.cuda.synchronize()
    return m.slot_state(slot).cpu().double().numpy()


def fresh(m, slots):
    m.reset(dev(slots))


def prompt(seed, n):
    return np.random.default_rng(seed).integers(0, S.vocab, size=n).astype(np.int32)


def test_tiny_workload_teacher_forced(model, W):
    """The tiny workload: 8-token prompt (7 prefilled, the 8th fed to the first
    decode step), then 16 decode steps on a teacher-forced stream."""
    wl = synth.WORKLOADS["tiny"]
    p = synth.prompt_tokens(wl, 0, 8)
    feeds = [int(p[7])] + [int(t) for t in synth.teacher_stream(wl, 0, 15)]
    fresh(model, [0])
    model.prefill(0, dev(p[:7]))
    st = O.State(S)
    O.seq(W, st, p[:7], want_logits=False)
    assert rel(gstate(model, 0), st.flat()) <= TOL
    logits = torch.empty(1, S.vocab, device="cuda")
    worst = 0.0
    for tok in feeds:
        model.decode_step(dev([0]), dev([tok]), logits)
        ref = O.step(W, [st], [tok])[0]
        e = rel(logits[0].cpu().numpy(), ref)
        worst = max(worst, e)
        assert e <= TOL
    assert rel(gstate(model, 0), st.flat()) <= TOL
    assert int(model.counters()[0].item()) == 7 + 16
    assert model.poll_error() == 0
    print(f"tiny worst step logits rel L2 = {worst:.3e}")


def test_tiny_free_running_greedy(model, W, R):
    wl = synth.WORKLOADS["tiny"]
    p = synth.prompt_tokens(wl, 0, 8)
    fresh(model, [1])
    model.prefill(1, dev(p[:7]))
    st = O.State(S)
    O.seq(W, st, p[:7], want_logits=False)
    occ = torch.zeros(NSLOT, S.vocab, device="cuda")
    zeros = torch.zeros(1, device="cuda")
    ones = torch.ones(1, device="cuda")
    ids = torch.zeros(1, dtype=torch.int32, device="cuda")
    logits = torch.empty(1, S.vocab, device="cuda")
    tok = int(p[7])
    for step in range(16):
        model.decode_step(dev([1]), dev([tok]), logits)
        model.greedy(logits, occ, dev([1]), zeros, zeros, ones, ids)
        ref = O.step(W, [st], [tok])[0]
        g = int(ids.item())
        r = int(np.argmax(ref))
        if g != r:
            srt = np.sort(ref)
            err = float(np.abs(logits[0].cpu().double().numpy() - ref).max())
            assert srt[-1] - srt[-2] < err, f"step {step}: ids differ with margin above the error"
            break
        tok = g


@pytest.mark.parametrize("B,gemv,sparse,fuse,fval", [
    (1, 2, 4, 1, 1), (1, 2, 4, 1, 0), (1, 2, 4, 0, 1), (1, 0, 4, 1, 1), (1, 2, 0, 1, 1),
    (1, 2, 0, 0, 1), (2, 2, 4, 1, 1), (2, 2, 4, 1, 0), (2, 2, 4, 0, 1), (2, 0, 0, 1, 1),
    (3, 2, 4, 1, 1), (4, 4, 4, 1, 1), (4, 4, 0, 1, 1), (4, 0, 4, 1, 1), (5, 2, 4, 1, 1),
    (8, 2, 4, 1, 1)])
def test_batched_step_paths(model, W, R, B, gemv, sparse, fuse, fval):
    """B independent rows through the GEMV / MFMA, sparse / dense, fused /
    separate LayerNorm and fused / separate sparse value paths."""
    model.set_option(R.OPT_GEMV_MAX_B, gemv)
    model.set_option(R.OPT_SPARSE_MAX_B, sparse)
    model.set_option(R.OPT_FUSE_LN, fuse)
    model.set_option(R.OPT_FUSE_VALUE, fval)
    try:
        slots = [(5 * i + 3) % NSLOT for i in range(B)]
        fresh(model, slots)
        states = []
        for i, s in enumerate(slots):
            pr = prompt(100 + i, 3 + i)
            model.prefill(s, dev(pr))
            st = O.State(S)
            O.seq(W, st, pr, want_logits=False)
            states.append(st)
        logits = torch.empty(B, S.vocab, device="cuda")
        for step in range(3):
            toks = [int(t) for t in prompt(200 + step, B)]
            model.decode_step(dev(slots), dev(toks), logits)
            ref = O.step(W, states, toks)
            got = logits.cpu().numpy()
            for b in range(B):
                assert rel(got[b], ref[b]) <= TOL, (step, b)
        for b, s in enumerate(slots):
            assert rel(gstate(model, s), states[b].flat()) <= TOL
        assert model.poll_error() == 0
    finally:
        model.set_option(R.OPT_GEMV_MAX_B, 2)
        model.set_option(R.OPT_SPARSE_MAX_B, 4)
        model.set_option(R.OPT_FUSE_LN, 1)
        model.set_option(R.OPT_FUSE_VALUE, 1)


def test_wkv_adapter_paths(weights, W, R):
    """The adapters' second stage on the MFMA decode path, computed by the WKV
    kernel (1, 2 or 4 rows per wave: blocks of 4, 8 or 16 rows of a head, the
    16-row matrix-core tile padded) or by a separate MFMA projection: every
    variant against the oracle, and the in-kernel ones against the separate
    projection (the same fp16 products, summed in another order).  Row
    counts 3, 8 and 21 give partial, whole and ragged blocks; the slots are
    a permutation so rows and slots differ."""
    n = 24
    m = R.Model.from_numpy(S, weights, n_slots=n, max_B=n, max_T=16)
    try:
        for B in (3, 8, 21):
            slots = [(7 * i + 5) % n for i in range(B)]
            prompts = [prompt(300 + i, 2 + i % 5) for i in range(B)]
            feeds = [[int(t) for t in prompt(400 + st, B)] for st in range(3)]
            refs = []
            states = [O.State(S) for _ in range(B)]
            for st_, pr in zip(states, prompts):
                O.seq(W, st_, pr, want_logits=False)
            for toks in feeds:
                refs.append(O.step(W, states, toks))
            runs = {}
            for opt in (1, 2, 3, 4, 0):
                m.set_option(R.OPT_WKV_ADAPTERS, opt)
                m.reset(dev(slots))
                for s_, pr in zip(slots, prompts):
                    m.prefill(s_, dev(pr))
                out = torch.empty(3, B, S.vocab, device="cuda")
                for t, toks in enumerate(feeds):
                    m.decode_step(dev(slots), dev(toks), out[t])
                got = out.cpu().numpy()
                runs[opt] = (got, np.stack([gstate(m, s_) for s_ in slots]))
                assert m.poll_error() == 0
                for t in range(3):
                    for b in range(B):
                        assert rel(got[t, b], refs[t][b]) <= TOL, (B, opt, t, b)
                for b in range(B):
                    assert rel(runs[opt][1][b], states[b].flat()) <= TOL, (B, opt, b)
            for opt in (2, 3, 4, 0):
                assert rel(runs[opt][0], runs[1][0]) <= 1e-4, (B, opt)
                assert rel(runs[opt][1], runs[1][1]) <= 1e-4, (B, opt)
        # the kernel-name query follows the option (rows per wave as the last argument)
        for opt, name in ((0, "k_wkv_decode_ad<32, 32, 32, 64, 1>"), (2, "k_wkv_decode_ad<32, 32, 32, 64, 1>"),
                          (3, "k_wkv_decode_ad<32, 32, 32, 64, 2>"), (4, "k_wkv_decode_ad<32, 32, 32, 64, 4>"),
                          (1, "k_wkv_decode_rows<")):
            m.set_option(R.OPT_WKV_ADAPTERS, opt)
            assert R.rwkv7_kernel_name(m.handle, R.K_WKV, 8).startswith(name), (opt, name)
        assert R.rwkv7_kernel_name(m.handle, R.K_WKV, 1).startswith("k_wkv_decode<")
        with pytest.raises(R.RWKV7Error):
            m.set_option(R.OPT_WKV_ADAPTERS, 5)
    finally:
        m.close()


GEMM_PLAN_KEYS = (8, 9, 10, 11, 12, 13)   # OPT_GEMM_PLAN_PROJ_IN .. _HEAD


@pytest.mark.parametrize("tm,tn,ks,pipe,split", [
    (1, 2, 128, 0, 0), (2, 2, 32, 1, 0), (2, 4, 64, 1, 1), (4, 4, 64, 0, 3),
    (2, 2, 64, 2, 0), (2, 2, 128, 2, 0), (1, 2, 64, 2, 0), (2, 4, 32, 2, 2),
    (4, 2, 64, 2, 1), (1, 4, 64, 2, 3),
    (2, 2, 64, 3, 0), (4, 4, 64, 3, 0), (1, 2, 128, 3, 0), (2, 4, 32, 3, 2),
    (4, 2, 64, 3, 1), (1, 4, 64, 3, 3), (2, 2, 128, 3, 0), (2, 5, 64, 3, 0), (2, 5, 64, 3, 2),
    (2, 2, 64, 4, 0), (4, 4, 64, 4, 0), (2, 4, 64, 4, 2), (4, 2, 64, 4, 1), (2, 2, 32, 4, 0),
    (4, 4, 32, 4, 3), (2, 2, 128, 4, 0), (4, 8, 64, 4, 0), (2, 8, 64, 4, 2), (8, 8, 32, 4, 3), (8, 8, 32, 4, 0),
    (8, 10, 32, 4, 0), (8, 10, 32, 4, 2), (4, 1, 64, 3, 0), (4, 1, 128, 3, 3), (4, 5, 64, 3, 0), (4, 5, 64, 3, 4),
    (4, 4, 32, 3, 2),
    (1, 2, 128, 5, 0), (2, 2, 64, 5, 0), (2, 2, 64, 5, 3), (2, 4, 64, 5, 0), (4, 4, 64, 5, 0),
    (4, 2, 64, 5, 2), (1, 4, 64, 6, 2), (1, 2, 128, 6, 0), (4, 2, 64, 6, 1), (2, 2, 64, 6, 2)])
def test_gemm_plans_match_oracle(model, W, R, tm, tn, ks, pipe, split):
    """Every MFMA projection (prefill and an 8-row step) forced onto one tile
    plan: tile shapes, stage depths, the seven K loops and K splits, with K
    from 32 (adapter ranks) to 1024 (channel-mix value) and ragged row
    counts, against the oracle and against the built-in plans."""
    code = R.gemm_plan_code(tm, tn, ks, pipe, split)
    B = 8
    slots = [(3 * i + 1) % NSLOT for i in range(B)]
    toks = [[int(t) for t in prompt(400 + step, B)] for step in range(2)]

    def run():
        fresh(model, slots)
        for i, s in enumerate(slots):
            model.prefill(s, dev(prompt(300 + i, 5 + 3 * i)))
        out = []
        logits = torch.empty(B, S.vocab, device="cuda")
        for t in toks:
            model.decode_step(dev(slots), dev(t), logits)
            out.append(logits.cpu().numpy().copy())
        return out, [gstate(model, s) for s in slots]

    base, base_states = run()
    for k in GEMM_PLAN_KEYS:
        model.set_option(k, code)
    try:
        got, got_states = run()
    finally:
        for k in GEMM_PLAN_KEYS:
            model.set_option(k, 0)
    states = []
    for i in range(B):
        st = O.State(S)
        O.seq(W, st, prompt(300 + i, 5 + 3 * i), want_logits=False)
        states.append(st)
    # Plans differ in fp32 summation order; the fp16 activations written
    # between projections can then round one ulp (2^-11 relative) apart, so
    # the plans agree to about 1e-3, not bitwise.  A wrong tile is O(1) off.
    for step, t in enumerate(toks):
        ref = O.step(W, states, t)
        for b in range(B):
            assert rel(got[step][b], ref[b]) <= TOL, (step, b)
            assert rel(got[step][b], base[step][b]) <= 2e-3, (step, b)
    for b in range(B):
        assert rel(got_states[b], states[b].flat()) <= TOL
        assert rel(got_states[b], base_states[b]) <= 2e-3
    assert model.poll_error() == 0


def test_gemm_plan_option_validation(model, R):
    for bad in (R.gemm_plan_code(3, 2, 64), R.gemm_plan_code(2, 2, 48), R.gemm_plan_code(4, 4, 64, 2),
                R.gemm_plan_code(4, 4, 128), R.gemm_plan_code(1, 4, 64, 4), R.gemm_plan_code(2, 4, 128, 3),
                R.gemm_plan_code(1, 2, 32, 3), R.gemm_plan_code(2, 5, 32, 3), R.gemm_plan_code(2, 5, 64, 2),
                R.gemm_plan_code(4, 5, 128, 3), R.gemm_plan_code(4, 5, 32, 3), R.gemm_plan_code(1, 2, 64, 4), R.gemm_plan_code(2, 4, 32, 4),
                R.gemm_plan_code(2, 4, 128, 4), R.gemm_plan_code(2, 2, 64, 7), R.gemm_plan_code(4, 8, 64, 3),
                R.gemm_plan_code(4, 4, 128, 5), R.gemm_plan_code(2, 2, 32, 5), R.gemm_plan_code(2, 2, 128, 6),
                R.gemm_plan_code(2, 5, 64, 5),
                R.gemm_plan_code(4, 8, 128, 4), R.gemm_plan_code(1, 8, 64, 4), R.gemm_plan_code(8, 8, 64, 4),
                R.gemm_plan_code(8, 8, 32, 3), R.gemm_plan_code(8, 4, 32, 4), R.gemm_plan_code(8, 10, 64, 4),
                R.gemm_plan_code(8, 10, 32, 3), R.gemm_plan_code(9, 0, 64, 4), R.gemm_plan_code(4, 1, 32, 3),
                R.gemm_plan_code(2, 1, 64, 3), R.gemm_plan_code(4, 1, 64, 4), -5, 10 ** 8):
        with pytest.raises(R.RWKV7Error):
            model.set_option(8, bad)
    model.set_option(8, 0)


def test_prefill_equals_steps_on_gpu(model, R):
    toks = prompt(7, 37)
    fresh(model, [2, 3, 4])
    model.prefill(2, dev(toks))
    logits = torch.empty(1, S.vocab, device="cuda")
    for t in toks:
        model.decode_step(dev([3]), dev([int(t)]), logits)
    # 3 chunks: 16 + 16 + 5, with the same (chunked) WKV scan as the one 37-token chunk
    model.set_option(R.OPT_PREFILL_CHUNK, 16)
    model.set_option(R.OPT_PREFILL_SCAN, 2)
    try:
        model.prefill(4, dev(toks))
    finally:
        model.set_option(R.OPT_PREFILL_CHUNK, 2048)
        model.set_option(R.OPT_PREFILL_SCAN, 0)
    a, b, c = gstate(model, 2), gstate(model, 3), gstate(model, 4)
    assert rel(a, b) <= TOL
    # 37 rows and 16 rows take different GEMM tile plans (K split 6 against none),
    # so the fp32 sums run in another order and the fp16 activations between the
    # projections can round an ulp (2^-11) apart: ~3e-5, not the bitwise agreement
    # of one plan
    assert rel(c, a) <= 1e-4
    cnt = model.counters().cpu().numpy()
    assert cnt[2] == cnt[3] == cnt[4] == 37


@pytest.mark.parametrize("T", [1, 5, 16, 37, 100])
def test_prefill_scan_forms_agree(model, W, R, T):
    """The serial WKV scan and the chunked one (16-token blocks in closed form,
    ragged last block) land on the same state, and both on the oracle's."""
    toks = prompt(20 + T, T)
    fresh(model, [7, 8])
    try:
        model.set_option(R.OPT_PREFILL_SCAN, 1)
        model.prefill(7, dev(toks))
        model.set_option(R.OPT_PREFILL_SCAN, 2)
        model.prefill(8, dev(toks))
    finally:
        model.set_option(R.OPT_PREFILL_SCAN, 0)
    a, b = gstate(model, 7), gstate(model, 8)
    st = O.State(S)
    O.seq(W, st, toks, want_logits=False)
    print(f"T={T}: chunked vs serial {rel(b, a):.3e}, chunked vs oracle {rel(b, st.flat()):.3e}")
    # the two scans round differently (~1e-7); downstream that can flip an fp16
    # activation rounding (relative step 4.9e-4) in the next layer's projections
    assert rel(b, a) <= 1e-3
    assert rel(b, st.flat()) <= TOL
    assert rel(a, st.flat()) <= TOL


def test_prefill_scan_option_validation(model, R):
    for bad in (-1, 3):
        with pytest.raises(R.RWKV7Error):
            model.set_option(R.OPT_PREFILL_SCAN, bad)
    assert R.rwkv7_get_option(model.handle, R.OPT_PREFILL_SCAN) == 0


@pytest.mark.parametrize("C", [1024, 3072])
def test_ln_split_bit_identical(R, C):
    """The batched LayerNorm kernel's column blocks (OPT_LN_SPLIT) change who
    computes which columns, never the arithmetic: logits and states are
    bit-identical for every split, and match the oracle.  C 1024 has two
    512-column pairs, C 3072 six (splits 4 and 5 deal them unevenly)."""
    import dataclasses
    sh = dataclasses.replace(S, name=f"tiny-c{C}", n_embd=C, n_head=C // 64, ffn=4 * C)
    wts = synth.make_weights(sh, bkey=synth.bkey_table(S))   # the tiny shape's key bias
    B, steps = 8, 3
    m = R.Model.from_numpy(sh, wts, n_slots=B, max_B=B, max_T=16)
    prompts = [np.random.default_rng(40 + b).integers(0, sh.vocab, 5).astype(np.int32) for b in range(B)]
    feeds = np.random.default_rng(50).integers(0, sh.vocab, (steps, B)).astype(np.int32)
    slots = dev(list(range(B)))
    runs = {}
    units = C // 512 if (C // 256) % 2 == 0 else C // 256
    for split in [1] + list(range(2, units + 1)) + [0]:
        m.set_option(R.OPT_LN_SPLIT, split)
        m.reset(slots)
        for b in range(B):
            m.prefill(b, dev(prompts[b]))
        out = torch.empty(steps, B, sh.vocab, device="cuda")
        for t in range(steps):
            m.decode_step(slots, dev(feeds[t]), out[t])
        torch.cuda.synchronize()
        runs[split] = (out.cpu().numpy(), np.stack([m.slot_state(b).cpu().numpy() for b in range(B)]))
        assert m.poll_error() == 0
    for split, (lg, stt) in runs.items():
        assert np.array_equal(lg, runs[1][0]), split
        assert np.array_equal(stt, runs[1][1]), split
    with pytest.raises(R.RWKV7Error):
        m.set_option(R.OPT_LN_SPLIT, 17)
    Wo = O.Weights(sh, wts)
    for b in (0, B - 1):
        st = O.State(sh)
        O.seq(Wo, st, prompts[b], want_logits=False)
        ref = O.seq(Wo, st, feeds[:, b], want_logits=True)
        assert rel(runs[1][0][:, b], ref) <= TOL
        assert rel(runs[1][1][b], st.flat()) <= TOL
    m.close()


def test_read_bandwidth_reads_only(R):
    """rwkv7_read_bandwidth streams a buffer and leaves it as it was; a size that
    is not a multiple of 16 bytes reads the whole 16-byte chunks only."""
    buf = torch.arange(1 << 20, dtype=torch.float32, device="cuda")
    ref = buf.clone()
    for nt in (True, False):
        gbs = R.rwkv7_read_bandwidth(buf, nontemporal=nt, iters=3)
        assert gbs > 0
    tail = buf.view(torch.uint8)[: (1 << 22) - 8]
    assert R.rwkv7_read_bandwidth(tail, iters=1) > 0
    torch.cuda.synchronize()
    assert torch.equal(buf, ref)


def test_prefill_matches_oracle(model, W):
    toks = prompt(8, 50)
    fresh(model, [5])
    model.prefill(5, dev(toks))
    st = O.State(S)
    O.seq(W, st, toks, want_logits=False)
    assert rel(gstate(model, 5), st.flat()) <= TOL


def test_zero_length_prefill_is_noop(model):
    fresh(model, [6])
    before = model.slot_state(6).clone()
    model.prefill(6, torch.zeros(0, dtype=torch.int32, device="cuda"))
    assert torch.equal(before, model.slot_state(6))


def test_pure_decay_closed_form_on_gpu(weights, R):
    """Zero decay adapters, w0 = 0, zero key/value weights: every decay is
    exp(-e^-1/2 / 2) = 0.7384031 and k = v = 0, so S_T = 0.7384031^T S_0."""
    w = dict(weights)
    for l in range(S.n_layer):
        p = f"blocks.{l}."
        for n in ("att.w0", "att.w1", "att.w2", "att.key.weight", "att.value.weight"):
            w[p + n] = np.zeros_like(w[p + n])
    m = R.Model.from_numpy(S, w, n_slots=2, max_B=1, max_T=8)
    try:
        view = m.slot_state(0)
        g = torch.Generator(device="cpu").manual_seed(3)
        C = S.n_embd
        init = torch.randn(view.shape, generator=g)
        init[:, :2 * C] = 0.0
        view.copy_(init.cuda())
        S0 = view[:, 2 * C:].double().cpu().numpy()
        T = 5
        logits = torch.empty(1, S.vocab, device="cuda")
        for t in range(T):
            m.decode_step(dev([0]), dev([t + 11]), logits)
        ST = gstate(m, 0)[:, 2 * C:]
        assert rel(ST, S0 * 0.7384031 ** T) <= 1e-5
    finally:
        m.close()


def test_unlisted_slots_bit_identical_and_counters(model):
    g = torch.Generator(device="cpu").manual_seed(5)
    n = model.counter_offset // 4
    fpool = model.pool[: model.counter_offset].view(torch.float32)
    fpool.copy_(torch.randn(n, generator=g).cuda() * 0.1)
    cnt = model.counters()
    cnt.copy_(torch.arange(NSLOT, dtype=torch.int64, device="cuda") * 10)
    before = model.pool.clone()
    logits = torch.empty(2, S.vocab, device="cuda")
    model.decode_step(dev([5, 2]), dev([7, 9]), logits)
    torch.cuda.synchronize()
    after = model.pool
    sf = model.slot_floats * 4
    for s in range(NSLOT):
        same = torch.equal(before[s * sf:(s + 1) * sf], after[s * sf:(s + 1) * sf])
        assert same == (s not in (2, 5)), s
    c = model.counters().cpu().numpy()
    exp = np.arange(NSLOT) * 10
    exp[2] += 1
    exp[5] += 1
    np.testing.assert_array_equal(c, exp)


def test_device_error_flags(model, R):
    logits = torch.empty(2, S.vocab, device="cuda")
    model.poll_error()
    model.decode_step(dev([1]), dev([S.vocab + 5]), logits[:1])
    assert model.poll_error() == R.ERR_TOKEN_RANGE
    model.decode_step(dev([1, 1]), dev([3, 4]), logits)
    assert model.poll_error() == R.ERR_SLOT_DUP
    model.decode_step(dev([1, NSLOT + 3]), dev([3, 4]), logits)
    assert model.poll_error() == R.ERR_SLOT_RANGE
    assert model.poll_error() == 0


def test_selection_slot_errors(model, R):
    """rwkv7_greedy and rwkv7_sample with a slot listed twice or outside the
    pool: the error bit is set, the first row of a repeated slot keeps its
    occurrence update, the later row and the out-of-range row touch none, and
    their picks are the plain argmax of their logits."""
    V = S.vocab
    g = torch.Generator().manual_seed(3)
    logits = torch.randn(3, V, generator=g).cuda()
    occ0 = torch.rand(NSLOT, V, generator=g).cuda() * (torch.rand(NSLOT, V, generator=g).cuda() < 0.1)
    ones = torch.ones(3, device="cuda")
    dec = torch.full((3,), 0.5, device="cuda")
    ids = torch.zeros(3, dtype=torch.int32, device="cuda")
    sws = torch.zeros(R.rwkv7_sample_workspace_bytes(3, V), dtype=torch.uint8, device="cuda")
    plain = logits.argmax(1).cpu().numpy()
    for use_sample in (False, True):
        for slots, bit in (([2, 5, 2], R.ERR_SLOT_DUP), ([2, 5, NSLOT + 1], R.ERR_SLOT_RANGE)):
            occ = occ0.clone()
            if use_sample:
                R.rwkv7_sample(logits, occ, NSLOT, dev(slots), ones, ones, dec, torch.zeros(3, device="cuda"),
                               ones, torch.zeros(3, dtype=torch.int32, device="cuda"), None,
                               torch.full((3,), 0.5, device="cuda"), ids, sws)
                flags = R.rwkv7_poll_error(sws)
            else:
                R.rwkv7_greedy(logits, occ, NSLOT, dev(slots), ones, ones, dec, ids, model.ws)
                flags = model.poll_error()
            assert flags == bit, (use_sample, slots, flags)
            got = ids.cpu().numpy()
            assert got[2] == plain[2]                       # unpenalised pick on the flagged row
            o = occ.cpu().numpy()
            o0 = occ0.cpu().numpy()
            untouched = [s for s in range(NSLOT) if s not in (2, 5)]
            assert np.array_equal(o[untouched], o0[untouched])
            for b, s in ((0, 2), (1, 5)):                   # the rows that own their slots
                want = (o0[s] * np.float32(0.5)).astype(np.float32)
                want[got[b]] += np.float32(1.0)
                assert np.array_equal(o[s], want), (use_sample, slots, b)


def test_host_errors_with_model(model, R):
    logits = torch.empty(1, S.vocab, device="cuda")
    with pytest.raises(R.RWKV7Error):
        R.rwkv7_decode_step(model.handle, model.pool, NSLOT, dev([]), dev([]), logits, model.ws)
    with pytest.raises(R.RWKV7Error):   # workspace too small for B = 9 > max_B
        R.rwkv7_decode_step(model.handle, model.pool, NSLOT, dev(list(range(9))), dev([1] * 9),
                            torch.empty(9, S.vocab, device="cuda"), model.ws[:4096])
    with pytest.raises(R.RWKV7Error):
        R.rwkv7_prefill_seq(model.handle, model.pool, NSLOT, NSLOT, dev([1, 2]), model.ws)


def test_graph_matches_eager_bitwise(model, R):
    fresh(model, [7])
    model.prefill(7, dev(prompt(9, 5)))
    torch.cuda.synchronize()
    snap = model.slot_state(7).clone()
    toks = [int(t) for t in prompt(10, 4)]
    outs = []
    for graph in (1, 0, 1):
        model.slot_state(7).copy_(snap)
        model.set_option(R.OPT_USE_GRAPH, graph)
        seq = []
        logits = torch.empty(1, S.vocab, device="cuda")
        for t in toks:
            model.decode_step(dev([7]), dev([t]), logits)
            seq.append(logits.clone())
        outs.append((torch.stack(seq), model.slot_state(7).clone()))
    model.set_option(R.OPT_USE_GRAPH, 1)
    for o in outs[1:]:
        assert torch.equal(o[0], outs[0][0])
        assert torch.equal(o[1], outs[0][1])


def test_greedy_bit_exact_vs_float32_replica(model):
    rng = np.random.default_rng(11)
    B, V = 6, S.vocab
    slots = [3, 0, 9, 4, 12, 1]
    L = (rng.integers(-4, 5, size=(B, V)) * 0.25).astype(np.float32)
    L[2] = np.nan
    L[4, rng.integers(0, V, 50)] = np.nan
    L[5] = rng.standard_normal(V).astype(np.float32)
    occ = np.zeros((NSLOT, V), np.float32)
    occ[:, rng.integers(0, V, 300)] = rng.random((NSLOT, 300)).astype(np.float32) * 3
    pres = np.array([1.0, 0.0, 0.5, 1.0, 0.25, 1.0], np.float32)
    freq = np.array([1.0, 0.5, 0.0, 1.0, 2.0, 1.0], np.float32)
    dec = np.array([0.996, 1.0, 0.9, 0.996, 0.5, 0.996], np.float32)
    occ_d = torch.from_numpy(occ).cuda()
    ids = torch.zeros(B, dtype=torch.int32, device="cuda")
    model.poll_error()
    model.greedy(torch.from_numpy(L).cuda(), occ_d, dev(slots), torch.from_numpy(pres).cuda(),
                 torch.from_numpy(freq).cuda(), torch.from_numpy(dec).cuda(), ids)
    flags = model.poll_error()
    rid, rocc, rerr = O.greedy_penalized(L, occ[slots], pres, freq, dec)
    np.testing.assert_array_equal(ids.cpu().numpy(), rid)
    got = occ_d.cpu().numpy()
    for b, s in enumerate(slots):
        assert np.array_equal(got[s].view(np.uint32), rocc[b].view(np.uint32)), b
    untouched = [s for s in range(NSLOT) if s not in slots]
    np.testing.assert_array_equal(got[untouched], occ[untouched])
    assert rerr[2] and flags == 8


def test_sparse_active_set_exact(model, W, R):
    """The skipped value rows are exactly those with pre-activation <= 0
    (against the GPU's own pre-activations), and match the oracle's set
    wherever the oracle's pre-activation is not within 1e-3 rms of zero."""
    B = 2
    slots = [10, 11]
    fresh(model, slots)
    states = [O.State(S), O.State(S)]
    for i, s in enumerate(slots):
        pr = prompt(300 + i, 6)
        model.prefill(s, dev(pr))
        O.seq(W, states[i], pr, want_logits=False)
    toks = [5, 77]
    logits = torch.empty(B, S.vocab, device="cuda")
    model.decode_step(dev(slots), dev(toks), logits)
    torch.cuda.synchronize()
    p_pre, p_mask, p_act, p_cnt = R.rwkv7_debug_cmix_buffers(model.handle, model.ws, B)
    base = model.ws.data_ptr()
    F = S.ffn

    def view(addr, n, dt):
        off = addr - base
        return model.ws[off: off + n * torch.tensor([], dtype=dt).element_size()].view(dt)

    pre = view(p_pre, B * F, torch.float32).cpu().numpy().reshape(B, F)
    mask = view(p_mask, F, torch.uint8).cpu().numpy()
    cnt = int(view(p_cnt, 1, torch.int32).item())
    act = view(p_act, F, torch.int32).cpu().numpy()[:cnt]
    exp_mask = (pre > 0).any(axis=0)
    np.testing.assert_array_equal(mask.astype(bool), exp_mask)
    np.testing.assert_array_equal(act, np.nonzero(exp_mask)[0])
    # against the oracle's last-layer pre-activations
    zs = []
    orig = O.cmix_key

    def spy(W_, l, u, prev):
        z = orig(W_, l, u, prev)
        zs.append(z + W_.L(l, "ffn.key.bias"))
        return z
    O.cmix_key = spy
    try:
        O.step(W, states, toks)
    finally:
        O.cmix_key = orig
    zref = zs[-1]
    assert rel(pre, zref) <= TOL
    rms = np.sqrt(np.mean(zref ** 2))
    clear = np.abs(zref) >= 1e-3 * rms
    assert np.array_equal((pre > 0)[clear], (zref > 0)[clear])
    assert 0.6 < 1 - (pre > 0).mean() < 0.97   # ~85 % zeros


def test_time_kernel_after_greedy(model, R):
    """rwkv7_greedy shares the decode workspace; rwkv7_time_kernel after it
    must rebuild the rows it reads (regression: greedy partials once
    overwrote the sanitized slot list at the head of the workspace)."""
    slots = dev([4, 9])
    toks = dev([3, 8])
    fresh(model, [4, 9])
    logits = torch.empty(2, S.vocab, device="cuda")
    occ = torch.zeros(NSLOT, S.vocab, device="cuda")
    z = torch.zeros(2, device="cuda")
    one = torch.ones(2, device="cuda")
    ids = torch.zeros(2, dtype=torch.int32, device="cuda")
    model.decode_step(slots, toks, logits)
    model.greedy(logits, occ, slots, z, z, one, ids)
    for cls in range(8):
        for layer in (0, S.n_layer):
            ms = R.rwkv7_time_kernel(model.handle, model.pool, NSLOT, slots, toks, logits, cls,
                                     layer, 3, model.ws)
            assert ms >= 0.0
    assert model.poll_error() == 0
    fresh(model, [4, 9])


def test_kernel_timing_counts(model, R):
    model.set_option(R.OPT_KERNEL_TIMING, 1)
    try:
        R.rwkv7_kernel_timing(model.handle, 0, reset=True)
        logits = torch.empty(1, S.vocab, device="cuda")
        model.decode_step(dev([0]), dev([1]), logits)
        counts = {R.K_NAMES[k]: R.rwkv7_kernel_timing(model.handle, k)[1] for k in range(8)}
        Lr = S.n_layer
        assert counts["ln_mix"] == 0          # fused into the GEMV prologues at B = 1
        assert counts["other"] == 1           # validation + embedding, one launch
        assert counts["proj_in"] == counts["wkv"] == counts["proj_out"] == Lr
        assert counts["cmix_key"] == counts["cmix_value"] == Lr
        assert counts["head"] == 1
        ms = R.rwkv7_kernel_timing(model.handle, R.K_HEAD)[0]
        assert ms > 0
    finally:
        model.set_option(R.OPT_KERNEL_TIMING, 0)
