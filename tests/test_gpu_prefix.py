"""Slot snapshots, slot offload and the prefix-state cache (include/rwkv7_prefix.h)
on the tiny model.

A snapshot is a copy, so everything restored is compared bit for bit with
the slot it came from.  A slot restored from a cached prefix and then
prefilled with the rest of a prompt is compared with the oracle's state after
the whole prompt (the state is a function of the tokens alone), within the
state tolerance.  The scheduler's GPU backend with a cache attached is checked
as in test_gpu_sched: its streams are replayed through the oracle."""
import numpy as np
import pytest
import torch

import synth
from oracle import rwkv7 as O
from test_gpu_sched import replay

pytestmark = pytest.mark.gpu

S = synth.TINY
V = S.vocab
NS = 8


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
    m = R.Model.from_numpy(S, weights, n_slots=NS, max_B=6, max_T=64)
    yield m
    m.close()


def toks(seed, n):
    return np.random.default_rng(seed).integers(0, V, n).astype(np.int32)


def dev(x):
    return torch.as_tensor(np.asarray(x, np.int32), device="cuda")


def snap(m, slot):
    torch.cuda.synchronize()
    return m.slot_state(slot).cpu().numpy().copy(), int(m.counters()[slot].item())


def oracle_state(W, t):
    st = O.State(S)
    O.seq(W, st, t.tolist(), want_logits=False)
    return st


def gpu_vs_oracle(m, slot, st):
    """Relative L2 of the slot (shifts and WKV state) against the oracle's state."""
    g = m.slot_state(slot).cpu().double().numpy()
    ref = st.flat()
    return float(np.linalg.norm(g - ref) / np.linalg.norm(ref))


def test_snapshot_bytes(R):
    cfg = R.make_config(S)
    assert R.rwkv7_snapshot_bytes(cfg) == R.rwkv7_slot_floats(cfg) * 4 + 8


def test_export_import_round_trip(model, R):
    m = model
    m.reset(dev(range(NS)))
    m.prefill(0, dev(toks(1, 20)))
    nb = R.rwkv7_snapshot_bytes(m.cfg)
    d = torch.empty(nb, dtype=torch.uint8, device="cuda")
    h = torch.empty(nb, dtype=torch.uint8).pin_memory()
    R.rwkv7_slot_export(m.handle, m.pool, NS, 0, d)
    R.rwkv7_slot_export(m.handle, m.pool, NS, 0, h)
    torch.cuda.synchronize()
    assert torch.equal(d.cpu(), h)
    R.rwkv7_slot_import(m.handle, m.pool, NS, 2, d)
    R.rwkv7_slot_import(m.handle, m.pool, NS, 3, h)
    s0, c0 = snap(m, 0)
    for sl in (2, 3):
        s, c = snap(m, sl)
        assert np.array_equal(s, s0) and c == c0 == 20
    # a restored slot continues exactly as the original (two rows of one step)
    logits = torch.empty(2, V, device="cuda")
    m.decode_step(dev([0, 2]), dev([5, 5]), logits)
    lg = logits.cpu().numpy()
    assert np.array_equal(lg[0], lg[1])
    assert np.array_equal(snap(m, 0)[0], snap(m, 2)[0])
    with pytest.raises(R.RWKV7Error):
        R.rwkv7_slot_export(m.handle, m.pool, NS, NS, d)


def test_prefix_restore_then_rest_matches_oracle(model, W, R):
    m = model
    m.reset(dev(range(NS)))
    t = toks(2, 50)
    arena = torch.empty(2 * R.rwkv7_snapshot_bytes(m.cfg) + 512, dtype=torch.uint8, device="cuda")
    c = R.rwkv7_prefix_cache_create(m.handle, arena)
    m.prefill(0, dev(t[:30]))
    R.rwkv7_prefix_cache_store(c, m.pool, NS, 0, t[:30])
    assert R.rwkv7_prefix_cache_lookup(c, m.pool, NS, 1, t[:49]) == 30
    s0, c0 = snap(m, 0)
    s1, c1 = snap(m, 1)
    assert np.array_equal(s0, s1) and c0 == c1 == 30
    m.prefill(1, dev(t[30:49]))
    m.prefill(2, dev(t[:49]))
    torch.cuda.synchronize()
    ref = oracle_state(W, t[:49])
    e1 = gpu_vs_oracle(m, 1, ref)
    e2 = gpu_vs_oracle(m, 2, ref)
    print(f"state vs oracle: restored + rest {e1:.2e}, whole prompt {e2:.2e}")
    assert e1 <= 1e-2 and e2 <= 1e-2
    g1, g2 = m.slot_state(1).cpu().double().numpy(), m.slot_state(2).cpu().double().numpy()
    assert np.linalg.norm(g1 - g2) / np.linalg.norm(g2) <= 1e-3
    assert int(m.counters()[1].item()) == 49
    # no match: the slot is untouched; a shorter stored prefix is not longer than asked
    assert R.rwkv7_prefix_cache_lookup(c, m.pool, NS, 3, toks(3, 40)) == 0
    assert R.rwkv7_prefix_cache_lookup(c, m.pool, NS, 3, t[:29]) == 0
    assert R.rwkv7_prefix_cache_lookup(c, m.pool, NS, 3, []) == 0
    st = R.rwkv7_prefix_cache_stats(c)
    assert (st.lookups, st.hits, st.hit_tokens, st.stores) == (4, 1, 30, 1)
    R.rwkv7_prefix_cache_free(c)


def test_lru_offload_and_drop(model, R):
    m = model
    m.reset(dev(range(NS)))
    nb = R.rwkv7_snapshot_bytes(m.cfg)
    stride = (nb + 255) // 256 * 256
    arena = torch.empty(2 * stride, dtype=torch.uint8, device="cuda")
    host = torch.empty(stride, dtype=torch.uint8).pin_memory()
    c = R.rwkv7_prefix_cache_create(m.handle, arena, host)
    seqs = [toks(10 + i, 12 + 3 * i) for i in range(4)]
    for i, t in enumerate(seqs):
        m.prefill(i, dev(t))
    orig = [snap(m, i) for i in range(4)]
    for i in range(3):
        R.rwkv7_prefix_cache_store(c, m.pool, NS, i, seqs[i])
    st = R.rwkv7_prefix_cache_stats(c)
    assert (st.device_entries, st.host_entries, st.offloads, st.drops) == (2, 1, 1, 0)
    R.rwkv7_prefix_cache_store(c, m.pool, NS, 1, seqs[1])      # already cached: only marked used
    R.rwkv7_prefix_cache_store(c, m.pool, NS, 3, seqs[3])      # offloads the LRU (seq 2), drops seq 0
    st = R.rwkv7_prefix_cache_stats(c)
    assert (st.stores, st.offloads, st.drops, st.device_entries, st.host_entries) == (4, 2, 1, 2, 1)
    assert R.rwkv7_prefix_cache_lookup(c, m.pool, NS, 5, seqs[0]) == 0
    for i in (1, 2, 3):
        ext = np.concatenate([seqs[i], toks(99, 7)])
        assert R.rwkv7_prefix_cache_lookup(c, m.pool, NS, 5, ext) == len(seqs[i])
        s, cnt = snap(m, 5)
        assert np.array_equal(s, orig[i][0]) and cnt == orig[i][1] == len(seqs[i])
    R.rwkv7_prefix_cache_free(c)
    small = torch.empty(stride - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(R.RWKV7Error):
        R.rwkv7_prefix_cache_create(m.handle, small)


def test_scheduler_backend_reuses_prefixes(weights, W, R):
    n_slots, max_b = 4, 4
    m = R.Model.from_numpy(S, weights, n_slots=n_slots, max_B=max_b, max_T=64)
    occ = torch.zeros(n_slots * V, device="cuda")
    sws = torch.zeros(R.rwkv7_sample_workspace_bytes(max_b, V), dtype=torch.uint8, device="cuda")
    arena = torch.empty(8 * R.rwkv7_snapshot_bytes(m.cfg) + 2048, dtype=torch.uint8, device="cuda")
    cache = R.rwkv7_prefix_cache_create(m.handle, arena)
    be = R.rwkv7_sched_gpu_backend(m.handle, m.pool, n_slots, occ, None, max_b, m.ws, sws, m.max_T)
    R.rwkv7_sched_gpu_backend_set_cache(be, cache)
    s = R.rwkv7_sched_create(R.SchedConfig(max_b, 1, 0, 10, V), be)
    p1 = toks(40, 30).tolist()
    p2 = p1 + toks(41, 25).tolist()          # the next turn: extends p1
    prompts = [p1, p2, list(p1), p2 + toks(42, 12).tolist()]
    tasks = {}
    for i, p in enumerate(prompts):
        prm = R.SchedParams(1.0 if i % 2 else 0.0, 0.5, 0, 0.3, 0.3, 0.996, 8, -1, 555 + i)
        tasks[R.rwkv7_sched_submit(s, p, prm)] = (p, prm)
    events = []
    for _ in range(300):
        R.rwkv7_sched_step(s)
        events += R.rwkv7_sched_poll(s)
        if all(R.rwkv7_sched_task_state(s, t) == R.TASK_FINISHED for t in tasks):
            break
    streams = {}
    for task, kind, value, index in events:
        if kind == R.EV_TOKEN:
            streams.setdefault(task, []).append(value)
    restored, prefilled = R.rwkv7_sched_gpu_backend_counts(be)
    # p1: 29 computed; p2: 29 restored + 25; p1 again: 29 restored; p3: 54 restored + 12
    assert (restored, prefilled) == (29 + 29 + 54, 29 + 25 + 12)
    forb = np.zeros(V, bool)
    near = sum(replay(W, p, prm, streams[t], forb) for t, (p, prm) in tasks.items())
    assert all(len(streams[t]) == 8 for t in tasks) and near <= 4
    R.rwkv7_sched_free(s)
    R.rwkv7_sched_gpu_backend_free(be)
    R.rwkv7_prefix_cache_free(cache)
    m.close()


def test_scheduler_restores_from_host_tier_and_stops(weights, W, R):
    """One device snapshot and two host ones: the second task's store moves
    the first prompt's state to the host arena, and the third task (which
    extends the first prompt) is restored from there.  The first task stops
    on its stop token (the oracle's third greedy pick)."""
    n_slots = max_b = 2
    m = R.Model.from_numpy(S, weights, n_slots=n_slots, max_B=max_b, max_T=64)
    stride = (R.rwkv7_snapshot_bytes(m.cfg) + 255) // 256 * 256
    arena = torch.empty(stride, dtype=torch.uint8, device="cuda")
    host = torch.empty(2 * stride, dtype=torch.uint8).pin_memory()
    cache = R.rwkv7_prefix_cache_create(m.handle, arena, host)
    occ = torch.zeros(n_slots * V, device="cuda")
    sws = torch.zeros(R.rwkv7_sample_workspace_bytes(max_b, V), dtype=torch.uint8, device="cuda")
    be = R.rwkv7_sched_gpu_backend(m.handle, m.pool, n_slots, occ, None, max_b, m.ws, sws, m.max_T)
    R.rwkv7_sched_gpu_backend_set_cache(be, cache)
    s = R.rwkv7_sched_create(R.SchedConfig(max_b, 1, 0, 10, V), be)
    p1, p2 = toks(60, 20).tolist(), toks(61, 24).tolist()
    p3 = p1 + toks(62, 5).tolist()
    # the oracle's greedy stream of p1 (penalties as below) gives the stop token
    st = O.State(S)
    O.seq(W, st, p1[:-1], want_logits=False)
    occ0 = np.zeros((1, V), np.float32)
    tok, greedy = p1[-1], []
    for _ in range(3):
        lg = O.step(W, [st], [tok])[0].astype(np.float32)[None]
        ids, occ0, _ = O.sample_penalized(lg, occ0, [0.3], [0.3], [0.996], [0.0], [1.0], [0], None, [0.5])
        tok = int(ids[0])
        greedy.append(tok)
    prm = [R.SchedParams(0.0, 1.0, 0, 0.3, 0.3, 0.996, 10, greedy[2], 1),
           R.SchedParams(1.0, 0.3, 0, 0.3, 0.3, 0.996, 6, -1, 2),
           R.SchedParams(0.0, 1.0, 0, 0.3, 0.3, 0.996, 6, -1, 3)]
    if greedy[2] in greedy[:2]:
        pytest.skip("the stop token occurs earlier in the stream")
    tasks = {}
    for p, q in zip((p1, p2, p3), prm):
        tasks[R.rwkv7_sched_submit(s, p, q)] = (p, q)
    events = []
    for _ in range(200):
        R.rwkv7_sched_step(s)
        events += R.rwkv7_sched_poll(s)
        if all(R.rwkv7_sched_task_state(s, t) == R.TASK_FINISHED for t in tasks):
            break
    streams, fin = {}, {}
    for task, kind, value, index in events:
        if kind == R.EV_TOKEN:
            streams.setdefault(task, []).append(value)
        else:
            fin[task] = (value, index)
    t1, t2, t3 = list(tasks)
    assert streams[t1] == greedy and fin[t1] == (R.FIN_STOP, 3)
    assert fin[t2] == (R.FIN_LENGTH, 6) and fin[t3] == (R.FIN_LENGTH, 6)
    assert R.rwkv7_sched_gpu_backend_counts(be) == (19, 19 + 23 + 5)
    cs = R.rwkv7_prefix_cache_stats(cache)
    assert cs.hits == 1 and cs.hit_tokens == 19 and cs.offloads >= 1 and cs.host_entries >= 1
    near = sum(replay(W, p, q, streams[t], np.zeros(V, bool)) for t, (p, q) in tasks.items())
    assert near <= 2
    R.rwkv7_sched_free(s)
    R.rwkv7_sched_gpu_backend_free(be)
    R.rwkv7_prefix_cache_free(cache)
    m.close()
