"""The continuous-batching scheduler on the GPU backend (rwkv7_sched_gpu_backend
over the tiny model) against the oracle.

Each task's emitted stream is replayed through the fp64 oracle, teacher
forced: the oracle consumes the task's prompt (prompt[:-1] as a sequence, the
last token as the first decode input) and then each emitted token, and at
every position draws with the oracle's sampler from its own logits, the same
uniform (the task's SplitMix64 stream) and the same occurrence row.  The
emitted id must be the oracle's, or, where GPU and oracle logits differ
within the logits tolerance and the draw sits at a boundary, one the oracle
picks for a uniform within 0.01 (a greedy pick within 2 % of a standard
deviation of the top logit).  Such near-boundary draws are expected: with
the whole vocabulary kept (temperature 1.3, top_p 1.0) about a thousand
interval boundaries lie in [0, 1), and logits that differ at the 1e-3 level
move one of them past u in a few percent of draws; they are counted and must
stay under 15 % of all draws, while a wrong slot, state, uniform or parameter
sends draws outside the window.  Tasks mix one-token and sequence prefills, greedy and sampled
rows, top-k / top-p, penalties and a forbidden mask; slots are reused as tasks
finish, and one task is aborted."""
import numpy as np
import pytest
import torch

import synth
from oracle import rwkv7 as O
from test_sched_host import uniform

pytestmark = pytest.mark.gpu

S = synth.TINY
V = S.vocab


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


def replay(W, prompt, prm, stream, forb):
    """Near-boundary count of one task's stream; asserts every emitted id is valid."""
    st = O.State(S)
    if len(prompt) >= 2:
        O.seq(W, st, prompt[:-1], want_logits=False)
    occ = np.zeros((1, V), np.float32)
    tok = prompt[-1]
    near = 0
    f32 = np.float32
    for j, g in enumerate(stream):
        lg = O.step(W, [st], [tok])[0].astype(np.float32)[None]
        u = uniform(prm.seed, j)

        def draw(x):
            ids, _, err = O.sample_penalized(lg, occ, [prm.presence], [prm.frequency], [prm.decay],
                                             [prm.temperature], [prm.top_p], [prm.top_k], forb, [x])
            assert not err.any()
            return int(ids[0])

        if draw(u) != g:
            if prm.temperature > 0:
                window = {draw(x) for x in np.clip(np.linspace(u - 0.01, u + 0.01, 81), 0.0, 1.0)}
                assert g in window, (j, g, sorted(window))
            else:
                lp = lg[0].astype(np.float64) - np.where(occ[0] > 0, prm.frequency * occ[0] + prm.presence, 0.0)
                lp[forb] = -np.inf
                assert not forb[g] and lp[g] >= lp.max() - 0.02 * np.std(lg[0]), (j, g)
            near += 1
        occ = (occ * f32(prm.decay)).astype(np.float32)
        occ[0, g] = occ[0, g] + f32(1)
        tok = g
    return near


def test_scheduler_streams_match_oracle(weights, W, R):
    n_slots, max_b = 6, 6
    # max_T 16: prompts of 17..64 tokens are prefilled by the backend in 16-token pieces
    m = R.Model.from_numpy(S, weights, n_slots=n_slots, max_B=max_b, max_T=16)
    occ = torch.zeros(n_slots * V, device="cuda")
    forb = np.zeros(V, bool)
    forb[:8] = True
    forb[500:520] = True
    forb_t = torch.tensor(forb.astype(np.uint8), device="cuda")
    sws = torch.zeros(R.rwkv7_sample_workspace_bytes(max_b, V), dtype=torch.uint8, device="cuda")
    be = R.rwkv7_sched_gpu_backend(m.handle, m.pool, n_slots, occ, forb_t, max_b, m.ws, sws, m.max_T)
    s = R.rwkv7_sched_create(R.SchedConfig(max_b, 2, 3, 10, V), be)
    kinds = [(0.0, 1.0, 0), (1.0, 0.3, 0), (0.8, 0.9, 5), (1.3, 1.0, 0)]
    tasks = {}
    for i, n in enumerate([1, 2, 5, 9, 10, 16, 33, 3, 12, 1, 40, 7, 64, 2]):
        T, p, k = kinds[i % 4]
        prm = R.SchedParams(T, p, k, 0.5, 0.5, 0.996, 6 + i % 7, -1, 1000 + 77 * i)
        pr = np.random.default_rng(700 + i).integers(0, V, n).tolist()
        tasks[R.rwkv7_sched_submit(s, pr, prm)] = (pr, prm)
    aborted = list(tasks)[5]
    events, stats = [], []
    for r in range(400):
        if r == 8:
            R.rwkv7_sched_abort(s, aborted)
        stats.append(R.rwkv7_sched_step(s))
        events += R.rwkv7_sched_poll(s)
        if all(R.rwkv7_sched_task_state(s, t) == R.TASK_FINISHED for t in tasks):
            break
    else:
        raise AssertionError("tasks did not finish")
    streams, fin = {}, {}
    for task, kind, value, index in events:
        if kind == R.EV_TOKEN:
            assert index == len(streams.setdefault(task, []))
            streams[task].append(value)
        else:
            fin[task] = (value, index)
    assert sum(st.seq_prefills for st in stats) >= 4 and sum(st.one_prefill_rows for st in stats) > 0
    assert max(st.decode_rows + st.one_prefill_rows for st in stats) >= 4
    near = 0
    for t, (pr, prm) in tasks.items():
        got = streams.get(t, [])
        if t == aborted:
            assert fin[t] == (R.FIN_ABORT, len(got)) and len(got) < prm.max_new_tokens
        else:
            assert fin[t] == (R.FIN_LENGTH, prm.max_new_tokens) and len(got) == prm.max_new_tokens
        assert not any(forb[g] for g in got)
        near += replay(W, pr, prm, got, forb)
    total = sum(len(v) for v in streams.values())
    print("near-boundary draws:", near, "of", total)
    assert near <= 0.15 * total
    R.rwkv7_sched_free(s)
    R.rwkv7_sched_gpu_backend_free(be)
    assert R.rwkv7_poll_error(m.ws) == 0
    m.close()


def test_gpu_backend_rejects_bad_sizes(weights, R):
    m = R.Model.from_numpy(S, weights, n_slots=2, max_B=2, max_T=16)
    occ = torch.zeros(2 * V, device="cuda")
    small = torch.zeros(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(R.RWKV7Error):
        R.rwkv7_sched_gpu_backend(m.handle, m.pool, 2, occ, None, 2, m.ws, small, m.max_T)
    sws = torch.zeros(R.rwkv7_sample_workspace_bytes(3, V), dtype=torch.uint8, device="cuda")
    with pytest.raises(R.RWKV7Error):
        R.rwkv7_sched_gpu_backend(m.handle, m.pool, 2, occ, None, 3, m.ws, sws, m.max_T)
    # caller-owned staging: too small (ESHAPE), misaligned (EINVAL), max_T < 1 (EINVAL)
    sws2 = torch.zeros(R.rwkv7_sample_workspace_bytes(2, V), dtype=torch.uint8, device="cuda")
    nd, nh = R.rwkv7_sched_gpu_backend_bytes(m.handle, 2, m.max_T)
    assert nd >= 2 * V * 4 + m.max_T * 4 and nh >= 9 * 2 * 4
    dev = torch.empty(nd + 256, dtype=torch.uint8, device="cuda")
    host = torch.empty(nh + 256, dtype=torch.uint8, pin_memory=True)
    with pytest.raises(R.RWKV7Error) as e:
        R.rwkv7_sched_gpu_backend(m.handle, m.pool, 2, occ, None, 2, m.ws, sws2, m.max_T, dev[:nd - 256], host)
    assert e.value.status == R.RWKV7_ESHAPE
    with pytest.raises(R.RWKV7Error) as e:
        R.rwkv7_sched_gpu_backend(m.handle, m.pool, 2, occ, None, 2, m.ws, sws2, m.max_T, dev[4:], host)
    assert e.value.status == R.RWKV7_EINVAL
    with pytest.raises(R.RWKV7Error) as e:
        R.rwkv7_sched_gpu_backend(m.handle, m.pool, 2, occ, None, 2, m.ws, sws2, 0, dev, host)
    assert e.value.status == R.RWKV7_EINVAL
    be = R.rwkv7_sched_gpu_backend(m.handle, m.pool, 2, occ, None, 2, m.ws, sws2, m.max_T, dev, host)
    R.rwkv7_sched_gpu_backend_free(be)
    m.close()
