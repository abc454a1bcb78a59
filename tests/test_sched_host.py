"""Host logic of the continuous-batching scheduler (include/rwkv7_sched.h),
driven through the C ABI with a mock model and no GPU.

The mock's "state" of a slot is the list of tokens the slot has consumed, and
its sampled id is a hash of that list, the row's uniform and its sampling
parameters.  A task's stream is therefore fixed by its own prompt, its
parameters and its uniform stream alone, as for a real model: any mix-up of
slots, tokens, rows, parameters, uniforms, resets or prefill ranges changes
some stream.  The reference for each task is the plain sequential definition:
consume the prompt, then draw, emit and consume one token at a time until the
stop token or max_new_tokens.  CPU only."""
import struct
import zlib

import numpy as np
import pytest

import rwkv_linear_attention_decode_amd as R

V = 1000
MASK64 = (1 << 64) - 1


def splitmix64(seed, n):
    """Output number n (n >= 1) of SplitMix64 started at `seed` (Steele, Lea and
    Flood, OOPSLA 2014), written from the published definition."""
    z = (seed + n * 0x9E3779B97F4A7C15) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def uniform(seed, j):
    return np.float32((splitmix64(seed, j + 1) >> 40) / 16777216.0)


def test_splitmix64_published_value():
    # the generator's first output from state 0, as listed with its reference code
    assert splitmix64(0, 1) == 0xE220A8397B1DCDAF


def mock_id(hist, u, temp, top_p, top_k, pres, freq, dec):
    blob = np.asarray(hist, np.int32).tobytes() + struct.pack("<ffiffff", temp, top_p, top_k, pres, freq, dec,
                                                              u)
    return zlib.crc32(blob) % V


class Mock:
    def __init__(self, max_batch):
        self.hist = {}
        self.log = []        # ("reset"|"prefill"|"step", ...)
        self.max_batch = max_batch
        self.fail_next_step = False

    def reset(self, slot):
        assert 0 <= slot < self.max_batch
        self.hist[slot] = []
        self.log.append(("reset", slot))

    def prefill(self, slot, toks):
        assert len(toks) >= 1
        self.hist[slot].extend(toks)
        self.log.append(("prefill", slot, list(toks)))

    def step(self, slots, tokens, S, p):
        if self.fail_next_step:
            self.fail_next_step = False
            raise RuntimeError("planted backend failure")
        assert len(set(slots)) == len(slots) <= self.max_batch
        out = []
        for r, (sl, tok) in enumerate(zip(slots, tokens)):
            self.hist[sl].append(tok)
            if r < S:
                out.append(mock_id(self.hist[sl], p["uniform"][r], p["temperature"][r], p["top_p"][r],
                                   p["top_k"][r], p["presence"][r], p["frequency"][r], p["decay"][r]))
        self.log.append(("step", list(slots), list(tokens), S, dict(p)))
        return out


def reference(prompt, prm):
    hist = list(prompt)
    out = []
    f32 = lambda x: float(np.float32(x))
    for j in range(prm.max_new_tokens):
        t = mock_id(hist, uniform(prm.seed, j), f32(prm.temperature), f32(prm.top_p), prm.top_k,
                    f32(prm.presence), f32(prm.frequency), f32(prm.decay))
        out.append(t)
        if t == prm.stop_token:
            return out, R.FIN_STOP
        hist.append(t)
    return out, R.FIN_LENGTH


def params(rng, stop=-1):
    return R.SchedParams(float(rng.choice([0.0, 0.7, 1.0])), float(rng.choice([0.3, 1.0])),
                         int(rng.choice([0, 5])), 0.5, float(rng.random()), 0.996,
                         int(rng.integers(1, 12)), stop, int(rng.integers(0, 1 << 63)))


def make(max_batch, **cfg):
    m = Mock(max_batch)
    be = R.sched_backend(m.reset, m.prefill, m.step)
    c = R.SchedConfig(max_batch, cfg.get("max_prefill_count", 0), cfg.get("decode_prefill_ratio", 0),
                      cfg.get("min_forward_seq_len", 0), V)
    s = R.rwkv7_sched_create(c, be)
    return m, be, s


def run_to_end(s, live_ids, limit=10000, check=None):
    events, stats = [], []
    for _ in range(limit):
        st = R.rwkv7_sched_step(s)
        stats.append(st)
        events += R.rwkv7_sched_poll(s)
        if check:
            check(st)
        if all(R.rwkv7_sched_task_state(s, t) == R.TASK_FINISHED for t in live_ids):
            return events, stats
    raise AssertionError("tasks did not finish")


def streams(events):
    out, fin = {}, {}
    for task, kind, value, index in events:
        if kind == R.EV_TOKEN:
            assert task not in fin
            lst = out.setdefault(task, [])
            assert index == len(lst)
            lst.append(value)
        else:
            assert task not in fin
            fin[task] = (value, index)
    return out, fin


@pytest.mark.parametrize("max_batch", [1, 4, 16])
def test_streams_equal_sequential_definition(max_batch):
    rng = np.random.default_rng(max_batch)
    m, be, s = make(max_batch)
    tasks = {}
    for i in range(40):
        n = int(rng.choice([1, 2, 3, 9, 10, 11, 25, 60]))
        prompt = rng.integers(0, V, n).tolist()
        prm = params(rng)
        if i % 5 == 0:                      # a stop token the task reaches at its third token
            prm.max_new_tokens = 8
            prm.stop_token = reference(prompt, prm)[0][2]
        tasks[R.rwkv7_sched_submit(s, prompt, prm)] = (prompt, prm)
    limit_prefill = max(int(max_batch * 0.125), 1)

    def check(st):
        assert st.decode_rows + st.one_prefill_rows <= max_batch
        n_pf = sum(R.rwkv7_sched_task_state(s, t) == R.TASK_PREFILL for t in tasks)
        assert n_pf <= limit_prefill

    events, stats = run_to_end(s, tasks, check=check)
    got, fin = streams(events)
    n_stop = 0
    for t, (prompt, prm) in tasks.items():
        ref, why = reference(prompt, prm)
        assert got[t] == ref, t
        assert fin[t] == (why, len(ref))
        n_stop += why == R.FIN_STOP
    assert n_stop >= 8
    # prefill paths: prompts of >= 10 tokens through one sequence prefill of prompt[:-1],
    # shorter ones token by token inside the batch
    pf = [e for e in m.log if e[0] == "prefill"]
    long_prompts = sorted(tuple(p[:-1]) for p, _ in tasks.values() if len(p) >= 10)
    assert sorted(tuple(e[2]) for e in pf) == long_prompts
    assert sum(st.seq_prefills for st in stats) == len(long_prompts)
    R.rwkv7_sched_free(s)


def test_sequence_prefills_are_paced():
    """A sequence prefill runs when nothing else is waiting, or once
    decode_prefill_ratio decode rounds have passed since the previous one."""
    rng = np.random.default_rng(5)
    m, be, s = make(8, max_prefill_count=8, decode_prefill_ratio=3)
    ids = []
    for i in range(12):
        n = 30 if i % 2 else 2
        prm = params(rng)
        prm.max_new_tokens = 20
        ids.append(R.rwkv7_sched_submit(s, rng.integers(0, V, n).tolist(), prm))
    events, stats = run_to_end(s, ids)
    last, decode_since = None, 0
    n = 0
    for st in stats:
        if st.seq_prefills:
            n += 1
            alone = st.decode_rows == 1 and st.one_prefill_rows == 0
            assert last is None or decode_since >= 3 or alone
            last, decode_since = st, 0
        decode_since += st.decode_rows > 0
    assert n == 6


def test_abort_queued_and_running():
    rng = np.random.default_rng(9)
    m, be, s = make(1)
    p1, p2 = params(rng), params(rng)
    p1.max_new_tokens = p2.max_new_tokens = 50
    a = R.rwkv7_sched_submit(s, [1, 2, 3], p1)
    b = R.rwkv7_sched_submit(s, [4], p2)
    assert R.rwkv7_sched_task_state(s, b) == R.TASK_QUEUED
    R.rwkv7_sched_abort(s, b)
    for _ in range(5):
        R.rwkv7_sched_step(s)
    assert R.rwkv7_sched_task_state(s, a) == R.TASK_RUNNING
    R.rwkv7_sched_abort(s, a)
    R.rwkv7_sched_step(s)
    got, fin = streams(R.rwkv7_sched_poll(s))
    assert b not in got and fin[b] == (R.FIN_ABORT, 0)
    assert fin[a] == (R.FIN_ABORT, len(got[a])) and got[a] == reference([1, 2, 3], p1)[0][:len(got[a])]
    for t in (a, b):
        assert R.rwkv7_sched_task_state(s, t) == R.TASK_FINISHED
        with pytest.raises(R.RWKV7Error):
            R.rwkv7_sched_abort(s, t)
    with pytest.raises(R.RWKV7Error):
        R.rwkv7_sched_task_state(s, 99)
    st = R.rwkv7_sched_step(s)               # nothing left: an empty round
    assert (st.decode_rows, st.active, st.queued) == (0, 0, 0)


def test_failed_round_is_retried_without_loss():
    rng = np.random.default_rng(13)
    m, be, s = make(3)
    tasks = {}
    for n in (1, 4, 12, 2, 30):
        prm = params(rng)
        prm.max_new_tokens = 6
        p = rng.integers(0, V, n).tolist()
        tasks[R.rwkv7_sched_submit(s, p, prm)] = (p, prm)
    events = []
    for r in range(4):
        R.rwkv7_sched_step(s)
    events += R.rwkv7_sched_poll(s)
    m.fail_next_step = True
    with pytest.raises(R.RWKV7Error):
        R.rwkv7_sched_step(s)
    ev, _ = run_to_end(s, tasks)
    got, fin = streams(events + ev)
    for t, (p, prm) in tasks.items():
        assert got[t] == reference(p, prm)[0]


def test_host_validation():
    rng = np.random.default_rng(1)
    m, be, s = make(2)
    prm = params(rng)
    for bad in ([], [V], [-1]):
        with pytest.raises(R.RWKV7Error):
            R.rwkv7_sched_submit(s, bad, prm)
    prm.max_new_tokens = 0
    with pytest.raises(R.RWKV7Error):
        R.rwkv7_sched_submit(s, [1], prm)
    prm.max_new_tokens, prm.stop_token = 3, V
    with pytest.raises(R.RWKV7Error):
        R.rwkv7_sched_submit(s, [1], prm)
    with pytest.raises(R.RWKV7Error):
        R.rwkv7_sched_create(R.SchedConfig(0, 0, 0, 0, V), be)
    with pytest.raises(R.RWKV7Error):
        R.rwkv7_sched_create(R.SchedConfig(2, 0, 0, 0, 0), be)
    with pytest.raises(R.RWKV7Error):    # only backends it made can be freed as GPU backends
        R.rwkv7_sched_gpu_backend_free(be)
    R.rwkv7_sched_free(s)


def test_admission_is_fifo_and_capped():
    """With max_batch 16 the prefill cap defaults to 2: the queue head waits
    while two tasks are in a prefill phase, and nothing overtakes it."""
    rng = np.random.default_rng(3)
    m, be, s = make(16)
    ids = []
    for i in range(6):
        prm = params(rng)
        prm.max_new_tokens = 3
        ids.append(R.rwkv7_sched_submit(s, rng.integers(0, V, 5).tolist(), prm))
    st = R.rwkv7_sched_step(s)
    assert st.admitted == 2 and st.queued == 4
    states = [R.rwkv7_sched_task_state(s, t) for t in ids]
    assert states == [R.TASK_PREFILL] * 2 + [R.TASK_QUEUED] * 4
    resets = [e[1] for e in m.log if e[0] == "reset"]
    assert resets == [0, 1]
