"""Seeded synthetic inputs for the RWKV-7 decode / prefill workloads.

This module only *draws numbers*: model shapes, random-init weights, prompt
lengths, prompt ids and teacher-forced token streams.  It holds none of the
model's arithmetic and imports neither the oracle nor the HIP library; both
sides consume exactly the arrays produced here.

The workloads follow the RWKV-Server article ("RWKV 批量推理中 Prefill 的正确打开方式",
section 2 table: prompts of 20-2000 tokens, single-token decode steps) and the
RWKV-Runner Albatross article (sampling defaults: frequency penalty 1, penalty
decay 0.996).  No public dataset is involved; uniform token ids stand in for
real text.

Determinism: every tensor is generated from its own ``SeedSequence`` child,
in fixed chunks, so the bytes do not depend on the thread count.
"""
from __future__ import annotations

import concurrent.futures as _cf
import json
import math
import os
from dataclasses import dataclass, field
from typing import Dict, Iterator, List, Tuple

import numpy as np

__all__ = [
    "ModelShape", "SHAPES", "TINY", "R7_2B9", "R7_7B2",
    "tensor_specs", "make_weights", "iter_layer_weights",
    "Workload", "WORKLOADS", "prompt_lengths", "prompt_tokens",
    "teacher_stream", "calibration_stream", "bkey_table",
]

_ROOT_ENTROPY = 0x52574B37  # "RWK7"


@dataclass(frozen=True)
class ModelShape:
    """RWKV-7 dimensions.  Matrices are stored (out, in) like ``torch.nn.Linear``."""
    name: str
    n_layer: int
    n_embd: int
    n_head: int
    head_size: int
    ffn: int
    d_w: int
    d_a: int
    d_v: int
    d_g: int
    vocab: int
    weight_dtype: str  # "f32" or "f16": the dtype the generated values are rounded to
    shape_id: int = 0

    @property
    def np_dtype(self):
        return np.float16 if self.weight_dtype == "f16" else np.float32


TINY = ModelShape("tiny", 2, 256, 4, 64, 1024, 32, 32, 32, 64, 1024, "f32", 1)
R7_2B9 = ModelShape("2.9b", 32, 2560, 40, 64, 10240, 64, 64, 32, 320, 65536, "f16", 2)
R7_7B2 = ModelShape("7.2b", 32, 4096, 64, 64, 16384, 128, 128, 64, 480, 65536, "f16", 3)
SHAPES = {s.name: s for s in (TINY, R7_2B9, R7_7B2)}


# --------------------------------------------------------------------------
# weight table
# --------------------------------------------------------------------------
# kind: ("normal", fan_in) | ("std", mean, scale) | ("uniform", lo, hi) | ("bkey",)
def tensor_specs(s: ModelShape) -> List[Tuple[str, Tuple[int, ...], tuple]]:
    """Every tensor of the model, in the fixed order that assigns seeds."""
    C, F, V, H, N = s.n_embd, s.ffn, s.vocab, s.n_head, s.head_size
    gamma = ("std", 1.0, 0.1)
    beta = ("std", 0.0, 0.1)
    specs: List[Tuple[str, Tuple[int, ...], tuple]] = [
        ("emb.weight", (V, C), ("normal", 1)),
        ("ln0.weight", (C,), gamma),
        ("ln0.bias", (C,), beta),
    ]
    for l in range(s.n_layer):
        p = f"blocks.{l}."
        specs += [
            (p + "ln1.weight", (C,), gamma),
            (p + "ln1.bias", (C,), beta),
        ]
        for q in "rwkvag":
            specs.append((p + f"att.x_{q}", (C,), ("uniform", 0.0, 1.0)))
        specs += [
            (p + "att.w0", (C,), ("uniform", -6.0, 0.0)),
            (p + "att.w1", (s.d_w, C), ("normal", C)),
            (p + "att.w2", (C, s.d_w), ("normal", s.d_w)),
            (p + "att.a0", (C,), ("std", 0.0, 1.0)),
            (p + "att.a1", (s.d_a, C), ("normal", C)),
            (p + "att.a2", (C, s.d_a), ("normal", s.d_a)),
            (p + "att.v0", (C,), ("std", 0.0, 1.0)),
            (p + "att.v1", (s.d_v, C), ("normal", C)),
            (p + "att.v2", (C, s.d_v), ("normal", s.d_v)),
            (p + "att.g1", (s.d_g, C), ("normal", C)),
            (p + "att.g2", (C, s.d_g), ("normal", s.d_g)),
            (p + "att.k_k", (C,), ("std", 1.0, 0.1)),
            (p + "att.k_a", (C,), ("uniform", 0.0, 1.0)),
            (p + "att.r_k", (H, N), ("std", 0.0, 0.1)),
            (p + "att.receptance.weight", (C, C), ("normal", C)),
            (p + "att.key.weight", (C, C), ("normal", C)),
            (p + "att.value.weight", (C, C), ("normal", C)),
            (p + "att.output.weight", (C, C), ("normal", C)),
            # per-head GroupNorm gain 0.1: at gain 1 this random network
            # amplifies a 1e-7 relative perturbation of its weights up to
            # ~4e4-fold in the logits over 32 layers, too much for fp16
            # activations to stay within 1e-2; at 0.1 such perturbations
            # grow at most ~10x (oracle/gn_gain_sensitivity.py measures both).
            (p + "att.ln_x.weight", (C,), ("std", 0.1, 0.01)),
            (p + "att.ln_x.bias", (C,), ("std", 0.0, 0.01)),
            (p + "ln2.weight", (C,), gamma),
            (p + "ln2.bias", (C,), beta),
            (p + "ffn.x_k", (C,), ("uniform", 0.0, 1.0)),
            (p + "ffn.key.weight", (F, C), ("normal", C)),
            (p + "ffn.key.bias", (F,), ("bkey",)),
            (p + "ffn.value.weight", (C, F), ("normal", F)),
        ]
    specs += [
        ("ln_out.weight", (C,), gamma),
        ("ln_out.bias", (C,), beta),
        ("head.weight", (V, C), ("normal", C)),
    ]
    return specs


_CHUNK = 1 << 22  # elements per independently seeded chunk


def _draw_chunk(args):
    seed, n, kind, out_dtype = args
    g = np.random.Generator(np.random.PCG64(seed))
    if kind[0] == "normal":
        x = g.standard_normal(n, dtype=np.float32)
        if kind[1] != 1:
            x *= np.float32(1.0 / math.sqrt(kind[1]))
    elif kind[0] == "std":
        x = g.standard_normal(n, dtype=np.float32)
        x *= np.float32(kind[2])
        x += np.float32(kind[1])
    elif kind[0] == "uniform":
        x = g.random(n, dtype=np.float32)
        x *= np.float32(kind[2] - kind[1])
        x += np.float32(kind[1])
    else:
        raise ValueError(kind)
    return x.astype(out_dtype, copy=False)


_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        n = int(os.environ.get("RWKV7_SYNTH_THREADS", "0")) or min(16, os.cpu_count() or 4)
        _POOL = _cf.ThreadPoolExecutor(max_workers=n)
    return _POOL


def _tensor_seed(s: ModelShape, index: int) -> np.random.SeedSequence:
    return np.random.SeedSequence([_ROOT_ENTROPY, s.shape_id, index])


def _gen_tensor(s: ModelShape, index: int, shape, kind, bkey_value=None) -> np.ndarray:
    n = int(np.prod(shape))
    dt = s.np_dtype
    if kind[0] == "bkey":
        return np.full(shape, bkey_value, dtype=np.float32).astype(dt)
    n_chunks = (n + _CHUNK - 1) // _CHUNK
    seeds = _tensor_seed(s, index).spawn(n_chunks)
    jobs = [(seeds[i], min(_CHUNK, n - i * _CHUNK), kind, dt) for i in range(n_chunks)]
    if n_chunks == 1:
        parts = [_draw_chunk(jobs[0])]
    else:
        parts = list(_pool().map(_draw_chunk, jobs))
    out = np.concatenate(parts) if len(parts) > 1 else parts[0]
    return out.reshape(shape)


_BKEY_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "bkey.json")


def bkey_table(s: ModelShape) -> List[float]:
    """Per-layer channel-mix key bias (one scalar per layer).

    The values were written by ``oracle/calibrate_bkey.py``: for each layer,
    minus the 0.85-quantile of the key pre-activations over a seeded
    64-token calibration stream, so that about 85 % of ReLU^2 outputs are
    zero.  This module only reads them.
    """
    with open(_BKEY_FILE) as f:
        tab = json.load(f)
    if s.name not in tab:
        raise KeyError(f"no calibrated key bias for shape {s.name!r}; run oracle/calibrate_bkey.py")
    vals = tab[s.name]["bkey"]
    if len(vals) != s.n_layer:
        raise ValueError("bkey table has the wrong number of layers")
    return [float(v) for v in vals]


def make_weights(s: ModelShape, bkey: List[float] | None = None,
                 names: List[str] | None = None) -> Dict[str, np.ndarray]:
    """Generate the model's weights (all of them, or only ``names``).

    ``bkey`` overrides the stored per-layer key bias (the calibration script
    passes zeros for layers it has not calibrated yet).
    """
    if bkey is None:
        bkey = bkey_table(s)
    want = None if names is None else set(names)
    out: Dict[str, np.ndarray] = {}
    for idx, (name, shape, kind) in enumerate(tensor_specs(s)):
        if want is not None and name not in want:
            continue
        bv = None
        if kind[0] == "bkey":
            bv = bkey[int(name.split(".")[1])]
        out[name] = _gen_tensor(s, idx, shape, kind, bv)
    return out


def iter_layer_weights(s: ModelShape, bkey: List[float] | None = None) -> Iterator[Tuple[str, Dict[str, np.ndarray]]]:
    """Yield ("global", {...}) then ("blocks.l", {...}) groups, to bound host memory."""
    specs = tensor_specs(s)
    groups: Dict[str, List[str]] = {}
    order: List[str] = []
    for name, _, _ in specs:
        g = ".".join(name.split(".")[:2]) if name.startswith("blocks.") else "global"
        if g not in groups:
            groups[g] = []
            order.append(g)
        groups[g].append(name)
    if bkey is None:
        bkey = bkey_table(s)
    for g in order:
        yield g, make_weights(s, bkey, groups[g])


# --------------------------------------------------------------------------
# workloads (token streams)
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    """One decode / prefill workload on a model shape."""
    name: str
    shape: ModelShape
    batch: int                 # decode rows B (1 for prefill workloads)
    prompt_len: int            # fixed prompt length; 0 = log-uniform 20..2000
    steps: int                 # decode steps after the prompt
    presence: float = 0.0      # presence penalty
    frequency: float = 0.0     # frequency penalty
    decay: float = 1.0         # penalty decay per step
    workload_id: int = 0
    prefill_T: Tuple[int, ...] = field(default_factory=tuple)


WORKLOADS = {
    w.name: w for w in (
        Workload("tiny", TINY, 1, 8, 16, workload_id=1),
        Workload("decode_b1_2.9b", R7_2B9, 1, 64, 256, workload_id=2),
        Workload("decode_b64_2.9b", R7_2B9, 64, 0, 512, 1.0, 1.0, 0.996, workload_id=3),
        Workload("decode_b256_2.9b", R7_2B9, 256, 0, 512, 1.0, 1.0, 0.996, workload_id=4),
        Workload("decode_b256_7.2b", R7_7B2, 256, 0, 512, 1.0, 1.0, 0.996, workload_id=5),
        Workload("prefill_2.9b", R7_2B9, 1, 0, 64, workload_id=6, prefill_T=(128, 512, 2048)),
    )
}


def _wl_seed(w: Workload, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([_ROOT_ENTROPY, 1000 + w.workload_id, stream])))


def prompt_lengths(w: Workload, n: int | None = None) -> np.ndarray:
    """Prompt length per slot: fixed, or floor(exp(U(ln 20, ln 2001))) in [20, 2000]."""
    n = w.batch if n is None else n
    if w.prompt_len > 0:
        return np.full(n, w.prompt_len, dtype=np.int64)
    g = _wl_seed(w, 0)
    u = g.random(n)
    L = np.floor(np.exp(np.log(20.0) + u * (np.log(2001.0) - np.log(20.0)))).astype(np.int64)
    return np.clip(L, 20, 2000)


def prompt_tokens(w: Workload, slot: int, length: int) -> np.ndarray:
    """Uniform token ids of one slot's prompt (int32)."""
    g = _wl_seed(w, 10_000 + slot)
    return g.integers(0, w.shape.vocab, size=length, dtype=np.int64).astype(np.int32)


def prefill_tokens(w: Workload, T: int) -> np.ndarray:
    """Uniform ids for a T-token prefill."""
    g = _wl_seed(w, 20_000 + T)
    return g.integers(0, w.shape.vocab, size=T, dtype=np.int64).astype(np.int32)


def teacher_stream(w: Workload, slot: int, steps: int) -> np.ndarray:
    """Teacher-forced decode inputs for one slot (int32, uniform ids)."""
    g = _wl_seed(w, 30_000 + slot)
    return g.integers(0, w.shape.vocab, size=steps, dtype=np.int64).astype(np.int32)


def calibration_stream(s: ModelShape, T: int = 64) -> np.ndarray:
    """The 64-token stream the key-bias calibration runs over."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([_ROOT_ENTROPY, 500, s.shape_id])))
    return g.integers(0, s.vocab, size=T, dtype=np.int64).astype(np.int32)


def random_state_like(n: int, seed: int, scale: float = 1.0) -> np.ndarray:
    """Seeded N(0, scale^2) fp32 values, for tests that start from non-zero states."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([_ROOT_ENTROPY, 700, seed])))
    return (g.standard_normal(n, dtype=np.float32) * np.float32(scale))
