"""RWKV-7 decode / prefill hot path for AMD MI355X (gfx950).

A thin ctypes binding over ``librwkv7.so`` (include/rwkv7.h).  The functions
below carry the C names and only marshal arguments: torch CUDA(HIP) tensors
are passed as device pointers, the stream defaults to torch's current
stream.  Every step of the computation runs in the library's HIP kernels;
there is no Python or CPU fallback, and a missing library raises.

``Model`` is a convenience holder that allocates the packed weights, the
state pool and the workspace through torch and keeps the handle.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librwkv7.so")

RWKV7_OK, RWKV7_EINVAL, RWKV7_ESHAPE, RWKV7_EHIP, RWKV7_EDEVICE, RWKV7_ENOTSUP = range(6)
ERR_SLOT_RANGE, ERR_SLOT_DUP, ERR_TOKEN_RANGE, ERR_ALL_NAN = 1, 2, 4, 8
F32, F16 = 0, 1
OPT_USE_GRAPH, OPT_GEMV_MAX_B, OPT_SPARSE_MAX_B, OPT_KERNEL_TIMING, OPT_PREFILL_CHUNK = 1, 2, 3, 4, 5
OPT_FUSE_LN = 6
OPT_FUSE_VALUE = 7
# tile plan per MFMA projection: decimal digits "T N KKK P S" (0 = built-in)
OPT_GEMM_PLAN_PROJ_IN = 8
OPT_GEMM_PLAN_ADAPTERS = 9
OPT_GEMM_PLAN_PROJ_OUT = 10
OPT_GEMM_PLAN_CMIX_KEY = 11
OPT_GEMM_PLAN_CMIX_VALUE = 12
OPT_GEMM_PLAN_HEAD = 13
OPT_PREFILL_SCAN = 14
OPT_INT8 = 15
# workgroups per row of the batched decode LayerNorm kernel (0 = automatic)
OPT_LN_SPLIT = 16
OPT_WKV_ADAPTERS = 17


def gemm_plan_code(tm, tn, ks, pipe=0, split=0):
    """Value of an OPT_GEMM_PLAN_* option: tile 32*tm x 32*tn, stage depth ks,
    K loop `pipe` (0 plain, 1 pipelined LDS reads, 2 two stages of global loads in
    flight, 3 LDS-DMA ring, 4 the same with eight waves, 5 a deep LDS-DMA ring filling
    about 144 KB of LDS, 6 the same in about 72 KB), K split (0 = automatic).
    tm = 8, tn = 10 (256 x 320 tiles) gives the digits 9 0, which the library reads so."""
    return ((tm * 10 + tn) * 1000 + ks) * 100 + pipe * 10 + split
K_LN_MIX, K_PROJ_IN, K_WKV, K_PROJ_OUT, K_CMIX_KEY, K_CMIX_VALUE, K_HEAD, K_OTHER = range(8)
K_NAMES = ("ln_mix", "proj_in", "wkv", "proj_out", "cmix_key", "cmix_value", "head", "other")


class RWKV7Error(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: status {status}: {msg}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layer", "n_embd", "n_head", "head_size", "ffn", "d_w", "d_a", "d_v", "d_g", "vocab")]


class Tensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("data", ctypes.c_void_p)]


# ---- scheduler structures (include/rwkv7_sched.h)
TASK_QUEUED, TASK_PREFILL, TASK_READY, TASK_RUNNING, TASK_FINISHED = range(5)
EV_TOKEN, EV_FINISHED = 1, 2
FIN_LENGTH, FIN_STOP, FIN_ABORT = 1, 2, 3


class SchedConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "max_batch", "max_prefill_count", "decode_prefill_ratio", "min_forward_seq_len", "vocab")]


class SchedParams(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_p", ctypes.c_float), ("top_k", ctypes.c_int32),
                ("presence", ctypes.c_float), ("frequency", ctypes.c_float), ("decay", ctypes.c_float),
                ("max_new_tokens", ctypes.c_int32), ("stop_token", ctypes.c_int32), ("seed", ctypes.c_uint64)]


class SchedBatch(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("slots", ctypes.POINTER(ctypes.c_int32)),
                ("tokens", ctypes.POINTER(ctypes.c_int32)), ("n_sample", ctypes.c_int32),
                ("temperature", ctypes.POINTER(ctypes.c_float)), ("top_p", ctypes.POINTER(ctypes.c_float)),
                ("top_k", ctypes.POINTER(ctypes.c_int32)), ("presence", ctypes.POINTER(ctypes.c_float)),
                ("frequency", ctypes.POINTER(ctypes.c_float)), ("decay", ctypes.POINTER(ctypes.c_float)),
                ("uniform", ctypes.POINTER(ctypes.c_float))]


RESET_FN = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_int32)
PREFILL_FN = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                              ctypes.c_int32)
STEP_FN = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(SchedBatch),
                           ctypes.POINTER(ctypes.c_int32))


class SchedBackend(ctypes.Structure):
    _fields_ = [("ctx", ctypes.c_void_p), ("reset", RESET_FN), ("prefill", PREFILL_FN), ("step", STEP_FN)]


class SchedEvent(ctypes.Structure):
    _fields_ = [("task", ctypes.c_int64), ("kind", ctypes.c_int32), ("value", ctypes.c_int32),
                ("index", ctypes.c_int32), ("pad", ctypes.c_int32)]


class SchedStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "decode_rows", "one_prefill_rows", "seq_prefills", "seq_prefill_tokens", "admitted", "finished",
        "queued", "active")]


class PrefixStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("lookups", "hits", "hit_tokens", "stores", "offloads", "drops")] + \
               [(n, ctypes.c_int32) for n in ("device_entries", "host_entries", "device_capacity", "host_capacity")]


_lib = None


def lib() -> ctypes.CDLL:
    """Load librwkv7.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m rwkv_linear_attention_decode_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, u64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p
    P = ctypes.POINTER
    sig = {
        "rwkv7_packed_bytes": [P(Config), P(u64)],
        "rwkv7_slot_floats": [P(Config), P(u64)],
        "rwkv7_state_bytes": [P(Config), i64, P(u64), P(u64)],
        "rwkv7_workspace_bytes": [P(Config), i32, i32, P(u64)],
        "rwkv7_load": [P(Config), P(Tensor), i32, vp, u64, vp, P(vp)],
        "rwkv7_free": [vp],
        "rwkv7_reset_slots": [vp, vp, i64, vp, i32, vp, u64, vp],
        "rwkv7_decode_step": [vp, vp, i64, i32, vp, vp, vp, vp, u64, vp],
        "rwkv7_prefill_seq": [vp, vp, i64, i32, vp, i32, vp, u64, vp],
        "rwkv7_greedy_workspace_bytes": [i32, i32, P(u64)],
        "rwkv7_greedy": [i32, i32, vp, vp, i64, vp, vp, vp, vp, vp, vp, u64, vp],
        "rwkv7_greedy_noalloc": [i32, i32, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp],
        "rwkv7_sample_workspace_bytes": [i32, i32, P(u64)],
        "rwkv7_sample": [i32, i32, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, u64, vp],
        "rwkv7_poll_error": [vp, vp, P(ctypes.c_uint32)],
        "rwkv7_set_option": [vp, i32, i64],
        "rwkv7_get_option": [vp, i32, P(i64)],
        "rwkv7_kernel_timing": [vp, i32, P(ctypes.c_double), P(i64), i32],
        "rwkv7_debug_cmix_buffers": [vp, vp, i32, P(vp), P(vp), P(vp), P(vp)],
        "rwkv7_debug_wkv_out": [vp, vp, i32, P(vp), P(i32)],
        "rwkv7_read_bandwidth": [vp, u64, i32, i32, vp, P(ctypes.c_double)],
        "rwkv7_time_kernel": [vp, vp, i64, i32, vp, vp, vp, i32, i32, i32, vp, u64, vp,
                              P(ctypes.c_double)],
        "rwkv7_sched_create": [P(SchedConfig), P(SchedBackend), P(vp)],
        "rwkv7_sched_free": [vp],
        "rwkv7_sched_submit": [vp, P(i32), i32, P(SchedParams), P(i64)],
        "rwkv7_sched_abort": [vp, i64],
        "rwkv7_sched_step": [vp, P(SchedStats)],
        "rwkv7_sched_poll": [vp, P(SchedEvent), i32, P(i32)],
        "rwkv7_sched_task_state": [vp, i64, P(i32)],
        "rwkv7_sched_gpu_backend_bytes": [vp, i32, i32, P(u64), P(u64)],
        "rwkv7_sched_gpu_backend": [vp, vp, i64, vp, vp, i32, i32, vp, u64, vp, u64, vp, u64, vp, u64, vp,
                                    P(SchedBackend)],
        "rwkv7_sched_gpu_backend_free": [P(SchedBackend)],
        "rwkv7_sched_gpu_backend_set_cache": [P(SchedBackend), vp],
        "rwkv7_sched_gpu_backend_counts": [P(SchedBackend), P(i64), P(i64)],
        "rwkv7_int8_bytes": [P(Config), P(u64)],
        "rwkv7_quantize_int8": [vp, vp, u64, vp],
        "rwkv7_debug_int8_matrix": [vp, i32, i32, P(vp), P(vp), P(i64), P(i32)],
        "rwkv7_snapshot_bytes": [P(Config), P(u64)],
        "rwkv7_slot_export": [vp, vp, i64, i32, vp, vp],
        "rwkv7_slot_import": [vp, vp, i64, i32, vp, vp],
        "rwkv7_prefix_cache_create": [vp, vp, u64, vp, u64, P(vp)],
        "rwkv7_prefix_cache_free": [vp],
        "rwkv7_prefix_cache_store": [vp, vp, i64, i32, P(i32), i32, vp],
        "rwkv7_prefix_cache_lookup": [vp, vp, i64, i32, P(i32), i32, P(i32), vp],
        "rwkv7_prefix_cache_stats": [vp, P(PrefixStats)],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    for name, args in {"rwkv7_status_string": [ctypes.c_int], "rwkv7_last_error": [],
                       "rwkv7_kernel_name": [vp, i32, i32]}.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(rc: int, where: str):
    if rc != RWKV7_OK:
        L = lib()
        raise RWKV7Error(rc, where, (L.rwkv7_last_error() or L.rwkv7_status_string(rc)).decode())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def make_config(shape) -> Config:
    """rwkv7_config from any object with the RWKV-7 dimension attributes."""
    return Config(shape.n_layer, shape.n_embd, shape.n_head, shape.head_size, shape.ffn,
                  shape.d_w, shape.d_a, shape.d_v, shape.d_g, shape.vocab)


# ------------------------------------------------------------------ sizes
def rwkv7_packed_bytes(cfg: Config) -> int:
    v = ctypes.c_uint64()
    _check(lib().rwkv7_packed_bytes(ctypes.byref(cfg), ctypes.byref(v)), "rwkv7_packed_bytes")
    return v.value


def rwkv7_slot_floats(cfg: Config) -> int:
    v = ctypes.c_uint64()
    _check(lib().rwkv7_slot_floats(ctypes.byref(cfg), ctypes.byref(v)), "rwkv7_slot_floats")
    return v.value


def rwkv7_state_bytes(cfg: Config, n_slots: int) -> Tuple[int, int]:
    v, off = ctypes.c_uint64(), ctypes.c_uint64()
    _check(lib().rwkv7_state_bytes(ctypes.byref(cfg), n_slots, ctypes.byref(v), ctypes.byref(off)),
           "rwkv7_state_bytes")
    return v.value, off.value


def rwkv7_workspace_bytes(cfg: Config, max_B: int, max_T: int) -> int:
    v = ctypes.c_uint64()
    _check(lib().rwkv7_workspace_bytes(ctypes.byref(cfg), max_B, max_T, ctypes.byref(v)),
           "rwkv7_workspace_bytes")
    return v.value


def rwkv7_greedy_workspace_bytes(B: int, V: int) -> int:
    v = ctypes.c_uint64()
    _check(lib().rwkv7_greedy_workspace_bytes(B, V, ctypes.byref(v)), "rwkv7_greedy_workspace_bytes")
    return v.value


# ------------------------------------------------------------------ model
def rwkv7_load(cfg: Config, tensors: Dict[str, "object"], packed, stream=None) -> int:
    """Pack device tensors (name -> torch tensor, fp16 or fp32) into ``packed`` (uint8)."""
    import torch
    arr = (Tensor * len(tensors))()
    keep = []
    for i, (name, t) in enumerate(tensors.items()):
        if not t.is_contiguous():
            t = t.contiguous()
        keep.append(t)
        if t.dtype == torch.float16:
            dt = F16
        elif t.dtype == torch.float32:
            dt = F32
        else:
            raise TypeError(f"{name}: dtype {t.dtype} is not float16/float32")
        nm = name.encode()
        keep.append(nm)
        arr[i].name = nm
        arr[i].dtype = dt
        arr[i].ndim = t.dim()
        for k in range(t.dim()):
            arr[i].shape[k] = t.shape[k]
        arr[i].data = t.data_ptr()
    h = ctypes.c_void_p()
    _check(lib().rwkv7_load(ctypes.byref(cfg), arr, len(tensors), packed.data_ptr(), packed.numel(),
                            _stream(stream), ctypes.byref(h)), "rwkv7_load")
    return h.value


def rwkv7_free(model: int):
    _check(lib().rwkv7_free(model), "rwkv7_free")


def rwkv7_reset_slots(model: int, pool, n_slots: int, slot_idx, ws, stream=None):
    _check(lib().rwkv7_reset_slots(model, pool.data_ptr(), n_slots, _ptr(slot_idx), slot_idx.numel(),
                                   ws.data_ptr(), ws.numel(), _stream(stream)), "rwkv7_reset_slots")


def rwkv7_decode_step(model: int, pool, n_slots: int, slot_idx, token_ids, logits_out, ws,
                      stream=None):
    _check(lib().rwkv7_decode_step(model, pool.data_ptr(), n_slots, slot_idx.numel(),
                                   _ptr(slot_idx), _ptr(token_ids), _ptr(logits_out),
                                   ws.data_ptr(), ws.numel(), _stream(stream)), "rwkv7_decode_step")


def rwkv7_prefill_seq(model: int, pool, n_slots: int, slot: int, token_ids, ws, stream=None):
    _check(lib().rwkv7_prefill_seq(model, pool.data_ptr(), n_slots, slot, _ptr(token_ids),
                                   token_ids.numel(), ws.data_ptr(), ws.numel(), _stream(stream)),
           "rwkv7_prefill_seq")


def rwkv7_greedy(logits, occ_pool, n_slots: int, slot_idx, presence, frequency, decay, ids_out,
                 ws, stream=None):
    B, V = logits.shape
    _check(lib().rwkv7_greedy(B, V, _ptr(logits), _ptr(occ_pool), n_slots, _ptr(slot_idx),
                              _ptr(presence), _ptr(frequency), _ptr(decay), _ptr(ids_out),
                              ws.data_ptr(), ws.numel(), _stream(stream)), "rwkv7_greedy")


def rwkv7_greedy_noalloc(logits, occ_pool, n_slots: int, slot_idx, presence, frequency, decay, ids_out,
                         flags_out, stream=None):
    """rwkv7_greedy without a workspace (its partials in the library's static
    device array); device error bits are ORed into flags_out (uint32/int32 [1])."""
    B, V = logits.shape
    _check(lib().rwkv7_greedy_noalloc(B, V, _ptr(logits), _ptr(occ_pool), n_slots, _ptr(slot_idx),
                                      _ptr(presence), _ptr(frequency), _ptr(decay), _ptr(ids_out),
                                      _ptr(flags_out), _stream(stream)), "rwkv7_greedy_noalloc")


def rwkv7_sample_workspace_bytes(B: int, V: int) -> int:
    v = ctypes.c_uint64()
    _check(lib().rwkv7_sample_workspace_bytes(B, V, ctypes.byref(v)), "rwkv7_sample_workspace_bytes")
    return v.value


def rwkv7_sample(logits, occ_pool, n_slots: int, slot_idx, presence, frequency, decay, temperature,
                 top_p, top_k, forbidden, uniform, ids_out, ws, stream=None):
    """Penalised temperature / top-k / top-p sampling (see include/rwkv7.h).
    forbidden: uint8 [V] tensor or None; ws: a uint8 tensor of
    rwkv7_sample_workspace_bytes(B, V) bytes (its first word is an error word)."""
    B, V = logits.shape
    _check(lib().rwkv7_sample(B, V, _ptr(logits), _ptr(occ_pool), n_slots, _ptr(slot_idx),
                              _ptr(presence), _ptr(frequency), _ptr(decay), _ptr(temperature),
                              _ptr(top_p), _ptr(top_k), None if forbidden is None else _ptr(forbidden),
                              _ptr(uniform), _ptr(ids_out), ws.data_ptr(), ws.numel(), _stream(stream)),
           "rwkv7_sample")


def rwkv7_poll_error(ws, stream=None) -> int:
    """Synchronise, return and clear the device error bits (0 = none)."""
    f = ctypes.c_uint32()
    rc = lib().rwkv7_poll_error(ws.data_ptr(), _stream(stream), ctypes.byref(f))
    if rc not in (RWKV7_OK, RWKV7_EDEVICE):
        _check(rc, "rwkv7_poll_error")
    return f.value


def rwkv7_set_option(model: int, key: int, value: int):
    _check(lib().rwkv7_set_option(model, key, value), "rwkv7_set_option")


def rwkv7_get_option(model: int, key: int) -> int:
    v = ctypes.c_int64()
    _check(lib().rwkv7_get_option(model, key, ctypes.byref(v)), "rwkv7_get_option")
    return v.value


def rwkv7_kernel_timing(model: int, cls: int, reset: bool = False) -> Tuple[float, int]:
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(lib().rwkv7_kernel_timing(model, cls, ctypes.byref(ms), ctypes.byref(n), int(reset)),
           "rwkv7_kernel_timing")
    return ms.value, n.value


def rwkv7_kernel_name(model: int, cls: int, B: int) -> str:
    return lib().rwkv7_kernel_name(model, cls, B).decode()


def rwkv7_time_kernel(model: int, pool, n_slots: int, slot_idx, token_ids, logits_out,
                      kernel_class: int, layer: int, iters: int, ws, stream=None) -> float:
    """Average ms per launch of one kernel class at ``layer``, replayed ``iters`` times
    (``layer`` -1: swept over every layer ``iters`` times)."""
    v = ctypes.c_double()
    _check(lib().rwkv7_time_kernel(model, pool.data_ptr(), n_slots, slot_idx.numel(),
                                   _ptr(slot_idx), _ptr(token_ids), _ptr(logits_out), kernel_class,
                                   layer, iters, ws.data_ptr(), ws.numel(), _stream(stream),
                                   ctypes.byref(v)), "rwkv7_time_kernel")
    return v.value


def rwkv7_debug_cmix_buffers(model: int, ws, B: int) -> Tuple[int, int, int, int]:
    """Device addresses (pre, mask, active, active_count) inside ``ws``."""
    out = [ctypes.c_void_p() for _ in range(4)]
    _check(lib().rwkv7_debug_cmix_buffers(model, ws.data_ptr(), B, *[ctypes.byref(o) for o in out]),
           "rwkv7_debug_cmix_buffers")
    return tuple(o.value for o in out)


def rwkv7_read_bandwidth(buf, nontemporal: bool = True, iters: int = 5, stream=None) -> float:
    """GB/s of a plain streaming read of the device tensor ``buf``."""
    v = ctypes.c_double()
    _check(lib().rwkv7_read_bandwidth(buf.data_ptr(), buf.numel() * buf.element_size(), int(nontemporal), iters,
                                      _stream(stream), ctypes.byref(v)), "rwkv7_read_bandwidth")
    return v.value


def rwkv7_debug_wkv_out(model: int, ws, B: int) -> Tuple[int, bool]:
    """(device address inside ``ws`` of the last layer's time-mix output
    before W_o, [B][C], whether it is fp16)."""
    out, f16 = ctypes.c_void_p(), ctypes.c_int32()
    _check(lib().rwkv7_debug_wkv_out(model, ws.data_ptr(), B, ctypes.byref(out), ctypes.byref(f16)),
           "rwkv7_debug_wkv_out")
    return out.value, bool(f16.value)


# ------------------------------------------------------------------ scheduler
def sched_backend(reset, prefill, step) -> SchedBackend:
    """A backend whose callbacks are Python callables (used by host-logic tests):
    reset(slot); prefill(slot, tokens: list); step(slots, tokens, n_sample, params) -> ids,
    where params maps temperature/top_p/top_k/presence/frequency/decay/uniform to lists of
    n_sample values.  A callable that raises makes the round fail with RWKV7_EINVAL.
    The returned structure holds the C callbacks: keep it alive while a
    scheduler created over it is in use."""
    names = ("temperature", "top_p", "top_k", "presence", "frequency", "decay", "uniform")

    def c_reset(_ctx, slot):
        try:
            reset(slot)
            return RWKV7_OK
        except Exception:
            return RWKV7_EINVAL

    def c_prefill(_ctx, slot, toks, T):
        try:
            prefill(slot, toks[:T])
            return RWKV7_OK
        except Exception:
            return RWKV7_EINVAL

    def c_step(_ctx, bp, ids):
        try:
            b = bp.contents
            S = b.n_sample
            params = {n: getattr(b, n)[:S] for n in names}
            out = step(b.slots[:b.B], b.tokens[:b.B], S, params)
            for i in range(S):
                ids[i] = int(out[i])
            return RWKV7_OK
        except Exception:
            return RWKV7_EINVAL

    be = SchedBackend(None, RESET_FN(c_reset), PREFILL_FN(c_prefill), STEP_FN(c_step))
    be._keep = (be.reset, be.prefill, be.step)
    return be


def rwkv7_sched_create(cfg: SchedConfig, backend: SchedBackend) -> int:
    h = ctypes.c_void_p()
    _check(lib().rwkv7_sched_create(ctypes.byref(cfg), ctypes.byref(backend), ctypes.byref(h)),
           "rwkv7_sched_create")
    return h.value


def rwkv7_sched_free(s: int):
    _check(lib().rwkv7_sched_free(s), "rwkv7_sched_free")


def rwkv7_sched_submit(s: int, prompt, params: SchedParams) -> int:
    n = len(prompt)
    arr = (ctypes.c_int32 * max(n, 1))(*[int(x) for x in prompt])
    tid = ctypes.c_int64()
    _check(lib().rwkv7_sched_submit(s, arr, n, ctypes.byref(params), ctypes.byref(tid)), "rwkv7_sched_submit")
    return tid.value


def rwkv7_sched_abort(s: int, task_id: int):
    _check(lib().rwkv7_sched_abort(s, task_id), "rwkv7_sched_abort")


def rwkv7_sched_step(s: int) -> SchedStats:
    st = SchedStats()
    _check(lib().rwkv7_sched_step(s, ctypes.byref(st)), "rwkv7_sched_step")
    return st


def rwkv7_sched_poll(s: int, cap: int = 4096):
    """Pending events, oldest first, as (task, kind, value, index) tuples."""
    buf = (SchedEvent * cap)()
    n = ctypes.c_int32()
    _check(lib().rwkv7_sched_poll(s, buf, cap, ctypes.byref(n)), "rwkv7_sched_poll")
    return [(e.task, e.kind, e.value, e.index) for e in buf[:n.value]]


def rwkv7_sched_task_state(s: int, task_id: int) -> int:
    v = ctypes.c_int32()
    _check(lib().rwkv7_sched_task_state(s, task_id, ctypes.byref(v)), "rwkv7_sched_task_state")
    return v.value


def rwkv7_sched_gpu_backend_bytes(model: int, max_B: int, max_T: int) -> Tuple[int, int]:
    """(device bytes, pinned host bytes) of the GPU backend's staging."""
    d, h = ctypes.c_uint64(), ctypes.c_uint64()
    _check(lib().rwkv7_sched_gpu_backend_bytes(model, max_B, max_T, ctypes.byref(d), ctypes.byref(h)),
           "rwkv7_sched_gpu_backend_bytes")
    return d.value, h.value


def rwkv7_sched_gpu_backend(model: int, pool, n_slots: int, occ_pool, forbidden, max_B: int, ws, sample_ws,
                            max_T: int, dev_buf=None, host_buf=None, stream=None) -> SchedBackend:
    """The GPU backend over caller-owned staging.  dev_buf / host_buf (uint8
    tensors, device and pinned host) default to torch allocations of the sizes
    rwkv7_sched_gpu_backend_bytes gives; the returned record keeps them alive."""
    import torch
    if dev_buf is None or host_buf is None:
        nd, nh = rwkv7_sched_gpu_backend_bytes(model, max_B, max_T)
        if dev_buf is None:
            dev_buf = torch.empty(nd, dtype=torch.uint8, device=pool.device)
        if host_buf is None:
            host_buf = torch.empty(nh, dtype=torch.uint8, pin_memory=True)
    be = SchedBackend()
    _check(lib().rwkv7_sched_gpu_backend(model, pool.data_ptr(), n_slots, _ptr(occ_pool), _ptr(forbidden),
                                         max_B, max_T, ws.data_ptr(), ws.numel(), sample_ws.data_ptr(),
                                         sample_ws.numel(), dev_buf.data_ptr(), dev_buf.numel(),
                                         host_buf.data_ptr(), host_buf.numel(), _stream(stream),
                                         ctypes.byref(be)),
           "rwkv7_sched_gpu_backend")
    be.buffers = (dev_buf, host_buf)
    return be


def rwkv7_sched_gpu_backend_free(backend: SchedBackend):
    _check(lib().rwkv7_sched_gpu_backend_free(ctypes.byref(backend)), "rwkv7_sched_gpu_backend_free")


def rwkv7_sched_gpu_backend_set_cache(backend: SchedBackend, cache: Optional[int]):
    _check(lib().rwkv7_sched_gpu_backend_set_cache(ctypes.byref(backend), cache), "rwkv7_sched_gpu_backend_set_cache")


def rwkv7_sched_gpu_backend_counts(backend: SchedBackend) -> Tuple[int, int]:
    """(tokens restored from the prefix cache, tokens prefilled) so far."""
    a, b = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().rwkv7_sched_gpu_backend_counts(ctypes.byref(backend), ctypes.byref(a), ctypes.byref(b)),
           "rwkv7_sched_gpu_backend_counts")
    return a.value, b.value


# ------------------------------------------------------------------ int8 weights
def rwkv7_int8_bytes(cfg: Config) -> int:
    v = ctypes.c_uint64()
    _check(lib().rwkv7_int8_bytes(ctypes.byref(cfg), ctypes.byref(v)), "rwkv7_int8_bytes")
    return v.value


def rwkv7_quantize_int8(model: int, buf, stream=None):
    """Fill ``buf`` (a device uint8 tensor of rwkv7_int8_bytes) with the int8 copies."""
    _check(lib().rwkv7_quantize_int8(model, buf.data_ptr(), buf.numel(), _stream(stream)), "rwkv7_quantize_int8")


def rwkv7_debug_int8_matrix(model: int, layer: int, which: int) -> Tuple[int, int, int, int]:
    """(codes address, scales address, rows, K) of one int8 matrix."""
    c, s_, r, k = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_int64(), ctypes.c_int32()
    _check(lib().rwkv7_debug_int8_matrix(model, layer, which, ctypes.byref(c), ctypes.byref(s_), ctypes.byref(r),
                                         ctypes.byref(k)), "rwkv7_debug_int8_matrix")
    return c.value, s_.value, r.value, k.value


# ------------------------------------------------------------------ snapshots, prefix cache
def rwkv7_snapshot_bytes(cfg: Config) -> int:
    v = ctypes.c_uint64()
    _check(lib().rwkv7_snapshot_bytes(ctypes.byref(cfg), ctypes.byref(v)), "rwkv7_snapshot_bytes")
    return v.value


def rwkv7_slot_export(model: int, pool, n_slots: int, slot: int, dst, stream=None):
    """Copy one slot (state, then its int64 step counter) into dst (a uint8 tensor, device or pinned host)."""
    _check(lib().rwkv7_slot_export(model, pool.data_ptr(), n_slots, slot, dst.data_ptr(), _stream(stream)),
           "rwkv7_slot_export")


def rwkv7_slot_import(model: int, pool, n_slots: int, slot: int, src, stream=None):
    _check(lib().rwkv7_slot_import(model, pool.data_ptr(), n_slots, slot, src.data_ptr(), _stream(stream)),
           "rwkv7_slot_import")


def rwkv7_prefix_cache_create(model: int, arena, host_arena=None) -> int:
    """A prefix-state cache over a device uint8 tensor and an optional pinned host one."""
    h = ctypes.c_void_p()
    _check(lib().rwkv7_prefix_cache_create(model, arena.data_ptr(), arena.numel(), _ptr(host_arena),
                                           0 if host_arena is None else host_arena.numel(), ctypes.byref(h)),
           "rwkv7_prefix_cache_create")
    return h.value


def rwkv7_prefix_cache_free(cache: int):
    _check(lib().rwkv7_prefix_cache_free(cache), "rwkv7_prefix_cache_free")


def _tok_array(tokens):
    n = len(tokens)
    return (ctypes.c_int32 * max(n, 1))(*[int(x) for x in tokens]), n


def rwkv7_prefix_cache_store(cache: int, pool, n_slots: int, slot: int, tokens, stream=None):
    arr, n = _tok_array(tokens)
    _check(lib().rwkv7_prefix_cache_store(cache, pool.data_ptr(), n_slots, slot, arr, n, _stream(stream)),
           "rwkv7_prefix_cache_store")


def rwkv7_prefix_cache_lookup(cache: int, pool, n_slots: int, slot: int, tokens, stream=None) -> int:
    """Restore the longest cached prefix of tokens into the slot; its length (0: none)."""
    arr, n = _tok_array(tokens)
    m = ctypes.c_int32()
    _check(lib().rwkv7_prefix_cache_lookup(cache, pool.data_ptr(), n_slots, slot, arr, n, ctypes.byref(m),
                                           _stream(stream)), "rwkv7_prefix_cache_lookup")
    return m.value


def rwkv7_prefix_cache_stats(cache: int) -> PrefixStats:
    st = PrefixStats()
    _check(lib().rwkv7_prefix_cache_stats(cache, ctypes.byref(st)), "rwkv7_prefix_cache_stats")
    return st


# ------------------------------------------------------------------ holder
class Model:
    """Packed weights + state pool + workspace on one device, allocated by torch."""

    def __init__(self, cfg: Config, tensors: Dict[str, "object"], n_slots: int, max_B: int,
                 max_T: int = 512, device: str = "cuda:0"):
        import torch
        self.cfg = cfg
        self.device = torch.device(device)
        self.n_slots = n_slots
        self.max_B, self.max_T = max_B, max_T
        self.packed = torch.empty(rwkv7_packed_bytes(cfg), dtype=torch.uint8, device=self.device)
        self.handle = rwkv7_load(cfg, tensors, self.packed)
        nbytes, self.counter_offset = rwkv7_state_bytes(cfg, n_slots)
        self.pool = torch.zeros(nbytes, dtype=torch.uint8, device=self.device)
        self.slot_floats = rwkv7_slot_floats(cfg)
        self.ws = torch.zeros(rwkv7_workspace_bytes(cfg, max_B, max_T), dtype=torch.uint8,
                              device=self.device)
        torch.cuda.synchronize(self.device)

    @classmethod
    def from_numpy(cls, shape, weights: Dict[str, "object"], n_slots: int, max_B: int,
                   max_T: int = 512, device: str = "cuda:0") -> "Model":
        """Upload host arrays (name -> numpy fp16/fp32) and pack them; the
        uploaded copies are freed once packing has finished."""
        import torch
        dev = torch.device(device)
        t = {k: torch.from_numpy(v).to(dev) for k, v in weights.items()}
        m = cls(make_config(shape), t, n_slots, max_B, max_T, device)
        del t
        torch.cuda.synchronize(dev)
        return m

    # views of the pool
    def slot_state(self, slot: int):
        """fp32 view of one slot: [n_layer, 2C + H*64*64]."""
        import torch
        f = self.pool[: self.counter_offset].view(torch.float32)
        n = self.slot_floats
        return f[slot * n:(slot + 1) * n].view(self.cfg.n_layer, -1)

    def counters(self):
        import torch
        return self.pool[self.counter_offset: self.counter_offset + 8 * self.n_slots].view(torch.int64)

    def reset(self, slots):
        rwkv7_reset_slots(self.handle, self.pool, self.n_slots, slots, self.ws)

    def decode_step(self, slot_idx, token_ids, logits_out):
        rwkv7_decode_step(self.handle, self.pool, self.n_slots, slot_idx, token_ids, logits_out, self.ws)

    def prefill(self, slot: int, token_ids):
        rwkv7_prefill_seq(self.handle, self.pool, self.n_slots, slot, token_ids, self.ws)

    def greedy(self, logits, occ_pool, slot_idx, presence, frequency, decay, ids_out):
        rwkv7_greedy(logits, occ_pool, self.n_slots, slot_idx, presence, frequency, decay, ids_out,
                     self.ws)

    def poll_error(self) -> int:
        return rwkv7_poll_error(self.ws)

    def set_option(self, key: int, value: int):
        rwkv7_set_option(self.handle, key, value)

    def close(self):
        if getattr(self, "handle", None):
            rwkv7_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
