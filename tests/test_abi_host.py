"""C-ABI checks that need no GPU: the library loads, exports every function
include/*.h declares, and rejects host-checkable misuse synchronously."""
import ctypes
import glob
import os
import re

import pytest

import rwkv_linear_attention_decode_amd as R
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        txt = open(h).read()
        names |= set(re.findall(r"^(?:int|const char\*)\s+(rwkv7_\w+)\s*\(", txt, flags=re.M))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    L = R.lib()
    declared = _declared()
    assert len(declared) >= 18
    missing = [n for n in declared if not hasattr(L, n)]
    assert not missing, missing


def test_binding_wraps_every_symbol():
    for n in _declared():
        if n in ("rwkv7_status_string", "rwkv7_last_error"):
            continue
        assert hasattr(R, n), n


def test_sizes_tiny():
    cfg = R.make_config(synth.TINY)
    s = synth.TINY
    sf = R.rwkv7_slot_floats(cfg)
    assert sf == s.n_layer * (2 * s.n_embd + s.n_head * 64 * 64)
    nbytes, off = R.rwkv7_state_bytes(cfg, 3)
    assert off >= 3 * sf * 4 and off % 256 == 0 and nbytes >= off + 3 * 8
    assert R.rwkv7_packed_bytes(cfg) > 2 * s.vocab * s.n_embd * 2
    ws1 = R.rwkv7_workspace_bytes(cfg, 1, 1)
    ws8 = R.rwkv7_workspace_bytes(cfg, 8, 1)
    assert ws8 > ws1 > 0


def test_sizes_2b9_fit_hbm():
    cfg = R.make_config(synth.R7_2B9)
    assert R.rwkv7_packed_bytes(cfg) < 8 << 30
    nbytes, _ = R.rwkv7_state_bytes(cfg, 256)
    assert abs(nbytes / 256 - 21.63e6) / 21.63e6 < 0.01   # 21.63 MB fp32 state per slot


@pytest.mark.parametrize("field,value,code", [
    ("head_size", 32, R.RWKV7_ENOTSUP),
    ("n_embd", 250, R.RWKV7_ESHAPE),
    ("ffn", 1000, R.RWKV7_ENOTSUP),
    ("d_v", 12, R.RWKV7_ENOTSUP),
    ("n_layer", 0, R.RWKV7_ESHAPE),
])
def test_bad_config_rejected(field, value, code):
    cfg = R.make_config(synth.TINY)
    setattr(cfg, field, value)
    with pytest.raises(R.RWKV7Error) as ei:
        R.rwkv7_packed_bytes(cfg)
    assert ei.value.status == code


def test_null_and_range_checks_without_device():
    L = R.lib()
    u = ctypes.c_uint64()
    assert L.rwkv7_packed_bytes(None, ctypes.byref(u)) == R.RWKV7_EINVAL
    assert L.rwkv7_decode_step(None, None, 1, 1, None, None, None, None, 0, None) == R.RWKV7_EINVAL
    assert L.rwkv7_prefill_seq(None, None, 1, 0, None, 4, None, 0, None) == R.RWKV7_EINVAL
    assert L.rwkv7_greedy(0, 10, None, None, 1, None, None, None, None, None, None, 0, None) == R.RWKV7_EINVAL
    assert L.rwkv7_greedy_workspace_bytes(0, 5, ctypes.byref(u)) == R.RWKV7_EINVAL
    assert L.rwkv7_poll_error(None, None, None) == R.RWKV7_EINVAL
    assert L.rwkv7_set_option(None, 1, 1) == R.RWKV7_EINVAL
    assert L.rwkv7_set_option(None, R.OPT_LN_SPLIT, 2) == R.RWKV7_EINVAL
    d = ctypes.c_double()
    assert L.rwkv7_read_bandwidth(None, 1 << 20, 1, 1, None, ctypes.byref(d)) == R.RWKV7_EINVAL
    buf = ctypes.create_string_buffer(64)
    assert L.rwkv7_read_bandwidth(buf, 8, 1, 1, None, ctypes.byref(d)) == R.RWKV7_EINVAL   # under 16 bytes
    assert L.rwkv7_read_bandwidth(buf, 64, 1, 0, None, ctypes.byref(d)) == R.RWKV7_EINVAL  # no iterations
    assert L.rwkv7_greedy_noalloc(0, 10, None, None, 1, None, None, None, None, None, None, None) == R.RWKV7_EINVAL
    # beyond the static scratch: rejected on the host, before any pointer is used
    assert L.rwkv7_greedy_noalloc(257, 65536, buf, buf, 1, buf, buf, buf, buf, buf, buf, None) == R.RWKV7_ESHAPE
    u2 = ctypes.c_uint64()
    assert L.rwkv7_sched_gpu_backend_bytes(None, 4, 16, ctypes.byref(u), ctypes.byref(u2)) == R.RWKV7_EINVAL
    cfg = R.make_config(synth.TINY)
    assert L.rwkv7_workspace_bytes(ctypes.byref(cfg), 0, 1, ctypes.byref(u)) == R.RWKV7_EINVAL
    assert L.rwkv7_state_bytes(ctypes.byref(cfg), 0, ctypes.byref(u), None) == R.RWKV7_EINVAL
    assert b"n_slots" in L.rwkv7_last_error()
    assert L.rwkv7_status_string(R.RWKV7_ESHAPE) == b"wrong shape or size"


def test_load_rejects_bad_tables_before_touching_memory():
    """Table validation (names, shapes, dtypes) happens before any launch."""
    L = R.lib()
    cfg = R.make_config(synth.TINY)
    h = ctypes.c_void_p()
    arr = (R.Tensor * 1)()
    arr[0].name = b"emb.weight"
    arr[0].dtype = R.F32
    arr[0].ndim = 2
    arr[0].shape[0], arr[0].shape[1] = 1024, 256
    arr[0].data = 0x1000
    # packed buffer too small
    assert L.rwkv7_load(ctypes.byref(cfg), arr, 1, ctypes.c_void_p(0x1000), 16, None, ctypes.byref(h)) == R.RWKV7_ESHAPE
    big = R.rwkv7_packed_bytes(cfg)
    rc = L.rwkv7_load(ctypes.byref(cfg), arr, 1, ctypes.c_void_p(0x1000), big, None, ctypes.byref(h))
    assert rc == R.RWKV7_EINVAL and b"missing tensor" in L.rwkv7_last_error()
    arr[0].shape[1] = 255
    rc = L.rwkv7_load(ctypes.byref(cfg), arr, 1, ctypes.c_void_p(0x1000), big, None, ctypes.byref(h))
    assert rc in (R.RWKV7_EINVAL, R.RWKV7_ESHAPE)
    assert h.value is None


def test_snapshot_bytes_formula():
    cfg = R.make_config(synth.TINY)
    assert R.rwkv7_snapshot_bytes(cfg) == R.rwkv7_slot_floats(cfg) * 4 + 8
    cfg = R.make_config(synth.R7_2B9)
    assert R.rwkv7_snapshot_bytes(cfg) == 32 * (2 * 2560 + 40 * 64 * 64) * 4 + 8
