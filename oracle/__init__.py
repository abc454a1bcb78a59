"""ORACLE: test infrastructure only (see oracle/rwkv7.py).

Imported by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg,
never by the product path.
"""
from . import rwkv7  # noqa: F401
