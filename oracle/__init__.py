"""fp64 CPU oracle (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or run anything here. The product path never
does: it has no CPU fallback.
"""
