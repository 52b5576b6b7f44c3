"""RouteRelay event-triggered cross-layer routing on MI355X (gfx950).

The routing pass runs in hand-written HIP kernels behind the C ABI declared in
``include/rr.h`` (library ``librr.so``); ``rr`` is a thin ctypes binding with the
same entry points.  ``workloads`` and ``synth`` describe and generate the
seeded synthetic inputs.  Importing this package loads nothing native; the
binding loads ``librr.so`` on first use and raises if it is missing.
"""
