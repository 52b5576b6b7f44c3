"""CPU oracle for the RouteRelay routing pass — TEST INFRASTRUCTURE, NOT PRODUCT CODE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run anything in this package.  The GPU library never
calls it, shares no code with it, and must fail loudly when its HIP extension is
missing rather than fall back to anything here.

It is plain NumPy, row by row, in the page's own order of steps ("RouteRelay:
Event-Triggered Cross-Layer Route Reuse for Efficient Dynamic Sparse
Attention", Sections 2.1, 3.1-3.5, 4.1-4.2, 5).  Every function is pinned by
``tests/test_oracle_*.py`` against brute force, closed forms, invariants and
the page's printed tables; see each test's docstring for the pin it provides.
"""
from .attention import sparse_attention  # noqa: F401
from .philox import philox4x32_10, philox4x64_10  # noqa: F401
from .routing import (  # noqa: F401
    Ledger, LayerRecord, RelayResult, RouteConfig, anchor_layer, decode, exact_routes,
    ledger_bytes, mandatory_sentinels, n_allowed, pair_counts, preference_order, query_rows,
    random_sentinels, rebuild_row, relay_decision, relay_gap, relay_layer, relay_layer_rows, reroute_fraction,
    route_recall, run_chain, score_rows, select, selection_gap, SAMPLER_DRAW_CAP,
)
