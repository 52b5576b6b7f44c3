"""GPU parity: the C-ABI HIP path against the oracle, element by element.

Every test prints the case it is about to run (flushed) before touching the GPU.
"""
import numpy as np
import pytest

import oracle as O
from long_context_prefill_anchor_amd import rr, synth, workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rr.lib()
    yield


def make(heads, nq, nk, k=12, m=12, r=8, dtype="bf16", causal=False, seed=0, gamma=0.0,
         sink=0, recent=0):
    led = rr.Ledger(heads, nq, nk, 64, k, m, r, gamma, causal, dtype, seed, sink=sink, recent=recent)
    return led, U.oracle_cfg(led, dtype, gamma, causal, seed)


ANCHOR_CASES = [
    # name, heads, nq, nk, k, m, r, dtype, causal, seed, input kind
    ("tiny_f32", 1, 128, 128, 12, 12, 8, "f32", False, 0, "gauss"),
    ("ragged_f32", 3, 100, 77, 12, 12, 8, "f32", False, 1, "gauss"),
    ("bf16_256", 2, 256, 256, 12, 12, 8, "bf16", False, 2, "gauss"),
    ("bf16_ragged", 2, 130, 301, 12, 12, 8, "bf16", False, 3, "gauss"),
    ("causal_bf16", 2, 200, 200, 12, 12, 8, "bf16", True, 4, "gauss"),
    ("causal_f32", 1, 97, 97, 12, 12, 8, "f32", True, 5, "gauss"),
    ("comparator_m0r0", 2, 256, 256, 12, 0, 0, "bf16", False, 6, "gauss"),
    ("k1_only", 1, 70, 64, 1, 0, 0, "f32", False, 7, "gauss"),
    ("small_widths", 2, 65, 40, 4, 3, 5, "bf16", False, 8, "gauss"),
    ("nk_below_k", 1, 33, 5, 12, 12, 8, "f32", False, 9, "gauss"),
    ("wide_32", 1, 96, 512, 16, 16, 32, "bf16", False, 10, "gauss"),
    ("big_seed", 1, 64, 256, 12, 12, 8, "bf16", False, (1 << 63) + 12345, "gauss"),
    ("int_ties_f32", 2, 128, 128, 12, 12, 8, "f32", False, 11, "int"),
    ("int_ties_bf16_causal", 2, 150, 150, 12, 12, 8, "bf16", True, 12, "int"),
    ("int_ties_narrow", 1, 64, 200, 12, 12, 8, "f32", False, 13, "int1"),
    ("equal_keys", 2, 64, 100, 12, 12, 8, "f32", False, 14, "equal"),
    # long rows: 8192 and 16384 key chunks (1M / 2M tokens in 128-token chunks), one route
    # block per compute unit (the sentinel bitmaps fill the LDS)
    ("long_keys_bf16", 1, 96, 16384, 12, 12, 8, "bf16", False, 15, "gauss"),
    ("long_keys_f32", 1, 64, 8192, 12, 12, 8, "f32", False, 16, "gauss"),
]


def inputs(kind, heads, nq, nk, dtype, seed):
    if kind == "gauss":
        return synth.gaussian_inputs(heads, nq, nk, 64, seed=seed, dtype=dtype)
    if kind in ("int", "int1"):
        lo, hi = (-2, 2) if kind == "int" else (-1, 1)
        q, _ = synth.integer_inputs(heads, nq, 64, seed=seed, lo=lo, hi=hi, dtype=dtype)
        _, k = synth.integer_inputs(heads, nk, 64, seed=seed + 1, lo=lo, hi=hi, dtype=dtype)
        return q, k
    if kind == "equal":
        q, k = synth.gaussian_inputs(heads, nq, 1, 64, seed=seed, dtype=dtype)
        return q, np.ascontiguousarray(np.repeat(k, nk, axis=1))
    raise ValueError(kind)


# Mandatory sink / recent sentinels (Section 3.1, item 3): name, heads, nq, nk, k, m, r, sink,
# recent, dtype, causal, seed, input kind
MAND_ANCHOR_CASES = [
    ("mand_f32", 2, 100, 77, 8, 8, 8, 2, 2, "f32", False, 20, "gauss"),
    ("mand_bf16_causal", 2, 200, 200, 12, 12, 4, 2, 2, "bf16", True, 21, "gauss"),
    ("mand_int_ties", 1, 128, 128, 12, 12, 4, 1, 3, "f32", False, 22, "int"),
    ("mand_c64", 1, 96, 512, 12, 12, 24, 8, 8, "bf16", False, 23, "gauss"),
    ("mand_only", 1, 64, 100, 12, 0, 0, 4, 4, "f32", False, 24, "gauss"),
    ("mand_tiny_pool", 1, 40, 10, 4, 2, 2, 3, 3, "f32", False, 25, "gauss"),
    ("mand_equal_keys", 1, 64, 100, 12, 12, 8, 2, 2, "f32", False, 26, "equal"),
]
ANCHOR_CASES_ALL = ([c[:7] + (0, 0) + c[7:] for c in ANCHOR_CASES] + MAND_ANCHOR_CASES)


@pytest.mark.parametrize("case", ANCHOR_CASES_ALL, ids=[c[0] for c in ANCHOR_CASES_ALL])
def test_anchor_parity(case):
    name, H, nq, nk, k, m, r, sink, recent, dtype, causal, seed, kind = case
    U.log(f"[anchor] {name} H={H} nq={nq} nk={nk} k={k} m={m} r={r} sink={sink} recent={recent} "
          f"{dtype} causal={causal}")
    led, cfg = make(H, nq, nk, k, m, r, dtype, causal, seed, sink=sink, recent=recent)
    q, kk = inputs(kind, H, nq, nk, dtype, seed)
    tol = 0.0 if kind != "gauss" else U.GAP_TOL
    rep = U.Report()
    U.anchor_parity(led, cfg, q, kk, 3, tol, rep)
    U.log(f"   rows={rep.rows} excluded={rep.excluded}")
    if kind != "gauss":
        assert rep.excluded == 0
    assert rep.excluded <= max(2, rep.rows // 200)
    led.close()


RELAY_CASES = [
    ("relay_f32", 2, 128, 128, 12, 12, 8, "f32", False, 0.05, "gauss"),
    ("relay_bf16", 2, 256, 256, 12, 12, 8, "bf16", False, 0.03, "gauss"),
    ("relay_ragged", 3, 100, 130, 12, 12, 8, "bf16", False, 0.05, "gauss"),
    ("relay_causal", 2, 180, 180, 12, 12, 8, "bf16", True, 0.04, "gauss"),
    ("relay_small", 1, 70, 50, 4, 3, 5, "f32", False, 0.1, "gauss"),
    ("relay_int", 2, 128, 160, 12, 12, 8, "f32", False, 0.0, "int"),
    ("relay_int_causal", 1, 140, 140, 12, 12, 8, "bf16", True, 0.0, "int"),
    ("relay_guard", 2, 128, 256, 12, 12, 8, "bf16", False, 0.02, "gauss"),
    # c = 64 (two candidate passes)
    ("relay_wide64_bf16", 1, 96, 512, 16, 16, 32, "bf16", False, 0.05, "gauss"),
    ("relay_wide64_f32", 1, 70, 200, 16, 16, 32, "f32", False, 0.05, "gauss"),
    # more keys than the main workloads (1300-1500 bf16, 600 fp32)
    ("relay_gather_bf16", 2, 96, 1500, 12, 12, 8, "bf16", False, 0.05, "gauss"),
    ("relay_gather_f32", 1, 100, 600, 12, 12, 8, "f32", False, 0.05, "gauss"),
    ("relay_gather_wide", 1, 80, 1300, 16, 16, 32, "bf16", False, 0.05, "gauss"),
    # more than 64 rescore blocks per head (nq > 4096): the reroute finds its rows by scanning flags
    ("relay_many_rows", 1, 4160, 96, 12, 12, 8, "bf16", False, 0.05, "gauss"),
    # long rows (see the anchor cases)
    ("relay_long_keys_bf16", 1, 96, 16384, 12, 12, 8, "bf16", False, 0.05, "gauss"),
    ("relay_long_keys_f32", 1, 64, 8192, 12, 12, 8, "f32", False, 0.05, "gauss"),
]


# with mandatory sentinels: name, heads, nq, nk, k, m, r, sink, recent, dtype, causal, drift, kind
MAND_RELAY_CASES = [
    ("relay_mand_bf16", 2, 256, 256, 12, 12, 4, 2, 2, "bf16", False, 0.03, "gauss"),
    ("relay_mand_causal", 2, 180, 180, 12, 12, 4, 2, 2, "bf16", True, 0.04, "gauss"),
    ("relay_mand_int", 2, 128, 160, 12, 12, 4, 1, 3, "f32", False, 0.0, "int"),
    ("relay_mand_c64", 1, 96, 512, 12, 12, 24, 8, 8, "bf16", False, 0.05, "gauss"),
    ("relay_mand_only", 1, 70, 50, 4, 0, 0, 2, 2, "f32", False, 0.1, "gauss"),
    # 32-entry lists with a ledger past 64 IDs (c = 80): main kernels, two-chunk rescore
    ("relay_mand_c80", 1, 96, 300, 12, 20, 32, 8, 8, "bf16", False, 0.05, "gauss"),
]
RELAY_CASES_ALL = ([c[:7] + (0, 0) + c[7:] for c in RELAY_CASES] + MAND_RELAY_CASES)


RELAY_MODES = ["fused", "compacted"]


def fused_supported(led: rr.Ledger, dtype: str) -> bool:
    """The fused relay's documented limits (include/rr.h, rr_ledger_set_relay_mode): k + m <= 32,
    c <= 32, a head's keys in 128 KB."""
    return led.k + led.m <= 32 and led.c <= 32 and led.nk * (128 if dtype == "bf16" else 256) <= 128 * 1024


def require_mode(led: rr.Ledger, dtype: str, mode: str):
    """Skip a fused-mode case outside the fused relay's limits, after checking that the library
    refuses it."""
    if mode == "fused" and not fused_supported(led, dtype):
        with pytest.raises(rr.RRError) as e:
            led.set_relay_mode("fused")
        assert e.value.status == rr.RR_EUNSUPPORTED
        led.close()
        pytest.skip("outside the fused relay's limits (refused with RR_EUNSUPPORTED)")


@pytest.mark.parametrize("mode", RELAY_MODES)
@pytest.mark.parametrize("case", RELAY_CASES_ALL, ids=[c[0] for c in RELAY_CASES_ALL])
def test_relay_lockstep(case, mode):
    """Same ledger in (oracle anchor at layer 4, injected with rr_ledger_set), relay at layer 5,
    through the fused relay kernel and through the two-kernel compacted schedule."""
    name, H, nq, nk, k, m, r, sink, recent, dtype, causal, drift, kind = case
    gamma = 0.01 if name == "relay_guard" else 0.0
    U.log(f"[relay {mode}] {name} H={H} nq={nq} nk={nk} sink={sink} recent={recent} {dtype} causal={causal} "
          f"drift={drift} gamma={gamma}")
    led, cfg = make(H, nq, nk, k, m, r, dtype, causal, 21, gamma, sink=sink, recent=recent)
    require_mode(led, dtype, mode)
    q0, k0 = inputs(kind, H, nq, nk, dtype, 31)
    if kind == "int":
        qn, kn = inputs(kind, H, nq, nk, dtype, 32)
        # change every 4th query row and every 9th key row: most rows relay, some refresh
        q1, k1 = q0.copy(), k0.copy()
        q1[:, 1::4] = qn[:, 1::4]
        k1[:, ::9] = kn[:, ::9]
    else:
        q1 = synth.perturb(q0, drift / 8, seed=41, dtype=dtype)
        k1 = synth.perturb(k0, drift / 8, seed=42, dtype=dtype)
    ora0 = O.anchor_layer(cfg, q0, k0, 4)
    tol = 0.0 if kind != "gauss" else U.GAP_TOL
    rel = 1e-5 if dtype == "f32" else 1e-3
    rep = U.Report()
    gpu, res, ex = U.relay_parity(led, cfg, q1, k1, 5, ora0, tol, rel, rep, mode=mode)
    nflag = int(res.flags.sum())
    U.log(f"   rows={rep.rows} flagged={nflag} excluded={rep.excluded} max|ds|={rep.max_score_err:.2e}")
    assert 0 < nflag < H * nq
    if kind != "gauss":
        assert rep.excluded == 0
    led.close()


def run_chain_gpu_vs_oracle(w: W.Workload, heads=None, tol=U.GAP_TOL, mode="auto"):
    """Both sides run the whole chain on their own state; per-layer comparison with the
    exclusion rule (an excluded row stays excluded until the next anchor layer).
    ``rep.excluded`` counts exclusion events (a row newly excluded at a layer);
    ``rep.notes`` holds the number of rows under exclusion at each layer."""
    import torch
    H = w.heads if heads is None else heads
    nq = w.nq
    led = rr.Ledger(H, w.nq, w.nk, 64, w.k, w.m, w.r, w.gamma, w.causal, w.dtype, w.seed,
                    sink=w.sink, recent=w.recent, min_reuse=w.min_reuse, gamma_extra=w.gamma_extra)
    led.set_relay_mode(mode)
    cfg = U.oracle_cfg(led, w.dtype, w.gamma, w.causal, w.seed)
    rel = 1e-5 if w.dtype == "f32" else 1e-3
    rep = U.Report()
    ora_led = None
    ex = np.zeros((H, nq), bool)
    hs = slice(0, H) if heads is not None else None
    for li in synth.generate(w, hs):
        if ora_led is None or w.is_anchor(li.layer):
            gpu, ora_led = U.anchor_parity(led, cfg, li.q, li.k, li.layer, tol, rep)
            S = U.oracle_scores(cfg, li.q, li.k)
            ex = U.selection_excluded(cfg, S, tol)
            rep.notes.append(int(ex.sum()))
        else:
            prev_ex = int(ex.sum())
            out = led.alloc_outputs()
            led.relay(U.upload(li.q), U.upload(li.k), li.layer, out)
            torch.cuda.synchronize()
            gpu = U.ledger_np(led)
            res = O.relay_layer(cfg, li.q, li.k, li.layer, ora_led)
            g_flags = out.flags.cpu().numpy().reshape(H, nq)
            if tol > 0:
                for h in range(H):
                    for i in range(nq):
                        if U.relay_excluded(cfg, li.layer, ora_led, h, i, res.alpha[h, i],
                                            res.beta[h, i], tol):
                            ex[h, i] = True
                S = U.oracle_scores(cfg, li.q, li.k)
                for h, i in np.argwhere(res.flags == 1):
                    if O.selection_gap(S[h, i], O.n_allowed(i, cfg), cfg.k, cfg.m) < tol:
                        ex[h, i] = True
            mask = ~ex
            rep.rows += H * nq
            rep.excluded += int(ex.sum()) - prev_ex
            rep.notes.append(int(ex.sum()))
            assert np.array_equal(g_flags[mask], res.flags[mask]), f"{w.name} layer {li.layer}: flags"
            n_rows = int(out.n_rows.cpu().numpy()[0])
            g_rows = out.rows.cpu().numpy()[:n_rows]
            assert np.array_equal(g_rows, np.flatnonzero(g_flags.reshape(-1)))
            U.check_compaction(g_rows, out.head_counts.cpu().numpy(), g_flags, res, mask,
                               f"{w.name} relay layer {li.layer}")
            U.compare_ledgers(gpu, res.ledger, mask, f"{w.name} relay layer {li.layer}")
            ora_led = res.ledger
    led.close()
    return rep


def chain_report(rep):
    held = sum(rep.notes)
    U.log(f"   row-layers={rep.rows} exclusion events={rep.excluded} row-layers under exclusion={held}")
    assert rep.excluded <= max(2, rep.rows // 100)
    assert held <= max(4, rep.rows // 20)


@pytest.mark.parametrize("mode", RELAY_MODES)
def test_chain_tiny(mode):
    U.log(f"[chain {mode}] tiny_chain")
    rep = run_chain_gpu_vs_oracle(W.tiny_chain(), mode=mode)
    chain_report(rep)


def test_chain_preferred_chunks():
    """The persistent-preferred-chunk chain (384 query rows, 192 key chunks: nq != nk,
    layer-local drift, 12 + 24 near-miss + 12 random sentinels, on the wide kernel)."""
    U.log("[chain] preferred_chunks sigma=0.03 seed=0")
    rep = run_chain_gpu_vs_oracle(W.preferred_chunks(0.03, 0))
    chain_report(rep)


# Width buckets (Section 4.4): name, heads, query rows, nk, dtype, causal, narrow and wide (k, m, r)
BUCKET_CASES = [
    ("buckets_bf16", 2, 300, 256, "bf16", False, (8, 8, 8), (16, 12, 8)),
    ("buckets_f32_causal", 2, 200, 200, "f32", True, (4, 4, 6), (12, 12, 8)),
    ("buckets_ragged", 1, 130, 1100, "bf16", False, (12, 0, 0), (20, 12, 16)),
    # every option at once: mandatory sentinels and hysteresis inside causal buckets
    ("buckets_all_options", 2, 180, 180, "bf16", True, (6, 6, 4), (12, 8, 6)),
    # a bucket past 32 near-miss + route entries: the wide kernel through the query-row map
    ("buckets_wide_bf16", 2, 200, 300, "bf16", False, (8, 8, 8), (12, 24, 8)),
    ("buckets_wide_all_options", 1, 180, 180, "bf16", True, (6, 6, 4), (12, 30, 6)),
]
_ALL = dict(sink=1, recent=2, min_reuse=1, gamma_extra=0.005)
BUCKET_EXTRA = {"buckets_all_options": _ALL, "buckets_wide_all_options": _ALL}


@pytest.mark.parametrize("mode", ["auto", "compacted"])
@pytest.mark.parametrize("case", BUCKET_CASES, ids=[c[0] for c in BUCKET_CASES])
def test_width_buckets(case, mode):
    """Two width buckets over complementary query-row sets, each with its own k, m, r: both
    anchor at layer 3 and relay at layer 4 on the full Q, against the oracle bucket (pinned on
    the CPU to the same rows of a ledger over every row)."""
    name, H, nq, nk, dtype, causal, narrow, wide = case
    rng = np.random.default_rng(7)
    pick = rng.random(nq) < 0.35
    q0, k0 = inputs("gauss", H, nq, nk, dtype, 51)
    q1 = synth.perturb(q0, 0.04 / 8, seed=52, dtype=dtype)
    k1 = synth.perturb(k0, 0.04 / 8, seed=53, dtype=dtype)
    rel = 1e-5 if dtype == "f32" else 1e-3
    for rows, (k, m, r) in ((np.flatnonzero(pick), narrow), (np.flatnonzero(~pick), wide)):
        U.log(f"[bucket] {name} rows={len(rows)} of {nq} k={k} m={m} r={r} {dtype} causal={causal}")
        led = rr.Ledger(H, nq, nk, 64, k, m, r, 0.0, causal, dtype, 61, q_rows=rows,
                        **BUCKET_EXTRA.get(name, {}))
        cfg = U.oracle_cfg(led, dtype, 0.0, causal, 61)
        rep = U.Report()
        _, ora = U.anchor_parity(led, cfg, q0, k0, 3, U.GAP_TOL, rep)
        _, res, _ = U.relay_parity(led, cfg, q1, k1, 4, ora, U.GAP_TOL, rel, rep, mode=mode)
        U.log(f"   rows={rep.rows} flagged={int(res.flags.sum())} excluded={rep.excluded}")
        assert rep.excluded <= max(2, rep.rows // 100)
        led.close()


# Near-miss sets past 32 entries (Table 3's 24-wide row and beyond): the wide kernel.
# name, heads, nq, nk, k, m, r, sink, recent, dtype, causal, seed, input kind
WIDE_ANCHOR_CASES = [
    ("wide_nm24_f32", 1, 64, 256, 12, 24, 12, 0, 0, "f32", False, 30, "gauss"),
    ("wide_nm40_bf16", 2, 100, 300, 16, 40, 8, 0, 0, "bf16", False, 31, "gauss"),
    ("wide_causal_bf16", 2, 150, 150, 12, 24, 12, 0, 0, "bf16", True, 32, "gauss"),
    ("wide_mandatory", 1, 70, 200, 12, 30, 10, 2, 2, "f32", False, 33, "gauss"),
    ("wide_int_ties", 1, 96, 128, 12, 24, 12, 0, 0, "f32", False, 34, "int"),
    ("wide_short_rows", 1, 40, 30, 12, 24, 12, 1, 1, "f32", False, 35, "gauss"),
    ("wide_nk1024", 1, 64, 1024, 12, 48, 4, 0, 0, "bf16", False, 36, "gauss"),
    ("wide_km64", 1, 80, 200, 16, 48, 0, 0, 0, "bf16", False, 37, "gauss"),     # c = k + m = 64
    ("wide_route40", 1, 72, 160, 40, 0, 8, 0, 0, "f32", False, 38, "gauss"),    # wide route, no near-miss
    ("wide_km64_ties", 1, 64, 96, 16, 48, 0, 0, 0, "f32", False, 39, "int"),
    # ledgers past 64 IDs: Table 3's 48 near-miss + 12 random (c = 72) and the widest (c = 128)
    ("wide_nm48_r12_bf16", 2, 96, 256, 12, 48, 12, 0, 0, "bf16", False, 40, "gauss"),
    ("wide_c128_f32", 1, 70, 200, 32, 32, 32, 16, 16, "f32", False, 41, "gauss"),
]


@pytest.mark.parametrize("case", WIDE_ANCHOR_CASES, ids=[c[0] for c in WIDE_ANCHOR_CASES])
def test_anchor_parity_wide(case):
    name, H, nq, nk, k, m, r, sink, recent, dtype, causal, seed, kind = case
    U.log(f"[anchor wide] {name} H={H} nq={nq} nk={nk} k={k} m={m} r={r} sink={sink} recent={recent} "
          f"{dtype} causal={causal}")
    led, cfg = make(H, nq, nk, k, m, r, dtype, causal, seed, sink=sink, recent=recent)
    q, kk = inputs(kind, H, nq, nk, dtype, seed)
    tol = 0.0 if kind != "gauss" else U.GAP_TOL
    rep = U.Report()
    U.anchor_parity(led, cfg, q, kk, 3, tol, rep)
    U.log(f"   rows={rep.rows} excluded={rep.excluded}")
    if kind != "gauss":
        assert rep.excluded == 0
    # Gaps between neighbouring ranks shrink deeper in the order (rank k + m = 56 of 300 keys
    # sits ~1e-3 from its neighbour): a few rows more fall under the 1e-5 exclusion rule.
    assert rep.excluded <= max(2, rep.rows // 20)
    led.close()


WIDE_RELAY_CASES = [
    ("wide_relay_f32", 2, 128, 256, 12, 24, 12, 0, 0, "f32", False, 0.05, "gauss"),
    ("wide_relay_causal", 1, 160, 160, 12, 36, 8, 1, 2, "bf16", True, 0.04, "gauss"),
    # c > 64: the rescore takes each row's candidates as two chunks of 64
    ("wide_relay_nm48_r12_bf16", 2, 128, 256, 12, 48, 12, 0, 0, "bf16", False, 0.05, "gauss"),
    ("wide_relay_c128_f32", 1, 96, 160, 32, 32, 32, 16, 16, "f32", False, 0.05, "gauss"),
    ("wide_relay_nm48_causal", 1, 150, 150, 12, 48, 12, 0, 0, "bf16", True, 0.04, "gauss"),
    ("wide_relay_int", 1, 128, 200, 12, 24, 12, 0, 0, "f32", False, 0.0, "int"),
    ("wide_relay_route40", 1, 96, 300, 40, 8, 8, 0, 0, "bf16", False, 0.05, "gauss"),
]


@pytest.mark.parametrize("case", WIDE_RELAY_CASES, ids=[c[0] for c in WIDE_RELAY_CASES])
def test_relay_lockstep_wide(case):
    name, H, nq, nk, k, m, r, sink, recent, dtype, causal, drift, kind = case
    U.log(f"[relay wide] {name} H={H} nq={nq} nk={nk} k={k} m={m} r={r} {dtype} causal={causal}")
    led, cfg = make(H, nq, nk, k, m, r, dtype, causal, 21, 0.0, sink=sink, recent=recent)
    q0, k0 = inputs(kind, H, nq, nk, dtype, 31)
    if kind == "int":
        qn, kn = inputs(kind, H, nq, nk, dtype, 32)
        q1, k1 = q0.copy(), k0.copy()
        q1[:, 1::4] = qn[:, 1::4]
        k1[:, ::9] = kn[:, ::9]
    else:
        q1 = synth.perturb(q0, drift / 8, seed=41, dtype=dtype)
        k1 = synth.perturb(k0, drift / 8, seed=42, dtype=dtype)
    ora0 = O.anchor_layer(cfg, q0, k0, 4)
    tol = 0.0 if kind != "gauss" else U.GAP_TOL
    rel = 1e-5 if dtype == "f32" else 1e-3
    rep = U.Report()
    gpu, res, ex = U.relay_parity(led, cfg, q1, k1, 5, ora0, tol, rel, rep)
    nflag = int(res.flags.sum())
    U.log(f"   rows={rep.rows} flagged={nflag} excluded={rep.excluded}")
    assert 0 < nflag < H * nq
    led.close()


def test_chain_wide_near_miss():
    """Table 3's 24-wide near-miss mix on its setting (256 chunks, fp32, drift 0.003, 24 layers)."""
    U.log("[chain] sentinel ablation setting with 24 near-miss + 12 random")
    rep = run_chain_gpu_vs_oracle(W.drift_sweep(0.003, 0).with_(layers=24, anchors=W.stride_anchors(24, 8),
                                                                m=24, r=12))
    chain_report(rep)


# Hysteresis (Section 3.2, after Eq. 8): min_reuse, gamma_extra
HYST_CASES = [
    ("hyst_horizon", 1, 0.0),
    ("hyst_guard", 0, 0.02),
    ("hyst_both", 2, 0.01),
]


@pytest.mark.parametrize("mode", RELAY_MODES)
@pytest.mark.parametrize("case", HYST_CASES, ids=[c[0] for c in HYST_CASES])
def test_relay_lockstep_hysteresis(case, mode):
    """Oracle anchor at layer 4 and relay at 5 (which refreshes some rows and marks them),
    injected with rr_ledger_set + rr_ledger_set_refreshed; then relay layer 6 on both sides."""
    name, min_reuse, gamma_extra = case
    H, nq, nk, dtype = 2, 256, 256, "bf16"
    U.log(f"[relay] {name} min_reuse={min_reuse} gamma_extra={gamma_extra}")
    led = rr.Ledger(H, nq, nk, 64, 12, 12, 8, 0.0, False, dtype, 21, min_reuse=min_reuse,
                    gamma_extra=gamma_extra)
    cfg = U.oracle_cfg(led, dtype, 0.0, False, 21)
    q0, k0 = inputs("gauss", H, nq, nk, dtype, 31)
    q1 = synth.perturb(q0, 0.03 / 8, seed=41, dtype=dtype)
    k1 = synth.perturb(k0, 0.03 / 8, seed=42, dtype=dtype)
    q2 = synth.perturb(q1, 0.03 / 8, seed=43, dtype=dtype)
    k2 = synth.perturb(k1, 0.03 / 8, seed=44, dtype=dtype)
    ora5 = O.relay_layer(cfg, q1, k1, 5, O.anchor_layer(cfg, q0, k0, 4)).ledger
    assert ora5.refreshed.sum() > 0
    rep = U.Report()
    gpu, res, ex = U.relay_parity(led, cfg, q2, k2, 6, ora5, U.GAP_TOL, 1e-3, rep, mode=mode)
    skipped = int(((ora5.refreshed == 1) & (6 - ora5.anchor <= min_reuse)).sum())
    U.log(f"   rows={rep.rows} flagged={int(res.flags.sum())} untested={skipped} "
          f"still marked={int(res.ledger.refreshed.sum())} excluded={rep.excluded}")
    if min_reuse >= 1:
        assert skipped == int(ora5.refreshed.sum())
    led.close()


def test_chain_hysteresis():
    """The drift-sweep chain with a one-layer reuse horizon and a 0.01 post-refresh guard;
    both sides carry their own hysteresis state through the chain."""
    U.log("[chain] drift_sweep sigma=0.03 with min_reuse=1 gamma_extra=0.01")
    rep = run_chain_gpu_vs_oracle(W.drift_sweep(0.03, 0).with_(min_reuse=1, gamma_extra=0.01))
    chain_report(rep)


def test_chain_all_options_causal():
    """The causal drift-sweep chain with mandatory sentinels and hysteresis together."""
    U.log("[chain] drift_sweep sigma=0.03 causal, sink=1 recent=1 r=6 min_reuse=1 gamma_extra=0.005")
    rep = run_chain_gpu_vs_oracle(W.drift_sweep(0.03, 1).with_(causal=True, sink=1, recent=1, r=6,
                                                               min_reuse=1, gamma_extra=0.005))
    chain_report(rep)


def test_chain_mandatory_sentinels():
    """The drift-sweep chain (256 chunks, 16 fp32 layers) with one sink and two recent
    sentinels in place of three random ones."""
    U.log("[chain] drift_sweep sigma=0.03 with sink=1 recent=2 r=5")
    rep = run_chain_gpu_vs_oracle(W.drift_sweep(0.03, 0).with_(sink=1, recent=2, r=5))
    chain_report(rep)


@pytest.mark.parametrize("sigma", [0.01, 0.03, 0.06])
@pytest.mark.parametrize("seed", [0, 1])
def test_chain_drift_sweep(sigma, seed):
    U.log(f"[chain] drift_sweep sigma={sigma} seed={seed}")
    rep = run_chain_gpu_vs_oracle(W.drift_sweep(sigma, seed))
    chain_report(rep)


def test_chain_drift_sweep_compacted():
    """The drift-sweep chain through the two-kernel compacted relay schedule."""
    U.log("[chain compacted] drift_sweep sigma=0.03 seed=2")
    rep = run_chain_gpu_vs_oracle(W.drift_sweep(0.03, 2), mode="compacted")
    chain_report(rep)


@pytest.mark.parametrize("n", [128, 256, 512, 1024])
def test_chain_scale_sweep(n):
    U.log(f"[chain] scale_sweep n={n}")
    rep = run_chain_gpu_vs_oracle(W.scale_sweep(n).with_(layers=12 if n == 1024 else 32))
    chain_report(rep)


def test_chain_batched_heads_subset():
    """32-head workload's first 4 heads, 10 layers (two anchors)."""
    U.log("[chain] batched_heads heads 0-3, layers 0-9")
    rep = run_chain_gpu_vs_oracle(W.batched_heads().with_(layers=10), heads=4)
    chain_report(rep)


@pytest.mark.parametrize("mode", RELAY_MODES)
def test_full_size_batched_heads_layers(mode):
    """Full 32 x 1024 bf16 anchor layer, then one relay layer, every row compared."""
    w = W.batched_heads()
    U.log(f"[full {mode}] batched_heads anchor layer 0 + relay layer 1, all 32768 rows")
    gen = synth.generate(w)
    l0, l1 = next(gen), next(gen)
    led, cfg = make(w.heads, w.n, w.n, w.k, w.m, w.r, w.dtype, False, w.seed)
    rep = U.Report()
    _, ora0 = U.anchor_parity(led, cfg, l0.q, l0.k, 0, U.GAP_TOL, rep)
    _, res, _ = U.relay_parity(led, cfg, l1.q, l1.k, 1, ora0, U.GAP_TOL, 1e-3, rep, mode=mode)
    U.log(f"   rows={rep.rows} excluded={rep.excluded} flagged={int(res.flags.sum())} max|ds|={rep.max_score_err:.2e}")
    # the exclusion rate is a property of the data (oracle gaps), ~0.5% at 1024 chunks
    assert rep.excluded <= rep.rows // 50
    led.close()


def test_full_size_causal_large_sampled():
    """Full 64 x 4096 causal bf16 anchor layer; oracle on a sample of rows (all heads' first
    64 rows, plus 1024 random (head, row) pairs)."""
    w = W.causal_large()
    U.log("[full] causal_large anchor layer 0, sampled rows")
    l0 = next(synth.generate(w))
    led, cfg = make(w.heads, w.n, w.n, w.k, w.m, w.r, w.dtype, True, w.seed)
    rng = np.random.default_rng(0)
    rows = {(h, i) for h in range(w.heads) for i in range(64)}
    rows |= {(int(h), int(i)) for h, i in zip(rng.integers(0, w.heads, 1024), rng.integers(0, w.n, 1024))}
    rows |= {(h, w.n - 1) for h in range(0, w.heads, 8)}
    rep = U.Report()
    U.anchor_parity(led, cfg, l0.q, l0.k, 0, U.GAP_TOL, rep, rows=sorted(rows))
    U.log(f"   rows={rep.rows} excluded={rep.excluded}")
    assert rep.excluded <= max(2, rep.rows // 50)
    led.close()


@pytest.mark.parametrize("mode", ["auto", "compacted"])
def test_full_size_causal_large_relay_sampled(mode):
    """Full 64 x 4096 causal bf16: GPU anchor at layer 0 and relay at layer 1 on every row (the
    reroute's flagged-row search then spans 64 rescore blocks per head, the edge of its
    block-count scan); the oracle relays sampled rows from its own anchor entries: every head's
    first 64 rows (rows shorter than k + m, sentinel segments still filling), the last 64 rows
    of every 8th head (rows near 4095) and 2000 random (head, row) pairs."""
    w = W.causal_large()
    U.log(f"[full {mode}] causal_large anchor layer 0 + relay layer 1, sampled rows")
    gen = synth.generate(w)
    l0, l1 = next(gen), next(gen)
    led, cfg = make(w.heads, w.n, w.n, w.k, w.m, w.r, w.dtype, True, w.seed)
    rng = np.random.default_rng(1)
    rows = {(h, i) for h in range(w.heads) for i in range(64)}
    rows |= {(h, i) for h in range(0, w.heads, 8) for i in range(w.n - 64, w.n)}
    rows |= {(int(h), int(i)) for h, i in zip(rng.integers(0, w.heads, 2000), rng.integers(0, w.n, 2000))}
    rep = U.Report()
    compared, flagged = U.relay_parity_sampled(led, cfg, l0.q, l0.k, l1.q, l1.k, rows, U.GAP_TOL, 1e-3, rep,
                                               mode=mode)
    U.log(f"   sampled={rep.rows} compared={compared} flagged={flagged} excluded={rep.excluded} "
          f"max|ds|={rep.max_score_err:.2e}")
    assert compared >= 6000 and flagged > 1000
    assert rep.excluded <= max(2, rep.rows // 50)
    led.close()


@pytest.mark.parametrize("mode", ["auto", "compacted"])
def test_long_keys_causal_relay_sampled(mode):
    """One head of 16384 causal bf16 chunks (2M tokens in 128-token chunks): GPU anchor at layer
    0 and relay at layer 1 on every row; the oracle on sampled rows: the first 64 (rows shorter
    than k + m), the last 64 (rows of ~16K keys, one route block per compute unit) and 400
    random rows."""
    w = W.causal_large().with_(name="causal_16k", heads=1, n=16384)
    U.log(f"[long keys {mode}] 1 x 16384 causal anchor layer 0 + relay layer 1, sampled rows")
    gen = synth.generate(w)
    l0, l1 = next(gen), next(gen)
    led, cfg = make(w.heads, w.n, w.n, w.k, w.m, w.r, w.dtype, True, w.seed)
    rng = np.random.default_rng(2)
    rows = {(0, i) for i in range(64)} | {(0, i) for i in range(w.n - 64, w.n)}
    rows |= {(0, int(i)) for i in rng.integers(0, w.n, 400)}
    rep = U.Report()
    compared, flagged = U.relay_parity_sampled(led, cfg, l0.q, l0.k, l1.q, l1.k, rows, U.GAP_TOL, 1e-3, rep,
                                               mode=mode)
    U.log(f"   sampled={rep.rows} compared={compared} flagged={flagged} excluded={rep.excluded} "
          f"max|ds|={rep.max_score_err:.2e}")
    assert compared >= 400 and flagged > 50
    assert rep.excluded <= max(2, rep.rows // 50)
    led.close()


@pytest.mark.parametrize("mode", RELAY_MODES)
def test_repeat_runs_are_bit_identical(mode):
    import torch
    w = W.scale_sweep(1024)
    U.log(f"[determinism {mode}] scale_sweep n=1024, anchor + relay twice")
    gen = synth.generate(w)
    l0, l1 = next(gen), next(gen)
    outs = []
    for _ in range(2):
        led = rr.Ledger(1, 1024, 1024, 64, 12, 12, 8, 0.0, False, "bf16", 0)
        led.set_relay_mode(mode)
        led.anchor(U.upload(l0.q), U.upload(l0.k), 0)
        o = led.alloc_outputs()
        led.relay(U.upload(l1.q), U.upload(l1.k), 1, o)
        torch.cuda.synchronize()
        outs.append((U.ledger_np(led), o.flags.cpu().numpy(), o.alpha.cpu().numpy(), o.cand_scores.cpu().numpy()))
        led.close()
    (a, fa, aa, ca), (b, fb, ab, cb) = outs
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert np.array_equal(fa, fb) and np.array_equal(aa.view(np.uint32), ab.view(np.uint32))
    assert np.array_equal(ca.view(np.uint32), cb.view(np.uint32))


def test_state_rules_on_device():
    import torch
    U.log("[state] relay before anchor, non-increasing layer")
    led = rr.Ledger(1, 64, 64, 64, 12, 12, 8, 0.0, False, "f32", 0)
    q, k = synth.gaussian_inputs(1, 64, 64, 64, seed=0)
    qd, kd = U.upload(q), U.upload(k)
    with pytest.raises(rr.RRError) as e:
        led.relay(qd, kd, 1)
    assert e.value.status == rr.RR_ESTATE
    led.anchor(qd, kd, 3)
    with pytest.raises(rr.RRError) as e:
        led.relay(qd, kd, 3)
    assert e.value.status == rr.RR_ESTATE
    before = U.ledger_np(led)
    led.relay(qd, kd, 4)
    torch.cuda.synchronize()
    after = U.ledger_np(led)
    # same inputs as the anchor: every row is stable unless it ties (alpha == beta)
    assert np.array_equal(before[0], after[0])
    led.close()


def test_ledger_set_from_host_checks_the_ids():
    """rr_ledger_set from host memory: an oracle ledger is taken as is (rr_ledger_get returns
    it); a ledger with a repeated chunk is refused with RR_EINVAL and leaves the ledger as it
    was."""
    import torch
    U.log("[state] rr_ledger_set from host memory: valid and repeated-chunk ledgers")
    led, cfg = make(2, 48, 64, k=8, m=6, r=5, dtype="f32", seed=3)
    q, k = synth.gaussian_inputs(2, 48, 64, 64, seed=1)
    ora = O.anchor_layer(cfg, q, k, 2)
    rr.rr_ledger_set(led.handle, ora.route, ora.sent, ora.anchor, 2, True)
    got = U.ledger_np(led)
    assert np.array_equal(got[0], ora.route) and np.array_equal(got[1], ora.sent)
    assert np.array_equal(got[2], ora.anchor)
    bad_sent = ora.sent.copy()
    bad_sent[1, 4, 0] = ora.route[1, 4, 0]
    bad_sent[1, 4, :6] = np.sort(bad_sent[1, 4, :6])
    with pytest.raises(rr.RRError) as e:
        rr.rr_ledger_set(led.handle, ora.route, np.ascontiguousarray(bad_sent), ora.anchor, 3, True)
    assert e.value.status == rr.RR_EINVAL and "head 1 row 4" in str(e.value)
    torch.cuda.synchronize()
    again = U.ledger_np(led)
    assert all(np.array_equal(a, b) for a, b in zip(got, again))
    qd, kd = U.upload(q), U.upload(k)
    led.relay(qd, kd, 3)                             # last layer still 2: the refused set changed nothing
    led.close()


@pytest.mark.gpu
@pytest.mark.parametrize("mode", RELAY_MODES)
def test_kernel_timing_records_every_launch(mode):
    import torch
    U.log(f"[profile {mode}] per-kernel launch events")
    led = rr.Ledger(2, 128, 128, 64, 12, 12, 8, 0.0, False, "f32", 0)
    led.set_relay_mode(mode)
    q, k = synth.gaussian_inputs(2, 128, 128, 64, seed=1)
    qd, kd = U.upload(q), U.upload(k)
    led.profile(True)
    led.anchor(qd, kd, 0)
    led.relay(qd, kd, 1)
    out = led.alloc_outputs(with_scores=False)
    led.relay(qd, kd, 2, out)                                      # with the compacted-list outputs
    kt = led.kernel_times()
    want = [1, 0, 0, 2, 1] if mode == "fused" else [1, 2, 2, 0, 0]
    assert [n for n, _ in kt] == want
    assert all(ms > 0.0 for n, ms in kt if n)
    assert [n for n, _ in led.kernel_times()] == [0] * rr.RR_KERNEL_KINDS    # reading clears the record
    led.profile(False)
    led.anchor(qd, kd, 3)
    torch.cuda.synchronize()
    assert [n for n, _ in led.kernel_times()] == [0] * rr.RR_KERNEL_KINDS
    led.close()


def test_relay_mode_rules():
    U.log("[state] relay modes")
    led = rr.Ledger(1, 64, 64, 64, 12, 24, 8, 0.0, False, "f32", 0)     # k + m = 36: wide kernel
    with pytest.raises(rr.RRError) as e:
        led.set_relay_mode("fused")
    assert e.value.status == rr.RR_EUNSUPPORTED
    led.set_relay_mode("compacted")
    with pytest.raises(rr.RRError) as e:
        rr.rr_ledger_set_relay_mode(led.handle, 7)
    assert e.value.status == rr.RR_EINVAL
    led.close()
