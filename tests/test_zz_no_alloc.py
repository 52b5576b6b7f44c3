"""The allocation-free relay layer (rr_relay_layer_noalloc) against rr_relay_layer.

Both entry points run the same kernels; the allocation-free one keeps its working memory in
one fixed device array of the library instead of the ledger's own buffers.  Each case runs two
calls in a row through it, the second on a smaller input, so that anything the first call left
in the fixed array and the second read back would show up as a difference.  Ledger state, refresh
flags, compacted list, head counts and scores must be bit-equal to rr_relay_layer's on the same
state and inputs.
"""
import numpy as np
import pytest

from long_context_prefill_anchor_amd import rr, synth
from tests import gpu_util as U

MAX_ROWS = 1 << 18


def test_noalloc_rejects_oversize_and_null_state():
    """Host-side checks only: they return before any device call."""
    cfg = rr.make_config(5, 65536, 64)          # 5 * 65536 padded rows > 2^18
    fake = 1 << 20
    with pytest.raises(rr.RRError) as e:
        rr.rr_relay_layer_noalloc(cfg, fake, fake, fake, fake, fake, 1, stream=0, out=False)
    assert e.value.status == rr.RR_EUNSUPPORTED
    assert "fixed working memory" in rr.rr_last_error()
    cfg = rr.make_config(4, 65536, 64)          # exactly 2^18 rows: passes the size check ...
    with pytest.raises(rr.RRError) as e:        # ... and stops at the missing state
        rr.rr_relay_layer_noalloc(cfg, None, fake, fake, fake, fake, 1, stream=0, out=False)
    assert e.value.status == rr.RR_EINVAL
    with pytest.raises(rr.RRError) as e:
        rr.rr_relay_layer_noalloc(cfg, fake, fake, fake, fake, fake, -1, stream=0, out=False)
    assert e.value.status == rr.RR_EINVAL
    bad = rr.make_config(2, 64, 64, k=40, m=30)
    with pytest.raises(rr.RRError) as e:
        rr.rr_relay_layer_noalloc(bad, fake, fake, fake, fake, fake, 1, stream=0, out=False)
    assert e.value.status == rr.RR_EUNSUPPORTED


# (name, heads, nq, nk, k, m, r, sink, recent, dtype, causal, min_reuse, gamma_extra, drift)
# Pairs: the second call of each pair is smaller than the first.
PAIRS = [
    ("fused",
     ("batched_bf16", 16, 1024, 1024, 12, 12, 8, 0, 0, "bf16", False, 0, 0.0, 0.03),
     ("ragged_f32_causal", 3, 300, 300, 12, 12, 5, 1, 2, "f32", True, 1, 0.005, 0.05)),
    ("compacted",
     ("many_blocks_bf16", 64, 2048, 2048, 12, 12, 8, 0, 0, "bf16", False, 0, 0.0, 0.03),
     ("long_keys_bf16", 2, 130, 2100, 12, 12, 8, 0, 0, "bf16", False, 0, 0.0, 0.05)),
    ("wide",
     ("wide_bf16", 4, 512, 512, 12, 24, 8, 0, 0, "bf16", False, 0, 0.0, 0.03),
     ("wide_f32_causal", 1, 70, 70, 12, 24, 8, 0, 0, "f32", True, 0, 0.0, 0.05)),
]


def run_case(case, with_out):
    import torch
    name, H, nq, nk, k, m, r, sink, recent, dtype, causal, min_reuse, gx, drift = case
    U.log(f"[noalloc] {name} H={H} nq={nq} nk={nk} k={k} m={m} r={r} sink={sink} recent={recent} "
          f"{dtype} causal={causal} min_reuse={min_reuse} gamma_extra={gx} outputs={with_out}")
    assert H * ((nq + 63) // 64) * 64 <= MAX_ROWS
    led = rr.Ledger(H, nq, nk, 64, k, m, r, 0.0, causal, dtype, 77, sink=sink, recent=recent,
                    min_reuse=min_reuse, gamma_extra=gx)
    q0, k0 = synth.gaussian_inputs(H, nq, nk, 64, seed=5, dtype=dtype)
    q1 = synth.perturb(q0, drift / 8, seed=6, dtype=dtype)
    k1 = synth.perturb(k0, drift / 8, seed=7, dtype=dtype)
    q2 = synth.perturb(q1, drift / 8, seed=8, dtype=dtype)
    k2 = synth.perturb(k1, drift / 8, seed=9, dtype=dtype)
    dq0, dk0, dq1, dk1, dq2, dk2 = (U.upload(x) for x in (q0, k0, q1, k1, q2, k2))
    led.anchor(dq0, dk0, 4)
    led.relay(dq1, dk1, 5)          # leaves some rows refreshed: the hysteresis state matters
    route, sent, anchor = led.get()
    ids = torch.cat([route, sent], dim=2).contiguous()
    anchor = anchor.clone()
    refreshed = led.get_refreshed().clone()
    torch.cuda.synchronize()

    ref = led.alloc_outputs() if with_out else None
    led.relay(dq2, dk2, 6, ref)
    got = led.alloc_outputs() if with_out else None
    if with_out:
        rr.rr_relay_layer_noalloc(led.cfg, ids, anchor, refreshed, dq2, dk2, 6, None, got.flags,
                                  got.rows, got.head_counts, got.n_rows, got.alpha, got.beta,
                                  got.cand_scores)
    else:
        rr.rr_relay_layer_noalloc(led.cfg, ids, anchor, refreshed, dq2, dk2, 6, None, out=False)
    torch.cuda.synchronize()

    r_route, r_sent, r_anchor = led.get()
    r_ids = torch.cat([r_route, r_sent], dim=2)
    r_refreshed = led.get_refreshed()
    torch.cuda.synchronize()
    assert torch.equal(ids, r_ids), f"{name}: ledger IDs differ"
    assert torch.equal(anchor, r_anchor), f"{name}: anchor layers differ"
    assert torch.equal(refreshed, r_refreshed), f"{name}: hysteresis state differs"
    nflag = int((r_anchor == 6).sum())
    if with_out:
        for f in ("flags", "rows", "head_counts", "n_rows"):
            assert torch.equal(getattr(got, f), getattr(ref, f)), f"{name}: {f} differ"
        for f in ("alpha", "beta", "cand_scores"):
            a, b = getattr(got, f).cpu().numpy(), getattr(ref, f).cpu().numpy()
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{name}: {f} differ"
        assert int(ref.n_rows.item()) == nflag
    U.log(f"   rerouted={nflag} of {H * nq}")
    assert 0 < nflag < H * nq
    led.close()


@pytest.mark.gpu
@pytest.mark.parametrize("pair", PAIRS, ids=[p[0] for p in PAIRS])
def test_noalloc_matches_relay_layer_twice(pair):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rr.lib()
    _, first, second = pair
    run_case(first, with_out=True)
    run_case(second, with_out=True)
    run_case(second, with_out=False)
