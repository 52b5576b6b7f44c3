"""GPU parity of the sparse attention over routed chunks (rr_sparse_attention) against the
oracle (oracle/attention.py), through the C ABI.

Tolerance, from the arithmetic: scores and the softmax are fp32 and the probabilities enter
the value product rounded to bf16 (relative error <= 2^-9 each, all non-negative), so an
output differs from the exact one by at most 2^-9 * max |v| over the routed tokens plus fp32
rounding; the test allows twice that: 2^-8 * max |V[:, d]| of the head + 1e-5 |ref|."""
import numpy as np
import pytest

import oracle as O
from long_context_prefill_anchor_amd import rr, synth
from tests import gpu_util as U

pytestmark = pytest.mark.gpu
T = 64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rr.lib()
    yield


def tokens(H, n_chunks, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((3, H, n_chunks * T, 64)) / 8).astype(np.float32)
    return [synth.fp32_to_bf16_bits(a) for a in x]


def vt_of(v_bits, H, nk):
    """[H, nk*T, 64] -> per-chunk transposed [H, nk, 64 (d), T]."""
    return np.ascontiguousarray(v_bits.reshape(H, nk, T, 64).transpose(0, 1, 3, 2))


def random_routes(H, nq, nk, kr, causal, seed, pad_frac=0.15):
    rng = np.random.default_rng(seed)
    r = np.full((H, nq, kr), -1, np.int32)
    for h in range(H):
        for i in range(nq):
            n = (i + 1) if causal else nk
            take = rng.permutation(n)[: min(kr, n)]
            if causal and rng.random() < 0.7 and i not in take:
                take[-1] = i                      # most causal rows hold their own chunk
            take = np.sort(take)
            keep = rng.random(len(take)) >= pad_frac
            r[h, i, : keep.sum()] = take[keep]
    return r


def run_gpu(q, k, vt, routes, H, nq, nk, causal):
    import torch
    kr = routes.shape[2]
    out = torch.empty((H, nq * T, 64), dtype=torch.float32, device="cuda")
    rr.rr_sparse_attention(U.upload(q), U.upload(k), U.upload(vt), torch.from_numpy(routes).cuda(),
                           H, nq, nk, kr, out, causal=causal)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def check(got, ref, v_bits, what):
    vmax = np.abs(synth.bf16_bits_to_fp32(v_bits)).max(axis=1).astype(np.float64)   # [H, 64]
    lim = 2.0 ** -8 * vmax[:, None, :] + 1e-5 * np.abs(ref)
    err = np.abs(got - ref)
    bad = err > lim
    if bad.any():
        idx = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} outputs out of tolerance, first {idx}: "
                             f"gpu={got[idx]} oracle={ref[idx]} lim={lim[idx]}")
    return float((err / np.maximum(lim, 1e-30)).max())


CASES = [
    # name, heads, nq, nk, kr, causal, seed
    ("dense_small", 2, 10, 14, 6, False, 1),
    ("causal_small", 2, 12, 12, 5, True, 2),
    ("wide_route", 1, 6, 40, 32, False, 3),
    ("single_chunk", 1, 9, 9, 1, True, 4),
    ("k12_ragged", 3, 7, 23, 12, False, 5),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_sparse_attention_parity(case):
    name, H, nq, nk, kr, causal, seed = case
    U.log(f"[attention] {name} H={H} nq={nq} nk={nk} kr={kr} causal={causal}")
    n_tok = max(nq, nk)
    q, k, v = tokens(H, n_tok, seed)
    q = np.ascontiguousarray(q[:, : nq * T])
    k = np.ascontiguousarray(k[:, : nk * T])
    v = np.ascontiguousarray(v[:, : nk * T])
    routes = random_routes(H, nq, nk, kr, causal, seed + 100)
    routes[0, 0] = -1                                    # a chunk with nothing routed
    got = run_gpu(q, k, vt_of(v, H, nk), routes, H, nq, nk, causal)
    ref = O.sparse_attention(q, k, v, routes, T, causal, "bf16")
    assert np.all(got[0, :T] == 0)
    worst = check(got, ref, v, name)
    U.log(f"   worst error / bound = {worst:.3f}")


def test_sparse_attention_on_ledger_routes_sampled():
    """Routes straight from a ledger's device route tensor (32 heads x 1024 chunks, k = 12,
    65,536 tokens per head), outputs of sampled query chunks against the oracle."""
    import torch
    H, n, kr = 32, 1024, 12
    U.log(f"[attention] ledger routes H={H} chunks={n} k={kr}, sampled rows")
    qc, kc = synth.gaussian_inputs(H, n, n, 64, seed=9, dtype="bf16")
    led = rr.Ledger(H, n, n, 64, kr, 12, 8, 0.0, False, "bf16", 0)
    led.anchor(U.upload(qc), U.upload(kc), 0)
    routes_d = led.get()[0]
    torch.cuda.synchronize()
    routes = routes_d.cpu().numpy()
    g = torch.Generator(device="cuda").manual_seed(11)
    qt = (torch.randn((H, n * T, 64), generator=g, device="cuda") / 8).to(torch.bfloat16)
    kt = (torch.randn((H, n * T, 64), generator=g, device="cuda") / 8).to(torch.bfloat16)
    vtok = (torch.randn((H, n * T, 64), generator=g, device="cuda") / 8).to(torch.bfloat16)
    vt = vtok.view(H, n, T, 64).transpose(2, 3).contiguous()
    out = torch.empty((H, n * T, 64), dtype=torch.float32, device="cuda")
    rr.rr_sparse_attention(qt, kt, vt, routes_d, H, n, n, kr, out)
    torch.cuda.synchronize()
    bits = lambda x: x.view(torch.int16).cpu().numpy().view(np.uint16)
    qb, kb, vb = bits(qt), bits(kt), bits(vtok)
    rng = np.random.default_rng(3)
    for h, i in zip(rng.integers(0, H, 6), rng.integers(0, n, 6)):
        sl = slice(i * T, (i + 1) * T)
        ref = O.sparse_attention(qb[h:h + 1, sl], kb[h:h + 1], vb[h:h + 1], routes[h:h + 1, i:i + 1], T,
                                 False, "bf16")
        got = out[h:h + 1, sl].cpu().numpy().astype(np.float64)
        check(got, ref, vb[h:h + 1], f"head {h} chunk {i}")
    led.close()
