"""Host-side checks of the C ABI: librr.so loads, exports every entry point of include/rr.h,
and rejects bad arguments before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

from long_context_prefill_anchor_amd import rr
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "rr.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:rr_status|void|const char\*|int32_t)\s+(rr_\w+)\s*\(", text, flags=re.M)


def test_header_and_binding_agree():
    names = declared_functions()
    assert len(names) == len(set(names)) >= 10
    assert set(names) == set(rr.ENTRY_POINTS)


def test_library_exports_every_declared_symbol():
    L = rr.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert rr.rr_abi_version() == 5


def cfg(**kw):
    base = dict(heads=2, nq=64, nk=64, d=64, k=12, m=12, r=8, gamma=0.0, causal=False,
                dtype="bf16", seed=0)
    base.update(kw)
    return rr.make_config(**base)


def test_config_check_accepts_every_named_workload():
    from long_context_prefill_anchor_amd import workloads as W
    for w in W.all_named():
        c = rr.make_config(w.heads, w.n, w.n, w.d, w.k, w.m, w.r, w.gamma, w.causal, w.dtype, w.seed)
        assert rr.rr_config_check(c) == rr.RR_OK, (w.name, rr.rr_last_error())
    # the full-routing comparator: m = r = 0
    assert rr.rr_config_check(cfg(m=0, r=0)) == rr.RR_OK
    # mandatory sentinels up to c = 64
    assert rr.rr_config_check(cfg(k=12, m=12, r=24, sink=8, recent=8)) == rr.RR_OK
    # Table 3's widest mix (48 near-miss + 12 random, c = 72) and the widest ledger (c = 128)
    assert rr.rr_config_check(cfg(k=12, m=48, r=12)) == rr.RR_OK
    assert rr.rr_config_check(cfg(k=32, m=32, r=32, sink=16, recent=16)) == rr.RR_OK
    # long rows: 16384 key chunks (2M tokens in 128-token chunks) with up to 86 IDs per row
    assert rr.rr_config_check(cfg(nk=16384)) == rr.RR_OK
    assert rr.rr_config_check(cfg(nk=16384, r=32, sink=15, recent=15)) == rr.RR_OK
    assert rr.rr_config_check(cfg(nk=8192, k=16, m=16, r=32, sink=16, recent=16)) == rr.RR_OK


def test_config_struct_layout_matches_the_header(tmp_path):
    """The binding's rr_config and relay-output structs have the size and field offsets a C
    compiler gives the header's declarations."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    src = tmp_path / "layout.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"rr.h\"\n"
                   "int main(void) { printf(\"%zu %zu %zu %zu %zu %zu %zu %zu\\n\", sizeof(rr_config), "
                   "offsetof(rr_config, seed), offsetof(rr_config, sink), offsetof(rr_config, recent), "
                   "offsetof(rr_config, min_reuse), offsetof(rr_config, gamma_extra), "
                   "sizeof(rr_relay_out), offsetof(rr_relay_out, cand_scores)); return 0; }\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", inc, str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    assert got == [ctypes.sizeof(rr.rr_config), rr.rr_config.seed.offset, rr.rr_config.sink.offset,
                   rr.rr_config.recent.offset, rr.rr_config.min_reuse.offset,
                   rr.rr_config.gamma_extra.offset, ctypes.sizeof(rr.rr_relay_out),
                   rr.rr_relay_out.cand_scores.offset]


@pytest.mark.parametrize("kw,status,needle", [
    (dict(heads=0), rr.RR_EINVAL, "heads"),
    (dict(nq=0), rr.RR_EINVAL, "nq"),
    (dict(nk=-5), rr.RR_EINVAL, "nk"),
    (dict(k=0), rr.RR_EINVAL, "k >= 1"),
    (dict(m=-1), rr.RR_EINVAL, "m >= 0"),
    (dict(r=-1), rr.RR_EINVAL, "r >= 0"),
    (dict(gamma=-0.5), rr.RR_EINVAL, "gamma"),
    (dict(gamma=float("inf")), rr.RR_EINVAL, "gamma"),
    (dict(gamma=float("nan")), rr.RR_EINVAL, "gamma"),
    (dict(causal=True, nk=32), rr.RR_EINVAL, "causal"),
    (dict(d=128), rr.RR_EUNSUPPORTED, "d = 64"),
    (dict(k=20, m=45), rr.RR_EUNSUPPORTED, "k + m"),
    (dict(k=20, m=13, r=4, nk=2048), rr.RR_EUNSUPPORTED, "nk <= 1024"),
    (dict(r=33), rr.RR_EUNSUPPORTED, "r must"),
    (dict(nk=32768), rr.RR_EUNSUPPORTED, "nk must be <= 16384"),
    # c = 88 IDs per row at 16384 chunks: the route block's LDS would exceed 160 KB
    (dict(nk=16384, r=32, sink=16, recent=16), rr.RR_EUNSUPPORTED, "LDS"),
    (dict(sink=-1), rr.RR_EINVAL, "sink >= 0"),
    (dict(recent=-2), rr.RR_EINVAL, "recent >= 0"),
    (dict(sink=20, recent=13), rr.RR_EUNSUPPORTED, "sink + recent"),
    (dict(min_reuse=-1), rr.RR_EINVAL, "min_reuse"),
    (dict(gamma_extra=-0.1), rr.RR_EINVAL, "gamma_extra"),
    (dict(gamma_extra=float("inf")), rr.RR_EINVAL, "gamma_extra"),
])
def test_config_check_rejects(kw, status, needle):
    assert rr.rr_config_check(cfg(**kw)) == status
    assert needle in rr.rr_last_error()


def test_width_bucket_rejects_bad_row_lists():
    """rr_ledger_create_rows validates its row list on the host before touching the device."""
    L = rr.lib()
    h = ctypes.c_void_p(77)

    def create(rows, nq_q, **kw):
        arr = (ctypes.c_int32 * max(1, len(rows)))(*rows)
        return L.rr_ledger_create_rows(ctypes.byref(cfg(nq=len(rows), **kw)), arr if rows else None,
                                       nq_q, ctypes.byref(h))
    assert create([], 64) == rr.RR_EINVAL                      # NULL list
    assert create([3, 2, 9], 64) == rr.RR_EINVAL and "ascend" in rr.rr_last_error()
    assert create([1, 1], 64) == rr.RR_EINVAL                  # not strictly ascending
    assert create([0, 64], 64) == rr.RR_EINVAL                 # outside [0, nq_q)
    assert create([0, 5], 1) == rr.RR_EINVAL and "nq_q" in rr.rr_last_error()
    assert create([0, 5], 64, causal=True, nk=32) == rr.RR_EINVAL and "causal" in rr.rr_last_error()
    assert h.value is None


def test_sparse_attention_rejects_bad_arguments():
    """rr_sparse_attention validates on the host: nothing is launched for these."""
    L = rr.lib()
    f = L.rr_sparse_attention
    ok = dict(q=1, k=1, vt=1, routes=1, heads=2, nq=4, nk=4, kr=3, T=64, causal=0, out=1)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["q"], a["k"], a["vt"], a["routes"], a["heads"], a["nq"], a["nk"], a["kr"], a["T"],
                 a["causal"], a["out"], None)
    assert call(q=None) == rr.RR_EINVAL and "required" in rr.rr_last_error()
    assert call(out=None) == rr.RR_EINVAL
    assert call(heads=0) == rr.RR_EINVAL
    assert call(kr=0) == rr.RR_EINVAL
    assert call(causal=2) == rr.RR_EINVAL
    assert call(causal=1, nk=5) == rr.RR_EINVAL and "nq == nk" in rr.rr_last_error()
    assert call(T=128) == rr.RR_EUNSUPPORTED and "64-token" in rr.rr_last_error()
    assert call(kr=65) == rr.RR_EUNSUPPORTED


def test_bad_dtype_and_causal_flag():
    c = cfg()
    c.dtype = 7
    assert rr.rr_config_check(c) == rr.RR_EINVAL
    c = cfg()
    c.causal = 2
    assert rr.rr_config_check(c) == rr.RR_EINVAL


def test_create_rejects_bad_config_without_touching_the_device():
    h = ctypes.c_void_p(1234)
    st = rr.lib().rr_ledger_create(ctypes.byref(cfg(k=0)), ctypes.byref(h))
    assert st == rr.RR_EINVAL and h.value is None
    assert rr.lib().rr_ledger_create(None, ctypes.byref(h)) == rr.RR_EINVAL
    assert rr.lib().rr_ledger_create(ctypes.byref(cfg()), None) == rr.RR_EINVAL


def test_null_ledger_is_rejected_by_every_call():
    L = rr.lib()
    assert L.rr_anchor_route(None, 1, 1, 0, None) == rr.RR_EINVAL
    assert L.rr_relay_layer(None, 1, 1, 1, None, None) == rr.RR_EINVAL
    assert L.rr_ledger_get(None, None, None, None, 1, None) == rr.RR_EINVAL
    assert L.rr_ledger_set(None, 1, 1, 1, 0, 1, None) == rr.RR_EINVAL
    assert L.rr_ledger_config(None, None) == rr.RR_EINVAL
    assert L.rr_ledger_get_refreshed(None, 1, 1, None) == rr.RR_EINVAL
    assert L.rr_ledger_set_refreshed(None, 1, 1, None) == rr.RR_EINVAL
    assert L.rr_ledger_profile(None, 1) == rr.RR_EINVAL
    assert L.rr_ledger_kernel_times(None, None, None) == rr.RR_EINVAL
    assert "NULL" in rr.rr_last_error() or "required" in rr.rr_last_error()
    L.rr_ledger_destroy(None)     # ignored


def test_group_calls_reject_bad_groups_before_any_launch():
    """The width-bucket group calls check the group on the host: NULL arrays or members, sizes
    outside 1 .. RR_GROUP_MAX (nothing is dereferenced or launched for these)."""
    L = rr.lib()
    none2 = (ctypes.c_void_p * 2)(None, None)
    for fn, extra in ((L.rr_anchor_route_group, ()), (L.rr_relay_layer_group, (None,))):
        assert fn(None, 1, 1, 1, 0, None, *extra) == rr.RR_EINVAL and "NULL" in rr.rr_last_error()
        assert fn(none2, 0, 1, 1, 0, None, *extra) == rr.RR_EINVAL and "1 to 4" in rr.rr_last_error()
        assert fn(none2, rr.RR_GROUP_MAX + 1, 1, 1, 0, None, *extra) == rr.RR_EINVAL
        assert fn(none2, 2, 1, 1, 0, None, *extra) == rr.RR_EINVAL and "ledger 0 is NULL" in rr.rr_last_error()


def test_last_error_clears_on_success():
    assert rr.rr_config_check(cfg(k=0)) == rr.RR_EINVAL
    assert rr.rr_last_error() != ""
    assert rr.rr_config_check(cfg()) == rr.RR_OK
    assert rr.rr_last_error() == ""
