"""Thin ctypes binding of librr.so (include/rr.h): same entry points, argument marshalling only.

Every compute step runs in the library's HIP kernels; this module only turns torch
tensors (or raw integers) into device pointers and the current HIP stream.  It raises
``RuntimeError`` when ``librr.so`` is missing; there is no other implementation to fall
back to.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librr.so")

RR_OK, RR_EINVAL, RR_EUNSUPPORTED, RR_ENOMEM, RR_EDEVICE, RR_ESTATE = 0, -1, -2, -3, -4, -5
RR_F32, RR_BF16 = 0, 1
STATUS_NAMES = {0: "RR_OK", -1: "RR_EINVAL", -2: "RR_EUNSUPPORTED", -3: "RR_ENOMEM",
                -4: "RR_EDEVICE", -5: "RR_ESTATE"}

# Entry points declared in include/rr.h, in declaration order.
ENTRY_POINTS = ("rr_config_check", "rr_ledger_create", "rr_ledger_create_rows", "rr_ledger_destroy",
                "rr_anchor_route",
                "rr_relay_layer", "rr_anchor_route_group", "rr_relay_layer_group", "rr_relay_layer_noalloc",
                "rr_ledger_set_relay_mode", "rr_ledger_get", "rr_ledger_validate",
                "rr_ledger_set", "rr_ledger_config",
                "rr_ledger_get_refreshed", "rr_ledger_set_refreshed", "rr_sparse_attention",
                "rr_ledger_profile",
                "rr_ledger_kernel_times", "rr_last_error", "rr_abi_version")
RR_KERNEL_ROUTE, RR_KERNEL_RESCORE, RR_KERNEL_REROUTE, RR_KERNEL_RELAY, RR_KERNEL_LIST = 0, 1, 2, 3, 4
RR_KERNEL_KINDS = 5
RR_RELAY_AUTO, RR_RELAY_FUSED, RR_RELAY_COMPACTED = 0, 1, 2
RR_GROUP_MAX = 4
RELAY_MODES = {"auto": RR_RELAY_AUTO, "fused": RR_RELAY_FUSED, "compacted": RR_RELAY_COMPACTED}


class rr_config(ctypes.Structure):
    _fields_ = [("heads", ctypes.c_int32), ("nq", ctypes.c_int32), ("nk", ctypes.c_int32),
                ("d", ctypes.c_int32), ("k", ctypes.c_int32), ("m", ctypes.c_int32),
                ("r", ctypes.c_int32), ("gamma", ctypes.c_float), ("causal", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("seed", ctypes.c_uint64), ("sink", ctypes.c_int32),
                ("recent", ctypes.c_int32), ("min_reuse", ctypes.c_int32), ("gamma_extra", ctypes.c_float)]


class rr_relay_out(ctypes.Structure):
    _fields_ = [("flags", ctypes.c_void_p), ("rows", ctypes.c_void_p),
                ("head_counts", ctypes.c_void_p), ("n_rows", ctypes.c_void_p),
                ("alpha", ctypes.c_void_p), ("beta", ctypes.c_void_p),
                ("cand_scores", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m long_context_prefill_anchor_amd.build`")
        # torch's HIP runtime must see the devices before this library's first HIP call; bring
        # it up first, whatever the caller imported or called before.
        import torch
        torch.cuda.is_available()
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, P = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER
        L.rr_config_check.argtypes = [P(rr_config)]
        L.rr_ledger_create.argtypes = [P(rr_config), P(vp)]
        L.rr_ledger_create_rows.argtypes = [P(rr_config), P(i32), i32, P(vp)]
        L.rr_ledger_destroy.argtypes = [vp]
        L.rr_ledger_destroy.restype = None
        L.rr_anchor_route.argtypes = [vp, vp, vp, i32, vp]
        L.rr_relay_layer.argtypes = [vp, vp, vp, i32, vp, P(rr_relay_out)]
        L.rr_anchor_route_group.argtypes = [P(vp), i32, vp, vp, i32, vp]
        L.rr_relay_layer_group.argtypes = [P(vp), i32, vp, vp, i32, vp, P(P(rr_relay_out))]
        L.rr_ledger_set_relay_mode.argtypes = [vp, i32]
        L.rr_relay_layer_noalloc.argtypes = [P(rr_config), vp, vp, vp, vp, vp, i32, vp, P(rr_relay_out)]
        L.rr_ledger_get.argtypes = [vp, vp, vp, vp, i32, vp]
        L.rr_ledger_validate.argtypes = [P(rr_config), P(i32), i32, vp, vp, vp, i32]
        L.rr_ledger_set.argtypes = [vp, vp, vp, vp, i32, i32, vp]
        L.rr_ledger_config.argtypes = [vp, P(rr_config)]
        L.rr_ledger_get_refreshed.argtypes = [vp, vp, i32, vp]
        L.rr_sparse_attention.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp]
        L.rr_ledger_set_refreshed.argtypes = [vp, vp, i32, vp]
        L.rr_ledger_profile.argtypes = [vp, i32]
        L.rr_ledger_kernel_times.argtypes = [vp, P(i32), P(ctypes.c_double)]
        L.rr_last_error.restype = ctypes.c_char_p
        L.rr_last_error.argtypes = []
        L.rr_abi_version.restype = i32
        L.rr_abi_version.argtypes = []
        for name in ENTRY_POINTS:
            fn = getattr(L, name)
            if fn.restype is ctypes.c_int:
                fn.restype = i32
        _lib = L
    return _lib


class RRError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().rr_last_error().decode()
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")


def _check(status: int, where: str) -> None:
    if status != RR_OK:
        raise RRError(status, where)


def _ptr(x) -> Optional[int]:
    """Device (or host) address of a tensor, a contiguous NumPy array or a raw int; None stays
    None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if not x.flags["C_CONTIGUOUS"]:
        raise ValueError("host arrays must be C-contiguous")
    return x.ctypes.data


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_config(heads, nq, nk, d=64, k=12, m=12, r=8, gamma=0.0, causal=False,
                dtype="bf16", seed=0, sink=0, recent=0, min_reuse=0, gamma_extra=0.0) -> rr_config:
    return rr_config(heads, nq, nk, d, k, m, r, float(gamma), int(bool(causal)),
                     RR_BF16 if dtype == "bf16" else RR_F32, int(seed) & (2**64 - 1),
                     int(sink), int(recent), int(min_reuse), float(gamma_extra))


# ------------------------------------------------------------------------- raw entry points

def rr_config_check(cfg: rr_config) -> int:
    return lib().rr_config_check(ctypes.byref(cfg))


def rr_ledger_create(cfg: rr_config) -> int:
    h = ctypes.c_void_p()
    _check(lib().rr_ledger_create(ctypes.byref(cfg), ctypes.byref(h)), "rr_ledger_create")
    return h.value


def rr_ledger_create_rows(cfg: rr_config, q_rows, nq_q: int) -> int:
    rows = (ctypes.c_int32 * len(q_rows))(*[int(x) for x in q_rows])
    h = ctypes.c_void_p()
    _check(lib().rr_ledger_create_rows(ctypes.byref(cfg), rows, int(nq_q), ctypes.byref(h)),
           "rr_ledger_create_rows")
    return h.value


def rr_ledger_destroy(handle: int) -> None:
    lib().rr_ledger_destroy(handle)


def rr_anchor_route(handle, q, k, layer: int, stream=None) -> None:
    _check(lib().rr_anchor_route(handle, _ptr(q), _ptr(k), int(layer), _stream(stream)),
           "rr_anchor_route")


def rr_relay_layer(handle, q, k, layer: int, stream=None, flags=None, rows=None, head_counts=None,
                   n_rows=None, alpha=None, beta=None, cand_scores=None, out: bool = True) -> None:
    o = rr_relay_out(_ptr(flags), _ptr(rows), _ptr(head_counts), _ptr(n_rows), _ptr(alpha),
                     _ptr(beta), _ptr(cand_scores))
    _check(lib().rr_relay_layer(handle, _ptr(q), _ptr(k), int(layer), _stream(stream),
                                ctypes.byref(o) if out else None), "rr_relay_layer")


def _handles(handles):
    return (ctypes.c_void_p * max(1, len(handles)))(*[h for h in handles]), len(handles)


def rr_anchor_route_group(handles, q, k, layer: int, stream=None) -> None:
    arr, n = _handles(handles)
    _check(lib().rr_anchor_route_group(arr, n, _ptr(q), _ptr(k), int(layer), _stream(stream)),
           "rr_anchor_route_group")


def rr_relay_layer_group(handles, q, k, layer: int, stream=None, outs=None) -> None:
    """outs: None, or one rr_relay_out (or None) per ledger."""
    arr, n = _handles(handles)
    po = None
    if outs is not None:
        po = (ctypes.POINTER(rr_relay_out) * max(1, len(outs)))(
            *[ctypes.pointer(o) if o is not None else ctypes.POINTER(rr_relay_out)() for o in outs])
    _check(lib().rr_relay_layer_group(arr, n, _ptr(q), _ptr(k), int(layer), _stream(stream), po),
           "rr_relay_layer_group")


def rr_relay_layer_noalloc(cfg: rr_config, ids, anchor_layer, refreshed, q, k, layer: int, stream=None,
                           flags=None, rows=None, head_counts=None, n_rows=None, alpha=None, beta=None,
                           cand_scores=None, out: bool = True) -> None:
    o = rr_relay_out(_ptr(flags), _ptr(rows), _ptr(head_counts), _ptr(n_rows), _ptr(alpha),
                     _ptr(beta), _ptr(cand_scores))
    _check(lib().rr_relay_layer_noalloc(ctypes.byref(cfg), _ptr(ids), _ptr(anchor_layer), _ptr(refreshed),
                                        _ptr(q), _ptr(k), int(layer), _stream(stream),
                                        ctypes.byref(o) if out else None), "rr_relay_layer_noalloc")


def rr_ledger_set_relay_mode(handle, mode) -> None:
    """mode: RR_RELAY_AUTO / _FUSED / _COMPACTED, or "auto" / "fused" / "compacted"."""
    m = RELAY_MODES[mode] if isinstance(mode, str) else int(mode)
    _check(lib().rr_ledger_set_relay_mode(handle, m), "rr_ledger_set_relay_mode")


def rr_ledger_get(handle, route, sent, anchor_layer, dst_is_host: bool, stream=None) -> None:
    _check(lib().rr_ledger_get(handle, _ptr(route), _ptr(sent), _ptr(anchor_layer),
                               int(bool(dst_is_host)), _stream(stream)), "rr_ledger_get")


def rr_ledger_validate(cfg: rr_config, route, sent, anchor_layer, last_layer: int, q_rows=None,
                       nq_q: int = 0) -> None:
    """Host-memory check of ledger tensors (numpy int32 arrays, rr_ledger_get layout); raises
    RRError naming the first offending row."""
    import numpy as np
    arrs = [None if x is None else np.ascontiguousarray(x, dtype=np.int32) for x in (route, sent, anchor_layer)]
    rows = None
    if q_rows is not None:
        rows = (ctypes.c_int32 * len(q_rows))(*[int(x) for x in q_rows])
    ptr = [None if a is None or a.size == 0 else a.ctypes.data for a in arrs]
    _check(lib().rr_ledger_validate(ctypes.byref(cfg), rows, int(nq_q), ptr[0], ptr[1], ptr[2], int(last_layer)),
           "rr_ledger_validate")


def rr_ledger_set(handle, route, sent, anchor_layer, last_layer: int, src_is_host: bool,
                  stream=None) -> None:
    _check(lib().rr_ledger_set(handle, _ptr(route), _ptr(sent), _ptr(anchor_layer),
                               int(last_layer), int(bool(src_is_host)), _stream(stream)),
           "rr_ledger_set")


def rr_ledger_get_refreshed(handle, refreshed, dst_is_host: bool, stream=None) -> None:
    _check(lib().rr_ledger_get_refreshed(handle, _ptr(refreshed), int(bool(dst_is_host)), _stream(stream)),
           "rr_ledger_get_refreshed")


def rr_ledger_set_refreshed(handle, refreshed, src_is_host: bool, stream=None) -> None:
    _check(lib().rr_ledger_set_refreshed(handle, _ptr(refreshed), int(bool(src_is_host)), _stream(stream)),
           "rr_ledger_set_refreshed")


def rr_sparse_attention(q, k, vt, routes, heads: int, nq: int, nk: int, kr: int, out,
                        causal: bool = False, chunk_tokens: int = 64, stream=None) -> None:
    _check(lib().rr_sparse_attention(_ptr(q), _ptr(k), _ptr(vt), _ptr(routes), int(heads), int(nq),
                                     int(nk), int(kr), int(chunk_tokens), int(bool(causal)), _ptr(out),
                                     _stream(stream)), "rr_sparse_attention")


def rr_ledger_profile(handle, enable: bool) -> None:
    _check(lib().rr_ledger_profile(handle, int(bool(enable))), "rr_ledger_profile")


def rr_ledger_kernel_times(handle):
    """[(launches, total_ms)] indexed by RR_KERNEL_ROUTE / _RESCORE / _REROUTE / _RELAY / _LIST."""
    n = (ctypes.c_int32 * RR_KERNEL_KINDS)()
    ms = (ctypes.c_double * RR_KERNEL_KINDS)()
    _check(lib().rr_ledger_kernel_times(handle, n, ms), "rr_ledger_kernel_times")
    return [(int(n[i]), float(ms[i])) for i in range(RR_KERNEL_KINDS)]


def rr_last_error() -> str:
    return lib().rr_last_error().decode()


def rr_abi_version() -> int:
    return lib().rr_abi_version()


# ------------------------------------------------------------------------- convenience wrapper

@dataclass
class RelayOutputs:
    flags: object
    rows: object
    head_counts: object
    n_rows: object
    alpha: object
    beta: object
    cand_scores: object


class Ledger:
    """Owns one rr_ledger handle; torch tensors in, torch tensors out (device memory only)."""

    def __init__(self, heads, nq, nk, d=64, k=12, m=12, r=8, gamma=0.0, causal=False,
                 dtype="bf16", seed=0, sink=0, recent=0, min_reuse=0, gamma_extra=0.0,
                 q_rows=None):
        """``q_rows``: a width bucket over these query rows (ascending) of a Q with ``nq``
        rows per head; the ledger then has len(q_rows) rows."""
        self.q_rows = None if q_rows is None else tuple(int(x) for x in q_rows)
        self.nq_q = nq
        if self.q_rows is not None:
            nq = len(self.q_rows)
        self.cfg = make_config(heads, nq, nk, d, k, m, r, gamma, causal, dtype, seed, sink, recent,
                               min_reuse, gamma_extra)
        self.min_reuse, self.gamma_extra = min_reuse, gamma_extra
        self.heads, self.nq, self.nk, self.k, self.m, self.r = heads, nq, nk, k, m, r
        self.sink, self.recent = sink, recent
        self.c = k + m + sink + recent + r
        if self.q_rows is None:
            self.handle = rr_ledger_create(self.cfg)
        else:
            self.handle = rr_ledger_create_rows(self.cfg, self.q_rows, self.nq_q)

    def close(self):
        if getattr(self, "handle", None):
            rr_ledger_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def anchor(self, q, k, layer, stream=None):
        rr_anchor_route(self.handle, q, k, layer, stream)

    def set_relay_mode(self, mode):
        """"auto", "fused" or "compacted" (see rr_ledger_set_relay_mode in include/rr.h)."""
        rr_ledger_set_relay_mode(self.handle, mode)

    def alloc_outputs(self, device="cuda", with_scores=True) -> RelayOutputs:
        import torch
        H, nq = self.heads, self.nq
        return RelayOutputs(
            flags=torch.zeros(H * nq, dtype=torch.uint8, device=device),
            rows=torch.full((H * nq,), -1, dtype=torch.int32, device=device),
            head_counts=torch.zeros(H, dtype=torch.int32, device=device),
            n_rows=torch.zeros(1, dtype=torch.int32, device=device),
            alpha=torch.zeros(H * nq, dtype=torch.float32, device=device),
            beta=torch.zeros(H * nq, dtype=torch.float32, device=device),
            cand_scores=(torch.zeros(H * nq * self.c, dtype=torch.float32, device=device)
                         if with_scores else None))

    def relay(self, q, k, layer, out: Optional[RelayOutputs] = None, stream=None):
        if out is None:
            rr_relay_layer(self.handle, q, k, layer, stream, out=False)
        else:
            rr_relay_layer(self.handle, q, k, layer, stream, out.flags, out.rows, out.head_counts,
                           out.n_rows, out.alpha, out.beta, out.cand_scores)

    def out_struct(self, out: Optional[RelayOutputs]):
        if out is None:
            return None
        return rr_relay_out(_ptr(out.flags), _ptr(out.rows), _ptr(out.head_counts), _ptr(out.n_rows),
                            _ptr(out.alpha), _ptr(out.beta), _ptr(out.cand_scores))

    def get(self, stream=None):
        """(route [H,nq,k], sent [H,nq,c-k], anchor [H,nq]) as device int32 tensors."""
        import torch
        H, nq = self.heads, self.nq
        route = torch.empty((H, nq, self.k), dtype=torch.int32, device="cuda")
        sent = torch.empty((H, nq, self.c - self.k), dtype=torch.int32, device="cuda")
        anchor = torch.empty((H, nq), dtype=torch.int32, device="cuda")
        rr_ledger_get(self.handle, route, sent if self.c > self.k else None, anchor, False, stream)
        return route, sent, anchor

    def get_refreshed(self, stream=None):
        """Hysteresis state [H, nq] as a device uint8 tensor."""
        import torch
        out = torch.empty((self.heads, self.nq), dtype=torch.uint8, device="cuda")
        rr_ledger_get_refreshed(self.handle, out, False, stream)
        return out

    def set_refreshed(self, refreshed, stream=None):
        rr_ledger_set_refreshed(self.handle, refreshed, False, stream)

    def profile(self, enable=True):
        rr_ledger_profile(self.handle, enable)

    def kernel_times(self):
        return rr_ledger_kernel_times(self.handle)

    def set(self, route, sent, anchor, last_layer, stream=None):
        rr_ledger_set(self.handle, route, sent if self.c > self.k else None, anchor, last_layer,
                      False, stream)


class LedgerGroup:
    """Width-bucket ledgers (Ledger objects over the same Q and K) advanced together, one launch
    per layer where the kernels allow it (rr_anchor_route_group / rr_relay_layer_group)."""

    def __init__(self, ledgers):
        self.ledgers = list(ledgers)

    def anchor(self, q, k, layer, stream=None):
        rr_anchor_route_group([x.handle for x in self.ledgers], q, k, layer, stream)

    def relay(self, q, k, layer, outs=None, stream=None):
        """outs: None, or one RelayOutputs (or None) per ledger."""
        structs = None if outs is None else [x.out_struct(o) for x, o in zip(self.ledgers, outs)]
        rr_relay_layer_group([x.handle for x in self.ledgers], q, k, layer, stream, structs)
