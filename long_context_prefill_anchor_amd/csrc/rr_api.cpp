// C ABI of librr.so (declared in include/rr.h): argument validation, ledger ownership and
// the launch sequence of the anchor and relay layers (Sections 4.1-4.2 of "RouteRelay:
// Event-Triggered Cross-Layer Route Reuse for Efficient Dynamic Sparse Attention").
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "rr.h"
#include "rr_internal.h"

struct rr_ledger {
    rr_config cfg;
    int c;        // k + m + sink + recent + r
    int sel;      // k + m
    int G;        // blocks of 64 rows per head
    int device;
    int32_t* ids = nullptr;      // [H, nq, c]
    int32_t* anchor = nullptr;   // [H, nq]
    uint8_t* refreshed = nullptr; // [H, nq] hysteresis state (1 = refreshed at a relay layer)
    int32_t* qmap = nullptr;     // width bucket: [nq] query row of each ledger row (else null)
    int nq_q = 0;                // query rows per head of the Q handed to compute calls
    uint8_t* flags_ws = nullptr; // [H, nq]
    float* hint_ws = nullptr;    // [H, nq]
    int32_t* bcount = nullptr;   // [H, G]
    int32_t* blist = nullptr;    // [H, G, 64]
    int32_t last_layer = -1;
    bool anchored = false;
    bool poisoned = false;
    // Kernel timing (rr_ledger_profile): recorded (kind, start, stop) triples and a pool of
    // spare events.
    struct Timed { int kind; hipEvent_t start, stop; };
    bool profiling = false;
    std::vector<Timed> timed;
    std::vector<hipEvent_t> spare;
};

namespace {

thread_local std::string g_err;

rr_status fail(rr_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
rr_status fail(rr_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

rr_status ok() {
    g_err.clear();
    return RR_OK;
}

rr_status check_cfg(const rr_config* c, bool bucket) {
    if (!c) return fail(RR_EINVAL, "config is NULL");
    if (c->heads < 1 || c->nq < 1 || c->nk < 1)
        return fail(RR_EINVAL, "heads, nq and nk must be >= 1 (got %d, %d, %d)", c->heads, c->nq, c->nk);
    if (c->k < 1 || c->m < 0 || c->r < 0)
        return fail(RR_EINVAL, "need k >= 1, m >= 0, r >= 0 (got %d, %d, %d)", c->k, c->m, c->r);
    if (!(std::isfinite(c->gamma) && c->gamma >= 0.f)) return fail(RR_EINVAL, "gamma must be finite and >= 0");
    if (c->causal != 0 && c->causal != 1) return fail(RR_EINVAL, "causal must be 0 or 1");
    if (c->dtype != RR_F32 && c->dtype != RR_BF16) return fail(RR_EINVAL, "dtype must be RR_F32 or RR_BF16");
    if (c->causal && !bucket && c->nq != c->nk) return fail(RR_EINVAL, "causal routing needs nq == nk");
    if ((int64_t)c->heads * c->nq >= (int64_t)1 << 31 || (int64_t)c->heads * c->nk * 64 >= (int64_t)1 << 40)
        return fail(RR_EINVAL, "problem too large");
    if (c->d != 64) return fail(RR_EUNSUPPORTED, "only d = 64 is implemented (got %d)", c->d);
    if (c->k + c->m > 64) return fail(RR_EUNSUPPORTED, "k + m must be <= 64 (got %d)", c->k + c->m);
    if (c->k + c->m > 32 && c->nk > 1024)
        return fail(RR_EUNSUPPORTED, "k + m > 32 needs nk <= 1024 (got k + m = %d, nk = %d)", c->k + c->m, c->nk);
    if (c->r > 32) return fail(RR_EUNSUPPORTED, "r must be <= 32 (got %d)", c->r);
    if (c->sink < 0 || c->recent < 0)
        return fail(RR_EINVAL, "need sink >= 0, recent >= 0 (got %d, %d)", c->sink, c->recent);
    if (c->sink + c->recent > 32)
        return fail(RR_EUNSUPPORTED, "sink + recent must be <= 32 (got %d)", c->sink + c->recent);
    if (c->min_reuse < 0) return fail(RR_EINVAL, "min_reuse must be >= 0 (got %d)", c->min_reuse);
    if (!(std::isfinite(c->gamma_extra) && c->gamma_extra >= 0.f))
        return fail(RR_EINVAL, "gamma_extra must be finite and >= 0");
    if (c->k + c->m + c->sink + c->recent + c->r > 64)
        return fail(RR_EUNSUPPORTED, "k + m + sink + recent + r must be <= 64 (got %d)",
                    c->k + c->m + c->sink + c->recent + c->r);
    if (c->nk > 4096) return fail(RR_EUNSUPPORTED, "nk must be <= 4096 (got %d)", c->nk);
    if (c->nq > 65536) return fail(RR_EUNSUPPORTED, "nq must be <= 65536 (got %d)", c->nq);
    return RR_OK;
}

rr_status hip_fail(rr_ledger* L, hipError_t e, const char* what) {
    if (L) L->poisoned = true;
    return fail(RR_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

void free_all(rr_ledger* L) {
    (void)hipFree(L->ids);
    (void)hipFree(L->anchor);
    (void)hipFree(L->refreshed);
    (void)hipFree(L->qmap);
    (void)hipFree(L->flags_ws);
    (void)hipFree(L->hint_ws);
    (void)hipFree(L->bcount);
    (void)hipFree(L->blist);
}

hipEvent_t take_event(rr_ledger* L) {
    hipEvent_t ev = nullptr;
    if (!L->spare.empty()) {
        ev = L->spare.back();
        L->spare.pop_back();
    } else if (hipEventCreateWithFlags(&ev, hipEventDisableSystemFence) != hipSuccess) {
        // timing only: no system-scope fence (cache writeback) when the event is recorded
        ev = nullptr;
    }
    return ev;
}

// Record the start of a timed launch; returns the index of its record or -1.
int time_begin(rr_ledger* L, int kind, hipStream_t st) {
    if (!L->profiling) return -1;
    hipEvent_t a = take_event(L), b = take_event(L);
    if (!a || !b || hipEventRecord(a, st) != hipSuccess) {
        if (a) L->spare.push_back(a);
        if (b) L->spare.push_back(b);
        return -1;
    }
    L->timed.push_back({kind, a, b});
    return (int)L->timed.size() - 1;
}

void time_end(rr_ledger* L, int idx, hipStream_t st) {
    if (idx < 0) return;
    if (hipEventRecord(L->timed[idx].stop, st) != hipSuccess) {
        L->spare.push_back(L->timed[idx].start);
        L->spare.push_back(L->timed[idx].stop);
        L->timed.erase(L->timed.begin() + idx);
    }
}

void release_events(rr_ledger* L) {
    for (auto& t : L->timed) {
        (void)hipEventDestroy(t.start);
        (void)hipEventDestroy(t.stop);
    }
    for (auto e : L->spare) (void)hipEventDestroy(e);
    L->timed.clear();
    L->spare.clear();
}

rr::RouteArgs route_args(const rr_ledger* L, const void* q, const void* k, int layer) {
    rr::RouteArgs a{};
    a.qp = q;
    a.kp = k;
    a.ids = L->ids;
    a.anchor = L->anchor;
    a.refreshed = L->refreshed;
    a.qmap = L->qmap;
    a.nq_q = L->nq_q;
    a.flags = L->flags_ws;
    a.hint = L->hint_ws;
    a.bcount = L->bcount;
    a.blist = L->blist;
    a.H = L->cfg.heads;
    a.nq = L->cfg.nq;
    a.nk = L->cfg.nk;
    a.k = L->cfg.k;
    a.m = L->cfg.m;
    a.r = L->cfg.r;
    a.sink = L->cfg.sink;
    a.recent = L->cfg.recent;
    a.c = L->c;
    a.sel = L->sel;
    a.layer = layer;
    a.seed_lo = (uint32_t)(L->cfg.seed & 0xFFFFFFFFull);
    a.seed_hi = (uint32_t)(L->cfg.seed >> 32);
    return a;
}

}  // namespace

extern "C" {

int32_t rr_abi_version(void) { return RR_ABI_VERSION; }

const char* rr_last_error(void) { return g_err.c_str(); }

rr_status rr_config_check(const rr_config* cfg) {
    const rr_status st = check_cfg(cfg, false);
    return st == RR_OK ? ok() : st;
}

}  // extern "C"

namespace {

// Shared by rr_ledger_create and rr_ledger_create_rows (q_rows: validated host array or null).
rr_status create_ledger(const rr_config* cfg, const int32_t* q_rows, int32_t nq_q, rr_ledger** out) {
    rr_ledger* L = new (std::nothrow) rr_ledger;
    if (!L) return fail(RR_ENOMEM, "host allocation failed");
    L->cfg = *cfg;
    L->c = cfg->k + cfg->m + cfg->sink + cfg->recent + cfg->r;
    L->sel = cfg->k + cfg->m;
    L->G = (cfg->nq + rr::ROUTE_ROWS - 1) / rr::ROUTE_ROWS;
    L->nq_q = q_rows ? nq_q : cfg->nq;
    hipError_t e = hipGetDevice(&L->device);
    if (e != hipSuccess) {
        delete L;
        return fail(RR_EDEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    }
    const size_t rows = (size_t)cfg->heads * cfg->nq;
    struct { void** p; size_t bytes; } allocs[] = {
        {(void**)&L->ids, rows * L->c * sizeof(int32_t)},
        {(void**)&L->anchor, rows * sizeof(int32_t)},
        {(void**)&L->flags_ws, rows},
        {(void**)&L->hint_ws, rows * sizeof(float)},
        {(void**)&L->refreshed, rows},
        {(void**)&L->bcount, (size_t)cfg->heads * L->G * sizeof(int32_t)},
        {(void**)&L->blist, (size_t)cfg->heads * L->G * rr::ROUTE_ROWS * sizeof(int32_t)},
        {(void**)&L->qmap, q_rows ? (size_t)cfg->nq * sizeof(int32_t) : 0},
    };
    for (auto& a : allocs) {
        if (a.p == (void**)&L->qmap && !q_rows) continue;
        e = hipMalloc(a.p, a.bytes ? a.bytes : 4);
        if (e != hipSuccess) {
            free_all(L);
            delete L;
            return fail(RR_ENOMEM, "hipMalloc(%zu): %s", a.bytes, hipGetErrorString(e));
        }
    }
    e = hipMemset(L->anchor, 0xFF, rows * sizeof(int32_t));
    if (e == hipSuccess) e = hipMemset(L->ids, 0xFF, rows * L->c * sizeof(int32_t));
    if (e == hipSuccess) e = hipMemset(L->refreshed, 0, rows);
    if (e == hipSuccess && q_rows)
        e = hipMemcpy(L->qmap, q_rows, (size_t)cfg->nq * sizeof(int32_t), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        free_all(L);
        delete L;
        return fail(RR_EDEVICE, "initialising the ledger: %s", hipGetErrorString(e));
    }
    *out = L;
    return ok();
}

}  // namespace

extern "C" {

rr_status rr_ledger_create(const rr_config* cfg, rr_ledger** out) {
    if (!out) return fail(RR_EINVAL, "out is NULL");
    *out = nullptr;
    const rr_status st = check_cfg(cfg, false);
    if (st != RR_OK) return st;
    return create_ledger(cfg, nullptr, 0, out);
}

rr_status rr_ledger_create_rows(const rr_config* cfg, const int32_t* q_rows, int32_t nq_q, rr_ledger** out) {
    if (!out) return fail(RR_EINVAL, "out is NULL");
    *out = nullptr;
    if (!q_rows) return fail(RR_EINVAL, "q_rows is NULL");
    const rr_status st = check_cfg(cfg, true);
    if (st != RR_OK) return st;
    if (nq_q < cfg->nq || nq_q > 65536)
        return fail(RR_EINVAL, "nq_q must be in [nq, 65536] (got %d for nq = %d)", nq_q, cfg->nq);
    if (cfg->causal && nq_q != cfg->nk) return fail(RR_EINVAL, "causal routing needs nq_q == nk");
    for (int r = 0; r < cfg->nq; ++r) {
        if (q_rows[r] < 0 || q_rows[r] >= nq_q || (r > 0 && q_rows[r] <= q_rows[r - 1]))
            return fail(RR_EINVAL, "q_rows must ascend strictly within [0, nq_q) (entry %d = %d)", r, q_rows[r]);
    }
    return create_ledger(cfg, q_rows, nq_q, out);
}

void rr_ledger_destroy(rr_ledger* L) {
    if (!L) return;
    (void)hipDeviceSynchronize();
    release_events(L);
    free_all(L);
    delete L;
}

rr_status rr_ledger_profile(rr_ledger* L, int32_t enable) {
    if (!L) return fail(RR_EINVAL, "ledger is NULL");
    if (enable != 0 && enable != 1) return fail(RR_EINVAL, "enable must be 0 or 1");
    if (enable) {
        for (auto& t : L->timed) {
            (void)hipEventSynchronize(t.stop);
            L->spare.push_back(t.start);
            L->spare.push_back(t.stop);
        }
        L->timed.clear();
    }
    L->profiling = enable != 0;
    return ok();
}

rr_status rr_ledger_kernel_times(rr_ledger* L, int32_t* launches, double* total_ms) {
    if (!L || !launches || !total_ms) return fail(RR_EINVAL, "ledger, launches and total_ms are required");
    for (int i = 0; i < RR_KERNEL_KINDS; ++i) {
        launches[i] = 0;
        total_ms[i] = 0.0;
    }
    hipError_t bad = hipSuccess;
    for (auto& t : L->timed) {
        float ms = 0.f;
        hipError_t e = hipEventSynchronize(t.stop);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.start, t.stop);
        if (e == hipSuccess) {
            launches[t.kind] += 1;
            total_ms[t.kind] += ms;
        } else {
            bad = e;
        }
        L->spare.push_back(t.start);
        L->spare.push_back(t.stop);
    }
    L->timed.clear();
    if (bad != hipSuccess) return fail(RR_EDEVICE, "kernel timing events: %s", hipGetErrorString(bad));
    return ok();
}

rr_status rr_ledger_config(const rr_ledger* L, rr_config* out) {
    if (!L || !out) return fail(RR_EINVAL, "ledger or out is NULL");
    *out = L->cfg;
    return ok();
}

rr_status rr_anchor_route(rr_ledger* L, const void* q, const void* k, int32_t layer, void* stream) {
    if (!L) return fail(RR_EINVAL, "ledger is NULL");
    if (!q || !k) return fail(RR_EINVAL, "q and k must be device pointers");
    if (layer < 0) return fail(RR_EINVAL, "layer must be >= 0 (got %d)", layer);
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    rr::RouteArgs a = route_args(L, q, k, layer);
    a.refresh_mark = 0;
    const int tix = time_begin(L, RR_KERNEL_ROUTE, st);
    // Near-miss sets past the main kernel's 32-entry lists go to the one-wave-per-row kernel.
    const hipError_t e = L->sel > 32 ? rr::launch_route_wide(a, L->cfg.dtype == RR_BF16, L->cfg.causal != 0, false, st)
                                     : rr::launch_route(a, L->cfg.dtype == RR_BF16, L->cfg.causal != 0, false, st);
    time_end(L, tix, st);
    if (e != hipSuccess) return hip_fail(L, e, "anchor route launch");
    L->anchored = true;
    L->poisoned = false;
    L->last_layer = layer;
    return ok();
}

rr_status rr_relay_layer(rr_ledger* L, const void* q, const void* k, int32_t layer, void* stream,
                         const rr_relay_out* out) {
    if (!L) return fail(RR_EINVAL, "ledger is NULL");
    if (L->poisoned) return fail(RR_ESTATE, "ledger is poisoned by an earlier device error; anchor first");
    if (!L->anchored) return fail(RR_ESTATE, "relay layer before any anchor layer");
    if (layer <= L->last_layer)
        return fail(RR_ESTATE, "relay layer %d is not after the last layer %d", layer, L->last_layer);
    if (!q || !k) return fail(RR_EINVAL, "q and k must be device pointers");
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);

    rr::RescoreArgs s{};
    s.qp = q;
    s.kp = k;
    s.ids = L->ids;
    s.flags_ws = L->flags_ws;
    s.hint_ws = L->hint_ws;
    s.bcount = L->bcount;
    s.blist = L->blist;
    s.out_flags = out ? out->flags : nullptr;
    s.out_alpha = out ? out->alpha : nullptr;
    s.out_beta = out ? out->beta : nullptr;
    s.cand_scores = out ? out->cand_scores : nullptr;
    s.H = L->cfg.heads;
    s.nq = L->cfg.nq;
    s.nk = L->cfg.nk;
    s.k = L->cfg.k;
    s.m = L->cfg.m;
    s.r = L->cfg.r;
    s.c = L->c;
    s.sel = L->sel;
    s.gamma = L->cfg.gamma;
    s.anchor = L->anchor;
    s.refreshed = L->refreshed;
    s.qmap = L->qmap;
    s.nq_q = L->nq_q;
    s.layer = layer;
    s.min_reuse = L->cfg.min_reuse;
    s.gamma_extra = L->cfg.gamma_extra;
    int tix = time_begin(L, RR_KERNEL_RESCORE, st);
    hipError_t e = rr::launch_rescore(s, L->cfg.dtype == RR_BF16, st);
    time_end(L, tix, st);
    if (e != hipSuccess) return hip_fail(L, e, "rescore launch");

    rr::RouteArgs a = route_args(L, q, k, layer);
    a.refresh_mark = 1;
    a.out_rows = out ? out->rows : nullptr;
    a.out_head_counts = out ? out->head_counts : nullptr;
    a.out_n_rows = out ? out->n_rows : nullptr;
    tix = time_begin(L, RR_KERNEL_REROUTE, st);
    e = L->sel > 32 ? rr::launch_route_wide(a, L->cfg.dtype == RR_BF16, L->cfg.causal != 0, true, st)
                    : rr::launch_route(a, L->cfg.dtype == RR_BF16, L->cfg.causal != 0, true, st);
    time_end(L, tix, st);
    if (e != hipSuccess) return hip_fail(L, e, "reroute launch");
    L->last_layer = layer;
    return ok();
}

rr_status rr_ledger_get(const rr_ledger* L, int32_t* route, int32_t* sent, int32_t* anchor_layer,
                        int32_t dst_is_host, void* stream) {
    if (!L) return fail(RR_EINVAL, "ledger is NULL");
    if (L->poisoned) return fail(RR_ESTATE, "ledger is poisoned by an earlier device error");
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const hipMemcpyKind kind = dst_is_host ? hipMemcpyDeviceToHost : hipMemcpyDeviceToDevice;
    const size_t rows = (size_t)L->cfg.heads * L->cfg.nq;
    const size_t pitch = (size_t)L->c * sizeof(int32_t);
    hipError_t e = hipSuccess;
    if (route)
        e = hipMemcpy2DAsync(route, L->cfg.k * sizeof(int32_t), L->ids, pitch, L->cfg.k * sizeof(int32_t), rows, kind, st);
    if (e == hipSuccess && sent && (L->c - L->cfg.k) > 0)
        e = hipMemcpy2DAsync(sent, (L->c - L->cfg.k) * sizeof(int32_t), L->ids + L->cfg.k, pitch,
                             (L->c - L->cfg.k) * sizeof(int32_t), rows, kind, st);
    if (e == hipSuccess && anchor_layer)
        e = hipMemcpyAsync(anchor_layer, L->anchor, rows * sizeof(int32_t), kind, st);
    if (e == hipSuccess && dst_is_host) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(RR_EDEVICE, "ledger copy out: %s", hipGetErrorString(e));
    return ok();
}

rr_status rr_ledger_set(rr_ledger* L, const int32_t* route, const int32_t* sent, const int32_t* anchor_layer,
                        int32_t last_layer, int32_t src_is_host, void* stream) {
    if (!L) return fail(RR_EINVAL, "ledger is NULL");
    if (!route || !anchor_layer || (!sent && (L->c - L->cfg.k) > 0))
        return fail(RR_EINVAL, "route, sent and anchor_layer are required");
    if (last_layer < 0) return fail(RR_EINVAL, "last_layer must be >= 0 (got %d)", last_layer);
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const hipMemcpyKind kind = src_is_host ? hipMemcpyHostToDevice : hipMemcpyDeviceToDevice;
    const size_t rows = (size_t)L->cfg.heads * L->cfg.nq;
    const size_t pitch = (size_t)L->c * sizeof(int32_t);
    hipError_t e = hipMemcpy2DAsync(L->ids, pitch, route, L->cfg.k * sizeof(int32_t), L->cfg.k * sizeof(int32_t),
                                    rows, kind, st);
    if (e == hipSuccess && (L->c - L->cfg.k) > 0)
        e = hipMemcpy2DAsync(L->ids + L->cfg.k, pitch, sent, (L->c - L->cfg.k) * sizeof(int32_t),
                             (L->c - L->cfg.k) * sizeof(int32_t), rows, kind, st);
    if (e == hipSuccess) e = hipMemcpyAsync(L->anchor, anchor_layer, rows * sizeof(int32_t), kind, st);
    if (e == hipSuccess) e = hipMemsetAsync(L->refreshed, 0, rows, st);
    if (e == hipSuccess && src_is_host) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(L, e, "ledger copy in");
    L->anchored = true;
    L->poisoned = false;
    L->last_layer = last_layer;
    return ok();
}

rr_status rr_ledger_get_refreshed(const rr_ledger* L, uint8_t* refreshed, int32_t dst_is_host, void* stream) {
    if (!L || !refreshed) return fail(RR_EINVAL, "ledger or refreshed is NULL");
    if (L->poisoned) return fail(RR_ESTATE, "ledger is poisoned by an earlier device error");
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const size_t rows = (size_t)L->cfg.heads * L->cfg.nq;
    hipError_t e = hipMemcpyAsync(refreshed, L->refreshed, rows,
                                  dst_is_host ? hipMemcpyDeviceToHost : hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess && dst_is_host) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(RR_EDEVICE, "hysteresis state copy out: %s", hipGetErrorString(e));
    return ok();
}

rr_status rr_ledger_set_refreshed(rr_ledger* L, const uint8_t* refreshed, int32_t src_is_host, void* stream) {
    if (!L || !refreshed) return fail(RR_EINVAL, "ledger or refreshed is NULL");
    if (L->poisoned) return fail(RR_ESTATE, "ledger is poisoned by an earlier device error");
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const size_t rows = (size_t)L->cfg.heads * L->cfg.nq;
    hipError_t e = hipMemcpyAsync(L->refreshed, refreshed, rows,
                                  src_is_host ? hipMemcpyHostToDevice : hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess && src_is_host) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(L, e, "hysteresis state copy in");
    return ok();
}

rr_status rr_sparse_attention(const void* q, const void* k, const void* vt, const int32_t* routes,
                              int32_t heads, int32_t nq, int32_t nk, int32_t kr, int32_t chunk_tokens,
                              int32_t causal, float* out, void* stream) {
    if (!q || !k || !vt || !routes || !out) return fail(RR_EINVAL, "q, k, vt, routes and out are required");
    if (heads < 1 || nq < 1 || nk < 1 || kr < 1)
        return fail(RR_EINVAL, "heads, nq, nk and kr must be >= 1 (got %d, %d, %d, %d)", heads, nq, nk, kr);
    if (causal != 0 && causal != 1) return fail(RR_EINVAL, "causal must be 0 or 1");
    if (causal && nq != nk) return fail(RR_EINVAL, "causal attention needs nq == nk");
    if (chunk_tokens != 64) return fail(RR_EUNSUPPORTED, "only 64-token chunks are implemented (got %d)", chunk_tokens);
    if (kr > 64) return fail(RR_EUNSUPPORTED, "kr must be <= 64 (got %d)", kr);
    if ((int64_t)heads * nq >= (int64_t)1 << 31 || (int64_t)heads * nk * 64 * 64 >= (int64_t)1 << 40)
        return fail(RR_EINVAL, "problem too large");
    rr::AttnArgs a{};
    a.q = q;
    a.k = k;
    a.vt = vt;
    a.routes = routes;
    a.out = out;
    a.H = heads;
    a.nq = nq;
    a.nk = nk;
    a.kr = kr;
    a.causal = causal;
    const hipError_t e = rr::launch_sparse_attn(a, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(RR_EDEVICE, "sparse attention launch: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"
