// C ABI of librr.so (declared in include/rr.h): argument validation, ledger ownership and
// the launch sequence of the anchor and relay layers (Sections 4.1-4.2 of "RouteRelay:
// Event-Triggered Cross-Layer Route Reuse for Efficient Dynamic Sparse Attention").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "rr.h"
#include "rr_internal.h"

// Working memory of rr_relay_layer_noalloc: the relay kernels' refresh flags (1 byte per row),
// reroute thresholds (4), per-block flagged-row lists (4) and per-block counts (4 per 64 rows),
// for at most NOALLOC_MAX_ROWS rows (heads * ceil(nq / 64) * 64).  One copy per GPU, held until
// the process ends; host code reaches it only through the address hipGetSymbolAddress returns.
constexpr size_t NOALLOC_MAX_ROWS = size_t(1) << 18;
constexpr size_t NOALLOC_SCRATCH_BYTES = NOALLOC_MAX_ROWS * (1 + 4 + 4) + NOALLOC_MAX_ROWS / 64 * 4;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

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
    std::vector<int32_t> qmap_host;  // the same on the host (snapshot checks)
    int nq_q = 0;                // query rows per head of the Q handed to compute calls
    uint8_t* flags_ws = nullptr; // [H, nq]
    float* hint_ws = nullptr;    // [H, nq]
    int32_t* bcount = nullptr;   // [H, G]
    int32_t* blist = nullptr;    // [H, G, 64]
    int32_t relay_mode = RR_RELAY_AUTO;
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
    if (c->k + c->m + c->sink + c->recent + c->r > 128)
        return fail(RR_EUNSUPPORTED, "k + m + sink + recent + r must be <= 128 (got %d)",
                    c->k + c->m + c->sink + c->recent + c->r);
    if (c->nk > 16384) return fail(RR_EUNSUPPORTED, "nk must be <= 16384 (got %d)", c->nk);
    {
        const int ids = c->k + c->m + c->sink + c->recent + c->r;
        if (!rr::route_fits(c->nk, ids))
            return fail(RR_EUNSUPPORTED,
                        "nk = %d with %d ledger IDs per row exceeds the route kernel's LDS (per-row sentinel "
                        "bitmaps of nk bits and staging rows of c IDs in 160 KB)", c->nk, ids);
    }
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

// Fused relay layers serve layers of FUSED_MIN_BLOCKS .. FUSED_MAX_BLOCKS 128-row blocks (half
// to two of them per compute unit): there the fixed latency of a reroute block, not its work,
// sets the time, and one launch per layer that rescores from LDS beats the two-kernel schedule.
// Smaller layers leave most of the GPU idle, and a fused block's serial rescore-then-reroute
// chain is longer than the two short launches of the compacted schedule (measured: one head of
// 128-1024 chunks, 2-7 us per layer in favour of the compacted schedule; 32 heads x 1024 chunks,
// 2 us in favour of the fused one).
constexpr long long FUSED_MIN_BLOCKS = 128;
constexpr long long FUSED_MAX_BLOCKS = 512;

// Non-owning view of a ledger's device state and of the working memory a relay layer's kernels
// use: taken from an rr_ledger, or from caller memory and the fixed scratch array
// (rr_relay_layer_noalloc).
struct LedgerView {
    rr_config cfg;
    int c, sel, nq_q;
    int32_t relay_mode;
    int32_t* ids;
    int32_t* anchor;
    uint8_t* refreshed;
    const int32_t* qmap;
    uint8_t* flags_ws;
    float* hint_ws;
    int32_t* bcount;
    int32_t* blist;
};

LedgerView view_of(const rr_ledger* L) {
    return LedgerView{L->cfg, L->c, L->sel, L->nq_q, L->relay_mode, L->ids, L->anchor, L->refreshed, L->qmap,
                      L->flags_ws, L->hint_ws, L->bcount, L->blist};
}

bool fused_fits(const LedgerView& v) {
    return rr::relay_fits(v.cfg.nk, v.c, v.sel, v.cfg.dtype == RR_BF16);
}

bool use_fused(const LedgerView& v) {
    if (!fused_fits(v)) return false;
    if (v.relay_mode != RR_RELAY_AUTO) return v.relay_mode == RR_RELAY_FUSED;
    const long long blocks = (long long)v.cfg.heads * ((v.cfg.nq + 127) / 128);
    return blocks >= FUSED_MIN_BLOCKS && blocks <= FUSED_MAX_BLOCKS;
}

rr::RouteArgs route_args(const LedgerView& v, const void* q, const void* k, int layer) {
    rr::RouteArgs a{};
    a.qp = q;
    a.kp = k;
    a.ids = v.ids;
    a.anchor = v.anchor;
    a.refreshed = v.refreshed;
    a.qmap = v.qmap;
    a.nq_q = v.nq_q;
    a.flags = v.flags_ws;
    a.hint = v.hint_ws;
    a.bcount = v.bcount;
    a.blist = v.blist;
    a.H = v.cfg.heads;
    a.nq = v.cfg.nq;
    a.nk = v.cfg.nk;
    a.k = v.cfg.k;
    a.m = v.cfg.m;
    a.r = v.cfg.r;
    a.sink = v.cfg.sink;
    a.recent = v.cfg.recent;
    a.c = v.c;
    a.sel = v.sel;
    a.layer = layer;
    a.seed_lo = (uint32_t)(v.cfg.seed & 0xFFFFFFFFull);
    a.seed_hi = (uint32_t)(v.cfg.seed >> 32);
    return a;
}

rr::RouteArgs route_args(const rr_ledger* L, const void* q, const void* k, int layer) {
    return route_args(view_of(L), q, k, layer);
}

// Device address of this GPU's copy of `scratch`, looked up once per device with that device
// current (each GPU holds its own copy at its own address; in host code the array's name is
// not a device address).
constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[NOALLOC_MAX_DEVICES] = {};

rr_status scratch_for_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(RR_EDEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return fail(RR_EUNSUPPORTED, "device %d past the scratch table", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(RR_EDEVICE, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return RR_OK;
}

// The launch sequence of one relay layer (Sections 3.2, 4.1, 4.2) on a view: the fused relay
// kernel (plus the compacted-list kernel when those outputs are asked for), or the rescoring
// kernel then the reroute of the compacted rows.  `T`: ledger whose profiling records the
// launches (null: none).  On failure *what names the launch.
rr::RescoreArgs rescore_args(const LedgerView& v, const void* q, const void* k, int32_t layer,
                             const rr_relay_out* out) {
    rr::RescoreArgs s{};
    s.qp = q;
    s.kp = k;
    s.ids = v.ids;
    s.flags_ws = v.flags_ws;
    s.hint_ws = v.hint_ws;
    s.bcount = v.bcount;
    s.blist = v.blist;
    s.out_flags = out ? out->flags : nullptr;
    s.out_alpha = out ? out->alpha : nullptr;
    s.out_beta = out ? out->beta : nullptr;
    s.cand_scores = out ? out->cand_scores : nullptr;
    s.H = v.cfg.heads;
    s.nq = v.cfg.nq;
    s.nk = v.cfg.nk;
    s.k = v.cfg.k;
    s.m = v.cfg.m;
    s.r = v.cfg.r;
    s.c = v.c;
    s.sel = v.sel;
    s.gamma = v.cfg.gamma;
    s.anchor = v.anchor;
    s.refreshed = v.refreshed;
    s.qmap = v.qmap;
    s.nq_q = v.nq_q;
    s.layer = layer;
    s.min_reuse = v.cfg.min_reuse;
    s.gamma_extra = v.cfg.gamma_extra;
    return s;
}

bool wants_list(const rr_relay_out* out) { return out && (out->rows || out->head_counts || out->n_rows); }

hipError_t relay_launch(const LedgerView& v, const void* q, const void* k, int32_t layer, hipStream_t st,
                        const rr_relay_out* out, rr_ledger* T, const char** what) {
    const rr::RescoreArgs s = rescore_args(v, q, k, layer, out);
    rr::RouteArgs a = route_args(v, q, k, layer);
    a.refresh_mark = 1;
    const bool bf16 = v.cfg.dtype == RR_BF16, causal = v.cfg.causal != 0;
    const bool timed = T != nullptr;
    if (use_fused(v)) {
        int tix = timed ? time_begin(T, RR_KERNEL_RELAY, st) : -1;
        hipError_t e = rr::launch_relay(s, a, bf16, causal, st);
        if (timed) time_end(T, tix, st);
        if (e != hipSuccess) {
            *what = "relay launch";
            return e;
        }
        if (wants_list(out)) {
            tix = timed ? time_begin(T, RR_KERNEL_LIST, st) : -1;
            e = rr::launch_compact_out(v.bcount, v.blist, v.cfg.heads, v.cfg.nq, out->rows, out->head_counts,
                                       out->n_rows, st);
            if (timed) time_end(T, tix, st);
            if (e != hipSuccess) {
                *what = "compacted-list launch";
                return e;
            }
        }
        return hipSuccess;
    }
    int tix = timed ? time_begin(T, RR_KERNEL_RESCORE, st) : -1;
    hipError_t e = rr::launch_rescore(s, bf16, st);
    if (timed) time_end(T, tix, st);
    if (e != hipSuccess) {
        *what = "rescore launch";
        return e;
    }
    a.out_rows = out ? out->rows : nullptr;
    a.out_head_counts = out ? out->head_counts : nullptr;
    a.out_n_rows = out ? out->n_rows : nullptr;
    tix = timed ? time_begin(T, RR_KERNEL_REROUTE, st) : -1;
    e = v.sel > 32 ? rr::launch_route_wide(a, bf16, causal, true, st) : rr::launch_route(a, bf16, causal, true, st);
    if (timed) time_end(T, tix, st);
    if (e != hipSuccess) *what = "reroute launch";
    return e;
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

// Host check of ledger IDs (Section 4.1's three tensors, layout of rr_ledger_get) against the
// rules every routing call leaves them in, row by row: each segment ascending with -1 padding
// only at its end; IDs inside the row's allowed range [0, n_i) (n_i = query row + 1 under the
// causal mask, else nk) and distinct across the row's segments; a full route (min(k, n_i)
// IDs) and near-miss segment (min(m, n_i - k_i)); mandatory IDs among the sink chunks or the
// row's last `recent` allowed chunks; min(r, pool) random IDs; anchor layers in [0, last_layer].
rr_status check_ledger_ids(const rr_config& c, const int32_t* q_rows, const int32_t* route, const int32_t* sent,
                           const int32_t* anchor_layer, int32_t last_layer) {
    const int cc = c.k + c.m + c.sink + c.recent + c.r;
    const int ns = cc - c.k;
    const int seg_len[4] = {c.k, c.m, c.sink + c.recent, c.r};
    const char* seg_name[4] = {"route", "near-miss", "mandatory", "random"};
    std::vector<uint32_t> seen((size_t)c.nk, 0u);
    uint32_t stamp = 0;
    for (int h = 0; h < c.heads; ++h) {
        for (int i = 0; i < c.nq; ++i) {
            const size_t flat = (size_t)h * c.nq + i;
            const int qrow = q_rows ? q_rows[i] : i;
            const int n = c.causal ? qrow + 1 : c.nk;
            const int a = anchor_layer[flat];
            if (a < 0 || a > last_layer)
                return fail(RR_EINVAL, "head %d row %d: anchor layer %d outside [0, %d]", h, i, a, last_layer);
            ++stamp;
            const int ki = std::min(c.k, n), mi = std::min(c.m, n - ki);
            int count[4] = {0, 0, 0, 0};
            int pos = 0;
            for (int sg = 0; sg < 4; ++sg) {
                int prev = -1;
                bool padded = false;
                for (int t = 0; t < seg_len[sg]; ++t, ++pos) {
                    const int id = pos < c.k ? route[flat * c.k + pos] : sent[flat * ns + (pos - c.k)];
                    if (id == -1) {
                        padded = true;
                        continue;
                    }
                    if (padded)
                        return fail(RR_EINVAL, "head %d row %d: %s ID %d after -1 padding", h, i, seg_name[sg], id);
                    if (id < 0 || id >= n)
                        return fail(RR_EINVAL, "head %d row %d: %s ID %d outside the allowed chunks [0, %d)", h, i,
                                    seg_name[sg], id, n);
                    if (id <= prev)
                        return fail(RR_EINVAL, "head %d row %d: %s segment not ascending (%d after %d)", h, i,
                                    seg_name[sg], id, prev);
                    if (seen[id] == stamp) return fail(RR_EINVAL, "head %d row %d: chunk %d appears twice", h, i, id);
                    if (sg == 2 && !(id < c.sink || id >= n - c.recent))
                        return fail(RR_EINVAL, "head %d row %d: mandatory ID %d is neither a sink nor a recent chunk",
                                    h, i, id);
                    seen[id] = stamp;
                    prev = id;
                    ++count[sg];
                }
            }
            const int rwant = std::min(c.r, n - ki - mi - count[2]);
            if (count[0] != ki || count[1] != mi || count[3] != rwant)
                return fail(RR_EINVAL, "head %d row %d: %d route, %d near-miss and %d random IDs where the row holds "
                            "%d, %d and %d", h, i, count[0], count[1], count[3], ki, mi, rwant);
        }
    }
    return RR_OK;
}

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
    if (e == hipSuccess && q_rows) {
        e = hipMemcpy(L->qmap, q_rows, (size_t)cfg->nq * sizeof(int32_t), hipMemcpyHostToDevice);
        L->qmap_host.assign(q_rows, q_rows + cfg->nq);
    }
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

rr_status rr_ledger_validate(const rr_config* cfg, const int32_t* q_rows, int32_t nq_q, const int32_t* route,
                             const int32_t* sent, const int32_t* anchor_layer, int32_t last_layer) {
    const rr_status st = check_cfg(cfg, q_rows != nullptr);
    if (st != RR_OK) return st;
    const int c = cfg->k + cfg->m + cfg->sink + cfg->recent + cfg->r;
    if (!route || !anchor_layer || (!sent && c > cfg->k))
        return fail(RR_EINVAL, "route, sent and anchor_layer are required");
    if (last_layer < 0) return fail(RR_EINVAL, "last_layer must be >= 0 (got %d)", last_layer);
    if (q_rows) {
        if (nq_q < cfg->nq || nq_q > 65536)
            return fail(RR_EINVAL, "nq_q must be in [nq, 65536] (got %d for nq = %d)", nq_q, cfg->nq);
        if (cfg->causal && nq_q != cfg->nk) return fail(RR_EINVAL, "causal routing needs nq_q == nk");
        for (int r = 0; r < cfg->nq; ++r) {
            if (q_rows[r] < 0 || q_rows[r] >= nq_q || (r > 0 && q_rows[r] <= q_rows[r - 1]))
                return fail(RR_EINVAL, "q_rows must ascend strictly within [0, nq_q) (entry %d = %d)", r, q_rows[r]);
        }
    }
    const rr_status v = check_ledger_ids(*cfg, q_rows, route, sent, anchor_layer, last_layer);
    return v == RR_OK ? ok() : v;
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
    const char* what = "";
    const hipError_t e = relay_launch(view_of(L), q, k, layer, st, out, L, &what);
    if (e != hipSuccess) return hip_fail(L, e, what);
    L->last_layer = layer;
    return ok();
}

}  // extern "C"

namespace {

// A width-bucket group: 1 .. RR_GROUP_MAX distinct ledgers over the same Q and K (same heads,
// nk, element type, causal mask, query rows per head and device).
rr_status check_group(rr_ledger* const* L, int32_t n, const void* q, const void* k, int32_t layer) {
    if (!L) return fail(RR_EINVAL, "ledgers is NULL");
    if (n < 1 || n > RR_GROUP_MAX) return fail(RR_EINVAL, "a group holds 1 to %d ledgers (got %d)", RR_GROUP_MAX, n);
    for (int b = 0; b < n; ++b) {
        if (!L[b]) return fail(RR_EINVAL, "ledger %d is NULL", b);
        for (int a = 0; a < b; ++a)
            if (L[a] == L[b]) return fail(RR_EINVAL, "ledger %d appears twice in the group", b);
        const rr_config& c0 = L[0]->cfg;
        const rr_config& c = L[b]->cfg;
        if (c.heads != c0.heads || c.nk != c0.nk || c.dtype != c0.dtype || c.causal != c0.causal ||
            L[b]->nq_q != L[0]->nq_q || L[b]->device != L[0]->device)
            return fail(RR_EINVAL, "ledger %d differs from ledger 0 in heads, nk, dtype, causal, query rows or device", b);
    }
    if (!q || !k) return fail(RR_EINVAL, "q and k must be device pointers");
    if (layer < 0) return fail(RR_EINVAL, "layer must be >= 0 (got %d)", layer);
    return RR_OK;
}

rr_status group_launch_failed(rr_ledger* const* L, int32_t n, hipError_t e, const char* what) {
    for (int b = 1; b < n; ++b) L[b]->poisoned = true;
    return hip_fail(L[0], e, what);
}

}  // namespace

extern "C" {

rr_status rr_anchor_route_group(rr_ledger* const* L, int32_t n, const void* q, const void* k, int32_t layer,
                                void* stream) {
    const rr_status st0 = check_group(L, n, q, k, layer);
    if (st0 != RR_OK) return st0;
    bool one_grid = n > 1;
    for (int b = 0; b < n; ++b) one_grid = one_grid && L[b]->sel <= 32;
    if (!one_grid) {
        for (int b = 0; b < n; ++b) {
            const rr_status e = rr_anchor_route(L[b], q, k, layer, stream);
            if (e != RR_OK) return e;
        }
        return ok();
    }
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    rr::RouteGroup g{};
    g.n = n;
    for (int b = 0; b < n; ++b) {
        g.p[b] = route_args(L[b], q, k, layer);
        g.p[b].refresh_mark = 0;
        g.off[b + 1] = g.off[b] + (L[b]->cfg.nq + rr::ROUTE_ROWS - 1) / rr::ROUTE_ROWS;
    }
    g.per_head = g.off[n];
    int tix[RR_GROUP_MAX];
    for (int b = 0; b < n; ++b) tix[b] = time_begin(L[b], RR_KERNEL_ROUTE, st);
    const hipError_t e = rr::launch_route_group(g, L[0]->cfg.dtype == RR_BF16, L[0]->cfg.causal != 0, st);
    for (int b = 0; b < n; ++b) time_end(L[b], tix[b], st);
    if (e != hipSuccess) return group_launch_failed(L, n, e, "grouped anchor route launch");
    for (int b = 0; b < n; ++b) {
        L[b]->anchored = true;
        L[b]->poisoned = false;
        L[b]->last_layer = layer;
    }
    return ok();
}

rr_status rr_relay_layer_group(rr_ledger* const* L, int32_t n, const void* q, const void* k, int32_t layer,
                               void* stream, const rr_relay_out* const* outs) {
    const rr_status st0 = check_group(L, n, q, k, layer);
    if (st0 != RR_OK) return st0;
    for (int b = 0; b < n; ++b) {
        if (L[b]->poisoned) return fail(RR_ESTATE, "ledger %d is poisoned by an earlier device error; anchor first", b);
        if (!L[b]->anchored) return fail(RR_ESTATE, "ledger %d: relay layer before any anchor layer", b);
        if (layer <= L[b]->last_layer)
            return fail(RR_ESTATE, "ledger %d: relay layer %d is not after the last layer %d", b, layer, L[b]->last_layer);
    }
    // One grid when every ledger takes the fused kernel: each fits it, none asks for the
    // compacted schedule, and either one asks for the fused one or the group's 128-row blocks
    // are in the automatic schedule's range.
    bool one_grid = n > 1, forced = false;
    long long blocks = 0;
    for (int b = 0; b < n; ++b) {
        one_grid = one_grid && fused_fits(view_of(L[b])) && L[b]->relay_mode != RR_RELAY_COMPACTED;
        forced = forced || L[b]->relay_mode == RR_RELAY_FUSED;
        blocks += (long long)L[b]->cfg.heads * ((L[b]->cfg.nq + 127) / 128);
    }
    one_grid = one_grid && (forced || (blocks >= FUSED_MIN_BLOCKS && blocks <= FUSED_MAX_BLOCKS));
    if (!one_grid) {
        for (int b = 0; b < n; ++b) {
            const rr_status e = rr_relay_layer(L[b], q, k, layer, stream, outs ? outs[b] : nullptr);
            if (e != RR_OK) return e;
        }
        return ok();
    }
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    rr::RelayGroup g{};
    g.n = n;
    for (int b = 0; b < n; ++b) {
        const LedgerView v = view_of(L[b]);
        g.s[b] = rescore_args(v, q, k, layer, outs ? outs[b] : nullptr);
        g.p[b] = route_args(v, q, k, layer);
        g.p[b].refresh_mark = 1;
        g.off[b + 1] = g.off[b] + (L[b]->cfg.nq + 127) / 128;
    }
    g.per_head = g.off[n];
    int tix[RR_GROUP_MAX];
    for (int b = 0; b < n; ++b) tix[b] = time_begin(L[b], RR_KERNEL_RELAY, st);
    hipError_t e = rr::launch_relay_group(g, L[0]->cfg.dtype == RR_BF16, L[0]->cfg.causal != 0, st);
    for (int b = 0; b < n; ++b) time_end(L[b], tix[b], st);
    if (e != hipSuccess) return group_launch_failed(L, n, e, "grouped relay launch");
    for (int b = 0; b < n; ++b) {
        const rr_relay_out* out = outs ? outs[b] : nullptr;
        if (!wants_list(out)) continue;
        const int t = time_begin(L[b], RR_KERNEL_LIST, st);
        e = rr::launch_compact_out(L[b]->bcount, L[b]->blist, L[b]->cfg.heads, L[b]->cfg.nq, out->rows,
                                   out->head_counts, out->n_rows, st);
        time_end(L[b], t, st);
        if (e != hipSuccess) return group_launch_failed(L, n, e, "compacted-list launch");
    }
    for (int b = 0; b < n; ++b) L[b]->last_layer = layer;
    return ok();
}

rr_status rr_relay_layer_noalloc(const rr_config* cfg, int32_t* ids, int32_t* anchor_layer, uint8_t* refreshed,
                                 const void* q, const void* k, int32_t layer, void* stream, const rr_relay_out* out) {
    const rr_status st0 = check_cfg(cfg, false);
    if (st0 != RR_OK) return st0;
    if (!ids || !anchor_layer || !refreshed) return fail(RR_EINVAL, "ids, anchor_layer and refreshed are required");
    if (!q || !k) return fail(RR_EINVAL, "q and k must be device pointers");
    if (layer < 0) return fail(RR_EINVAL, "layer must be >= 0 (got %d)", layer);
    const long long padded = (long long)cfg->heads * ((cfg->nq + 63) / 64) * 64;
    if (padded > (long long)NOALLOC_MAX_ROWS)
        return fail(RR_EUNSUPPORTED, "heads * ceil(nq / 64) * 64 = %lld rows exceed the fixed working memory (%zu rows)",
                    padded, NOALLOC_MAX_ROWS);
    void* base = nullptr;
    const rr_status st1 = scratch_for_current_device(&base);
    if (st1 != RR_OK) return st1;
    unsigned char* b = static_cast<unsigned char*>(base);
    constexpr size_t P = NOALLOC_MAX_ROWS;
    LedgerView v{*cfg, cfg->k + cfg->m + cfg->sink + cfg->recent + cfg->r, cfg->k + cfg->m, cfg->nq, RR_RELAY_AUTO,
                 ids, anchor_layer, refreshed, nullptr,
                 b,                                              // refresh flags      [P] u8
                 reinterpret_cast<float*>(b + P),                // reroute thresholds [P] f32
                 reinterpret_cast<int32_t*>(b + 5 * P),          // per-block counts   [P / 64] i32
                 reinterpret_cast<int32_t*>(b + 5 * P + P / 16)};  // per-block lists  [P] i32
    const char* what = "";
    const hipError_t e = relay_launch(v, q, k, layer, reinterpret_cast<hipStream_t>(stream), out, nullptr, &what);
    if (e != hipSuccess) return fail(RR_EDEVICE, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

rr_status rr_ledger_set_relay_mode(rr_ledger* L, int32_t mode) {
    if (!L) return fail(RR_EINVAL, "ledger is NULL");
    if (mode != RR_RELAY_AUTO && mode != RR_RELAY_FUSED && mode != RR_RELAY_COMPACTED)
        return fail(RR_EINVAL, "unknown relay mode %d", mode);
    if (mode == RR_RELAY_FUSED && !fused_fits(view_of(L)))
        return fail(RR_EUNSUPPORTED, "the fused relay needs k + m <= 32, c <= 32 and a head's keys in 128 KB "
                    "(got k + m = %d, c = %d, nk = %d)", L->sel, L->c, L->cfg.nk);
    L->relay_mode = mode;
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
    if (src_is_host) {
        const rr_status v = check_ledger_ids(L->cfg, L->qmap_host.empty() ? nullptr : L->qmap_host.data(), route,
                                             sent, anchor_layer, last_layer);
        if (v != RR_OK) return v;
    }
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
