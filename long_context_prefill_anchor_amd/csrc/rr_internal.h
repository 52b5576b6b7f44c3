// Internal interface between the C ABI host code (rr_api.cpp) and the kernels (rr_kernels.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rr {

struct RouteArgs {
    const void* qp;             // [H, nq_q, 64] f32 or bf16
    const int32_t* qmap;        // width bucket: ledger row r is query row qmap[r]; null = identity
    const void* kp;             // [H, nk, 64]
    int32_t* ids;               // ledger IDs [H, nq, c]: route k | near-miss m | mandatory sink+recent | random r
    int32_t* anchor;            // [H, nq]
    uint8_t* refreshed;         // [H, nq] hysteresis state: each emitted row gets refresh_mark
    const uint8_t* flags;       // reroute: refresh flags [H, nq] from the rescore kernel
    const float* hint;          // reroute: first selection threshold per row [H, nq]
    const int32_t* bcount;      // reroute: flagged rows per rescore block [H, G]
    const int32_t* blist;       // reroute: per rescore block, its flagged rows (ascending) [H, G, 64]
    int32_t* out_rows;          // reroute, optional: compacted list (ascending h*nq+i)
    int32_t* out_head_counts;   // reroute, optional: [H]
    int32_t* out_n_rows;        // reroute, optional: [1]
    int H, nq, nk, k, m, r, c, sel;
    int sink, recent;           // mandatory sentinels: chunks [0, sink) and the row's last `recent`
    int layer;
    int refresh_mark;           // 0 for an anchor launch, 1 for a reroute
    int nq_q;                   // query rows per head in qp (nq when qmap is null)
    uint32_t seed_lo, seed_hi;
};

struct RescoreArgs {
    const void* qp;             // [H, nq_q, 64]
    const int32_t* qmap;        // as in RouteArgs
    int nq_q;
    const void* kp;
    const int32_t* ids;         // [H, nq, c]
    const int32_t* anchor;      // [H, nq] layer of each row's last full routing (hysteresis)
    uint8_t* refreshed;         // [H, nq] hysteresis state, cleared when a refreshed row passes
    uint8_t* flags_ws;          // [H, nq]
    float* hint_ws;             // [H, nq]
    int32_t* bcount;            // [H, G] flagged rows per block of 64 rows
    int32_t* blist;             // [H, G, 64] those rows (row index within the head), ascending
    uint8_t* out_flags;         // optional
    float* out_alpha;           // optional
    float* out_beta;            // optional
    float* cand_scores;         // optional [H, nq, c]
    int H, nq, nk, k, m, r, c, sel;
    float gamma;
    int layer, min_reuse;       // hysteresis (on when min_reuse > 0 or gamma_extra > 0)
    float gamma_extra;
};

// Sparse attention over routed chunks (rr_attention.hip).
struct AttnArgs {
    const void* q;              // [H, nq*64, 64] bf16
    const void* k;              // [H, nk*64, 64] bf16
    const void* vt;             // [H, nk, 64 (d), 64 (token)] bf16
    const int32_t* routes;      // [H, nq, kr], -1 padded
    float* out;                 // [H, nq*64, 64]
    int H, nq, nk, kr, causal;
};

constexpr int ROUTE_ROWS = 64;   // rows per route block and per rescore block

// Width-bucket ledgers over the same Q and K launched as one grid: logical blocks run head-major
// over the group, ledger b taking blocks off[b] .. off[b + 1] - 1 of each head's per_head.
constexpr int GROUP_MAX = 4;
struct RouteGroup {
    int n;                      // ledgers in the group, 1 .. GROUP_MAX
    int per_head;               // blocks per head over all of them
    int off[GROUP_MAX + 1];
    RouteArgs p[GROUP_MAX];
};
struct RelayGroup {
    int n, per_head;
    int off[GROUP_MAX + 1];
    RescoreArgs s[GROUP_MAX];
    RouteArgs p[GROUP_MAX];
};

hipError_t launch_route(const RouteArgs& a, bool bf16, bool causal, bool reroute, hipStream_t st);
hipError_t launch_rescore(const RescoreArgs& a, bool bf16, hipStream_t st);
// Fused relay layer: rescoring, in-block compaction and reroute of every 128-row block in one
// launch, with the head's keys staged in LDS; leaves bcount / blist for launch_compact_out.
// Only where relay_fits (k + m <= 32, c <= 32, the keys of a head in 128 KB).
bool relay_fits(int nk, int c, int sel, bool bf16);
hipError_t launch_relay(const RescoreArgs& s, const RouteArgs& a, bool bf16, bool causal, hipStream_t st);
// Compacted list (ascending h*nq+i), per-head counts and total from bcount / blist.
// Anchor routing (sel <= 32) / fused relay layers (relay_fits) of a group of ledgers that share
// H, nk, the element type and the causal mask.
hipError_t launch_route_group(const RouteGroup& g, bool bf16, bool causal, hipStream_t st);
hipError_t launch_relay_group(const RelayGroup& g, bool bf16, bool causal, hipStream_t st);
hipError_t launch_compact_out(const int32_t* bcount, const int32_t* blist, int H, int nq, int32_t* out_rows,
                              int32_t* out_head_counts, int32_t* out_n_rows, hipStream_t st);
size_t route_lds_bytes(int nk, int c);
// The route kernels' LDS for nk key chunks and c ledger IDs per row fits a compute unit.
bool route_fits(int nk, int c);
hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t st);
// k + m > 32 (rr_wide.hip): one wave per row, same ledger rules; nk <= 1024.
hipError_t launch_route_wide(const RouteArgs& a, bool bf16, bool causal, bool reroute, hipStream_t st);

}  // namespace rr
