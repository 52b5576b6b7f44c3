// RouteRelay routing kernels for gfx950 (MI355X).
//
// Source: "RouteRelay: Event-Triggered Cross-Layer Route Reuse for Efficient Dynamic Sparse
// Attention" (arXiv 2609.07306), Sections 2.1, 3.1-3.2, 4.1-4.2.
//
// k_route    — full routing of 64 query rows of one head: S = Q K^T (Eq. 1) on MFMA, exact
//              top-(k+m) selection (Eq. 2 + near-miss sentinels, Section 3.1), random
//              sentinels, ledger write.  Anchor mode routes rows 64g..64g+63; reroute mode
//              routes the g-th slice of 64 flagged rows of the head (the compacted list of
//              Sections 4.1/4.2), found from the rescore kernel's per-block lists of
//              flagged rows.
// k_rescore  — relay candidate rescoring (Eq. 5-8): per row, gather the ledger's candidate key
//              rows, dot them with the query row, alpha / beta / refresh flag, plus a lower
//              bound on the row's (k+m)-th best score that the reroute uses as its first
//              selection threshold.  Lists each 64-row block's flagged rows for the
//              compaction.
//
// k_route layout.  A block is SPLIT = 4 waves; all four own the same 64 rows (one row per
// lane) and wave w scores the key tiles t = w, w+4, ... (32 keys per tile).  One tile is two
// v_mfma_f32_32x32x16_bf16 groups (rows 0-31 and 32-63) of D = K_tile Q^T; a
// v_permlane32_swap between the two accumulators leaves every lane with the 32 scores of its
// own row, so selection runs one row per lane with no LDS traffic for the scores.
//
// Selection.  Each lane keeps its row's best keys (64-bit: orderable score, inverted index) in
// a sorted register list of 32.  Scores at or above the row's threshold are appended to a
// per-wave, per-row LDS buffer; when a buffer holds 16 or more entries the lane sorts them
// (odd-even merge network) and merges them into its list, and publishes the list's (k+m)-th key
// as the row's threshold (LDS atomic max shared by the four waves).  At the end the four lists
// are exchanged through LDS and merged by the row's quad of lanes (DPP bitonic exchanges).  A key below the threshold cannot be among the best k+m, so
// the result is exact.  The first threshold is a proven lower bound on the (k+m)-th best score:
// anchor mode — the (k+m)-th largest of 32 maxima of disjoint 8-key groups taken from a first
// MFMA pass (each wave contributes its 8 largest group maxima); reroute mode — the smallest
// current score of the row's k+m ledger route and near-miss chunks, minus a rounding margin
// (a row that ends with fewer than k+m keys is recomputed from -inf).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <algorithm>

#include "rr_device.h"
#include "rr_internal.h"

namespace rr {

// Phase timestamps for measurement builds (RR_PHASE_TRACE defined; the library is built
// without): the first lane of every wave of the first TRACE_BLOCKS blocks of a launch records
// the 100 MHz real-time counter at fixed points of the route and relay kernels, and counts its
// mid-stream drains; rr_debug_phase_trace / rr_debug_phase_clear (end of this file) copy the
// tables out and clear them.  Work and results are unchanged.
#ifdef RR_PHASE_TRACE
constexpr int TRACE_BLOCKS = 4096, TRACE_WAVES = 8, TRACE_SLOTS = 16;
__device__ uint64_t g_phase[TRACE_BLOCKS * TRACE_WAVES * TRACE_SLOTS];
__device__ uint32_t g_drains[TRACE_BLOCKS * TRACE_WAVES];
#define RR_STAMP(LB, W, K)                                                                                   \
    do {                                                                                                     \
        if ((threadIdx.x & 63) == 0 && (LB) >= 0 && (LB) < TRACE_BLOCKS)                                     \
            g_phase[((size_t)(LB) * TRACE_WAVES + (W)) * TRACE_SLOTS + (K)] = __builtin_amdgcn_s_memrealtime(); \
    } while (0)
#define RR_COUNT_DRAIN(LB, W)                                                                                \
    do {                                                                                                     \
        if ((threadIdx.x & 63) == 0 && (LB) >= 0 && (LB) < TRACE_BLOCKS) g_drains[(LB) * TRACE_WAVES + (W)] += 1; \
    } while (0)
#else
#define RR_STAMP(LB, W, K) do {} while (0)
#define RR_COUNT_DRAIN(LB, W) do {} while (0)
#endif

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int ROWS = 64;           // rows per route block (one per lane)
constexpr int SPLIT = 4;           // waves per block, each scoring a quarter of the key tiles
constexpr int TK = 32;             // keys per tile
constexpr int TOPW = 32;           // register top list width (k + m <= TOPW)
constexpr int CAP = 31;            // per-wave per-row buffer: <= 15 held + 16 slots appended
constexpr int BUF_IDX = CAP * ROWS; // words from a buffered score to its key index
// The per-wave buffers are slot-major ([CAP][ROWS] per wave): a lane's consecutive entries are
// ROWS apart, so whatever count each lane is at, the 32 lanes of a half-wave write 64-bit entries
// to 32 distinct bank pairs.
constexpr int GSTRIDE = 33;        // f32 row stride of the pass-1 group maxima table
constexpr int XSTRIDE = TOPW + 1;  // u64 row stride of the cross-wave exchange lists
constexpr int XWAVE = ROWS * XSTRIDE + 8;  // u64 stride between waves' exchange lists: the pad puts
                                           // the four lists a quad reads in different banks
constexpr uint64_t NO_PASS_KEY = ~0ull;   // threshold whose score part is NaN: nothing passes

struct bf16_t { uint16_t bits; };
template <typename DT> struct Elem { typedef float type; };
template <> struct Elem<bf16_t> { typedef uint16_t type; };

// ------------------------------------------------------------------------------ MFMA tiles
// acc0 / acc1: D = K_tile * Q^T for query groups 0 (rows 0-31) and 1 (rows 32-63); lane L holds
// D[key 8(v/4) + 4(L/32) + v%4][query L%32] in register v.

template <typename DT> struct Tile;

template <> struct Tile<bf16_t> {
    typedef bf16x8 KReg[4];
    static constexpr int NBUF = 2;        // K register ring: loads run one tile ahead (a third
                                          // buffer measured ~3% slower: the freed registers
                                          // serve the scheduler better)
    bf16x8 q[2][4];                       // B operand: group g, k-step s: d = 16s + 8(L/32) + t
    __device__ __forceinline__ void load_q(const uint16_t* Q, int row0, int row1, int lane) {
        const int sub = lane >> 5;
        const int rows[2] = {row0, row1};
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if (rows[g] >= 0) {
                    q[g][s] = *reinterpret_cast<const bf16x8*>(Q + (size_t)rows[g] * 64 + 16 * s + 8 * sub);
                } else {
                    u32x4 z = {0u, 0u, 0u, 0u};
                    q[g][s] = __builtin_bit_cast(bf16x8, z);
                }
            }
    }
    // Rows past nk read row nk-1 instead: those keys are masked out of every row afterwards.
    // FENCED keeps the loads in program order (see fill_ring).
    template <bool FENCED = false>
    __device__ __forceinline__ void load_k(KReg& dst, const uint16_t* K, int key0, int nk, int lane) const {
        const int key = min(key0 + (lane & 31), nk - 1);
        const int sub = lane >> 5;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            dst[s] = *reinterpret_cast<const bf16x8*>(K + (size_t)key * 64 + 16 * s + 8 * sub);
            if constexpr (FENCED) __builtin_amdgcn_sched_barrier(0);
        }
    }
    __device__ __forceinline__ void mma(const KReg& ka, f32x16& acc0, f32x16& acc1) const {
        acc0 = f32x16{};
        acc1 = f32x16{};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s], q[0][s], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s], q[1][s], acc1, 0, 0, 0);
        }
    }
};

template <> struct Tile<float> {
    typedef float KReg[32];
    // 32-register tiles: one buffer (the load of the next tile follows the tile's MMA).  A
    // second buffer made every fp32 route kernel spill 164-332 bytes per lane to scratch; fp32
    // inputs serve the small one-head configurations, which are latency-bound either way.
    static constexpr int NBUF = 1;
    float q[2][32];                       // k-step s: d = 32(L/32) + s
    __device__ __forceinline__ void load_q(const float* Q, int row0, int row1, int lane) {
        const int sub = lane >> 5;
        const int rows[2] = {row0, row1};
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            if (rows[g] >= 0) {
                const float4* src = reinterpret_cast<const float4*>(Q + (size_t)rows[g] * 64 + 32 * sub);
#pragma unroll
                for (int v = 0; v < 8; ++v) {
                    const float4 x = src[v];
                    q[g][4 * v] = x.x; q[g][4 * v + 1] = x.y; q[g][4 * v + 2] = x.z; q[g][4 * v + 3] = x.w;
                }
            } else {
#pragma unroll
                for (int s = 0; s < 32; ++s) q[g][s] = 0.f;
            }
        }
    }
    template <bool FENCED = false>
    __device__ __forceinline__ void load_k(KReg& dst, const float* K, int key0, int nk, int lane) const {
        const int key = min(key0 + (lane & 31), nk - 1);
        const int sub = lane >> 5;
        const float4* src = reinterpret_cast<const float4*>(K + (size_t)key * 64 + 32 * sub);
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            const float4 x = src[v];
            dst[4 * v] = x.x; dst[4 * v + 1] = x.y; dst[4 * v + 2] = x.z; dst[4 * v + 3] = x.w;
            if constexpr (FENCED) __builtin_amdgcn_sched_barrier(0);
        }
    }
    __device__ __forceinline__ void mma(const KReg& ka, f32x16& acc0, f32x16& acc1) const {
        acc0 = f32x16{};
        acc1 = f32x16{};
#pragma unroll
        for (int s = 0; s < 32; ++s) {
            acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(ka[s], q[0][s], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(ka[s], q[1][s], acc1, 0, 0, 0);
        }
    }
};

// After the swap every lane holds its own row: lo[v] is key lo_key(v) of the tile, hi[v] is
// key hi_key(v).  (v_permlane32_swap exchanges lanes 32-63 of its first operand with lanes
// 0-31 of its second.)
__device__ __forceinline__ void rows_per_lane(f32x16& acc0, f32x16& acc1) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc0[v]), __float_as_uint(acc1[v]), false, false);
        acc0[v] = __uint_as_float(r[0]);
        acc1[v] = __uint_as_float(r[1]);
    }
}

// Fill the K register ring with tiles wave, wave + SPLIT, ... in the order in which the
// streaming loop reissues them, oldest first.  The wait at the loop head has to hold both on
// entry and on the back edge; if the entry issued the loads in another order (the scheduler
// would reverse them), that wait would drain every load in flight instead of only the oldest
// tile's.
template <typename DT, typename E, typename KRing>
__device__ __forceinline__ void fill_ring(const Tile<DT>& tile, KRing& kbuf, const E* Kh, int wave, int nk, int lane) {
#pragma unroll
    for (int u = 0; u < Tile<DT>::NBUF; ++u) tile.template load_k<true>(kbuf[u], Kh, TK * (wave + u * SPLIT), nk, lane);
}

__device__ __forceinline__ constexpr int lo_key(int v) { return 8 * (v >> 2) + (v & 3); }
__device__ __forceinline__ constexpr int hi_key(int v) { return 8 * (v >> 2) + 4 + (v & 3); }

// ------------------------------------------------------------------------------ top lists

__device__ __forceinline__ uint64_t pick(const uint64_t (&v)[TOPW], int idx) {
    uint64_t out = EMPTY_KEY;
#pragma unroll
    for (int s = 0; s < TOPW; ++s) out = (s == idx) ? v[s] : out;
    return out;
}

// top (sorted desc, 32) <- the 32 largest of top U x, x sorted desc (16 entries).
__device__ __forceinline__ void merge16_into_top(uint64_t (&top)[TOPW], const uint64_t (&x)[16]) {
#pragma unroll
    for (int i = 16; i < 32; ++i) {
        const uint64_t c = x[31 - i];
        top[i] = c > top[i] ? c : top[i];
    }
#pragma unroll
    for (int s = 16; s >= 1; s >>= 1) {
#pragma unroll
        for (int i = 0; i < 32; ++i)
            if ((i & s) == 0) ce_desc(top[i], top[i + s]);
    }
}

// Sort the lane's buffered (score bits, index) pairs and merge them into its top list.
// `fresh`: every lane's list is still empty, so the first sorted chunk is copied in.
// buf: slot-major, scores at buf[j * ROWS], their key indices BUF_IDX words further on.
// A last chunk of at most 8 (common once the threshold is tight) takes an 8-key network and
// merges through the same 32-key cascade: the slots past 8 would only add empty keys.
__device__ __forceinline__ void drain8(uint64_t (&top)[TOPW], const uint32_t* buf, int c0, int cnt, bool& fresh) {
    uint64_t x[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        if (c0 + s < cnt) {
            const uint32_t* e = buf + (c0 + s) * ROWS;
            x[s] = make_key(__uint_as_float(e[0]), e[BUF_IDX]);
        } else {
            x[s] = EMPTY_KEY;
        }
    }
    sort_desc<8>(x);
    if (fresh) {
#pragma unroll
        for (int s = 0; s < 8; ++s) top[s] = x[s];
        fresh = false;
        return;
    }
    // max(top[i], x'[31 - i]) with x' = x followed by empty keys: only the last 8 change.
#pragma unroll
    for (int i = 24; i < 32; ++i) {
        const uint64_t c = x[31 - i];
        top[i] = c > top[i] ? c : top[i];
    }
#pragma unroll
    for (int s = 16; s >= 1; s >>= 1) {
#pragma unroll
        for (int i = 0; i < 32; ++i)
            if ((i & s) == 0) ce_desc(top[i], top[i + s]);
    }
}

__device__ __forceinline__ void drain(uint64_t (&top)[TOPW], const uint32_t* buf, int cnt, bool& fresh) {
    const int maxc = wave_max_i(cnt);
    if (maxc <= 8) {                                                  // uniform
        if (maxc > 0) drain8(top, buf, 0, cnt, fresh);
        return;
    }
    for (int c0 = 0; c0 < maxc; c0 += 16) {
        uint64_t x[16];
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            if (c0 + s < cnt) {
                const uint32_t* e = buf + (c0 + s) * ROWS;
                x[s] = make_key(__uint_as_float(e[0]), e[BUF_IDX]);
            } else {
                x[s] = EMPTY_KEY;
            }
        }
        sort_desc<16>(x);
        if (fresh) {
#pragma unroll
            for (int s = 0; s < 16; ++s) top[s] = x[s];
            fresh = false;
        } else {
            merge16_into_top(top, x);
        }
    }
}

// Workgroups are handed to the 8 XCDs round-robin (block b runs on XCD b % 8), and each XCD
// has its own L2.  Renumbering so that XCD x runs the contiguous logical range
// [x * per, (x + 1) * per) keeps all blocks of a head, which share that head's K, on one XCD.
// The grid is padded to a multiple of 8; padding blocks get -1.
constexpr int XCDS = 8;

__device__ __forceinline__ int xcd_block(int nlogical) {
    const int per = (int)gridDim.x / XCDS;
    const int l = ((int)blockIdx.x % XCDS) * per + (int)blockIdx.x / XCDS;
    return l < nlogical ? l : -1;
}

// Reroute grids are sized for every slice of 64 rows of every head, but a slice past the head's
// flagged count exits at once.  The dispatcher deals an XCD's blocks to its CUs in turn, so in
// head-major order the live slices (the first few of each head) would stack two to a CU while
// others idle.  When an XCD's range holds whole heads, its blocks are handed out slice-major
// (slice 0 of each of its heads, then slice 1, ...), which puts the live ones first.
__device__ __forceinline__ int slice_major_block(int H, int G) {
    const int per = (int)gridDim.x / XCDS;
    const int l0 = ((int)blockIdx.x % XCDS) * per;
    const int local = (int)blockIdx.x / XCDS;
    if (per % G == 0 && l0 + per <= H * G) {
        const int nh = per / G;
        return l0 + (local % nh) * G + local / nh;
    }
    return xcd_block(H * G);
}

__host__ __forceinline__ int xcd_grid(int nlogical) { return (nlogical + XCDS - 1) / XCDS * XCDS; }

// Words of a row's sentinel bitmap: one bit per key chunk plus a spare word, padded to a multiple
// of four so that every row's bitmap starts 16-byte aligned (cleared with 16-byte stores).
__host__ __device__ __forceinline__ constexpr int bitmap_words(int nk) { return ((nk + 31) / 32 + 1 + 3) & ~3; }

// LDS a route block (64 rows, SPLIT waves) needs: the per-wave candidate buffers, the cross-wave
// exchange lists, the pass-1 group maxima and the ledger-write area, which alias; rounded up to
// 16 bytes.
__host__ __device__ __forceinline__ size_t route_lds_bytes_dev(int nk, int c) {
    const size_t cand = (size_t)SPLIT * CAP * ROWS * sizeof(uint2);
    const size_t xl = (size_t)SPLIT * XWAVE * sizeof(uint64_t);
    const size_t gm = (size_t)ROWS * GSTRIDE * sizeof(float);
    const size_t em = (size_t)ROWS * (bitmap_words(nk) + 32 + c + 1) * sizeof(uint32_t);
    size_t m = cand > xl ? cand : xl;
    m = m > gm ? m : gm;
    m = m > em ? m : em;
    return (m + 15) / 16 * 16;
}

size_t route_lds_bytes(int nk, int c) { return route_lds_bytes_dev(nk, c); }

struct RouteShared {
    uint64_t thr[ROWS];      // shared threshold key per row (max over the waves' lower bounds)
    int32_t rows[ROWS];      // ledger row of each slot (-1: none)
    int32_t qrows[ROWS];     // its query row (differs in a width bucket)
    int32_t redo;
};

// A route block's LDS (the dynamic area and its shared row state) fits a compute unit's 160 KB.
// Past 4096 key chunks the per-row sentinel bitmaps dominate: one block per compute unit.
bool route_fits(int nk, int c) { return route_lds_bytes_dev(nk, c) + sizeof(RouteShared) + 64 <= (160u << 10); }

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t min_u64(uint64_t a, uint64_t b) { return a > b ? b : a; }
// keep_max ? max(a, b) : min(a, b) with one compare (the lane's choice flips the compare's mask).
__device__ __forceinline__ uint64_t max_or_min_u64(uint64_t a, uint64_t b, bool keep_max) {
    return ((a > b) == keep_max) ? a : b;
}

// Sort a bitonic sequence descending (half-cleaner cascade).
template <int N, typename T>
__device__ __forceinline__ void bitonic_clean_desc(T (&v)[N]) {
#pragma unroll
    for (int st = N / 2; st >= 1; st >>= 1) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            if ((i & st) == 0) ce_desc(v[i], v[i + st]);
    }
}

// Merge the four sorted lists (descending, TOPW = 32 keys) held by the lanes of a quad into
// the quad's best 32, split between lanes: lanes 0 and 3 end with entries [0, 16) and lanes 1
// and 2 with entries [16, 32), each sorted descending.  Level 1 merges lists 0+1 and 2+3
// (partners lane ^ 1), level 2 merges the two results (partners lane ^ 3, then lane ^ 1).
// Each step is a bitonic merge: the element-wise max of one list and the other reversed holds
// exactly the best half, as a bitonic sequence; a half-cleaner splits it between two lanes.
// Keys are distinct (the index is part of the key), so partners agree on every split.
__device__ __forceinline__ void quad_merge_split(const uint64_t (&a)[TOPW], uint64_t (&hv)[16], int sub) {
    static_assert(TOPW == 32, "the split merge is written for 32-key lists");
    {
        uint64_t b[32];
#pragma unroll
        for (int s = 0; s < 32; ++s) b[s] = dpp_u64<DPP_XOR1>(a[s]);
        const bool keep_max = (sub & 1) == 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint64_t x = max_u64(a[i], b[31 - i]);
            const uint64_t y = max_u64(a[i + 16], b[15 - i]);
            hv[i] = max_or_min_u64(x, y, keep_max);
        }
        bitonic_clean_desc<16>(hv);
    }
    {
        uint64_t b[16], d[16];
#pragma unroll
        for (int s = 0; s < 16; ++s) b[s] = dpp_u64<DPP_REVERSE>(hv[s]);
#pragma unroll
        for (int i = 0; i < 16; ++i) d[i] = max_u64(hv[i], b[15 - i]);
#pragma unroll
        for (int s = 0; s < 16; ++s) b[s] = dpp_u64<DPP_XOR1>(d[s]);
        const bool keep_max = (sub == 0) || (sub == 3);
#pragma unroll
        for (int i = 0; i < 16; ++i) hv[i] = max_or_min_u64(d[i], b[i], keep_max);
        bitonic_clean_desc<16>(hv);
    }
}

// Sum of x over the quad lanes below this one; *total gets the sum over all four.
__device__ __forceinline__ int quad_excl_sum(int x, int sub, int* total) {
    const int x0 = dpp_i<DPP_BCAST0>(x), x1 = dpp_i<DPP_BCAST1>(x);
    const int x2 = dpp_i<DPP_BCAST2>(x), x3 = dpp_i<DPP_BCAST3>(x);
    *total = x0 + x1 + x2 + x3;
    return (sub > 0 ? x0 : 0) + (sub > 1 ? x1 : 0) + (sub > 2 ? x2 : 0);
}

// Ascending sort of 16 32-bit keys (Batcher's network, min / max compare-exchanges).
__device__ __forceinline__ void sort16_asc_u32(uint32_t (&v)[16]) {
#pragma unroll
    for (int p = 1; p < 16; p <<= 1) {
#pragma unroll
        for (int k = p; k >= 1; k >>= 1) {
#pragma unroll
            for (int j = k % p; j + k < 16; j += 2 * k) {
#pragma unroll
                for (int i = 0; i < k; ++i) {
                    if (i < 16 - j - k && (i + j) / (2 * p) == (i + j + k) / (2 * p)) {
                        const uint32_t a = v[i + j], b = v[i + j + k];
                        v[i + j] = min(a, b);
                        v[i + j + k] = max(a, b);
                    }
                }
            }
        }
    }
}

constexpr int RLIST = 32;          // per-row list of drawn random sentinels (r <= 32)

// Mandatory and random sentinels (Section 3.1, items 3 and 2) and the ledger write of one row,
// split over the row's quad of lanes (sub = lane & 3).  hv: this lane's half of the row's final
// list (see quad_merge_split: lanes 0 and 3 hold positions [0, 16), lanes 1 and 2 [16, 32)).
// LDS per row slot: a bitmap of W = (nk + 31) / 32 + 1 words holding route, near-miss,
// mandatory and drawn chunks (what a draw must avoid), the list of drawn chunks in draw order,
// then a staging row of c IDs plus a spare slot.
// The first 16 draws (Philox blocks 0..3, one block per lane) are decided in parallel: draw t
// is taken iff its chunk is not in the bitmap, no earlier draw hit the same chunk, and fewer
// than r draws before it were taken.  Rows that need more draws continue one draw at a time.
// Output order: lanes 0 and 1 sort the route and near-miss chunks by (segment, index) and
// lanes 2 and 3 the drawn chunks by index, each pair with a 16-key network per lane and one
// bitonic exchange between the two lanes, which leaves every segment in ascending index order.
__device__ __forceinline__ void emit_split(const RouteArgs& p, const uint64_t (&hv)[16], int slot, int sub,
                                           int my_row, int my_qrow, int my_n, int h, unsigned char* lds,
                                           int tlb, int tw) {
    (void)tlb;
    (void)tw;
    const int ki = min(p.k, my_n);
    const int mi = min(p.m, my_n - ki);
    const int words = (p.nk + 31) >> 5;
    const int W = bitmap_words(p.nk);                 // words + 1, padded to 16 bytes
    uint32_t* bm = reinterpret_cast<uint32_t*>(lds) + (size_t)slot * (W + RLIST);
    int32_t* rlist = reinterpret_cast<int32_t*>(bm + W);
    int32_t* stage = reinterpret_cast<int32_t*>(lds) + (size_t)ROWS * (W + RLIST) + (size_t)slot * (p.c + 1);
    // Bitmap of the chunks a draw must avoid (route, near-miss, mandatory, drawn): only rows
    // with sentinels need it.
    const int mw = p.sink + p.recent;
    if (p.r > 0 || mw > 0) {                          // uniform
        for (int w = 4 * sub; w < W; w += 16) *reinterpret_cast<uint4*>(bm + w) = make_uint4(0u, 0u, 0u, 0u);
        if (sub < 2) {                                // lanes 0 / 1 own positions [0,16) / [16,32)
            // Branch-free: an unused position ORs zero into word 0 (per-entry branches cost
            // four scalar instructions and an exec round trip each).
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int pos = 16 * sub + i;
                const bool use = pos < ki + mi && hv[i] != EMPTY_KEY;
                const uint32_t j = use ? key_index(hv[i]) : 0u;
                atomicOr(&bm[j >> 5], use ? 1u << (j & 31) : 0u);
            }
        }
    }

    RR_STAMP(tlb, tw, 13);
    // Mandatory sentinels (Section 3.1, item 3): the sink chunks [0, sink) and the row's last
    // `recent` allowed chunks, ascending, skipping those already in the route or near-miss
    // set; marked so that the draws avoid them.  One lane walks them (sink + recent <= 32).
    int mand = 0;
    if (mw > 0) {
        if (sub == 0) {
            int32_t* mseg = stage + p.k + p.m;
            const int s_end = min(p.sink, my_n);
            const int r_beg = max(s_end, my_n - p.recent);
            for (int pass = 0; pass < 2; ++pass) {
                const int j0 = pass ? r_beg : 0, j1 = pass ? my_n : s_end;
                for (int j = j0; j < j1; ++j) {
                    const uint32_t bit = 1u << (j & 31);
                    const uint32_t word = bm[j >> 5];
                    if ((word & bit) == 0u) {
                        bm[j >> 5] = word | bit;
                        mseg[mand++] = j;
                    }
                }
            }
            for (int s2 = mand; s2 < mw; ++s2) mseg[s2] = -1;
        }
        mand = dpp_i<DPP_BCAST0>(mand);
    }
    const int pool = my_n - ki - mi - mand;
    const int rwant = min(p.r, pool);
    int taken = 0;                                    // random sentinels taken so far
    if (p.r > 0 && pool > p.r) {
        // Draws 4 sub .. 4 sub + 3 from Philox block `sub`.
        const P4 w4 = philox4x32_10(P4{(uint32_t)sub, (uint32_t)my_qrow, (uint32_t)p.layer, (uint32_t)h},
                                    p.seed_lo, p.seed_hi);
        uint32_t jj[4];
        jj[0] = __umulhi(w4.x, (uint32_t)my_n);
        jj[1] = __umulhi(w4.y, (uint32_t)my_n);
        jj[2] = __umulhi(w4.z, (uint32_t)my_n);
        jj[3] = __umulhi(w4.w, (uint32_t)my_n);
        bool ok[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) ok[q] = (bm[jj[q] >> 5] & (1u << (jj[q] & 31))) == 0u;
        // Earlier draws of the quad: blocks 0 .. sub-1 (all four words each).
        uint32_t e[12];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            e[q] = (uint32_t)dpp_i<DPP_BCAST0>((int)jj[q]);
            e[4 + q] = (uint32_t)dpp_i<DPP_BCAST1>((int)jj[q]);
            e[8 + q] = (uint32_t)dpp_i<DPP_BCAST2>((int)jj[q]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            bool dup = false;
#pragma unroll
            for (int t = 0; t < 12; ++t) dup = dup || (t < 4 * sub && e[t] == jj[q]);
#pragma unroll
            for (int t = 0; t < 4; ++t) dup = dup || (t < q && jj[t] == jj[q]);
            ok[q] = ok[q] && !dup;
        }
        const int mine = (int)ok[0] + (int)ok[1] + (int)ok[2] + (int)ok[3];
        int tot;
        int rank = quad_excl_sum(mine, sub, &tot);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (ok[q] && rank < p.r) {
                atomicOr(&bm[jj[q] >> 5], 1u << (jj[q] & 31));
                rlist[rank] = (int32_t)jj[q];
            }
            rank += ok[q] ? 1 : 0;
        }
        taken = min(tot, p.r);
        if (sub == 0) {
            // Rarely more than 16 draws are needed: continue one draw at a time.
            bool drawing = taken < p.r;
            P4 v4 = {0u, 0u, 0u, 0u};
            for (int t = 16; t < 65536 && __ballot(drawing); ++t) {
                if ((t & 3) == 0) {
                    P4 c = {(uint32_t)(t >> 2), (uint32_t)my_qrow, (uint32_t)p.layer, (uint32_t)h};
                    v4 = philox4x32_10(c, p.seed_lo, p.seed_hi);
                }
                const uint32_t uu = ((t & 3) == 0) ? v4.x : ((t & 3) == 1) ? v4.y : ((t & 3) == 2) ? v4.z : v4.w;
                if (drawing) {
                    const uint32_t j = __umulhi(uu, (uint32_t)my_n);
                    const uint32_t bit = 1u << (j & 31);
                    if ((bm[j >> 5] & bit) == 0u) {
                        bm[j >> 5] |= bit;
                        rlist[taken] = (int32_t)j;
                        ++taken;
                        drawing = taken < p.r;
                    }
                }
            }
        }
    }
    if (sub == 0 && taken < rwant) {
        // Fill: lowest-index chunks still free (whole pool when pool <= r; draw cap reached).
        for (int w = 0; w < words && taken < rwant; ++w) {
            uint32_t free_bits = ~bm[w];
            while (free_bits && taken < rwant) {
                const uint32_t j = (uint32_t)(w * 32 + __builtin_ctz(free_bits));
                free_bits &= free_bits - 1u;
                if ((int)j >= my_n) { free_bits = 0; break; }
                bm[w] |= 1u << (j & 31);
                rlist[taken] = (int32_t)j;
                ++taken;
            }
        }
    }
    taken = dpp_i<DPP_BCAST0>(taken);                 // lane 0 holds the final count
    RR_STAMP(tlb, tw, 14);
    if (sub == 0) {
        p.anchor[(size_t)h * p.nq + my_row] = p.layer;
        p.refreshed[(size_t)h * p.nq + my_row] = (uint8_t)p.refresh_mark;
    }

    // Sort keys: lanes 0 / 1 take list positions [0,16) / [16,32) as (segment << 16) | index
    // (segment 0 route, 1 near-miss, 2 none), lanes 2 / 3 the drawn chunks [0,16) / [16,32)
    // (absent: all ones).  Indices are below 65536.
    const int half = sub & 1;
    uint32_t key[16];
    int cr = 0, cn = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int pos = 16 * half + i;
        const bool used = sub < 2 && pos < ki + mi && hv[i] != EMPTY_KEY;
        const bool route = used && pos < ki;
        cr += route ? 1 : 0;
        cn += (used && !route) ? 1 : 0;
        const uint32_t sel_key = used ? ((route ? 0u : 0x10000u) | key_index(hv[i])) : 0x2FFFFu;
        const uint32_t rnd_key = (pos < taken) ? (uint32_t)rlist[pos] : 0xFFFFFFFFu;
        key[i] = (sub < 2) ? sel_key : rnd_key;
    }
    sort16_asc_u32(key);
    {
        // Bitonic exchange with the partner lane (lane ^ 1): the even lane keeps the lower 16 of
        // the pair's 32 keys, the odd lane the upper 16.
        uint32_t b[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) b[i] = (uint32_t)dpp_i<DPP_XOR1>((int)key[15 - i]);
#pragma unroll
        for (int i = 0; i < 16; ++i) key[i] = half ? max(key[i], b[i]) : min(key[i], b[i]);
#pragma unroll
        for (int st = 8; st >= 1; st >>= 1) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if ((i & st) == 0) {
                    const uint32_t x = key[i], y = key[i + st];
                    key[i] = min(x, y);
                    key[i + st] = max(x, y);
                }
        }
    }
    RR_STAMP(tlb, tw, 15);
    int tr, tn;
    quad_excl_sum(cr, sub, &tr);
    quad_excl_sum(cn, sub, &tn);
    // Every lane stores all 16 keys; those past its segments go to the row's spare slot c.
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int q = 16 * half + i;
        const int d_sel = (q < tr) ? q : (q < tr + tn) ? p.k + (q - tr) : p.c;
        const int d_rnd = (q < taken) ? p.k + p.m + mw + q : p.c;
        stage[(sub < 2) ? d_sel : d_rnd] = (int32_t)((sub < 2) ? (key[i] & 0xFFFFu) : key[i]);
    }
    for (int s2 = tr + sub; s2 < p.k; s2 += 4) stage[s2] = -1;
    for (int s2 = tn + sub; s2 < p.m; s2 += 4) stage[p.k + s2] = -1;
    for (int s2 = taken + sub; s2 < p.r; s2 += 4) stage[p.k + p.m + mw + s2] = -1;
    // The quad copies the staged row out: four consecutive IDs per instruction and row.
    int32_t* dst = p.ids + ((size_t)h * p.nq + my_row) * p.c;
    for (int e2 = sub; e2 < p.c; e2 += 4) dst[e2] = stage[e2];
}

// ------------------------------------------------------------------------------ route kernel

// Per-lane state of the route kernel shared by the selection pass and the redo path.
template <typename DT>
struct RowCtx {
    typedef typename Elem<DT>::type E;
    int lane, wave, h, my_row, my_n, nmin, ntiles;
    const E* Qh;
    const E* Kh;
    uint32_t* my_buf;
    int qslot, qsub, q_row, q_n, q_qrow;
    bool q_redo;
    int trace_lb, trace_w;      // phase-trace block and wave (measurement builds only)
};

// Streaming selection pass from the rows' shared thresholds (sh.thr), final merge and ledger
// write.  attempt 0 emits every row that holds min(k+m, n) keys; in reroute mode the others are
// marked for a redo from -inf (attempt 1, which emits only them).
// kbuf: the K register ring (shared with the anchor's first pass).  `primed`: the query rows
// and the ring's first tiles are already loaded (the reroute's first attempt issues them beside
// its threshold load).
template <typename DT, bool CAUSAL, bool REROUTE>
__device__ __forceinline__ void select_and_emit(const RouteArgs& p, RouteShared& sh, unsigned char* dyn_lds,
                                                Tile<DT>& tile, typename Tile<DT>::KReg (&kbuf)[Tile<DT>::NBUF],
                                                bool primed, RowCtx<DT>& cx, int attempt) {
    const int lane = cx.lane, wave = cx.wave, h = cx.h, my_row = cx.my_row, my_n = cx.my_n;
    // Block-uniform by construction; readfirstlane makes the loops scalar.
    const int nmin = __builtin_amdgcn_readfirstlane(cx.nmin), ntiles = __builtin_amdgcn_readfirstlane(cx.ntiles);
    const auto* Qh = cx.Qh;
    const auto* Kh = cx.Kh;
    uint32_t* my_buf = cx.my_buf;
    const int qslot = cx.qslot, qsub = cx.qsub, q_row = cx.q_row, q_n = cx.q_n, q_qrow = cx.q_qrow;
    if constexpr (REROUTE) {
        if (!primed) tile.load_q(Qh, sh.qrows[lane & 31], sh.qrows[32 + (lane & 31)], lane);
    } else {
        (void)Qh;
    }
    uint64_t top[TOPW];
#pragma unroll
    for (int s = 0; s < TOPW; ++s) top[s] = EMPTY_KEY;
    {
        int cnt = 0;
        bool fresh = true;                                              // list empty in every lane
        float ts = key_score(sh.thr[lane]);
        constexpr int NB = Tile<DT>::NBUF;
        if (!primed) fill_ring<DT>(tile, kbuf, Kh, wave, p.nk, lane);
        for (int t0 = wave; t0 < ntiles; t0 += NB * SPLIT) {
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                const int t = t0 + u * SPLIT;
                const bool live = t < ntiles;                        // uniform
                f32x16 lo, hi;
                if (live) tile.mma(kbuf[u], lo, hi);
                // Issued on every path (past the end it rereads the last key row), so the load
                // counter sees one fixed sequence and waits only for the oldest buffer.
                tile.load_k(kbuf[u], Kh, TK * (t + NB * SPLIT), p.nk, lane);
                if (live) {
                rows_per_lane(lo, hi);
                const int key0 = TK * t;
                if (key0 + TK > nmin) {                                 // keys past a row's end
                    const int lim = my_n - key0;
                    const float nan = __builtin_nanf("");
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        lo[v] = (lo_key(v) < lim) ? lo[v] : nan;            // NaN never passes >=
                        hi[v] = (hi_key(v) < lim) ? hi[v] : nan;
                    }
                }
                // The key index in a vector register: each slot's index is then one add, and
                // score and index go out as one two-address store.
                uint32_t vkey0 = (uint32_t)key0;
                asm volatile("" : "+v"(vkey0));
                // Branch-free append: every slot stores its (score, index) at the row's current
                // count and the count advances only when the score passes, so a failing slot's
                // store is overwritten by the next one (<= 15 held + 16 slots: index <= 30).
#pragma unroll
                for (int half = 0; half < 2; ++half) {
#pragma unroll
                    for (int v = 8 * half; v < 8 * half + 8; ++v) {
                        my_buf[cnt * ROWS] = __float_as_uint(lo[v]);
                        my_buf[cnt * ROWS + BUF_IDX] = vkey0 + lo_key(v);
                        cnt += (lo[v] >= ts) ? 1 : 0;
                        my_buf[cnt * ROWS] = __float_as_uint(hi[v]);
                        my_buf[cnt * ROWS + BUF_IDX] = vkey0 + hi_key(v);
                        cnt += (hi[v] >= ts) ? 1 : 0;
                    }
                    if (__ballot(cnt >= 16)) {
                        RR_COUNT_DRAIN(cx.trace_lb, cx.trace_w);
                        drain(top, my_buf, cnt, fresh);
                        cnt = 0;
                        const uint64_t own = pick(top, p.sel - 1);
                        if (own != EMPTY_KEY && my_row >= 0) atomicMax((unsigned long long*)&sh.thr[lane], own);
                    }
                }
                ts = key_score(sh.thr[lane]);
                }
            }
        }
        RR_STAMP(cx.trace_lb, cx.trace_w, 5);
        drain(top, my_buf, cnt, fresh);
        RR_STAMP(cx.trace_lb, cx.trace_w, 6);

        // Final merge, one row per quad: wave w takes rows 16w .. 16w+15 and lane 4j + s of it
        // holds wave s's list of row 16w + j.
        uint64_t* xl = reinterpret_cast<uint64_t*>(dyn_lds);            // [SPLIT][XWAVE]: [ROWS][XSTRIDE] + pad
        __syncthreads();                                                // every buffer is drained
        RR_STAMP(cx.trace_lb, cx.trace_w, 7);
        // A block (slice) without rows has nothing to publish: no wave of it reads these lists
        // (ntiles is 0 exactly when none of the 64 rows exists, the same in its four waves).
        // bf16 only, as the skip below: the fp32 instantiations are at their register limit.
        constexpr bool SKIP_EMPTY = sizeof(typename Elem<DT>::type) == 2;
        if (!SKIP_EMPTY || ntiles > 0) {
#pragma unroll
            for (int s = 0; s < TOPW; ++s) xl[wave * XWAVE + lane * XSTRIDE + s] = top[s];
        }
        __syncthreads();
        uint64_t hv[16];
        // A wave whose 16 merge rows are all empty (the tail of a partly filled slice) skips
        // the reads and the merge: it would only hold back the busy waves on its SIMD.
        const bool any_row = !SKIP_EMPTY || __ballot(q_row >= 0) != 0ull;   // uniform over the wave
        if (any_row) {
#pragma unroll
            for (int s = 0; s < TOPW; ++s) top[s] = xl[qsub * XWAVE + qslot * XSTRIDE + s];
        }
        RR_STAMP(cx.trace_lb, cx.trace_w, 8);
        if (any_row) {
            quad_merge_split(top, hv, qsub);
        } else {
#pragma unroll
            for (int s = 0; s < 16; ++s) hv[s] = EMPTY_KEY;
        }
        RR_STAMP(cx.trace_lb, cx.trace_w, 9);
        __syncthreads();                                                // xl is free again
        RR_STAMP(cx.trace_lb, cx.trace_w, 10);

        bool emit_now = q_row >= 0;
        if constexpr (REROUTE) {
            // Each row must now hold min(sel, n) keys.  Only a reroute threshold taken from the
            // rescore kernel's arithmetic can miss (rounding); such rows are redone from -inf
            // while every other row keeps the result it emits now.
            if (attempt == 0) {
                int have = 0;
#pragma unroll
                for (int s = 0; s < 16; ++s) have += (hv[s] != EMPTY_KEY);
                have += dpp_i<DPP_XOR1>(have);                          // the other half's count
                cx.q_redo = (q_row >= 0) && have < min(p.sel, q_n);
                if (cx.q_redo) sh.redo = 1;
                if (qsub == 0) sh.thr[qslot] = cx.q_redo ? make_key(-INFINITY, 0xFFFFFFFFu) : NO_PASS_KEY;
                emit_now = emit_now && !cx.q_redo;
            } else {
                emit_now = emit_now && cx.q_redo;
            }
        }
        if (emit_now) emit_split(p, hv, qslot, qsub, q_row, q_qrow, q_n, h, dyn_lds, cx.trace_lb, cx.trace_w);
        RR_STAMP(cx.trace_lb, cx.trace_w, 11);
        __syncthreads();                                                // LDS free, sh.redo final
        RR_STAMP(cx.trace_lb, cx.trace_w, 12);
    }
}

// Rows whose reroute threshold missed (see select_and_emit) are selected again from -inf.  It
// runs only when a row needs it.  The context goes through an empty asm so the compiler cannot
// share address arithmetic with the first pass, which would keep that pass's registers alive
// through the merge.
template <typename DT, bool CAUSAL>
__device__ __forceinline__ void redo_rows(const RouteArgs& p, RouteShared& sh, unsigned char* dyn_lds, RowCtx<DT>& cx) {
    __syncthreads();                                                    // everyone has read sh.redo
    if (cx.wave == 0 && cx.lane == 0) sh.redo = 0;
    asm volatile("" : "+v"(cx.my_n), "+v"(cx.nmin), "+v"(cx.my_row), "+v"(cx.ntiles));
    asm volatile("" : "+v"(cx.Kh), "+v"(cx.Qh), "+v"(cx.my_buf));
    asm volatile("" : "+v"(cx.q_row), "+v"(cx.q_n), "+v"(cx.qslot), "+v"(cx.qsub), "+v"(cx.q_qrow));
    Tile<DT> tile;
    typename Tile<DT>::KReg kbuf[Tile<DT>::NBUF];
    select_and_emit<DT, CAUSAL, true>(p, sh, dyn_lds, tile, kbuf, false, cx, 1);
}

// Per-lane state of a route block once sh.rows / sh.qrows name its rows: one row per lane for
// the scoring passes (all four waves cover all 64 slots), one row per quad of lanes for the
// merge and the ledger write.
template <typename DT, bool CAUSAL>
__device__ __forceinline__ RowCtx<DT> row_context(const RouteArgs& p, const RouteShared& sh, unsigned char* dyn_lds,
                                                  int h, int wave, int lane) {
    typedef typename Elem<DT>::type E;
    RowCtx<DT> cx;
    cx.lane = lane;
    cx.wave = wave;
    cx.h = h;
    cx.my_row = sh.rows[lane];
    cx.my_n = (cx.my_row < 0) ? 0 : (CAUSAL ? sh.qrows[lane] + 1 : p.nk);
    // Wave-uniform after the reductions; readfirstlane lets the compiler see it.
    const int kmax = __builtin_amdgcn_readfirstlane(wave_max_i(cx.my_n));
    cx.nmin = __builtin_amdgcn_readfirstlane(wave_min_i((cx.my_row < 0) ? (1 << 30) : cx.my_n));
    cx.ntiles = (kmax + TK - 1) / TK;
    cx.Qh = reinterpret_cast<const E*>(p.qp) + (size_t)h * p.nq_q * 64;
    cx.Kh = reinterpret_cast<const E*>(p.kp) + (size_t)h * p.nk * 64;
    cx.my_buf = reinterpret_cast<uint32_t*>(dyn_lds) + (size_t)wave * 2 * CAP * ROWS + lane;
    // Final merge and ledger write run one row per quad of lanes over all four waves.
    cx.qslot = 16 * wave + (lane >> 2);
    cx.qsub = lane & 3;
    cx.q_row = sh.rows[cx.qslot];
    cx.q_qrow = sh.qrows[cx.qslot];
    cx.q_n = (cx.q_row < 0) ? 0 : (CAUSAL ? cx.q_qrow + 1 : p.nk);
    cx.q_redo = false;
    cx.trace_lb = -1;
    cx.trace_w = wave;
    return cx;
}

// One route block: 64 ledger rows of one head (block lb = h * G + g of the ledger's grid).
// tlb: the block's number in phase traces.
template <typename DT, bool CAUSAL, bool REROUTE>
__device__ __forceinline__ void route_block(const RouteArgs& p, int lb, int tlb, RouteShared& sh,
                                            unsigned char* dyn_lds) {
    typedef typename Elem<DT>::type E;
    (void)tlb;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = (p.nq + ROWS - 1) / ROWS;
    const int h = lb / G;
    const int g = lb % G;
    RR_STAMP(tlb, wave, 0);

    // ------------------------------------------------------------------ rows of this block
    if constexpr (REROUTE) {
        const int32_t* bc = p.bcount + (size_t)h * G;
        if (G <= 64) {
            // Ranks of flagged rows within the head: block b of the rescore kernel holds ranks
            // [incl_b - cnt_b, incl_b), listed ascending in blist.
            const int cnt = (lane < G) ? bc[lane] : 0;
            const int incl = wave_incl_scan_i(cnt);
            const int count_h = __builtin_amdgcn_readlane(incl, 63);
            const int32_t* bl = p.blist + (size_t)h * G * ROWS;
            if (g == 0 && wave == 0) {
                // Compacted list output (ascending h*nq + i), per-head count and total.
                if (p.out_head_counts && lane == 0) p.out_head_counts[h] = count_h;
                int offset = 0;
                if (p.out_rows || p.out_n_rows) {
                    int acc = 0;
                    for (int x = lane; x < h * G; x += 64) acc += p.bcount[x];
                    offset = wave_sum_i(acc);
                    if (p.out_n_rows && h == p.H - 1 && lane == 0) p.out_n_rows[0] = offset + count_h;
                }
                if (p.out_rows) {
                    for (int bb = 0; bb < G; ++bb) {
                        const int cb = __builtin_amdgcn_readlane(cnt, bb);
                        const int base = __builtin_amdgcn_readlane(incl, bb) - cb;
                        if (lane < cb) p.out_rows[offset + base + lane] = h * p.nq + bl[bb * ROWS + lane];
                    }
                }
            }
            if (g * ROWS >= count_h) return;                   // uniform over the block
            if (wave == 0) {
                // The rescore block holding this lane's rank, and the rank's entry in its list;
                // only entries below that block's count are ever read.
                const int rank = g * ROWS + lane;
                int start = 0, bsel = -1, csel = 0;
                for (int bb = 0; bb < G; ++bb) {
                    const int ib = __builtin_amdgcn_readlane(incl, bb);
                    const int cb = __builtin_amdgcn_readlane(cnt, bb);
                    if (ib <= rank) {
                        start = ib;
                    } else if (bsel < 0) {
                        bsel = bb;
                        csel = cb;
                    }
                }
                const int ent = rank - start;
                sh.rows[lane] = (bsel >= 0 && ent >= 0 && ent < csel) ? bl[bsel * ROWS + ent] : -1;
            }
        } else {
            int total = 0;
            for (int b0 = 0; b0 < G; b0 += 64) total += wave_sum_i((b0 + lane < G) ? bc[b0 + lane] : 0);
            const int count_h = total;
            if (g == 0 && wave == 0) {
                // Compacted list output (ascending h*nq + i), per-head count and total.
                if (p.out_head_counts && lane == 0) p.out_head_counts[h] = count_h;
                int offset = 0;
                if (p.out_rows || p.out_n_rows) {
                    int acc = 0;
                    for (int x = lane; x < h * G; x += 64) acc += p.bcount[x];
                    offset = wave_sum_i(acc);
                    if (p.out_n_rows && h == p.H - 1 && lane == 0) p.out_n_rows[0] = offset + count_h;
                }
                if (p.out_rows) {
                    int run = 0;
                    for (int b = 0; b < G; ++b) {
                        const int i = b * ROWS + lane;
                        const bool f = i < p.nq && p.flags[(size_t)h * p.nq + i];
                        const uint64_t m = __ballot(f);
                        const int pos = run + __popcll(m & ((1ull << lane) - 1ull));
                        if (f) p.out_rows[offset + pos] = h * p.nq + i;
                        run += __popcll(m);
                    }
                }
            }
            if (g * ROWS >= count_h) return;                       // uniform over the block
            if (wave == 0) {
                const int want0 = g * ROWS;
                int run = 0;
                sh.rows[lane] = -1;
                for (int b = 0; b < G && run < want0 + ROWS; ++b) {
                    const int cb = bc[b];
                    if (run + cb > want0) {
                        const int i = b * ROWS + lane;
                        const bool f = i < p.nq && p.flags[(size_t)h * p.nq + i];
                        const uint64_t m = __ballot(f);
                        const int pos = run + __popcll(m & ((1ull << lane) - 1ull));
                        if (f && pos >= want0 && pos < want0 + ROWS) sh.rows[pos - want0] = i;
                    }
                    run += cb;
                }
            }
        }
    } else {
        if (wave == 0) {
            const int i = g * ROWS + lane;
            sh.rows[lane] = (i < p.nq) ? i : -1;
        }
    }
    if (wave == 0) {
        // Query row of each slot: a width bucket's ledger rows are a subset of the query rows.
        const int r = sh.rows[lane];
        sh.qrows[lane] = (r < 0) ? -1 : (p.qmap ? p.qmap[r] : r);
    }
    if (threadIdx.x == 0) sh.redo = 0;
    __syncthreads();

    // ------------------------------------------------------------------ per-row setup
    RowCtx<DT> cx = row_context<DT, CAUSAL>(p, sh, dyn_lds, h, wave, lane);
    const int my_row = cx.my_row, my_n = cx.my_n, nmin = cx.nmin, ntiles = cx.ntiles;
    const E* Qh = cx.Qh;
    const E* Kh = cx.Kh;
    Tile<DT> tile;
    typename Tile<DT>::KReg kbuf[Tile<DT>::NBUF];
    if constexpr (!REROUTE) tile.load_q(Qh, sh.qrows[lane & 31], sh.qrows[32 + (lane & 31)], lane);

    // ------------------------------------------------------------------ first threshold
    uint64_t base_thr;
    if constexpr (REROUTE) {
        // The threshold load first, then the query rows and the first key tiles: the three
        // round trips overlap, and waiting for the threshold does not wait for the others.
        const float hraw = p.hint[(size_t)h * p.nq + max(my_row, 0)];
        tile.load_q(Qh, sh.qrows[lane & 31], sh.qrows[32 + (lane & 31)], lane);
        fill_ring<DT>(tile, kbuf, Kh, wave, p.nk, lane);
        const float hv = (my_row >= 0) ? hraw : -INFINITY;
        const float t = (hv == -INFINITY) ? -INFINITY : hv - (fabsf(hv) * 1e-4f + 1e-6f);
        base_thr = make_key(t, 0xFFFFFFFFu);
    } else {
        // Pass 1: per row and wave, the 8 largest maxima of disjoint 8-key groups.
        float top8[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) top8[s] = -INFINITY;
        // K tiles stream through a ring of NBUF register buffers, NBUF - 1 tiles ahead (a
        // statically indexed ring: copying registers would make the loop wait on the newest
        // load).
        constexpr int NB = Tile<DT>::NBUF;
        fill_ring<DT>(tile, kbuf, Kh, wave, p.nk, lane);
        for (int t0 = wave; t0 < ntiles; t0 += NB * SPLIT) {
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                const int t = t0 + u * SPLIT;
                const bool live = t < ntiles;                        // uniform
                f32x16 lo, hi;
                if (live) tile.mma(kbuf[u], lo, hi);
                // Issued on every path (past the end it rereads the last key row), so the load
                // counter sees one fixed sequence and waits only for the oldest buffer.
                tile.load_k(kbuf[u], Kh, TK * (t + NB * SPLIT), p.nk, lane);
                if (live) {
                rows_per_lane(lo, hi);
                const int key0 = TK * t;
                if (key0 + TK > nmin) {
                    const int lim = my_n - key0;
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        lo[v] = (lo_key(v) < lim) ? lo[v] : -INFINITY;
                        hi[v] = (hi_key(v) < lim) ? hi[v] : -INFINITY;
                    }
                }
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const float x = vmax3(vmax3(lo[4 * a], lo[4 * a + 1], lo[4 * a + 2]),
                                          vmax3(lo[4 * a + 3], hi[4 * a], hi[4 * a + 1]),
                                          vmax2(hi[4 * a + 2], hi[4 * a + 3]));
                    // insert x into the sorted list: entry s becomes med3(top[s-1], top[s], x)
#pragma unroll
                    for (int s = 7; s >= 1; --s) top8[s] = __builtin_amdgcn_fmed3f(top8[s - 1], top8[s], x);
                    top8[0] = vmax2(top8[0], x);
                }
                }
            }
        }
        float* gm = reinterpret_cast<float*>(dyn_lds);                 // [ROWS][GSTRIDE]
#pragma unroll
        for (int s = 0; s < 8; ++s) gm[lane * GSTRIDE + 8 * wave + s] = top8[s];
        __syncthreads();
        float v[32];
#pragma unroll
        for (int s = 0; s < 32; ++s) v[s] = gm[lane * GSTRIDE + s];
        sort_desc<32>(v);
        float t0 = -INFINITY;
#pragma unroll
        for (int s = 0; s < 32; ++s) t0 = (s == p.sel - 1) ? v[s] : t0;
        base_thr = make_key(t0, 0xFFFFFFFFu);
        __syncthreads();                                               // gm aliases the buffers
    }
    RR_STAMP(tlb, wave, 1);
    if (wave == 0) sh.thr[lane] = (my_row < 0) ? NO_PASS_KEY : base_thr;
    __syncthreads();
    RR_STAMP(tlb, wave, 2);
    cx.trace_lb = tlb;

    // ------------------------------------------------------------------ streaming pass
    select_and_emit<DT, CAUSAL, REROUTE>(p, sh, dyn_lds, tile, kbuf, REROUTE, cx, 0);
    if constexpr (REROUTE) {
        if (sh.redo) redo_rows<DT, CAUSAL>(p, sh, dyn_lds, cx);         // uniform; rare
    }
}

template <typename DT, bool CAUSAL, bool REROUTE>
__global__ __launch_bounds__(ROWS * SPLIT) __attribute__((amdgpu_waves_per_eu(2))) void k_route(RouteArgs p) {
    extern __shared__ __align__(16) unsigned char dyn_lds[];
    __shared__ RouteShared sh;
    const int G = (p.nq + ROWS - 1) / ROWS;
    const int lb = REROUTE ? slice_major_block(p.H, G) : xcd_block(p.H * G);
    if (lb < 0) return;
    route_block<DT, CAUSAL, REROUTE>(p, lb, lb, sh, dyn_lds);
}

// The block of a grouped launch (width buckets sharing Q and K): logical blocks run head-major
// over all ledgers of the group, so one head's blocks of every bucket share an XCD (and its L2
// copy of that head's keys).  Returns the ledger, and its own block number in *lb_out (-1 for
// grid padding).
template <typename A>
__device__ __forceinline__ int group_block(int n, int per_head, const int (&off)[GROUP_MAX + 1], const A (&args)[GROUP_MAX],
                                           int rows_per_block, int H, int* lb_out) {
    const int lb = xcd_block(H * per_head);
    if (lb < 0) {
        *lb_out = -1;
        return 0;
    }
    const int h = lb / per_head;
    const int x = lb % per_head;
    int b = 0;
    while (b + 1 < n && x >= off[b + 1]) ++b;            // uniform
    const int G = (args[b].nq + rows_per_block - 1) / rows_per_block;
    *lb_out = h * G + (x - off[b]);
    return b;
}

template <typename DT, bool CAUSAL>
__global__ __launch_bounds__(ROWS * SPLIT) __attribute__((amdgpu_waves_per_eu(2))) void k_route_group(RouteGroup g) {
    extern __shared__ __align__(16) unsigned char dyn_lds[];
    __shared__ RouteShared sh;
    int lb;
    const int b = group_block(g.n, g.per_head, g.off, g.p, ROWS, g.p[0].H, &lb);
    if (lb < 0) return;
    route_block<DT, CAUSAL, false>(g.p[b], lb, (int)blockIdx.x, sh, dyn_lds);
}

// ------------------------------------------------------------------------------ rescore

// Dot product of 16-byte chunks of a query row and a key row, accumulated into a.
template <typename DT> struct Dot;
template <> struct Dot<bf16_t> {
    __device__ __forceinline__ static float acc(const uint4& q, const uint4& k, float a) {
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.x), __builtin_bit_cast(bf16x2, k.x), a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.y), __builtin_bit_cast(bf16x2, k.y), a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.z), __builtin_bit_cast(bf16x2, k.z), a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.w), __builtin_bit_cast(bf16x2, k.w), a, false);
        return a;
    }
};
template <> struct Dot<float> {
    __device__ __forceinline__ static float acc(const uint4& q, const uint4& k, float a) {
        a = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), a);
        a = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), a);
        a = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), a);
        a = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), a);
        return a;
    }
};

constexpr int RESCORE_THREADS = 1024;     // 16 waves x 4 rows: rows 64b..64b+63 of head h
constexpr int RS_WAVES = RESCORE_THREADS / 64;
constexpr int RS_ROWS = ROWS / RS_WAVES;  // rows per wave

// Raw buffer loads: a uniform base in a buffer resource plus a 32-bit per-lane offset (one
// VALU op of address arithmetic instead of a 64-bit add); offsets past `bytes` read zeros.
// Word 3 is the gfx9-family raw-buffer format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ int buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
constexpr uint32_t OOB = 0x7FFFFFF0u;                 // offset past any buffer here: reads zeros

// Reduce-scatter of per-lane partial dot products over the LPR lanes that share key rows (LPR = 8
// for bf16 rows, 16 for fp32): part[j] is this lane's share of candidate RPI j + L / LPR.  Each
// step pairs lanes that differ in one bit of the group position; a lane keeps the half of its
// values selected by that bit and adds the partner's copy of the same half.  Returns the full
// dot product of candidate cand_of_lane<LPR, NP>(L); with 32 candidates (NP = 1) lanes L and
// L ^ 1 end with the same candidate and bit-identical sums.
template <int LPR, int NP>
__device__ __forceinline__ float reduce_scatter(const float (&part)[32 * NP * LPR / 64], int lane) {
    const int b3 = (lane >> 3) & 1, b2 = (lane >> 2) & 1, b1 = (lane >> 1) & 1, b0 = lane & 1;
    (void)b3;
    float s;
    if constexpr (LPR == 8) {
        // partners: 7 - (L % 8) (bit 2 differs), L ^ 2, L ^ 1
        if constexpr (NP == 1) {
            float k0 = b2 ? part[2] : part[0], k1 = b2 ? part[3] : part[1];
            const float s0 = b2 ? part[0] : part[2], s1 = b2 ? part[1] : part[3];
            k0 += dpp_f<DPP_HALF_MIRROR>(s0);
            k1 += dpp_f<DPP_HALF_MIRROR>(s1);
            s = b1 ? k1 : k0;
            s += dpp_f<DPP_XOR2>(b1 ? k0 : k1);
            s += dpp_f<DPP_XOR1>(s);
        } else {
            float k[4], t[2];
#pragma unroll
            for (int u = 0; u < 4; ++u) k[u] = (b2 ? part[4 + u] : part[u]) + dpp_f<DPP_HALF_MIRROR>(b2 ? part[u] : part[4 + u]);
#pragma unroll
            for (int u = 0; u < 2; ++u) t[u] = (b1 ? k[2 + u] : k[u]) + dpp_f<DPP_XOR2>(b1 ? k[u] : k[2 + u]);
            s = (b0 ? t[1] : t[0]) + dpp_f<DPP_XOR1>(b0 ? t[0] : t[1]);
        }
    } else {
        // fp32 rows, 16 lanes per row: partners L ^ 8 (row rotation by 8), 7 - (L % 8), L ^ 2 [, L ^ 1]
        if constexpr (NP == 1) {
            float k[4], t[2];
#pragma unroll
            for (int u = 0; u < 4; ++u) k[u] = (b3 ? part[4 + u] : part[u]) + dpp_f<DPP_ROR8>(b3 ? part[u] : part[4 + u]);
#pragma unroll
            for (int u = 0; u < 2; ++u) t[u] = (b2 ? k[2 + u] : k[u]) + dpp_f<DPP_HALF_MIRROR>(b2 ? k[u] : k[2 + u]);
            s = (b1 ? t[1] : t[0]) + dpp_f<DPP_XOR2>(b1 ? t[0] : t[1]);
            s += dpp_f<DPP_XOR1>(s);
        } else {
            float k[8], t[4], v[2];
#pragma unroll
            for (int u = 0; u < 8; ++u) k[u] = (b3 ? part[8 + u] : part[u]) + dpp_f<DPP_ROR8>(b3 ? part[u] : part[8 + u]);
#pragma unroll
            for (int u = 0; u < 4; ++u) t[u] = (b2 ? k[4 + u] : k[u]) + dpp_f<DPP_HALF_MIRROR>(b2 ? k[u] : k[4 + u]);
#pragma unroll
            for (int u = 0; u < 2; ++u) v[u] = (b1 ? t[2 + u] : t[u]) + dpp_f<DPP_XOR2>(b1 ? t[u] : t[2 + u]);
            s = (b0 ? v[1] : v[0]) + dpp_f<DPP_XOR1>(b0 ? v[0] : v[1]);
        }
    }
    return s;
}

template <int LPR, int NP>
__device__ __forceinline__ int cand_of_lane(int lane) {
    const int b3 = (lane >> 3) & 1, b2 = (lane >> 2) & 1, b1 = (lane >> 1) & 1, b0 = lane & 1;
    const int j = (LPR == 8) ? (NP == 1 ? 2 * b2 + b1 : 4 * b2 + 2 * b1 + b0)
                             : (NP == 1 ? 4 * b3 + 2 * b2 + b1 : 8 * b3 + 4 * b2 + 2 * b1 + b0);
    return (64 / LPR) * j + lane / LPR;
}

// Rescoring of ledger rows i0 .. i0 + nrow - 1 of head h (nrow <= RPW) by one wave, one row at a
// time; afterwards lane rr (rr < RPW) holds row rr's alpha, its minimum over route + near-miss
// (the reroute threshold hint), beta, and whether a route or near-miss slot had no ID.
//
// Loads.  Each load instruction reads 8 whole key rows: lane L takes 16-byte chunk L % 8 of
// candidate 8 j + L / 8 in instruction j, so an instruction touches 8 cache lines (the address
// unit handles a load in about one cycle per line it touches, so spreading a row's candidates
// over more lines per instruction would cost more than the extra lane arithmetic below).  Each
// lane dots its chunk with the matching 16 bytes of the query row, giving partial sums for 4
// (8 when c > 32) candidates, which a reduce-scatter over the 8-lane group turns into full dot
// products: afterwards lane L holds candidate 8 (2 b2 + b1) + L / 8 (b2, b1: bits 2 and 1 of L),
// and with c <= 32 lanes L and L ^ 1 hold the same candidate.
//
// Flags.  Even lanes fold the route scores and odd lanes the route + near-miss scores into one
// min over their parity, which gives alpha (Eq. 6) and the reroute threshold hint together;
// the max over sentinel scores is beta (Eq. 7).  Two rows are reduced together.  Candidates
// without an ID count as +inf for the minima and -inf for the max; a route or near-miss slot
// without one makes the hint -inf.
//
// The wave's query rows (sq: RPW rows) and candidate IDs (sid: RPW rows of 32 * NP * NCH entries,
// -1 past c) are staged in LDS, read back by this wave only (LDS operations of one wave complete
// in order), and the key rows of the next DEPTH rows stay in flight while a row is reduced.
// Ledgers wider than 64 entries (NCH = 2, with NP = 2) take each row's candidates as two chunks
// of 64 in turn and fold the two chunks' route, near-miss and sentinel scores per lane before
// the cross-lane reduction.
template <typename DT, int NP, int RPW, int DEPTH, int NCH = 1>
__device__ __forceinline__ void rescore_rows(const RescoreArgs& p, int h, int i0, int nrow, int lane,
                                             unsigned char* sq, int32_t* sid, float& res_alpha, float& res_mu,
                                             float& res_beta, bool& res_bad) {
    static_assert(NCH == 1 || (NCH == 2 && NP == 2 && DEPTH == 1), "two chunks of 64 candidates");
    constexpr int SROW = 32 * NP * NCH;                // staged IDs per row
    typedef typename Elem<DT>::type E;
    constexpr uint32_t ROW_BYTES = 64 * sizeof(E);
    static_assert(ROW_BYTES == 128 || ROW_BYTES == 256, "bf16 or fp32 rows");
    static_assert(RPW % 2 == 0 && RPW <= 64, "rows are reduced in pairs, one result lane per row");
    constexpr int LPR = ROW_BYTES / 16;                // lanes per key row in one instruction: 8 or 16
    constexpr int RPI = 64 / LPR;                      // key rows per instruction: 8 or 4
    constexpr int NI = 32 * NP / RPI;                  // instructions per query row
    const __amdgpu_buffer_rsrc_t rQ = make_rsrc(reinterpret_cast<const char*>(p.qp) + (size_t)h * p.nq_q * ROW_BYTES,
                                                (uint32_t)p.nq_q * ROW_BYTES);
    const __amdgpu_buffer_rsrc_t rK = make_rsrc(reinterpret_cast<const char*>(p.kp) + (size_t)h * p.nk * ROW_BYTES,
                                                (uint32_t)p.nk * ROW_BYTES);
    const __amdgpu_buffer_rsrc_t rI = make_rsrc(p.ids + (size_t)h * p.nq * p.c, (uint32_t)(p.nq * p.c * 4));

    // Stage the wave's query rows and its rows' candidate IDs (contiguous in the ledger).
    {
        constexpr int PIECES = RPW * ROW_BYTES / 16;
        for (int x = lane; x < PIECES; x += 64) {
            const int rr = x / (ROW_BYTES / 16), piece = x % (ROW_BYTES / 16);
            // a width bucket's ledger row names its query row through qmap
            const int qr = p.qmap ? (rr < nrow ? p.qmap[i0 + rr] : 0) : i0 + rr;
            const uint4 v = buf_load16(rQ, rr < nrow ? (uint32_t)qr * ROW_BYTES + 16u * piece : OOB);
            *reinterpret_cast<uint4*>(sq + rr * ROW_BYTES + 16 * piece) = v;
        }
        // rows padded to SROW IDs (-1 past c), so that every later read is unconditional
        for (int x = lane; x < RPW * SROW; x += 64) {
            const int rr = x / SROW, c = x % SROW;
            const bool in = rr < nrow && c < p.c;
            const int id = buf_load4(rI, in ? (uint32_t)((i0 + rr) * p.c + c) * 4u : OOB);
            // -1 for padding, rows outside the head and any index outside K.
            sid[x] = (in && (unsigned)id < (unsigned)p.nk) ? id : -1;
        }
    }
    const int grp = lane / LPR;                         // key row within an instruction
    const uint32_t coff = 16u * (lane % LPR);           // this lane's chunk of it
    // Candidate held after the reduce-scatter (pass ps adds 32 ps).
    const int b0 = lane & 1;
    const int cown = cand_of_lane<LPR, NP>(lane);       // candidate index 0 .. 32 NP - 1 (chunk 0)

    uint4 kv[DEPTH][NI];
    auto issue = [&](int slot, int rr, int ch) {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int id = sid[rr * SROW + 32 * NP * ch + RPI * j + grp];
            kv[slot][j] = buf_load16(rK, id >= 0 ? (uint32_t)id * ROW_BYTES + coff : OOB);
        }
    };
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) issue(d, d, 0);

    res_alpha = 0.f;
    res_mu = 0.f;
    res_beta = 0.f;
    res_bad = false;
#pragma unroll
    for (int pr = 0; pr < RPW; pr += 2) {
        float A[2], B[2];
        bool bad[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int rr = pr + t;
            const int slot = rr % DEPTH;
            const int i = i0 + rr;
            const uint4 qv = *reinterpret_cast<const uint4*>(sq + rr * ROW_BYTES + coff);
            float vr = INFINITY, vsel = INFINITY;
            B[t] = -INFINITY;
            bool badc = false;
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) {
                float part[NI];
#pragma unroll
                for (int j = 0; j < NI; ++j) part[j] = Dot<DT>::acc(qv, kv[slot][j], 0.f);
                // Two candidate passes (c > 32), bf16 and fp32 alike: the next loads (8 or 16 of
                // them) would stay live through the reduce-scatter and push the kernel past its
                // register budget (64 VGPRs for bf16 at eight waves per SIMD), so they go out
                // after it.  The build's resource report and its test check that no k_rescore
                // spills.
                constexpr bool LATE = NP == 2;
                if (!LATE && rr + DEPTH < RPW) issue(slot, rr + DEPTH, 0);
                const float sc = reduce_scatter<LPR, NP>(part, lane);
                // (the fence keeps the next ID reads from being hoisted above the reduce-scatter)
                if constexpr (LATE) __builtin_amdgcn_sched_barrier(0);
                if (LATE) {
                    if (ch + 1 < NCH) issue(slot, rr, ch + 1);
                    else if (rr + DEPTH < RPW) issue(slot, rr + DEPTH, 0);
                }
                const int cc = cown + 32 * NP * ch;               // this lane's candidate
                const bool valid = sid[rr * SROW + cc] >= 0;      // -1 also past c
                const bool cR = cc < p.k, cSel = cc < p.sel, cS = cc >= p.k && cc < p.c;
                vr = vmin2(vr, (cR && valid) ? sc : INFINITY);
                vsel = vmin2(vsel, (cSel && valid) ? sc : INFINITY);
                B[t] = vmax2(B[t], (cS && valid) ? sc : -INFINITY);
                badc = badc || (cSel && !valid);
                if (p.cand_scores && i < p.nq && cc < p.c && (NP == 2 || b0 == 0))
                    p.cand_scores[((size_t)h * p.nq + i) * p.c + cc] = valid ? sc : __builtin_nanf("");
            }
            if constexpr (NP == 1) {
                A[t] = b0 ? vsel : vr;                  // lanes L and L ^ 1 hold the same candidate
            } else {
                // Pair up: the even lane takes the pair's route minimum, the odd lane its route +
                // near-miss minimum.
                A[t] = vmin2(b0 ? vsel : vr, dpp_f<DPP_XOR1>(b0 ? vr : vsel));
                B[t] = vmax2(B[t], dpp_f<DPP_XOR1>(B[t]));
            }
            bad[t] = __ballot(badc) != 0ull;
        }
        // Min / max over each parity of lanes, two rows at once: one exchange with lane ^ 2 leaves
        // the first row in lanes with bit 1 clear and the second in the others, then the common
        // steps (partners 4 and 8 apart within a row of 16, then the row swaps) reduce both.
        const bool second = (lane & 2) != 0;
        float a = vmin2(second ? A[1] : A[0], dpp_f<DPP_XOR2>(second ? A[0] : A[1]));
        float bb = vmax2(second ? B[1] : B[0], dpp_f<DPP_XOR2>(second ? B[0] : B[1]));
        a = vmin2(a, dpp_f<DPP_ROR4>(a));
        bb = vmax2(bb, dpp_f<DPP_ROR4>(bb));
        a = vmin2(a, dpp_f<DPP_ROR8>(a));
        bb = vmax2(bb, dpp_f<DPP_ROR8>(bb));
        {
            auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
            auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(bb), __float_as_uint(bb), false, false);
            a = vmin2(__uint_as_float(x[0]), __uint_as_float(x[1]));
            bb = vmax2(__uint_as_float(y[0]), __uint_as_float(y[1]));
            auto z = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
            auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(bb), __float_as_uint(bb), false, false);
            a = vmin2(__uint_as_float(z[0]), __uint_as_float(z[1]));
            bb = vmax2(__uint_as_float(w[0]), __uint_as_float(w[1]));
        }
        // Lane 0: alpha (Eq. 6) and beta (Eq. 7) of the first row, lane 1: its minimum over route
        // + near-miss (the reroute hint); lanes 2 and 3 the same for the second row.
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const float al = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 2 * t));
            const float mu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 2 * t + 1));
            const float be = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bb), 2 * t));
            const bool mine = lane == pr + t;
            res_alpha = mine ? al : res_alpha;
            res_mu = mine ? mu : res_mu;
            res_beta = mine ? be : res_beta;
            res_bad = mine ? bad[t] : res_bad;
        }
    }
}

// Eq. 8 for ledger row i of head h from its rescoring results: reuse iff alpha > beta + gamma
// (a row without any route ID is refreshed).  Hysteresis (Section 3.2, after Eq. 8): a row
// refreshed at a relay layer a is reused untested up to layer a + min_reuse, then tested with
// gamma + gamma_extra until it passes once, which clears its state.  Writes the optional
// outputs (and, for the reroute kernel, the flag / hint workspaces); returns true when the row
// is to be rerouted.
__device__ __forceinline__ bool relay_decide(const RescoreArgs& p, int h, int i, float alpha, float mu, float beta,
                                             bool bad, bool write_ws) {
    bool reuse;
    if (p.min_reuse > 0 || p.gamma_extra > 0.f) {                       // uniform
        const size_t fl = (size_t)h * p.nq + min(i, p.nq - 1);
        const bool ref = p.refreshed[fl] != 0;
        const bool skip = ref && p.layer - p.anchor[fl] <= p.min_reuse;
        const float guard = ref ? p.gamma + p.gamma_extra : p.gamma;
        reuse = skip || (alpha < INFINITY && alpha > beta + guard);
        if (i < p.nq && ref && reuse && !skip) p.refreshed[fl] = 0;
    } else {
        reuse = alpha < INFINITY && alpha > beta + p.gamma;
    }
    if (i < p.nq) {
        const size_t flat = (size_t)h * p.nq + i;
        if (write_ws) {
            p.flags_ws[flat] = reuse ? 0 : 1;
            p.hint_ws[flat] = bad ? -INFINITY : mu;
        }
        if (p.out_flags) p.out_flags[flat] = reuse ? 0 : 1;
        if (p.out_alpha) p.out_alpha[flat] = alpha;
        if (p.out_beta) p.out_beta[flat] = beta;
    }
    return i < p.nq && !reuse;
}

// Block (h, b): rows 64b..64b+63 of head h; wave w takes rows 4w..4w+3, one at a time.  The
// block ends by listing its flagged rows (ascending) for the reroute kernel.
template <typename DT, int NP, int NCH>
__global__ __launch_bounds__(RESCORE_THREADS) __attribute__((amdgpu_waves_per_eu(sizeof(typename Elem<DT>::type) == 2 ? 8 : 4)))
void k_rescore(RescoreArgs p) {
    typedef typename Elem<DT>::type E;
    constexpr uint32_t ROW_BYTES = 64 * sizeof(E);
    constexpr int LPR = ROW_BYTES / 16;
    constexpr int DEPTH = (NP == 1 && LPR == 8) ? 2 : 1;
    __shared__ uint32_t row_flag[ROWS];
    __shared__ __align__(16) unsigned char sq[RS_WAVES][RS_ROWS * ROW_BYTES];
    __shared__ int32_t sid[RS_WAVES][RS_ROWS * 32 * NP * NCH];
    const int G = (p.nq + ROWS - 1) / ROWS;
    const int lb = xcd_block(p.H * G);
    if (lb < 0) return;
    const int h = lb / G;
    const int b = lb % G;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int i0 = b * ROWS + wave * RS_ROWS;
    const int nrow = max(0, min(RS_ROWS, p.nq - i0));   // rows of this wave inside the head
    float alpha, mu, beta;
    bool bad;
    rescore_rows<DT, NP, RS_ROWS, DEPTH, NCH>(p, h, i0, nrow, lane, sq[wave], sid[wave], alpha, mu, beta, bad);
    if (lane < RS_ROWS) {
        const bool f = relay_decide(p, h, i0 + lane, alpha, mu, beta, bad, true);
        row_flag[wave * RS_ROWS + lane] = f ? 1u : 0u;
    }
    __syncthreads();
    if (wave == 0) {
        // This block's flagged rows, ascending, and their count (the reroute's compaction input).
        const bool f = row_flag[lane] != 0u;
        const uint64_t m = __ballot(f);
        const int pos = __popcll(m & ((1ull << lane) - 1ull));
        if (f) p.blist[(size_t)lb * ROWS + pos] = b * ROWS + lane;
        if (lane == 0) p.bcount[lb] = __popcll(m);
    }
}

// ------------------------------------------------------------------------------ fused relay

constexpr int RELAY_ROWS = 2 * ROWS;              // ledger rows per fused relay block
constexpr int RELAY_WAVES = 2 * SPLIT;            // its waves: two reroute slices of SPLIT waves
constexpr int RELAY_RPW = RELAY_ROWS / RELAY_WAVES;  // rows rescored per wave
constexpr uint32_t RELAY_MAX_K_BYTES = 128u << 10;  // a head's keys staged in LDS (1024 bf16 rows)
// Words between two rows' staged candidate IDs: 32 IDs plus a pad, so that the 16 rows a
// quarter-wave reads at once start in 16 different 4-bank groups (16-byte aligned rows).
constexpr int RELAY_SID_STRIDE = 36;

// Rescoring of ledger rows i0 .. i0 + nrow - 1 (nrow <= RPW) by one wave with the head's key rows
// resident in LDS (kl: nk rows of 64 elements) and the candidate IDs staged per wave (sid: RPW
// rows of 32 entries, -1 past c <= 32): the same candidate-to-lane layout, reduce-scatter and min / max folding as
// rescore_rows, with every key chunk read from LDS (one 16-byte read per lane and 8 candidates).
// qv[rr]: this lane's 16-byte chunk of row rr's query.  Results as rescore_rows (lane rr).
template <typename DT, int RPW>
__device__ __forceinline__ void rescore_rows_lds(const RescoreArgs& p, int h, int i0, int lane, const unsigned char* kl,
                                                 const int32_t* sid, const uint4 (&qv)[RPW], float* res_lds,
                                                 float& res_alpha, float& res_mu, float& res_beta, bool& res_bad) {
    typedef typename Elem<DT>::type E;
    constexpr uint32_t ROW_BYTES = 64 * sizeof(E);
    constexpr int LPR = ROW_BYTES / 16;
    constexpr int RPI = 64 / LPR;
    constexpr int NI = 32 / RPI;                       // one pass of 32 candidates
    const int grp = lane / LPR;
    const uint32_t coff = 16u * (lane % LPR);
    const int b0 = lane & 1;
    const int cown = cand_of_lane<LPR, 1>(lane);
    const bool ownR = cown < p.k, ownSel = cown < p.sel, ownS = cown >= p.k && cown < p.c;
    uint32_t badmask = 0u;                             // bit rr: row rr has a missing route / near-miss ID
#pragma unroll
    for (int pr = 0; pr < RPW; pr += 2) {
        float A[2], B[2];
        bool bad[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int rr = pr + t;
            const int i = i0 + rr;
            float part[NI];
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                // Unconditional: a missing ID reads row 0, and its score is masked by `valid`
                // below (a branch here would serialise every read behind its ID read).
                const int id = sid[rr * RELAY_SID_STRIDE + RPI * j + grp];
                const uint4 kv = *reinterpret_cast<const uint4*>(kl + (size_t)max(id, 0) * ROW_BYTES + coff);
                part[j] = Dot<DT>::acc(qv[rr], kv, 0.f);
            }
            const float sc = reduce_scatter<LPR, 1>(part, lane);
            const bool valid = sid[rr * RELAY_SID_STRIDE + cown] >= 0;   // -1 also past c
            const float vr = (ownR && valid) ? sc : INFINITY;
            const float vsel = (ownSel && valid) ? sc : INFINITY;
            B[t] = (ownS && valid) ? sc : -INFINITY;
            A[t] = b0 ? vsel : vr;                      // lanes L and L ^ 1 hold the same candidate
            bad[t] = __ballot(ownSel && !valid) != 0ull;
            if (p.cand_scores) {                        // uniform
                if (i < p.nq && cown < p.c && b0 == 0)
                    p.cand_scores[((size_t)h * p.nq + i) * p.c + cown] = valid ? sc : __builtin_nanf("");
            }
        }
        const bool second = (lane & 2) != 0;
        float a = vmin2(second ? A[1] : A[0], dpp_f<DPP_XOR2>(second ? A[0] : A[1]));
        float bb = vmax2(second ? B[1] : B[0], dpp_f<DPP_XOR2>(second ? B[0] : B[1]));
        a = vmin2(a, dpp_f<DPP_ROR4>(a));
        bb = vmax2(bb, dpp_f<DPP_ROR4>(bb));
        a = vmin2(a, dpp_f<DPP_ROR8>(a));
        bb = vmax2(bb, dpp_f<DPP_ROR8>(bb));
        {
            auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
            auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(bb), __float_as_uint(bb), false, false);
            a = vmin2(__uint_as_float(x[0]), __uint_as_float(x[1]));
            bb = vmax2(__uint_as_float(y[0]), __uint_as_float(y[1]));
            auto z = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
            auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(bb), __float_as_uint(bb), false, false);
            a = vmin2(__uint_as_float(z[0]), __uint_as_float(z[1]));
            bb = vmax2(__uint_as_float(w[0]), __uint_as_float(w[1]));
        }
        // Lanes 2t and 2t + 1 hold alpha and mu of row pr + t, lane 2t its beta: straight to the
        // wave's result slot (alpha, mu at 2 rr, 2 rr + 1; beta at 2 RPW + rr).
        if (lane < 4) res_lds[2 * pr + lane] = a;
        if (lane < 4 && (lane & 1) == 0) res_lds[2 * RPW + pr + (lane >> 1)] = bb;
        badmask |= (bad[0] ? 1u : 0u) << pr;
        badmask |= (bad[1] ? 1u : 0u) << (pr + 1);
    }
    // The same wave wrote the slot: its LDS operations complete in order.
    const int rr = lane < RPW ? lane : 0;
    res_alpha = res_lds[2 * rr];
    res_mu = res_lds[2 * rr + 1];
    res_beta = res_lds[2 * RPW + rr];
    res_bad = ((badmask >> rr) & 1u) != 0u;
}

// The same rescoring for bf16 keys on the matrix cores (Section 3.2, Eq. 5-7).  For candidate
// slot c, two 16x16x32 products give D[m][n] = K[id(m, c)] . Q[n] over the wave's 16 rows m, n;
// the scores wanted are the diagonal D[n][n], which lands in register n % 4 of lane
// n + 16 (n / 4) (lane L holds D[4 (L / 16) + v][L % 16]).  The four lanes L with L % 16 = n
// supply row n's candidate key (A) and query (B), each a 16-byte chunk of the 64 dims per
// product; A and B take the same chunk in the same lane, so a diagonal entry sums all 64 dims
// whatever chunk each lane takes (off-diagonal entries mix chunks and are never read).  Lane
// (n, g = L / 16) takes chunk relay_chunk(n, g, s) in product s: the 8 lanes n = 8a .. 8a + 7 of a
// quarter-wave then read 8 different 16-byte columns of their 8 key rows, which fall in 8
// different bank groups whatever the rows.  Fifteen of every sixteen products are discarded:
// the matrix cores are otherwise idle here, and the dot products cost no vector instructions.
// The diagonal lanes fold alpha (route), mu (route + near-miss: the reroute hint) and beta
// (sentinels) over the slots; the other lanes' folds are never read.
// qb[s]: this lane's query chunk relay_chunk(L % 16, L / 16, s).
__device__ __forceinline__ constexpr int relay_chunk(int n, int g, int s) {
    return 4 * (s ^ ((n >> 2) & 1)) + ((g + n) & 3);
}

// One pass over the 32 candidate slots, eight at a time: the key reads of the next eight slots
// are issued before the products of the current eight (scheduling barriers keep the compiler
// from sinking them back, which would leave one LDS round trip per slot).  The slot classes
// (route c < k, route + near-miss c < k + m, sentinel c >= k) are compared in vector registers:
// as scalar conditions the compiler hoisted all 96 of them and spilled them.  SCORES also writes
// every candidate's score (a uniform choice made outside the loop).
template <bool SCORES>
__device__ __forceinline__ void rescore_slots_mfma(const RescoreArgs& p, const int (&id)[32], const unsigned char* kl,
                                                   uint32_t off0, uint32_t off1, const bf16x8 (&qb)[2], int v,
                                                   float* srow_out, float& a, float& mu, float& b, bool& bad) {
    constexpr int GS = 8;                              // slots per group
    int kv = p.k, selv = p.sel, cv = p.c;
    asm volatile("" : "+v"(kv), "+v"(selv), "+v"(cv));
    bf16x8 kb[2][GS][2];
    auto issue = [&](int grp, int buf) {
#pragma unroll
        for (int j = 0; j < GS; ++j) {
            // A missing ID reads key row 0; its score is masked by `valid`.
            const unsigned char* kr = kl + (uint32_t)max(id[GS * grp + j], 0) * 128u;
            kb[buf][j][0] = *reinterpret_cast<const bf16x8*>(kr + off0);
            kb[buf][j][1] = *reinterpret_cast<const bf16x8*>(kr + off1);
        }
    };
    issue(0, 0);
#pragma unroll
    for (int grp = 0; grp < 32 / GS; ++grp) {
        const int buf = grp & 1;
        if (grp + 1 < 32 / GS) issue(grp + 1, buf ^ 1);
        __builtin_amdgcn_sched_barrier(0);
        // All products of the group first, each slot in its own accumulator, so that the
        // matrix core runs them back to back while the folds of earlier slots proceed.
        f32x4 dd[GS];
#pragma unroll
        for (int j = 0; j < GS; ++j) {
            dd[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            dd[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[buf][j][0], qb[0], dd[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < GS; ++j)
            dd[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[buf][j][1], qb[1], dd[j], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < GS; ++j) {
            const int c = GS * grp + j;
            const bool valid = id[c] >= 0;             // -1: padding, past c, outside K
            const f32x4 d = dd[j];
            const float lo = (v & 1) ? d[1] : d[0];
            const float hi = (v & 1) ? d[3] : d[2];
            const float sc = (v & 2) ? hi : lo;
            const bool isR = c < kv, isSel = c < selv;
            a = vmin2(a, (isR && valid) ? sc : INFINITY);
            mu = vmin2(mu, (isSel && valid) ? sc : INFINITY);
            bad = bad || (isSel && !valid);
            b = vmax2(b, (!isR && valid) ? sc : -INFINITY);   // past c the ID is -1
            if constexpr (SCORES) {
                if (srow_out != nullptr && c < cv) srow_out[c] = valid ? sc : __builtin_nanf("");
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int RPW>
__device__ __forceinline__ void rescore_rows_lds_mfma(const RescoreArgs& p, int h, int i0, int lane,
                                                      const unsigned char* kl, const int32_t* sid,
                                                      const bf16x8 (&qb)[2], float* res_lds, float& res_alpha,
                                                      float& res_mu, float& res_beta, bool& res_bad) {
    static_assert(RPW == 16, "one 16x16 product per candidate slot");
    const int n = lane & 15, g = lane >> 4, v = lane & 3;
    const bool diag = (n >> 2) == g;
    int id[32];
    {
        const int4* srow = reinterpret_cast<const int4*>(sid + n * RELAY_SID_STRIDE);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int4 x = srow[u];
            id[4 * u] = x.x;
            id[4 * u + 1] = x.y;
            id[4 * u + 2] = x.z;
            id[4 * u + 3] = x.w;
        }
    }
    const uint32_t off0 = 16u * relay_chunk(n, g, 0), off1 = 16u * relay_chunk(n, g, 1);
    float a = INFINITY, mu = INFINITY, b = -INFINITY;
    bool bad = false;
    if (p.cand_scores) {                                // uniform: checks only
        float* out = (diag && i0 + n < p.nq) ? p.cand_scores + ((size_t)h * p.nq + i0 + n) * p.c : nullptr;
        rescore_slots_mfma<true>(p, id, kl, off0, off1, qb, v, out, a, mu, b, bad);
    } else {
        rescore_slots_mfma<false>(p, id, kl, off0, off1, qb, v, nullptr, a, mu, b, bad);
    }
    if (diag) {
        res_lds[2 * n] = a;
        res_lds[2 * n + 1] = mu;
        res_lds[2 * RPW + n] = b;
    }
    const uint64_t badmask = __ballot(diag && bad);
    // The same wave wrote the slot: its LDS operations complete in order.
    const int rr = lane < RPW ? lane : 0;
    res_alpha = res_lds[2 * rr];
    res_mu = res_lds[2 * rr + 1];
    res_beta = res_lds[2 * RPW + rr];
    res_bad = ((badmask >> (rr + 16 * (rr >> 2))) & 1ull) != 0ull;
}

// One relay layer (Sections 3.2, 4.1, 4.2) for 128 ledger rows of one head in one block of
// eight waves (one block per compute unit):
//   1. the head's keys (nk rows, at most 128 KB) are staged in LDS once, together with each
//      wave's 16 rows of candidate IDs, and every row is rescored from LDS (rescore_rows_lds)
//      and decided (Eq. 8);
//   2. compaction: the block's flagged rows, ascending, go to the row slots 0 .. n-1 (ballot +
//      prefix count over the two 64-row halves), each with its reroute threshold from its own
//      rescoring (the smallest current score over its route and near-miss chunks, less a
//      rounding margin: a lower bound on its (k+m)-th best score); per 64-row half, the flagged
//      rows and their count also go to blist / bcount for the compacted-list output;
//   3. reroute: slots 0-63 and 64-127 are two independent 64-row slices, each routed by four
//      waves with the route kernel's streaming selection and ledger write (select_and_emit);
//      the keys' LDS area is reused for the slices' buffers.  A slice without rows streams no
//      key tile.  The block-wide barriers inside select_and_emit are met by both slices in the
//      same order; a redo (rare) runs in both when either needs it.
// At the usual flagged fractions (around 0.6) the ~77 flagged rows of a block fill one slice
// and part of the other, so the reroute runs at the occupancy of full routing (two 64-row
// slices per compute unit) without its threshold pass, and the rescoring reads keys from LDS
// instead of gathering them from L2.  A block without a flagged row stops after step 2.
// Block-shared state of a fused relay block.
struct RelayShared {
    RouteShared sh[2];
    uint32_t rflag[RELAY_ROWS];
    float rhint[RELAY_ROWS];
    float rres[RELAY_WAVES][3 * RELAY_RPW];   // each wave's rescoring results (alpha, mu | beta)
    int nflag[2];
};

// One fused relay block: 128 ledger rows of one head (block lb = h * G2 + g2 of the ledger's
// grid).  tlb: the block's number in phase traces.
template <typename DT, bool CAUSAL>
__device__ __forceinline__ void relay_block(const RescoreArgs& s, const RouteArgs& p, int lb, int tlb,
                                            RelayShared& rs, unsigned char* dyn_lds) {
    typedef typename Elem<DT>::type E;
    constexpr uint32_t ROW_BYTES = 64 * sizeof(E);
    constexpr int LPR = ROW_BYTES / 16;
    constexpr int KPIECES = RELAY_MAX_K_BYTES / 16 / (ROWS * RELAY_WAVES);   // 16-byte pieces per thread
    RouteShared (&sh)[2] = rs.sh;
    uint32_t (&rflag)[RELAY_ROWS] = rs.rflag;
    float (&rhint)[RELAY_ROWS] = rs.rhint;
    int (&nflag)[2] = rs.nflag;
    (void)tlb;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G2 = (p.nq + RELAY_ROWS - 1) / RELAY_ROWS;
    const int h = lb / G2;
    const int g2 = lb % G2;
    const uint32_t kbytes = (uint32_t)p.nk * ROW_BYTES;
    unsigned char* kl = dyn_lds;
    int32_t* sid = reinterpret_cast<int32_t*>(dyn_lds + RELAY_MAX_K_BYTES) + (size_t)wave * RELAY_RPW * RELAY_SID_STRIDE;
    const int i0 = g2 * RELAY_ROWS + wave * RELAY_RPW;
    const int nrow = max(0, min(RELAY_RPW, p.nq - i0));
    RR_STAMP(tlb, wave, 0);

    // ------------------------------------------------------------------ 1. staging + rescoring
    {
        const __amdgpu_buffer_rsrc_t rK = make_rsrc(reinterpret_cast<const char*>(s.kp) + (size_t)h * p.nk * ROW_BYTES,
                                                    kbytes);
        const __amdgpu_buffer_rsrc_t rQ = make_rsrc(reinterpret_cast<const char*>(s.qp) + (size_t)h * s.nq_q * ROW_BYTES,
                                                    (uint32_t)s.nq_q * ROW_BYTES);
        const __amdgpu_buffer_rsrc_t rI = make_rsrc(s.ids + (size_t)h * s.nq * s.c, (uint32_t)(s.nq * s.c * 4));
        // The keys go straight from memory to LDS (buffer loads with an LDS destination, 1 KB per
        // wave and instruction; bytes past the head's keys read as zeros), beside the IDs and the
        // query chunks, which go through registers.
#pragma unroll
        for (int x = 0; x < KPIECES; ++x) {
            const uint32_t chunk = (uint32_t)(wave * KPIECES + x) * 1024u;
            if (chunk < kbytes)                         // uniform
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rK, (__attribute__((address_space(3))) void*)(kl + chunk), 16,
                    (int)(chunk + 16u * (uint32_t)lane), 0, 0, 0);
        }
        int idv[RELAY_RPW * 32 / 64];                   // rows padded to 32 IDs
#pragma unroll
        for (int u = 0; u < RELAY_RPW * 32 / 64; ++u) {
            const int x = lane + 64 * u, rr = x / 32, c = x % 32;
            idv[u] = buf_load4(rI, (rr < nrow && c < s.c) ? (uint32_t)((i0 + rr) * s.c + c) * 4u : OOB);
        }
        constexpr bool MFMA_RESCORE = sizeof(E) == 2;   // bf16: rescoring on the matrix cores
        uint4 qv[MFMA_RESCORE ? 1 : RELAY_RPW];
        bf16x8 qb[2];
        if constexpr (MFMA_RESCORE) {
            // Row L % 16, chunk relay_chunk(L % 16, L / 16, s) (see rescore_rows_lds_mfma).
            const int rr = lane & 15;
            const int qr = s.qmap ? (rr < nrow ? s.qmap[i0 + rr] : 0) : i0 + rr;
#pragma unroll
            for (int hs = 0; hs < 2; ++hs) {
                const uint32_t off = 16u * (uint32_t)relay_chunk(rr, lane >> 4, hs);
                const uint4 x = buf_load16(rQ, rr < nrow ? (uint32_t)qr * ROW_BYTES + off : OOB);
                qb[hs] = __builtin_bit_cast(bf16x8, x);
            }
            qv[0] = make_uint4(0u, 0u, 0u, 0u);
        } else {
            const uint32_t coff = 16u * (lane % LPR);
#pragma unroll
            for (int rr = 0; rr < RELAY_RPW; ++rr) {
                const int qr = s.qmap ? (rr < nrow ? s.qmap[i0 + rr] : 0) : i0 + rr;
                qv[rr] = buf_load16(rQ, rr < nrow ? (uint32_t)qr * ROW_BYTES + coff : OOB);
            }
        }
#pragma unroll
        for (int u = 0; u < RELAY_RPW * 32 / 64; ++u) {
            const int x = lane + 64 * u, rr = x / 32, c = x % 32;
            // -1 for padding (also past c), rows outside the head and any index outside K
            sid[rr * RELAY_SID_STRIDE + c] = (rr < nrow && c < s.c && (unsigned)idv[u] < (unsigned)s.nk) ? idv[u] : -1;
        }
        __builtin_amdgcn_s_waitcnt(0);                  // this wave's key chunks have landed
        __syncthreads();                                // the keys are in LDS
        RR_STAMP(tlb, wave, 1);
        float alpha, mu, beta;
        bool bad;
        if constexpr (MFMA_RESCORE) {
            (void)qv;
            rescore_rows_lds_mfma<RELAY_RPW>(s, h, i0, lane, kl, sid, qb, rs.rres[wave], alpha, mu, beta, bad);
        } else {
            (void)qb;
            rescore_rows_lds<DT, RELAY_RPW>(s, h, i0, lane, kl, sid, qv, rs.rres[wave], alpha, mu, beta, bad);
        }
        if (lane < RELAY_RPW) {
            const bool f = relay_decide(s, h, i0 + lane, alpha, mu, beta, bad, false);
            rflag[wave * RELAY_RPW + lane] = f ? 1u : 0u;
            rhint[wave * RELAY_RPW + lane] = bad ? -INFINITY : mu;
        }
    }
    RR_STAMP(tlb, wave, 2);
    __syncthreads();                                    // flags ready; the keys' LDS is free
    RR_STAMP(tlb, wave, 3);

    // ------------------------------------------------------------------ 2. compaction
    if (wave < 2) {
        // wave w takes the rows of half w (64 w .. 64 w + 63 of the block)
        const int G = (p.nq + ROWS - 1) / ROWS;        // 64-row groups per head (blist / bcount)
        const int grp = 2 * g2 + wave;
        const bool f = rflag[64 * wave + lane] != 0u;
        const uint64_t m = __ballot(f);
        const int cnt = __popcll(m);
        const int pos = __popcll(m & ((1ull << lane) - 1ull));
        const int cnt0 = __popcll(__ballot(rflag[lane] != 0u));
        const int total = cnt0 + __popcll(__ballot(rflag[64 + lane] != 0u));
        const int row = 64 * grp + lane;                // ledger row within the head
        if (f) {                                        // slot: half 0 first, then half 1
            const int slot = (wave == 0 ? 0 : cnt0) + pos;
            RouteShared& dst = sh[slot >> 6];
            const int sl = slot & 63;
            dst.rows[sl] = row;
            dst.qrows[sl] = p.qmap ? p.qmap[row] : row;
            const float hv = rhint[64 * wave + lane];
            const float t = (hv == -INFINITY) ? -INFINITY : hv - (fabsf(hv) * 1e-4f + 1e-6f);
            dst.thr[sl] = make_key(t, 0xFFFFFFFFu);
            s.blist[((size_t)h * G + grp) * ROWS + pos] = row;
        }
        if (64 * wave + lane >= total) {                // slots past the flagged rows: no row
            sh[wave].rows[lane] = -1;
            sh[wave].qrows[lane] = -1;
            sh[wave].thr[lane] = NO_PASS_KEY;
        }
        if (lane == 0) {
            if (grp < G) s.bcount[(size_t)h * G + grp] = cnt;
            nflag[wave] = wave == 0 ? min(total, 64) : max(total - 64, 0);
            sh[wave].redo = 0;
        }
    }
    __syncthreads();
    RR_STAMP(tlb, wave, 4);
    if (nflag[0] == 0) return;                          // uniform: nothing to reroute

    // ------------------------------------------------------------------ 3. reroute, two slices
    const int slice = wave / SPLIT;
    const int wv = wave % SPLIT;
    unsigned char* lds_s = dyn_lds + (size_t)slice * route_lds_bytes_dev(p.nk, p.c);
    RowCtx<DT> cx = row_context<DT, CAUSAL>(p, sh[slice], lds_s, h, wv, lane);
    cx.trace_lb = tlb;
    cx.trace_w = wave;
    Tile<DT> tile;
    typename Tile<DT>::KReg kbuf[Tile<DT>::NBUF];
    select_and_emit<DT, CAUSAL, true>(p, sh[slice], lds_s, tile, kbuf, false, cx, 0);
    if (sh[0].redo || sh[1].redo) redo_rows<DT, CAUSAL>(p, sh[slice], lds_s, cx);    // uniform; rare
}

template <typename DT, bool CAUSAL>
__global__ __launch_bounds__(ROWS * RELAY_WAVES) __attribute__((amdgpu_waves_per_eu(2)))
void k_relay(RescoreArgs s, RouteArgs p) {
    extern __shared__ __align__(16) unsigned char dyn_lds[];
    __shared__ RelayShared rs;
    const int G2 = (p.nq + RELAY_ROWS - 1) / RELAY_ROWS;
    const int lb = xcd_block(p.H * G2);
    if (lb < 0) return;
    relay_block<DT, CAUSAL>(s, p, lb, lb, rs, dyn_lds);
}

// A fused relay layer over several width-bucket ledgers in one grid (see group_block).
template <typename DT, bool CAUSAL>
__global__ __launch_bounds__(ROWS * RELAY_WAVES) __attribute__((amdgpu_waves_per_eu(2)))
void k_relay_group(RelayGroup g) {
    extern __shared__ __align__(16) unsigned char dyn_lds[];
    __shared__ RelayShared rs;
    int lb;
    const int b = group_block(g.n, g.per_head, g.off, g.p, RELAY_ROWS, g.p[0].H, &lb);
    if (lb < 0) return;
    relay_block<DT, CAUSAL>(g.s[b], g.p[b], lb, (int)blockIdx.x, rs, dyn_lds);
}

// The compacted list of a relay layer (Sections 4.1-4.2: ascending h * nq + i of the flagged
// rows), the flagged rows per head and their total, from the per-block flag counts and
// ascending row lists (bcount [H, G], blist [H, G, 64]) that the relay leaves: one wave per
// head.  Launched only when the caller asks for these outputs.
__global__ __launch_bounds__(64) void k_compact_out(const int32_t* bcount, const int32_t* blist, int H, int nq,
                                                     int32_t* out_rows, int32_t* out_head_counts,
                                                     int32_t* out_n_rows) {
    const int h = blockIdx.x;
    const int lane = threadIdx.x;
    const int G = (nq + ROWS - 1) / ROWS;
    int acc = 0;                                        // flagged rows in the heads before h
    for (int x = lane; x < h * G; x += 64) acc += bcount[x];
    const int offset = wave_sum_i(acc);
    const int32_t* bc = bcount + (size_t)h * G;
    const int32_t* bl = blist + (size_t)h * G * ROWS;
    int run = 0;
    for (int b0 = 0; b0 < G; b0 += 64) {                // uniform
        const int cnt = (b0 + lane < G) ? bc[b0 + lane] : 0;
        const int incl = wave_incl_scan_i(cnt);
        if (out_rows) {
            const int nb = min(64, G - b0);
            for (int bb = 0; bb < nb; ++bb) {
                const int cb = __builtin_amdgcn_readlane(cnt, bb);
                const int base = run + __builtin_amdgcn_readlane(incl, bb) - cb;
                if (lane < cb) out_rows[offset + base + lane] = h * nq + bl[(size_t)(b0 + bb) * ROWS + lane];
            }
        }
        run += __builtin_amdgcn_readlane(incl, 63);
    }
    if (lane == 0) {
        if (out_head_counts) out_head_counts[h] = run;
        if (out_n_rows && h == H - 1) out_n_rows[0] = offset + run;
    }
}

// ------------------------------------------------------------------------------ launchers



template <typename DT, bool CAUSAL, bool REROUTE>
static hipError_t launch_route_t(const RouteArgs& a, hipStream_t st) {
    const int G = (a.nq + ROWS - 1) / ROWS;
    const size_t lds = route_lds_bytes(a.nk, a.c);
    hipLaunchKernelGGL((k_route<DT, CAUSAL, REROUTE>), dim3(xcd_grid(a.H * G)), dim3(ROWS * SPLIT), lds, st, a);
    return hipGetLastError();
}

hipError_t launch_route(const RouteArgs& a, bool bf16, bool causal, bool reroute, hipStream_t st) {
    if (bf16) {
        if (causal) return reroute ? launch_route_t<bf16_t, true, true>(a, st) : launch_route_t<bf16_t, true, false>(a, st);
        return reroute ? launch_route_t<bf16_t, false, true>(a, st) : launch_route_t<bf16_t, false, false>(a, st);
    }
    if (causal) return reroute ? launch_route_t<float, true, true>(a, st) : launch_route_t<float, true, false>(a, st);
    return reroute ? launch_route_t<float, false, true>(a, st) : launch_route_t<float, false, false>(a, st);
}

size_t relay_lds_bytes(int nk, int c, bool bf16) {
    const size_t stage = RELAY_MAX_K_BYTES + (size_t)RELAY_WAVES * RELAY_RPW * RELAY_SID_STRIDE * sizeof(int32_t);
    const size_t slices = 2 * route_lds_bytes_dev(nk, c);
    (void)bf16;
    return stage > slices ? stage : slices;
}

bool relay_fits(int nk, int c, int sel, bool bf16) {
    const size_t row_bytes = bf16 ? 128 : 256;
    return sel <= 32 && c <= 32 && (size_t)nk * row_bytes <= RELAY_MAX_K_BYTES &&
           relay_lds_bytes(nk, c, bf16) + sizeof(RelayShared) + 64 <= (160u << 10);
}

template <typename DT, bool CAUSAL>
static hipError_t launch_relay_t(const RescoreArgs& s, const RouteArgs& a, hipStream_t st) {
    const int G2 = (a.nq + RELAY_ROWS - 1) / RELAY_ROWS;
    const size_t lds = relay_lds_bytes(a.nk, a.c, sizeof(typename Elem<DT>::type) == 2);
    hipLaunchKernelGGL((k_relay<DT, CAUSAL>), dim3(xcd_grid(a.H * G2)), dim3(ROWS * RELAY_WAVES), lds, st, s, a);
    return hipGetLastError();
}

hipError_t launch_relay(const RescoreArgs& s, const RouteArgs& a, bool bf16, bool causal, hipStream_t st) {
    if (!relay_fits(a.nk, a.c, a.sel, bf16)) return hipErrorInvalidValue;
    if (bf16) return causal ? launch_relay_t<bf16_t, true>(s, a, st) : launch_relay_t<bf16_t, false>(s, a, st);
    return causal ? launch_relay_t<float, true>(s, a, st) : launch_relay_t<float, false>(s, a, st);
}

template <typename DT, bool CAUSAL>
static hipError_t launch_route_group_t(const RouteGroup& g, hipStream_t st) {
    size_t lds = 0;
    for (int b = 0; b < g.n; ++b) lds = std::max(lds, route_lds_bytes(g.p[b].nk, g.p[b].c));
    hipLaunchKernelGGL((k_route_group<DT, CAUSAL>), dim3(xcd_grid(g.p[0].H * g.per_head)), dim3(ROWS * SPLIT), lds,
                       st, g);
    return hipGetLastError();
}

hipError_t launch_route_group(const RouteGroup& g, bool bf16, bool causal, hipStream_t st) {
    if (g.n < 1 || g.n > GROUP_MAX) return hipErrorInvalidValue;
    for (int b = 0; b < g.n; ++b)
        if (g.p[b].sel > 32) return hipErrorInvalidValue;
    if (bf16) return causal ? launch_route_group_t<bf16_t, true>(g, st) : launch_route_group_t<bf16_t, false>(g, st);
    return causal ? launch_route_group_t<float, true>(g, st) : launch_route_group_t<float, false>(g, st);
}

template <typename DT, bool CAUSAL>
static hipError_t launch_relay_group_t(const RelayGroup& g, hipStream_t st) {
    size_t lds = 0;
    for (int b = 0; b < g.n; ++b)
        lds = std::max(lds, relay_lds_bytes(g.p[b].nk, g.p[b].c, sizeof(typename Elem<DT>::type) == 2));
    hipLaunchKernelGGL((k_relay_group<DT, CAUSAL>), dim3(xcd_grid(g.p[0].H * g.per_head)), dim3(ROWS * RELAY_WAVES),
                       lds, st, g);
    return hipGetLastError();
}

hipError_t launch_relay_group(const RelayGroup& g, bool bf16, bool causal, hipStream_t st) {
    if (g.n < 1 || g.n > GROUP_MAX) return hipErrorInvalidValue;
    for (int b = 0; b < g.n; ++b)
        if (!relay_fits(g.p[b].nk, g.p[b].c, g.p[b].sel, bf16)) return hipErrorInvalidValue;
    if (bf16) return causal ? launch_relay_group_t<bf16_t, true>(g, st) : launch_relay_group_t<bf16_t, false>(g, st);
    return causal ? launch_relay_group_t<float, true>(g, st) : launch_relay_group_t<float, false>(g, st);
}

hipError_t launch_compact_out(const int32_t* bcount, const int32_t* blist, int H, int nq, int32_t* out_rows,
                              int32_t* out_head_counts, int32_t* out_n_rows, hipStream_t st) {
    hipLaunchKernelGGL(k_compact_out, dim3(H), dim3(64), 0, st, bcount, blist, H, nq, out_rows, out_head_counts,
                       out_n_rows);
    return hipGetLastError();
}

hipError_t launch_rescore(const RescoreArgs& a, bool bf16, hipStream_t st) {
    const dim3 grid(xcd_grid(a.H * ((a.nq + ROWS - 1) / ROWS)));
    // candidate passes of 32: one (c <= 32), two (c <= 64), or two chunks of two (c <= 128)
    const int passes = (a.c + 31) / 32;
    if (passes > 4) return hipErrorInvalidValue;
    if (bf16) {
        if (passes > 2) hipLaunchKernelGGL((k_rescore<bf16_t, 2, 2>), grid, dim3(RESCORE_THREADS), 0, st, a);
        else if (passes == 2) hipLaunchKernelGGL((k_rescore<bf16_t, 2, 1>), grid, dim3(RESCORE_THREADS), 0, st, a);
        else hipLaunchKernelGGL((k_rescore<bf16_t, 1, 1>), grid, dim3(RESCORE_THREADS), 0, st, a);
    } else {
        if (passes > 2) hipLaunchKernelGGL((k_rescore<float, 2, 2>), grid, dim3(RESCORE_THREADS), 0, st, a);
        else if (passes == 2) hipLaunchKernelGGL((k_rescore<float, 2, 1>), grid, dim3(RESCORE_THREADS), 0, st, a);
        else hipLaunchKernelGGL((k_rescore<float, 1, 1>), grid, dim3(RESCORE_THREADS), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace rr

#ifdef RR_PHASE_TRACE
// Measurement builds only: copy out / clear the phase tables ([block][wave][slot] timestamps,
// [block][wave] mid-stream drain counts).  Return 0 on success.
extern "C" int rr_debug_phase_trace(uint64_t* stamps, size_t n_stamps, uint32_t* drains, size_t n_drains) {
    if (n_stamps > sizeof(rr::g_phase) / 8 || n_drains > sizeof(rr::g_drains) / 4) return -1;
    if (hipMemcpyFromSymbol(stamps, HIP_SYMBOL(rr::g_phase), n_stamps * 8, 0, hipMemcpyDeviceToHost) != hipSuccess)
        return -1;
    return hipMemcpyFromSymbol(drains, HIP_SYMBOL(rr::g_drains), n_drains * 4, 0, hipMemcpyDeviceToHost) ==
                   hipSuccess ? 0 : -1;
}
extern "C" int rr_debug_phase_clear(void) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(rr::g_phase)) != hipSuccess) return -1;
    if (hipMemset(p, 0, sizeof(rr::g_phase)) != hipSuccess) return -1;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(rr::g_drains)) != hipSuccess) return -1;
    return hipMemset(p, 0, sizeof(rr::g_drains)) == hipSuccess ? 0 : -1;
}
#endif
