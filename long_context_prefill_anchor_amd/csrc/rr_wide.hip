// Routing with near-miss sets wider than the main route kernel's 32-entry lists
// (32 < k + m <= 64): MFMA scores into LDS, then one wave per query row for the selection.
//
// "RouteRelay: Event-Triggered Cross-Layer Route Reuse for Efficient Dynamic Sparse
// Attention", Section 2.1 Eq. 1-2 (scores, top-k route), Section 3.1 items 1-3 (near-miss,
// random and mandatory sentinels, Eq. 4 ledger), Sections 4.1-4.2 (reroute of flagged rows);
// Table 3 evaluates 24- and 48-wide near-miss sets.
//
// A block takes 16 consecutive query rows of one head.  Its eight waves first score the rows
// against every key with v_mfma_f32_16x16x32_bf16 (fp32 inputs: v_mfma_f32_16x16x4f32), 16
// keys per tile and tiles dealt round-robin to the waves, into an LDS table of orderable fp32
// scores (0 = no key).  Each row then goes to one wave (two rows per wave, side by side, so
// that their exchange chains interleave), which finds its exact top-(k+m) over
// the 64-bit keys (orderable score, then lower index first): lane l holds keys l, l + 64, ...;
// the (k+m)-th largest of the 64 lane maxima is a lower bound of the (k+m)-th largest key, so
// the keys at or above it (at least k+m of them, at most 64 in the common case) are compacted
// and sorted across lanes with a bitonic network, leaving rank r in lane r; when more than 64
// keys pass the bound, an exact radix select over the 64-bit keys finds the threshold instead.
// Route and near-miss are put in index order by a second lane sort.  Lane exchanges are DPP
// moves and the 16- and 32-lane swaps, so the sorts stay in the VALU.  Route = the k largest,
// near-miss = the next m.  The ledger row is then written with the same
// rules as the main kernel: segments ascending by index, mandatory sink / recent chunks not
// already routed, random draws from Philox4x32-10 (counter = (t div 4, query row, layer,
// head)) accepted in draw order when the chunk is still in the pool, a fill with the
// lowest-index free chunks when the pool is not larger than r or the draw cap is reached.
// The kernel keeps no threshold state, so anchor and reroute use it alike; in a reroute the
// blocks of a head take its flagged rows in ascending order, 16 per block, from the rescore
// kernel's per-64-row counts and lists (the compaction of Sections 4.1-4.2), so that only
// ceil(flagged / 16) blocks per head score and select; the head's first block also writes its
// entries of the compacted list.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rr_device.h"
#include "rr_internal.h"

namespace rr {

namespace {

constexpr int WR = 16;                 // query rows per block (the MFMA's row count)
constexpr int WWAVES = 8;              // waves per block
constexpr int WKT = 16;                // keys per lane in the selection: nk <= 1024
constexpr int WBM = 1024 / 32 + 1;     // bitmap words per row
constexpr int SST = 1024 + 4;          // u32 row stride of the score table (the pad spreads the
                                       // four 4-row groups of an MFMA result over the banks)

struct WideShared {
    uint32_t s[WR][SST];               // orderable scores of the block's rows; 0 = no key
    uint64_t list[WWAVES][2][64];      // candidate keys of a wave's two rows; then random draws (u32)
    uint32_t bm[WWAVES][WBM];          // chunks already in the row's ledger
    int32_t stage[WWAVES][129];        // the row's ledger entries (c <= 128) before the copy out
};

// The value of lane (lane ^ J), all in the VALU: quad permutes for J = 1, 2; a row shift each
// way for J = 4; a row rotation for J = 8; the 16- and 32-lane swaps for J = 16, 32 (the swap of
// a register with itself returns the own value in one result and the partner's in the other).
template <int J> __device__ __forceinline__ uint32_t xor_lane(uint32_t v, int lane) {
    if constexpr (J == 1) return (uint32_t)dpp_i<0xB1>((int)v);               // quad_perm [1,0,3,2]
    else if constexpr (J == 2) return (uint32_t)dpp_i<0x4E>((int)v);          // quad_perm [2,3,0,1]
    else if constexpr (J == 4) {
        const uint32_t up = (uint32_t)dpp_i<0x104>((int)v);                    // row_shl:4, lane i <- i + 4
        const uint32_t dn = (uint32_t)dpp_i<0x114>((int)v);                    // row_shr:4, lane i <- i - 4
        return (lane & 4) ? dn : up;
    } else if constexpr (J == 8) return (uint32_t)dpp_i<0x128>((int)v);       // row_ror:8
    else if constexpr (J == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (r[0] == v) ? r[1] : r[0];
    } else {
        static_assert(J == 32, "lane distance");
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (r[0] == v) ? r[1] : r[0];
    }
}
template <int J> __device__ __forceinline__ uint64_t xor_lane(uint64_t v, int lane) {
    const uint32_t lo = xor_lane<J>((uint32_t)v, lane);
    const uint32_t hi = xor_lane<J>((uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

// Bitonic sort across the 64 lanes, one value per lane, ascending or descending.
template <int K, int J, bool DESC, typename T> __device__ __forceinline__ T bitonic_merge(T v, int lane) {
    const T o = xor_lane<J>(v, lane);
    const bool low = ((lane & K) == 0) == ((lane & J) == 0);   // keeps the smaller one (ascending)
    v = (low != DESC) ? (v < o ? v : o) : (v < o ? o : v);
    if constexpr (J > 1) v = bitonic_merge<K, J / 2, DESC>(v, lane);
    return v;
}
template <int K, bool DESC, typename T> __device__ __forceinline__ T bitonic_sort(T v, int lane) {
    if constexpr (K > 2) v = bitonic_sort<K / 2, DESC>(v, lane);
    return bitonic_merge<K, K / 2, DESC>(v, lane);
}
// The same over NR independent values per lane (one per row), stage by stage, so that the
// rows' exchange chains interleave.
template <int K, int J, bool DESC, int NR, typename T>
__device__ __forceinline__ void bitonic_merge_n(T (&v)[NR], int lane) {
    T o[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) o[r] = xor_lane<J>(v[r], lane);
    const bool low = ((lane & K) == 0) == ((lane & J) == 0);
#pragma unroll
    for (int r = 0; r < NR; ++r) v[r] = (low != DESC) ? (v[r] < o[r] ? v[r] : o[r]) : (v[r] < o[r] ? o[r] : v[r]);
    if constexpr (J > 1) bitonic_merge_n<K, J / 2, DESC>(v, lane);
}
template <int K, bool DESC, int NR, typename T>
__device__ __forceinline__ void bitonic_sort_n(T (&v)[NR], int lane) {
    if constexpr (K > 2) bitonic_sort_n<K / 2, DESC>(v, lane);
    bitonic_merge_n<K, K / 2, DESC>(v, lane);
}
__device__ __forceinline__ uint32_t lane_sort_asc_u32(uint32_t v, int lane) { return bitonic_sort<64, false>(v, lane); }

__device__ __forceinline__ int lanes_below(uint64_t mask, int lane) {
    return __popcll(mask & ((1ull << lane) - 1ull));
}

__device__ __forceinline__ uint64_t wkey(uint32_t o, int j) {
    return ((uint64_t)o << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
}

// The ledger row of query row `row` of head h, given its route and near-miss: `used` / `idx`
// (lanes below ki + mi hold the chosen chunks, in any order) and `sorted` (lane e < ki: the e-th
// route chunk ascending; lane ki + e < ki + mi: the e-th near-miss chunk ascending).
__device__ __forceinline__ void write_row(const RouteArgs& p, WideShared& sh, int wave, int lane, int h, int row,
                                          int qrow, int n, int ki, int mi, bool used, uint32_t idx,
                                          uint32_t sorted) {
    const size_t flat = (size_t)h * p.nq + row;
    uint64_t* list = sh.list[wave][0];
    uint32_t* bm = sh.bm[wave];
    int32_t* stage = sh.stage[wave];
    const int words = (n + 31) >> 5;
    if (lane < WBM) bm[lane] = 0u;
    if (used && idx < (uint32_t)n) atomicOr(&bm[idx >> 5], 1u << (idx & 31));
    for (int e = lane; e < p.c; e += 64) stage[e] = -1;
    if (lane < ki) stage[lane] = (int32_t)(sorted & 0xFFFFu);
    else if (lane < ki + mi) stage[p.k + (lane - ki)] = (int32_t)(sorted & 0xFFFFu);

    // ---------------------------------------------------------------- mandatory sentinels
    const int mw = p.sink + p.recent;
    int mand = 0;
    if (mw > 0) {
        const int s_end = min(p.sink, n);
        const int r_beg = max(s_end, n - p.recent);
        int j = -1;
        if (lane < s_end) j = lane;
        else if (lane - s_end < n - r_beg) j = r_beg + (lane - s_end);
        const bool keep = j >= 0 && (bm[j >> 5] & (1u << (j & 31))) == 0u;
        const uint64_t m = __ballot(keep);
        if (keep) {
            stage[p.k + p.m + lanes_below(m, lane)] = j;
            atomicOr(&bm[j >> 5], 1u << (j & 31));
        }
        mand = __popcll(m);
    }

    // ---------------------------------------------------------------- random sentinels
    // Accepted chunks go to the row's list (its key list is free again) in draw order.
    const int pool = n - ki - mi - mand;
    const int rwant = min(p.r, pool);
    uint32_t* rlist = reinterpret_cast<uint32_t*>(list);
    int taken = 0;
    if (p.r > 0 && pool > p.r) {
        // A round covers draws t0 .. t0 + L - 1, L ending at the draw that would fill the row if
        // none of them repeated an earlier one, so only those draws are checked against each other.
        for (int t0 = 0; t0 < 65536 && taken < p.r;) {
            const int t = t0 + lane;
            const P4 w4 = philox4x32_10(P4{(uint32_t)(t >> 2), (uint32_t)qrow, (uint32_t)p.layer, (uint32_t)h},
                                        p.seed_lo, p.seed_hi);
            const uint32_t u = ((t & 3) == 0) ? w4.x : ((t & 3) == 1) ? w4.y : ((t & 3) == 2) ? w4.z : w4.w;
            const uint32_t j = __umulhi(u, (uint32_t)n);
            const bool inpool = t < 65536 && (bm[j >> 5] & (1u << (j & 31))) == 0u;
            const uint64_t m_in = __ballot(inpool);
            const int need = p.r - taken;
            // in-pool draws up to and including this lane (for lane 63, 2 << 63 wraps to 0: all bits)
            const int upto = __popcll(m_in & ((2ull << lane) - 1ull));
            const uint64_t at_need = __ballot(inpool && upto == need);
            const int L = at_need ? (int)__builtin_ctzll(at_need) + 1 : 64;
            bool dup = false;                             // an earlier draw of this round hit j
            for (int l2 = 0; l2 < L - 1; ++l2) {
                const uint32_t jj = (uint32_t)__builtin_amdgcn_readlane((int)j, l2);
                dup = dup || (l2 < lane && ((m_in >> l2) & 1ull) != 0ull && jj == j);
            }
            const bool acc = inpool && !dup && lane < L;
            const uint64_t m = __ballot(acc);
            const int rank = lanes_below(m, lane);
            if (acc && taken + rank < p.r) {
                atomicOr(&bm[j >> 5], 1u << (j & 31));
                rlist[taken + rank] = j;
            }
            taken = min(p.r, taken + __popcll(m));
            t0 += L;
        }
    }
    if (taken < rwant && lane == 0) {
        // Fill (pool not larger than r, or the draw cap reached): lowest-index free chunks.
        for (int w = 0; w < words && taken < rwant; ++w) {
            uint32_t f = ~bm[w];
            while (f && taken < rwant) {
                const int j = w * 32 + __builtin_ctz(f);
                f &= f - 1u;
                if (j >= n) break;
                rlist[taken++] = (uint32_t)j;
            }
        }
    }
    if (rwant > 0) {
        const uint32_t rv = lane < rwant ? rlist[lane] : 0xFFFFFFFFu;
        // up to 16 draws sit in lanes 0-15: a sort within each 16-lane row is enough
        const uint32_t rsorted = (rwant <= 16) ? bitonic_sort<16, false>(rv, lane) : lane_sort_asc_u32(rv, lane);
        if (lane < rwant) stage[p.k + p.m + mw + lane] = (int32_t)rsorted;
    }

    // ---------------------------------------------------------------- ledger row
    int32_t* dst = p.ids + flat * p.c;
    for (int e = lane; e < p.c; e += 64) dst[e] = stage[e];
    if (lane == 0) {
        p.anchor[flat] = p.layer;
        p.refreshed[flat] = (uint8_t)p.refresh_mark;
    }
}

// One 16-row group: score table, then the ledger rows.  Called by every wave of the block.
// Exact top-(k+m) of NR rows (block rows bi[r], query rows row[r]) from the score table, the
// rows side by side, then each row's ledger write.
template <bool CAUSAL, bool REROUTE, int NR>
__device__ __forceinline__ void emit_rows(const RouteArgs& p, WideShared& sh, int wave, int lane, int h,
                                          const int (&row)[NR], const int (&bi)[NR]) {
    // Opaque per call: otherwise the sorts' per-lane stage conditions are hoisted out of the
    // row loop as 64-bit masks and spill.
    asm volatile("" : "+v"(lane));
    int qrow[NR], n[NR], sel[NR];
    uint32_t o[NR][WKT];
    uint32_t lm[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        qrow[r] = p.qmap ? p.qmap[row[r]] : row[r];
        n[r] = CAUSAL ? qrow[r] + 1 : p.nk;
        sel[r] = min(p.sel, n[r]);
        lm[r] = 0u;
#pragma unroll
        for (int t = 0; t < WKT; ++t) {
            const int j = lane + 64 * t;
            o[r][t] = (j < n[r]) ? sh.s[bi[r]][j] : 0u;
            lm[r] = max(lm[r], o[r][t]);
        }
    }
    // The prefilter bound tau: at least sel keys must reach it.  In a reroute, the rescore
    // kernel's hint (the row's lowest current score over its old route and near-miss, -inf if a
    // slot was empty) serves when between sel and 64 keys reach it (it comes from other
    // arithmetic, so a key it names may score a rounding lower here).  Otherwise: lanes
    // 0 .. min(n, 64) - 1 hold at least one key and sel <= min(n, 64), so the sel-th largest
    // lane maximum is a key's score that at least sel keys reach.
    uint32_t tau[NR];
    bool need_sort = !REROUTE;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        tau[r] = 0u;
        if constexpr (REROUTE) {
            const float hv = p.hint[(size_t)h * p.nq + row[r]];
            const uint32_t th = (hv > -INFINITY) ? orderable(hv) : 0u;
            int ch = 0;
#pragma unroll
            for (int t = 0; t < WKT; ++t) ch += (o[r][t] >= th) ? 1 : 0;
            const int C = wave_sum_i(ch);
            if (th != 0u && C >= sel[r] && C <= 64) tau[r] = th;
            else need_sort = true;
        }
    }
    if (need_sort) {
        bitonic_sort_n<64, false>(lm, lane);
#pragma unroll
        for (int r = 0; r < NR; ++r)
            if (tau[r] == 0u) tau[r] = (uint32_t)__builtin_amdgcn_readlane((int)lm[r], 64 - sel[r]);
    }
    uint64_t cand[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const uint32_t tau_r = tau[r];
        int cnt = 0;
#pragma unroll
        for (int t = 0; t < WKT; ++t) cnt += (o[r][t] >= tau_r) ? 1 : 0;
        const int C = wave_sum_i(cnt);
        uint64_t* list = sh.list[wave][r];
        int held;                                         // keys in the list, the top sel among them
        if (tau_r != 0u && C <= 64) {
            int pos = wave_incl_scan_i(cnt) - cnt;
#pragma unroll
            for (int t = 0; t < WKT; ++t)
                if (o[r][t] >= tau_r) list[pos++] = wkey(o[r][t], lane + 64 * t);
            held = C;
        } else {
            // More than 64 keys reach tau: an exact radix select over the 64-bit keys finds the
            // sel-th largest, and exactly the sel keys at or above it are kept.
            uint64_t thr = 0ull;
            for (int b = 63; b >= 0; --b) {
                const uint64_t c64 = thr | (1ull << b);
                int c = 0;
#pragma unroll
                for (int t = 0; t < WKT; ++t) c += (o[r][t] != 0u && wkey(o[r][t], lane + 64 * t) >= c64) ? 1 : 0;
                if (wave_sum_i(c) >= sel[r]) thr = c64;
            }
            int mine = 0;
#pragma unroll
            for (int t = 0; t < WKT; ++t) mine += (o[r][t] != 0u && wkey(o[r][t], lane + 64 * t) >= thr) ? 1 : 0;
            int pos = wave_incl_scan_i(mine) - mine;
#pragma unroll
            for (int t = 0; t < WKT; ++t)
                if (o[r][t] != 0u && wkey(o[r][t], lane + 64 * t) >= thr && pos < 64)
                    list[pos++] = wkey(o[r][t], lane + 64 * t);
            held = sel[r];
        }
        cand[r] = lane < held ? list[lane] : 0ull;
    }
    bitonic_sort_n<64, true>(cand, lane);                 // lane e: rank e
    int ki[NR], mi[NR];
    bool used[NR];
    uint32_t idx[NR], skey[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        ki[r] = min(p.k, n[r]);
        mi[r] = min(p.m, n[r] - ki[r]);
        used[r] = lane < ki[r] + mi[r];
        idx[r] = 0xFFFFFFFFu - (uint32_t)cand[r];
        skey[r] = used[r] ? (((lane < ki[r]) ? 0u : 0x10000u) | idx[r]) : 0xFFFFFFFFu;
    }
    bitonic_sort_n<64, false>(skey, lane);                // route ascending, then near-miss ascending
#pragma unroll
    for (int r = 0; r < NR; ++r)
        write_row(p, sh, wave, lane, h, row[r], qrow[r], n[r], ki[r], mi[r], used[r], idx[r], skey[r]);
}

// One group of nrows (<= 16) ledger rows, ascending: brow is the row of block row lane % 16 (for
// lane % 16 < nrows).  Every wave of the block calls it.
template <typename E, bool CAUSAL, bool REROUTE>
__device__ __forceinline__ void route_group(const RouteArgs& p, WideShared& sh, int wave, int lane, int h, int brow,
                                            int nrows) {
    const uint64_t todo = __ballot(lane < nrows);         // the same in every wave
    if (todo == 0ull) return;                             // whole block: nothing to write

    // ---------------------------------------------------------------- score table
    // Keys up to the last written row's limit (query rows ascend with the block's rows).
    const int last = __builtin_amdgcn_readlane(brow, 63 - __builtin_clzll(todo));
    const int nmax = CAUSAL ? (p.qmap ? p.qmap[last] : last) + 1 : p.nk;
    const int ntile = (nmax + 15) >> 4;
    const int g = lane >> 4, c = lane & 15;
    // A operand: block row c (rows past the group read its first row; their scores are unused).
    const int arow = (c < nrows) ? brow : __builtin_amdgcn_readlane(brow, 0);
    const E* qv = reinterpret_cast<const E*>(p.qp) + ((size_t)h * p.nq_q + (p.qmap ? p.qmap[arow] : arow)) * 64;
    const E* Kh = reinterpret_cast<const E*>(p.kp) + (size_t)h * p.nk * 64;
    int nlim[4];                                          // key limit of result rows 4g .. 4g+3
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int bi = 4 * g + v;
        const int r = __shfl(brow, bi);
        nlim[v] = (bi < nrows) ? (CAUSAL ? (p.qmap ? p.qmap[r] : r) + 1 : p.nk) : 0;
    }
    auto put = [&](int tile, const f32x4& acc) {
        // result lane layout: key 16 tile + c, rows 4g + v
        const int key = 16 * tile + c;
#pragma unroll
        for (int v = 0; v < 4; ++v) sh.s[4 * g + v][key] = (key < nlim[v]) ? orderable(acc[v]) : 0u;
    };
    if constexpr (sizeof(E) == 2) {
        // k-step s of a tile contracts d = 32 s + 8 g .. 32 s + 8 g + 7 in lane group g.
        const bf16x8 qa0 = *reinterpret_cast<const bf16x8*>(qv + 8 * g);
        const bf16x8 qa1 = *reinterpret_cast<const bf16x8*>(qv + 32 + 8 * g);
        constexpr int TG = 1024 / 16 / WWAVES;            // tiles per wave at nk = 1024
        bf16x8 kb[TG][2];
#pragma unroll
        for (int u = 0; u < TG; ++u) {
            const int tile = wave + WWAVES * u;
            if (tile < ntile) {
                const E* kr = Kh + (size_t)min(16 * tile + c, p.nk - 1) * 64 + 8 * g;
                kb[u][0] = *reinterpret_cast<const bf16x8*>(kr);
                kb[u][1] = *reinterpret_cast<const bf16x8*>(kr + 32);
            }
        }
#pragma unroll
        for (int u = 0; u < TG; ++u) {
            const int tile = wave + WWAVES * u;
            if (tile < ntile) {
                f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa0, kb[u][0], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa1, kb[u][1], acc, 0, 0, 0);
                put(tile, acc);
            }
        }
    } else {
        // k-step s contracts d = 16 g + s in lane group g (s = 0 .. 15).
        float qa[16];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(qv + 16 * g + 4 * u);
#pragma unroll
            for (int e = 0; e < 4; ++e) qa[4 * u + e] = __uint_as_float(w[e]);
        }
        for (int t0 = wave; t0 < ntile; t0 += 4 * WWAVES) {
            float kb[4][16];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int tile = t0 + WWAVES * u;
                if (tile < ntile) {
                    const E* kr = Kh + (size_t)min(16 * tile + c, p.nk - 1) * 64 + 16 * g;
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const u32x4 w = *reinterpret_cast<const u32x4*>(kr + 4 * q4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) kb[u][4 * q4 + e] = __uint_as_float(w[e]);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int tile = t0 + WWAVES * u;
                if (tile < ntile) {
                    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < 16; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[s], kb[u][s], acc, 0, 0, 0);
                    put(tile, acc);
                }
            }
        }
    }
    __syncthreads();

    // ---------------------------------------------------------------- ledger rows
    // The block's written rows in order, dealt round-robin to the waves: at most 16 rows, so a
    // wave takes the wave-th and, if present, the (wave + 8)-th.
    uint64_t rest = todo;
    for (int x = 0; x < wave && rest != 0ull; ++x) rest &= rest - 1ull;
    if (rest == 0ull) return;
    const int b0 = __builtin_ctzll(rest);
    for (int x = 0; x < WWAVES && rest != 0ull; ++x) rest &= rest - 1ull;
    if (rest != 0ull) {
        const int b1 = __builtin_ctzll(rest);
        const int rows[2] = {__builtin_amdgcn_readlane(brow, b0), __builtin_amdgcn_readlane(brow, b1)};
        const int bis[2] = {b0, b1};
        emit_rows<CAUSAL, REROUTE, 2>(p, sh, wave, lane, h, rows, bis);
    } else {
        const int rows[1] = {__builtin_amdgcn_readlane(brow, b0)}, bis[1] = {b0};
        emit_rows<CAUSAL, REROUTE, 1>(p, sh, wave, lane, h, rows, bis);
    }
}

// Reroute: the head's flagged rows, ascending, are ranks 0 .. count_h - 1 of the rescore
// kernel's per-64-row counts and ascending lists (bcount [H, G], blist [H, G, 64]).  Returns
// the row of rank `want` (-1 at or past the count) and the head's count in *count_h.
__device__ __forceinline__ int flagged_row(const RouteArgs& p, int h, int want, int lane, int* count_h) {
    const int G = (p.nq + ROUTE_ROWS - 1) / ROUTE_ROWS;
    const int32_t* bc = p.bcount + (size_t)h * G;
    const int32_t* bl = p.blist + (size_t)h * G * ROUTE_ROWS;
    int base = 0, row = -1;
    for (int c0 = 0; c0 < G; c0 += 64) {                  // uniform
        const int cnt = (c0 + lane < G) ? bc[c0 + lane] : 0;
        const int incl = wave_incl_scan_i(cnt);
        const int nb = min(64, G - c0);
        for (int bb = 0; bb < nb; ++bb) {
            const int hi = base + __builtin_amdgcn_readlane(incl, bb);
            const int lo = hi - __builtin_amdgcn_readlane(cnt, bb);
            if (want >= lo && want < hi) row = bl[(size_t)(c0 + bb) * ROUTE_ROWS + (want - lo)];
        }
        base += __builtin_amdgcn_readlane(incl, 63);
    }
    *count_h = base;
    return row;
}

// Reroute outputs of head h (one wave): its compacted rows (ascending h * nq + i), its count and,
// for the last head, the layer's total.
__device__ __forceinline__ void head_outputs(const RouteArgs& p, int h, int lane, int count_h) {
    const int G = (p.nq + ROUTE_ROWS - 1) / ROUTE_ROWS;
    int acc = 0;
    for (int x = lane; x < h * G; x += 64) acc += p.bcount[x];
    const int offset = wave_sum_i(acc);                   // flagged rows of the heads before h
    if (lane == 0) {
        if (p.out_head_counts) p.out_head_counts[h] = count_h;
        if (p.out_n_rows && h == p.H - 1) p.out_n_rows[0] = offset + count_h;
    }
    if (p.out_rows) {
        int run = 0;
        for (int bb = 0; bb < G; ++bb) {                  // uniform
            const int cb = p.bcount[(size_t)h * G + bb];
            if (lane < cb) p.out_rows[offset + run + lane] = h * p.nq + p.blist[((size_t)h * G + bb) * ROUTE_ROWS + lane];
            run += cb;
        }
    }
}

// E: uint16_t (bf16 bits) or float.
template <typename E, bool CAUSAL, bool REROUTE>
__global__ __launch_bounds__(64 * WWAVES) __attribute__((amdgpu_waves_per_eu(4))) void k_route_wide(RouteArgs p) {
    __shared__ WideShared sh;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int per_head = (p.nq + WR - 1) / WR;
    // Workgroups go to the 8 XCDs round-robin; renumber so that each XCD runs a contiguous
    // range of blocks, i.e. whole heads, whose key rows then stay in that XCD's L2.
    const int per_xcd = (int)gridDim.x / 8;
    const int lb = ((int)blockIdx.x % 8) * per_xcd + (int)blockIdx.x / 8;
    if (lb >= p.H * per_head) return;                     // grid padding (whole block)
    const int h = lb / per_head, b = lb % per_head;
    if constexpr (REROUTE) {
        // Block b takes ranks 16 b .. 16 b + 15 of the head's flagged rows (compacted, so that
        // only ceil(flagged / 16) blocks per head score and select); the rest exit.
        int count_h;
        const int brow = flagged_row(p, h, WR * b + (lane & 15), lane, &count_h);
        if (b == 0 && wave == 0 && (p.out_rows || p.out_head_counts || p.out_n_rows)) head_outputs(p, h, lane, count_h);
        if (WR * b >= count_h) return;                    // uniform
        route_group<E, CAUSAL, REROUTE>(p, sh, wave, lane, h, brow, min(WR, count_h - WR * b));
    } else {
        const int r0 = b * WR;
        route_group<E, CAUSAL, REROUTE>(p, sh, wave, lane, h, r0 + (lane & 15), min(WR, p.nq - r0));
    }
}

template <typename E, bool CAUSAL, bool REROUTE>
hipError_t launch_wide_t(const RouteArgs& a, hipStream_t st) {
    const int per_head = (a.nq + WR - 1) / WR;
    const unsigned blocks = (unsigned)((a.H * per_head + 7) / 8 * 8);      // a multiple of the 8 XCDs
    hipLaunchKernelGGL((k_route_wide<E, CAUSAL, REROUTE>), dim3(blocks), dim3(64 * WWAVES), 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route_wide(const RouteArgs& a, bool bf16, bool causal, bool reroute, hipStream_t st) {
    if (bf16) {
        if (causal) return reroute ? launch_wide_t<uint16_t, true, true>(a, st) : launch_wide_t<uint16_t, true, false>(a, st);
        return reroute ? launch_wide_t<uint16_t, false, true>(a, st) : launch_wide_t<uint16_t, false, false>(a, st);
    }
    if (causal) return reroute ? launch_wide_t<float, true, true>(a, st) : launch_wide_t<float, true, false>(a, st);
    return reroute ? launch_wide_t<float, false, true>(a, st) : launch_wide_t<float, false, false>(a, st);
}

}  // namespace rr
