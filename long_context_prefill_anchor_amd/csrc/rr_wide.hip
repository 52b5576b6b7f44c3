// Routing with near-miss sets wider than the main route kernel's 32-entry lists
// (32 < k + m <= 64): one wave per query row.
//
// "RouteRelay: Event-Triggered Cross-Layer Route Reuse for Efficient Dynamic Sparse
// Attention", Section 2.1 Eq. 1-2 (scores, top-k route), Section 3.1 items 1-3 (near-miss,
// random and mandatory sentinels, Eq. 4 ledger), Sections 4.1-4.2 (reroute of flagged rows);
// Table 3 evaluates 24- and 48-wide near-miss sets.
//
// Per row, in one wave: each lane scores the keys lane, lane + 64, ... (fp32 dot products of
// the row's query, held in LDS, with the key rows); an exact radix select over the 64-bit keys
// (orderable score, then lower index first) finds the (k+m)-th largest; the keys at or above
// it are compacted and sorted across lanes with a bitonic network, so lane r holds rank r.
// Route = ranks below k, near-miss = the next m.  The ledger row is then written with the same
// rules as the main kernel: segments ascending by index, mandatory sink / recent chunks not
// already routed, random draws from Philox4x32-10 (counter = (t div 4, query row, layer,
// head)) accepted in draw order when the chunk is still in the pool, a fill with the
// lowest-index free chunks when the pool is not larger than r or the draw cap is reached.
// The kernel keeps no threshold state, so anchor and reroute use it alike; a reroute wave
// returns at once for a row the rescore kernel did not flag.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rr_device.h"
#include "rr_internal.h"

namespace rr {

namespace {

constexpr int WW = 4;                  // waves (rows) per block
constexpr int WKT = 16;                // keys per lane: nk <= 1024
constexpr int WBM = 1024 / 32 + 1;     // bitmap words per row

// Element e of a 16-byte load: eight bf16 (raw bits) or four fp32 values.
__device__ __forceinline__ float elem_of(const u32x4& w, int e, const uint16_t*) {
    const uint32_t word = w[e >> 1];
    return __uint_as_float((e & 1) ? (word & 0xFFFF0000u) : (word << 16));
}
__device__ __forceinline__ float elem_of(const u32x4& w, int e, const float*) { return __uint_as_float(w[e]); }

struct WideShared {
    uint64_t list[WW][64];
    uint32_t bm[WW][WBM];
    int32_t stage[WW][65];
};

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
    const int lo = __shfl_xor((int)(uint32_t)v, m);
    const int hi = __shfl_xor((int)(uint32_t)(v >> 32), m);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Bitonic sort across the 64 lanes, one value per lane: descending (u64) or ascending (u32).
__device__ __forceinline__ uint64_t lane_sort_desc_u64(uint64_t v, int lane) {
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const uint64_t o = shfl_xor_u64(v, j);
            const bool keep_max = (((lane & k) == 0) == ((lane & j) == 0));
            v = keep_max ? (v > o ? v : o) : (v > o ? o : v);
        }
    }
    return v;
}

__device__ __forceinline__ uint32_t lane_sort_asc_u32(uint32_t v, int lane) {
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const uint32_t o = (uint32_t)__shfl_xor((int)v, j);
            const bool keep_min = (((lane & k) == 0) == ((lane & j) == 0));
            v = keep_min ? min(v, o) : max(v, o);
        }
    }
    return v;
}

__device__ __forceinline__ int lanes_below(uint64_t mask, int lane) {
    return __popcll(mask & ((1ull << lane) - 1ull));
}

// E: uint16_t (bf16 bits) or float.
template <typename E, bool CAUSAL, bool REROUTE>
__global__ __launch_bounds__(64 * WW) void k_route_wide(RouteArgs p) {
    __shared__ WideShared sh;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int per_head = (p.nq + WW - 1) / WW;
    // Workgroups go to the 8 XCDs round-robin; renumber so that each XCD runs a contiguous
    // range of blocks, i.e. whole heads, whose key rows then stay in that XCD's L2.
    const int per_xcd = (int)gridDim.x / 8;
    const int lb = ((int)blockIdx.x % 8) * per_xcd + (int)blockIdx.x / 8;
    if (lb >= p.H * per_head) return;                     // grid padding
    const int h = lb / per_head;
    const int row = (lb % per_head) * WW + wave;
    if (row >= p.nq) return;                              // whole wave; no block barriers below
    const size_t flat = (size_t)h * p.nq + row;
    if constexpr (REROUTE) {
        if (p.flags[flat] == 0) return;
    }
    const int qrow = p.qmap ? p.qmap[row] : row;
    const int n = CAUSAL ? qrow + 1 : p.nk;

    // ---------------------------------------------------------------- scores and keys
    // The query row in registers; each key row read with 16-byte loads.
    const E* qv = reinterpret_cast<const E*>(p.qp) + ((size_t)h * p.nq_q + qrow) * 64;
    constexpr int PER = 16 / sizeof(E);                   // elements per 16-byte load
    float qf[64];
#pragma unroll
    for (int c = 0; c < 64 / PER; ++c) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(qv + PER * c);
#pragma unroll
        for (int e = 0; e < PER; ++e) qf[PER * c + e] = elem_of(w, e, (const E*)nullptr);
    }
    const E* Kh = reinterpret_cast<const E*>(p.kp) + (size_t)h * p.nk * 64;
    uint64_t key[WKT];
#pragma unroll
    for (int t = 0; t < WKT; ++t) {
        const int j = lane + 64 * t;
        key[t] = EMPTY_KEY;
        if (j < n) {
            const E* kr = Kh + (size_t)j * 64;
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < 64 / PER; ++c) {
                const u32x4 w = *reinterpret_cast<const u32x4*>(kr + PER * c);
#pragma unroll
                for (int e = 0; e < PER; ++e) acc = fmaf(qf[PER * c + e], elem_of(w, e, (const E*)nullptr), acc);
            }
            key[t] = make_key(acc, (uint32_t)j);
        }
    }

    // ---------------------------------------------------------------- exact top-(k+m)
    const int sel = min(p.sel, n);
    uint64_t thr = 0ull;                                  // the sel-th largest key
    for (int b = 63; b >= 0; --b) {
        const uint64_t cand = thr | (1ull << b);
        int c = 0;
#pragma unroll
        for (int t = 0; t < WKT; ++t) c += (key[t] >= cand) ? 1 : 0;
        if (wave_sum_i(c) >= sel) thr = cand;
    }
    int mine = 0;
#pragma unroll
    for (int t = 0; t < WKT; ++t) mine += (key[t] >= thr && key[t] != EMPTY_KEY) ? 1 : 0;
    int pos = wave_incl_scan_i(mine) - mine;
#pragma unroll
    for (int t = 0; t < WKT; ++t)
        if (key[t] >= thr && key[t] != EMPTY_KEY && pos < 64) sh.list[wave][pos++] = key[t];
    const uint64_t ranked = lane_sort_desc_u64(lane < sel ? sh.list[wave][lane] : EMPTY_KEY, lane);

    // ---------------------------------------------------------------- route and near-miss
    const int ki = min(p.k, n);
    const int mi = min(p.m, n - ki);
    const bool used = lane < ki + mi;
    const uint32_t idx = key_index(ranked);
    const uint32_t skey = used ? (((lane < ki) ? 0u : 0x10000u) | idx) : 0xFFFFFFFFu;
    const uint32_t sorted = lane_sort_asc_u32(skey, lane);   // route ascending, then near-miss ascending
    uint32_t* bm = sh.bm[wave];
    int32_t* stage = sh.stage[wave];
    const int words = (n + 31) >> 5;
    if (lane < WBM) bm[lane] = 0u;
    if (used) atomicOr(&bm[idx >> 5], 1u << (idx & 31));
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
    uint32_t* rlist = reinterpret_cast<uint32_t*>(sh.list[wave]);
    int taken = 0;
    if (p.r > 0 && pool > p.r) {
        for (int t0 = 0; t0 < 65536 && taken < p.r; t0 += 64) {
            const int t = t0 + lane;
            const P4 w4 = philox4x32_10(P4{(uint32_t)(t >> 2), (uint32_t)qrow, (uint32_t)p.layer, (uint32_t)h},
                                        p.seed_lo, p.seed_hi);
            const uint32_t u = ((t & 3) == 0) ? w4.x : ((t & 3) == 1) ? w4.y : ((t & 3) == 2) ? w4.z : w4.w;
            const uint32_t j = __umulhi(u, (uint32_t)n);
            const bool inpool = (bm[j >> 5] & (1u << (j & 31))) == 0u;
            bool dup = false;                             // an earlier draw of this round hit j
            for (int l2 = 0; l2 < 63; ++l2) {
                const uint32_t jj = (uint32_t)__builtin_amdgcn_readlane((int)j, l2);
                const int ok2 = __builtin_amdgcn_readlane((int)inpool, l2);
                dup = dup || (l2 < lane && ok2 != 0 && jj == j);
            }
            const bool acc = inpool && !dup;
            const uint64_t m = __ballot(acc);
            const int rank = lanes_below(m, lane);
            if (acc && taken + rank < p.r) {
                atomicOr(&bm[j >> 5], 1u << (j & 31));
                rlist[taken + rank] = j;
            }
            taken = min(p.r, taken + __popcll(m));
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
    const uint32_t rsorted = lane_sort_asc_u32(lane < rwant ? rlist[lane] : 0xFFFFFFFFu, lane);
    if (lane < rwant) stage[p.k + p.m + mw + lane] = (int32_t)rsorted;

    // ---------------------------------------------------------------- ledger row
    int32_t* dst = p.ids + flat * p.c;
    for (int e = lane; e < p.c; e += 64) dst[e] = stage[e];
    if (lane == 0) {
        p.anchor[flat] = p.layer;
        p.refreshed[flat] = (uint8_t)p.refresh_mark;
    }
}

// Compacted list of flagged rows (ascending h*nq + i), per-head counts and total, for the
// wide reroute (the main reroute kernel writes these from its prologue).  One wave per head.
__global__ __launch_bounds__(64) void k_wide_outputs(RouteArgs p) {
    const int h = blockIdx.x;
    const int lane = threadIdx.x;
    const int G = (p.nq + 63) / 64;
    int acc = 0;
    for (int x = lane; x < h * G; x += 64) acc += p.bcount[x];
    const int offset = wave_sum_i(acc);
    int cnt = 0;
    for (int x = lane; x < G; x += 64) cnt += p.bcount[(size_t)h * G + x];
    const int count_h = wave_sum_i(cnt);
    if (lane == 0) {
        if (p.out_head_counts) p.out_head_counts[h] = count_h;
        if (p.out_n_rows && h == p.H - 1) p.out_n_rows[0] = offset + count_h;
    }
    if (p.out_rows) {
        int run = 0;
        for (int b = 0; b < G; ++b) {
            const int i = b * 64 + lane;
            const bool f = i < p.nq && p.flags[(size_t)h * p.nq + i];
            const uint64_t m = __ballot(f);
            if (f) p.out_rows[offset + run + lanes_below(m, lane)] = h * p.nq + i;
            run += __popcll(m);
        }
    }
}

template <typename E, bool CAUSAL, bool REROUTE>
hipError_t launch_wide_t(const RouteArgs& a, hipStream_t st) {
    const int per_head = (a.nq + WW - 1) / WW;
    const unsigned blocks = (unsigned)((a.H * per_head + 7) / 8 * 8);      // a multiple of the 8 XCDs
    hipLaunchKernelGGL((k_route_wide<E, CAUSAL, REROUTE>), dim3(blocks), dim3(64 * WW), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && REROUTE && (a.out_rows || a.out_head_counts || a.out_n_rows)) {
        hipLaunchKernelGGL(k_wide_outputs, dim3((unsigned)a.H), dim3(64), 0, st, a);
        e = hipGetLastError();
    }
    return e;
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
