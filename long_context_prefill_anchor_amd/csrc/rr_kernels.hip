// RouteRelay routing kernels for gfx950 (MI355X).
//
// Source: "RouteRelay: Event-Triggered Cross-Layer Route Reuse for Efficient Dynamic Sparse
// Attention" (arXiv 2609.07306), Sections 2.1, 3.1-3.2, 4.1-4.2.
//
// k_route    — full routing of 64 query rows of one head: S = Q K^T (Eq. 1) on MFMA, exact
//              top-(k+m) selection (Eq. 2 + near-miss sentinels, Section 3.1), random
//              sentinels, ledger write.  Anchor mode routes rows 64g..64g+63; reroute mode
//              routes the g-th slice of 64 flagged rows of the head (the compacted list of
//              Sections 4.1/4.2), recovered from the rescore kernel's flags.
// k_rescore  — relay candidate rescoring (Eq. 5-8): per row, gather the ledger's candidate key
//              rows, dot them with the query row, alpha / beta / refresh flag, plus a lower
//              bound on the row's (k+m)-th best score that the reroute uses as its first
//              selection threshold.  Writes per-block flag counts for the compaction.
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
// are merged pairwise through LDS.  A key below the threshold cannot be among the best k+m, so
// the result is exact.  The first threshold is a proven lower bound on the (k+m)-th best score:
// anchor mode — the (k+m)-th largest of 32 maxima of disjoint 8-key groups taken from a first
// MFMA pass (each wave contributes its 8 largest group maxima); reroute mode — the smallest
// current score of the row's k+m ledger route and near-miss chunks, minus a rounding margin
// (a row that ends with fewer than k+m keys is recomputed from -inf).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rr_device.h"
#include "rr_internal.h"

namespace rr {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int ROWS = 64;           // rows per route block (one per lane)
constexpr int SPLIT = 4;           // waves per block, each scoring a quarter of the key tiles
constexpr int TK = 32;             // keys per tile
constexpr int TOPW = 32;           // register top list width (k + m <= TOPW)
constexpr int CAP = 31;            // per-wave per-row buffer: <= 15 held + 16 slots appended
constexpr int CSTRIDE = CAP;       // row stride in entries (odd: spreads rows over LDS banks)
constexpr int GSTRIDE = 33;        // f32 row stride of the pass-1 group maxima table
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
    __device__ __forceinline__ void load_k(KReg& dst, const uint16_t* K, int key0, int nk, int lane) const {
        const int key = key0 + (lane & 31);
        const int sub = lane >> 5;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (key < nk) {
                dst[s] = *reinterpret_cast<const bf16x8*>(K + (size_t)key * 64 + 16 * s + 8 * sub);
            } else {
                u32x4 z = {0u, 0u, 0u, 0u};
                dst[s] = __builtin_bit_cast(bf16x8, z);
            }
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
    __device__ __forceinline__ void load_k(KReg& dst, const float* K, int key0, int nk, int lane) const {
        const int key = key0 + (lane & 31);
        const int sub = lane >> 5;
        if (key < nk) {
            const float4* src = reinterpret_cast<const float4*>(K + (size_t)key * 64 + 32 * sub);
#pragma unroll
            for (int v = 0; v < 8; ++v) {
                const float4 x = src[v];
                dst[4 * v] = x.x; dst[4 * v + 1] = x.y; dst[4 * v + 2] = x.z; dst[4 * v + 3] = x.w;
            }
        } else {
#pragma unroll
            for (int s = 0; s < 32; ++s) dst[s] = 0.f;
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

template <typename KR>
__device__ __forceinline__ void copy_k(KR& dst, const KR& src) {
#pragma unroll
    for (int s = 0; s < (int)(sizeof(KR) / sizeof(src[0])); ++s) dst[s] = src[s];
}

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
__device__ __forceinline__ void drain(uint64_t (&top)[TOPW], const uint2* buf, int cnt) {
    int maxc = cnt;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) maxc = max(maxc, __shfl_xor(maxc, o, 64));
    for (int c0 = 0; c0 < maxc; c0 += 16) {
        uint64_t x[16];
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            if (c0 + s < cnt) {
                const uint2 e = buf[c0 + s];
                x[s] = make_key(__uint_as_float(e.x), e.y);
            } else {
                x[s] = EMPTY_KEY;
            }
        }
        sort_desc<16>(x);
        merge16_into_top(top, x);
    }
}

struct RouteShared {
    uint64_t thr[ROWS];      // shared threshold key per row (max over the waves' lower bounds)
    int32_t rows[ROWS];
    int32_t redo;
};

// ------------------------------------------------------------------------------ route kernel

template <typename DT, bool CAUSAL, bool REROUTE>
__global__ __launch_bounds__(ROWS * SPLIT) void k_route(RouteArgs p) {
    typedef typename Elem<DT>::type E;
    extern __shared__ __align__(16) unsigned char dyn_lds[];
    __shared__ RouteShared sh;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int G = (p.nq + ROWS - 1) / ROWS;
    const int h = blockIdx.x / G;
    const int g = blockIdx.x % G;

    // ------------------------------------------------------------------ rows of this block
    if constexpr (REROUTE) {
        const int32_t* bc = p.bcount + (size_t)h * G;
        int total = 0;
        for (int b0 = 0; b0 < G; b0 += 64) total += wave_sum_in((b0 + lane < G) ? bc[b0 + lane] : 0, 64);
        const int count_h = total;
        if (g == 0 && wave == 0) {
            // Compacted list output (ascending h*nq + i), per-head count and total.
            if (p.out_head_counts && lane == 0) p.out_head_counts[h] = count_h;
            int offset = 0;
            if (p.out_rows || p.out_n_rows) {
                int acc = 0;
                for (int x = lane; x < h * G; x += 64) acc += p.bcount[x];
                offset = wave_sum_in(acc, 64);
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
    } else {
        if (wave == 0) {
            const int i = g * ROWS + lane;
            sh.rows[lane] = (i < p.nq) ? i : -1;
        }
    }
    if (threadIdx.x == 0) sh.redo = 0;
    __syncthreads();

    // ------------------------------------------------------------------ per-row setup
    const int my_row = sh.rows[lane];
    const int my_n = (my_row < 0) ? 0 : (CAUSAL ? my_row + 1 : p.nk);
    int kmax = my_n, nmin = (my_row < 0) ? (1 << 30) : my_n;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        kmax = max(kmax, __shfl_xor(kmax, o, 64));
        nmin = min(nmin, __shfl_xor(nmin, o, 64));
    }
    const int ntiles = (kmax + TK - 1) / TK;
    const E* Qh = reinterpret_cast<const E*>(p.qp) + (size_t)h * p.nq * 64;
    const E* Kh = reinterpret_cast<const E*>(p.kp) + (size_t)h * p.nk * 64;
    Tile<DT> tile;
    tile.load_q(Qh, sh.rows[lane & 31], sh.rows[32 + (lane & 31)], lane);

    uint2* my_buf = reinterpret_cast<uint2*>(dyn_lds) + ((size_t)wave * ROWS + lane) * CSTRIDE;

    // ------------------------------------------------------------------ first threshold
    uint64_t base_thr;
    if constexpr (REROUTE) {
        const float hv = (my_row >= 0) ? p.hint[(size_t)h * p.nq + my_row] : -INFINITY;
        const float t = (hv == -INFINITY) ? -INFINITY : hv - (fabsf(hv) * 1e-4f + 1e-6f);
        base_thr = make_key(t, 0xFFFFFFFFu);
    } else {
        // Pass 1: per row and wave, the 8 largest maxima of disjoint 8-key groups.
        float top8[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) top8[s] = -INFINITY;
        typename Tile<DT>::KReg ka, kb;
        if (wave < ntiles) tile.load_k(kb, Kh, TK * wave, p.nk, lane);
        for (int t = wave; t < ntiles; t += SPLIT) {
            copy_k(ka, kb);
            if (t + SPLIT < ntiles) tile.load_k(kb, Kh, TK * (t + SPLIT), p.nk, lane);
            f32x16 lo, hi;
            tile.mma(ka, lo, hi);
            rows_per_lane(lo, hi);
            const int key0 = TK * t;
            if (key0 + TK > nmin) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    if (key0 + lo_key(v) >= my_n) lo[v] = -INFINITY;
                    if (key0 + hi_key(v) >= my_n) hi[v] = -INFINITY;
                }
            }
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                float x = fmaxf(fmaxf(fmaxf(lo[4 * a], lo[4 * a + 1]), fmaxf(lo[4 * a + 2], lo[4 * a + 3])),
                                fmaxf(fmaxf(hi[4 * a], hi[4 * a + 1]), fmaxf(hi[4 * a + 2], hi[4 * a + 3])));
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const float up = fmaxf(top8[s], x);
                    x = fminf(top8[s], x);
                    top8[s] = up;
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
    if (wave == 0) sh.thr[lane] = (my_row < 0) ? NO_PASS_KEY : base_thr;
    __syncthreads();

    // ------------------------------------------------------------------ streaming pass
    uint64_t top[TOPW];
#pragma unroll
    for (int s = 0; s < TOPW; ++s) top[s] = EMPTY_KEY;

    for (int attempt = 0; attempt < 2; ++attempt) {
        int cnt = 0;
        float ts = key_score(sh.thr[lane]);
        typename Tile<DT>::KReg ka, kb;
        if (wave < ntiles) tile.load_k(kb, Kh, TK * wave, p.nk, lane);
        for (int t = wave; t < ntiles; t += SPLIT) {
            copy_k(ka, kb);
            if (t + SPLIT < ntiles) tile.load_k(kb, Kh, TK * (t + SPLIT), p.nk, lane);
            f32x16 lo, hi;
            tile.mma(ka, lo, hi);
            rows_per_lane(lo, hi);
            const int key0 = TK * t;
            const bool edge = key0 + TK > nmin;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
#pragma unroll
                for (int v = 8 * half; v < 8 * half + 8; ++v) {
                    const uint32_t jl = (uint32_t)(key0 + lo_key(v));
                    const uint32_t jh = (uint32_t)(key0 + hi_key(v));
                    const bool pl = lo[v] >= ts && (!edge || (int)jl < my_n);
                    const bool ph = hi[v] >= ts && (!edge || (int)jh < my_n);
                    if (pl) my_buf[cnt] = make_uint2(__float_as_uint(lo[v]), jl);
                    cnt += pl;
                    if (ph) my_buf[cnt] = make_uint2(__float_as_uint(hi[v]), jh);
                    cnt += ph;
                }
                if (__ballot(cnt >= 16)) {
                    drain(top, my_buf, cnt);
                    cnt = 0;
                    const uint64_t own = pick(top, p.sel - 1);
                    if (own != EMPTY_KEY && my_row >= 0) atomicMax((unsigned long long*)&sh.thr[lane], own);
                }
            }
            ts = key_score(sh.thr[lane]);
        }
        drain(top, my_buf, cnt);

        // Merge the four waves' lists through two LDS slots: 1 -> 0 and 3 -> 2, then 2 -> 0.
        uint64_t* xchg = reinterpret_cast<uint64_t*>(dyn_lds);          // [2][ROWS][TOPW]
        __syncthreads();                                                // every buffer is drained
        if (wave & 1) {
#pragma unroll
            for (int s = 0; s < TOPW; ++s) xchg[((size_t)(wave >> 1) * ROWS + lane) * TOPW + s] = top[s];
        }
        __syncthreads();
        if (!(wave & 1)) {
            uint64_t y[TOPW];
#pragma unroll
            for (int s = 0; s < TOPW; ++s) y[s] = xchg[((size_t)(wave >> 1) * ROWS + lane) * TOPW + s];
            merge_top_desc<TOPW>(top, y);
        }
        __syncthreads();
        if (wave == 2) {
#pragma unroll
            for (int s = 0; s < TOPW; ++s) xchg[(size_t)lane * TOPW + s] = top[s];
        }
        __syncthreads();
        if (wave == 0) {
            uint64_t y[TOPW];
#pragma unroll
            for (int s = 0; s < TOPW; ++s) y[s] = xchg[(size_t)lane * TOPW + s];
            merge_top_desc<TOPW>(top, y);
            // Each row must now hold min(sel, n) keys.  Only a reroute threshold taken from the
            // rescore kernel's arithmetic can miss (rounding); such rows are redone from -inf.
            int have = 0;
#pragma unroll
            for (int s = 0; s < TOPW; ++s) have += (top[s] != EMPTY_KEY);
            const bool redo = (my_row >= 0) && have < min(p.sel, my_n);
            if (__ballot(redo) && attempt == 0) {
                sh.thr[lane] = redo ? make_key(-INFINITY, 0xFFFFFFFFu) : NO_PASS_KEY;
                if (lane == 0) sh.redo = 1;
                if (redo) {
#pragma unroll
                    for (int s = 0; s < TOPW; ++s) top[s] = EMPTY_KEY;
                }
            }
        }
        __syncthreads();
        if (!sh.redo) break;                                            // uniform over the block
        if (wave != 0) {
#pragma unroll
            for (int s = 0; s < TOPW; ++s) top[s] = EMPTY_KEY;
        }
        __syncthreads();                                                // everyone has read sh.redo
        if (threadIdx.x == 0) sh.redo = 0;
    }
    if (wave != 0) return;                                              // no barriers below

    // ------------------------------------------------------------------ ledger update (wave 0)
    // Route = entries [0, ki), near-miss = [ki, ki+mi) of the sorted list; both emitted
    // ascending by chunk index via one ascending sort of (segment << 16 | index).
    const int ki = min(p.k, my_n);
    const int mi = min(p.m, my_n - ki);
    uint32_t cmb[TOPW];
#pragma unroll
    for (int s = 0; s < TOPW; ++s) {
        const uint32_t j = key_index(top[s]);
        cmb[s] = (s < ki) ? j : ((s < ki + mi) ? (0x10000u | j) : 0xFFFFFFFFu);
    }
    sort_asc<TOPW>(cmb);

    // Sampler bitmap over allowed chunks: route + near-miss + accepted draws are set.
    const int words = (p.nk + 31) >> 5;
    uint32_t* bm = reinterpret_cast<uint32_t*>(dyn_lds) + (size_t)lane * (words + 1);
    for (int w = 0; w < words; ++w) bm[w] = 0u;
#pragma unroll
    for (int s = 0; s < TOPW; ++s) {
        if (s < ki + mi) {
            const uint32_t j = cmb[s] & 0xFFFFu;
            bm[j >> 5] |= 1u << (j & 31);
        }
    }
    uint32_t rnd[TOPW];
#pragma unroll
    for (int s = 0; s < TOPW; ++s) rnd[s] = 0xFFFFFFFFu;
    int nr = 0;
    const int pool = my_n - ki - mi;
    const int rwant = (my_row < 0) ? 0 : min(p.r, pool);
    if (p.r > 0) {
        // Draws only for rows whose pool exceeds r; smaller pools are taken whole by the fill.
        bool drawing = (my_row >= 0) && pool > p.r;
        P4 w4 = {0u, 0u, 0u, 0u};
        for (int t = 0; t < 65536 && __ballot(drawing); ++t) {
            if ((t & 3) == 0) {
                P4 c = {(uint32_t)(t >> 2), (uint32_t)my_row, (uint32_t)p.layer, (uint32_t)h};
                w4 = philox4x32_10(c, p.seed_lo, p.seed_hi);
            }
            const uint32_t u = ((t & 3) == 0) ? w4.x : ((t & 3) == 1) ? w4.y : ((t & 3) == 2) ? w4.z : w4.w;
            if (drawing) {
                const uint32_t j = __umulhi(u, (uint32_t)my_n);
                const uint32_t bit = 1u << (j & 31);
                if (!(bm[j >> 5] & bit)) {
                    bm[j >> 5] |= bit;
#pragma unroll
                    for (int s = 0; s < TOPW; ++s) rnd[s] = (s == nr) ? j : rnd[s];
                    ++nr;
                    drawing = nr < p.r;
                }
            }
        }
        // Fill: lowest-index chunks still free (whole pool when pool <= r; draw cap reached).
        if (my_row >= 0 && nr < rwant) {
            for (int w = 0; w < words && nr < rwant; ++w) {
                uint32_t free_bits = ~bm[w];
                while (free_bits && nr < rwant) {
                    const uint32_t j = (uint32_t)(w * 32 + __builtin_ctz(free_bits));
                    free_bits &= free_bits - 1u;
                    if ((int)j >= my_n) { free_bits = 0; break; }
#pragma unroll
                    for (int s = 0; s < TOPW; ++s) rnd[s] = (s == nr) ? j : rnd[s];
                    ++nr;
                }
            }
        }
        sort_asc<TOPW>(rnd);
    }

    if (my_row >= 0) {
        int32_t* dst = p.ids + ((size_t)h * p.nq + my_row) * p.c;
#pragma unroll
        for (int s = 0; s < TOPW; ++s) {
            if (s < ki) dst[s] = (int32_t)cmb[s];
            else if (s < ki + mi) dst[p.k + (s - ki)] = (int32_t)(cmb[s] & 0xFFFFu);
        }
        for (int s = ki; s < p.k; ++s) dst[s] = -1;
        for (int s = mi; s < p.m; ++s) dst[p.k + s] = -1;
#pragma unroll
        for (int s = 0; s < TOPW; ++s)
            if (s < p.r) dst[p.k + p.m + s] = (s < nr) ? (int32_t)rnd[s] : -1;
        p.anchor[(size_t)h * p.nq + my_row] = p.layer;
    }
}

// ------------------------------------------------------------------------------ rescore

template <typename DT>
__device__ __forceinline__ float dot_row(const typename Elem<DT>::type* q, const typename Elem<DT>::type* k);

template <>
__device__ __forceinline__ float dot_row<bf16_t>(const uint16_t* q, const uint16_t* k) {
    // 32 packed bf16 pairs; v_dot2 adds two exact bf16 products into the fp32 sum.
    const uint4* qa = reinterpret_cast<const uint4*>(q);
    const uint4* ka = reinterpret_cast<const uint4*>(k);
    uint32_t qw[32], kw[32];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        const uint4 a = qa[v], b = ka[v];
        qw[4 * v + 0] = a.x; qw[4 * v + 1] = a.y; qw[4 * v + 2] = a.z; qw[4 * v + 3] = a.w;
        kw[4 * v + 0] = b.x; kw[4 * v + 1] = b.y; kw[4 * v + 2] = b.z; kw[4 * v + 3] = b.w;
    }
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e)
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw[e]),
                                              __builtin_bit_cast(bf16x2, kw[e]), acc, false);
    return acc;
}

template <>
__device__ __forceinline__ float dot_row<float>(const float* q, const float* k) {
    const float4* qa = reinterpret_cast<const float4*>(q);
    const float4* ka = reinterpret_cast<const float4*>(k);
    float acc = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const float4 a = qa[v], b = ka[v];
        acc = fmaf(a.x, b.x, acc);
        acc = fmaf(a.y, b.y, acc);
        acc = fmaf(a.z, b.z, acc);
        acc = fmaf(a.w, b.w, acc);
    }
    return acc;
}

constexpr int RESCORE_THREADS = 1024;     // 16 waves x 4 rows: rows 64b..64b+63 of head h

// Block (h, b): rows 64b..64b+63 of head h; `cp` lanes per row (power of two >= c).
template <typename DT>
__global__ __launch_bounds__(RESCORE_THREADS) void k_rescore(RescoreArgs p) {
    typedef typename Elem<DT>::type E;
    __shared__ int32_t wave_flags[RESCORE_THREADS / 64];
    const int G = (p.nq + ROWS - 1) / ROWS;
    const int h = blockIdx.x / G;
    const int b = blockIdx.x % G;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int cp = p.cp;
    const int rpp = 64 / cp;                          // rows per wave pass
    const int slot = lane & (cp - 1);
    const E* Qh = reinterpret_cast<const E*>(p.qp) + (size_t)h * p.nq * 64;
    const E* Kh = reinterpret_cast<const E*>(p.kp) + (size_t)h * p.nk * 64;
    const float nan = __builtin_nanf("");
    int flagged = 0;
    for (int r0 = 0; r0 < 4; r0 += rpp) {
        const int rl = r0 + lane / cp;                // row within this wave's 4
        const int i = b * ROWS + wave * 4 + rl;
        const bool row_ok = rl < 4 && i < p.nq;
        const size_t flat = (size_t)h * p.nq + (row_ok ? i : 0);
        int id = (row_ok && slot < p.c) ? p.ids[flat * p.c + slot] : -1;
        id = (id < p.nk) ? id : -1;                   // never gather outside K, whatever the ledger holds
        float s = nan;
        if (id >= 0) s = dot_row<DT>(Qh + (size_t)i * 64, Kh + (size_t)id * 64);
        const float alpha = wave_min_in(slot < p.k ? s : nan, cp);
        const float nmin = wave_min_in((slot >= p.k && slot < p.sel) ? s : nan, cp);
        float beta = wave_max_in((slot >= p.k && slot < p.c) ? s : nan, cp);
        const int nsel = wave_sum_in((slot < p.sel && id >= 0) ? 1 : 0, cp);
        beta = (beta != beta) ? -INFINITY : beta;
        const bool reuse = alpha > (beta + p.gamma);
        if (row_ok) {
            if (p.cand_scores && slot < p.c) p.cand_scores[flat * p.c + slot] = s;
            if (slot == 0) {
                p.flags_ws[flat] = reuse ? 0 : 1;
                p.hint_ws[flat] = (nsel == p.sel) ? fminf(alpha, nmin) : -INFINITY;
                if (p.out_flags) p.out_flags[flat] = reuse ? 0 : 1;
                if (p.out_alpha) p.out_alpha[flat] = alpha;
                if (p.out_beta) p.out_beta[flat] = beta;
                flagged += reuse ? 0 : 1;
            }
        }
    }
    int wsum = flagged;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) wsum += __shfl_xor(wsum, o, 64);
    if (lane == 0) wave_flags[wave] = wsum;
    __syncthreads();
    if (threadIdx.x == 0) {
        int tot = 0;
#pragma unroll
        for (int w = 0; w < RESCORE_THREADS / 64; ++w) tot += wave_flags[w];
        p.bcount[blockIdx.x] = tot;
    }
}

// ------------------------------------------------------------------------------ launchers

size_t route_lds_bytes(int nk) {
    const size_t cand = (size_t)SPLIT * ROWS * CSTRIDE * sizeof(uint2);
    const size_t xchg = (size_t)2 * ROWS * TOPW * sizeof(uint64_t);
    const size_t gm = (size_t)ROWS * GSTRIDE * sizeof(float);
    const size_t bm = (size_t)ROWS * ((nk + 31) / 32 + 1) * sizeof(uint32_t);
    size_t m = cand > xchg ? cand : xchg;
    m = m > gm ? m : gm;
    return m > bm ? m : bm;
}

template <typename DT, bool CAUSAL, bool REROUTE>
static hipError_t launch_route_t(const RouteArgs& a, hipStream_t st) {
    const int G = (a.nq + ROWS - 1) / ROWS;
    const size_t lds = route_lds_bytes(a.nk);
    hipLaunchKernelGGL((k_route<DT, CAUSAL, REROUTE>), dim3(a.H * G), dim3(ROWS * SPLIT), lds, st, a);
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

hipError_t launch_rescore(const RescoreArgs& a, bool bf16, hipStream_t st) {
    const int G = (a.nq + ROWS - 1) / ROWS;
    if (bf16) hipLaunchKernelGGL((k_rescore<bf16_t>), dim3(a.H * G), dim3(RESCORE_THREADS), 0, st, a);
    else hipLaunchKernelGGL((k_rescore<float>), dim3(a.H * G), dim3(RESCORE_THREADS), 0, st, a);
    return hipGetLastError();
}

}  // namespace rr
