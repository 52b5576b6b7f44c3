// RouteRelay routing kernels for gfx950 (MI355X).
//
// Source: "RouteRelay: Event-Triggered Cross-Layer Route Reuse for Efficient Dynamic Sparse
// Attention" (arXiv 2609.07306), Sections 2.1, 3.1-3.2, 4.1-4.2.
//
// k_route    — full routing of a set of query rows of one head: S = Q K^T (Eq. 1) on MFMA,
//              top-(k+m) selection (Eq. 2 + near-miss sentinels), random sentinels, ledger
//              write.  Anchor mode routes rows 64g..64g+63; reroute mode routes the g-th slice
//              of 64 flagged rows of the head (the compacted list of Section 4.1/4.2), which it
//              recovers from the rescore kernel's flags.  One wave per block, 64 rows per wave.
// k_rescore  — relay candidate rescoring (Eq. 5-8): per row, gather the ledger's candidate key
//              rows, dot them with the query row, alpha / beta / refresh flag, plus a lower
//              bound on the row's (k+m)-th best score that the reroute uses as its first
//              selection threshold.  Writes per-block flag counts for the compaction.
//
// Selection scheme (route kernel): every row keeps a sorted top-32 list of 64-bit keys in
// registers (one row per lane).  Scores come out of the MFMA four per lane per 16x16 tile;
// those whose key reaches the row's threshold are appended to a per-row LDS buffer; when any
// buffer reaches 32 entries, each lane sorts its row's buffer (odd-even merge network) and
// merges it into its top list, and the threshold becomes the exact key of the (k+m)-th
// entry.  Nothing below the threshold can enter the top k+m, so the result is exact.  The
// first threshold is a proven lower bound on the (k+m)-th best score: in anchor mode the
// (k+m)-th largest of per-lane group maxima from a first MFMA pass; in reroute mode the
// smallest current score of the row's k+m ledger route/near-miss chunks (minus a rounding
// margin; a row that ends with too few entries is redone from -inf).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rr_device.h"
#include "rr_internal.h"

namespace rr {

constexpr int ROWS = 64;      // rows per route block (one wave, one row per lane)
constexpr int TOPW = 32;      // width of the register top list (k + m <= TOPW)
constexpr int CAP = 48;       // per-row LDS candidate buffer; a tile adds <= 16 to a row < 32
constexpr int CSTRIDE = CAP + 1;   // u64 row stride of the candidate buffers (bank spread)
constexpr int GSTRIDE = 33;        // f32 row stride of the group-maxima table
constexpr uint64_t NO_PASS_KEY = ~0ull;   // threshold whose score is NaN: nothing passes

struct bf16_t { uint16_t bits; };

template <typename DT> struct Operands;

// bf16: one 16x16x32 MFMA per 32-wide slice of d; lane L feeds d = 32h + 8*(L/16) + t.
template <> struct Operands<bf16_t> {
    bf16x8 q[4][2];   // B operand per row group g and d-half h
    __device__ __forceinline__ void load_q(const uint16_t* Q, const int (&row)[4], int lane) {
        const int sub = lane >> 4;
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (row[g] >= 0) {
                    q[g][h] = *reinterpret_cast<const bf16x8*>(Q + (size_t)row[g] * 64 + 32 * h + 8 * sub);
                } else {
                    u32x4 z = {0u, 0u, 0u, 0u};
                    q[g][h] = __builtin_bit_cast(bf16x8, z);
                }
            }
    }
    // acc[g][v] = score(row of group g, key = key0 + 4*(lane/16) + v)
    __device__ __forceinline__ void tile(const uint16_t* K, int key0, int nk, int lane, f32x4 (&acc)[4]) const {
        const int key = key0 + (lane & 15);
        const int sub = lane >> 4;
        bf16x8 a[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (key < nk) {
                a[h] = *reinterpret_cast<const bf16x8*>(K + (size_t)key * 64 + 32 * h + 8 * sub);
            } else {
                u32x4 z = {0u, 0u, 0u, 0u};
                a[h] = __builtin_bit_cast(bf16x8, z);
            }
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            f32x4 c = {0.f, 0.f, 0.f, 0.f};
            c = mfma_bf16(a[0], q[g][0], c);
            c = mfma_bf16(a[1], q[g][1], c);
            acc[g] = c;
        }
    }
};

// fp32: sixteen 16x16x4 MFMAs cover d = 64; lane L feeds d = 16*(L/16) + s at step s.
template <> struct Operands<float> {
    float q[4][16];
    __device__ __forceinline__ void load_q(const float* Q, const int (&row)[4], int lane) {
        const int sub = lane >> 4;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            if (row[g] >= 0) {
                const float4* src = reinterpret_cast<const float4*>(Q + (size_t)row[g] * 64 + 16 * sub);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float4 x = src[v];
                    q[g][4 * v + 0] = x.x; q[g][4 * v + 1] = x.y;
                    q[g][4 * v + 2] = x.z; q[g][4 * v + 3] = x.w;
                }
            } else {
#pragma unroll
                for (int s = 0; s < 16; ++s) q[g][s] = 0.f;
            }
        }
    }
    __device__ __forceinline__ void tile(const float* K, int key0, int nk, int lane, f32x4 (&acc)[4]) const {
        const int key = key0 + (lane & 15);
        const int sub = lane >> 4;
        float a[16];
        if (key < nk) {
            const float4* src = reinterpret_cast<const float4*>(K + (size_t)key * 64 + 16 * sub);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float4 x = src[v];
                a[4 * v + 0] = x.x; a[4 * v + 1] = x.y; a[4 * v + 2] = x.z; a[4 * v + 3] = x.w;
            }
        } else {
#pragma unroll
            for (int s = 0; s < 16; ++s) a[s] = 0.f;
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 16; ++s) c = mfma_f32(a[s], q[g][s], c);
            acc[g] = c;
        }
    }
};

template <typename DT> struct Elem { typedef float type; };
template <> struct Elem<bf16_t> { typedef uint16_t type; };

struct RouteShared {
    uint64_t thr[ROWS];
    int32_t rows[ROWS];
    uint32_t cnt[ROWS];
    uint32_t flag_words[ROWS];
    int32_t scan[ROWS];
};

// Dynamic LDS: candidate buffers [ROWS][CSTRIDE] u64, reused for the group maxima
// [ROWS][GSTRIDE] f32 of the first pass and for the sampler's chunk bitmaps [ROWS][words+1].
// The odd strides spread consecutive rows over the LDS banks.

__device__ __forceinline__ uint64_t pick(const uint64_t (&v)[TOPW], int idx) {
    uint64_t out = EMPTY_KEY;
#pragma unroll
    for (int s = 0; s < TOPW; ++s) out = (s == idx) ? v[s] : out;
    return out;
}

// Lane-per-row merge of the row's LDS buffer into its register top list; returns nothing,
// updates thr (LDS) to the exact key of entry sel-1 when the list holds at least sel keys.
__device__ __forceinline__ void merge_buffer(uint64_t (&top)[TOPW], uint64_t* cand_row, RouteShared& sh,
                                             int lane, int sel, uint64_t base_thr) {
    const int c = (int)sh.cnt[lane];
    int maxc = c;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) maxc = max(maxc, __shfl_xor(maxc, o, 64));
    for (int c0 = 0; c0 < maxc; c0 += TOPW) {
        uint64_t x[TOPW];
#pragma unroll
        for (int s = 0; s < TOPW; ++s) x[s] = (c0 + s < c) ? cand_row[c0 + s] : EMPTY_KEY;
        sort_desc<TOPW>(x);
        merge_top_desc<TOPW>(top, x);
    }
    sh.cnt[lane] = 0;
    const uint64_t t = pick(top, sel - 1);
    if (t != EMPTY_KEY && t > base_thr && sh.thr[lane] != NO_PASS_KEY) sh.thr[lane] = t;
}

template <typename DT, bool CAUSAL, bool REROUTE>
__global__ __launch_bounds__(64) void k_route(RouteArgs p) {
    typedef typename Elem<DT>::type E;
    extern __shared__ __align__(16) unsigned char dyn_lds[];
    __shared__ RouteShared sh;
    uint64_t* cand = reinterpret_cast<uint64_t*>(dyn_lds);

    const int lane = threadIdx.x;
    const int G = (p.nq + ROWS - 1) / ROWS;
    const int h = blockIdx.x / G;
    const int g = blockIdx.x % G;

    // ------------------------------------------------------------------ rows of this block
    if constexpr (REROUTE) {
        // Flag counts of the rescore blocks of this head: prefix over blocks -> where the
        // g-th slice of 64 flagged rows starts.
        const int32_t* bc = p.bcount + (size_t)h * G;
        int total = 0;
        for (int b0 = 0; b0 < G; b0 += 64) {
            const int v = (b0 + lane < G) ? bc[b0 + lane] : 0;
            total += wave_sum_in(v, 64);
        }
        const int count_h = total;
        if (g == 0) {
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
        if (g * ROWS >= count_h) return;
        // Locate the slice [64g, 64g+64) of the head's compacted list.
        const int want0 = g * ROWS;
        int run = 0;
        sh.rows[lane] = -1;
        __syncthreads();
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
        __syncthreads();
    } else {
        const int i = g * ROWS + lane;
        sh.rows[lane] = (i < p.nq) ? i : -1;
        __syncthreads();
    }

    // ------------------------------------------------------------------ per-row setup
    const int my_row = sh.rows[lane];                       // lane-per-row view
    const int my_n = (my_row < 0) ? 0 : (CAUSAL ? my_row + 1 : p.nk);
    int kmax = my_n, nmin = (my_row < 0) ? (1 << 30) : my_n;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        kmax = max(kmax, __shfl_xor(kmax, o, 64));
        nmin = min(nmin, __shfl_xor(nmin, o, 64));
    }
    const int ntiles = (kmax + 15) >> 4;

    // MFMA view: lane holds rows 16g'+(lane&15) for g' = 0..3 and keys 4*(lane>>4)+v of a tile.
    int vrow[4], vn[4], vslot[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        vslot[q4] = 16 * q4 + (lane & 15);
        vrow[q4] = sh.rows[vslot[q4]];
        vn[q4] = (vrow[q4] < 0) ? 0 : (CAUSAL ? vrow[q4] + 1 : p.nk);
    }
    const E* Qh = reinterpret_cast<const E*>(p.qp) + (size_t)h * p.nq * 64;
    const E* Kh = reinterpret_cast<const E*>(p.kp) + (size_t)h * p.nk * 64;
    Operands<DT> ops;
    ops.load_q(Qh, vrow, lane);
    const int sub = lane >> 4;

    // ------------------------------------------------------------------ first threshold
    uint64_t base_thr;
    if constexpr (REROUTE) {
        const float hv = (my_row >= 0) ? p.hint[(size_t)h * p.nq + my_row] : -INFINITY;
        const float t = (hv == -INFINITY) ? -INFINITY : hv - (fabsf(hv) * 1e-4f + 1e-6f);
        base_thr = make_key(t, 0xFFFFFFFFu);
    } else {
        // Pass 1: per lane and row, the 8 largest maxima over groups of gt tiles.
        const int gt = max(1, min(4, ntiles / 8));
        float top8[4][8], gmax[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            gmax[q4] = -INFINITY;
#pragma unroll
            for (int s = 0; s < 8; ++s) top8[q4][s] = -INFINITY;
        }
        for (int t = 0; t < ntiles; ++t) {
            f32x4 acc[4];
            ops.tile(Kh, 16 * t, p.nk, lane, acc);
            const bool edge = (16 * t + 16 > nmin);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int j = 16 * t + 4 * sub + v;
                    const float s = (!edge || j < vn[q4]) ? acc[q4][v] : -INFINITY;
                    gmax[q4] = fmaxf(gmax[q4], s);
                }
            }
            if ((t + 1) % gt == 0 || t == ntiles - 1) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    float x = gmax[q4];
#pragma unroll
                    for (int s = 0; s < 8; ++s) {
                        const float hi = fmaxf(top8[q4][s], x);
                        x = fminf(top8[q4][s], x);
                        top8[q4][s] = hi;
                    }
                    gmax[q4] = -INFINITY;
                }
            }
        }
        float* gm = reinterpret_cast<float*>(dyn_lds);        // [ROWS][32]
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
            for (int s = 0; s < 8; ++s) gm[vslot[q4] * GSTRIDE + 8 * sub + s] = top8[q4][s];
        __syncthreads();
        float v[32];
#pragma unroll
        for (int s = 0; s < 32; ++s) v[s] = gm[lane * GSTRIDE + s];
        sort_desc<32>(v);
        float t0 = -INFINITY;
#pragma unroll
        for (int s = 0; s < 32; ++s) t0 = (s == p.sel - 1) ? v[s] : t0;
        base_thr = make_key(t0, 0xFFFFFFFFu);
        __syncthreads();
    }

    // ------------------------------------------------------------------ streaming pass
    uint64_t top[TOPW];
#pragma unroll
    for (int s = 0; s < TOPW; ++s) top[s] = EMPTY_KEY;
    uint64_t* my_cand = cand + (size_t)lane * CSTRIDE;
    sh.thr[lane] = (my_row < 0) ? NO_PASS_KEY : base_thr;
    sh.cnt[lane] = 0;

    for (int attempt = 0; attempt < 2; ++attempt) {
        __syncthreads();
        float ts[4];
        uint32_t tj[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const uint64_t k = sh.thr[vslot[q4]];
            ts[q4] = key_score(k);
            tj[q4] = key_index(k);
        }
        for (int t = 0; t < ntiles; ++t) {
            f32x4 acc[4];
            ops.tile(Kh, 16 * t, p.nk, lane, acc);
            const bool edge = (16 * t + 16 > nmin);
            bool full = false;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int j = 16 * t + 4 * sub + v;
                    const float s = acc[q4][v];
                    const bool ok = (!edge || j < vn[q4]) && s >= ts[q4] && (s > ts[q4] || (uint32_t)j <= tj[q4]);
                    if (ok) {
                        const uint32_t slot = atomicAdd(&sh.cnt[vslot[q4]], 1u);
                        cand[(size_t)vslot[q4] * CSTRIDE + slot] = make_key(s, (uint32_t)j);
                        full |= (slot >= 31u);
                    }
                }
            }
            if (__ballot(full)) {
                __syncthreads();
                merge_buffer(top, my_cand, sh, lane, p.sel, base_thr);
                __syncthreads();
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const uint64_t k = sh.thr[vslot[q4]];
                    ts[q4] = key_score(k);
                    tj[q4] = key_index(k);
                }
            }
        }
        __syncthreads();
        merge_buffer(top, my_cand, sh, lane, p.sel, base_thr);
        // A row must now hold min(sel, n) keys; only a reroute threshold taken from the
        // rescore kernel's arithmetic can miss (rounding).  Redo such rows from -inf.
        int have = 0;
#pragma unroll
        for (int s = 0; s < TOPW; ++s) have += (top[s] != EMPTY_KEY);
        const bool redo = (my_row >= 0) && have < min(p.sel, my_n);
        if (!__ballot(redo)) break;
        if (redo) {
#pragma unroll
            for (int s = 0; s < TOPW; ++s) top[s] = EMPTY_KEY;
            base_thr = make_key(-INFINITY, 0xFFFFFFFFu);
            sh.thr[lane] = base_thr;
        } else {
            sh.thr[lane] = NO_PASS_KEY;
        }
    }
    __syncthreads();

    // ------------------------------------------------------------------ ledger update
    // Route = entries [0, ki), near-miss = [ki, ki+mi) of the sorted top list.  Both are
    // emitted ascending by chunk index: one ascending sort of (segment << 16 | index).
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
        // Draws: only rows whose pool is larger than r sample; smaller pools are taken whole
        // by the fill below.
        bool drawing = (my_row >= 0) && pool > p.r;
        P4 words4 = {0u, 0u, 0u, 0u};
        for (int t = 0; t < 65536 && __ballot(drawing); ++t) {
            if ((t & 3) == 0) {
                P4 c = {(uint32_t)(t >> 2), (uint32_t)my_row, (uint32_t)p.layer, (uint32_t)h};
                words4 = philox4x32_10(c, p.seed_lo, p.seed_hi);
            }
            const uint32_t u = ((t & 3) == 0) ? words4.x : ((t & 3) == 1) ? words4.y
                             : ((t & 3) == 2) ? words4.z : words4.w;
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
        // Fill: lowest-index chunks still free (whole pool when pool <= r; cap reached).
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

// --------------------------------------------------------------------------- rescore

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

// Block (h, b): rows 64b..64b+63 of head h; 256 threads, `cp` lanes per row (power of two >= c).
template <typename DT>
__global__ __launch_bounds__(256) void k_rescore(RescoreArgs p) {
    typedef typename Elem<DT>::type E;
    __shared__ int32_t block_flags[4];
    const int G = (p.nq + ROWS - 1) / ROWS;
    const int h = blockIdx.x / G;
    const int b = blockIdx.x % G;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int cp = p.cp;
    const int rpp = 64 / cp;                 // rows per wave pass
    const int slot = lane & (cp - 1);
    const E* Qh = reinterpret_cast<const E*>(p.qp) + (size_t)h * p.nq * 64;
    const E* Kh = reinterpret_cast<const E*>(p.kp) + (size_t)h * p.nk * 64;
    int flagged = 0;
    for (int r0 = wave * rpp; r0 < ROWS; r0 += 4 * rpp) {
        const int i = b * ROWS + r0 + lane / cp;
        const bool row_ok = i < p.nq;
        const size_t flat = (size_t)h * p.nq + (row_ok ? i : 0);
        int id = (row_ok && slot < p.c) ? p.ids[flat * p.c + slot] : -1;
        id = (id < p.nk) ? id : -1;          // never gather outside K, whatever the ledger holds
        float s = __builtin_nanf("");
        if (id >= 0) s = dot_row<DT>(Qh + (size_t)i * 64, Kh + (size_t)id * 64);
        const float nan = __builtin_nanf("");
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
    // block count of flagged rows (lanes with slot == 0 carry the per-row flags)
    int wsum = flagged;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) wsum += __shfl_xor(wsum, o, 64);
    if (lane == 0) block_flags[wave] = wsum;
    __syncthreads();
    if (threadIdx.x == 0)
        p.bcount[blockIdx.x] = block_flags[0] + block_flags[1] + block_flags[2] + block_flags[3];
}

// --------------------------------------------------------------------------- launchers

size_t route_lds_bytes(int nk) {
    const size_t cand = (size_t)ROWS * CSTRIDE * sizeof(uint64_t);
    const size_t gm = (size_t)ROWS * GSTRIDE * sizeof(float);
    const size_t bm = (size_t)ROWS * ((nk + 31) / 32 + 1) * sizeof(uint32_t);
    size_t m = cand > gm ? cand : gm;
    return m > bm ? m : bm;
}

template <typename DT, bool CAUSAL, bool REROUTE>
static hipError_t launch_route_t(const RouteArgs& a, hipStream_t st) {
    const int G = (a.nq + ROWS - 1) / ROWS;
    const size_t lds = route_lds_bytes(a.nk);
    hipLaunchKernelGGL((k_route<DT, CAUSAL, REROUTE>), dim3(a.H * G), dim3(64), lds, st, a);
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
    if (bf16) hipLaunchKernelGGL((k_rescore<bf16_t>), dim3(a.H * G), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((k_rescore<float>), dim3(a.H * G), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace rr
