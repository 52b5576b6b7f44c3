// Device-side building blocks of the RouteRelay routing kernels (gfx950 / CDNA4).
//
//  * 64-bit selection keys: (orderable fp32 score << 32) | (0xFFFFFFFF - chunk index), so that
//    a larger key means "higher score, and on equal scores the lower chunk index" — the
//    order under which the route (Eq. 2) and the near-miss sentinels (Section 3.1, item 1)
//    are ranked.  -0.0 is folded to +0.0 before encoding so both zeros tie.
//  * Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11), the counter-based generator behind the
//    random sentinels (Section 3.1, item 2).
//  * Compile-time sorting networks over register arrays (Batcher odd-even merge sort and the
//    bitonic merge), used one query row per lane.
//  * MFMA wrappers: v_mfma_f32_16x16x32_bf16 and v_mfma_f32_16x16x4_f32 computing
//    D[key][query] = sum_d K[key][d] * Q[query][d] for a 16-key x 16-query tile.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------------- keys

__device__ __forceinline__ uint32_t orderable(float s) {
    // -0.0 + 0.0 is +0.0 in round-to-nearest, so both zeros tie; then negative values have all
    // bits flipped and non-negative ones only the sign bit (no compare, no select).
    const uint32_t u = __float_as_uint(s + 0.0f);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ float from_orderable(uint32_t o) {
    uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
    return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t make_key(float s, uint32_t j) {
    return ((uint64_t)orderable(s) << 32) | (uint64_t)(0xFFFFFFFFu - j);
}

__device__ __forceinline__ uint32_t key_index(uint64_t key) {
    return 0xFFFFFFFFu - (uint32_t)key;
}

__device__ __forceinline__ float key_score(uint64_t key) {
    return from_orderable((uint32_t)(key >> 32));
}

// Key 0 sits below every real key (the lowest real score, -inf, encodes to 0x007FFFFF).
constexpr uint64_t EMPTY_KEY = 0ull;

// ---------------------------------------------------------------------------------- Philox

struct P4 { uint32_t x, y, z, w; };

__device__ __forceinline__ P4 philox4x32_10(P4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int rnd = 0; rnd < 10; ++rnd) {
        if (rnd) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
        const uint32_t hi0 = __umulhi(0xD2511F53u, c.x), lo0 = 0xD2511F53u * c.x;
        const uint32_t hi1 = __umulhi(0xCD9E8D57u, c.z), lo1 = 0xCD9E8D57u * c.z;
        c = P4{hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0};
    }
    return c;
}

// min / max of non-NaN values as one med3 (the median of {a, b, -inf} is the smaller of a, b).
// Unlike fminf / fmaxf these need no canonicalising of operands the compiler cannot prove
// canonical (MFMA results, lane moves).
__device__ __forceinline__ float min_f(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, -INFINITY); }
__device__ __forceinline__ float max_f(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, INFINITY); }

// ---------------------------------------------------------------------------------- networks
// All indices are compile-time constants after unrolling, so the arrays stay in VGPRs.

template <typename T>
__device__ __forceinline__ void ce_desc(T& a, T& b) {       // larger first
    const bool sw = b > a;
    const T hi = sw ? b : a;
    const T lo = sw ? a : b;
    a = hi;
    b = lo;
}

template <typename T>
__device__ __forceinline__ void ce_asc(T& a, T& b) {        // smaller first
    const bool sw = b < a;
    const T lo = sw ? b : a;
    const T hi = sw ? a : b;
    a = lo;
    b = hi;
}

// 64-bit keys: there is no 64-bit min / max instruction, and the two selects above are each
// rewritten into a max or a min with a compare of its own.  Selecting the swapped pair as one
// two-element vector keeps a single compare per exchange (four 32-bit selects on its mask).
typedef uint64_t u64x2_t __attribute__((ext_vector_type(2)));

template <>
__device__ __forceinline__ void ce_desc<uint64_t>(uint64_t& a, uint64_t& b) {
    const bool sw = b > a;
    const u64x2_t v = sw ? (u64x2_t){b, a} : (u64x2_t){a, b};
    a = v.x;
    b = v.y;
}

template <>
__device__ __forceinline__ void ce_asc<uint64_t>(uint64_t& a, uint64_t& b) {
    const bool sw = b < a;
    const u64x2_t v = sw ? (u64x2_t){b, a} : (u64x2_t){a, b};
    a = v.x;
    b = v.y;
}

// Batcher's odd-even merge sort, descending.
template <int N, typename T>
__device__ __forceinline__ void sort_desc(T (&v)[N]) {
#pragma unroll
    for (int p = 1; p < N; p <<= 1) {
#pragma unroll
        for (int k = p; k >= 1; k >>= 1) {
#pragma unroll
            for (int j = k % p; j + k < N; j += 2 * k) {
#pragma unroll
                for (int i = 0; i < k; ++i) {
                    if (i < N - j - k && (i + j) / (2 * p) == (i + j + k) / (2 * p))
                        ce_desc(v[i + j], v[i + j + k]);
                }
            }
        }
    }
}

// Same network, ascending.
template <int N, typename T>
__device__ __forceinline__ void sort_asc(T (&v)[N]) {
#pragma unroll
    for (int p = 1; p < N; p <<= 1) {
#pragma unroll
        for (int k = p; k >= 1; k >>= 1) {
#pragma unroll
            for (int j = k % p; j + k < N; j += 2 * k) {
#pragma unroll
                for (int i = 0; i < k; ++i) {
                    if (i < N - j - k && (i + j) / (2 * p) == (i + j + k) / (2 * p))
                        ce_asc(v[i + j], v[i + j + k]);
                }
            }
        }
    }
}

// top (sorted desc, N) <- the N largest of top U chunk, chunk sorted desc (N).
// max(top[i], chunk[N-1-i]) keeps exactly the N largest and leaves a bitonic sequence,
// which the half-cleaner cascade then sorts.
template <int N, typename T>
__device__ __forceinline__ void merge_top_desc(T (&top)[N], const T (&chunk)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const T c = chunk[N - 1 - i];
        top[i] = c > top[i] ? c : top[i];
    }
#pragma unroll
    for (int s = N / 2; s >= 1; s >>= 1) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            if ((i & s) == 0) ce_desc(top[i], top[i + s]);
    }
}

// ---------------------------------------------------------------------------------- MFMA

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------------- wave ops

// Cross-lane moves that stay in the VALU (no LDS round trip, no wait): DPP within 16-lane rows
// and the gfx950 row swaps across rows.
enum : int {
    DPP_XOR1 = 0xB1,          // quad_perm [1,0,3,2]
    DPP_XOR2 = 0x4E,          // quad_perm [2,3,0,1]
    DPP_HALF_MIRROR = 0x141,  // lane i of each 8-lane half-row <- lane 7 - i
    DPP_ROR4 = 0x124,         // lane i of each row <- lane (i + 4) mod 16
    DPP_ROR8 = 0x128,         // lane i of each row <- lane (i + 8) mod 16
    DPP_REVERSE = 0x1B,       // quad_perm [3,2,1,0]
    DPP_BCAST0 = 0x00,        // quad_perm [0,0,0,0]: every lane of a quad <- its lane 0
    DPP_BCAST1 = 0x55,        // quad_perm [1,1,1,1]
    DPP_BCAST2 = 0xAA,        // quad_perm [2,2,2,2]
    DPP_BCAST3 = 0xFF,        // quad_perm [3,3,3,3]
};
// Lanes whose source lies outside their row (the row shifts) read 0 (bound_ctrl); every other
// pattern here has a source for every lane, so no "old" value has to be materialised.
template <int CTRL> __device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL> __device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}

template <int CTRL> __device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)dpp_i<CTRL>((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)dpp_i<CTRL>((int)(uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Sum over aligned groups of G consecutive lanes (G = 8 or 16); every lane of a group ends with
// the bit-identical total (each step adds the same two partial sums in either order).
template <int G> __device__ __forceinline__ float group_sum(float s) {
    static_assert(G == 8 || G == 16, "group of 8 or 16 lanes");
    s += dpp_f<DPP_XOR1>(s);
    s += dpp_f<DPP_XOR2>(s);
    s += dpp_f<DPP_HALF_MIRROR>(s);
    if (G == 16) s += dpp_f<DPP_ROR8>(s);
    return s;
}

// Reduce over the 64 / G groups of G lanes whose members already agree (G = 8 or 16): the
// partner group sits at lane offset 8 (within a row), then 16 and 32 (row swaps).
template <int G, typename F> __device__ __forceinline__ uint32_t across_groups(uint32_t v, F op) {
    static_assert(G == 8 || G == 16, "group of 8 or 16 lanes");
    if (G == 8) v = op(v, (uint32_t)dpp_i<DPP_ROR8>((int)v));
    auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = op(a[0], a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return op(b[0], b[1]);
}

// Reduce over all 64 lanes (every lane ends with the result), without an LDS round trip:
// quad, half-row and row steps in DPP, then the row swaps.
template <typename F> __device__ __forceinline__ int wave_reduce_i(int v, F op) {
    v = op(v, dpp_i<DPP_XOR1>(v));
    v = op(v, dpp_i<DPP_XOR2>(v));
    v = op(v, dpp_i<DPP_HALF_MIRROR>(v));
    return (int)across_groups<8>((uint32_t)v, [op](uint32_t a, uint32_t b) { return (uint32_t)op((int)a, (int)b); });
}
__device__ __forceinline__ int wave_max_i(int v) { return wave_reduce_i(v, [](int a, int b) { return a > b ? a : b; }); }
__device__ __forceinline__ int wave_min_i(int v) { return wave_reduce_i(v, [](int a, int b) { return a < b ? a : b; }); }
__device__ __forceinline__ int wave_sum_i(int v) { return wave_reduce_i(v, [](int a, int b) { return a + b; }); }

// Inclusive prefix sum over the 64 lanes: shifts within rows of 16 in DPP (lanes without a
// source add 0), then the row totals from lanes 15, 31 and 47.
__device__ __forceinline__ int wave_incl_scan_i(int v) {
    v += dpp_i<0x111>(v);                                             // row_shr:1
    v += dpp_i<0x112>(v);                                             // row_shr:2
    v += dpp_i<0x114>(v);                                             // row_shr:4
    v += dpp_i<0x118>(v);                                             // row_shr:8
    const int r0 = __builtin_amdgcn_readlane(v, 15);
    const int r1 = __builtin_amdgcn_readlane(v, 31);
    const int r2 = __builtin_amdgcn_readlane(v, 47);
    const int lane = (int)(threadIdx.x & 63);
    return v + (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) + (lane >= 48 ? r2 : 0);
}

// fp32 min / max of two or three values as one VALU op.  Written as instructions because the compiler
// canonicalises both operands of fmaxf (two extra ops each) when it cannot prove them canonical,
// as for MFMA results and lane moves; the inputs here are never NaN.
__device__ __forceinline__ float vmax2(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float vmin2(float a, float b) {
    float r;
    asm("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

}  // namespace rr
