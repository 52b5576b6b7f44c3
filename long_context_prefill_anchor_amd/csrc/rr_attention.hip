// Sparse attention over routed chunks on gfx950: the consumer of the routes.
//
// "RouteRelay: Event-Triggered Cross-Layer Route Reuse for Efficient Dynamic Sparse
// Attention", Section 2.1 (selected chunks are expanded into token indices for a sparse
// online-softmax kernel) and Section 2.2, Eq. 3: o_t = softmax(q_t K_R^T / sqrt(d)) V_R for
// every query token t of query chunk i, R being chunk i's route.
//
// Layout: chunk j covers tokens j*T .. j*T+T-1 (T = 64).  Q [H, nq*T, 64] and K [H, nk*T, 64]
// bf16 row-major; V handed over per chunk transposed, Vt [H, nk, 64 (d), T (token)], so that
// both MFMA operands of the second product are runs along one row; routes [H, nq, kr] int32
// (-1 padding; any entry outside [0, nk) is padding too); O [H, nq*T, 64] fp32.
//
// Block = one query chunk of one head, two waves of 32 query tokens each.  Each routed chunk's
// K (8 KB) and V^T (8 KB) are loaded once per block with whole-line loads (128 threads x 16 B
// per instruction) into registers one chunk ahead, then stored to LDS, where both waves read
// their MFMA operands (padded rows keep the reads free of bank conflicts).  Per 32-key half a
// wave computes S^T = K_half Q^T (v_mfma_f32_32x32x16_bf16, keys x queries, so each lane holds
// 16 scores of one query), updates its queries' running max and sum (online softmax; the lane
// pair L, L^32 shares a query and combines with v_permlane32_swap), and accumulates
// O^T += V^T P^T (d x queries: the per-query rescale is per lane).  The k index of the second
// product runs over the keys in the order the first product leaves them in registers (lane
// half h, slot t: key 8(t/4) + 4h + t%4 of each 16-key step), and V^T is read in that order,
// so P goes from the accumulator to the operand with one bf16 rounding and no data movement.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rr_device.h"
#include "rr_internal.h"

namespace rr {

namespace {

typedef float f32x16a __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int AT = 64;                 // tokens per chunk
constexpr int AW = 2;                  // waves per block (32 query tokens each)
constexpr int KSTR = 72;               // LDS row stride of K, bf16 (144 B: 16-B aligned, conflict-free b128 reads)
constexpr int VSTR = 68;               // LDS row stride of V^T, bf16 (136 B: 8-B aligned, conflict-free b64 reads)

struct Stage {                         // one chunk's K and V^T as this thread loads them
    u32x4 k[4];
    u32x4 v[4];
};

// Thread x of the block loads bytes 16x + 2048r of the chunk's K and of its V^T (r = 0..3):
// row 16r + x/8, columns 8(x%8) .. 8(x%8)+7.
__device__ __forceinline__ void load_stage(Stage& st, const uint16_t* Kh, const uint16_t* Vth, int chunk, int x) {
    const u32x4* kc = reinterpret_cast<const u32x4*>(Kh + (size_t)chunk * AT * 64);
    const u32x4* vc = reinterpret_cast<const u32x4*>(Vth + (size_t)chunk * 64 * AT);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        st.k[r] = kc[x + 128 * r];
        st.v[r] = vc[x + 128 * r];
    }
}

__device__ __forceinline__ void store_stage(const Stage& st, uint16_t* lk, uint16_t* lv, int x) {
    const int row = x >> 3, col = 8 * (x & 7);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        *reinterpret_cast<u32x4*>(lk + (16 * r + row) * KSTR + col) = st.k[r];
        u32x2* vd = reinterpret_cast<u32x2*>(lv + (16 * r + row) * VSTR + col);
        vd[0] = u32x2{st.v[r][0], st.v[r][1]};
        vd[1] = u32x2{st.v[r][2], st.v[r][3]};
    }
}

// Lanes L and L^32 hold the same query: combine their values (the swap of x with itself
// leaves one lane's own value and its partner's in the two results).
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t bf16_bits(float x) {   // round to nearest even (finite inputs)
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <bool CAUSAL>
__global__ __launch_bounds__(64 * AW) __attribute__((amdgpu_waves_per_eu(3))) void k_sparse_attn(AttnArgs p) {
    __shared__ __align__(16) uint16_t lk[AT * KSTR];     // K of the current chunk: [token][d]
    __shared__ __align__(16) uint16_t lv[64 * VSTR];     // V^T of the current chunk: [d][token]
    // Workgroups go to the 8 XCDs round-robin; renumbered so that XCD x runs the contiguous
    // range [x * per, (x + 1) * per) of query chunks, i.e. whole heads: the chunks a head's
    // routes name then meet again in that XCD's L2 instead of in all eight.
    const int per = (int)gridDim.x / 8;
    const int blk = ((int)blockIdx.x % 8) * per + (int)blockIdx.x / 8;
    if (blk >= p.H * p.nq) return;                       // grid padding
    const int h = blk / p.nq;
    const int i = blk % p.nq;
    const int x = threadIdx.x;
    const int wave = x >> 6;
    const int lane = x & 63;
    const int sub = lane >> 5;
    const int qloc = 32 * wave + (lane & 31);            // query token within the chunk
    const uint16_t* Qh = reinterpret_cast<const uint16_t*>(p.q) + (size_t)h * p.nq * AT * 64;
    const uint16_t* Kh = reinterpret_cast<const uint16_t*>(p.k) + (size_t)h * p.nk * AT * 64;
    const uint16_t* Vth = reinterpret_cast<const uint16_t*>(p.vt) + (size_t)h * p.nk * 64 * AT;
    const int32_t* route = p.routes + ((size_t)h * p.nq + i) * p.kr;

    auto next_valid = [&](int from) {                    // uniform over the block
        for (int j = from; j < p.kr; ++j) {
            const int c = route[j];
            if (c >= 0 && c < p.nk && (!CAUSAL || c <= i)) return j;
        }
        return -1;
    };
    int j = next_valid(0);
    Stage st;
    if (j >= 0) load_stage(st, Kh, Vth, route[j], x);

    // B operand of S^T: query qloc, d = 16s + 8 sub + 0..7.
    bf16x8 qb[4];
    {
        const uint16_t* qrow = Qh + ((size_t)i * AT + qloc) * 64;
#pragma unroll
        for (int s = 0; s < 4; ++s) qb[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * sub);
    }

    const float scale = 0.125f * 1.4426950408889634f;    // 1/sqrt(64) * log2(e): exp2 below
    f32x16a o0 = f32x16a{}, o1 = f32x16a{};              // O^T, d 0-31 and 32-63
    float mrun = -INFINITY, lrun = 0.f;
    while (j >= 0) {
        const int chunk = route[j];
        __syncthreads();                                 // the previous chunk's reads are done
        store_stage(st, lk, lv, x);
        __syncthreads();
        j = next_valid(j + 1);
        if (j >= 0) load_stage(st, Kh, Vth, route[j], x);    // one chunk ahead
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            // A operand of S^T: key row 32 half + L%32, d = 16 s + 8 sub + 0..7.
            const uint16_t* krow = lk + (32 * half + (lane & 31)) * KSTR + 8 * sub;
            f32x16a s = f32x16a{};
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4)
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(krow + 16 * k4),
                                                            qb[k4], s, 0, 0, 0);
            // lane L, register v: key 32 half + 8(v/4) + 4 sub + v%4 of this chunk, query qloc
            float mt = -INFINITY;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                float xv = s[v] * scale;
                if constexpr (CAUSAL) {
                    const int key = 32 * half + 8 * (v >> 2) + 4 * sub + (v & 3);
                    if (chunk == i && key > qloc) xv = -INFINITY;
                }
                s[v] = xv;
                mt = fmaxf(mt, xv);
            }
            mt = pair_max(mt);
            const float mnew = fmaxf(mrun, mt);
            const float muse = (mnew == -INFINITY) ? 0.f : mnew;
            const float corr = exp2f(mrun - muse);
            float ls = 0.f;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                s[v] = exp2f(s[v] - muse);
                ls += s[v];
            }
            lrun = lrun * corr + pair_sum(ls);
            mrun = mnew;
            o0 *= corr;
            o1 *= corr;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                // B operand of O^T, k-step u: slots t = 0..7 are registers 8u + t.
                u32x4 w;
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    w[t] = bf16_bits(s[8 * u + 2 * t]) | (bf16_bits(s[8 * u + 2 * t + 1]) << 16);
                const bf16x8 pb = __builtin_bit_cast(bf16x8, w);
                // A operand of O^T, d tile g: row d = 32 g + L%32, keys 32 half + 16 u + 4 sub
                // + 0..3 and the same + 8.
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    const uint16_t* vrow = lv + (32 * g + (lane & 31)) * VSTR + 32 * half + 16 * u + 4 * sub;
                    const u32x2 a = *reinterpret_cast<const u32x2*>(vrow);
                    const u32x2 b = *reinterpret_cast<const u32x2*>(vrow + 8);
                    const u32x4 av = {a[0], a[1], b[0], b[1]};
                    const bf16x8 va = __builtin_bit_cast(bf16x8, av);
                    if (g == 0) o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o0, 0, 0, 0);
                    else o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o1, 0, 0, 0);
                }
            }
        }
    }
    // O[query][d] = O^T[d][query] / l; lane L holds d = 8(v/4) + 4 sub + v%4 (+32): runs of four.
    const float inv = (lrun > 0.f) ? 1.f / lrun : 0.f;
    float* orow = p.out + ((size_t)h * p.nq * AT + (size_t)i * AT + qloc) * 64;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
        *reinterpret_cast<float4*>(orow + 8 * r4 + 4 * sub) =
            make_float4(o0[4 * r4] * inv, o0[4 * r4 + 1] * inv, o0[4 * r4 + 2] * inv, o0[4 * r4 + 3] * inv);
        *reinterpret_cast<float4*>(orow + 32 + 8 * r4 + 4 * sub) =
            make_float4(o1[4 * r4] * inv, o1[4 * r4 + 1] * inv, o1[4 * r4 + 2] * inv, o1[4 * r4 + 3] * inv);
    }
}

}  // namespace

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t st) {
    const dim3 grid((unsigned)((a.H * a.nq + 7) / 8 * 8));   // a multiple of the 8 XCDs
    if (a.causal)
        hipLaunchKernelGGL(k_sparse_attn<true>, grid, dim3(64 * AW), 0, st, a);
    else
        hipLaunchKernelGGL(k_sparse_attn<false>, grid, dim3(64 * AW), 0, st, a);
    return hipGetLastError();
}

}  // namespace rr
