// Sparse attention over routed chunks on gfx950: the consumer of the routes.
//
// "RouteRelay: Event-Triggered Cross-Layer Route Reuse for Efficient Dynamic Sparse
// Attention", Section 2.1 (selected chunks are expanded into token indices for a sparse
// online-softmax kernel) and Section 2.2, Eq. 3: o_t = softmax(q_t K_R^T / sqrt(d)) V_R for
// every query token t of query chunk i, R being chunk i's route.
//
// Layout: chunk j covers tokens j*T .. j*T+T-1 (T = 64).  Q [H, nq*T, 64] and K [H, nk*T, 64]
// bf16 row-major; V handed over per chunk transposed, Vt [H, nk, 64 (d), T (token)], so that
// both MFMA operands of the second product load contiguous runs; routes [H, nq, kr] int32
// (-1 padding; any entry outside [0, nk) is padding too); O [H, nq*T, 64] fp32.
//
// Block = one query chunk of one head, two waves of 32 query tokens each.  Per routed chunk
// and 32-key half, each wave computes S^T = K_half Q^T (v_mfma_f32_32x32x16_bf16, keys x
// queries, so each lane holds 16 scores of one query), updates its queries' running max and
// sum (online softmax; the lane pair L, L^32 shares a query and exchanges with
// v_permlane32_swap), and accumulates O^T += V^T P^T (d x queries: the per-query rescale is
// per lane).  The MFMA k index of the second product runs over the 16 keys of each half of a
// tile in the order the first product leaves them in registers (lane half h, slot t: key
// 8(t/4) + 4h + t%4), and V^T is read in the same order, so P needs no data movement.  The
// next half's K and V^T loads are issued before the current half is computed.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rr_device.h"
#include "rr_internal.h"

namespace rr {

namespace {

typedef float f32x16a __attribute__((ext_vector_type(16)));

constexpr int AT = 64;                 // tokens per chunk
constexpr int AW = 2;                  // waves per block (32 query tokens each)

struct Half {                          // one 32-key half of a routed chunk, in registers
    bf16x8 k[4];                       // A operand of S^T: key L%32, d = 16s + 8(L/32) + 0..7
    bf16x8 v[2][2];                    // A operand of O^T: [d tile][k-step]
};

__device__ __forceinline__ bf16x8 pack8(uint2 a, uint2 b) {     // four bf16 from each run
    u32x4 w = {a.x, a.y, b.x, b.y};
    return __builtin_bit_cast(bf16x8, w);
}

// Loads of one half: K rows key0 .. key0+31 of the head, and the matching V^T entries.
__device__ __forceinline__ void load_half(Half& hf, const uint16_t* Kh, const uint16_t* Vth, int chunk, int half,
                                          int lane) {
    const int sub = lane >> 5;
    const uint16_t* krow = Kh + ((size_t)chunk * AT + 32 * half + (lane & 31)) * 64;
#pragma unroll
    for (int s = 0; s < 4; ++s) hf.k[s] = *reinterpret_cast<const bf16x8*>(krow + 16 * s + 8 * sub);
    // V^T of this chunk: [64 d][64 tokens]; lane L, d tile g: d = 32g + L%32; k-step u: keys
    // 32*half + 16u + 4*sub + 0..3 and + 8.
    const uint16_t* vbase = Vth + (size_t)chunk * 64 * AT;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const uint16_t* vrow = vbase + (size_t)(32 * g + (lane & 31)) * AT + 32 * half + 4 * sub;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const uint2 a = *reinterpret_cast<const uint2*>(vrow + 16 * u);
            const uint2 b = *reinterpret_cast<const uint2*>(vrow + 16 * u + 8);
            hf.v[g][u] = pack8(a, b);
        }
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
    const int blk = blockIdx.x;
    const int h = blk / p.nq;
    const int i = blk % p.nq;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int sub = lane >> 5;
    const int qloc = 32 * wave + (lane & 31);            // query token within the chunk
    const uint16_t* Qh = reinterpret_cast<const uint16_t*>(p.q) + (size_t)h * p.nq * AT * 64;
    const uint16_t* Kh = reinterpret_cast<const uint16_t*>(p.k) + (size_t)h * p.nk * AT * 64;
    const uint16_t* Vth = reinterpret_cast<const uint16_t*>(p.vt) + (size_t)h * p.nk * 64 * AT;
    const int32_t* route = p.routes + ((size_t)h * p.nq + i) * p.kr;

    // B operand of S^T: query qloc, d = 16s + 8 sub + 0..7.
    bf16x8 qb[4];
    {
        const uint16_t* qrow = Qh + ((size_t)i * AT + qloc) * 64;
#pragma unroll
        for (int s = 0; s < 4; ++s) qb[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * sub);
    }

    // The routed chunks are walked in route order (uniform over the block), two 32-key halves
    // each; half buffers A (first half) and B (second half) alternate so that each load is
    // issued one half ahead of its use and nothing is copied between registers.
    const float scale = 0.125f * 1.4426950408889634f;    // 1/sqrt(64) * log2(e): exp2 below
    f32x16a o0 = f32x16a{}, o1 = f32x16a{};              // O^T, d 0-31 and 32-63
    float mrun = -INFINITY, lrun = 0.f;
    auto next_valid = [&](int from) {
        for (int j = from; j < p.kr; ++j) {
            const int c = route[j];
            if (c >= 0 && c < p.nk && (!CAUSAL || c <= i)) return j;
        }
        return -1;
    };
    // One half: S^T = K_half Q^T, online-softmax update, O^T += V_half^T P^T.
    auto process = [&](const Half& hf, int chunk, int half) {
        f32x16a s = f32x16a{};
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hf.k[k4], qb[k4], s, 0, 0, 0);
        // lane L, register v: key 32*half + 8(v/4) + 4 sub + v%4 of this chunk, query qloc
        float mt = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            float x = s[v] * scale;
            if constexpr (CAUSAL) {
                const int key = 32 * half + 8 * (v >> 2) + 4 * sub + (v & 3);
                if (chunk == i && key > qloc) x = -INFINITY;
            }
            s[v] = x;
            mt = fmaxf(mt, x);
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
        // B operand of O^T, k-step u: slots t = 0..7 are registers 8u + t.
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            u32x4 w;
#pragma unroll
            for (int t = 0; t < 4; ++t)
                w[t] = bf16_bits(s[8 * u + 2 * t]) | (bf16_bits(s[8 * u + 2 * t + 1]) << 16);
            const bf16x8 pb = __builtin_bit_cast(bf16x8, w);
            o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hf.v[0][u], pb, o0, 0, 0, 0);
            o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hf.v[1][u], pb, o1, 0, 0, 0);
        }
    };
    Half A, B;
    int j = next_valid(0);
    if (j >= 0) load_half(A, Kh, Vth, route[j], 0, lane);
    while (j >= 0) {
        const int chunk = route[j];
        load_half(B, Kh, Vth, chunk, 1, lane);
        process(A, chunk, 0);
        j = next_valid(j + 1);
        if (j >= 0) load_half(A, Kh, Vth, route[j], 0, lane);
        process(B, chunk, 1);
    }
    // O[query][d] = O^T[d][query] / l; lane L holds d = 8(v/4) + 4 sub + v%4 (+32): runs of four.
    const float inv = (lrun > 0.f) ? 1.f / lrun : 0.f;
    float* orow = p.out + ((size_t)h * p.nq * AT + (size_t)i * AT + qloc) * 64;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const f32x16a& o = g ? o1 : o0;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            float4 w = make_float4(o[4 * r4] * inv, o[4 * r4 + 1] * inv, o[4 * r4 + 2] * inv, o[4 * r4 + 3] * inv);
            *reinterpret_cast<float4*>(orow + 32 * g + 8 * r4 + 4 * sub) = w;
        }
    }
}

}  // namespace

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t st) {
    const dim3 grid((unsigned)(a.H * a.nq));
    if (a.causal)
        hipLaunchKernelGGL(k_sparse_attn<true>, grid, dim3(64 * AW), 0, st, a);
    else
        hipLaunchKernelGGL(k_sparse_attn<false>, grid, dim3(64 * AW), 0, st, a);
    return hipGetLastError();
}

}  // namespace rr
