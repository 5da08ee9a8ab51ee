// Mixture-of-experts decode: expert-indexed mat-vec with the weighted sum of
// each token's selected experts fused in.
//
// "Language models on the device: the cajeta-llm kernels", section 2.4: for a
// decode, every token's selected experts are visited in one launch and the
// experts' outputs are summed as they are produced; weights are read through
// the index of which expert each token chose (section intro).
//
// One wavefront owns output row r of every token.  It walks the experts in
// ascending order; for expert e it collects the (token, slot) pairs that chose
// e with a wave ballot over ids, reads row r of W_e once per group of up to
// MOE_GROUP pairs (once in total unless more than MOE_GROUP pairs chose e),
// dots it with each pair's q8_K codes exactly as the decode mat-vec does, and
// adds rw * dot into the token's running sum.  The running sums live in
// registers (token t in lane t % 64, slot t / 64), so the order of the sum is
// fixed (experts ascending) and no atomics are used.  An expert nobody chose
// is never read; an id outside [0, E) matches no expert and is dropped.
#include "kquant.h"
#include "q8k_launch.h"

namespace q8k {

constexpr int MOE_GROUP = 8;
constexpr int MOE_TSLOTS = 4;  // 4 * 64 = 256 tokens at most

__device__ __forceinline__ void add_to_token(float (&yreg)[MOE_TSLOTS], int lane, int tok, float v) {
#pragma unroll
    for (int i = 0; i < MOE_TSLOTS; ++i)
        if ((tok >> 6) == i && (tok & 63) == lane) yreg[i] += v;
}

template <bool Q6>
__global__ __launch_bounds__(256) void moe_kernel(const uint8_t* __restrict__ w, const uint16_t* __restrict__ prefix,
                                                  int64_t E, int64_t rows, int nb, const int8_t* __restrict__ qs,
                                                  const float* __restrict__ d8, const int16_t* __restrict__ bs,
                                                  int64_t K, int64_t T, const int32_t* __restrict__ ids,
                                                  const float* __restrict__ rw, int topk, float* __restrict__ y) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const int ci = lane & 7;
    // Q4_K lane constants
    const int c = ci >> 1, half = ci & 1;
    // Q6_K lane constants
    const int h = ci >> 2, tt = (ci >> 1) & 1, lh = ci & 1;
    const int s0 = 8 * h + 2 * tt + lh;
    const int a6 = 128 * h + 32 * tt + 16 * lh;

    float yreg[MOE_TSLOTS];
#pragma unroll
    for (int i = 0; i < MOE_TSLOTS; ++i) yreg[i] = 0.0f;
    const int64_t P = T * topk;

    for (int64_t e = 0; e < E; ++e) {
        const int64_t erow = e * rows + row;  // row of the stacked [E*rows] weight
        for (int64_t p0 = 0; p0 < P; p0 += 64) {
            const int64_t p = p0 + lane;
            const bool sel = p < P && ids[p] == (int32_t)e;
            uint64_t mask = __ballot(sel);
            while (mask) {
                int pidx[MOE_GROUP];
                int ng = 0;
#pragma unroll
                for (int g = 0; g < MOE_GROUP; ++g) {
                    pidx[g] = 0;
                    if (mask) {
                        pidx[g] = (int)p0 + __builtin_ctzll(mask);
                        mask &= mask - 1;
                        ng = g + 1;
                    }
                }
                float acc[MOE_GROUP];
#pragma unroll
                for (int g = 0; g < MOE_GROUP; ++g) acc[g] = 0.0f;
                for (int b = lane >> 3; b < nb; b += 8) {
                    if (!Q6) {
                        const uint8_t* blk = w + (erow * nb + b) * Q4K_BLOCK;
                        const uint4 hdr = *reinterpret_cast<const uint4*>(blk);
                        const uint4 qv = *reinterpret_cast<const uint4*>(blk + 16 + 16 * ci);
                        int sc0, sc1, m0, m1;
                        q4k_scales(hdr, c, sc0, sc1, m0, m1);
                        const float dd = half_bits_to_float(hdr.x & 0xffffu);
                        const float dm = half_bits_to_float(hdr.x >> 16);
                        uint32_t lo[4], hi[4];
                        q4k_unpack(qv, lo, hi);
#pragma unroll
                        for (int g = 0; g < MOE_GROUP; ++g) {
                            if (g < ng) {
                                const int64_t tok = pidx[g] / topk;
                                const int8_t* a = qs + tok * K + (int64_t)b * QK + 64 * c + 16 * half;
                                int S0, S1;
                                q4k_chunk_sums(lo, hi, *reinterpret_cast<const int4*>(a),
                                               *reinterpret_cast<const int4*>(a + 32), S0, S1);
                                const uint32_t bb =
                                    *reinterpret_cast<const uint32_t*>(bs + (tok * nb + b) * 8 + 2 * c);
                                const int isum = sc0 * S0 + sc1 * S1;
                                const int msum =
                                    half ? 0 : m0 * (int)(int16_t)(bb & 0xffffu) + m1 * (int)(int16_t)(bb >> 16);
                                acc[g] += d8[tok * nb + b] * (dd * (float)isum - dm * (float)msum);
                            }
                        }
                    } else {
                        const int64_t ib = erow * nb + b;
                        const uint8_t* body = w + ib * Q6K_BODY;
                        const uint4 qlv = *reinterpret_cast<const uint4*>(body + 16 * ci);
                        const uint4 qhv = *reinterpret_cast<const uint4*>(body + 128 + 16 * (2 * h + lh));
                        const uint4 scv = *reinterpret_cast<const uint4*>(body + 192);
                        const int sc0 = (int)(int8_t)byte_of(scv, s0);
                        const int sc1 = (int)(int8_t)byte_of(scv, s0 + 4);
                        const float dd = half_bits_to_float(prefix[ib]);
                        uint32_t lo[4], hi[4];
                        q6k_unpack(qlv, qhv, tt, lo, hi);
#pragma unroll
                        for (int g = 0; g < MOE_GROUP; ++g) {
                            if (g < ng) {
                                const int64_t tok = pidx[g] / topk;
                                const int8_t* a = qs + tok * K + (int64_t)b * QK + a6;
                                const int S0 = q6k_sum16(lo, *reinterpret_cast<const int4*>(a));
                                const int S1 = q6k_sum16(hi, *reinterpret_cast<const int4*>(a + 64));
                                acc[g] += d8[tok * nb + b] * dd * (float)(sc0 * S0 + sc1 * S1);
                            }
                        }
                    }
                }
#pragma unroll
                for (int g = 0; g < MOE_GROUP; ++g) {
                    if (g < ng) {
                        const float v = wave_sum(acc[g]);
                        add_to_token(yreg, lane, pidx[g] / topk, rw[pidx[g]] * v);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < MOE_TSLOTS; ++i) {
        const int64_t t = (int64_t)i * 64 + lane;
        if (t < T) y[t * rows + row] = yreg[i];
    }
}

hipError_t launch_moe_q4k(const uint8_t* w, int64_t E, int64_t rows, int nb, Acts a, int64_t T, const int32_t* ids,
                          const float* rw, int topk, float* y, hipStream_t s) {
    hipLaunchKernelGGL(moe_kernel<false>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, w,
                       (const uint16_t*)nullptr, E, rows, nb, a.qs, a.d, a.bs, a.K, T, ids, rw, topk, y);
    return hipGetLastError();
}

hipError_t launch_moe_q6k(const uint16_t* prefix, const uint8_t* bodies, int64_t E, int64_t rows, int nb, Acts a,
                          int64_t T, const int32_t* ids, const float* rw, int topk, float* y, hipStream_t s) {
    hipLaunchKernelGGL(moe_kernel<true>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, bodies, prefix, E, rows,
                       nb, a.qs, a.d, a.bs, a.K, T, ids, rw, topk, y);
    return hipGetLastError();
}

}  // namespace q8k
