// Mixture-of-experts decode: expert-indexed mat-vec with the weighted sum of
// each token's selected experts fused in.
//
// "Language models on the device: the cajeta-llm kernels", section 2.4: for a
// decode, every token's selected experts are visited in one launch and the
// experts' outputs are summed as they are produced; weights are read through
// the index of which expert each token chose (section intro).
//
// One wavefront owns MOE_ROWS consecutive output rows of every token.  It
// walks the experts in ascending order; for expert e it collects the
// (token, slot) pairs that chose e with a wave ballot over ids and takes them
// MOE_GROUP at a time (all of them in one group unless more than MOE_GROUP
// pairs chose e).  For each 2048-value segment of K it loads the group's q8_K
// codes into registers once, then streams the segment of each of its rows of
// W_e past them, issuing every row's loads before the arithmetic.  Each row of
// an expert is therefore read once, and each token's codes once per
// MOE_ROWS rows.  rw * dot is added into the token's running sum, held in
// registers (token t in lane t % 64, slot t / 64), so the order of the sum is
// fixed (experts ascending) and no atomics or workspace are used.  An expert
// nobody chose is never read; an id outside [0, E) matches no expert.
#include "kquant.h"
#include "q8k_launch.h"

namespace q8k {

#ifndef Q8K_MOE_GROUP
#define Q8K_MOE_GROUP 4
#endif
#ifndef Q8K_MOE_ROWS
#define Q8K_MOE_ROWS 2
#endif
constexpr int MOE_GROUP = Q8K_MOE_GROUP;
constexpr int MOE_ROWS = Q8K_MOE_ROWS;
constexpr int MOE_TSLOTS = 4;  // 4 * 64 = 256 tokens at most

template <bool Q6>
__global__ __launch_bounds__(256) void moe_kernel(const uint8_t* __restrict__ w, const uint16_t* __restrict__ prefix,
                                                  int64_t E, int64_t rows, int nb, const int8_t* __restrict__ qs,
                                                  const float* __restrict__ d8, const int16_t* __restrict__ bs,
                                                  int64_t K, int64_t T, const int32_t* __restrict__ ids,
                                                  const float* __restrict__ rw, int topk, float* __restrict__ y) {
    const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * MOE_ROWS;
    const int lane = threadIdx.x & 63;
    if (row0 >= rows) return;  // uniform per wave
    const int ci = lane & 7;
    // Q4_K lane constants
    const int c = ci >> 1, half = ci & 1;
    const int aoff4 = 64 * c + 16 * half;
    // Q6_K lane constants
    const int h = ci >> 2, tt = (ci >> 1) & 1, lh = ci & 1;
    const int s0 = 8 * h + 2 * tt + lh;
    const int aoff6 = 128 * h + 32 * tt + 16 * lh;
    const int qhoff = 128 + 16 * (2 * h + lh);
    const int aoff = Q6 ? aoff6 : aoff4;
    const int nseg = (nb + 7) / 8;

    float yreg[MOE_ROWS][MOE_TSLOTS];
#pragma unroll
    for (int r = 0; r < MOE_ROWS; ++r)
#pragma unroll
        for (int i = 0; i < MOE_TSLOTS; ++i) yreg[r][i] = 0.0f;
    const int64_t P = T * topk;

    for (int64_t e = 0; e < E; ++e) {
        for (int64_t p0 = 0; p0 < P; p0 += 64) {
            const int64_t p = p0 + lane;
            const bool sel = p < P && ids[p] == (int32_t)e;
            uint64_t mask = __ballot(sel);
            while (mask) {
                // ---- next group of up to MOE_GROUP pairs (wave-uniform)
                int tok[MOE_GROUP];
                float gw[MOE_GROUP];
                int ng = 0;
#pragma unroll
                for (int g = 0; g < MOE_GROUP; ++g) {
                    tok[g] = 0;
                    gw[g] = 0.0f;
                    if (mask) {
                        const int pi = (int)p0 + __builtin_ctzll(mask);
                        mask &= mask - 1;
                        tok[g] = pi / topk;
                        gw[g] = rw[pi];
                        ng = g + 1;
                    }
                }
                float acc[MOE_ROWS][MOE_GROUP];
#pragma unroll
                for (int r = 0; r < MOE_ROWS; ++r)
#pragma unroll
                    for (int g = 0; g < MOE_GROUP; ++g) acc[r][g] = 0.0f;

                for (int seg = 0; seg < nseg; ++seg) {
                    const int bq = seg * 8 + (lane >> 3);
                    const bool valid = bq < nb;
                    const int b = valid ? bq : nb - 1;
                    // ---- the group's codes for this segment
                    int4 alo[MOE_GROUP], ahi[MOE_GROUP];
                    uint32_t bsv[MOE_GROUP];
                    float dv[MOE_GROUP];
#pragma unroll
                    for (int g = 0; g < MOE_GROUP; ++g) {
                        if (g < ng) {
                            const int8_t* a = qs + (int64_t)tok[g] * K + (int64_t)b * QK + aoff;
                            alo[g] = *reinterpret_cast<const int4*>(a);
                            ahi[g] = *reinterpret_cast<const int4*>(a + (Q6 ? 64 : 32));
                            bsv[g] = Q6 ? 0u
                                        : *reinterpret_cast<const uint32_t*>(bs + ((int64_t)tok[g] * nb + b) * 8 + 2 * c);
                            dv[g] = d8[(int64_t)tok[g] * nb + b];
                        }
                    }
                    // ---- this segment of each row of W_e: loads first
                    uint4 wa[MOE_ROWS], wb[MOE_ROWS], wc[MOE_ROWS];
                    uint32_t wd[MOE_ROWS];
#pragma unroll
                    for (int r = 0; r < MOE_ROWS; ++r) {
                        const int64_t rr = row0 + r < rows ? row0 + r : rows - 1;
                        const int64_t ib = (e * rows + rr) * nb + b;
                        if (!Q6) {
                            const uint8_t* blk = w + ib * Q4K_BLOCK;
                            wa[r] = *reinterpret_cast<const uint4*>(blk);               // header
                            wb[r] = *reinterpret_cast<const uint4*>(blk + 16 + 16 * ci);  // quants
                        } else {
                            const uint8_t* body = w + ib * Q6K_BODY;
                            wa[r] = *reinterpret_cast<const uint4*>(body + 16 * ci);  // ql
                            wb[r] = *reinterpret_cast<const uint4*>(body + qhoff);    // qh
                            wc[r] = *reinterpret_cast<const uint4*>(body + 192);      // scales
                            wd[r] = prefix[ib];
                        }
                    }
#pragma unroll
                    for (int r = 0; r < MOE_ROWS; ++r) {
                        if (!Q6) {
                            int sc0, sc1, m0, m1;
                            q4k_scales(wa[r], c, sc0, sc1, m0, m1);
                            const float dd = half_bits_to_float(wa[r].x & 0xffffu);
                            const float dm = half_bits_to_float(wa[r].x >> 16);
                            uint32_t lo[4], hi[4];
                            q4k_unpack(wb[r], lo, hi);
#pragma unroll
                            for (int g = 0; g < MOE_GROUP; ++g) {
                                if (g < ng) {
                                    int S0, S1;
                                    q4k_chunk_sums(lo, hi, alo[g], ahi[g], S0, S1);
                                    const int isum = sc0 * S0 + sc1 * S1;
                                    const int msum = half ? 0
                                                          : m0 * (int)(int16_t)(bsv[g] & 0xffffu) +
                                                                m1 * (int)(int16_t)(bsv[g] >> 16);
                                    const float v = dv[g] * (dd * (float)isum - dm * (float)msum);
                                    acc[r][g] += valid ? v : 0.0f;
                                }
                            }
                        } else {
                            const int sc0 = (int)(int8_t)byte_of(wc[r], s0);
                            const int sc1 = (int)(int8_t)byte_of(wc[r], s0 + 4);
                            const float dd = half_bits_to_float(wd[r]);
                            uint32_t lo[4], hi[4];
                            q6k_unpack(wa[r], wb[r], tt, lo, hi);
#pragma unroll
                            for (int g = 0; g < MOE_GROUP; ++g) {
                                if (g < ng) {
                                    const int S0 = q6k_sum16(lo, alo[g]);
                                    const int S1 = q6k_sum16(hi, ahi[g]);
                                    const float v = dv[g] * dd * (float)(sc0 * S0 + sc1 * S1);
                                    acc[r][g] += valid ? v : 0.0f;
                                }
                            }
                        }
                    }
                }
                // ---- reduce and add rw * dot into the tokens' running sums
#pragma unroll
                for (int g = 0; g < MOE_GROUP; ++g) {
                    if (g < ng) {
#pragma unroll
                        for (int r = 0; r < MOE_ROWS; ++r) {
                            const float v = gw[g] * wave_sum_dpp(acc[r][g]);
#pragma unroll
                            for (int i = 0; i < MOE_TSLOTS; ++i)
                                if ((tok[g] >> 6) == i && (tok[g] & 63) == lane) yreg[r][i] += v;
                        }
                    }
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < MOE_ROWS; ++r) {
        if (row0 + r >= rows) break;
#pragma unroll
        for (int i = 0; i < MOE_TSLOTS; ++i) {
            const int64_t t = (int64_t)i * 64 + lane;
            if (t < T) y[t * rows + row0 + r] = yreg[r][i];
        }
    }
}

static unsigned moe_grid(int64_t rows) {
    const int64_t waves = (rows + MOE_ROWS - 1) / MOE_ROWS;
    return (unsigned)((waves + 3) / 4);
}

hipError_t launch_moe_q4k(const uint8_t* w, int64_t E, int64_t rows, int nb, Acts a, int64_t T, const int32_t* ids,
                          const float* rw, int topk, float* y, hipStream_t s) {
    hipLaunchKernelGGL(moe_kernel<false>, dim3(moe_grid(rows)), dim3(256), 0, s, w, (const uint16_t*)nullptr, E, rows,
                       nb, a.qs, a.d, a.bs, a.K, T, ids, rw, topk, y);
    return hipGetLastError();
}

hipError_t launch_moe_q6k(const uint16_t* prefix, const uint8_t* bodies, int64_t E, int64_t rows, int nb, Acts a,
                          int64_t T, const int32_t* ids, const float* rw, int topk, float* y, hipStream_t s) {
    hipLaunchKernelGGL(moe_kernel<true>, dim3(moe_grid(rows)), dim3(256), 0, s, bodies, prefix, E, rows, nb, a.qs,
                       a.d, a.bs, a.K, T, ids, rw, topk, y);
    return hipGetLastError();
}

}  // namespace q8k
