// Decode mat-vecs for Q4_K, Q5_K and relaid Q6_K weights against q8_K
// activations.
//
// "Language models on the device: the cajeta-llm kernels", section 2.1: one
// wavefront owns one output row; consecutive lanes read consecutive bytes of
// the row's blocks as whole words, dot them with the matching q8_K codes using
// the integer dot product, fold the sub-block scales, and a wave reduction
// finishes the row.  Section 2.2: the batched form reads each weight row once
// for up to Q8K_COLS_MAX activation columns.
//
// Lane map (gfx950 wave64): lane l serves block b = 8k + (l >> 3) of the row
// (k = 0, 1, ...) and its 16-byte quant chunk ci = l & 7, so each 64-lane
// load instruction covers the quant bytes of eight consecutive blocks.
//
// Latency: a decode mat-vec of a 4096-wide row is only two such 8-block
// groups per lane, so a wave would otherwise wait for two dependent HBM round
// trips.  Each trip of the main loop therefore issues every load of U groups
// (weight chunk, block header, q8_K codes, sums and scales) before any
// arithmetic.  Lanes whose block index runs past the row load the row's last
// block and contribute nothing, which keeps the wave convergent.
#include "kquant.h"
#include "q8k_launch.h"
#include "q8k_quant.h"

namespace q8k {

// Up to this many columns a wave keeps two 8-block groups (U = 2) in flight.
#ifndef Q8K_MV_U2_MAXNC
#define Q8K_MV_U2_MAXNC 4
#endif

// ---------------------------------------------------------- Q4_K, Q5_K ----
// Q5_K ("Language models on the device", section 2.3: the Q4_K member with
// the fifth-bit plane OR-ed into bit four) runs the Q4_K code with a 176-byte
// block, quants at byte 48 and each chunk's 16 qh bytes loaded beside it.
template <bool Q5>
constexpr int kblock() { return Q5 ? Q5K_BLOCK : Q4K_BLOCK; }

template <int NC, bool Q5>
struct Q4Chunk {
    uint4 hdr, qv, qh;
    int4 alo[NC], ahi[NC];
    uint32_t bs[NC];
    float d8[NC];
};

template <int NC, bool Q5>
__device__ __forceinline__ void q4k_load(Q4Chunk<NC, Q5>& L, const uint8_t* __restrict__ wr, int b, int ci, int aoff,
                                         int boff, const int8_t* __restrict__ qs, const float* __restrict__ d8,
                                         const int16_t* __restrict__ bs, int64_t K, int nb) {
    const uint8_t* blk = wr + (int64_t)b * kblock<Q5>();
    L.hdr = wload16<!Q5>(blk);
    L.qv = wload16<!Q5>(blk + (Q5 ? 48 : 16) + 16 * ci);
    if (Q5) L.qh = wload16<false>(blk + 16 + 16 * (ci & 1));
#pragma unroll
    for (int t = 0; t < NC; ++t) {
        const int8_t* a = qs + t * K + (int64_t)b * QK + aoff;
        L.alo[t] = *reinterpret_cast<const int4*>(a);
        L.ahi[t] = *reinterpret_cast<const int4*>(a + 32);
        L.bs[t] = *reinterpret_cast<const uint32_t*>(bs + ((int64_t)t * nb + b) * 8 + boff);
        L.d8[t] = d8[(int64_t)t * nb + b];
    }
}

// SUMS (test support, one column): also store the chunk's two exact sub-block
// sums to Sb[2c], Sb[2c + 1] (Sb: the block's eight sums); the two halves of
// each sub-block sit in lanes ci and ci ^ 1.
template <int NC, bool Q5, bool SUMS = false>
__device__ __forceinline__ void q4k_accum(const Q4Chunk<NC, Q5>& L, int c, int half, bool valid, float (&acc)[NC],
                                          int32_t* Sb = nullptr) {
    int sc0, sc1, m0, m1;
    q4k_scales(L.hdr, c, sc0, sc1, m0, m1);
    const float dd = half_bits_to_float(L.hdr.x & 0xffffu);
    const float dm = half_bits_to_float(L.hdr.x >> 16);
    uint32_t lo[4], hi[4];
    q4k_unpack(L.qv, lo, hi);
    if (Q5) q5k_fifth_bits(L.qh, c, lo, hi);
#pragma unroll
    for (int t = 0; t < NC; ++t) {
        int S0, S1;
        q4k_chunk_sums(lo, hi, L.alo[t], L.ahi[t], S0, S1);
        if constexpr (SUMS) {
            const int f0 = S0 + __shfl_xor(S0, 1, WAVE), f1 = S1 + __shfl_xor(S1, 1, WAVE);
            if (valid && !half) {
                Sb[2 * c] = f0;
                Sb[2 * c + 1] = f1;
            }
        }
        const int isum = sc0 * S0 + sc1 * S1;
        // the min term uses whole sub-block sums: counted once per chunk pair
        const int msum =
            half ? 0 : m0 * (int)(int16_t)(L.bs[t] & 0xffffu) + m1 * (int)(int16_t)(L.bs[t] >> 16);
        const float v = L.d8[t] * (dd * (float)isum - dm * (float)msum);
        acc[t] += valid ? v : 0.0f;
    }
}

// Rows (waves) per workgroup of the packed-activation mat-vec: up to two
// columns (narrow) and more.
#ifndef Q8K_MV_WAVES
#define Q8K_MV_WAVES 8
#endif
#ifndef Q8K_MV_WAVES_NARROW
#define Q8K_MV_WAVES_NARROW 4
#endif
template <int NC>
constexpr int mv_waves() { return NC <= 2 ? Q8K_MV_WAVES_NARROW : Q8K_MV_WAVES; }

// SUMS (test support, NC = 1): the same kernel also stores the exact
// sub-block sums S [rows][nb][8].
template <int NC, int U, bool Q5, bool SUMS = false>
__global__ __launch_bounds__(64 * mv_waves<NC>()) void matvec_q4k_kernel(const uint8_t* __restrict__ w, int64_t rows,
                                                                   int nb, const int8_t* __restrict__ qs,
                                                                   const float* __restrict__ d8,
                                                                   const int16_t* __restrict__ bs, int64_t K,
                                                                   float* __restrict__ y, int32_t* __restrict__ S) {
    static_assert(!SUMS || NC == 1, "sums of one column");
    const int64_t row = (int64_t)blockIdx.x * mv_waves<NC>() + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;  // uniform per wave
    const int ci = lane & 7, c = ci >> 1, half = ci & 1;
    const int aoff = 64 * c + 16 * half, boff = 2 * c;
    const uint8_t* wr = w + row * (int64_t)nb * kblock<Q5>();
    float acc[NC];
#pragma unroll
    for (int t = 0; t < NC; ++t) acc[t] = 0.0f;
    for (int b0 = lane >> 3; b0 - (lane >> 3) < nb; b0 += 8 * U) {
        Q4Chunk<NC, Q5> L[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int b = b0 + 8 * u;
            q4k_load(L[u], wr, b < nb ? b : nb - 1, ci, aoff, boff, qs, d8, bs, K, nb);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            q4k_accum<NC, Q5, SUMS>(L[u], c, half, b0 + 8 * u < nb, acc,
                                    SUMS ? S + (row * nb + b0 + 8 * u) * 8 : nullptr);
    }
#pragma unroll
    for (int t = 0; t < NC; ++t) {
        const float v = wave_sum_dpp(acc[t]);
        if (lane == 0) y[(int64_t)t * rows + row] = v;
    }
}

// ------------------------------------------------- fused pack + mat-vec ----
// One launch for a decode step from fp32 activations (the fused pack + GEMM
// of "Language models on the device", section 1 and the fused launches of
// section 3.3, which spare the packed activations a round trip through global
// memory and a launch).  A workgroup of four rows first issues the weight
// loads of its first loop trip, then its four waves quantise the activation
// columns into LDS (wave w takes blocks w, w+4, ...) with the same lane
// quantiser as q8k_pack, so the codes, sums and scales are the same bytes;
// after one barrier each wave runs the mat-vec of its row with the
// activations read from LDS.  Workgroup 0 also stores the packed columns when
// the caller asks for them (to feed further mat-vecs of the same tokens).
// The workgroup packs the NC activation columns x [NC][K] into LDS (codes
// [NC][K], sums [NC][nb][8], scales [NC][nb]); workgroup 0 also stores them
// to o when o.qs is not null.  Sixteen lanes take a block (16 values each),
// so the 256 threads pack 16 blocks at once: a 4096-wide column in one pass.
// The first pass (column 0, blocks 0..15) is loaded by pack_first, so that a
// caller can issue its own loads behind it: loads complete in issue order,
// and the packing must not wait for loads issued after its own.
struct PackFirst {
    float4 v[4];
};
// Workgroup size of the fused Q4_K/Q5_K kernel (one row per wave): every
// workgroup packs the whole activation, so fewer, larger workgroups repeat
// that work less often; up to two columns a wave's registers allow 16 waves.
#ifndef Q8K_FUSED_WAVES
#define Q8K_FUSED_WAVES 8
#endif
#ifndef Q8K_FUSED_WAVES_NARROW
#define Q8K_FUSED_WAVES_NARROW 16
#endif
template <int NC>
constexpr int fused_waves() { return NC <= 2 ? Q8K_FUSED_WAVES_NARROW : Q8K_FUSED_WAVES; }

__device__ __forceinline__ void pack_first(PackFirst& P, const float* __restrict__ x, int nb) {
    const int r = threadIdx.x & 15, b = threadIdx.x >> 4;
    if (b < nb) {
        const float4* src = reinterpret_cast<const float4*>(x + (int64_t)b * QK + 16 * r);
#pragma unroll
        for (int i = 0; i < 4; ++i) P.v[i] = src[i];
    }
}

__device__ __forceinline__ void pack_store(const float4 (&v)[4], int t, int b, int64_t K, int nb, int8_t* sqs,
                                           int16_t* sbs, float* sd, const PackedOut& o, bool out) {
    const int r = threadIdx.x & 15;
    int sub;
    float dd;
    const uint4 codes = q8k_quant_lane16(v, sub, dd);
    *reinterpret_cast<uint4*>(sqs + t * K + b * QK + 16 * r) = codes;
    if ((r & 1) == 0) sbs[(t * nb + b) * 8 + (r >> 1)] = (int16_t)sub;
    if (r == 0) sd[t * nb + b] = dd;
    if (out) {
        *reinterpret_cast<uint4*>(o.qs + t * K + (int64_t)b * QK + 16 * r) = codes;
        if ((r & 1) == 0) o.bs[((int64_t)t * nb + b) * 8 + (r >> 1)] = (int16_t)sub;
        if (r == 0) o.d[(int64_t)t * nb + b] = dd;
    }
}

// Ends with a workgroup barrier.
template <int NC>
__device__ __forceinline__ void pack_to_lds(const PackFirst& P, const float* __restrict__ x, int64_t K, int nb,
                                            int8_t* sqs, int16_t* sbs, float* sd, const PackedOut& o) {
    const int r = threadIdx.x & 15, b0 = threadIdx.x >> 4, bstep = blockDim.x >> 4;
    const bool out = o.qs != nullptr && blockIdx.x == 0;
#pragma unroll
    for (int t = 0; t < NC; ++t) {
        for (int b = b0; b < nb; b += bstep) {  // uniform per 16-lane row
            if (t == 0 && b == b0) {
                pack_store(P.v, 0, b, K, nb, sqs, sbs, sd, o, out);
                continue;
            }
            const float4* src = reinterpret_cast<const float4*>(x + t * K + (int64_t)b * QK + 16 * r);
            const float4 v[4] = {src[0], src[1], src[2], src[3]};
            pack_store(v, t, b, K, nb, sqs, sbs, sd, o, out);
        }
    }
    __syncthreads();
}

template <bool Q5>
struct Q4Weights {
    uint4 hdr, qv, qh;
};

template <bool Q5>
__device__ __forceinline__ void q4k_load_w(Q4Weights<Q5>& W, const uint8_t* __restrict__ wr, int b, int ci) {
    const uint8_t* blk = wr + (int64_t)b * kblock<Q5>();
    W.hdr = wload16<!Q5>(blk);
    W.qv = wload16<!Q5>(blk + (Q5 ? 48 : 16) + 16 * ci);
    if (Q5) W.qh = wload16<false>(blk + 16 + 16 * (ci & 1));
}

// The rows of one wave from activations in LDS (codes sqs [NC][K], sums sbs
// [NC][nb][8], scales sd [NC][nb]); W holds the weights of the first trip.
template <int NC, int U, bool Q5>
__device__ __forceinline__ void q4k_row_from_lds(Q4Weights<Q5> (&W)[U], const uint8_t* __restrict__ wr, int nb,
                                                 const int8_t* sqs, const int16_t* sbs, const float* sd, int64_t K,
                                                 int64_t rows, int64_t row, float* __restrict__ y) {
    const int lane = threadIdx.x & 63;
    const int ci = lane & 7, c = ci >> 1, half = ci & 1;
    const int aoff = 64 * c + 16 * half, boff = 2 * c;
    float acc[NC];
#pragma unroll
    for (int t = 0; t < NC; ++t) acc[t] = 0.0f;
    for (int b0 = lane >> 3; b0 - (lane >> 3) < nb; b0 += 8 * U) {
        Q4Chunk<NC, Q5> L[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int b = b0 + 8 * u;
            const int bc = b < nb ? b : nb - 1;
            L[u].hdr = W[u].hdr;
            L[u].qv = W[u].qv;
            L[u].qh = W[u].qh;
#pragma unroll
            for (int t = 0; t < NC; ++t) {
                const int8_t* a = sqs + t * K + bc * QK + aoff;
                L[u].alo[t] = *reinterpret_cast<const int4*>(a);
                L[u].ahi[t] = *reinterpret_cast<const int4*>(a + 32);
                L[u].bs[t] = *reinterpret_cast<const uint32_t*>(sbs + (t * nb + bc) * 8 + boff);
                L[u].d8[t] = sd[t * nb + bc];
            }
            // the next trip's weights
            const int bn = b + 8 * U;
            if (b0 - (lane >> 3) + 8 * U < nb) q4k_load_w(W[u], wr, bn < nb ? bn : nb - 1, ci);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) q4k_accum(L[u], c, half, b0 + 8 * u < nb, acc);
    }
#pragma unroll
    for (int t = 0; t < NC; ++t) {
        const float v = wave_sum_dpp(acc[t]);
        if (lane == 0) y[(int64_t)t * rows + row] = v;
    }
}

template <int NC, int U, bool Q5>
__device__ __forceinline__ void q4k_first_weights(Q4Weights<Q5> (&W)[U], const uint8_t* __restrict__ wr, int nb) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int b = (lane >> 3) + 8 * u;
        q4k_load_w(W[u], wr, b < nb ? b : nb - 1, lane & 7);
    }
}

// RW rows of one wave from the activations in LDS: each trip reads the
// columns' operands once and multiplies them into every row's accumulators.
// Each row's arithmetic (and its order) is that of q4k_row_from_lds, so the
// results are the same bits.  W[r] holds row r's weights of the first trip.
template <int NC, int U, bool Q5, int RW>
__device__ __forceinline__ void q4k_rows_from_lds(Q4Weights<Q5> (&W)[RW][U], const uint8_t* const (&wr)[RW], int nb,
                                                  const int8_t* sqs, const int16_t* sbs, const float* sd, int64_t K,
                                                  int64_t rows, const int64_t (&row)[RW], float* __restrict__ y) {
    const int lane = threadIdx.x & 63;
    const int ci = lane & 7, c = ci >> 1, half = ci & 1;
    const int aoff = 64 * c + 16 * half, boff = 2 * c;
    float acc[RW][NC];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int t = 0; t < NC; ++t) acc[r][t] = 0.0f;
    for (int b0 = lane >> 3; b0 - (lane >> 3) < nb; b0 += 8 * U) {
        Q4Chunk<NC, Q5> L[RW][U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int b = b0 + 8 * u;
            const int bc = b < nb ? b : nb - 1;
#pragma unroll
            for (int t = 0; t < NC; ++t) {
                const int8_t* a = sqs + t * K + bc * QK + aoff;
                L[0][u].alo[t] = *reinterpret_cast<const int4*>(a);
                L[0][u].ahi[t] = *reinterpret_cast<const int4*>(a + 32);
                L[0][u].bs[t] = *reinterpret_cast<const uint32_t*>(sbs + (t * nb + bc) * 8 + boff);
                L[0][u].d8[t] = sd[t * nb + bc];
            }
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                if (r > 0) {
#pragma unroll
                    for (int t = 0; t < NC; ++t) {
                        L[r][u].alo[t] = L[0][u].alo[t];
                        L[r][u].ahi[t] = L[0][u].ahi[t];
                        L[r][u].bs[t] = L[0][u].bs[t];
                        L[r][u].d8[t] = L[0][u].d8[t];
                    }
                }
                L[r][u].hdr = W[r][u].hdr;
                L[r][u].qv = W[r][u].qv;
                L[r][u].qh = W[r][u].qh;
                // the next trip's weights
                const int bn = b + 8 * U;
                if (b0 - (lane >> 3) + 8 * U < nb) q4k_load_w(W[r][u], wr[r], bn < nb ? bn : nb - 1, ci);
            }
        }
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int u = 0; u < U; ++u) q4k_accum(L[r][u], c, half, b0 + 8 * u < nb, acc[r]);
    }
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int t = 0; t < NC; ++t) {
            const float v = wave_sum_dpp(acc[r][t]);
            if (lane == 0 && row[r] < rows) y[(int64_t)t * rows + row[r]] = v;
        }
}

template <int NC, int U, bool Q5>
__global__ __launch_bounds__(64 * fused_waves<NC>()) void matvec_f32_q4k_kernel(const uint8_t* __restrict__ w,
                                                                                 int64_t rows, int nb,
                                                                                 const float* __restrict__ x, int64_t K,
                                                                                 float* __restrict__ y, PackedOut o) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    int8_t* sqs = reinterpret_cast<int8_t*>(lds);                                // [NC][K]
    int16_t* sbs = reinterpret_cast<int16_t*>(lds + (int64_t)NC * K);            // [NC][nb][8]
    float* sd = reinterpret_cast<float*>(lds + (int64_t)NC * K + 16 * NC * nb);  // [NC][nb]
    const int64_t row = (int64_t)blockIdx.x * fused_waves<NC>() + (threadIdx.x >> 6);
    const uint8_t* wr = w + (row < rows ? row : rows - 1) * (int64_t)nb * kblock<Q5>();
    PackFirst P;
    pack_first(P, x, nb);
    // weights of the first trip, in flight while the activations are packed
    Q4Weights<Q5> W[U];
    q4k_first_weights<NC, U, Q5>(W, wr, nb);
    pack_to_lds<NC>(P, x, K, nb, sqs, sbs, sd, o);
    if (row >= rows) return;  // uniform per wave, after the barrier
    q4k_row_from_lds<NC, U, Q5>(W, wr, nb, sqs, sbs, sd, K, rows, row, y);
}

// Packed-token form with the columns staged in LDS: the workgroup copies the
// NC packed columns (codes, sums, scales) into LDS once, so its waves read
// them there instead of each through the vector cache.  The first copy loads
// are issued before the weights (loads complete in issue order).
constexpr int STAGE_REGS = 4;  // 16-byte copy units per thread held across the weight loads
// Rows per wave of the staged kernel: each wave multiplies the columns' LDS
// operands into mv_rows_per_wave() rows, so the workgroup's one staging and
// every operand read serve that many rows.  Two rows raise the registers per
// wave; measured at 4096x4096 they pay for Q4_K at 3-4 columns and Q5_K from 3
// (4-5% faster) and cost elsewhere (6-7% slower at 2 and 8 Q4_K columns).
template <int NC, bool Q5>
constexpr int mv_rows_per_wave() { return NC >= 3 && (Q5 || NC <= 4) ? 2 : 1; }
template <int NC, int U, bool Q5>
__global__ __launch_bounds__(64 * mv_waves<NC>()) void matvec_staged_q4k_kernel(
    const uint8_t* __restrict__ w, int64_t rows, int nb, const int8_t* __restrict__ qs, const float* __restrict__ d8,
    const int16_t* __restrict__ bs, int64_t K, float* __restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    int8_t* sqs = reinterpret_cast<int8_t*>(lds);
    int16_t* sbs = reinterpret_cast<int16_t*>(lds + (int64_t)NC * K);
    float* sd = reinterpret_cast<float*>(lds + (int64_t)NC * K + 16 * NC * nb);
    constexpr int MV_RW = mv_rows_per_wave<NC, Q5>();
    const int T = 64 * mv_waves<NC>();
    // wave v takes rows first + v + r * waves (r < MV_RW) of the workgroup's run
    const int64_t first = (int64_t)blockIdx.x * mv_waves<NC>() * MV_RW;
    int64_t row[MV_RW];
    const uint8_t* wr[MV_RW];
#pragma unroll
    for (int r = 0; r < MV_RW; ++r) {
        row[r] = first + (threadIdx.x >> 6) + (int64_t)r * mv_waves<NC>();
        wr[r] = w + (row[r] < rows ? row[r] : rows - 1) * (int64_t)nb * kblock<Q5>();
    }
    // codes and sums as one run of 16-byte units: NC*K/16 of codes, then NC*nb of sums
    const int ncode = (int)(NC * K / 16), nunit = ncode + NC * nb;
    auto src = [&](int u) -> uint4 {
        return u < ncode ? reinterpret_cast<const uint4*>(qs)[u] : reinterpret_cast<const uint4*>(bs)[u - ncode];
    };
    auto dst = [&](int u) -> uint4* {
        return u < ncode ? reinterpret_cast<uint4*>(sqs) + u : reinterpret_cast<uint4*>(sbs) + (u - ncode);
    };
    uint4 R[STAGE_REGS];
#pragma unroll
    for (int i = 0; i < STAGE_REGS; ++i) {
        const int u = (int)threadIdx.x + i * T;
        if (u < nunit) R[i] = src(u);
    }
    float dv = 0.0f;
    if ((int)threadIdx.x < NC * nb) dv = d8[threadIdx.x];
    Q4Weights<Q5> W[MV_RW][U];
#pragma unroll
    for (int r = 0; r < MV_RW; ++r) q4k_first_weights<NC, U, Q5>(W[r], wr[r], nb);
#pragma unroll
    for (int i = 0; i < STAGE_REGS; ++i) {
        const int u = (int)threadIdx.x + i * T;
        if (u < nunit) *dst(u) = R[i];
    }
    for (int u = (int)threadIdx.x + STAGE_REGS * T; u < nunit; u += T) *dst(u) = src(u);
    if ((int)threadIdx.x < NC * nb) sd[threadIdx.x] = dv;
    for (int i = (int)threadIdx.x + T; i < NC * nb; i += T) sd[i] = d8[i];
    __syncthreads();
    if (row[0] >= rows) return;  // uniform per wave, after the barrier
    q4k_rows_from_lds<NC, U, Q5, MV_RW>(W, wr, nb, sqs, sbs, sd, K, rows, row, y);
}

// ---------------------------------------------------------------- Q6_K ----
// Lane map: lane l serves block b = 16k + (l >> 2) and the pair (h, lh) =
// ((l >> 1) & 1, l & 1): the two ql chunks 4h + lh and 4h + 2 + lh (tt = 0
// and 1), their shared qh chunk 2h + lh and the 8 scale bytes 8h..8h+7.  Four
// lanes cover a block, so a 64-lane pass spans 16 blocks (a 4096-wide row),
// every qh byte is read once and the scales need one 8-byte load per lane.
struct Q6W {  // one pass of one row
    uint4 ql0, ql1, qhv;
    uint2 scv;
    uint32_t dbits;
};
template <int NC>
struct Q6A {  // one pass of the activation columns
    int4 a[NC][4];  // codes of tt = 0 (low, high nibbles), tt = 1 (low, high)
    float d8[NC];
};

__device__ __forceinline__ void q6k_load_w(Q6W& W, const uint16_t* __restrict__ prefix,
                                           const uint8_t* __restrict__ bodies, int64_t row, int b, int h, int lh,
                                           int nb) {
    const int64_t ib = row * nb + b;
    const uint8_t* body = bodies + ib * Q6K_BODY;
    W.ql0 = *reinterpret_cast<const uint4*>(body + 16 * (4 * h + lh));
    W.ql1 = *reinterpret_cast<const uint4*>(body + 16 * (4 * h + 2 + lh));
    W.qhv = *reinterpret_cast<const uint4*>(body + 128 + 16 * (2 * h + lh));
    W.scv = *reinterpret_cast<const uint2*>(body + 192 + 8 * h);
    W.dbits = prefix[ib];
}

template <int NC>
__device__ __forceinline__ void q6k_load_a(Q6A<NC>& A, int b, int h, int lh, const int8_t* __restrict__ qs,
                                           const float* __restrict__ d8, int64_t K, int nb) {
    const int aoff = 128 * h + 16 * lh;
#pragma unroll
    for (int t = 0; t < NC; ++t) {
        const int8_t* a = qs + t * K + (int64_t)b * QK + aoff;
        A.a[t][0] = *reinterpret_cast<const int4*>(a);       // tt = 0, low nibbles
        A.a[t][1] = *reinterpret_cast<const int4*>(a + 64);  // tt = 0, high nibbles
        A.a[t][2] = *reinterpret_cast<const int4*>(a + 32);  // tt = 1, low nibbles
        A.a[t][3] = *reinterpret_cast<const int4*>(a + 96);  // tt = 1, high nibbles
        A.d8[t] = d8[(int64_t)t * nb + b];
    }
}

// SUMS (test support, one column): also store the lane's four exact
// sub-block sums to Sb[lh], Sb[2 + lh], Sb[4 + lh], Sb[6 + lh] (Sb: the
// block's sums from sub-block 8h on).
template <int NC, bool SUMS = false>
__device__ __forceinline__ void q6k_accum(const Q6W& W, const Q6A<NC>& A, int lh, bool valid, float (&acc)[NC],
                                          int32_t* Sb = nullptr) {
    // scale bytes (relative to 8h): sub-blocks 8h + 2tt + lh and +4
    const uint32_t sw0 = W.scv.x >> (8 * lh), sw1 = W.scv.y >> (8 * lh);
    const int sc00 = (int)(int8_t)(sw0 & 0xffu), sc01 = (int)(int8_t)(sw1 & 0xffu);                  // tt = 0
    const int sc10 = (int)(int8_t)((sw0 >> 16) & 0xffu), sc11 = (int)(int8_t)((sw1 >> 16) & 0xffu);  // tt = 1
    const float dd = half_bits_to_float(W.dbits);
    uint32_t lo0[4], hi0[4], lo1[4], hi1[4];
    q6k_unpack(W.ql0, W.qhv, 0, lo0, hi0);
    q6k_unpack(W.ql1, W.qhv, 1, lo1, hi1);
#pragma unroll
    for (int t = 0; t < NC; ++t) {
        const int s00 = q6k_sum16(lo0, A.a[t][0]), s01 = q6k_sum16(hi0, A.a[t][1]);
        const int s10 = q6k_sum16(lo1, A.a[t][2]), s11 = q6k_sum16(hi1, A.a[t][3]);
        if constexpr (SUMS) {
            if (valid) {
                Sb[lh] = s00;
                Sb[4 + lh] = s01;
                Sb[2 + lh] = s10;
                Sb[6 + lh] = s11;
            }
        }
        const int I = sc00 * s00 + sc01 * s01 + sc10 * s10 + sc11 * s11;
        const float v = A.d8[t] * dd * (float)I;
        acc[t] += valid ? v : 0.0f;
    }
}

template <int NC>
__device__ __forceinline__ void q6k_store(const float (&acc)[NC], int lane, int64_t rows, int64_t row,
                                          float* __restrict__ y) {
#pragma unroll
    for (int t = 0; t < NC; ++t) {
        const float v = wave_sum_dpp(acc[t]);
        if (lane == 0) y[(int64_t)t * rows + row] = v;
    }
}

// One wave walks rows row0, row0 + stride, ... (stride = all waves of the
// grid).  When a row fits one pass (K <= 4096) the activation codes are loaded
// once per wave and the weights of the wave's next Q6_DEPTH - 1 rows are
// issued before the current row is reduced, so Q6_DEPTH rows are in flight;
// a prefetch past the last row re-reads the wave's current row (cache-hot)
// and is not used.
#ifndef Q8K_Q6_DEPTH
#define Q8K_Q6_DEPTH 2
#endif
constexpr int Q6_DEPTH = Q8K_Q6_DEPTH;
//
// FUSED: the activations arrive as fp32 columns x and every workgroup packs
// them into LDS first (as the fused Q4_K kernel does); qs and d8 are unused.
//
// SUMS (test support, NC = 1, packed token): the same kernel also stores the
// exact sub-block sums S [rows][nb][16].
template <int NC, bool FUSED, bool SUMS = false>
__global__ __launch_bounds__(256) void matvec_q6k_kernel(const uint16_t* __restrict__ prefix,
                                                         const uint8_t* __restrict__ bodies, int64_t rows, int nb,
                                                         const int8_t* __restrict__ qs, const float* __restrict__ d8,
                                                         int64_t K, float* __restrict__ y, const float* __restrict__ x,
                                                         PackedOut o, int32_t* __restrict__ S) {
    static_assert(!SUMS || (NC == 1 && !FUSED), "sums of one packed column");
    if constexpr (FUSED) {
        extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
        int8_t* sqs = reinterpret_cast<int8_t*>(lds);
        int16_t* sbs = reinterpret_cast<int16_t*>(lds + (int64_t)NC * K);
        float* sd = reinterpret_cast<float*>(lds + (int64_t)NC * K + 16 * NC * nb);
        PackFirst P;
        pack_first(P, x, nb);
        pack_to_lds<NC>(P, x, K, nb, sqs, sbs, sd, o);
        qs = sqs;
        d8 = sd;
    }
    const int64_t stride = (int64_t)gridDim.x * 4;
    int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;  // uniform per wave
    const int h = (lane >> 1) & 1, lh = lane & 1;
    const int bl = lane >> 2;
    if (nb <= 16) {
        const bool valid = bl < nb;
        const int b = valid ? bl : nb - 1;
        Q6A<NC> A;
        q6k_load_a(A, b, h, lh, qs, d8, K, nb);
        Q6W W[Q6_DEPTH];
#pragma unroll
        for (int i = 0; i < Q6_DEPTH - 1; ++i) {
            const int64_t r = row + i * stride;
            q6k_load_w(W[i], prefix, bodies, r < rows ? r : row, b, h, lh, nb);
        }
        for (;;) {
#pragma unroll
            for (int i = 0; i < Q6_DEPTH; ++i) {
                const int64_t cur = row + i * stride;
                const int64_t pre = cur + (Q6_DEPTH - 1) * stride;
                q6k_load_w(W[(i + Q6_DEPTH - 1) % Q6_DEPTH], prefix, bodies, pre < rows ? pre : cur, b, h, lh, nb);
                float acc[NC];
#pragma unroll
                for (int t = 0; t < NC; ++t) acc[t] = 0.0f;
                q6k_accum<NC, SUMS>(W[i], A, lh, valid, acc, SUMS ? S + (cur * nb + b) * 16 + 8 * h : nullptr);
                q6k_store(acc, lane, rows, cur, y);
                if (cur + stride >= rows) return;
            }
            row += Q6_DEPTH * stride;
        }
    }
    for (; row < rows; row += stride) {
        float acc[NC];
#pragma unroll
        for (int t = 0; t < NC; ++t) acc[t] = 0.0f;
        for (int b0 = bl; b0 - bl < nb; b0 += 16) {
            const int b = b0 < nb ? b0 : nb - 1;
            Q6W W;
            Q6A<NC> A;
            q6k_load_w(W, prefix, bodies, row, b, h, lh, nb);
            q6k_load_a(A, b, h, lh, qs, d8, K, nb);
            q6k_accum<NC, SUMS>(W, A, lh, b0 < nb, acc, SUMS ? S + (row * nb + b) * 16 + 8 * h : nullptr);
        }
        q6k_store(acc, lane, rows, row, y);
    }
}

// Test support: the wave reduction on closed-form inputs.  Thread t of one
// 256-thread workgroup holds t; out[w] = wave w's wave_sum_dpp (sum over its
// 64 lanes: 4096 w + 2016) and out[4] = the four wave sums added in order
// (sum of 0..255 = 32640), the reduction checks that the pages print.
__global__ __launch_bounds__(256) void wave_sums_kernel(float* __restrict__ out) {
    __shared__ float part[4];
    const int w = threadIdx.x >> 6;
    const float s = wave_sum_dpp((float)threadIdx.x);
    if ((threadIdx.x & 63) == 0) {
        out[w] = s;
        part[w] = s;
    }
    __syncthreads();
    if (threadIdx.x == 0) out[4] = (part[0] + part[1]) + (part[2] + part[3]);
}

hipError_t launch_wave_sums(float* out, hipStream_t s) {
    Q8K_LAUNCH(wave_sums_kernel, dim3(1), dim3(256), 0, s, out);
    return hipGetLastError();
}

// ----------------------------------------------------------- launchers ----
// Q4_K: two 8-block groups per loop trip for up to Q8K_MV_U2_MAXNC columns
// (a 4096-wide row in one trip); one group per trip for more columns, where
// the activation registers of every column already give enough loads in
// flight.  Q6_K: one 16-block pass per trip.
// From this many columns the packed-token mat-vec stages the columns in LDS
// (when they fit one workgroup's LDS).
#ifndef Q8K_MV_STAGED_MINNC
#define Q8K_MV_STAGED_MINNC 2
#endif
template <int NC, bool Q5>
static void go_q4k(const uint8_t* w, int64_t rows, int nb, Acts a, float* y, hipStream_t s) {
    constexpr int U = NC <= Q8K_MV_U2_MAXNC ? 2 : 1;
    constexpr int WV = mv_waves<NC>();
    if (NC >= Q8K_MV_STAGED_MINNC && fused_lds_bytes(NC, a.K) <= FUSED_LDS_MAX) {
        constexpr int RW = mv_rows_per_wave<NC, Q5>();
        Q8K_LAUNCH((matvec_staged_q4k_kernel<NC, U, Q5>), dim3((unsigned)((rows + WV * RW - 1) / (WV * RW))),
                   dim3(64 * WV),
                   fused_lds_bytes(NC, a.K), s, w, rows, nb, a.qs, a.d, a.bs, a.K, y);
        return;
    }
    Q8K_LAUNCH((matvec_q4k_kernel<NC, U, Q5>), dim3((unsigned)((rows + WV - 1) / WV)), dim3(64 * WV), 0, s, w, rows, nb,
               a.qs, a.d, a.bs, a.K, y, nullptr);
}
#ifndef Q8K_Q6_GRID
#define Q8K_Q6_GRID 512
#endif
template <int NC>
static void go_q6k(const uint16_t* p, const uint8_t* bodies, int64_t rows, int nb, Acts a, float* y, hipStream_t s) {
    const int64_t wgs = (rows + 3) / 4;
    const unsigned grid = (unsigned)(wgs < Q8K_Q6_GRID ? wgs : Q8K_Q6_GRID);
    Q8K_LAUNCH((matvec_q6k_kernel<NC, false>), dim3(grid), dim3(256), 0, s, p, bodies, rows, nb, a.qs, a.d, a.K, y,
               nullptr, PackedOut{nullptr, nullptr, nullptr}, nullptr);
}

template <bool Q5>
static hipError_t launch_q4k_family(const uint8_t* w, int64_t rows, int nb, Acts a, int ncols, float* y,
                                    hipStream_t s) {
    switch (ncols) {
        case 1: go_q4k<1, Q5>(w, rows, nb, a, y, s); break;
        case 2: go_q4k<2, Q5>(w, rows, nb, a, y, s); break;
        case 3: go_q4k<3, Q5>(w, rows, nb, a, y, s); break;
        case 4: go_q4k<4, Q5>(w, rows, nb, a, y, s); break;
        case 5: go_q4k<5, Q5>(w, rows, nb, a, y, s); break;
        case 6: go_q4k<6, Q5>(w, rows, nb, a, y, s); break;
        case 7: go_q4k<7, Q5>(w, rows, nb, a, y, s); break;
        case 8: go_q4k<8, Q5>(w, rows, nb, a, y, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_matvec_q4k(const uint8_t* w, int64_t rows, int nb, Acts a, int ncols, float* y, hipStream_t s) {
    return launch_q4k_family<false>(w, rows, nb, a, ncols, y, s);
}

hipError_t launch_matvec_q5k(const uint8_t* w, int64_t rows, int nb, Acts a, int ncols, float* y, hipStream_t s) {
    return launch_q4k_family<true>(w, rows, nb, a, ncols, y, s);
}

template <int NC, bool Q5>
static void go_f32_q4k(const uint8_t* w, int64_t rows, int nb, const float* x, int64_t K, float* y, PackedOut o,
                       hipStream_t s) {
    constexpr int U = NC <= Q8K_MV_U2_MAXNC ? 2 : 1;
    const size_t lds = fused_lds_bytes(NC, K);
    constexpr int WV = fused_waves<NC>();
    Q8K_LAUNCH((matvec_f32_q4k_kernel<NC, U, Q5>), dim3((unsigned)((rows + WV - 1) / WV)), dim3(64 * WV), lds, s, w,
               rows, nb, x, K, y, o);
}

template <int NC>
static void go_f32_q6k(const uint16_t* p, const uint8_t* bodies, int64_t rows, int nb, const float* x, int64_t K,
                       float* y, PackedOut o, hipStream_t s) {
    const int64_t wgs = (rows + 3) / 4;
    const unsigned grid = (unsigned)(wgs < Q8K_Q6_GRID ? wgs : Q8K_Q6_GRID);
    Q8K_LAUNCH((matvec_q6k_kernel<NC, true>), dim3(grid), dim3(256), fused_lds_bytes(NC, K), s, p, bodies, rows, nb,
               nullptr, nullptr, K, y, x, o, nullptr);
}

hipError_t launch_matvec_f32(int fmt, const uint8_t* w, const uint16_t* prefix, int64_t rows, int nb, const float* x,
                             int64_t K, int ncols, float* y, PackedOut o, hipStream_t s) {
#define Q8K_F32_CASE(n)                                            \
    case n:                                                        \
        if (fmt == WFMT_Q6_K)                                   \
            go_f32_q6k<n>(prefix, w, rows, nb, x, K, y, o, s);     \
        else if (fmt == WFMT_Q5_K)                              \
            go_f32_q4k<n, true>(w, rows, nb, x, K, y, o, s);       \
        else                                                       \
            go_f32_q4k<n, false>(w, rows, nb, x, K, y, o, s);      \
        break;
    switch (ncols) {
        Q8K_F32_CASE(1)
        Q8K_F32_CASE(2)
        Q8K_F32_CASE(3)
        Q8K_F32_CASE(4)
        Q8K_F32_CASE(5)
        Q8K_F32_CASE(6)
        Q8K_F32_CASE(7)
        Q8K_F32_CASE(8)
        default: return hipErrorInvalidValue;
    }
#undef Q8K_F32_CASE
    return hipGetLastError();
}

hipError_t launch_matvec_q6k(const uint16_t* prefix, const uint8_t* bodies, int64_t rows, int nb, Acts a, int ncols,
                             float* y, hipStream_t s) {
    switch (ncols) {
        case 1: go_q6k<1>(prefix, bodies, rows, nb, a, y, s); break;
        case 2: go_q6k<2>(prefix, bodies, rows, nb, a, y, s); break;
        case 3: go_q6k<3>(prefix, bodies, rows, nb, a, y, s); break;
        case 4: go_q6k<4>(prefix, bodies, rows, nb, a, y, s); break;
        case 5: go_q6k<5>(prefix, bodies, rows, nb, a, y, s); break;
        case 6: go_q6k<6>(prefix, bodies, rows, nb, a, y, s); break;
        case 7: go_q6k<7>(prefix, bodies, rows, nb, a, y, s); break;
        case 8: go_q6k<8>(prefix, bodies, rows, nb, a, y, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_matvec_sums(int fmt, const uint8_t* w, const uint16_t* prefix, int64_t rows, int nb, Acts a,
                              float* y, int32_t* S, hipStream_t s) {
    // qmatvec's launch shapes for one column (go_q4k, go_q6k)
    constexpr int WV = mv_waves<1>();
    const dim3 g4((unsigned)((rows + WV - 1) / WV));
    if (fmt == WFMT_Q4_K) {
        Q8K_LAUNCH((matvec_q4k_kernel<1, 2, false, true>), g4, dim3(64 * WV), 0, s, w, rows, nb, a.qs, a.d, a.bs, a.K,
                   y, S);
    } else if (fmt == WFMT_Q5_K) {
        Q8K_LAUNCH((matvec_q4k_kernel<1, 2, true, true>), g4, dim3(64 * WV), 0, s, w, rows, nb, a.qs, a.d, a.bs, a.K,
                   y, S);
    } else {
        const int64_t wgs = (rows + 3) / 4;
        const unsigned grid = (unsigned)(wgs < Q8K_Q6_GRID ? wgs : Q8K_Q6_GRID);
        Q8K_LAUNCH((matvec_q6k_kernel<1, false, true>), dim3(grid), dim3(256), 0, s, prefix, w, rows, nb, a.qs, a.d,
                   a.K, y, nullptr, PackedOut{nullptr, nullptr, nullptr}, S);
    }
    return hipGetLastError();
}

}  // namespace q8k
