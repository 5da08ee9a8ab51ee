// Prefill GEMM: Q4_K weight [N rows][K] times M packed q8_K tokens on the
// gfx950 matrix cores.
//
// "Language models on the device: the cajeta-llm kernels", section 2.3: a
// workgroup computes a tile of tokens x weight rows; weight nibbles are
// widened into an int8 tile in shared memory beside the tokens' q8_K codes,
// staged ahead of the arithmetic, the waves multiply fragments on the matrix
// units, and the per-sub-block scales fold in through the accumulator
// epilogue (the scale/min epilogue of section 1).
//
// Per (token m, row n) the result is
//   y = sum_b d8_b * d_b * I_b  -  sum_b sum_j (d8_b * bsum_bj) * (dmin_b * m_bj)
// with I_b = sum_j sc_j * S_j the scale-weighted integer dot of block b.
//
// MI355X design.  On gfx950 the int8 matrix cores retire 32x more operations
// per clock than the vector ALUs, so the per-sub-block scale fold must not run
// on the vector ALUs.  It is moved into the matrix-core operands instead:
// each 6-bit scale is split as sc = 8a + b (a, b in 0..7) and the weight is
// staged as two int8 planes a*q and b*q (each <= 105); two int8 MFMA passes
// over the whole block give P_hi, P_lo and I_b = 8 P_hi + P_lo exactly.  The
// min term is a GEMM over the (block, sub-block) axis whose operands already
// carry their block scales, so it accumulates in fp32 across all blocks on
// the bf16 matrix path: both operands are split into bf16 high and low parts
// (a = ah + al exactly to ~2^-18) and all four cross products are taken, two
// 32x32x16 bf16 MFMAs per block.  What remains on the vector ALUs is the
// block epilogue, acc += (d8 * float(8 P_hi + P_lo)) * d: four operations per
// output and block.
//
// Tiles: workgroup 128 tokens x 64 weight rows, 4 waves; wave w holds tokens
// 64(w&1)..+63 (two 32-token MFMA tiles sharing one weight fragment) and rows
// 32(w>>1)..+31.  Per 256-value block the workgroup stages the two weight
// planes, the tokens' codes and the min-term operands in LDS (rows padded by
// 16 bytes); the next block's global loads are issued into registers before
// the current block's arithmetic.
//
// MFMA operand map (verified on gfx950): 32x32x32 int8 and 32x32x16 bf16 take
// row l % 32 of A and column l % 32 of B from lane l, k-group l / 32; result
// (i, j) is in lane j + 32 * ((i / 4) % 2), register (i % 4) + 4 * (i / 8).
// A = tokens, B = weight rows, so each lane owns one weight row.
#include "q8k_device.h"
#include "q8k_launch.h"

namespace q8k {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

// Four byte-wise products q_i * k (q_i <= 15, k <= 7, so every product stays
// inside its byte) as one packed 16-bit multiply (v_pk_mul_lo_u16).
__device__ __forceinline__ uint32_t mul_bytes(uint32_t q, uint32_t k) {
    const v2u16 kk = {(unsigned short)k, (unsigned short)k};
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2u16, q) * kk);
}

constexpr int PF_TM = 128;      // tokens per workgroup
constexpr int PF_TN = 64;       // weight rows per workgroup
constexpr int PF_LD = QK + 16;  // LDS row stride in bytes (bank spread)

struct PrefillSmem {
    int8_t whi[PF_TN * PF_LD];   // weight plane a*q
    int8_t wlo[PF_TN * PF_LD];   // weight plane b*q
    int8_t xa[PF_TM * PF_LD];    // token codes
    float dw[PF_TN];             // row block scale d
    float d8[PF_TM];             // token block scale
    uint16_t bj[PF_TN][16];      // dmin*m_j as bf16: [0..7] high, [8..15] low
    uint16_t aj[PF_TM][16];      // d8*bsum_j as bf16: [0..7] high, [8..15] low
};

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_val(uint32_t b) { return __builtin_bit_cast(float, b << 16); }

// Sub-block scale and min j (0..7) from the 12 packed bytes (hdr.y|z|w).
__device__ __forceinline__ void q4k_scale_min(uint4 hdr, int j, int& sc, int& mn) {
    if (j < 4) {
        sc = (int)((hdr.y >> (8 * j)) & 63);
        mn = (int)((hdr.z >> (8 * j)) & 63);
    } else {
        const uint32_t lo = (hdr.w >> (8 * (j - 4))) & 0xffu;
        sc = (int)((lo & 15) | (((hdr.y >> (8 * (j - 4))) >> 6 & 3) << 4));
        mn = (int)((lo >> 4) | (((hdr.z >> (8 * (j - 4))) >> 6 & 3) << 4));
    }
}

// Registers holding one block's global data for this thread, loaded ahead.
struct PrefillStage {
    uint4 hdr, q0, q1;  // weight: header and 32 quant bytes
    uint4 x[8];         // token: 128 codes
    float d8;
    uint4 bsv;          // token: eight int16 sums
};

__device__ __forceinline__ void prefill_load(PrefillStage& st, const uint8_t* __restrict__ w, int64_t rows, int nb,
                                             const int8_t* __restrict__ qs, const float* __restrict__ d8,
                                             const int16_t* __restrict__ bs, int64_t K, int64_t M, int64_t n0,
                                             int64_t m0, int b, int tid) {
    const int r = tid >> 2, p = tid & 3;
    const int64_t n = n0 + r;
    if (n < rows) {
        const uint8_t* blk = w + (n * nb + b) * Q4K_BLOCK;
        st.hdr = *reinterpret_cast<const uint4*>(blk);
        st.q0 = *reinterpret_cast<const uint4*>(blk + 16 + 32 * p);
        st.q1 = *reinterpret_cast<const uint4*>(blk + 16 + 32 * p + 16);
    } else {
        st.hdr = st.q0 = st.q1 = make_uint4(0, 0, 0, 0);
    }
    const int t = tid >> 1, hh = tid & 1;
    const int64_t m = m0 + t;
    if (m < M) {
        const int8_t* src = qs + m * K + (int64_t)b * QK + 128 * hh;
#pragma unroll
        for (int i = 0; i < 8; ++i) st.x[i] = *reinterpret_cast<const uint4*>(src + 16 * i);
        st.d8 = d8[m * nb + b];
        st.bsv = *reinterpret_cast<const uint4*>(bs + (m * nb + b) * 8);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) st.x[i] = make_uint4(0, 0, 0, 0);
        st.d8 = 0.0f;
        st.bsv = make_uint4(0, 0, 0, 0);
    }
}

__device__ __forceinline__ void prefill_store(const PrefillStage& st, PrefillSmem& sm, int tid) {
    // ---- weight planes: thread -> row tid/4, quant bytes 32p..32p+31, i.e.
    // values 64p..64p+31 (low nibbles, sub-block 2p) and 64p+32..64p+63 (high
    // nibbles, sub-block 2p+1).
    {
        const int r = tid >> 2, p = tid & 3;
        int sc0, mn0, sc1, mn1;
        q4k_scale_min(st.hdr, 2 * p, sc0, mn0);
        q4k_scale_min(st.hdr, 2 * p + 1, sc1, mn1);
        // plane multipliers, applied to four bytes at a time
        const uint32_t a0 = (uint32_t)(sc0 >> 3), b0 = (uint32_t)(sc0 & 7);
        const uint32_t a1 = (uint32_t)(sc1 >> 3), b1 = (uint32_t)(sc1 & 7);
        const uint32_t qw[8] = {st.q0.x, st.q0.y, st.q0.z, st.q0.w, st.q1.x, st.q1.y, st.q1.z, st.q1.w};
        uint32_t lh[8], ll[8], hh[8], hl[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t lo = qw[i] & 0x0F0F0F0Fu, hi = (qw[i] >> 4) & 0x0F0F0F0Fu;
            lh[i] = mul_bytes(lo, a0);
            ll[i] = mul_bytes(lo, b0);
            hh[i] = mul_bytes(hi, a1);
            hl[i] = mul_bytes(hi, b1);
        }
        int8_t* dh = sm.whi + r * PF_LD + 64 * p;
        int8_t* dl = sm.wlo + r * PF_LD + 64 * p;
        *reinterpret_cast<uint4*>(dh) = make_uint4(lh[0], lh[1], lh[2], lh[3]);
        *reinterpret_cast<uint4*>(dh + 16) = make_uint4(lh[4], lh[5], lh[6], lh[7]);
        *reinterpret_cast<uint4*>(dh + 32) = make_uint4(hh[0], hh[1], hh[2], hh[3]);
        *reinterpret_cast<uint4*>(dh + 48) = make_uint4(hh[4], hh[5], hh[6], hh[7]);
        *reinterpret_cast<uint4*>(dl) = make_uint4(ll[0], ll[1], ll[2], ll[3]);
        *reinterpret_cast<uint4*>(dl + 16) = make_uint4(ll[4], ll[5], ll[6], ll[7]);
        *reinterpret_cast<uint4*>(dl + 32) = make_uint4(hl[0], hl[1], hl[2], hl[3]);
        *reinterpret_cast<uint4*>(dl + 48) = make_uint4(hl[4], hl[5], hl[6], hl[7]);
        // min-term operand dmin * m_j (exact in fp32), split into bf16 parts
        const float dm = half_bits_to_float(st.hdr.x >> 16);
        const float v0 = dm * (float)mn0, v1 = dm * (float)mn1;
        const uint32_t h0 = bf16_bits(v0), h1 = bf16_bits(v1);
        sm.bj[r][2 * p] = (uint16_t)h0;
        sm.bj[r][2 * p + 1] = (uint16_t)h1;
        sm.bj[r][8 + 2 * p] = (uint16_t)bf16_bits(v0 - bf16_val(h0));
        sm.bj[r][8 + 2 * p + 1] = (uint16_t)bf16_bits(v1 - bf16_val(h1));
        if (p == 0) sm.dw[r] = half_bits_to_float(st.hdr.x & 0xffffu);
    }
    // ---- tokens: thread -> token tid/2, codes 128h..128h+127
    {
        const int t = tid >> 1, hh = tid & 1;
        int8_t* dst = sm.xa + t * PF_LD + 128 * hh;
#pragma unroll
        for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(dst + 16 * i) = st.x[i];
        const uint32_t bw[4] = {st.bsv.x, st.bsv.y, st.bsv.z, st.bsv.w};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int j = 4 * hh + jj;
            const uint32_t word = bw[j >> 1];
            const int s = (int)(int16_t)((j & 1) ? (word >> 16) : (word & 0xffffu));
            const float v = st.d8 * (float)s;
            const uint32_t hb = bf16_bits(v);
            sm.aj[t][j] = (uint16_t)hb;
            sm.aj[t][8 + j] = (uint16_t)bf16_bits(v - bf16_val(hb));
        }
        if (hh == 0) sm.d8[t] = st.d8;
    }
}

__global__ __launch_bounds__(256) void prefill_q4k_kernel(const uint8_t* __restrict__ w, int64_t rows, int nb,
                                                          const int8_t* __restrict__ qs, const float* __restrict__ d8,
                                                          const int16_t* __restrict__ bs, int64_t K, int64_t M,
                                                          float* __restrict__ y) {
    __shared__ __attribute__((aligned(16))) PrefillSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t ntn = (rows + PF_TN - 1) / PF_TN;
    const int64_t n0 = ((int64_t)blockIdx.x % ntn) * PF_TN;
    const int64_t m0 = ((int64_t)blockIdx.x / ntn) * PF_TM;
    const int th = wv & 1, rh = wv >> 1;
    const int kg = lane >> 5;
    const int nl = 32 * rh + (lane & 31);  // this lane's weight row in the tile
    const int tl0 = 64 * th;               // first token of this wave

    v16f accf[2], accj[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) accf[t][r] = accj[t][r] = 0.0f;

    PrefillStage st;
    prefill_load(st, w, rows, nb, qs, d8, bs, K, M, n0, m0, 0, tid);
    for (int b = 0; b < nb; ++b) {
        __syncthreads();  // the previous block's LDS reads are done
        prefill_store(st, sm, tid);
        __syncthreads();
        if (b + 1 < nb) prefill_load(st, w, rows, nb, qs, d8, bs, K, M, n0, m0, b + 1, tid);

        // ---- main term: two int8 planes over the whole block
        v16i phi[2], plo[2];
        const int8_t* bh = sm.whi + nl * PF_LD + 16 * kg;
        const int8_t* bl = sm.wlo + nl * PF_LD + 16 * kg;
        const int8_t* ap0 = sm.xa + (tl0 + (lane & 31)) * PF_LD + 16 * kg;
        const int8_t* ap1 = ap0 + 32 * PF_LD;
        {
            const v4i vh = *reinterpret_cast<const v4i*>(bh);
            const v4i vl = *reinterpret_cast<const v4i*>(bl);
            const v4i a0 = *reinterpret_cast<const v4i*>(ap0);
            const v4i a1 = *reinterpret_cast<const v4i*>(ap1);
            const v16i z = {};
            phi[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, vh, z, 0, 0, 0);
            plo[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, vl, z, 0, 0, 0);
            phi[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, vh, z, 0, 0, 0);
            plo[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, vl, z, 0, 0, 0);
        }
#pragma unroll
        for (int j = 1; j < 8; ++j) {
            const v4i vh = *reinterpret_cast<const v4i*>(bh + 32 * j);
            const v4i vl = *reinterpret_cast<const v4i*>(bl + 32 * j);
            const v4i a0 = *reinterpret_cast<const v4i*>(ap0 + 32 * j);
            const v4i a1 = *reinterpret_cast<const v4i*>(ap1 + 32 * j);
            phi[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, vh, phi[0], 0, 0, 0);
            plo[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, vl, plo[0], 0, 0, 0);
            phi[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, vh, phi[1], 0, 0, 0);
            plo[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, vl, plo[1], 0, 0, 0);
        }
        // ---- min term: [ah | al] x [bh | bh] and [ah | al] x [bl | bl]
        {
            const v8bf bhv = *reinterpret_cast<const v8bf*>(&sm.bj[nl][0]);
            const v8bf blv = *reinterpret_cast<const v8bf*>(&sm.bj[nl][8]);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const v8bf av = *reinterpret_cast<const v8bf*>(&sm.aj[tl0 + 32 * t + (lane & 31)][8 * kg]);
                accj[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bhv, accj[t], 0, 0, 0);
                accj[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, blv, accj[t], 0, 0, 0);
            }
        }
        // ---- block epilogue: acc += (d8 * float(8 P_hi + P_lo)) * d
        const float dd = sm.dw[nl];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 d8v = *reinterpret_cast<const float4*>(&sm.d8[tl0 + 32 * t + 8 * g + 4 * kg]);
                const float d8a[4] = {d8v.x, d8v.y, d8v.z, d8v.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * g + i;
                    const float If = (float)((phi[t][r] << 3) + plo[t][r]);
                    accf[t][r] = fmaf(If * d8a[i], dd, accf[t][r]);
                }
            }
        }
    }
    const int64_t n = n0 + nl;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t m = m0 + tl0 + 32 * t + 8 * (r >> 2) + 4 * kg + (r & 3);
            if (m < M && n < rows) y[m * rows + n] = accf[t][r] - accj[t][r];
        }
    }
}

hipError_t launch_prefill_q4k(const uint8_t* w, int64_t rows, int nb, Acts a, int64_t M, float* y, hipStream_t s) {
    const int64_t tiles = ((rows + PF_TN - 1) / PF_TN) * ((M + PF_TM - 1) / PF_TM);
    hipLaunchKernelGGL(prefill_q4k_kernel, dim3((unsigned)tiles), dim3(256), 0, s, w, rows, nb, a.qs, a.d, a.bs, a.K,
                       M, y);
    return hipGetLastError();
}

}  // namespace q8k
