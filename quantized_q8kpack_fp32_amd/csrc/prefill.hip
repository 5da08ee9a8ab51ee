// Prefill GEMM: Q4_K weight [N rows][K] times M packed q8_K tokens on the
// gfx950 matrix cores.
//
// "Language models on the device: the cajeta-llm kernels", section 2.3: a
// workgroup computes a tile of tokens x weight rows; weight nibbles are
// widened into int8 beside the tokens' q8_K codes staged in shared memory
// ahead of the arithmetic, the waves multiply fragments on the matrix units,
// and the per-sub-block scales fold in through the accumulator epilogue (the
// scale/min epilogue of section 1).
//
// Per (token m, row n) the result is
//   y = sum_b d8_b * d_b * I_b  -  sum_b sum_j (d8_b * bsum_bj) * (dmin_b * m_bj)
// with I_b = sum_j sc_j * S_j the scale-weighted integer dot of block b.
//
// MI355X design.  The int8 matrix cores retire 32x more operations per clock
// than the vector ALUs, so the per-sub-block scale fold must not run on the
// vector ALUs.  It goes into the matrix-core operands instead: each 6-bit
// scale is split as sc = 8a + b (a, b in 0..7) and the weight fragment is
// built as two int8 planes a*q and b*q (each <= 105) in registers, four bytes
// per packed 16-bit multiply; two int8 MFMA passes over the block give P_hi,
// P_lo and I_b = 8 P_hi + P_lo exactly.  The min term is a GEMM over the
// (block, sub-block) axis whose operands already carry their block scales, so
// it accumulates in fp32 across all blocks on the bf16 matrix path: both
// operands are split into bf16 high and low parts and all four cross products
// are taken (two 32x32x16 bf16 MFMAs per block).  The vector ALUs keep the
// plane build and the block epilogue acc += (d8 * float(8 P_hi + P_lo)) * d.
//
// Tiles: a workgroup of 8 waves owns PF_TM tokens x PF_TN weight rows
// (PF_TM * PF_TN = 8192).  Waves 0..3 take the even blocks of K and waves 4..7
// the odd ones (each wave: 64 tokens as two 32-token MFMA tiles against 32
// weight rows), so every SIMD holds
// two waves whose matrix, vector and LDS work interleave; the two halves'
// accumulators are summed through LDS at the end, in a fixed order.  Each half
// stages its block's raw quant nibbles (128 B per row), the tokens' codes and
// the small scale/min operands in LDS; the next block's global loads are
// issued into registers before the current block's arithmetic.
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

#ifndef Q8K_PREFILL_TM
#define Q8K_PREFILL_TM 64
#endif
constexpr int PF_TM = Q8K_PREFILL_TM;  // tokens per workgroup (64, 128 or 256)
constexpr int PF_TN = 8192 / PF_TM;    // weight rows per workgroup
constexpr int PF_TG = PF_TM / 64;      // 64-token groups per half
constexpr int PF_RG = PF_TN / 32;      // 32-row groups per half (PF_TG * PF_RG = 4 waves)
constexpr int PF_LDQ = 128 + 16;       // LDS stride of a row's packed quants (bytes)
constexpr int PF_LDX = QK + 16;        // LDS stride of a token's codes (bytes)
static_assert(PF_TG * PF_RG == 4, "four waves per half");

struct PrefillHalf {
    uint8_t wq[PF_TN * PF_LDQ];  // raw Q4_K quant bytes of the block
    int8_t xa[PF_TM * PF_LDX];   // token codes of the block
    uint32_t sc[PF_TN][2];       // the row's eight 6-bit scales, one per byte
    float dw[PF_TN];             // row block scale d
    float d8[PF_TM];             // token block scale
    uint16_t bj[PF_TN][16];      // dmin*m_j as bf16: [0..7] high, [8..15] low
    uint16_t aj[PF_TM][16];      // d8*bsum_j as bf16: [0..7] high, [8..15] low
};
struct PrefillSmem {
    PrefillHalf h[2];
};

// Four byte-wise products q_i * k (q_i <= 15, k <= 7: every product stays
// inside its byte) as one packed 16-bit multiply.
__device__ __forceinline__ uint32_t mul_bytes(uint32_t q, uint32_t k) {
    const v2u16 kk = {(unsigned short)k, (unsigned short)k};
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2u16, q) * kk);
}

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

// One thread's share of a block's global data (256 threads per half):
// PF_TN rows x 128 quant bytes and PF_TM tokens x 256 codes.
constexpr int PF_QL = PF_TN / 32;  // 16-byte quant loads per thread
constexpr int PF_XL = PF_TM / 16;  // 16-byte code loads per thread
constexpr int PF_QT = 8 / PF_QL;   // threads per weight row
constexpr int PF_XT = 16 / PF_XL;  // threads per token
struct PrefillStage {
    uint4 q[PF_QL];  // weight row t/PF_QT: quant bytes 16*PF_QL*(t%PF_QT) ..
    uint4 x[PF_XL];  // token t/PF_XT: codes 16*PF_XL*(t%PF_XT) ..
    uint4 hdr;       // weight row t (t < PF_TN): block header
    uint4 bsv;       // token t (t < PF_TM): eight int16 sums
    float d8;        // token t (t < PF_TM)
};

__device__ __forceinline__ void prefill_load(PrefillStage& st, const uint8_t* __restrict__ w, int64_t rows, int nb,
                                             const int8_t* __restrict__ qs, const float* __restrict__ d8,
                                             const int16_t* __restrict__ bs, int64_t K, int64_t M, int64_t n0,
                                             int64_t m0, int b, int t) {
    {
        const int64_t n = n0 + t / PF_QT;
        if (b < nb && n < rows) {
            const uint8_t* src = w + (n * nb + b) * Q4K_BLOCK + 16 + 16 * PF_QL * (t % PF_QT);
#pragma unroll
            for (int i = 0; i < PF_QL; ++i) st.q[i] = *reinterpret_cast<const uint4*>(src + 16 * i);
        } else {
#pragma unroll
            for (int i = 0; i < PF_QL; ++i) st.q[i] = make_uint4(0, 0, 0, 0);
        }
    }
    {
        const int64_t m = m0 + t / PF_XT;
        if (b < nb && m < M) {
            const int8_t* src = qs + m * K + (int64_t)b * QK + 16 * PF_XL * (t % PF_XT);
#pragma unroll
            for (int i = 0; i < PF_XL; ++i) st.x[i] = *reinterpret_cast<const uint4*>(src + 16 * i);
        } else {
#pragma unroll
            for (int i = 0; i < PF_XL; ++i) st.x[i] = make_uint4(0, 0, 0, 0);
        }
    }
    st.hdr = make_uint4(0, 0, 0, 0);
    if (t < PF_TN) {
        const int64_t n = n0 + t;
        if (b < nb && n < rows) st.hdr = *reinterpret_cast<const uint4*>(w + (n * nb + b) * Q4K_BLOCK);
    }
    st.bsv = make_uint4(0, 0, 0, 0);
    st.d8 = 0.0f;
    if (t < PF_TM) {
        const int64_t m = m0 + t;
        if (b < nb && m < M) {
            st.bsv = *reinterpret_cast<const uint4*>(bs + (m * nb + b) * 8);
            st.d8 = d8[m * nb + b];
        }
    }
}

__device__ __forceinline__ void prefill_store(const PrefillStage& st, PrefillHalf& sm, int t) {
    {
        uint8_t* dst = sm.wq + (t / PF_QT) * PF_LDQ + 16 * PF_QL * (t % PF_QT);
#pragma unroll
        for (int i = 0; i < PF_QL; ++i) *reinterpret_cast<uint4*>(dst + 16 * i) = st.q[i];
    }
    {
        int8_t* dst = sm.xa + (t / PF_XT) * PF_LDX + 16 * PF_XL * (t % PF_XT);
#pragma unroll
        for (int i = 0; i < PF_XL; ++i) *reinterpret_cast<uint4*>(dst + 16 * i) = st.x[i];
    }
    if (t < PF_TN) {
        uint32_t scw[2] = {0, 0};
        const float dm = half_bits_to_float(st.hdr.x >> 16);
        uint32_t hb[8], lb[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            int sc, mn;
            q4k_scale_min(st.hdr, j, sc, mn);
            scw[j >> 2] |= (uint32_t)sc << (8 * (j & 3));
            const float v = dm * (float)mn;  // exact in fp32
            hb[j] = bf16_bits(v);
            lb[j] = bf16_bits(v - bf16_val(hb[j]));
        }
        sm.sc[t][0] = scw[0];
        sm.sc[t][1] = scw[1];
        sm.dw[t] = half_bits_to_float(st.hdr.x & 0xffffu);
        uint4* bjp = reinterpret_cast<uint4*>(&sm.bj[t][0]);
        bjp[0] = make_uint4(hb[0] | hb[1] << 16, hb[2] | hb[3] << 16, hb[4] | hb[5] << 16, hb[6] | hb[7] << 16);
        bjp[1] = make_uint4(lb[0] | lb[1] << 16, lb[2] | lb[3] << 16, lb[4] | lb[5] << 16, lb[6] | lb[7] << 16);
    }
    if (t < PF_TM) {
        const uint32_t bw[4] = {st.bsv.x, st.bsv.y, st.bsv.z, st.bsv.w};
        uint32_t hb[8], lb[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int s = (int)(int16_t)((j & 1) ? (bw[j >> 1] >> 16) : (bw[j >> 1] & 0xffffu));
            const float v = st.d8 * (float)s;
            hb[j] = bf16_bits(v);
            lb[j] = bf16_bits(v - bf16_val(hb[j]));
        }
        uint4* ajp = reinterpret_cast<uint4*>(&sm.aj[t][0]);
        ajp[0] = make_uint4(hb[0] | hb[1] << 16, hb[2] | hb[3] << 16, hb[4] | hb[5] << 16, hb[6] | hb[7] << 16);
        ajp[1] = make_uint4(lb[0] | lb[1] << 16, lb[2] | lb[3] << 16, lb[4] | lb[5] << 16, lb[6] | lb[7] << 16);
        sm.d8[t] = st.d8;
    }
}

// One wave's work on one staged block: tokens tg0..tg0+63 (2 MFMA tiles) x
// rows 32rw..32rw+31.
__device__ __forceinline__ void prefill_block(const PrefillHalf& sm, int lane, int rw, int tg0, v16f (&accf)[2],
                                              v16f (&accj)[2]) {
    const int kg = lane >> 5;
    const int nl = 32 * rw + (lane & 31);
    const uint32_t sc0 = sm.sc[nl][0], sc1 = sm.sc[nl][1];
    const uint8_t* qrow = sm.wq + nl * PF_LDQ + 16 * kg;
    const int8_t* x0 = sm.xa + (tg0 + (lane & 31)) * PF_LDX + 16 * kg;
    const int8_t* x1 = x0 + 32 * PF_LDX;
    v16i ph[2], pl[2];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        // quant bytes 32c + 16kg .. +15 of this row: low nibbles are sub-block
        // 2c, high nibbles sub-block 2c+1, at k = 16kg .. 16kg+15.
        const uint4 qv = *reinterpret_cast<const uint4*>(qrow + 32 * c);
        const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int j = 2 * c + h;
            const uint32_t s = ((j < 4 ? sc0 : sc1) >> (8 * (j & 3))) & 63u;
            const uint32_t ka = s >> 3, kb = s & 7u;
            uint32_t qq[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) qq[i] = h ? (qw[i] >> 4) & 0x0F0F0F0Fu : qw[i] & 0x0F0F0F0Fu;
            const v4i bh = {(int)mul_bytes(qq[0], ka), (int)mul_bytes(qq[1], ka), (int)mul_bytes(qq[2], ka),
                            (int)mul_bytes(qq[3], ka)};
            const v4i bl = {(int)mul_bytes(qq[0], kb), (int)mul_bytes(qq[1], kb), (int)mul_bytes(qq[2], kb),
                            (int)mul_bytes(qq[3], kb)};
            const v4i a0 = *reinterpret_cast<const v4i*>(x0 + 32 * j);
            const v4i a1 = *reinterpret_cast<const v4i*>(x1 + 32 * j);
            if (j == 0) {
                const v16i z = {};
                ph[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, bh, z, 0, 0, 0);
                pl[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, bl, z, 0, 0, 0);
                ph[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, bh, z, 0, 0, 0);
                pl[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, bl, z, 0, 0, 0);
            } else {
                ph[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, bh, ph[0], 0, 0, 0);
                pl[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, bl, pl[0], 0, 0, 0);
                ph[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, bh, ph[1], 0, 0, 0);
                pl[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, bl, pl[1], 0, 0, 0);
            }
        }
    }
    // min term: [ah | al] x [bh | bh] and [ah | al] x [bl | bl]
    {
        const v8bf bhv = *reinterpret_cast<const v8bf*>(&sm.bj[nl][0]);
        const v8bf blv = *reinterpret_cast<const v8bf*>(&sm.bj[nl][8]);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const v8bf av = *reinterpret_cast<const v8bf*>(&sm.aj[tg0 + 32 * t + (lane & 31)][8 * kg]);
            accj[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bhv, accj[t], 0, 0, 0);
            accj[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, blv, accj[t], 0, 0, 0);
        }
    }
    // block epilogue: acc += (d8 * float(8 P_hi + P_lo)) * d
    const float dd = sm.dw[nl];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 d8v = *reinterpret_cast<const float4*>(&sm.d8[tg0 + 32 * t + 8 * g + 4 * kg]);
            const float d8a[4] = {d8v.x, d8v.y, d8v.z, d8v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * g + i;
                const float If = (float)((ph[t][r] << 3) + pl[t][r]);
                accf[t][r] = fmaf(If * d8a[i], dd, accf[t][r]);
            }
        }
    }
}

__global__ __launch_bounds__(512) void prefill_q4k_kernel(const uint8_t* __restrict__ w, int64_t rows, int nb,
                                                          const int8_t* __restrict__ qs, const float* __restrict__ d8,
                                                          const int16_t* __restrict__ bs, int64_t K, int64_t M,
                                                          float* __restrict__ y) {
    __shared__ __attribute__((aligned(16))) PrefillSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int half = wv >> 2, t = tid & 255;
    const int rw = (wv & 3) % PF_RG, tg0 = 64 * ((wv & 3) / PF_RG);
    const int64_t ntn = (rows + PF_TN - 1) / PF_TN;
    const int64_t n0 = ((int64_t)blockIdx.x % ntn) * PF_TN;
    const int64_t m0 = ((int64_t)blockIdx.x / ntn) * PF_TM;

    v16f accf[2], accj[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) accf[i][r] = accj[i][r] = 0.0f;

    PrefillStage st;
    prefill_load(st, w, rows, nb, qs, d8, bs, K, M, n0, m0, half, t);
    for (int b0 = 0; b0 < nb; b0 += 2) {
        const int b = b0 + half;  // this half's block
        __syncthreads();          // the previous blocks' LDS reads are done
        prefill_store(st, sm.h[half], t);
        __syncthreads();
        if (b0 + 2 < nb) prefill_load(st, w, rows, nb, qs, d8, bs, K, M, n0, m0, b + 2, t);
        if (b < nb) prefill_block(sm.h[half], lane, rw, tg0, accf, accj);
    }
    // ---- sum the two halves in a fixed order: even blocks + odd blocks
    __syncthreads();
    float* red = reinterpret_cast<float*>(&sm);  // 4 waves x 64 lanes x 32 floats = 32 KB
    const int wq4 = wv & 3;
    if (half == 1) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) red[((wq4 * 32 + 16 * i + r) * 64) + lane] = accf[i][r] - accj[i][r];
    }
    __syncthreads();
    if (half == 0) {
        const int64_t n = n0 + 32 * rw + (lane & 31);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + tg0 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const float v = (accf[i][r] - accj[i][r]) + red[((wq4 * 32 + 16 * i + r) * 64) + lane];
                if (m < M && n < rows) y[m * rows + n] = v;
            }
        }
    }
}

hipError_t launch_prefill_q4k(const uint8_t* w, int64_t rows, int nb, Acts a, int64_t M, float* y, hipStream_t s) {
    const int64_t tiles = ((rows + PF_TN - 1) / PF_TN) * ((M + PF_TM - 1) / PF_TM);
    hipLaunchKernelGGL(prefill_q4k_kernel, dim3((unsigned)tiles), dim3(512), 0, s, w, rows, nb, a.qs, a.d, a.bs, a.K,
                       M, y);
    return hipGetLastError();
}

}  // namespace q8k
