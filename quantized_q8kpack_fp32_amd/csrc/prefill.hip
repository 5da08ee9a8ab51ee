// Prefill GEMM: Q4_K weight [N rows][K] times M packed q8_K tokens on the
// gfx950 int8 matrix cores.
//
// "Language models on the device: the cajeta-llm kernels", section 2.3: a
// workgroup computes a tile of tokens x weight rows; weight nibbles are
// widened into an int8 tile in shared memory beside the tokens' q8_K codes,
// the waves multiply fragments on the matrix units, and the per-sub-block
// scales fold in through the accumulator epilogue.
//
// This kernel: workgroup tile 64 tokens x 64 weight rows, 4 waves, each wave
// one 32x32 output tile.  Per 256-value block the workgroup stages both
// operands into LDS (rows padded by 16 bytes), then per 32-value sub-block j a
// v_mfma_i32_32x32x32_i8 gives the exact int32 sums S_j for the wave's 32x32
// tile, folded as I += sc_j * S_j; after the block the min term
// J = sum_j m_j * bsums_j and the fp32 epilogue acc += d8 * (d * I - dmin * J)
// run on the vector ALUs.
//
// MFMA operand map (32x32x32 int8): lane l supplies row l % 32 of A and
// column l % 32 of B, 16 int8 each from the same k positions of its k-group
// l / 32; result element (i, j) is in lane j + 32 * ((i / 4) % 2), register
// (i % 4) + 4 * (i / 8).  A = tokens, B = weight rows, so every lane holds one
// weight row (its sub-block scales are lane-uniform).
#include "q8k_device.h"
#include "q8k_launch.h"

namespace q8k {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int PF_TM = 64;           // tokens per workgroup
constexpr int PF_TN = 64;           // weight rows per workgroup
constexpr int PF_LD = QK + 16;      // LDS row stride in bytes

__global__ __launch_bounds__(256) void prefill_q4k_kernel(const uint8_t* __restrict__ w, int64_t rows, int nb,
                                                          const int8_t* __restrict__ qs, const float* __restrict__ d8,
                                                          const int16_t* __restrict__ bs, int64_t K, int64_t M,
                                                          float* __restrict__ y) {
    __shared__ __attribute__((aligned(16))) int8_t a_lds[PF_TM * PF_LD];
    __shared__ __attribute__((aligned(16))) int8_t w_lds[PF_TN * PF_LD];
    __shared__ int sc_lds[PF_TN][8];
    __shared__ int mn_lds[PF_TN][8];
    __shared__ float dw_lds[PF_TN];
    __shared__ float dmw_lds[PF_TN];
    __shared__ float d8_lds[PF_TM];
    __shared__ int bs_lds[PF_TM][8];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    // 1-D grid: tile index -> (weight-row tile, token tile), row tiles fastest
    const int64_t ntn = (rows + PF_TN - 1) / PF_TN;
    const int64_t n0 = ((int64_t)blockIdx.x % ntn) * PF_TN;
    const int64_t m0 = ((int64_t)blockIdx.x / ntn) * PF_TM;
    const int mt = wv & 1, nt = wv >> 1;
    const int nl = nt * 32 + (lane & 31);  // this lane's weight row in the tile

    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

    for (int b = 0; b < nb; ++b) {
        // ---- stage weights: thread -> (row tid/4, quant bytes 32p..32p+31)
        {
            const int r = tid >> 2, p = tid & 3;
            const int64_t n = n0 + r;
            int8_t* dst = w_lds + r * PF_LD + 64 * p;
            uint4 lo0 = {0, 0, 0, 0}, lo1 = lo0, hi0 = lo0, hi1 = lo0;
            if (n < rows) {
                const uint8_t* blk = w + (n * nb + b) * Q4K_BLOCK;
                const uint4 q0 = *reinterpret_cast<const uint4*>(blk + 16 + 32 * p);
                const uint4 q1 = *reinterpret_cast<const uint4*>(blk + 16 + 32 * p + 16);
                const uint32_t M4 = 0x0F0F0F0Fu;
                lo0 = make_uint4(q0.x & M4, q0.y & M4, q0.z & M4, q0.w & M4);
                lo1 = make_uint4(q1.x & M4, q1.y & M4, q1.z & M4, q1.w & M4);
                hi0 = make_uint4((q0.x >> 4) & M4, (q0.y >> 4) & M4, (q0.z >> 4) & M4, (q0.w >> 4) & M4);
                hi1 = make_uint4((q1.x >> 4) & M4, (q1.y >> 4) & M4, (q1.z >> 4) & M4, (q1.w >> 4) & M4);
                if (p == 0) {
                    const uint4 hdr = *reinterpret_cast<const uint4*>(blk);
                    const uint32_t s[3] = {hdr.y, hdr.z, hdr.w};
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const uint32_t sj = (s[j >> 2] >> (8 * (j & 3))) & 0xffu;  // byte j
                        if (j < 4) {
                            sc_lds[r][j] = (int)(sj & 63);
                            mn_lds[r][j] = (int)((s[1] >> (8 * j)) & 63);
                        } else {
                            const uint32_t b8 = (s[2] >> (8 * (j - 4))) & 0xffu;      // byte j+4
                            const uint32_t bl = (s[0] >> (8 * (j - 4))) & 0xffu;      // byte j-4
                            sc_lds[r][j] = (int)((b8 & 15) | ((bl >> 6) << 4));
                            mn_lds[r][j] = (int)((b8 >> 4) | ((sj >> 6) << 4));
                        }
                    }
                    dw_lds[r] = half_bits_to_float(hdr.x & 0xffffu);
                    dmw_lds[r] = half_bits_to_float(hdr.x >> 16);
                }
            } else if (p == 0) {
#pragma unroll
                for (int j = 0; j < 8; ++j) sc_lds[r][j] = mn_lds[r][j] = 0;
                dw_lds[r] = 0.0f;
                dmw_lds[r] = 0.0f;
            }
            // quant byte 32p+l -> value 64p+l (low nibble), 64p+32+l (high)
            *reinterpret_cast<uint4*>(dst) = lo0;
            *reinterpret_cast<uint4*>(dst + 16) = lo1;
            *reinterpret_cast<uint4*>(dst + 32) = hi0;
            *reinterpret_cast<uint4*>(dst + 48) = hi1;
        }
        // ---- stage tokens: thread -> (token tid/4, codes 64p..64p+63)
        {
            const int t = tid >> 2, p = tid & 3;
            const int64_t m = m0 + t;
            int8_t* dst = a_lds + t * PF_LD + 64 * p;
            uint4 v[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
            if (m < M) {
                const int8_t* src = qs + m * K + (int64_t)b * QK + 64 * p;
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = *reinterpret_cast<const uint4*>(src + 16 * i);
                if (p == 0) d8_lds[t] = d8[m * nb + b];
                if (p == 1) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) bs_lds[t][j] = bs[(m * nb + b) * 8 + j];
                }
            } else {
                if (p == 0) d8_lds[t] = 0.0f;
                if (p == 1) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) bs_lds[t][j] = 0;
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(dst + 16 * i) = v[i];
        }
        __syncthreads();

        // ---- integer sums per sub-block on the matrix cores, scale fold
        v16i I = {};
        const v16i zero = {};
        const int8_t* ap = a_lds + (mt * 32 + (lane & 31)) * PF_LD + 16 * (lane >> 5);
        const int8_t* bp = w_lds + nl * PF_LD + 16 * (lane >> 5);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const v4i av = *reinterpret_cast<const v4i*>(ap + 32 * j);
            const v4i bv = *reinterpret_cast<const v4i*>(bp + 32 * j);
            const v16i S = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, zero, 0, 0, 0);
            I += sc_lds[nl][j] * S;
        }
        // ---- min term and fp32 block epilogue
        const float dd = dw_lds[nl], dm = dmw_lds[nl];
        int mrow[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) mrow[j] = mn_lds[nl][j];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int tl = mt * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            int J = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) J += mrow[j] * bs_lds[tl][j];
            acc[r] += d8_lds[tl] * (dd * (float)I[r] - dm * (float)J);
        }
        __syncthreads();
    }
    const int64_t n = n0 + nl;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + mt * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < M && n < rows) y[m * rows + n] = acc[r];
    }
}

hipError_t launch_prefill_q4k(const uint8_t* w, int64_t rows, int nb, Acts a, int64_t M, float* y, hipStream_t s) {
    const int64_t tiles = ((rows + PF_TN - 1) / PF_TN) * ((M + PF_TM - 1) / PF_TM);
    hipLaunchKernelGGL(prefill_q4k_kernel, dim3((unsigned)tiles), dim3(256), 0, s, w, rows, nb, a.qs, a.d, a.bs, a.K,
                       M, y);
    return hipGetLastError();
}

}  // namespace q8k
