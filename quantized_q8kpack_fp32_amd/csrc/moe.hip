// Mixture-of-experts decode: expert-indexed mat-vec with the weighted sum of
// each token's selected experts fused in.  These kernels serve K beyond the
// LDS token stage of the matrix-core kernels (moe_mfma.hip), which take every
// format below it.
//
// "Language models on the device: the cajeta-llm kernels", section 2.4: for a
// decode, every token's selected experts are visited in one launch and the
// experts' outputs are summed as they are produced; weights are read through
// the index of which expert each token chose (section intro).
//
// Q4_K and Q5_K (moe_rows_q4k_kernel<Q5>): one lane per weight row.  A workgroup owns 64
// consecutive rows of every expert; its MQ_WAVES waves take the experts
// w, w + MQ_WAVES, ... .  For expert e a wave collects the (token, slot) pairs
// that chose e with a ballot over ids and takes them MQ_G at a time.  Per
// block it loads the 64 rows' 144-byte (Q5_K: 176-byte) blocks with coalesced
// reads, passes
// them through its own LDS region so that lane r holds row r's block, and
// reads the group's q8_K codes from LDS as wave-uniform operands: one code
// read serves 64 rows, and a lane's sub-block sums, the scale/min fold and the
// block epilogue stay in that lane (no cross-lane reduction).  The dot of
// pair p and row r lands in an LDS slot owned by pair p; once every wave is
// done the workgroup adds each token's slots in slot order,
//   y[t][r] = sum_k rw[t][k] * dot(ids[t][k], t, r),
// so the order of the sum is fixed and no atomics or global workspace are
// used.  Tokens are taken in slabs of at most MQ_SLOT pairs.  An expert nobody
// chose is never read; an id outside [0, E) matches no expert and its slot is
// skipped.
//
// Q6_K (moe_chunk_kernel): one wave per MC_ROWS rows, lane l on 16-byte chunk
// l & 7 of a block, walking the experts in ascending order with the tokens'
// running sums in registers (token t in lane t % 64, slot t / 64).
#include "kquant.h"
#include "q8k.h"
#include "q8k_launch.h"

namespace q8k {

// ============================================================== Q4_K rows ====
constexpr int MQ_WAVES = 8;                            // waves per workgroup
constexpr int MQ_ROWS = 64;                            // rows per workgroup, one per lane
#ifndef Q8K_MOE_ROW_GROUP
#define Q8K_MOE_ROW_GROUP 8
#endif
constexpr int MQ_G = Q8K_MOE_ROW_GROUP;                // tokens per group
constexpr int MQ_SLOT = 128;                           // (token, slot) pairs per slab
// Block format: 16-byte pieces per row block (9 for Q4_K, 11 for Q5_K); the
// header is piece 0, Q5_K's qh pieces 1 and 2, the quants start at piece
// 1 (Q4_K) or 3 (Q5_K).
template <bool Q5>
struct MqFmt {
    static constexpr int BLK = Q5 ? Q5K_BLOCK : Q4K_BLOCK;
    static constexpr int PR = BLK / 16;
    static constexpr int QO = Q5 ? 3 : 1;
};
static_assert(MqFmt<false>::PR * 16 == Q4K_BLOCK && MqFmt<true>::PR * 16 == Q5K_BLOCK, "whole pieces");
static_assert(MQ_SLOT >= Q8K_MOE_MAX_TOPK, "a slab holds at least one token's pairs");

template <bool Q5>
struct MqWave {
    uint4 w[MQ_ROWS * MqFmt<Q5>::PR];  // one block of the 64 rows, row-major (row r at PR r)
    uint4 x[MQ_G * 16];                // the group's codes of that block, token g at 16g
    uint4 bs[MQ_G];                    // their eight int16 sub-block sums
    float d8[MQ_G];                    // their block scales
};
template <bool Q5>
struct MqSmem {
    MqWave<Q5> wave[MQ_WAVES];
    float slot[MQ_SLOT * MQ_ROWS];  // dot of (pair, row), pair-major
};
static_assert(sizeof(MqSmem<true>) <= 160 * 1024, "LDS of one workgroup");

// One block's worth of loads of a wave: piece 64i + lane of the 64 rows'
// block, 16 code bytes (token lane / 16, piece lane % 16), and the sums and
// scale of token lane % 4.
template <bool Q5>
struct MqStage {
    uint4 w[MqFmt<Q5>::PR];
    uint4 x[MQ_G / 4], bs;
    float d8;
};
static_assert(MQ_G == 4 || MQ_G == 8, "groups of 4 or 8 tokens");

template <bool Q5>
struct MqSrc {
    rsrc_t wr;                  // the 64 rows of expert e; reads past the last row give zeros
    int woff[MqFmt<Q5>::PR];    // byte offset of piece 64i + lane inside block 0
    const int8_t* x;            // codes of token tok[lane / 16], piece lane % 16, block 0
    const int8_t* x2;           // the same for token tok[lane / 16 + 4] (groups of 8)
    const int16_t* bs;          // sums of token tok[lane % 4], block 0
    const float* d8;            // scale of token tok[lane % 4], block 0
};

template <bool Q5>
__device__ __forceinline__ void mq_load(MqStage<Q5>& S, const MqSrc<Q5>& R, int b, int nb) {
#pragma unroll
    for (int i = 0; i < MqFmt<Q5>::PR; ++i) S.w[i] = load16(R.wr, R.woff[i] + b * MqFmt<Q5>::BLK);
    const int bc = b < nb ? b : nb - 1;  // steps past the end reload the last block (unused)
    S.x[0] = *reinterpret_cast<const uint4*>(R.x + (int64_t)bc * QK);
    if (MQ_G == 8) S.x[MQ_G / 4 - 1] = *reinterpret_cast<const uint4*>(R.x2 + (int64_t)bc * QK);
    S.bs = *reinterpret_cast<const uint4*>(R.bs + (int64_t)bc * 8);
    S.d8 = R.d8[bc];
}

// The wave hands data between its own lanes through LDS.  The hardware runs
// one wave's LDS instructions in order, but the compiler reasons per thread:
// it may forward a lane's earlier read past other lanes' writes, or hoist the
// writes above earlier reads.  The memory clobbers forbid both.
template <bool Q5>
__device__ __forceinline__ void mq_store(const MqStage<Q5>& S, MqWave<Q5>& L, int lane) {
    asm volatile("" ::: "memory");  // the previous block's reads come first
#pragma unroll
    for (int i = 0; i < MqFmt<Q5>::PR; ++i) L.w[64 * i + lane] = S.w[i];
    L.x[lane] = S.x[0];
    if (MQ_G == 8) L.x[64 + lane] = S.x[MQ_G / 4 - 1];
    if (lane < MQ_G) {
        L.bs[lane] = S.bs;
        L.d8[lane] = S.d8;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // visible to every lane before the reads
}

// Scale and min of sub-block j (compile-time) from the header's 12 bytes.
template <int j>
__device__ __forceinline__ void mq_scale_min(uint4 hdr, int& sc, int& mn) {
    constexpr int sh = 8 * (j & 3);
    const uint32_t yb = (hdr.y >> sh) & 0xffu, zb = (hdr.z >> sh) & 0xffu;
    if (j < 4) {
        sc = (int)(yb & 63);
        mn = (int)(zb & 63);
    } else {
        const uint32_t wb = (hdr.w >> sh) & 0xffu;
        sc = (int)((wb & 15) | ((yb >> 6) << 4));
        mn = (int)((wb >> 4) | ((zb >> 6) << 4));
    }
}

// sum over 32 values of sub-block (c, h) of row `lane` times token g's codes;
// Q5_K ORs bit j = 2c + h of each qh byte into bit 4 of the value (a rotate
// right by j - 4 puts it there in every byte of a word)
template <int c, int h, bool Q5>
__device__ __forceinline__ int mq_sub(const uint4 q0, const uint4 q1, const uint4 qh0, const uint4 qh1,
                                      const MqWave<Q5>& L, int g) {
    constexpr int j = 2 * c + h;
    constexpr int rot = (j + 28) & 31;
    const uint4 c0 = L.x[16 * g + 2 * j], c1 = L.x[16 * g + 2 * j + 1];
    auto val = [](uint32_t q, uint32_t qh) {
        uint32_t v = (h ? q >> 4 : q) & 0x0F0F0F0Fu;
        if (Q5) v |= __builtin_rotateright32(qh, rot) & 0x10101010u;
        return (int)v;
    };
    int s = sdot4(val(q0.x, qh0.x), (int)c0.x, 0);
    s = sdot4(val(q0.y, qh0.y), (int)c0.y, s);
    s = sdot4(val(q0.z, qh0.z), (int)c0.z, s);
    s = sdot4(val(q0.w, qh0.w), (int)c0.w, s);
    s = sdot4(val(q1.x, qh1.x), (int)c1.x, s);
    s = sdot4(val(q1.y, qh1.y), (int)c1.y, s);
    s = sdot4(val(q1.z, qh1.z), (int)c1.z, s);
    s = sdot4(val(q1.w, qh1.w), (int)c1.w, s);
    return s;
}

template <int c, bool Q5>
__device__ __forceinline__ void mq_pair(const MqWave<Q5>& L, int lane, uint4 hdr, int ng, int (&I)[MQ_G]) {
    // quant bytes 32c..32c+31: low nibbles are sub-block 2c, high 2c+1
    constexpr int PR = MqFmt<Q5>::PR, QO = MqFmt<Q5>::QO;
    const uint4 q0 = L.w[PR * lane + QO + 2 * c], q1 = L.w[PR * lane + QO + 1 + 2 * c];
    uint4 qh0 = q0, qh1 = q1;  // unused for Q4_K
    if (Q5) {
        qh0 = L.w[PR * lane + 1];
        qh1 = L.w[PR * lane + 2];
    }
    int sc0, mn0, sc1, mn1;
    mq_scale_min<2 * c>(hdr, sc0, mn0);
    mq_scale_min<2 * c + 1>(hdr, sc1, mn1);
#pragma unroll
    for (int g = 0; g < MQ_G; ++g) {
        if (g < ng) {  // wave-uniform
            I[g] += sc0 * mq_sub<c, 0, Q5>(q0, q1, qh0, qh1, L, g);
            I[g] += sc1 * mq_sub<c, 1, Q5>(q0, q1, qh0, qh1, L, g);
        }
    }
}

// Block b of row `lane` against the group's tokens: for each token g,
//   acc[g] += d8_g * (d * sum_j sc_j S_gj - dmin * sum_j m_j bsum_gj).
template <bool Q5>
__device__ __forceinline__ void mq_compute(const MqWave<Q5>& L, int lane, int ng, float (&acc)[MQ_G]) {
    const uint4 hdr = L.w[MqFmt<Q5>::PR * lane];
    int I[MQ_G];
#pragma unroll
    for (int g = 0; g < MQ_G; ++g) I[g] = 0;
    mq_pair<0, Q5>(L, lane, hdr, ng, I);
    mq_pair<1, Q5>(L, lane, hdr, ng, I);
    mq_pair<2, Q5>(L, lane, hdr, ng, I);
    mq_pair<3, Q5>(L, lane, hdr, ng, I);
    const float d = half_bits_to_float(hdr.x & 0xffffu);
    const float dmin = half_bits_to_float(hdr.x >> 16);
    // mins packed as int16 pairs (m0|m1, m2|m3, ...) against the sums' pairs
    int mn[8], sc_unused;
    mq_scale_min<0>(hdr, sc_unused, mn[0]);
    mq_scale_min<1>(hdr, sc_unused, mn[1]);
    mq_scale_min<2>(hdr, sc_unused, mn[2]);
    mq_scale_min<3>(hdr, sc_unused, mn[3]);
    mq_scale_min<4>(hdr, sc_unused, mn[4]);
    mq_scale_min<5>(hdr, sc_unused, mn[5]);
    mq_scale_min<6>(hdr, sc_unused, mn[6]);
    mq_scale_min<7>(hdr, sc_unused, mn[7]);
    typedef short v2s __attribute__((ext_vector_type(2)));
    v2s mp[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) mp[k] = __builtin_bit_cast(v2s, (uint32_t)mn[2 * k] | ((uint32_t)mn[2 * k + 1] << 16));
#pragma unroll
    for (int g = 0; g < MQ_G; ++g) {
        if (g < ng) {
            const uint4 bv = L.bs[g];
            int J = __builtin_amdgcn_sdot2(mp[0], __builtin_bit_cast(v2s, bv.x), 0, false);
            J = __builtin_amdgcn_sdot2(mp[1], __builtin_bit_cast(v2s, bv.y), J, false);
            J = __builtin_amdgcn_sdot2(mp[2], __builtin_bit_cast(v2s, bv.z), J, false);
            J = __builtin_amdgcn_sdot2(mp[3], __builtin_bit_cast(v2s, bv.w), J, false);
            acc[g] += L.d8[g] * (d * (float)I[g] - dmin * (float)J);
        }
    }
}

template <bool Q5>
__global__ __launch_bounds__(64 * MQ_WAVES) void moe_rows_q4k_kernel(
    const uint8_t* __restrict__ w, int64_t E, int64_t rows, int nb, const int8_t* __restrict__ qs,
    const float* __restrict__ d8, const int16_t* __restrict__ bs, int64_t K, int64_t T,
    const int32_t* __restrict__ ids, const float* __restrict__ rw, int topk, float* __restrict__ y) {
    constexpr int PR = MqFmt<Q5>::PR;
    __shared__ MqSmem<Q5> sm;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform, so e and rsrc are scalar
    const int lane = threadIdx.x & 63;
    const int64_t r0 = (int64_t)blockIdx.x * MQ_ROWS;
    const int64_t wrow = (int64_t)nb * MqFmt<Q5>::BLK;
    const int64_t live = rows - r0 < MQ_ROWS ? rows - r0 : MQ_ROWS;  // rows of this workgroup
    MqWave<Q5>& L = sm.wave[wv];
    int woff[PR];
#pragma unroll
    for (int i = 0; i < PR; ++i) {
        const int piece = 64 * i + lane;  // row piece / PR, 16-byte piece piece % PR of the block
        woff[i] = (piece / PR) * (int)wrow + 16 * (piece % PR);
    }
    const int64_t ts = MQ_SLOT / topk > 0 ? MQ_SLOT / topk : 1;  // tokens per slab
    for (int64_t t0 = 0; t0 < T; t0 += ts) {
        const int64_t t1 = t0 + ts < T ? t0 + ts : T;
        const int64_t pb = t0 * topk, pe = t1 * topk;
        for (int64_t e = wv; e < E; e += MQ_WAVES) {
            for (int64_t p0 = pb; p0 < pe; p0 += 64) {
                const int64_t p = p0 + lane;
                uint64_t mask = __ballot(p < pe && ids[p] == (int32_t)e);
                while (mask) {
                    // ---- next group of up to MQ_G pairs (wave-uniform); slot 0
                    // is always filled, empty slots repeat its token
                    int pidx[MQ_G], tok[MQ_G];
                    int ng = 0;
#pragma unroll
                    for (int g = 0; g < MQ_G; ++g) {
                        if (mask) {
                            pidx[g] = (int)p0 + __builtin_ctzll(mask);
                            mask &= mask - 1;
                            tok[g] = pidx[g] / topk;
                            ng = g + 1;
                        } else {
                            pidx[g] = pidx[0];
                            tok[g] = tok[0];
                        }
                    }
                    MqSrc<Q5> R;
                    R.wr = make_rsrc(w + (e * rows + r0) * wrow, live * wrow);
#pragma unroll
                    for (int i = 0; i < PR; ++i) R.woff[i] = woff[i];
                    {
                        // codes: piece lane % 16 of token lane / 16 (and of token
                        // lane / 16 + 4 for the second half of a group of 8);
                        // sums and scale: token lane % MQ_G
                        int tx = tok[0], tx2 = tok[0], tb = tok[0];
#pragma unroll
                        for (int g = 1; g < MQ_G; ++g) {
                            if ((lane >> 4) == g) tx = tok[g];
                            if ((lane >> 4) + 4 == g) tx2 = tok[g];
                            if ((lane % MQ_G) == g) tb = tok[g];
                        }
                        R.x = qs + (int64_t)tx * K + 16 * (lane & 15);
                        R.x2 = qs + (int64_t)tx2 * K + 16 * (lane & 15);
                        R.bs = bs + (int64_t)tb * nb * 8;
                        R.d8 = d8 + (int64_t)tb * nb;
                    }
                    float acc[MQ_G];
#pragma unroll
                    for (int g = 0; g < MQ_G; ++g) acc[g] = 0.0f;
                    // ---- blocks, two in flight: A holds even, B odd blocks
                    MqStage<Q5> A, B;
                    mq_load(A, R, 0, nb);
                    mq_load(B, R, 1, nb);
                    for (int b = 0; b < nb; b += 2) {
                        mq_store(A, L, lane);
                        mq_compute(L, lane, ng, acc);
                        mq_load(A, R, b + 2, nb);
                        if (b + 1 >= nb) break;
                        mq_store(B, L, lane);
                        mq_compute(L, lane, ng, acc);
                        mq_load(B, R, b + 3, nb);
                    }
#pragma unroll
                    for (int g = 0; g < MQ_G; ++g)
                        if (g < ng) sm.slot[(pidx[g] - (int)pb) * MQ_ROWS + lane] = acc[g];
                }
            }
        }
        __syncthreads();
        // ---- each token's slots, added in slot order
        for (int idx = threadIdx.x; idx < (int)(t1 - t0) * MQ_ROWS; idx += 64 * MQ_WAVES) {
            const int64_t t = t0 + idx / MQ_ROWS;
            const int r = idx % MQ_ROWS;
            if (r < live) {
                float s = 0.0f;
                for (int k = 0; k < topk; ++k) {
                    const int64_t pp = t * topk + k;
                    const int32_t id = ids[pp];
                    if (id >= 0 && id < E) s += rw[pp] * sm.slot[(pp - pb) * MQ_ROWS + r];
                }
                y[t * rows + r0 + r] = s;
            }
        }
        __syncthreads();
    }
}

// ============================================================= Q6_K chunks ===
#ifndef Q8K_MOE_GROUP
#define Q8K_MOE_GROUP 4
#endif
#ifndef Q8K_MOE_ROWS
#define Q8K_MOE_ROWS 2
#endif
constexpr int MC_GROUP = Q8K_MOE_GROUP;
constexpr int MC_ROWS = Q8K_MOE_ROWS;
constexpr int MC_TSLOTS = 4;  // 4 * 64 = 256 tokens at most
static_assert(MC_TSLOTS * 64 >= Q8K_MOE_MAX_TOKENS, "token slots");

template <bool Q6>
__global__ __launch_bounds__(256) void moe_chunk_kernel(const uint8_t* __restrict__ w, const uint16_t* __restrict__ prefix,
                                                  int64_t E, int64_t rows, int nb, const int8_t* __restrict__ qs,
                                                  const float* __restrict__ d8, const int16_t* __restrict__ bs,
                                                  int64_t K, int64_t T, const int32_t* __restrict__ ids,
                                                  const float* __restrict__ rw, int topk, float* __restrict__ y) {
    const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * MC_ROWS;
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

    float yreg[MC_ROWS][MC_TSLOTS];
#pragma unroll
    for (int r = 0; r < MC_ROWS; ++r)
#pragma unroll
        for (int i = 0; i < MC_TSLOTS; ++i) yreg[r][i] = 0.0f;
    const int64_t P = T * topk;

    for (int64_t e = 0; e < E; ++e) {
        for (int64_t p0 = 0; p0 < P; p0 += 64) {
            const int64_t p = p0 + lane;
            const bool sel = p < P && ids[p] == (int32_t)e;
            uint64_t mask = __ballot(sel);
            while (mask) {
                // ---- next group of up to MC_GROUP pairs (wave-uniform)
                int tok[MC_GROUP];
                float gw[MC_GROUP];
                int ng = 0;
#pragma unroll
                for (int g = 0; g < MC_GROUP; ++g) {
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
                float acc[MC_ROWS][MC_GROUP];
#pragma unroll
                for (int r = 0; r < MC_ROWS; ++r)
#pragma unroll
                    for (int g = 0; g < MC_GROUP; ++g) acc[r][g] = 0.0f;

                for (int seg = 0; seg < nseg; ++seg) {
                    const int bq = seg * 8 + (lane >> 3);
                    const bool valid = bq < nb;
                    const int b = valid ? bq : nb - 1;
                    // ---- the group's codes for this segment
                    int4 alo[MC_GROUP], ahi[MC_GROUP];
                    uint32_t bsv[MC_GROUP];
                    float dv[MC_GROUP];
#pragma unroll
                    for (int g = 0; g < MC_GROUP; ++g) {
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
                    uint4 wa[MC_ROWS], wb[MC_ROWS], wc[MC_ROWS];
                    uint32_t wd[MC_ROWS];
#pragma unroll
                    for (int r = 0; r < MC_ROWS; ++r) {
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
                    for (int r = 0; r < MC_ROWS; ++r) {
                        if (!Q6) {
                            int sc0, sc1, m0, m1;
                            q4k_scales(wa[r], c, sc0, sc1, m0, m1);
                            const float dd = half_bits_to_float(wa[r].x & 0xffffu);
                            const float dm = half_bits_to_float(wa[r].x >> 16);
                            uint32_t lo[4], hi[4];
                            q4k_unpack(wb[r], lo, hi);
#pragma unroll
                            for (int g = 0; g < MC_GROUP; ++g) {
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
                            for (int g = 0; g < MC_GROUP; ++g) {
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
                for (int g = 0; g < MC_GROUP; ++g) {
                    if (g < ng) {
#pragma unroll
                        for (int r = 0; r < MC_ROWS; ++r) {
                            const float v = gw[g] * wave_sum_dpp(acc[r][g]);
#pragma unroll
                            for (int i = 0; i < MC_TSLOTS; ++i)
                                if ((tok[g] >> 6) == i && (tok[g] & 63) == lane) yreg[r][i] += v;
                        }
                    }
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < MC_ROWS; ++r) {
        if (row0 + r >= rows) break;
#pragma unroll
        for (int i = 0; i < MC_TSLOTS; ++i) {
            const int64_t t = (int64_t)i * 64 + lane;
            if (t < T) y[t * rows + row0 + r] = yreg[r][i];
        }
    }
}


hipError_t launch_moe_q4k(const uint8_t* w, int64_t E, int64_t rows, int nb, Acts a, int64_t T, const int32_t* ids,
                          const float* rw, int topk, float* y, hipStream_t s) {
    const unsigned grid = (unsigned)((rows + MQ_ROWS - 1) / MQ_ROWS);
    Q8K_LAUNCH(moe_rows_q4k_kernel<false>, dim3(grid), dim3(64 * MQ_WAVES), 0, s, w, E, rows, nb, a.qs, a.d, a.bs,
               a.K, T, ids, rw, topk, y);
    return hipGetLastError();
}

hipError_t launch_moe_q5k(const uint8_t* w, int64_t E, int64_t rows, int nb, Acts a, int64_t T, const int32_t* ids,
                          const float* rw, int topk, float* y, hipStream_t s) {
    const unsigned grid = (unsigned)((rows + MQ_ROWS - 1) / MQ_ROWS);
    Q8K_LAUNCH(moe_rows_q4k_kernel<true>, dim3(grid), dim3(64 * MQ_WAVES), 0, s, w, E, rows, nb, a.qs, a.d, a.bs,
               a.K, T, ids, rw, topk, y);
    return hipGetLastError();
}

hipError_t launch_moe_q6k(const uint16_t* prefix, const uint8_t* bodies, int64_t E, int64_t rows, int nb, Acts a,
                          int64_t T, const int32_t* ids, const float* rw, int topk, float* y, hipStream_t s) {
    const int64_t waves = (rows + MC_ROWS - 1) / MC_ROWS;
    const unsigned grid = (unsigned)((waves + 3) / 4);
    Q8K_LAUNCH(moe_chunk_kernel<true>, dim3(grid), dim3(256), 0, s, bodies, prefix, E, rows, nb, a.qs, a.d, a.bs,
               a.K, T, ids, rw, topk, y);
    return hipGetLastError();
}

}  // namespace q8k
