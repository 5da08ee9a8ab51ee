// Prefill GEMM: Q4_K weight [N rows][K] times M packed q8_K tokens on the
// gfx950 matrix cores.
//
// "Language models on the device: the cajeta-llm kernels", section 2.3: a
// workgroup computes a tile of tokens x weight rows; weight nibbles are
// widened into int8 in shared memory beside the tokens' q8_K codes, staged
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
// scale is split as sc = 8a + b (a, b in 0..7) and the weight is staged as
// two int8 planes a*q and b*q (each <= 105, four bytes per packed 16-bit
// multiply); two int8 MFMA passes over the block give P_hi, P_lo and
// I_b = 8 P_hi + P_lo exactly.  The min term is a GEMM over the (block,
// sub-block) axis whose operands already carry their block scales, so it
// accumulates in fp32 across all blocks on the bf16 matrix path: both
// operands are split into bf16 high and low parts and all four cross products
// are taken (two 32x32x16 bf16 MFMAs per block and tile).
//
// Work split (producer / consumer waves).  A workgroup of 8 waves owns 128
// tokens x 64 weight rows.  Waves 4..7 are producers: they keep the global
// loads two blocks ahead in registers (coalesced buffer loads, one instruction
// covering four tokens' 256 code bytes) and, per block, build the two weight
// planes, the min-term operands and the token codes into one of two LDS
// buffers.  Waves 0..3 are consumers: each multiplies 64 tokens (two 32-token
// MFMA tiles) against 32 weight rows from the other buffer and folds the block
// into its fp32 accumulators.  Every SIMD thus holds one wave of each kind, so
// the vector work of the producer overlaps the matrix work of the consumer;
// one barrier per block hands the buffers over.  The planes of a weight tile
// are built once per workgroup, i.e. once per 128 tokens.
//
// MFMA operand map (verified on gfx950): 32x32x32 int8 and 32x32x16 bf16 take
// row l % 32 of A and column l % 32 of B from lane l, k-group l / 32; result
// (i, j) is in lane j + 32 * ((i / 4) % 2), register (i % 4) + 4 * (i / 8).
// A = tokens, B = weight rows, so each consumer lane owns one weight row.
#include "q8k_device.h"
#include "q8k_launch.h"

namespace q8k {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

constexpr int PF_TM = 128;      // tokens per workgroup
constexpr int PF_TN = 64;       // weight rows per workgroup
constexpr int PF_LD = QK + 16;  // LDS row stride in bytes (bank spread)

struct PrefillBuf {
    int8_t whi[PF_TN * PF_LD];  // weight plane a*q
    int8_t wlo[PF_TN * PF_LD];  // weight plane b*q
    int8_t xa[PF_TM * PF_LD];   // token codes
    float dw[PF_TN];            // row block scale d
    float d8[PF_TM];            // token block scale
    uint16_t bj[PF_TN][16];     // dmin*m_j as bf16: [0..7] high, [8..15] low
    uint16_t aj[PF_TM][16];     // d8*bsum_j as bf16: [0..7] high, [8..15] low
};
struct PrefillSmem {
    PrefillBuf buf[2];
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

// Sub-block scale and min j (0..7) from the 12 packed bytes (hdr.y|z|w),
// without branches (j differs across the lanes of a wave).
__device__ __forceinline__ void q4k_scale_min(uint4 hdr, int j, int& sc, int& mn) {
    const int sh = 8 * (j & 3);
    const uint32_t yb = (hdr.y >> sh) & 0xffu, zb = (hdr.z >> sh) & 0xffu, wb = (hdr.w >> sh) & 0xffu;
    const uint32_t sc_lo = yb & 63, mn_lo = zb & 63;
    const uint32_t sc_hi = (wb & 15) | ((yb >> 6) << 4), mn_hi = (wb >> 4) | ((zb >> 6) << 4);
    sc = (int)(j < 4 ? sc_lo : sc_hi);
    mn = (int)(j < 4 ? mn_lo : mn_hi);
}

// Workgroup barrier for the LDS hand-over only.  __syncthreads() also
// orders global memory, which makes every wave wait for all of its
// outstanding global loads (the prefetches of later blocks) at each barrier;
// here only the LDS writes and reads before the barrier must be complete.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ------------------------------------------------------------ producers ----
// Global reads go through buffer resources whose range ends at the last row
// (token) of the problem: a read past it returns zeros and touches no memory,
// so the tails of the row and token tiles need no clamping and no branches.
// Lane offsets stay 32-bit: one workgroup's rows span at most
// 64 * (K / 256) * 144 bytes and its tokens 128 * K bytes, both < 2^31.
// Producer thread p (0..255), wave w = p / 64, lane l = p % 64, owns:
//  * weight row p/4, quant bytes 32(p&3)..+31 (values 64c..64c+63 with
//    c = p&3, i.e. sub-blocks 2c and 2c+1) and that row's header;
//  * 16 bytes of the codes of each of 8 tokens, 16i + 4w + l/16 for
//    i = 0..7, at byte 16(l&15) of the block: one load instruction of a wave
//    reads four tokens' 256 contiguous code bytes;
//  * sub-block sums 4h..4h+3 (h = p&1) and the block scale of token p/2.
struct PrefillRegs {
    uint4 hdr, q0, q1;
    uint4 x[8];
    uint2 bsv;
    float d8;
};

// Per-workgroup sources (wave-uniform) and per-thread byte offsets.  For
// block b the resources are rebased to block b (scalar arithmetic), so the
// range check "offset < records" is exactly "inside the problem".
struct PrefillSrc {
    const uint8_t* w;
    const int8_t* x;
    const int16_t* bs;
    const float* d8;
    int64_t wbytes, xbytes, bsbytes, d8bytes;  // bytes from the tile's first row/token to the end
    int wo, xo[8], bso, d8o;
};

__device__ __forceinline__ void producer_src(PrefillSrc& S, const uint8_t* __restrict__ w, int64_t rows, int nb,
                                             const int8_t* __restrict__ qs, const float* __restrict__ d8,
                                             const int16_t* __restrict__ bs, int64_t K, int64_t M, int64_t n0,
                                             int64_t m0, int p) {
    const int64_t wrow = (int64_t)nb * Q4K_BLOCK;
    S.w = w + n0 * wrow;
    S.x = qs + m0 * K;
    S.bs = bs + m0 * nb * 8;
    S.d8 = d8 + m0 * nb;
    S.wbytes = (rows - n0) * wrow;
    S.xbytes = (M - m0) * K;
    S.bsbytes = (M - m0) * nb * 16;
    S.d8bytes = (M - m0) * nb * 4;
    const int wv = p >> 6, l = p & 63;
    S.wo = (p >> 2) * (int)wrow;
#pragma unroll
    for (int i = 0; i < 8; ++i) S.xo[i] = (16 * i + 4 * wv + (l >> 4)) * (int)K + 16 * (l & 15);
    S.bso = (p >> 1) * nb * 16 + 8 * (p & 1);
    S.d8o = (p >> 1) * nb * 4;
}

// Mixture-of-experts form: the tile's 128 token rows are the tokens tok[0..127]
// (gathered from anywhere in the q8_K buffer of T tokens; tok < 0 marks an
// empty row).  An empty row's offsets point past every record, so its reads
// return zeros.  Offsets stay 32-bit: T * K < 2^30 is checked by the caller.
constexpr int PF_NONE = 0x7ffffff0;
__device__ __forceinline__ void producer_src_gather(PrefillSrc& S, const uint8_t* __restrict__ w, int64_t rows,
                                                    int nb, const int8_t* __restrict__ qs,
                                                    const float* __restrict__ d8, const int16_t* __restrict__ bs,
                                                    int64_t K, int64_t T, int64_t n0, const int* tok, int p) {
    const int64_t wrow = (int64_t)nb * Q4K_BLOCK;
    S.w = w + n0 * wrow;
    S.x = qs;
    S.bs = bs;
    S.d8 = d8;
    S.wbytes = (rows - n0) * wrow;
    S.xbytes = T * K;
    S.bsbytes = T * nb * 16;
    S.d8bytes = T * nb * 4;
    const int wv = p >> 6, l = p & 63;
    S.wo = (p >> 2) * (int)wrow;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int t = tok[16 * i + 4 * wv + (l >> 4)];
        S.xo[i] = t >= 0 ? t * (int)K + 16 * (l & 15) : PF_NONE;
    }
    const int tb = tok[p >> 1];
    S.bso = tb >= 0 ? tb * nb * 16 + 8 * (p & 1) : PF_NONE;
    S.d8o = tb >= 0 ? tb * nb * 4 : PF_NONE;
}

__device__ __forceinline__ void producer_load(PrefillRegs& R, const PrefillSrc& S, int b, int p) {
    const rsrc_t rw = make_rsrc(S.w + (int64_t)b * Q4K_BLOCK, S.wbytes - (int64_t)b * Q4K_BLOCK);
    const rsrc_t rx = make_rsrc(S.x + (int64_t)b * QK, S.xbytes - (int64_t)b * QK);
    const rsrc_t rb = make_rsrc(S.bs + (int64_t)b * 8, S.bsbytes - (int64_t)b * 16);
    const rsrc_t rd = make_rsrc(S.d8 + b, S.d8bytes - (int64_t)b * 4);
    const int wq = S.wo + 32 * (p & 3);
    R.hdr = load16(rw, S.wo);
    R.q0 = load16(rw, wq + 16);
    R.q1 = load16(rw, wq + 32);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        R.x[i] = load16(rx, S.xo[i]);
    R.bsv = load8(rb, S.bso);
    R.d8 = __builtin_bit_cast(float, load4(rd, S.d8o));
}

__device__ __forceinline__ void producer_store(const PrefillRegs& R, PrefillBuf& sm, int p) {
    // ---- weight planes and min-term operands of row p/4, sub-blocks 2c, 2c+1
    {
        const int r = p >> 2, c = p & 3;
        int sc0, mn0, sc1, mn1;
        q4k_scale_min(R.hdr, 2 * c, sc0, mn0);
        q4k_scale_min(R.hdr, 2 * c + 1, sc1, mn1);
        const uint32_t a0 = (uint32_t)(sc0 >> 3), b0 = (uint32_t)(sc0 & 7);
        const uint32_t a1 = (uint32_t)(sc1 >> 3), b1 = (uint32_t)(sc1 & 7);
        const uint32_t qw[8] = {R.q0.x, R.q0.y, R.q0.z, R.q0.w, R.q1.x, R.q1.y, R.q1.z, R.q1.w};
        uint32_t lh[8], ll[8], hh[8], hl[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t lo = qw[i] & 0x0F0F0F0Fu, hi = (qw[i] >> 4) & 0x0F0F0F0Fu;
            lh[i] = mul_bytes(lo, a0);
            ll[i] = mul_bytes(lo, b0);
            hh[i] = mul_bytes(hi, a1);
            hl[i] = mul_bytes(hi, b1);
        }
        // quant byte 32c+l -> value 64c+l (low nibble), 64c+32+l (high)
        int8_t* dh = sm.whi + r * PF_LD + 64 * c;
        int8_t* dl = sm.wlo + r * PF_LD + 64 * c;
        *reinterpret_cast<uint4*>(dh) = make_uint4(lh[0], lh[1], lh[2], lh[3]);
        *reinterpret_cast<uint4*>(dh + 16) = make_uint4(lh[4], lh[5], lh[6], lh[7]);
        *reinterpret_cast<uint4*>(dh + 32) = make_uint4(hh[0], hh[1], hh[2], hh[3]);
        *reinterpret_cast<uint4*>(dh + 48) = make_uint4(hh[4], hh[5], hh[6], hh[7]);
        *reinterpret_cast<uint4*>(dl) = make_uint4(ll[0], ll[1], ll[2], ll[3]);
        *reinterpret_cast<uint4*>(dl + 16) = make_uint4(ll[4], ll[5], ll[6], ll[7]);
        *reinterpret_cast<uint4*>(dl + 32) = make_uint4(hl[0], hl[1], hl[2], hl[3]);
        *reinterpret_cast<uint4*>(dl + 48) = make_uint4(hl[4], hl[5], hl[6], hl[7]);
        const float dm = half_bits_to_float(R.hdr.x >> 16);
        const float v0 = dm * (float)mn0, v1 = dm * (float)mn1;  // exact in fp32
        const uint32_t h0 = bf16_bits(v0), h1 = bf16_bits(v1);
        const uint32_t l0 = bf16_bits(v0 - bf16_val(h0)), l1 = bf16_bits(v1 - bf16_val(h1));
        *reinterpret_cast<uint32_t*>(&sm.bj[r][2 * c]) = h0 | (h1 << 16);
        *reinterpret_cast<uint32_t*>(&sm.bj[r][8 + 2 * c]) = l0 | (l1 << 16);
        if (c == 0) sm.dw[r] = half_bits_to_float(R.hdr.x & 0xffffu);
    }
    // ---- token codes
    {
        const int wv = p >> 6, l = p & 63;
        int8_t* dst = sm.xa + (4 * wv + (l >> 4)) * PF_LD + 16 * (l & 15);
#pragma unroll
        for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(dst + 16 * i * PF_LD) = R.x[i];
    }
    // ---- token min-term operand d8 * bsum_j (j = 4h..4h+3) and scale
    {
        const int t = p >> 1, h = p & 1;
        const uint32_t bw[2] = {R.bsv.x, R.bsv.y};
        uint32_t hb[4], lb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int s = (int)(int16_t)((j & 1) ? (bw[j >> 1] >> 16) : (bw[j >> 1] & 0xffffu));
            const float v = R.d8 * (float)s;
            hb[j] = bf16_bits(v);
            lb[j] = bf16_bits(v - bf16_val(hb[j]));
        }
        *reinterpret_cast<uint2*>(&sm.aj[t][4 * h]) = make_uint2(hb[0] | hb[1] << 16, hb[2] | hb[3] << 16);
        *reinterpret_cast<uint2*>(&sm.aj[t][8 + 4 * h]) = make_uint2(lb[0] | lb[1] << 16, lb[2] | lb[3] << 16);
        if (h == 0) sm.d8[t] = R.d8;
    }
}

// ------------------------------------------------------------ consumers ----
// Consumer wave: tokens tg0..tg0+63 (two MFMA tiles) x rows 32rg..32rg+31.
__device__ __forceinline__ void consumer_block(const PrefillBuf& sm, int lane, int rg, int tg0, v16f (&accf)[2],
                                               v16f (&accj)[2]) {
    const int kg = lane >> 5;
    const int nl = 32 * rg + (lane & 31);
    const int8_t* bh = sm.whi + nl * PF_LD + 16 * kg;
    const int8_t* bl = sm.wlo + nl * PF_LD + 16 * kg;
    const int8_t* a0p = sm.xa + (tg0 + (lane & 31)) * PF_LD + 16 * kg;
    const int8_t* a1p = a0p + 32 * PF_LD;
    v16i ph[2], pl[2];
    {
        const v4i vh = *reinterpret_cast<const v4i*>(bh);
        const v4i vl = *reinterpret_cast<const v4i*>(bl);
        const v4i a0 = *reinterpret_cast<const v4i*>(a0p);
        const v4i a1 = *reinterpret_cast<const v4i*>(a1p);
        const v16i z = {};
        ph[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, vh, z, 0, 0, 0);
        pl[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, vl, z, 0, 0, 0);
        ph[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, vh, z, 0, 0, 0);
        pl[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, vl, z, 0, 0, 0);
    }
#pragma unroll
    for (int j = 1; j < 8; ++j) {
        const v4i vh = *reinterpret_cast<const v4i*>(bh + 32 * j);
        const v4i vl = *reinterpret_cast<const v4i*>(bl + 32 * j);
        const v4i a0 = *reinterpret_cast<const v4i*>(a0p + 32 * j);
        const v4i a1 = *reinterpret_cast<const v4i*>(a1p + 32 * j);
        ph[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, vh, ph[0], 0, 0, 0);
        pl[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, vl, pl[0], 0, 0, 0);
        ph[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, vh, ph[1], 0, 0, 0);
        pl[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, vl, pl[1], 0, 0, 0);
    }
    // min term: [ah | al] x [bh | bh] and [ah | al] x [bl | bl]; k-group 0 of
    // the token operand carries the high parts, k-group 1 the low parts
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

// One 128-token x 64-row tile over all nb blocks.  The producers' sources are
// in S (built by the caller); consumer output row m of the tile goes to
// y[orow(m) * rows + n] when ok(m).
template <class ORow, class OK>
__device__ __forceinline__ void prefill_tile(PrefillSmem& sm, const PrefillSrc& S, int nb, int64_t rows, int64_t n0,
                                             float* __restrict__ y, ORow orow, OK ok) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    // Both roles run the same number of barriers: one before the first
    // block and one after each block (checked for every block count).
    if (wv >= 4) {
        // ---------------- producers: block b is built into buf[b & 1] during
        // iteration b - 1 (block 0 before the loop) from registers loaded two
        // iterations earlier; the two register sets alternate.
        const int p = tid - 256;
        PrefillRegs RA, RB;
        // The loads are unconditional: past the last block the resources
        // have no records, so the reads return zeros without touching memory.
        // Branch-free loads keep the compiler's wait counts exact, so that a
        // store waits only for its own register set, two blocks old.
        producer_load(RA, S, 0, p);
        producer_load(RB, S, 1, p);
        producer_store(RA, sm.buf[0], p);
        producer_load(RA, S, 2, p);
        lds_barrier();
        for (int b = 0; b < nb; b += 2) {
            // after block b is consumed: build block b+1 (RB), refill RB with b+3
            if (b + 1 < nb) producer_store(RB, sm.buf[1], p);
            producer_load(RB, S, b + 3, p);
            lds_barrier();
            if (b + 1 >= nb) break;
            // after block b+1 is consumed: build block b+2 (RA), refill RA with b+4
            if (b + 2 < nb) producer_store(RA, sm.buf[0], p);
            producer_load(RA, S, b + 4, p);
            lds_barrier();
        }
    } else {
        // ---------------- consumers
        const int rg = wv & 1, tg0 = 64 * (wv >> 1);
        v16f accf[2], accj[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) accf[i][r] = accj[i][r] = 0.0f;
        lds_barrier();
        for (int b = 0; b < nb; ++b) {
            consumer_block(sm.buf[b & 1], lane, rg, tg0, accf, accj);
            lds_barrier();
        }
        const int64_t n = n0 + 32 * rg + (lane & 31);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = tg0 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (ok(m) && n < rows) y[orow(m) * rows + n] = accf[i][r] - accj[i][r];
            }
        }
    }
}

__global__ __launch_bounds__(512) void prefill_q4k_kernel(const uint8_t* __restrict__ w, int64_t rows, int nb,
                                                          const int8_t* __restrict__ qs, const float* __restrict__ d8,
                                                          const int16_t* __restrict__ bs, int64_t K, int64_t M,
                                                          float* __restrict__ y) {
    __shared__ __attribute__((aligned(16))) PrefillSmem sm;
    const int64_t ntn = (rows + PF_TN - 1) / PF_TN;
    const int64_t n0 = ((int64_t)blockIdx.x % ntn) * PF_TN;
    const int64_t m0 = ((int64_t)blockIdx.x / ntn) * PF_TM;
    PrefillSrc S;
    if (threadIdx.x >= 256) producer_src(S, w, rows, nb, qs, d8, bs, K, M, n0, m0, (int)threadIdx.x - 256);
    prefill_tile(
        sm, S, nb, rows, n0, y, [&](int m) { return m0 + m; }, [&](int m) { return m0 + m < M; });
}

// ----------------------------------------------------- mixture of experts ----
// "Language models on the device", section 2.4: the prefill of an MoE layer
// groups each expert's (token, slot) pairs into chunks and runs the prefill
// tile per (expert, chunk), with a ragged last chunk.  Here workgroup
// (e, row tile) walks the pairs in ascending order, collects the next 128
// that chose expert e (a block-wide compaction of ids == e) and runs the
// tile on them; pair p's dot products go to row p of the per-pair output
// `out` [T * topk][rows].  A second kernel adds each token's pairs in slot
// order: y[t][r] = sum_k rw[t][k] * out[t * topk + k][r], skipping ids
// outside [0, E) (no workgroup writes those rows).
struct MoeLists {
    int tok[PF_TM];   // token of each tile row, -1 past the chunk's end
    int pair[PF_TM];  // pair index of each tile row
    int wcount[8];    // per-wave match counts of one 512-pair slab
    int count, pos;   // pairs collected, next pair to examine
};

// Collect the next up-to-128 pairs p >= L.pos with ids[p] == e, in ascending
// order.  Block-wide and barrier-synchronised; returns the count (uniform).
__device__ __forceinline__ int moe_collect(MoeLists& L, const int32_t* __restrict__ ids, int64_t P, int64_t e,
                                           int topk) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    if (tid == 0) L.count = 0;
    __syncthreads();
    for (;;) {
        const int count = L.count;
        const int64_t pos = L.pos;
        if (count >= PF_TM || pos >= P) break;  // uniform: read after a barrier
        const int64_t p = pos + tid;
        const bool m = p < P && ids[p] == (int32_t)e;
        const uint64_t ball = __ballot(m);
        const int below = __builtin_popcountll(ball & ((1ull << lane) - 1ull));
        if (lane == 0) L.wcount[wv] = __builtin_popcountll(ball);
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = L.wcount[i];
            before += i < wv ? c : 0;
            total += c;
        }
        const int idx = count + before + below;
        if (m && idx < PF_TM) {
            L.tok[idx] = (int)(p / topk);
            L.pair[idx] = (int)p;
        }
        __syncthreads();  // every thread has read count, pos and wcount
        if (count + total <= PF_TM) {
            if (tid == 0) {
                L.count = count + total;
                L.pos = pos + 512;
            }
        } else if (m && idx == PF_TM) {
            // the first pair that did not fit: the next chunk starts there
            L.count = PF_TM;
            L.pos = p;
        }
        __syncthreads();
    }
    const int count = L.count;
    for (int i = count + (int)threadIdx.x; i < PF_TM; i += 512) L.tok[i] = -1;
    __syncthreads();
    return count;
}

__global__ __launch_bounds__(512) void prefill_moe_q4k_kernel(const uint8_t* __restrict__ w, int64_t E, int64_t rows,
                                                              int nb, const int8_t* __restrict__ qs,
                                                              const float* __restrict__ d8,
                                                              const int16_t* __restrict__ bs, int64_t K, int64_t T,
                                                              const int32_t* __restrict__ ids, int topk,
                                                              float* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) PrefillSmem sm;
    __shared__ MoeLists L;
    const int64_t ntn = (rows + PF_TN - 1) / PF_TN;
    const int64_t e = (int64_t)blockIdx.x / ntn;
    const int64_t n0 = ((int64_t)blockIdx.x % ntn) * PF_TN;
    const uint8_t* we = w + e * rows * (int64_t)nb * Q4K_BLOCK;
    const int64_t P = T * topk;
    if (threadIdx.x == 0) L.pos = 0;
    for (;;) {
        const int count = moe_collect(L, ids, P, e, topk);
        if (count == 0) break;  // uniform
        PrefillSrc S;
        if (threadIdx.x >= 256)
            producer_src_gather(S, we, rows, nb, qs, d8, bs, K, T, n0, L.tok, (int)threadIdx.x - 256);
        prefill_tile(
            sm, S, nb, rows, n0, out, [&](int m) { return (int64_t)L.pair[m]; }, [&](int m) { return m < count; });
        __syncthreads();  // the lists are rebuilt next
    }
}

// y[t][r] = sum_k rw[t][k] * out[t * topk + k][r] over ids in [0, E), k ascending.
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ out, int64_t rows, int64_t T,
                                                          const int32_t* __restrict__ ids,
                                                          const float* __restrict__ rw, int topk, int64_t E,
                                                          float* __restrict__ y) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= T * rows) return;
    const int64_t t = i / rows, r = i % rows;
    float s = 0.0f;
    for (int k = 0; k < topk; ++k) {
        const int64_t pp = t * topk + k;
        const int32_t id = ids[pp];
        if (id >= 0 && id < E) s += rw[pp] * out[pp * rows + r];
    }
    y[i] = s;
}

hipError_t launch_prefill_moe_q4k(const uint8_t* w, int64_t E, int64_t rows, int nb, Acts a, int64_t T,
                                  const int32_t* ids, const float* rw, int topk, float* y, float* ws, hipStream_t s) {
    const int64_t ntn = (rows + PF_TN - 1) / PF_TN;
    hipLaunchKernelGGL(prefill_moe_q4k_kernel, dim3((unsigned)(E * ntn)), dim3(512), 0, s, w, E, rows, nb, a.qs, a.d,
                       a.bs, a.K, T, ids, topk, ws);
    const int64_t n = T * rows;
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ws, rows, T, ids, rw,
                       topk, E, y);
    return hipGetLastError();
}

hipError_t launch_prefill_q4k(const uint8_t* w, int64_t rows, int nb, Acts a, int64_t M, float* y, hipStream_t s) {
    const int64_t tiles = ((rows + PF_TN - 1) / PF_TN) * ((M + PF_TM - 1) / PF_TM);
    hipLaunchKernelGGL(prefill_q4k_kernel, dim3((unsigned)tiles), dim3(512), 0, s, w, rows, nb, a.qs, a.d, a.bs, a.K,
                       M, y);
    return hipGetLastError();
}

}  // namespace q8k
