// Per-chunk K-quant arithmetic shared by the decode mat-vec, batched and
// MoE kernels (one wavefront per output row, lane l on 16-byte chunk l & 7 of
// block 8k + (l >> 3)).
#pragma once
#include "q8k_device.h"

namespace q8k {

// ---------------------------------------------------------------- Q4_K ----
// Q4_K block: fp16 d, fp16 dmin, 12 bytes of 6-bit scales/mins, 128 quant
// bytes; quant byte 32c+l holds value 64c+l (low nibble) and 64c+32+l (high).
// Chunk ci covers bytes 16ci..16ci+15, i.e. c = ci/2, l = 16(ci&1) + 0..15:
// 16 values of sub-block 2c and 16 values of sub-block 2c+1.

// Scales and mins of sub-blocks 2c and 2c+1 from the header's 12 bytes
// (hdr.y = bytes 0..3, hdr.z = 4..7, hdr.w = 8..11).  Sub-blocks 0..3 keep 6
// bits in bytes 0..3 (scale) and 4..7 (min); sub-blocks 4..7 keep their low
// nibbles in bytes 8..11 and their top two bits in the spare bits 6..7 of
// bytes 0..3 (scale) and 4..7 (min).
__device__ __forceinline__ void q4k_scales(uint4 hdr, int c, int& sc0, int& sc1, int& m0, int& m1) {
    const int k = 16 * (c & 1);
    const uint32_t y = hdr.y >> k, z = hdr.z >> k, w = hdr.w >> k;
    if (c < 2) {
        sc0 = y & 63;
        sc1 = (y >> 8) & 63;
        m0 = z & 63;
        m1 = (z >> 8) & 63;
    } else {
        sc0 = (w & 15) | ((y >> 2) & 0x30);
        sc1 = ((w >> 8) & 15) | ((y >> 10) & 0x30);
        m0 = ((w >> 4) & 15) | ((z >> 2) & 0x30);
        m1 = ((w >> 12) & 15) | ((z >> 10) & 0x30);
    }
}

// Exact half sub-block sums of one chunk: S0 over the 16 low nibbles (against
// codes alo), S1 over the 16 high nibbles (against codes ahi).
__device__ __forceinline__ void q4k_chunk_sums(const uint32_t lo[4], const uint32_t hi[4], int4 alo, int4 ahi, int& S0,
                                               int& S1) {
    S0 = sdot4((int)lo[0], alo.x, 0);
    S0 = sdot4((int)lo[1], alo.y, S0);
    S0 = sdot4((int)lo[2], alo.z, S0);
    S0 = sdot4((int)lo[3], alo.w, S0);
    S1 = sdot4((int)hi[0], ahi.x, 0);
    S1 = sdot4((int)hi[1], ahi.y, S1);
    S1 = sdot4((int)hi[2], ahi.z, S1);
    S1 = sdot4((int)hi[3], ahi.w, S1);
}

__device__ __forceinline__ void q4k_unpack(uint4 qv, uint32_t lo[4], uint32_t hi[4]) {
    lo[0] = qv.x & 0x0F0F0F0Fu;
    lo[1] = qv.y & 0x0F0F0F0Fu;
    lo[2] = qv.z & 0x0F0F0F0Fu;
    lo[3] = qv.w & 0x0F0F0F0Fu;
    hi[0] = (qv.x >> 4) & 0x0F0F0F0Fu;
    hi[1] = (qv.y >> 4) & 0x0F0F0F0Fu;
    hi[2] = (qv.z >> 4) & 0x0F0F0F0Fu;
    hi[3] = (qv.w >> 4) & 0x0F0F0F0Fu;
}

// Q5_K: the same fields and quant packing as Q4_K (quants at byte 48), plus
// qh[32] at byte 16: bit j of qh[l] is bit 4 of value l of sub-block j.  For
// the chunk of quant bytes 32c + 16h .. +15 (qh bytes 16h .. +15), bit 2c of
// each qh byte goes to bit 4 of the low-nibble value and bit 2c + 1 to bit 4
// of the high-nibble value: one rotate and one masked OR per word, so the
// 5-bit quants (0..31) stay byte-wise for sdot4.
__device__ __forceinline__ void q5k_fifth_bits(uint4 qhv, int c, uint32_t lo[4], uint32_t hi[4]) {
    const uint32_t h[4] = {qhv.x, qhv.y, qhv.z, qhv.w};
    const int rl = (2 * c + 28) & 31, rh = (2 * c + 29) & 31;  // rotate right by 2c - 4 and 2c - 3
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lo[i] |= __builtin_rotateright32(h[i], rl) & 0x10101010u;
        hi[i] |= __builtin_rotateright32(h[i], rh) & 0x10101010u;
    }
}

// ---------------------------------------------------------------- Q6_K ----
// Relaid Q6_K: fp16 d in the prefix, body = ql[128] | qh[64] | int8 scales[16].
// Value v = 128h + 32t + l: low 4 bits in ql[64h + 32(t&1) + l] (nibble t>>1),
// high 2 bits in qh[32h + l] (bits 2t, 2t+1); value q - 32; sub-block v/16.
// Chunk ci of ql: h = ci>>2, tt = (ci>>1)&1, l = 16(ci&1) + 0..15; its low
// nibbles are t = tt (sub-block 8h+2tt+(ci&1)), its high nibbles t = tt+2
// (that sub-block + 4); the matching qh bytes are qh chunk 2h + (ci&1).

__device__ __forceinline__ void q6k_unpack(uint4 qlv, uint4 qhv, int tt, uint32_t lo[4], uint32_t hi[4]) {
    const int sh = 2 * tt;
    const uint32_t ql[4] = {qlv.x, qlv.y, qlv.z, qlv.w};
    const uint32_t qh[4] = {qhv.x, qhv.y, qhv.z, qhv.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        lo[k] = (ql[k] & 0x0F0F0F0Fu) | (((qh[k] >> sh) & 0x03030303u) << 4);
        hi[k] = ((ql[k] >> 4) & 0x0F0F0F0Fu) | (((qh[k] >> (sh + 4)) & 0x03030303u) << 4);
    }
}

// sum (q - 32) * code over 16 values: q*code plus (-32)*code, both by sdot4.
__device__ __forceinline__ int q6k_sum16(const uint32_t q[4], int4 a) {
    const int m32 = (int)0xE0E0E0E0u;  // four int8 -32
    int s = sdot4((int)q[0], a.x, 0);
    s = sdot4((int)q[1], a.y, s);
    s = sdot4((int)q[2], a.z, s);
    s = sdot4((int)q[3], a.w, s);
    s = sdot4(m32, a.x, s);
    s = sdot4(m32, a.y, s);
    s = sdot4(m32, a.z, s);
    s = sdot4(m32, a.w, s);
    return s;
}

}  // namespace q8k
