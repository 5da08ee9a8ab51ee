// Q4_K weight blocks as int8 matrix-core operands (gfx950, wave64), shared by
// the prefill tile and the mixture-of-experts decode.
//
// "Language models on the device: the cajeta-llm kernels", section 2.3 (weight
// nibbles widened to int8 for the matrix units) and section 1 (the per-sub-block
// scale and min epilogue).  Each 6-bit scale is split sc = 8a + b and the
// weight enters the int8 MFMA as two planes a*q and b*q (each <= 105), so the
// scale-weighted integer dot of a block is I = 8 P_hi + P_lo exactly.
//
// Lane map of the 32x32x32 int8 MFMA (verified on gfx950): A takes row l % 32
// from lane l, B column l % 32, and k-group g = l / 32 holds 16 of the 32 k;
// result (i, j) is in lane j + 32 ((i / 4) % 2), register (i % 4) + 4 (i / 8).
// The k order inside a 256-value block is free as long as both operands follow
// it: the weight lane (j, g) owns quant bytes 64g .. 64g+63 of row j's block
// (the values of sub-blocks 4g .. 4g+3), and k-step kk (0..7) takes the low (kk
// even) or high (kk odd) nibbles of its quant dwords 4(kk/2) .. 4(kk/2)+3:
// values 64(2g + kk/4) + 32(kk%2) + 16((kk/2)%2) + 0..15, all in sub-block
// 4g + 2(kk/4) + kk%2.  The other operand's lane (i, g) supplies the 16
// contiguous q8_K code bytes of those values (kstep_off).
#pragma once
#include "q8k_device.h"

namespace q8k {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

// Four byte-wise products q_i * k (q_i <= 15, k <= 7: every product stays
// inside its byte) as one packed 16-bit multiply.
__device__ __forceinline__ uint32_t mul_bytes(uint32_t q, uint32_t k) {
    const v2u16 kk = {(unsigned short)k, (unsigned short)k};
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2u16, q) * kk);
}

// bf16 high and low parts of v (round to nearest even both times): v - hi is
// exact in fp32, so hi + lo carries 16 significant bits of v.
__device__ __forceinline__ void bf16_split(float v, __bf16& hi, __bf16& lo) {
    hi = (__bf16)v;
    lo = (__bf16)(v - (float)hi);
}

// Byte offset inside a 256-value block of the 16 codes lane (i, g) supplies at
// k-step kk: values 64(2g + kk/4) + 32(kk%2) + 16((kk/2)%2) .. +15.
__host__ __device__ constexpr int kstep_off(int g, int kk) {
    return 128 * g + 64 * (kk >> 2) + 32 * (kk & 1) + 16 * ((kk >> 1) & 1);
}

// Raw bytes of one (row, block) for weight lane (j, g): the 16-byte header (d,
// dmin, 12 scale bytes) and quant bytes 64g .. 64g+63.
struct Q4kRaw {
    uint4 hdr, q[4];
};

// The operands of one (row, block) for weight lane (j, g), built from its raw
// bytes: the two planes of the 8 k-steps, the row's min-term operands
// (-dmin * m_j for sub-blocks 4g .. 4g+3, high and low bf16 parts, each
// repeated in both halves of the 8-element fragment) and the row's d.
struct Q4kPlanes {
    v4i ph[8], pl[8];
    v8bf bh, bl;
    float dd;
};
__device__ __forceinline__ void build_q4k_planes(Q4kPlanes& P, const Q4kRaw& R, int lane) {
    const int g = lane >> 5;
    // ---- scales and mins of sub-blocks 4g .. 4g+3 as bytes
    const uint32_t y = R.hdr.y, z = R.hdr.z, wq = R.hdr.w;
    // (branch-free: g differs between the two halves of the wave)
    const uint32_t hm = 0u - (uint32_t)g;
    const uint32_t sc = (hm & ((wq & 0x0F0F0F0Fu) | ((y >> 2) & 0x30303030u))) | (~hm & y & 0x3F3F3F3Fu);
    const uint32_t mn = (hm & (((wq >> 4) & 0x0F0F0F0Fu) | ((z >> 2) & 0x30303030u))) | (~hm & z & 0x3F3F3F3Fu);
    const uint32_t av = (sc >> 3) & 0x07070707u, bvv = sc & 0x07070707u;
    P.dd = half_bits_to_float(R.hdr.x & 0xffffu);
    const float dmin = half_bits_to_float(R.hdr.x >> 16);
    // ---- row min-term operands: -dmin * m_j (exact in fp32), high / low bf16
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        __bf16 hi, lo;
        bf16_split(-dmin * (float)((mn >> (8 * e)) & 0xffu), hi, lo);
        P.bh[e] = P.bh[4 + e] = hi;
        P.bl[e] = P.bl[4 + e] = lo;
    }
    // ---- the two planes of the 8 k-steps
    const uint32_t raw[16] = {R.q[0].x, R.q[0].y, R.q[0].z, R.q[0].w, R.q[1].x, R.q[1].y, R.q[1].z, R.q[1].w,
                              R.q[2].x, R.q[2].y, R.q[2].z, R.q[2].w, R.q[3].x, R.q[3].y, R.q[3].z, R.q[3].w};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        const int e = 2 * (kk >> 2) + (kk & 1);
        const uint32_t ka = (av >> (8 * e)) & 0xffu, kb = (bvv >> (8 * e)) & 0xffu;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const uint32_t r = raw[4 * (kk >> 1) + x];
            const uint32_t nib = (kk & 1) ? ((r >> 4) & 0x0F0F0F0Fu) : (r & 0x0F0F0F0Fu);
            P.ph[kk][x] = (int)mul_bytes(nib, ka);
            P.pl[kk][x] = (int)mul_bytes(nib, kb);
        }
    }
}

}  // namespace q8k
