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
// Q6_K (relaid: fp16 d in a prefix, 208-byte body).  The value weight is
// w = sc * (q - 32) with a signed 8-bit scale, an integer in [-4064, 4096]
// that no product of two int8 factors covers.  The producers compute w in
// 16-bit lanes (one packed multiply-add per two values) and stage its two
// base-128 digits as the planes: w1 = w >> 7 in [-32, 32] and w0 = w & 127,
// so I_b = 128 P_1 + P_0 exactly.  Q6_K has no min term.
//
// MFMA operand map (verified on gfx950): 32x32x32 int8 and 32x32x16 bf16 take
// row l % 32 of A and column l % 32 of B from lane l, k-group l / 32; result
// (i, j) is in lane j + 32 * ((i / 4) % 2), register (i % 4) + 4 * (i / 8).
// A = tokens, B = weight rows, so each consumer lane owns one weight row.
#include "q8k_device.h"
#include "q8k_launch.h"
#include "prefill_pack.h"

#include <mutex>

namespace q8k {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

constexpr int PF_TM = 128;      // tokens per workgroup
constexpr int PF_TN = 64;       // weight rows per workgroup
constexpr int PF_LD = QK + 16;  // LDS row stride in bytes (bank spread)

// Q5_K (a 5-bit quant q = l + 16h times a 6-bit scale does not split into
// two int8 factors): the nibble l takes the two planes a*l and b*l as in
// Q4_K, and the fifth bit h a third plane sc*h (<= 63), built by each
// consumer in registers from the row's qh bytes and scales staged beside the
// planes: I = 8 P_hi + P_lo + 16 P_h.
// Weight formats of the tile.
constexpr int PF_Q4 = WFMT_Q4_K, PF_Q5 = WFMT_Q5_K, PF_Q6 = WFMT_Q6_K;

template <int F>
struct PrefillQ5 {};
template <>
struct PrefillQ5<PF_Q5> {
    uint8_t qh[PF_TN][32];  // each row's fifth-bit plane (bit j of qh[l]: value l of sub-block j)
    uint8_t sc[PF_TN][8];   // each row's sub-block scales
};
template <int F>
struct PrefillMin {
    uint16_t bj[PF_TN][16];  // dmin*m_j as bf16: [0..7] high, [8..15] low
    uint16_t aj[PF_TM][16];  // d8*bsum_j as bf16: [0..7] high, [8..15] low
};
template <>
struct PrefillMin<PF_Q6> {};  // Q6_K has no min term

struct PrefillCore {
    int8_t whi[PF_TN * PF_LD];  // weight plane a*q (Q6_K: w >> 7)
    int8_t wlo[PF_TN * PF_LD];  // weight plane b*q (Q6_K: w & 127)
    int8_t xa[PF_TM * PF_LD];   // token codes
    float dw[PF_TN];            // row block scale d
    float d8[PF_TM];            // token block scale
};
// Bases are laid out in order: the planes and codes first, then the format's
// extra arrays.
template <int F>
struct PrefillBuf : PrefillCore, PrefillMin<F>, PrefillQ5<F> {};
template <int F>
struct PrefillSmem {
    PrefillBuf<F> buf[2];
};
// Bytes per (row, block) in the weight stream the tile reads (Q6_K: the body).
template <int F>
constexpr int kblock() { return F == PF_Q5 ? Q5K_BLOCK : F == PF_Q6 ? Q6K_BODY : Q4K_BLOCK; }

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
//  Q6_K: row p/4, quarter c = p&3 (h = c>>1, t = c&1): ql bytes
//    64h+32t..+31 (values 128h+32t+l and 128h+32t+64+l), qh bytes 32h..32h+31,
//    scale bytes 8h..8h+7 and the row's d; no sub-block sums (no min term).
struct PrefillRegs {
    uint4 hdr, q0, q1;
    uint2 qh;   // Q5_K: qh bytes 8c..8c+7 of the row; Q6_K: scale bytes 8h..8h+7
    uint4 qh2;  // Q6_K: qh bytes 32h+16..32h+31 (hdr holds 32h..32h+15)
    uint32_t dq;  // Q6_K: the row's fp16 d
    uint4 x[8];
    uint2 bsv;
    float d8;
};

// Per-workgroup sources (wave-uniform) and per-thread byte offsets.  For
// block b the resources are rebased to block b (scalar arithmetic), so the
// range check "offset < records" is exactly "inside the problem".
struct PrefillSrc {
    const uint8_t* w;
    const uint16_t* pf;  // Q6_K: the fp16 d prefix
    const int8_t* x;
    const int16_t* bs;
    const float* d8;
    int64_t wbytes, pfbytes, xbytes, bsbytes, d8bytes;  // bytes from the tile's first row/token to the end
    int wo, pfo, xo[8], bso, d8o;
};

template <int F>
__device__ __forceinline__ void producer_src_weights(PrefillSrc& S, const uint8_t* __restrict__ w,
                                                     const uint16_t* __restrict__ prefix, int64_t rows, int nb,
                                                     int64_t n0, int p) {
    const int64_t wrow = (int64_t)nb * kblock<F>();
    S.w = w + n0 * wrow;
    S.wbytes = (rows - n0) * wrow;
    S.wo = (p >> 2) * (int)wrow;
    if constexpr (F == PF_Q6) {
        S.pf = prefix + n0 * nb;
        S.pfbytes = (rows - n0) * nb * 2;
        S.pfo = (p >> 2) * nb * 2;
    }
}

template <int F>
__device__ __forceinline__ void producer_src(PrefillSrc& S, const uint8_t* __restrict__ w,
                                             const uint16_t* __restrict__ prefix, int64_t rows, int nb,
                                             const int8_t* __restrict__ qs, const float* __restrict__ d8,
                                             const int16_t* __restrict__ bs, int64_t K, int64_t M, int64_t n0,
                                             int64_t m0, int p) {
    producer_src_weights<F>(S, w, prefix, rows, nb, n0, p);
    S.x = qs + m0 * K;
    S.bs = bs + m0 * nb * 8;
    S.d8 = d8 + m0 * nb;
    S.xbytes = (M - m0) * K;
    S.bsbytes = (M - m0) * nb * 16;
    S.d8bytes = (M - m0) * nb * 4;
    const int wv = p >> 6, l = p & 63;
#pragma unroll
    for (int i = 0; i < 8; ++i) S.xo[i] = (16 * i + 4 * wv + (l >> 4)) * (int)K + 16 * (l & 15);
    S.bso = (p >> 1) * nb * 16 + 8 * (p & 1);
    S.d8o = (p >> 1) * nb * 4;
}

// Split-K: the sources start at block kb0 of every row and token (the strides
// between rows and tokens are unchanged), so the tile's block loop covers
// blocks kb0 .. of the problem.
template <int F>
__device__ __forceinline__ void producer_src_from_block(PrefillSrc& S, int kb0) {
    S.w += (int64_t)kb0 * kblock<F>();
    S.wbytes -= (int64_t)kb0 * kblock<F>();
    if constexpr (F == PF_Q6) {
        S.pf += kb0;
        S.pfbytes -= (int64_t)kb0 * 2;
    }
    S.x += (int64_t)kb0 * QK;
    S.xbytes -= (int64_t)kb0 * QK;
    S.bs += (int64_t)kb0 * 8;
    S.bsbytes -= (int64_t)kb0 * 16;
    S.d8 += kb0;
    S.d8bytes -= (int64_t)kb0 * 4;
}

// Mixture-of-experts form: the tile's 128 token rows are the tokens tok[0..127]
// (gathered from anywhere in the q8_K buffer of T tokens; tok < 0 marks an
// empty row).  An empty row's offsets point past every record, so its reads
// return zeros.  Offsets stay 32-bit: T * K < 2^30 is checked by the caller.
constexpr int PF_NONE = 0x7ffffff0;
template <int F>
__device__ __forceinline__ void producer_src_gather(PrefillSrc& S, const uint8_t* __restrict__ w,
                                                    const uint16_t* __restrict__ prefix, int64_t rows, int nb,
                                                    const int8_t* __restrict__ qs, const float* __restrict__ d8,
                                                    const int16_t* __restrict__ bs, int64_t K, int64_t T, int64_t n0,
                                                    const int* tok, int p) {
    producer_src_weights<F>(S, w, prefix, rows, nb, n0, p);
    S.x = qs;
    S.bs = bs;
    S.d8 = d8;
    S.xbytes = T * K;
    S.bsbytes = T * nb * 16;
    S.d8bytes = T * nb * 4;
    const int wv = p >> 6, l = p & 63;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int t = tok[16 * i + 4 * wv + (l >> 4)];
        S.xo[i] = t >= 0 ? t * (int)K + 16 * (l & 15) : PF_NONE;
    }
    const int tb = tok[p >> 1];
    S.bso = tb >= 0 ? tb * nb * 16 + 8 * (p & 1) : PF_NONE;
    S.d8o = tb >= 0 ? tb * nb * 4 : PF_NONE;
}

template <int F>
__device__ __forceinline__ void producer_load(PrefillRegs& R, const PrefillSrc& S, int b, int p) {
    constexpr bool Q5 = F == PF_Q5;
    const rsrc_t rw = make_rsrc(S.w + (int64_t)b * kblock<F>(), S.wbytes - (int64_t)b * kblock<F>());
    const rsrc_t rx = make_rsrc(S.x + (int64_t)b * QK, S.xbytes - (int64_t)b * QK);
    const rsrc_t rd = make_rsrc(S.d8 + b, S.d8bytes - (int64_t)b * 4);
    if constexpr (F == PF_Q6) {
        const rsrc_t rp = make_rsrc(S.pf + b, S.pfbytes - (int64_t)b * 2);
        const int c = p & 3, h = c >> 1;
        R.q0 = load16(rw, S.wo + 64 * h + 32 * (c & 1));
        R.q1 = load16(rw, S.wo + 64 * h + 32 * (c & 1) + 16);
        R.hdr = load16(rw, S.wo + 128 + 32 * h);
        R.qh2 = load16(rw, S.wo + 128 + 32 * h + 16);
        R.qh = load8(rw, S.wo + 192 + 8 * h);
        R.dq = load2(rp, S.pfo);
    } else {
        const int wq = S.wo + (Q5 ? 48 : 16) + 32 * (p & 3);
        R.hdr = load16(rw, S.wo);
        R.q0 = load16(rw, wq);
        R.q1 = load16(rw, wq + 16);
        if (Q5) R.qh = load8(rw, S.wo + 16 + 8 * (p & 3));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
        R.x[i] = load16(rx, S.xo[i]);
    if constexpr (F != PF_Q6) {
        const rsrc_t rb = make_rsrc(S.bs + (int64_t)b * 8, S.bsbytes - (int64_t)b * 16);
        R.bsv = load8(rb, S.bso);
    }
    R.d8 = __builtin_bit_cast(float, load4(rd, S.d8o));
}

// Q6_K: the two base-128 digit planes of w = sc * (q - 32) for four values
// q (bytes of q4, each 0..63) sharing one signed scale sc.  The values go to
// 16-bit lanes in pairs (bytes 0, 2 and bytes 1, 3), one packed multiply-add
// per pair forms w, and byte permutes put the four digits back in order.
__device__ __forceinline__ void q6k_digits(uint32_t q4, int sc, uint32_t& w1, uint32_t& w0) {
    const uint32_t qe = __builtin_amdgcn_perm(0u, q4, 0x0c020c00u);  // values 0, 2
    const uint32_t qo = __builtin_amdgcn_perm(0u, q4, 0x0c030c01u);  // values 1, 3
    const unsigned short s = (unsigned short)sc, o = (unsigned short)(-32 * sc);
    const v2u16 ss = {s, s}, oo = {o, o};
    const v2u16 we = __builtin_bit_cast(v2u16, qe) * ss + oo;
    const v2u16 wo = __builtin_bit_cast(v2u16, qo) * ss + oo;
    const v2u16 seven = {7, 7};
    const uint32_t he = __builtin_bit_cast(uint32_t, we >> seven), ho = __builtin_bit_cast(uint32_t, wo >> seven);
    // byte k of the result: value k's low byte (even values from `e`, odd from `o`)
    w1 = __builtin_amdgcn_perm(ho, he, 0x06020400u);
    w0 = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, wo), __builtin_bit_cast(uint32_t, we), 0x06020400u) &
         0x7F7F7F7Fu;
}

template <int F>
__device__ __forceinline__ void producer_store(const PrefillRegs& R, PrefillBuf<F>& sm, int p) {
    constexpr bool Q5 = F == PF_Q5;
    if constexpr (F == PF_Q6) {
        // ---- digit planes of row p/4: values 128h+32t+l (low nibbles, quarter
        // t, sub-blocks 8h+2t, 8h+2t+1) and 128h+32t+64+l (high nibbles,
        // quarter t+2, sub-blocks 8h+2t+4, 8h+2t+5), l = 0..31
        const int r = p >> 2, c = p & 3, h = c >> 1, t = c & 1;
        const uint32_t ql[8] = {R.q0.x, R.q0.y, R.q0.z, R.q0.w, R.q1.x, R.q1.y, R.q1.z, R.q1.w};
        const uint32_t qh[8] = {R.hdr.x, R.hdr.y, R.hdr.z, R.hdr.w, R.qh2.x, R.qh2.y, R.qh2.z, R.qh2.w};
        const int sh = 16 * t;  // scale bytes 2t, 2t+1 of each half of the 8 loaded
        const int s_lo0 = (int)(int8_t)(R.qh.x >> sh), s_lo1 = (int)(int8_t)(R.qh.x >> (sh + 8));
        const int s_hi0 = (int)(int8_t)(R.qh.y >> sh), s_hi1 = (int)(int8_t)(R.qh.y >> (sh + 8));
        uint32_t l1[8], l0[8], h1[8], h0[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t hb = qh[i] >> (2 * t);  // bits 2t, 2t+1 -> 0, 1; bits 2t+4, 2t+5 -> 4, 5
            const uint32_t qlo = (ql[i] & 0x0F0F0F0Fu) | ((hb << 4) & 0x30303030u);
            const uint32_t qhi = ((ql[i] >> 4) & 0x0F0F0F0Fu) | (hb & 0x30303030u);
            q6k_digits(qlo, i < 4 ? s_lo0 : s_lo1, l1[i], l0[i]);
            q6k_digits(qhi, i < 4 ? s_hi0 : s_hi1, h1[i], h0[i]);
        }
        int8_t* dh = sm.whi + r * PF_LD + 128 * h + 32 * t;
        int8_t* dl = sm.wlo + r * PF_LD + 128 * h + 32 * t;
        *reinterpret_cast<uint4*>(dh) = make_uint4(l1[0], l1[1], l1[2], l1[3]);
        *reinterpret_cast<uint4*>(dh + 16) = make_uint4(l1[4], l1[5], l1[6], l1[7]);
        *reinterpret_cast<uint4*>(dh + 64) = make_uint4(h1[0], h1[1], h1[2], h1[3]);
        *reinterpret_cast<uint4*>(dh + 80) = make_uint4(h1[4], h1[5], h1[6], h1[7]);
        *reinterpret_cast<uint4*>(dl) = make_uint4(l0[0], l0[1], l0[2], l0[3]);
        *reinterpret_cast<uint4*>(dl + 16) = make_uint4(l0[4], l0[5], l0[6], l0[7]);
        *reinterpret_cast<uint4*>(dl + 64) = make_uint4(h0[0], h0[1], h0[2], h0[3]);
        *reinterpret_cast<uint4*>(dl + 80) = make_uint4(h0[4], h0[5], h0[6], h0[7]);
        if (c == 0) sm.dw[r] = half_bits_to_float(R.dq & 0xffffu);
    } else {
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
        if constexpr (Q5) {
            *reinterpret_cast<uint2*>(&sm.qh[r][8 * c]) = R.qh;
            *reinterpret_cast<uint16_t*>(&sm.sc[r][2 * c]) = (uint16_t)(sc0 | (sc1 << 8));
        }
    }
    // ---- token codes
    {
        const int wv = p >> 6, l = p & 63;
        int8_t* dst = sm.xa + (4 * wv + (l >> 4)) * PF_LD + 16 * (l & 15);
#pragma unroll
        for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(dst + 16 * i * PF_LD) = R.x[i];
    }
    // ---- token min-term operand d8 * bsum_j (j = 4h..4h+3) and scale
    if constexpr (F == PF_Q6) {
        if ((p & 1) == 0) sm.d8[p >> 1] = R.d8;
    } else {
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
// Test support (SUMS): where the block sums I_b go, [M][rows][nb] from the
// tile's first token and row (int32).
struct PfSums {
    int32_t* I;
    int64_t rows, live, nrow;  // problem rows; tokens and rows of this tile still inside the problem
    int nb;
};

// Consumer wave: tokens tg0..tg0+63 (two MFMA tiles) x rows 32rg..32rg+31.
// SUMS: also store each (token, row)'s exact block sum I_b of block b to D.
template <int F, bool SUMS = false>
__device__ __forceinline__ void consumer_block(const PrefillBuf<F>& sm, int lane, int rg, int tg0, v16f (&accf)[2],
                                               v16f (&accj)[2], const PfSums& D = PfSums{}, int b = 0) {
    constexpr bool Q5 = F == PF_Q5;
    const int kg = lane >> 5;
    const int nl = 32 * rg + (lane & 31);
    const int8_t* bh = sm.whi + nl * PF_LD + 16 * kg;
    const int8_t* bl = sm.wlo + nl * PF_LD + 16 * kg;
    const int8_t* a0p = sm.xa + (tg0 + (lane & 31)) * PF_LD + 16 * kg;
    const int8_t* a1p = a0p + 32 * PF_LD;
    v16i ph[2], pl[2], pq[2];
    // Q5_K: this lane's 16 values of each sub-block are positions 16kg..16kg+15,
    // whose fifth bits are bit j of qh bytes 16kg..16kg+15
    // (read from LDS at each use: keeping them in registers would spill the
    // mixture-of-experts form)
    auto hplane = [&](int j) {
        v4i v = {0, 0, 0, 0};
        if constexpr (Q5) {
            const uint4 qhv = *reinterpret_cast<const uint4*>(&sm.qh[nl][16 * kg]);
            const uint32_t scj = sm.sc[nl][j];
            const uint32_t h[4] = {qhv.x, qhv.y, qhv.z, qhv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = (int)mul_bytes(__builtin_rotateright32(h[i], j) & 0x01010101u, scj);
        }
        return v;
    };
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
        if constexpr (Q5) {
            const v4i vq = hplane(0);
            pq[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, vq, z, 0, 0, 0);
            pq[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, vq, z, 0, 0, 0);
        }
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
        if constexpr (Q5) {
            const v4i vq = hplane(j);
            pq[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, vq, pq[0], 0, 0, 0);
            pq[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, vq, pq[1], 0, 0, 0);
        }
    }
    // min term: [ah | al] x [bh | bh] and [ah | al] x [bl | bl]; k-group 0 of
    // the token operand carries the high parts, k-group 1 the low parts
    if constexpr (F != PF_Q6) {
        const v8bf bhv = *reinterpret_cast<const v8bf*>(&sm.bj[nl][0]);
        const v8bf blv = *reinterpret_cast<const v8bf*>(&sm.bj[nl][8]);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const v8bf av = *reinterpret_cast<const v8bf*>(&sm.aj[tg0 + 32 * t + (lane & 31)][8 * kg]);
            accj[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bhv, accj[t], 0, 0, 0);
            accj[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, blv, accj[t], 0, 0, 0);
        }
    }
    // block epilogue: acc += (d8 * float(8 P_hi + P_lo (+ 16 P_h))) * d
    // (Q6_K: float(128 P_1 + P_0))
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
                const int I = (ph[t][r] << (F == PF_Q6 ? 7 : 3)) + pl[t][r];
                const int Ib = Q5 ? I + (pq[t][r] << 4) : I;
                if constexpr (SUMS) {
                    const int m = tg0 + 32 * t + 8 * g + 4 * kg + i;
                    if (m < D.live && nl < D.nrow) D.I[((int64_t)m * D.rows + nl) * D.nb + b] = Ib;
                }
                const float If = (float)Ib;
                accf[t][r] = fmaf(If * d8a[i], dd, accf[t][r]);
            }
        }
    }
}

// One 128-token x 64-row tile over all nb blocks.  The producers' sources are
// in S (built by the caller); consumer output row m of the tile goes to
// y[orow(m) * rows + n] when ok(m).
template <int F, bool SUMS = false, class ORow, class OK>
__device__ __forceinline__ void prefill_tile(PrefillSmem<F>& sm, const PrefillSrc& S, int nb, int64_t rows,
                                             int64_t n0, float* __restrict__ y, ORow orow, OK ok,
                                             const PfSums& D = PfSums{}) {
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
        producer_load<F>(RA, S, 0, p);
        producer_load<F>(RB, S, 1, p);
        producer_store<F>(RA, sm.buf[0], p);
        producer_load<F>(RA, S, 2, p);
        lds_barrier();
        for (int b = 0; b < nb; b += 2) {
            // after block b is consumed: build block b+1 (RB), refill RB with b+3
            if (b + 1 < nb) producer_store<F>(RB, sm.buf[1], p);
            producer_load<F>(RB, S, b + 3, p);
            lds_barrier();
            if (b + 1 >= nb) break;
            // after block b+1 is consumed: build block b+2 (RA), refill RA with b+4
            if (b + 2 < nb) producer_store<F>(RA, sm.buf[0], p);
            producer_load<F>(RA, S, b + 4, p);
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
            consumer_block<F, SUMS>(sm.buf[b & 1], lane, rg, tg0, accf, accj, D, b);
            lds_barrier();
        }
        // the results to LDS as [token][row] (the buffers are free after the
        // last block's barrier)
        float* out = reinterpret_cast<float*>(&sm.buf[0]);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = tg0 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                out[m * PF_TN + 32 * rg + (lane & 31)] = F == PF_Q6 ? accf[i][r] : accf[i][r] - accj[i][r];
            }
        }
    }
    // Every wave stores: lane l of wave wv takes rows 4 (l & 15) .. +3 of
    // tokens 16 wv + 4 k + (l >> 4), one 16-byte store each (4-byte stores
    // for a ragged or unaligned row end).
    lds_barrier();
    static_assert(sizeof(PrefillBuf<F>) >= PF_TM * PF_TN * sizeof(float), "the results fit one buffer");
    const float* out = reinterpret_cast<const float*>(&sm.buf[0]);
    const int64_t n = n0 + 4 * (lane & 15);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int m = 16 * wv + 4 * k + (lane >> 4);
        const float4 o = *reinterpret_cast<const float4*>(&out[m * PF_TN + 4 * (lane & 15)]);
        if (ok(m) && n < rows) {
            float* dst = y + orow(m) * rows + n;
            if (n + 4 <= rows && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
                *reinterpret_cast<float4*>(dst) = o;
            } else {
                const float oo[4] = {o.x, o.y, o.z, o.w};
                for (int e = 0; e < 4 && n + e < rows; ++e) dst[e] = oo[e];
            }
        }
    }
}

// SUMS (test support): the same kernel also stores every block's exact
// integer sum I_b to Isum [M][rows][nb].  Split-K (ksplit > 1, "Language
// models on the device", section 2.3): workgroup split ks multiplies blocks
// [kb0, kb0 + nbk) and stores its partial [M][rows] at y + ks * M * rows, for
// prefill_fixup_kernel to add.  PACK: the tokens arrive as fp32 and the
// workgroups pack them first (prefill_pack.h).
template <int F, bool SUMS = false, bool PACK = false>
__global__ __launch_bounds__(512) void prefill_q4k_kernel(const uint8_t* __restrict__ w,
                                                          const uint16_t* __restrict__ prefix, int64_t rows, int nb,
                                                          const int8_t* __restrict__ qs, const float* __restrict__ d8,
                                                          const int16_t* __restrict__ bs, int64_t K, int64_t M,
                                                          float* __restrict__ y, int32_t* __restrict__ Isum,
                                                          int ksplit, PackDst pk) {
    __shared__ __attribute__((aligned(16))) PrefillSmem<F> sm;
    // (tile counts are below 2^31, as the grid is: 32-bit divisions, which
    // cost far fewer scalar instructions ahead of the first load)
    const uint32_t ntn = (uint32_t)((rows + PF_TN - 1) / PF_TN);
    const uint32_t ntm = (uint32_t)((M + PF_TM - 1) / PF_TM);
    const uint32_t ks32 = blockIdx.x / (ntn * ntm);
    const uint32_t tile = blockIdx.x - ks32 * (ntn * ntm);
    const uint32_t tm = tile / ntn, tn = tile - tm * ntn;
    const int64_t n0 = (int64_t)tn * PF_TN;
    const int64_t m0 = (int64_t)tm * PF_TM;
    const int ks = (int)ks32;
    const int per = (nb + ksplit - 1) / ksplit;
    const int kb0 = ks * per;
    const int nbk = nb - kb0 < per ? nb - kb0 : per;
    y += (int64_t)ks * M * rows;
    if constexpr (PACK)
        pack_group<512>(pk, nb, M, PF_TM, m0, kb0, nbk, tn, ntn, (int64_t)ks * ntm + tm, (int)threadIdx.x);
    // Only producers use the sources.  Q6_K: every thread builds them, outside a
    // branch on the thread index, so their wave-uniform parts stay scalar (2%
    // faster); Q5_K measured 4% slower that way and builds them in the
    // producers' branch.
    PrefillSrc S;
    if (F == PF_Q6 || threadIdx.x >= 256) {
        producer_src<F>(S, w, prefix, rows, nb, qs, d8, bs, K, M, n0, m0, (int)threadIdx.x & 255);
        producer_src_from_block<F>(S, kb0);
    }
    PfSums D{};
    if constexpr (SUMS) D = PfSums{Isum + (m0 * rows + n0) * nb, rows, M - m0, rows - n0, nb};
    prefill_tile<F, SUMS>(
        sm, S, nbk, rows, n0, y, [&](int m) { return m0 + m; }, [&](int m) { return m0 + m < M; }, D);
}

// y[i] = sum over the ksplit partials part[s][i], s ascending (a fixed order:
// the result does not depend on scheduling).  V = 4: 16-byte accesses.
template <int V>
__global__ __launch_bounds__(256) void prefill_fixup_kernel(const float* __restrict__ part, int ksplit, int64_t n,
                                                            float* __restrict__ y) {
    typedef float fv __attribute__((ext_vector_type(V)));
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * V;
    if (i >= n) return;
    fv acc = *reinterpret_cast<const fv*>(part + i);
    for (int s = 1; s < ksplit; ++s) acc += *reinterpret_cast<const fv*>(part + (int64_t)s * n + i);
    *reinterpret_cast<fv*>(y + i) = acc;
}

hipError_t launch_prefill_fixup(const float* part, int ksplit, int64_t n, float* y, hipStream_t s) {
    if (n % 4 == 0 && reinterpret_cast<uintptr_t>(y) % 16 == 0)
        Q8K_LAUNCH(prefill_fixup_kernel<4>, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, s, part, ksplit, n,
                   y);
    else
        Q8K_LAUNCH(prefill_fixup_kernel<1>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, ksplit, n, y);
    return hipGetLastError();
}

// ----------------------------------------------------- mixture of experts ----
// "Language models on the device", section 2.4: the prefill of an MoE layer
// groups each expert's (token, slot) pairs into chunks and runs the prefill
// tile per (expert, chunk), with a ragged last chunk.  Three launches:
//   1. moe_group_kernel (one workgroup) counts the pairs of every expert,
//      lists the pair indices grouped by expert in `order` and cuts each
//      expert's run into chunks of at most 128 pairs (the chunk table);
//   2. prefill_moe_q4k_kernel runs one prefill tile per (chunk, row tile):
//      the chunk's tokens are gathered as the tile's 128 token rows and pair
//      p's dot products go to row p of the per-pair output `out` [P][rows];
//   3. moe_combine_kernel adds each token's pairs in slot order.
// Within an expert the pairs may be listed in any order: every output
// element is one row's own dot product, so the order changes no value.

// Grouping of P pairs over E experts: pair counts and cursors in LDS.
__global__ __launch_bounds__(1024) void moe_group_kernel(const int32_t* __restrict__ ids, int64_t P, int E,
                                                         int32_t* __restrict__ nchunks, int4* __restrict__ chunks,
                                                         int32_t* __restrict__ order) {
    __shared__ int cnt[MOE_GROUP_MAX_E];
    __shared__ int cur[MOE_GROUP_MAX_E];
    __shared__ int wsum[16][2];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    for (int e = tid; e < E; e += 1024) cnt[e] = 0;
    __syncthreads();
    for (int64_t p = tid; p < P; p += 1024) {
        const int32_t e = ids[p];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    // Exclusive scans over experts of the pair counts and of the chunk counts
    // ceil(cnt / 128); thread tid owns the experts [per * tid, per * tid + per).
    const int per = (E + 1023) / 1024;
    const int e0 = per * tid;
    int sp = 0, sc = 0;
    for (int i = 0; i < per; ++i) {
        const int e = e0 + i;
        if (e < E) {
            sp += cnt[e];
            sc += (cnt[e] + PF_TM - 1) / PF_TM;
        }
    }
    int ip = sp, ic = sc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int tp = __shfl_up(ip, o), tc = __shfl_up(ic, o);
        if (lane >= o) {
            ip += tp;
            ic += tc;
        }
    }
    if (lane == 63) {
        wsum[wv][0] = ip;
        wsum[wv][1] = ic;
    }
    __syncthreads();
    int pbase = ip - sp, cbase = ic - sc;
    for (int i = 0; i < wv; ++i) {
        pbase += wsum[i][0];
        cbase += wsum[i][1];
    }
    for (int i = 0; i < per; ++i) {
        const int e = e0 + i;
        if (e < E) {
            const int n = cnt[e];
            cur[e] = pbase;
            for (int c = 0; PF_TM * c < n; ++c)
                chunks[cbase + c] = make_int4(e, pbase + PF_TM * c, min(PF_TM, n - PF_TM * c), 0);
            pbase += n;
            cbase += (n + PF_TM - 1) / PF_TM;
        }
    }
    if (tid == 1023) *nchunks = cbase;  // the last thread ends on the total
    __syncthreads();
    for (int64_t p = tid; p < P; p += 1024) {
        const int32_t e = ids[p];
        if (e >= 0 && e < E) order[atomicAdd(&cur[e], 1)] = (int32_t)p;
    }
}

template <int F>
__global__ __launch_bounds__(512) void prefill_moe_q4k_kernel(const uint8_t* __restrict__ w,
                                                              const uint16_t* __restrict__ prefix, int64_t rows, int nb,
                                                              const int8_t* __restrict__ qs,
                                                              const float* __restrict__ d8,
                                                              const int16_t* __restrict__ bs, int64_t K, int64_t T,
                                                              const int32_t* __restrict__ nchunks,
                                                              const int4* __restrict__ chunks,
                                                              const int32_t* __restrict__ order, int topk,
                                                              float* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) PrefillSmem<F> sm;
    __shared__ int tok[PF_TM];   // token of each tile row, -1 past the chunk's end
    __shared__ int pair[PF_TM];  // pair index of each tile row
    const uint32_t ntn = (uint32_t)((rows + PF_TN - 1) / PF_TN);
    const uint32_t c = blockIdx.x / ntn;
    if ((int64_t)c >= nchunks[0]) return;  // uniform: the grid covers the most chunks P pairs can make
    const int64_t n0 = (int64_t)(blockIdx.x - c * ntn) * PF_TN;
    const int4 ch = chunks[c];
    const int count = ch.z;
    for (int i = threadIdx.x; i < PF_TM; i += 512) {
        const int p = i < count ? order[ch.y + i] : -1;
        pair[i] = p;
        tok[i] = p < 0 ? -1 : p / topk;
    }
    __syncthreads();
    const int64_t eb = (int64_t)ch.x * rows * (int64_t)nb;  // the expert's first (row, block)
    const uint8_t* we = w + eb * kblock<F>();
    const uint16_t* pe = F == PF_Q6 ? prefix + eb : prefix;
    PrefillSrc S;  // used by the producers (see prefill_q4k_kernel)
    if (F == PF_Q6 || threadIdx.x >= 256)
        producer_src_gather<F>(S, we, pe, rows, nb, qs, d8, bs, K, T, n0, tok, (int)threadIdx.x & 255);
    prefill_tile(
        sm, S, nb, rows, n0, out, [&](int m) { return (int64_t)pair[m]; }, [&](int m) { return m < count; });
}

// y[t][r] = sum_k rw[t][k] * out[t * topk + k][r] over ids in [0, E), k ascending.
// A workgroup takes one token and 256 * V consecutive rows (V = 4 when rows is
// a multiple of 4 and y 16-byte aligned: 16-byte loads and stores); the
// token's ids and router weights are the same for all its threads.
template <int V>
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ out, int64_t rows,
                                                          const int32_t* __restrict__ ids,
                                                          const float* __restrict__ rw, int topk, int64_t E,
                                                          float* __restrict__ y) {
    typedef float fv __attribute__((ext_vector_type(V)));
    const uint32_t nrb = (uint32_t)((rows + 256 * V - 1) / (256 * V));  // the grid is below 2^31
    const uint32_t tt = blockIdx.x / nrb;
    const int64_t t = tt;
    const int64_t r = ((int64_t)(blockIdx.x - tt * nrb) * 256 + threadIdx.x) * V;
    if (r >= rows) return;
    fv s = {};
    for (int k = 0; k < topk; ++k) {
        const int64_t pp = t * topk + k;
        const int32_t id = ids[pp];
        if (id >= 0 && id < E) s += rw[pp] * *reinterpret_cast<const fv*>(out + pp * rows + r);
    }
    *reinterpret_cast<fv*>(y + t * rows + r) = s;
}

hipError_t launch_prefill_moe(int fmt, const uint8_t* w, const uint16_t* prefix, int64_t E, int64_t rows, int nb,
                              Acts a, int64_t T, const int32_t* ids, const float* rw, int topk, float* y, void* ws,
                              hipStream_t s) {
    const MoePrefillWs L = moe_prefill_ws(E, rows, T, topk);
    float* out = static_cast<float*>(ws);
    int32_t* nchunks = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + L.meta);
    int4* chunks = reinterpret_cast<int4*>(static_cast<char*>(ws) + L.chunks);
    int32_t* order = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + L.order);
    Q8K_LAUNCH(moe_group_kernel, dim3(1), dim3(1024), 0, s, ids, L.P, (int)E, nchunks, chunks, order);
    const int64_t ntn = (rows + PF_TN - 1) / PF_TN;
    const dim3 grid((unsigned)(L.max_chunks * ntn));
    if (fmt == PF_Q4) {
        const hipError_t e = launch_prefill_regw_moe_q4k(w, rows, nb, a, T, L.max_chunks, nchunks, chunks, order,
                                                         topk, out, s);
        if (e != hipSuccess) return e;
    } else if (fmt == PF_Q6)
        Q8K_LAUNCH(prefill_moe_q4k_kernel<PF_Q6>, grid, dim3(512), 0, s, w, prefix, rows, nb, a.qs, a.d, a.bs, a.K, T,
                   nchunks, chunks, order, topk, out);
    else if (fmt == PF_Q5)
        Q8K_LAUNCH(prefill_moe_q4k_kernel<PF_Q5>, grid, dim3(512), 0, s, w, prefix, rows, nb, a.qs, a.d, a.bs, a.K, T,
                   nchunks, chunks, order, topk, out);
    if (rows % 4 == 0 && reinterpret_cast<uintptr_t>(y) % 16 == 0)
        Q8K_LAUNCH(moe_combine_kernel<4>, dim3((unsigned)(T * ((rows + 1023) / 1024))), dim3(256), 0, s, out, rows,
                   ids, rw, topk, E, y);
    else
        Q8K_LAUNCH(moe_combine_kernel<1>, dim3((unsigned)(T * ((rows + 255) / 256))), dim3(256), 0, s, out, rows, ids,
                   rw, topk, E, y);
    return hipGetLastError();
}

// ------------------------------------------------- allocation-free form ----
// The MoE prefill's workspace for callers that cannot allocate: a file-scope
// device array, one copy per device, held until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory: its device
// address is asked of the runtime once per device (with that device current)
// and only that address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[SCRATCH_MAX_DEVICES] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

// Q4_K runs the register-plane tile (prefill_regw.hip); Q5_K and relaid Q6_K
// the producer/consumer tile above.
hipError_t launch_prefill(int fmt, const uint8_t* w, const uint16_t* prefix, int64_t rows, int nb, Acts a,
                          int64_t M, float* y, float* part, hipStream_t s) {
    const int ksplit = prefill_ksplit(rows, nb, M);
    if (fmt == PF_Q4) return launch_prefill_regw_q4k(w, rows, nb, a, M, y, ksplit, part, s);
    const dim3 grid((unsigned)(((rows + PF_TN - 1) / PF_TN) * ((M + PF_TM - 1) / PF_TM) * ksplit));
    float* out = ksplit > 1 ? part : y;
    if (fmt == PF_Q6)
        Q8K_LAUNCH(prefill_q4k_kernel<PF_Q6>, grid, dim3(512), 0, s, w, prefix, rows, nb, a.qs, a.d, a.bs, a.K, M, out,
                   nullptr, ksplit, PackDst{});
    else
        Q8K_LAUNCH(prefill_q4k_kernel<PF_Q5>, grid, dim3(512), 0, s, w, prefix, rows, nb, a.qs, a.d, a.bs, a.K, M, out,
                   nullptr, ksplit, PackDst{});
    if (ksplit > 1) return launch_prefill_fixup(part, ksplit, M * rows, y, s);
    return hipGetLastError();
}

// The same tiles from fp32 tokens: the q8_K pack inside the launch.  `a` is
// the q8_K buffer the workgroups fill (pk.qs/d/bs are its sections).
hipError_t launch_prefill_f32(int fmt, const uint8_t* w, const uint16_t* prefix, int64_t rows, int nb, Acts a,
                              int64_t M, float* y, float* part, PackDst pk, hipStream_t s) {
    const int ksplit = prefill_ksplit(rows, nb, M);
    if (fmt == PF_Q4) return launch_prefill_regw_q4k_f32(w, rows, nb, a, M, y, ksplit, part, pk, s);
    const dim3 grid((unsigned)(((rows + PF_TN - 1) / PF_TN) * ((M + PF_TM - 1) / PF_TM) * ksplit));
    float* out = ksplit > 1 ? part : y;
    if (fmt == PF_Q6)
        Q8K_LAUNCH((prefill_q4k_kernel<PF_Q6, false, true>), grid, dim3(512), 0, s, w, prefix, rows, nb, a.qs, a.d,
                   a.bs, a.K, M, out, nullptr, ksplit, pk);
    else
        Q8K_LAUNCH((prefill_q4k_kernel<PF_Q5, false, true>), grid, dim3(512), 0, s, w, prefix, rows, nb, a.qs, a.d,
                   a.bs, a.K, M, out, nullptr, ksplit, pk);
    if (ksplit > 1) return launch_prefill_fixup(part, ksplit, M * rows, y, s);
    return hipGetLastError();
}

hipError_t launch_prefill_sums(int fmt, const uint8_t* w, const uint16_t* prefix, int64_t rows, int nb, Acts a,
                               int64_t M, float* y, int32_t* I, hipStream_t s) {
    if (fmt == PF_Q4) return launch_prefill_regw_q4k_sums(w, rows, nb, a, M, y, I, s);
    const dim3 grid((unsigned)(((rows + PF_TN - 1) / PF_TN) * ((M + PF_TM - 1) / PF_TM)));
    if (fmt == PF_Q6)
        Q8K_LAUNCH((prefill_q4k_kernel<PF_Q6, true>), grid, dim3(512), 0, s, w, prefix, rows, nb, a.qs, a.d, a.bs, a.K,
                   M, y, I, 1, PackDst{});
    else
        Q8K_LAUNCH((prefill_q4k_kernel<PF_Q5, true>), grid, dim3(512), 0, s, w, prefix, rows, nb, a.qs, a.d, a.bs, a.K,
                   M, y, I, 1, PackDst{});
    return hipGetLastError();
}

}  // namespace q8k
