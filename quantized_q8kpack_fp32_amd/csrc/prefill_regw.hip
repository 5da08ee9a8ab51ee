// Prefill GEMM with the weight planes built in registers: Q4_K weight
// [N rows][K] times M packed q8_K tokens on the gfx950 matrix cores.
//
// "Language models on the device: the cajeta-llm kernels", section 2.3 (the
// prefill tile: widen the weight nibbles to int8, stage ahead, multiply on
// the matrix units, fold the per-sub-block scales through the accumulator
// epilogue) and section 1 (the scale/min epilogue).  Per (token m, row n):
//   y = sum_b d8_b * d_b * I_b  -  sum_b sum_j (d8_b * bsum_bj) * (dmin_b * m_bj)
// with I_b = sum_j sc_j * S_j, the scale-weighted integer dot of block b.
//
// Arithmetic (as in the producer/consumer tile of prefill.hip): each 6-bit
// scale is split sc = 8a + b and the weight enters the int8 matrix cores as
// two planes a*q and b*q (each <= 105), so I_b = 8 P_hi + P_lo exactly from
// two 32x32x32 int8 MFMA passes; the min term runs on the bf16 matrix cores
// with both operands split into high and low bf16 parts, accumulating in
// fp32 across blocks.
//
// Work split.  The int8 planes of a weight row are reused by every token of
// the tile, and the token codes by every row.  Here the planes never leave
// the registers of the wave that builds them: a workgroup of 8 waves (two per
// SIMD, so one wave's vector work runs beside the other's matrix work) owns
// 128 tokens x 64 rows; wave w takes rows 32 (w & 1) .. +31 for all 128
// tokens (four 32-token MFMA tiles, so each plane fragment feeds eight MFMAs)
// over the blocks b with b % 4 == w >> 1 (a quarter of K).  Only the token
// codes go through LDS: the buffer unit copies them there (loads that write
// LDS directly, no registers), double-buffered in stages of 64 tokens x one
// block per quarter; a wave's planes serve the two stages of its block.  Every
// token fragment read from LDS feeds two MFMAs (both planes).  The four
// quarters meet at the end through LDS in a fixed order.
//
// Lane map.  32x32x32 int8 MFMA: A = tokens (row l % 32 from lane l), B =
// weight rows (column l % 32), k-group g = l / 32 holds 16 of the 32 k.  The
// k order inside a block is free as long as both operands follow it: lane
// (j, g) owns quant bytes 64g .. 64g+63 of row j's block (values of
// sub-blocks 4g .. 4g+3), and k-step kk (0..7) takes the low (kk even) or
// high (kk odd) nibbles of its quant dwords 4(kk/2) .. 4(kk/2)+3: values
// 64(2g + kk/4) + 32(kk%2) + 16((kk/2)%2) + 0..15, all in sub-block
// 4g + 2(kk/4) + kk%2, the same 16 contiguous code bytes the token lane reads.
//
// Result (i, j) of a 32x32 MFMA is in lane j + 32 ((i / 4) % 2), register
// (i % 4) + 4 (i / 8): each lane holds one weight row and 16 tokens.
#include "q4k_planes.h"
#include "q8k_launch.h"
#include "prefill_pack.h"

namespace q8k {
namespace {

constexpr int RW_TM = 128;  // tokens per workgroup
constexpr int RW_TN = 64;   // weight rows per workgroup
constexpr int RW_KQ = 4;    // K quarters (waves per row group)
constexpr int RW_SM = 64;   // tokens per stage
constexpr int RW_THREADS = 512;

// LDS, all double-buffered by stage parity: token codes (64 tokens x one
// block per quarter), the raw block scales and sub-block sums (copied two
// stages ahead, to build the min-term operands one stage ahead), and from
// those the min-term operands and the block scales the epilogue reads.  A
// stage's copies and its reads always touch opposite parities.  Token code
// rows keep their 256 bytes together (one copy moves four whole rows, so its
// global reads are contiguous) with the 16-byte chunks XOR-swizzled by the
// token index: the 16 lanes of a read phase then hit 16 different bank
// groups.  The min-term operands are stored fragment-major (64 lanes x 16
// bytes in lane order).  The arrays written by buffer-unit copies and those
// written by ds stores are separate objects.
struct RwCopied {
    int8_t codes[2][RW_KQ][RW_SM][QK];  // [parity][quarter][token][chunk ^ (token & 15)]
    float d8raw[2][RW_KQ][RW_SM];       // [parity][quarter][token]
    int16_t bs[2][RW_KQ][RW_SM][8];     // [parity][quarter][token][sub-block]
};
struct RwBuilt {
    float d8[2][RW_KQ][RW_SM];     // [parity][quarter][token]
    uint4 amin[2][RW_KQ][2][64];   // [parity][quarter][tile][lane (token i, g)]: bf16 d8*bsum_j, j = 4g..4g+3, high then low
};
// Mixture-of-experts tiles: the tile's 128 rows are the pairs of one chunk
// (pairs of one expert, grouped beforehand), so token rows are gathered: the
// byte offset of each tile row's token in the q8_K codes, and its pair index
// (the row of the per-pair result).
struct RwGather {
    int tokoff[RW_TM];
    int pair[RW_TM];
};
static_assert(sizeof(RwCopied) + sizeof(RwBuilt) + sizeof(RwGather) <= 160 * 1024, "LDS of one workgroup");

typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ uint32_t lds_addr(void* p) { return (uint32_t)(uintptr_t)(lds_void*)p; }

// Buffer-unit copy of 16 (4) bytes per lane from `off` into LDS at base +
// 16 (4) * lane; out-of-range reads write zeros.  Issued as inline assembly:
// the compiler then does not count the copies among its own loads, so it
// inserts no waits for them before unrelated LDS reads (it cannot tell the
// two parities of a buffer apart).  Every read of copied data comes after a
// stage_barrier(), whose vmcnt wait covers the copies.  (M0 holds the LDS
// base; one wait state between writing M0 and the copy.)
__device__ __forceinline__ void dma16(rsrc_t r, void* lds_base, int off) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_addr(lds_base)), "v"(off), "s"(r)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4(rsrc_t r, void* lds_base, int off) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"(lds_addr(lds_base)), "v"(off), "s"(r)
                 : "memory", "m0");
}

// Sources of one workgroup: tokens m0.., rows n0...  Offsets stay 32-bit: a
// tile's rows span at most 64 * (K / 256) * 144 bytes, its tokens 128 * K <=
// 2^31 bytes.  Each buffer's extent from the tile's start is kept as the
// index of its last byte (int32: a span of 2^31 bytes has last byte 2^31 - 1;
// an empty span -1), so every resource range below is the count left after
// the copy's own start offset, with one scalar signed compare.
struct RwSrc {
    const uint8_t* w;
    const int8_t* x;
    const float* d8;
    const int16_t* bs;
    int wlast, xlast, d8last, bslast;  // index of the last byte of each source (-1: empty)
    int wrow;  // bytes per weight row
    int nb;
    int K;
    const int* tokoff;  // gathered tiles: LDS offsets of the tile's token rows
};
// Index of the last byte of a span of v bytes, for spans of at most 2^31
// bytes (-1 when the span is empty or negative).
__device__ __forceinline__ int last_of(int64_t v) { return v <= 0 ? -1 : v < 0x80000000LL ? (int)(v - 1) : 0x7fffffff; }
// Raw buffer resource over [base + off, base + last + 1): the records left
// after the start offset `off` (none when off > last).  The compare is signed
// 32-bit (a scalar instruction; an unsigned compare-and-subtract would become
// a saturating subtract, which only the vector unit has, and the descriptor
// must stay in scalar registers for the copies' inline assembly).
__device__ __forceinline__ rsrc_t rsrc32(const void* base, int last, int off) {
    const uint32_t left = off <= last ? (uint32_t)last - (uint32_t)off + 1u : 0u;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(static_cast<const char*>(base)) + off, (short)0,
                                             __builtin_bit_cast(int, left), 0x00020000 /* raw, untyped dwords */);
}

// The buffer-unit copies of stage sg = 2 s + h (tokens 64 h .. 64 h + 63 of
// the tile, block 4 s + q of quarter q) by wave wv: codes of 32 token rows of
// quarter wv >> 1 (8 copies of four whole rows), and one copy of block scales
// (waves 0..3) or sub-block sums (waves 4..7) of one quarter.
template <bool GATHER>
__device__ __forceinline__ void issue_codes(RwCopied& sm, const RwSrc& S, int sg, int wv, int lane) {
    const int s = sg >> 1, h = sg & 1;
    const int q = wv >> 1, half = wv & 1;
    const int tq = lane >> 4, pc = lane & 15;
    if constexpr (GATHER) {
        // copy i covers stage tokens 32 half + 4i + tq, each at its own row
        const int bo = (4 * s + q) * QK;
        const rsrc_t rx = rsrc32(S.x, S.xlast, bo);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int m = RW_SM * h + 32 * half + 4 * i + tq;
            dma16(rx, &sm.codes[sg & 1][q][32 * half + 4 * i][0], S.tokoff[m] + 16 * (pc ^ (4 * (i & 3) + tq)));
        }
        return;
    }
    // copy i covers stage tokens 32 half + 4i + tq; its resource starts at that
    // group's first token (scalar), so the lane offsets repeat with period 4 in i
    const int base = (RW_SM * h + 32 * half) * S.K + (4 * s + q) * QK;
    int vo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) vo[j] = tq * S.K + 16 * (pc ^ (4 * j + tq));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int o = base + 4 * i * S.K;
        const rsrc_t rx = rsrc32(S.x, S.xlast, o);
        dma16(rx, &sm.codes[sg & 1][q][32 * half + 4 * i][0], vo[i & 3]);
    }
}
template <bool GATHER>
__device__ __forceinline__ void issue_aux(RwCopied& sm, const RwSrc& S, int sg, int wv, int lane) {
    const int s = sg >> 1, h = sg & 1, st = sg & 1;
    const int q = wv & 3;
    const int t0 = RW_SM * h;  // first token of the stage
    if constexpr (GATHER) {
        // token row r's records start at r * nb * 4 (scales) and r * nb * 16
        // (sums) bytes, i.e. at its code offset r * K over 64 and over 16
        const int tok = S.tokoff[t0 + lane];
        if (wv < 4) {
            const int o = (4 * s + q) * 4;
            dma4(rsrc32(S.d8, S.d8last, o), &sm.d8raw[st][q][0], tok >> 6);
        } else {
            const int o = (4 * s + q) * 16;
            dma16(rsrc32(S.bs, S.bslast, o), &sm.bs[st][q][0][0], tok >> 4);
        }
        return;
    }
    const int off = lane * S.nb;  // token 64 h + lane, block 4 s + q, in units of one block's record
    if (wv < 4) {
        const int o = (t0 * S.nb + 4 * s + q) * 4;
        dma4(rsrc32(S.d8, S.d8last, o), &sm.d8raw[st][q][0], off * 4);
    } else {
        const int o = (t0 * S.nb + 4 * s + q) * 16;
        dma16(rsrc32(S.bs, S.bslast, o), &sm.bs[st][q][0][0], off * 16);
    }
}

__device__ __forceinline__ void load_weights(Q4kRaw& R, const RwSrc& S, int b, int rg, int lane) {
    // (blocks past the row's end read the next row's bytes or, past the last
    // row, zeros: they are never multiplied)
    const int boff = b * Q4K_BLOCK;
    const rsrc_t rw = rsrc32(S.w, S.wlast, boff);
    const int o = (32 * rg + (lane & 31)) * S.wrow;
    R.hdr = load16(rw, o);
    const int oq = o + 16 + 64 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) R.q[i] = load16(rw, oq + 16 * i);
}

// Min-term operands and block scales of the tokens of stage sg from the raw
// scales and sums:
// thread tid takes quarter (tid >> 6) & 3, token tid & 63, sub-blocks 4g ..
// 4g+3 with g = tid >> 8.
__device__ __forceinline__ void build_amin(const RwCopied& sm, RwBuilt& sb, int sg, int tid) {
    const int q = (tid >> 6) & 3, t = tid & 63, g = tid >> 8;
    const int st = sg & 1;
    const float d8 = sm.d8raw[st][q][t];
    if (g == 0) sb.d8[st][q][t] = d8;
    const uint2 bv = *reinterpret_cast<const uint2*>(&sm.bs[st][q][t][4 * g]);
    const uint32_t bw[2] = {bv.x, bv.y};
    v8bf o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int sj = (int)(int16_t)(bw[j >> 1] >> (16 * (j & 1)));
        __bf16 hi, lo;
        bf16_split(d8 * (float)sj, hi, lo);
        o[j] = hi;
        o[4 + j] = lo;
    }
    *reinterpret_cast<v8bf*>(&sb.amin[sg & 1][q][t >> 5][(t & 31) + 32 * g]) = o;
}

// Test support (SUMS): where the block sums I_b go, [M][rows][nb] from the
// tile's first token and row (int32).
struct RwSums {
    int32_t* I;
    int64_t rows, live, nrow;  // problem rows; tokens and rows of this tile still inside the problem
    int nb;
};

// One stage of one wave: 64 tokens x 32 rows of block 4 s + q, two MFMA tiles
// of 32 tokens, into the accumulators of tiles 2h and 2h + 1.  SUMS: also
// store each (token, row)'s exact block sum I_b to D.
template <bool SUMS = false>
__device__ __forceinline__ void wave_stage(const RwCopied& sm, const RwBuilt& sb, const Q4kPlanes& P, int sg, int q,
                                           int lane, v16f (&acc)[4], const RwSums& D = RwSums{}, int rg = 0) {
    const int g = lane >> 5, h = sg & 1;
    // Code fragment of lane (i, g) at k-step kk: row i of the tile, logical
    // chunk kstep_off(g, kk) / 16 stored at chunk ^ (i & 15): one XOR per read.
    const int i = lane & 31;
    const int8_t* rowp = &sm.codes[sg & 1][q][i][0];
    const int y16 = 16 * (i & 15) ^ 128 * g;
    auto frag = [&](int t, int kk) {
        return *reinterpret_cast<const v4i*>(rowp + (y16 ^ kstep_off(0, kk)) + t * 32 * QK);
    };
    const float* d8row = &sb.d8[sg & 1][q][0];
    // The eight code fragments of a tile are read before its MFMAs (one LDS
    // latency per tile).  Both planes use them: the high plane's chain first,
    // then its sum times 8, then the low plane's chain into the same
    // accumulator, which then holds I = 8 P_hi + P_lo.
    auto chains = [&](int t, v16i& I) {
        v4i a[8];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) a[kk] = frag(t, kk);
        {
            const v16i zero = {};
            I = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[0], P.ph[0], zero, 0, 0, 0);
        }
#pragma unroll
        for (int kk = 1; kk < 8; ++kk) I = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[kk], P.ph[kk], I, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) I[r] <<= 3;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) I = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[kk], P.pl[kk], I, 0, 0, 0);
    };
    // min term: [ah | al] x [bh | bh] and [ah | al] x [bl | bl]
    auto minterm = [&](int t) {
        v16f& ac = acc[2 * h + t];
        const v8bf am = *reinterpret_cast<const v8bf*>(&sb.amin[sg & 1][q][t][lane]);
        ac = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, P.bh, ac, 0, 0, 0);
        ac = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, P.bl, ac, 0, 0, 0);
    };
    // block epilogue: acc += (d8 * float(I)) * d
    auto fold = [&](int t, const v16i& I) {
        v16f& ac = acc[2 * h + t];
#pragma unroll
        for (int G = 0; G < 4; ++G) {
            const float4 dv = *reinterpret_cast<const float4*>(d8row + 32 * t + 8 * G + 4 * g);
            const float d8a[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * G + e;
                ac[r] = fmaf((float)I[r] * d8a[e], P.dd, ac[r]);
            }
        }
    };
    // The matrix chains run at raised wave priority: the SIMD's other wave,
    // usually in its vector phase (plane build, folds), then fills the issue
    // slots between them instead of competing for the matrix unit.
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        v16i I;
        __builtin_amdgcn_s_setprio(1);
        chains(t, I);
        minterm(t);
        __builtin_amdgcn_s_setprio(0);
        if constexpr (SUMS) {
            // lane (j, g) register r: row 32 rg + j, token 8 (r / 4) + 4 g + r % 4 of tile t
            const int b = 2 * (sg & ~1) + q;
            const int j = lane & 31;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = 64 * h + 32 * t + 8 * (r >> 2) + 4 * g + (r & 3);
                if (m < D.live && 32 * rg + j < D.nrow)
                    D.I[((int64_t)m * D.rows + 32 * rg + j) * D.nb + b] = I[r];
            }
        }
        fold(t, I);
    }
}

// The stage's LDS writes (ds stores of this wave and buffer-unit copies) done,
// then the workgroup barrier.  `keep` loads issued last may stay in flight
// (the next block's weight bytes, which land in registers).
template <int keep>
__device__ __forceinline__ void stage_barrier() {
    if constexpr (keep == 0)
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(keep) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
constexpr int RW_RAW_LOADS = 5;  // load_weights() issues five loads

// GATHER = false: y[m][n] for tokens m0 .. m0+127 of M.  GATHER = true (the
// mixture-of-experts prefill): workgroup (chunk c, row tile) multiplies the
// chunk's expert by the tokens of its pairs (chunks[c] = {expert, first index
// in order, count}); the result of pair p goes to row p of y ([P][rows]);
// workgroups past the chunk count return at once.
//
// Split-K (dense tiles, "Language models on the device", section 2.3: when a
// problem is too small to fill the device, workgroups are added along the
// reduction and a fixup sums the partials): with ksplit > 1, workgroup split
// ks multiplies blocks [kb0, kb0 + nbk) of every row and stores its partial
// [M][rows] at y + ks * M * rows; prefill_fixup_kernel adds the splits.
//
// SUMS (test support, dense tiles): the same kernel also stores every block's
// exact integer sum I_b = 8 P_hi + P_lo to Isum [M][rows][nb].
template <bool GATHER, bool SUMS = false, bool PACK = false>
__global__ __launch_bounds__(RW_THREADS) void prefill_regw_q4k_kernel(
    const uint8_t* __restrict__ w, int64_t rows, int nb, const int8_t* __restrict__ qs,
    const float* __restrict__ d8, const int16_t* __restrict__ bs, int64_t K, int64_t M, float* __restrict__ y,
    const int32_t* __restrict__ nchunks, const int4* __restrict__ chunks, const int32_t* __restrict__ order,
    int topk, int32_t* __restrict__ Isum, int ksplit, PackDst pk) {
    static_assert(!(SUMS && GATHER), "block sums of the dense tile");
    static_assert(!(PACK && GATHER), "the pack runs in the dense tile");
    __shared__ __attribute__((aligned(16))) RwCopied sm;
    __shared__ __attribute__((aligned(16))) RwBuilt sb;
    __shared__ RwGather gat;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int rg = wv & 1, q = wv >> 1;
    // Row tiles vary fastest: the workgroups on one XCD (b, b + 8, ...) then
    // cover every token tile and a set of row tiles, so each weight row is
    // fetched into one L2 (measured: fewer L2 misses and faster than giving
    // each XCD one token tile).
    // (gathered tiles: workgroup = (chunk, row tile), no split)
    // The tile counts are below 2^31 (the grid is), so the workgroup index is
    // split with 32-bit divisions: 64-bit ones cost a few hundred scalar
    // instructions ahead of the first load.
    const uint32_t ntn = (uint32_t)((rows + RW_TN - 1) / RW_TN);
    const uint32_t ntm = GATHER ? 1u : (uint32_t)((M + RW_TM - 1) / RW_TM);
    const uint32_t bid = blockIdx.x;
    const uint32_t ks32 = GATHER ? 0u : bid / (ntn * ntm);
    const uint32_t tile = bid - ks32 * (ntn * ntm);
    const uint32_t tm = tile / ntn, tn = tile - tm * ntn;  // token tile (gathered: chunk), row tile
    const int64_t n0 = (int64_t)tn * RW_TN, m0 = GATHER ? 0 : (int64_t)tm * RW_TM;
    // this workgroup's blocks [kb0, kb0 + nbk) (all of them without split-K)
    const int ks = (int)ks32;
    const int per = (nb + ksplit - 1) / ksplit;
    const int kb0 = ks * per;
    const int nbk = nb - kb0 < per ? nb - kb0 : per;
    if constexpr (!GATHER) y += (int64_t)ks * M * rows;

    RwSrc S;
    S.nb = nb;
    S.K = (int)K;
    S.wrow = nb * Q4K_BLOCK;
    S.tokoff = gat.tokoff;
    int64_t live;  // tokens of the tile
    Q4kRaw R;
    if constexpr (GATHER) {
        const int64_t c = tm;
        if (c >= *nchunks) return;  // the whole workgroup
        const int4 ch = chunks[c];
        live = ch.z;
        S.w = w + ((int64_t)ch.x * rows + n0) * S.wrow;
        S.wlast = last_of((rows - n0) * S.wrow);
        S.x = qs;
        S.xlast = last_of(M * K);
        S.d8 = d8;
        S.d8last = last_of(M * nb * 4);
        S.bs = bs;
        S.bslast = last_of(M * nb * 16);
        // The tile's pair indices, then its first weights: the weights (from
        // HBM) stay in flight while the indices land and the token offsets go
        // to LDS (loads complete in issue order, so the indices are issued
        // first).  Rows past the chunk's count repeat its first pair (never
        // stored).
        static_assert(RW_TM <= RW_THREADS, "one pair index per thread");
        const int p = tid < RW_TM ? order[ch.y + (tid < ch.z ? tid : 0)] : 0;
        load_weights(R, S, q, rg, lane);
        if (tid < RW_TM) {
            gat.pair[tid] = p;
            gat.tokoff[tid] = (int)((int64_t)(p / topk) * K);
        }
        __syncthreads();
    } else {
        // sources start at block kb0 of the tile's first token / row; the
        // strides between tokens and rows stay those of whole rows
        live = M - m0;
        S.w = w + n0 * S.wrow + kb0 * Q4K_BLOCK;
        S.x = qs + m0 * K + (int64_t)kb0 * QK;
        S.xlast = last_of((M - m0) * K - (int64_t)kb0 * QK);
        S.d8 = d8 + m0 * nb + kb0;
        S.d8last = last_of(((M - m0) * nb - kb0) * 4);
        S.bs = bs + (m0 * nb + kb0) * 8;
        S.bslast = last_of(((M - m0) * nb - kb0) * 16);
    }
    if constexpr (!GATHER) S.wlast = last_of((rows - n0) * S.wrow - (int64_t)kb0 * Q4K_BLOCK);
    RwSums D{};
    if constexpr (SUMS) D = RwSums{Isum + (m0 * rows + n0) * nb, rows, live, rows - n0, nb};

    const int steps = (nbk + RW_KQ - 1) / RW_KQ;
    const int nst = 2 * steps;                        // stages
    const bool half2 = live > RW_SM;                  // the tile's second 64 tokens exist
    v16f acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;

    if constexpr (PACK) {
        // fp32 tokens: the first weights (which do not depend on the tokens)
        // are loaded first; then this workgroup packs its share of the tile's
        // blocks and waits for the rest of its group (prefill_pack.h)
        load_weights(R, S, q, rg, lane);
        pack_group<RW_THREADS>(pk, nb, M, RW_TM, m0, kb0, nbk, tn, ntn, (int64_t)ks * ntm + tm, tid);
    }
    issue_codes<GATHER>(sm, S, 0, wv, lane);
    issue_aux<GATHER>(sm, S, 0, wv, lane);
    if (half2) issue_aux<GATHER>(sm, S, 1, wv, lane);
    if constexpr (!PACK && !GATHER) load_weights(R, S, q, rg, lane);
    stage_barrier<0>();
    build_amin(sm, sb, 0, tid);
    stage_barrier<0>();
    Q4kPlanes PL;
    for (int sg = 0; sg < nst; sg += 2) {
        const int b = 2 * sg + q;  // block of this wave in step sg / 2
        // ---- first 64 tokens: copies of the next stage (codes) and the one
        // after (scales, sums); this block's operands, then the next block's raw
        // bytes into the same registers (issued last: they may stay in flight
        // across the barrier)
        // (R landed at the last barrier; the empty use makes the compiler place
        // its own wait for R here, before copies it does not know about)
        asm volatile("" ::"v"(__builtin_bit_cast(v4i, R.hdr)), "v"(__builtin_bit_cast(v4i, R.q[0])),
                     "v"(__builtin_bit_cast(v4i, R.q[1])), "v"(__builtin_bit_cast(v4i, R.q[2])),
                     "v"(__builtin_bit_cast(v4i, R.q[3])));
        if (half2) issue_codes<GATHER>(sm, S, sg + 1, wv, lane);
        if (sg + 2 < nst) issue_aux<GATHER>(sm, S, sg + 2, wv, lane);
        build_q4k_planes(PL, R, lane);
        load_weights(R, S, b + RW_KQ, rg, lane);
        if (b < nbk) wave_stage<SUMS>(sm, sb, PL, sg, q, lane, acc, D, rg);
        if (half2) build_amin(sm, sb, sg + 1, tid);
        stage_barrier<RW_RAW_LOADS>();
        // ---- second 64 tokens
        if (sg + 2 < nst) issue_codes<GATHER>(sm, S, sg + 2, wv, lane);
        if (half2 && sg + 3 < nst) issue_aux<GATHER>(sm, S, sg + 3, wv, lane);
        if (b < nbk && half2) wave_stage<SUMS>(sm, sb, PL, sg + 1, q, lane, acc, D, rg);
        if (sg + 2 < nst) build_amin(sm, sb, sg + 2, tid);
        stage_barrier<0>();
    }
    // The quarters meet in LDS: every wave stores its partial sums there, then
    // wave (q, rg) adds tile t = q of row group rg over the quarters in the
    // fixed order 0, 1, 2, 3 (register r of lane (j, g) in tile
    // t: token 32 t + 8 (r / 4) + 4 g + r % 4, row 32 rg + j; partials move as
    // float4 of registers 4 r4 .. 4 r4 + 3, so the 64 lanes of an access touch
    // 1 KB of consecutive LDS).  The lane index is read afresh (mbcnt) so that
    // nothing lane-dependent stays live across the loop for this epilogue.
    const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    float4* red = reinterpret_cast<float4*>(&sm.codes[0][0][0][0]);  // [q][rg][t][r4][lane], 128 KB
    static_assert(sizeof(sm.codes) == RW_KQ * 2 * 4 * 4 * 64 * sizeof(float4), "partials fill the code buffers");
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
            red[(((q * 2 + rg) * 4 + t) * 4 + r4) * 64 + ln] =
                make_float4(acc[t][4 * r4], acc[t][4 * r4 + 1], acc[t][4 * r4 + 2], acc[t][4 * r4 + 3]);
    __syncthreads();
    // The sums go back to LDS as [token][row] (the partials are read: one
    // barrier) and leave as 16-byte stores, four rows of one token per lane.
    float4 v[4];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
        v[r4] = red[((rg * 4 + q) * 4 + r4) * 64 + ln];
#pragma unroll
        for (int qq = 1; qq < RW_KQ; ++qq) {
            const float4 u = red[(((qq * 2 + rg) * 4 + q) * 4 + r4) * 64 + ln];
            v[r4].x += u.x;
            v[r4].y += u.y;
            v[r4].z += u.z;
            v[r4].w += u.w;
        }
    }
    __syncthreads();
    float* out = reinterpret_cast<float*>(&sm.codes[0][0][0][0]);  // [RW_TM][RW_TN]
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
        const float vv[4] = {v[r4].x, v[r4].y, v[r4].z, v[r4].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            out[(32 * q + 8 * r4 + 4 * (ln >> 5) + e) * RW_TN + 32 * rg + (ln & 31)] = vv[e];
    }
    __syncthreads();
    // lane l of wave wv: rows 4 (l & 15) .. +3 of tokens 16 wv + 4 k + (l >> 4)
    const int64_t n = n0 + 4 * (ln & 15);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int mt = 16 * wv + 4 * k + (ln >> 4);  // tile row
        const float4 o = *reinterpret_cast<const float4*>(&out[mt * RW_TN + 4 * (ln & 15)]);
        if (mt < live && n < rows) {
            float* dst = GATHER ? y + (int64_t)gat.pair[mt] * rows + n : y + (m0 + mt) * rows + n;
            if (n + 4 <= rows && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
                *reinterpret_cast<float4*>(dst) = o;
            } else {
                const float oo[4] = {o.x, o.y, o.z, o.w};
                for (int e = 0; e < 4 && n + e < rows; ++e) dst[e] = oo[e];
            }
        }
    }
}

}  // namespace

hipError_t launch_prefill_regw_q4k(const uint8_t* w, int64_t rows, int nb, Acts a, int64_t M, float* y,
                                   int ksplit, float* part, hipStream_t s) {
    const dim3 grid((unsigned)(((rows + RW_TN - 1) / RW_TN) * ((M + RW_TM - 1) / RW_TM) * ksplit));
    Q8K_LAUNCH((prefill_regw_q4k_kernel<false>), grid, dim3(RW_THREADS), 0, s, w, rows, nb, a.qs, a.d, a.bs, a.K, M,
               ksplit > 1 ? part : y, nullptr, nullptr, nullptr, 1, nullptr, ksplit, PackDst{});
    if (ksplit > 1) return launch_prefill_fixup(part, ksplit, M * rows, y, s);
    return hipGetLastError();
}

hipError_t launch_prefill_regw_q4k_f32(const uint8_t* w, int64_t rows, int nb, Acts a, int64_t M, float* y,
                                       int ksplit, float* part, PackDst pk, hipStream_t s) {
    const dim3 grid((unsigned)(((rows + RW_TN - 1) / RW_TN) * ((M + RW_TM - 1) / RW_TM) * ksplit));
    Q8K_LAUNCH((prefill_regw_q4k_kernel<false, false, true>), grid, dim3(RW_THREADS), 0, s, w, rows, nb, a.qs, a.d,
               a.bs, a.K, M, ksplit > 1 ? part : y, nullptr, nullptr, nullptr, 1, nullptr, ksplit, pk);
    if (ksplit > 1) return launch_prefill_fixup(part, ksplit, M * rows, y, s);
    return hipGetLastError();
}

hipError_t launch_prefill_regw_q4k_sums(const uint8_t* w, int64_t rows, int nb, Acts a, int64_t M, float* y,
                                        int32_t* I, hipStream_t s) {
    const dim3 grid((unsigned)(((rows + RW_TN - 1) / RW_TN) * ((M + RW_TM - 1) / RW_TM)));
    Q8K_LAUNCH((prefill_regw_q4k_kernel<false, true>), grid, dim3(RW_THREADS), 0, s, w, rows, nb, a.qs, a.d, a.bs, a.K,
               M, y, nullptr, nullptr, nullptr, 1, I, 1, PackDst{});
    return hipGetLastError();
}

hipError_t launch_prefill_regw_moe_q4k(const uint8_t* w, int64_t rows, int nb, Acts a, int64_t T, int64_t max_chunks,
                                       const int32_t* nchunks, const int4* chunks, const int32_t* order, int topk,
                                       float* out, hipStream_t s) {
    const dim3 grid((unsigned)(((rows + RW_TN - 1) / RW_TN) * max_chunks));
    Q8K_LAUNCH((prefill_regw_q4k_kernel<true>), grid, dim3(RW_THREADS), 0, s, w, rows, nb, a.qs, a.d, a.bs, a.K, T,
               out, nchunks, chunks, order, topk, nullptr, 1, PackDst{});
    return hipGetLastError();
}

}  // namespace q8k
