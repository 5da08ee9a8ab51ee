// Mixture-of-experts decode on the int8 matrix cores: Q4_K and Q5_K here,
// relaid Q6_K further below.
//
// "Language models on the device: the cajeta-llm kernels", section 2.4: for a
// decode, every token's selected experts are visited in one launch and each
// token's expert outputs are summed as they are produced; weights are read
// through the index of which expert each token chose (section intro).
//
// A workgroup walks row tiles of at most 32 rows of every expert; its
// MM_WAVES waves take the experts w, w + MM_WAVES, ... .  For expert e a wave
// lists the (token, slot) pairs that chose e (a ballot over ids) and
// multiplies its tile's rows against up to MM_GROUP of those pairs at a time
// on the int8 matrix cores, one 32x32x32 MFMA per 32-value sub-block: the
// pairs' q8_K codes are the A operand (row i = pair i of the group), the
// rows' raw 4-bit quants the B operand, and the result is the integer sum S_j
// of sub-block j for every (pair, row), exactly.  The six-bit scales then
// fold in int32 on the vector unit, I = sum_j sc_j * S_j, in the four result
// registers that hold the group's pairs; the min term runs on the bf16 matrix
// path (both operands split in high and low parts) into the fp32
// accumulator; then acc += (d8 * float(I)) * d.  One weight read serves every
// pair of the group, and the vector work per weight byte is a nibble mask and
// a quarter of a multiply-add.
//
// The dot of pair p and row r lands in an LDS slot owned by p; once every wave
// is done the workgroup adds each token's slots in slot order,
//   y[t][r] = sum_k rw[t][k] * dot(ids[t][k], t, r),
// so the order of the sum is fixed and no atomics or global workspace are
// used.  Tokens are taken in slabs of at most MM_SLOT pairs whose packed
// tokens fit the workgroup's LDS stage (codes, sub-block sums and scales of
// every slab token, copied once per slab): the pairs' operands are then LDS
// reads, so the only vector-memory loads in flight during the block walk are
// the weight blocks, and each wave keeps the next one in flight while it
// multiplies the current one (vector loads complete in issue order, so token
// loads interleaved with them would be waited for with every block).  The
// slab, the ids and the router weights reach LDS through buffer-unit copies,
// and each walk's first block is fetched into the cache ahead of the walk
// (during the staging, and across the previous tile's barrier and slot sums),
// so no walk starts on a cold memory latency.  An expert nobody
// chose is never read; an id outside [0, E) matches no expert and its slot is
// skipped.
#include "q4k_planes.h"  // vector types, bf16 split
#include "q8k.h"
#include "q8k_launch.h"

#include <atomic>

namespace q8k {
namespace {

constexpr int MM_WAVES = 8;   // waves per workgroup
constexpr int MM_ROWS = 32;   // rows per workgroup (the MFMA's B columns)
constexpr int MM_SLOT = 128;  // (token, slot) pairs per slab
constexpr int MM_GROUP = 8;   // pairs per MFMA tile (its first 8 rows; the rest repeat pair 0)
static_assert(MM_SLOT >= Q8K_MOE_MAX_TOPK, "a slab holds at least one token's pairs");
constexpr int MM_TOK_BYTES = 98304;  // LDS stage of the slab's packed tokens

// Block formats: Q4_K (144 bytes: d, dmin, 12 scale bytes, 128 quant bytes) and
// Q5_K (176 bytes: the same 16-byte header, 32 bytes of fifth bits, then the
// 128 low-nibble bytes).  A tile of 32 rows' blocks is CH 16-byte chunks per
// row, NL loads per lane.
template <bool Q5>
struct MmFmt {
    static constexpr int BLK = Q5 ? Q5K_BLOCK : Q4K_BLOCK;
    static constexpr int CH = BLK / 16;    // 9 or 11
    static constexpr int NL = Q5 ? 6 : 5;  // ceil(32 * CH / 64)
    static constexpr int QOFF = Q5 ? 48 : 16;
    static constexpr int TILE = MM_ROWS * BLK;
    static_assert(32 * CH - 64 * (NL - 1) == 32, "the last load takes the last 32 chunks");
};

// LDS bytes of one staged token: codes padded by 16 bytes (consecutive tokens
// start 4 banks apart), sub-block sums, block scales.
__host__ __device__ constexpr int64_t mm_tok_bytes(int64_t K) { return (K + 16) + K / 16 + K / 64; }

template <bool Q5>
struct MmWave {
    int plist[64];  // pair indices of the current 64-pair window that chose the wave's expert, by rank
    float d8[32];   // the group's block scales (pair i at i) for the epilogue
    __attribute__((aligned(16))) uint8_t tile[MmFmt<Q5>::TILE];  // block b of the tile's rows, [row][block]
};
template <bool Q5>
struct MmSmem {
    MmWave<Q5> wave[MM_WAVES];
    float slot[MM_SLOT * MM_ROWS];  // dot of (pair, row), pair-major
    int32_t sid[MM_SLOT];           // the slab's expert ids and router weights, by pair
    float srw[MM_SLOT];
    // slab tokens: codes [ts][K + 16], then sums [ts][K / 32] int16, then scales [ts][K / 256] fp32
    int8_t tok[MM_TOK_BYTES];
};

// One block of the tile's 32 rows, loaded by hand in a sector-contiguous lane
// map: load x of lane l takes 16-byte chunk c = 64x + l of the 288 chunks
// (row c / 9, chunk c % 9 of its 144-byte block; the fifth load's upper half
// repeats the lower half), so consecutive lanes read consecutive bytes and a
// load instruction touches 2-3 cache lines per row instead of 32 scattered
// pieces.  The wave then moves the block through its LDS tile into the
// matrix-core lane map.  The walk keeps the next block in flight behind the
// one it multiplies and waits for that one with an explicit count (it issues
// no other vector-memory load); the wait names the registers it covers, so
// the compiler neither reads them earlier nor reuses them while a load into
// them is in flight.
template <int NL>
struct MmW {
    v4i c[NL];
};
__device__ __forceinline__ v4i mm_vload16(rsrc_t r, int off) {
    v4i v;
    asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(v) : "v"(off), "s"(r));
    return v;
}
// Lane l's chunk offsets inside a row-major run of 32 rows (block 0).
template <int NL>
struct MmLane {
    int go[NL];  // global: row * row_bytes + 16 * chunk
    int lo[NL];  // LDS tile: 16 * c
};
template <bool Q5>
__device__ __forceinline__ MmLane<MmFmt<Q5>::NL> mm_lane(int lane, int64_t wrow) {
    using F = MmFmt<Q5>;
    MmLane<F::NL> m;
#pragma unroll
    for (int x = 0; x < F::NL; ++x) {
        const int c = x < F::NL - 1 ? 64 * x + lane : 64 * (F::NL - 1) + (lane & 31);
        m.go[x] = (c / F::CH) * (int)wrow + 16 * (c % F::CH);
        m.lo[x] = 16 * c;
    }
    return m;
}
template <bool Q5>
__device__ __forceinline__ void mm_issue_w(MmW<MmFmt<Q5>::NL>& W, rsrc_t wr, const MmLane<MmFmt<Q5>::NL>& m,
                                           int b) {
    const int boff = b * MmFmt<Q5>::BLK;
#pragma unroll
    for (int x = 0; x < MmFmt<Q5>::NL; ++x) W.c[x] = mm_vload16(wr, m.go[x] + boff);
}
template <int N>
__device__ __forceinline__ void mm_wait_w(MmW<5>& W) {
    asm volatile("s_waitcnt vmcnt(%5)" : "+v"(W.c[0]), "+v"(W.c[1]), "+v"(W.c[2]), "+v"(W.c[3]), "+v"(W.c[4]) : "n"(N));
}
template <int N>
__device__ __forceinline__ void mm_wait_w(MmW<6>& W) {
    asm volatile("s_waitcnt vmcnt(%6)"
                 : "+v"(W.c[0]), "+v"(W.c[1]), "+v"(W.c[2]), "+v"(W.c[3]), "+v"(W.c[4]), "+v"(W.c[5])
                 : "n"(N));
}

// Buffer-unit copies straight into LDS: 16 (4) bytes per lane land at
// base + 16 (4) * lane (M0 holds the LDS base, with one wait state between
// writing M0 and the copy).  No register receives the data, so a copy may stay
// in flight across barriers and loops; a vmcnt wait covers it.  A partial copy
// runs on the lowest lanes only.  mm_issue_tile copies a block into the wave's
// tile in the register loads' lane map (the last copy's upper half-wave would
// repeat the lower one past the tile, so it runs on lanes 0-31).
typedef __attribute__((address_space(3))) void mm_lds_void;
__device__ __forceinline__ void mm_dma16(rsrc_t r, void* lds_base, int off) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"((uint32_t)(uintptr_t)(mm_lds_void*)lds_base), "v"(off), "s"(r)
                 : "memory", "m0");
}
__device__ __forceinline__ void mm_dma4(rsrc_t r, void* lds_base, int off) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"((uint32_t)(uintptr_t)(mm_lds_void*)lds_base), "v"(off), "s"(r)
                 : "memory", "m0");
}
template <bool Q5>
__device__ __forceinline__ void mm_issue_tile(uint8_t* tile, rsrc_t wr, const MmLane<MmFmt<Q5>::NL>& m, int lane,
                                              int b) {
    using F = MmFmt<Q5>;
    const int boff = b * F::BLK;
#pragma unroll
    for (int x = 0; x < F::NL - 1; ++x) mm_dma16(wr, tile + 1024 * x, m.go[x] + boff);
    if (lane < 32) mm_dma16(wr, tile + 1024 * (F::NL - 1), m.go[F::NL - 1] + boff);
}

// The wave hands data between its own lanes through LDS.  The hardware runs
// one wave's LDS instructions in order, but the compiler reasons per thread:
// the memory clobbers keep a lane's reads behind the other lanes' writes and
// the next writes behind the reads.
__device__ __forceinline__ void wave_lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// SUMS (test support): the same kernel also stores each pair's exact sub-block
// sums, Sout [T * topk][rows][nb][8], as its matrix cores produce them.
template <bool Q5, bool SUMS = false>
__global__ __launch_bounds__(64 * MM_WAVES) void moe_mfma_q4k_kernel(
    const uint8_t* __restrict__ w, int64_t E, int64_t rows, int nb, const int8_t* __restrict__ qs,
    const float* __restrict__ d8, const int16_t* __restrict__ bs, int64_t K, int64_t T,
    const int32_t* __restrict__ ids, const float* __restrict__ rw, int topk, float* __restrict__ y, int rt,
    int64_t ntiles, int32_t* __restrict__ Sout) {
    using F = MmFmt<Q5>;
    __shared__ __attribute__((aligned(16))) MmSmem<Q5> sm;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: expert and rsrc are scalar
    const int lane = threadIdx.x & 63;
    const int i = lane & 31, g = lane >> 5;
    const int64_t wrow = (int64_t)nb * F::BLK;
    MmWave<Q5>& L = sm.wave[wv];
    const MmLane<F::NL> ml = mm_lane<Q5>(lane, wrow);  // rows past `live` read zeros
    const int64_t KS = K + 16, cpt = K / 16;  // staged code row stride; 16-byte chunks of codes per token
    // (32-bit divisions: the slab bounds K, so these fit, and 64-bit ones cost
    // about a hundred instructions each)
    const int tsl = MM_TOK_BYTES / (int)mm_tok_bytes(K);  // >= 1 (checked by the launcher)
    const int64_t ts = MM_SLOT / topk < tsl ? MM_SLOT / topk : tsl;  // tokens per slab
    int8_t* const tokc = sm.tok;
    int8_t* const tokb = sm.tok + ts * KS;
    float* const tokd = reinterpret_cast<float*>(sm.tok + ts * KS + ts * cpt);
    // expert e's rows of a tile (rows past the tile's live rows read zeros)
    auto tile_rsrc = [&](int64_t tile, int64_t e) {
        const int64_t r0 = tile * rt;
        const int64_t live = rows - r0 < rt ? rows - r0 : rt;
        return make_rsrc(w + (e * rows + r0) * wrow, live * wrow);
    };
    // Each wave's first walk of a tile (expert wv) finds its first block in the
    // cache: the block is copied into the wave's tile ahead (at the start of a
    // slab, right behind the staging copies; at the end of the previous tile's
    // walks, across the barrier and the slot sums).  The walk then loads it again into
    // registers, a cache hit, and overwrites the tile only after waiting for its
    // own load, which is younger than the copy.
    for (int64_t t0 = 0; t0 < T; t0 += ts) {
        const int64_t t1 = t0 + ts < T ? t0 + ts : T;
        const int64_t pb = t0 * topk, pe = t1 * topk;
        // ---- stage the slab's packed tokens, ids and router weights with
        // buffer-unit copies (waves take copies w, w + MM_WAVES, ...); then the
        // first block of this wave's first walk, and a wait for everything but
        // that block: the staging never waits for the weight fetch.
        {
            const int nt = (int)(t1 - t0), cp = (int)cpt, nbt = nt * nb, np = (int)(pe - pb);
            const int ipt = (cp + 63) >> 6;  // copies per token (64 chunks of 16 bytes each)
            const rsrc_t rq = make_rsrc(qs + t0 * K, (int64_t)nt * K);
            for (int n = wv; n < nt * ipt; n += MM_WAVES) {
                const int t = n / ipt, j = n - t * ipt, c = 64 * j + lane;
                if (c < cp) mm_dma16(rq, tokc + t * KS + 1024 * j, t * (int)K + 16 * c);
            }
            // sums: one 16-byte chunk per block; scales: one fp32 per block
            const rsrc_t rb = make_rsrc(bs + t0 * nb * 8, (int64_t)nbt * 16);
            const rsrc_t rd = make_rsrc(d8 + t0 * nb, (int64_t)nbt * 4);
            for (int n = wv; n < (nbt + 63) >> 6; n += MM_WAVES) {
                const int c = 64 * n + lane;
                if (c < nbt) {
                    mm_dma16(rb, tokb + 1024 * n, 16 * c);
                    mm_dma4(rd, tokd + 64 * n, 4 * c);
                }
            }
            const rsrc_t ri = make_rsrc(ids + pb, (int64_t)np * 4);
            const rsrc_t rr = make_rsrc(rw + pb, (int64_t)np * 4);
            for (int n = wv; n < (np + 63) >> 6; n += MM_WAVES) {
                const int c = 64 * n + lane;
                if (c < np) {
                    mm_dma4(ri, sm.sid + 64 * n, 4 * c);
                    mm_dma4(rr, sm.srw + 64 * n, 4 * c);
                }
            }
        }
        if (wv < E) {
            mm_issue_tile<Q5>(L.tile, tile_rsrc(blockIdx.x, wv), ml, lane, 0);  // grid <= ntiles
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(F::NL) : "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        __syncthreads();
        for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
            const int64_t r0 = tile * rt;
            const int64_t live = rows - r0 < rt ? rows - r0 : rt;  // rows of this tile
            for (int64_t e = wv; e < E; e += MM_WAVES) {
                const rsrc_t wr = tile_rsrc(tile, e);
                for (int64_t p0 = pb; p0 < pe; p0 += 64) {
                    const int64_t p = p0 + lane;
                    const bool hit = p < pe && sm.sid[p - pb] == (int32_t)e;
                    const uint64_t mask = __ballot(hit);
                    if (mask == 0) continue;
                    const int count = __popcll(mask);
                    // pair indices by rank in the window
                    wave_lds_fence();
                    const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
                    if (hit) L.plist[rank] = (int)p;
                    wave_lds_fence();
                    for (int k0 = 0; k0 < count; k0 += MM_GROUP) {
                        const int n = count - k0 < MM_GROUP ? count - k0 : MM_GROUP;  // pairs of this group
                        // code lane (i, g) takes pair k0 + i (pair k0 when the group has fewer)
                        const int pi = L.plist[k0 + (i < n ? i : 0)];
                        const int tl = (int)(pi / topk - t0);  // the pair's token in the slab stage
                        const int8_t* xrow = tokc + tl * KS;
                        const int8_t* bsrow = tokb + tl * cpt + 8 * g;
                        const float* d8row = tokd + tl * nb;
                        // The block walk.  The weights of two blocks are in registers at
                        // once: block b's (multiplied now) and block b+1's (in flight), in W0
                        // and W1 by parity (no register copies); the walk starts at b = -1
                        // with a load-only step.  The last step reloads the row's last block
                        // (a cache hit, never used) and the walk ends by draining it: no load
                        // outlives it.
                        v16f acc = {};
                        MmW<F::NL> W0, W1;
                        auto step = [&](int b, MmW<F::NL>& Wc, MmW<F::NL>& Wfree) __attribute__((always_inline)) {
                            mm_issue_w<Q5>(Wfree, wr, ml, b + 1 < nb ? b + 1 : nb - 1);
                            if (b < 0) return;
                            // the pairs' side of block b (staged codes, sums and scale) is
                            // read before the wait for the weights, so its LDS latency hides
                            // behind the memory wait and the MFMAs wait on no LDS read
                            v4i av[8];
#pragma unroll
                            for (int j = 0; j < 8; ++j)
                                av[j] = *reinterpret_cast<const v4i*>(xrow + b * QK + 32 * j + 16 * g);
                            const uint2 bsv = *reinterpret_cast<const uint2*>(bsrow + 16 * b);
                            const float a8 = d8row[b];
                            mm_wait_w<F::NL>(Wc);
                            // block b through the tile into this wave's lane map
                            wave_lds_fence();
#pragma unroll
                            for (int x = 0; x < F::NL; ++x)
                                *reinterpret_cast<v4i*>(L.tile + ml.lo[x]) = Wc.c[x];
                            wave_lds_fence();
                            const uint8_t* tr = L.tile + i * F::BLK;
                            const uint4 hdr = *reinterpret_cast<const uint4*>(tr);
                            // the row's min-term operands for sub-blocks 4g..4g+3 (-dmin *
                            // m_j, high and low bf16 parts, repeated in both fragment
                            // halves) and d
                            const uint32_t hy = hdr.y, hz = hdr.z, hw = hdr.w;
                            const uint32_t hm = 0u - (uint32_t)g;  // (branch-free: g differs inside the wave)
                            const uint32_t mn = (hm & (((hw >> 4) & 0x0F0F0F0Fu) | ((hz >> 2) & 0x30303030u))) |
                                                (~hm & hz & 0x3F3F3F3Fu);
                            const float dd = half_bits_to_float(hdr.x & 0xffffu);
                            const float dmin = half_bits_to_float(hdr.x >> 16);
                            v8bf bh, bl;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                __bf16 hi, lo;
                                bf16_split(-dmin * (float)((mn >> (8 * e)) & 0xffu), hi, lo);
                                bh[e] = bh[4 + e] = hi;
                                bl[e] = bl[4 + e] = lo;
                            }
                            v16i I;
                            {
                                // One MFMA per 32-value sub-block j on the raw nibbles gives
                                // the sums S_j of every (pair, row); the six-bit scales fold
                                // in int32 in the registers that hold pairs: I = sum_j sc_j *
                                // S_j (|S_j| <= 127*15*32, sc_j <= 63: 24-bit products).  Lane
                                // (i, g) holds quant bytes 32m + 16g .. +15 (m = 0..3): values
                                // 16g .. 16g+15 of sub-blocks 2m (low nibbles) and 2m + 1
                                // (high nibbles).  Sub-block j + 1's MFMA is issued before
                                // sub-block j's fold.
                                v4i qb[4];
#pragma unroll
                                for (int m = 0; m < 4; ++m)
                                    qb[m] = *reinterpret_cast<const v4i*>(tr + F::QOFF + 32 * m + 16 * g);
                                // Q5_K: fifth bits of values 16g .. 16g+15 (bit j of byte t: sub-block j)
                                v4i qh = {};
                                if constexpr (Q5) qh = *reinterpret_cast<const v4i*>(tr + 16 + 16 * g);
                                const uint32_t sc03 = hy & 0x3F3F3F3Fu;
                                const uint32_t sc47 = (hw & 0x0F0F0F0Fu) | ((hy >> 2) & 0x30303030u);
                                auto sums = [&](int j) {
                                    const v4i aj = av[j];
                                    v4i bj;
#pragma unroll
                                    for (int x = 0; x < 4; ++x) {
                                        const int q4 = qb[j >> 1][x];
                                        const int nib = (j & 1) ? ((q4 >> 4) & 0x0F0F0F0F) : (q4 & 0x0F0F0F0F);
                                        bj[x] = nib | (Q5 ? ((qh[x] >> j) & 0x01010101) << 4 : 0);
                                    }
                                    const v16i zero = {};
                                    return __builtin_amdgcn_mfma_i32_32x32x32_i8(aj, bj, zero, 0, 0, 0);
                                };
                                auto fold = [&](int j, const v16i& S) {
                                    if constexpr (SUMS) {
                                        // register r < 4 of lane (i, g) holds pair 4g + r of the group, row i
#pragma unroll
                                        for (int r = 0; r < 4; ++r)
                                            if (4 * g + r < n && i < live)
                                                Sout[((int64_t)L.plist[k0 + 4 * g + r] * rows + r0 + i) * (nb * 8) +
                                                     8 * b + j] = S[r];
                                    }
                                    const int sc = (int)(((j < 4 ? sc03 : sc47) >> (8 * (j & 3))) & 0xffu);
#pragma unroll
                                    for (int r = 0; r < 4; ++r)
                                        I[r] = j == 0 ? __mul24(sc, S[r]) : I[r] + __mul24(sc, S[r]);
                                };
                                v16i S0 = sums(0), S1;
#pragma unroll
                                for (int j = 0; j < 8; j += 2) {
                                    S1 = sums(j + 1);
                                    fold(j, S0);
                                    __builtin_amdgcn_sched_barrier(0);
                                    if (j + 2 < 8) S0 = sums(j + 2);
                                    fold(j + 1, S1);
                                    __builtin_amdgcn_sched_barrier(0);
                                }
                            }
                            // ---- min term: the pair's d8 * bsum_j (j = 4g..4g+3), high
                            // then low bf16 parts, against [bh | bh] and [bl | bl]
                            {
                                v8bf am;
                                const uint32_t bw[2] = {bsv.x, bsv.y};
#pragma unroll
                                for (int j = 0; j < 4; ++j) {
                                    const int sj = (int)(int16_t)(bw[j >> 1] >> (16 * (j & 1)));
                                    __bf16 hi, lo;
                                    bf16_split(a8 * (float)sj, hi, lo);
                                    am[j] = hi;
                                    am[4 + j] = lo;
                                }
                                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, bh, acc, 0, 0, 0);
                                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, bl, acc, 0, 0, 0);
                            }
                            // ---- epilogue: acc += (d8 * float(I)) * d; register r < 4 of
                            // lane (i, g) holds pair 4g + r (the other registers hold the
                            // tile's repeated rows)
                            wave_lds_fence();
                            if (g == 0) L.d8[i] = a8;
                            wave_lds_fence();
                            {
                                const float4 dv = *reinterpret_cast<const float4*>(&L.d8[4 * g]);
                                const float d8a[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
                                for (int r = 0; r < 4; ++r) acc[r] = fmaf((float)I[r] * d8a[r], dd, acc[r]);
                            }
                        };
                        for (int b = -1; b < nb; b += 2) {
                            step(b, W1, W0);
                            if (b + 1 == nb) break;
                            step(b + 1, W0, W1);
                        }
                        mm_wait_w<0>(W0);
                        mm_wait_w<0>(W1);
                        // ---- the group's dots into their pairs' slots (row i of the
                        // workgroup is this lane's weight row)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int pr = 8 * (r >> 2) + 4 * g + (r & 3);  // pair of register r
                            if (pr < n) sm.slot[(L.plist[k0 + pr] - (int)pb) * MM_ROWS + i] = acc[r];
                        }
                    }
                }
            }
            // the next tile's first block for this wave's first expert, fetched
            // while the workgroup meets and adds its slots (this wave's reads of
            // the tile are done: every step ends with an LDS wait)
            if (wv < E && tile + gridDim.x < ntiles) {
                wave_lds_fence();
                mm_issue_tile<Q5>(L.tile, tile_rsrc(tile + gridDim.x, wv), ml, lane, 0);
            }
            __syncthreads();
            // ---- each token's slots, added in slot order
            for (int idx = threadIdx.x; idx < (int)(t1 - t0) * MM_ROWS; idx += 64 * MM_WAVES) {
                const int64_t t = t0 + idx / MM_ROWS;
                const int r = idx % MM_ROWS;
                if (r < live) {
                    float s = 0.0f;
                    for (int k = 0; k < topk; ++k) {
                        const int64_t pp = t * topk + k;
                        const int32_t id = sm.sid[pp - pb];
                        if (id >= 0 && id < E) s += sm.srw[pp - pb] * sm.slot[(pp - pb) * MM_ROWS + r];
                    }
                    y[t * rows + r0 + r] = s;
                }
            }
            __syncthreads();
        }
    }
    // a copy ahead for a walk that did not come (an expert nobody chose)
    // lands before the wave ends
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}


// ================================================================ relaid Q6_K
// The same walk over relaid Q6_K experts (fp16 d per (row, block) in the
// prefix; bodies ql[128] | qh[64] | int8 scales[16]).  A Q6_K sub-block is 16
// values with its own signed 8-bit scale, so each takes one 32x32x16 int8
// MFMA: lane (i, g) supplies values 16s + 8g .. +7 of sub-block s, the pairs'
// q8_K codes as A and the rows' 6-bit values q (0..63, before the -32 offset)
// as B.  A second MFMA of the same codes against -32 in every byte adds
// -32 times each pair's code sum, so the accumulator holds S_s = sum (q - 32) x
// exactly; the scales then fold in int32, I = sum_s sc_s * S_s, and
// acc += (d8 * float(I)) * d.
// Value v = 128h + 32t + l of a block has its low four bits in
// ql[64h + 32(t&1) + l] (nibble t >> 1) and its high two in qh[32h + l] (bits
// 2t, 2t + 1); sub-block s = v / 16.
constexpr int M6_CH = Q6K_BODY / 16;  // 13 chunks of a body
constexpr int M6_NL = 7;              // ceil(32 * 13 / 64) loads per lane and block
static_assert(32 * M6_CH - 64 * (M6_NL - 1) == 32, "the last load takes the last 32 chunks");
constexpr int M6_TOK_BYTES = 86016;   // LDS stage of the slab's packed tokens

// LDS bytes of one staged token: codes padded by 16 bytes, block scales (no
// sub-block sums: Q6_K has no min term).
__host__ __device__ constexpr int64_t m6_tok_bytes(int64_t K) { return (K + 16) + K / 64; }

struct Mm6Wave {
    int plist[64];
    float d8[32];
    uint32_t dd[2][64];  // by block parity: lane l's dword of the prefix run holding row l % 32's d
    __attribute__((aligned(16))) uint8_t tile[MM_ROWS * Q6K_BODY];  // block b of the tile's rows, [row][body]
};
struct Mm6Smem {
    Mm6Wave wave[MM_WAVES];
    float slot[MM_SLOT * MM_ROWS];
    int32_t sid[MM_SLOT];
    float srw[MM_SLOT];
    int8_t tok[M6_TOK_BYTES];  // codes [ts][K + 16], then scales [ts][K / 256] fp32
};
static_assert(sizeof(Mm6Smem) <= 160 * 1024, "LDS of one workgroup");

// One block of the tile's rows: the body chunks in the sector-contiguous lane
// map (chunk c = 64x + l of the 416, row c / 13) into registers, and the rows'
// d by a buffer-unit copy into LDS (lane l: the aligned dword of the prefix run
// that holds row l % 32's d).  The wait names every register it covers.
struct M6W {
    v4i c[M6_NL];
};
__device__ __forceinline__ MmLane<M6_NL> m6_lane(int lane, int64_t brow) {
    MmLane<M6_NL> m;
#pragma unroll
    for (int x = 0; x < M6_NL; ++x) {
        const int c = x < M6_NL - 1 ? 64 * x + lane : 64 * (M6_NL - 1) + (lane & 31);
        m.go[x] = (c / M6_CH) * (int)brow + 16 * (c % M6_CH);
        m.lo[x] = 16 * c;
    }
    return m;
}
__device__ __forceinline__ void m6_issue(M6W& W, rsrc_t wr, rsrc_t pr, const MmLane<M6_NL>& m, uint32_t (&dd)[2][64],
                                         int drow, int b) {
    const int boff = b * Q6K_BODY;
#pragma unroll
    for (int x = 0; x < M6_NL; ++x) W.c[x] = mm_vload16(wr, m.go[x] + boff);
    mm_dma4(pr, &dd[b & 1][0], ((drow + b) * 2) & ~3);
}
template <int N>
__device__ __forceinline__ void m6_wait(M6W& W) {
    asm volatile("s_waitcnt vmcnt(%7)"
                 : "+v"(W.c[0]), "+v"(W.c[1]), "+v"(W.c[2]), "+v"(W.c[3]), "+v"(W.c[4]), "+v"(W.c[5]), "+v"(W.c[6])
                 : "n"(N));
}
constexpr int M6_LOADS = M6_NL + 1;  // loads per block

// SUMS (test support): also store each pair's exact sub-block sums, Sout
// [T * topk][rows][nb][16], as its matrix cores produce them.
template <bool SUMS = false>
__global__ __launch_bounds__(64 * MM_WAVES) void moe_mfma_q6k_kernel(
    const uint16_t* __restrict__ prefix, const uint8_t* __restrict__ bodies, int64_t E, int64_t rows, int nb,
    const int8_t* __restrict__ qs, const float* __restrict__ d8, int64_t K, int64_t T,
    const int32_t* __restrict__ ids, const float* __restrict__ rw, int topk, float* __restrict__ y, int rt,
    int64_t ntiles, int32_t* __restrict__ Sout) {
    __shared__ __attribute__((aligned(16))) Mm6Smem sm;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: expert and rsrc are scalar
    const int lane = threadIdx.x & 63;
    const int i = lane & 31, g = lane >> 5;
    const int64_t brow = (int64_t)nb * Q6K_BODY;  // body bytes per row
    Mm6Wave& L = sm.wave[wv];
    const MmLane<M6_NL> ml = m6_lane(lane, brow);  // rows past `live` read zeros
    const int drow = i * nb;                       // index of row i's d of block 0 in the tile's prefix run
    const int64_t KS = K + 16, cpt = K / 16;
    const int tsl = M6_TOK_BYTES / (int)m6_tok_bytes(K);  // >= 1 (checked by the launcher)
    const int64_t ts = MM_SLOT / topk < tsl ? MM_SLOT / topk : tsl;  // tokens per slab
    int8_t* const tokc = sm.tok;
    float* const tokd = reinterpret_cast<float*>(sm.tok + ts * KS);
    // expert e's rows of a tile: bodies and the prefix run of their d
    auto tile_rsrc = [&](int64_t tile, int64_t e) {
        const int64_t r0 = tile * rt;
        const int64_t live = rows - r0 < rt ? rows - r0 : rt;
        return make_rsrc(bodies + (e * rows + r0) * brow, live * brow);
    };
    // (2 bytes past the run: a dword copy may end there; they are the next
    // row's entries or the prefix array's padding to 256 bytes)
    auto tile_prsrc = [&](int64_t tile, int64_t e) {
        const int64_t r0 = tile * rt;
        const int64_t live = rows - r0 < rt ? rows - r0 : rt;
        return make_rsrc(prefix + (e * rows + r0) * nb, live * nb * 2 + 2);
    };
    for (int64_t t0 = 0; t0 < T; t0 += ts) {
        const int64_t t1 = t0 + ts < T ? t0 + ts : T;
        const int64_t pb = t0 * topk, pe = t1 * topk;
        // ---- stage the slab's codes, block scales, ids and router weights
        // with buffer-unit copies; then the first body block of this wave's
        // first walk, and a wait for everything but that block
        {
            const int nt = (int)(t1 - t0), cp = (int)cpt, nbt = nt * nb, np = (int)(pe - pb);
            const int ipt = (cp + 63) >> 6;
            const rsrc_t rq = make_rsrc(qs + t0 * K, (int64_t)nt * K);
            for (int n = wv; n < nt * ipt; n += MM_WAVES) {
                const int t = n / ipt, j = n - t * ipt, c = 64 * j + lane;
                if (c < cp) mm_dma16(rq, tokc + t * KS + 1024 * j, t * (int)K + 16 * c);
            }
            const rsrc_t rd = make_rsrc(d8 + t0 * nb, (int64_t)nbt * 4);
            for (int n = wv; n < (nbt + 63) >> 6; n += MM_WAVES)
                if (64 * n + lane < nbt) mm_dma4(rd, tokd + 64 * n, 4 * (64 * n + lane));
            const rsrc_t ri = make_rsrc(ids + pb, (int64_t)np * 4);
            const rsrc_t rr = make_rsrc(rw + pb, (int64_t)np * 4);
            for (int n = wv; n < (np + 63) >> 6; n += MM_WAVES) {
                const int c = 64 * n + lane;
                if (c < np) {
                    mm_dma4(ri, sm.sid + 64 * n, 4 * c);
                    mm_dma4(rr, sm.srw + 64 * n, 4 * c);
                }
            }
        }
        if (wv < E) {
            // block 0 of the first walk into the wave's tile (a cache fill, as
            // in the Q4_K walk; the last copy on lanes 0-31)
            const rsrc_t wr0 = tile_rsrc(blockIdx.x, wv);  // grid <= ntiles
#pragma unroll
            for (int x = 0; x < M6_NL - 1; ++x) mm_dma16(wr0, L.tile + 1024 * x, ml.go[x]);
            if (lane < 32) mm_dma16(wr0, L.tile + 1024 * (M6_NL - 1), ml.go[M6_NL - 1]);
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(M6_NL) : "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        __syncthreads();
        for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
            const int64_t r0 = tile * rt;
            const int64_t live = rows - r0 < rt ? rows - r0 : rt;
            for (int64_t e = wv; e < E; e += MM_WAVES) {
                const rsrc_t wr = tile_rsrc(tile, e);
                const rsrc_t pr = tile_prsrc(tile, e);
                for (int64_t p0 = pb; p0 < pe; p0 += 64) {
                    const int64_t p = p0 + lane;
                    const bool hit = p < pe && sm.sid[p - pb] == (int32_t)e;
                    const uint64_t mask = __ballot(hit);
                    if (mask == 0) continue;
                    const int count = __popcll(mask);
                    wave_lds_fence();
                    const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
                    if (hit) L.plist[rank] = (int)p;
                    wave_lds_fence();
                    for (int k0 = 0; k0 < count; k0 += MM_GROUP) {
                        const int n = count - k0 < MM_GROUP ? count - k0 : MM_GROUP;
                        const int pi = L.plist[k0 + (i < n ? i : 0)];
                        const int tl = (int)(pi / topk - t0);
                        // the pair's codes and scales as 32-bit offsets into the stage
                        // (under 2^17 bytes), so every address stays an LDS address
                        const int xoff = tl * (int)KS;
                        const float* d8row = tokd + tl * nb;
                        // The block walk, as for Q4_K: block b's registers are
                        // multiplied while block b + 1's are in flight (M0 / M1 by
                        // parity); the last step reloads the last block and the
                        // walk ends by draining it.
                        v16f acc = {};
                        M6W M0, M1;
                        auto step = [&](int b, M6W& Wc, M6W& Wfree) __attribute__((always_inline)) {
                            m6_issue(Wfree, wr, pr, ml, L.dd, drow, b + 1 < nb ? b + 1 : nb - 1);
                            if (b < 0) return;
                            // the pairs' codes and scale of block b, read before the wait
                            // for the weights (as in the Q4_K walk)
                            long av[16];
#pragma unroll
                            for (int sb = 0; sb < 16; ++sb)
                                av[sb] = *reinterpret_cast<const long*>(&sm.tok[xoff + b * QK + 16 * sb + 8 * g]);
                            const float a8 = d8row[b];
                            m6_wait<M6_LOADS>(Wc);
                            wave_lds_fence();
#pragma unroll
                            for (int x = 0; x < M6_NL; ++x)
                                *reinterpret_cast<v4i*>(L.tile + ml.lo[x]) = Wc.c[x];
                            if (g == 0) L.d8[i] = a8;
                            wave_lds_fence();
                            const uint8_t* tr = L.tile + i * Q6K_BODY;
                            // this lane's ql pieces (h, t & 1, s & 1) and qh pieces
                            // (h, s & 1): 8 bytes each at value offset 16 (s & 1) + 8g
                            uint2 lq[8], hq[4];
#pragma unroll
                            for (int k = 0; k < 8; ++k)
                                lq[k] = *reinterpret_cast<const uint2*>(tr + 64 * (k >> 2) + 32 * ((k >> 1) & 1) +
                                                                         16 * (k & 1) + 8 * g);
#pragma unroll
                            for (int k = 0; k < 4; ++k)
                                hq[k] = *reinterpret_cast<const uint2*>(tr + 128 + 32 * (k >> 1) + 16 * (k & 1) + 8 * g);
                            const uint4 scv = *reinterpret_cast<const uint4*>(tr + 192);
                            const uint32_t scw[4] = {scv.x, scv.y, scv.z, scv.w};
                            int I[4] = {0, 0, 0, 0};
                            const long m32 = (long)0xE0E0E0E0E0E0E0E0uLL;  // eight int8 -32
                            const v16i zero = {};
                            // sub-block sb's two MFMAs; sub-block sb + 1's are issued
                            // before sb's fold
                            auto sums = [&](int sb) {
                                const int h = sb >> 3, t = (sb >> 1) & 3, c = sb & 1;
                                const uint2 l2 = lq[4 * h + 2 * (t & 1) + c], h2 = hq[2 * h + c];
                                const uint32_t bx = ((l2.x >> (4 * (t >> 1))) & 0x0F0F0F0Fu) |
                                                    (((h2.x >> (2 * t)) & 0x03030303u) << 4);
                                const uint32_t by = ((l2.y >> (4 * (t >> 1))) & 0x0F0F0F0Fu) |
                                                    (((h2.y >> (2 * t)) & 0x03030303u) << 4);
                                const long B = (long)((uint64_t)bx | ((uint64_t)by << 32));
                                const long A = av[sb];
                                const v16i S = __builtin_amdgcn_mfma_i32_32x32x16_i8(A, B, zero, 0, 0, 0);
                                return __builtin_amdgcn_mfma_i32_32x32x16_i8(A, m32, S, 0, 0, 0);
                            };
                            auto fold = [&](int sb, const v16i& S) {
                                const int sc = (int)(int8_t)((scw[sb >> 2] >> (8 * (sb & 3))) & 0xffu);
#pragma unroll
                                for (int r = 0; r < 4; ++r) {
                                    const int Ss = S[r];
                                    if constexpr (SUMS) {
                                        // register r < 4 of lane (i, g): pair 4g + r of the group, row i
                                        if (4 * g + r < n && i < live)
                                            Sout[((int64_t)L.plist[k0 + 4 * g + r] * rows + r0 + i) * (nb * 16) +
                                                 16 * b + sb] = Ss;
                                    }
                                    I[r] += __mul24(sc, Ss);  // |Ss| <= 65024, |sc| <= 128
                                }
                            };
                            v16i S0 = sums(0), S1;
#pragma unroll
                            for (int sb = 0; sb < 16; sb += 2) {
                                S1 = sums(sb + 1);
                                fold(sb, S0);
                                __builtin_amdgcn_sched_barrier(0);
                                if (sb + 2 < 16) S0 = sums(sb + 2);
                                fold(sb + 1, S1);
                                __builtin_amdgcn_sched_barrier(0);
                            }
                            // acc += (d8 * float(I)) * d: register r < 4 of lane (i, g)
                            // holds pair 4g + r
                            const float4 dv = *reinterpret_cast<const float4*>(&L.d8[4 * g]);
                            const float d8a[4] = {dv.x, dv.y, dv.z, dv.w};
                            const uint32_t dw = L.dd[b & 1][i];
                            const float dd = half_bits_to_float(((drow + b) & 1 ? dw >> 16 : dw) & 0xffffu);
#pragma unroll
                            for (int r = 0; r < 4; ++r) acc[r] = fmaf((float)I[r] * d8a[r], dd, acc[r]);
                            wave_lds_fence();
                        };
                        for (int b = -1; b < nb; b += 2) {
                            step(b, M1, M0);
                            if (b + 1 == nb) break;
                            step(b + 1, M0, M1);
                        }
                        m6_wait<0>(M0);
                        m6_wait<0>(M1);
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int prr = 8 * (r >> 2) + 4 * g + (r & 3);
                            if (prr < n) sm.slot[(L.plist[k0 + prr] - (int)pb) * MM_ROWS + i] = acc[r];
                        }
                    }
                }
            }
            if (wv < E && tile + gridDim.x < ntiles) {
                wave_lds_fence();
                const rsrc_t wn = tile_rsrc(tile + gridDim.x, wv);
#pragma unroll
                for (int x = 0; x < M6_NL - 1; ++x) mm_dma16(wn, L.tile + 1024 * x, ml.go[x]);
                if (lane < 32) mm_dma16(wn, L.tile + 1024 * (M6_NL - 1), ml.go[M6_NL - 1]);
            }
            __syncthreads();
            for (int idx = threadIdx.x; idx < (int)(t1 - t0) * MM_ROWS; idx += 64 * MM_WAVES) {
                const int64_t t = t0 + idx / MM_ROWS;
                const int r = idx % MM_ROWS;
                if (r < live) {
                    float s = 0.0f;
                    for (int k = 0; k < topk; ++k) {
                        const int64_t pp = t * topk + k;
                        const int32_t id = sm.sid[pp - pb];
                        if (id >= 0 && id < E) s += sm.srw[pp - pb] * sm.slot[(pp - pb) * MM_ROWS + r];
                    }
                    y[t * rows + r0 + r] = s;
                }
            }
            __syncthreads();
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace

// Compute units of the current device, asked once per device.
int64_t device_cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    const int slot = dev >= 0 && dev < 64 ? dev : 0;
    int n = cached[slot].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[slot].store(n, std::memory_order_relaxed);
    }
    return n;
}

bool moe_mfma_q4k_fits(int64_t K) { return mm_tok_bytes(K) <= MM_TOK_BYTES; }

template <bool Q5, bool SUMS = false>
hipError_t launch_moe_mfma(const uint8_t* w, int64_t E, int64_t rows, int nb, Acts a, int64_t T, const int32_t* ids,
                           const float* rw, int topk, float* y, hipStream_t s, int32_t* Sout = nullptr) {
    if (!moe_mfma_q4k_fits(a.K)) return hipErrorInvalidValue;
    // One workgroup per compute unit (its LDS allows no second), each walking
    // row tiles of rt <= 32 rows: rt is chosen so the tiles come out as whole
    // rounds over the compute units (14336 rows: 512 tiles of 28 on 256 units)
    // and a workgroup stages its tokens once for all its tiles.
    const int64_t cus = device_cu_count();
    const int64_t rounds = ((rows + MM_ROWS - 1) / MM_ROWS + cus - 1) / cus;
    int64_t rt = (rows + rounds * cus - 1) / (rounds * cus);
    rt = rt < 16 ? 16 : rt > MM_ROWS ? MM_ROWS : rt;
    const int64_t ntiles = (rows + rt - 1) / rt;
    const unsigned grid = (unsigned)(ntiles < cus ? ntiles : cus);
    Q8K_LAUNCH((moe_mfma_q4k_kernel<Q5, SUMS>), dim3(grid), dim3(64 * MM_WAVES), 0, s, w, E, rows, nb, a.qs, a.d, a.bs,
               a.K, T, ids, rw, topk, y, (int)rt, ntiles, Sout);
    return hipGetLastError();
}

bool moe_mfma_q6k_fits(int64_t K) { return m6_tok_bytes(K) <= M6_TOK_BYTES; }

template <bool SUMS = false>
hipError_t launch_moe_mfma6(const uint16_t* prefix, const uint8_t* bodies, int64_t E, int64_t rows, int nb, Acts a,
                            int64_t T, const int32_t* ids, const float* rw, int topk, float* y, hipStream_t s,
                            int32_t* Sout = nullptr) {
    if (!moe_mfma_q6k_fits(a.K)) return hipErrorInvalidValue;
    // the grid and row tiles of the Q4_K kernel
    const int64_t cus = device_cu_count();
    const int64_t rounds = ((rows + MM_ROWS - 1) / MM_ROWS + cus - 1) / cus;
    int64_t rt = (rows + rounds * cus - 1) / (rounds * cus);
    rt = rt < 16 ? 16 : rt > MM_ROWS ? MM_ROWS : rt;
    const int64_t ntiles = (rows + rt - 1) / rt;
    const unsigned grid = (unsigned)(ntiles < cus ? ntiles : cus);
    Q8K_LAUNCH((moe_mfma_q6k_kernel<SUMS>), dim3(grid), dim3(64 * MM_WAVES), 0, s, prefix, bodies, E, rows, nb, a.qs,
               a.d, a.K, T, ids, rw, topk, y, (int)rt, ntiles, Sout);
    return hipGetLastError();
}

hipError_t launch_moe_mfma_q6k(const uint16_t* prefix, const uint8_t* bodies, int64_t E, int64_t rows, int nb, Acts a,
                               int64_t T, const int32_t* ids, const float* rw, int topk, float* y, hipStream_t s) {
    return launch_moe_mfma6(prefix, bodies, E, rows, nb, a, T, ids, rw, topk, y, s);
}
hipError_t launch_moe_mfma6_sums(const uint16_t* prefix, const uint8_t* bodies, int64_t E, int64_t rows, int nb,
                                 Acts a, int64_t T, const int32_t* ids, const float* rw, int topk, float* y,
                                 int32_t* S, hipStream_t s) {
    return launch_moe_mfma6<true>(prefix, bodies, E, rows, nb, a, T, ids, rw, topk, y, s, S);
}

hipError_t launch_moe_mfma_q4k(const uint8_t* w, int64_t E, int64_t rows, int nb, Acts a, int64_t T,
                               const int32_t* ids, const float* rw, int topk, float* y, hipStream_t s) {
    return launch_moe_mfma<false>(w, E, rows, nb, a, T, ids, rw, topk, y, s);
}
hipError_t launch_moe_mfma_q5k(const uint8_t* w, int64_t E, int64_t rows, int nb, Acts a, int64_t T,
                               const int32_t* ids, const float* rw, int topk, float* y, hipStream_t s) {
    return launch_moe_mfma<true>(w, E, rows, nb, a, T, ids, rw, topk, y, s);
}
hipError_t launch_moe_mfma_sums(bool q5, const uint8_t* w, int64_t E, int64_t rows, int nb, Acts a, int64_t T,
                                const int32_t* ids, const float* rw, int topk, float* y, int32_t* S, hipStream_t s) {
    return q5 ? launch_moe_mfma<true, true>(w, E, rows, nb, a, T, ids, rw, topk, y, s, S)
              : launch_moe_mfma<false, true>(w, E, rows, nb, a, T, ids, rw, topk, y, s, S);
}

}  // namespace q8k
