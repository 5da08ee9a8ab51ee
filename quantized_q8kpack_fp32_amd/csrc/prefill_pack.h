// The q8_K pack inside the prefill launch ("Language models on the device:
// the cajeta-llm kernels", section 1 and section 3.3: launches are fused
// where it pays; the pack is the device quantiser of section 2.6).
//
// qmatmul_prefill_f32 runs the prefill tiles on fp32 tokens.  The workgroups
// that share a token tile and a K range (a "group": the tile's row tiles,
// whose workgroup numbers are consecutive) split that tile's 256-value blocks
// into equal shares.  Each packs its share into the caller's q8_K buffer with
// the pack kernel's quantiser (so the bytes are q8k_pack's), publishes it, and
// waits until every member of its group has published before the tile reads
// any packed code.
//
// Progress.  A group has at most as many members as the device has compute
// units and one workgroup fills a compute unit, so a group's members fit on
// the device together; the hardware starts workgroups in order, so a group
// only waits for members that are running or about to start, never for
// workgroups that wait on it.  Each wait is still bounded: after
// PACK_WAIT_POLLS polls the workgroup gives up, sets the error word and goes
// on (its outputs are then not valid), so every wave always finishes.
//
// Sync words (in the caller's workspace, zero before the first call): word 0
// is the error word (set, never cleared, by a workgroup that gave up), words
// 4 + 2g and 5 + 2g count the members of group g that have arrived and that
// have left the wait.  The last member to leave sets both back to zero, so a
// finished call leaves them as it found them.
#pragma once
#include "q8k_launch.h"
#include "q8k_quant.h"

namespace q8k {

constexpr int PACK_WAIT_POLLS = 1 << 20;

// Blocks [i0, i1) of the group's live x nbk blocks (token-major), sixteen
// lanes per block as in the pack kernel.  Up to four blocks per 16-lane row
// are loaded before any is quantised.  THREADS: the workgroup size.
template <int THREADS>
__device__ __forceinline__ void pack_share(const PackDst& P, int nb, int64_t m0, int64_t live, int kb0, int nbk,
                                           int64_t member, int64_t members, int tid) {
    constexpr int ROWS = THREADS / 16;  // blocks per round
    constexpr int U = 4;                // rounds in flight
    // block indices inside the group stay below 2^31 (at most a token tile
    // times the blocks of a row), so they are divided in 32 bits
    const int total = (int)live * nbk;
    const int per = (total + (int)members - 1) / (int)members;
    const int i0 = (int)member * per;
    const int i1 = i0 + per < total ? i0 + per : total;
    const int r = tid & 15;
    for (int ib = i0 + (tid >> 4); ib < i1; ib += U * ROWS) {
        float4 v[U][4];
        int64_t blk[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = ib + u * ROWS;  // the same for the 16 lanes of a row
            blk[u] = -1;
            if (i < i1) {
                const int tok = i / nbk;
                blk[u] = (m0 + tok) * nb + kb0 + (i - tok * nbk);
                const float4* src = reinterpret_cast<const float4*>(P.x + blk[u] * QK + 16 * r);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[u][e] = src[e];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (blk[u] >= 0) {
                int s;
                float dd;
                const uint4 codes = q8k_quant_lane16(v[u], s, dd);
                // device-scope stores: written through to the device's point
                // of coherence, so no cache write-back is needed before the
                // hand-off (group_sync)
                uint64_t* dst = reinterpret_cast<uint64_t*>(P.qs + blk[u] * QK + 16 * r);
                __hip_atomic_store(dst, (uint64_t)codes.x | ((uint64_t)codes.y << 32), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(dst + 1, (uint64_t)codes.z | ((uint64_t)codes.w << 32), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                if ((r & 1) == 0)
                    __hip_atomic_store(P.bs + blk[u] * 8 + (r >> 1), (int16_t)s, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                if (r == 0) __hip_atomic_store(P.d + blk[u], dd, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

// Publish this workgroup's share and wait for the rest of group g.
// Visibility across XCDs (each has its own L2): the packed bytes were stored
// at device scope (written through, so nothing waits in an L2 to be written
// back), every wave waits for its stores before the workgroup meets, and only
// then does wave 0 raise the count.  After the wait, wave 0 invalidates the
// compute unit's vector cache (shared by the workgroup's waves) and the L2's
// stale lines once for the whole workgroup.  Cache maintenance per wave
// instead cost about 85 us per launch (it acts on a whole L2, and every wave
// of 32 workgroups per XCD queued two write-backs and two invalidations).
__device__ __forceinline__ void group_sync(int32_t* sync, int64_t g, int members, int tid) {
    // each wave's packed stores are complete before the workgroup meets
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid < 64) {
        if (tid == 0) {
            int32_t* arrived = sync + PACK_SYNC_HEAD + 2 * g;
            int32_t* left = arrived + 1;
            __hip_atomic_fetch_add(arrived, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            int polls = 0;
            while (__hip_atomic_load(arrived, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < members) {
                if (++polls > PACK_WAIT_POLLS) {
                    __hip_atomic_fetch_or(sync, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
            if (__hip_atomic_fetch_add(left, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == members - 1) {
                // every member has arrived and stopped reading the counts
                __hip_atomic_store(arrived, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(left, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        // the peers' bytes are then read afresh (the wait lets the
        // invalidation finish before the barrier)
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
}

// Pack this workgroup's share of its group and wait for the group.  The tile
// decomposition is the prefill's: tile = (token tile tm, row tile tn) with row
// tiles fastest, split ks of K.
template <int THREADS>
__device__ __forceinline__ void pack_group(const PackDst& P, int nb, int64_t M, int64_t TM, int64_t m0, int kb0,
                                           int nbk, int64_t tn, int64_t ntn, int64_t g, int tid) {
    const int64_t live = M - m0 < TM ? M - m0 : TM;
    pack_share<THREADS>(P, nb, m0, live, kb0, nbk, tn, ntn, tid);
    group_sync(P.sync, g, (int)ntn, tid);
}

}  // namespace q8k
