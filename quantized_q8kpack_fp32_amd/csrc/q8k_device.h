// Internal device helpers for the gfx950 kernels (wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q8k {

constexpr int QK = 256;          // values per K-quant super-block and q8_K block
constexpr int Q4K_BLOCK = 144;   // GGUF Q4_K block bytes
constexpr int Q5K_BLOCK = 176;   // GGUF Q5_K block bytes
constexpr int Q6K_BLOCK = 210;   // GGUF Q6_K block bytes
constexpr int Q6K_BODY = 208;    // Q6_K body after the bind relayout
constexpr int WAVE = 64;

__host__ __device__ constexpr size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// q8_K activation buffer sections (see include/q8k.h).
struct ActLayout {
    size_t off_d, off_bs, total;
};
__host__ __device__ inline ActLayout act_layout(int64_t T, int64_t K) {
    ActLayout l;
    size_t nb = (size_t)T * (size_t)(K / QK);
    l.off_d = align256((size_t)T * (size_t)K);
    l.off_bs = align256(l.off_d + 4 * nb);
    l.total = align256(l.off_bs + 2 * 8 * nb);
    return l;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// Raw buffer resource over [base, base + bytes): a read at a byte offset at
// or past `bytes` returns zeros and touches no memory.  The record count is a
// 32-bit field, so ranges are capped at 2^31 - 1 bytes; callers keep their
// offsets below that.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
// (The clamp compares the two 32-bit halves: the scalar unit has no signed
// 64-bit compare, and a wave-uniform range should not cost vector
// instructions.)
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int hi = (int)(bytes >> 32);
    const uint32_t lo = (uint32_t)bytes;
    const uint32_t lim = hi < 0 ? 0u : hi > 0 ? 0x7fffffffu : (lo < 0x7fffffffu ? lo : 0x7fffffffu);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)lim,
                                             0x00020000 /* raw, untyped dwords */);
}
__device__ __forceinline__ uint4 load16(rsrc_t r, int off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint2 load8(rsrc_t r, int off) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t load4(rsrc_t r, int off) { return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0); }
__device__ __forceinline__ uint32_t load2(rsrc_t r, int off) { return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0); }

// A 16-byte weight load, non-temporal when NT (the weights of the Q4_K decode
// mat-vec, read once per launch: a plain streaming read is fastest with the
// hint on gfx950, and the Q4_K mat-vec measured 6% faster with it; Q5_K,
// Q6_K and the MoE decode measured slower, because some of their 128-byte
// lines are touched by more than one load and the hint evicts them between).
typedef unsigned int v4u_nt __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ uint4 wload16(const void* p) {
    if constexpr (NT) {
        const v4u_nt v = __builtin_nontemporal_load(static_cast<const v4u_nt*>(p));
        return make_uint4(v[0], v[1], v[2], v[3]);
    } else {
        return *static_cast<const uint4*>(p);
    }
}

// int8x4 . int8x4 + acc, signed (v_dot4_i32_i8).
__device__ __forceinline__ int sdot4(int a, int b, int acc) { return __builtin_amdgcn_sdot4(a, b, acc, false); }

// Butterfly sums / max over the 64 lanes of a wavefront.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, WAVE);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, WAVE));
    return v;
}

__device__ __forceinline__ uint32_t byte_of(uint4 v, int i) {
    uint32_t w = (i < 4) ? v.x : (i < 8) ? v.y : (i < 12) ? v.z : v.w;
    return (w >> (8 * (i & 3))) & 0xffu;
}

}  // namespace q8k

namespace q8k {

// DPP lane shuffles (gfx9 encodings): quad_perm [1,0,3,2] and [2,3,0,1],
// row_ror:4 and row_ror:8 within each 16-lane row.
__device__ __forceinline__ float dpp_f(float v, int ctrl_id) {
    const int x = __builtin_bit_cast(int, v);
    int r;
    switch (ctrl_id) {
        case 0: r = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false); break;   // quad_perm 1,0,3,2
        case 1: r = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false); break;   // quad_perm 2,3,0,1
        case 2: r = __builtin_amdgcn_update_dpp(0, x, 0x124, 0xF, 0xF, false); break;  // row_ror:4
        default: r = __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false); break; // row_ror:8
    }
    return __builtin_bit_cast(float, r);
}

// Sum over all 64 lanes of a wavefront (all lanes must be active); the total
// is returned in every lane.  Four DPP steps give each 16-lane row its sum,
// then the four row sums are read as scalars.
__device__ __forceinline__ float wave_sum_dpp(float v) {
    v += dpp_f(v, 0);
    v += dpp_f(v, 1);
    v += dpp_f(v, 2);
    v += dpp_f(v, 3);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (r0 + r1) + (r2 + r3);
}

}  // namespace q8k
