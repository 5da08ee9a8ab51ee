// q8_K activation packing and the bind-time Q6_K relayout.
//
// q8_K: 256 values a block, one scale and eight sub-block sums ("Language
// models on the device: the cajeta-llm kernels", section 1; the device
// quantiser is listed among the utility kernels of section 2.6).
// Q6_K relayout: split each block into a scale prefix and a 208-byte body so
// that kernels read bodies with aligned 16-byte loads (same page, section 1).
#include "q8k_device.h"
#include "q8k_launch.h"
#include "q8k_quant.h"

namespace q8k {

// Sixteen lanes per 256-value block, 16 values each (four 16-byte loads), so
// a 256-thread workgroup packs 16 blocks and every reduction stays in DPP row
// operations (a shuffle-based wave-per-block form took 9.0 us for 512 x 14336
// values against 6.3 us for this one).
__global__ __launch_bounds__(256) void pack_kernel(const float* __restrict__ x, int64_t nblocks,
                                                   int8_t* __restrict__ qs, float* __restrict__ d,
                                                   int16_t* __restrict__ bsums) {
    const int64_t blk = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int r = threadIdx.x & 15;
    if (blk >= nblocks) return;  // uniform per 16-lane row
    const float4* src = reinterpret_cast<const float4*>(x + blk * QK + 16 * r);
    const float4 v[4] = {src[0], src[1], src[2], src[3]};
    int s;
    float dd;
    const uint4 codes = q8k_quant_lane16(v, s, dd);
    *reinterpret_cast<uint4*>(qs + blk * QK + 16 * r) = codes;
    if ((r & 1) == 0) bsums[blk * 8 + (r >> 1)] = (int16_t)s;
    if (r == 0) d[blk] = dd;
}

hipError_t launch_pack(const float* x, int64_t nblocks, int8_t* qs, float* d, int16_t* bsums, hipStream_t s) {
    Q8K_LAUNCH(pack_kernel, dim3((unsigned)((nblocks + 15) / 16)), dim3(256), 0, s, x, nblocks, qs, d, bsums);
    return hipGetLastError();
}

// One wavefront per block.  The 210-byte source blocks are only 2-byte
// aligned: lanes 0..51 each assemble one 32-bit word of the body from two
// halfwords; lane 52 moves the fp16 scale into the prefix.
__global__ __launch_bounds__(256) void bind_q6k_kernel(const uint8_t* __restrict__ src, int64_t nblocks,
                                                       uint16_t* __restrict__ prefix, uint8_t* __restrict__ bodies) {
    const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (blk >= nblocks) return;
    const uint16_t* s16 = reinterpret_cast<const uint16_t*>(src + blk * Q6K_BLOCK);
    if (lane < Q6K_BODY / 4) {
        const uint32_t word = (uint32_t)s16[2 * lane] | ((uint32_t)s16[2 * lane + 1] << 16);
        reinterpret_cast<uint32_t*>(bodies + blk * Q6K_BODY)[lane] = word;
    } else if (lane == Q6K_BODY / 4) {
        prefix[blk] = s16[Q6K_BODY / 2];
    }
}

hipError_t launch_bind_q6k(const uint8_t* src, int64_t nblocks, uint16_t* prefix, uint8_t* bodies, hipStream_t s) {
    const int64_t grid = (nblocks + 3) / 4;
    Q8K_LAUNCH(bind_q6k_kernel, dim3((unsigned)grid), dim3(256), 0, s, src, nblocks, prefix, bodies);
    return hipGetLastError();
}

}  // namespace q8k
