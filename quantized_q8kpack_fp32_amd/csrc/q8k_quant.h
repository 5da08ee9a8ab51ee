// q8_K quantisation of one 256-value block ("Language models on the device:
// the cajeta-llm kernels", section 1: 256 values a block, one scale and eight
// sub-block sums; the device quantiser of section 2.6).  Shared by the pack
// kernel and the mat-vecs that pack their own activations, so both produce
// the same bytes.
#pragma once
#include "q8k_device.h"

namespace q8k {

// Sixteen lanes per block: lane r of a 16-lane row (DPP row) holds values
// 16r..16r+15 in v[0..3].  The block scale is amax/127 (0 for an all-zero
// block); each value is rounded half-to-even from x * (127/amax), both fp32
// divisions correctly rounded, and clamped to [-127, 127].  amax is a max and
// the sums are integers, so any lane layout gives the same bytes.  Returns the
// 16 codes; `sub` is the sum of sub-block r/2 (lanes 2j and 2j+1 hold
// sub-block j).  Every lane of the row must be active.
__device__ __forceinline__ uint4 q8k_quant_lane16(const float4 (&v)[4], int& sub, float& d) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
#pragma unroll
    for (int k = 0; k < 4; ++k) amax = fmaxf(amax, dpp_f(amax, k));
    uint32_t words[4] = {0u, 0u, 0u, 0u};
    int s = 0;
    if (amax != 0.0f) {
        const float iscale = 127.0f / amax;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float xs[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float r = __builtin_rintf(xs[e] * iscale);
                if (r != r) r = 0.0f;  // 0 * inf when 127/amax overflows
                r = r > 127.0f ? 127.0f : r;
                r = r < -127.0f ? -127.0f : r;
                const int qi = (int)r;
                s += qi;
                words[i] |= (uint32_t)(qi & 255) << (8 * e);
            }
        }
    }
    s += __builtin_amdgcn_update_dpp(0, s, 0xB1, 0xF, 0xF, false);  // the pair's other lane (quad_perm 1,0,3,2)
    sub = s;
    d = amax != 0.0f ? amax / 127.0f : 0.0f;
    return make_uint4(words[0], words[1], words[2], words[3]);
}

}  // namespace q8k
