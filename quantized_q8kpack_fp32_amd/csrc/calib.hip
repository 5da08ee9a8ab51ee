// Streaming-read calibration for the benchmark (not part of libq8k): a plain
// read-only kernel that moves `bytes` from device memory with 16-byte loads,
// so each bandwidth-bound workload can be reported against what a plain read
// of the same bytes achieves on the same device, beside the nominal HBM peak
// (the measurement discipline of "One kernel, any device", section 5: a
// number is read against the ceiling it can reach).
//
// Each thread issues U 16-byte loads before using any of them; load u of a
// workgroup covers 4 KB of contiguous bytes (consecutive lanes, consecutive
// 16-byte words), and the grid strides over the buffer.  The loaded words are
// folded with XOR into one word per workgroup, stored to `sink`, so no load
// can be removed.  A few variants (loads per thread, non-temporal loads) are
// built; the benchmark times each and takes the fastest as the ceiling.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int CAL_THREADS = 256;
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// U 16-byte loads per thread per trip, issued before any is used; NT: loads
// marked non-temporal (streamed data that will not be reused).
template <int U, bool NT>
__global__ __launch_bounds__(CAL_THREADS) void stream_read_kernel(const uint4* __restrict__ buf, int64_t n16,
                                                                  uint32_t* __restrict__ sink) {
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * CAL_THREADS * U;
    for (int64_t i = (int64_t)blockIdx.x * CAL_THREADS * U + threadIdx.x; i < n16; i += stride) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t k = i + (int64_t)u * CAL_THREADS;
            if (k < n16) {
                if constexpr (NT) {
                    const v4u w = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(buf) + k);
                    v[u] = make_uint4(w[0], w[1], w[2], w[3]);
                } else {
                    v[u] = buf[k];
                }
            } else {
                v[u] = make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    // one word per workgroup: a wave-level fold, then lane 0 of each wave
    for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
    __shared__ uint32_t part[CAL_THREADS / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

constexpr int CAL_VARIANTS = 6;
constexpr int CAL_U[CAL_VARIANTS] = {1, 2, 4, 8, 2, 4};  // loads per lane; variants 4 and 5 non-temporal
constexpr int64_t CAL_GRID_CAP = 8192;

int64_t workgroups(int64_t bytes, int variant) {
    const int64_t trip = (int64_t)CAL_THREADS * CAL_U[variant] * 16;
    const int64_t trips = (bytes + trip - 1) / trip;
    return trips < 1 ? 1 : trips < CAL_GRID_CAP ? trips : CAL_GRID_CAP;
}

}  // namespace

extern "C" {

int q8k_calib_stream_variants(void) { return CAL_VARIANTS; }

// Words the sink of one streaming read needs (the most workgroups of any variant).
int64_t q8k_calib_stream_workgroups(int64_t bytes) { return workgroups(bytes, 0); }

// Read `bytes` (a multiple of 16) from buf with variant v (0 <= v <
// q8k_calib_stream_variants()): 0 on success, else the HIP error.
int q8k_calib_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int variant, void* stream) {
    if (!buf || !sink || bytes <= 0 || bytes % 16 != 0 || ((uintptr_t)buf & 15) != 0 || variant < 0 ||
        variant >= CAL_VARIANTS)
        return (int)hipErrorInvalidValue;
    const dim3 grid((unsigned)workgroups(bytes, variant)), block(CAL_THREADS);
    const uint4* b = static_cast<const uint4*>(buf);
    const int64_t n = bytes / 16;
    hipStream_t s = (hipStream_t)stream;
    switch (variant) {
        case 0: hipLaunchKernelGGL((stream_read_kernel<1, false>), grid, block, 0, s, b, n, sink); break;
        case 1: hipLaunchKernelGGL((stream_read_kernel<2, false>), grid, block, 0, s, b, n, sink); break;
        case 2: hipLaunchKernelGGL((stream_read_kernel<4, false>), grid, block, 0, s, b, n, sink); break;
        case 3: hipLaunchKernelGGL((stream_read_kernel<8, false>), grid, block, 0, s, b, n, sink); break;
        case 4: hipLaunchKernelGGL((stream_read_kernel<2, true>), grid, block, 0, s, b, n, sink); break;
        default: hipLaunchKernelGGL((stream_read_kernel<4, true>), grid, block, 0, s, b, n, sink); break;
    }
    return (int)hipGetLastError();
}

}  // extern "C"
