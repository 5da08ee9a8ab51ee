// Internal launch functions (host side), one per kernel family.  Arguments
// are validated by the C-ABI layer before any of these is called; each
// returns the hipError_t of its launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8k {

hipError_t launch_pack(const float* x, int64_t nblocks, int8_t* qs, float* d, int16_t* bsums, hipStream_t s);
hipError_t launch_bind_q6k(const uint8_t* src, int64_t nblocks, uint16_t* prefix, uint8_t* bodies, hipStream_t s);

// Packed-token view: T tokens, K values each, sections as in act_layout().
struct Acts {
    const int8_t* qs;
    const float* d;
    const int16_t* bs;
    int64_t K;
};

hipError_t launch_matvec_q4k(const uint8_t* w, int64_t rows, int nb, Acts a, int ncols, float* y, hipStream_t s);
hipError_t launch_matvec_q6k(const uint16_t* prefix, const uint8_t* bodies, int64_t rows, int nb, Acts a, int ncols,
                             float* y, hipStream_t s);
hipError_t launch_sums_q4k(const uint8_t* w, int64_t rows, int nb, Acts a, int32_t* S, hipStream_t s);
hipError_t launch_matvec_q5k(const uint8_t* w, int64_t rows, int nb, Acts a, int ncols, float* y, hipStream_t s);
hipError_t launch_sums_q5k(const uint8_t* w, int64_t rows, int nb, Acts a, int32_t* S, hipStream_t s);
hipError_t launch_sums_q6k(const uint16_t* prefix, const uint8_t* bodies, int64_t rows, int nb, Acts a, int32_t* S,
                           hipStream_t s);
hipError_t launch_moe_q4k(const uint8_t* w, int64_t E, int64_t rows, int nb, Acts a, int64_t T, const int32_t* ids,
                          const float* rw, int topk, float* y, hipStream_t s);
hipError_t launch_moe_q5k(const uint8_t* w, int64_t E, int64_t rows, int nb, Acts a, int64_t T, const int32_t* ids,
                          const float* rw, int topk, float* y, hipStream_t s);
hipError_t launch_moe_q6k(const uint16_t* prefix, const uint8_t* bodies, int64_t E, int64_t rows, int nb, Acts a,
                          int64_t T, const int32_t* ids, const float* rw, int topk, float* y, hipStream_t s);
hipError_t launch_prefill_q4k(const uint8_t* w, int64_t rows, int nb, Acts a, int64_t M, float* y, hipStream_t s);
hipError_t launch_prefill_moe_q4k(const uint8_t* w, int64_t E, int64_t rows, int nb, Acts a, int64_t T,
                                  const int32_t* ids, const float* rw, int topk, float* y, float* ws, hipStream_t s);

}  // namespace q8k
