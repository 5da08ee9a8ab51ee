// Internal launch functions (host side), one per kernel family.  Arguments
// are validated by the C-ABI layer before any of these is called; each
// returns the hipError_t of its launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8k {

// Launch census: every launch notes its kernel's host handle for the calling
// thread (the C ABI resets the record at the start of each call), so a test
// can tell which kernels produced the values it checks ("One kernel, any
// device", section 5: every registered kernel must be value-checked by some
// test).
void note_launch(const void* kernel);
#define Q8K_LAUNCH(kernel, grid, block, lds, stream, ...)                         \
    do {                                                                          \
        ::q8k::note_launch(reinterpret_cast<const void*>(&kernel));               \
        hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);        \
    } while (0)

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
hipError_t launch_matvec_q5k(const uint8_t* w, int64_t rows, int nb, Acts a, int ncols, float* y, hipStream_t s);
// Weight formats of the prefill and fused kernels: Q4_K and Q5_K read one
// weight stream `w` (prefix unused); relaid Q6_K reads the bodies as `w` and
// the fp16 d prefix.
constexpr int WFMT_Q4_K = 0, WFMT_Q5_K = 1, WFMT_Q6_K = 2;

// Fused pack + mat-vec from fp32 activations [ncols][K] (fmt: WFMT_*).  The packed
// columns are also stored to `o` when o.qs is not null.  LDS per workgroup:
// the packed columns, fused_lds_bytes(ncols, K) <= FUSED_LDS_MAX.
struct PackedOut {
    int8_t* qs;
    float* d;
    int16_t* bs;
};
inline size_t fused_lds_bytes(int64_t ncols, int64_t K) { return (size_t)(ncols * (K + K / 256 * 20)); }
constexpr size_t FUSED_LDS_MAX = 65536;
hipError_t launch_matvec_f32(int fmt, const uint8_t* w, const uint16_t* prefix, int64_t rows, int nb, const float* x,
                             int64_t K, int ncols, float* y, PackedOut o, hipStream_t s);
hipError_t launch_moe_q4k(const uint8_t* w, int64_t E, int64_t rows, int nb, Acts a, int64_t T, const int32_t* ids,
                          const float* rw, int topk, float* y, hipStream_t s);
// Q4_K mixture-of-experts decode on the int8 matrix cores (moe_mfma.hip); it
// stages a token's packed row in LDS, so it serves K with moe_mfma_q4k_fits(K).
bool moe_mfma_q4k_fits(int64_t K);
// relaid Q6_K on the matrix cores (32x32x16 per 16-value sub-block); K with
// moe_mfma_q6k_fits(K), launch_moe_q6k beyond
bool moe_mfma_q6k_fits(int64_t K);
hipError_t launch_moe_mfma_q6k(const uint16_t* prefix, const uint8_t* bodies, int64_t E, int64_t rows, int nb, Acts a,
                               int64_t T, const int32_t* ids, const float* rw, int topk, float* y, hipStream_t s);
hipError_t launch_moe_mfma6_sums(const uint16_t* prefix, const uint8_t* bodies, int64_t E, int64_t rows, int nb,
                                 Acts a, int64_t T, const int32_t* ids, const float* rw, int topk, float* y,
                                 int32_t* S, hipStream_t s);
hipError_t launch_moe_mfma_q4k(const uint8_t* w, int64_t E, int64_t rows, int nb, Acts a, int64_t T,
                               const int32_t* ids, const float* rw, int topk, float* y, hipStream_t s);
hipError_t launch_moe_mfma_q5k(const uint8_t* w, int64_t E, int64_t rows, int nb, Acts a, int64_t T,
                               const int32_t* ids, const float* rw, int topk, float* y, hipStream_t s);
hipError_t launch_moe_q5k(const uint8_t* w, int64_t E, int64_t rows, int nb, Acts a, int64_t T, const int32_t* ids,
                          const float* rw, int topk, float* y, hipStream_t s);
hipError_t launch_moe_q6k(const uint16_t* prefix, const uint8_t* bodies, int64_t E, int64_t rows, int nb, Acts a,
                          int64_t T, const int32_t* ids, const float* rw, int topk, float* y, hipStream_t s);
// Split-K of the prefill ("Language models on the device", section 2.3): a
// problem whose 128-token x 64-row tiles number fewer than the device's 256
// compute units gets ksplit workgroups along the reduction, each with at least
// PREFILL_SPLIT_MIN_BLOCKS blocks of K; their fp32 partials [ksplit][M][rows]
// live in the caller's workspace and a fixup kernel adds them in split order.
constexpr int PREFILL_TARGET_WGS = 256;
constexpr int PREFILL_SPLIT_MAX = 8;
constexpr int PREFILL_SPLIT_MIN_BLOCKS = 8;
inline int prefill_ksplit(int64_t rows, int64_t nb, int64_t M) {
    const int64_t tiles = ((rows + 63) / 64) * ((M + 127) / 128);
    if (tiles <= 0 || tiles >= PREFILL_TARGET_WGS) return 1;
    int64_t k = (PREFILL_TARGET_WGS + tiles - 1) / tiles;
    if (k > PREFILL_SPLIT_MAX) k = PREFILL_SPLIT_MAX;
    if (k > nb / PREFILL_SPLIT_MIN_BLOCKS) k = nb / PREFILL_SPLIT_MIN_BLOCKS;
    return k < 1 ? 1 : (int)k;
}
// part: the workspace (ksplit * M * rows fp32) when prefill_ksplit(...) > 1.
hipError_t launch_prefill(int fmt, const uint8_t* w, const uint16_t* prefix, int64_t rows, int nb, Acts a, int64_t M,
                          float* y, float* part, hipStream_t s);
hipError_t launch_prefill_fixup(const float* part, int ksplit, int64_t n, float* y, hipStream_t s);
// The prefill from fp32 tokens with the q8_K pack inside the launch
// (prefill_pack.h): the tiles' workgroups pack their group's blocks into the
// q8_K buffer (qs, d, bs) and meet on sync words in the caller's workspace:
// word 0 the error word, then two words per group (token tile x K split),
// zero before the first call.  The split-K partials follow the sync words.
struct PackDst {
    const float* x;  // fp32 tokens [M][K]
    int8_t* qs;      // the q8_K buffer's sections (act_layout(M, K))
    float* d;
    int16_t* bs;
    int32_t* sync;
};
constexpr int PACK_SYNC_HEAD = 4;  // words before the first group's
inline int64_t prefill_groups(int64_t M, int ksplit) { return ((M + 127) / 128) * ksplit; }
inline int64_t prefill_sync_bytes(int64_t M, int ksplit) {
    return (4 * (PACK_SYNC_HEAD + 2 * prefill_groups(M, ksplit)) + 255) / 256 * 256;
}
// Compute units of the current device (asked once per device): a group of
// workgroups that wait for each other must fit on the device together.
int64_t device_cu_count();
hipError_t launch_prefill_f32(int fmt, const uint8_t* w, const uint16_t* prefix, int64_t rows, int nb, Acts a,
                              int64_t M, float* y, float* part, PackDst pk, hipStream_t s);
// Q4_K prefill with the weight planes built in the registers of the waves that
// multiply them (prefill_regw.hip).
hipError_t launch_prefill_regw_q4k(const uint8_t* w, int64_t rows, int nb, Acts a, int64_t M, float* y, int ksplit,
                                   float* part, hipStream_t s);
hipError_t launch_prefill_regw_q4k_f32(const uint8_t* w, int64_t rows, int nb, Acts a, int64_t M, float* y,
                                       int ksplit, float* part, PackDst pk, hipStream_t s);
// The same tile over the chunks of a mixture-of-experts prefill (T tokens;
// chunk table and pair order as in the workspace below; out: [P][rows]).
hipError_t launch_prefill_regw_moe_q4k(const uint8_t* w, int64_t rows, int nb, Acts a, int64_t T, int64_t max_chunks,
                                       const int32_t* nchunks, const int4* chunks, const int32_t* order, int topk,
                                       float* out, hipStream_t s);

// Workspace of the MoE prefill, byte offsets from its start: the fp32 result
// of every (token, slot) pair [P][rows]; then, 256-aligned, the chunk count
// (int32, padded to 16 bytes), the chunk table (int4 {expert, first index in
// order, count, 0} per chunk) and `order` (the P pair indices grouped by
// expert).  P pairs over E experts make at most floor(P / 128) + min(E, P)
// chunks of at most 128 pairs: each expert with n > 0 pairs makes
// ceil(n / 128) <= floor(n / 128) + 1 of them.  No workspace is needed when
// there are no pairs or no rows.
constexpr int MOE_GROUP_MAX_E = 4096;  // most experts the grouping kernel counts in LDS
struct MoePrefillWs {
    int64_t P, max_chunks;
    int64_t meta, chunks, order, total;
};
inline int64_t align256(int64_t b) { return (b + 255) / 256 * 256; }
inline MoePrefillWs moe_prefill_ws(int64_t E, int64_t rows, int64_t T, int64_t topk) {
    MoePrefillWs L;
    L.P = T * topk;
    L.max_chunks = L.P / 128 + (E < L.P ? E : L.P);
    L.meta = align256(L.P * rows * 4);
    L.chunks = L.meta + 16;
    L.order = L.chunks + 16 * L.max_chunks;
    L.total = (L.P == 0 || rows == 0) ? 0 : align256(L.order + 4 * L.P);  // nothing is enqueued then
    return L;
}
// Allocation-free MoE prefill: the device address of the library's own
// scratch array (NOALLOC_SCRATCH_BYTES on every device), found on the first
// call per device.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)64 << 20;
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_prefill_moe(int fmt, const uint8_t* w, const uint16_t* prefix, int64_t E, int64_t rows, int nb,
                              Acts a, int64_t T, const int32_t* ids, const float* rw, int topk, float* y, void* ws,
                              hipStream_t s);

// ---- test support: the shipped kernels' integer sums (template flags of the
// same kernels, which also write y as they ship)
// qmatvec's kernel for one packed token: y [rows] and the exact sub-block sums
// S [rows][nb][8] (Q4_K, Q5_K) or [rows][nb][16] (relaid Q6_K).
hipError_t launch_matvec_sums(int fmt, const uint8_t* w, const uint16_t* prefix, int64_t rows, int nb, Acts a,
                              float* y, int32_t* S, hipStream_t s);
// qmatmul_prefill's tile: y [M][rows] and the block sums I [M][rows][nb]
// (sum_j sc_j * S_j per block, the integer the tile folds into y).
hipError_t launch_prefill_sums(int fmt, const uint8_t* w, const uint16_t* prefix, int64_t rows, int nb, Acts a,
                               int64_t M, float* y, int32_t* I, hipStream_t s);
hipError_t launch_prefill_regw_q4k_sums(const uint8_t* w, int64_t rows, int nb, Acts a, int64_t M, float* y,
                                        int32_t* I, hipStream_t s);
// qmatvec_moe's matrix-core kernel (Q4_K, Q5_K): y [T][rows] and the sub-block
// sums S [T * topk][rows][nb][8] of every (token, slot) pair that selects an
// expert in [0, E) (other pairs' entries are not written).
// The wave reduction on closed-form inputs: out [5] (four wave sums, total).
hipError_t launch_wave_sums(float* out, hipStream_t s);
hipError_t launch_moe_mfma_sums(bool q5, const uint8_t* w, int64_t E, int64_t rows, int nb, Acts a, int64_t T,
                                const int32_t* ids, const float* rw, int topk, float* y, int32_t* S, hipStream_t s);

}  // namespace q8k
