/*
 * q8k.h -- C ABI of libq8k: GGUF K-quant weights (Q4_K, Q5_K, Q6_K) times
 * activations packed on the GPU into q8_K blocks, on AMD Instinct MI355X
 * (gfx950).
 *
 * The operations follow "Language models on the device: the cajeta-llm
 * kernels" (cajeta.dev/xpu/kernels-llm/):
 *   - section 1: weights arrive in GGUF K-quant blocks (256 values, per
 *     sub-block scales); activations are quantised on the device to q8_K
 *     (256 values a block, one scale, eight sub-block sums); an integer dot
 *     product does the arithmetic and the per-sub-block scales and mins are
 *     applied in an epilogue; at bind, Q6_K blocks may be split into a scale
 *     prefix and 208-byte bodies so kernels read them with aligned 16-byte
 *     loads;
 *   - section 2.1: decode mat-vec, one wavefront owns one output row;
 *   - section 2.2: batched decode, one pass over a weight row serves several
 *     activation columns;
 *   - section 2.3: prefill, a tiled matrix-core GEMM with a scale epilogue;
 *     a Q5_K member is the Q4_K one with the fifth-bit plane supplying bit
 *     four of each value (every operation here serves Q4_K, Q5_K and relaid
 *     Q6_K weights, the prefill and its MoE form included);
 *   - section 2.4: mixture of experts, a decode mat-vec that visits each
 *     token's selected experts and sums their weighted outputs, and the
 *     prefill form that runs the prefill tile per expert chunk;
 *   - section 3.2 (and SKaiNET's "Kernel SPI and the selection algorithm",
 *     decline reasons): the input width must be a multiple of 256.
 *
 * Conventions for every entry point
 *   - Buffers are device pointers owned by the caller; the library never
 *     allocates and never synchronises.  Its only state: the calling
 *     thread's last-error text and launch record (q8k_debug_last_launches),
 *     the compute-unit count of each device, asked of the runtime once (it
 *     sizes the MoE decode grid and bounds qmatmul_prefill_f32), and the
 *     static device scratch of qmatmul_prefill_moe_noalloc with its address
 *     on each device (below).  Buffers must stay alive until the work
 *     enqueued on `stream` has finished.
 *   - `stream` is a hipStream_t (NULL = the default stream).
 *   - Arguments are validated on the host before anything is enqueued.  A
 *     refusal returns a non-zero q8k_status, enqueues nothing, leaves every
 *     output untouched and sets q8k_last_error() to a message naming the
 *     rule and the values.  Refusals are never replaced by a fallback.
 *   - Q8K_OK means the kernels were enqueued and will overwrite every element
 *     of the outputs (nothing is accumulated into what the caller passed).
 *   - Sizes: K (the reduction width) must be a positive multiple of 256.
 *     Zero rows / tokens are accepted and enqueue nothing.
 *   - Alignment: weights, packed activations, fp32 inputs and workspaces must
 *     be 16-byte aligned; fp32 outputs, ids and router weights 4-byte aligned.
 *   - Device-side values are not inspected (that would need a sync): x must be
 *     finite; an expert id outside [0, E) selects nothing.
 */
#ifndef Q8K_H
#define Q8K_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    Q8K_OK = 0,
    Q8K_ERR_NULL = 1,      /* a required pointer is NULL                        */
    Q8K_ERR_SHAPE = 2,     /* K not a positive multiple of 256, negative size,  */
                           /* or a size beyond the supported maximum            */
    Q8K_ERR_ALIGN = 3,     /* a pointer is not aligned as required              */
    Q8K_ERR_QTYPE = 4,     /* weight format not served by this entry point      */
    Q8K_ERR_ARG = 5,       /* topk / ncols / E / token count out of range       */
    Q8K_ERR_WORKSPACE = 6, /* workspace smaller than the size helper reports    */
    Q8K_ERR_LAUNCH = 7     /* the HIP runtime refused the launch                */
} q8k_status;

typedef enum {
    Q8K_Q4_K = 1,        /* GGUF Q4_K: 144-byte blocks, row-major block order   */
    Q8K_Q6_K_RELAID = 2, /* Q6_K after q8k_bind_q6k: fp16 prefix + 208-B bodies */
    Q8K_Q6_K_GGUF = 3,   /* raw GGUF Q6_K (210-byte blocks): bind input only    */
    Q8K_Q5_K = 4         /* GGUF Q5_K: 176-byte blocks, row-major block order   */
} q8k_qtype;

#define Q8K_QK 256         /* values per K-quant super-block / q8_K block       */
#define Q8K_COLS_MAX 8     /* most activation columns qmatvec_batched serves    */
#define Q8K_MOE_MAX_TOKENS 256 /* most tokens qmatvec_moe serves per call       */
#define Q8K_MOE_MAX_TOPK 64    /* most experts per token qmatvec_moe serves     */

/* ---------------------------------------------------------------- sizing --
 * q8_K activation buffer for T tokens of K values: three sections, each
 * starting on a 256-byte boundary:
 *   qs    int8  [T][K]          at offset 0
 *   d     fp32  [T][K/256]      at *off_d      (block scale, amax/127)
 *   bsums int16 [T][K/32]       at *off_bsums  (sum of the 32 codes of each of
 *                                               the block's eight sub-blocks)
 * Returns the total size in bytes (0 if K is not a positive multiple of 256
 * or T < 0).  off_d / off_bsums may be NULL. */
size_t q8k_act_bytes(int64_t T, int64_t K);
size_t q8k_act_layout(int64_t T, int64_t K, size_t* off_d, size_t* off_bsums);

/* Bytes of a rows x K weight in the given layout (0 on a bad shape):
 *   Q8K_Q4_K         rows*K/256 blocks of 144 B;
 *   Q8K_Q5_K         rows*K/256 blocks of 176 B;
 *   Q8K_Q6_K_GGUF    rows*K/256 blocks of 210 B;
 *   Q8K_Q6_K_RELAID  fp16 d prefix [rows*K/256] padded to 256 B, then
 *                    rows*K/256 bodies of 208 B (ql[128] | qh[64] | scales[16]);
 *                    block (r, b) is entry r*K/256 + b of both arrays. */
size_t q8k_weight_bytes(int qtype, int64_t rows, int64_t K);

/* ------------------------------------------------------------ operations --
 * q8k_pack: quantise x (fp32 [T][K], row-major) into the q8_K buffer xq.
 * Per 256-value block: amax = max |x|; d = amax/127 (0 for an all-zero
 * block); qs = round-half-even(x * (127/amax)) clamped to [-127, 127], all in
 * fp32 (correctly rounded division, single multiply); bsums = int16 sums of
 * the eight 32-value groups of qs. */
int q8k_pack(const float* x, int64_t T, int64_t K, void* xq, void* stream);

/* q8k_bind_q6k: bind-time relayout of a raw GGUF Q6_K weight (rows x K) into
 * the Q8K_Q6_K_RELAID layout (scale prefix + 208-byte bodies).  Byte moves
 * only.  w_gguf may be 2-byte aligned; w_relaid must be 16-byte aligned and
 * q8k_weight_bytes(Q8K_Q6_K_RELAID, rows, K) long. */
int q8k_bind_q6k(const void* w_gguf, int64_t rows, int64_t K, void* w_relaid, void* stream);

/* qmatvec: decode mat-vec for one packed token.
 *   y[r] = sum_b d8_b * (d_rb * sum_j sc_rbj * S_rbj - dmin_rb * sum_j m_rbj * bsums_bj)   (Q4_K, Q5_K)
 *   y[r] = sum_b d8_b * d_rb * sum_s sc_rbs * S_rbs                                        (Q6_K)
 * with S the exact int32 sub-block sums of quant x code (Q6_K quants minus 32;
 * Q5_K quants 0..31 with the fifth bit from the block's qh plane).
 * qtype: Q8K_Q4_K, Q8K_Q5_K or Q8K_Q6_K_RELAID.  xq: q8_K buffer of one token (T = 1).
 * y: fp32 [rows]. */
int qmatvec(int qtype, const void* w, int64_t rows, int64_t K, const void* xq, float* y, void* stream);

/* qmatvec_batched: the same for ncols packed tokens (1 <= ncols <=
 * Q8K_COLS_MAX), each weight row read once for all columns.
 * xq: q8_K buffer of T = ncols tokens.  y: fp32 [ncols][rows]. */
int qmatvec_batched(int qtype, const void* w, int64_t rows, int64_t K, const void* xq, int64_t ncols, float* y,
                    void* stream);

/* qmatvec_f32: the decode step in one launch, from fp32 activations.  Each
 * workgroup first packs the ncols columns x [ncols][K] to q8_K in its own
 * shared memory, with the same arithmetic as q8k_pack, then runs
 * qmatvec_batched's arithmetic on them: y equals q8k_pack followed by
 * qmatvec_batched bit for bit, without the packed activations' round trip
 * through global memory or the second launch (the fused launches of
 * "Language models on the device", sections 1 and 3.3; a q|k|v or gate|up
 * weight concatenated row-wise is one weight here, so one launch serves all
 * of its parts).
 * qtype: Q8K_Q4_K, Q8K_Q5_K or Q8K_Q6_K_RELAID.  1 <= ncols <= Q8K_COLS_MAX
 * and ncols * (K + K/256 * 20) <= 65536 bytes (the packed columns fit one
 * workgroup's shared memory), else Q8K_ERR_ARG / Q8K_ERR_SHAPE.  x: fp32
 * [ncols][K], 16-byte aligned.  xq_out: NULL, or a q8_K buffer of ncols
 * tokens (q8k_act_bytes(ncols, K)) that also receives the packed columns,
 * for further mat-vecs of the same tokens.  y: fp32 [ncols][rows]. */
int qmatvec_f32(int qtype, const void* w, int64_t rows, int64_t K, const float* x, int64_t ncols, float* y,
                void* xq_out, void* stream);

/* qmatvec_moe: expert-indexed decode.  w holds E experts, each a rows x K
 * weight in the given layout, expert e's blocks following expert e-1's.
 * xq: q8_K buffer of T tokens (0 <= T <= Q8K_MOE_MAX_TOKENS); ids int32
 * [T][topk]; rw fp32 [T][topk]; 1 <= topk <= min(E, Q8K_MOE_MAX_TOPK).
 *   y[t][r] = sum_k rw[t][k] * (W_{ids[t][k]} x_t)[r]
 * Each expert row that at least one token selected is read once for all of
 * its tokens; an expert nobody selected is not read.  y: fp32 [T][rows]. */
int qmatvec_moe(int qtype, const void* w, int64_t E, int64_t rows, int64_t K, const void* xq, int64_t T,
                const int32_t* ids, const float* rw, int32_t topk, float* y, void* stream);

/* qmatmul_prefill: y[m][n] = qmatvec's formula for every token m < M and
 * weight row n < rows, computed as a tiled int8 matrix-core GEMM.
 * qtype: Q8K_Q4_K, Q8K_Q5_K or Q8K_Q6_K_RELAID (raw Q8K_Q6_K_GGUF is
 * refused with Q8K_ERR_QTYPE: bind it first).  xq: q8_K buffer of M tokens.
 * y: fp32 [M][rows].
 * ws / ws_bytes: caller-owned workspace of at least
 * qmatmul_prefill_workspace_bytes(...) bytes, 16-byte aligned (may be NULL
 * when that is 0).  It is non-zero when the problem's 128-token x 64-row tiles
 * are fewer than the 256 compute units of the device: the reduction is then
 * split across S <= 8 workgroups (at least 8 blocks of K each; split-K and its
 * fixup, "Language models on the device", section 2.3) and the workspace holds
 * their fp32 partials, S * M * rows * 4 bytes, added in a fixed order. */
size_t qmatmul_prefill_workspace_bytes(int qtype, int64_t rows, int64_t K, int64_t M);
int qmatmul_prefill(int qtype, const void* w, int64_t rows, int64_t K, const void* xq, int64_t M, float* y, void* ws,
                    size_t ws_bytes, void* stream);

/* qmatmul_prefill_f32: qmatmul_prefill from fp32 tokens, with the q8_K pack
 * inside the same launch (the fused launches of "Language models on the
 * device", sections 1 and 3.3).  The workgroups that share a 128-token tile
 * and a K range first pack that tile's blocks into xq, each an equal share,
 * with q8k_pack's arithmetic, and wait for one another before multiplying:
 * xq receives exactly q8k_pack's bytes and y equals q8k_pack followed by
 * qmatmul_prefill bit for bit.
 * qtype, w, rows, K, M, y: as qmatmul_prefill.  x: fp32 [M][K], 16-byte
 * aligned.  xq: a q8_K buffer of M tokens (q8k_act_bytes(M, K) bytes,
 * 16-byte aligned), written by the call; it must not overlap x, y or ws.
 * ws / ws_bytes: caller-owned workspace of at least
 * qmatmul_prefill_f32_workspace_bytes(...) bytes, 16-byte aligned, never NULL
 * (for M, rows > 0).  It starts with the sync words of the waiting
 * workgroups, which must be zero before the first call with this workspace;
 * every call leaves them zero, so stream-ordered calls may share it (calls
 * that overlap in time may not).  The split-K partials of qmatmul_prefill
 * follow them.  The int32 at ws[0] is an error word: a workgroup that has
 * polled for its peers 2^20 times (far longer than any call takes) gives up,
 * sets it to non-zero and finishes (its results are then not valid); the
 * library never clears it.
 * The workgroups of one token tile wait for each other, so they must fit on
 * the device together: ceil(rows / 64) may not exceed the device's compute
 * units (256 on MI355X: rows <= 16384), else Q8K_ERR_SHAPE (use q8k_pack +
 * qmatmul_prefill); this check asks the runtime for the compute-unit count. */
size_t qmatmul_prefill_f32_workspace_bytes(int qtype, int64_t rows, int64_t K, int64_t M);
int qmatmul_prefill_f32(int qtype, const void* w, int64_t rows, int64_t K, const float* x, int64_t M, void* xq,
                        float* y, void* ws, size_t ws_bytes, void* stream);

/* qmatmul_prefill_moe: the prefill of a mixture-of-experts layer ("Language
 * models on the device", section 2.4: each expert's (token, slot) pairs are
 * grouped into chunks and the prefill tile runs per expert and chunk).
 * Same weights, tokens, ids, router weights and result as qmatvec_moe,
 *   y[t][r] = sum_k rw[t][k] * (W_{ids[t][k]} x_t)[r],
 * for T tokens (0 <= T, T * K < 2^30) instead of at most 256.
 * qtype: Q8K_Q4_K, Q8K_Q5_K or Q8K_Q6_K_RELAID (w: E experts' weights
 * bound as one E*rows-row matrix).  1 <= E <= 4096;
 * 1 <= topk <= min(E, Q8K_MOE_MAX_TOPK).  An id outside [0, E) selects
 * nothing.  ws / ws_bytes: caller-owned workspace, 16-byte aligned, of at
 * least qmatmul_prefill_moe_workspace_bytes(...) bytes, not overlapping y:
 * the fp32 result of every (token, slot) pair, then the pairs grouped by
 * expert and the chunk table (about 4 * T * topk * (rows + 1) bytes; 0 when
 * T or rows is 0).  Its contents are scratch: stream-ordered calls may share
 * one workspace, calls that overlap in time may not.  y: fp32 [T][rows]. */
size_t qmatmul_prefill_moe_workspace_bytes(int qtype, int64_t E, int64_t rows, int64_t K, int64_t T, int32_t topk);
int qmatmul_prefill_moe(int qtype, const void* w, int64_t E, int64_t rows, int64_t K, const void* xq, int64_t T,
                        const int32_t* ids, const float* rw, int32_t topk, float* y, void* ws, size_t ws_bytes,
                        void* stream);

/* qmatmul_prefill_moe_noalloc: qmatmul_prefill_moe for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, refusals and result,
 * without the workspace: the library's own scratch, a static device array of
 * Q8K_NOALLOC_SCRATCH_BYTES (64 MiB) that each device the library runs on
 * holds until the process ends, takes its place.  A call whose workspace
 * (qmatmul_prefill_moe_workspace_bytes) would exceed it is refused with
 * Q8K_ERR_WORKSPACE.  The call allocates nothing; its first call on a device
 * asks the runtime for that device's scratch address.  Every call on one
 * device shares the scratch (it keeps the last call's contents; nothing in it
 * needs to start at zero): calls that overlap in time on one device race,
 * stream-ordered calls do not. */
#define Q8K_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int qmatmul_prefill_moe_noalloc(int qtype, const void* w, int64_t E, int64_t rows, int64_t K, const void* xq,
                                int64_t T, const int32_t* ids, const float* rw, int32_t topk, float* y, void* stream);

/* ---------------------------------------------------------- test support --
 * The exact integer sums of the path ("Language models on the device",
 * section 1: the integer dot product does the arithmetic, the sub-block
 * scales and mins fold in afterwards), exported by the kernels that ship:
 * each call runs the operation's own kernel, instantiated with a flag that
 * also stores its integer sums, and writes y exactly as the operation does.
 * Validation, refusals and ownership as for the operations.
 *
 * q8k_debug_subblock_sums: qmatvec's kernel for one packed token (xq, T = 1).
 *   y: fp32 [rows]; S: int32 sub-block sums of quant x code, [rows][K/32]
 *   for Q8K_Q4_K and Q8K_Q5_K, [rows][K/16] (quants minus 32) for
 *   Q8K_Q6_K_RELAID. */
int q8k_debug_subblock_sums(int qtype, const void* w, int64_t rows, int64_t K, const void* xq, float* y, int32_t* S,
                            void* stream);

/* q8k_debug_prefill_block_sums: qmatmul_prefill's tile for M packed tokens.
 *   y: fp32 [M][rows]; I: int32 block sums [M][rows][K/256], the integer the
 *   tile folds into y per block: sum_j sc_j * S_j (Q4_K, Q5_K; 8 sub-blocks)
 *   or sum_s sc_s * S_s (Q6_K; 16 sub-blocks). */
int q8k_debug_prefill_block_sums(int qtype, const void* w, int64_t rows, int64_t K, const void* xq, int64_t M,
                                 float* y, int32_t* I, void* stream);

/* q8k_debug_moe_subblock_sums: qmatvec_moe's matrix-core kernels (Q8K_Q4_K,
 *   Q8K_Q5_K or Q8K_Q6_K_RELAID; K small enough that a packed token fits the
 *   kernel's shared-memory stage, else Q8K_ERR_SHAPE).  y: fp32 [T][rows]; S:
 *   int32 sub-block sums of pair (t, k) against expert ids[t][k],
 *   [T * topk][rows][K/32] (Q4_K, Q5_K) or [T * topk][rows][K/16] (Q6_K);
 *   entries of pairs whose id is outside [0, E) are not written. */
int q8k_debug_moe_subblock_sums(int qtype, const void* w, int64_t E, int64_t rows, int64_t K, const void* xq,
                                int64_t T, const int32_t* ids, const float* rw, int32_t topk, float* y, int32_t* S,
                                void* stream);

/* q8k_debug_wave_sums: the wave reduction every mat-vec ends with, on
 * closed-form inputs ("One kernel, any device" prints the sum of 0..255,
 * 32640, as the check of its reduce helpers).  One workgroup of 256 threads,
 * thread t holding t: out[w] = the sum over wave w's 64 lanes (4096 w + 2016)
 * and out[4] = the four wave sums added (32640).  out: fp32 [5]. */
int q8k_debug_wave_sums(float* out, void* stream);

/* q8k_debug_last_launches: the kernels the calling thread's last operation
 * (any call above that takes a stream) enqueued, as host kernel handles in
 * launch order: the first min(count, max) go to handles.  Returns the count.
 * A test maps each handle to its kernel's name through the library's symbol
 * table ("One kernel, any device", section 5: the census of value-checked
 * kernels). */
int q8k_debug_last_launches(const void** handles, int max);

/* ---------------------------------------------------------------- errors -- */
const char* q8k_status_str(int status);
const char* q8k_last_error(void); /* calling thread's last refusal message */

#ifdef __cplusplus
}
#endif
#endif /* Q8K_H */
