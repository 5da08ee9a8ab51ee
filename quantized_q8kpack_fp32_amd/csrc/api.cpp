// C ABI of libq8k: argument validation, sizing helpers and dispatch to the
// gfx950 kernels.  Every refusal is named and enqueues nothing (the launch
// checks with named reasons of "One kernel, any device", section 1; the
// 256-multiple width rule of "Language models on the device: the cajeta-llm
// kernels", section 3.2).  Validation touches no HIP API, so refusals work on
// a machine without a GPU.
#include <stdarg.h>
#include <stdio.h>

#include "../../include/q8k.h"
#include "q8k_device.h"
#include "q8k_launch.h"

using namespace q8k;

namespace {

thread_local char g_err[512] = "";

// The launch record of the calling thread's last operation (test support: the
// kernel census).  Every operation clears it first; each launch appends its
// kernel's host handle.
constexpr int LAUNCH_RECORD_MAX = 16;
thread_local const void* g_launched[LAUNCH_RECORD_MAX];
thread_local int g_nlaunched = 0;
void begin_call() { g_nlaunched = 0; }

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

// Sizes are kept well inside int32 block counts per row and 2^31 rows so that
// grid sizes and per-row indexing cannot overflow.
constexpr int64_t MAX_ROWS = (int64_t)1 << 30;
constexpr int64_t MAX_K = (int64_t)1 << 24;
constexpr int64_t MAX_TOKENS = (int64_t)1 << 24;
constexpr int64_t MAX_EXPERTS = 4096;
static_assert(MAX_EXPERTS <= MOE_GROUP_MAX_E, "the MoE prefill groups pairs of at most MOE_GROUP_MAX_E experts");

// Every launch uses a 1-D grid of at most 2^31 - 1 workgroups.
constexpr int64_t MAX_GRID = ((int64_t)1 << 31) - 1;

int check_grid(const char* fn, int64_t workgroups) {
    if (workgroups > MAX_GRID)
        return fail(Q8K_ERR_SHAPE, "%s: problem needs %lld workgroups (at most %lld)", fn, (long long)workgroups,
                    (long long)MAX_GRID);
    return Q8K_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int check_k(const char* fn, int64_t K) {
    if (K <= 0 || K % QK != 0 || K > MAX_K)
        return fail(Q8K_ERR_SHAPE, "%s: K=%lld must be a positive multiple of 256 (at most %lld)", fn, (long long)K,
                    (long long)MAX_K);
    return Q8K_OK;
}

int check_count(const char* fn, const char* what, int64_t v, int64_t maxv) {
    if (v < 0 || v > maxv)
        return fail(Q8K_ERR_SHAPE, "%s: %s=%lld out of range [0, %lld]", fn, what, (long long)v, (long long)maxv);
    return Q8K_OK;
}

int check_ptr(const char* fn, const char* what, const void* p, size_t align) {
    if (!p) return fail(Q8K_ERR_NULL, "%s: %s is NULL", fn, what);
    if (!aligned(p, align))
        return fail(Q8K_ERR_ALIGN, "%s: %s=%p is not %zu-byte aligned", fn, what, p, align);
    return Q8K_OK;
}

Acts acts_of(const void* xq, int64_t T, int64_t K) {
    const ActLayout l = act_layout(T, K);
    const uint8_t* base = static_cast<const uint8_t*>(xq);
    Acts a;
    a.qs = reinterpret_cast<const int8_t*>(base);
    a.d = reinterpret_cast<const float*>(base + l.off_d);
    a.bs = reinterpret_cast<const int16_t*>(base + l.off_bs);
    a.K = K;
    return a;
}

struct Q6View {
    const uint16_t* prefix;
    const uint8_t* bodies;
};
Q6View q6_view(const void* w, int64_t nblocks) {
    const uint8_t* base = static_cast<const uint8_t*>(w);
    return Q6View{reinterpret_cast<const uint16_t*>(base), base + align256(2 * (size_t)nblocks)};
}

int launched(const char* fn, hipError_t e) {
    if (e != hipSuccess) return fail(Q8K_ERR_LAUNCH, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return Q8K_OK;
}

#define Q8K_TRY(x)                    \
    do {                              \
        int _st = (x);                \
        if (_st != Q8K_OK) return _st; \
    } while (0)

// Every operation serves Q4_K, Q5_K and relaid Q6_K weights.
int check_weight(const char* fn, int qtype, const void* w) {
    if (qtype == Q8K_Q4_K || qtype == Q8K_Q5_K || qtype == Q8K_Q6_K_RELAID) return check_ptr(fn, "w", w, 16);
    if (qtype == Q8K_Q6_K_GGUF)
        return fail(Q8K_ERR_QTYPE, "%s: raw GGUF Q6_K must be bound first (q8k_bind_q6k -> Q8K_Q6_K_RELAID)", fn);
    return fail(Q8K_ERR_QTYPE, "%s: qtype=%d not served here (use Q8K_Q4_K=1, Q8K_Q6_K_RELAID=2 or Q8K_Q5_K=4)", fn,
                qtype);
}

// The prefill tile's format index and weight streams (Q6_K: bodies and prefix).
struct PrefillWeights {
    int fmt;
    const uint8_t* w;
    const uint16_t* prefix;
};
PrefillWeights prefill_weights(int qtype, const void* w, int64_t nblocks) {
    if (qtype == Q8K_Q6_K_RELAID) {
        const Q6View v = q6_view(w, nblocks);
        return PrefillWeights{WFMT_Q6_K, v.bodies, v.prefix};
    }
    return PrefillWeights{qtype == Q8K_Q5_K ? WFMT_Q5_K : WFMT_Q4_K, static_cast<const uint8_t*>(w), nullptr};
}

}  // namespace

void q8k::note_launch(const void* kernel) {
    if (g_nlaunched < LAUNCH_RECORD_MAX) g_launched[g_nlaunched] = kernel;
    ++g_nlaunched;  // counts past the record's end too, so an overflow is visible
}

extern "C" {

size_t q8k_act_layout(int64_t T, int64_t K, size_t* off_d, size_t* off_bsums) {
    if (T < 0 || K <= 0 || K % QK != 0) return 0;
    const ActLayout l = act_layout(T, K);
    if (off_d) *off_d = l.off_d;
    if (off_bsums) *off_bsums = l.off_bs;
    return l.total;
}

size_t q8k_act_bytes(int64_t T, int64_t K) { return q8k_act_layout(T, K, nullptr, nullptr); }

size_t q8k_weight_bytes(int qtype, int64_t rows, int64_t K) {
    if (rows < 0 || K <= 0 || K % QK != 0) return 0;
    const size_t nblk = (size_t)rows * (size_t)(K / QK);
    switch (qtype) {
        case Q8K_Q4_K: return nblk * Q4K_BLOCK;
        case Q8K_Q5_K: return nblk * Q5K_BLOCK;
        case Q8K_Q6_K_GGUF: return nblk * Q6K_BLOCK;
        case Q8K_Q6_K_RELAID: return align256(2 * nblk) + nblk * Q6K_BODY;
        default: return 0;
    }
}

int q8k_pack(const float* x, int64_t T, int64_t K, void* xq, void* stream) {
    begin_call();
    const char* fn = "q8k_pack";
    Q8K_TRY(check_k(fn, K));
    Q8K_TRY(check_count(fn, "T", T, MAX_TOKENS));
    Q8K_TRY(check_ptr(fn, "x", x, 16));
    Q8K_TRY(check_ptr(fn, "xq", xq, 16));
    Q8K_TRY(check_grid(fn, (T * (K / QK) + 15) / 16));  // 16 blocks per workgroup
    if (T == 0) return Q8K_OK;
    const ActLayout l = act_layout(T, K);
    uint8_t* base = static_cast<uint8_t*>(xq);
    return launched(fn, launch_pack(x, T * (K / QK), reinterpret_cast<int8_t*>(base),
                                    reinterpret_cast<float*>(base + l.off_d),
                                    reinterpret_cast<int16_t*>(base + l.off_bs), (hipStream_t)stream));
}

int q8k_bind_q6k(const void* w_gguf, int64_t rows, int64_t K, void* w_relaid, void* stream) {
    begin_call();
    const char* fn = "q8k_bind_q6k";
    Q8K_TRY(check_k(fn, K));
    Q8K_TRY(check_count(fn, "rows", rows, MAX_ROWS));
    Q8K_TRY(check_ptr(fn, "w_gguf", w_gguf, 2));
    Q8K_TRY(check_ptr(fn, "w_relaid", w_relaid, 16));
    Q8K_TRY(check_grid(fn, (rows * (K / QK) + 3) / 4));
    if (rows == 0) return Q8K_OK;
    const int64_t nblk = rows * (K / QK);
    uint8_t* base = static_cast<uint8_t*>(w_relaid);
    return launched(fn, launch_bind_q6k(static_cast<const uint8_t*>(w_gguf), nblk, reinterpret_cast<uint16_t*>(base),
                                        base + align256(2 * (size_t)nblk), (hipStream_t)stream));
}

static int matvec_common(const char* fn, int qtype, const void* w, int64_t rows, int64_t K, const void* xq,
                         int64_t ncols, float* y, void* stream) {
    Q8K_TRY(check_k(fn, K));
    Q8K_TRY(check_count(fn, "rows", rows, MAX_ROWS));
    Q8K_TRY(check_weight(fn, qtype, w));
    Q8K_TRY(check_ptr(fn, "xq", xq, 16));
    Q8K_TRY(check_ptr(fn, "y", y, 4));
    if (rows == 0) return Q8K_OK;
    const int nb = (int)(K / QK);
    const Acts a = acts_of(xq, ncols, K);
    hipError_t e;
    if (qtype == Q8K_Q4_K) {
        e = launch_matvec_q4k(static_cast<const uint8_t*>(w), rows, nb, a, (int)ncols, y, (hipStream_t)stream);
    } else if (qtype == Q8K_Q5_K) {
        e = launch_matvec_q5k(static_cast<const uint8_t*>(w), rows, nb, a, (int)ncols, y, (hipStream_t)stream);
    } else {
        const Q6View v = q6_view(w, rows * nb);
        e = launch_matvec_q6k(v.prefix, v.bodies, rows, nb, a, (int)ncols, y, (hipStream_t)stream);
    }
    return launched(fn, e);
}

int qmatvec_f32(int qtype, const void* w, int64_t rows, int64_t K, const float* x, int64_t ncols, float* y,
                void* xq_out, void* stream) {
    begin_call();
    const char* fn = "qmatvec_f32";
    Q8K_TRY(check_k(fn, K));
    Q8K_TRY(check_count(fn, "rows", rows, MAX_ROWS));
    if (ncols < 1 || ncols > Q8K_COLS_MAX)
        return fail(Q8K_ERR_ARG, "%s: ncols=%lld must be in [1, %d]", fn, (long long)ncols, Q8K_COLS_MAX);
    if (fused_lds_bytes(ncols, K) > FUSED_LDS_MAX)
        return fail(Q8K_ERR_SHAPE,
                    "%s: ncols*K=%lld: the packed columns (%zu bytes) exceed one workgroup's %zu bytes of LDS "
                    "(use q8k_pack + qmatvec_batched)",
                    fn, (long long)(ncols * K), fused_lds_bytes(ncols, K), FUSED_LDS_MAX);
    Q8K_TRY(check_weight(fn, qtype, w));
    Q8K_TRY(check_ptr(fn, "x", x, 16));
    Q8K_TRY(check_ptr(fn, "y", y, 4));
    if (xq_out) Q8K_TRY(check_ptr(fn, "xq_out", xq_out, 16));
    if (rows == 0) return Q8K_OK;
    const int nb = (int)(K / QK);
    PackedOut o{nullptr, nullptr, nullptr};
    if (xq_out) {
        const Acts a = acts_of(xq_out, ncols, K);
        o = PackedOut{const_cast<int8_t*>(a.qs), const_cast<float*>(a.d), const_cast<int16_t*>(a.bs)};
    }
    const PrefillWeights pw = prefill_weights(qtype, w, rows * nb);
    return launched(fn, launch_matvec_f32(pw.fmt, pw.w, pw.prefix, rows, nb, x, K, (int)ncols, y, o,
                                          (hipStream_t)stream));
}

int qmatvec(int qtype, const void* w, int64_t rows, int64_t K, const void* xq, float* y, void* stream) {
    begin_call();
    return matvec_common("qmatvec", qtype, w, rows, K, xq, 1, y, stream);
}

int qmatvec_batched(int qtype, const void* w, int64_t rows, int64_t K, const void* xq, int64_t ncols, float* y,
                    void* stream) {
    begin_call();
    if (ncols < 1 || ncols > Q8K_COLS_MAX)
        return fail(Q8K_ERR_ARG, "qmatvec_batched: ncols=%lld must be in [1, %d]", (long long)ncols, Q8K_COLS_MAX);
    return matvec_common("qmatvec_batched", qtype, w, rows, K, xq, ncols, y, stream);
}

int qmatvec_moe(int qtype, const void* w, int64_t E, int64_t rows, int64_t K, const void* xq, int64_t T,
                const int32_t* ids, const float* rw, int32_t topk, float* y, void* stream) {
    begin_call();
    const char* fn = "qmatvec_moe";
    Q8K_TRY(check_k(fn, K));
    Q8K_TRY(check_count(fn, "rows", rows, MAX_ROWS));
    if (E < 1 || E > MAX_EXPERTS)
        return fail(Q8K_ERR_ARG, "%s: E=%lld must be in [1, %lld]", fn, (long long)E, (long long)MAX_EXPERTS);
    if (E * rows > MAX_ROWS)
        return fail(Q8K_ERR_SHAPE, "%s: E*rows=%lld exceeds %lld", fn, (long long)(E * rows), (long long)MAX_ROWS);
    if (T < 0 || T > Q8K_MOE_MAX_TOKENS)
        return fail(Q8K_ERR_ARG, "%s: T=%lld must be in [0, %d]", fn, (long long)T, Q8K_MOE_MAX_TOKENS);
    if (topk < 1 || topk > E || topk > Q8K_MOE_MAX_TOPK)
        return fail(Q8K_ERR_ARG, "%s: topk=%d must be in [1, min(E=%lld, %d)]", fn, topk, (long long)E,
                    Q8K_MOE_MAX_TOPK);
    Q8K_TRY(check_weight(fn, qtype, w));
    Q8K_TRY(check_ptr(fn, "xq", xq, 16));
    Q8K_TRY(check_ptr(fn, "ids", ids, 4));
    Q8K_TRY(check_ptr(fn, "rw", rw, 4));
    Q8K_TRY(check_ptr(fn, "y", y, 4));
    if (rows == 0 || T == 0) return Q8K_OK;
    const int nb = (int)(K / QK);
    const Acts a = acts_of(xq, T, K);
    hipError_t e;
    if (qtype == Q8K_Q4_K) {
        // matrix-core kernel while a packed token fits its LDS stage (K up to
        // about 89k), the one-lane-per-row kernel beyond
        if (moe_mfma_q4k_fits(K))
            e = launch_moe_mfma_q4k(static_cast<const uint8_t*>(w), E, rows, nb, a, T, ids, rw, topk, y,
                                    (hipStream_t)stream);
        else
            e = launch_moe_q4k(static_cast<const uint8_t*>(w), E, rows, nb, a, T, ids, rw, topk, y,
                               (hipStream_t)stream);
    } else if (qtype == Q8K_Q5_K) {
        if (moe_mfma_q4k_fits(K))
            e = launch_moe_mfma_q5k(static_cast<const uint8_t*>(w), E, rows, nb, a, T, ids, rw, topk, y,
                                    (hipStream_t)stream);
        else
            e = launch_moe_q5k(static_cast<const uint8_t*>(w), E, rows, nb, a, T, ids, rw, topk, y,
                               (hipStream_t)stream);
    } else {
        // relaid Q6_K: the matrix-core kernel while a packed token fits its
        // stage (K up to about 84k), the per-chunk kernel beyond
        const Q6View v = q6_view(w, E * rows * nb);
        if (moe_mfma_q6k_fits(K))
            e = launch_moe_mfma_q6k(v.prefix, v.bodies, E, rows, nb, a, T, ids, rw, topk, y, (hipStream_t)stream);
        else
            e = launch_moe_q6k(v.prefix, v.bodies, E, rows, nb, a, T, ids, rw, topk, y, (hipStream_t)stream);
    }
    return launched(fn, e);
}

size_t qmatmul_prefill_workspace_bytes(int qtype, int64_t rows, int64_t K, int64_t M) {
    (void)qtype;
    if (rows <= 0 || M <= 0 || K <= 0 || K % QK != 0) return 0;
    const int ks = prefill_ksplit(rows, K / QK, M);
    return ks > 1 ? (size_t)ks * (size_t)M * (size_t)rows * 4 : 0;
}

int qmatmul_prefill(int qtype, const void* w, int64_t rows, int64_t K, const void* xq, int64_t M, float* y, void* ws,
                    size_t ws_bytes, void* stream) {
    begin_call();
    const char* fn = "qmatmul_prefill";
    Q8K_TRY(check_k(fn, K));
    Q8K_TRY(check_count(fn, "rows", rows, MAX_ROWS));
    Q8K_TRY(check_count(fn, "M", M, MAX_TOKENS));
    Q8K_TRY(check_weight(fn, qtype, w));
    Q8K_TRY(check_ptr(fn, "xq", xq, 16));
    Q8K_TRY(check_ptr(fn, "y", y, 4));
    const size_t need = qmatmul_prefill_workspace_bytes(qtype, rows, K, M);
    if (ws_bytes < need)
        return fail(Q8K_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, ws_bytes, need);
    if (need > 0) Q8K_TRY(check_ptr(fn, "ws", ws, 16));
    Q8K_TRY(check_grid(fn, ((rows + 31) / 32) * ((M + 63) / 64)));  // bound for every tile shape
    if (rows == 0 || M == 0) return Q8K_OK;
    const int nb = (int)(K / QK);
    const PrefillWeights pw = prefill_weights(qtype, w, rows * nb);
    return launched(fn, launch_prefill(pw.fmt, pw.w, pw.prefix, rows, nb, acts_of(xq, M, K), M, y,
                                       static_cast<float*>(ws), (hipStream_t)stream));
}

size_t qmatmul_prefill_f32_workspace_bytes(int qtype, int64_t rows, int64_t K, int64_t M) {
    (void)qtype;
    if (rows <= 0 || M <= 0 || K <= 0 || K % QK != 0) return 0;
    const int ks = prefill_ksplit(rows, K / QK, M);
    return (size_t)prefill_sync_bytes(M, ks) + (ks > 1 ? (size_t)ks * (size_t)M * (size_t)rows * 4 : 0);
}

int qmatmul_prefill_f32(int qtype, const void* w, int64_t rows, int64_t K, const float* x, int64_t M, void* xq,
                        float* y, void* ws, size_t ws_bytes, void* stream) {
    begin_call();
    const char* fn = "qmatmul_prefill_f32";
    Q8K_TRY(check_k(fn, K));
    Q8K_TRY(check_count(fn, "rows", rows, MAX_ROWS));
    Q8K_TRY(check_count(fn, "M", M, MAX_TOKENS));
    Q8K_TRY(check_weight(fn, qtype, w));
    Q8K_TRY(check_ptr(fn, "x", x, 16));
    Q8K_TRY(check_ptr(fn, "xq", xq, 16));
    Q8K_TRY(check_ptr(fn, "y", y, 4));
    const size_t need = qmatmul_prefill_f32_workspace_bytes(qtype, rows, K, M);
    if (ws_bytes < need)
        return fail(Q8K_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, ws_bytes, need);
    if (need > 0) Q8K_TRY(check_ptr(fn, "ws", ws, 16));
    Q8K_TRY(check_grid(fn, ((rows + 31) / 32) * ((M + 63) / 64)));
    if (rows == 0 || M == 0) return Q8K_OK;
    // the row tiles of a token tile wait for each other: they must fit on the
    // device together (one workgroup per compute unit)
    const int64_t tiles = (rows + 63) / 64, cus = device_cu_count();
    if (tiles > cus)
        return fail(Q8K_ERR_SHAPE,
                    "%s: rows=%lld make %lld row tiles that wait for each other, more than the device's %lld compute "
                    "units (rows <= %lld; use q8k_pack + qmatmul_prefill)",
                    fn, (long long)rows, (long long)tiles, (long long)cus, (long long)(64 * cus));
    const int nb = (int)(K / QK);
    const int ks = prefill_ksplit(rows, nb, M);
    const Acts a = acts_of(xq, M, K);
    PackDst pk{x, const_cast<int8_t*>(a.qs), const_cast<float*>(a.d), const_cast<int16_t*>(a.bs),
               static_cast<int32_t*>(ws)};
    float* part = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + prefill_sync_bytes(M, ks));
    const PrefillWeights pw = prefill_weights(qtype, w, rows * nb);
    return launched(fn, launch_prefill_f32(pw.fmt, pw.w, pw.prefix, rows, nb, a, M, y, part, pk,
                                           (hipStream_t)stream));
}

size_t qmatmul_prefill_moe_workspace_bytes(int qtype, int64_t E, int64_t rows, int64_t K, int64_t T, int32_t topk) {
    if ((qtype != Q8K_Q4_K && qtype != Q8K_Q5_K && qtype != Q8K_Q6_K_RELAID) || E < 1 || rows < 0 || K <= 0 ||
        K % QK != 0 || T < 0 || topk < 1)
        return 0;
    return (size_t)moe_prefill_ws(E, rows, T, topk).total;
}

static int prefill_moe_common(const char* fn, int qtype, const void* w, int64_t E, int64_t rows, int64_t K,
                              const void* xq, int64_t T, const int32_t* ids, const float* rw, int32_t topk, float* y,
                              void* ws, size_t ws_bytes, bool noalloc, void* stream);

int qmatmul_prefill_moe(int qtype, const void* w, int64_t E, int64_t rows, int64_t K, const void* xq, int64_t T,
                        const int32_t* ids, const float* rw, int32_t topk, float* y, void* ws, size_t ws_bytes,
                        void* stream) {
    begin_call();
    return prefill_moe_common("qmatmul_prefill_moe", qtype, w, E, rows, K, xq, T, ids, rw, topk, y, ws, ws_bytes,
                              false, stream);
}

int qmatmul_prefill_moe_noalloc(int qtype, const void* w, int64_t E, int64_t rows, int64_t K, const void* xq,
                                int64_t T, const int32_t* ids, const float* rw, int32_t topk, float* y,
                                void* stream) {
    begin_call();
    return prefill_moe_common("qmatmul_prefill_moe_noalloc", qtype, w, E, rows, K, xq, T, ids, rw, topk, y, nullptr,
                              0, true, stream);
}

static int prefill_moe_common(const char* fn, int qtype, const void* w, int64_t E, int64_t rows, int64_t K,
                              const void* xq, int64_t T, const int32_t* ids, const float* rw, int32_t topk, float* y,
                              void* ws, size_t ws_bytes, bool noalloc, void* stream) {
    Q8K_TRY(check_k(fn, K));
    Q8K_TRY(check_count(fn, "rows", rows, MAX_ROWS));
    if (E < 1 || E > MAX_EXPERTS)
        return fail(Q8K_ERR_ARG, "%s: E=%lld must be in [1, %lld]", fn, (long long)E, (long long)MAX_EXPERTS);
    if (E * rows > MAX_ROWS)
        return fail(Q8K_ERR_SHAPE, "%s: E*rows=%lld exceeds %lld", fn, (long long)(E * rows), (long long)MAX_ROWS);
    Q8K_TRY(check_count(fn, "T", T, MAX_TOKENS));
    if (T * K >= ((int64_t)1 << 30))
        return fail(Q8K_ERR_SHAPE, "%s: T*K=%lld must be below 2^30 (32-bit gather offsets)", fn,
                    (long long)(T * K));
    if (topk < 1 || topk > E || topk > Q8K_MOE_MAX_TOPK)
        return fail(Q8K_ERR_ARG, "%s: topk=%d must be in [1, min(E=%lld, %d)]", fn, topk, (long long)E,
                    Q8K_MOE_MAX_TOPK);
    Q8K_TRY(check_weight(fn, qtype, w));
    Q8K_TRY(check_ptr(fn, "xq", xq, 16));
    Q8K_TRY(check_ptr(fn, "ids", ids, 4));
    Q8K_TRY(check_ptr(fn, "rw", rw, 4));
    Q8K_TRY(check_ptr(fn, "y", y, 4));
    const size_t need = qmatmul_prefill_moe_workspace_bytes(qtype, E, rows, K, T, topk);
    if (noalloc) {
        if (need > NOALLOC_SCRATCH_BYTES)
            return fail(Q8K_ERR_WORKSPACE,
                        "%s: the call needs %zu bytes of workspace, more than the library's %zu-byte scratch "
                        "(use qmatmul_prefill_moe with a caller workspace)",
                        fn, need, NOALLOC_SCRATCH_BYTES);
    } else {
        if (ws_bytes < need)
            return fail(Q8K_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, ws_bytes, need);
        if (need > 0) Q8K_TRY(check_ptr(fn, "ws", ws, 16));
    }
    Q8K_TRY(check_grid(fn, moe_prefill_ws(E, rows, T, topk).max_chunks * ((rows + 63) / 64)));
    Q8K_TRY(check_grid(fn, T * ((rows + 255) / 256)));  // the combine's workgroups, at most
    if (rows == 0 || T == 0) return Q8K_OK;
    if (noalloc) {
        const hipError_t e = noalloc_scratch(&ws);
        if (e != hipSuccess)
            return fail(Q8K_ERR_LAUNCH, "%s: the library's scratch is not available: %s", fn, hipGetErrorString(e));
    }
    const int nb = (int)(K / QK);
    const PrefillWeights pw = prefill_weights(qtype, w, E * rows * nb);
    return launched(fn, launch_prefill_moe(pw.fmt, pw.w, pw.prefix, E, rows, nb, acts_of(xq, T, K), T, ids, rw, topk,
                                           y, ws, (hipStream_t)stream));
}

int q8k_debug_subblock_sums(int qtype, const void* w, int64_t rows, int64_t K, const void* xq, float* y, int32_t* S,
                            void* stream) {
    begin_call();
    const char* fn = "q8k_debug_subblock_sums";
    Q8K_TRY(check_k(fn, K));
    Q8K_TRY(check_count(fn, "rows", rows, MAX_ROWS));
    Q8K_TRY(check_weight(fn, qtype, w));
    Q8K_TRY(check_ptr(fn, "xq", xq, 16));
    Q8K_TRY(check_ptr(fn, "y", y, 4));
    Q8K_TRY(check_ptr(fn, "S", S, 4));
    if (rows == 0) return Q8K_OK;
    const int nb = (int)(K / QK);
    const PrefillWeights pw = prefill_weights(qtype, w, rows * nb);
    return launched(fn, launch_matvec_sums(pw.fmt, pw.w, pw.prefix, rows, nb, acts_of(xq, 1, K), y, S,
                                           (hipStream_t)stream));
}

int q8k_debug_prefill_block_sums(int qtype, const void* w, int64_t rows, int64_t K, const void* xq, int64_t M,
                                 float* y, int32_t* I, void* stream) {
    begin_call();
    const char* fn = "q8k_debug_prefill_block_sums";
    Q8K_TRY(check_k(fn, K));
    Q8K_TRY(check_count(fn, "rows", rows, MAX_ROWS));
    Q8K_TRY(check_count(fn, "M", M, MAX_TOKENS));
    Q8K_TRY(check_weight(fn, qtype, w));
    Q8K_TRY(check_ptr(fn, "xq", xq, 16));
    Q8K_TRY(check_ptr(fn, "y", y, 4));
    Q8K_TRY(check_ptr(fn, "I", I, 4));
    Q8K_TRY(check_grid(fn, ((rows + 31) / 32) * ((M + 63) / 64)));
    if (rows == 0 || M == 0) return Q8K_OK;
    const int nb = (int)(K / QK);
    const PrefillWeights pw = prefill_weights(qtype, w, rows * nb);
    return launched(fn, launch_prefill_sums(pw.fmt, pw.w, pw.prefix, rows, nb, acts_of(xq, M, K), M, y, I,
                                            (hipStream_t)stream));
}

int q8k_debug_moe_subblock_sums(int qtype, const void* w, int64_t E, int64_t rows, int64_t K, const void* xq,
                                int64_t T, const int32_t* ids, const float* rw, int32_t topk, float* y, int32_t* S,
                                void* stream) {
    begin_call();
    const char* fn = "q8k_debug_moe_subblock_sums";
    Q8K_TRY(check_k(fn, K));
    Q8K_TRY(check_count(fn, "rows", rows, MAX_ROWS));
    if (qtype != Q8K_Q4_K && qtype != Q8K_Q5_K && qtype != Q8K_Q6_K_RELAID)
        return fail(Q8K_ERR_QTYPE,
                    "%s: qtype=%d: the matrix-core MoE kernels serve Q8K_Q4_K, Q8K_Q5_K and Q8K_Q6_K_RELAID", fn, qtype);
    if (qtype == Q8K_Q6_K_RELAID ? !moe_mfma_q6k_fits(K) : !moe_mfma_q4k_fits(K))
        return fail(Q8K_ERR_SHAPE, "%s: K=%lld: a packed token exceeds the matrix-core MoE kernel's LDS stage", fn,
                    (long long)K);
    if (E < 1 || E > MAX_EXPERTS)
        return fail(Q8K_ERR_ARG, "%s: E=%lld must be in [1, %lld]", fn, (long long)E, (long long)MAX_EXPERTS);
    if (E * rows > MAX_ROWS)
        return fail(Q8K_ERR_SHAPE, "%s: E*rows=%lld exceeds %lld", fn, (long long)(E * rows), (long long)MAX_ROWS);
    if (T < 0 || T > Q8K_MOE_MAX_TOKENS)
        return fail(Q8K_ERR_ARG, "%s: T=%lld must be in [0, %d]", fn, (long long)T, Q8K_MOE_MAX_TOKENS);
    if (topk < 1 || topk > E || topk > Q8K_MOE_MAX_TOPK)
        return fail(Q8K_ERR_ARG, "%s: topk=%d must be in [1, min(E=%lld, %d)]", fn, topk, (long long)E,
                    Q8K_MOE_MAX_TOPK);
    Q8K_TRY(check_ptr(fn, "w", w, 16));
    Q8K_TRY(check_ptr(fn, "xq", xq, 16));
    Q8K_TRY(check_ptr(fn, "ids", ids, 4));
    Q8K_TRY(check_ptr(fn, "rw", rw, 4));
    Q8K_TRY(check_ptr(fn, "y", y, 4));
    Q8K_TRY(check_ptr(fn, "S", S, 4));
    if (rows == 0 || T == 0) return Q8K_OK;
    if (qtype == Q8K_Q6_K_RELAID) {
        const Q6View v = q6_view(w, E * rows * (K / QK));
        return launched(fn, launch_moe_mfma6_sums(v.prefix, v.bodies, E, rows, (int)(K / QK), acts_of(xq, T, K), T, ids,
                                                  rw, topk, y, S, (hipStream_t)stream));
    }
    return launched(fn, launch_moe_mfma_sums(qtype == Q8K_Q5_K, static_cast<const uint8_t*>(w), E, rows, (int)(K / QK),
                                             acts_of(xq, T, K), T, ids, rw, topk, y, S, (hipStream_t)stream));
}

int q8k_debug_wave_sums(float* out, void* stream) {
    begin_call();
    Q8K_TRY(check_ptr("q8k_debug_wave_sums", "out", out, 4));
    return launched("q8k_debug_wave_sums", launch_wave_sums(out, (hipStream_t)stream));
}

int q8k_debug_last_launches(const void** handles, int max) {
    const int n = g_nlaunched < LAUNCH_RECORD_MAX ? g_nlaunched : LAUNCH_RECORD_MAX;
    for (int i = 0; i < n && i < max; ++i) handles[i] = g_launched[i];
    return g_nlaunched;
}

const char* q8k_status_str(int status) {
    switch (status) {
        case Q8K_OK: return "Q8K_OK";
        case Q8K_ERR_NULL: return "Q8K_ERR_NULL";
        case Q8K_ERR_SHAPE: return "Q8K_ERR_SHAPE";
        case Q8K_ERR_ALIGN: return "Q8K_ERR_ALIGN";
        case Q8K_ERR_QTYPE: return "Q8K_ERR_QTYPE";
        case Q8K_ERR_ARG: return "Q8K_ERR_ARG";
        case Q8K_ERR_WORKSPACE: return "Q8K_ERR_WORKSPACE";
        case Q8K_ERR_LAUNCH: return "Q8K_ERR_LAUNCH";
        default: return "Q8K_ERR_UNKNOWN";
    }
}

const char* q8k_last_error(void) { return g_err; }

}  // extern "C"
