/*
 * oracle.c -- plain, slow, obviously correct CPU oracle for the q8_K-packed
 * K-quant mat-vec / GEMM path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check of the entry module and
 * the CPU-baseline leg of the benchmark use it.  It shares no code, header,
 * table or constant with the HIP library (it includes only the C standard
 * library and pthreads) and is built with plain gcc.
 *
 * What it computes follows "Language models on the device: the cajeta-llm
 * kernels" (cajeta.dev/xpu/kernels-llm/), section 1 "The weights, and what the
 * kernels read": weights come as GGUF K-quant blocks of 256 values with
 * per-sub-block scales; activations are quantised to q8_K (256 values a block,
 * one scale, eight sub-block sums); an integer dot product does the arithmetic
 * and the sub-block scales and mins are applied afterwards.
 *
 * Readings taken where the pages are silent (each one is listed with its
 * reason in the design notes of the repository):
 *  - Q4_K, Q5_K and Q6_K byte layouts are the public GGUF block definitions
 *    (the pages name the formats but print no layout; for Q5_K they say only
 *    that it is Q4_K with a fifth-bit plane that supplies bit 4 of each value).
 *  - q8_K: d = amax/127 (positive), qs = round-half-even(x * (127/amax))
 *    clamped to [-127,127], computed in fp32 (a floating-point decision that
 *    produces integers is taken in the kernel's precision); an all-zero block
 *    has d = 0 and qs = 0.  The eight sub-block sums are int16 sums over the 32
 *    consecutive values that match Q4_K's eight 32-value sub-blocks.
 *  - Epilogue in fp64 over exact integer sums, blocks and sub-blocks ascending.
 *
 * Parity pins: every function here is checked in tests/test_oracle_pins.py
 * against closed forms, invariants, hand-built blocks and an independent
 * brute-force dequantise-then-dot in numpy.  The GGUF byte layout itself is
 * pinned only by self-consistency (no GGUF file is available): interop with
 * real GGUF files is "parity unpinned".
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define QK 256 /* values per K-quant super-block and per q8_K block */

/* ------------------------------------------------------------------------ */
/* O1. IEEE binary16 -> binary32, including subnormals, inf and NaN.         */
/* ------------------------------------------------------------------------ */
float or_f16_to_f32(uint16_t h) {
    uint32_t sign = (uint32_t)(h >> 15);
    uint32_t ex = (uint32_t)((h >> 10) & 31u);
    uint32_t man = (uint32_t)(h & 1023u);
    if (ex == 31u) {
        /* inf or NaN: keep the payload, as a widening conversion does */
        uint32_t bits = (sign << 31) | (255u << 23) | (man << 13);
        if (man) bits |= 1u << 22; /* quiet NaN */
        float f;
        memcpy(&f, &bits, 4);
        return f;
    }
    float v;
    if (ex == 0u)
        v = ldexpf((float)man, -24); /* zero or subnormal: man * 2^-24 */
    else
        v = ldexpf((float)(man + 1024u), (int)ex - 25); /* (1.man) * 2^(ex-15) */
    return sign ? -v : v;
}

static float f16_at(const uint8_t* p) { return or_f16_to_f32((uint16_t)(p[0] | (p[1] << 8))); }

/* ------------------------------------------------------------------------ */
/* O2. Q4_K block (144 bytes): fp16 d @0, fp16 dmin @2, 12 bytes of packed   */
/* 6-bit scales and mins @4, 128 bytes of 4-bit quants @16.                  */
/* ------------------------------------------------------------------------ */
void or_q4k_fields(const uint8_t* blk, float* d, float* dmin, uint8_t sc[8], uint8_t mn[8],
                   uint8_t q[QK]) {
    const uint8_t* s = blk + 4;
    const uint8_t* qs = blk + 16;
    *d = f16_at(blk);
    *dmin = f16_at(blk + 2);
    for (int j = 0; j < 8; ++j) {
        if (j < 4) {
            sc[j] = s[j] & 63;
            mn[j] = s[j + 4] & 63;
        } else {
            /* low four bits in byte j+4, top two bits in the spare bits of
               bytes j-4 (scale) and j (min) */
            sc[j] = (uint8_t)((s[j + 4] & 15) | ((s[j - 4] >> 6) << 4));
            mn[j] = (uint8_t)((s[j + 4] >> 4) | ((s[j] >> 6) << 4));
        }
    }
    /* values 64c..64c+31 are the low nibbles of bytes 32c..32c+31, values
       64c+32..64c+63 their high nibbles */
    for (int c = 0; c < 4; ++c)
        for (int h = 0; h < 2; ++h)
            for (int l = 0; l < 32; ++l) q[64 * c + 32 * h + l] = (uint8_t)((qs[32 * c + l] >> (4 * h)) & 15);
}

/* ------------------------------------------------------------------------ */
/* O2b. Q5_K block (176 bytes): fp16 d @0, fp16 dmin @2, the 12 scale/min    */
/* bytes @4 packed as in Q4_K, qh[32] @16, 128 bytes of low nibbles @48.     */
/* Value l (0..31) of sub-block j is the nibble Q4_K would give it plus 16   */
/* times bit j of qh[l], so q is in 0..31.                                    */
/* ------------------------------------------------------------------------ */
void or_q5k_fields(const uint8_t* blk, float* d, float* dmin, uint8_t sc[8], uint8_t mn[8],
                   uint8_t q[QK]) {
    /* d, dmin and the scale bytes sit where Q4_K has them; Q4_K's decode of
       a block whose quant bytes are ours gives the four low bits */
    uint8_t tmp[144];
    memcpy(tmp, blk, 16);
    memcpy(tmp + 16, blk + 48, 128);
    or_q4k_fields(tmp, d, dmin, sc, mn, q);
    const uint8_t* qh = blk + 16;
    for (int j = 0; j < 8; ++j)
        for (int l = 0; l < 32; ++l) q[32 * j + l] = (uint8_t)(q[32 * j + l] | (((qh[l] >> j) & 1) << 4));
}

/* ------------------------------------------------------------------------ */
/* O3. Q6_K block (210 bytes): ql[128] @0 (low 4 bits), qh[64] @128 (high 2  */
/* bits), int8 scales[16] @192, fp16 d @208.  Quant q in 0..63, value q-32.  */
/* ------------------------------------------------------------------------ */
void or_q6k_fields(const uint8_t* blk, float* d, int8_t sc[16], uint8_t q[QK]) {
    const uint8_t* ql = blk;
    const uint8_t* qh = blk + 128;
    for (int s = 0; s < 16; ++s) sc[s] = (int8_t)blk[192 + s];
    *d = f16_at(blk + 208);
    for (int h = 0; h < 2; ++h)
        for (int t = 0; t < 4; ++t)
            for (int l = 0; l < 32; ++l) {
                int lo = (ql[64 * h + 32 * (t & 1) + l] >> (4 * (t >> 1))) & 15;
                int hi = (qh[32 * h + l] >> (2 * t)) & 3;
                q[128 * h + 32 * t + l] = (uint8_t)(lo | (hi << 4));
            }
}

/* Full dequantisation to fp64 (used only by the brute-force checks). */
void or_dequant_q4k(const uint8_t* w, int64_t rows, int64_t K, double* out) {
    int64_t nb = K / QK;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            float d, dmin;
            uint8_t sc[8], mn[8], q[QK];
            or_q4k_fields(w + (r * nb + b) * 144, &d, &dmin, sc, mn, q);
            for (int v = 0; v < QK; ++v)
                out[r * K + b * QK + v] = (double)d * sc[v / 32] * q[v] - (double)dmin * mn[v / 32];
        }
}

void or_dequant_q5k(const uint8_t* w, int64_t rows, int64_t K, double* out) {
    int64_t nb = K / QK;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            float d, dmin;
            uint8_t sc[8], mn[8], q[QK];
            or_q5k_fields(w + (r * nb + b) * 176, &d, &dmin, sc, mn, q);
            for (int v = 0; v < QK; ++v)
                out[r * K + b * QK + v] = (double)d * sc[v / 32] * q[v] - (double)dmin * mn[v / 32];
        }
}

void or_dequant_q6k(const uint8_t* w, int64_t rows, int64_t K, double* out) {
    int64_t nb = K / QK;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            float d;
            int8_t sc[16];
            uint8_t q[QK];
            or_q6k_fields(w + (r * nb + b) * 210, &d, sc, q);
            for (int v = 0; v < QK; ++v) out[r * K + b * QK + v] = (double)d * sc[v / 16] * ((int)q[v] - 32);
        }
}

/* ------------------------------------------------------------------------ */
/* O4. q8_K pack of T rows of K fp32 values (K a multiple of 256).           */
/* qs[T*K] int8, d[T*K/256] fp32, bsums[T*K/32] int16.                       */
/* ------------------------------------------------------------------------ */
void or_q8k_pack(const float* x, int64_t T, int64_t K, int8_t* qs, float* d, int16_t* bsums) {
    int64_t nb = K / QK;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t b = 0; b < nb; ++b) {
            const float* xb = x + t * K + b * QK;
            int8_t* qb = qs + t * K + b * QK;
            int16_t* sb = bsums + (t * nb + b) * 8;
            float amax = 0.0f;
            for (int i = 0; i < QK; ++i) {
                float a = fabsf(xb[i]);
                if (a > amax) amax = a;
            }
            if (amax == 0.0f) {
                d[t * nb + b] = 0.0f;
                memset(qb, 0, QK);
                memset(sb, 0, 8 * sizeof(int16_t));
                continue;
            }
            float iscale = 127.0f / amax; /* one correctly rounded fp32 division */
            for (int i = 0; i < QK; ++i) {
                float v = xb[i] * iscale; /* one fp32 multiply */
                float r = nearbyintf(v);  /* default mode: round half to even */
                /* When 127/amax overflows to inf (amax below ~3.7e-37) a zero
                   value gives 0*inf = NaN: its code is 0; nonzero values
                   saturate to +-127 through the clamp below. */
                if (r != r) r = 0.0f;
                if (r > 127.0f) r = 127.0f;
                if (r < -127.0f) r = -127.0f;
                qb[i] = (int8_t)r;
            }
            for (int j = 0; j < 8; ++j) {
                int s = 0;
                for (int i = 0; i < 32; ++i) s += qb[32 * j + i];
                sb[j] = (int16_t)s;
            }
            d[t * nb + b] = amax / 127.0f;
        }
}

/* ------------------------------------------------------------------------ */
/* O5. Exact integer sub-block sums.                                         */
/* Q4_K: S[r][b*8+j]  = sum over the 32 values of sub-block j of q*qs.       */
/* Q6_K: S[r][b*16+s] = sum over the 16 values of sub-block s of (q-32)*qs.  */
/* qs is one token's K int8 codes.                                           */
/* ------------------------------------------------------------------------ */
void or_subblock_sums_q4k(const uint8_t* w, int64_t rows, int64_t K, const int8_t* qs, int32_t* S) {
    int64_t nb = K / QK;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            float d, dmin;
            uint8_t sc[8], mn[8], q[QK];
            or_q4k_fields(w + (r * nb + b) * 144, &d, &dmin, sc, mn, q);
            for (int j = 0; j < 8; ++j) {
                int32_t s = 0;
                for (int i = 0; i < 32; ++i) s += (int32_t)q[32 * j + i] * qs[b * QK + 32 * j + i];
                S[r * nb * 8 + b * 8 + j] = s;
            }
        }
}

/* Q5_K: as Q4_K, over the 5-bit quants. */
void or_subblock_sums_q5k(const uint8_t* w, int64_t rows, int64_t K, const int8_t* qs, int32_t* S) {
    int64_t nb = K / QK;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            float d, dmin;
            uint8_t sc[8], mn[8], q[QK];
            or_q5k_fields(w + (r * nb + b) * 176, &d, &dmin, sc, mn, q);
            for (int j = 0; j < 8; ++j) {
                int32_t s = 0;
                for (int i = 0; i < 32; ++i) s += (int32_t)q[32 * j + i] * qs[b * QK + 32 * j + i];
                S[r * nb * 8 + b * 8 + j] = s;
            }
        }
}

void or_subblock_sums_q6k(const uint8_t* w, int64_t rows, int64_t K, const int8_t* qs, int32_t* S) {
    int64_t nb = K / QK;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            float d;
            int8_t sc[16];
            uint8_t q[QK];
            or_q6k_fields(w + (r * nb + b) * 210, &d, sc, q);
            for (int s = 0; s < 16; ++s) {
                int32_t acc = 0;
                for (int i = 0; i < 16; ++i) acc += ((int32_t)q[16 * s + i] - 32) * qs[b * QK + 16 * s + i];
                S[r * nb * 16 + b * 16 + s] = acc;
            }
        }
}

/* ------------------------------------------------------------------------ */
/* O5b. Exact integer block sums: the scale-weighted integer dot of each     */
/* block before the floating-point epilogue ("Language models on the        */
/* device", section 1: the integer dot product does the arithmetic, the      */
/* sub-block scales fold in afterwards).                                     */
/*   Q4_K, Q5_K: I[t][r][b] = sum_j sc_j * S_j over the 8 sub-blocks;        */
/*   Q6_K:       I[t][r][b] = sum_s sc_s * S_s over the 16 sub-blocks.       */
/* qtype as in or_matvec (1 Q4_K, 2 Q6_K, 3 Q5_K; GGUF blocks); qs holds T   */
/* tokens' K codes.  The min term (sum_j m_j * bsum_j) is not part of I.     */
/* ------------------------------------------------------------------------ */
int or_block_sums(int qtype, const uint8_t* w, int64_t rows, int64_t K, const int8_t* qs, int64_t T, int64_t* I) {
    if (qtype < 1 || qtype > 3 || rows < 0 || T < 0 || K % QK) return -1;
    int64_t nb = K / QK;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t b = 0; b < nb; ++b) {
                const int8_t* x = qs + t * K + b * QK;
                int64_t acc = 0;
                if (qtype == 2) {
                    float d;
                    int8_t sc[16];
                    uint8_t q[QK];
                    or_q6k_fields(w + (r * nb + b) * 210, &d, sc, q);
                    for (int s = 0; s < 16; ++s) {
                        int64_t S = 0;
                        for (int i = 0; i < 16; ++i) S += ((int64_t)q[16 * s + i] - 32) * x[16 * s + i];
                        acc += (int64_t)sc[s] * S;
                    }
                } else {
                    float d, dmin;
                    uint8_t sc[8], mn[8], q[QK];
                    if (qtype == 3)
                        or_q5k_fields(w + (r * nb + b) * 176, &d, &dmin, sc, mn, q);
                    else
                        or_q4k_fields(w + (r * nb + b) * 144, &d, &dmin, sc, mn, q);
                    for (int j = 0; j < 8; ++j) {
                        int64_t S = 0;
                        for (int i = 0; i < 32; ++i) S += (int64_t)q[32 * j + i] * x[32 * j + i];
                        acc += (int64_t)sc[j] * S;
                    }
                }
                I[(t * rows + r) * nb + b] = acc;
            }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O6. One output element: weight row `wr` (nb blocks) against one packed    */
/* token (qs, d8, bsums of that token).  fp64 epilogue over exact integers;  */
/* *A receives the sum of |terms| at sub-block granularity.                  */
/* ------------------------------------------------------------------------ */
/* Q4_K and Q5_K share the epilogue: y = sum_b d8 (d sum_j sc_j S_j - dmin
   sum_j m_j bsum_j); `five` selects the 176-byte Q5_K block. */
static double dot_q4k_row(const uint8_t* wr, int64_t nb, const int8_t* qs, const float* d8,
                          const int16_t* bsums, double* A, int five) {
    double y = 0.0, a = 0.0;
    for (int64_t b = 0; b < nb; ++b) {
        float d, dmin;
        uint8_t sc[8], mn[8], q[QK];
        if (five)
            or_q5k_fields(wr + b * 176, &d, &dmin, sc, mn, q);
        else
            or_q4k_fields(wr + b * 144, &d, &dmin, sc, mn, q);
        int64_t isum = 0, msum = 0;
        for (int j = 0; j < 8; ++j) {
            int64_t S = 0;
            for (int i = 0; i < 32; ++i) S += (int64_t)q[32 * j + i] * qs[b * QK + 32 * j + i];
            int64_t B = bsums[b * 8 + j];
            isum += (int64_t)sc[j] * S;
            msum += (int64_t)mn[j] * B;
            a += fabs((double)d8[b] * (double)d * (double)sc[j] * (double)S) +
                 fabs((double)d8[b] * (double)dmin * (double)mn[j] * (double)B);
        }
        y += (double)d8[b] * ((double)d * (double)isum - (double)dmin * (double)msum);
    }
    *A = a;
    return y;
}

static double dot_q6k_row(const uint8_t* wr, int64_t nb, const int8_t* qs, const float* d8, double* A) {
    double y = 0.0, a = 0.0;
    for (int64_t b = 0; b < nb; ++b) {
        float d;
        int8_t sc[16];
        uint8_t q[QK];
        or_q6k_fields(wr + b * 210, &d, sc, q);
        int64_t isum = 0;
        for (int s = 0; s < 16; ++s) {
            int64_t S = 0;
            for (int i = 0; i < 16; ++i) S += ((int64_t)q[16 * s + i] - 32) * qs[b * QK + 16 * s + i];
            isum += (int64_t)sc[s] * S;
            a += fabs((double)d8[b] * (double)d * (double)sc[s] * (double)S);
        }
        y += (double)d8[b] * (double)d * (double)isum;
    }
    *A = a;
    return y;
}

/* ------------------------------------------------------------------------ */
/* O7. Mat-vec over T packed tokens: y[t][r], A[t][r].  qtype 1 = Q4_K       */
/* (144-byte GGUF blocks), 2 = Q6_K (210-byte GGUF blocks), 3 = Q5_K         */
/* (176-byte GGUF blocks).  Rows are split                                   */
/* across `nthreads` pthreads (each output is computed by one thread, so the */
/* result does not depend on the thread count).                              */
/* ------------------------------------------------------------------------ */
int64_t or_block_bytes(int qtype) { return qtype == 1 ? 144 : qtype == 2 ? 210 : qtype == 3 ? 176 : 0; }

typedef struct {
    int qtype;
    const uint8_t* w;
    int64_t rows, K, T;
    const int8_t* qs;
    const float* d8;
    const int16_t* bsums;
    double* y;
    double* A;
    int64_t r0, r1;
} mv_job;

static void* mv_worker(void* p) {
    mv_job* j = (mv_job*)p;
    int64_t nb = j->K / QK;
    int64_t bb = or_block_bytes(j->qtype);
    for (int64_t t = 0; t < j->T; ++t)
        for (int64_t r = j->r0; r < j->r1; ++r) {
            const uint8_t* wr = j->w + r * nb * bb;
            double a;
            double y = j->qtype == 2 ? dot_q6k_row(wr, nb, j->qs + t * j->K, j->d8 + t * nb, &a)
                                     : dot_q4k_row(wr, nb, j->qs + t * j->K, j->d8 + t * nb, j->bsums + t * nb * 8,
                                                   &a, j->qtype == 3);
            j->y[t * j->rows + r] = y;
            if (j->A) j->A[t * j->rows + r] = a;
        }
    return NULL;
}

int or_matvec(int qtype, const uint8_t* w, int64_t rows, int64_t K, const int8_t* qs, const float* d8,
              const int16_t* bsums, int64_t T, double* y, double* A, int nthreads) {
    if (or_block_bytes(qtype) == 0 || rows < 0 || T < 0 || K % QK) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > rows) nthreads = rows > 0 ? (int)rows : 1;
    mv_job jobs[256];
    pthread_t th[256];
    for (int i = 0; i < nthreads; ++i) {
        mv_job jb = {qtype, w, rows, K, T, qs, d8, bsums, y, A, rows * i / nthreads, rows * (i + 1) / nthreads};
        jobs[i] = jb;
    }
    if (nthreads == 1) {
        mv_worker(&jobs[0]);
        return 0;
    }
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, mv_worker, &jobs[i]);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    return 0;
}

/* MoE expert-indexed mat-vec: w holds E experts of `rows` rows each (same
   format); token t selects experts ids[t][k] with router weights rw[t][k]:
   y[t][r] = sum_k rw[t][k] * (W_{ids[t][k]} x_t)[r], k ascending.
   A[t][r] = sum_k |rw[t][k]| * A_{ids[t][k]}[t][r]. */
int or_moe(int qtype, const uint8_t* w, int64_t E, int64_t rows, int64_t K, const int8_t* qs, const float* d8,
           const int16_t* bsums, int64_t T, const int32_t* ids, const float* rw, int64_t topk, double* y, double* A,
           int nthreads) {
    if (or_block_bytes(qtype) == 0 || K % QK || E < 1 || topk < 1) return -1;
    int64_t nb = K / QK;
    int64_t bb = or_block_bytes(qtype);
    double* ye = (double*)malloc(sizeof(double) * (size_t)(rows > 0 ? rows : 1));
    double* ae = (double*)malloc(sizeof(double) * (size_t)(rows > 0 ? rows : 1));
    if (!ye || !ae) {
        free(ye);
        free(ae);
        return -2;
    }
    for (int64_t i = 0; i < T * rows; ++i) {
        y[i] = 0.0;
        if (A) A[i] = 0.0;
    }
    for (int64_t t = 0; t < T; ++t)
        for (int64_t k = 0; k < topk; ++k) {
            int32_t e = ids[t * topk + k];
            if (e < 0 || e >= E) {
                free(ye);
                free(ae);
                return -3;
            }
            or_matvec(qtype, w + (int64_t)e * rows * nb * bb, rows, K, qs + t * K, d8 + t * nb, bsums + t * nb * 8, 1,
                      ye, ae, nthreads);
            double g = (double)rw[t * topk + k];
            for (int64_t r = 0; r < rows; ++r) {
                y[t * rows + r] += g * ye[r];
                if (A) A[t * rows + r] += fabs(g) * ae[r];
            }
        }
    free(ye);
    free(ae);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Bind-time Q6_K relayout: each 210-byte block -> its fp16 d into the       */
/* prefix array and its first 208 bytes (ql, qh, scales) into the body array. */
/* ------------------------------------------------------------------------ */
void or_q6k_relayout(const uint8_t* src, int64_t nblocks, uint16_t* prefix, uint8_t* bodies) {
    for (int64_t i = 0; i < nblocks; ++i) {
        const uint8_t* b = src + i * 210;
        memcpy(bodies + i * 208, b, 208);
        prefix[i] = (uint16_t)(b[208] | (b[209] << 8));
    }
}
