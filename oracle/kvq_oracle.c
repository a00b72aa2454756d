/*
 * kvq_oracle.c -- plain, slow CPU oracle for the quantized-KV decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the CPU-baseline
 * leg of bench.py may load this library.  It shares no code, header, table or
 * constant generator with the HIP library: every conversion below is written
 * from the format definition, every codec step from the pages' description.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp (see oracle/build.py).
 * fp32 steps are fp32 C expressions (x86-64 SSE, FLT_EVAL_METHOD == 0, no
 * contraction), fmaf() appears only where the definition says fma.
 * Attention is computed in double from explicitly reconstructed rows.
 *
 * Sources (cited by page title and section):
 *  [KV8]  colibri PR #399 "KV cache quantization: fp8 (KV8) + 4-bit TurboQuant
 *         (KV_TQ) on CPU, CUDA, and Metal" -- Summary (per-row amax/448 scale,
 *         RNE e4m3), "Why rotated-int4 for the 4-bit tier" (randomized Hadamard
 *         rotation, 16-level N(0,1) Lloyd-Max codebook scaled by radius/sqrt(n),
 *         one per-row radius), the rebase note on HIP portability (e4m3 grid:
 *         normals (1+M/8)*2^(E-7), denormals M*2^-9, S.1111.111 reads as 0),
 *         the "Ready for review" note (rotation identities q.xhat = Rq.c and
 *         sum w xhat = R^T sum w c), and the rebase note refusing
 *         non-power-of-two widths.
 *  [Q4]   Strata PR #2533 "metal: q4_0 KV cache on the Mac engine" -- the first
 *         commit message (FWHT-256 orthonormal 1/16, tie in |x| resolves to the
 *         larger value, fp16 scale by round-to-nearest-even, codeword
 *         int(fma(x, id, 8.5f)) truncated toward zero), the fixtures commit
 *         (all-zero group: d = -0.0 -> scale bits 0x8000, id = 0 -> q = 8,
 *         bytes 0x88; 18-byte blocks), the QSA_KV_Q4 commit (pools
 *         [cell][kv head][144], dequant (nibble - 8) * f32(d)), and the k4
 *         commit (four consecutive k share one nibble side of a block).
 *
 * Readings of points the pages leave open are stated at each
 * function below.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_UNSUPPORTED 2
#define ORACLE_ERR_NOMEM 3

/* ------------------------------------------------------------------------- */
/* Threads                                                                    */
/* ------------------------------------------------------------------------- */

int oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/* ------------------------------------------------------------------------- */
/* Small-float formats, from their definitions                                */
/* ------------------------------------------------------------------------- */

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits.
 * Value of a code per [KV8] HIP portability note: E > 0 -> (1 + M/8) 2^(E-7),
 * E == 0 -> M 2^-9, and S.1111.111 (the format's NaN) reads back as 0. */
double oracle_e4m3_decode(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return 0.0;
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* Magnitude of positive code c (0x00..0x7E), increasing in c. */
static double e4m3_mag(int c) { return oracle_e4m3_decode((uint8_t)c); }

/* Round |v| to the nearest e4m3 grid value, ties to the even code, after
 * saturating |v| to 448 (the largest finite e4m3).  The sign of the input is
 * kept, also for results that round to zero.  NaN input is outside the
 * contract (returns 0). */
uint8_t oracle_e4m3_encode(double v) {
    if (isnan(v)) return 0;
    int s = signbit(v) ? 1 : 0;
    double a = fabs(v);
    if (a >= 448.0) return (uint8_t)((s << 7) | 0x7E);
    int lo = 0, hi = 0x7E;
    while (lo < hi) { /* largest code with magnitude <= a */
        int mid = (lo + hi + 1) / 2;
        if (e4m3_mag(mid) <= a) lo = mid; else hi = mid - 1;
    }
    int c = lo;
    if (e4m3_mag(lo) < a) { /* a strictly between lo and lo+1 (lo < 0x7E) */
        double mid = (e4m3_mag(lo) + e4m3_mag(lo + 1)) / 2.0; /* exact */
        if (a > mid || (a == mid && (lo & 1))) c = lo + 1;
    }
    return (uint8_t)((s << 7) | c);
}

/* IEEE 754 binary16. */
double oracle_f16_decode(uint16_t h) {
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 31) v = m ? NAN : INFINITY;
    else if (e == 0) v = ldexp((double)m, -24);
    else v = ldexp(1.0 + m / 1024.0, e - 15);
    return s ? -v : v;
}

/* Round to nearest binary16, ties to even; beyond the overflow threshold
 * (the midpoint between 65504 and 2^16) the result is +-Inf. */
uint16_t oracle_f16_encode(double v) {
    if (isnan(v)) return 0x7E00;
    int s = signbit(v) ? 1 : 0;
    double a = fabs(v);
    uint16_t r;
    if (a >= 65520.0) r = 0x7C00;
    else {
        int lo = 0, hi = 0x7BFF;
        while (lo < hi) {
            int mid = (lo + hi + 1) / 2;
            if (oracle_f16_decode((uint16_t)mid) <= a) lo = mid; else hi = mid - 1;
        }
        r = (uint16_t)lo;
        double v0 = oracle_f16_decode((uint16_t)lo);
        if (v0 < a) {
            double v1 = (lo < 0x7BFF) ? oracle_f16_decode((uint16_t)(lo + 1)) : 65536.0;
            double mid = (v0 + v1) / 2.0;
            if (a > mid || (a == mid && (lo & 1))) r = (uint16_t)(lo + 1);
        }
    }
    return (uint16_t)((s << 15) | r);
}

/* bfloat16: the top half of a binary32. */
double oracle_bf16_decode(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round to nearest bfloat16, ties to even; overflow to +-Inf past the
 * midpoint between the largest finite bf16 and 2^128. */
uint16_t oracle_bf16_encode(double v) {
    if (isnan(v)) return 0x7FC0;
    int s = signbit(v) ? 1 : 0;
    double a = fabs(v);
    double top = oracle_bf16_decode(0x7F7F);
    double over = (top + ldexp(1.0, 128)) / 2.0;
    uint16_t r;
    if (a >= over) r = 0x7F80;
    else {
        int lo = 0, hi = 0x7F7F;
        while (lo < hi) {
            int mid = (lo + hi + 1) / 2;
            if (oracle_bf16_decode((uint16_t)mid) <= a) lo = mid; else hi = mid - 1;
        }
        r = (uint16_t)lo;
        double v0 = oracle_bf16_decode((uint16_t)lo);
        if (v0 < a) {
            double v1 = (lo < 0x7F7F) ? oracle_bf16_decode((uint16_t)(lo + 1)) : ldexp(1.0, 128);
            double mid = (v0 + v1) / 2.0;
            if (a > mid || (a == mid && (lo & 1))) r = (uint16_t)(lo + 1);
        }
    }
    return (uint16_t)((s << 15) | r);
}

/* Array forms (numpy-friendly). */
void oracle_e4m3_encode_array(const float* x, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; i++) out[i] = oracle_e4m3_encode((double)x[i]);
}
void oracle_e4m3_decode_array(const uint8_t* c, int64_t n, double* out) {
    for (int64_t i = 0; i < n; i++) out[i] = oracle_e4m3_decode(c[i]);
}
void oracle_f16_encode_array(const float* x, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; i++) out[i] = oracle_f16_encode((double)x[i]);
}
void oracle_f16_encode_array_f64(const double* x, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; i++) out[i] = oracle_f16_encode(x[i]);
}
void oracle_f16_decode_array(const uint16_t* h, int64_t n, double* out) {
    for (int64_t i = 0; i < n; i++) out[i] = oracle_f16_decode(h[i]);
}
void oracle_bf16_encode_array(const float* x, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; i++) out[i] = oracle_bf16_encode((double)x[i]);
}
void oracle_bf16_encode_array_f64(const double* x, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; i++) out[i] = oracle_bf16_encode(x[i]);
}

/* ------------------------------------------------------------------------- */
/* Walsh-Hadamard transform                                                   */
/* ------------------------------------------------------------------------- */

static int is_pow2(int n) { return n > 0 && (n & (n - 1)) == 0; }

/* Unnormalized radix-2 FWHT in fp32, stages h = 1, 2, 4, ..., n/2; within a
 * stage every pair (i, i+h) with (i & h) == 0 becomes (a + b, a - b) where
 * a = v[i], b = v[i+h].  The pages fix only "the CUDA register order" for this
 * (Strata PR #2533, the qsa_prep commit); ascending h is the reading taken. */
int oracle_fwht_f32(float* v, int n) {
    if (!is_pow2(n)) return ORACLE_ERR_UNSUPPORTED;
    for (int h = 1; h < n; h <<= 1)
        for (int i = 0; i < n; i++)
            if (!(i & h)) {
                float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
    return ORACLE_OK;
}

/* The same transform in double (used for reconstruction in attention). */
static void fwht_f64(double* v, int n) {
    for (int h = 1; h < n; h <<= 1)
        for (int i = 0; i < n; i++)
            if (!(i & h)) {
                double a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
}

/* FWHT-256, orthonormal: the unnormalized transform, then x 1/16 (exact in
 * fp32).  [Q4] first commit message. */
int oracle_fwht256_orthonormal(float* v) {
    oracle_fwht_f32(v, 256);
    for (int i = 0; i < 256; i++) v[i] = v[i] * 0.0625f;
    return ORACLE_OK;
}

int oracle_fwht_rows_f32(float* v, int64_t n_rows, int n) {
    if (!is_pow2(n)) return ORACLE_ERR_UNSUPPORTED;
    for (int64_t r = 0; r < n_rows; r++) oracle_fwht_f32(v + r * n, n);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------- */
/* a1: fp8 e4m3 per-row encoder ([KV8] Summary / commit 1)                    */
/* ------------------------------------------------------------------------- */

/* amax = max |x_i|; s = fl32(amax / 448); code_i = e4m3(fl32(x_i / s)).
 * All-zero row: s = 0 and every code 0x00 (reading: the pages name inert rows
 * only for the 4-bit codec). */
int oracle_encode_fp8(const float* x, int64_t n_rows, int dim, uint8_t* codes, float* scales) {
    if (!x || !codes || !scales || n_rows < 0 || dim <= 0) return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_rows; r++) {
        const float* xr = x + r * dim;
        uint8_t* cr = codes + r * dim;
        float amax = 0.0f;
        for (int i = 0; i < dim; i++) {
            float a = fabsf(xr[i]);
            if (a > amax) amax = a;
        }
        if (amax == 0.0f) {
            scales[r] = 0.0f;
            memset(cr, 0, (size_t)dim);
            continue;
        }
        float s = amax / 448.0f;
        scales[r] = s;
        for (int i = 0; i < dim; i++) {
            float q = xr[i] / s;
            cr[i] = oracle_e4m3_encode((double)q);
        }
    }
    return ORACLE_OK;
}

/* x_hat = e4m3(code) * s, in double. */
int oracle_decode_fp8_rows(const uint8_t* codes, const float* scales, int64_t n_rows, int dim, double* out) {
    for (int64_t r = 0; r < n_rows; r++)
        for (int i = 0; i < dim; i++)
            out[r * dim + i] = oracle_e4m3_decode(codes[r * dim + i]) * (double)scales[r];
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------- */
/* Codec-1 codebooks: 2^b-level Lloyd-Max quantizers for N(0,1), b = 3, 4, 6  */
/* ([KV8] Why rotated-int4; the KV_TQ=4,6 tiers of the teacher-forcing table; */
/* the "codec 1, 3-bit" tier of the .coli_kv reply)                          */
/* ------------------------------------------------------------------------- */

static double phi(double x) { return exp(-0.5 * x * x) / sqrt(2.0 * M_PI); }
static double Phi(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }
static double Qtail(double x) { return 0.5 * erfc(x / sqrt(2.0)); } /* 1 - Phi(x), no cancellation */

/* Number of codebook levels of a codec-1 tier: 8 (3-bit), 16 (4-bit) or 64
 * (6-bit); 0 for any other width. */
static int tq_levels(int bits) { return (bits == 3 || bits == 4 || bits == 6) ? 1 << bits : 0; }

/* Lloyd-Max for N(0,1) with N = 2^bits levels, in double.  Only the positive
 * half is iterated (the density is symmetric, so the optimum is symmetric with
 * a threshold at 0): thresholds are midpoints of neighbouring levels, levels
 * are the conditional means (phi(a) - phi(b)) / (Q(a) - Q(b)) of their cells
 * (Q the upper tail, Q(a) - Q(b) = Phi(b) - Phi(a)).  Once no level moves by
 * 1e-14 it runs as many iterations again: the 64-level iteration contracts
 * slowly (about 0.2% per step), so a small step still leaves the levels about
 * 1e-12 from the fixed point, and its rounding noise (a few 1e-15) rules out a
 * much smaller step bound.  Outputs (any may be NULL):
 *   levels_exact[N]   the converged levels, ascending;
 *   levels_bf16[N]    each level rounded to the nearest bfloat16 (reading:
 *                     the decode feeds 16-bit tiles, so the stored levels are
 *                     bf16 values);
 *   thresholds[N-1]   fp32 midpoints of neighbouring bf16 levels (exact);
 *   iters             iterations to convergence. */
int oracle_tq_codebook(int bits, double* levels_exact, float* levels_bf16, float* thresholds, int* iters) {
    const int N = tq_levels(bits);
    if (!N) return ORACLE_ERR_UNSUPPORTED;
    const int h = N / 2;
    double c[32], t[33];
    for (int k = 0; k < h; k++) c[k] = (k + 0.5) * 3.0 / h; /* initial guess */
    int it, stop = -1;
    for (it = 0; it < 2000000; it++) {
        t[0] = 0.0;
        for (int k = 1; k < h; k++) t[k] = 0.5 * (c[k - 1] + c[k]);
        double delta = 0.0;
        for (int k = 0; k < h; k++) {
            double a = t[k];
            double nc = (k == h - 1) ? phi(a) / Qtail(a)
                                     : (phi(a) - phi(t[k + 1])) / (Qtail(a) - Qtail(t[k + 1]));
            double d = fabs(nc - c[k]);
            if (d > delta) delta = d;
            c[k] = nc;
        }
        if (stop < 0 && delta < 1e-14) stop = 2 * it + 1;
        if (it == stop) break;
    }
    if (stop < 0) return ORACLE_ERR_UNSUPPORTED; /* did not converge */
    double full[64];
    for (int k = 0; k < h; k++) {
        full[h + k] = c[k];
        full[h - 1 - k] = -c[k];
    }
    if (levels_exact)
        for (int k = 0; k < N; k++) levels_exact[k] = full[k];
    float lb[64];
    for (int k = 0; k < N; k++) lb[k] = (float)oracle_bf16_decode(oracle_bf16_encode(full[k]));
    if (levels_bf16)
        for (int k = 0; k < N; k++) levels_bf16[k] = lb[k];
    if (thresholds)
        for (int k = 0; k < N - 1; k++) {
            double m = ((double)lb[k] + (double)lb[k + 1]) / 2.0;
            float mf = (float)m;
            if ((double)mf != m) return ORACLE_ERR_UNSUPPORTED; /* must be exact */
            thresholds[k] = mf;
        }
    if (iters) *iters = it;
    return ORACLE_OK;
}

int oracle_tq4_codebook(double* levels_exact, float* levels_bf16, float* thresholds, int* iters) {
    return oracle_tq_codebook(4, levels_exact, levels_bf16, thresholds, iters);
}

/* Mean squared error of an n-level scalar quantizer (levels[n], cell
 * boundaries thresholds[n-1]) on N(0,1), closed form from the truncated
 * moments. */
double oracle_quantizer_mse_n(int n, const double* levels, const double* thresholds) {
    double mse = 0.0;
    for (int k = 0; k < n; k++) {
        double a = (k == 0) ? -INFINITY : thresholds[k - 1];
        double b = (k == n - 1) ? INFINITY : thresholds[k];
        double Pa = isinf(a) ? 0.0 : Phi(a), Pb = isinf(b) ? 1.0 : Phi(b);
        double pa = isinf(a) ? 0.0 : phi(a), pb = isinf(b) ? 0.0 : phi(b);
        double apa = isinf(a) ? 0.0 : a * pa, bpb = isinf(b) ? 0.0 : b * pb;
        double m0 = Pb - Pa;                 /* int phi       */
        double m1 = pa - pb;                 /* int x phi     */
        double m2 = (Pb - Pa) + apa - bpb;   /* int x^2 phi   */
        double c = levels[k];
        mse += m2 - 2.0 * c * m1 + c * c * m0;
    }
    return mse;
}

double oracle_quantizer_mse(const double* levels, const double* thresholds) {
    return oracle_quantizer_mse_n(16, levels, thresholds);
}

/* ------------------------------------------------------------------------- */
/* a2: codec-1 row encoder ([KV8] Why rotated-int4; rebase 85852e2 refusal)  */
/* ------------------------------------------------------------------------- */

static int sign_bit(const uint8_t* mask, int i) { return (mask[i >> 3] >> (i & 7)) & 1; }

/* Packing of b-bit indices (reading: the pages fix the index width per tier but
 * not the byte layout; the plainest layout that is the 4-bit tier's nibble
 * layout at b = 4): the row is a little-endian bit stream and index i occupies
 * bits b*i .. b*i + b - 1, least significant bit first, so bit j of the stream
 * is bit j % 8 of byte j / 8.  A row of dim indices takes dim * b / 8 bytes. */
static void put_index(uint8_t* row, int i, int bits, unsigned v) {
    for (int j = 0; j < bits; j++) {
        int pos = i * bits + j;
        if ((v >> j) & 1u) row[pos >> 3] |= (uint8_t)(1u << (pos & 7));
    }
}

static unsigned get_index(const uint8_t* row, int i, int bits) {
    unsigned v = 0;
    for (int j = 0; j < bits; j++) {
        int pos = i * bits + j;
        v |= (unsigned)((row[pos >> 3] >> (pos & 7)) & 1) << j;
    }
    return v;
}

/* Code bytes per row of a b-bit tier, or -1 if dim cannot be encoded: dim must
 * be a power of two (refusal of non-power-of-two widths) whose indices fill
 * whole bytes. */
int64_t oracle_tq_code_bytes(int bits, int dim) {
    if (!tq_levels(bits) || !is_pow2(dim) || dim < 2 || (dim * bits) % 8 != 0) return -1;
    return (int64_t)dim * bits / 8;
}

/* For each row x (dim a power of two):
 *   z_i = -x_i where sign bit i is set, else x_i;
 *   w   = FWHT(z), unnormalized, fp32 (oracle_fwht_f32 order);
 *   r   = sqrt of the pairwise-tree sum of x_i*x_i (level 0 is fl(x_i*x_i),
 *         each level adds adjacent pairs), correctly rounded;
 *   T_k = fl(t_k * r), k = 0 .. N-2 (t_k the fp32 thresholds of the codebook);
 *   idx_i = #{k : w_i > T_k}  (a value exactly on a threshold goes low);
 *   the indices packed as above (b = 4: byte j = idx_{2j} | idx_{2j+1} << 4).
 * The orthonormal coordinate is y = w / sqrt(n) and the scaled levels are
 * c_k r / sqrt(n), so the nearest level is found by comparing w with t_k r.
 * Non-power-of-two widths are refused. */
int oracle_encode_tq(int bits, const float* x, int64_t n_rows, int dim, const uint8_t* sign_mask,
                     uint8_t* codes, float* radii) {
    if (!x || !codes || !radii || !sign_mask || n_rows < 0) return ORACLE_ERR_ARG;
    const int64_t cb = oracle_tq_code_bytes(bits, dim);
    if (cb < 0) return ORACLE_ERR_UNSUPPORTED;
    const int N = tq_levels(bits);
    float thr[63];
    if (oracle_tq_codebook(bits, NULL, NULL, thr, NULL) != ORACLE_OK) return ORACLE_ERR_UNSUPPORTED;
    int rc = ORACLE_OK;
#pragma omp parallel
    {
        float* z = (float*)malloc(sizeof(float) * (size_t)dim);
        float* sq = (float*)malloc(sizeof(float) * (size_t)dim);
        if (!z || !sq) {
#pragma omp atomic write
            rc = ORACLE_ERR_NOMEM;
        } else {
#pragma omp for schedule(static)
            for (int64_t r = 0; r < n_rows; r++) {
                const float* xr = x + r * dim;
                for (int i = 0; i < dim; i++) z[i] = sign_bit(sign_mask, i) ? -xr[i] : xr[i];
                oracle_fwht_f32(z, dim);
                for (int i = 0; i < dim; i++) sq[i] = xr[i] * xr[i];
                for (int len = dim; len > 1; len >>= 1)
                    for (int i = 0; i < len / 2; i++) sq[i] = sq[2 * i] + sq[2 * i + 1];
                float rad = sqrtf(sq[0]);
                radii[r] = rad;
                float T[63];
                for (int k = 0; k < N - 1; k++) T[k] = thr[k] * rad;
                uint8_t* cr = codes + r * cb;
                memset(cr, 0, (size_t)cb);
                for (int i = 0; i < dim; i++) {
                    unsigned idx = 0;
                    for (int k = 0; k < N - 1; k++)
                        if (z[i] > T[k]) idx++;
                    put_index(cr, i, bits, idx);
                }
            }
        }
        free(z);
        free(sq);
    }
    return rc;
}

int oracle_encode_tq4(const float* x, int64_t n_rows, int dim, const uint8_t* sign_mask,
                      uint8_t* codes, float* radii) {
    return oracle_encode_tq(4, x, n_rows, dim, sign_mask, codes, radii);
}

/* Reconstruction in double: y_i = c[idx_i] r / sqrt(n), x_hat = D H y / sqrt(n)
 * (R = H D / sqrt(n) is orthonormal, so R^-1 = R^T = D H / sqrt(n)). */
static void decode_tq_rows_with(int bits, const float* lv, const uint8_t* codes, const float* radii,
                                int64_t n_rows, int dim, const uint8_t* sign_mask, double* out) {
    const int64_t cb = (int64_t)dim * bits / 8;
    double rs = sqrt((double)dim);
    for (int64_t r = 0; r < n_rows; r++) {
        double* o = out + r * dim;
        const uint8_t* cr = codes + r * cb;
        for (int i = 0; i < dim; i++) o[i] = (double)lv[get_index(cr, i, bits)] * (double)radii[r] / rs;
        fwht_f64(o, dim);
        for (int i = 0; i < dim; i++) o[i] = (sign_bit(sign_mask, i) ? -o[i] : o[i]) / rs;
    }
}

int oracle_decode_tq_rows(int bits, const uint8_t* codes, const float* radii, int64_t n_rows, int dim,
                          const uint8_t* sign_mask, double* out) {
    if (oracle_tq_code_bytes(bits, dim) < 0) return ORACLE_ERR_UNSUPPORTED;
    float lv[64];
    oracle_tq_codebook(bits, NULL, lv, NULL, NULL);
    decode_tq_rows_with(bits, lv, codes, radii, n_rows, dim, sign_mask, out);
    return ORACLE_OK;
}

int oracle_decode_tq4_rows(const uint8_t* codes, const float* radii, int64_t n_rows, int dim,
                           const uint8_t* sign_mask, double* out) {
    return oracle_decode_tq_rows(4, codes, radii, n_rows, dim, sign_mask, out);
}

/* The rotation identities of the native codec-1 consumer ([KV8] Ready for
 * review): for a query q and weights w over rows,
 *   q . x_hat_t        == (R q) . y_t
 *   sum_t w_t x_hat_t  == R^T (sum_t w_t y_t)
 * Both sides are formed in double; returns the largest relative discrepancy
 * (against the magnitude of the terms) over all rows and coordinates.
 *
 * `plant` exists only so that a test can show the check is sensitive: 0 is the
 * definition; 1 leaves the query unrotated (R q := q); 2 drops the signs from
 * the query rotation (R q := H q / sqrt(n)); 3 drops the signs from the
 * un-rotation (R^T v := H v / sqrt(n)); 4 leaves the weighted sum unrotated
 * (R^T v := v).  Each planted mistake must show up as a large discrepancy. */
static double tq_identity_check_planted(int bits, const uint8_t* codes, const float* radii, int64_t n_rows,
                                        int dim, const uint8_t* sign_mask, const double* q, const double* w,
                                        int plant) {
    if (oracle_tq_code_bytes(bits, dim) < 0) return -1.0;
    const int64_t cb = (int64_t)dim * bits / 8;
    float lv[64];
    oracle_tq_codebook(bits, NULL, lv, NULL, NULL);
    double rs = sqrt((double)dim);
    double* xh = (double*)malloc(sizeof(double) * (size_t)dim);
    double* y = (double*)malloc(sizeof(double) * (size_t)dim);
    double* rq = (double*)malloc(sizeof(double) * (size_t)dim);
    double* sx = (double*)calloc((size_t)dim, sizeof(double));
    double* sy = (double*)calloc((size_t)dim, sizeof(double));
    double* sxa = (double*)calloc((size_t)dim, sizeof(double));
    double worst = 0.0;
    /* R q = H D q / sqrt(n) */
    for (int i = 0; i < dim; i++) rq[i] = (sign_bit(sign_mask, i) && plant != 2) ? -q[i] : q[i];
    if (plant != 1) {
        fwht_f64(rq, dim);
        for (int i = 0; i < dim; i++) rq[i] /= rs;
    }
    for (int64_t r = 0; r < n_rows; r++) {
        const uint8_t* cr = codes + r * cb;
        decode_tq_rows_with(bits, lv, cr, radii + r, 1, dim, sign_mask, xh);
        for (int i = 0; i < dim; i++) y[i] = (double)lv[get_index(cr, i, bits)] * (double)radii[r] / rs;
        double a = 0.0, b = 0.0, mag = 0.0;
        for (int i = 0; i < dim; i++) {
            a += q[i] * xh[i];
            b += rq[i] * y[i];
            mag += fabs(q[i] * xh[i]) + fabs(rq[i] * y[i]);
        }
        if (mag > 0) {
            double e = fabs(a - b) / mag;
            if (e > worst) worst = e;
        }
        for (int i = 0; i < dim; i++) {
            sx[i] += w[r] * xh[i];
            sxa[i] += fabs(w[r] * xh[i]);
            sy[i] += w[r] * y[i];
        }
    }
    /* R^T sy = D H sy / sqrt(n) */
    if (plant != 4) fwht_f64(sy, dim);
    for (int i = 0; i < dim; i++) {
        double v = plant == 4 ? sy[i] : ((sign_bit(sign_mask, i) && plant != 3) ? -sy[i] : sy[i]) / rs;
        if (sxa[i] > 0) {
            double e = fabs(v - sx[i]) / sxa[i];
            if (e > worst) worst = e;
        }
    }
    free(xh); free(y); free(rq); free(sx); free(sy); free(sxa);
    return worst;
}

double oracle_tq_identity_check(int bits, const uint8_t* codes, const float* radii, int64_t n_rows, int dim,
                                const uint8_t* sign_mask, const double* q, const double* w, int plant) {
    return tq_identity_check_planted(bits, codes, radii, n_rows, dim, sign_mask, q, w, plant);
}

double oracle_tq4_identity_check(const uint8_t* codes, const float* radii, int64_t n_rows, int dim,
                                 const uint8_t* sign_mask, const double* q, const double* w) {
    return tq_identity_check_planted(4, codes, radii, n_rows, dim, sign_mask, q, w, 0);
}

/* The same check with a planted mistake (see above); tests only. */
double oracle_tq4_identity_check_planted(const uint8_t* codes, const float* radii, int64_t n_rows, int dim,
                                         const uint8_t* sign_mask, const double* q, const double* w, int plant) {
    return tq_identity_check_planted(4, codes, radii, n_rows, dim, sign_mask, q, w, plant);
}

/* ------------------------------------------------------------------------- */
/* a3..a8: absorbed-MLA decode attention over quantized rows, in double       */
/* ------------------------------------------------------------------------- */

/* For every sequence s (rows seq_offsets[s] .. seq_offsets[s+1]-1) and head h:
 *   x_hat_t  = reconstructed latent row (fp8: e4m3(code) * scale;
 *              codec 1: oracle_decode_tq_rows), explicitly, in double;
 *   s_t      = sm_scale * (q_lat[s,h] . x_hat_t + q_rope[s,h] . k_rope_t);
 *   p        = softmax over all rows of the sequence (max subtracted);
 *   out[s,h] = sum_t p_t x_hat_t;   lse[s,h] = m + log(sum_t exp(s_t - m)).
 * qmode 1 = fp8 rows (codes [rows][dim]); codec-1 rows, codes [rows][dim*b/8]:
 * qmode 2 = 4-bit (TQ4), 3 = 3-bit (TQ3), 4 = 6-bit (TQ6).
 * k_rope holds bfloat16 bit patterns.  A sequence with no rows gives zeros and
 * lse = -Inf.  Decode attends to every cached row (no mask). */
int oracle_decode_attn(int qmode, int n_seqs, int n_heads, int dim, int dim_rope,
                       const int64_t* seq_offsets, const uint8_t* codes, const float* row_scale,
                       const uint16_t* k_rope, const uint8_t* sign_mask, const float* q_lat,
                       const float* q_rope, double sm_scale, double* out, double* lse) {
    if (n_seqs < 0 || n_heads <= 0 || dim <= 0 || dim_rope < 0 || !seq_offsets || !out)
        return ORACLE_ERR_ARG;
    const int bits = qmode == 2 ? 4 : qmode == 3 ? 3 : qmode == 4 ? 6 : 0;
    if (qmode != 1 && !bits) return ORACLE_ERR_UNSUPPORTED;
    if (bits && (oracle_tq_code_bytes(bits, dim) < 0 || !sign_mask)) return ORACLE_ERR_UNSUPPORTED;
    const int64_t cb = (qmode == 1) ? dim : oracle_tq_code_bytes(bits, dim);
    float lv[64];
    if (bits) oracle_tq_codebook(bits, NULL, lv, NULL, NULL);
    for (int s = 0; s < n_seqs; s++) {
        int64_t t0 = seq_offsets[s], t1 = seq_offsets[s + 1];
        int64_t T = t1 - t0;
        if (T < 0) return ORACLE_ERR_ARG;
        if (T == 0) {
            for (int h = 0; h < n_heads; h++) {
                for (int d = 0; d < dim; d++) out[((int64_t)s * n_heads + h) * dim + d] = 0.0;
                if (lse) lse[(int64_t)s * n_heads + h] = -INFINITY;
            }
            continue;
        }
        double* X = (double*)malloc(sizeof(double) * (size_t)T * (size_t)dim);
        double* KR = (double*)malloc(sizeof(double) * (size_t)T * (size_t)(dim_rope > 0 ? dim_rope : 1));
        if (!X || !KR) { free(X); free(KR); return ORACLE_ERR_NOMEM; }
#pragma omp parallel for schedule(static)
        for (int64_t t = 0; t < T; t++) {
            if (qmode == 1)
                oracle_decode_fp8_rows(codes + (t0 + t) * cb, row_scale + t0 + t, 1, dim, X + t * dim);
            else
                decode_tq_rows_with(bits, lv, codes + (t0 + t) * cb, row_scale + t0 + t, 1, dim, sign_mask,
                                     X + t * dim);
            for (int r = 0; r < dim_rope; r++)
                KR[t * dim_rope + r] = oracle_bf16_decode(k_rope[(t0 + t) * dim_rope + r]);
        }
        int rc = ORACLE_OK;
#pragma omp parallel
        {
            double* sc = (double*)malloc(sizeof(double) * (size_t)T);
            double* acc = (double*)malloc(sizeof(double) * (size_t)dim);
            if (!sc || !acc) {
#pragma omp atomic write
                rc = ORACLE_ERR_NOMEM;
            } else {
#pragma omp for schedule(dynamic, 1)
                for (int h = 0; h < n_heads; h++) {
                    const float* ql = q_lat + ((int64_t)s * n_heads + h) * dim;
                    const float* qr = q_rope ? q_rope + ((int64_t)s * n_heads + h) * dim_rope : NULL;
                    double m = -INFINITY;
                    for (int64_t t = 0; t < T; t++) {
                        double a = 0.0, b = 0.0;
                        const double* xt = X + t * dim;
                        for (int d = 0; d < dim; d++) a += (double)ql[d] * xt[d];
                        if (qr)
                            for (int r = 0; r < dim_rope; r++) b += (double)qr[r] * KR[t * dim_rope + r];
                        sc[t] = sm_scale * (a + b);
                        if (sc[t] > m) m = sc[t];
                    }
                    double l = 0.0;
                    for (int64_t t = 0; t < T; t++) {
                        sc[t] = exp(sc[t] - m);
                        l += sc[t];
                    }
                    for (int d = 0; d < dim; d++) acc[d] = 0.0;
                    for (int64_t t = 0; t < T; t++) {
                        const double* xt = X + t * dim;
                        double p = sc[t];
                        for (int d = 0; d < dim; d++) acc[d] += p * xt[d];
                    }
                    double* o = out + ((int64_t)s * n_heads + h) * dim;
                    for (int d = 0; d < dim; d++) o[d] = acc[d] / l;
                    if (lse) lse[(int64_t)s * n_heads + h] = m + log(l);
                }
            }
            free(sc);
            free(acc);
        }
        free(X);
        free(KR);
        if (rc != ORACLE_OK) return rc;
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------- */
/* a9/a10: q4_0 paged tier ([Q4])                                             */
/* ------------------------------------------------------------------------- */

#define Q4_BLOCK 32
#define Q4_BLOCK_BYTES 18

/* One block of 32 values -> 18 bytes:
 *   mval = the element of largest |x|; a tie in |x| goes to the larger signed
 *          value (and between +0 and -0 to +0, a reading: the pages do not
 *          speak of signed zeros);
 *   d    = mval / -8 (fp32);  id = d != 0 ? fl32(1/d) : 0;
 *   q_j  = int(fma(x_j, id, 8.5)) truncated toward zero (NaN -> 0),
 *          then clamped to [0, 15] (reading: {v,-v,...} gives 16 for -v);
 *   bytes 0..1 = binary16(d) rounded to nearest even, little-endian;
 *   byte 2+j   = q_j | q_{j+16} << 4, j = 0..15. */
void oracle_q4_0_block(const float* x, uint8_t* out) {
    float mval = x[0], amax = fabsf(x[0]);
    for (int j = 1; j < Q4_BLOCK; j++) {
        float a = fabsf(x[j]);
        if (a > amax || (a == amax && (x[j] > mval || (x[j] == mval && !signbit(x[j]))))) {
            amax = a;
            mval = x[j];
        }
    }
    float d = mval / -8.0f;
    float id = (d != 0.0f) ? 1.0f / d : 0.0f;
    uint16_t hb = oracle_f16_encode((double)d);
    out[0] = (uint8_t)(hb & 0xFF);
    out[1] = (uint8_t)(hb >> 8);
    int q[Q4_BLOCK];
    for (int j = 0; j < Q4_BLOCK; j++) {
        float v = fmaf(x[j], id, 8.5f);
        int qi;
        if (!(v >= 0.0f)) qi = 0;       /* NaN and negatives (trunc -> <= 0) */
        else if (v >= 15.0f) qi = 15;
        else qi = (int)v;               /* truncation toward zero */
        q[j] = qi;
    }
    for (int j = 0; j < 16; j++) out[2 + j] = (uint8_t)(q[j] | (q[j + 16] << 4));
}

/* Dequantize one block to binary16 bits: out_j = fp16_rne((q_j - 8) * f32(d)),
 * the product taken in fp32. */
void oracle_q4_0_block_dequant(const uint8_t* blk, uint16_t* out) {
    uint16_t hb = (uint16_t)(blk[0] | (blk[1] << 8));
    float d = (float)oracle_f16_decode(hb);
    for (int j = 0; j < 16; j++) {
        int lo = blk[2 + j] & 15, hi = blk[2 + j] >> 4;
        float v0 = (float)(lo - 8) * d;
        float v1 = (float)(hi - 8) * d;
        out[j] = oracle_f16_encode((double)v0);
        out[j + 16] = oracle_f16_encode((double)v1);
    }
}

/* Append new K and V rows of each sequence into paged q4_0 pools.
 *   pools      [n_cells][n_kv_heads][head_dim/32 * 18] bytes (K and V);
 *   table      int32 [n_seqs][max_pages], physical page ids;
 *   src rows   k_src/v_src fp32 [total_new][n_kv_heads][head_dim], the new
 *              rows of sequence s are src_off[s] .. src_off[s+1]-1;
 *   position   of new row i of sequence s is pos0[s] + i;
 *   cell       = table[s][pos / page_size] * page_size + pos % page_size.
 * Each head-row goes through FWHT-256 x 1/16 (skipped with no_rotate, for
 * fixtures already in the rotated domain) and then 8 blocks of 32.
 * Rows whose page is outside the table or the pool are not written. */
int oracle_append_q4_0(uint8_t* k_pool, uint8_t* v_pool, int64_t n_cells, const int32_t* table,
                       int max_pages, int page_size, int n_kv_heads, int head_dim, int n_seqs,
                       const int32_t* pos0, const int64_t* src_off, const float* k_src,
                       const float* v_src, int no_rotate) {
    if (head_dim != 256 || page_size <= 0 || n_kv_heads <= 0 || n_seqs < 0) return ORACLE_ERR_ARG;
    int row_bytes = head_dim / Q4_BLOCK * Q4_BLOCK_BYTES;
    for (int s = 0; s < n_seqs; s++) {
        for (int64_t r = src_off[s]; r < src_off[s + 1]; r++) {
            int64_t pos = pos0[s] + (r - src_off[s]);
            int64_t page = pos / page_size;
            if (pos < 0 || page >= max_pages) continue;
            int64_t phys = table[(int64_t)s * max_pages + page];
            int64_t cell = phys * page_size + pos % page_size;
            if (phys < 0 || cell >= n_cells) continue;
            for (int plane = 0; plane < 2; plane++) {
                const float* src = plane ? v_src : k_src;
                uint8_t* pool = plane ? v_pool : k_pool;
                for (int h = 0; h < n_kv_heads; h++) {
                    float v[256];
                    memcpy(v, src + (r * n_kv_heads + h) * head_dim, sizeof(v));
                    if (!no_rotate) oracle_fwht256_orthonormal(v);
                    uint8_t* dst = pool + (cell * n_kv_heads + h) * row_bytes;
                    for (int b = 0; b < head_dim / Q4_BLOCK; b++)
                        oracle_q4_0_block(v + b * Q4_BLOCK, dst + b * Q4_BLOCK_BYTES);
                }
            }
        }
    }
    return ORACLE_OK;
}

/* Gather sequence s's positions 0 .. (dst_off[s+1]-dst_off[s])-1 from the
 * pools into binary16 rows (rotated domain, no inverse transform):
 * k_dst/v_dst [total][n_kv_heads][head_dim] at row dst_off[s] + pos.
 * Rows whose page is outside the table or the pool are left untouched. */
int oracle_gather_q4_0(const uint8_t* k_pool, const uint8_t* v_pool, int64_t n_cells,
                       const int32_t* table, int max_pages, int page_size, int n_kv_heads,
                       int head_dim, int n_seqs, const int64_t* dst_off, uint16_t* k_dst,
                       uint16_t* v_dst) {
    if (head_dim != 256 || page_size <= 0 || n_kv_heads <= 0 || n_seqs < 0) return ORACLE_ERR_ARG;
    int row_bytes = head_dim / Q4_BLOCK * Q4_BLOCK_BYTES;
    for (int s = 0; s < n_seqs; s++) {
        int64_t len = dst_off[s + 1] - dst_off[s];
        for (int64_t pos = 0; pos < len; pos++) {
            int64_t page = pos / page_size;
            if (page >= max_pages) continue;
            int64_t phys = table[(int64_t)s * max_pages + page];
            int64_t cell = phys * page_size + pos % page_size;
            if (phys < 0 || cell >= n_cells) continue;
            for (int plane = 0; plane < 2; plane++) {
                const uint8_t* pool = plane ? v_pool : k_pool;
                uint16_t* dst = plane ? v_dst : k_dst;
                for (int h = 0; h < n_kv_heads; h++) {
                    const uint8_t* src = pool + (cell * n_kv_heads + h) * row_bytes;
                    uint16_t* o = dst + ((dst_off[s] + pos) * n_kv_heads + h) * head_dim;
                    for (int b = 0; b < head_dim / Q4_BLOCK; b++)
                        oracle_q4_0_block_dequant(src + b * Q4_BLOCK_BYTES, o + b * Q4_BLOCK);
                }
            }
        }
    }
    return ORACLE_OK;
}
