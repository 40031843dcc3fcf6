/*
 * q4k_oracle.c — plain, slow, obviously-correct CPU reference (double
 * precision) for the GGUF Q4_K weight-only-quantised matmul path.
 *
 * TEST INFRASTRUCTURE ONLY: only tests/, the package smoke check and the
 * benchmark's CPU-baseline leg may load this library; the HIP library never
 * does, and the two share no code.
 *
 * Sources.  The pages ("Mac Qwen3.6-27B Metal Q4_K perf diagnosis", TL;DR and
 * §3; "Qwen3.6-27B on Apple M3 Pro — the llama.cpp parity bar", reconciliation
 * table) name the format — raw GGUF q4_k blocks kept resident and multiplied
 * by an f32 activation, checked against a CPU f32 reference — but do not spell
 * out its bits.  The layout below is the public GGUF Q4_K super-block
 * convention, taken as the plainest reading of "GGUF Q4_K":
 *
 *   bytes 0..1    d     IEEE binary16, little-endian (super-scale of the scales)
 *   bytes 2..3    dmin  IEEE binary16, little-endian (super-scale of the mins)
 *   bytes 4..15   s[12] eight 6-bit scales sc[] and eight 6-bit mins m[]
 *   bytes 16..143 qs    256 four-bit quants; in 32-byte group g, byte l holds
 *                       weight 64g+l in its low nibble and weight 64g+32+l in
 *                       its high nibble
 *
 * and weight k of the block, in sub-block j = k/32, is d*sc[j]*q_k - dmin*m[j].
 *
 * Parity pins (tests/test_oracle_*.py): every binary16 pattern against numpy;
 * hand-worked blocks (tests/golden/worked_blocks.txt); the all-ones closed
 * form; zero/one-hot/linearity invariants; exact-rational brute force; bf16
 * rounding against torch.
 */
#include "q4k_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define Q4K_WEIGHTS_PER_BLOCK 256
#define Q4K_BYTES_PER_BLOCK 144

static int g_threads = 0;

void oracle_set_threads(int32_t n) {
    g_threads = n;
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#endif
}

int32_t oracle_get_threads(void) {
#ifdef _OPENMP
    return (int32_t)omp_get_max_threads();
#else
    return 1;
#endif
}

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 31;
    int frac = h & 1023;
    double mag;
    if (expo == 0) {
        mag = ldexp((double)frac, -24);                 /* subnormal: frac * 2^-24 */
    } else if (expo == 31) {
        mag = frac ? NAN : INFINITY;
    } else {
        mag = ldexp((double)(1024 + frac), expo - 25);  /* (1 + frac/1024) * 2^(expo-15) */
    }
    return sign ? -mag : mag;
}

void oracle_unpack_scales(const uint8_t s[12], int32_t sc[8], int32_t mn[8]) {
    for (int j = 0; j < 4; ++j) {
        sc[j] = s[j] & 63;
        mn[j] = s[j + 4] & 63;
    }
    for (int j = 4; j < 8; ++j) {
        /* low four bits in s[8..11], high two bits in the top of s[0..7] */
        sc[j] = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        mn[j] = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

static int quant_at(const uint8_t *qs, int k) {
    int g = k / 64, r = k % 64;
    return (r < 32) ? (qs[32 * g + r] & 15) : (qs[32 * g + (r - 32)] >> 4);
}

void oracle_dequant_block(const uint8_t *blk, float out[256]) {
    uint16_t hd = (uint16_t)(blk[0] | (blk[1] << 8));
    uint16_t hm = (uint16_t)(blk[2] | (blk[3] << 8));
    double d = oracle_half_to_double(hd);
    double dmin = oracle_half_to_double(hm);
    int32_t sc[8], mn[8];
    oracle_unpack_scales(blk + 4, sc, mn);
    const uint8_t *qs = blk + 16;
    for (int k = 0; k < Q4K_WEIGHTS_PER_BLOCK; ++k) {
        int j = k / 32;
        /* Both products are exact in double; the difference is exact too
         * (a multiple of 2^-24 below 2^27), so the single cast is the only
         * rounding. */
        double w = d * (double)sc[j] * (double)quant_at(qs, k) - dmin * (double)mn[j];
        out[k] = (float)w;
    }
}

static int check_shape(int64_t M, int64_t K) {
    if (M < 0 || K < 0 || K % Q4K_WEIGHTS_PER_BLOCK) return -2;
    return 0;
}

int oracle_dequant(const uint8_t *w, int64_t M, int64_t K, float *out) {
    if (check_shape(M, K)) return -2;
    int64_t nb = K / Q4K_WEIGHTS_PER_BLOCK;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < M; ++r)
        for (int64_t b = 0; b < nb; ++b)
            oracle_dequant_block(w + (r * nb + b) * Q4K_BYTES_PER_BLOCK,
                                 out + r * K + b * Q4K_WEIGHTS_PER_BLOCK);
    return 0;
}

/* One row's dot product, k ascending, in double. */
static void row_dot(const uint8_t *row, const double *x, int64_t K, double *y, double *S) {
    float wblk[Q4K_WEIGHTS_PER_BLOCK];
    double acc = 0.0, aabs = 0.0;
    for (int64_t b = 0; b < K / Q4K_WEIGHTS_PER_BLOCK; ++b) {
        oracle_dequant_block(row + b * Q4K_BYTES_PER_BLOCK, wblk);
        for (int k = 0; k < Q4K_WEIGHTS_PER_BLOCK; ++k) {
            double p = (double)wblk[k] * x[b * Q4K_WEIGHTS_PER_BLOCK + k];
            acc += p;
            aabs += fabs(p);
        }
    }
    *y = acc;
    if (S) *S = aabs;
}

int oracle_gemv_rows_d(const uint8_t *w, const double *x, int64_t M, int64_t K,
                       const int64_t *rows, int64_t nrows, double *y, double *S) {
    if (check_shape(M, K)) return -2;
    int64_t n = rows ? nrows : M;
    int64_t row_bytes = (K / Q4K_WEIGHTS_PER_BLOCK) * Q4K_BYTES_PER_BLOCK;
    for (int64_t r = 0; r < n; ++r)
        if (rows && (rows[r] < 0 || rows[r] >= M)) return -1;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < n; ++r) {
        int64_t i = rows ? rows[r] : r;
        row_dot(w + i * row_bytes, x, K, &y[r], S ? &S[r] : NULL);
    }
    return 0;
}

int oracle_gemv_rows(const uint8_t *w, const float *x, int64_t M, int64_t K,
                     const int64_t *rows, int64_t nrows, double *y, double *S) {
    if (check_shape(M, K)) return -2;
    double *xd = (double *)malloc(sizeof(double) * (size_t)(K ? K : 1));
    if (!xd) return -4;
    for (int64_t k = 0; k < K; ++k) xd[k] = (double)x[k];
    int rc = oracle_gemv_rows_d(w, xd, M, K, rows, nrows, y, S);
    free(xd);
    return rc;
}

int oracle_gemv_batch_rows(const uint8_t *w, const float *X, int64_t M, int64_t K, int64_t N,
                           const int64_t *rows, int64_t nrows, double *Y, double *S) {
    if (check_shape(M, K) || N < 0) return -2;
    int64_t n = rows ? nrows : M;
    for (int64_t v = 0; v < N; ++v) {
        int rc = oracle_gemv_rows(w, X + v * K, M, K, rows, nrows, Y + v * n, S ? S + v * n : NULL);
        if (rc) return rc;
    }
    return 0;
}

/* bf16 keeps the upper 16 bits of a binary32 pattern.  The two candidates are
 * the value with the low 16 bits cleared (smaller magnitude) and the next bf16
 * of larger magnitude; pick the nearer, and on a tie the one whose last kept
 * bit is 0. */
float oracle_bf16_round(float v) {
    uint32_t bits;
    memcpy(&bits, &v, 4);
    uint32_t lo_bits = bits & 0xFFFF0000u;
    uint32_t hi_bits = lo_bits + 0x10000u;
    float lo, hi;
    memcpy(&lo, &lo_bits, 4);
    memcpy(&hi, &hi_bits, 4);
    double e_lo = fabs((double)v - (double)lo);
    double e_hi = fabs((double)hi - (double)v);
    if (e_lo < e_hi) return lo;
    if (e_hi < e_lo) return hi;
    return ((lo_bits >> 16) & 1u) ? hi : lo;
}

int oracle_gemm_sub(const uint8_t *w, const float *X, int64_t M, int64_t K, int64_t P,
                    const int64_t *rows, int64_t nrows, const int64_t *toks, int64_t ntok,
                    int32_t bf16_inputs, double *Y, double *S) {
    if (check_shape(M, K) || P < 0) return -2;
    int64_t nr = rows ? nrows : M;
    int64_t nt = toks ? ntok : P;
    int64_t nb = K / Q4K_WEIGHTS_PER_BLOCK;
    int64_t row_bytes = nb * Q4K_BYTES_PER_BLOCK;
    for (int64_t r = 0; r < nr; ++r)
        if (rows && (rows[r] < 0 || rows[r] >= M)) return -1;
    for (int64_t t = 0; t < nt; ++t)
        if (toks && (toks[t] < 0 || toks[t] >= P)) return -1;
    int fail = 0;
    #pragma omp parallel for schedule(dynamic, 4) reduction(|:fail)
    for (int64_t r = 0; r < nr; ++r) {
        int64_t i = rows ? rows[r] : r;
        float *wrow = (float *)malloc(sizeof(float) * (size_t)(K ? K : 1));
        if (!wrow) { fail = 1; continue; }
        for (int64_t b = 0; b < nb; ++b)
            oracle_dequant_block(w + i * row_bytes + b * Q4K_BYTES_PER_BLOCK,
                                 wrow + b * Q4K_WEIGHTS_PER_BLOCK);
        if (bf16_inputs)
            for (int64_t k = 0; k < K; ++k) wrow[k] = oracle_bf16_round(wrow[k]);
        for (int64_t t = 0; t < nt; ++t) {
            int64_t p = toks ? toks[t] : t;
            const float *xrow = X + p * K;
            double acc = 0.0, aabs = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double xv = bf16_inputs ? (double)oracle_bf16_round(xrow[k]) : (double)xrow[k];
                double prod = (double)wrow[k] * xv;
                acc += prod;
                aabs += fabs(prod);
            }
            Y[t * nr + r] = acc;
            if (S) S[t * nr + r] = aabs;
        }
        free(wrow);
    }
    return fail ? -4 : 0;
}

/* ---------------------------------------------------------------- Q8_0
 * The other GGUF block type the pages use (the lm_head matmul in Q8, "Mac
 * Qwen3.6-27B Metal Q4_K perf diagnosis", §2 decode profile; the GGUF->Q8
 * path of "Qwen3.6-27B on Apple M3 Pro — the llama.cpp parity bar").  Layout
 * per the public GGUF convention: 34 bytes per 32 weights, a binary16 scale d
 * (little-endian) followed by 32 two's-complement int8 quants; w_i = d * q_i.
 * The product of an 11-bit and an 8-bit significand is exact in f32. */
static int check_shape_q8(int64_t M, int64_t K) {
    return (M < 0 || K <= 0 || K % 32 != 0) ? -2 : 0;
}

void oracle_dequant_q8_0_block(const uint8_t *b, float out[32]) {
    const double d = oracle_half_to_double((uint16_t)(b[0] | (b[1] << 8)));
    for (int i = 0; i < 32; ++i) out[i] = (float)(d * (double)(int8_t)b[2 + i]);
}

int oracle_dequant_q8_0(const uint8_t *w, int64_t M, int64_t K, float *out) {
    if (check_shape_q8(M, K)) return -2;
    const int64_t nb = K / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < M; ++r)
        for (int64_t j = 0; j < nb; ++j)
            oracle_dequant_q8_0_block(w + (r * nb + j) * 34, out + r * K + j * 32);
    return 0;
}

/* y[r] = sum_k w_rk x_k in double, and S[r] = sum_k |w_rk x_k| (either may
 * be NULL), for the listed rows (rows NULL: all M). */
int oracle_gemv_q8_0_rows_d(const uint8_t *w, const double *x, int64_t M, int64_t K,
                            const int64_t *rows, int64_t nrows, double *y, double *S) {
    if (check_shape_q8(M, K)) return -2;
    const int64_t nb = K / 32, n = rows ? nrows : M;
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        const int64_t r = rows ? rows[t] : t;
        double acc = 0.0, sab = 0.0;
        float v[32];
        for (int64_t j = 0; j < nb; ++j) {
            oracle_dequant_q8_0_block(w + (r * nb + j) * 34, v);
            for (int i = 0; i < 32; ++i) {
                const double p = (double)v[i] * x[j * 32 + i];
                acc += p;
                sab += fabs(p);
            }
        }
        if (y) y[t] = acc;
        if (S) S[t] = sab;
    }
    return 0;
}

/* ---------------------------------------------------------------- Q6_K
 * The six-bit GGUF k-quant that q4_k_m files use next to Q4_K for some
 * tensors (the pages run the Qwen3.6-27B q4_k_m file: "Mac Qwen3.6-27B Metal
 * Q4_K perf diagnosis", §1).  Layout per the public GGUF convention, 210
 * bytes per 256 weights:
 *   bytes   0..127  ql: the low four bits of the quants
 *   bytes 128..191  qh: the high two bits
 *   bytes 192..207  sixteen two's-complement int8 scales, one per 16
 *                   consecutive weights
 *   bytes 208..209  d, binary16 (little-endian)
 * Write weight k as 128h + 32c + l (h in 0..1, c in 0..3, l in 0..31).  Its
 * low four bits are the low nibble (c = 0, 1) or the high nibble (c = 2, 3)
 * of ql[64h + 32(c mod 2) + l]; its high two bits are bits 2c and 2c+1 of
 * qh[32h + l].  With q_k in 0..63 the value is
 *   w_k = d * (sc[k / 16] * (q_k - 32)),
 * the integer product taken first.  It has at most 12 significant bits and d
 * at most 11, so w_k is exact in f32 (no rounding in any order; the stated
 * order fixes only the sign of a zero). */
static int check_shape_q6(int64_t M, int64_t K) {
    return (M < 0 || K <= 0 || K % 256 != 0) ? -2 : 0;
}

static int q6_quant(const uint8_t *b, int k) {
    const int h = k / 128, c = (k % 128) / 32, l = k % 32;
    const int lo_byte = b[64 * h + 32 * (c % 2) + l];
    const int lo = c < 2 ? (lo_byte & 15) : (lo_byte >> 4);
    const int hi = (b[128 + 32 * h + l] >> (2 * c)) & 3;
    return lo | (hi << 4);
}

void oracle_dequant_q6_k_block(const uint8_t *b, float out[256]) {
    const double d = oracle_half_to_double((uint16_t)(b[208] | (b[209] << 8)));
    for (int k = 0; k < 256; ++k) {
        const int sc = (int8_t)b[192 + k / 16];
        out[k] = (float)(d * (double)(sc * (q6_quant(b, k) - 32)));
    }
}

int oracle_dequant_q6_k(const uint8_t *w, int64_t M, int64_t K, float *out) {
    if (check_shape_q6(M, K)) return -2;
    const int64_t nb = K / 256;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < M; ++r)
        for (int64_t j = 0; j < nb; ++j)
            oracle_dequant_q6_k_block(w + (r * nb + j) * 210, out + r * K + j * 256);
    return 0;
}

/* y[r] = sum_k w_rk x_k in double, and S[r] = sum_k |w_rk x_k| (either may
 * be NULL), for the listed rows (rows NULL: all M). */
int oracle_gemv_q6_k_rows_d(const uint8_t *w, const double *x, int64_t M, int64_t K,
                            const int64_t *rows, int64_t nrows, double *y, double *S) {
    if (check_shape_q6(M, K)) return -2;
    const int64_t nb = K / 256, n = rows ? nrows : M;
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        const int64_t r = rows ? rows[t] : t;
        double acc = 0.0, sab = 0.0;
        float v[256];
        for (int64_t j = 0; j < nb; ++j) {
            oracle_dequant_q6_k_block(w + (r * nb + j) * 210, v);
            for (int i = 0; i < 256; ++i) {
                const double p = (double)v[i] * x[j * 256 + i];
                acc += p;
                sab += fabs(p);
            }
        }
        if (y) y[t] = acc;
        if (S) S[t] = sab;
    }
    return 0;
}

double oracle_rms(const double *v, int64_t n, double eps) {
    double ss = 0.0;
    for (int64_t i = 0; i < n; ++i) ss += v[i] * v[i];
    return sqrt(ss / (double)n + eps);
}

double oracle_silu(double g) { return g / (1.0 + exp(-g)); }

/* Normalised GEMV: out = W * (v / rms(v)).  Everything in double. */
static int gemv_rmsn(const uint8_t *w, int64_t M, int64_t K, const double *v, double eps,
                     double *out) {
    double *vn = (double *)malloc(sizeof(double) * (size_t)K);
    if (!vn) return -4;
    double r = oracle_rms(v, K, eps);
    for (int64_t k = 0; k < K; ++k) vn[k] = v[k] / r;
    int rc = oracle_gemv_rows_d(w, vn, M, K, NULL, 0, out, NULL);
    free(vn);
    return rc;
}

/* One MLP block of a token: the model's SwiGLU feed-forward with its RMSNorm
 * in the (1 + w) form ("Qwen3.6-27B on Apple M3 Pro — the llama.cpp parity
 * bar": the model description lists hidden 5120, intermediate 17408 with
 * SwiGLU and rms_norm_eps 1e-6; the fak-native status list names the
 * (1 + w) RMSNorm):
 *   n = x / rms(x) * (1 + nw)          (nw NULL: gain 1)
 *   g = W_gate n,  u = W_up n,  a = silu(g) * u
 *   y = r + W_down a                   (r NULL: no residual)
 * Everything in double.  Any of the outputs may be NULL; Sg, Su, Sd are the
 * sums of |w_ik n_k| (|w_ik a_k| for down) of the three matmuls. */
int oracle_mlp(const uint8_t *wg, const uint8_t *wu, const uint8_t *wd, int64_t hidden,
               int64_t inter, const float *x, const float *nw, double eps, const float *r,
               double *g_out, double *u_out, double *a_out, double *y_out, double *Sg,
               double *Su, double *Sd) {
    if (check_shape(inter, hidden) || check_shape(hidden, inter) || !x || eps < 0.0) return -2;
    double *n = (double *)malloc(sizeof(double) * (size_t)hidden);
    double *g = (double *)malloc(sizeof(double) * (size_t)inter);
    double *u = (double *)malloc(sizeof(double) * (size_t)inter);
    double *a = (double *)malloc(sizeof(double) * (size_t)inter);
    double *y = (double *)malloc(sizeof(double) * (size_t)hidden);
    int rc = (n && g && u && a && y) ? 0 : -4;
    if (!rc) {
        for (int64_t k = 0; k < hidden; ++k) n[k] = (double)x[k];
        const double rm = oracle_rms(n, hidden, eps);
        for (int64_t k = 0; k < hidden; ++k)
            n[k] = n[k] / rm * (nw ? 1.0 + (double)nw[k] : 1.0);
        rc = oracle_gemv_rows_d(wg, n, inter, hidden, NULL, 0, g, Sg);
    }
    if (!rc) rc = oracle_gemv_rows_d(wu, n, inter, hidden, NULL, 0, u, Su);
    if (!rc) {
        for (int64_t i = 0; i < inter; ++i) a[i] = oracle_silu(g[i]) * u[i];
        rc = oracle_gemv_rows_d(wd, a, hidden, inter, NULL, 0, y, Sd);
    }
    if (!rc) {
        if (r)
            for (int64_t j = 0; j < hidden; ++j) y[j] += (double)r[j];
        if (g_out) memcpy(g_out, g, sizeof(double) * (size_t)inter);
        if (u_out) memcpy(u_out, u, sizeof(double) * (size_t)inter);
        if (a_out) memcpy(a_out, a, sizeof(double) * (size_t)inter);
        if (y_out) memcpy(y_out, y, sizeof(double) * (size_t)hidden);
    }
    free(n); free(g); free(u); free(a); free(y);
    return rc;
}

/* The per-token chain of projection and MLP matmuls, with every matmul input
 * RMS-normalised (no gain) and the stand-in mixer taking the first mix_out.K
 * outputs of mix_in:
 *   u = W_in rmsn(h);          h += W_out rmsn(u[0:K_out])
 *   g = W_gate rmsn(h);        a = W_up rmsn(h)
 *   h += W_down rmsn(silu(g) * a)
 *   logits = W_lm rmsn(h)
 * Shapes follow the model card on "Qwen3.6-27B on Apple M3 Pro — the llama.cpp
 * parity bar" (architecture list) and the per-phase matmuls of "Mac Qwen3.6-27B
 * Metal Q4_K perf diagnosis", §2 decode table. */
int oracle_stack(const uint8_t *const *mats, const int64_t *Ms, const int64_t *Ks,
                 int32_t n_layers, int64_t hidden, double eps, const float *h0,
                 double *logits, double *hid_out) {
    if (n_layers < 0 || hidden <= 0) return -2;
    int64_t maxM = hidden;
    for (int64_t i = 0; i < 5 * (int64_t)n_layers + 1; ++i) {
        if (check_shape(Ms[i], Ks[i])) return -2;
        if (Ms[i] > maxM) maxM = Ms[i];
    }
    for (int32_t l = 0; l < n_layers; ++l) {
        const int64_t *m = Ms + 5 * l, *k = Ks + 5 * l;
        if (k[0] != hidden || k[1] > m[0] || m[1] != hidden || k[2] != hidden ||
            k[3] != hidden || m[2] != m[3] || k[4] != m[2] || m[4] != hidden)
            return -2;
    }
    if (Ks[5 * n_layers] != hidden) return -2;

    double *h = (double *)malloc(sizeof(double) * (size_t)hidden);
    double *u = (double *)malloc(sizeof(double) * (size_t)maxM);
    double *g = (double *)malloc(sizeof(double) * (size_t)maxM);
    double *a = (double *)malloc(sizeof(double) * (size_t)maxM);
    double *o = (double *)malloc(sizeof(double) * (size_t)hidden);
    int rc = (h && u && g && a && o) ? 0 : -4;
    if (!rc) {
        for (int64_t i = 0; i < hidden; ++i) h[i] = (double)h0[i];
        for (int32_t l = 0; l < n_layers && !rc; ++l) {
            const uint8_t *const *W = mats + 5 * l;
            const int64_t *m = Ms + 5 * l, *k = Ks + 5 * l;
            rc = gemv_rmsn(W[0], m[0], k[0], h, eps, u);                 /* mixer in  */
            if (!rc) rc = gemv_rmsn(W[1], m[1], k[1], u, eps, o);        /* mixer out */
            if (!rc) for (int64_t i = 0; i < hidden; ++i) h[i] += o[i];
            if (!rc) rc = gemv_rmsn(W[2], m[2], k[2], h, eps, g);        /* gate */
            if (!rc) rc = gemv_rmsn(W[3], m[3], k[3], h, eps, a);        /* up   */
            if (!rc) for (int64_t i = 0; i < m[2]; ++i) a[i] = oracle_silu(g[i]) * a[i];
            if (!rc) rc = gemv_rmsn(W[4], m[4], k[4], a, eps, o);        /* down */
            if (!rc) for (int64_t i = 0; i < hidden; ++i) h[i] += o[i];
            if (!rc && hid_out) memcpy(hid_out + (int64_t)l * hidden, h, sizeof(double) * (size_t)hidden);
        }
        if (!rc) rc = gemv_rmsn(mats[5 * n_layers], Ms[5 * n_layers], hidden, h, eps, logits);
    }
    free(h); free(u); free(g); free(a); free(o);
    return rc;
}
