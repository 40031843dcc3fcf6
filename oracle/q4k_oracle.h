/*
 * q4k_oracle.h — plain, slow CPU reference for the Q4_K matmul path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may call this library.  The product path
 * (the HIP library) never links, loads or calls it, and the two share no
 * code, headers, tables or constants.
 *
 * Every routine computes in double and keeps the plain definition of the
 * operation: no blocking, no fusion, no reordering.  Rows are distributed over
 * OpenMP threads, but each output is computed by one thread in a fixed order,
 * so results are bitwise identical for any thread count.
 */
#ifndef Q4K_ORACLE_H
#define Q4K_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* IEEE binary16 bit pattern -> double, from the format definition. */
double oracle_half_to_double(uint16_t h);

/* 12 packed bytes -> 8 six-bit scales and 8 six-bit mins. */
void oracle_unpack_scales(const uint8_t s[12], int32_t sc[8], int32_t mn[8]);

/* One 144-byte super-block -> 256 f32 weights (exact value rounded once). */
void oracle_dequant_block(const uint8_t *blk, float out[256]);

/* M x K matrix of super-blocks (row-major, K/256 blocks per row) -> f32 [M][K]. */
int oracle_dequant(const uint8_t *w, int64_t M, int64_t K, float *out);

/* y[r] = sum_k w[rows[r]][k] * x[k] and S[r] = sum_k |w*x| for the listed rows
 * (rows == NULL: all M rows, in order).  x is f32 [K]. */
int oracle_gemv_rows(const uint8_t *w, const float *x, int64_t M, int64_t K,
                     const int64_t *rows, int64_t nrows, double *y, double *S);

/* Same with a double input vector. */
int oracle_gemv_rows_d(const uint8_t *w, const double *x, int64_t M, int64_t K,
                       const int64_t *rows, int64_t nrows, double *y, double *S);

/* Batched: X f32 [N][K] -> Y[n][r], S[n][r] for the listed rows. */
int oracle_gemv_batch_rows(const uint8_t *w, const float *X, int64_t M, int64_t K, int64_t N,
                           const int64_t *rows, int64_t nrows, double *Y, double *S);

/* Nearest bf16 value (ties to even) of a finite f32, returned as f32. */
float oracle_bf16_round(float v);

/* GEMM sub-block: X f32 [P][K].  For tokens toks[t] (NULL: all P) and rows
 * rows[r] (NULL: all M):  Y[t][r] = sum_k w*X, S[t][r] = sum_k |w*X|.
 * With bf16_inputs != 0, w and X are first rounded to bf16 (RNE). */
int oracle_gemm_sub(const uint8_t *w, const float *X, int64_t M, int64_t K, int64_t P,
                    const int64_t *rows, int64_t nrows, const int64_t *toks, int64_t ntok,
                    int32_t bf16_inputs, double *Y, double *S);

/* Q8_0 (34 bytes per 32 weights: binary16 d, 32 int8 q; w = d*q). */
void oracle_dequant_q8_0_block(const uint8_t *b, float out[32]);
int oracle_dequant_q8_0(const uint8_t *w, int64_t M, int64_t K, float *out);
int oracle_gemv_q8_0_rows_d(const uint8_t *w, const double *x, int64_t M, int64_t K,
                            const int64_t *rows, int64_t nrows, double *y, double *S);

/* Q6_K (210 bytes per 256 weights: ql[128], qh[64], int8 sc[16], binary16 d;
 * w = d * (sc * (q - 32)), q six bits). */
void oracle_dequant_q6_k_block(const uint8_t *b, float out[256]);
int oracle_dequant_q6_k(const uint8_t *w, int64_t M, int64_t K, float *out);
int oracle_gemv_q6_k_rows_d(const uint8_t *w, const double *x, int64_t M, int64_t K,
                            const int64_t *rows, int64_t nrows, double *y, double *S);

/* Root mean square with epsilon: sqrt(mean(v^2) + eps). */
double oracle_rms(const double *v, int64_t n, double eps);

/* SiLU: g / (1 + exp(-g)). */
double oracle_silu(double g);

/* One MLP block: n = x / rms(x) * (1 + nw) (nw NULL: gain 1), a = silu(W_gate n)
 * * (W_up n), y = r + W_down a (r NULL: 0).  wg, wu: [inter][hidden];
 * wd: [hidden][inter].  Outputs double, each may be NULL: g, u, a [inter],
 * y [hidden], and the sums of |w x| of the three matmuls Sg, Su [inter],
 * Sd [hidden]. */
int oracle_mlp(const uint8_t *wg, const uint8_t *wu, const uint8_t *wd, int64_t hidden,
               int64_t inter, const float *x, const float *nw, double eps, const float *r,
               double *g_out, double *u_out, double *a_out, double *y_out, double *Sg,
               double *Su, double *Sd);

/* Decode matmul chain.  mats holds 5*n_layers + 1 matrices in the order
 * (mix_in, mix_out, gate, up, down) per layer, then lm_head; Ms/Ks their
 * shapes.  h0 is f32 [hidden]; logits (double) gets lm_head's M outputs.
 * If hid_out != NULL it receives the residual stream after every layer,
 * double [n_layers][hidden]. */
int oracle_stack(const uint8_t *const *mats, const int64_t *Ms, const int64_t *Ks,
                 int32_t n_layers, int64_t hidden, double eps, const float *h0,
                 double *logits, double *hid_out);

/* Number of OpenMP threads used by the row loops (0 = leave the default). */
void oracle_set_threads(int32_t n);
int32_t oracle_get_threads(void);

/* Token mixers (mixer_oracle.c): one decode step of the Gated DeltaNet
 * recurrence and of gated full attention, in double.  See that file for the
 * equations.  Return 0, or -1 for bad sizes. */
int oracle_gdn_step(int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv, double eps, const double *u,
                    const double *conv_w, const double *a_log, const double *dt_bias,
                    const double *norm_w, double *conv_state, double *S, double *out);
int oracle_attn_step(int32_t Hq, int32_t Hkv, int32_t D, int32_t R, double theta, double eps,
                     const double *u, const double *q_norm_w, const double *k_norm_w,
                     double *k_cache, double *v_cache, int64_t cap, int64_t pos, double *out);

#ifdef __cplusplus
}
#endif
#endif
