/*
 * sanitize_driver.c — runs every entry point of the CPU oracle (oracle/*.c)
 * and of the input generator (synth/synth.c) on small ragged shapes, with
 * every buffer allocated at exactly the size the functions are documented to
 * touch.  Built with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitizers_cpu.py: an out-of-bounds access, a use after free or
 * an undefined operation anywhere in those sources aborts the run.  Also
 * checks that the documented bad-size returns are taken.
 * Host code only; no device is involved.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../oracle/q4k_oracle.h"

uint64_t synth_word(uint64_t key, uint64_t i);
uint16_t synth_half_bits(double v);
int synth_q4k_blocks(uint64_t key, uint64_t block0, uint64_t nblocks, uint8_t *out, double lo,
                     double hi);
int synth_q8_0_blocks(uint64_t key, uint64_t block0, uint64_t nblocks, uint8_t *out, double lo,
                      double hi);
int synth_q6_k_blocks(uint64_t key, uint64_t block0, uint64_t nblocks, uint8_t *out, double lo,
                      double hi);
void synth_normal_f32(uint64_t key, uint64_t n, float *out);
void synth_bytes(uint64_t key, uint64_t n, uint8_t *out);

static int failures = 0;
#define CHECK(c)                                                  \
    do {                                                          \
        if (!(c)) {                                               \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            ++failures;                                           \
        }                                                         \
    } while (0)

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static uint8_t *q4k(uint64_t key, int64_t M, int64_t K) {
    uint8_t *w = xmalloc((size_t)(M * (K / 256) * 144));
    CHECK(synth_q4k_blocks(key, 0, (uint64_t)(M * (K / 256)), w, 1e-4, 1e-3) == 0);
    return w;
}

static float *normal(uint64_t key, int64_t n) {
    float *v = xmalloc(sizeof(float) * (size_t)n);
    synth_normal_f32(key, (uint64_t)n, v);
    return v;
}

static double *dnormal(uint64_t key, int64_t n, double s) {
    float *f = normal(key, n);
    double *d = xmalloc(sizeof(double) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) d[i] = s * f[i];
    free(f);
    return d;
}

static int finite_all(const double *v, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(v[i])) return 0;
    return 1;
}

int main(void) {
    oracle_set_threads(3);
    CHECK(oracle_get_threads() == 3);
    /* generator */
    (void)synth_word(1, 2);
    CHECK(synth_half_bits(1.0) == 0x3C00);
    uint8_t *bytes = xmalloc(37);
    synth_bytes(5, 37, bytes);
    uint8_t *q8 = xmalloc(7 * 2 * 34);
    CHECK(synth_q8_0_blocks(6, 0, 14, q8, 1e-4, 1e-3) == 0);
    uint8_t *q6 = xmalloc(7 * 2 * 210);
    CHECK(synth_q6_k_blocks(7, 0, 14, q6, 1e-4, 1e-3) == 0);
    uint8_t *one = xmalloc(144);
    CHECK(synth_q4k_blocks(8, 0, 1, one, 1e9, 2e9) != 0); /* d outside binary16: flagged */
    free(one);

    /* half decode and scale unpack */
    for (uint32_t h = 0; h < 65536; h += 97) (void)oracle_half_to_double((uint16_t)h);
    int32_t sc[8], mn[8];
    oracle_unpack_scales(bytes, sc, mn);

    /* Q4_K: ragged row count, two and three blocks per row */
    const int64_t M = 37, K = 512, N = 3, P = 5;
    uint8_t *w = q4k(9, M, K);
    float blk[256];
    oracle_dequant_block(w, blk);
    float *deq = xmalloc(sizeof(float) * (size_t)(M * K));
    CHECK(oracle_dequant(w, M, K, deq) == 0);
    CHECK(oracle_dequant(w, M, 100, deq) != 0);
    float *x = normal(10, K);
    double *y = xmalloc(sizeof(double) * (size_t)M), *S = xmalloc(sizeof(double) * (size_t)M);
    CHECK(oracle_gemv_rows(w, x, M, K, NULL, M, y, S) == 0);
    CHECK(finite_all(y, M));
    const int64_t rows[3] = {0, 17, 36};
    CHECK(oracle_gemv_rows(w, x, M, K, rows, 3, y, S) == 0);
    double *xd = dnormal(11, K, 1.0);
    CHECK(oracle_gemv_rows_d(w, xd, M, K, NULL, M, y, S) == 0);
    float *X = normal(12, N * K);
    double *Y = xmalloc(sizeof(double) * (size_t)(N * M)), *SY = xmalloc(sizeof(double) * (size_t)(N * M));
    CHECK(oracle_gemv_batch_rows(w, X, M, K, N, NULL, M, Y, SY) == 0);
    (void)oracle_bf16_round(1.2345f);
    float *XP = normal(13, P * K);
    double *G = xmalloc(sizeof(double) * (size_t)(P * M)), *SG = xmalloc(sizeof(double) * (size_t)(P * M));
    CHECK(oracle_gemm_sub(w, XP, M, K, P, NULL, M, NULL, P, 0, G, SG) == 0);
    const int64_t toks[2] = {0, 4};
    CHECK(oracle_gemm_sub(w, XP, M, K, P, rows, 3, toks, 2, 1, G, SG) == 0);
    CHECK(finite_all(G, 6));

    /* Q8_0 and Q6_K: 7 rows */
    float *d8 = xmalloc(sizeof(float) * 7 * 64);
    CHECK(oracle_dequant_q8_0(q8, 7, 64, d8) == 0);
    double *x64 = dnormal(14, 64, 1.0), *y7 = xmalloc(sizeof(double) * 7), *s7 = xmalloc(sizeof(double) * 7);
    CHECK(oracle_gemv_q8_0_rows_d(q8, x64, 7, 64, NULL, 7, y7, s7) == 0);
    float *d6 = xmalloc(sizeof(float) * 7 * 512);
    CHECK(oracle_dequant_q6_k(q6, 7, 512, d6) == 0);
    CHECK(oracle_gemv_q6_k_rows_d(q6, xd, 7, 512, NULL, 7, y7, s7) == 0);

    /* glue, MLP block and the decode chain: hidden 256, inter 512, two layers */
    const int64_t H = 256, I = 512, MI = 384, V = 100;
    CHECK(oracle_rms(xd, K, 1e-6) > 0.0);
    (void)oracle_silu(-3.0);
    uint8_t *wg = q4k(20, I, H), *wu = q4k(21, I, H), *wd = q4k(22, H, I);
    float *xh = normal(23, H), *nw = normal(24, H), *rr = normal(25, H);
    double *g = xmalloc(sizeof(double) * I), *u = xmalloc(sizeof(double) * I), *a = xmalloc(sizeof(double) * I);
    double *yo = xmalloc(sizeof(double) * H), *Sg = xmalloc(sizeof(double) * I), *Su = xmalloc(sizeof(double) * I);
    double *Sd = xmalloc(sizeof(double) * H);
    CHECK(oracle_mlp(wg, wu, wd, H, I, xh, nw, 1e-6, rr, g, u, a, yo, Sg, Su, Sd) == 0);
    CHECK(oracle_mlp(wg, wu, wd, H, I, xh, NULL, 1e-6, NULL, NULL, NULL, NULL, yo, NULL, NULL, NULL) == 0);
    CHECK(finite_all(yo, H));
    const uint8_t *mats[11];
    int64_t Ms[11], Ks[11];
    for (int l = 0; l < 2; ++l) {
        const int64_t sh[5][2] = {{MI, H}, {H, 256}, {I, H}, {I, H}, {H, I}};
        for (int m = 0; m < 5; ++m) {
            Ms[5 * l + m] = sh[m][0];
            Ks[5 * l + m] = sh[m][1];
            mats[5 * l + m] = q4k(30 + 5 * l + m, sh[m][0], sh[m][1]);
        }
    }
    Ms[10] = V;
    Ks[10] = H;
    mats[10] = q4k(40, V, H);
    double *logits = xmalloc(sizeof(double) * V), *hid = xmalloc(sizeof(double) * 2 * H);
    CHECK(oracle_stack(mats, Ms, Ks, 2, H, 1e-6, xh, logits, hid) == 0);
    CHECK(finite_all(logits, V));

    /* token mixers: GDN with Hk = 2, Hv = 4 (128-dim heads); attention with
     * Hq = 2, Hkv = 1 (256-dim heads), rotary over 64 dims, four positions */
    {
        const int Hk = 2, Hv = 4, D = 128;
        const int64_t C = (int64_t)(2 * Hk + Hv) * D, NU = C + (int64_t)Hv * D + 2 * Hv;
        double *uu = dnormal(50, NU, 1.0), *cw = dnormal(51, 4 * C, 0.5), *al = dnormal(52, Hv, 0.5);
        double *dt = dnormal(53, Hv, 0.5), *nwd = dnormal(54, D, 0.1), *cs = dnormal(55, 3 * C, 1.0);
        double *Sst = dnormal(56, (int64_t)Hv * D * D, 0.05), *o = xmalloc(sizeof(double) * Hv * D);
        CHECK(oracle_gdn_step(Hk, Hv, D, D, 1e-6, uu, cw, al, dt, nwd, cs, Sst, o) == 0);
        CHECK(finite_all(o, (int64_t)Hv * D));
        CHECK(oracle_gdn_step(3, Hv, D, D, 1e-6, uu, cw, al, dt, nwd, cs, Sst, o) != 0);
        free(uu); free(cw); free(al); free(dt); free(nwd); free(cs); free(Sst); free(o);
    }
    {
        const int Hq = 2, Hkv = 1, D = 256, R = 64;
        const int64_t cap = 4, NA = (int64_t)Hq * 2 * D + 2 * (int64_t)Hkv * D;
        double *qw = dnormal(60, D, 0.2), *kw = dnormal(61, D, 0.2);
        double *kc = xmalloc(sizeof(double) * Hkv * cap * D), *vc = xmalloc(sizeof(double) * Hkv * cap * D);
        double *o = xmalloc(sizeof(double) * Hq * D);
        for (int64_t pos = 0; pos < cap; ++pos) {
            double *uu = dnormal(62 + pos, NA, 1.0);
            CHECK(oracle_attn_step(Hq, Hkv, D, R, 1e7, 1e-6, uu, qw, kw, kc, vc, cap, pos, o) == 0);
            CHECK(finite_all(o, (int64_t)Hq * D));
            free(uu);
        }
        double *uu = dnormal(70, NA, 1.0);
        CHECK(oracle_attn_step(Hq, Hkv, D, R, 1e7, 1e-6, uu, qw, kw, kc, vc, cap, cap, o) != 0);
        CHECK(oracle_attn_step(Hq, Hkv, D, 63, 1e7, 1e-6, uu, qw, kw, kc, vc, cap, 0, o) != 0);
        free(uu); free(qw); free(kw); free(kc); free(vc); free(o);
    }

    for (int i = 0; i < 11; ++i) free((void *)mats[i]);
    free(logits); free(hid); free(wg); free(wu); free(wd); free(xh); free(nw); free(rr);
    free(g); free(u); free(a); free(yo); free(Sg); free(Su); free(Sd);
    free(d8); free(x64); free(y7); free(s7); free(d6);
    free(G); free(SG); free(XP); free(Y); free(SY); free(X); free(xd); free(y); free(S); free(x);
    free(deq); free(w); free(q8); free(q6); free(bytes);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("sanitized oracle and generator runs clean\n");
    return 0;
}
