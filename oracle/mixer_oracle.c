/*
 * mixer_oracle.c — plain double-precision CPU reference for the two token
 * mixers of the hybrid model, one decode token at a time.
 *
 * TEST INFRASTRUCTURE ONLY (see q4k_oracle.h): shares no code with the HIP
 * library.
 *
 * Source.  "Qwen3.6-27B on Apple M3 Pro — the llama.cpp parity bar",
 * architecture list: 48 linear-attention layers are Gated DeltaNet with a
 * depthwise causal convolution of kernel 4, 16 key heads and 48 value heads
 * of dimension 128, a swish output gate and an f32 recurrent state; 16
 * full-attention layers have 24 query heads and 4 key/value heads of
 * dimension 256, an output gate, partial rotary embedding over a quarter of
 * each head (theta 1e7), per-head q/k RMSNorm, and the (1 + w) RMSNorm form.
 * The status list of the same page names the pieces (Gated DeltaNet
 * recurrence, sigmoid output gate, per-head qk-norm, partial RoPE).  The
 * pages give no equations; the readings below are the published Gated
 * DeltaNet delta rule and standard rotary attention, with every choice the
 * pages leave open listed in the file that documents the design.
 *
 * Gated DeltaNet step (per token):
 *   u = [q (Hk*Dk) | k (Hk*Dk) | v (Hv*Dv) | z (Hv*Dv) | b (Hv) | a (Hv)]
 *   conv: for each of the C = 2*Hk*Dk + Hv*Dv channels of [q|k|v],
 *         c = silu(sum_{i=0..3} conv_w[ch][i] * win[i]),
 *         win = (state[0], state[1], state[2], input), oldest first;
 *         the state becomes (win[1], win[2], win[3]).
 *   q_j, k_j (key head j): divided by sqrt(sum of squares + eps); q also by
 *         sqrt(Dk).
 *   value head h uses key head j = h / (Hv/Hk);
 *   beta_h = sigmoid(b_h);  g_h = -exp(a_log_h) * softplus(a_h + dt_bias_h);
 *   S_h (Dk x Dv) <- exp(g_h) * S_h;
 *   delta = beta_h * (v_h - S_h^T k_j);   S_h <- S_h + k_j delta^T;
 *   o_h = S_h^T q_j;
 *   out_h = norm_w * o_h / sqrt(mean(o_h^2) + eps) * silu(z_h).
 *   S is stored value-dimension major: S[h][dv][dk].
 *
 * Gated attention step at position pos (caches hold positions 0 .. pos-1):
 *   u = [per query head: q (D) | gate (D)] (Hq times), then k (Hkv*D), v (Hkv*D)
 *   q_h, k_g: x / sqrt(mean(x^2) + eps) * (1 + w)
 *   rotary on the first R dims: pairs (i, i + R/2), angle pos * theta^(-2i/R),
 *         (x_i, x_{i+R/2}) -> (x_i cos - x_{i+R/2} sin, x_{i+R/2} cos + x_i sin)
 *   caches[g][pos] <- (k_g, v_g)
 *   query head h attends with key/value head g = h / (Hq/Hkv):
 *   o_h = sum_t softmax_t(q_h . k_t / sqrt(D)) v_t,  t = 0 .. pos
 *   out_h = o_h * sigmoid(gate_h).
 */
#include "q4k_oracle.h"

#include <math.h>
#include <stdlib.h>

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }
static double silu(double x) { return x * sigmoid(x); }
static double softplus(double x) { return x > 30.0 ? x : log1p(exp(x)); }

int oracle_gdn_step(int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv, double eps, const double *u,
                    const double *conv_w, const double *a_log, const double *dt_bias,
                    const double *norm_w, double *conv_state, double *S, double *out) {
    if (Hk <= 0 || Hv <= 0 || Dk <= 0 || Dv <= 0 || Hv % Hk != 0) return -1;
    const int64_t nq = (int64_t)Hk * Dk, nv = (int64_t)Hv * Dv;
    const int64_t C = 2 * nq + nv;
    const double *z = u + C, *b = u + C + nv, *a = u + C + nv + Hv;
    double *c = (double *)malloc(sizeof(double) * C);
    double *kv = (double *)malloc(sizeof(double) * Dv);
    if (!c || !kv) {
        free(c);
        free(kv);
        return -2;
    }
    /* causal depthwise convolution over the last four inputs, then silu */
    for (int64_t ch = 0; ch < C; ++ch) {
        double *st = conv_state + 3 * ch;
        const double win[4] = {st[0], st[1], st[2], u[ch]};
        double s = 0.0;
        for (int i = 0; i < 4; ++i) s += conv_w[4 * ch + i] * win[i];
        c[ch] = silu(s);
        st[0] = win[1];
        st[1] = win[2];
        st[2] = win[3];
    }
    double *q = c, *k = c + nq, *v = c + 2 * nq;
    /* L2 normalisation of every query and key head; queries also by 1/sqrt(Dk) */
    for (int32_t j = 0; j < Hk; ++j) {
        double sq = 0.0, sk = 0.0;
        for (int32_t d = 0; d < Dk; ++d) {
            sq += q[(int64_t)j * Dk + d] * q[(int64_t)j * Dk + d];
            sk += k[(int64_t)j * Dk + d] * k[(int64_t)j * Dk + d];
        }
        const double fq = 1.0 / sqrt(sq + eps) / sqrt((double)Dk), fk = 1.0 / sqrt(sk + eps);
        for (int32_t d = 0; d < Dk; ++d) {
            q[(int64_t)j * Dk + d] *= fq;
            k[(int64_t)j * Dk + d] *= fk;
        }
    }
    const int32_t rep = Hv / Hk;
    for (int32_t h = 0; h < Hv; ++h) {
        const double *kj = k + (int64_t)(h / rep) * Dk, *qj = q + (int64_t)(h / rep) * Dk;
        const double *vh = v + (int64_t)h * Dv;
        double *Sh = S + (int64_t)h * Dv * Dk; /* Sh[dv * Dk + dk] = S_h[dk][dv] */
        const double beta = sigmoid(b[h]);
        const double g = -exp(a_log[h]) * softplus(a[h] + dt_bias[h]);
        const double alpha = exp(g);
        for (int64_t e = 0; e < (int64_t)Dv * Dk; ++e) Sh[e] *= alpha;
        for (int32_t dv = 0; dv < Dv; ++dv) { /* (S^T k)[dv] */
            double s = 0.0;
            for (int32_t dk = 0; dk < Dk; ++dk) s += Sh[(int64_t)dv * Dk + dk] * kj[dk];
            kv[dv] = s;
        }
        for (int32_t dv = 0; dv < Dv; ++dv) {
            const double delta = beta * (vh[dv] - kv[dv]);
            for (int32_t dk = 0; dk < Dk; ++dk) Sh[(int64_t)dv * Dk + dk] += kj[dk] * delta;
        }
        double ms = 0.0;
        double *oh = out + (int64_t)h * Dv;
        for (int32_t dv = 0; dv < Dv; ++dv) { /* (S^T q)[dv] */
            double s = 0.0;
            for (int32_t dk = 0; dk < Dk; ++dk) s += Sh[(int64_t)dv * Dk + dk] * qj[dk];
            oh[dv] = s;
            ms += s * s;
        }
        const double inv = 1.0 / sqrt(ms / Dv + eps);
        const double *zh = z + (int64_t)h * Dv;
        for (int32_t dv = 0; dv < Dv; ++dv) oh[dv] = norm_w[dv] * (oh[dv] * inv) * silu(zh[dv]);
    }
    free(c);
    free(kv);
    return 0;
}

/* x <- x / sqrt(mean(x^2) + eps) * (1 + w) over n values */
static void rmsnorm_1pw(double *x, const double *w, int32_t n, double eps) {
    double s = 0.0;
    for (int32_t i = 0; i < n; ++i) s += x[i] * x[i];
    const double inv = 1.0 / sqrt(s / n + eps);
    for (int32_t i = 0; i < n; ++i) x[i] = x[i] * inv * (1.0 + w[i]);
}

static void rotate(double *x, int32_t R, double theta, int64_t pos) {
    const int32_t half = R / 2;
    for (int32_t i = 0; i < half; ++i) {
        const double ang = (double)pos * pow(theta, -2.0 * i / R);
        const double cs = cos(ang), sn = sin(ang);
        const double x1 = x[i], x2 = x[i + half];
        x[i] = x1 * cs - x2 * sn;
        x[i + half] = x2 * cs + x1 * sn;
    }
}

int oracle_attn_step(int32_t Hq, int32_t Hkv, int32_t D, int32_t R, double theta, double eps,
                     const double *u, const double *q_norm_w, const double *k_norm_w,
                     double *k_cache, double *v_cache, int64_t cap, int64_t pos, double *out) {
    if (Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0 || R < 0 || R > D || R % 2 != 0 ||
        pos < 0 || pos >= cap)
        return -1;
    double *qh = (double *)malloc(sizeof(double) * D);
    double *sc = (double *)malloc(sizeof(double) * (pos + 1));
    if (!qh || !sc) {
        free(qh);
        free(sc);
        return -2;
    }
    const double *ku = u + (int64_t)Hq * 2 * D, *vu = ku + (int64_t)Hkv * D;
    for (int32_t g = 0; g < Hkv; ++g) {
        double *kc = k_cache + ((int64_t)g * cap + pos) * D;
        double *vc = v_cache + ((int64_t)g * cap + pos) * D;
        for (int32_t d = 0; d < D; ++d) {
            kc[d] = ku[(int64_t)g * D + d];
            vc[d] = vu[(int64_t)g * D + d];
        }
        rmsnorm_1pw(kc, k_norm_w, D, eps);
        rotate(kc, R, theta, pos);
    }
    const int32_t rep = Hq / Hkv;
    for (int32_t h = 0; h < Hq; ++h) {
        const double *uq = u + (int64_t)h * 2 * D, *gate = uq + D;
        for (int32_t d = 0; d < D; ++d) qh[d] = uq[d];
        rmsnorm_1pw(qh, q_norm_w, D, eps);
        rotate(qh, R, theta, pos);
        const int32_t g = h / rep;
        double mx = -INFINITY;
        for (int64_t t = 0; t <= pos; ++t) {
            const double *kt = k_cache + ((int64_t)g * cap + t) * D;
            double s = 0.0;
            for (int32_t d = 0; d < D; ++d) s += qh[d] * kt[d];
            sc[t] = s / sqrt((double)D);
            if (sc[t] > mx) mx = sc[t];
        }
        double den = 0.0;
        for (int64_t t = 0; t <= pos; ++t) {
            sc[t] = exp(sc[t] - mx);
            den += sc[t];
        }
        double *oh = out + (int64_t)h * D;
        for (int32_t d = 0; d < D; ++d) {
            double s = 0.0;
            for (int64_t t = 0; t <= pos; ++t) s += sc[t] * v_cache[((int64_t)g * cap + t) * D + d];
            oh[d] = s / den * sigmoid(gate[d]);
        }
    }
    free(qh);
    free(sc);
    return 0;
}
