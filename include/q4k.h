/*
 * q4k.h — C ABI of the MI355X (gfx950) Q4_K weight-only-quantised matmul
 * library (libq4k.so).
 *
 * What it computes.  The pages ("Mac Qwen3.6-27B Metal Q4_K perf diagnosis",
 * TL;DR, §2 decode profile and §4b batched-GEMV witness; "Qwen3.6-27B on Apple
 * M3 Pro — the llama.cpp parity bar", architecture list) describe a
 * single-stream Qwen3.6-27B decode/prefill whose time is dominated by matmuls
 * against weights kept resident as raw GGUF q4_k blocks, multiplied by an f32
 * activation.  This library provides those matmuls: dequantisation, the
 * batch-1 GEMV, an N-vector GEMV that reads the weights once, the prefill GEMM
 * (bf16 MFMA), and the per-token chain of projection/MLP GEMVs replayed as one
 * HIP graph — the one-submission-per-token decode that the diagnosis page
 * names as the lever (§4).
 *
 * Weight format (public GGUF Q4_K convention; the pages name the format only).
 * A matrix of M rows and K columns (K a multiple of 256) is M rows of K/256
 * consecutive 144-byte super-blocks, each covering 256 consecutive weights:
 *   bytes 0..1   d     binary16, little-endian
 *   bytes 2..3   dmin  binary16, little-endian
 *   bytes 4..15  eight 6-bit scales sc[] and eight 6-bit mins m[]:
 *                s[j]&63 = sc[j], s[j+4]&63 = m[j] (j<4);
 *                sc[j] = (s[j+4]&15) | (s[j-4]>>6)<<4,
 *                m[j]  = (s[j+4]>>4) | (s[j]>>6)<<4     (j>=4)
 *   bytes 16..143 quants: in 32-byte group g, byte l holds weight 64g+l (low
 *                nibble) and weight 64g+32+l (high nibble)
 * Weight k (sub-block j = k/32) is  w = d*sc[j]*q - dmin*m[j].
 * The row stride is K/256*144 bytes; every block is 16-byte aligned when the
 * base pointer is.
 *
 * Conventions for every entry point.
 *  - Pointers are DEVICE pointers owned by the caller (e.g. from hipMalloc or a
 *    torch CUDA tensor).  The library never frees them.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls only enqueue work and return; results are valid once the stream
 *    has been synchronised.  Outputs are overwritten (not accumulated).
 *  - Inputs and outputs must not alias.
 *  - Arguments are validated before anything is enqueued; on error nothing is
 *    enqueued, a negative q4k_status is returned and q4k_last_error() gives a
 *    message (per calling thread).
 *  - M, N or P equal to 0 is a valid no-op.  K must be a positive multiple of
 *    256.  Dimension limits: see "Supported sizes" below.
 *  - Required alignment: 16 bytes for w, x/X, y/Y and out.
 *  - Results are deterministic: the same call on the same inputs returns the
 *    same bits (all reductions run in a fixed order; no float atomics).
 *  - Workspaces.  The GEMV-family calls, the MLP block and the GEMM use device
 *    scratch memory besides their inputs and outputs (partial sums of work
 *    split between workgroups and their arrival counters, the bf16 copy of
 *    X, the MLP's intermediate vectors).  The caller owns it:
 *    q4k_workspace_size() gives the bytes a call needs for its shape; pass
 *    a device buffer `ws` of at least `ws_bytes` >= that many bytes,
 *    256-byte aligned and zero-filled before its first use.  Every call
 *    returns the buffer to a state valid for the next call (its counters to
 *    zero), so a buffer is zeroed once, not per call.  If a call did not run
 *    to completion (a failed launch, a device fault), zero it again.  Calls
 *    that may execute at the same time (on different streams, or a captured
 *    graph replayed while other work runs) need distinct workspaces; calls
 *    ordered on one stream may share one, whatever their kind (every layout
 *    starts with the same counter region, which no call writes data into).
 *    A HIP graph that captured a call keeps using that call's workspace,
 *    which must outlive the graph.
 *  - Hot calls (everything except q4k_decode_stack_create and _destroy)
 *    allocate no memory and never synchronise; they may be captured into a
 *    HIP graph, the first call included.
 *  - Supported sizes: K <= 2^24 (so that 32-bit offsets inside a 64-row tile
 *    cannot wrap), M <= 2^30 rows; N and P <= 2^31 - 1.  Larger shapes return
 *    Q4K_EUNSUPPORTED before anything is enqueued.
 *  - Non-finite d/dmin propagate as IEEE arithmetic does; they are outside
 *    the tested contract.
 *  - Hardware assumption of the split-tile hand-off (gfx950): a tile cut
 *    between workgroups is finished by its last-arriving contributor.  The
 *    contributors store their partial sums with device-coherent (sc1) stores,
 *    wait until those stores have completed, and count themselves in with a
 *    device-scope atomic; the last one reads the partials with
 *    device-coherent loads.  sc1 accesses bypass the per-XCD L2, so the
 *    completed stores are visible to those loads without a cache-wide
 *    write-back/invalidate.  Under the HIP memory model the atomics are
 *    relaxed (release/acquire ordering would add an L2 write-back and
 *    invalidate per hand-off, which measured twice the GEMV's time).
 */
#ifndef Q4K_H
#define Q4K_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4K_BLOCK_WEIGHTS 256
#define Q4K_BLOCK_BYTES 144

typedef enum {
    Q4K_OK = 0,
    Q4K_EINVAL = -1,      /* null pointer with nonzero size, or bad enum/flag */
    Q4K_ESHAPE = -2,      /* negative dims, K not a positive multiple of 256, chain mismatch */
    Q4K_EALIGN = -3,      /* a pointer is not 16-byte aligned */
    Q4K_ENOMEM = -4,      /* device or host allocation failed */
    Q4K_EHIP = -5,        /* a HIP runtime call or kernel launch failed */
    Q4K_EUNSUPPORTED = -6 /* no gfx950 device, or a size beyond the supported range */
} q4k_status;

/* Message describing the last error returned on the calling thread ("" if none). */
const char *q4k_last_error(void);

/* Library version: major*10000 + minor*100 + patch. */
int q4k_version(void);

/*
 * Dequantise: out[i][k] = w_ik as f32, row-major [M][K] (the per-weight value
 * d*sc*q - dmin*m of a Q4_K super-block; the decode path reads the weights as
 * raw q4_k blocks, "Mac Qwen3.6-27B Metal Q4_K perf diagnosis", TL;DR and §4b,
 * and its prefill dequantises them for the matrix cores, §4b q4k_gemm).
 * Bit-exact: the value is the exact d*sc*q - dmin*m rounded once to f32, the
 * same for any evaluation order (every product is exact in f32).  w, out:
 * device pointers, 16-byte aligned; out holds M*K floats.  Needs no
 * workspace.  Errors: Q4K_ESHAPE, Q4K_EINVAL (NULL), Q4K_EALIGN.
 */
int q4k_dequant(const void *w, float *out, int64_t M, int64_t K, void *stream);

/*
 * Bytes of workspace a call needs (see "Workspaces" above), for the current
 * device and the current tuning knobs:
 *   Q4K_OP_GEMV, Q4K_OP_GEMV_Q8_0, Q4K_OP_GEMV_Q6_K:  M x K matrix;
 *   Q4K_OP_GEMV_BATCH: M x K matrix, N vectors;
 *   Q4K_OP_GEMM: M x K matrix, P = N tokens;
 *   Q4K_OP_MLP: M = inter, K = hidden (N ignored);
 *   Q4K_OP_GDN_STEP: M = key heads, K = value heads (N ignored);
 *   Q4K_OP_ATTN_STEP: M = query heads, K = kv heads, N = cache capacity.
 * Writes *bytes (a multiple of 256, possibly 0).  Errors: Q4K_EINVAL for an
 * unknown op or NULL bytes, and the shape errors of the call itself.
 */
enum {
    Q4K_OP_GEMV = 0, Q4K_OP_GEMV_BATCH = 1, Q4K_OP_GEMM = 2, Q4K_OP_GEMV_Q8_0 = 3,
    Q4K_OP_GEMV_Q6_K = 4, Q4K_OP_MLP = 5, Q4K_OP_GDN_STEP = 6, Q4K_OP_ATTN_STEP = 7
};
int q4k_workspace_size(int32_t op, int64_t M, int64_t K, int64_t N, size_t *bytes);

/*
 * Batch-1 GEMV: y[i] = sum_k w_ik * x[k], x f32 [K], y f32 [M].
 * The decode matmul ("Mac Qwen3.6-27B Metal Q4_K perf diagnosis", §2 decode
 * profile and §3): bandwidth-bound, one pass over the weight bytes.
 * f32 accumulation; |y - exact| stays within 1e-4 * sum_k |w_ik x_k| + 1e-6.
 * Each weight is formed exactly (d*sc*q - dmin*m rounded once) before it
 * meets x, so the bound also holds on rows whose weights cancel (a row of
 * zero weights gives exactly 0).  ws/ws_bytes: the call's workspace (see
 * "Workspaces"); Q4K_EINVAL if ws is NULL or ws_bytes is below
 * q4k_workspace_size(Q4K_OP_GEMV, M, K, 1), Q4K_EALIGN if ws is not
 * 256-byte aligned.
 */
int q4k_gemv(const void *w, const float *x, float *y, int64_t M, int64_t K, void *ws,
             size_t ws_bytes, void *stream);

/*
 * q4k_gemv for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture that must not call hipMalloc,
 * tight serving loops, harnesses that forbid allocation): same kernel, same
 * launch shape and the same output bits as q4k_gemv, with the split-tile
 * scratch (partial sums and arrival counters, about 0.6 MB) in a fixed
 * device array that the library holds on each GPU it runs on until the
 * process ends.  Every call on a GPU shares that GPU's array: calls that may
 * overlap in time on one GPU (different streams, concurrent graph replays)
 * race and must be ordered by the caller.  The counters start at zero and
 * every completed call leaves them at zero.  Limit: the launch may use at
 * most 1024 workgroups (the GEMV uses at most two per CU); beyond it the
 * call returns Q4K_EUNSUPPORTED before anything is enqueued.  Other errors
 * as q4k_gemv.  Allocates nothing, never synchronises.
 */
int q4k_gemv_noalloc(const void *w, const float *x, float *y, int64_t M, int64_t K,
                     void *stream);

/*
 * Q8_0 GEMV: y[i] = sum_k w_ik * x[k] for a Q8_0 matrix (public GGUF layout:
 * 34 bytes per 32 weights, a little-endian binary16 scale d then 32
 * two's-complement int8 quants, w = d * q; rows of K / 32 consecutive
 * blocks).  The pages run the lm_head matmul in Q8 ("Mac Qwen3.6-27B Metal
 * Q4_K perf diagnosis", §2 decode profile).  K must be a positive multiple
 * of 256 (so row runs stay 16-byte aligned), x f32 [K], y f32 [M]; w, x, y
 * 16-byte aligned.  f32 accumulation within the q4k_gemv bound (each quant
 * enters as the exact small integer q, the scale once per block).
 * Workspace: q4k_workspace_size(Q4K_OP_GEMV_Q8_0, M, K, 1).  Same error
 * codes as q4k_gemv.
 */
int q4k_gemv_q8_0(const void *w, const float *x, float *y, int64_t M, int64_t K, void *ws,
                  size_t ws_bytes, void *stream);

/*
 * Q6_K GEMV: y[i] = sum_k w_ik * x[k] for a Q6_K matrix (public GGUF layout,
 * the six-bit k-quant that q4_k_m files carry next to Q4_K; the pages run the
 * Qwen3.6-27B q4_k_m file, "Mac Qwen3.6-27B Metal Q4_K perf diagnosis", §1):
 * 210 bytes per 256 weights, ql[128] (low four bits of the quants), qh[64]
 * (high two bits), sixteen int8 scales (one per 16 weights), then a
 * little-endian binary16 d; w = d * sc * (q - 32) with q in 0..63; rows of
 * K / 256 consecutive blocks.  K must be a positive multiple of 1024 (rows
 * of a multiple of four blocks, so row runs stay 8-byte aligned; every
 * Qwen3.6-27B shape qualifies), otherwise Q4K_ESHAPE.  x f32 [K], y f32 [M];
 * w, x, y 16-byte aligned.  f32 accumulation within the q4k_gemv bound (each
 * quant enters as the exact small integer q - 32, the scales once per 16
 * weights).  Workspace: q4k_workspace_size(Q4K_OP_GEMV_Q6_K, M, K, 1).
 * Other error codes as q4k_gemv.
 */
int q4k_gemv_q6_k(const void *w, const float *x, float *y, int64_t M, int64_t K, void *ws,
                  size_t ws_bytes, void *stream);

/*
 * MLP block of one token (the model's SwiGLU feed-forward with its RMSNorm in
 * the (1 + w) form, "Qwen3.6-27B on Apple M3 Pro — the llama.cpp parity bar",
 * model description and the fak-native status list; the gate/up/down matmuls
 * are the decode GEMVs of "Mac Qwen3.6-27B Metal Q4_K perf diagnosis", §2):
 *   n = x / sqrt(mean(x^2) + eps) * (1 + norm_w)     (norm_w NULL: gain 1)
 *   a = silu(W_gate n) * (W_up n),  silu(g) = g / (1 + e^-g)
 *   y = resid + W_down a                              (resid NULL: 0)
 * w_gate, w_up: Q4_K [inter][hidden]; w_down: Q4_K [hidden][inter]; hidden and
 * inter positive multiples of 256.  x, norm_w, resid: f32 [hidden]; y: f32
 * [hidden]; act: optional f32 [inter] that receives a (NULL: kept in the
 * workspace).  Two GEMV launches (gate and up fused into one pass
 * with the SwiGLU in its epilogue, then down with the residual add) after a
 * small prologue that applies the gain.  y may alias x or resid (the down
 * pass runs after gate|up has read x); act must not alias the other vectors.
 * Each GEMV meets the q4k_gemv bound on its own inputs.  Workspace:
 * q4k_workspace_size(Q4K_OP_MLP, inter, hidden, 0).  Errors: Q4K_ESHAPE for
 * bad dims, Q4K_EINVAL for NULL w/x/y/ws, a workspace below that size, or
 * eps < 0 or not finite, Q4K_EALIGN for w, x, y, act not 16-byte aligned or
 * ws not 256-byte aligned.
 */
int q4k_mlp(const void *w_gate, const void *w_up, const void *w_down, int64_t hidden,
            int64_t inter, const float *x, const float *norm_w, float eps, const float *resid,
            float *y, float *act, void *ws, size_t ws_bytes, void *stream);

/*
 * N-vector GEMV in one launch, weights read once:
 *   Y[n][i] = sum_k w_ik * X[n][k],  X f32 [N][K], Y f32 [N][M].
 * The batched witness of "Mac Qwen3.6-27B Metal Q4_K perf diagnosis", §4b,
 * with N distinct activation vectors.  Any N >= 0; the kernels handle up to 16
 * vectors per weight pass (N = 1 gives the q4k_gemv bits).  Every weight is
 * formed exactly in f32.  Passes of up to eight vectors multiply in f32; a
 * pass of sixteen splits each weight and activation into two bf16 parts and
 * accumulates three bf16 products in f32 (w1 x1 + w1 x2 + w2 x1), which
 * leaves out at most about 3 * 2^-18 |w x| per product.  Workspace:
 * q4k_workspace_size(Q4K_OP_GEMV_BATCH, M, K, N).  Errors as q4k_gemv.
 */
int q4k_gemv_batch(const void *w, const float *X, float *Y, int64_t M, int64_t K, int64_t N,
                   void *ws, size_t ws_bytes, void *stream);

/*
 * Prefill GEMM:  Y[p][i] = sum_k w_ik * X[p][k],  X f32 [P][K], Y f32 [P][M].
 * The prompt-phase matmul ("Mac Qwen3.6-27B Metal Q4_K perf diagnosis", §2
 * prefill phases and §4b; "Qwen3.6-27B on Apple M3 Pro — the llama.cpp
 * parity bar", the compute-bound prefill argument).  Each weight is
 * dequantised exactly and rounded to bf16 (round to nearest even) straight
 * into a matrix-core fragment in registers, X is rounded to bf16 and staged
 * in LDS, products accumulate in f32 on the matrix cores; |y - exact| stays
 * within 5e-3 * sum_k |w_ik x_pk| + 1e-6.  The result is deterministic for a
 * given shape and device.  Workspace (the bf16 copy of X and the partial
 * tiles of stream-K): q4k_workspace_size(Q4K_OP_GEMM, M, K, P).
 * Errors as q4k_gemv.
 */
int q4k_gemm(const void *w, const float *X, float *Y, int64_t M, int64_t K, int64_t P,
             void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Token mixers of the hybrid model, one decode token ("Qwen3.6-27B on Apple
 * M3 Pro — the llama.cpp parity bar", architecture list: Gated DeltaNet
 * layers with a kernel-4 causal conv, 16 key / 48 value heads of 128, swish
 * output gate and an f32 recurrent state; full-attention layers with 24
 * query / 4 key-value heads of 256, output gate, partial rotary over a
 * quarter of each head with theta 1e7, (1 + w) q/k RMSNorm).  They run
 * between a layer's mixer-in and mixer-out projections ("Mac Qwen3.6-27B
 * Metal Q4_K perf diagnosis", §2: the recurrence and the attention/conv/
 * norm/gate work outside the matmuls; §4: on the device, one submission per
 * token).  All pointers are device pointers, f32, 16-byte aligned.
 * ---------------------------------------------------------------------- */

/* Gated DeltaNet, one token.  With Hk key heads, Hv value heads (a multiple
 * of Hk) and head dimension 128, C = (2*Hk + Hv) * 128 conv channels:
 *   u       [C + Hv*128 + 2*Hv]  mixer-in output: q | k | v | z | b | a
 *   conv_w  [C][4]   depthwise causal conv taps, oldest input first
 *   conv_state [C][3] the channel's last three inputs, oldest first (updated)
 *   a_log, dt_bias [Hv];  norm_w [128]
 *   state   [Hv][128][128] recurrent state, value-dimension major:
 *           state[h][dv][dk] (updated)
 *   out     [Hv*128]
 * Per token: c = silu(conv), q and k L2-normalised per key head (q also by
 * 1/sqrt(128)), value head h reads key head h / (Hv/Hk);
 * beta = sigmoid(b), alpha = exp(-exp(a_log) * softplus(a + dt_bias));
 * S <- alpha S; S <- S + k (beta (v - S^T k))^T; o = S^T q;
 * out = norm_w * o / sqrt(mean(o^2) + eps) * silu(z).
 * Workspace: q4k_workspace_size(Q4K_OP_GDN_STEP, Hk, Hv, 0).  One kernel,
 * four workgroups per value head, each taking 32 of the head's 128 state
 * rows (the state is read and written once, 64 KB per value head) and
 * forming the conv of the channels it reads; the last of a head's
 * workgroups applies the norm, and the last reader of a key head's q and k
 * channels shifts their conv state, each counted in on arrival counters in
 * the workspace's counter region that the call leaves at zero.  Errors:
 * Q4K_EINVAL (NULL, bad eps, small workspace), Q4K_ESHAPE (Hk, Hv not
 * positive or Hv not a multiple of Hk, key_dim or value_dim not 128),
 * Q4K_EALIGN. */
typedef struct {
    int32_t key_heads, value_heads, key_dim, value_dim; /* dims must be 128 */
    float eps;                                           /* e.g. 1e-6 */
    const float *conv_w, *a_log, *dt_bias, *norm_w;
} q4k_gdn_params;
int q4k_gdn_step(const q4k_gdn_params *p, const float *u, float *conv_state, float *state,
                 float *out, void *ws, size_t ws_bytes, void *stream);

/* Gated full attention, one token at position pos (0 <= pos < capacity;
 * the caches hold positions 0 .. pos-1 from earlier calls):
 *   u       [Hq*2*256 + 2*Hkv*256]  per query head [q | gate], then k, then v
 *   q_norm_w, k_norm_w [256]  (1 + w) RMSNorm weights
 *   k_cache, v_cache [Hkv][capacity][256]  position pos is written
 *   out     [Hq*256]
 * q and k: x / sqrt(mean(x^2) + eps) * (1 + w), then rotary on the first
 * rope_dim dims (pairs i, i + rope_dim/2; angle pos * theta^(-2i/rope_dim));
 * query head h attends with key/value head h / (Hq/Hkv):
 * out_h = softmax(q . k_t / 16) v over t = 0..pos, times sigmoid(gate_h).
 * Split-KV: the positions are cut into chunks of 64 spread over up to 64
 * workgroups per (kv head, group of query heads: at most 4, evened out), each
 * key and value row read once per group, then merged per query head in a
 * fixed order.
 * Workspace: q4k_workspace_size(Q4K_OP_ATTN_STEP, Hq, Hkv, capacity)
 * (per-chunk partials).  Errors: Q4K_EINVAL (NULL,
 * small workspace), Q4K_ESHAPE (head_dim not 256, Hq not a multiple of Hkv,
 * rope_dim odd or above 256, pos outside 0..capacity-1), Q4K_EALIGN. */
typedef struct {
    int32_t q_heads, kv_heads, head_dim, rope_dim; /* head_dim must be 256 */
    float rope_theta, eps;                          /* e.g. 1e7, 1e-6 */
    const float *q_norm_w, *k_norm_w;
} q4k_attn_params;
int q4k_attn_step(const q4k_attn_params *p, const float *u, float *k_cache, float *v_cache,
                  int64_t capacity, int64_t pos, float *out, void *ws, size_t ws_bytes,
                  void *stream);

/* ------------------------------------------------------------------------
 * Decode stack: the per-token chain of projection and MLP GEMVs of a
 * hybrid Gated-DeltaNet / attention model, with the activation kept on the
 * device and the whole chain replayed as ONE hipGraph launch per token
 * ("Mac Qwen3.6-27B Metal Q4_K perf diagnosis", §4, the one-submission-per-
 * token lever; layer shapes from "Qwen3.6-27B on Apple M3 Pro — the llama.cpp
 * parity bar", architecture list).
 *
 * Per layer l (rmsn(v) = v / sqrt(mean(v^2) + eps), no gain):
 *   u      = W_in  rmsn(h)                     mixer-in projection
 *   h_mid  = h + W_out rmsn(u[0 : mix_out.K])  stand-in mixer + out projection
 *   g      = W_gate rmsn(h_mid),  v = W_up rmsn(h_mid)
 *   a      = silu(g) * v
 *   h      = h_mid + W_down rmsn(a)
 * and finally logits = W_lm rmsn(h).  The stand-in mixer (first mix_out.K
 * outputs of the mixer-in projection) replaces the Gated-DeltaNet recurrence
 * and attention body, which are not matmuls.
 *
 * With Q4K_STACK_MIXERS in flags the stand-in gives way to each layer's real
 * token mixer: o = q4k_gdn_step(u) (kind 0) or q4k_attn_step(u, pos) (kind
 * 1), and h_mid = h + W_out rmsn(o).  The plan then owns every layer's
 * recurrent state (GDN conv state and S) or KV cache (attn_capacity
 * positions), all zero at creation and after q4k_decode_stack_reset; the
 * position lives on the device and the graph advances it by one per token,
 * so a token is still one graph launch.
 *
 * With Q4K_STACK_PERSISTENT in flags (stand-in mixer only) a token is ONE
 * cooperative kernel instead of a graph of kernels: every workgroup walks
 * the whole node list, loads its share of the next matrix while it waits for
 * the current one to finish (16 arrival counters per node), and hands activations over
 * through device-coherent stores.  The arithmetic of every node is that of
 * the graph plan, so both give the same logits bit for bit.  Each wait is
 * bounded (spin_limit polls, default 2^20); a wait that runs out records an
 * error that q4k_decode_stack_status reports, and the kernel still ends.
 * ---------------------------------------------------------------------- */

typedef struct {
    const void *w; /* borrowed device pointer to the super-blocks; must outlive the plan */
    int64_t M, K;
} q4k_mat;

typedef struct {
    int32_t kind; /* 0 = Gated-DeltaNet-shaped, 1 = attention-shaped (informational) */
    q4k_mat mix_in, mix_out, gate, up, down;
} q4k_layer;

typedef struct {
    q4k_gdn_params gdn;   /* kind 0 layers */
    q4k_attn_params attn; /* kind 1 layers */
} q4k_mixer;

#define Q4K_STACK_MIXERS 1
#define Q4K_STACK_PERSISTENT 2

typedef struct {
    int64_t hidden;          /* residual width (K of mix_in/gate/up/lm_head, M of mix_out/down) */
    int32_t n_layers;        /* >= 0 */
    const q4k_layer *layers; /* n_layers entries, copied at create time */
    q4k_mat lm_head;
    float eps;               /* RMS epsilon, e.g. 1e-6 */
    int32_t flags;           /* 0 (stand-in mixer, graph), Q4K_STACK_MIXERS or
                                Q4K_STACK_PERSISTENT (not both) */
    const q4k_mixer *mixers; /* Q4K_STACK_MIXERS: n_layers entries, copied (their weight
                                pointers are borrowed); otherwise ignored */
    int64_t attn_capacity;   /* Q4K_STACK_MIXERS: KV-cache positions of each attention layer */
    int32_t spin_limit;      /* Q4K_STACK_PERSISTENT: polls before a wait between nodes
                                gives up (0 = 2^20, about a second); otherwise ignored */
} q4k_stack_desc;

typedef struct q4k_stack q4k_stack; /* opaque plan: owns its graph and activation arena */

/* Validate the chain, allocate the arena, capture and instantiate the graph.
 * Synchronises `stream`.  Requirements: every K is a multiple of 256;
 * mix_in.K = gate.K = up.K = lm_head.K = hidden; mix_out.M = down.M = hidden;
 * mix_out.K <= mix_in.M; gate.M = up.M = down.K.  With Q4K_STACK_MIXERS, in
 * addition: a kind-0 layer's mix_in.M is (2*Hk + 2*Hv)*128 + 2*Hv and its
 * mix_out.K is Hv*128 (q4k_gdn_step's sizes); a kind-1 layer's mix_in.M is
 * (2*Hq + 2*Hkv)*256 and its mix_out.K is Hq*256 (q4k_attn_step's); the
 * mixer parameters as those calls require; attn_capacity >= 1. */
int q4k_decode_stack_create(const q4k_stack_desc *desc, void *stream, q4k_stack **out);

/* One token: copy h_in (f32 [hidden], device) into the arena, launch the
 * graph, copy the logits (f32 [lm_head.M], device) out.  logits may be NULL
 * to leave them in the arena only.  Enqueue-only; h_in/logits must stay valid
 * until the stream reaches this point.  A plan must not run on two streams
 * at once.  With mixers, Q4K_EINVAL once attn_capacity tokens have run
 * since creation or the last reset (nothing is enqueued then). */
int q4k_decode_stack(q4k_stack *s, const float *h_in, float *logits, void *stream);

/* Mixer states back to zero and the position to 0 (enqueued on `stream`);
 * a no-op without mixers. */
int q4k_decode_stack_reset(q4k_stack *s, void *stream);

/* Tokens launched since creation or the last reset. */
int q4k_decode_stack_position(q4k_stack *s, int64_t *pos);

/* Health of a persistent plan: synchronises `stream`, sets *status to 0 if
 * every wait between nodes ended normally since the last call, 1 if one ran
 * out of polls (the logits of the tokens since the last call are then not to
 * be trusted), and clears the record together with the plan's split-tile
 * counters, so that later tokens are sound again.  Always 0 for graph plans.  Not a hot call (it waits
 * for the device). */
int q4k_decode_stack_status(q4k_stack *s, void *stream, int32_t *status);

/* Arena buffers of the last token, for per-stage checks.  `which`:
 *   Q4K_BUF_H     residual stream entering layer `layer` (layer = n_layers:
 *                 the final residual that feeds lm_head)        [hidden]
 *   Q4K_BUF_U     mixer-in output u of `layer`                  [mix_in.M]
 *   Q4K_BUF_HMID  h_mid of `layer`                              [hidden]
 *   Q4K_BUF_G     gate output g of `layer` (after rmsn scaling) [gate.M]
 *   Q4K_BUF_V     up output v of `layer`                        [gate.M]
 *   Q4K_BUF_A     silu(g) * v of `layer`                        [gate.M]
 *   Q4K_BUF_LOGITS logits (layer ignored)                       [lm_head.M]
 * and with mixers:
 *   Q4K_BUF_MIX   mixer output o of `layer`                     [mix_out.K]
 *   Q4K_BUF_CONV_STATE, Q4K_BUF_GDN_STATE  a kind-0 layer's conv state
 *                 [C][3] and recurrent state [Hv][128][128] (current values)
 *   Q4K_BUF_K_CACHE, Q4K_BUF_V_CACHE  a kind-1 layer's caches
 *                 [Hkv][attn_capacity][256]
 * Sets *ptr to the device address and *n to the element count. */
enum {
    Q4K_BUF_H = 0, Q4K_BUF_U = 1, Q4K_BUF_HMID = 2, Q4K_BUF_G = 3,
    Q4K_BUF_V = 4, Q4K_BUF_A = 5, Q4K_BUF_LOGITS = 6, Q4K_BUF_MIX = 7,
    Q4K_BUF_CONV_STATE = 8, Q4K_BUF_GDN_STATE = 9, Q4K_BUF_K_CACHE = 10, Q4K_BUF_V_CACHE = 11
};
int q4k_decode_stack_buffer(q4k_stack *s, int32_t layer, int32_t which,
                            const float **ptr, int64_t *n);

/* Number of kernel nodes in the plan's graph (for launch-overhead
 * accounting); for a persistent plan, the number of GEMV nodes its one
 * kernel walks. */
int q4k_decode_stack_nodes(q4k_stack *s, int64_t *n_nodes);

/* Free the plan (graph, arena, workspace).  NULL-safe.  Synchronises the
 * device work the plan may still have in flight. */
void q4k_decode_stack_destroy(q4k_stack *s);

/* ------------------------------------------------------------------------
 * Self-check of the work partitions (host only, no device needed).
 * ---------------------------------------------------------------------- */

/* Runs, on the host, the range / owner / cut-tile arithmetic that the
 * kernels of `op` (Q4K_OP_GEMV, _GEMV_BATCH with N vectors, _MLP with M =
 * intermediate and K = hidden, _GEMM with P = N tokens, _GEMV_Q8_0,
 * _GEMV_Q6_K) would receive for an M x K matrix over `workgroups`
 * workgroups (0: the count the launch heuristics pick; the GEMM tile width
 * follows q4k_tune_gemm), for every workgroup, and checks that the ranges
 * cover the work exactly once, that every tile cut between workgroups has
 * consecutive contributors which all hold part of it, that every partial-sum
 * slot and arrival counter the kernels index lies inside the workspace
 * q4k_workspace_size reserves, and that every weight or activation byte a
 * fetch forms lies inside its operand (with 32-bit lane offsets that do not
 * wrap).  Q4K_OK, or Q4K_EINVAL naming the first violation in
 * q4k_last_error; Q4K_ESHAPE for shapes the entry points refuse. */
int q4k_check_partition(int32_t op, int64_t M, int64_t K, int64_t N, int32_t workgroups);

/* ------------------------------------------------------------------------
 * Launch-shape reporting and benchmark knobs.
 * ---------------------------------------------------------------------- */

/* Launch shape that q4k_gemv / q4k_gemv_batch pick for a shape (N
 * vectors): waves per workgroup (always 4) and the number of workgroups
 * (as many as the device holds at once for that kernel, at most one per
 * 64-row x 4-block work unit).  Without a device the count assumes 1024. */
int q4k_gemv_config(int64_t M, int64_t K, int64_t N, int32_t *waves_per_group,
                    int32_t *workgroups);

/* Tile width (tokens per workgroup tile: 32, 64, 128 or 256) and workgroup count
 * (the stream-K partition of the tile x super-block work) that q4k_gemm picks
 * for a shape. */
int q4k_gemm_config(int64_t M, int64_t K, int64_t P, int32_t *tile_tokens, int32_t *workgroups);

/* Force the GEMV workgroup count (workgroups in 1..16384, capped at the
 * number of work units; waves_per_group must be 0 or 4), or the GEMM tile
 * width (tile_tokens 0, 32, 64, 128 or 256) and workgroup count (0..4096, capped at
 * the number of tile x super-block work items); 0 restores the default of
 * that knob.  Process-wide and not synchronised with calls in flight: meant
 * for benchmark sweeps. */
int q4k_tune_gemv(int32_t waves_per_group, int32_t workgroups);
int q4k_tune_gemm(int32_t tile_tokens, int32_t workgroups);

#ifdef __cplusplus
}
#endif
#endif /* Q4K_H */
