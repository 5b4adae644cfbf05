/*
 * Plain CPU oracle for the Gated DeltaNet record / replay / GQA-expand path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this file: only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code, header, table or helper with the
 * HIP library.
 *
 * Every operation is written from the equations of the method, one pass per
 * equation, in double precision, with floating-point contraction disabled at
 * build time (-ffp-contract=off) so that each product and sum is rounded once,
 * in the order written here.  Inputs arrive already widened to double; the
 * widening of fp32 / fp16 / bf16 to double is exact, so the oracle sees the
 * same numbers the device sees.
 *
 * Sources (pages as published):
 *   [P1] metaltile-std 0.1.0, src/ffai/gated_delta_replay.rs -- the module
 *        documentation ("Two kernels", "Tape layout"), the record kernel
 *        (macro `gated_delta_record!`) and the replay kernel (macro
 *        `state_replay!`).
 *   [P3] mlx-native 0.6.5, mlx_native/ops/repeat_tiled.rs -- the module
 *        documentation ("Mapping") and `dispatch_repeat_tiled_f32`.
 *   [P2] moeflux 0.1.0-pre.3, src/riir/backend/gpu/gpu_norm.rs -- the
 *        documentation of `gpu_rms_norm_fused` (GPU RMSNorm with bf16 weights)
 *        and of `encode_rms_norm_bf16_fused_n_tokens` (one row per token).
 *
 * Layouts (dense, row-major, no strides), following [P1] "Tape layout" and the
 * index arithmetic of both [P1] kernels:
 *   q, k          [B, T, Hk, Dk]
 *   v, y, delta   [B, T, Hv, Dv]
 *   g, beta       [B, T, Hv]
 *   state         [B, Hv, Dv, Dk]   (row = value index dv, column = key index dk)
 *   mask          [B, T]            (uint32, step active iff value > 0)
 *   k_log         [B, T, Hv, Dk]    (keys already expanded to value heads)
 *   g_log         [B, T, Hv]
 *
 * Parity status: every function below is pinned by the CPU test suite against
 * hand-computed values, closed forms and independent formulations (the
 * transition-matrix form of the gated delta rule, numpy repeat / tile for the
 * head maps).  The summation order of the two Dk-length dot products is not
 * fixed by the pages; that order is "parity unpinned" beyond tolerance.  The
 * RMSNorm is pinned by a hand-worked case, closed forms (constant and one-hot
 * rows, unit RMS), scale invariance and the per-column weight; the order of
 * its sum of squares is likewise unpinned beyond tolerance.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

enum { ORACLE_GQA_BLOCK = 0, ORACLE_GQA_TILED = 1 };

/* Key head that serves value head hv.
 * Block map: consecutive value heads share one key head, hk = hv / (Hv / Hk)
 * ([P1] record kernel, head-index derivation).
 * Tiled map: value head hv reads key head hv mod Hk ([P3] "Mapping",
 * dst[t, h, k] = src[t, h % Hg, k]). */
static uint32_t oracle_key_head(uint32_t hv, uint32_t Hk, uint32_t Hv, int map)
{
    if (map == ORACLE_GQA_BLOCK) {
        uint32_t group = Hv / Hk;
        return hv / group;
    }
    return hv % Hk;
}

/* sum_i a[i] * b[i], in index order. */
static double oracle_dot(const double* a, const double* b, uint32_t n)
{
    double acc = 0.0;
    for (uint32_t i = 0; i < n; ++i) acc = acc + a[i] * b[i];
    return acc;
}

static int oracle_step_active(const uint32_t* mask, uint32_t T, uint32_t b, uint32_t t)
{
    /* [P1] record kernel: with has_mask == 0 every step is active, otherwise
     * the step runs iff mask[b*T + t] > 0.  A NULL mask plays has_mask == 0. */
    if (mask == NULL) return 1;
    return mask[(size_t)b * T + t] > 0u;
}

/*
 * Gated delta-rule forward step with innovation-tape capture
 * ([P1] macro `gated_delta_record!`, and the module documentation's
 * description of `gated_delta_step_record`).
 *
 * For every (b, hv) and every value row dv of S, for t = 0 .. T-1 with the step
 * active, the gated delta rule on row dv:
 *     (1) S[dv, :] <- g_t S[dv, :]                       (the gate decays the row first)
 *     (2) kv = S[dv, :] . k_t                            (prediction of the decayed row)
 *     (3) delta = beta_t (v_t[dv] - kv)                  (innovation)
 *     (4) delta_log[b, t, hv, dv] = delta                (tape)
 *     (5) S[dv, :] <- S[dv, :] + delta k_t               (rank-one correction)
 *     (6) y[b, t, hv, dv] = S[dv, :] . q_t               (output from the corrected row)
 * Inactive steps change nothing and write nothing.  The final S goes to
 * state_out.  delta_log may be NULL (the plain forward step without a tape).
 *
 * Returns 0, or -1 when Hk does not divide Hv or a dimension is zero.
 */
int oracle_gdn_record(const double* q, const double* k, const double* v,
                      const double* g, const double* beta,
                      const double* state_in, const uint32_t* mask,
                      double* y, double* state_out, double* delta_log,
                      uint32_t B, uint32_t T, uint32_t Hk, uint32_t Hv,
                      uint32_t Dk, uint32_t Dv, int gqa_map)
{
    if (B == 0 || T == 0 || Hk == 0 || Hv == 0 || Dk == 0 || Dv == 0) return -1;
    if (Hv % Hk != 0) return -1;
    if (gqa_map != ORACLE_GQA_BLOCK && gqa_map != ORACLE_GQA_TILED) return -1;

    for (uint32_t b = 0; b < B; ++b) {
        for (uint32_t hv = 0; hv < Hv; ++hv) {
            uint32_t hk = oracle_key_head(hv, Hk, Hv, gqa_map);
            for (uint32_t dv = 0; dv < Dv; ++dv) {
                size_t row = (((size_t)b * Hv + hv) * Dv + dv) * Dk;
                double* S = state_out + row;
                /* The row starts from the input state (copy first so that
                 * state_out may alias state_in exactly). */
                if (S != state_in + row)
                    for (uint32_t i = 0; i < Dk; ++i) S[i] = state_in[row + i];

                for (uint32_t t = 0; t < T; ++t) {
                    if (!oracle_step_active(mask, T, b, t)) continue;
                    size_t bt = (size_t)b * T + t;
                    const double* kt = k + (bt * Hk + hk) * Dk;
                    const double* qt = q + (bt * Hk + hk) * Dk;
                    double gt = g[bt * Hv + hv];
                    double bet = beta[bt * Hv + hv];
                    size_t vo = (bt * Hv + hv) * Dv + dv;

                    /* (1) decay the row by the step's gate */
                    for (uint32_t i = 0; i < Dk; ++i) S[i] = gt * S[i];
                    /* (2) what the decayed row predicts for this key */
                    double kv = oracle_dot(S, kt, Dk);
                    /* (3) innovation: the prediction error, scaled by beta */
                    double delta = bet * (v[vo] - kv);
                    /* (4) the tape keeps the innovation */
                    if (delta_log != NULL) delta_log[vo] = delta;
                    /* (5) rank-one correction along the key */
                    for (uint32_t i = 0; i < Dk; ++i) S[i] = S[i] + delta * kt[i];
                    /* (6) output: the corrected row read against the query */
                    y[vo] = oracle_dot(S, qt, Dk);
                }
            }
        }
    }
    return 0;
}

/*
 * Tape replay onto a pre-record snapshot ([P1] macro `state_replay!`, and the
 * module documentation's description of `state_replay`).
 *
 * For every (b, hv, dv), starting from the snapshot row, for t = 0 .. T_log-1:
 *     take the step iff t < accepted and the mask passes;
 *     if taken:  S[dv, :] <- S[dv, :] * g_log_t + k_log_t[:] * delta_log_t[dv]
 *     else:      S unchanged
 * The page writes this as a select between the new and the old value, so an
 * untaken step contributes nothing whatever its tape slot holds; reading only
 * taken slots is the same function.  An `accepted` beyond T_log has no further
 * effect.
 *
 * Returns 0, or -1 when a dimension is zero.
 */
int oracle_gdn_replay(const double* delta_log, const double* k_log, const double* g_log,
                      const double* state_in, const uint32_t* mask, double* state_out,
                      uint32_t B, uint32_t T_log, uint32_t Hv, uint32_t Dk, uint32_t Dv,
                      uint32_t accepted)
{
    if (B == 0 || T_log == 0 || Hv == 0 || Dk == 0 || Dv == 0) return -1;

    for (uint32_t b = 0; b < B; ++b) {
        for (uint32_t hv = 0; hv < Hv; ++hv) {
            for (uint32_t dv = 0; dv < Dv; ++dv) {
                size_t row = (((size_t)b * Hv + hv) * Dv + dv) * Dk;
                double* S = state_out + row;
                if (S != state_in + row)
                    for (uint32_t i = 0; i < Dk; ++i) S[i] = state_in[row + i];

                for (uint32_t t = 0; t < T_log; ++t) {
                    int take = (t < accepted) && oracle_step_active(mask, T_log, b, t);
                    if (!take) continue;
                    size_t bt = (size_t)b * T_log + t;
                    double gt = g_log[bt * Hv + hv];
                    double d = delta_log[(bt * Hv + hv) * Dv + dv];
                    const double* kt = k_log + (bt * Hv + hv) * Dk;
                    for (uint32_t i = 0; i < Dk; ++i)
                        S[i] = S[i] * gt + kt[i] * d;
                }
            }
        }
    }
    return 0;
}

/*
 * GQA head broadcast [seq, hg, k] -> [seq, h, k] ([P3] "Mapping":
 * dst[t, h, k] = src[t, h % Hg, k] for the tiled map; the block map sends
 * destination head h to source head h / (h_total / hg), as in [P1]).
 * A pure copy of elem_bytes-wide elements; no arithmetic on the values.
 *
 * Returns 0, or -1 for a zero dimension, hg not dividing h, or a bad map.
 */
int oracle_gqa_expand(const void* src, void* dst, uint32_t seq, uint32_t hg, uint32_t h,
                      uint32_t k, uint32_t elem_bytes, int gqa_map)
{
    if (seq == 0 || hg == 0 || h == 0 || k == 0 || elem_bytes == 0) return -1;
    if (h % hg != 0) return -1;
    if (gqa_map != ORACLE_GQA_BLOCK && gqa_map != ORACLE_GQA_TILED) return -1;

    const unsigned char* s = (const unsigned char*)src;
    unsigned char* d = (unsigned char*)dst;
    for (uint32_t t = 0; t < seq; ++t) {
        for (uint32_t hh = 0; hh < h; ++hh) {
            uint32_t from = oracle_key_head(hh, hg, h, gqa_map);
            for (uint32_t e = 0; e < k; ++e) {
                size_t so = (((size_t)t * hg + from) * k + e) * elem_bytes;
                size_t dO = (((size_t)t * h + hh) * k + e) * elem_bytes;
                for (uint32_t c = 0; c < elem_bytes; ++c) d[dO + c] = s[so + c];
            }
        }
    }
    return 0;
}

/*
 * oracle_rms_norm_bf16 -- [P2] "GPU RMSNorm": for every token t of an
 * [n, dim] float32 input,
 *     r = 1 / sqrt( (sum_i x[t,i]^2) / dim + eps )
 *     out[t,i] = x[t,i] * r * w[i]
 * where w[i] is the bf16 weight widened exactly (its 16 bits are the upper
 * half of a float32).  The sum runs over i in order, in double.
 *
 * Returns 0, or -1 for a zero dimension.
 */
int oracle_rms_norm_bf16(const float* x, const uint16_t* w, double* out, uint32_t n,
                         uint32_t dim, double eps)
{
    if (n == 0 || dim == 0) return -1;
    for (uint32_t t = 0; t < n; ++t) {
        const float* xt = x + (size_t)t * dim;
        double ss = 0.0;
        for (uint32_t i = 0; i < dim; ++i) ss = ss + (double)xt[i] * (double)xt[i];
        double r = 1.0 / sqrt(ss / (double)dim + eps);
        for (uint32_t i = 0; i < dim; ++i) {
            uint32_t bits = (uint32_t)w[i] << 16;
            float wf;
            memcpy(&wf, &bits, sizeof wf);
            out[(size_t)t * dim + i] = (double)xt[i] * r * (double)wf;
        }
    }
    return 0;
}
