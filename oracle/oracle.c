/*
 * CPU oracle of the MoE expert combine -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library. It is a plain, slow, obviously correct statement of what
 * the combine computes, written from the documentation pages:
 *
 *   [A] flashinfer.comm.moe_a2a_combine  (FlashInfer API reference)
 *   [B] Struct_ep_combine_skip_a2a        (MAX Mojo API reference, execute)
 *   [C] flashinfer.megamoe.nvfp4_mega_moe (FlashInfer API reference)
 *   [D] flashinfer.comm.trtllm_moe_allreduce_fusion (FlashInfer API reference)
 *
 * It shares no code with the GPU library and includes none of its headers.
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fused
 * multiply-add is formed implicitly; every fma below is an explicit fmaf).
 *
 * Definition (one token t, one hidden index h):
 *   acc = +0.0f
 *   for j = 0 .. top_k-1 in ascending order:            [B] execute summary,
 *       (r, row) = src_info[t, j]; skip if r < 0          [B] Args src_info,
 *       w = router_weights ? router_weights[t, j] : 1    [C] Parameters
 *       acc = fmaf(w, float(payload[r, row, h]), acc)        num_tokens ("-1")
 *   if shared: acc = acc + float(shared[t, h])           [B] Parameters
 *                                                            fused_shared_expert
 *   epilogue: bf16 store [A] output_dtype / [B] output_tokens, or
 *             residual add + RMSNorm [D] Parameters, or
 *             MXFP8 e4m3 + UE8M0 per 32 [A] output_dtype, output_scales.
 *
 * Precision: the routed sum is accumulated in fp32 in fixed slot order (the
 * workload fixes fp32 accumulation); the RMSNorm statistic and scaling are
 * done in double; every output rounding is round-to-nearest-even.
 * Every function returns 0 on success, 1 on an out-of-range slot when
 * `checked` is set, 2 on a bad argument.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- scalar conversions ------------------------------------------------ */

/* bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits. */
static float bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* fp32 -> bf16, round to nearest, ties to even. NaN becomes the quiet NaN
 * 0x7FC0 with the input's sign; overflow rounds to infinity as RNE does.
 * ([A] Parameters output_dtype: bf16 output.) */
uint16_t oracle_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if (isnan(f))
        return (uint16_t)(((u >> 16) & 0x8000u) | 0x7FC0u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/* Shared exponent of one 32-element MX block from its largest magnitude:
 * floor(log2(amax)) - 8, where 8 is the exponent of e4m3's largest normal
 * (448 = 1.75 * 2^8), clamped to the UE8M0 range [-127, 127]; amax == 0 gives
 * -127. Returns 128 for a NaN or infinite amax (the UE8M0 NaN byte 0xFF).
 * ([A] Parameters output_scales: UE8M0, vector size 32.) */
int oracle_mx_exponent(float amax)
{
    if (isnan(amax) || isinf(amax))
        return 128;
    if (amax == 0.0f)
        return -127;
    int ex;
    (void)frexp((double)amax, &ex);      /* amax = m * 2^ex, m in [0.5, 1) */
    int e = (ex - 1) - 8;                /* floor(log2 amax) - 8 */
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* fp32 -> float8 e4m3fn (bias 7, no infinities, 0x7F/0xFF = NaN, largest
 * finite 448), round to nearest even on the e4m3 grid, saturating: any
 * magnitude >= 448 (infinity included) becomes +-448. Zero keeps its sign.
 * ([A] Parameters output_dtype: float8_e4m3fn.) */
uint8_t oracle_e4m3_rne_sat(float q)
{
    uint32_t u;
    memcpy(&u, &q, sizeof u);
    uint8_t s = (uint8_t)((u >> 24) & 0x80u);
    if (isnan(q))
        return (uint8_t)(s | 0x7F);
    double a = fabs((double)q);
    if (a >= 448.0)
        return (uint8_t)(s | 0x7E);
    if (a < 0x1p-6) {
        /* subnormal range: grid step 2^-9; n = 8 is the smallest normal */
        double n = rint(a * 512.0);             /* ties to even */
        return (uint8_t)(s | (uint8_t)n);
    }
    int ex;
    (void)frexp(a, &ex);
    int E = ex - 1;                              /* floor(log2 a), -6..8 */
    double n = rint(ldexp(a, 3 - E));            /* 8..16, ties to even */
    int code = ((E + 7) << 3) + (int)n - 8;      /* n == 16 carries into E+1 */
    return (uint8_t)(s | (uint8_t)code);
}

/* Shared exponent of one 32-element MXFP4 block: floor(log2(amax)) - 2,
 * where 2 is the exponent of e2m1's largest value (6 = 1.5 * 2^2), clamped to
 * [-127, 127]; amax == 0 gives -127; NaN/inf amax gives 128 (byte 0xFF). */
int oracle_mx4_exponent(float amax)
{
    if (isnan(amax) || isinf(amax))
        return 128;
    if (amax == 0.0f)
        return -127;
    int ex;
    (void)frexp((double)amax, &ex);
    int e = (ex - 1) - 2;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* fp32 -> float4 e2m1 code (4 bits: sign, 2 exponent bits with bias 1, 1
 * mantissa bit; values 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinity or NaN):
 * round to nearest even on that grid, saturating at 6. e2m1 has no NaN, so
 * NaN and infinity both saturate (a block holding them has the NaN scale). */
uint8_t oracle_e2m1_rne_sat(float q)
{
    uint32_t u;
    memcpy(&u, &q, sizeof u);
    uint8_t s = (uint8_t)((u >> 28) & 0x8u);
    if (isnan(q))
        return (uint8_t)(s | 0x7);
    double a = fabs((double)q);
    if (a >= 6.0)
        return (uint8_t)(s | 0x7);
    if (a < 1.0)                      /* subnormal step 0.5: codes 0, 1, 2 */
        return (uint8_t)(s | (uint8_t)rint(a * 2.0));
    int ex;
    (void)frexp(a, &ex);
    int E = ex - 1;                   /* 0, 1 or 2 */
    double n = rint(ldexp(a, 1 - E)); /* 2..4, ties to even */
    int code = ((E + 1) << 1) + (int)n - 2;
    return (uint8_t)(s | (uint8_t)code);
}

/* ---- the routed sum ----------------------------------------------------- */

static int check_dims(int64_t T, int64_t H, int k, int ep, int64_t mtpr)
{
    return T < 0 || H <= 0 || k < 1 || ep < 1 || mtpr < 1;
}

static int check_slots(const int32_t *src, int64_t T, int k, int ep, int64_t mtpr)
{
    for (int64_t i = 0; i < T * k; ++i) {
        int32_t r = src[2 * i], row = src[2 * i + 1];
        if (r < 0)
            continue;
        if (r >= ep || row < 0 || row >= mtpr)
            return 1;
    }
    return 0;
}

/* fp32 value of output element (t, h) before the epilogue. */
static float routed_sum(const uint16_t *payload, const int32_t *src,
                        const float *w, const uint16_t *shared, int64_t t,
                        int64_t h, int64_t H, int k, int64_t mtpr)
{
    float acc = 0.0f;
    for (int j = 0; j < k; ++j) {
        int32_t r = src[(t * k + j) * 2 + 0];
        int32_t row = src[(t * k + j) * 2 + 1];
        if (r < 0)
            continue;                            /* dropped slot: no term */
        float wj = w ? w[t * k + j] : 1.0f;
        float x = bf16_to_float(payload[((int64_t)r * mtpr + row) * H + h]);
        acc = fmaf(wj, x, acc);
    }
    if (shared)
        acc = acc + bf16_to_float(shared[t * H + h]);
    return acc;
}

/* acc_out[t, h] = fp32 routed sum (+ shared), for pins and tests. */
int oracle_routed_sum_f32(const uint16_t *payload, const int32_t *src_info,
                          const float *weights, const uint16_t *shared,
                          float *acc_out, int64_t T, int64_t H, int k, int ep,
                          int64_t mtpr, int checked)
{
    if (check_dims(T, H, k, ep, mtpr)) return 2;
    if (checked && check_slots(src_info, T, k, ep, mtpr)) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t h = 0; h < H; ++h)
            acc_out[t * H + h] = routed_sum(payload, src_info, weights, shared,
                                            t, h, H, k, mtpr);
    return 0;
}

/* bf16 combine: out[t, h] = bf16_rne(acc). Rows >= T of out are untouched
 * ([C] Parameters y: the first num_tokens rows are written). */
int oracle_combine(const uint16_t *payload, const int32_t *src_info,
                   const float *weights, const uint16_t *shared, uint16_t *out,
                   int64_t T, int64_t H, int k, int ep, int64_t mtpr, int checked)
{
    if (check_dims(T, H, k, ep, mtpr)) return 2;
    if (checked && check_slots(src_info, T, k, ep, mtpr)) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t h = 0; h < H; ++h)
            out[t * H + h] = oracle_bf16_rne(routed_sum(
                payload, src_info, weights, shared, t, h, H, k, mtpr));
    return 0;
}

/* Combine + residual add + RMSNorm ([D] Parameters residual_in, rms_gamma,
 * rms_eps, residual_out, norm_out, weight_bias):
 *   s            = acc + float(residual_in)                     (fp32)
 *   residual_out = bf16_rne(s)
 *   rstd         = 1 / sqrt(mean_h residual_out^2 + eps)        (double)
 *   norm_out     = bf16_rne(residual_out * rstd * (gamma + weight_bias))
 * weight_bias 0 is the standard RMSNorm, 1 the (1 + gamma) form. */
int oracle_combine_residual_rmsnorm(
    const uint16_t *payload, const int32_t *src_info, const float *weights,
    const uint16_t *shared, const uint16_t *residual_in, const uint16_t *gamma,
    float eps, float weight_bias, uint16_t *residual_out, uint16_t *norm_out,
    int64_t T, int64_t H, int k, int ep, int64_t mtpr, int checked)
{
    if (check_dims(T, H, k, ep, mtpr)) return 2;
    if (checked && check_slots(src_info, T, k, ep, mtpr)) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double ss = 0.0;
        for (int64_t h = 0; h < H; ++h) {
            float acc = routed_sum(payload, src_info, weights, shared, t, h, H,
                                   k, mtpr);
            float s = acc + bf16_to_float(residual_in[t * H + h]);
            uint16_t ro = oracle_bf16_rne(s);
            residual_out[t * H + h] = ro;
            double x = (double)bf16_to_float(ro);
            ss += x * x;
        }
        double rstd = 1.0 / sqrt(ss / (double)H + (double)eps);
        for (int64_t h = 0; h < H; ++h) {
            double x = (double)bf16_to_float(residual_out[t * H + h]);
            float g = bf16_to_float(gamma[h]) + weight_bias;
            norm_out[t * H + h] = oracle_bf16_rne((float)(x * rstd * (double)g));
        }
    }
    return 0;
}

/* Combine with MXFP8 output ([A] Parameters output_dtype float8_e4m3fn,
 * output_scales UE8M0 with vector size 32, sf_layout linear): for each block
 * of 32 consecutive hidden elements of a token, e = oracle_mx_exponent(amax
 * of the fp32 sums), scale byte = e + 127, code = e4m3_rne_sat(acc * 2^-e).
 * Scales are row-major [T, H/32]. A block with a NaN or infinite element
 * gets the NaN scale byte 0xFF and its codes are taken with e = 0. */
int oracle_combine_mxfp8(const uint16_t *payload, const int32_t *src_info,
                         const float *weights, const uint16_t *shared,
                         uint8_t *out_fp8, uint8_t *out_scales, int64_t T,
                         int64_t H, int k, int ep, int64_t mtpr, int checked)
{
    if (check_dims(T, H, k, ep, mtpr) || H % 32) return 2;
    if (checked && check_slots(src_info, T, k, ep, mtpr)) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t b = 0; b < H / 32; ++b) {
            float acc[32];
            float amax = 0.0f;
            int nonfinite = 0;
            for (int i = 0; i < 32; ++i) {
                acc[i] = routed_sum(payload, src_info, weights, shared, t,
                                    b * 32 + i, H, k, mtpr);
                if (!isfinite(acc[i]))
                    nonfinite = 1;
                else if (fabsf(acc[i]) > amax)
                    amax = fabsf(acc[i]);
            }
            int e = nonfinite ? 128 : oracle_mx_exponent(amax);
            out_scales[t * (H / 32) + b] = (uint8_t)(e + 127);
            if (e == 128)
                e = 0;
            for (int i = 0; i < 32; ++i)
                out_fp8[t * H + b * 32 + i] =
                    oracle_e4m3_rne_sat(ldexpf(acc[i], -e));
        }
    }
    return 0;
}

/* Combine + residual add + RMSNorm, with the normalised row quantised to
 * MXFP8. This composes the two epilogues above: the RMSNorm of
 * flashinfer.comm.trtllm_moe_allreduce_fusion (Parameters residual_out,
 * norm_out, weight_bias; its quant_out is a quantised copy of the normalised
 * output) with the MXFP8 format of flashinfer.comm.moe_a2a_combine
 * (Parameters output_dtype, output_scales).
 *   residual_out = bf16_rne(acc + residual_in)                      (as above)
 *   n_h          = (float)(residual_out_h * rstd * (gamma_h + weight_bias))
 *   norm_out_h   = bf16_rne(n_h)               (written only if norm_out)
 *   per block of 32 of n: e = oracle_mx_exponent(amax), scale = e + 127,
 *   code = e4m3_rne_sat(n_h * 2^-e)            (NaN/inf blocks as above).
 * The quantiser reads the fp32 values n_h, not their bf16 rounding. */
int oracle_combine_residual_rmsnorm_mxfp8(
    const uint16_t *payload, const int32_t *src_info, const float *weights,
    const uint16_t *shared, const uint16_t *residual_in, const uint16_t *gamma,
    float eps, float weight_bias, uint16_t *residual_out, uint16_t *norm_out,
    uint8_t *out_fp8, uint8_t *out_scales, int64_t T, int64_t H, int k, int ep,
    int64_t mtpr, int checked)
{
    if (check_dims(T, H, k, ep, mtpr) || H % 32) return 2;
    if (checked && check_slots(src_info, T, k, ep, mtpr)) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double ss = 0.0;
        for (int64_t h = 0; h < H; ++h) {
            float acc = routed_sum(payload, src_info, weights, shared, t, h, H,
                                   k, mtpr);
            float s = acc + bf16_to_float(residual_in[t * H + h]);
            uint16_t ro = oracle_bf16_rne(s);
            residual_out[t * H + h] = ro;
            double x = (double)bf16_to_float(ro);
            ss += x * x;
        }
        double rstd = 1.0 / sqrt(ss / (double)H + (double)eps);
        for (int64_t b = 0; b < H / 32; ++b) {
            float n[32];
            float amax = 0.0f;
            int nonfinite = 0;
            for (int i = 0; i < 32; ++i) {
                int64_t h = b * 32 + i;
                double x = (double)bf16_to_float(residual_out[t * H + h]);
                float g = bf16_to_float(gamma[h]) + weight_bias;
                n[i] = (float)(x * rstd * (double)g);
                if (norm_out)
                    norm_out[t * H + h] = oracle_bf16_rne(n[i]);
                if (!isfinite(n[i]))
                    nonfinite = 1;
                else if (fabsf(n[i]) > amax)
                    amax = fabsf(n[i]);
            }
            int e = nonfinite ? 128 : oracle_mx_exponent(amax);
            out_scales[t * (H / 32) + b] = (uint8_t)(e + 127);
            if (e == 128)
                e = 0;
            for (int i = 0; i < 32; ++i)
                out_fp8[t * H + b * 32 + i] = oracle_e4m3_rne_sat(ldexpf(n[i], -e));
        }
    }
    return 0;
}

/* Combine with an MXFP4 output (flashinfer.comm.moe_a2a_combine, Parameters
 * output_scales: UE8M0 scales with vector size 32; output_scalar_scale: the
 * per-tensor scale is ignored by the MXFP4 path). For each block of 32 fp32
 * sums, e = oracle_mx4_exponent(amax), scale byte = e + 127, code =
 * e2m1_rne_sat(acc * 2^-e); two codes per byte, element 2i in the low nibble.
 * out_fp4 is [T, H/2] bytes, scales [T, H/32] row-major. A block with a NaN or
 * infinite element gets scale 0xFF and its codes are taken with e = 0. */
int oracle_combine_mxfp4(const uint16_t *payload, const int32_t *src_info,
                         const float *weights, const uint16_t *shared,
                         uint8_t *out_fp4, uint8_t *out_scales, int64_t T,
                         int64_t H, int k, int ep, int64_t mtpr, int checked)
{
    if (check_dims(T, H, k, ep, mtpr) || H % 32) return 2;
    if (checked && check_slots(src_info, T, k, ep, mtpr)) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t b = 0; b < H / 32; ++b) {
            float acc[32];
            float amax = 0.0f;
            int nonfinite = 0;
            for (int i = 0; i < 32; ++i) {
                acc[i] = routed_sum(payload, src_info, weights, shared, t,
                                    b * 32 + i, H, k, mtpr);
                if (!isfinite(acc[i]))
                    nonfinite = 1;
                else if (fabsf(acc[i]) > amax)
                    amax = fabsf(acc[i]);
            }
            int e = nonfinite ? 128 : oracle_mx4_exponent(amax);
            out_scales[t * (H / 32) + b] = (uint8_t)(e + 127);
            if (e == 128)
                e = 0;
            for (int i = 0; i < 32; i += 2) {
                uint8_t lo = oracle_e2m1_rne_sat(ldexpf(acc[i], -e));
                uint8_t hi = oracle_e2m1_rne_sat(ldexpf(acc[i + 1], -e));
                out_fp4[t * (H / 2) + (b * 32 + i) / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
    return 0;
}

/* Dense MoE reduction: inputs are expert-major rows [n_in, T, H] (one row per
 * (input, token); for the local reduce that replaces the all-to-all, the
 * inputs are the n_in partial sums of the ranks), per-(token, input) fp32
 * scales or none, and an optional token input added unweighted:
 *   out[t, h] = bf16_rne( (sum over i ascending of s[t, i] * x[i, t, h]) + tok[t, h] )
 * with one fp32 fused multiply-add per input from +0, then one fp32 add.
 * Sources: flashinfer.comm.trtllm_moe_allreduce_fusion, Parameters
 * moe_reduction_scale_input, moe_reduction_active_experts_token_input and
 * moe_reduction_token_input; Struct_ep_combine_skip_a2a, Parameters
 * skip_a2a and allreduce_world_size (reduce locally instead of exchanging).
 * The residual + RMSNorm epilogue, if residual_in is given, is the one of
 * oracle_combine_residual_rmsnorm (out is then residual_out). */
int oracle_reduce_dense(const uint16_t *x, int n_in, const float *scales,
                        const uint16_t *tok, const uint16_t *residual_in,
                        const uint16_t *gamma, float eps, float weight_bias,
                        uint16_t *out, uint16_t *norm_out, int64_t T, int64_t H)
{
    if (T < 0 || H <= 0 || n_in < 1) return 2;
    if (residual_in && (!gamma || !norm_out)) return 2;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double ss = 0.0;
        for (int64_t h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int i = 0; i < n_in; ++i) {
                float s = scales ? scales[t * n_in + i] : 1.0f;
                acc = fmaf(s, bf16_to_float(x[((int64_t)i * T + t) * H + h]), acc);
            }
            if (tok)
                acc = acc + bf16_to_float(tok[t * H + h]);
            if (residual_in)
                acc = acc + bf16_to_float(residual_in[t * H + h]);
            uint16_t o = oracle_bf16_rne(acc);
            out[t * H + h] = o;
            double v = (double)bf16_to_float(o);
            ss += v * v;
        }
        if (!residual_in)
            continue;
        double rstd = 1.0 / sqrt(ss / (double)H + (double)eps);
        for (int64_t h = 0; h < H; ++h) {
            double v = (double)bf16_to_float(out[t * H + h]);
            float g = bf16_to_float(gamma[h]) + weight_bias;
            norm_out[t * H + h] = oracle_bf16_rne((float)(v * rstd * (double)g));
        }
    }
    return 0;
}

/* Dispatch: the forward scatter the combine inverts
 * (flashinfer.comm.moe_a2a_combine summary: the combine is the inverse of
 * moe_a2a_dispatch; flashinfer.megamoe.nvfp4_mega_moe, Parameters num_tokens:
 * slots routed to -1 carry nothing, and cumulative_local_expert_recv_stats:
 * per-expert receive counts accumulated in place).
 * Pairs (t, j) with topk_ids[t, j] >= 0 are taken expert by expert in
 * ascending expert id, and within an expert in token-major, slot-minor order;
 * expert e lives on rank e / (E / ep); the next free row of that rank is
 * assigned. A row at or past mtpr drops the pair. For a placed pair:
 *   src_info[t, j] = (rank, row), payload[rank, row, :] = x[t, :],
 *   recv_counts[e] += 1 (if recv_counts is given);
 * dropped pairs get (-1, -1). Unassigned payload rows are left untouched. */
int oracle_dispatch(const uint16_t *x, const int32_t *topk_ids, int64_t T,
                    int64_t H, int k, int E, int ep, int64_t mtpr,
                    uint16_t *payload, int32_t *src_info, int32_t *recv_counts)
{
    if (T < 0 || H <= 0 || k < 1 || E < 1 || ep < 1 || E % ep || mtpr < 1)
        return 2;
    for (int64_t i = 0; i < T * k; ++i)
        if (topk_ids[i] >= E || topk_ids[i] < -1)
            return 1;
    int64_t *next_row = calloc((size_t)ep, sizeof(int64_t));
    if (!next_row)
        return 2;
    for (int64_t i = 0; i < T * k; ++i)
        src_info[2 * i] = src_info[2 * i + 1] = -1;
    int epr = E / ep;
    for (int e = 0; e < E; ++e) {
        int r = e / epr;
        for (int64_t i = 0; i < T * k; ++i) {       /* i = t * k + j */
            if (topk_ids[i] != e)
                continue;
            int64_t row = next_row[r]++;
            if (row >= mtpr)
                continue;                            /* over capacity */
            src_info[2 * i] = r;
            src_info[2 * i + 1] = (int32_t)row;
            memcpy(payload + ((int64_t)r * mtpr + row) * H, x + (i / k) * H,
                   (size_t)H * sizeof(uint16_t));
            if (recv_counts)
                recv_counts[e] += 1;
        }
    }
    free(next_row);
    return 0;
}

/* ---- threading ----------------------------------------------------------- */

void oracle_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int oracle_max_threads(void) { return omp_get_max_threads(); }
