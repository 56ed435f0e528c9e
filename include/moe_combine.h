/*
 * moe_combine.h -- C ABI of the MI355X (gfx950) MoE expert-combine library.
 *
 * The combine returns each token's routed expert outputs to it and reduces
 * them. For token t, hidden index h, and slots j = 0..top_k-1 in ascending
 * order:
 *
 *   (rank, row) = src_info[t, j]              -- kept only if 0 <= rank < ep_size
 *                                                and 0 <= row < max_tokens_per_rank
 *   acc  = +0.0f
 *   acc  = fmaf(w[t, j], payload[rank, row, h], acc)   for every kept slot
 *   acc += shared_out[t, h]                   -- only if shared_out != NULL
 *
 * The sum is accumulated in fp32 in that fixed order. It is followed by one
 * of five epilogues:
 *  - a bf16 store (moe_combine);
 *  - residual add plus RMSNorm (moe_combine_residual_rmsnorm);
 *  - MXFP8 quantisation (moe_combine_mxfp8);
 *  - residual add, RMSNorm and MXFP8 of the normalised row
 *    (moe_combine_residual_rmsnorm_mxfp8);
 *  - MXFP4 quantisation (moe_combine_mxfp4).
 *
 * Sources (documentation pages):
 *  - flashinfer.comm.moe_a2a_combine, Parameters: payload, output_dtype,
 *    output_scales, sf_layout, output; and Returns.
 *  - Struct_ep_combine_skip_a2a, execute: the summary, the Parameters
 *    fused_shared_expert and has_epilogue_fusion, and the Args
 *    output_tokens, src_info, router_weights and topk_ids.
 *  - flashinfer.megamoe.nvfp4_mega_moe, Parameters: y and num_tokens
 *    ("-1" rows contribute nothing); and Notes (contiguous tensors on one
 *    device).
 *  - flashinfer.comm.trtllm_moe_allreduce_fusion, Parameters: residual_in,
 *    rms_gamma, rms_eps, residual_out, norm_out and weight_bias.
 *
 * Conventions common to every entry point:
 *  - Pointers are device pointers to caller-owned, contiguous, row-major
 *    memory on the current HIP device. The library allocates nothing, keeps
 *    no state between calls, and never synchronises. Work is enqueued on
 *    `stream`, a hipStream_t; NULL means the default stream. Inputs must be
 *    unchanged, and outputs untouched, until that work completes.
 *  - bf16 tensors use 16-bit bfloat16 elements.
 *  - payload: [ep_size, max_tokens_per_rank, hidden] bf16. Per-expert-rank
 *    output rows are in dispatch order.
 *  - src_info: [num_tokens, top_k, 2] int32 = (rank, row) per (token, slot).
 *    A slot with rank < 0 is dropped: it reads nothing, and its weight is
 *    ignored (the other weights are not renormalised). The pages only
 *    require a kept slot to name a payload row; any slot outside the payload
 *    (rank >= ep_size, row < 0 or row >= max_tokens_per_rank) is dropped the
 *    same way. The kernels check both bounds before every row read, so no
 *    slot map can make them read outside the payload.
 *  - router_weights: [num_tokens, top_k] fp32, or NULL for unit weights.
 *  - shared_out: [num_tokens, hidden] bf16, or NULL. It is added unweighted,
 *    after the routed sum.
 *  - Outputs have at least num_tokens rows. Exactly the first num_tokens
 *    rows are written; rows past them are untouched. No byte of an output's
 *    first num_tokens rows may lie in an input or in another output (the
 *    payload counts with all its ep_size * max_tokens_per_rank rows), except
 *    where an entry point allows it; a call that breaks this is rejected.
 *  - hidden must be a positive multiple of 8 (16-byte rows), at most 2^28
 *    (output rows are addressed with 32-bit byte offsets). bf16 pointers
 *    must be 16-byte aligned, src_info 8-byte aligned, router_weights 4-byte
 *    aligned. 1 <= top_k <= 32, ep_size >= 1, max_tokens_per_rank >= 1, and
 *    num_tokens >= 0. num_tokens == 0 returns MOE_OK and launches nothing.
 *  - Rounding: every float -> bf16 conversion rounds to nearest, ties to even.
 *  - Errors: argument errors return MOE_ERR_INVALID_ARG before any HIP call.
 *    A failed launch returns MOE_ERR_HIP. moe_combine_last_error() describes
 *    the last failure on the calling thread.
 */
#ifndef MOE_COMBINE_H_
#define MOE_COMBINE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,
    MOE_ERR_UNSUPPORTED = 2,
    MOE_ERR_HIP = 3
} moe_status_t;

#define MOE_COMBINE_ABI_VERSION 2

/* Entry-point kinds, for moe_combine_check_args and
 * moe_combine_describe_launch. */
enum {
    MOE_KIND_COMBINE = 0,                        /* moe_combine */
    MOE_KIND_COMBINE_RESIDUAL_RMSNORM = 1,       /* moe_combine_residual_rmsnorm */
    MOE_KIND_COMBINE_MXFP8 = 2,                  /* moe_combine_mxfp8 */
    MOE_KIND_COMBINE_RESIDUAL_RMSNORM_MXFP8 = 3, /* moe_combine_residual_rmsnorm_mxfp8 */
    MOE_KIND_COMBINE_MXFP4 = 4,                  /* moe_combine_mxfp4 */
    MOE_KIND_DISPATCH = 5,                       /* moe_dispatch */
    MOE_KIND_REDUCE_DENSE = 6,                   /* moe_reduce_dense */
    MOE_KIND_REDUCE_DENSE_RESIDUAL_RMSNORM = 7   /* moe_reduce_dense_residual_rmsnorm */
};

/* The arguments of one entry-point call, by the entry point's parameter
 * names. A kind reads the fields its entry point takes and ignores the
 * rest (leave them zero). For MOE_KIND_DISPATCH, payload and src_info are
 * the call's outputs. */
typedef struct moe_call_args {
    int32_t kind;                   /* MOE_KIND_* */
    int32_t hidden;
    int64_t num_tokens;
    int32_t top_k;                  /* combine kinds, dispatch */
    int32_t ep_size;                /* combine kinds, dispatch */
    int64_t max_tokens_per_rank;    /* combine kinds, dispatch */
    int32_t n_in;                   /* local-reduce kinds */
    int32_t num_experts;            /* dispatch */
    float eps;                      /* RMSNorm kinds */
    float weight_bias;              /* RMSNorm kinds (any value is valid) */
    const void *payload;
    const int32_t *src_info;
    const float *router_weights;
    const void *shared_out;
    const void *inputs;             /* local-reduce kinds */
    const float *scales;            /* local-reduce kinds */
    const void *token_input;        /* local-reduce kinds */
    const void *residual_in;
    const void *gamma;
    const void *x;                  /* dispatch */
    const int32_t *topk_ids;        /* dispatch */
    void *out;                      /* moe_combine, moe_reduce_dense */
    void *residual_out;
    void *norm_out;
    void *out_fp8;
    void *out_fp4;
    uint8_t *out_scales;
    int32_t *recv_counts;           /* dispatch */
    void *workspace;                /* dispatch */
    size_t workspace_bytes;         /* dispatch */
} moe_call_args_t;

/*
 * Validates the arguments of one call without touching the GPU: pure host
 * code, no HIP call, no allocation. Every entry point runs exactly this
 * validation before its first HIP call, so MOE_OK here means the entry
 * point will not reject these arguments (a MOE_COMBINE_TILE override can
 * still make a launch shape unsupported). It checks:
 *  - sizes (the ranges stated with each entry point);
 *  - required pointers, for num_tokens > 0 (num_tokens == 0 needs none);
 *  - alignment;
 *  - byte ranges: every output's written range (first num_tokens rows) must
 *    not intersect an input's range or another output's, except
 *    residual_out == residual_in exactly.
 * Returns MOE_OK, MOE_ERR_INVALID_ARG, or MOE_ERR_UNSUPPORTED (an RMSNorm
 * row longer than 32768); moe_combine_last_error() names the argument.
 * Sources: flashinfer.comm.moe_a2a_combine, Parameters output (a contiguous
 * caller-provided output of matching shape and dtype on the same device);
 * flashinfer.megamoe.nvfp4_mega_moe, Parameters y (the first num_tokens
 * rows are written in place) and Notes (contiguous tensors on one device);
 * flashinfer.comm.trtllm_moe_allreduce_fusion, Parameters residual_out.
 */
moe_status_t moe_combine_check_args(const moe_call_args_t *args);

/* Version of this ABI (MOE_COMBINE_ABI_VERSION). */
int moe_combine_abi_version(void);

/* Static name of a status code. */
const char *moe_combine_status_string(int status);

/* Message for the last failing call on the calling thread. The string is
 * owned by the library and valid until this thread's next call. */
const char *moe_combine_last_error(void);

/*
 * Routed combine with a bf16 output.
 *   out[t, h] = bf16(acc)       out: [>= num_tokens, hidden] bf16
 * Sources: flashinfer.comm.moe_a2a_combine (summary; Parameters payload,
 * output_dtype = bf16, output), and Struct_ep_combine_skip_a2a, execute
 * (summary; Args output_tokens, src_info, router_weights; Parameter
 * fused_shared_expert).
 */
moe_status_t moe_combine(const void *payload, const int32_t *src_info,
                         const float *router_weights, const void *shared_out,
                         void *out, int64_t num_tokens, int32_t hidden,
                         int32_t top_k, int32_t ep_size,
                         int64_t max_tokens_per_rank, void *stream);

/*
 * Routed combine fused with a residual add and an RMSNorm.
 *   s                = acc + residual_in[t, h]                      (fp32)
 *   residual_out     = bf16(s)
 *   rstd             = 1 / sqrt(mean_h(residual_out^2) + eps)
 *   norm_out[t, h]   = bf16(residual_out * rstd * (gamma[h] + weight_bias))
 * rstd and the product are evaluated in fp64 and rounded once to fp32, then
 * to bf16. Rows of up to 32768 elements are supported (MOE_ERR_UNSUPPORTED
 * beyond).
 * weight_bias = 0 gives the standard RMSNorm; 1 gives the (1 + gamma) form.
 * residual_in, residual_out and norm_out are [>= num_tokens, hidden] bf16;
 * gamma is [hidden] bf16. residual_out may equal residual_in (in-place
 * update). norm_out must differ from both of them.
 * Source: flashinfer.comm.trtllm_moe_allreduce_fusion, Parameters
 * residual_in, rms_gamma, rms_eps, residual_out, norm_out, weight_bias.
 */
moe_status_t moe_combine_residual_rmsnorm(
    const void *payload, const int32_t *src_info, const float *router_weights,
    const void *shared_out, const void *residual_in, const void *gamma,
    float eps, float weight_bias, void *residual_out, void *norm_out,
    int64_t num_tokens, int32_t hidden, int32_t top_k, int32_t ep_size,
    int64_t max_tokens_per_rank, void *stream);

/*
 * Routed combine with an MXFP8 output: float8 e4m3fn codes plus one UE8M0
 * scale byte per 32 consecutive elements of a row.
 *
 * For each block of 32 sums, amax is their largest magnitude. Then:
 *   e     = clamp(floor(log2(amax)) - 8, -127, 127), with e = -127 if amax == 0
 *   scale = e + 127                       (0xFF if the block holds NaN or inf)
 *   code  = e4m3(acc * 2^-e), rounded to nearest even and saturated to +-448
 *
 * A NaN or inf block has its codes taken with e = 0: NaN encodes as 0x7F or
 * 0xFF, and inf saturates. Here 8 is the exponent of e4m3's largest finite
 * value, 448 = 1.75 * 2^8.
 *
 * out_fp8 is [>= num_tokens, hidden] e4m3fn (8-byte aligned). out_scales is
 * [>= num_tokens, hidden / 32] uint8, linear row-major. hidden must be a
 * multiple of 32.
 *
 * Source: flashinfer.comm.moe_a2a_combine, Parameters output_dtype
 * (float8_e4m3fn), output_scales (UE8M0, vector size 32) and sf_layout
 * (linear).
 */
moe_status_t moe_combine_mxfp8(const void *payload, const int32_t *src_info,
                               const float *router_weights,
                               const void *shared_out, void *out_fp8,
                               uint8_t *out_scales, int64_t num_tokens,
                               int32_t hidden, int32_t top_k, int32_t ep_size,
                               int64_t max_tokens_per_rank, void *stream);

/*
 * Routed combine fused with a residual add, an RMSNorm, and MXFP8
 * quantisation of the normalised row (the quantised copy that feeds the next
 * layer's fp8 GEMM).
 *   residual_out  = bf16(acc + residual_in)                  as above
 *   n[t, h]       = residual_out * rstd * (gamma[h] + weight_bias)
 *   norm_out      = bf16(n)          written only if norm_out != NULL
 *   out_fp8, out_scales = MXFP8 of n, per the rule of moe_combine_mxfp8
 * The quantiser reads n as fp32, not its bf16 rounding. The RMSNorm
 * statistic and n are evaluated in fp64 and rounded once to fp32.
 * residual_out may equal residual_in. No other pair of arguments may
 * overlap. hidden must be a multiple of 32.
 * Sources: flashinfer.comm.trtllm_moe_allreduce_fusion, Parameters
 * residual_out, norm_out, weight_bias and quant_out / scale_out (a quantised
 * copy of the normalised output); flashinfer.comm.moe_a2a_combine,
 * Parameters output_dtype (float8_e4m3fn) and output_scales (UE8M0, 32).
 */
moe_status_t moe_combine_residual_rmsnorm_mxfp8(
    const void *payload, const int32_t *src_info, const float *router_weights,
    const void *shared_out, const void *residual_in, const void *gamma,
    float eps, float weight_bias, void *residual_out, void *norm_out,
    void *out_fp8, uint8_t *out_scales, int64_t num_tokens, int32_t hidden,
    int32_t top_k, int32_t ep_size, int64_t max_tokens_per_rank, void *stream);

/*
 * Routed combine with an MXFP4 output: float4 e2m1 codes (two per byte)
 * plus one UE8M0 scale byte per 32 consecutive elements.
 *
 * e2m1 has a sign, 2 exponent bits (bias 1) and 1 mantissa bit, with
 * magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6, and no inf or NaN. For each block
 * of 32 sums:
 *   e     = clamp(floor(log2(amax)) - 2, -127, 127), e = -127 if amax == 0
 *   scale = e + 127                     (0xFF if the block holds NaN or inf)
 *   code  = e2m1(acc * 2^-e), rounded to nearest even, saturated at +-6
 * Here 2 is the exponent of e2m1's largest value, 6 = 1.5 * 2^2. A NaN or
 * inf block has its codes taken with e = 0, and NaN and inf saturate.
 *
 * Layout: out_fp4 is [>= num_tokens, hidden / 2] bytes (4-byte aligned).
 * Element 2i of a row sits in the low nibble of byte i and element 2i+1 in
 * the high nibble. out_scales is [>= num_tokens, hidden / 32] uint8,
 * row-major. hidden must be a multiple of 32.
 *
 * Source: flashinfer.comm.moe_a2a_combine, Parameters output_scales (UE8M0,
 * vector size 32) and output_scalar_scale (ignored by the MXFP4 path).
 */
moe_status_t moe_combine_mxfp4(const void *payload, const int32_t *src_info,
                               const float *router_weights,
                               const void *shared_out, void *out_fp4,
                               uint8_t *out_scales, int64_t num_tokens,
                               int32_t hidden, int32_t top_k, int32_t ep_size,
                               int64_t max_tokens_per_rank, void *stream);

/*
 * Dense MoE reduction: the local reduce of the expert-parallel combine. It
 * replaces the all-to-all exchange when skip_a2a is set, and it is the MoE
 * reduction in front of the all-reduce of the allreduce-fusion kernel.
 *
 * inputs is [n_in, num_tokens, hidden] bf16, expert-major: row t of input i
 * is expert i's (or rank i's partial) output for token t. scales is
 * [num_tokens, n_in] fp32, or NULL for unit scales, which gives the plain
 * sum of n_in partial buffers. token_input is [num_tokens, hidden] bf16, or
 * NULL.
 *   acc = +0;  acc = fmaf(scales[t, i], inputs[i, t, h], acc) for i ascending
 *   acc += token_input[t, h];  out[t, h] = bf16(acc)
 * This is moe_combine with the slot map (rank, row) = (i, t). Arguments
 * follow that entry point's rules, with 1 <= n_in <= 32.
 *
 * Sources: Struct_ep_combine_skip_a2a, Parameters skip_a2a and
 * allreduce_world_size; flashinfer.comm.trtllm_moe_allreduce_fusion,
 * Parameters moe_reduction_scale_input,
 * moe_reduction_active_experts_token_input and moe_reduction_token_input.
 */
moe_status_t moe_reduce_dense(const void *inputs, int32_t n_in,
                              const float *scales, const void *token_input,
                              void *out, int64_t num_tokens, int32_t hidden,
                              void *stream);

/*
 * moe_reduce_dense followed by the residual add and RMSNorm of
 * moe_combine_residual_rmsnorm: the single-GPU body of the MoE reduction
 * + residual + RMSNorm fusion (the all-reduce between them has one
 * participant here). Outputs and aliasing follow
 * moe_combine_residual_rmsnorm.
 * Source: flashinfer.comm.trtllm_moe_allreduce_fusion, Parameters
 * residual_in, rms_gamma, rms_eps, residual_out, norm_out, weight_bias.
 */
moe_status_t moe_reduce_dense_residual_rmsnorm(
    const void *inputs, int32_t n_in, const float *scales,
    const void *token_input, const void *residual_in, const void *gamma,
    float eps, float weight_bias, void *residual_out, void *norm_out,
    int64_t num_tokens, int32_t hidden, void *stream);

/*
 * Dispatch: the forward scatter the combine inverts. It builds the payload
 * and slot map that moe_combine consumes.
 *
 * Inputs:
 *  - x: [num_tokens, hidden] bf16;
 *  - topk_ids: [num_tokens, top_k] int32 expert ids in [0, num_experts).
 *    -1 marks a dropped slot, and ids outside the range are treated as -1.
 *  - ep_size: number of ranks. Expert e lives on rank e / (num_experts /
 *    ep_size), so ep_size must divide num_experts (<= 4096).
 *
 * Placement: kept (token, slot) pairs are enumerated token-major and stably
 * sorted by expert id. A pair's row is its position among its rank's pairs
 * in that order. A row at or past max_tokens_per_rank drops the pair.
 *
 * For each placed pair, it writes:
 *  - src_info[t, j] = (rank, row);
 *  - payload[rank, row, :] = x[t, :];
 *  - recv_counts[e] += 1 (counts accumulate in place; NULL skips them).
 * Dropped pairs get (-1, -1). payload rows no pair is placed in are left
 * untouched.
 *
 * workspace: caller-provided device memory of at least
 * moe_dispatch_workspace_size(num_tokens, top_k, num_experts, ep_size,
 * max_tokens_per_rank) bytes (4-byte aligned). Its contents on entry do not
 * matter, and are overwritten. Calls that share a workspace must not
 * overlap.
 *
 * Launches: up to 65536 pairs (num_tokens * top_k), one placement kernel
 * and the row scatter; above, a count kernel, a scan kernel and the row
 * scatter (the workspace holds their intermediate counts). Tuning
 * overrides, read at each call: MOE_DISPATCH_PATH=place or count_scan
 * takes that path at any size (both are exact at every size), and
 * MOE_DISPATCH_TILE="<threads>x<vectors>" sets the scatter's workgroup size
 * (a multiple of 64, at most 1024) and 16-byte vectors per thread (1, 2, 4
 * or 8). Invalid values are ignored.
 *
 * Sources: flashinfer.comm.moe_a2a_combine (summary: the combine is the
 * inverse of moe_a2a_dispatch); flashinfer.megamoe.nvfp4_mega_moe,
 * Parameters num_tokens (rows routed to -1) and
 * cumulative_local_expert_recv_stats (receive counts accumulated in place);
 * Struct_ep_combine_skip_a2a, Args recv_count_ptrs and topk_ids.
 */
size_t moe_dispatch_workspace_size(int64_t num_tokens, int32_t top_k,
                                   int32_t num_experts, int32_t ep_size,
                                   int64_t max_tokens_per_rank);

moe_status_t moe_dispatch(const void *x, const int32_t *topk_ids,
                          int64_t num_tokens, int32_t hidden, int32_t top_k,
                          int32_t num_experts, int32_t ep_size,
                          int64_t max_tokens_per_rank, void *payload,
                          int32_t *src_info, int32_t *recv_counts,
                          void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * moe_dispatch without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * and harnesses that forbid allocation. The call allocates nothing. Its
 * count + scan path keeps its per-chunk expert offsets and per-pair ranks in
 * the library's own device scratch array of 8 MiB (MOE_DISPATCH_SCRATCH_BYTES),
 * which each GPU the library runs on holds from the library's load until the
 * process ends. Arguments, results and errors are those of moe_dispatch.
 * A call whose count + scan path would need more than 8 MiB of scratch
 * (dispatch_workspace_size) returns MOE_ERR_UNSUPPORTED; the placement path
 * (up to 65536 pairs unless MOE_DISPATCH_PATH overrides it) needs none.
 * Every call on one GPU shares that GPU's scratch array, which keeps the
 * last call's contents (the kernels overwrite what they read), so calls that
 * may overlap on one GPU, from any stream or thread, race and must be
 * ordered by the caller.
 */
#define MOE_DISPATCH_SCRATCH_BYTES (8u << 20)

moe_status_t moe_dispatch_noalloc(const void *x, const int32_t *topk_ids,
                                  int64_t num_tokens, int32_t hidden,
                                  int32_t top_k, int32_t num_experts,
                                  int32_t ep_size,
                                  int64_t max_tokens_per_rank, void *payload,
                                  int32_t *src_info, int32_t *recv_counts,
                                  void *stream);

/*
 * Describes the launch an entry point would make for these sizes, without
 * touching the GPU. kind is a MOE_KIND_* value; for the local-reduce kinds
 * top_k is n_in.
 *
 * On success, writes a NUL-terminated text into buf, such as
 * "threads=128 vec_per_thread=1 chunks=7 blocks=28672 slot_tile=8 masked=0"
 * (or, for the dispatch, "path=place place_blocks=128 scatter_threads=64
 * scatter_vec_per_thread=2 scatter_blocks=28672"), and returns MOE_OK. It
 * validates the sizes like the entry point does.
 * The environment variable MOE_COMBINE_TILE="<threads>x<vectors>[x<kt>]"
 * overrides the threads per block and the 16-byte vectors per thread of
 * every combine entry point. kt, one of 2, 4 or 8, caps the slot tile, the
 * number of slots whose rows are loaded together.
 */
moe_status_t moe_combine_describe_launch(int kind, int64_t num_tokens,
                                         int32_t hidden, int32_t top_k,
                                         char *buf, int32_t buflen);

#ifdef __cplusplus
}
#endif

#endif /* MOE_COMBINE_H_ */
