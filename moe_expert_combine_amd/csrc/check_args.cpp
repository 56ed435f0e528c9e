// Argument validation of every entry point, as pure host code: sizes,
// required pointers, alignment, and byte-range overlap of outputs with
// inputs and with each other. The entry points call check_call() before any
// HIP call; moe_combine_check_args() exports it. Nothing here includes a HIP
// header, so the same file also builds with a plain host compiler (and under
// the host sanitizers).
//
// Ownership rules enforced (documentation pages):
//  - flashinfer.comm.moe_a2a_combine, Parameters output: the caller provides
//    a contiguous output of matching shape and dtype on the same device;
//  - flashinfer.megamoe.nvfp4_mega_moe, Parameters y (the first num_tokens
//    rows are written in place) and Notes (contiguous tensors on one device);
//  - flashinfer.comm.trtllm_moe_allreduce_fusion, Parameters residual_out
//    (the updated residual, which may replace residual_in) and norm_out.
// An output is never allowed to share a byte with an input or with another
// output, except residual_out == residual_in exactly (the in-place update).
#include "host_check.h"

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

namespace moe_host {

namespace {

thread_local char g_err[256] = "";

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool is_combine(int kind) { return kind >= MOE_KIND_COMBINE && kind <= MOE_KIND_COMBINE_MXFP4; }
bool is_reduce(int kind) { return kind == MOE_KIND_REDUCE_DENSE || kind == MOE_KIND_REDUCE_DENSE_RESIDUAL_RMSNORM; }
bool is_rmsnorm(int kind) {
    return kind == MOE_KIND_COMBINE_RESIDUAL_RMSNORM || kind == MOE_KIND_COMBINE_RESIDUAL_RMSNORM_MXFP8 ||
           kind == MOE_KIND_REDUCE_DENSE_RESIDUAL_RMSNORM;
}
bool is_mx(int kind) {
    return kind == MOE_KIND_COMBINE_MXFP8 || kind == MOE_KIND_COMBINE_RESIDUAL_RMSNORM_MXFP8 ||
           kind == MOE_KIND_COMBINE_MXFP4;
}

// Byte range [p, p + n) of one argument.
struct Span {
    const char *name;
    const void *p;
    uint64_t n;
};

bool overlap(const Span &a, const Span &b) {
    if (!a.p || !b.p || !a.n || !b.n) return false;
    const unsigned __int128 a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.n && b0 < a0 + a.n;
}

// Every written span against every read span and every other written span.
// residual_out may coincide exactly with residual_in (in-place update).
moe_status_t check_overlaps(const Span *rd, int nr, const Span *wr, int nw) {
    for (int i = 0; i < nw; ++i) {
        for (int j = 0; j < nr; ++j) {
            if (!overlap(wr[i], rd[j])) continue;
            if (!strcmp(wr[i].name, "residual_out") && !strcmp(rd[j].name, "residual_in") &&
                wr[i].p == rd[j].p)
                continue;
            return fail(MOE_ERR_INVALID_ARG, "%s aliases %s: outputs must not overlap an input", wr[i].name,
                        rd[j].name);
        }
        for (int j = 0; j < i; ++j)
            if (overlap(wr[i], wr[j]))
                return fail(MOE_ERR_INVALID_ARG, "%s aliases %s: outputs must not overlap each other",
                            wr[i].name, wr[j].name);
    }
    return MOE_OK;
}

// Sizes of a combine or local-reduce call; k = top_k or n_in.
moe_status_t check_combine_sizes(const moe_call_args_t &c) {
    const int kind = c.kind;
    const int64_t T = c.num_tokens;
    const int32_t H = c.hidden;
    if (is_reduce(kind) && (c.n_in < 1 || c.n_in > kMaxTopK))
        return fail(MOE_ERR_INVALID_ARG, "n_in must be in [1, %d] (got %d)", kMaxTopK, c.n_in);
    if (T < 0) return fail(MOE_ERR_INVALID_ARG, "num_tokens must be >= 0 (got %lld)", (long long)T);
    if (H <= 0 || H % 8) return fail(MOE_ERR_INVALID_ARG, "hidden must be a positive multiple of 8 (got %d)", H);
    if (H > kMaxHidden) return fail(MOE_ERR_INVALID_ARG, "hidden must be <= %d (got %d)", kMaxHidden, H);
    if (is_combine(kind)) {
        if (c.top_k < 1 || c.top_k > kMaxTopK)
            return fail(MOE_ERR_INVALID_ARG, "top_k must be in [1, %d] (got %d)", kMaxTopK, c.top_k);
        if (c.ep_size < 1) return fail(MOE_ERR_INVALID_ARG, "ep_size must be >= 1 (got %d)", c.ep_size);
        if (c.max_tokens_per_rank < 1 || c.max_tokens_per_rank > 0x7FFFFFFFLL)
            return fail(MOE_ERR_INVALID_ARG, "max_tokens_per_rank must be in [1, 2^31) (got %lld)",
                        (long long)c.max_tokens_per_rank);
    }
    if (T > 0x7FFFFFFFLL) return fail(MOE_ERR_INVALID_ARG, "num_tokens must be < 2^31");
    const double rows = is_combine(kind) ? (double)c.ep_size * (double)c.max_tokens_per_rank
                                         : (double)c.n_in * (double)T;
    if (rows * (double)H * 2.0 > 9.0e18) return fail(MOE_ERR_INVALID_ARG, "payload size overflows");
    if (is_mx(kind) && H % 32)
        return fail(MOE_ERR_INVALID_ARG, "hidden must be a multiple of 32 for MXFP8 / MXFP4 (got %d)", H);
    if (is_rmsnorm(kind) && H > kMaxRmsHidden)
        return fail(MOE_ERR_UNSUPPORTED, "hidden %d too large for the RMSNorm epilogue (max %d)", H, kMaxRmsHidden);
    return MOE_OK;
}

moe_status_t check_dispatch_sizes(const moe_call_args_t &c) {
    const int64_t T = c.num_tokens;
    if (T < 0 || T > 0x7FFFFFFFLL) return fail(MOE_ERR_INVALID_ARG, "num_tokens must be in [0, 2^31)");
    if (c.hidden <= 0 || c.hidden % 8)
        return fail(MOE_ERR_INVALID_ARG, "hidden must be a positive multiple of 8 (got %d)", c.hidden);
    if (c.hidden > kMaxHidden) return fail(MOE_ERR_INVALID_ARG, "hidden must be <= %d (got %d)", kMaxHidden, c.hidden);
    if (c.top_k < 1 || c.top_k > kMaxTopK)
        return fail(MOE_ERR_INVALID_ARG, "top_k must be in [1, %d] (got %d)", kMaxTopK, c.top_k);
    if (c.num_experts < 1 || c.num_experts > kMaxExperts)
        return fail(MOE_ERR_INVALID_ARG, "num_experts must be in [1, %d] (got %d)", kMaxExperts, c.num_experts);
    if (c.ep_size < 1 || c.num_experts % c.ep_size)
        return fail(MOE_ERR_INVALID_ARG, "ep_size must divide num_experts (got %d, %d)", c.ep_size, c.num_experts);
    if (c.max_tokens_per_rank < 1 || c.max_tokens_per_rank > 0x7FFFFFFFLL)
        return fail(MOE_ERR_INVALID_ARG, "max_tokens_per_rank must be in [1, 2^31)");
    if (T * (int64_t)c.top_k > 0x7FFFFFFFLL) return fail(MOE_ERR_INVALID_ARG, "num_tokens * top_k must be < 2^31");
    if ((double)c.ep_size * (double)c.max_tokens_per_rank * (double)c.hidden * 2.0 > 9.0e18)
        return fail(MOE_ERR_INVALID_ARG, "payload size overflows");
    return MOE_OK;
}

moe_status_t check_combine_call(const moe_call_args_t &c) {
    moe_status_t st = check_combine_sizes(c);
    if (st != MOE_OK || c.num_tokens == 0) return st;
    const int kind = c.kind;
    const uint64_t T = (uint64_t)c.num_tokens, H = (uint64_t)c.hidden;
    const uint64_t row16 = T * H * 2;
    Span rd[8];
    int nr = 0;
    if (is_combine(kind)) {
        if (!c.payload) return fail(MOE_ERR_INVALID_ARG, "payload is NULL");
        if (!c.src_info) return fail(MOE_ERR_INVALID_ARG, "src_info is NULL");
        if (!aligned(c.payload, 16)) return fail(MOE_ERR_INVALID_ARG, "payload must be 16-byte aligned");
        if (!aligned(c.src_info, 8)) return fail(MOE_ERR_INVALID_ARG, "src_info must be 8-byte aligned");
        if (c.router_weights && !aligned(c.router_weights, 4))
            return fail(MOE_ERR_INVALID_ARG, "router_weights must be 4-byte aligned");
        if (c.shared_out && !aligned(c.shared_out, 16))
            return fail(MOE_ERR_INVALID_ARG, "shared_out must be 16-byte aligned");
        const uint64_t k = (uint64_t)c.top_k;
        rd[nr++] = {"payload", c.payload, (uint64_t)c.ep_size * (uint64_t)c.max_tokens_per_rank * H * 2};
        rd[nr++] = {"src_info", c.src_info, T * k * 8};
        rd[nr++] = {"router_weights", c.router_weights, T * k * 4};
        rd[nr++] = {"shared_out", c.shared_out, row16};
    } else {
        if (!c.inputs) return fail(MOE_ERR_INVALID_ARG, "inputs is NULL");
        if (!aligned(c.inputs, 16)) return fail(MOE_ERR_INVALID_ARG, "inputs must be 16-byte aligned");
        if (c.scales && !aligned(c.scales, 4)) return fail(MOE_ERR_INVALID_ARG, "scales must be 4-byte aligned");
        if (c.token_input && !aligned(c.token_input, 16))
            return fail(MOE_ERR_INVALID_ARG, "token_input must be 16-byte aligned");
        rd[nr++] = {"inputs", c.inputs, (uint64_t)c.n_in * row16};
        rd[nr++] = {"scales", c.scales, T * (uint64_t)c.n_in * 4};
        rd[nr++] = {"token_input", c.token_input, row16};
    }
    Span wr[4];
    int nw = 0;
    if (kind == MOE_KIND_COMBINE || kind == MOE_KIND_REDUCE_DENSE) {
        if (!c.out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
        if (!aligned(c.out, 16)) return fail(MOE_ERR_INVALID_ARG, "out must be 16-byte aligned");
        wr[nw++] = {"out", c.out, row16};
    } else if (is_rmsnorm(kind)) {
        const bool mx = kind == MOE_KIND_COMBINE_RESIDUAL_RMSNORM_MXFP8;
        if (!c.residual_in || !c.gamma || !c.residual_out || (!mx && !c.norm_out))
            return fail(MOE_ERR_INVALID_ARG, mx ? "residual_in, gamma, residual_out, out_fp8 and out_scales are required"
                                                : "residual_in, gamma, residual_out and norm_out are required");
        if (mx && (!c.out_fp8 || !c.out_scales))
            return fail(MOE_ERR_INVALID_ARG, "residual_in, gamma, residual_out, out_fp8 and out_scales are required");
        if (!aligned(c.residual_in, 16) || !aligned(c.gamma, 16) || !aligned(c.residual_out, 16) ||
            (c.norm_out && !aligned(c.norm_out, 16)))
            return fail(MOE_ERR_INVALID_ARG, "residual_in, gamma, residual_out and norm_out must be 16-byte aligned");
        if (mx && !aligned(c.out_fp8, 8)) return fail(MOE_ERR_INVALID_ARG, "out_fp8 must be 8-byte aligned");
        if (!(c.eps >= 0.0f)) return fail(MOE_ERR_INVALID_ARG, "eps must be >= 0");
        rd[nr++] = {"residual_in", c.residual_in, row16};
        rd[nr++] = {"gamma", c.gamma, H * 2};
        wr[nw++] = {"residual_out", c.residual_out, row16};
        wr[nw++] = {"norm_out", c.norm_out, row16};
        if (mx) {
            wr[nw++] = {"out_fp8", c.out_fp8, T * H};
            wr[nw++] = {"out_scales", c.out_scales, T * (H / 32)};
        }
    } else if (kind == MOE_KIND_COMBINE_MXFP8) {
        if (!c.out_fp8 || !c.out_scales) return fail(MOE_ERR_INVALID_ARG, "out_fp8 and out_scales are required");
        if (!aligned(c.out_fp8, 8)) return fail(MOE_ERR_INVALID_ARG, "out_fp8 must be 8-byte aligned");
        wr[nw++] = {"out_fp8", c.out_fp8, T * H};
        wr[nw++] = {"out_scales", c.out_scales, T * (H / 32)};
    } else {
        if (!c.out_fp4 || !c.out_scales) return fail(MOE_ERR_INVALID_ARG, "out_fp4 and out_scales are required");
        if (!aligned(c.out_fp4, 4)) return fail(MOE_ERR_INVALID_ARG, "out_fp4 must be 4-byte aligned");
        wr[nw++] = {"out_fp4", c.out_fp4, T * (H / 2)};
        wr[nw++] = {"out_scales", c.out_scales, T * (H / 32)};
    }
    return check_overlaps(rd, nr, wr, nw);
}

// own_scratch: the workspace is the library's own device array (a separate
// allocation), so the workspace fields are not the caller's and are not
// checked.
moe_status_t check_dispatch_call(const moe_call_args_t &c, bool own_scratch) {
    moe_status_t st = check_dispatch_sizes(c);
    if (st != MOE_OK || c.num_tokens == 0) return st;
    if (!c.x || !c.topk_ids || !c.payload || !c.src_info || (!own_scratch && !c.workspace))
        return fail(MOE_ERR_INVALID_ARG, own_scratch ? "x, topk_ids, payload and src_info are required"
                                                     : "x, topk_ids, payload, src_info and workspace are required");
    if (!aligned(c.x, 16) || !aligned(c.payload, 16) || !aligned(c.src_info, 8) || !aligned(c.topk_ids, 4) ||
        (c.recv_counts && !aligned(c.recv_counts, 4)) || (!own_scratch && !aligned(c.workspace, 4)))
        return fail(MOE_ERR_INVALID_ARG, "misaligned pointer (x, payload 16 B; src_info 8 B; others 4 B)");
    const size_t need = dispatch_workspace_bytes(c.num_tokens, c.top_k, c.num_experts);
    if (!own_scratch && c.workspace_bytes < need)
        return fail(MOE_ERR_INVALID_ARG, "workspace too small (%zu < %zu bytes)", c.workspace_bytes, need);
    const uint64_t T = (uint64_t)c.num_tokens, H = (uint64_t)c.hidden, k = (uint64_t)c.top_k;
    const Span rd[2] = {{"x", c.x, T * H * 2}, {"topk_ids", c.topk_ids, T * k * 4}};
    const Span wr[4] = {{"payload", c.payload, (uint64_t)c.ep_size * (uint64_t)c.max_tokens_per_rank * H * 2},
                        {"src_info", c.src_info, T * k * 8},
                        {"recv_counts", c.recv_counts, (uint64_t)c.num_experts * 4},
                        {"workspace", own_scratch ? nullptr : c.workspace, (uint64_t)need}};
    return check_overlaps(rd, 2, wr, 4);
}

}  // namespace

moe_status_t fail(moe_status_t st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

moe_status_t ok() {
    g_err[0] = '\0';
    return MOE_OK;
}

size_t dispatch_workspace_bytes(int64_t T, int32_t k, int32_t E) {
    // per-chunk expert offsets [chunks, E] + per-pair ranks [T * k], int32,
    // rounded up to 256 bytes
    const int64_t chunks = (T * k + kDispatchChunk - 1) / kDispatchChunk;
    const int64_t n = (chunks * (int64_t)E + T * k) * 4;
    return (size_t)((n + 255) / 256 * 256);
}

moe_status_t check_sizes(const moe_call_args_t &c) {
    if (c.kind == MOE_KIND_DISPATCH) return check_dispatch_sizes(c);
    if (is_combine(c.kind) || is_reduce(c.kind)) return check_combine_sizes(c);
    return fail(MOE_ERR_INVALID_ARG, "kind must be in [0, 7] (got %d)", c.kind);
}

moe_status_t check_call(const moe_call_args_t &c) {
    if (c.kind == MOE_KIND_DISPATCH) return check_dispatch_call(c, false);
    if (is_combine(c.kind) || is_reduce(c.kind)) return check_combine_call(c);
    return fail(MOE_ERR_INVALID_ARG, "kind must be in [0, 7] (got %d)", c.kind);
}

moe_status_t check_dispatch_own_scratch(const moe_call_args_t &c) { return check_dispatch_call(c, true); }

}  // namespace moe_host

extern "C" {

int moe_combine_abi_version(void) { return MOE_COMBINE_ABI_VERSION; }

const char *moe_combine_status_string(int status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
        default: return "MOE_ERR_UNKNOWN";
    }
}

const char *moe_combine_last_error(void) { return moe_host::g_err; }

moe_status_t moe_combine_check_args(const moe_call_args_t *args) {
    if (!args) return moe_host::fail(MOE_ERR_INVALID_ARG, "args is NULL");
    const moe_status_t st = moe_host::check_call(*args);
    return st == MOE_OK ? moe_host::ok() : st;
}

size_t moe_dispatch_workspace_size(int64_t num_tokens, int32_t top_k, int32_t num_experts, int32_t ep_size,
                                   int64_t max_tokens_per_rank) {
    if (num_tokens < 0 || top_k < 1 || num_experts < 1 || ep_size < 1 || max_tokens_per_rank < 1) return 0;
    return moe_host::dispatch_workspace_bytes(num_tokens, top_k, num_experts);
}

}  // extern "C"
