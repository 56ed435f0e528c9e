// Host side of the MoE expert-combine library: argument validation, launch
// planning, kernel dispatch and the C ABI declared in include/moe_combine.h.
//
// Validation is pure host code and runs before any HIP call, so argument
// errors are reported identically on machines without a GPU. The library
// allocates nothing, keeps no state between calls and never synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_combine.h"
#include "combine_kernels.h"
#include "dispatch_kernels.h"

namespace {

thread_local char g_err[256] = "";

moe_status_t fail(moe_status_t st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
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

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr int kMaxTopK = 32;
constexpr int64_t kPlaceMaxPairs = 1 << 16;   // one-kernel dispatch placement up to here (measured crossover)
constexpr int kMaxThreads = 1024;
constexpr int kMaxRmsHidden = 512 * 8 * 8;   // 512 threads x 8 vectors x 8 bf16
constexpr int kMaxHidden = 1 << 28;           // output rows are addressed with 32-bit byte offsets

// Launch shape of one call.
struct Plan {
    int threads;   // workgroup size (multiple of 64)
    int vec;       // 16-byte vectors per thread per chunk (1, 2, 4, 8)
    int chunks;    // workgroups per token
    int kt;        // slot tile (2, 4, 8)
    bool masked;   // tail vectors past hidden/8 exist
    int64_t blocks;
};

// Optional override "<threads>x<vectors>[x<slot tile>]" for tuning sweeps.
bool tile_override(int *threads, int *vec, int *kt) {
    const char *s = getenv("MOE_COMBINE_TILE");
    if (!s || !*s || !strcmp(s, "auto")) return false;
    int t = 0, v = 0, k = 0;
    const int n = sscanf(s, "%dx%dx%d", &t, &v, &k);
    if (n < 2) return false;
    if (t < 64 || t > kMaxThreads || t % 64 || !(v == 1 || v == 2 || v == 4 || v == 8)) return false;
    if (v >= 4 && t > 512) return false;   // register budget of the V >= 4 kernels
    if (n == 3 && !(k == 2 || k == 4 || k == 8)) return false;
    *threads = t;
    *vec = v;
    *kt = n == 3 ? k : 0;
    return true;
}

// Scatter shape of the dispatch: "<threads>x<vectors>" from
// MOE_DISPATCH_TILE for tuning sweeps, else one wave of two 16-byte vectors
// per lane.
void dispatch_tile(int *threads, int *vec) {
    *threads = 64;
    *vec = 2;
    const char *s = getenv("MOE_DISPATCH_TILE");
    if (!s || !*s || !strcmp(s, "auto")) return;
    int t = 0, v = 0;
    if (sscanf(s, "%dx%d", &t, &v) != 2) return;
    if (t < 64 || t > kMaxThreads || t % 64 || !(v == 1 || v == 2 || v == 4 || v == 8)) return;
    *threads = t;
    *vec = v;
}

// Dispatch paths. Placement by redundant per-workgroup histograms (place)
// grows with the pair count; the count + scan path pays one more launch. Up
// to kPlaceMaxPairs pairs: place + scatter; above: count + scan + scatter.
// MOE_DISPATCH_PATH = place | count_scan forces a path for tuning sweeps and
// tests (both are correct at every size).
enum DispatchPath { PATH_COUNT_SCAN = 0, PATH_PLACE = 1 };

DispatchPath dispatch_path(int64_t pairs) {
    DispatchPath p = pairs <= kPlaceMaxPairs ? PATH_PLACE : PATH_COUNT_SCAN;
    const char *s = getenv("MOE_DISPATCH_PATH");
    if (s && !strcmp(s, "count_scan")) p = PATH_COUNT_SCAN;
    if (s && !strcmp(s, "place")) p = PATH_PLACE;
    return p;
}

template <bool FROM_OFFS>
void launch_scatter(int vec, dim3 grid, dim3 block, hipStream_t s, const moe::DispatchArgs &a) {
    switch (vec) {
        case 1: hipLaunchKernelGGL((moe::dispatch_scatter<1, FROM_OFFS>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((moe::dispatch_scatter<2, FROM_OFFS>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((moe::dispatch_scatter<4, FROM_OFFS>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((moe::dispatch_scatter<8, FROM_OFFS>), grid, block, 0, s, a); break;
    }
}

moe_status_t make_plan(int kind, int64_t T, int32_t H, int32_t k, Plan *p) {
    const int nvec = H / 8;
    p->kt = k <= 2 ? 2 : (k <= 4 ? 4 : 8);
    int threads = 0, vec = 0, kt = 0;
    const bool forced = tile_override(&threads, &vec, &kt);
    if (forced && kt && kt < p->kt) p->kt = kt;
    if (kind == moe::EPI_RMSNORM || kind == moe::EPI_RMSNORM_MXFP8) {
        // The row reduction needs the whole token in one workgroup.
        if (!forced) {
            vec = 0;
            for (int v : {1, 2, 4, 8}) {
                const int t = ((nvec + v - 1) / v + 63) / 64 * 64;
                if (t <= 512) {
                    vec = v;
                    threads = t;
                    break;
                }
            }
            if (!vec) return fail(MOE_ERR_UNSUPPORTED, "hidden %d too large for the RMSNorm epilogue (max %d)", H, kMaxRmsHidden);
        }
        if ((int64_t)threads * vec < nvec)
            return fail(MOE_ERR_UNSUPPORTED, "tile %dx%d does not cover hidden %d for RMSNorm", threads, vec, H);
        p->chunks = 1;
    } else {
        if (!forced) {
            // one wave per workgroup, two 16-byte vectors per lane: each wave
            // reads 2 KiB of every routed row (fastest measured on MI355X)
            threads = 64;
            vec = nvec >= 128 ? 2 : 1;
        }
        p->chunks = (nvec + threads * vec - 1) / (threads * vec);
    }
    p->threads = threads;
    p->vec = vec;
    // at most 16 loads in flight per lane: shrink the slot tile for wide rows
    while (p->kt * vec > 16) p->kt /= 2;
    // The RMSNorm epilogues run after a workgroup barrier; a smaller slot
    // tile frees registers for more resident workgroups, which hides that
    // serial tail (measured on MI355X at T=2048, H=7168: slot tile 4 for
    // RMSNorm, 2 when the normalised row is also quantised).
    if (!(forced && kt)) {
        if (kind == moe::EPI_RMSNORM && p->kt > 4) p->kt = 4;
        if (kind == moe::EPI_RMSNORM_MXFP8 && p->kt > 2) p->kt = 2;
    }
    p->masked = (int64_t)p->chunks * threads * vec != nvec;
    p->blocks = T * (int64_t)p->chunks;
    if (p->blocks > 0x7FFFFFFFLL) return fail(MOE_ERR_UNSUPPORTED, "grid too large (%lld workgroups)", (long long)p->blocks);
    return MOE_OK;
}

moe_status_t check_common(const void *payload, const int32_t *src_info, const float *w, const void *shared,
                          int64_t T, int32_t H, int32_t k, int32_t ep, int64_t mtpr) {
    if (T < 0) return fail(MOE_ERR_INVALID_ARG, "num_tokens must be >= 0 (got %lld)", (long long)T);
    if (H <= 0 || H % 8) return fail(MOE_ERR_INVALID_ARG, "hidden must be a positive multiple of 8 (got %d)", H);
    if (H > kMaxHidden) return fail(MOE_ERR_INVALID_ARG, "hidden must be <= %d (got %d)", kMaxHidden, H);
    if (k < 1 || k > kMaxTopK) return fail(MOE_ERR_INVALID_ARG, "top_k must be in [1, %d] (got %d)", kMaxTopK, k);
    if (ep < 1) return fail(MOE_ERR_INVALID_ARG, "ep_size must be >= 1 (got %d)", ep);
    if (mtpr < 1 || mtpr > 0x7FFFFFFFLL) return fail(MOE_ERR_INVALID_ARG, "max_tokens_per_rank must be in [1, 2^31) (got %lld)", (long long)mtpr);
    if (T > 0x7FFFFFFFLL) return fail(MOE_ERR_INVALID_ARG, "num_tokens must be < 2^31");
    if ((double)ep * (double)mtpr * (double)H * 2.0 > 9.0e18) return fail(MOE_ERR_INVALID_ARG, "payload size overflows");
    if (T == 0) return MOE_OK;
    if (!payload) return fail(MOE_ERR_INVALID_ARG, "payload is NULL");
    if (!src_info) return fail(MOE_ERR_INVALID_ARG, "src_info is NULL");
    if (!aligned(payload, 16)) return fail(MOE_ERR_INVALID_ARG, "payload must be 16-byte aligned");
    if (!aligned(src_info, 8)) return fail(MOE_ERR_INVALID_ARG, "src_info must be 8-byte aligned");
    if (w && !aligned(w, 4)) return fail(MOE_ERR_INVALID_ARG, "router_weights must be 4-byte aligned");
    if (shared && !aligned(shared, 16)) return fail(MOE_ERR_INVALID_ARG, "shared_out must be 16-byte aligned");
    return MOE_OK;
}

template <int KT, int V, int EPI, bool MASK, bool SH>
void launch_one(const Plan &p, const moe::KernelArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((moe::combine_kernel<KT, V, EPI, MASK, SH>), dim3((unsigned)p.blocks), dim3(p.threads), 0, s, a);
}

template <int KT, int V, int EPI>
void launch_mask(const Plan &p, const moe::KernelArgs &a, hipStream_t s) {
    if (a.shared) {
        if (p.masked) launch_one<KT, V, EPI, true, true>(p, a, s);
        else launch_one<KT, V, EPI, false, true>(p, a, s);
    } else {
        if (p.masked) launch_one<KT, V, EPI, true, false>(p, a, s);
        else launch_one<KT, V, EPI, false, false>(p, a, s);
    }
}

// Largest slot tile for V vectors per lane: KT * V <= 16 (no register spills).
template <int V>
constexpr int kt_cap() { return 16 / V > 8 ? 8 : 16 / V; }

template <int V, int EPI>
void launch_kt(const Plan &p, const moe::KernelArgs &a, hipStream_t s) {
    constexpr int C = kt_cap<V>();
    if (p.kt <= 2) launch_mask<2, V, EPI>(p, a, s);
    else if (p.kt <= 4) launch_mask<(C < 4 ? C : 4), V, EPI>(p, a, s);
    else launch_mask<C, V, EPI>(p, a, s);
}

template <int EPI>
moe_status_t launch(const Plan &p, const moe::KernelArgs &a, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (p.vec) {
        case 1: launch_kt<1, EPI>(p, a, s); break;
        case 2: launch_kt<2, EPI>(p, a, s); break;
        case 4: launch_kt<4, EPI>(p, a, s); break;
        default: launch_kt<8, EPI>(p, a, s); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

moe::KernelArgs base_args(const void *payload, const int32_t *src_info, const float *w, const void *shared,
                          int32_t H, int32_t k, int64_t mtpr, const Plan &p) {
    moe::KernelArgs a;
    memset(&a, 0, sizeof a);
    a.payload = static_cast<const uint16_t *>(payload);
    a.src_info = src_info;
    a.weights = w;
    a.shared = static_cast<const uint16_t *>(shared);
    a.mtpr = mtpr;
    a.H = H;
    a.nvec = H / 8;
    a.k = k;
    a.chunks = p.chunks;
    return a;
}

}  // namespace

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

const char *moe_combine_last_error(void) { return g_err; }

moe_status_t moe_combine(const void *payload, const int32_t *src_info, const float *router_weights,
                         const void *shared_out, void *out, int64_t num_tokens, int32_t hidden, int32_t top_k,
                         int32_t ep_size, int64_t max_tokens_per_rank, void *stream) {
    moe_status_t st = check_common(payload, src_info, router_weights, shared_out, num_tokens, hidden, top_k,
                                   ep_size, max_tokens_per_rank);
    if (st != MOE_OK) return st;
    if (num_tokens == 0) return ok();
    if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
    if (!aligned(out, 16)) return fail(MOE_ERR_INVALID_ARG, "out must be 16-byte aligned");
    if (out == payload || out == shared_out) return fail(MOE_ERR_INVALID_ARG, "out must not alias an input");
    Plan p;
    if ((st = make_plan(moe::EPI_BF16, num_tokens, hidden, top_k, &p)) != MOE_OK) return st;
    moe::KernelArgs a = base_args(payload, src_info, router_weights, shared_out, hidden, top_k, max_tokens_per_rank, p);
    a.out0 = out;
    return launch<moe::EPI_BF16>(p, a, stream);
}

moe_status_t moe_combine_residual_rmsnorm(const void *payload, const int32_t *src_info, const float *router_weights,
                                          const void *shared_out, const void *residual_in, const void *gamma,
                                          float eps, float weight_bias, void *residual_out, void *norm_out,
                                          int64_t num_tokens, int32_t hidden, int32_t top_k, int32_t ep_size,
                                          int64_t max_tokens_per_rank, void *stream) {
    moe_status_t st = check_common(payload, src_info, router_weights, shared_out, num_tokens, hidden, top_k,
                                   ep_size, max_tokens_per_rank);
    if (st != MOE_OK) return st;
    Plan p;
    if ((st = make_plan(moe::EPI_RMSNORM, num_tokens, hidden, top_k, &p)) != MOE_OK) return st;
    if (num_tokens == 0) return ok();
    if (!residual_in || !gamma || !residual_out || !norm_out)
        return fail(MOE_ERR_INVALID_ARG, "residual_in, gamma, residual_out and norm_out are required");
    if (!aligned(residual_in, 16) || !aligned(gamma, 16) || !aligned(residual_out, 16) || !aligned(norm_out, 16))
        return fail(MOE_ERR_INVALID_ARG, "residual_in, gamma, residual_out and norm_out must be 16-byte aligned");
    if (norm_out == residual_out || norm_out == residual_in)
        return fail(MOE_ERR_INVALID_ARG, "norm_out must differ from residual_in and residual_out");
    const void *outs[2] = {residual_out, norm_out};
    for (const void *o : outs)
        if (o == payload || o == shared_out || o == gamma) return fail(MOE_ERR_INVALID_ARG, "outputs must not alias an input");
    if (!(eps >= 0.0f)) return fail(MOE_ERR_INVALID_ARG, "eps must be >= 0");
    moe::KernelArgs a = base_args(payload, src_info, router_weights, shared_out, hidden, top_k, max_tokens_per_rank, p);
    a.residual = static_cast<const uint16_t *>(residual_in);
    a.gamma = static_cast<const uint16_t *>(gamma);
    a.out0 = residual_out;
    a.out1 = norm_out;
    a.eps = eps;
    a.wb = weight_bias;
    return launch<moe::EPI_RMSNORM>(p, a, stream);
}

moe_status_t moe_combine_mxfp8(const void *payload, const int32_t *src_info, const float *router_weights,
                               const void *shared_out, void *out_fp8, uint8_t *out_scales, int64_t num_tokens,
                               int32_t hidden, int32_t top_k, int32_t ep_size, int64_t max_tokens_per_rank,
                               void *stream) {
    moe_status_t st = check_common(payload, src_info, router_weights, shared_out, num_tokens, hidden, top_k,
                                   ep_size, max_tokens_per_rank);
    if (st != MOE_OK) return st;
    if (hidden % 32) return fail(MOE_ERR_INVALID_ARG, "hidden must be a multiple of 32 for MXFP8 (got %d)", hidden);
    if (num_tokens == 0) return ok();
    if (!out_fp8 || !out_scales) return fail(MOE_ERR_INVALID_ARG, "out_fp8 and out_scales are required");
    if (!aligned(out_fp8, 8)) return fail(MOE_ERR_INVALID_ARG, "out_fp8 must be 8-byte aligned");
    if (out_fp8 == payload || out_fp8 == shared_out || (const void *)out_scales == payload ||
        (const void *)out_scales == shared_out || (const void *)out_scales == out_fp8)
        return fail(MOE_ERR_INVALID_ARG, "outputs must not alias an input or each other");
    Plan p;
    if ((st = make_plan(moe::EPI_MXFP8, num_tokens, hidden, top_k, &p)) != MOE_OK) return st;
    moe::KernelArgs a = base_args(payload, src_info, router_weights, shared_out, hidden, top_k, max_tokens_per_rank, p);
    a.out0 = out_fp8;
    a.out1 = out_scales;
    return launch<moe::EPI_MXFP8>(p, a, stream);
}

moe_status_t moe_combine_mxfp4(const void *payload, const int32_t *src_info, const float *router_weights,
                               const void *shared_out, void *out_fp4, uint8_t *out_scales, int64_t num_tokens,
                               int32_t hidden, int32_t top_k, int32_t ep_size, int64_t max_tokens_per_rank,
                               void *stream) {
    moe_status_t st = check_common(payload, src_info, router_weights, shared_out, num_tokens, hidden, top_k,
                                   ep_size, max_tokens_per_rank);
    if (st != MOE_OK) return st;
    if (hidden % 32) return fail(MOE_ERR_INVALID_ARG, "hidden must be a multiple of 32 for MXFP4 (got %d)", hidden);
    if (num_tokens == 0) return ok();
    if (!out_fp4 || !out_scales) return fail(MOE_ERR_INVALID_ARG, "out_fp4 and out_scales are required");
    if (!aligned(out_fp4, 4)) return fail(MOE_ERR_INVALID_ARG, "out_fp4 must be 4-byte aligned");
    if (out_fp4 == payload || out_fp4 == shared_out || (const void *)out_scales == payload ||
        (const void *)out_scales == shared_out || (const void *)out_scales == out_fp4)
        return fail(MOE_ERR_INVALID_ARG, "outputs must not alias an input or each other");
    Plan p;
    if ((st = make_plan(moe::EPI_MXFP4, num_tokens, hidden, top_k, &p)) != MOE_OK) return st;
    moe::KernelArgs a = base_args(payload, src_info, router_weights, shared_out, hidden, top_k, max_tokens_per_rank, p);
    a.out0 = out_fp4;
    a.out1 = out_scales;
    return launch<moe::EPI_MXFP4>(p, a, stream);
}

moe_status_t moe_combine_residual_rmsnorm_mxfp8(const void *payload, const int32_t *src_info,
                                                const float *router_weights, const void *shared_out,
                                                const void *residual_in, const void *gamma, float eps,
                                                float weight_bias, void *residual_out, void *norm_out,
                                                void *out_fp8, uint8_t *out_scales, int64_t num_tokens,
                                                int32_t hidden, int32_t top_k, int32_t ep_size,
                                                int64_t max_tokens_per_rank, void *stream) {
    moe_status_t st = check_common(payload, src_info, router_weights, shared_out, num_tokens, hidden, top_k,
                                   ep_size, max_tokens_per_rank);
    if (st != MOE_OK) return st;
    if (hidden % 32) return fail(MOE_ERR_INVALID_ARG, "hidden must be a multiple of 32 for MXFP8 (got %d)", hidden);
    Plan p;
    if ((st = make_plan(moe::EPI_RMSNORM_MXFP8, num_tokens, hidden, top_k, &p)) != MOE_OK) return st;
    if (num_tokens == 0) return ok();
    if (!residual_in || !gamma || !residual_out || !out_fp8 || !out_scales)
        return fail(MOE_ERR_INVALID_ARG, "residual_in, gamma, residual_out, out_fp8 and out_scales are required");
    if (!aligned(residual_in, 16) || !aligned(gamma, 16) || !aligned(residual_out, 16) ||
        (norm_out && !aligned(norm_out, 16)) || !aligned(out_fp8, 8))
        return fail(MOE_ERR_INVALID_ARG, "misaligned residual_in, gamma, residual_out, norm_out or out_fp8");
    const void *outs[4] = {residual_out, norm_out, out_fp8, out_scales};
    for (int i = 0; i < 4; ++i) {
        if (!outs[i]) continue;
        if (outs[i] == payload || outs[i] == shared_out || outs[i] == gamma)
            return fail(MOE_ERR_INVALID_ARG, "outputs must not alias an input");
        if (i > 0 && outs[i] == residual_in) return fail(MOE_ERR_INVALID_ARG, "only residual_out may alias residual_in");
        for (int j = 0; j < i; ++j)
            if (outs[j] == outs[i]) return fail(MOE_ERR_INVALID_ARG, "outputs must not alias each other");
    }
    if (!(eps >= 0.0f)) return fail(MOE_ERR_INVALID_ARG, "eps must be >= 0");
    moe::KernelArgs a = base_args(payload, src_info, router_weights, shared_out, hidden, top_k, max_tokens_per_rank, p);
    a.residual = static_cast<const uint16_t *>(residual_in);
    a.gamma = static_cast<const uint16_t *>(gamma);
    a.out0 = residual_out;
    a.out1 = out_fp8;
    a.out2 = out_scales;
    a.out3 = norm_out;
    a.eps = eps;
    a.wb = weight_bias;
    return launch<moe::EPI_RMSNORM_MXFP8>(p, a, stream);
}

static moe_status_t check_dense(const void *inputs, int32_t n_in, const float *scales, const void *token_input,
                                int64_t T, int32_t H) {
    if (n_in < 1 || n_in > kMaxTopK) return fail(MOE_ERR_INVALID_ARG, "n_in must be in [1, %d] (got %d)", kMaxTopK, n_in);
    moe_status_t st = check_common(inputs, reinterpret_cast<const int32_t *>(16), scales, token_input, T, H, n_in,
                                   n_in, T > 0 ? T : 1);
    if (st != MOE_OK) return st;
    if (T > 0 && !inputs) return fail(MOE_ERR_INVALID_ARG, "inputs is NULL");
    return MOE_OK;
}

moe_status_t moe_reduce_dense(const void *inputs, int32_t n_in, const float *scales, const void *token_input,
                              void *out, int64_t num_tokens, int32_t hidden, void *stream) {
    moe_status_t st = check_dense(inputs, n_in, scales, token_input, num_tokens, hidden);
    if (st != MOE_OK) return st;
    if (num_tokens == 0) return ok();
    if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
    if (!aligned(out, 16)) return fail(MOE_ERR_INVALID_ARG, "out must be 16-byte aligned");
    if (out == inputs || out == token_input) return fail(MOE_ERR_INVALID_ARG, "out must not alias an input");
    Plan p;
    if ((st = make_plan(moe::EPI_BF16, num_tokens, hidden, n_in, &p)) != MOE_OK) return st;
    moe::KernelArgs a = base_args(inputs, nullptr, scales, token_input, hidden, n_in, num_tokens, p);
    a.out0 = out;
    return launch<moe::EPI_BF16>(p, a, stream);
}

moe_status_t moe_reduce_dense_residual_rmsnorm(const void *inputs, int32_t n_in, const float *scales,
                                               const void *token_input, const void *residual_in, const void *gamma,
                                               float eps, float weight_bias, void *residual_out, void *norm_out,
                                               int64_t num_tokens, int32_t hidden, void *stream) {
    moe_status_t st = check_dense(inputs, n_in, scales, token_input, num_tokens, hidden);
    if (st != MOE_OK) return st;
    Plan p;
    if ((st = make_plan(moe::EPI_RMSNORM, num_tokens, hidden, n_in, &p)) != MOE_OK) return st;
    if (num_tokens == 0) return ok();
    if (!residual_in || !gamma || !residual_out || !norm_out)
        return fail(MOE_ERR_INVALID_ARG, "residual_in, gamma, residual_out and norm_out are required");
    if (!aligned(residual_in, 16) || !aligned(gamma, 16) || !aligned(residual_out, 16) || !aligned(norm_out, 16))
        return fail(MOE_ERR_INVALID_ARG, "residual_in, gamma, residual_out and norm_out must be 16-byte aligned");
    if (norm_out == residual_out || norm_out == residual_in)
        return fail(MOE_ERR_INVALID_ARG, "norm_out must differ from residual_in and residual_out");
    const void *outs[2] = {residual_out, norm_out};
    for (const void *o : outs)
        if (o == inputs || o == token_input || o == gamma) return fail(MOE_ERR_INVALID_ARG, "outputs must not alias an input");
    if (!(eps >= 0.0f)) return fail(MOE_ERR_INVALID_ARG, "eps must be >= 0");
    moe::KernelArgs a = base_args(inputs, nullptr, scales, token_input, hidden, n_in, num_tokens, p);
    a.residual = static_cast<const uint16_t *>(residual_in);
    a.gamma = static_cast<const uint16_t *>(gamma);
    a.out0 = residual_out;
    a.out1 = norm_out;
    a.eps = eps;
    a.wb = weight_bias;
    return launch<moe::EPI_RMSNORM>(p, a, stream);
}

static int64_t dispatch_chunks(int64_t T, int32_t k) { return (T * k + moe::kChunk - 1) / moe::kChunk; }

size_t moe_dispatch_workspace_size(int64_t num_tokens, int32_t top_k, int32_t num_experts, int32_t ep_size,
                                   int64_t max_tokens_per_rank) {
    if (num_tokens < 0 || top_k < 1 || num_experts < 1 || ep_size < 1 || max_tokens_per_rank < 1) return 0;
    // offs [nchunks, E] + local [T * k], int32 (ep_size and capacity are
    // part of the signature so that the layout may depend on them)
    const int64_t n = (dispatch_chunks(num_tokens, top_k) * (int64_t)num_experts + num_tokens * top_k) * 4;
    return (size_t)((n + 255) / 256 * 256);
}

moe_status_t moe_dispatch(const void *x, const int32_t *topk_ids, int64_t num_tokens, int32_t hidden,
                          int32_t top_k, int32_t num_experts, int32_t ep_size, int64_t max_tokens_per_rank,
                          void *payload, int32_t *src_info, int32_t *recv_counts, void *workspace,
                          size_t workspace_bytes, void *stream) {
    if (num_tokens < 0 || num_tokens > 0x7FFFFFFFLL)
        return fail(MOE_ERR_INVALID_ARG, "num_tokens must be in [0, 2^31)");
    if (hidden <= 0 || hidden % 8) return fail(MOE_ERR_INVALID_ARG, "hidden must be a positive multiple of 8 (got %d)", hidden);
    if (top_k < 1 || top_k > kMaxTopK) return fail(MOE_ERR_INVALID_ARG, "top_k must be in [1, %d] (got %d)", kMaxTopK, top_k);
    if (num_experts < 1 || num_experts > moe::kMaxExperts)
        return fail(MOE_ERR_INVALID_ARG, "num_experts must be in [1, %d] (got %d)", moe::kMaxExperts, num_experts);
    if (ep_size < 1 || num_experts % ep_size)
        return fail(MOE_ERR_INVALID_ARG, "ep_size must divide num_experts (got %d, %d)", ep_size, num_experts);
    if (max_tokens_per_rank < 1 || max_tokens_per_rank > 0x7FFFFFFFLL)
        return fail(MOE_ERR_INVALID_ARG, "max_tokens_per_rank must be in [1, 2^31)");
    if (num_tokens * (int64_t)top_k > 0x7FFFFFFFLL) return fail(MOE_ERR_INVALID_ARG, "num_tokens * top_k must be < 2^31");
    if (num_tokens == 0) return ok();
    if (!x || !topk_ids || !payload || !src_info || !workspace)
        return fail(MOE_ERR_INVALID_ARG, "x, topk_ids, payload, src_info and workspace are required");
    if (!aligned(x, 16) || !aligned(payload, 16) || !aligned(src_info, 8) || !aligned(topk_ids, 4) ||
        (recv_counts && !aligned(recv_counts, 4)) || !aligned(workspace, 4))
        return fail(MOE_ERR_INVALID_ARG, "misaligned pointer (x, payload 16 B; src_info 8 B; others 4 B)");
    const size_t need = moe_dispatch_workspace_size(num_tokens, top_k, num_experts, ep_size, max_tokens_per_rank);
    if (workspace_bytes < need)
        return fail(MOE_ERR_INVALID_ARG, "workspace too small (%zu < %zu bytes)", workspace_bytes, need);
    if (payload == x || (const void *)src_info == (const void *)topk_ids)
        return fail(MOE_ERR_INVALID_ARG, "outputs must not alias inputs");
    moe::DispatchArgs a;
    memset(&a, 0, sizeof a);
    a.x = static_cast<const uint16_t *>(x);
    a.ids = topk_ids;
    a.payload = static_cast<uint16_t *>(payload);
    a.src_info = src_info;
    a.recv_counts = recv_counts;
    a.pairs = num_tokens * top_k;
    a.nchunks = (int)dispatch_chunks(num_tokens, top_k);
    a.offs = static_cast<int32_t *>(workspace);
    a.local = a.offs + (int64_t)a.nchunks * num_experts;
    a.mtpr = max_tokens_per_rank;
    a.T = (int)num_tokens;
    a.H = hidden;
    a.k = top_k;
    a.E = num_experts;
    a.epr = num_experts / ep_size;
    a.segs = std::max(1, std::min(a.nchunks, 1024 / a.epr));
    a.idbits = 32 - __builtin_clz((unsigned)num_experts);
    int sthreads = 0, svec = 0;
    dispatch_tile(&sthreads, &svec);
    a.hchunks = (hidden / 8 + sthreads * svec - 1) / (sthreads * svec);
    if ((int64_t)a.T * a.hchunks > 0x7FFFFFFFLL) return fail(MOE_ERR_UNSUPPORTED, "grid too large");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 sg((unsigned)((int64_t)a.T * a.hchunks)), sb(sthreads);
    if (dispatch_path(a.pairs) == PATH_PLACE) {
        hipLaunchKernelGGL(moe::dispatch_place, dim3((unsigned)((a.pairs + moe::kPlaceChunk - 1) / moe::kPlaceChunk)),
                           dim3(moe::kPlace), 0, s, a);
        launch_scatter<false>(svec, sg, sb, s, a);
    } else {
        hipLaunchKernelGGL(moe::dispatch_count, dim3(a.nchunks), dim3(64), 0, s, a);
        hipLaunchKernelGGL(moe::dispatch_scan, dim3(ep_size), dim3(1024), 0, s, a);
        launch_scatter<true>(svec, sg, sb, s, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

moe_status_t moe_combine_describe_launch(int kind, int64_t num_tokens, int32_t hidden, int32_t top_k, char *buf,
                                         int32_t buflen) {
    if (kind < 0 || kind > 5) return fail(MOE_ERR_INVALID_ARG, "kind must be in [0, 5]");
    if (!buf || buflen < 1) return fail(MOE_ERR_INVALID_ARG, "buf is NULL or empty");
    if (kind == 5) {
        if (num_tokens < 0 || num_tokens > 0x7FFFFFFFLL) return fail(MOE_ERR_INVALID_ARG, "num_tokens must be in [0, 2^31)");
        if (hidden <= 0 || hidden % 8) return fail(MOE_ERR_INVALID_ARG, "hidden must be a positive multiple of 8 (got %d)", hidden);
        if (top_k < 1 || top_k > kMaxTopK) return fail(MOE_ERR_INVALID_ARG, "top_k must be in [1, %d] (got %d)", kMaxTopK, top_k);
        if (num_tokens * (int64_t)top_k > 0x7FFFFFFFLL) return fail(MOE_ERR_INVALID_ARG, "num_tokens * top_k must be < 2^31");
        int sthreads = 0, svec = 0;
        dispatch_tile(&sthreads, &svec);
        const int64_t pairs = num_tokens * top_k;
        const int64_t hchunks = (hidden / 8 + sthreads * svec - 1) / (sthreads * svec);
        const bool place = dispatch_path(pairs) == PATH_PLACE;
        snprintf(buf, (size_t)buflen, "path=%s place_blocks=%lld scatter_threads=%d scatter_vec_per_thread=%d "
                 "scatter_blocks=%lld", place ? "place" : "count_scan",
                 place ? (long long)((pairs + moe::kPlaceChunk - 1) / moe::kPlaceChunk) : 0LL, sthreads, svec,
                 (long long)(num_tokens * hchunks));
        return ok();
    }
    moe_status_t st = check_common(reinterpret_cast<const void *>(16), reinterpret_cast<const int32_t *>(16), nullptr,
                                   nullptr, num_tokens, hidden, top_k, 1, 1);
    if (st != MOE_OK) return st;
    if (kind >= 2 && hidden % 32)
        return fail(MOE_ERR_INVALID_ARG, "hidden must be a multiple of 32 for MXFP8 / MXFP4");
    Plan p;
    if ((st = make_plan(kind, num_tokens, hidden, top_k, &p)) != MOE_OK) return st;
    snprintf(buf, (size_t)buflen, "threads=%d vec_per_thread=%d chunks=%d blocks=%lld slot_tile=%d masked=%d",
             p.threads, p.vec, p.chunks, (long long)p.blocks, p.kt, (int)p.masked);
    return ok();
}

}  // extern "C"
