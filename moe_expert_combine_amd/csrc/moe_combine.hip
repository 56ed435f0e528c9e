// Host side of the MoE expert-combine library: launch planning, kernel
// dispatch and the compute entry points of the C ABI declared in
// include/moe_combine.h. Argument validation (check_args.cpp) is pure host
// code and runs before any HIP call, so argument errors are reported
// identically on machines without a GPU. The library allocates nothing,
// keeps no state between calls and never synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_combine.h"
#include "host_check.h"
#include "combine_kernels.h"
#include "dispatch_kernels.h"

namespace {

using moe_host::fail;
using moe_host::ok;

static_assert(moe::kChunk == moe_host::kDispatchChunk, "dispatch chunk size");
static_assert(moe::kMaxExperts == moe_host::kMaxExperts, "dispatch expert limit");

constexpr int64_t kPlaceMaxPairs = 1 << 16;   // one-kernel dispatch placement up to here (measured crossover)
constexpr int kMaxThreads = 1024;
static_assert(moe_host::kMaxRmsHidden <= 512 * 8 * 8, "RMSNorm rows: 512 threads x 8 vectors x 8 bf16");

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

int64_t dispatch_chunks(int64_t T, int32_t k) { return (T * k + moe::kChunk - 1) / moe::kChunk; }

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
            // Rows of 6144 to 16384 elements: four vectors per lane (at
            // H = 7168, 256 threads with the last 128 vectors masked). With
            // slot tile 2 that measured 53.9 us against 54.3 us for 448 x 2 at
            // T = 2048 (52.9 against 53.3 us with the MXFP8 copy) on MI355X:
            // 4-wave workgroups, so more tokens are resident at once.
            if (nvec >= 768 && (nvec + 3) / 4 <= 512) {
                vec = 4;
                threads = ((nvec + 3) / 4 + 63) / 64 * 64;
            }
            for (int v : {1, 2, 4, 8}) {
                if (vec) break;
                const int t = ((nvec + v - 1) / v + 63) / 64 * 64;
                if (t <= 512) {
                    vec = v;
                    threads = t;
                    break;
                }
            }
            if (!vec) return fail(MOE_ERR_UNSUPPORTED, "hidden %d too large for the RMSNorm epilogue (max %d)", H,
                                  moe_host::kMaxRmsHidden);
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
    // serial tail (measured on MI355X at T=2048, H=7168: slot tile 2 with
    // four vectors per lane; with two vectors per lane, slot tile 4 for
    // RMSNorm and 2 when the normalised row is also quantised).
    if (!(forced && kt)) {
        if (kind == moe::EPI_RMSNORM && p->kt > (vec >= 4 ? 2 : 4)) p->kt = vec >= 4 ? 2 : 4;
        if (kind == moe::EPI_RMSNORM_MXFP8 && p->kt > 2) p->kt = 2;
    }
    p->masked = (int64_t)p->chunks * threads * vec != nvec;
    p->blocks = T * (int64_t)p->chunks;
    if (p->blocks > 0x7FFFFFFFLL) return fail(MOE_ERR_UNSUPPORTED, "grid too large (%lld workgroups)", (long long)p->blocks);
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

// ranks, mtpr: the payload's first two dimensions (for the dense reduce, the
// inputs and the tokens), which bound the slots the kernel reads.
moe::KernelArgs base_args(const void *payload, const int32_t *src_info, const float *w, const void *shared,
                          int32_t H, int32_t k, int32_t ranks, int64_t mtpr, const Plan &p) {
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
    a.ranks = ranks;
    // every int32 row >= 0 is below 2^31, so this bound is exact for any mtpr
    a.rows = (uint32_t)std::min<int64_t>(mtpr, int64_t(1) << 31);
    a.rank_elems = mtpr * H;
    a.chunks = p.chunks;
    return a;
}

// The arguments of a combine-kind call, for the validator.
moe_call_args_t combine_call(int kind, const void *payload, const int32_t *src_info, const float *w,
                             const void *shared, int64_t T, int32_t H, int32_t k, int32_t ep, int64_t mtpr) {
    moe_call_args_t c;
    memset(&c, 0, sizeof c);
    c.kind = kind;
    c.payload = payload;
    c.src_info = src_info;
    c.router_weights = w;
    c.shared_out = shared;
    c.num_tokens = T;
    c.hidden = H;
    c.top_k = k;
    c.ep_size = ep;
    c.max_tokens_per_rank = mtpr;
    return c;
}

moe_call_args_t reduce_call(int kind, const void *inputs, int32_t n_in, const float *scales,
                            const void *token_input, int64_t T, int32_t H) {
    moe_call_args_t c;
    memset(&c, 0, sizeof c);
    c.kind = kind;
    c.inputs = inputs;
    c.n_in = n_in;
    c.scales = scales;
    c.token_input = token_input;
    c.num_tokens = T;
    c.hidden = H;
    return c;
}

moe_call_args_t dispatch_call(const void *x, const int32_t *topk_ids, int64_t T, int32_t H, int32_t k, int32_t E,
                              int32_t ep, int64_t mtpr, void *payload, int32_t *src_info, int32_t *recv_counts) {
    moe_call_args_t c;
    memset(&c, 0, sizeof c);
    c.kind = MOE_KIND_DISPATCH;
    c.x = x;
    c.topk_ids = topk_ids;
    c.num_tokens = T;
    c.hidden = H;
    c.top_k = k;
    c.num_experts = E;
    c.ep_size = ep;
    c.max_tokens_per_rank = mtpr;
    c.payload = payload;
    c.src_info = src_info;
    c.recv_counts = recv_counts;
    return c;
}

// The dispatch's kernels for a validated call with num_tokens > 0; ws holds
// at least dispatch_workspace_bytes() on the count + scan path.
moe_status_t dispatch_launch(const moe_call_args_t &c, int32_t *ws, void *stream) {
    moe::DispatchArgs a;
    memset(&a, 0, sizeof a);
    a.x = static_cast<const uint16_t *>(c.x);
    a.ids = c.topk_ids;
    a.payload = static_cast<uint16_t *>(const_cast<void *>(c.payload));
    a.src_info = const_cast<int32_t *>(c.src_info);
    a.recv_counts = c.recv_counts;
    a.pairs = c.num_tokens * c.top_k;
    a.nchunks = (int)dispatch_chunks(c.num_tokens, c.top_k);
    a.offs = ws;
    a.local = a.offs + (int64_t)a.nchunks * c.num_experts;
    a.mtpr = c.max_tokens_per_rank;
    a.T = (int)c.num_tokens;
    a.H = c.hidden;
    a.k = c.top_k;
    a.E = c.num_experts;
    a.epr = c.num_experts / c.ep_size;
    a.segs = std::max(1, std::min(a.nchunks, 1024 / a.epr));
    a.idbits = 32 - __builtin_clz((unsigned)c.num_experts);
    int sthreads = 0, svec = 0;
    dispatch_tile(&sthreads, &svec);
    a.hchunks = (c.hidden / 8 + sthreads * svec - 1) / (sthreads * svec);
    if ((int64_t)a.T * a.hchunks > 0x7FFFFFFFLL) return fail(MOE_ERR_UNSUPPORTED, "grid too large");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 sg((unsigned)((int64_t)a.T * a.hchunks)), sb(sthreads);
    if (dispatch_path(a.pairs) == PATH_PLACE) {
        hipLaunchKernelGGL(moe::dispatch_place, dim3((unsigned)((a.pairs + moe::kPlaceChunk - 1) / moe::kPlaceChunk)),
                           dim3(moe::kPlace), 0, s, a);
        launch_scatter<false>(svec, sg, sb, s, a);
    } else {
        hipLaunchKernelGGL(moe::dispatch_count, dim3(a.nchunks), dim3(64), 0, s, a);
        hipLaunchKernelGGL(moe::dispatch_scan, dim3(c.ep_size), dim3(1024), 0, s, a);
        launch_scatter<true>(svec, sg, sb, s, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

// Scratch of the allocation-free dispatch: a file-scope device array that
// each GPU holds from the library's load until the process ends. On the host
// its name is only a stand-in for the symbol, not a device address: kernels
// and copies take the address that hipGetSymbolAddress returns for the
// current device, looked up once per device and kept.
constexpr size_t kScratchBytes = MOE_DISPATCH_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
__device__ __align__(256) uint8_t scratch[kScratchBytes];
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

moe_status_t scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

// Validation, then the launch plan; MOE_OK with *skip set means nothing to do.
moe_status_t prepare(const moe_call_args_t &c, int epi, int32_t k, Plan *p, bool *skip) {
    *skip = false;
    moe_status_t st = moe_host::check_call(c);
    if (st != MOE_OK) return st;
    if (c.num_tokens == 0) {
        *skip = true;
        return ok();
    }
    return make_plan(epi, c.num_tokens, c.hidden, k, p);
}

}  // namespace

extern "C" {

moe_status_t moe_combine(const void *payload, const int32_t *src_info, const float *router_weights,
                         const void *shared_out, void *out, int64_t num_tokens, int32_t hidden, int32_t top_k,
                         int32_t ep_size, int64_t max_tokens_per_rank, void *stream) {
    moe_call_args_t c = combine_call(MOE_KIND_COMBINE, payload, src_info, router_weights, shared_out, num_tokens,
                                     hidden, top_k, ep_size, max_tokens_per_rank);
    c.out = out;
    Plan p;
    bool skip;
    moe_status_t st = prepare(c, moe::EPI_BF16, top_k, &p, &skip);
    if (st != MOE_OK || skip) return st;
    moe::KernelArgs a = base_args(payload, src_info, router_weights, shared_out, hidden, top_k, ep_size, max_tokens_per_rank, p);
    a.out0 = out;
    return launch<moe::EPI_BF16>(p, a, stream);
}

moe_status_t moe_combine_residual_rmsnorm(const void *payload, const int32_t *src_info, const float *router_weights,
                                          const void *shared_out, const void *residual_in, const void *gamma,
                                          float eps, float weight_bias, void *residual_out, void *norm_out,
                                          int64_t num_tokens, int32_t hidden, int32_t top_k, int32_t ep_size,
                                          int64_t max_tokens_per_rank, void *stream) {
    moe_call_args_t c = combine_call(MOE_KIND_COMBINE_RESIDUAL_RMSNORM, payload, src_info, router_weights,
                                     shared_out, num_tokens, hidden, top_k, ep_size, max_tokens_per_rank);
    c.residual_in = residual_in;
    c.gamma = gamma;
    c.eps = eps;
    c.weight_bias = weight_bias;
    c.residual_out = residual_out;
    c.norm_out = norm_out;
    Plan p;
    bool skip;
    moe_status_t st = prepare(c, moe::EPI_RMSNORM, top_k, &p, &skip);
    if (st != MOE_OK || skip) return st;
    moe::KernelArgs a = base_args(payload, src_info, router_weights, shared_out, hidden, top_k, ep_size, max_tokens_per_rank, p);
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
    moe_call_args_t c = combine_call(MOE_KIND_COMBINE_MXFP8, payload, src_info, router_weights, shared_out,
                                     num_tokens, hidden, top_k, ep_size, max_tokens_per_rank);
    c.out_fp8 = out_fp8;
    c.out_scales = out_scales;
    Plan p;
    bool skip;
    moe_status_t st = prepare(c, moe::EPI_MXFP8, top_k, &p, &skip);
    if (st != MOE_OK || skip) return st;
    moe::KernelArgs a = base_args(payload, src_info, router_weights, shared_out, hidden, top_k, ep_size, max_tokens_per_rank, p);
    a.out0 = out_fp8;
    a.out1 = out_scales;
    return launch<moe::EPI_MXFP8>(p, a, stream);
}

moe_status_t moe_combine_mxfp4(const void *payload, const int32_t *src_info, const float *router_weights,
                               const void *shared_out, void *out_fp4, uint8_t *out_scales, int64_t num_tokens,
                               int32_t hidden, int32_t top_k, int32_t ep_size, int64_t max_tokens_per_rank,
                               void *stream) {
    moe_call_args_t c = combine_call(MOE_KIND_COMBINE_MXFP4, payload, src_info, router_weights, shared_out,
                                     num_tokens, hidden, top_k, ep_size, max_tokens_per_rank);
    c.out_fp4 = out_fp4;
    c.out_scales = out_scales;
    Plan p;
    bool skip;
    moe_status_t st = prepare(c, moe::EPI_MXFP4, top_k, &p, &skip);
    if (st != MOE_OK || skip) return st;
    moe::KernelArgs a = base_args(payload, src_info, router_weights, shared_out, hidden, top_k, ep_size, max_tokens_per_rank, p);
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
    moe_call_args_t c = combine_call(MOE_KIND_COMBINE_RESIDUAL_RMSNORM_MXFP8, payload, src_info, router_weights,
                                     shared_out, num_tokens, hidden, top_k, ep_size, max_tokens_per_rank);
    c.residual_in = residual_in;
    c.gamma = gamma;
    c.eps = eps;
    c.weight_bias = weight_bias;
    c.residual_out = residual_out;
    c.norm_out = norm_out;
    c.out_fp8 = out_fp8;
    c.out_scales = out_scales;
    Plan p;
    bool skip;
    moe_status_t st = prepare(c, moe::EPI_RMSNORM_MXFP8, top_k, &p, &skip);
    if (st != MOE_OK || skip) return st;
    moe::KernelArgs a = base_args(payload, src_info, router_weights, shared_out, hidden, top_k, ep_size, max_tokens_per_rank, p);
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

moe_status_t moe_reduce_dense(const void *inputs, int32_t n_in, const float *scales, const void *token_input,
                              void *out, int64_t num_tokens, int32_t hidden, void *stream) {
    moe_call_args_t c = reduce_call(MOE_KIND_REDUCE_DENSE, inputs, n_in, scales, token_input, num_tokens, hidden);
    c.out = out;
    Plan p;
    bool skip;
    moe_status_t st = prepare(c, moe::EPI_BF16, n_in, &p, &skip);
    if (st != MOE_OK || skip) return st;
    moe::KernelArgs a = base_args(inputs, nullptr, scales, token_input, hidden, n_in, n_in, num_tokens, p);
    a.out0 = out;
    return launch<moe::EPI_BF16>(p, a, stream);
}

moe_status_t moe_reduce_dense_residual_rmsnorm(const void *inputs, int32_t n_in, const float *scales,
                                               const void *token_input, const void *residual_in, const void *gamma,
                                               float eps, float weight_bias, void *residual_out, void *norm_out,
                                               int64_t num_tokens, int32_t hidden, void *stream) {
    moe_call_args_t c = reduce_call(MOE_KIND_REDUCE_DENSE_RESIDUAL_RMSNORM, inputs, n_in, scales, token_input,
                                    num_tokens, hidden);
    c.residual_in = residual_in;
    c.gamma = gamma;
    c.eps = eps;
    c.weight_bias = weight_bias;
    c.residual_out = residual_out;
    c.norm_out = norm_out;
    Plan p;
    bool skip;
    moe_status_t st = prepare(c, moe::EPI_RMSNORM, n_in, &p, &skip);
    if (st != MOE_OK || skip) return st;
    moe::KernelArgs a = base_args(inputs, nullptr, scales, token_input, hidden, n_in, n_in, num_tokens, p);
    a.residual = static_cast<const uint16_t *>(residual_in);
    a.gamma = static_cast<const uint16_t *>(gamma);
    a.out0 = residual_out;
    a.out1 = norm_out;
    a.eps = eps;
    a.wb = weight_bias;
    return launch<moe::EPI_RMSNORM>(p, a, stream);
}

moe_status_t moe_dispatch(const void *x, const int32_t *topk_ids, int64_t num_tokens, int32_t hidden,
                          int32_t top_k, int32_t num_experts, int32_t ep_size, int64_t max_tokens_per_rank,
                          void *payload, int32_t *src_info, int32_t *recv_counts, void *workspace,
                          size_t workspace_bytes, void *stream) {
    moe_call_args_t c = dispatch_call(x, topk_ids, num_tokens, hidden, top_k, num_experts, ep_size,
                                      max_tokens_per_rank, payload, src_info, recv_counts);
    c.workspace = workspace;
    c.workspace_bytes = workspace_bytes;
    moe_status_t st = moe_host::check_call(c);
    if (st != MOE_OK) return st;
    if (num_tokens == 0) return ok();
    return dispatch_launch(c, static_cast<int32_t *>(workspace), stream);
}

moe_status_t moe_dispatch_noalloc(const void *x, const int32_t *topk_ids, int64_t num_tokens, int32_t hidden,
                                  int32_t top_k, int32_t num_experts, int32_t ep_size,
                                  int64_t max_tokens_per_rank, void *payload, int32_t *src_info,
                                  int32_t *recv_counts, void *stream) {
    moe_call_args_t c = dispatch_call(x, topk_ids, num_tokens, hidden, top_k, num_experts, ep_size,
                                      max_tokens_per_rank, payload, src_info, recv_counts);
    moe_status_t st = moe_host::check_dispatch_own_scratch(c);
    if (st != MOE_OK) return st;
    if (num_tokens == 0) return ok();
    // only the count + scan path keeps data in the workspace
    const size_t need = dispatch_path(num_tokens * top_k) == PATH_PLACE
                            ? 0 : moe_host::dispatch_workspace_bytes(num_tokens, top_k, num_experts);
    if (need > kScratchBytes)
        return fail(MOE_ERR_UNSUPPORTED,
                    "this dispatch needs %zu bytes of scratch; moe_dispatch_noalloc holds at most %zu "
                    "(use moe_dispatch with a workspace)", need, kScratchBytes);
    void *ws = nullptr;
    if ((st = scratch_address(&ws)) != MOE_OK) return st;
    return dispatch_launch(c, static_cast<int32_t *>(ws), stream);
}

moe_status_t moe_combine_describe_launch(int kind, int64_t num_tokens, int32_t hidden, int32_t top_k, char *buf,
                                         int32_t buflen) {
    if (kind < 0 || kind > MOE_KIND_REDUCE_DENSE_RESIDUAL_RMSNORM)
        return fail(MOE_ERR_INVALID_ARG, "kind must be in [0, 7]");
    if (!buf || buflen < 1) return fail(MOE_ERR_INVALID_ARG, "buf is NULL or empty");
    moe_call_args_t c;
    memset(&c, 0, sizeof c);
    c.kind = kind;
    c.num_tokens = num_tokens;
    c.hidden = hidden;
    c.top_k = top_k;
    c.n_in = top_k;
    c.ep_size = 1;
    c.max_tokens_per_rank = 1;
    c.num_experts = 1;
    moe_status_t st = moe_host::check_sizes(c);
    if (st != MOE_OK) return st;
    if (kind == MOE_KIND_DISPATCH) {
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
    const int epi = kind == MOE_KIND_REDUCE_DENSE ? moe::EPI_BF16
                    : kind == MOE_KIND_REDUCE_DENSE_RESIDUAL_RMSNORM ? moe::EPI_RMSNORM : kind;
    Plan p;
    if ((st = make_plan(epi, num_tokens, hidden, top_k, &p)) != MOE_OK) return st;
    snprintf(buf, (size_t)buflen, "threads=%d vec_per_thread=%d chunks=%d blocks=%lld slot_tile=%d masked=%d",
             p.threads, p.vec, p.chunks, (long long)p.blocks, p.kt, (int)p.masked);
    return ok();
}

}  // extern "C"
