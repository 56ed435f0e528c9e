// Device code of the MoE dispatch (the forward scatter the combine inverts)
// for CDNA4 (gfx950).
//
// Order of placement (flashinfer.comm.moe_a2a_combine summary: the combine is
// the inverse of the dispatch): kept (token, slot) pairs, enumerated
// token-major, are stably sorted by expert id; expert e lives on rank
// e / (E / ep); a pair's row is its position among its rank's pairs in that
// order, and a row at or past the rank's capacity drops the pair. Expert id
// -1 is a dropped slot (flashinfer.megamoe.nvfp4_mega_moe, Parameters
// num_tokens); ids outside [0, E) are treated the same way.
//
// A stable counting sort in three small kernels, then one scatter kernel:
//   1. dispatch_hist:  per chunk of kChunk pairs, a per-expert histogram in
//                      LDS (LDS atomics), written to hist[chunk][E];
//   2. dispatch_scan:  per expert, exclusive prefix over chunks (in place),
//                      the expert's first row within its rank, and the
//                      per-expert receive counts;
//   3. dispatch_rank:  one wave per chunk walks its pairs in order, 64 at a
//                      time; the stable rank among equal ids inside the wave
//                      comes from a ballot match on the 13 id bits, and a
//                      running per-expert row in LDS carries it across
//                      groups; writes src_info;
//   4. dispatch_scatter: workgroup per (token, hidden chunk) reads the token's
//                      row once and stores it to each of its placed rows (on
//                      MI355X this beats copying in payload order, whose
//                      randomly ordered re-reads of token rows cost more than
//                      sequential writes save).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kChunk = 256;           // pairs per histogram / rank chunk
constexpr int kMaxExperts = 4096;     // LDS counters and 13-bit id match
constexpr int kIdBits = 13;           // ids 0..E-1 plus the sentinel E < 8192

struct DispatchArgs {
    const uint16_t *x;        // [T, H] bf16
    const int32_t *ids;       // [T, k]
    uint16_t *payload;        // [ep, mtpr, H]
    int32_t *src_info;        // [T, k, 2]
    int32_t *recv_counts;     // [E] or null (accumulated)
    int32_t *hist;            // workspace [nchunks, E]
    int32_t *base;            // workspace [E]: first row of the expert in its rank
    int64_t pairs;            // T * k
    int64_t mtpr;
    int32_t T, H, k, E, epr, nchunks, hchunks;
};

__device__ __forceinline__ int clean_id(int id, int E) { return (id >= 0 && id < E) ? id : -1; }

__global__ __launch_bounds__(256) void dispatch_hist(DispatchArgs a) {
    __shared__ int cnt[kMaxExperts];
    for (int e = threadIdx.x; e < a.E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    const int64_t p0 = (int64_t)blockIdx.x * kChunk;
    for (int i = threadIdx.x; i < kChunk; i += blockDim.x) {
        const int64_t p = p0 + i;
        if (p < a.pairs) {
            const int id = clean_id(a.ids[p], a.E);
            if (id >= 0) atomicAdd(&cnt[id], 1);
        }
    }
    __syncthreads();
    int32_t *h = a.hist + (int64_t)blockIdx.x * a.E;
    for (int e = threadIdx.x; e < a.E; e += blockDim.x) h[e] = cnt[e];
}

// One workgroup. Thread e (strided) owns expert e; chunk counts are read 16
// at a time before their prefixes are written back, so the loads overlap.
__global__ __launch_bounds__(1024) void dispatch_scan(DispatchArgs a) {
    __shared__ int total[kMaxExperts];
    for (int e = threadIdx.x; e < a.E; e += blockDim.x) {
        int run = 0;
        for (int c0 = 0; c0 < a.nchunks; c0 += 16) {
            int v[16];
#pragma unroll
            for (int i = 0; i < 16; ++i)
                v[i] = (c0 + i < a.nchunks) ? a.hist[(int64_t)(c0 + i) * a.E + e] : 0;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (c0 + i < a.nchunks) a.hist[(int64_t)(c0 + i) * a.E + e] = run;
                run += v[i];
            }
        }
        total[e] = run;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < a.E; e += blockDim.x) {
        const int first = (e / a.epr) * a.epr;
        int b = 0;
        for (int f = first; f < e; ++f) b += total[f];
        a.base[e] = b;
        if (a.recv_counts) {
            // rows [b, b + total) of the rank, cut at the capacity
            const int64_t room = a.mtpr - b;
            const int kept = room <= 0 ? 0 : (room < total[e] ? (int)room : total[e]);
            a.recv_counts[e] += kept;
        }
    }
}

// One wave per chunk of pairs.
__global__ __launch_bounds__(64) void dispatch_rank(DispatchArgs a) {
    __shared__ int row_of[kMaxExperts];
    const int c = blockIdx.x;
    const int lane = threadIdx.x;
    for (int e = lane; e < a.E; e += 64) row_of[e] = a.base[e] + a.hist[(int64_t)c * a.E + e];
    __syncthreads();
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));   // lanes below
    const uint64_t gt = (lane == 63) ? 0ull : (~0ull << (lane + 1));   // lanes above
    const int64_t p0 = (int64_t)c * kChunk;
    int ids[kChunk / 64];                                // the chunk's ids, prefetched
#pragma unroll
    for (int i = 0; i < kChunk / 64; ++i) {
        const int64_t p = p0 + i * 64 + lane;
        ids[i] = p < a.pairs ? a.ids[p] : -1;
    }
#pragma unroll
    for (int gi = 0; gi < kChunk / 64; ++gi) {
        const int64_t p = p0 + gi * 64 + lane;
        const bool in = p < a.pairs;
        int id = in ? clean_id(ids[gi], a.E) : -1;
        const int key = id >= 0 ? id : a.E;             // sentinel for dropped
        // lanes holding the same key: intersect the ballots of all key bits
        uint64_t same = ~0ull;
#pragma unroll
        for (int b = 0; b < kIdBits; ++b) {
            const uint64_t ones = __ballot((key >> b) & 1);
            same &= ((key >> b) & 1) ? ones : ~ones;
        }
        const int before = __popcll(same & lt);
        // All lanes read row_of in one LDS instruction; only the last lane of
        // each id then writes it (its value depends on that read), so every
        // read sees the value from before this group.
        int row = -1;
        if (id >= 0) row = row_of[id] + before;
        if (id >= 0 && (same & gt) == 0) row_of[id] = row + 1;   // last of its id
        __builtin_amdgcn_wave_barrier();
        if (in) {
            int2 o = make_int2(-1, -1);
            if (id >= 0 && row < a.mtpr) o = make_int2(id / a.epr, row);
            reinterpret_cast<int2 *>(a.src_info)[p] = o;
        }
    }
}

typedef unsigned int du32x4 __attribute__((ext_vector_type(4)));

// Workgroup per (token, chunk of 64 * V 16-byte vectors); the token row is
// read once and written to each placed row. The scattered row writes go
// through L2 (write-back): on MI355X that is about 3% faster here than
// non-temporal stores, unlike the combine's sequential output rows.
template <int V>
__global__ __launch_bounds__(64) void dispatch_scatter(DispatchArgs a) {
    const int t = blockIdx.x / a.hchunks;
    const int c = blockIdx.x - t * a.hchunks;
    const int nvec = a.H / 8;
    du32x4 v[V];
    bool ok[V];
    int vi[V];
#pragma unroll
    for (int u = 0; u < V; ++u) {
        vi[u] = (c * V + u) * 64 + threadIdx.x;
        ok[u] = vi[u] < nvec;
        if (ok[u]) v[u] = *reinterpret_cast<const du32x4 *>(a.x + (int64_t)t * a.H + (int64_t)vi[u] * 8);
    }
    const int2 *si = reinterpret_cast<const int2 *>(a.src_info) + (int64_t)t * a.k;
    for (int j = 0; j < a.k; ++j) {
        const int2 rr = si[j];
        if (rr.x < 0) continue;
        uint16_t *dst = a.payload + ((int64_t)rr.x * a.mtpr + rr.y) * a.H;
#pragma unroll
        for (int u = 0; u < V; ++u)
            if (ok[u]) *reinterpret_cast<du32x4 *>(dst + (int64_t)vi[u] * 8) = v[u];
    }
}

}  // namespace moe
