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
// Two kernels for small inputs (up to 65536 pairs by default):
//   1. dispatch_place:   every workgroup histograms all ids in LDS, finds the
//                        rows its own chunk of pairs starts from, ranks the
//                        chunk (stable: a ballot match on the id bits inside a
//                        wave, waves in order) and writes src_info;
//   2. dispatch_scatter: workgroup per (token, hidden chunk) reads the token
//                        row once and stores it to each of its placed rows.
// Three for large inputs, where the redundant histograms would cost more than
// a launch (a stable counting sort):
//   1. dispatch_count:   one wave per chunk of kChunk pairs walks them in
//                        order, 64 at a time, with the same ballot match and a
//                        running per-expert count in LDS. Writes each pair's
//                        (id, rank in chunk) and the chunk's per-expert counts;
//   2. dispatch_scan:    one workgroup per rank turns the counts into the first
//                        row of every (chunk, expert) within the rank: a
//                        segmented sum over chunks, a prefix over segments, a
//                        block prefix over the rank's experts; adds the receive
//                        counts;
//   3. dispatch_scatter: as above; its rows follow from steps 1 and 2 (first
//                        row of the chunk's expert + rank in chunk), and the
//                        first hidden chunk of each token writes src_info.
// The scatter goes in token order (on MI355X this beats copying in payload
// order, whose randomly ordered re-reads of token rows cost more than
// sequential writes save). On MI355X an empty kernel still costs about 3 us
// back to back (4.6 us as a profiled kernel duration), so the number of
// kernels, more than their work, sets the time of the routing metadata.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kChunk = 256;           // pairs per count chunk
constexpr int kMaxExperts = 4096;     // LDS counters and 13-bit id match
constexpr int kScanBatch = 32;        // chunk counts loaded per batch in the scan
constexpr int kPlace = 1024;          // threads per workgroup of dispatch_place
constexpr int kPlaceChunk = 256;      // pairs it ranks per workgroup (multiple of 64, <= kPlace)
constexpr int kPlaceBatch = 16;       // ids loaded per batch in its histogram

struct DispatchArgs {
    const uint16_t *x;        // [T, H] bf16
    const int32_t *ids;       // [T, k]
    uint16_t *payload;        // [ep, mtpr, H]
    int32_t *src_info;        // [T, k, 2]
    int32_t *recv_counts;     // [E] or null (accumulated)
    int32_t *offs;            // workspace [nchunks, E]: counts, then first rows
    int32_t *local;           // workspace [pairs]: id << 16 | rank in chunk; -1 dropped
    int64_t pairs;
    int64_t mtpr;
    int32_t T, H, k, E, epr, nchunks, hchunks;
    int32_t segs;             // scan segments per expert
    int32_t idbits;           // bits of the largest key (E, the dropped sentinel)
};

__device__ __forceinline__ int clean_id(int id, int E) { return (id >= 0 && id < E) ? id : -1; }

// One wave per chunk of pairs.
__global__ __launch_bounds__(64) void dispatch_count(DispatchArgs a) {
    __shared__ int cnt[kMaxExperts];
    const int c = blockIdx.x;
    const int lane = threadIdx.x;
    const int64_t p0 = (int64_t)c * kChunk;
    int ids[kChunk / 64];                                // the chunk's ids, prefetched
#pragma unroll
    for (int i = 0; i < kChunk / 64; ++i) {
        const int64_t p = p0 + i * 64 + lane;
        ids[i] = p < a.pairs ? a.ids[p] : -1;
    }
    for (int e = lane; e < a.E; e += 64) cnt[e] = 0;
    __syncthreads();
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));   // lanes below
    const uint64_t gt = (lane == 63) ? 0ull : (~0ull << (lane + 1));   // lanes above
#pragma unroll
    for (int gi = 0; gi < kChunk / 64; ++gi) {
        const int64_t p = p0 + gi * 64 + lane;
        const bool in = p < a.pairs;
        const int id = in ? clean_id(ids[gi], a.E) : -1;
        const int key = id >= 0 ? id : a.E;             // sentinel for dropped
        // lanes holding the same key: intersect the ballots of all key bits
        uint64_t same = ~0ull;
        for (int b = 0; b < a.idbits; ++b) {
            const uint64_t ones = __ballot((key >> b) & 1);
            same &= ((key >> b) & 1) ? ones : ~ones;
        }
        const int before = __popcll(same & lt);
        // All lanes read cnt in one LDS instruction; only the last lane of
        // each id then writes it (its value depends on that read), so every
        // read sees the value from before this group.
        int loc = -1;
        if (id >= 0) loc = cnt[id] + before;
        if (id >= 0 && (same & gt) == 0) cnt[id] = loc + 1;   // last of its id
        __builtin_amdgcn_wave_barrier();
        if (in) a.local[p] = id >= 0 ? (id << 16) | loc : -1;
    }
    __syncthreads();
    int32_t *h = a.offs + (int64_t)c * a.E;
    for (int e = lane; e < a.E; e += 64) h[e] = cnt[e];
}

// One workgroup per rank, for its experts [g * epr, (g + 1) * epr): every
// row offset depends only on counts of the same rank, so ranks scan
// independently. Thread (local expert e, segment s) owns chunks
// [s * L, (s + 1) * L) of the expert's column; consecutive threads take
// consecutive experts, so each load and store of a chunk row coalesces.
__global__ __launch_bounds__(1024) void dispatch_scan(DispatchArgs a) {
    __shared__ int part[kMaxExperts];   // [segs][epr]: segment sums, then their prefixes
    __shared__ int tot[kMaxExperts];    // expert totals
    __shared__ int pre[kMaxExperts];    // first row of each expert in the rank
    __shared__ int wsum[16];
    const int E = a.E, n = a.epr, S = a.segs;
    const int g0 = blockIdx.x * n;      // first expert of this rank
    const int L = (a.nchunks + S - 1) / S;
    for (int i = threadIdx.x; i < n * S; i += blockDim.x) {
        const int e = g0 + i % n, s = i / n;
        const int c0 = s * L, c1 = min(a.nchunks, c0 + L);
        int sum = 0;
        for (int c = c0; c < c1; c += kScanBatch) {
            int v[kScanBatch];
#pragma unroll
            for (int u = 0; u < kScanBatch; ++u) v[u] = (c + u < c1) ? a.offs[(int64_t)(c + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < kScanBatch; ++u) sum += v[u];
        }
        part[i] = sum;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < n; e += blockDim.x) {
        int run = 0;
        for (int s = 0; s < S; ++s) {
            const int v = part[s * n + e];
            part[s * n + e] = run;
            run += v;
        }
        tot[e] = run;
    }
    __syncthreads();
    // exclusive prefix of tot over the rank's experts: thread i sums experts
    // [i * per, (i + 1) * per), then a scan over the threads
    const int per = (n + (int)blockDim.x - 1) / (int)blockDim.x;
    const int e0 = threadIdx.x * per;
    int mine = 0;
    for (int u = 0; u < per; ++u)
        if (e0 + u < n) mine += tot[e0 + u];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int inc = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(inc, off, 64);
        if (lane >= off) inc += y;
    }
    if (lane == 63) wsum[wid] = inc;
    __syncthreads();
    int run = inc - mine;
    for (int w = 0; w < wid; ++w) run += wsum[w];
    for (int u = 0; u < per; ++u)
        if (e0 + u < n) {
            pre[e0 + u] = run;
            run += tot[e0 + u];
        }
    __syncthreads();
    // receive counts: the expert's rows [pre, pre + tot) cut at the capacity
    if (a.recv_counts)
        for (int e = threadIdx.x; e < n; e += blockDim.x) {
            const int64_t room = a.mtpr - pre[e];
            const int kept = room <= 0 ? 0 : (room < tot[e] ? (int)room : tot[e]);
            if (kept) atomicAdd(a.recv_counts + g0 + e, kept);
        }
    for (int i = threadIdx.x; i < n * S; i += blockDim.x) {
        const int e = g0 + i % n, s = i / n;
        const int c0 = s * L, c1 = min(a.nchunks, c0 + L);
        int r = pre[i % n] + part[i];
        for (int c = c0; c < c1; c += kScanBatch) {
            int v[kScanBatch];
#pragma unroll
            for (int u = 0; u < kScanBatch; ++u) v[u] = (c + u < c1) ? a.offs[(int64_t)(c + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < kScanBatch; ++u)
                if (c + u < c1) {
                    a.offs[(int64_t)(c + u) * E + e] = r;
                    r += v[u];
                }
        }
    }
}

// Placement of one chunk of pairs by a workgroup of kPlace threads, with no
// other workgroup involved. It histograms ALL ids in LDS, split at the
// chunk's first pair p0 (lo: pairs before p0, hi: the rest), so it knows
// every expert's total and the row the chunk's first pair of each expert
// takes. It then ranks the chunk's cnt <= kPlace pairs in order (wave w holds
// pairs p0 + 64 w .. p0 + 64 w + 63; the waves take their turns at the
// running rows in LDS between barriers), writes their src_info, and returns
// thread i's pair p0 + i as (rank, row), (-1, -1) if dropped or past the
// chunk. Workgroup 0 also adds the receive counts. Every thread of the
// workgroup must call it. The redundant histograms cost O(pairs) per
// workgroup, so the host uses it for small pair counts only.
__device__ __forceinline__ int2 place_chunk(const DispatchArgs &a, int64_t p0, int cnt, int *lo, int *hi,
                                            int *wsum) {
    const int E = a.E;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int64_t pm = p0 + tid;                        // this thread's own pair
    const bool mine_ok = tid < cnt && pm < a.pairs;
    const int myid = mine_ok ? clean_id(a.ids[pm], E) : -1;
    for (int e = tid; e < E; e += kPlace) lo[e] = hi[e] = 0;
    __syncthreads();
    for (int64_t q = tid; q < a.pairs; q += (int64_t)kPlace * kPlaceBatch) {
        int v[kPlaceBatch];
#pragma unroll
        for (int u = 0; u < kPlaceBatch; ++u) {
            const int64_t p = q + (int64_t)u * kPlace;
            v[u] = p < a.pairs ? a.ids[p] : -1;
        }
#pragma unroll
        for (int u = 0; u < kPlaceBatch; ++u) {
            const int id = clean_id(v[u], E);
            if (id >= 0) atomicAdd(q + (int64_t)u * kPlace < p0 ? &lo[id] : &hi[id], 1);
        }
    }
    __syncthreads();
    // hi <- exclusive prefix of the expert totals over all experts: thread i
    // sums experts [i * per, (i + 1) * per), then a scan over the threads
    const int per = (E + kPlace - 1) / kPlace;          // <= kMaxExperts / kPlace
    const int e0 = tid * per;
    int tv[kMaxExperts / kPlace];
    int mine = 0;
#pragma unroll
    for (int u = 0; u < kMaxExperts / kPlace; ++u) {
        tv[u] = (u < per && e0 + u < E) ? lo[e0 + u] + hi[e0 + u] : 0;
        mine += tv[u];
    }
    int inc = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(inc, off, 64);
        if (lane >= off) inc += y;
    }
    if (lane == 63) wsum[wid] = inc;
    __syncthreads();
    int run = inc - mine, grand = 0;
    for (int w = 0; w < kPlace / 64; ++w) {
        if (w < wid) run += wsum[w];
        grand += wsum[w];
    }
#pragma unroll
    for (int u = 0; u < kMaxExperts / kPlace; ++u)
        if (u < per && e0 + u < E) {
            hi[e0 + u] = run;
            run += tv[u];
        }
    __syncthreads();
    // lo <- row of the expert's first pair at or after p0, within its rank;
    // workgroup 0 adds the receive counts (rows cut at the capacity)
    for (int e = tid; e < E; e += kPlace) {
        const int base = hi[e] - hi[(e / a.epr) * a.epr];
        if (blockIdx.x == 0 && a.recv_counts) {
            const int tot = (e + 1 < E ? hi[e + 1] : grand) - hi[e];
            const int64_t room = a.mtpr - base;
            const int kept = room <= 0 ? 0 : (room < tot ? (int)room : tot);
            if (kept) atomicAdd(a.recv_counts + e, kept);
        }
        lo[e] += base;
    }
    __syncthreads();
    // stable rank among equal ids inside the wave: intersect the ballots of
    // all key bits (dropped pairs share the sentinel key E)
    const int key = myid >= 0 ? myid : E;
    uint64_t same = ~0ull;
    for (int b = 0; b < a.idbits; ++b) {
        const uint64_t ones = __ballot((key >> b) & 1);
        same &= ((key >> b) & 1) ? ones : ~ones;
    }
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const uint64_t gt = (lane == 63) ? 0ull : (~0ull << (lane + 1));
    const int before = __popcll(same & lt);
    int row = -1;
    for (int w = 0; w * 64 < cnt; ++w) {
        // one LDS read by all lanes, then the last lane of each id writes
        if (wid == w && myid >= 0) {
            row = lo[myid] + before;
            if ((same & gt) == 0) lo[myid] = row + 1;
        }
        __syncthreads();
    }
    int2 o = make_int2(-1, -1);
    if (myid >= 0 && row < a.mtpr) o = make_int2(myid / a.epr, row);
    if (mine_ok) reinterpret_cast<int2 *>(a.src_info)[pm] = o;
    return o;
}

// Small inputs, general hidden size: placement only, kPlaceChunk pairs per
// workgroup (on MI355X at 32768 pairs, 256 experts: 8.2 us against 11.4 us
// for count + scan); the scatter follows.
__global__ __launch_bounds__(kPlace) void dispatch_place(DispatchArgs a) {
    __shared__ int lo[kMaxExperts];
    __shared__ int hi[kMaxExperts];
    __shared__ int wsum[kPlace / 64];
    place_chunk(a, (int64_t)blockIdx.x * kPlaceChunk, kPlaceChunk, lo, hi, wsum);
}

typedef unsigned int du32x4 __attribute__((ext_vector_type(4)));

// Workgroup per (token, chunk of blockDim.x * V 16-byte vectors); the token
// row is read once and written to each placed row. While the row loads are in
// flight, lane j < k of each wave fetches slot j's (rank, row): from src_info
// as dispatch_place wrote it, or (FROM_OFFS) from the pair's (id, rank in
// chunk) and the scanned first rows, the first hidden chunk then writing
// src_info. The loop over slots takes them with readlane. The scattered row
// writes go through L2 (write-back): on MI355X that is about 3% faster here
// than non-temporal stores, unlike the combine's sequential output rows.
template <int V, bool FROM_OFFS>
__global__ __launch_bounds__(1024) void dispatch_scatter(DispatchArgs a) {
    // Workgroups are dealt to the 8 XCDs round-robin; renumber them so that
    // each XCD takes one contiguous range of (token, chunk) pairs. All chunks
    // of a token then run on one XCD, so each placed row is assembled in one
    // L2 (write-back stores) before it goes to HBM: 113.3 against 116.5 us
    // for the whole dispatch at T = 4096, H = 7168 on MI355X.
    const unsigned nb = gridDim.x, per = nb >> 3, rem = nb & 7;
    const unsigned xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    const unsigned lb = xcd * per + (xcd < rem ? xcd : rem) + idx;
    const int t = (int)(lb / (unsigned)a.hchunks);
    const int c = (int)(lb - (unsigned)t * (unsigned)a.hchunks);
    const int nvec = a.H / 8;
    const int nt = blockDim.x;
    du32x4 v[V];
    bool ok[V];
    int vi[V];
#pragma unroll
    for (int u = 0; u < V; ++u) {
        vi[u] = (c * V + u) * nt + threadIdx.x;
        ok[u] = vi[u] < nvec;
        if (ok[u]) v[u] = *reinterpret_cast<const du32x4 *>(a.x + (int64_t)t * a.H + (int64_t)vi[u] * 8);
    }
    // lane j < k of every wave resolves slot j of the token
    const int lane = threadIdx.x & 63;
    int rk = -1, rw = -1;
    if (lane < a.k) {
        const int64_t p = (int64_t)t * a.k + lane;
        if constexpr (FROM_OFFS) {
            const int lv = a.local[p];
            if (lv >= 0) {
                const int id = lv >> 16;
                const int row = a.offs[(p / kChunk) * a.E + id] + (lv & 0xFFFF);
                if (row < a.mtpr) {
                    rk = id / a.epr;
                    rw = row;
                }
            }
            if (c == 0 && threadIdx.x < 64)
                reinterpret_cast<int2 *>(a.src_info)[p] = make_int2(rk, rw);
        } else {
            const int2 o = reinterpret_cast<const int2 *>(a.src_info)[p];
            rk = o.x;
            rw = o.y;
        }
    }
    for (int j = 0; j < a.k; ++j) {
        const int r = __builtin_amdgcn_readlane(rk, j);
        if (r < 0) continue;
        const int w = __builtin_amdgcn_readlane(rw, j);
        uint16_t *dst = a.payload + ((int64_t)r * a.mtpr + w) * a.H;
#pragma unroll
        for (int u = 0; u < V; ++u)
            if (ok[u]) *reinterpret_cast<du32x4 *>(dst + (int64_t)vi[u] * 8) = v[u];
    }
}

}  // namespace moe
