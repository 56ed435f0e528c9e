// Device code of the MoE expert combine for CDNA4 (gfx950).
//
// One kernel template covers the three outputs. A workgroup of `blockDim.x`
// threads owns one (token, chunk) pair; a chunk is `blockDim.x * V`
// consecutive 16-byte vectors (8 bf16) of the hidden dimension. Thread i
// holds vectors chunk_base + v * blockDim.x + i, v < V, so every load and
// store instruction of a wavefront covers 1 KiB of contiguous memory.
//
// Per token the slot map and weights are wave-uniform (scalar loads). For
// each group of KT slots all row loads are issued before any arithmetic, so
// a lane keeps KT * V 16-byte loads in flight; dropped slots are skipped
// with a uniform branch and read nothing.
//
// A slot reads its row only if 0 <= rank < ep and 0 <= row < rows per rank
// (two scalar compares); any other slot, rank < 0 included, is dropped, so a
// bad slot map cannot read outside the payload.
//
// Arithmetic (Struct_ep_combine_skip_a2a, execute: weighted sum of the
// routed expert outputs; Parameter fused_shared_expert): acc starts at +0 and
// takes one fp32 fused multiply-add per kept slot in ascending slot order,
// then the unweighted shared-expert term. No MFMA: the work is a gather and
// a weighted sum, bound by HBM bandwidth.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

enum Epilogue { EPI_BF16 = 0, EPI_RMSNORM = 1, EPI_MXFP8 = 2, EPI_RMSNORM_MXFP8 = 3, EPI_MXFP4 = 4 };

struct KernelArgs {
    const uint16_t *payload;   // [ep, mtpr, H] bf16
    const int32_t *src_info;   // [T, k, 2]; null: slot j of token t is row t of input j
    const float *weights;      // [T, k] or null (unit weights)
    const uint16_t *shared;    // [T, H] or null
    const uint16_t *residual;  // [T, H]   (RMSNorm)
    const uint16_t *gamma;     // [H]      (RMSNorm)
    void *out0;                // bf16 out | residual_out | e4m3 codes
    void *out1;                // norm_out | UE8M0 scales | e4m3 codes of the norm
    void *out2;                // UE8M0 scales of the norm (RMSNorm + MXFP8)
    void *out3;                // bf16 norm_out or null (RMSNorm + MXFP8)
    int64_t mtpr;              // rows per rank
    int32_t H;                 // hidden
    int32_t nvec;              // H / 8
    int32_t k;                 // top_k
    int32_t ranks;             // ep: the payload's first dimension
    uint32_t rows;             // min(mtpr, 2^31): a slot's row must be below it (unsigned)
    int64_t rank_elems;        // mtpr * H: elements per rank of the payload
    int32_t chunks;            // workgroups per token
    float eps;
    float wb;
};

// bf16 element e (0..7) of a 16-byte vector, widened exactly to fp32.
__device__ __forceinline__ float bf16_elem(const u32x4 &x, int e) {
    const unsigned w = x[e >> 1];
    return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
}

// Two fp32 -> packed bf16 pair (low half = a), round to nearest even; on
// gfx950 this is the hardware v_cvt_pk_bf16_f32.
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
    f32x2 v = {a, b};
    bf16x2 r = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(unsigned, r);
}

// fp32 magnitude bits -> float8 e4m3fn code magnitude (0..0x7F): round to
// nearest even on the e4m3 grid, saturate at 448, NaN -> 0x7F. Integer route:
// for normal e4m3 values the fp32 pattern is rounded to 3 mantissa bits and
// rebiased (fp32 bias 127 -> e4m3 bias 7); below 2^-6 the value is scaled by
// 2^9 (exact) and rounded to an integer number of subnormal steps.
__device__ __forceinline__ unsigned e4m3_mag(unsigned a) {
    if (a > 0x7F800000u) return 0x7Fu;               // NaN
    if (a >= 0x43E00000u) return 0x7Eu;              // >= 448 (and inf)
    if (a >= 0x3C800000u) {                          // >= 2^-6
        const unsigned r = a + 0x7FFFFu + ((a >> 20) & 1u);
        return (r >> 20) - (120u << 3);
    }
    return (unsigned)__builtin_rintf(__uint_as_float(a) * 512.0f);
}

// Memory access helpers. Rows that are read once (payload, shared expert,
// residual) use non-temporal loads: on MI355X the streaming hint takes the
// bf16 combine at T = 4096, H = 7168 from 103.5 to 86.8 us (5.1 to 6.1 TB/s).
// gamma, reused by every token, takes ordinary loads.
__device__ __forceinline__ u32x4 ld_stream(const uint16_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ u32x4 ld_cached(const uint16_t *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

// Output stores, with the cache policy chosen per epilogue by measurement on
// MI355X. The output stores are what a gather-sum pays most for beyond its
// reads (the bf16 kernel without them runs in 71 us instead of 87 us at
// T = 4096, H = 7168).
//  - The bf16, MXFP8 and MXFP4 combines and the local reduce write through a
//    buffer resource over the output row (its size as the range, so the
//    hardware drops any store past it) with the SC1 cache policy:
//    device-scope write-through, the L2 forwarding the lines at once instead
//    of holding them dirty for a later eviction. That is 2-6% faster than
//    non-temporal stores (bf16 at T = 4096, H = 7168: 87.7 against 90.5 us).
//  - The RMSNorm epilogues write residual_out the same way, before the row
//    reduction, but the rows and codes written after it with non-temporal
//    global stores and the scales with write-back byte stores: at T = 2048,
//    H = 7168 that mix takes 54.5 us (55.9 with MXFP8), against 55.9 us with
//    every store non-temporal and 57.1 us with every store SC1.
constexpr int kPolSC1 = 16;   // CPol bits of the buffer stores

__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_row(void *row, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(row, (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ void st_sc1(__amdgpu_buffer_rsrc_t r, int off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kPolSC1);
}
__device__ __forceinline__ void st_sc1(__amdgpu_buffer_rsrc_t r, int off, u32x2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kPolSC1);
}
__device__ __forceinline__ void st_sc1(__amdgpu_buffer_rsrc_t r, int off, unsigned v) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kPolSC1);
}
__device__ __forceinline__ void st_sc1_byte(__amdgpu_buffer_rsrc_t r, int off, unsigned char v) {
    __builtin_amdgcn_raw_buffer_store_b8(v, r, off, 0, kPolSC1);
}
__device__ __forceinline__ void st_stream(uint16_t *p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}
__device__ __forceinline__ void st_stream(uint8_t *p, u32x2 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(p));
}

// fp32 magnitude bits -> float4 e2m1 code magnitude (0..7 for 0, 0.5, 1, 1.5,
// 2, 3, 4, 6): round to nearest even on that grid, saturate at 6; e2m1 has no
// NaN, so NaN and infinity saturate too. Integer route: at or above 1 the fp32
// pattern is rounded to 1 mantissa bit and rebiased (127 -> 1); below 1 the
// value is doubled (exact) and rounded to an integer number of 0.5 steps.
__device__ __forceinline__ unsigned e2m1_mag(unsigned a) {
    if (a > 0x7F800000u || a >= 0x40C00000u) return 7u;   // NaN, >= 6 (and inf)
    if (a >= 0x3F800000u) {                               // >= 1
        const unsigned r = a + 0x1FFFFFu + ((a >> 22) & 1u);
        return (r >> 22) - 252u;
    }
    return (unsigned)__builtin_rintf(__uint_as_float(a) * 2.0f);
}

// Max over the 4 lanes of a DPP quad (lanes 4m..4m+3).
__device__ __forceinline__ int quad_max(int v) {
    v = max(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true));  // [1,0,3,2]
    v = max(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true));  // [2,3,0,1]
    return v;
}

// Sum over the workgroup in fp64; every thread gets the same value (butterfly
// within each wave, then the wave partials in a fixed order from LDS).
__device__ __forceinline__ double block_sum(double v, double *lds) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    const int wid = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) lds[wid] = v;
    __syncthreads();
    const int nw = (blockDim.x + 63) >> 6;
    double s = 0.0;
    for (int i = 0; i < nw; ++i) s += lds[i];
    return s;
}

// Whether a chunk of the MXFP8 or MXFP4 combine may take the paired code
// stores and the word scale stores: two vectors per lane, the whole chunk in
// range, and rows (H % 128 == 0) and array bases aligned for the wider
// stores (codes to cbytes, scales to 4). The RMSNorm + MXFP8 epilogue keeps
// per-vector stores (pairing measured 0.5 us slower there).
template <int V>
__device__ __forceinline__ bool mx_pairable(const KernelArgs &a, int c, const void *codes, const void *scales,
                                            int cbytes) {
    return V == 2 && (c + 1) * V * (int)blockDim.x <= a.nvec && (a.H & 127) == 0 &&
           (reinterpret_cast<uintptr_t>(codes) & (uintptr_t)(cbytes - 1)) == 0 &&
           (reinterpret_cast<uintptr_t>(scales) & 3u) == 0;
}

// The UE8M0 scale bytes of one wave holding two vectors per lane, all in
// range: 16 bytes for each vector index v (one per DPP quad), stored as
// eight 4-byte words (lanes 0..3: v = 0, lanes 4..7: v = 1) instead of 32
// byte stores. vi0, vi1: this lane's two vector indices.
__device__ __forceinline__ void st_scales_wave(__amdgpu_buffer_rsrc_t rs, unsigned sb0, unsigned sb1, int vi0,
                                               int vi1) {
    const int lane = threadIdx.x & 63;
    const int qs = (lane & 3) * 16;                     // first of the word's 4 quads
    unsigned w0 = 0u, w1 = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        w0 |= (unsigned)__shfl((int)sb0, qs + 4 * i) << (8 * i);
        w1 |= (unsigned)__shfl((int)sb1, qs + 4 * i) << (8 * i);
    }
    const bool second = lane & 4;
    const int first_vec = (second ? vi1 : vi0) - lane;   // the wave's first vector of that half
    if (lane < 8) st_sc1(rs, (first_vec >> 2) + (lane & 3) * 4, second ? w1 : w0);
}

// MXFP8 quantisation of V vectors of 8 fp32 values held by this lane
// (flashinfer.comm.moe_a2a_combine, Parameters output_dtype float8_e4m3fn and
// output_scales UE8M0 with 32 elements per scale). A 32-element block is the
// 4 vectors of one DPP quad of lanes: amax is a quad max of the integer
// magnitudes (NaN patterns sort above infinity), the scale byte is the
// exponent field of amax minus 8, clamped at 0 (floor(log2 amax) - 8 + 127),
// 0xFF for NaN/inf blocks, and codes are e4m3 of x * 2^-e. Must be reached by
// every lane of the wave (no divergence around the DPP reads).
template <int V, bool SC1>
__device__ __forceinline__ void mx_quantize_store(const float (&x)[V][8], const bool (&ok)[V],
                                                  const int (&vi)[V], int H, uint8_t *codes_row,
                                                  uint8_t *scales_row, bool full = false) {
    const __amdgpu_buffer_rsrc_t rc = out_row(codes_row, H), rs = out_row(scales_row, H >> 5);
    u32x2 ov[V];
    unsigned sb[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        int m = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) m = max(m, (int)(__float_as_uint(x[v][e]) & 0x7FFFFFFFu));
        m = quad_max(m);
        const unsigned ef = (unsigned)m >> 23;                  // exponent field of amax
        const unsigned sbyte = ef == 255u ? 255u : (ef > 8u ? ef - 8u : 0u);
        // 2^-e as an fp32 bit pattern, e = sbyte - 127 (e = 0 for NaN/inf blocks)
        const float inv = ef == 255u ? 1.0f : __uint_as_float((254u - sbyte) << 23);
        if (!ok[v]) continue;
        u32x2 o = {0u, 0u};
        if (ef != 255u) {
            // finite block: clamp to +-448 (v_med3), then the hardware
            // e4m3 conversion, round to nearest even; the same codes as the
            // integer route (checked on every bf16 pattern and on 29M
            // fp32 sums), in far fewer instructions
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float q[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) q[i] = __builtin_amdgcn_fmed3f(x[v][4 * h + i] * inv, -448.0f, 448.0f);
                const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
                o[h] = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], lo, true);
            }
        } else {
            // NaN / infinity in the block: the integer route (NaN -> 0x7F)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const unsigned sgn = (__float_as_uint(x[v][e]) >> 24) & 0x80u;
                const float q = x[v][e] * inv;
                const unsigned code = sgn | e4m3_mag(__float_as_uint(q) & 0x7FFFFFFFu);
                o[e >> 2] |= code << ((e & 3) * 8);
            }
        }
        ov[v] = o;
        sb[v] = sbyte;
        if constexpr (SC1 && V == 2) {
            if (full) continue;                    // merged store below
        }
        if constexpr (SC1) {
            st_sc1(rc, vi[v] * 8, o);
            if ((threadIdx.x & 3) == 0) st_sc1_byte(rs, vi[v] >> 2, (unsigned char)sbyte);
        } else {
            st_stream(codes_row + (int64_t)vi[v] * 8, o);
            if ((threadIdx.x & 3) == 0) scales_row[vi[v] >> 2] = (uint8_t)sbyte;
        }
    }
    if constexpr (SC1 && V == 2) {
        if (full) {
            // lane l stores the codes of vectors 2j, 2j + 1 (j = l % 32) of
            // half l / 32, gathered from lanes 2j and 2j + 1: one 16-byte
            // store per lane instead of two 8-byte ones
            const int lane = threadIdx.x & 63, j = lane & 31, h = lane >> 5;
            const int s0 = 2 * j, s1 = 2 * j + 1;
            const unsigned a0 = __shfl(ov[0][0], s0), a1 = __shfl(ov[0][1], s0);
            const unsigned b0 = __shfl(ov[0][0], s1), b1 = __shfl(ov[0][1], s1);
            const unsigned c0 = __shfl(ov[1][0], s0), c1 = __shfl(ov[1][1], s0);
            const unsigned d0 = __shfl(ov[1][0], s1), d1 = __shfl(ov[1][1], s1);
            const u32x4 w = h ? (u32x4){c0, c1, d0, d1} : (u32x4){a0, a1, b0, b1};
            st_sc1(rc, (vi[h] - lane + 2 * j) * 8, w);
            st_scales_wave(rs, sb[0], sb[1], vi[0], vi[1]);
        }
    }
}

// MXFP4 quantisation (flashinfer.comm.moe_a2a_combine, Parameters
// output_scales UE8M0 with 32 elements per scale; the MXFP4 path ignores
// output_scalar_scale): like mx_quantize_store with the e2m1 element format,
// whose largest value is 6 = 1.5 * 2^2, so the scale byte is the exponent
// field of amax minus 2. Eight 4-bit codes per vector, element 2i in the low
// nibble of byte i, stored as one 4-byte word.
template <int V>
__device__ __forceinline__ void mx4_quantize_store(const float (&x)[V][8], const bool (&ok)[V],
                                                   const int (&vi)[V], int H, uint8_t *codes_row,
                                                   uint8_t *scales_row, bool full = false) {
    const __amdgpu_buffer_rsrc_t rc = out_row(codes_row, H >> 1), rs = out_row(scales_row, H >> 5);
    unsigned ov[V], sb[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        int m = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) m = max(m, (int)(__float_as_uint(x[v][e]) & 0x7FFFFFFFu));
        m = quad_max(m);
        const unsigned ef = (unsigned)m >> 23;
        const unsigned sbyte = ef == 255u ? 255u : (ef > 2u ? ef - 2u : 0u);
        const float inv = ef == 255u ? 1.0f : __uint_as_float((254u - sbyte) << 23);
        if (!ok[v]) continue;
        unsigned o = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const unsigned sgn = (__float_as_uint(x[v][e]) >> 28) & 0x8u;
            const float q = x[v][e] * inv;
            o |= (sgn | e2m1_mag(__float_as_uint(q) & 0x7FFFFFFFu)) << (4 * e);
        }
        ov[v] = o;
        sb[v] = sbyte;
        if constexpr (V == 2) {
            if (full) continue;                    // merged store below
        }
        st_sc1(rc, vi[v] * 4, o);
        if ((threadIdx.x & 3) == 0) st_sc1_byte(rs, vi[v] >> 2, (unsigned char)sbyte);
    }
    if constexpr (V == 2) {
        if (full) {
            // as for MXFP8: lane l stores the codes of vectors 2j, 2j + 1
            // (j = l % 32) of half l / 32 as one 8-byte word
            const int lane = threadIdx.x & 63, j = lane & 31, h = lane >> 5;
            const unsigned a0 = __shfl(ov[0], 2 * j), a1 = __shfl(ov[0], 2 * j + 1);
            const unsigned b0 = __shfl(ov[1], 2 * j), b1 = __shfl(ov[1], 2 * j + 1);
            const u32x2 w = h ? (u32x2){b0, b1} : (u32x2){a0, a1};
            st_sc1(rc, (vi[h] - lane + 2 * j) * 4, w);
            st_scales_wave(rs, sb[0], sb[1], vi[0], vi[1]);
        }
    }
}

// The routed sum of one (token, chunk): for each group of KT slots, load the
// slot map and weights (wave-uniform), issue every row load of the group,
// then take one fp32 fused multiply-add per kept slot in ascending slot
// order (Struct_ep_combine_skip_a2a, execute: the weighted sum of the routed
// expert outputs). A null slot map means dense inputs [k, T, H]: slot j of
// token t is row t of input j.
template <int KT, int V>
__device__ __forceinline__ void gather_sum(const KernelArgs &a, int t, const int (&vi)[V],
                                           const bool (&ok)[V], float (&acc)[V][8]) {
    const int32_t *__restrict__ si = a.src_info ? a.src_info + (int64_t)t * a.k * 2 : nullptr;
    const float *__restrict__ wt = a.weights ? a.weights + (int64_t)t * a.k : nullptr;

    for (int g = 0; g < a.k; g += KT) {
        const uint16_t *base[KT];
        bool valid[KT];
        float w[KT];
        int r[KT], row[KT];
        if (!a.src_info) {
            // dense inputs [k, T, H]: slot j of token t is row t of input j
#pragma unroll
            for (int jj = 0; jj < KT; ++jj) {
                const int j = g + jj;
                r[jj] = j < a.k ? j : -1;
                row[jj] = t;
                w[jj] = (j < a.k && wt) ? wt[j] : 1.0f;
            }
        } else if (g + KT <= a.k) {
            // full group: straight-line loads that merge into wide scalar loads
#pragma unroll
            for (int jj = 0; jj < KT; ++jj) {
                r[jj] = si[2 * (g + jj)];
                row[jj] = si[2 * (g + jj) + 1];
            }
            if (wt) {
#pragma unroll
                for (int jj = 0; jj < KT; ++jj) w[jj] = wt[g + jj];
            } else {
#pragma unroll
                for (int jj = 0; jj < KT; ++jj) w[jj] = 1.0f;
            }
        } else {
#pragma unroll
            for (int jj = 0; jj < KT; ++jj) {
                const int j = g + jj;
                const bool in = j < a.k;
                r[jj] = in ? si[2 * j] : -1;
                row[jj] = in ? si[2 * j + 1] : 0;
                w[jj] = (in && wt) ? wt[j] : 1.0f;
            }
        }
#pragma unroll
        for (int jj = 0; jj < KT; ++jj) {
            // rank < 0 marks a dropped slot; a slot outside the payload
            // reads nothing either. Both bounds in one unsigned compare
            // each, combined without a branch; the row offset is formed
            // from the per-rank stride (fewer 64-bit scalar multiplies).
            const unsigned ur = (unsigned)r[jj], uw = (unsigned)row[jj];
            valid[jj] = (ur < (unsigned)a.ranks) & (uw < a.rows);
            const int64_t off = (int64_t)ur * a.rank_elems + (int64_t)((uint64_t)uw * (unsigned)a.H);
            base[jj] = a.payload + (valid[jj] ? off : 0);
        }
        u32x4 x[KT][V];
#pragma unroll
        for (int jj = 0; jj < KT; ++jj) {
#pragma unroll
            for (int v = 0; v < V; ++v) {
                x[jj][v] = (u32x4){0u, 0u, 0u, 0u};
                if (valid[jj] && ok[v])
                    x[jj][v] = ld_stream(base[jj] + (int64_t)vi[v] * 8);
            }
        }
#pragma unroll
        for (int jj = 0; jj < KT; ++jj) {
            if (!valid[jj]) continue;
#pragma unroll
            for (int v = 0; v < V; ++v)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[v][e] = __builtin_fmaf(w[jj], bf16_elem(x[jj][v], e), acc[v][e]);
        }
    }
}

// Register budget: KT * V 16-byte loads are in flight per lane (KT * V <= 16,
// 64 VGPRs) plus 8 * V fp32 sums and up to 3 * 4 * V VGPRs of prefetched
// shared / residual / gamma vectors, so V >= 4 needs more than the 128 VGPRs a
// 1024-thread workgroup allows and is launched with at most 512 threads.
template <int V>
constexpr int max_threads_for() { return V >= 4 ? 512 : 1024; }

// KT: slot tile; V: 16-byte vectors per lane; EPI: output kind; MASK: the
// chunk may run past hidden / 8 vectors; SH: a shared-expert row is added.
template <int KT, int V, int EPI, bool MASK, bool SH>
__global__ __launch_bounds__(max_threads_for<V>()) void combine_kernel(KernelArgs a) {
    __shared__ double lds_red[16];
    const int nt = blockDim.x;
    const int tid = threadIdx.x;
    const int t = blockIdx.x / a.chunks;
    const int c = blockIdx.x - t * a.chunks;
    const int64_t row_off = (int64_t)t * a.H;          // output/shared row

    int vi[V];
    bool ok[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        vi[v] = (c * V + v) * nt + tid;
        ok[v] = !MASK || vi[v] < a.nvec;
    }

    float acc[V][8];
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[v][e] = 0.0f;

    // Rows that do not depend on the slot map are requested first, so their
    // latency overlaps the gathers instead of following them.
    u32x4 shv[V], resv[V], gmv[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        shv[v] = resv[v] = gmv[v] = (u32x4){0u, 0u, 0u, 0u};
        if (!ok[v]) continue;
        if constexpr (SH) shv[v] = ld_stream(a.shared + row_off + (int64_t)vi[v] * 8);
        if constexpr (EPI == EPI_RMSNORM || EPI == EPI_RMSNORM_MXFP8) {
            resv[v] = ld_stream(a.residual + row_off + (int64_t)vi[v] * 8);
            if constexpr (V <= 4) gmv[v] = ld_cached(a.gamma + (int64_t)vi[v] * 8);
        }
    }

    gather_sum<KT, V>(a, t, vi, ok, acc);

    if constexpr (SH) {
#pragma unroll
        for (int v = 0; v < V; ++v) {
            if (!ok[v]) continue;
            const u32x4 s = shv[v];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[v][e] = acc[v][e] + bf16_elem(s, e);
        }
    }

    if constexpr (EPI == EPI_BF16) {
        const __amdgpu_buffer_rsrc_t ro = out_row(static_cast<uint16_t *>(a.out0) + row_off, a.H * 2);
#pragma unroll
        for (int v = 0; v < V; ++v) {
            if (!ok[v]) continue;
            u32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[v][2 * i], acc[v][2 * i + 1]);
            st_sc1(ro, vi[v] * 16, o);
        }
    } else if constexpr (EPI == EPI_RMSNORM || EPI == EPI_RMSNORM_MXFP8) {
        // flashinfer.comm.trtllm_moe_allreduce_fusion, Parameters residual_in,
        // residual_out, rms_gamma, rms_eps, norm_out, weight_bias:
        //   residual_out = bf16(acc + residual_in)                   (fp32 add)
        //   n = residual_out * rstd * (gamma + weight_bias)
        // The statistic and the scaling are done in fp64 (each x^2 of a bf16
        // value is exact), so n matches a double-precision evaluation.
        const __amdgpu_buffer_rsrc_t rro = out_row(static_cast<uint16_t *>(a.out0) + row_off, a.H * 2);
        double ss = 0.0;
#pragma unroll
        for (int v = 0; v < V; ++v) {
            if (!ok[v]) continue;
            const u32x4 r = resv[v];
            u32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                o[i] = pack_bf16x2(acc[v][2 * i] + bf16_elem(r, 2 * i),
                                   acc[v][2 * i + 1] + bf16_elem(r, 2 * i + 1));
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xr = bf16_elem(o, e);     // the stored residual
                acc[v][e] = xr;
                ss = __builtin_fma((double)xr, (double)xr, ss);
            }
            st_sc1(rro, vi[v] * 16, o);
        }
        const double tot = block_sum(ss, lds_red);
        const double rstd = 1.0 / __builtin_sqrt(tot / (double)a.H + (double)a.eps);
#pragma unroll
        for (int v = 0; v < V; ++v) {
            // the widest rows re-read gamma here (L2-resident) to save registers
            const u32x4 gm = (V <= 4) ? gmv[v] : (ok[v] ? ld_cached(a.gamma + (int64_t)vi[v] * 8)
                                                       : (u32x4){0u, 0u, 0u, 0u});
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float g = bf16_elem(gm, e) + a.wb;
                acc[v][e] = (float)((double)acc[v][e] * rstd * (double)g);
            }
        }
        uint16_t *norm_out = static_cast<uint16_t *>(EPI == EPI_RMSNORM ? a.out1 : a.out3);
        if (norm_out) {
#pragma unroll
            for (int v = 0; v < V; ++v) {
                if (!ok[v]) continue;
                u32x4 o;
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[v][2 * i], acc[v][2 * i + 1]);
                st_stream(norm_out + row_off + (int64_t)vi[v] * 8, o);
            }
        }
        if constexpr (EPI == EPI_RMSNORM_MXFP8)
            mx_quantize_store<V, false>(acc, ok, vi, a.H, static_cast<uint8_t *>(a.out1) + row_off,
                                 static_cast<uint8_t *>(a.out2) + (int64_t)t * (a.H >> 5));
    } else if constexpr (EPI == EPI_MXFP8) {
        mx_quantize_store<V, true>(acc, ok, vi, a.H, static_cast<uint8_t *>(a.out0) + row_off,
                             static_cast<uint8_t *>(a.out1) + (int64_t)t * (a.H >> 5),
                             mx_pairable<V>(a, c, a.out0, a.out1, 16));
    } else {
        mx4_quantize_store<V>(acc, ok, vi, a.H, static_cast<uint8_t *>(a.out0) + (int64_t)t * (a.H >> 1),
                              static_cast<uint8_t *>(a.out1) + (int64_t)t * (a.H >> 5),
                              mx_pairable<V>(a, c, a.out0, a.out1, 8));
    }
}

}  // namespace moe
