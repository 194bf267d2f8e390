// Predictor kernels: the per-layer MLP that marks the neurons expected to fire
// (PowerInfer reading report, Part A section 2.3, module 3), with the active
// set compacted into an ascending index list on the device.
//
//   k_pred_hidden  h = act(P1 x + b1)                  P1 r x d fp16, h fp32
//   k_pred_logits  z = P2 h + b2 ; active = z > ln(tau/(1-tau))
//                  -> per-tile bitmaps, then the last tile to finish writes
//                     idx (ascending) and count         P2 ffn x r fp16
//
// Both stream a weight matrix from HBM once.  Weight loads are issued before
// the small vector (x or h) is staged into LDS, so staging overlaps them.
// Cross-workgroup data travels through device-coherent stores and loads and
// relaxed arrival counters: no workgroup ever waits for another, so the
// kernels cannot stall on dispatch order, and no L2 write-back is needed.
#include "common.hpp"
#include "internal.hpp"

namespace pi {

// ---------------------------------------------------------------------------
// Hidden layer.  One wave per row of P1: the 64 lanes read the row in 1 KB
// steps (16 B per lane), up to 16 steps in flight, and fold the fp16
// products into fp32 with v_dot2 against x in LDS.  Tokens are taken TB at a
// time, so each row is read once per TB tokens.  The kernel also zeroes the
// arrival counters of the logits kernel that follows it on the stream.
template <int TB>
__global__ __launch_bounds__(256) void k_pred_hidden(const h16* __restrict__ x, int B, int d,
                                                     const h16* __restrict__ P1,
                                                     const float* __restrict__ b1, int relu,
                                                     int r, float* __restrict__ h,
                                                     uint32_t* __restrict__ ctr) {
    extern __shared__ u32x4 sx[];  // TB x (d/8) chunks of x
    const int tid = threadIdx.x;
    for (int i = blockIdx.x * 256 + tid; i < B * (kArriveGroups + 1); i += gridDim.x * 256)
        ctr[(size_t)(i / (kArriveGroups + 1)) * kCtrWords + (i % (kArriveGroups + 1)) * kCtrStride] = 0u;

    const int wave = tid >> 6, lane = tid & 63;
    const int row = blockIdx.x * 4 + wave;
    const bool valid = row < r;
    const h16* prow = P1 + (size_t)(valid ? row : 0) * d;
    const int nch = d >> 3;
    const float bias = (b1 && valid) ? b1[row] : 0.f;

    for (int t0 = 0; t0 < B; t0 += TB) {
        u32x4 w[16];
        if (valid) {
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int c = lane + u * 64;
                if (c < nch) w[u] = ld16_stream(prow + (size_t)c * 8);
            }
        }
        __syncthreads();  // the previous token group is done with sx
        for (int i = tid; i < TB * nch; i += 256) {
            const int t = t0 + i / nch;
            sx[i] = (t < B) ? ld16(x + (size_t)t * d + (size_t)(i % nch) * 8) : u32x4{0u, 0u, 0u, 0u};
        }
        __syncthreads();
        float acc[TB];
#pragma unroll
        for (int t = 0; t < TB; ++t) acc[t] = 0.f;
        if (valid) {
            for (int c0 = lane; c0 < nch; c0 += 64 * 16) {
                if (c0 != lane) {
#pragma unroll
                    for (int u = 0; u < 16; ++u) {
                        const int c = c0 + u * 64;
                        if (c < nch) w[u] = ld16_stream(prow + (size_t)c * 8);
                    }
                }
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int c = c0 + u * 64;
                    if (c < nch) {
#pragma unroll
                        for (int t = 0; t < TB; ++t) acc[t] = dot8_h(w[u], sx[t * nch + c], acc[t]);
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            const float s = group_sum<64>(acc[t]) + bias;
            if (valid && lane == 0 && t0 + t < B) h[(size_t)(t0 + t) * r + row] = relu ? fmaxf(s, 0.f) : s;
        }
    }
}

// ---------------------------------------------------------------------------
// Logits, threshold and ordered compaction.  A workgroup owns a tile of 64
// consecutive neurons for one token: LPR lanes cooperate on a row of P2 (16 B
// each, so a load instruction covers 64/LPR rows x LPR*16 B contiguous), all
// of a thread's row loads are issued first, then h is staged in LDS, and
// each row's flag is the strict test z > thr.
//
// The tile's 64 flags become one ballot; the bitmap is published with a
// device-coherent store, then the tile arrives on a
// two-level counter.  The workgroup that completes the count scans every
// tile's popcount in tile order and writes the ascending index list and the
// total, so positions never depend on which tile finished first.
template <int LPR>
__global__ __launch_bounds__(256) void k_pred_logits(const h16* __restrict__ P2,
                                                     const float* __restrict__ b2,
                                                     const float* __restrict__ h, int r, int ffn,
                                                     float thr, int ntiles,
                                                     uint64_t* __restrict__ masks,
                                                     uint32_t* __restrict__ ctr,
                                                     int32_t* __restrict__ idx,
                                                     int32_t* __restrict__ count) {
    extern __shared__ float sh_h[];
    __shared__ uint32_t s_act[kPredTile];
    __shared__ int s_last;
    __shared__ uint32_t s_part[4];
    constexpr int RP = 256 / LPR;  // rows per pass
    constexpr int NP = kPredTile / RP;
    constexpr int U = 16;
    static_assert(kPredTile % RP == 0, "tile must be a whole number of passes");

    const int tile = blockIdx.x, tok = blockIdx.y;
    const int tid = threadIdx.x;
    const int grp = tid / LPR, p = tid % LPR;
    const int nch = r >> 3;
    // Full steps give every lane a valid chunk, so their guards are wave-uniform
    // and the loads issue back to back; a ragged r leaves one per-lane tail step.
    // Rows past ffn (last tile only) read row ffn-1 and their flags are dropped.
    const int nsteps = nch / LPR, tail = nch % LPR;
    const h16* prow[NP];
#pragma unroll
    for (int pp = 0; pp < NP; ++pp)
        prow[pp] = P2 + (size_t)min(tile * kPredTile + pp * RP + grp, ffn - 1) * r;

    float acc[NP];
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) acc[pp] = 0.f;
    // Whole batches of U steps carry no guard at all (a guarded batch makes the
    // compiler wait for every earlier load before reusing its registers).
    int s0 = 0;
    bool staged = false;
    for (; s0 + U <= nsteps; s0 += U) {
        u32x4 w[NP][U];
#pragma unroll
        for (int pp = 0; pp < NP; ++pp)
#pragma unroll
            for (int u = 0; u < U; ++u) w[pp][u] = ld16_stream(prow[pp] + (size_t)(p + (s0 + u) * LPR) * 8);
        if (!staged) {  // first batch in flight: stage h meanwhile
            for (int i = tid; i < r; i += 256) sh_h[i] = h[(size_t)tok * r + i];
            __syncthreads();
            staged = true;
        }
#pragma unroll
        for (int pp = 0; pp < NP; ++pp)
#pragma unroll
            for (int u = 0; u < U; ++u) acc[pp] = dot8_hf(w[pp][u], sh_h + (p + (s0 + u) * LPR) * 8, acc[pp]);
    }
    if (!staged) {
        for (int i = tid; i < r; i += 256) sh_h[i] = h[(size_t)tok * r + i];
        __syncthreads();
    }
    for (; s0 < nsteps; ++s0) {
        const int c = p + s0 * LPR;
#pragma unroll
        for (int pp = 0; pp < NP; ++pp) acc[pp] = dot8_hf(ld16_stream(prow[pp] + (size_t)c * 8), sh_h + c * 8, acc[pp]);
    }
    if (p < tail) {
        const int c = p + nsteps * LPR;
#pragma unroll
        for (int pp = 0; pp < NP; ++pp) acc[pp] = dot8_hf(ld16_stream(prow[pp] + (size_t)c * 8), sh_h + c * 8, acc[pp]);
    }
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
        const int rl = pp * RP + grp;
        const int row = tile * kPredTile + rl;
        const float z = group_sum<LPR>(acc[pp]);
        if (p == 0) s_act[rl] = (row < ffn) && (z + (b2 ? b2[row] : 0.f) > thr);
    }
    __syncthreads();

    uint32_t* tc = ctr + (size_t)tok * kCtrWords;
    if (tid < 64) {
        const uint64_t m = __ballot(s_act[tid] != 0u);
        if (tid == 0) {
            __hip_atomic_store(&masks[(size_t)tok * ntiles + tile], m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            wait_own_memory();
            const int g = tile % kArriveGroups;
            const uint32_t n1 = (uint32_t)((ntiles - g + kArriveGroups - 1) / kArriveGroups);
            const uint32_t groups = (uint32_t)min(ntiles, kArriveGroups);
            bool last = false;
            if (fetch_add(&tc[g * kCtrStride], 1u) == n1 - 1u)
                last = fetch_add(&tc[kArriveGroups * kCtrStride], 1u) == groups - 1u;
            s_last = last;
        }
    }
    __syncthreads();
    if (!s_last) return;

    // Ordered compaction by the last tile, 1024 tiles per round (4 per thread):
    // per-thread sums -> wave prefix sums -> workgroup offsets, then each
    // thread writes the ids of its own tiles' set bits in ascending order.
    const int wave = tid >> 6, lane = tid & 63;
    uint32_t base = 0;
    for (int t0 = 0; t0 < ntiles; t0 += 1024) {
        uint64_t m4[4];
        uint32_t mine = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int t = t0 + tid * 4 + q;
            m4[q] = t < ntiles ? __hip_atomic_load(&masks[(size_t)tok * ntiles + t], __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT) : 0ull;
            mine += (uint32_t)__popcll(m4[q]);
        }
        uint32_t incl = mine;  // inclusive prefix within the wave
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t v = __shfl_up(incl, off, 64);
            if (lane >= off) incl += v;
        }
        if (lane == 63) s_part[wave] = incl;
        __syncthreads();
        uint32_t pos = base + incl - mine;
        for (int w2 = 0; w2 < wave; ++w2) pos += s_part[w2];
        const uint32_t chunk_total = s_part[0] + s_part[1] + s_part[2] + s_part[3];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint64_t m = m4[q];
            const int t = t0 + tid * 4 + q;
            while (m) {
                idx[(size_t)tok * ffn + pos++] = t * kPredTile + __builtin_ctzll(m);
                m &= m - 1;
            }
        }
        base += chunk_total;
        __syncthreads();
    }
    if (tid == 0) count[tok] = (int32_t)base;
    if (tid <= kArriveGroups) st_flag(&tc[tid * kCtrStride], 0u);
}

hipError_t launch_pred_hidden(const h16* x, int B, int d, const h16* P1, const float* b1,
                              bool relu, int r, float* h, uint32_t* ctr, hipStream_t s) {
    dim3 grid((r + 3) / 4);
    const int TB = B == 1 ? 1 : (d <= 4096 ? 4 : (d <= 8192 ? 2 : 1));
    const size_t shm = (size_t)TB * d * 2;
    if (TB == 4)
        hipLaunchKernelGGL(k_pred_hidden<4>, grid, dim3(256), shm, s, x, B, d, P1, b1, (int)relu, r, h, ctr);
    else if (TB == 2)
        hipLaunchKernelGGL(k_pred_hidden<2>, grid, dim3(256), shm, s, x, B, d, P1, b1, (int)relu, r, h, ctr);
    else
        hipLaunchKernelGGL(k_pred_hidden<1>, grid, dim3(256), shm, s, x, B, d, P1, b1, (int)relu, r, h, ctr);
    return hipGetLastError();
}

hipError_t launch_pred_compact(const h16* P2, const float* b2, const float* h, int B, int r,
                               int ffn, float thr, uint64_t* masks, uint32_t* ctr, int32_t* idx, int32_t* count, hipStream_t s) {
    const int ntiles = pred_tiles(ffn);
    dim3 grid(ntiles, B);
    const size_t shm = (size_t)r * sizeof(float);
    if (r / 8 >= 8)
        hipLaunchKernelGGL(k_pred_logits<8>, grid, dim3(256), shm, s, P2, b2, h, r, ffn, thr, ntiles,
                           masks, ctr, idx, count);
    else
        hipLaunchKernelGGL(k_pred_logits<4>, grid, dim3(256), shm, s, P2, b2, h, r, ffn, thr, ntiles,
                           masks, ctr, idx, count);
    return hipGetLastError();
}

}  // namespace pi
