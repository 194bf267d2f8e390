// Neuron-aware sparse FFN kernels (PowerInfer reading report, Part A section
// 2.3 module 4 and section 4.3): only the rows of active neurons are read,
// straight from the dense neuron-major weights, with no sparse format.
//
//   k_up_act    a_j = act(W_up[i].x + b_up_i [, W_gate[i].x + b_gate_i]),  i = idx[j]
//   k_down_acc  y   = sum_j a_j * W_down[i, :]
//
// The active count stays on the device; both kernels read it and stride over
// the list, so no host round trip separates prediction from the FFN.
#include "common.hpp"
#include "internal.hpp"

namespace pi {

// The active count and ids come from device memory; a count outside [0, ffn]
// (the compaction's -1 error marker included) or an id outside [0, ffn) is
// clamped so that no input can make the kernels read outside the weights.
__device__ __forceinline__ int clamp_count(int c, int ffn) { return c < 0 ? 0 : (c > ffn ? ffn : c); }
__device__ __forceinline__ int clamp_row(int i, int ffn) { return i < 0 ? 0 : (i >= ffn ? ffn - 1 : i); }

// ---------------------------------------------------------------------------
// Gathered up(/gate) GEMV.  One wave per active neuron: the row (d fp16) is
// streamed 1 KB per step, 8 steps in flight per lane, against x held in LDS.
// Workgroup 0 of each token also zeroes that token's arrival counters for
// the accumulate kernel that follows on the stream.
template <bool REGLU, bool DENSE>
__global__ __launch_bounds__(256) void k_up_act(const h16* __restrict__ x, int d, int ffn,
                                                const h16* __restrict__ Wup,
                                                const float* __restrict__ bup,
                                                const h16* __restrict__ Wg,
                                                const float* __restrict__ bg,
                                                const int32_t* __restrict__ idx,
                                                const int32_t* __restrict__ count,
                                                float* __restrict__ a, uint32_t* __restrict__ ctr,
                                                int T) {
    extern __shared__ u32x4 sx[];
    const int tok = blockIdx.y;
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i < T; i += 256) ctr[(size_t)tok * T + i] = 0u;
    const int nch = d >> 3;
    for (int i = threadIdx.x; i < nch; i += 256) sx[i] = ld16(x + (size_t)tok * d + (size_t)i * 8);
    __syncthreads();

    const int cnt = DENSE ? ffn : clamp_count(count[tok], ffn);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int32_t* ip = idx + (size_t)tok * ffn;
    for (int j = blockIdx.x * 4 + wave; j < cnt; j += gridDim.x * 4) {
        const int i = DENSE ? j : clamp_row(ip[j], ffn);
        const h16* ru = Wup + (size_t)i * d;
        const h16* rg = REGLU ? Wg + (size_t)i * d : nullptr;
        float au = 0.f, ag = 0.f;
        for (int c0 = lane; c0 < nch; c0 += 64 * 8) {
            u32x4 wu[8], wg[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int c = c0 + u * 64;
                if (c < nch) {
                    wu[u] = ld16_stream(ru + (size_t)c * 8);
                    if (REGLU) wg[u] = ld16_stream(rg + (size_t)c * 8);
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int c = c0 + u * 64;
                if (c < nch) {
                    const u32x4 xv = sx[c];
                    au = dot8_h(wu[u], xv, au);
                    if (REGLU) ag = dot8_h(wg[u], xv, ag);
                }
            }
        }
        au = group_sum<64>(au);
        if (REGLU) ag = group_sum<64>(ag);
        if (lane == 0) {
            const float uval = au + (bup ? bup[i] : 0.f);
            float act;
            if (REGLU)
                act = fmaxf(ag + (bg ? bg[i] : 0.f), 0.f) * uval;
            else
                act = fmaxf(uval, 0.f);
            a[(size_t)tok * ffn + j] = act;
        }
    }
}

// ---------------------------------------------------------------------------
// W_down accumulate.  Grid = (column tiles, neuron chunks, tokens).  A
// workgroup of 128 threads owns 1024 output columns (8 per thread) and a
// contiguous slice of the active list; each active row contributes one
// coalesced 2 KB segment.  Per-chunk partial sums go to the workspace; the
// last chunk of a column tile to arrive (atomic arrival counter) adds the
// partials in chunk order and writes y, so the result does not depend on
// scheduling, and resets the counter.
template <bool DENSE>
__global__ __launch_bounds__(kDownThreads) void k_down_acc(const h16* __restrict__ Wd, int d,
                                                           int ffn,
                                                           const int32_t* __restrict__ idx,
                                                           const int32_t* __restrict__ count,
                                                           const float* __restrict__ a,
                                                           float* __restrict__ y,
                                                           float* __restrict__ partial,
                                                           uint32_t* __restrict__ ctr, int T,
                                                           int G) {
    __shared__ int s_last;
    const int tile = blockIdx.x, chunk = blockIdx.y, tok = blockIdx.z;
    const int cnt = DENSE ? ffn : clamp_count(count[tok], ffn);
    const int per = (cnt + G - 1) / G;
    const int j0 = min(cnt, chunk * per), j1 = min(cnt, j0 + per);
    const int col = tile * kDownCols + threadIdx.x * 8;
    const bool on = col < d;
    const int32_t* ip = idx + (size_t)tok * ffn;
    const float* ap = a + (size_t)tok * ffn;

    float acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.f;
    if (on) {
        int j = j0;
        for (; j + 8 <= j1; j += 8) {
            u32x4 w[8];
            float s[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = DENSE ? j + u : clamp_row(ip[j + u], ffn);
                w[u] = ld16_stream(Wd + (size_t)i * d + col);
                s[u] = ap[j + u];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) axpy8(acc, s[u], w[u]);
        }
        for (; j < j1; ++j) {
            const int i = DENSE ? j : clamp_row(ip[j], ffn);
            axpy8(acc, ap[j], ld16_stream(Wd + (size_t)i * d + col));
        }
        float* pp = partial + ((size_t)tok * G + chunk) * d + col;
        *reinterpret_cast<f32x4*>(pp) = f32x4{acc[0], acc[1], acc[2], acc[3]};
        *reinterpret_cast<f32x4*>(pp + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0)
        s_last = fetch_add_acq_rel(&ctr[(size_t)tok * T + tile], 1u) == (uint32_t)(G - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    if (on) {
        float sum[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) sum[k] = 0.f;
        const float* q = partial + (size_t)tok * G * d + col;
        for (int g = 0; g < G; ++g) {
            const f32x4 v0 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(q + (size_t)g * d));
            const f32x4 v1 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(q + (size_t)g * d + 4));
            sum[0] += v0.x; sum[1] += v0.y; sum[2] += v0.z; sum[3] += v0.w;
            sum[4] += v1.x; sum[5] += v1.y; sum[6] += v1.z; sum[7] += v1.w;
        }
        float* yp = y + (size_t)tok * d + col;
        *reinterpret_cast<f32x4*>(yp) = f32x4{sum[0], sum[1], sum[2], sum[3]};
        *reinterpret_cast<f32x4*>(yp + 4) = f32x4{sum[4], sum[5], sum[6], sum[7]};
    }
    if (threadIdx.x == 0) ctr[(size_t)tok * T + tile] = 0u;
}

hipError_t launch_up_act(bool reglu, bool dense, const h16* x, int B, int d, int ffn,
                         const h16* Wup, const float* bup, const h16* Wg, const float* bg,
                         const int32_t* idx, const int32_t* count, float* a, uint32_t* ctr,
                         int T, hipStream_t s) {
    int gx = (ffn + 3) / 4;
    if (gx > 1024) gx = 1024;
    dim3 grid(gx, B);
    const size_t shm = (size_t)d * 2;
#define PI_UP(R, D)                                                                          \
    hipLaunchKernelGGL((k_up_act<R, D>), grid, dim3(256), shm, s, x, d, ffn, Wup, bup, Wg, bg, \
                       idx, count, a, ctr, T)
    if (reglu) {
        if (dense) PI_UP(true, true); else PI_UP(true, false);
    } else {
        if (dense) PI_UP(false, true); else PI_UP(false, false);
    }
#undef PI_UP
    return hipGetLastError();
}

hipError_t launch_down_acc(bool dense, const h16* Wd, int B, int d, int ffn, const int32_t* idx,
                           const int32_t* count, const float* a, float* y, float* partial,
                           uint32_t* ctr, int T, int G, hipStream_t s) {
    dim3 grid(T, G, B);
    if (dense)
        hipLaunchKernelGGL(k_down_acc<true>, grid, dim3(kDownThreads), 0, s, Wd, d, ffn, idx, count,
                           a, y, partial, ctr, T, G);
    else
        hipLaunchKernelGGL(k_down_acc<false>, grid, dim3(kDownThreads), 0, s, Wd, d, ffn, idx,
                           count, a, y, partial, ctr, T, G);
    return hipGetLastError();
}

}  // namespace pi
