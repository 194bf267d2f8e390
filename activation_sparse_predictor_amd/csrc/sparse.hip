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

// ---------------------------------------------------------------------------
// Gathered up(/gate) GEMV.  One wave per active neuron: the row (d fp16) is
// streamed 1 KB per step, 16 steps (ReGLU: 8 per matrix) in flight per lane,
// so a d <= 8192 row is requested in one round.  The first row's loads are
// issued before x is staged into LDS, so the staging overlaps them.
// Workgroup 0 of each token also zeroes that token's arrival counters for
// the accumulate kernel that follows on the stream.
template <int KIND, bool DENSE>
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
    constexpr bool REGLU = KIND != 0;   // gated: a W_gate row per neuron (ReGLU, SwiGLU)
    constexpr int U = REGLU ? 8 : 16;
    const int tok = blockIdx.y;
    const int tid = threadIdx.x;
    if (blockIdx.x == 0)
        for (int i = tid; i < T; i += 256) ctr[((size_t)tok * T + i) * kCtrStride] = 0u;
    const int nch = d >> 3;
    const int cnt = DENSE ? ffn : clamp_count(count[tok], ffn);
    const int wave = tid >> 6, lane = tid & 63;
    const int32_t* ip = idx + (size_t)tok * ffn;
    const int stride = gridDim.x * 4;

    int j = blockIdx.x * 4 + wave;
    int i = 0;
    u32x4 wu[U], wg[U];
    auto issue = [&](int c0) {
        const h16* ru = Wup + (size_t)i * d;
        const h16* rg = REGLU ? Wg + (size_t)i * d : nullptr;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * 64;
            if (c < nch) {
                wu[u] = ld16_stream(ru + (size_t)c * 8);
                if (REGLU) wg[u] = ld16_stream(rg + (size_t)c * 8);
            }
        }
    };
    if (j < cnt) {
        i = DENSE ? j : clamp_row(ip[j], ffn);
        issue(lane);
    }
    for (int k = tid; k < nch; k += 256) sx[k] = ld16(x + (size_t)tok * d + (size_t)k * 8);
    __syncthreads();

    bool first = true;
    for (; j < cnt; j += stride) {
        if (!first) {
            i = DENSE ? j : clamp_row(ip[j], ffn);
            issue(lane);
        }
        first = false;
        float au = 0.f, ag = 0.f;
        for (int c0 = lane; c0 < nch; c0 += 64 * U) {
            if (c0 != lane) issue(c0);
#pragma unroll
            for (int u = 0; u < U; ++u) {
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
            const float gval = REGLU ? ag + (bg ? bg[i] : 0.f) : 0.f;
            a[(size_t)tok * ffn + j] = ffn_act<KIND>(uval, gval);
        }
    }
}

// ---------------------------------------------------------------------------
// W_down accumulate.  Grid = (column tiles, neuron chunks, tokens).  A
// workgroup of 1024 threads owns 1024 output columns and a contiguous slice
// of the active list.  The slice's row ids and activations are staged in
// LDS, then 8 row groups of 128 threads each take every 8th row, so a row
// contributes one coalesced 2 KB segment and a thread keeps 8 row loads in
// flight with no dependent global load in between.  The row groups are
// summed in LDS in a fixed order and the chunk's partial goes to the
// workspace through device-coherent stores.  Once its stores have completed,
// one thread per workgroup arrives on the tile's counter (a relaxed atomic on
// its own 128-byte line); the last chunk to arrive adds the G partials in
// chunk order (one column per thread, all loads issued together, read from
// the coherent level), writes y and resets the counter.  The result never
// depends on scheduling, and no L2 write-back is needed.
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
    // Staged list slice, transposed so row group g finds its rows (window
    // entries g, g+8, g+16, ...) contiguous: 8 ids in two 16-byte LDS reads.
    constexpr int kPerGroup = kDownWindow / kDownGroups;
    __shared__ float s_red[kDownGroups][kDownCols];
    __shared__ __align__(16) int32_t s_row[kDownGroups][kPerGroup];
    __shared__ __align__(16) float s_act[kDownGroups][kPerGroup];
    __shared__ int s_last;
    const int tile = blockIdx.x, chunk = blockIdx.y, tok = blockIdx.z;
    const int tid = threadIdx.x;
    const int cnt = DENSE ? ffn : clamp_count(count[tok], ffn);
    const int per = (cnt + G - 1) / G;
    const int j0 = min(cnt, chunk * per), j1 = min(cnt, j0 + per);
    const int ct = tid % kDownColThreads;
    const int rg = __builtin_amdgcn_readfirstlane(tid / kDownColThreads);
    const int lcol = ct * 8;
    const int col = tile * kDownCols + lcol;
    const int32_t* ip = idx + (size_t)tok * ffn;
    const float* ap = a + (size_t)tok * ffn;

    float acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.f;
    for (int w0 = j0; w0 < j1; w0 += kDownWindow) {
        const int wn = min(kDownWindow, j1 - w0);
        if (tid < wn) {
            s_row[tid % kDownGroups][tid / kDownGroups] = DENSE ? w0 + tid : clamp_row(ip[w0 + tid], ffn);
            s_act[tid % kDownGroups][tid / kDownGroups] = ap[w0 + tid];
        }
        __syncthreads();
        const int nk = (wn - rg + kDownGroups - 1) / kDownGroups;  // rows of this group
        if (col < d) {
            for (int k0 = 0; k0 < nk; k0 += 8) {
                const i32x4 r0 = *reinterpret_cast<const i32x4*>(&s_row[rg][k0]);
                const i32x4 r1 = *reinterpret_cast<const i32x4*>(&s_row[rg][k0 + 4]);
                const f32x4 a0 = *reinterpret_cast<const f32x4*>(&s_act[rg][k0]);
                const f32x4 a1 = *reinterpret_cast<const f32x4*>(&s_act[rg][k0 + 4]);
                const int rows[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
                const float s[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                u32x4 w[8];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (k0 + u < nk) w[u] = ld16_stream(Wd + (size_t)rows[u] * d + col);
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (k0 + u < nk) axpy8(acc, s[u], w[u]);
            }
        }
        __syncthreads();
    }
    *reinterpret_cast<f32x4*>(&s_red[rg][lcol]) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4*>(&s_red[rg][lcol + 4]) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    __syncthreads();

    const int gc = tile * kDownCols + tid;  // one output column per thread from here on
    if (gc < d) {
        float v = 0.f;
#pragma unroll
        for (int g = 0; g < kDownGroups; ++g) v += s_red[g][tid];
        st_coherent(&partial[((size_t)tok * G + chunk) * d + gc], v);
    }
    wait_own_memory();
    __syncthreads();
    uint32_t* my_ctr = &ctr[((size_t)tok * T + tile) * kCtrStride];
    if (tid == 0) s_last = fetch_add(my_ctr, 1u) == (uint32_t)(G - 1);
    __syncthreads();
    if (!s_last) return;
    if (gc < d) {
        const float* q = partial + (size_t)tok * G * d + gc;
        float sum = 0.f;
        for (int g0 = 0; g0 < G; g0 += 16) {
            float v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = (g0 + u < G) ? ld_coherent(q + (size_t)(g0 + u) * d) : 0.f;
#pragma unroll
            for (int u = 0; u < 16; ++u) sum += v[u];
        }
        // a negative count is an overrun report of the predictor: answered with NaN
        y[(size_t)tok * d + gc] = (!DENSE && count[tok] < 0) ? __builtin_nanf("") : sum;
    }
    if (tid == 0) st_flag(my_ctr, 0u);
}

hipError_t launch_up_act(int kind, bool dense, const h16* x, int B, int d, int ffn,
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
    if (kind == 2) {
        if (dense) PI_UP(2, true); else PI_UP(2, false);
    } else if (kind == 1) {
        if (dense) PI_UP(1, true); else PI_UP(1, false);
    } else {
        if (dense) PI_UP(0, true); else PI_UP(0, false);
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
