// INT4 neuron rows: group-wise 4-bit weights for W_up, W_gate and W_down.
//
// Format (this library's own).  A row of d weights (d % 64 == 0) is cut into
// groups of 64.  Group g has one fp16 scale s = fp16(max|w| / 7) and its
// weights are q = clamp(rint(w / s), -8, 7) (rint: round half to even; q = 0
// when s = 0), stored offset by 8 as 4-bit codes, two per byte: element e of
// the row is the low nibble of byte e / 2 when e is even, the high nibble
// when odd.  The dequantised weight is (code - 8) * s, exactly representable
// in fp32.  A row therefore takes d / 2 bytes of codes and d / 32 bytes of
// scales: 3.9x fewer bytes than fp16 for an active neuron's row.
//
// The quantiser runs one thread per (row, group).  The FFN kernels mirror
// the staged fp16 pair (k_up_act, k_down_acc): one wave per listed neuron for
// the up (and gate) rows, then a column-tiled W_down accumulate whose tile
// chunks are added in a fixed order, so results are deterministic.
#include "common.hpp"
#include "internal.hpp"

namespace pi {

constexpr int kQGroup = 64;   // weights per scale

__global__ __launch_bounds__(256) void k_quantize_rows(const h16* __restrict__ W, int rows, int d,
                                                       uint8_t* __restrict__ q, h16* __restrict__ s) {
    const int ng = d / kQGroup;
    const long long n = (long long)rows * ng;
    for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < n; e += (long long)gridDim.x * 256) {
        const int row = (int)(e / ng), g = (int)(e % ng);
        const h16* src = W + (size_t)row * d + (size_t)g * kQGroup;
        u32x4 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = ld16(src + k * 8);
        float w[kQGroup];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t u[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f16x2 p = as_h2(u[j]);
                w[k * 8 + 2 * j] = (float)p.x;
                w[k * 8 + 2 * j + 1] = (float)p.y;
            }
        }
        float amax = 0.f;
#pragma unroll
        for (int k = 0; k < kQGroup; ++k) amax = fmaxf(amax, fabsf(w[k]));
        const h16 sh = (h16)(amax / 7.0f);   // IEEE division, then round to nearest even fp16
        const float sf = (float)sh;
        uint32_t out[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            uint32_t word = 0u;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                int c = 0;
                if (sf != 0.f) c = (int)fminf(fmaxf(rintf(w[k * 8 + j] / sf), -8.f), 7.f);
                word |= (uint32_t)(c + 8) << (4 * j);
            }
            out[k] = word;
        }
        uint32_t* dst = reinterpret_cast<uint32_t*>(q + (size_t)row * (d / 2) + (size_t)g * (kQGroup / 2));
#pragma unroll
        for (int k = 0; k < 8; k += 4) *reinterpret_cast<u32x4*>(dst + k) = u32x4{out[k], out[k + 1], out[k + 2], out[k + 3]};
        s[(size_t)row * ng + g] = sh;
    }
}

// Up (and gate) rows: one wave per listed neuron.  Lane l takes the 16-byte
// code chunks l + 64 u of the row (32 weights each, half a group), with the
// chunk's scale; the chunk's products are summed in fp32 and then scaled.
template <int KIND, bool DENSE>
__global__ __launch_bounds__(256) void k_up_act_q4(const h16* __restrict__ x, int d, int ffn,
                                                   const uint8_t* __restrict__ qu, const h16* __restrict__ su,
                                                   const float* __restrict__ bup, const uint8_t* __restrict__ qg,
                                                   const h16* __restrict__ sg, const float* __restrict__ bg,
                                                   const int32_t* __restrict__ idx, const int32_t* __restrict__ count,
                                                   float* __restrict__ a, uint32_t* __restrict__ ctr, int T) {
    extern __shared__ u32x4 sx[];
    constexpr bool GATED = KIND != 0;
    constexpr int U = 4;   // chunks in flight per lane and matrix: a row of 8192 weights in one round
    const int tok = blockIdx.y;
    const int tid = threadIdx.x;
    if (blockIdx.x == 0)
        for (int i = tid; i < T; i += 256) ctr[((size_t)tok * T + i) * kCtrStride] = 0u;
    const int nch = d >> 3;    // 8-weight x chunks in LDS
    const int ncq = d >> 5;    // 32-weight code chunks per row
    const int ng = d / kQGroup;
    const int cnt = DENSE ? ffn : clamp_count(count[tok], ffn);
    const int wave = tid >> 6, lane = tid & 63;
    const int32_t* ip = idx + (size_t)tok * ffn;
    for (int k = tid; k < nch; k += 256) sx[k] = ld16(x + (size_t)tok * d + (size_t)k * 8);
    __syncthreads();
    for (int j = blockIdx.x * 4 + wave; j < cnt; j += gridDim.x * 4) {
        const int i = DENSE ? j : clamp_row(ip[j], ffn);
        const uint8_t* ru = qu + (size_t)i * (d / 2);
        const uint8_t* rg = GATED ? qg + (size_t)i * (d / 2) : nullptr;
        float au = 0.f, ag = 0.f;
        for (int c0 = lane; c0 < ncq; c0 += 64 * U) {
            u32x4 wu[U], wg[U];
            float cu[U], cg[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = min(c0 + u * 64, ncq - 1);   // a clamped slot is loaded but not used
                wu[u] = ld16_stream(ru + (size_t)c * 16);
                cu[u] = (float)su[(size_t)i * ng + (c >> 1)];
                if (GATED) {
                    wg[u] = ld16_stream(rg + (size_t)c * 16);
                    cg[u] = (float)sg[(size_t)i * ng + (c >> 1)];
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * 64;
                if (c < ncq) {
                    const uint32_t qw[4] = {wu[u].x, wu[u].y, wu[u].z, wu[u].w};
                    float pu = 0.f, pg = 0.f;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const u32x4 xv = sx[c * 4 + k];
                        pu = dot8_q4(qw[k], xv, pu);
                        if (GATED) {
                            const uint32_t gw[4] = {wg[u].x, wg[u].y, wg[u].z, wg[u].w};
                            pg = dot8_q4(gw[k], xv, pg);
                        }
                    }
                    au = fmaf(cu[u], pu, au);
                    if (GATED) ag = fmaf(cg[u], pg, ag);
                }
            }
        }
        au = group_sum<64>(au);
        if (GATED) ag = group_sum<64>(ag);
        if (lane == 0) {
            const float uval = au + (bup ? bup[i] : 0.f);
            const float gval = GATED ? ag + (bg ? bg[i] : 0.f) : 0.f;
            a[(size_t)tok * ffn + j] = ffn_act<KIND>(uval, gval);
        }
    }
}

// W_down accumulate over INT4 rows.  Grid = (column tiles, neuron chunks,
// tokens), 1024 threads: 128 column threads x 8 columns (one 32-bit code word
// and one scale per row, 16 rows in flight) and 8 row groups taking every 8th
// row of the chunk's slice; the row groups are summed in LDS, the chunk partials in
// chunk order by the tile's last chunk to arrive.
template <bool DENSE>
__global__ __launch_bounds__(kDownThreads) void k_down_acc_q4(const uint8_t* __restrict__ qd,
                                                              const h16* __restrict__ sd, int d, int ffn,
                                                              const int32_t* __restrict__ idx,
                                                              const int32_t* __restrict__ count,
                                                              const float* __restrict__ a, float* __restrict__ y,
                                                              float* __restrict__ partial, uint32_t* __restrict__ ctr,
                                                              int T, int G) {
    __shared__ float s_red[kDownGroups][kDownCols];
    __shared__ int32_t s_row[kDownWindow];
    __shared__ float s_act[kDownWindow];
    __shared__ int s_last;
    const int tile = blockIdx.x, chunk = blockIdx.y, tok = blockIdx.z;
    const int tid = threadIdx.x;
    const int cnt = DENSE ? ffn : clamp_count(count[tok], ffn);
    const int per = (cnt + G - 1) / G;
    const int j0 = min(cnt, chunk * per), j1 = min(cnt, j0 + per);
    const int ct = tid % kDownColThreads;
    const int rg = tid / kDownColThreads;
    const int lcol = ct * 8;
    const int col = tile * kDownCols + lcol;
    const int ng = d / kQGroup;
    const int32_t* ip = idx + (size_t)tok * ffn;
    const float* ap = a + (size_t)tok * ffn;
    float acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.f;
    for (int w0 = j0; w0 < j1; w0 += kDownWindow) {
        const int wn = min(kDownWindow, j1 - w0);
        if (tid < wn) {
            s_row[tid] = DENSE ? w0 + tid : clamp_row(ip[w0 + tid], ffn);
            s_act[tid] = ap[w0 + tid];
        }
        __syncthreads();
        if (col < d) {
            for (int k0 = rg; k0 < wn; k0 += 16 * kDownGroups) {
                uint32_t w[16];
                float sc[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int r = s_row[min(k0 + u * kDownGroups, wn - 1)];
                    w[u] = *reinterpret_cast<const uint32_t*>(qd + (size_t)r * (d / 2) + col / 2);
                    sc[u] = (float)sd[(size_t)r * ng + col / kQGroup];
                }
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int k = k0 + u * kDownGroups;
                    if (k < wn) {
                        const float f = s_act[k] * sc[u];
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            acc[e] = fmaf(f, (float)((int)((w[u] >> (4 * e)) & 0xFu) - 8), acc[e]);
                    }
                }
            }
        }
        __syncthreads();
    }
    *reinterpret_cast<f32x4*>(&s_red[rg][lcol]) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4*>(&s_red[rg][lcol + 4]) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    __syncthreads();
    const int gc = tile * kDownCols + tid;
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

hipError_t launch_quantize_rows(const h16* W, int rows, int d, uint8_t* q, h16* s, hipStream_t st) {
    const long long n = (long long)rows * (d / kQGroup);
    long long g = (n + 255) / 256;
    if (g > 4096) g = 4096;
    if (g < 1) g = 1;
    hipLaunchKernelGGL(k_quantize_rows, dim3((unsigned)g), dim3(256), 0, st, W, rows, d, q, s);
    return hipGetLastError();
}

hipError_t launch_ffn_q4(int kind, bool dense, const h16* x, int B, int d, int ffn, const uint8_t* qu,
                         const h16* su, const float* bup, const uint8_t* qg, const h16* sg, const float* bg,
                         const uint8_t* qd, const h16* sd, const int32_t* idx, const int32_t* count, float* y,
                         const SparseLayout& L, char* data, hipStream_t s) {
    float* a = reinterpret_cast<float*>(data + L.a);
    float* partial = reinterpret_cast<float*>(data + L.partial);
    uint32_t* ctr = reinterpret_cast<uint32_t*>(data + L.ctr);
    int gx = (ffn + 3) / 4;
    if (gx > 1024) gx = 1024;
    const dim3 gu(gx, B);
    const size_t shm = (size_t)d * 2;
#define PI_UQ(K, D) hipLaunchKernelGGL((k_up_act_q4<K, D>), gu, dim3(256), shm, s, x, d, ffn, qu, su, bup, qg, sg, bg, \
                                       idx, count, a, ctr, L.T)
    if (kind == 2) { if (dense) PI_UQ(2, true); else PI_UQ(2, false); }
    else if (kind == 1) { if (dense) PI_UQ(1, true); else PI_UQ(1, false); }
    else { if (dense) PI_UQ(0, true); else PI_UQ(0, false); }
#undef PI_UQ
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 gd(L.T, L.G, B);
    if (dense)
        hipLaunchKernelGGL(k_down_acc_q4<true>, gd, dim3(kDownThreads), 0, s, qd, sd, d, ffn, idx, count, a, y,
                           partial, ctr, L.T, L.G);
    else
        hipLaunchKernelGGL(k_down_acc_q4<false>, gd, dim3(kDownThreads), 0, s, qd, sd, d, ffn, idx, count, a, y,
                           partial, ctr, L.T, L.G);
    return hipGetLastError();
}

}  // namespace pi
