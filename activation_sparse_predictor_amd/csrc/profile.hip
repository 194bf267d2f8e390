// Offline profiler and reorder plumbing (PowerInfer reading report, Part A
// section 2.2 "offline profiling", section 2.3 module 1 and neuron impact
// v_i = f_i): count, per neuron, the calibration tokens whose ReLU input is
// positive, then apply a hot-first row order to the weights.
//
//   k_profile  counts[i] += #{t : W[i].X_t + b_i > 0}   (fp16 MFMA, fp32 accumulate)
//   k_permute  dst[j, :] = src[perm[j], :]
#include "common.hpp"
#include "internal.hpp"

namespace pi {

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// v_mfma_f32_32x32x8_f16 operand layout (wave64): lane l supplies row l%32 of
// the A block and column l%32 of the B block, with the K slice selected by
// l/32; the 32x32 fp32 result gives lane l column l%32 and rows
// 8*(e/4) + 4*(l/32) + e%4 for its 16 values e.  A and B use the same K
// slices, so any consistent assignment of K values to (lane half, element)
// yields the same dot products; the kernel loads 8 consecutive K values per
// lane and feeds them as two MFMA steps.
//
// Tile: a wave computes 32 neurons x 64 tokens (two accumulators sharing the
// W fragment); a workgroup of 4 waves covers 64 neurons x 128 tokens.  The
// epilogue turns each fp32 pre-activation into a predicate, ballots it, and
// adds one popcount per neuron per wave with a device atomic.
__global__ __launch_bounds__(256) void k_profile(const h16* __restrict__ X, int n, int d, int ffn,
                                                 const h16* __restrict__ W,
                                                 const float* __restrict__ b,
                                                 uint32_t* __restrict__ counts) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nb = blockIdx.x * 64 + (wave & 1) * 32;
    const int tb = blockIdx.y * 128 + (wave >> 1) * 64;
    const int li = lane & 31, half = lane >> 5;
    const int wrow = min(nb + li, ffn - 1);
    const int t0 = min(tb + li, n - 1), t1 = min(tb + 32 + li, n - 1);
    const h16* wp = W + (size_t)wrow * d;
    const h16* xp0 = X + (size_t)t0 * d;
    const h16* xp1 = X + (size_t)t1 * d;

    f32x16 acc0 = {}, acc1 = {};
    int k = 0;
    for (; k + 64 <= d; k += 64) {
        u32x4 aw[4], bx0[4], bx1[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int kk = k + u * 16 + half * 8;
            aw[u] = ld16(wp + kk);
            bx0[u] = ld16(xp0 + kk);
            bx1[u] = ld16(xp1 + kk);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const f16x8 a8 = __builtin_bit_cast(f16x8, aw[u]);
            const f16x8 p8 = __builtin_bit_cast(f16x8, bx0[u]);
            const f16x8 q8 = __builtin_bit_cast(f16x8, bx1[u]);
            const f16x4 alo = {a8[0], a8[1], a8[2], a8[3]}, ahi = {a8[4], a8[5], a8[6], a8[7]};
            const f16x4 plo = {p8[0], p8[1], p8[2], p8[3]}, phi = {p8[4], p8[5], p8[6], p8[7]};
            const f16x4 qlo = {q8[0], q8[1], q8[2], q8[3]}, qhi = {q8[4], q8[5], q8[6], q8[7]};
            acc0 = __builtin_amdgcn_mfma_f32_32x32x8f16(alo, plo, acc0, 0, 0, 0);
            acc0 = __builtin_amdgcn_mfma_f32_32x32x8f16(ahi, phi, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x8f16(alo, qlo, acc1, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x8f16(ahi, qhi, acc1, 0, 0, 0);
        }
    }
    for (; k < d; k += 8) {  // d % 8 == 0: 8 K values per MFMA, 4 per lane
        const int kk = k + half * 4;
        const f16x4 a4 = *reinterpret_cast<const f16x4*>(wp + kk);
        const f16x4 p4 = *reinterpret_cast<const f16x4*>(xp0 + kk);
        const f16x4 q4 = *reinterpret_cast<const f16x4*>(xp1 + kk);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x8f16(a4, p4, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x8f16(a4, q4, acc1, 0, 0, 0);
    }

    const bool tok0_ok = tb + li < n, tok1_ok = tb + 32 + li < n;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int i = nb + 8 * (e / 4) + 4 * half + (e % 4);
        const float bias = (b && i < ffn) ? b[i] : 0.f;
        const uint64_t m0 = __ballot(tok0_ok && (acc0[e] + bias > 0.f));
        const uint64_t m1 = __ballot(tok1_ok && (acc1[e] + bias > 0.f));
        const uint32_t c = (uint32_t)__popcll(half ? (m0 >> 32) : (m0 & 0xffffffffull)) +
                           (uint32_t)__popcll(half ? (m1 >> 32) : (m1 & 0xffffffffull));
        if (li == 0 && i < ffn && c) fetch_add(&counts[i], c);
    }
}

// Row gather with 16-byte (or 4-byte) granularity; one workgroup per row,
// rows strided over the grid.  An out-of-range perm entry leaves its
// destination row untouched instead of reading out of bounds.
template <typename V>
__global__ __launch_bounds__(256) void k_permute(const V* __restrict__ src, V* __restrict__ dst,
                                                 int rows, int vec_per_row,
                                                 const int32_t* __restrict__ perm) {
    for (int row = blockIdx.x; row < rows; row += gridDim.x) {
        const int sr = perm[row];
        if (sr < 0 || sr >= rows) continue;
        const V* s = src + (size_t)sr * vec_per_row;
        V* t = dst + (size_t)row * vec_per_row;
        for (int v = threadIdx.x; v < vec_per_row; v += 256) t[v] = s[v];
    }
}

hipError_t launch_profile(const h16* X, int n, int d, int ffn, const h16* W, const float* b,
                          uint32_t* counts, hipStream_t s) {
    dim3 grid((ffn + 63) / 64, (n + 127) / 128);
    hipLaunchKernelGGL(k_profile, grid, dim3(256), 0, s, X, n, d, ffn, W, b, counts);
    return hipGetLastError();
}

hipError_t launch_permute(const void* src, void* dst, int rows, int row_bytes,
                          const int32_t* perm, hipStream_t s) {
    int gx = rows < 65536 ? rows : 65536;
    if (row_bytes % 16 == 0 && ((uintptr_t)src % 16 == 0) && ((uintptr_t)dst % 16 == 0))
        hipLaunchKernelGGL(k_permute<u32x4>, dim3(gx), dim3(256), 0, s,
                           static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), rows,
                           row_bytes / 16, perm);
    else
        hipLaunchKernelGGL(k_permute<uint32_t>, dim3(gx), dim3(256), 0, s,
                           static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst), rows,
                           row_bytes / 4, perm);
    return hipGetLastError();
}

}  // namespace pi
