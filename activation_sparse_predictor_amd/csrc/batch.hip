// Batched decode (B >= 2 tokens): the union of the tokens' active lists is
// loaded once and multiplied on the matrix cores (PowerInfer reading report,
// Part A section 4.4: the gain falls as the batch grows because the tokens'
// active sets overlap less than fully; the union is what must be read).
//
//   k_union_clear / k_union_mark   per-neuron token bitmask from the lists
//   k_union_compact                ascending union list U, |U|, masks per entry
//   k_union_up      (MFMA)         A[u][t] = W_up[U_u].x_t (+ gate), bias,
//                                  activation, zeroed where t did not select U_u
//   k_union_down    (MFMA)         Y[t] = sum_u A[u][t] * W_down[U_u, :]
//
// Each token's result equals its single-token result up to fp32 rounding:
// a neuron outside a token's own list contributes exactly 0 to that token.
// A is kept as an fp16 pair (hi + lo, about 22 significant bits) so that the
// fp16 matrix-core down product loses no accuracy against fp32 activations.
#include "common.hpp"
#include "internal.hpp"

namespace pi {

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_union_clear(uint32_t* __restrict__ tmask, size_t n,
                                                     uint32_t* __restrict__ ctr) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) tmask[i] = 0u;
    if (blockIdx.x == 0 && threadIdx.x <= kArriveGroups) ctr[threadIdx.x * kCtrStride] = 0u;
}

// tmask[i * W + t / 32] has bit t % 32 set when token t selected neuron i.
__global__ __launch_bounds__(256) void k_union_mark(const int32_t* __restrict__ idx,
                                                    const int32_t* __restrict__ count, int ffn, int W,
                                                    uint32_t* __restrict__ tmask) {
    const int t = blockIdx.y;
    const int cnt = clampi(count[t], 0, ffn);
    for (int j = blockIdx.x * 256 + threadIdx.x; j < cnt; j += gridDim.x * 256) {
        const int i = clampi(idx[(size_t)t * ffn + j], 0, ffn - 1);
        atomicOr(&tmask[(size_t)i * W + (t >> 5)], 1u << (t & 31));
    }
}

// Union compaction: each wave turns 64 neurons into one bitmap (any token
// selected the neuron), published with a coherent store; workgroups arrive on
// a two-level counter and the last one scans the bitmaps in neuron order and
// writes the ascending union list, each entry's token mask and |U|.
__global__ __launch_bounds__(256) void k_union_compact(const uint32_t* __restrict__ tmask, int ffn, int W,
                                                       uint64_t* __restrict__ umasks,
                                                       uint32_t* __restrict__ ctr,
                                                       int32_t* __restrict__ ulist,
                                                       uint32_t* __restrict__ umask,
                                                       uint32_t* __restrict__ ucount) {
    __shared__ uint32_t s_part[4];
    __shared__ int s_last;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ntiles = (ffn + 63) / 64;
    const int tile = blockIdx.x * 4 + wave;
    if (tile < ntiles) {
        const int i = tile * 64 + lane;
        bool sel = false;
        if (i < ffn)
            for (int w = 0; w < W; ++w) sel = sel || tmask[(size_t)i * W + w] != 0u;
        const uint64_t m = __ballot(sel);
        if (lane == 0) __hip_atomic_store(&umasks[tile], m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    wait_own_memory();
    __syncthreads();
    if (tid == 0) {
        const int nwg = gridDim.x;
        const int g = blockIdx.x % kArriveGroups;
        const uint32_t n1 = (uint32_t)((nwg - g + kArriveGroups - 1) / kArriveGroups);
        const uint32_t groups = (uint32_t)min(nwg, kArriveGroups);
        bool last = false;
        if (fetch_add(&ctr[g * kCtrStride], 1u) == n1 - 1u)
            last = fetch_add(&ctr[kArriveGroups * kCtrStride], 1u) == groups - 1u;
        s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    uint32_t base = 0;
    for (int t0 = 0; t0 < ntiles; t0 += 1024) {
        uint64_t m4[4];
        uint32_t mine = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int t = t0 + tid * 4 + q;
            m4[q] = t < ntiles ? __hip_atomic_load(&umasks[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
            mine += (uint32_t)__popcll(m4[q]);
        }
        uint32_t incl = mine;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t v = __shfl_up(incl, off, 64);
            if (lane >= off) incl += v;
        }
        if (lane == 63) s_part[wave] = incl;
        __syncthreads();
        uint32_t pos = base + incl - mine;
        for (int w2 = 0; w2 < wave; ++w2) pos += s_part[w2];
        const uint32_t total = s_part[0] + s_part[1] + s_part[2] + s_part[3];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint64_t m = m4[q];
            const int t = t0 + tid * 4 + q;
            while (m) {
                const int i = t * 64 + __builtin_ctzll(m);
                ulist[pos] = i;
                for (int w = 0; w < W; ++w) umask[(size_t)pos * W + w] = tmask[(size_t)i * W + w];
                ++pos;
                m &= m - 1;
            }
        }
        base += total;
        __syncthreads();
    }
    if (tid == 0) *ucount = base;
    if (tid <= kArriveGroups) st_flag(&ctr[tid * kCtrStride], 0u);
}

// ---------------------------------------------------------------------------
// Up GEMM.  A workgroup owns 32 union entries; its 4 waves split K = d in
// quarters and each computes the 32 x 32 products for every 32-token block
// with v_mfma_f32_32x32x8_f16 (lane l: row l%32 of the W block, token l%32
// of the x block, K slice by l/32).  Both operands are K-contiguous in
// memory: a 16-byte load gives a lane 8 values; the two lane halves take the
// two chunks of a chunk pair, and every MFMA sums over both halves' slices.
// The loop runs over whole pairs in unrolled batches of 8, so every lane
// executes the same MFMAs (an odd final chunk is fed as zeros by half 1).
// The quarters are summed in LDS, then bias, activation and the token mask
// give A, stored token-major as hi/lo fp16 pairs: aT[t][u].
constexpr int kUpBatch = 8;   // chunk pairs in flight per lane

template <bool REGLU, int NB>
__global__ __launch_bounds__(256) void k_union_up(const h16* __restrict__ x, int B, int d, int ffn,
                                                  const h16* __restrict__ Wup,
                                                  const float* __restrict__ bup,
                                                  const h16* __restrict__ Wg,
                                                  const float* __restrict__ bg,
                                                  const int32_t* __restrict__ ulist,
                                                  const uint32_t* __restrict__ umask,
                                                  const uint32_t* __restrict__ ucount, int W,
                                                  int Bp, int lda, h16* __restrict__ a_hi,
                                                  h16* __restrict__ a_lo) {
    constexpr int NM = REGLU ? 2 : 1;
    __shared__ float s_red[4][16][64];       // one (matrix, token block) of partial tiles
    __shared__ float s_sum[NM][32][33];      // reduced 32 x 32 block per matrix
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 31, half = lane >> 5;
    const int U = (int)min(*ucount, (uint32_t)ffn);
    const int nrb = (U + 31) / 32;
    const int nch = d >> 3;
    const int npair = nch >> 1;
    const int p0 = (npair * wave) / 4, p1 = (npair * (wave + 1)) / 4;

    auto mfma_pair = [&](f32x16 (&acc)[NM][NB], u32x4 av, u32x4 gv, int c) {
        const f16x8 a8 = __builtin_bit_cast(f16x8, av);
        const f16x4 alo = {a8[0], a8[1], a8[2], a8[3]}, ahi = {a8[4], a8[5], a8[6], a8[7]};
        f16x4 glo = {0, 0, 0, 0}, ghi = {0, 0, 0, 0};
        if (REGLU) {
            const f16x8 g8 = __builtin_bit_cast(f16x8, gv);
            glo = f16x4{g8[0], g8[1], g8[2], g8[3]};
            ghi = f16x4{g8[4], g8[5], g8[6], g8[7]};
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int t = min(nb * 32 + li, B - 1);
            const f16x8 x8 = __builtin_bit_cast(f16x8, ld16(x + (size_t)t * d + (size_t)c * 8));
            const f16x4 xlo = {x8[0], x8[1], x8[2], x8[3]}, xhi = {x8[4], x8[5], x8[6], x8[7]};
            acc[0][nb] = __builtin_amdgcn_mfma_f32_32x32x8f16(alo, xlo, acc[0][nb], 0, 0, 0);
            acc[0][nb] = __builtin_amdgcn_mfma_f32_32x32x8f16(ahi, xhi, acc[0][nb], 0, 0, 0);
            if (REGLU) {
                acc[NM - 1][nb] = __builtin_amdgcn_mfma_f32_32x32x8f16(glo, xlo, acc[NM - 1][nb], 0, 0, 0);
                acc[NM - 1][nb] = __builtin_amdgcn_mfma_f32_32x32x8f16(ghi, xhi, acc[NM - 1][nb], 0, 0, 0);
            }
        }
    };

    for (int rb = blockIdx.x; rb < nrb; rb += gridDim.x) {
        const int u = rb * 32 + li;
        const int row = ulist[min(u, U - 1)];
        const h16* wu = Wup + (size_t)row * d;
        const h16* wg = REGLU ? Wg + (size_t)row * d : Wup;
        f32x16 acc[NM][NB];
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[m][nb] = f32x16{};
        int p = p0;
        for (; p + kUpBatch <= p1; p += kUpBatch) {
            u32x4 av[kUpBatch], gv[kUpBatch];
#pragma unroll
            for (int k = 0; k < kUpBatch; ++k) {
                const int c = 2 * (p + k) + half;
                av[k] = ld16_stream(wu + (size_t)c * 8);
                if (REGLU) gv[k] = ld16_stream(wg + (size_t)c * 8);
            }
#pragma unroll
            for (int k = 0; k < kUpBatch; ++k) mfma_pair(acc, av[k], REGLU ? gv[k] : av[k], 2 * (p + k) + half);
        }
        for (; p < p1; ++p) {
            const int c = 2 * p + half;
            mfma_pair(acc, ld16_stream(wu + (size_t)c * 8), REGLU ? ld16_stream(wg + (size_t)c * 8) : u32x4{}, c);
        }
        if ((nch & 1) && wave == 3) {   // odd chunk count: the last chunk, half 1 feeds zeros
            const int c = nch - 1;
            const u32x4 z = {0u, 0u, 0u, 0u};
            const u32x4 av = half ? z : ld16_stream(wu + (size_t)c * 8);
            const u32x4 gv = (REGLU && !half) ? ld16_stream(wg + (size_t)c * 8) : z;
            // x must be zero where the weight half is zero: feed chunk c for both halves,
            // the zero weights cancel half 1's contribution.
            mfma_pair(acc, av, gv, c);
        }
        // Reduce the K quarters block by block, then apply bias, activation, mask.
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int m = 0; m < NM; ++m) {
#pragma unroll
                for (int e = 0; e < 16; ++e) s_red[wave][e][lane] = acc[m][nb][e];
                __syncthreads();
                // output (row r, token n): element e = (r/8)*4 + r%4, lane n + 32*((r/4)%2)
                for (int o = threadIdx.x; o < 1024; o += 256) {
                    const int r = o >> 5, n = o & 31;
                    const int e = (r >> 3) * 4 + (r & 3), ln = n + 32 * ((r >> 2) & 1);
                    s_sum[m][r][n] = s_red[0][e][ln] + s_red[1][e][ln] + s_red[2][e][ln] + s_red[3][e][ln];
                }
                __syncthreads();
            }
            for (int o = threadIdx.x; o < 1024; o += 256) {
                const int r = o >> 5, n = o & 31;
                const int uu = rb * 32 + r, t = nb * 32 + n;
                if (uu < U && t < Bp) {
                    float av = 0.f;
                    if (t < B && ((umask[(size_t)uu * W + (t >> 5)] >> (t & 31)) & 1u)) {
                        const int nrow = ulist[uu];
                        const float uval = s_sum[0][r][n] + (bup ? bup[nrow] : 0.f);
                        av = REGLU ? fmaxf(s_sum[NM - 1][r][n] + (bg ? bg[nrow] : 0.f), 0.f) * uval
                                   : fmaxf(uval, 0.f);
                    }
                    const h16 hi = (h16)av;
                    a_hi[(size_t)t * lda + uu] = hi;
                    a_lo[(size_t)t * lda + uu] = (h16)(av - (float)hi);
                }
            }
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------------------
// Down GEMM.  Grid = (128-column tiles, G chunks of the union).  Rows of
// W_down are neuron-major, so the contraction index (the union entry) runs
// across rows: each stage of 128 union rows x 128 columns is loaded with
// coalesced 16-byte loads into registers, written to LDS, and the next
// stage's loads are issued before the current one is multiplied, so one
// 32 KB stage per workgroup is always in flight.  The MFMA operand (4
// consecutive union rows of one column per lane) is read back from LDS.
// Wave w owns columns 32w..32w+31 of the tile; A (hi and lo) is the other
// operand, 4 consecutive union entries of one token per lane.  Chunk
// partials go to the workspace with coherent stores; the last chunk of a
// column tile to arrive sums them in chunk order and writes Y.
constexpr int kDnCols = 128;
constexpr int kDnStage = 128;
constexpr int kDnIds = 4096;   // union entries per chunk staged in LDS (G is sized for it)

template <int NB>
__global__ __launch_bounds__(256) void k_union_down(const h16* __restrict__ Wd, int d, int ffn,
                                                    const int32_t* __restrict__ ulist,
                                                    const uint32_t* __restrict__ ucount,
                                                    const h16* __restrict__ a_hi,
                                                    const h16* __restrict__ a_lo, int Bp, int lda,
                                                    float* __restrict__ partial, int G) {
    __shared__ h16 s_w[kDnStage][kDnCols + 8];   // padded rows
    __shared__ int32_t s_ids[kDnIds];
    const int tile = blockIdx.x, chunk = blockIdx.y;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 31, half = lane >> 5;
    const int U = (int)min(*ucount, (uint32_t)ffn);
    // chunk starts are multiples of 8 so the 4-entry A loads stay 8-byte aligned
    const int per = min((((U + G - 1) / G) + 7) & ~7, kDnIds);
    const int u0 = min(U, chunk * per), u1 = min(U, u0 + per);
    const int n_ids = u1 - u0;
    const int c0 = tile * kDnCols;
    for (int i = tid; i < n_ids; i += 256) s_ids[i] = ulist[u0 + i];
    __syncthreads();

    f32x16 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16{};

    // staging map: thread -> rows tid/16 + 16*k (k < 8), 8 columns at 8*(tid%16)
    const int sr = tid >> 4, sc = (tid & 15) * 8;
    const bool col_ok = c0 + sc < d;
    u32x4 v[8];
    auto issue = [&](int s0) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int rr = s0 + sr + 16 * k;   // chunk-relative union row
            v[k] = (rr < n_ids && col_ok) ? ld16_stream(Wd + (size_t)s_ids[rr] * d + c0 + sc)
                                          : u32x4{0u, 0u, 0u, 0u};
        }
    };
    if (n_ids > 0) issue(0);
    const int col = wave * 32 + li;   // column within the tile
    for (int s0 = 0; s0 < n_ids; s0 += kDnStage) {
        __syncthreads();   // the previous stage is no longer read from LDS
#pragma unroll
        for (int k = 0; k < 8; ++k) *reinterpret_cast<u32x4*>(&s_w[sr + 16 * k][sc]) = v[k];
        __syncthreads();
        if (s0 + kDnStage < n_ids) issue(s0 + kDnStage);
        const int sn = min(kDnStage, n_ids - s0);
        for (int kk = 0; kk < sn; kk += 8) {
            const int kr = kk + 4 * half;     // this lane's 4 union rows: kr .. kr+3 (zero rows past sn)
            const f16x4 wv = {s_w[kr][col], s_w[kr + 1][col], s_w[kr + 2][col], s_w[kr + 3][col]};
            const int ue = u0 + s0 + kr;      // union entries ue .. ue+3
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int t = nb * 32 + li;
                const size_t off = (size_t)t * lda + ue;
                f16x4 ah = {0, 0, 0, 0}, al = {0, 0, 0, 0};
                if (ue + 3 < u1) {
                    ah = *reinterpret_cast<const f16x4*>(a_hi + off);
                    al = *reinterpret_cast<const f16x4*>(a_lo + off);
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (ue + q < u1) { ah[q] = a_hi[off + q]; al[q] = a_lo[off + q]; }
                }
                acc[nb] = __builtin_amdgcn_mfma_f32_32x32x8f16(wv, ah, acc[nb], 0, 0, 0);
                acc[nb] = __builtin_amdgcn_mfma_f32_32x32x8f16(wv, al, acc[nb], 0, 0, 0);
            }
        }
    }
    // acc[nb] element e of lane l: column wave*32 + 8*(e/4) + 4*half + e%4, token nb*32 + li
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int t = nb * 32 + li;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int cc = c0 + wave * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
            if (cc < d) partial[((size_t)chunk * Bp + t) * d + cc] = acc[nb][e];
        }
    }
}

// y[t][c] = sum over chunks g (in order) of partial[g][t][c]: one output per
// thread, the G loads issued 8 at a time.
__global__ __launch_bounds__(256) void k_union_reduce(const float* __restrict__ partial, int B, int Bp,
                                                      int d, int G, float* __restrict__ y) {
    const size_t o = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (o >= (size_t)B * d) return;
    const int t = (int)(o / d), c = (int)(o % d);
    float sum = 0.f;
    for (int g0 = 0; g0 < G; g0 += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = (g0 + u < G) ? partial[((size_t)(g0 + u) * Bp + t) * d + c] : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) sum += v[u];
    }
    y[o] = sum;
}

hipError_t launch_union(bool reglu, const h16* x, int B, int d, int ffn, const h16* Wup,
                        const float* bup, const h16* Wg, const float* bg, const h16* Wd,
                        const int32_t* idx, const int32_t* count, float* y, const BatchLayout& L,
                        char* ws, hipStream_t s) {
    uint32_t* tmask = reinterpret_cast<uint32_t*>(ws + L.tmask);
    uint64_t* umasks = reinterpret_cast<uint64_t*>(ws + L.umasks);
    uint32_t* umask = reinterpret_cast<uint32_t*>(ws + L.umask);
    int32_t* ulist = reinterpret_cast<int32_t*>(ws + L.ulist);
    uint32_t* ucount = reinterpret_cast<uint32_t*>(ws + L.ucount);
    h16* a_hi = reinterpret_cast<h16*>(ws + L.a_hi);
    h16* a_lo = reinterpret_cast<h16*>(ws + L.a_lo);
    float* partial = reinterpret_cast<float*>(ws + L.partial);
    uint32_t* ctr = reinterpret_cast<uint32_t*>(ws + L.ctr);
    const size_t nmask = (size_t)ffn * L.W;
    int gclear = (int)((nmask + 255) / 256);
    if (gclear > 2048) gclear = 2048;
    hipLaunchKernelGGL(k_union_clear, dim3(gclear), dim3(256), 0, s, tmask, nmask, ctr);
    int gm = (ffn + 255) / 256;
    if (gm > 64) gm = 64;
    hipLaunchKernelGGL(k_union_mark, dim3(gm, B), dim3(256), 0, s, idx, count, ffn, L.W, tmask);
    const int ntiles = (ffn + 63) / 64;
    hipLaunchKernelGGL(k_union_compact, dim3((ntiles + 3) / 4), dim3(256), 0, s, tmask, ffn, L.W, umasks,
                       ctr, ulist, umask, ucount);
    int gu = (ffn + 31) / 32;
    if (gu > 1024) gu = 1024;
#define PI_UP(R, N)                                                                                  \
    hipLaunchKernelGGL((k_union_up<R, N>), dim3(gu), dim3(256), 0, s, x, B, d, ffn, Wup, bup, Wg, bg, \
                       ulist, umask, ucount, L.W, L.Bp, L.lda, a_hi, a_lo)
#define PI_DN(N)                                                                                     \
    hipLaunchKernelGGL((k_union_down<N>), dim3(L.T, L.G), dim3(256), 0, s, Wd, d, ffn, ulist, ucount, \
                       a_hi, a_lo, L.Bp, L.lda, partial, L.G)
    const int NB = L.Bp / 32;
    if (reglu) {
        if (NB == 1) PI_UP(true, 1); else if (NB == 2) PI_UP(true, 2); else if (NB == 3) PI_UP(true, 3); else PI_UP(true, 4);
    } else {
        if (NB == 1) PI_UP(false, 1); else if (NB == 2) PI_UP(false, 2); else if (NB == 3) PI_UP(false, 3); else PI_UP(false, 4);
    }
    if (NB == 1) PI_DN(1); else if (NB == 2) PI_DN(2); else if (NB == 3) PI_DN(3); else PI_DN(4);
#undef PI_UP
#undef PI_DN
    const size_t nout = (size_t)B * d;
    hipLaunchKernelGGL(k_union_reduce, dim3((unsigned)((nout + 255) / 256)), dim3(256), 0, s, partial, B, L.Bp,
                       d, L.G, y);
    return hipGetLastError();
}

}  // namespace pi
