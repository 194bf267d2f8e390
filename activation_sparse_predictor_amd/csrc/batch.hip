// Batched decode (B >= 2 tokens): the union of the tokens' active lists is
// loaded once and multiplied on the matrix cores (PowerInfer reading report,
// Part A section 4.4: the gain falls as the batch grows because the tokens'
// active sets overlap less than fully; the union is what must be read).
//
//   k_union_clear / k_union_mark   per-neuron token bitmask from the lists
//   k_union_compact                ascending union list U and |U|
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
// writes the ascending union list and |U|.
__global__ __launch_bounds__(256) void k_union_compact(const uint32_t* __restrict__ tmask, int ffn, int W,
                                                       uint64_t* __restrict__ umasks,
                                                       uint32_t* __restrict__ ctr,
                                                       int32_t* __restrict__ ulist,
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
                ulist[pos++] = t * 64 + __builtin_ctzll(m);
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
// Rows x tokens on the matrix cores.  A workgroup owns 32 weight rows; its 4
// waves split K in quarters and each computes the 32 x 32 products for every
// 32-token block with v_mfma_f32_32x32x8_f16 (lane l: row l%32 of the
// weight block, token l%32 of the activation block, K slice by l/32).  Both
// operands are K-contiguous in memory: a 16-byte load gives a lane 8 values;
// the two lane halves take the two chunks of a chunk pair, and every MFMA sums
// over both halves' slices.  The loop runs over whole pairs in batches, so
// every lane executes the same MFMAs (an odd final chunk is fed as zero
// weights by half 1).  NM weight matrices share the activation loads (gate +
// up); NX activation arrays share the weight loads and add into the same
// accumulators (an fp32 activation carried as fp16 hi + lo).
constexpr int kUpBatch = 8;   // loads per operand kind in flight per lane

template <int NM, int NX, int NB>
__device__ __forceinline__ void gemm_quarters(f32x16 (&acc)[NM][NB], const h16* const (&wrow)[NM],
                                              const h16* const (&xs)[NX], int ldx, int nch, int B,
                                              int wave, int li, int half) {
    const int npair = nch >> 1;
    const int p0 = (npair * wave) / 4, p1 = (npair * (wave + 1)) / 4;
    constexpr int UB = kUpBatch / (NB * NX) > 1 ? kUpBatch / (NB * NX) : 2;   // pairs per batch
    auto ldx_ = [&](int ix, int nb, int c) {
        return ld16(xs[ix] + (size_t)min(nb * 32 + li, B - 1) * ldx + (size_t)c * 8);
    };
    auto mfma = [&](const u32x4 (&wv)[NM], const u32x4 (&xv)[NX][NB]) {
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const f16x8 a8 = __builtin_bit_cast(f16x8, wv[m]);
            const f16x4 alo = {a8[0], a8[1], a8[2], a8[3]}, ahi = {a8[4], a8[5], a8[6], a8[7]};
#pragma unroll
            for (int ix = 0; ix < NX; ++ix)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const f16x8 x8 = __builtin_bit_cast(f16x8, xv[ix][nb]);
                    const f16x4 xlo = {x8[0], x8[1], x8[2], x8[3]}, xhi = {x8[4], x8[5], x8[6], x8[7]};
                    acc[m][nb] = __builtin_amdgcn_mfma_f32_32x32x8f16(alo, xlo, acc[m][nb], 0, 0, 0);
                    acc[m][nb] = __builtin_amdgcn_mfma_f32_32x32x8f16(ahi, xhi, acc[m][nb], 0, 0, 0);
                }
        }
    };
    int p = p0;
    for (; p + UB <= p1; p += UB) {
        u32x4 wv[UB][NM], xv[UB][NX][NB];
#pragma unroll
        for (int k = 0; k < UB; ++k) {
            const int c = 2 * (p + k) + half;
#pragma unroll
            for (int m = 0; m < NM; ++m) wv[k][m] = ld16_stream(wrow[m] + (size_t)c * 8);
#pragma unroll
            for (int ix = 0; ix < NX; ++ix)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) xv[k][ix][nb] = ldx_(ix, nb, c);
        }
#pragma unroll
        for (int k = 0; k < UB; ++k) mfma(wv[k], xv[k]);
        // keep the batch's loads ahead of its MFMAs: left alone, the scheduler
        // interleaves them and only one or two loads are ever in flight
        __builtin_amdgcn_sched_group_barrier(0x0020, UB * (NM + NX * NB), 0);   // VMEM reads
        __builtin_amdgcn_sched_group_barrier(0x0008, UB * 2 * NM * NX * NB, 0); // MFMA
    }
    for (; p < p1; ++p) {
        const int c = 2 * p + half;
        u32x4 wv[NM], xv[NX][NB];
#pragma unroll
        for (int m = 0; m < NM; ++m) wv[m] = ld16_stream(wrow[m] + (size_t)c * 8);
#pragma unroll
        for (int ix = 0; ix < NX; ++ix)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) xv[ix][nb] = ldx_(ix, nb, c);
        mfma(wv, xv);
    }
    if ((nch & 1) && wave == 3) {   // odd chunk count: the last chunk, half 1 feeds zero weights
        const int c = nch - 1;
        u32x4 wv[NM], xv[NX][NB];
#pragma unroll
        for (int m = 0; m < NM; ++m) wv[m] = half ? u32x4{0u, 0u, 0u, 0u} : ld16_stream(wrow[m] + (size_t)c * 8);
#pragma unroll
        for (int ix = 0; ix < NX; ++ix)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) xv[ix][nb] = ldx_(ix, nb, c);
        mfma(wv, xv);
    }
}

// Sum the four K quarters of accumulator block acc (one matrix, one token
// block) into out[32][33]: output (row r, token n) lives at element
// e = (r/8)*4 + r%4, lane n + 32*((r/4)%2) of every wave.  Two barriers.
__device__ __forceinline__ void sum_quarters(const f32x16& acc, float (&red)[4][16][64], float (&out)[32][33],
                                             int wave, int lane) {
#pragma unroll
    for (int e = 0; e < 16; ++e) red[wave][e][lane] = acc[e];
    __syncthreads();
    for (int o = threadIdx.x; o < 1024; o += 256) {
        const int r = o >> 5, n = o & 31;
        const int e = (r >> 3) * 4 + (r & 3), ln = n + 32 * ((r >> 2) & 1);
        out[r][n] = red[0][e][ln] + red[1][e][ln] + red[2][e][ln] + red[3][e][ln];
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Up GEMM over the union rows: bias, activation and the token mask give A,
// stored token-major as hi/lo fp16 pairs: aT[t][u].
template <bool REGLU, int NB>
__global__ __launch_bounds__(256) void k_union_up(const h16* __restrict__ x, int B, int d, int ffn,
                                                  const h16* __restrict__ Wup,
                                                  const float* __restrict__ bup,
                                                  const h16* __restrict__ Wg,
                                                  const float* __restrict__ bg,
                                                  const int32_t* __restrict__ ulist,
                                                  const uint32_t* __restrict__ tmask,
                                                  const uint32_t* __restrict__ ucount, int W,
                                                  int Bp, int lda, h16* __restrict__ a_hi,
                                                  h16* __restrict__ a_lo) {
    constexpr int NM = REGLU ? 2 : 1;
    __shared__ float s_red[4][16][64];
    __shared__ float s_sum[NM][32][33];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 31, half = lane >> 5;
    const int U = (int)min(*ucount, (uint32_t)ffn);
    const int nrb = (U + 31) / 32;
    for (int rb = blockIdx.x; rb < nrb; rb += gridDim.x) {
        const int row = ulist[min(rb * 32 + li, U - 1)];
        const h16* wrow[NM];
        wrow[0] = Wup + (size_t)row * d;
        if (REGLU) wrow[NM - 1] = Wg + (size_t)row * d;
        const h16* xs[1] = {x};
        f32x16 acc[NM][NB];
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[m][nb] = f32x16{};
        gemm_quarters<NM, 1, NB>(acc, wrow, xs, d, d >> 3, B, wave, li, half);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int m = 0; m < NM; ++m) sum_quarters(acc[m][nb], s_red, s_sum[m], wave, lane);
            for (int o = threadIdx.x; o < 1024; o += 256) {
                const int r = o >> 5, n = o & 31;
                const int uu = rb * 32 + r, t = nb * 32 + n;
                if (uu < U && t < Bp) {
                    float av = 0.f;
                    const int nrow = ulist[uu];
                    if (t < B && ((tmask[(size_t)nrow * W + (t >> 5)] >> (t & 31)) & 1u)) {
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
// Batched predictor.  Hidden layer: H = act(P1 X^T + b1), rows of P1 against
// the tokens.  Grid = (32-row blocks, KS splits of K): each workgroup writes
// the fp32 partial of its K range with device-coherent stores and arrives on
// its row block's counter; the last of the KS to arrive adds the partials in
// split order, applies b1 and the activation, writes h token-major as an fp16
// hi/lo pair (h itself is never rounded to fp16: hi + lo carries about 22
// significant bits) and puts the counter back to 0.
template <int NB>
__global__ __launch_bounds__(256) void k_bpred_hidden(const h16* __restrict__ x, int B, int d,
                                                      const h16* __restrict__ P1,
                                                      const float* __restrict__ b1, int relu, int r,
                                                      int ldh, h16* __restrict__ h_hi,
                                                      h16* __restrict__ h_lo, float* __restrict__ part,
                                                      uint32_t* __restrict__ ctr, int KS) {
    __shared__ float s_red[4][16][64];
    __shared__ float s_sum[32][33];
    __shared__ int s_last;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 31, half = lane >> 5;
    const int rb = blockIdx.x, ks = blockIdx.y;
    const int nch = d >> 3;
    const int c0 = (int)(((long long)nch * ks) / KS), c1 = (int)(((long long)nch * (ks + 1)) / KS);
    const int Bp = NB * 32;
    const h16* wrow[1] = {P1 + (size_t)min(rb * 32 + li, r - 1) * d + (size_t)c0 * 8};
    const h16* xs[1] = {x + (size_t)c0 * 8};
    f32x16 acc[1][NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[0][nb] = f32x16{};
    gemm_quarters<1, 1, NB>(acc, wrow, xs, d, c1 - c0, B, wave, li, half);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        sum_quarters(acc[0][nb], s_red, s_sum, wave, lane);
        for (int o = threadIdx.x; o < 1024; o += 256) {
            const int rr = o >> 5, n = o & 31;
            const int j = rb * 32 + rr, t = nb * 32 + n;
            if (j < r && t < B) st_coherent(&part[((size_t)ks * Bp + t) * r + j], s_sum[rr][n]);
        }
        __syncthreads();
    }
    wait_own_memory();
    __syncthreads();
    if (threadIdx.x == 0) {
        const int last = fetch_add(&ctr[rb], 1u) == (uint32_t)(KS - 1);
        if (last) st_flag(&ctr[rb], 0u);
        s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    for (int o = threadIdx.x; o < 32 * B; o += 256) {
        const int rr = o / B, t = o % B;
        const int j = rb * 32 + rr;
        if (j >= r) continue;
        float sv = b1 ? b1[j] : 0.f;
        for (int k = 0; k < KS; ++k) sv += ld_coherent(&part[((size_t)k * Bp + t) * r + j]);
        const float hv = relu ? fmaxf(sv, 0.f) : sv;
        const h16 hi = (h16)hv;
        h_hi[(size_t)t * ldh + j] = hi;
        h_lo[(size_t)t * ldh + j] = (h16)(hv - (float)hi);
    }
}

// Logits: Z = P2 H^T + b2 with both halves of h, then the strict test
// z > thr per (neuron, token); each 32-neuron tile gives one 32-bit mask per
// token (bit r = neuron 32*tile + r).
template <int NB>
__global__ __launch_bounds__(256) void k_bpred_logits(const h16* __restrict__ P2,
                                                      const float* __restrict__ b2, int B, int r,
                                                      int ffn, float thr, int ldh,
                                                      const h16* __restrict__ h_hi,
                                                      const h16* __restrict__ h_lo,
                                                      uint32_t* __restrict__ masks32) {
    __shared__ float s_red[4][16][64];
    __shared__ float s_sum[32][33];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 31, half = lane >> 5;
    const int nrb = (ffn + 31) / 32;
    for (int rb = blockIdx.x; rb < nrb; rb += gridDim.x) {
        const h16* wrow[1] = {P2 + (size_t)min(rb * 32 + li, ffn - 1) * r};
        const h16* xs[2] = {h_hi, h_lo};
        f32x16 acc[1][NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[0][nb] = f32x16{};
        gemm_quarters<1, 2, NB>(acc, wrow, xs, ldh, r >> 3, B, wave, li, half);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            sum_quarters(acc[0][nb], s_red, s_sum, wave, lane);
            if (threadIdx.x < 32) {
                const int n = threadIdx.x, t = nb * 32 + n;
                uint32_t m = 0;
                for (int rr = 0; rr < 32; ++rr) {
                    const int i = rb * 32 + rr;
                    if (i < ffn && s_sum[rr][n] + (b2 ? b2[i] : 0.f) > thr) m |= 1u << rr;
                }
                if (t < B) masks32[(size_t)t * nrb + rb] = m;
            }
            __syncthreads();
        }
    }
}

// One workgroup per token: the token's 32-bit tile masks in neuron order ->
// popcount prefix -> ascending idx and count.
__global__ __launch_bounds__(256) void k_bpred_compact(const uint32_t* __restrict__ masks32, int ffn,
                                                       int32_t* __restrict__ idx, int32_t* __restrict__ count) {
    __shared__ uint32_t s_part[4];
    const int tok = blockIdx.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ntiles = (ffn + 31) / 32;
    const uint32_t* mk = masks32 + (size_t)tok * ntiles;
    int32_t* out = idx + (size_t)tok * ffn;
    uint32_t base = 0;
    for (int t0 = 0; t0 < ntiles; t0 += 2048) {
        uint32_t m8[8];
        uint32_t mine = 0;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int t = t0 + tid * 8 + q;
            m8[q] = t < ntiles ? mk[t] : 0u;
            mine += (uint32_t)__popc(m8[q]);
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
        for (int q = 0; q < 8; ++q) {
            uint32_t m = m8[q];
            const int t = t0 + tid * 8 + q;
            while (m) {
                out[pos++] = t * 32 + __builtin_ctz(m);
                m &= m - 1;
            }
        }
        base += total;
        __syncthreads();
    }
    if (tid == 0) count[tok] = (int32_t)base;
}

// ---------------------------------------------------------------------------
// Down GEMM.  Grid = (128-column tiles, G chunks of the union).  Rows of
// W_down are neuron-major, so the contraction index (the union entry) runs
// across rows: each stage of KS union rows x 128 columns, and the stage's
// activations (hi and lo, KS entries x 32*NB tokens), are loaded with
// coalesced 16-byte loads into registers and written to LDS; the next
// stage's loads are issued before the current one is multiplied.  The MFMA
// operands come from LDS: 4 consecutive union rows of one column per lane
// (W) and 4 consecutive union entries of one token per lane (A).  Wave w
// owns columns 32w..32w+31 of the tile.  Chunk partials go to the
// workspace; k_union_reduce adds them in chunk order.
constexpr int kDnCols = 128;
constexpr int kDnIds = 4096;   // union entries per chunk staged in LDS (G is sized for it)

template <int NB>
__global__ __launch_bounds__(256) void k_union_down(const h16* __restrict__ Wd, int d, int ffn,
                                                    const int32_t* __restrict__ ulist,
                                                    const uint32_t* __restrict__ ucount,
                                                    const h16* __restrict__ a_hi,
                                                    const h16* __restrict__ a_lo, int Bp, int lda,
                                                    float* __restrict__ partial, int G) {
    constexpr int KS = NB == 1 ? 128 : (NB == 2 ? 64 : 32);   // union rows per stage
    constexpr int BT = NB * 32;                               // tokens in the tile
    constexpr int NW = KS / 16;                               // W loads per thread per stage
    constexpr int NA = 2 * BT * KS / 8 / 256;                 // A loads per thread per stage (= 4)
    static_assert(NA * 256 * 8 == 2 * BT * KS, "A stage must split evenly");
    __shared__ h16 s_w[KS][kDnCols + 8];
    __shared__ __align__(16) h16 s_a[2][BT][KS + 8];          // [hi/lo][token][entry]
    __shared__ int32_t s_ids[kDnIds];
    const int tile = blockIdx.x, chunk = blockIdx.y;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 31, half = lane >> 5;
    const int U = (int)min(*ucount, (uint32_t)ffn);
    // chunk starts are multiples of 8 so 16-byte A loads stay aligned
    const int per = min((((U + G - 1) / G) + 7) & ~7, kDnIds);
    const int u0 = min(U, chunk * per), u1 = min(U, u0 + per);
    const int n_ids = u1 - u0;
    const int c0 = tile * kDnCols;
    for (int i = tid; i < n_ids; i += 256) s_ids[i] = ulist[u0 + i];
    __syncthreads();

    f32x16 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16{};

    const int sr = tid >> 4, sc = (tid & 15) * 8;   // W staging: rows sr + 16k, 8 columns at sc
    const bool col_ok = c0 + sc < d;
    u32x4 vw[NW], va[NA];
    auto issue = [&](int s0) {
#pragma unroll
        for (int k = 0; k < NW; ++k) {
            const int rr = s0 + sr + 16 * k;   // chunk-relative union row
            vw[k] = (rr < n_ids && col_ok) ? ld16_stream(Wd + (size_t)s_ids[rr] * d + c0 + sc)
                                           : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int k = 0; k < NA; ++k) {
            const int q = tid + 256 * k;
            const int which = q / (BT * KS / 8), rem = q % (BT * KS / 8);
            const int t = rem / (KS / 8), e = (rem % (KS / 8)) * 8;   // entries s0+e .. +7
            const h16* src = (which ? a_lo : a_hi) + (size_t)t * lda + u0 + s0 + e;
            va[k] = (s0 + e < n_ids) ? *reinterpret_cast<const u32x4*>(src) : u32x4{0u, 0u, 0u, 0u};
        }
    };
    if (n_ids > 0) issue(0);
    const int col = wave * 32 + li;   // column within the tile
    for (int s0 = 0; s0 < n_ids; s0 += KS) {
        __syncthreads();   // the previous stage is no longer read from LDS
#pragma unroll
        for (int k = 0; k < NW; ++k) *reinterpret_cast<u32x4*>(&s_w[sr + 16 * k][sc]) = vw[k];
#pragma unroll
        for (int k = 0; k < NA; ++k) {
            const int q = tid + 256 * k;
            const int which = q / (BT * KS / 8), rem = q % (BT * KS / 8);
            const int t = rem / (KS / 8), e = (rem % (KS / 8)) * 8;
            f16x8 v = __builtin_bit_cast(f16x8, va[k]);
#pragma unroll
            for (int j = 0; j < 8; ++j)   // entries past the chunk hold stale data: zero them
                if (s0 + e + j >= n_ids) v[j] = (h16)0.f;
            *reinterpret_cast<f16x8*>(&s_a[which][t][e]) = v;
        }
        __syncthreads();
        if (s0 + KS < n_ids) issue(s0 + KS);
        const int sn = min(KS, n_ids - s0);
        for (int kk = 0; kk < sn; kk += 8) {
            const int kr = kk + 4 * half;     // this lane's 4 union rows: kr .. kr+3 (zero past sn)
            const f16x4 wv = {s_w[kr][col], s_w[kr + 1][col], s_w[kr + 2][col], s_w[kr + 3][col]};
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int t = nb * 32 + li;
                const f16x4 ah = *reinterpret_cast<const f16x4*>(&s_a[0][t][kr]);
                const f16x4 al = *reinterpret_cast<const f16x4*>(&s_a[1][t][kr]);
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
                       ctr, ulist, ucount);
    int gu = (ffn + 31) / 32;
    if (gu > 1024) gu = 1024;
#define PI_UP(R, N)                                                                                  \
    hipLaunchKernelGGL((k_union_up<R, N>), dim3(gu), dim3(256), 0, s, x, B, d, ffn, Wup, bup, Wg, bg, \
                       ulist, tmask, ucount, L.W, L.Bp, L.lda, a_hi, a_lo)
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

hipError_t launch_bpredict(const h16* x, int B, int d, const h16* P1, const float* b1, bool relu,
                          const h16* P2, const float* b2, int r, int ffn, float thr, int32_t* idx,
                          int32_t* count, const BPredLayout& L, char* ws, char* hdr, hipStream_t s) {
    h16* h_hi = reinterpret_cast<h16*>(ws + L.h_hi);
    h16* h_lo = reinterpret_cast<h16*>(ws + L.h_lo);
    uint32_t* masks32 = reinterpret_cast<uint32_t*>(ws + L.masks32);
    float* hpart = reinterpret_cast<float*>(ws + L.hpart);
    uint32_t* ctr = reinterpret_cast<uint32_t*>(hdr + Sync::bpred_ctr);
    const int NB = L.Bp / 32;
    const dim3 gh((r + 31) / 32, L.KS);
    int gl = (ffn + 31) / 32;
    if (gl > 2048) gl = 2048;
#define PI_BH(N) hipLaunchKernelGGL((k_bpred_hidden<N>), gh, dim3(256), 0, s, x, B, d, P1, b1, (int)relu, r, L.ldh, h_hi, h_lo, hpart, ctr, L.KS)
#define PI_BL(N) hipLaunchKernelGGL((k_bpred_logits<N>), dim3(gl), dim3(256), 0, s, P2, b2, B, r, ffn, thr, L.ldh, h_hi, h_lo, masks32)
    if (NB == 1) { PI_BH(1); PI_BL(1); }
    else if (NB == 2) { PI_BH(2); PI_BL(2); }
    else if (NB == 3) { PI_BH(3); PI_BL(3); }
    else { PI_BH(4); PI_BL(4); }
#undef PI_BH
#undef PI_BL
    hipLaunchKernelGGL(k_bpred_compact, dim3(B), dim3(256), 0, s, masks32, ffn, idx, count);
    return hipGetLastError();
}

}  // namespace pi
