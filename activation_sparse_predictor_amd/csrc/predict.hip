// Predictor kernels: the per-layer MLP that marks the neurons expected to fire
// (PowerInfer reading report, Part A section 2.3, module 3), with the active
// set compacted into an ascending index list on the device.
//
//   k_pred_hidden   h = act(P1 x + b1)            P1 r x d fp16, h fp32
//   k_pred_compact  z = P2 h + b2 ; active = z > ln(tau/(1-tau))
//                   -> idx (ascending), count     P2 ffn x r fp16
//
// Both stream a weight matrix from HBM once; every step stays on the device.
#include "common.hpp"
#include "internal.hpp"

namespace pi {

// ---------------------------------------------------------------------------
// Hidden layer.  One wave per row of P1; the 64 lanes read the row in 1 KB
// steps (16 B per lane), up to 8 steps in flight, and fold the fp16 products
// into fp32 with v_dot2.  Tokens are handled TB at a time so each row is read
// from HBM once per TB tokens.  The kernel also zeroes the look-back words
// and tickets that the compaction kernel after it on the stream relies on.
template <int TB>
__global__ __launch_bounds__(256) void k_pred_hidden(const h16* __restrict__ x, int B, int d,
                                                     const h16* __restrict__ P1,
                                                     const float* __restrict__ b1, int relu,
                                                     int r, float* __restrict__ h,
                                                     uint32_t* __restrict__ clear, int n_clear) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n_clear; i += gridDim.x * 256) clear[i] = 0u;

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + wave;
    if (row >= r) return;
    const h16* prow = P1 + (size_t)row * d;
    const int nch = d >> 3;
    const float bias = b1 ? b1[row] : 0.f;

    for (int t0 = 0; t0 < B; t0 += TB) {
        float acc[TB];
#pragma unroll
        for (int t = 0; t < TB; ++t) acc[t] = 0.f;
        for (int c0 = lane; c0 < nch; c0 += 64 * 8) {
            u32x4 w[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int c = c0 + u * 64;
                if (c < nch) w[u] = ld16_stream(prow + (size_t)c * 8);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int c = c0 + u * 64;
                if (c < nch) {
#pragma unroll
                    for (int t = 0; t < TB; ++t)
                        if (t0 + t < B)
                            acc[t] = dot8_h(w[u], ld16(x + (size_t)(t0 + t) * d + (size_t)c * 8), acc[t]);
                }
            }
        }
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            const float s = group_sum<64>(acc[t]) + bias;
            if (lane == 0 && t0 + t < B) h[(size_t)(t0 + t) * r + row] = relu ? fmaxf(s, 0.f) : s;
        }
    }
}

// ---------------------------------------------------------------------------
// Logits, threshold and ordered compaction.  A workgroup owns a tile of 64
// consecutive neurons for one token: LPR lanes cooperate on a row of P2 (16 B
// each, so a load instruction covers 256/LPR rows x LPR*16 B contiguous), h
// sits in LDS, and each row's flag is the strict test z > thr.
//
// The tile's 64 flags become one wave ballot.  Its position in the global
// list is found with a decoupled look-back over the preceding tiles of the
// same token: each tile publishes its own count as soon as it is known
// (kAgg) and its running total once its predecessors are resolved (kInc);
// wave 0 inspects 64 predecessors per step.  Tile numbers are taken from an
// atomic ticket, so every tile waits only on tiles that have already
// started, which guarantees progress whatever the dispatch order.  Waiting
// is bounded; on overrun the token's count is set to -1 (an impossible
// value the host can detect) instead of hanging.
constexpr uint32_t kAgg = 1u << 30;
constexpr uint32_t kInc = 1u << 31;
constexpr uint32_t kVal = (1u << 30) - 1u;
constexpr int kSpinLimit = 1 << 20;

template <int LPR>
__global__ __launch_bounds__(256) void k_pred_compact(const h16* __restrict__ P2,
                                                      const float* __restrict__ b2,
                                                      const float* __restrict__ h, int r, int ffn,
                                                      float thr, int ntiles,
                                                      uint32_t* __restrict__ status,
                                                      uint32_t* __restrict__ tickets,
                                                      int32_t* __restrict__ idx,
                                                      int32_t* __restrict__ count) {
    extern __shared__ float sh_h[];
    __shared__ uint32_t s_tile;
    __shared__ uint32_t s_act[kPredTile];
    constexpr int RP = 256 / LPR;  // rows per pass
    static_assert(kPredTile % RP == 0, "tile must be a whole number of passes");

    const int tok = blockIdx.y;
    const int tid = threadIdx.x;
    if (tid == 0) s_tile = fetch_add(&tickets[tok], 1u);
    for (int i = tid; i < r; i += 256) sh_h[i] = h[(size_t)tok * r + i];
    __syncthreads();
    const int tile = (int)s_tile;

    const int grp = tid / LPR, p = tid % LPR;
    const int nch = r >> 3;
#pragma unroll
    for (int pass = 0; pass < kPredTile / RP; ++pass) {
        const int rl = pass * RP + grp;
        const int row = tile * kPredTile + rl;
        float acc = 0.f;
        if (row < ffn) {
            const h16* prow = P2 + (size_t)row * r;
            for (int c0 = p; c0 < nch; c0 += LPR * 8) {
                u32x4 w[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int c = c0 + u * LPR;
                    if (c < nch) w[u] = ld16_stream(prow + (size_t)c * 8);
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int c = c0 + u * LPR;
                    if (c < nch) acc = dot8_hf(w[u], sh_h + c * 8, acc);
                }
            }
        }
        acc = group_sum<LPR>(acc);
        if (p == 0) s_act[rl] = (row < ffn) && (acc + (b2 ? b2[row] : 0.f) > thr);
    }
    __syncthreads();
    if (tid >= 64) return;

    const int lane = tid;
    const uint64_t m = __ballot(s_act[lane] != 0u);
    const uint32_t agg = (uint32_t)__popcll(m);
    uint32_t* st = status + (size_t)tok * ntiles;
    uint32_t excl = 0;
    bool fail = false;
    if (tile == 0) {
        if (lane == 0) st_flag(&st[0], kInc | agg);
    } else {
        if (lane == 0) st_flag(&st[tile], kAgg | agg);
        int base = tile - 1;
        int spins = 0;
        for (;;) {
            const int j = base - lane;
            const uint32_t v = (j >= 0) ? ld_flag(&st[j]) : kInc;
            const uint64_t inc = __ballot((v & kInc) != 0u);
            const uint64_t ready = __ballot(v != 0u);
            if (inc != 0ull) {
                const int k = __ffsll((unsigned long long)inc) - 1;
                const uint64_t need = (k >= 63) ? ~0ull : ((2ull << k) - 1ull);
                if ((ready & need) == need) {
                    excl += group_sum_u32<64>(lane <= k ? (v & kVal) : 0u);
                    break;
                }
            } else if (ready == ~0ull) {
                excl += group_sum_u32<64>(v & kVal);
                base -= 64;
                continue;
            }
            if (++spins > kSpinLimit) {
                fail = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        fail = fail || excl >= kVal || excl + agg > (uint32_t)ffn;
        if (lane == 0) st_flag(&st[tile], kInc | (fail ? kVal : (excl + agg)));
    }
    if (!fail && ((m >> lane) & 1ull))
        idx[(size_t)tok * ffn + excl + rank_below(m)] = tile * kPredTile + lane;
    if (tile == ntiles - 1 && lane == 0) count[tok] = fail ? -1 : (int32_t)(excl + agg);
}

hipError_t launch_pred_hidden(const h16* x, int B, int d, const h16* P1, const float* b1,
                              bool relu, int r, float* h, uint32_t* clear, int n_clear,
                              hipStream_t s) {
    dim3 grid((r + 3) / 4);
    if (B == 1)
        hipLaunchKernelGGL(k_pred_hidden<1>, grid, dim3(256), 0, s, x, B, d, P1, b1, (int)relu, r,
                           h, clear, n_clear);
    else
        hipLaunchKernelGGL(k_pred_hidden<4>, grid, dim3(256), 0, s, x, B, d, P1, b1, (int)relu, r,
                           h, clear, n_clear);
    return hipGetLastError();
}

hipError_t launch_pred_compact(const h16* P2, const float* b2, const float* h, int B, int r,
                               int ffn, float thr, uint32_t* status, uint32_t* tickets,
                               int32_t* idx, int32_t* count, hipStream_t s) {
    const int ntiles = pred_tiles(ffn);
    dim3 grid(ntiles, B);
    const size_t shm = (size_t)r * sizeof(float);
    const int nch = r / 8;
    if (nch >= 16)
        hipLaunchKernelGGL(k_pred_compact<16>, grid, dim3(256), shm, s, P2, b2, h, r, ffn, thr,
                           ntiles, status, tickets, idx, count);
    else if (nch >= 8)
        hipLaunchKernelGGL(k_pred_compact<8>, grid, dim3(256), shm, s, P2, b2, h, r, ffn, thr,
                           ntiles, status, tickets, idx, count);
    else
        hipLaunchKernelGGL(k_pred_compact<4>, grid, dim3(256), shm, s, P2, b2, h, r, ffn, thr,
                           ntiles, status, tickets, idx, count);
    return hipGetLastError();
}

}  // namespace pi
